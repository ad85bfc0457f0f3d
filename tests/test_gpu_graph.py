"""HIP graph capture of the library's calls: a captured call replays to the same bits as
the eager call, replay after replay, with other eager work and synchronisations between
the replays. Covers the key-split forward (forward + combine, its workspace taken from
the graph's memory pool), the plain forward, the split-KV decode and the backward."""
import pytest
import torch

from tests.gpu_util import announce, device


def _capture(fn):
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    g = torch.cuda.CUDAGraph()
    with torch.cuda.stream(side):
        fn()                                  # warm-up on the capture stream
        torch.cuda.synchronize()
        with torch.cuda.graph(g, stream=side):
            outs = fn()
    torch.cuda.synchronize()
    return g, outs


def _replays_match(fn, n=4):
    """Capture fn, replay it n times with unrelated eager work in between, and check
    every replay against a fresh eager call bit for bit."""
    ref = [t.clone() for t in fn()]
    torch.cuda.synchronize()
    g, outs = _capture(fn)
    junk = torch.randn(1 << 20, device=device())
    for i in range(n):
        for t in outs:
            t.zero_()                         # replays must rewrite every output element
        torch.cuda.synchronize()
        g.replay()
        junk.mul_(1.0001).add_(0.5)           # eager work between replays
        torch.cuda.synchronize()
        for r, t in zip(ref, outs):
            assert torch.equal(r, t), f"replay {i} differs from the eager call"


@pytest.mark.gpu
@pytest.mark.parametrize("shape", [(1, 256, 8192, 8, 128, "causal"), (1, 2048, 2048, 16, 64, "none"),
                                   (2, 300, 5000, 3, 128, "sliding_window")])
def test_graph_replay_forward(shape):
    import block_sparse_attention_fmha_amd as fa
    B, Nq, Nk, H, D, kind = shape
    gen = torch.Generator(device="cpu").manual_seed(11)
    q = torch.randn(B, Nq, H, D, generator=gen).bfloat16().to(device())
    k = torch.randn(B, Nk, H, D, generator=gen).bfloat16().to(device())
    v = torch.randn(B, Nk, H, D, generator=gen).bfloat16().to(device())
    m = fa.Mask(kind, window=1000)
    split = fa.fwd_workspace_size(q, k, v, mask=m) > 0
    announce(f"graph replay fwd B={B} Nq={Nq} Nk={Nk} H={H} D={D} mask={kind} key_split={split}")
    _replays_match(lambda: fa.fmha_fwd(q, k, v, mask=m, bias_slope=-0.01))


@pytest.mark.gpu
def test_graph_replay_splitkv_and_backward():
    import block_sparse_attention_fmha_amd as fa
    gen = torch.Generator(device="cpu").manual_seed(12)
    q1 = torch.randn(2, 1, 8, 128, generator=gen).bfloat16().to(device())
    kc = torch.randn(2, 4096, 2, 128, generator=gen).bfloat16().to(device())
    vc = torch.randn(2, 4096, 2, 128, generator=gen).bfloat16().to(device())
    announce("graph replay split-KV decode B=2 H=8 Hkv=2 Nk=4096 splits=8")
    _replays_match(lambda: fa.fmha_fwd_splitkv(q1, kc, vc, 8))
    q, k, v, do = (torch.randn(1, 1024, 4, 128, generator=gen).bfloat16().to(device()) for _ in range(4))
    m = fa.Mask("causal")
    o, lse = fa.fmha_fwd(q, k, v, mask=m)
    announce("graph replay backward B=1 H=4 N=1024 D=128 causal")
    _replays_match(lambda: fa.fmha_bwd(q, k, v, o, lse, do, mask=m))
