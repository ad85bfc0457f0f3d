"""The rocprofv3 summariser of bench.py (--summarize-profiles) on small synthetic
databases: dispatches of one kernel are split by launch order, and a kernel the summary
lists but the databases lack stops it with an error instead of a made-up row."""
import os
import sqlite3

import pytest

import bench

COUNTER_SETS = {
    "fetch": ["FETCH_SIZE"],
    "write": ["WRITE_SIZE"],
    "sq1": ["SQ_VALU_MFMA_BUSY_CYCLES", "GRBM_GUI_ACTIVE", "SQ_LDS_BANK_CONFLICT", "SQ_LDS_IDX_ACTIVE"],
    "sq2": ["SQ_INSTS_MFMA", "SQ_INSTS_VALU", "SQ_INSTS_VALU_TRANS_F32", "SQ_INSTS_SALU", "SQ_INSTS_LDS"],
}


def _kernels(drop=None):
    names = bench.PROFILE_HEAD + [k for _, k, _ in bench.PROFILE_OTHER] + [bench.PROFILE_COPY]
    out, seen = [], set()
    for n in names:
        if n in seen or n == drop:
            continue
        seen.add(n)
        launches = 10 if n == "splitkv_mfma_kernel<128>" else (15 if "combine" in n else 5)
        out.append((n, launches))
    return out


def _write_dbs(root, drop=None):
    kernels = _kernels(drop)
    os.makedirs(os.path.join(root, "trace"))
    c = sqlite3.connect(os.path.join(root, "trace", "run_results.db"))
    c.execute("create table kernels (name text, start integer, end integer)")
    t = 0
    for name, n in kernels:
        for i in range(n):
            # grouped decode: the first half of the launches take 200 us, the second 40 us
            us = (200 if i < n // 2 else 40) if name == "splitkv_mfma_kernel<128>" else 100
            c.execute("insert into kernels values (?, ?, ?)", (f"void fmha::(anonymous namespace)::{name}(x)", t, t + us * 1000))
            t += us * 1000 + 10
    c.commit()
    for pass_name, cnames in COUNTER_SETS.items():
        os.makedirs(os.path.join(root, pass_name))
        c = sqlite3.connect(os.path.join(root, pass_name, "run_results.db"))
        c.execute("create table counters_collection (kernel_name text, counter_name text, value real, dispatch_id integer)")
        disp = 0
        for name, n in kernels:
            for i in range(n):
                for cn in cnames:
                    v = 1000.0 + i
                    if name == bench.PROFILE_COPY and cn in ("FETCH_SIZE", "WRITE_SIZE"):
                        v = 512 * 1024.0
                    c.execute("insert into counters_collection values (?, ?, ?, ?)", (name, cn, v, disp))
                disp += 1
        c.commit()


def test_summaries_split_dispatches_by_launch_order(tmp_path):
    _write_dbs(str(tmp_path / "prof"))
    out = tmp_path / "profiles"
    bench.summarize_profiles(str(tmp_path / "prof"), str(out))
    text = (out / "splitkv_fp32wide_blocksparse_kernels.md").read_text()
    assert "| `split-KV on the matrix cores, 8 K/V heads` | 5 | 200.0 | 200.0 |" in text
    assert "| `split-KV on the matrix cores, 1 K/V head` | 5 | 40.0 | 40.0 |" in text
    assert "1024 MiB of K/V per launch in 200.0 µs = **5369 GB/s**" in text
    assert sorted(os.listdir(out)) == ["fwd_bwd_causal_b1h16n16384d128_hbm_counters.md",
                                       "fwd_bwd_causal_b1h16n16384d128_sq_counters.md",
                                       "fwd_bwd_causal_b1h16n16384d128_trace.md",
                                       "splitkv_fp32wide_blocksparse_kernels.md"]


@pytest.mark.parametrize("drop", ["splitkv_mfma_kernel<128>", "bwd_dq_kernel<128, 128, false, false, false>"])
def test_missing_kernel_is_an_error(tmp_path, drop):
    _write_dbs(str(tmp_path / "prof"), drop=drop)
    with pytest.raises(SystemExit, match="has no kernel-trace row"):
        bench.summarize_profiles(str(tmp_path / "prof"), str(tmp_path / "profiles"))


def test_missing_pass_is_an_error(tmp_path):
    with pytest.raises(SystemExit, match="missing"):
        bench.summarize_profiles(str(tmp_path), str(tmp_path / "profiles"))
