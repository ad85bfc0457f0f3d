"""The localized gradient check of the GPU parity tests, exercised on the CPU: one wrong
128-row block must fail it even where the whole-tensor norm stays inside 1e-2, and
rounding-level noise everywhere must pass."""
import numpy as np
import pytest

from tests.gpu_util import GRAD_RTOL, check_grad, grad_local_errors


def _ref(seed, shape=(1, 4096, 4, 64)):
    return np.random.default_rng(seed).standard_normal(shape)


def test_uniform_rounding_noise_passes():
    ref = _ref(1)
    got = ref * (1 + 3e-3 * np.random.default_rng(2).standard_normal(ref.shape))
    check_grad("g", got, ref)


def test_one_bad_block_hides_in_the_global_norm_but_not_locally():
    ref = _ref(3)
    got = ref.copy()
    got[0, 1024:1152, 2] *= 1.05          # 5 % error in one 128-row block of head 2
    rel = np.linalg.norm(got - ref) / np.linalg.norm(ref)
    assert rel < GRAD_RTOL                # the whole-tensor check alone would pass
    _, ratio = grad_local_errors(got, ref)
    assert np.unravel_index(np.argmax(ratio), ratio.shape) == (0, 2, 8)
    with pytest.raises(AssertionError, match=r"head 2\) rows 1024\.\.1151"):
        check_grad("g", got, ref)


def test_one_bad_head_fails_the_slice_check():
    ref = _ref(4, (2, 512, 8, 32))
    got = ref.copy()
    got[1, :, 5] += 0.015 * ref[1, :, 5]   # 1.5 % on one head: under 1e-2 globally
    assert np.linalg.norm(got - ref) / np.linalg.norm(ref) < GRAD_RTOL
    with pytest.raises(AssertionError, match=r"\(batch 1, head 5\) norm-relative"):
        check_grad("g", got, ref)


def test_packed_layout_and_ragged_last_block():
    ref = _ref(5, (1000, 2, 16))          # [T, H, D]; last block has 1000 - 896 = 104 rows
    got = ref.copy()
    check_grad("g", got, ref)
    # block 896..999 of head 1: bound ~0.9 (2e-2 x ~41 + floor); slice bound ~1.26, whole ~1.79
    got[990, 1, 0] += 1.0
    with pytest.raises(AssertionError, match=r"rows 896\.\.1023"):
        check_grad("g", got, ref)


def test_zero_reference_blocks():
    ref = _ref(6, (1, 512, 1, 16))
    ref[0, 128:256] = 0.0                 # a block with no gradient (e.g. keys nobody sees)
    got = ref.copy()
    check_grad("g", got, ref)
    got[0, 130, 0, 3] = 1e-3              # under the block's floor share (~0.08): passes
    check_grad("g", got, ref)
    got[0, 130, 0, 3] = 0.5               # over it, still under 1e-2 of the whole (~0.78)
    with pytest.raises(AssertionError, match=r"rows 128\.\.255"):
        check_grad("g", got, ref)
