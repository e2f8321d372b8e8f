"""The GPU tests' comparison (tests/gpu_util.py) on planted CPU arrays: a mistake confined to one
chunk of one head of one document passes the whole-tensor relative L2 but fails the
per-(document, head) and per-block checks."""
import numpy as np
import pytest

from gpu_util import BLOCK_TOKENS, blocks_of, rel_l2, report, worst_part


def test_blocks_cover_documents_and_long_blocks():
    cu = np.array([0, 10, 74, 74 + 2 * BLOCK_TOKENS + 30, 74 + 2 * BLOCK_TOKENS + 30 + 4097])
    got = list(blocks_of(cu))
    # the 10-token document is skipped; the 64-token one is checked whole
    assert got[0] == (1, 10, 74)
    long0 = 74
    assert got[1] == (2, long0, long0 + 2 * BLOCK_TOKENS + 30)
    # the 30-token tail joins the second block
    assert got[2] == (2, long0, long0 + BLOCK_TOKENS)
    assert got[3] == (2, long0 + BLOCK_TOKENS, long0 + 2 * BLOCK_TOKENS + 30)
    last0 = long0 + 2 * BLOCK_TOKENS + 30
    assert got[4] == (3, last0, last0 + 4097)
    assert got[5] == (3, last0, last0 + BLOCK_TOKENS + 1)  # 1-token tail joins
    assert len(got) == 6


def test_planted_chunk_error_is_caught():
    rng = np.random.default_rng(0)
    T, H, D = 32768, 8, 32
    ref = rng.standard_normal((T, H, D))
    x = ref * (1 + 2.9e-3 * rng.standard_normal(ref.shape))  # the bf16 floor
    cu = np.array([0, T])
    assert rel_l2(x, ref) < 5e-3
    report("clean", x, ref, 5e-3, cu=cu)
    bad = x.copy()
    bad[64 * 100:64 * 101, 5] *= 1.25  # one chunk of one head, 25 % off
    assert rel_l2(bad, ref) < 5e-3  # the whole-tensor metric lets it through
    worst, where = worst_part(bad, ref, cu)
    assert worst > 5e-3 and "head 5" in where
    with pytest.raises(AssertionError):
        report("planted", bad, ref, 5e-3, cu=cu)


def test_planted_state_error_is_caught():
    rng = np.random.default_rng(1)
    N, H, D = 20, 16, 16
    ref = rng.standard_normal((N, H, D, D))
    bad = ref.copy()
    bad[7, 3] *= 1.01
    cu = np.arange(N + 1) * 64
    assert rel_l2(bad, ref) < 5e-3
    worst, where = worst_part(bad, ref, cu, states=True)
    assert abs(worst - 0.01) < 1e-9 and where == "sequence 7, head 3"
