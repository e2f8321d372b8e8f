"""The allocation-free forward (gdn_chunk_fwd_noalloc, for callers that cannot allocate) against
the workspace entry point gdn_chunk_fwd, through the C ABI: two calls in a row, the second with a
smaller input, each bitwise equal to gdn_chunk_fwd on the same inputs (the same kernels run on
the same values; only the workspace's address differs)."""
import numpy as np
import pytest

from gdn_inputs import make_inputs
from gpu_util import args_of, to_dev

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")


@pytest.fixture(scope="module")
def gdn():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import linear_attention_recurrence_prefill_amd as m

    m.load_library()
    return m


def _both(gdn, inp, **kw):
    d = to_dev(inp)
    N = len(inp["cu_seqlens"]) - 1
    T, H, D = inp["v"].shape
    ref_o, ref_ht = gdn.chunk_fwd(*args_of(d), d["cu_seqlens"], d["h0"], **kw)
    o = torch.full_like(d["v"], float("nan"))
    ht = torch.full((N, H, D, D), float("nan"), device="cuda")
    gdn.chunk_fwd_noalloc(*args_of(d), d["cu_seqlens"], d["h0"], out=o, final_state=ht, **kw)
    torch.cuda.synchronize()
    return o, ht, ref_o, ref_ht


def test_noalloc_matches_the_workspace_entry_point(gdn):
    # 1: the 32K x 8-head prefill in exact mode (its split uses 48 MiB of scratch)
    big = make_inputs([32768], H=8, dk=128, dv=128, dtype="bf16", seed=601, h0_scale=0.3)
    cu_h = big["cu_seqlens"]
    from linear_attention_recurrence_prefill_amd.gdn import fwd_workspace_bytes

    d = to_dev(big)
    need = fwd_workspace_bytes(d["q"], d["cu_seqlens"], mode="exact", cu_seqlens_host=cu_h)
    print(f"[noalloc] call 1: 1 x 32768 tokens, H=8, exact, workspace {need} bytes", flush=True)
    assert need > 0
    o, ht, ro, rht = _both(gdn, big, mode="exact", cu_seqlens_host=cu_h)
    assert torch.equal(o, ro) and torch.equal(ht, rht)
    # 2: a smaller ragged batch with forced 2-chunk segments (more units per token), after it
    small = make_inputs([700, 65, 0, 1300], H=3, dk=128, dv=128, dtype="bf16", seed=602,
                        h0_scale=0.5, g_mu=-6.0)
    print("[noalloc] call 2: 4 documents, H=3, exact split into 2-chunk segments", flush=True)
    o, ht, ro, rht = _both(gdn, small, mode="exact", seg_chunks=2,
                           cu_seqlens_host=small["cu_seqlens"])
    assert torch.equal(o, ro) and torch.equal(ht, rht)
    # 3: truncate mode (no scratch needed) still runs through it
    o, ht, ro, rht = _both(gdn, small, mode="truncate", seg_chunks=2)
    assert torch.equal(o, ro) and torch.equal(ht, rht)
    assert not bool(torch.isnan(o).any())
