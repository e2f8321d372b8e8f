"""Misuse handling on the GPU ("Step 10 · Making it fast": wrong boundaries in a packed batch mix
documents; "How to Speed Up GDN Kernels for Qwen Models", section "Using it, and the fine
print": misuse is refused).  Malformed tables reach only the validation kernel: the debug-mode
calls below return before any compute launch, and no forward or backward kernel is ever run on a
malformed table here."""
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


def _cu(vals):
    return torch.tensor(vals, dtype=torch.int32, device="cuda")


@pytest.mark.parametrize("vals,T,flags", [
    ([0, 100, 100, 300], 300, 0),
    ([0, 0], 0, 0),
    ([1, 100, 300], 300, 1),               # cu[0] != 0
    ([0, 200, 100, 300], 300, 2),          # descending
    ([0, 100, 299], 300, 4),               # cu[N] != T
    ([0, 100, 400], 300, 4 | 8),           # past T
    ([0, -5, 300], 300, 2 | 8),            # negative offset, then a rise
    ([5, 3, 400], 300, 1 | 2 | 4 | 8),
])
def test_validate_cu_seqlens(gdn, vals, T, flags):
    assert gdn.validate_cu_seqlens(_cu(vals), T) == flags


def test_validate_many_sequences(gdn):
    cu = np.arange(0, 64 * 5001, 64, dtype=np.int32)
    T = int(cu[-1])
    assert gdn.validate_cu_seqlens(torch.from_numpy(cu).cuda(), T) == 0
    cu[3777] = cu[3776] - 1
    assert gdn.validate_cu_seqlens(torch.from_numpy(cu).cuda(), T) == 2


def test_debug_mode_refuses_a_malformed_table_before_launching(gdn):
    """In debug mode the forward, the plan and the backward validate the device table first and
    return GDN_ERR_BAD_SHAPE (status 2) with the outputs untouched."""
    inp = make_inputs([100, 200], H=2, dk=128, dv=128, dtype="bf16", seed=11, with_dout=True)
    d = to_dev(inp)
    bad = _cu([0, 250, 200])  # descending: the host is never told (no cu_seqlens_host)
    o = torch.full_like(d["v"], 7.0)
    ht = torch.full((2, 2, 128, 128), 7.0, device="cuda")
    before = gdn.get_debug()
    gdn.set_debug(True)
    try:
        assert gdn.get_debug()
        for mode in ("exact", "truncate"):
            with pytest.raises(gdn.GdnError) as ei:
                gdn.chunk_fwd(*args_of(d), bad, None, mode=mode, out=o, final_state=ht)
            assert ei.value.status == 2 and "descending" in str(ei.value)
        with pytest.raises(gdn.GdnError) as ei:
            gdn.chunk_fwd_plan(d["g"], bad, 2, 128, torch.bfloat16, mode="truncate")
        assert ei.value.status == 2
        with pytest.raises(gdn.GdnError) as ei:
            gdn.chunk_bwd(*args_of(d), bad, d["dout"])
        assert ei.value.status == 2
        torch.cuda.synchronize()
        assert bool((o == 7.0).all()) and bool((ht == 7.0).all())
        # a valid table runs, and gives the same result as without the debug mode
        o1, ht1 = gdn.chunk_fwd(*args_of(d), d["cu_seqlens"], None)
    finally:
        gdn.set_debug(before)
    o2, ht2 = gdn.chunk_fwd(*args_of(d), d["cu_seqlens"], None)
    assert torch.equal(o1, o2) and torch.equal(ht1, ht2)


def test_debug_mode_refuses_a_host_copy_that_differs(gdn):
    """The host copy of cu_seqlens plans the split; in debug mode a copy that differs from the
    device table (both well formed) is refused with nothing launched, and a matching copy runs."""
    inp = make_inputs([100, 200], H=2, dk=128, dv=128, dtype="bf16", seed=14, with_dout=True)
    d = to_dev(inp)
    other = np.array([0, 150, 300], dtype=np.int32)  # well formed, not the device's [0, 100, 300]
    o = torch.full_like(d["v"], 7.0)
    before = gdn.get_debug()
    gdn.set_debug(True)
    try:
        for mode in ("exact", "truncate"):
            with pytest.raises(gdn.GdnError) as ei:
                gdn.chunk_fwd(*args_of(d), d["cu_seqlens"], None, mode=mode, out=o,
                              cu_seqlens_host=other)
            assert ei.value.status == 2 and "differs" in str(ei.value)
        with pytest.raises(gdn.GdnError) as ei:
            gdn.chunk_fwd_plan(d["g"], d["cu_seqlens"], 2, 128, torch.bfloat16, mode="truncate",
                               cu_seqlens_host=other)
        assert ei.value.status == 2
        with pytest.raises(gdn.GdnError) as ei:
            gdn.chunk_bwd(*args_of(d), d["cu_seqlens"], d["dout"], cu_seqlens_host=other)
        assert ei.value.status == 2
        torch.cuda.synchronize()
        assert bool((o == 7.0).all())
        o1, _ = gdn.chunk_fwd(*args_of(d), d["cu_seqlens"], None,
                              cu_seqlens_host=inp["cu_seqlens"])
    finally:
        gdn.set_debug(before)
    o2, _ = gdn.chunk_fwd(*args_of(d), d["cu_seqlens"], None)
    assert torch.equal(o1, o2)


def test_no_fault_flags_after_normal_runs(gdn):
    inp = make_inputs([3000], H=8, dk=128, dv=128, dtype="bf16", seed=12)
    d = to_dev(inp)
    for mode in ("exact", "truncate"):
        gdn.chunk_fwd(*args_of(d), d["cu_seqlens"], None, mode=mode)
    assert gdn.device_faults(clear=False) == 0


def test_binding_checks_caller_outputs(gdn):
    inp = make_inputs([100], H=2, dk=128, dv=128, dtype="bf16", seed=13)
    d = to_dev(inp)
    with pytest.raises(ValueError):
        gdn.chunk_fwd(*args_of(d), d["cu_seqlens"], None, out=torch.empty(100, 2, 64,
                                                                          device="cuda"))
    with pytest.raises(ValueError):
        gdn.chunk_fwd(*args_of(d), d["cu_seqlens"], None,
                      final_state=torch.empty(1, 2, 128, 128, dtype=torch.bfloat16,
                                              device="cuda"))
    with pytest.raises(ValueError):
        gdn.chunk_fwd(*args_of(d), d["cu_seqlens"], None,
                      final_state=torch.empty(1, 2, 128, 256, device="cuda")[..., :128])
