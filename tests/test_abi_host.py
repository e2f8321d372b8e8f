"""Host-side checks of the C ABI (no GPU needed): the library loads, exports every function
include/*.h declares, and rejects bad arguments before touching the device."""
import ctypes
import glob
import os
import re

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADERS = sorted(glob.glob(os.path.join(ROOT, "include", "*.h")))


def _declared_functions():
    names = set()
    for h in HEADERS:
        text = re.sub(r"/\*.*?\*/", "", open(h).read(), flags=re.S)
        names |= set(re.findall(r"\b(gdn_[a-z0-9_]+)\s*\(", text))
    return sorted(names)


@pytest.fixture(scope="module")
def lib():
    from linear_attention_recurrence_prefill_amd import gdn

    if not os.path.exists(gdn.LIB_PATH):
        pytest.fail("libgdn_mi355x.so is not built (run __graft_entry__.build())")
    return gdn.load_library()


def test_header_declares_the_boundary():
    names = _declared_functions()
    for required in ("gdn_chunk_fwd", "gdn_chunk_bwd", "gdn_chunk_fwd_workspace_size",
                     "gdn_chunk_bwd_workspace_size", "gdn_status_string", "gdn_last_error"):
        assert required in names


def test_library_exports_every_declared_function(lib):
    from linear_attention_recurrence_prefill_amd import gdn

    names = _declared_functions()
    assert set(names) == set(gdn.EXPORTS)
    for name in names:
        assert hasattr(lib, name), name


def _problem(**kw):
    from linear_attention_recurrence_prefill_amd.gdn import GdnProblem

    lib = _lib()
    p = GdnProblem()
    assert lib.gdn_problem_init(ctypes.byref(p), 1024, 2, 8, 128) == 0
    for k, v in kw.items():
        setattr(p, k, v)
    return p


def _lib():
    from linear_attention_recurrence_prefill_amd import gdn

    return gdn.load_library()


def test_problem_defaults(lib):
    p = _problem()
    assert (p.chunk, p.dtype, p.mode, p.scale, p.trunc_log_threshold) == (64, 1, 0, 1.0, -10.0)
    assert p.h0_seq_stride == 8 * 128 * 128


@pytest.mark.parametrize("field,value,status", [
    ("chunk", 32, 2), ("d_k", 96, 2), ("d_v", 64, 2), ("num_heads", 0, 2), ("num_seqs", 0, 2),
    ("total_tokens", -1, 2), ("dtype", 7, 3), ("mode", 5, 4), ("num_k_heads", 3, 2),
    ("num_k_heads", -1, 2), ("num_k_heads", 16, 2), ("qk_l2norm", 2, 4), ("reserved", 1, 2),
    ("h0_seq_stride", -1, 2)])
def test_bad_problem_rejected_on_host(lib, field, value, status):
    p = _problem(**{field: value})
    n = ctypes.c_size_t(0)
    assert lib.gdn_chunk_fwd_workspace_size(ctypes.byref(p), None, ctypes.byref(n)) == status
    assert lib.gdn_chunk_bwd_workspace_size(ctypes.byref(p), None, ctypes.byref(n)) == status
    assert lib.gdn_last_error()


def test_truncate_threshold_must_be_negative(lib):
    p = _problem(mode=1, trunc_log_threshold=0.5, seg_chunks=4)
    n = ctypes.c_size_t(0)
    assert lib.gdn_chunk_fwd_workspace_size(ctypes.byref(p), None, ctypes.byref(n)) == 4


def test_null_pointers_rejected_before_launch(lib):
    p = _problem()
    buf = (ctypes.c_char * 64)()
    ptr = ctypes.cast(buf, ctypes.c_void_p)
    # q missing
    st = lib.gdn_chunk_fwd(ctypes.byref(p), None, ptr, ptr, ptr, ptr, ptr, None, None, ptr, None,
                           None, 0, None)
    assert st == 1
    st = lib.gdn_chunk_bwd(ctypes.byref(p), ptr, ptr, ptr, ptr, ptr, ptr, None, None, None, None,
                           ptr, ptr, ptr, ptr, ptr, None, None, 0, None)
    assert st == 1


def test_misaligned_pointer_rejected(lib):
    p = _problem()
    buf = (ctypes.c_char * 256)()
    base = ctypes.addressof(buf)
    al = ctypes.c_void_p((base + 15) & ~15)
    mis = ctypes.c_void_p(((base + 15) & ~15) + 4)
    st = lib.gdn_chunk_fwd(ctypes.byref(p), mis, al, al, al, al, al, None, None, al, None, None,
                           0, None)
    assert st == 7


def test_host_cu_seqlens_checked(lib):
    p = _problem(mode=1, seg_chunks=4)
    cu = (ctypes.c_int32 * 3)(0, 700, 900)  # does not end at total_tokens = 1024
    n = ctypes.c_size_t(0)
    assert lib.gdn_chunk_fwd_workspace_size(ctypes.byref(p), cu, ctypes.byref(n)) == 2


def test_workspace_sizes(lib):
    # num_slots (P of the latency model) is given, so no device is queried
    n = ctypes.c_size_t(123)
    p = _problem(num_slots=1)  # num_seqs * H >= P: no split, no scratch
    assert lib.gdn_chunk_fwd_workspace_size(ctypes.byref(p), None, ctypes.byref(n)) == 0
    assert n.value == 0
    p = _problem(num_slots=256, dtype=0)  # fp32: the exact mode is never split
    assert lib.gdn_chunk_fwd_workspace_size(ctypes.byref(p), None, ctypes.byref(n)) == 0
    assert n.value == 0
    p = _problem(num_slots=256, mode=1)  # truncate mode: no scratch
    assert lib.gdn_chunk_fwd_workspace_size(ctypes.byref(p), None, ctypes.byref(n)) == 0
    assert n.value == 0
    assert lib.gdn_chunk_bwd_workspace_size(ctypes.byref(p), None, ctypes.byref(n)) == 0
    assert n.value > 1024 * 8 * 128 * 4


def test_exact_split_workspace(lib):
    """The exact mode's split (bf16, d = 128, num_seqs * H < P) needs per unit and head a pair
    (B, M) and a start state: 3 fp32 states of 128 x 128."""
    n = ctypes.c_size_t(0)
    state = 128 * 128 * 4
    p = _problem(num_slots=256, seg_chunks=4)
    cu = (ctypes.c_int32 * 3)(0, 512, 1024)  # 8 chunks each: 2 units each
    assert lib.gdn_chunk_fwd_workspace_size(ctypes.byref(p), cu, ctypes.byref(n)) == 0
    assert n.value == 3 * 4 * 8 * state
    cu = (ctypes.c_int32 * 3)(0, 256, 1024)  # 4 + 12 chunks: 1 + 3 units
    assert lib.gdn_chunk_fwd_workspace_size(ctypes.byref(p), cu, ctypes.byref(n)) == 0
    assert n.value == 3 * 4 * 8 * state
    p = _problem(num_slots=256, seg_chunks=16)  # every sequence is one unit: no split
    assert lib.gdn_chunk_fwd_workspace_size(ctypes.byref(p), cu, ctypes.byref(n)) == 0
    assert n.value == 0
    p = _problem(num_slots=256)  # latency model: L = 4 (floor); without cu a bound on the units
    assert lib.gdn_chunk_fwd_workspace_size(ctypes.byref(p), None, ctypes.byref(n)) == 0
    assert n.value >= 3 * 4 * 8 * state


def test_status_strings(lib):
    for s in range(9):
        assert lib.gdn_status_string(s)


def test_bwd_recompute_split_workspace(lib):
    """bf16, d = 128 with num_seqs * H < P: the backward's forward recompute runs the exact split,
    which adds per (unit, head) a pair (B, M), a start state and M transposed for the reverse
    walk (4 fp32 states of 128 x 128).
    Without the host cu_seqlens the unit count is bounded by ceil((ceil(T / 64) + N) / L) + N:
    T = 1024, N = 2, L = 4 (the forward's rule: 3 sqrt(8 * 16 / 256) rounds to 2, floored at 4)
    gives 7 units."""
    n1, n2 = ctypes.c_size_t(0), ctypes.c_size_t(0)
    p = _problem(num_slots=1)  # num_seqs * H >= P: the recompute is not split
    assert lib.gdn_chunk_bwd_workspace_size(ctypes.byref(p), None, ctypes.byref(n1)) == 0
    p = _problem(num_slots=256)
    assert lib.gdn_chunk_bwd_workspace_size(ctypes.byref(p), None, ctypes.byref(n2)) == 0
    assert n2.value - n1.value == 4 * 7 * 8 * 128 * 128 * 4
    p = _problem(num_slots=256, dtype=0)  # fp32: the general kernel, never split
    assert lib.gdn_chunk_bwd_workspace_size(ctypes.byref(p), None, ctypes.byref(n2)) == 0
    assert n2.value < n1.value * 2
    # truncate mode: the same split with warmup windows, no per-unit maps or states
    n3 = ctypes.c_size_t(0)
    p = _problem(num_slots=256, mode=1)
    assert lib.gdn_chunk_bwd_workspace_size(ctypes.byref(p), None, ctypes.byref(n3)) == 0
    assert n3.value == n1.value


@pytest.mark.parametrize("args,status", [
    ((0, 8, 0, 128, 1, 0), 2), ((4, 0, 0, 128, 1, 0), 2), ((4, 8, 0, 96, 1, 0), 2),
    ((4, 8, 0, 128, 5, 0), 3), ((4, 8, 3, 128, 1, 0), 2), ((4, 8, 16, 128, 1, 0), 2),
    ((4, 8, -1, 128, 1, 0), 2), ((4, 8, 2, 128, 1, 2), 4)])
def test_decode_step_rejects_bad_sizes(lib, args, status):
    buf = (ctypes.c_char * 64)()
    ptr = ctypes.cast(buf, ctypes.c_void_p)
    st = lib.gdn_decode_step(*args, 1.0, ptr, ptr, ptr, ptr, ptr, ptr, ptr, None)
    assert st == status
    assert lib.gdn_last_error()


def test_decode_step_rejects_null_pointer(lib):
    buf = (ctypes.c_char * 64)()
    ptr = ctypes.cast(buf, ctypes.c_void_p)
    assert lib.gdn_decode_step(4, 8, 0, 128, 1, 0, 1.0, ptr, None, ptr, ptr, ptr, ptr, ptr,
                               None) == 1


def _aligned_ptr(buf):
    return ctypes.c_void_p((ctypes.addressof(buf) + 15) & ~15)


@pytest.mark.parametrize("nbytes,status", [(0, 2), (24, 2), (15, 2)])
def test_calib_copy_rejects_bad_sizes(lib, nbytes, status):
    buf = (ctypes.c_char * 128)()
    ptr = _aligned_ptr(buf)
    assert lib.gdn_calib_copy(ptr, ptr, nbytes, None) == status
    assert lib.gdn_last_error()


def test_calib_copy_rejects_null_and_misaligned(lib):
    buf = (ctypes.c_char * 128)()
    ptr = _aligned_ptr(buf)
    assert lib.gdn_calib_copy(None, ptr, 64, None) == 1
    assert lib.gdn_calib_copy(ctypes.c_void_p(ptr.value + 4), ptr, 64, None) == 7


@pytest.mark.parametrize("waves,iters", [(0, 10), (9, 10), (4, 0), (4, (1 << 20) + 1)])
def test_calib_mfma_rejects_bad_sizes(lib, waves, iters):
    buf = (ctypes.c_char * 128)()
    assert lib.gdn_calib_mfma_bf16(_aligned_ptr(buf), waves, iters, None) == 2
    assert lib.gdn_calib_mfma_bf16(None, 4, 10, None) == 1


@pytest.mark.parametrize("dtype,d", [(1, 64), (1, 128), (0, 64), (0, 128)])
def test_qk_l2norm_accepted_for_every_dtype_and_size(lib, dtype, d):
    n = ctypes.c_size_t(0)
    p = _problem(qk_l2norm=1, d_k=d, d_v=d, dtype=dtype, num_slots=256)
    assert lib.gdn_chunk_fwd_workspace_size(ctypes.byref(p), None, ctypes.byref(n)) == 0
    assert lib.gdn_chunk_bwd_workspace_size(ctypes.byref(p), None, ctypes.byref(n)) == 0


def test_binding_has_every_compute_entry_point():
    """The Python binding offers each C compute entry point under its C name."""
    import linear_attention_recurrence_prefill_amd as pkg

    names = [n for n in _declared_functions()
             if n not in ("gdn_problem_init", "gdn_chunk_fwd_workspace_size",
                          "gdn_chunk_bwd_workspace_size", "gdn_status_string", "gdn_last_error")]
    for n in names:
        assert callable(getattr(pkg, n)), n


def test_validate_cu_seqlens_rejects_bad_arguments_on_the_host(lib):
    status = ctypes.c_void_p(16)  # never dereferenced: every call below fails its host checks
    assert lib.gdn_validate_cu_seqlens(None, 2, 10, status, None) == 1
    assert lib.gdn_validate_cu_seqlens(status, 2, 10, None, None) == 1
    assert lib.gdn_validate_cu_seqlens(status, 0, 10, status, None) == 2
    assert lib.gdn_validate_cu_seqlens(status, 2, -1, status, None) == 2
    assert lib.gdn_validate_cu_seqlens(status, 2, 1 << 31, status, None) == 2


def test_debug_switch(lib):
    before = lib.gdn_get_debug()
    try:
        assert lib.gdn_set_debug(1) == 0 and lib.gdn_get_debug() == 1
        assert lib.gdn_set_debug(0) == 0 and lib.gdn_get_debug() == 0
        assert lib.gdn_set_debug(2) == 4
    finally:
        lib.gdn_set_debug(before)
    assert lib.gdn_device_faults(None, 0) == 1
    assert lib.gdn_status_string(9) == b"a device-side check failed"


def test_noalloc_refuses_problems_beyond_its_scratch(lib):
    """gdn_chunk_fwd_noalloc refuses, on the host and before any device call, a problem whose
    workspace exceeds the static scratch (GDN_NOALLOC_SCRATCH_BYTES): here an exact split of
    1 x 2^21 tokens over 32 heads (8192 units of 192 KiB)."""
    from linear_attention_recurrence_prefill_amd.gdn import NOALLOC_SCRATCH_BYTES

    p = _problem(total_tokens=1 << 21, num_seqs=1, num_heads=32, mode=0, seg_chunks=4,
                 num_slots=256)
    n = ctypes.c_size_t(0)
    assert lib.gdn_chunk_fwd_workspace_size(ctypes.byref(p), None, ctypes.byref(n)) == 0
    assert n.value > NOALLOC_SCRATCH_BYTES
    fake = ctypes.c_void_p(1 << 20)  # aligned, never dereferenced
    rc = lib.gdn_chunk_fwd_noalloc(ctypes.byref(p), fake, fake, fake, fake, fake, fake, None,
                                   None, fake, None, None)
    assert rc == 6, lib.gdn_last_error()
    assert b"static scratch" in lib.gdn_last_error()


def test_exact_split_segment_length_fills_one_round(lib):
    """The exact split's segment length: the shortest (not below the latency model's) whose last
    pass fits in one round of P workgroups, so a non-power of two when the documents ask for it.
    65536 tokens in documents of 191, 231, 83, 209, 245 and 68 chunks, 8 heads, P = 256: the
    latency model gives 16 (68 units, 544 workgroups); 35 gives 6 + 7 + 3 + 6 + 7 + 2 = 31 units
    (248 workgroups) and 34 gives 33.  The forward's workspace holds 3 states per (unit, head),
    the backward's 4 per (unit, head) on top of its per-chunk arrays."""
    chunks = [191, 231, 83, 209, 245, 68]
    lens = [64 * c for c in chunks]
    lens[-1] -= 64 * sum(chunks) - 65536 if sum(lens) > 65536 else 0
    cu = [0]
    for n in lens:
        cu.append(cu[-1] + n)
    T = cu[-1]
    arr = (ctypes.c_int32 * len(cu))(*cu)
    p = _problem(total_tokens=T, num_seqs=6, num_heads=8, mode=0, num_slots=256)
    n = ctypes.c_size_t(0)
    assert lib.gdn_chunk_fwd_workspace_size(ctypes.byref(p), arr, ctypes.byref(n)) == 0
    state = 128 * 128 * 4
    units = sum((c + 34) // 35 for c in chunks)
    assert units == 31
    assert n.value == 3 * units * 8 * state
    nb1, nb2 = ctypes.c_size_t(0), ctypes.c_size_t(0)
    assert lib.gdn_chunk_bwd_workspace_size(ctypes.byref(p), arr, ctypes.byref(nb1)) == 0
    p1 = _problem(total_tokens=T, num_seqs=6, num_heads=8, mode=0, num_slots=6 * 8)
    assert lib.gdn_chunk_bwd_workspace_size(ctypes.byref(p1), arr, ctypes.byref(nb2)) == 0
    assert nb1.value - nb2.value == 4 * units * 8 * state  # num_seqs * H >= P: no split
