"""Python binding of the gfx950 gated delta rule library (argument marshalling only).

Every step of the computation runs in the HIP kernels of ``libgdn_mi355x.so``; this module
checks tensor shapes, takes device pointers from torch tensors, allocates outputs and workspace
with torch (memory plumbing) and calls the C ABI declared in ``include/gdn.h`` on torch's
current stream.  There is no fallback: if the library is missing or the device is not gfx950,
the call raises.
"""
from __future__ import annotations

import ctypes
import os

import torch

_PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_PKG, "libgdn_mi355x.so")

GDN_DTYPE_F32, GDN_DTYPE_BF16 = 0, 1
GDN_MODE_EXACT, GDN_MODE_TRUNCATE = 0, 1
_MODES = {"exact": GDN_MODE_EXACT, "truncate": GDN_MODE_TRUNCATE}

# Every exported entry point of include/gdn.h.
EXPORTS = ("gdn_problem_init", "gdn_chunk_fwd_workspace_size", "gdn_chunk_fwd",
           "gdn_chunk_fwd_noalloc", "gdn_chunk_fwd_plan", "gdn_chunk_fwd_intermediates",
           "gdn_chunk_bwd_workspace_size",
           "gdn_chunk_bwd", "gdn_decode_step", "gdn_validate_cu_seqlens", "gdn_set_debug",
           "gdn_get_debug", "gdn_device_faults", "gdn_status_string", "gdn_last_error",
           "gdn_calib_copy", "gdn_calib_mfma_bf16")

# Status bits of gdn_validate_cu_seqlens.
CU_FIRST_NOT_ZERO, CU_DESCENDING, CU_LAST_NOT_TOTAL, CU_OUT_OF_RANGE = 1, 2, 4, 8


class GdnError(RuntimeError):
    def __init__(self, status: int, msg: str):
        super().__init__(msg)
        self.status = status


class GdnProblem(ctypes.Structure):
    _fields_ = [("total_tokens", ctypes.c_int64), ("num_seqs", ctypes.c_int32),
                ("num_heads", ctypes.c_int32), ("d_k", ctypes.c_int32),
                ("d_v", ctypes.c_int32), ("chunk", ctypes.c_int32), ("dtype", ctypes.c_int32),
                ("mode", ctypes.c_int32), ("seg_chunks", ctypes.c_int32),
                ("num_slots", ctypes.c_int32), ("trunc_log_threshold", ctypes.c_float),
                ("scale", ctypes.c_float), ("num_k_heads", ctypes.c_int32),
                ("qk_l2norm", ctypes.c_int32), ("reserved", ctypes.c_int32),
                ("h0_seq_stride", ctypes.c_int64)]


_lib = None


def load_library() -> ctypes.CDLL:
    """Load libgdn_mi355x.so (raises if it has not been built)."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(LIB_PATH):
        raise RuntimeError(f"{LIB_PATH} is missing: build it with "
                           "`python -m linear_attention_recurrence_prefill_amd.build`")
    lib = ctypes.CDLL(LIB_PATH)
    vp, sz, i32p = ctypes.c_void_p, ctypes.c_size_t, ctypes.POINTER(ctypes.c_int32)
    P = ctypes.POINTER(GdnProblem)
    st = ctypes.c_int
    lib.gdn_problem_init.argtypes = [P, ctypes.c_int64, ctypes.c_int32, ctypes.c_int32,
                                     ctypes.c_int32]
    lib.gdn_problem_init.restype = st
    lib.gdn_chunk_fwd_workspace_size.argtypes = [P, i32p, ctypes.POINTER(sz)]
    lib.gdn_chunk_fwd_workspace_size.restype = st
    lib.gdn_chunk_fwd.argtypes = [P, vp, vp, vp, vp, vp, vp, i32p, vp, vp, vp, vp, sz, vp]
    lib.gdn_chunk_fwd.restype = st
    lib.gdn_chunk_fwd_noalloc.argtypes = [P, vp, vp, vp, vp, vp, vp, i32p, vp, vp, vp, vp]
    lib.gdn_chunk_fwd_noalloc.restype = st
    lib.gdn_chunk_fwd_plan.argtypes = [P, vp, vp, i32p, vp, ctypes.c_int64, vp, sz, vp]
    lib.gdn_chunk_fwd_plan.restype = st
    lib.gdn_chunk_fwd_intermediates.argtypes = [P, vp, vp, vp, vp, vp, vp, vp, vp, vp, vp, vp,
                                                vp, vp, vp, vp, vp, sz, vp]
    lib.gdn_chunk_fwd_intermediates.restype = st
    lib.gdn_chunk_bwd_workspace_size.argtypes = [P, i32p, ctypes.POINTER(sz)]
    lib.gdn_chunk_bwd_workspace_size.restype = st
    lib.gdn_chunk_bwd.argtypes = [P, vp, vp, vp, vp, vp, vp, i32p, vp, vp, vp, vp, vp, vp, vp,
                                  vp, vp, vp, sz, vp]
    lib.gdn_chunk_bwd.restype = st
    lib.gdn_decode_step.argtypes = [ctypes.c_int32, ctypes.c_int32, ctypes.c_int32, ctypes.c_int32,
                                    ctypes.c_int32,
                                    ctypes.c_int32, ctypes.c_float, vp, vp, vp, vp, vp, vp, vp,
                                    vp]
    lib.gdn_decode_step.restype = st
    lib.gdn_calib_copy.argtypes = [vp, vp, sz, vp]
    lib.gdn_calib_copy.restype = st
    lib.gdn_calib_mfma_bf16.argtypes = [vp, ctypes.c_int, ctypes.c_int, vp]
    lib.gdn_calib_mfma_bf16.restype = st
    lib.gdn_validate_cu_seqlens.argtypes = [vp, ctypes.c_int32, ctypes.c_int64, vp, vp]
    lib.gdn_validate_cu_seqlens.restype = st
    lib.gdn_set_debug.argtypes = [ctypes.c_int32]
    lib.gdn_set_debug.restype = st
    lib.gdn_get_debug.argtypes = []
    lib.gdn_get_debug.restype = ctypes.c_int32
    lib.gdn_device_faults.argtypes = [ctypes.POINTER(ctypes.c_uint32), ctypes.c_int32]
    lib.gdn_device_faults.restype = st
    lib.gdn_status_string.argtypes = [st]
    lib.gdn_status_string.restype = ctypes.c_char_p
    lib.gdn_last_error.argtypes = []
    lib.gdn_last_error.restype = ctypes.c_char_p
    _lib = lib
    return lib


def _check(status: int):
    if status != 0:
        lib = load_library()
        raise GdnError(status, f"{lib.gdn_status_string(status).decode()}: "
                               f"{lib.gdn_last_error().decode()}")


def _ptr(t):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _stream():
    return ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)


def make_problem(total_tokens, num_seqs, num_heads, head_dim, dtype, mode="exact", scale=1.0,
                 seg_chunks=0, num_slots=0, trunc_log_threshold=-10.0, h0_seq_stride=None,
                 num_k_heads=0, qk_l2norm=False):
    lib = load_library()
    p = GdnProblem()
    _check(lib.gdn_problem_init(ctypes.byref(p), int(total_tokens), int(num_seqs),
                                int(num_heads), int(head_dim)))
    p.dtype = GDN_DTYPE_BF16 if dtype == torch.bfloat16 else GDN_DTYPE_F32
    p.mode = _MODES[mode]
    p.scale = float(scale)
    p.seg_chunks = int(seg_chunks)
    p.num_slots = int(num_slots)
    p.trunc_log_threshold = float(trunc_log_threshold)
    if h0_seq_stride is not None:
        p.h0_seq_stride = int(h0_seq_stride)
    p.num_k_heads = int(num_k_heads)
    p.qk_l2norm = 1 if qk_l2norm else 0
    return p


def _validate(q, k, v, g, beta, cu_seqlens, h0):
    """Sizes of a call: q, k [T, Hk, D], v [T, H, D] with Hk dividing H (grouped heads: value
    head h reads key head h // (H // Hk)), g, beta [T, H]."""
    if q.dim() != 3 or v.dim() != 3:
        raise ValueError("q, k, v must be [T, heads, D]")
    T, Hk, D = q.shape
    H = v.shape[1]
    if k.shape != (T, Hk, D) or v.shape != (T, H, D) or Hk < 1 or H % Hk != 0:
        raise ValueError("q and k must be [T, Hk, D] and v [T, H, D] with Hk dividing H")
    if g.shape != (T, H) or beta.shape != (T, H):
        raise ValueError("g and beta must be [T, H]")
    if q.dtype not in (torch.bfloat16, torch.float32):
        raise ValueError("q must be bfloat16 or float32")
    if k.dtype != q.dtype or v.dtype != q.dtype or beta.dtype != q.dtype:
        raise ValueError("k, v and beta must have q's dtype")
    if g.dtype != torch.float32:
        raise ValueError("g must be float32")
    if cu_seqlens.dtype != torch.int32 or cu_seqlens.dim() != 1:
        raise ValueError("cu_seqlens must be a 1-D int32 tensor")
    for t in (q, k, v, g, beta, cu_seqlens):
        if not t.is_cuda or not t.is_contiguous():
            raise ValueError("inputs must be contiguous device tensors")
    N = cu_seqlens.numel() - 1
    stride = None
    if h0 is not None:
        if h0.dtype != torch.float32 or not h0.is_cuda or not h0.is_contiguous():
            raise ValueError("h0 must be a contiguous float32 device tensor")
        if h0.shape == (H, D, D):
            stride = 0
        elif h0.shape == (N, H, D, D):
            stride = H * D * D
        else:
            raise ValueError("h0 must be [N, H, D, D] or [H, D, D] (shared by all sequences)")
    return T, H, D, N, stride, Hk


def _host_cu(cu_seqlens, cu_seqlens_host):
    if cu_seqlens_host is None:
        return None
    arr = (ctypes.c_int32 * len(cu_seqlens_host))(*[int(x) for x in cu_seqlens_host])
    return arr


def chunk_fwd(q, k, v, g, beta, cu_seqlens, h0=None, *, mode="exact", scale=1.0,
              seg_chunks=0, num_slots=0, trunc_log_threshold=-10.0, output_final_state=True,
              cu_seqlens_host=None, out=None, final_state=None, workspace=None,
              qk_l2norm=False):
    """Forward of the chunked gated delta rule.  Returns (o, ht or None).  qk_l2norm: q and k
    are L2-normalised per (token, head) row inside the kernels."""
    lib = load_library()
    T, H, D, N, stride, Hk = _validate(q, k, v, g, beta, cu_seqlens, h0)
    p = make_problem(T, N, H, D, q.dtype, mode, scale, seg_chunks, num_slots,
                     trunc_log_threshold, stride, num_k_heads=Hk, qk_l2norm=qk_l2norm)
    cu_h = _host_cu(cu_seqlens, cu_seqlens_host)
    ws_bytes = ctypes.c_size_t(0)
    _check(lib.gdn_chunk_fwd_workspace_size(ctypes.byref(p), cu_h, ctypes.byref(ws_bytes)))
    workspace = _workspace(workspace, ws_bytes.value, q.device)
    if out is not None:
        _check_out("out", out, tuple(v.shape), v.dtype, q.device)
    o = out if out is not None else torch.empty_like(v)
    ht = None
    if output_final_state:
        if final_state is not None:
            _check_out("final_state", final_state, (N, H, D, D), torch.float32, q.device)
        ht = final_state if final_state is not None else torch.empty(
            (N, H, D, D), dtype=torch.float32, device=q.device)
    _check(lib.gdn_chunk_fwd(ctypes.byref(p), _ptr(q), _ptr(k), _ptr(v), _ptr(g), _ptr(beta),
                             _ptr(cu_seqlens), cu_h, _ptr(h0), _ptr(o), _ptr(ht),
                             _ptr(workspace), _nbytes(workspace), _stream()))
    return o, ht


NOALLOC_SCRATCH_BYTES = 128 << 20  # GDN_NOALLOC_SCRATCH_BYTES of include/gdn.h


def chunk_fwd_noalloc(q, k, v, g, beta, cu_seqlens, h0=None, *, out, final_state=None,
                      mode="exact", scale=1.0, seg_chunks=0, num_slots=0,
                      trunc_log_threshold=-10.0, cu_seqlens_host=None, qk_l2norm=False):
    """The forward through gdn_chunk_fwd_noalloc: the library allocates nothing (its workspace
    is a static device array), and the caller passes the outputs (``out`` like v; optional
    ``final_state`` [N, H, D, D] fp32).  Returns (out, final_state)."""
    lib = load_library()
    T, H, D, N, stride, Hk = _validate(q, k, v, g, beta, cu_seqlens, h0)
    p = make_problem(T, N, H, D, q.dtype, mode, scale, seg_chunks, num_slots,
                     trunc_log_threshold, stride, num_k_heads=Hk, qk_l2norm=qk_l2norm)
    _check_out("out", out, tuple(v.shape), v.dtype, q.device)
    if final_state is not None:
        _check_out("final_state", final_state, (N, H, D, D), torch.float32, q.device)
    _check(lib.gdn_chunk_fwd_noalloc(ctypes.byref(p), _ptr(q), _ptr(k), _ptr(v), _ptr(g),
                                     _ptr(beta), _ptr(cu_seqlens),
                                     _host_cu(cu_seqlens, cu_seqlens_host), _ptr(h0), _ptr(out),
                                     _ptr(final_state), _stream()))
    return out, final_state


def _check_out(name, t, shape, dtype, device):
    """A caller-supplied output: the shape, dtype and device the call writes, contiguous."""
    if tuple(t.shape) != tuple(shape) or t.dtype != dtype or t.device != device or \
            not t.is_contiguous():
        raise ValueError(f"{name} must be a contiguous {dtype} tensor of shape {list(shape)} on "
                         f"{device}")


def _nbytes(t):
    return t.numel() * t.element_size()


def _workspace(workspace, nbytes, device):
    """The caller's workspace if it is a contiguous device tensor of at least ``nbytes`` bytes
    (any dtype), else a new uint8 one."""
    if workspace is not None:
        if workspace.device != device or not workspace.is_contiguous():
            raise ValueError("workspace must be a contiguous tensor on the inputs' device")
        if _nbytes(workspace) >= nbytes:
            return workspace
    return torch.empty(max(nbytes, 1), dtype=torch.uint8, device=device)


def fwd_workspace_bytes(q, cu_seqlens, H=None, *, mode="exact", seg_chunks=0, num_slots=0,
                        cu_seqlens_host=None):
    """Workspace bytes of chunk_fwd for q [T, Hk, D] and H value heads (H = Hk if not given)."""
    lib = load_library()
    T, Hq, D = q.shape
    heads = Hq if H is None else H
    p = make_problem(T, cu_seqlens.numel() - 1, heads, D, q.dtype, mode, 1.0, seg_chunks,
                     num_slots, num_k_heads=Hq)
    n = ctypes.c_size_t(0)
    _check(lib.gdn_chunk_fwd_workspace_size(ctypes.byref(p), _host_cu(cu_seqlens,
                                                                      cu_seqlens_host),
                                            ctypes.byref(n)))
    return n.value


def chunk_fwd_plan(g, cu_seqlens, num_heads, head_dim, dtype, *, mode="truncate", seg_chunks=0,
                   num_slots=0, trunc_log_threshold=-10.0, cu_seqlens_host=None):
    """The segment plan the forward uses.  Returns dict(L, seq, c0, c1, warm [U, H])."""
    lib = load_library()
    T = g.shape[0]
    N = cu_seqlens.numel() - 1
    p = make_problem(T, N, num_heads, head_dim, dtype, mode, 1.0, seg_chunks, num_slots,
                     trunc_log_threshold)
    cu_h = _host_cu(cu_seqlens, cu_seqlens_host)
    ws_bytes = ctypes.c_size_t(0)
    _check(lib.gdn_chunk_fwd_workspace_size(ctypes.byref(p), cu_h, ctypes.byref(ws_bytes)))
    ws = torch.empty(max(ws_bytes.value, 1), dtype=torch.uint8, device=g.device)
    cap = 2 + (T // 64 + N + 1) * (3 + num_heads)
    out = torch.full((cap,), -1, dtype=torch.int32, device=g.device)
    _check(lib.gdn_chunk_fwd_plan(ctypes.byref(p), _ptr(g), _ptr(cu_seqlens), cu_h, _ptr(out),
                                  cap, _ptr(ws), ws.numel(), _stream()))
    host = out.cpu()
    U, L = int(host[0]), int(host[1])
    body = host[2:2 + U * (3 + num_heads)].reshape(U, 3 + num_heads)
    return dict(L=L, seq=body[:, 0].numpy(), c0=body[:, 1].numpy(), c1=body[:, 2].numpy(),
                warm=body[:, 3:].numpy())


def chunk_fwd_intermediates(q, k, v, g, beta, cu_seqlens, h0=None, *, scale=1.0,
                            num_chunks=None, qk_l2norm=False):
    """Exact forward that also returns the per-chunk intermediates (fp32):
    o, ht, dict(gamma [T,H], tmat [Nc,H,64,64], w [Nc,H,64,D], u [Nc,H,64,D],
    hc [Nc,H,D,D], delta [T,H,D])."""
    lib = load_library()
    T, H, D, N, stride, Hk = _validate(q, k, v, g, beta, cu_seqlens, h0)
    if num_chunks is None:
        cu = cu_seqlens.cpu().tolist()
        num_chunks = sum((cu[i + 1] - cu[i] + 63) // 64 for i in range(N))
    p = make_problem(T, N, H, D, q.dtype, "exact", scale, h0_seq_stride=stride, num_k_heads=Hk,
                     qk_l2norm=qk_l2norm)
    ws_bytes = ctypes.c_size_t(0)
    _check(lib.gdn_chunk_fwd_workspace_size(ctypes.byref(p), None, ctypes.byref(ws_bytes)))
    ws = torch.empty(max(ws_bytes.value, 1), dtype=torch.uint8, device=q.device)
    dev = q.device
    f32 = torch.float32
    inter = dict(gamma=torch.zeros((T, H), dtype=f32, device=dev),
                 tmat=torch.zeros((num_chunks, H, 64, 64), dtype=f32, device=dev),
                 w=torch.zeros((num_chunks, H, 64, D), dtype=f32, device=dev),
                 u=torch.zeros((num_chunks, H, 64, D), dtype=f32, device=dev),
                 hc=torch.zeros((num_chunks, H, D, D), dtype=f32, device=dev),
                 delta=torch.zeros((T, H, D), dtype=f32, device=dev))
    o = torch.empty_like(v)
    ht = torch.empty((N, H, D, D), dtype=f32, device=dev)
    _check(lib.gdn_chunk_fwd_intermediates(
        ctypes.byref(p), _ptr(q), _ptr(k), _ptr(v), _ptr(g), _ptr(beta), _ptr(cu_seqlens),
        _ptr(h0), _ptr(o), _ptr(ht), _ptr(inter["gamma"]), _ptr(inter["tmat"]),
        _ptr(inter["w"]), _ptr(inter["u"]), _ptr(inter["hc"]), _ptr(inter["delta"]), _ptr(ws),
        ws.numel(), _stream()))
    return o, ht, inter


def chunk_bwd(q, k, v, g, beta, cu_seqlens, dout, h0=None, dht=None, *, scale=1.0,
              need_dh0=True, workspace=None, seg_chunks=0, num_slots=0, qk_l2norm=False,
              cu_seqlens_host=None, mode="exact", trunc_log_threshold=-10.0):
    """Backward of the exact forward.  Returns dict(dq, dk, dv, dg, dbeta, dh0).  dh0 is
    [N, H, D, D], or [H, D, D] summed over sequences when h0 is shared ([H, D, D]).
    seg_chunks / num_slots set the segment length of the split (the forward recompute and the
    reverse chain) and the workgroup slots it is planned for (0: chosen by the library).
    mode "truncate": where the backward splits (bf16, d = 128), each unit starts from a warmup
    window (summed g below trunc_log_threshold) instead of the exact split's extra passes.
    qk_l2norm: backward of the forward with q and k normalised inside the kernels (dq, dk are
    the raw inputs' gradients).  cu_seqlens_host: an optional host copy of cu_seqlens (sets the
    split exactly)."""
    lib = load_library()
    T, H, D, N, stride, Hk = _validate(q, k, v, g, beta, cu_seqlens, h0)
    if dout.shape != v.shape or dout.dtype != q.dtype or not dout.is_contiguous():
        raise ValueError("dout must be contiguous with v's shape and q's dtype")
    if dht is not None and (dht.shape != (N, H, D, D) or dht.dtype != torch.float32):
        raise ValueError("dht must be float32 [N, H, D, D]")
    p = make_problem(T, N, H, D, q.dtype, mode, scale, seg_chunks=seg_chunks,
                     num_slots=num_slots, trunc_log_threshold=trunc_log_threshold,
                     h0_seq_stride=stride if stride is not None else H * D * D, num_k_heads=Hk,
                     qk_l2norm=qk_l2norm)
    cu_h = _host_cu(cu_seqlens, cu_seqlens_host)
    ws_bytes = ctypes.c_size_t(0)
    _check(lib.gdn_chunk_bwd_workspace_size(ctypes.byref(p), cu_h, ctypes.byref(ws_bytes)))
    workspace = _workspace(workspace, ws_bytes.value, q.device)
    out = dict(dq=torch.empty_like(q), dk=torch.empty_like(k), dv=torch.empty_like(v),
               dg=torch.empty_like(g), dbeta=torch.empty_like(beta), dh0=None)
    if need_dh0:
        shape = (H, D, D) if stride == 0 else (N, H, D, D)
        out["dh0"] = torch.empty(shape, dtype=torch.float32, device=q.device)
    _check(lib.gdn_chunk_bwd(ctypes.byref(p), _ptr(q), _ptr(k), _ptr(v), _ptr(g), _ptr(beta),
                             _ptr(cu_seqlens), cu_h, _ptr(h0), _ptr(dout), _ptr(dht),
                             _ptr(out["dq"]), _ptr(out["dk"]), _ptr(out["dv"]), _ptr(out["dg"]),
                             _ptr(out["dbeta"]), _ptr(out["dh0"]), _ptr(workspace),
                             _nbytes(workspace), _stream()))
    return out


def decode_step(q, k, v, g, beta, state, *, scale=1.0, out=None, qk_l2norm=False):
    """One decode step (gdn_decode_step): q, k [B, Hk, D] and v [B, H, D] (bf16 or fp32; Hk
    dividing H, value head h reading key head h // (H // Hk)), g [B, H] fp32, beta [B, H] (q's
    dtype), state [B, H, D, D] fp32, advanced in place by one token.  qk_l2norm: q and k rows
    are L2-normalised in the kernel.  Returns o [B, H, D] (q's dtype)."""
    lib = load_library()
    if q.dim() != 3 or v.dim() != 3:
        raise ValueError("q, k and v must be [B, heads, D]")
    B, Hk, D = q.shape
    H = v.shape[1]
    if Hk < 1 or H % Hk != 0:
        raise ValueError("q's heads must divide v's heads")
    for name, t, shape in (("q", q, (B, Hk, D)), ("k", k, (B, Hk, D)), ("v", v, (B, H, D)),
                           ("g", g, (B, H)), ("beta", beta, (B, H)),
                           ("state", state, (B, H, D, D))):
        if tuple(t.shape) != shape or not t.is_contiguous():
            raise ValueError(f"{name} must be contiguous {list(shape)}")
    if q.dtype not in (torch.bfloat16, torch.float32) or k.dtype != q.dtype or \
            v.dtype != q.dtype or beta.dtype != q.dtype:
        raise ValueError("q, k, v, beta must share a dtype (bfloat16 or float32)")
    if g.dtype != torch.float32 or state.dtype != torch.float32:
        raise ValueError("g and state must be float32")
    if out is None:
        out = torch.empty_like(v)
    dt = GDN_DTYPE_BF16 if q.dtype == torch.bfloat16 else GDN_DTYPE_F32
    _check(lib.gdn_decode_step(B, H, Hk, D, dt, 1 if qk_l2norm else 0, float(scale), _ptr(q),
                               _ptr(k), _ptr(v), _ptr(g), _ptr(beta), _ptr(state), _ptr(out),
                               _stream()))
    return out


def validate_cu_seqlens(cu_seqlens, total_tokens):
    """Checks a device cu_seqlens table on the device (gdn_validate_cu_seqlens) and returns its
    status bits (0: valid; CU_* bits otherwise).  Synchronises torch's current stream."""
    lib = load_library()
    if cu_seqlens.dtype != torch.int32 or cu_seqlens.dim() != 1 or not cu_seqlens.is_cuda or \
            not cu_seqlens.is_contiguous():
        raise ValueError("cu_seqlens must be a contiguous 1-D int32 device tensor")
    status = torch.full((1,), -1, dtype=torch.int32, device=cu_seqlens.device)
    _check(lib.gdn_validate_cu_seqlens(_ptr(cu_seqlens), cu_seqlens.numel() - 1,
                                       int(total_tokens), _ptr(status), _stream()))
    return int(status.item())


def set_debug(on):
    """Debug mode (gdn_set_debug): compute calls validate cu_seqlens on the device first and
    check the kernels' fault flags after their launches (synchronising the stream)."""
    _check(load_library().gdn_set_debug(1 if on else 0))


def get_debug():
    return bool(load_library().gdn_get_debug())


def device_faults(clear=False):
    """The current device's fault flags (gdn_device_faults; synchronises the device)."""
    flags = ctypes.c_uint32(0)
    _check(load_library().gdn_device_faults(ctypes.byref(flags), 1 if clear else 0))
    return int(flags.value)


def calib_copy(src, dst):
    """Stream copy of ``src`` into ``dst`` (same byte size, a multiple of 16) by the library's
    calibration kernel (gdn_calib_copy): the HBM bandwidth a plain kernel reaches."""
    lib = load_library()
    nbytes = src.numel() * src.element_size()
    if dst.numel() * dst.element_size() != nbytes or not src.is_contiguous() or \
            not dst.is_contiguous():
        raise ValueError("src and dst must be contiguous and of the same byte size")
    _check(lib.gdn_calib_copy(_ptr(src), _ptr(dst), nbytes, _stream()))


def calib_mfma_bf16(out, waves_per_cu, iters):
    """The calibration loop of bf16 MFMAs (gdn_calib_mfma_bf16); ``out`` float32 with at least
    waves_per_cu * 256 * 64 elements.  Returns the flop count of the call."""
    lib = load_library()
    if out.dtype != torch.float32 or out.numel() < waves_per_cu * 256 * 64:
        raise ValueError("out must be float32 with waves_per_cu * 256 * 64 elements")
    _check(lib.gdn_calib_mfma_bf16(_ptr(out), int(waves_per_cu), int(iters), _stream()))
    return waves_per_cu * 256 * iters * 4 * 32768


# The C entry points' names (include/gdn.h, include/gdn_calib.h), one binding each.
gdn_chunk_fwd = chunk_fwd
gdn_chunk_fwd_noalloc = chunk_fwd_noalloc
gdn_chunk_fwd_plan = chunk_fwd_plan
gdn_chunk_fwd_intermediates = chunk_fwd_intermediates
gdn_chunk_bwd = chunk_bwd
gdn_decode_step = decode_step
gdn_validate_cu_seqlens = validate_cu_seqlens
gdn_set_debug = set_debug
gdn_get_debug = get_debug
gdn_device_faults = device_faults
gdn_calib_copy = calib_copy
gdn_calib_mfma_bf16 = calib_mfma_bf16
