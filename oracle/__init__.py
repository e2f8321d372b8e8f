"""Gated DeltaNet oracle: plain fp64 CPU implementation (test infrastructure only).

Only the test suite, ``__graft_entry__.smoke()`` and the CPU-baseline leg of ``bench.py`` may
import this package.  The product path (the HIP library and its Python binding) never imports,
loads or calls it, and it shares no code with that path.

The arithmetic lives in ``gdn_oracle.c`` (plain C, fp64, OpenMP over independent
(sequence, head) pairs).  This module compiles it with gcc and wraps it with ctypes; every
function takes numpy arrays and returns fp64 numpy arrays.

Sources, cited by page title and section:

* "How to Speed Up GDN Kernels for Qwen Models": section "What GDN actually computes" (the
  gated delta rule, 64-token chunks, one triangular system per chunk per head); section
  "Lever 1" (truncated history, warmup windows, the segment-length latency model); section
  "Lever 2" (gate cumsum once per chunk, triangular inverse reused).
* "Musings on long-context fine-tuning": section "Isolating the recurrent layers" (decay first,
  then correct; the query reads the updated state; ``initial_state`` and ``cu_seqlens``);
  section "Backward through P" (gradients of a shared state add up); the q/k L2 normalisation
  whose backward kernel that page times (its OOM in the normalisation backward) is the optional
  first step ``qk_l2norm``: each (token, head) row of q and k divided by sqrt(|row|^2 + 1e-6).

Parity pins for every function are in ``tests/test_oracle_pins.py``.
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "gdn_oracle.c")
_LIB_PATH = os.path.join(_HERE, "libgdn_oracle.so")
_lib = None

_D = ctypes.POINTER(ctypes.c_double)
_I32 = ctypes.POINTER(ctypes.c_int32)


def build(force: bool = True) -> str:
    """Compile gdn_oracle.c into libgdn_oracle.so with gcc (-O2, OpenMP, no fast-math)."""
    if force or not os.path.exists(_LIB_PATH):
        tmp = _LIB_PATH + ".tmp"
        cmd = ["gcc", "-O2", "-fopenmp", "-fPIC", "-shared", "-std=c11", "-Wall",
               "-o", tmp, _SRC, "-lm"]
        subprocess.run(cmd, check=True)
        os.replace(tmp, _LIB_PATH)
    return _LIB_PATH


def _load():
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(_LIB_PATH) or os.path.getmtime(_LIB_PATH) < os.path.getmtime(_SRC):
        build()
    lib = ctypes.CDLL(_LIB_PATH)
    i64, i32, dbl = ctypes.c_int64, ctypes.c_int32, ctypes.c_double
    lib.gdn_oracle_fwd_recurrent.argtypes = [i64, i32, i32, i32, i32, _I32, _D, _D, _D, _D, _D,
                                             _D, i64, dbl, _D, _D, ctypes.c_int]
    lib.gdn_oracle_fwd_chunked.argtypes = [i64, i32, i32, i32, i32, _I32, i32, _D, _D, _D, _D,
                                           _D, _D, i64, dbl, _D, _D, _D, _D, _D, _D, _D, _D,
                                           ctypes.c_int]
    lib.gdn_oracle_num_chunks.argtypes = [i32, _I32, i32]
    lib.gdn_oracle_num_chunks.restype = i64
    lib.gdn_oracle_segment_chunks.argtypes = [i32, i64, i32, i32, i32]
    lib.gdn_oracle_segment_chunks.restype = i32
    lib.gdn_oracle_plan.argtypes = [i64, i32, i32, _I32, _D, i32, i32, i32, dbl, i32, _I32,
                                    _I32, _I32, _I32]
    lib.gdn_oracle_plan.restype = i32
    lib.gdn_oracle_fwd_truncated.argtypes = [i64, i32, i32, i32, i32, _I32, i32, _D, _D, _D,
                                             _D, _D, _D, i64, dbl, i32, _I32, _I32, _I32, _I32,
                                             _D, _D, ctypes.c_int]
    lib.gdn_oracle_bwd.argtypes = [i64, i32, i32, i32, i32, _I32, _D, _D, _D, _D, _D, _D, i64,
                                   dbl, _D, _D, _D, _D, _D, _D, _D, _D, ctypes.c_int]
    lib.gdn_oracle_l2norm.argtypes = [i64, i32, _D, dbl, _D]
    lib.gdn_oracle_l2norm_bwd.argtypes = [i64, i32, _D, _D, dbl, _D]
    lib.gdn_oracle_max_threads.restype = ctypes.c_int
    _lib = lib
    return lib


def _f64(x):
    if x is None:
        return None
    return np.ascontiguousarray(np.asarray(x, dtype=np.float64))


def _ptr(a, typ=_D):
    if a is None:
        return ctypes.cast(None, typ)
    return a.ctypes.data_as(typ)


def _cu(cu_seqlens):
    return np.ascontiguousarray(np.asarray(cu_seqlens, dtype=np.int32))


def _shape(q, v, cu):
    T, H, dk = q.shape
    dv = v.shape[2]
    return T, len(cu) - 1, H, dk, dv


def _h0(h0, N, H, dk, dv):
    """h0 may be None, [H, dk, dv] (one state broadcast to all sequences) or [N, H, dk, dv]."""
    if h0 is None:
        return None, 0
    h0 = _f64(h0)
    if h0.ndim == 3:
        return h0, 0
    assert h0.shape == (N, H, dk, dv)
    return h0, H * dk * dv


def max_threads() -> int:
    return int(_load().gdn_oracle_max_threads())


L2NORM_EPS = 1e-6


def l2norm(x, eps=L2NORM_EPS):
    """Each row over the last axis divided by sqrt(|row|^2 + eps)."""
    lib = _load()
    x = _f64(x)
    y = np.zeros_like(x)
    d = x.shape[-1]
    if lib.gdn_oracle_l2norm(x.size // d, d, _ptr(x), float(eps), _ptr(y)):
        raise ValueError("gdn_oracle_l2norm: bad arguments")
    return y


def l2norm_bwd(x, dy, eps=L2NORM_EPS):
    """Gradient with respect to x of <l2norm(x), dy>."""
    lib = _load()
    x, dy = _f64(x), _f64(dy)
    dx = np.zeros_like(x)
    d = x.shape[-1]
    if lib.gdn_oracle_l2norm_bwd(x.size // d, d, _ptr(x), _ptr(dy), float(eps), _ptr(dx)):
        raise ValueError("gdn_oracle_l2norm_bwd: bad arguments")
    return dx


def fwd_recurrent(q, k, v, g, beta, cu_seqlens, h0=None, scale=1.0, nthreads=0,
                  qk_l2norm=False):
    """Token-by-token forward (the plain definition).  Returns (o [T,H,dv], ht [N,H,dk,dv]).
    qk_l2norm: q and k are L2-normalised per (token, head) row first."""
    lib = _load()
    if qk_l2norm:
        q, k = l2norm(q), l2norm(k)
    q, k, v, g, beta = map(_f64, (q, k, v, g, beta))
    cu = _cu(cu_seqlens)
    T, N, H, dk, dv = _shape(q, v, cu)
    h0a, stride = _h0(h0, N, H, dk, dv)
    o = np.zeros((T, H, dv))
    ht = np.zeros((N, H, dk, dv))
    rc = lib.gdn_oracle_fwd_recurrent(T, N, H, dk, dv, _ptr(cu, _I32), _ptr(q), _ptr(k),
                                      _ptr(v), _ptr(g), _ptr(beta), _ptr(h0a), stride,
                                      float(scale), _ptr(o), _ptr(ht), nthreads)
    if rc:
        raise ValueError(f"gdn_oracle_fwd_recurrent: bad arguments ({rc})")
    return o, ht


def num_chunks(cu_seqlens, chunk=64) -> int:
    cu = _cu(cu_seqlens)
    return int(_load().gdn_oracle_num_chunks(len(cu) - 1, _ptr(cu, _I32), chunk))


def fwd_chunked(q, k, v, g, beta, cu_seqlens, h0=None, scale=1.0, chunk=64,
                intermediates=False, nthreads=0):
    """Chunked forward (separately written).  Returns (o, ht) or (o, ht, dict of intermediates:
    gamma [T,H], tm [nc,H,C,C], w [nc,H,C,dk], u [nc,H,C,dv], hc [nc,H,dk,dv],
    delta [T,H,dv])."""
    lib = _load()
    q, k, v, g, beta = map(_f64, (q, k, v, g, beta))
    cu = _cu(cu_seqlens)
    T, N, H, dk, dv = _shape(q, v, cu)
    h0a, stride = _h0(h0, N, H, dk, dv)
    o = np.zeros((T, H, dv))
    ht = np.zeros((N, H, dk, dv))
    inter = None
    if intermediates:
        nc = num_chunks(cu, chunk)
        C = chunk
        inter = dict(gamma=np.zeros((T, H)), tm=np.zeros((nc, H, C, C)),
                     w=np.zeros((nc, H, C, dk)), u=np.zeros((nc, H, C, dv)),
                     hc=np.zeros((nc, H, dk, dv)), delta=np.zeros((T, H, dv)))
    get = (lambda n: _ptr(inter[n])) if inter else (lambda n: _ptr(None))
    rc = lib.gdn_oracle_fwd_chunked(T, N, H, dk, dv, _ptr(cu, _I32), chunk, _ptr(q), _ptr(k),
                                    _ptr(v), _ptr(g), _ptr(beta), _ptr(h0a), stride,
                                    float(scale), _ptr(o), _ptr(ht), get("gamma"), get("tm"),
                                    get("w"), get("u"), get("hc"), get("delta"), nthreads)
    if rc:
        raise ValueError(f"gdn_oracle_fwd_chunked: bad arguments ({rc})")
    return (o, ht, inter) if intermediates else (o, ht)


def segment_chunks(H, total_chunks, num_seqs, P, forced=0) -> int:
    """Segment length L (chunks) of the latency model; 0 means no split."""
    return int(_load().gdn_oracle_segment_chunks(H, total_chunks, num_seqs, P, forced))


def plan(g, cu_seqlens, H, chunk=64, P=256, seg_chunks=0, log_threshold=-10.0):
    """Truncation plan.  Returns dict(seq, c0, c1 [S], warm [S, H]) with chunk numbers counted
    from each sequence's first chunk."""
    lib = _load()
    g = _f64(g)
    cu = _cu(cu_seqlens)
    T = g.shape[0]
    N = len(cu) - 1
    cap = num_chunks(cu, chunk) + N + 1
    seq = np.zeros(cap, np.int32)
    c0 = np.zeros(cap, np.int32)
    c1 = np.zeros(cap, np.int32)
    warm = np.zeros((cap, H), np.int32)
    ns = lib.gdn_oracle_plan(T, N, H, _ptr(cu, _I32), _ptr(g), chunk, P, seg_chunks,
                             float(log_threshold), cap, _ptr(seq, _I32), _ptr(c0, _I32),
                             _ptr(c1, _I32), _ptr(warm, _I32))
    if ns < 0:
        raise ValueError(f"gdn_oracle_plan failed ({ns})")
    return dict(seq=seq[:ns].copy(), c0=c0[:ns].copy(), c1=c1[:ns].copy(),
                warm=warm[:ns].copy())


def fwd_truncated(q, k, v, g, beta, cu_seqlens, plan_dict, h0=None, scale=1.0, chunk=64,
                  nthreads=0, qk_l2norm=False):
    """Truncated-history forward following ``plan_dict`` (from :func:`plan`)."""
    lib = _load()
    if qk_l2norm:
        q, k = l2norm(q), l2norm(k)
    q, k, v, g, beta = map(_f64, (q, k, v, g, beta))
    cu = _cu(cu_seqlens)
    T, N, H, dk, dv = _shape(q, v, cu)
    h0a, stride = _h0(h0, N, H, dk, dv)
    seq = np.ascontiguousarray(plan_dict["seq"], np.int32)
    c0 = np.ascontiguousarray(plan_dict["c0"], np.int32)
    c1 = np.ascontiguousarray(plan_dict["c1"], np.int32)
    warm = np.ascontiguousarray(plan_dict["warm"], np.int32)
    o = np.zeros((T, H, dv))
    ht = np.zeros((N, H, dk, dv))
    rc = lib.gdn_oracle_fwd_truncated(T, N, H, dk, dv, _ptr(cu, _I32), chunk, _ptr(q), _ptr(k),
                                      _ptr(v), _ptr(g), _ptr(beta), _ptr(h0a), stride,
                                      float(scale), len(seq), _ptr(seq, _I32), _ptr(c0, _I32),
                                      _ptr(c1, _I32), _ptr(warm, _I32), _ptr(o), _ptr(ht),
                                      nthreads)
    if rc:
        raise ValueError(f"gdn_oracle_fwd_truncated: bad arguments ({rc})")
    return o, ht


def bwd(q, k, v, g, beta, cu_seqlens, dout, h0=None, dht=None, scale=1.0, nthreads=0,
        qk_l2norm=False):
    """Backward of the token recurrence.  Returns dict(dq, dk, dv, dg, dbeta, dh0) with dh0 per
    sequence [N, H, dk, dv] (sum it over sequences that share one initial state).  qk_l2norm:
    the gradients of the normalised q, k pass back through the normalisation."""
    if qk_l2norm:
        out = bwd(l2norm(q), l2norm(k), v, g, beta, cu_seqlens, dout, h0=h0, dht=dht, scale=scale,
                  nthreads=nthreads)
        out["dq"] = l2norm_bwd(q, out["dq"])
        out["dk"] = l2norm_bwd(k, out["dk"])
        return out
    lib = _load()
    q, k, v, g, beta, dout = map(_f64, (q, k, v, g, beta, dout))
    cu = _cu(cu_seqlens)
    T, N, H, dk, dv = _shape(q, v, cu)
    h0a, stride = _h0(h0, N, H, dk, dv)
    dhta = None if dht is None else _f64(dht)
    out = dict(dq=np.zeros((T, H, dk)), dk=np.zeros((T, H, dk)), dv=np.zeros((T, H, dv)),
               dg=np.zeros((T, H)), dbeta=np.zeros((T, H)), dh0=np.zeros((N, H, dk, dv)))
    rc = lib.gdn_oracle_bwd(T, N, H, dk, dv, _ptr(cu, _I32), _ptr(q), _ptr(k), _ptr(v),
                            _ptr(g), _ptr(beta), _ptr(h0a), stride, float(scale), _ptr(dout),
                            _ptr(dhta), _ptr(out["dq"]), _ptr(out["dk"]), _ptr(out["dv"]),
                            _ptr(out["dg"]), _ptr(out["dbeta"]), _ptr(out["dh0"]), nthreads)
    if rc:
        raise ValueError(f"gdn_oracle_bwd: bad arguments ({rc})")
    return out
