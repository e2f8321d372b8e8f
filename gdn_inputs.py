"""Seeded synthetic inputs for the gated delta rule (shared by the tests, the smoke check and the
benchmark; holds none of the method's arithmetic).

Recipe (the pages print no input values; these stand in for their workloads):

* numpy PCG64, one seed per workload; values drawn in fp64, then rounded to the compute dtype
  with round-to-nearest-even.  Callers give both sides (kernel and oracle) the *rounded*
  values, so a parity check measures the kernel and not input quantisation.
* q, k: per-element N(0, 1), each (token, head) row L2-normalised over d_k in fp64 before the
  cast.  v: N(0, 1).
* g = -softplus(x), x ~ N(-3, 1), kept in fp32 (mean about -0.075 per token, so a 64-token
  chunk decays by about e^-4.8).  beta = sigmoid(N(0, 1)) in the dtype of q.
* Documents are packed into one token-major buffer with int32 ``cu_seqlens`` offsets.

Workloads (the shapes of the pages' prefill and training cases):

* ``tiny``:    1 x 256 tokens, H=2, d=64, fp32.
* ``packed``:  8192 tokens from documents of U{256..2048} tokens, last trimmed; H=8, d=128, bf16.
* ``long``:    1 x 32768 tokens, H=8, d=128, bf16 (a 32K prefill on one GPU's 8-head share).
* ``fork``:    a 65536-token prefix, then 80 branches of U{1024..4096} tokens sharing the
               prefix's final state; H=16, d=128, bf16.
* ``train``:   65536 tokens from documents of U{4096..16384}, last trimmed; H=8, d=128, bf16,
               with dO ~ N(0, 1).
"""
from __future__ import annotations

import numpy as np

WORKLOAD_SEEDS = {"tiny": 1000, "packed": 1001, "long": 1002, "fork": 1003, "train": 1004}


def bf16_round(x) -> np.ndarray:
    """Round to the nearest bfloat16 (ties to even); returns float32 holding bf16 values.

    Works on the uint32 bit patterns in place: adding 0x7FFF plus the kept part's lowest bit
    cannot carry out of 32 bits for finite values or infinities (the generated inputs are
    finite)."""
    x32 = np.ascontiguousarray(np.asarray(x, dtype=np.float32))
    b = x32.view(np.uint32)
    r = (b >> 16) & np.uint32(1)
    r += np.uint32(0x7FFF)
    r += b
    r &= np.uint32(0xFFFF0000)
    return r.view(np.float32).reshape(x32.shape)


def bf16_bits(x) -> np.ndarray:
    """uint16 bit patterns of bf16-representable float32 values (e.g. from :func:`bf16_round`)."""
    x32 = np.ascontiguousarray(np.asarray(x, dtype=np.float32))
    return (x32.view(np.uint32) >> 16).astype(np.uint16)


def to_dtype(x, dtype: str) -> np.ndarray:
    """Round fp64 values to ``dtype`` ('f32' or 'bf16'); returns float32 arrays."""
    if dtype == "f32":
        return np.asarray(x, dtype=np.float32)
    if dtype == "bf16":
        return bf16_round(np.asarray(x, dtype=np.float32))
    raise ValueError(dtype)


def cu_from_lengths(lengths) -> np.ndarray:
    cu = np.zeros(len(lengths) + 1, np.int32)
    cu[1:] = np.cumsum(np.asarray(lengths, np.int64))
    return cu


def lengths_until(rng, lo, hi, total):
    """Draw lengths uniform in [lo, hi] until they reach ``total``; trim the last one."""
    lens = []
    acc = 0
    while acc < total:
        n = int(rng.integers(lo, hi + 1))
        n = min(n, total - acc)
        lens.append(n)
        acc += n
    return lens


def make_inputs(lengths, H, dk, dv, dtype, seed, h0_scale=0.0, n_h0=None, g_mu=-3.0,
                with_dout=False):
    """Inputs for documents of the given lengths.

    Returns a dict with float32 numpy arrays q, k [T,H,dk], v [T,H,dv], g, beta [T,H],
    ``cu_seqlens`` (int32), ``h0`` ([n_h0 or N, H, dk, dv] float32 or None), ``dout`` (if asked),
    and ``dtype``.  All values are exactly representable in ``dtype`` (g is always fp32).
    """
    rng = np.random.Generator(np.random.PCG64(seed))
    cu = cu_from_lengths(lengths)
    T = int(cu[-1])
    N = len(lengths)
    q = rng.standard_normal((T, H, dk))
    k = rng.standard_normal((T, H, dk))
    q /= np.linalg.norm(q, axis=-1, keepdims=True)
    k /= np.linalg.norm(k, axis=-1, keepdims=True)
    v = rng.standard_normal((T, H, dv))
    x = rng.standard_normal((T, H)) + g_mu
    g = -np.logaddexp(0.0, x)  # -softplus(x)
    beta = 1.0 / (1.0 + np.exp(-rng.standard_normal((T, H))))
    out = dict(q=to_dtype(q, dtype), k=to_dtype(k, dtype), v=to_dtype(v, dtype),
               g=g.astype(np.float32), beta=to_dtype(beta, dtype), cu_seqlens=cu,
               dtype=dtype, h0=None)
    if h0_scale:
        nh = N if n_h0 is None else n_h0
        out["h0"] = (h0_scale * rng.standard_normal((nh, H, dk, dv))).astype(np.float32)
    if with_dout:
        out["dout"] = to_dtype(rng.standard_normal((T, H, dv)), dtype)
    return out


def scale_qk_rows(inp, seed, lo=0.3, hi=3.0):
    """A copy of ``inp`` whose q and k rows are scaled by factors drawn from U[lo, hi] per
    (token, head) and rounded back to the input dtype: inputs for the in-kernel L2
    normalisation, whose rows are not of unit length."""
    rng = np.random.Generator(np.random.PCG64(seed))
    out = dict(inp)
    for name in ("q", "k"):
        x = inp[name] * rng.uniform(lo, hi, inp[name].shape[:2] + (1,))
        out[name] = bf16_round(x) if inp["dtype"] == "bf16" else x.astype(np.float32)
    return out


def workload_shape(name: str):
    """Document lengths and sizes of one named workload, without drawing any values: the same
    lengths :func:`workload` uses.  Returns dict(lengths, H, d, dtype) and, for ``fork``,
    prefix_len (the branches' lengths are ``lengths``)."""
    seed = WORKLOAD_SEEDS[name]
    rng = np.random.Generator(np.random.PCG64(seed + 7919))
    if name == "tiny":
        return dict(lengths=[256], H=2, d=64, dtype="f32")
    if name == "packed":
        return dict(lengths=lengths_until(rng, 256, 2048, 8192), H=8, d=128, dtype="bf16")
    if name == "long":
        return dict(lengths=[32768], H=8, d=128, dtype="bf16")
    if name == "fork":
        return dict(lengths=[int(rng.integers(1024, 4097)) for _ in range(80)], H=16, d=128,
                    dtype="bf16", prefix_len=65536)
    if name == "train":
        return dict(lengths=lengths_until(rng, 4096, 16384, 65536), H=8, d=128, dtype="bf16")
    raise KeyError(name)


def workload(name: str, **overrides):
    """Inputs of one named workload (see the module docstring)."""
    seed = WORKLOAD_SEEDS[name]
    sh = workload_shape(name)
    spec = dict(lengths=sh["lengths"], H=sh["H"], dk=sh["d"], dv=sh["d"], dtype=sh["dtype"])
    if name == "train":
        spec["with_dout"] = True
    spec.update(overrides)
    if name == "fork":
        # the prefix and the branches are drawn as two documents sets with related seeds
        prefix = make_inputs([sh["prefix_len"]], spec["H"], spec["dk"], spec["dv"],
                             spec["dtype"], seed)
        branches = make_inputs(spec["lengths"], spec["H"], spec["dk"], spec["dv"],
                               spec["dtype"], seed + 1)
        return dict(prefix=prefix, branches=branches)
    return make_inputs(spec.pop("lengths"), spec.pop("H"), spec.pop("dk"), spec.pop("dv"),
                       spec.pop("dtype"), seed, **spec)
