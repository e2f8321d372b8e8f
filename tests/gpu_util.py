"""Helpers shared by the GPU tests: moving seeded inputs to the device and comparing results."""
import numpy as np
import torch

BF16_TOL = 5e-3  # relative L2 for bf16 inputs with an fp32 state
F32_TOL = 1e-4   # relative L2 for fp32 inputs
BLOCK_TOKENS = 4096  # longer documents are also checked per block of at most this many tokens
MIN_DOC_TOKENS = 64  # per-(document, head) checks cover documents of at least one full chunk


def tol_for(dtype: str) -> float:
    return BF16_TOL if dtype == "bf16" else F32_TOL


def to_dev(inp, device="cuda"):
    """Device tensors of a gdn_inputs dict (bf16 or fp32 as the dict's dtype says)."""
    tdt = torch.bfloat16 if inp["dtype"] == "bf16" else torch.float32
    out = {}
    for name in ("q", "k", "v", "beta"):
        out[name] = torch.from_numpy(np.ascontiguousarray(inp[name])).to(device).to(tdt)
    out["g"] = torch.from_numpy(np.ascontiguousarray(inp["g"])).to(device)
    out["cu_seqlens"] = torch.from_numpy(np.ascontiguousarray(inp["cu_seqlens"])).to(device)
    out["h0"] = None
    if inp.get("h0") is not None:
        out["h0"] = torch.from_numpy(np.ascontiguousarray(inp["h0"])).to(device)
    if inp.get("dout") is not None:
        out["dout"] = torch.from_numpy(np.ascontiguousarray(inp["dout"])).to(device).to(tdt)
    return out


def args_of(d):
    return [d[x] for x in ("q", "k", "v", "g", "beta")]


def np64(t):
    return t.detach().float().cpu().numpy().astype(np.float64)


def rel_l2(x, ref):
    x = np.asarray(x, np.float64).ravel()
    ref = np.asarray(ref, np.float64).ravel()
    den = np.linalg.norm(ref)
    return float(np.linalg.norm(x - ref) / (den if den > 0 else 1.0))


def _per_head(x, ref):
    """Relative L2 per head of [n, H, ...] slices (head axis 1); absolute where ref is zero."""
    n, H = ref.shape[0], ref.shape[1]
    d = (x - ref).reshape(n, H, -1)
    num = np.sqrt(np.einsum("nhk,nhk->h", d, d))
    r = ref.reshape(n, H, -1)
    den = np.sqrt(np.einsum("nhk,nhk->h", r, r))
    return num / np.where(den > 0, den, 1.0)


def blocks_of(cu, block=BLOCK_TOKENS, min_tokens=MIN_DOC_TOKENS):
    """Token ranges checked separately: every document of at least ``min_tokens`` tokens, and
    each block of at most ``block`` tokens of a longer one (a tail shorter than ``min_tokens``
    joins the block before it).  Yields (document, first token, end token)."""
    cu = np.asarray(cu, np.int64)
    for n in range(len(cu) - 1):
        t0, t1 = int(cu[n]), int(cu[n + 1])
        if t1 - t0 < min_tokens:
            continue
        yield n, t0, t1
        if t1 - t0 > block:
            starts = list(range(t0, t1, block))
            if len(starts) > 1 and t1 - starts[-1] < min_tokens:
                starts.pop()
            for i, s in enumerate(starts):
                yield n, s, (starts[i + 1] if i + 1 < len(starts) else t1)


def worst_part(x, ref, cu, states=False):
    """Largest relative L2 over (document, head) pairs, and over (block, head) pairs of long
    documents, with where it occurs.  ``states``: x and ref are [N, H, ...] per-sequence arrays
    (one entry per document); otherwise token-major [T, H, ...]."""
    x = np.asarray(x, np.float64)
    ref = np.asarray(ref, np.float64)
    worst, where = 0.0, None
    cu = np.asarray(cu, np.int64)
    if states:
        for n in range(len(cu) - 1):
            if cu[n + 1] - cu[n] < MIN_DOC_TOKENS:
                continue
            e = _per_head(x[n:n + 1], ref[n:n + 1])
            h = int(np.argmax(e))
            if e[h] > worst:
                worst, where = float(e[h]), f"sequence {n}, head {h}"
        return worst, where
    for n, t0, t1 in blocks_of(cu):
        e = _per_head(x[t0:t1], ref[t0:t1])
        h = int(np.argmax(e))
        if e[h] > worst:
            worst, where = float(e[h]), f"document {n} tokens [{t0}, {t1}), head {h}"
    return worst, where


def report(name, x, ref, tol, cu=None, states=False):
    """Asserts the relative L2 of x against ref over the whole tensor is within tol.  With
    ``cu`` (the documents' offsets) it also asserts the same bound per (document, head) for
    documents of at least 64 tokens, and per (block of at most 4096 tokens, head) within longer
    documents, so that a wrong chunk or head cannot hide in a large norm."""
    x = np.asarray(x, np.float64)
    ref = np.asarray(ref, np.float64)
    err = rel_l2(x, ref)
    msg = f"  {name}: rel_l2 = {err:.3e} (tol {tol:.0e})"
    worst = None
    if cu is not None:
        worst, where = worst_part(x, ref, cu, states)
        if where is not None:
            msg += f"; worst per (document, head) {worst:.3e} at {where}"
    print(msg, flush=True)
    assert err <= tol, f"{name}: rel_l2 {err:.3e} > {tol:.0e}"
    if worst is not None:
        assert worst <= tol, f"{name}: {worst:.3e} > {tol:.0e} at {where}"
    return err
