"""Helpers shared by the GPU tests: moving seeded inputs to the device and comparing results."""
import numpy as np
import torch

BF16_TOL = 5e-3  # relative L2 for bf16 inputs with an fp32 state
F32_TOL = 1e-4   # relative L2 for fp32 inputs


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


def report(name, x, ref, tol):
    err = rel_l2(x, ref)
    print(f"  {name}: rel_l2 = {err:.3e} (tol {tol:.0e})", flush=True)
    assert err <= tol, f"{name}: rel_l2 {err:.3e} > {tol:.0e}"
    return err
