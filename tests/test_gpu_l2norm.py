"""GPU parity of the in-kernel q/k L2 normalisation (``qk_l2norm``) against the fp64 oracle,
which normalises each (token, head) row of q and k, row / sqrt(|row|^2 + 1e-6), before the
recurrence.  Inputs have rows of length 0.3 .. 3 so that the normalisation matters (gfx950 only;
marked ``gpu``)."""
import numpy as np
import pytest

from gdn_inputs import make_inputs, scale_qk_rows, workload
from gpu_util import np64, report, tol_for

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")
NAMES = ("q", "k", "v", "g", "beta")


@pytest.fixture(scope="module")
def gdn():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import linear_attention_recurrence_prefill_amd as m

    m.load_library()
    return m


def _dev(a, dtype=None):
    t = torch.from_numpy(np.ascontiguousarray(a)).cuda()
    return t.to(dtype) if dtype is not None else t


def _tdt(inp):
    return torch.bfloat16 if inp["dtype"] == "bf16" else torch.float32


def _run_fwd(gdn, oracle_mod, inp, label, mode="exact", seg=0, slots=256, scale=1.0, G=1):
    inp = scale_qk_rows(inp, seed=501)
    gi = dict(inp)
    if G > 1:  # grouped heads: q, k keep every G-th head; the oracle repeats them
        for x in ("q", "k"):
            gi[x] = np.ascontiguousarray(inp[x][:, ::G])
    ref = dict(gi)
    for x in ("q", "k"):
        ref[x] = np.ascontiguousarray(np.repeat(gi[x], G, axis=1))
    tdt = _tdt(inp)
    args = [_dev(gi[x], tdt if x != "g" else None) for x in NAMES]
    h0 = None if inp["h0"] is None else _dev(inp["h0"])
    print(f"[{label}]", flush=True)
    o, ht = gdn.chunk_fwd(*args, _dev(inp["cu_seqlens"]), h0, mode=mode, seg_chunks=seg,
                          num_slots=slots, scale=scale, qk_l2norm=True)
    torch.cuda.synchronize()
    H = inp["g"].shape[1]
    oargs = [ref[x] for x in NAMES]
    if mode == "exact":
        o_ref, ht_ref = oracle_mod.fwd_recurrent(*oargs, inp["cu_seqlens"], h0=inp["h0"],
                                                 scale=scale, qk_l2norm=True)
    else:
        plan = oracle_mod.plan(inp["g"], inp["cu_seqlens"], H, P=slots, seg_chunks=seg)
        o_ref, ht_ref = oracle_mod.fwd_truncated(*oargs, inp["cu_seqlens"], plan, h0=inp["h0"],
                                                 scale=scale, qk_l2norm=True)
    tol = tol_for(inp["dtype"])
    report("o", np64(o), o_ref, tol, cu=inp["cu_seqlens"])
    report("ht", np64(ht), ht_ref, tol, cu=inp["cu_seqlens"], states=True)
    # without the normalisation the same inputs give a different result
    o_plain, _ = oracle_mod.fwd_recurrent(*oargs, inp["cu_seqlens"], h0=inp["h0"], scale=scale)
    assert np.linalg.norm(o_plain - o_ref) > 10 * tol * np.linalg.norm(o_ref)


@pytest.mark.parametrize("mode,seg", [("exact", 0), ("exact", 2), ("truncate", 2)])
def test_l2norm_bf16_d128_ragged(gdn, oracle_mod, mode, seg):
    inp = make_inputs([1, 63, 64, 65, 130, 0, 300], H=4, dk=128, dv=128, dtype="bf16", seed=511,
                      h0_scale=0.5)
    _run_fwd(gdn, oracle_mod, inp, f"l2norm bf16 d=128 {mode} seg={seg}", mode=mode, seg=seg,
             scale=0.7)


def test_l2norm_bf16_d128_grouped_heads(gdn, oracle_mod):
    inp = make_inputs([500, 200], H=8, dk=128, dv=128, dtype="bf16", seed=512, h0_scale=0.5)
    _run_fwd(gdn, oracle_mod, inp, "l2norm bf16 d=128 grouped G=4", mode="exact", seg=2, G=4)


@pytest.mark.parametrize("d,mode,seg", [(64, "exact", 0), (128, "exact", 0), (64, "truncate", 2)])
def test_l2norm_fp32(gdn, oracle_mod, d, mode, seg):
    inp = make_inputs([100, 0, 200, 64], H=2, dk=d, dv=d, dtype="f32", seed=513, h0_scale=0.5)
    _run_fwd(gdn, oracle_mod, inp, f"l2norm fp32 d={d} {mode}", mode=mode, seg=seg, scale=0.5)


def test_l2norm_long_32k_truncate(gdn, oracle_mod):
    """The 32768-token, 8-head workload with q and k rows of length 0.3 .. 3, normalised in the
    kernel (truncate mode, the benchmarked launch configuration)."""
    inp = workload("long")
    inp = scale_qk_rows(inp, seed=514)
    d = {x: _dev(inp[x], torch.bfloat16 if x != "g" else None) for x in NAMES}
    cu = _dev(inp["cu_seqlens"])
    o, ht = gdn.chunk_fwd(*[d[x] for x in NAMES], cu, None, mode="truncate", num_slots=256,
                          cu_seqlens_host=inp["cu_seqlens"], qk_l2norm=True)
    torch.cuda.synchronize()
    plan = oracle_mod.plan(inp["g"], inp["cu_seqlens"], 8, P=256)
    o_t, ht_t = oracle_mod.fwd_truncated(*[inp[x] for x in NAMES], inp["cu_seqlens"], plan,
                                         qk_l2norm=True)
    print("[l2norm long 32K truncate]", flush=True)
    report("o", np64(o), o_t, 5e-3, cu=inp["cu_seqlens"])
    report("ht", np64(ht), ht_t, 5e-3, cu=inp["cu_seqlens"], states=True)


@pytest.mark.parametrize("mode,seg", [("exact", 0), ("truncate", 2)])
def test_l2norm_bf16_d64(gdn, oracle_mod, mode, seg):
    """bf16 with d = 64 (the rows normalised as they are staged and rounded to bf16)."""
    inp = make_inputs([1, 63, 64, 65, 130, 0, 300], H=4, dk=64, dv=64, dtype="bf16", seed=515,
                      h0_scale=0.5)
    _run_fwd(gdn, oracle_mod, inp, f"l2norm bf16 d=64 {mode}", mode=mode, seg=seg, scale=0.7)


@pytest.mark.parametrize("dtype,d,G,seg,mode", [
    ("bf16", 128, 1, 0, "exact"), ("bf16", 128, 2, 2, "exact"), ("bf16", 64, 1, 0, "exact"),
    ("bf16", 64, 2, 0, "exact"), ("f32", 64, 1, 0, "exact"), ("f32", 128, 2, 0, "exact"),
    ("bf16", 128, 1, 2, "truncate"), ("bf16", 128, 2, 2, "truncate")])
def test_l2norm_backward(gdn, oracle_mod, dtype, d, G, seg, mode):
    """Gradients of the raw q, k (through the normalisation) and of v, g, beta, h0 against the
    oracle's backward with the normalisation; grouped heads sum dq, dk over each group.  The
    truncate mode's backward (2-chunk segments: warmup windows that stop inside a document and
    ones that reach its start or end) against the same exact gradients."""
    inp = make_inputs([300, 65, 0, 260], H=4, dk=d, dv=d, dtype=dtype, seed=521, h0_scale=0.5,
                      with_dout=True)
    inp = scale_qk_rows(inp, seed=522)
    gi = dict(inp)
    for x in ("q", "k"):
        gi[x] = np.ascontiguousarray(inp[x][:, ::G])
    ref = dict(gi)
    for x in ("q", "k"):
        ref[x] = np.ascontiguousarray(np.repeat(gi[x], G, axis=1))
    tdt = _tdt(inp)
    rng = np.random.default_rng(523)
    N = len(inp["cu_seqlens"]) - 1
    dht = (0.3 * rng.standard_normal((N, 4, d, d))).astype(np.float32)
    args = [_dev(gi[x], tdt if x != "g" else None) for x in NAMES]
    print(f"[l2norm bwd {dtype} d={d} G={G} seg={seg} {mode}]", flush=True)
    gr = gdn.chunk_bwd(*args, _dev(inp["cu_seqlens"]), _dev(inp["dout"], tdt), _dev(inp["h0"]),
                       _dev(dht), scale=0.7, seg_chunks=seg, num_slots=256 if seg else 0,
                       qk_l2norm=True, mode=mode)
    torch.cuda.synchronize()
    r = oracle_mod.bwd(*[ref[x] for x in NAMES], inp["cu_seqlens"], inp["dout"], h0=inp["h0"],
                       dht=dht, scale=0.7, qk_l2norm=True)
    T = inp["g"].shape[0]
    tol = tol_for(dtype)
    for n in ("dq", "dk"):
        summed = np.asarray(r[n]).reshape(T, 4 // G, G, d).sum(axis=2)
        report(n, np64(gr[n]), summed, tol, cu=inp["cu_seqlens"])
    for n in ("dv", "dg", "dbeta"):
        report(n, np64(gr[n]), r[n], tol, cu=inp["cu_seqlens"])
    report("dh0", np64(gr["dh0"]), r["dh0"], tol, cu=inp["cu_seqlens"], states=True)
