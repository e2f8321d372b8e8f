"""Degenerate inputs of the method on the GPU against the fp64 oracle: beta = 0 (pure decay),
g = 0 (no decay: the truncation window never closes, so truncate mode must reach back to each
document's start), very negative g (the state forgets everything between tokens), and all-zero
q and k rows under the L2 normalisation (they stay zero).  The forward of each, and the backward
of the first three (every gradient against the oracle's exact backward, per (document, head);
with g = -30 the decay factors above the diagonal of a chunk overflow and must be masked, not
multiplied).  bf16 with d = 128 on the pipelined kernels, and fp32 with d = 64 on the general
kernels (gfx950 only; marked ``gpu``)."""
import numpy as np
import pytest

from gdn_inputs import bf16_round, make_inputs
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


def _run(gdn, oracle_mod, inp, label, mode, norm=False, seg=2):
    tdt = torch.bfloat16 if inp["dtype"] == "bf16" else torch.float32
    args = [torch.from_numpy(np.ascontiguousarray(inp[x])).cuda().to(tdt if x != "g" else torch.float32)
            for x in NAMES]
    cu = torch.from_numpy(inp["cu_seqlens"]).cuda()
    h0 = None if inp["h0"] is None else torch.from_numpy(inp["h0"]).cuda()
    o, ht = gdn.chunk_fwd(*args, cu, h0, mode=mode, seg_chunks=seg, num_slots=256, qk_l2norm=norm)
    torch.cuda.synchronize()
    H = inp["g"].shape[1]
    oargs = [inp[x] for x in NAMES]
    if mode == "exact":
        o_ref, ht_ref = oracle_mod.fwd_recurrent(*oargs, inp["cu_seqlens"], h0=inp["h0"],
                                                 qk_l2norm=norm)
    else:
        plan = oracle_mod.plan(inp["g"], inp["cu_seqlens"], H, P=256, seg_chunks=seg)
        o_ref, ht_ref = oracle_mod.fwd_truncated(*oargs, inp["cu_seqlens"], plan, h0=inp["h0"],
                                                 qk_l2norm=norm)
    print(f"[{label} {mode}]", flush=True)
    tol = tol_for(inp["dtype"])
    report("o", np64(o), o_ref, tol)
    report("ht", np64(ht), ht_ref, tol)
    return o, ht, o_ref, ht_ref


def _run_bwd(gdn, oracle_mod, inp, label, mode, seg=2, rel=("dq", "dk", "dv", "dg", "dbeta")):
    """The backward in ``mode`` against the oracle's exact gradients, per (document, head), for
    the gradients named in ``rel``."""
    tdt = torch.bfloat16 if inp["dtype"] == "bf16" else torch.float32
    dev = lambda a, t=None: torch.from_numpy(np.ascontiguousarray(a)).cuda().to(
        t if t is not None else torch.float32)
    args = [dev(inp[x], tdt if x != "g" else None) for x in NAMES]
    cu = torch.from_numpy(inp["cu_seqlens"]).cuda()
    h0 = None if inp["h0"] is None else dev(inp["h0"])
    print(f"[{label} {mode} backward]", flush=True)
    gr = gdn.chunk_bwd(*args, cu, dev(inp["dout"], tdt), h0, seg_chunks=seg, num_slots=256,
                       mode=mode)
    torch.cuda.synchronize()
    r = oracle_mod.bwd(*[inp[x] for x in NAMES], inp["cu_seqlens"], inp["dout"], h0=inp["h0"])
    tol = tol_for(inp["dtype"])
    cu_h = inp["cu_seqlens"]
    for n in rel:
        report(n, np64(gr[n]), r[n], tol, cu=cu_h)
    if h0 is not None:
        report("dh0", np64(gr["dh0"]), r["dh0"], tol, cu=cu_h, states=True)
    return gr, r


CASES = [("bf16", 128), ("f32", 64)]


@pytest.mark.parametrize("dtype,d", CASES)
@pytest.mark.parametrize("mode", ["exact", "truncate"])
def test_beta_zero_is_pure_decay(gdn, oracle_mod, dtype, d, mode):
    inp = make_inputs([300, 130], H=2, dk=d, dv=d, dtype=dtype, seed=601, h0_scale=0.5)
    inp["beta"] = np.zeros_like(inp["beta"])
    _, ht, _, _ = _run(gdn, oracle_mod, inp, f"beta=0 {dtype} d={d}", mode)
    # exact mode: the final state is h0 scaled by e^{sum g} of each document (truncate mode keeps
    # h0 only where the last segment's window reaches the document's start; _run compared it with
    # the oracle's truncated recurrence)
    if mode == "exact":
        cu = inp["cu_seqlens"]
        for n in range(2):
            decay = np.exp(inp["g"][cu[n]:cu[n + 1]].astype(np.float64).sum(axis=0))
            report(f"ht[{n}] closed form", np64(ht)[n], inp["h0"][n] * decay[:, None, None],
                   tol_for(dtype))


@pytest.mark.parametrize("dtype,d", CASES)
@pytest.mark.parametrize("mode", ["exact", "truncate"])
def test_no_decay(gdn, oracle_mod, dtype, d, mode):
    """g = 0: no history is ever truncated; truncate mode equals exact mode."""
    inp = make_inputs([600, 200], H=2, dk=d, dv=d, dtype=dtype, seed=602)
    inp["g"] = np.zeros_like(inp["g"])
    _, _, o_ref, _ = _run(gdn, oracle_mod, inp, f"g=0 {dtype} d={d}", mode)
    o_exact, _ = oracle_mod.fwd_recurrent(*[inp[x] for x in NAMES], inp["cu_seqlens"])
    assert np.allclose(o_ref, o_exact, rtol=0, atol=1e-12)


@pytest.mark.parametrize("dtype,d", CASES)
@pytest.mark.parametrize("mode", ["exact", "truncate"])
def test_total_forgetting(gdn, oracle_mod, dtype, d, mode):
    """g = -30 everywhere: the state forgets all but the current token (o_t depends on token t
    only), and the truncation window is one chunk."""
    inp = make_inputs([257, 64], H=2, dk=d, dv=d, dtype=dtype, seed=603, h0_scale=0.5)
    inp["g"] = np.full_like(inp["g"], -30.0)
    _run(gdn, oracle_mod, inp, f"g=-30 {dtype} d={d}", mode)


@pytest.mark.parametrize("dtype,d", [("bf16", 128), ("f32", 64)])
def test_zero_rows_under_l2norm(gdn, oracle_mod, dtype, d):
    """Rows of q and k that are all zero stay zero after the normalisation (|row|^2 + eps > 0)."""
    inp = make_inputs([200, 70], H=2, dk=d, dv=d, dtype=dtype, seed=604, h0_scale=0.5)
    rng = np.random.default_rng(605)
    for x in ("q", "k"):
        a = inp[x].copy()
        a[rng.random(a.shape[:2]) < 0.2] = 0.0
        inp[x] = bf16_round(a) if dtype == "bf16" else a
    _run(gdn, oracle_mod, inp, f"zero rows l2norm {dtype} d={d}", "exact", norm=True)


@pytest.mark.parametrize("dtype,d", CASES)
def test_all_documents_empty(gdn, dtype, d):
    """T = 0 (every document empty): the final states are the initial states, nothing else is
    written, and the backward passes dht through to dh0."""
    tdt = torch.bfloat16 if dtype == "bf16" else torch.float32
    H, N = 2, 3
    q = torch.zeros((0, H, d), device="cuda", dtype=tdt)
    g = torch.zeros((0, H), device="cuda")
    cu = torch.zeros(N + 1, dtype=torch.int32, device="cuda")
    h0 = torch.randn((N, H, d, d), device="cuda")
    for mode in ("exact", "truncate"):
        o, ht = gdn.chunk_fwd(q, q, q, g, g.to(tdt), cu, h0, mode=mode, num_slots=256)
        torch.cuda.synchronize()
        assert o.shape == (0, H, d) and torch.equal(ht, h0), mode
    dht = torch.randn((N, H, d, d), device="cuda")
    gr = gdn.chunk_bwd(q, q, q, g, g.to(tdt), cu, q, h0, dht)
    torch.cuda.synchronize()
    assert gr["dq"].shape == (0, H, d)
    assert torch.equal(gr["dh0"], dht)


@pytest.mark.parametrize("dtype,d", CASES)
@pytest.mark.parametrize("mode", ["exact", "truncate"])
def test_beta_zero_backward(gdn, oracle_mod, dtype, d, mode):
    """beta = 0: dv is zero, dbeta is not (the gradient at beta = 0)."""
    inp = make_inputs([300, 130], H=2, dk=d, dv=d, dtype=dtype, seed=601, h0_scale=0.5,
                      with_dout=True)
    inp["beta"] = np.zeros_like(inp["beta"])
    gr, _ = _run_bwd(gdn, oracle_mod, inp, f"beta=0 {dtype} d={d}", mode)
    assert np.all(np64(gr["dv"]) == 0.0)


@pytest.mark.parametrize("dtype,d", CASES)
@pytest.mark.parametrize("mode", ["exact", "truncate"])
def test_no_decay_backward(gdn, oracle_mod, dtype, d, mode):
    """g = 0: the truncate mode's windows reach every document's ends, as exact mode."""
    inp = make_inputs([600, 200], H=2, dk=d, dv=d, dtype=dtype, seed=602, with_dout=True)
    inp["g"] = np.zeros_like(inp["g"])
    _run_bwd(gdn, oracle_mod, inp, f"g=0 {dtype} d={d}", mode)


@pytest.mark.parametrize("dtype,d", CASES)
@pytest.mark.parametrize("mode", ["exact", "truncate"])
def test_total_forgetting_backward(gdn, oracle_mod, dtype, d, mode):
    """g = -30: every gradient is local to its token and the chunk maps vanish.  dg itself is
    then of order e^-30 (the oracle's is about 1e-13): the chunked form obtains it as the row
    minus the column sums of a chunk's products, whose diagonal terms are of order one and
    cancel, so the e^-30 remainder lies below fp32 resolution of those sums.  dg is held to the
    tolerance absolutely, on the scale of those per-row products (dbeta is formed from the same
    kind), and the other gradients relatively as everywhere."""
    inp = make_inputs([257, 64], H=2, dk=d, dv=d, dtype=dtype, seed=603, h0_scale=0.5,
                      with_dout=True)
    inp["g"] = np.full_like(inp["g"], -30.0)
    gr, r = _run_bwd(gdn, oracle_mod, inp, f"g=-30 {dtype} d={d}", mode,
                     rel=("dq", "dk", "dv", "dbeta"))
    dg = np64(gr["dg"])
    assert np.all(np.isfinite(dg))
    err = np.linalg.norm(dg - r["dg"]) / np.linalg.norm(r["dbeta"])
    print(f"  dg: |error| / |dbeta| = {err:.3e}", flush=True)
    assert err <= tol_for(dtype)
