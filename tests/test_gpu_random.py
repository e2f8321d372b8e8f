"""Randomised GPU parity across combinations of the options: dtype, head size, grouped heads,
the in-kernel q/k L2 normalisation, exact and truncate modes with forced segment lengths, per-
sequence or broadcast initial states, the output scale, and document lengths that include empty
and one-token documents.  Each case checks the forward (o, final states) against the fp64 oracle
and the backward in the case's mode against the oracle's exact gradients (the truncate mode's
backward approximates them within the same bound as its forward; gfx950 only; marked
``gpu``).

With bf16 inputs, d = 64 and the normalisation, the kernels round the normalised rows to bf16
before using them, as an unfused normalise-then-cast would (with d = 128 they fold the norms into
fp32 factors instead and round nothing).  On a short document that rounding alone moves a
(document, head) slice of dg by more than the bf16 bound, so those cases check each (document,
head) against the oracle run on the rounded rows and the whole tensors against the exact
oracle."""
import numpy as np
import pytest

from gdn_inputs import bf16_round, make_inputs, scale_qk_rows
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


def _case(seed):
    rng = np.random.default_rng(1000 + seed)
    dtype = ["bf16", "f32"][rng.integers(2)]
    d = [64, 128][rng.integers(2)]
    H = int(rng.choice([1, 2, 4, 6]))
    G = int(rng.choice([g for g in (1, 2, 3, 6) if H % g == 0]))
    norm = bool(rng.integers(2))
    mode = ["exact", "truncate"][rng.integers(2)]
    seg = int(rng.choice([0, 2, 3]))
    lengths = [int(x) for x in rng.choice([0, 1, 63, 64, 65, 130, 257, 400], rng.integers(1, 6))]
    if sum(lengths) == 0:
        lengths[0] = 70
    h0 = ["none", "seq", "broadcast"][rng.integers(3)]
    scale = float(rng.uniform(0.3, 1.5))
    return dict(dtype=dtype, d=d, H=H, G=G, norm=norm, mode=mode, seg=seg, lengths=lengths,
                h0=h0, scale=scale)


def _check(name, x, exact, used, tol, cu, states=False):
    """x against the exact oracle; with ``used`` (the oracle on the rows the kernels consume),
    per (document, head) against that and as a whole against the exact result."""
    if used is None:
        report(name, x, exact, tol, cu=cu, states=states)
    else:
        report(name + " (rows as used)", x, used, tol, cu=cu, states=states)
        report(name, x, exact, tol)


@pytest.mark.parametrize("seed", range(40))
def test_random_combination(gdn, oracle_mod, seed):
    c = _case(seed)
    print(f"[random {seed}: {c}]", flush=True)
    inp = make_inputs(c["lengths"], H=c["H"], dk=c["d"], dv=c["d"], dtype=c["dtype"],
                      seed=2000 + seed, h0_scale=0.5, with_dout=True)
    if c["norm"]:
        inp = scale_qk_rows(inp, seed=3000 + seed)
    G = c["G"]
    gi = dict(inp)
    for x in ("q", "k"):
        gi[x] = np.ascontiguousarray(inp[x][:, ::G])
    ref = dict(gi)
    for x in ("q", "k"):
        ref[x] = np.ascontiguousarray(np.repeat(gi[x], G, axis=1))
    h0 = None
    if c["h0"] == "seq":
        h0 = inp["h0"]
    elif c["h0"] == "broadcast":
        h0 = np.ascontiguousarray(inp["h0"][0])
    tdt = torch.bfloat16 if c["dtype"] == "bf16" else torch.float32
    dev = lambda a, t=None: (None if a is None else
                             torch.from_numpy(np.ascontiguousarray(a)).cuda().to(t) if t is not None
                             else torch.from_numpy(np.ascontiguousarray(a)).cuda())
    args = [dev(gi[x], tdt if x != "g" else None) for x in NAMES]
    cu = dev(inp["cu_seqlens"])
    o, ht = gdn.chunk_fwd(*args, cu, dev(h0), mode=c["mode"], seg_chunks=c["seg"], num_slots=256,
                          scale=c["scale"], qk_l2norm=c["norm"])
    torch.cuda.synchronize()
    oargs = [ref[x] for x in NAMES]
    rounded = c["norm"] and c["dtype"] == "bf16" and c["d"] == 64
    uargs = None
    if rounded:
        used = dict(ref)
        for x in ("q", "k"):
            used[x] = bf16_round(oracle_mod.l2norm(ref[x]))
        uargs = [used[x] for x in NAMES]

    def fwd_ref(a, norm):
        if c["mode"] == "exact":
            return oracle_mod.fwd_recurrent(*a, inp["cu_seqlens"], h0=h0, scale=c["scale"],
                                            qk_l2norm=norm)
        plan = oracle_mod.plan(inp["g"], inp["cu_seqlens"], c["H"], P=256, seg_chunks=c["seg"])
        return oracle_mod.fwd_truncated(*a, inp["cu_seqlens"], plan, h0=h0, scale=c["scale"],
                                        qk_l2norm=norm)

    o_ref, ht_ref = fwd_ref(oargs, c["norm"])
    o_u, ht_u = fwd_ref(uargs, False) if rounded else (None, None)
    tol = tol_for(c["dtype"])
    cu_h = inp["cu_seqlens"]
    _check("o", np64(o), o_ref, o_u, tol, cu_h)
    _check("ht", np64(ht), ht_ref, ht_u, tol, cu_h, states=True)
    gr = gdn.chunk_bwd(*args, cu, dev(inp["dout"], tdt), dev(h0), scale=c["scale"],
                       seg_chunks=c["seg"], num_slots=256, qk_l2norm=c["norm"], mode=c["mode"])
    torch.cuda.synchronize()
    r = oracle_mod.bwd(*oargs, inp["cu_seqlens"], inp["dout"], h0=h0, scale=c["scale"],
                       qk_l2norm=c["norm"])
    ru = None
    if rounded:
        ru = dict(oracle_mod.bwd(*uargs, inp["cu_seqlens"], inp["dout"], h0=h0,
                                 scale=c["scale"]))
        for n, x in (("dq", "q"), ("dk", "k")):
            ru[n] = oracle_mod.l2norm_bwd(ref[x], ru[n])
    T, d = inp["g"].shape[0], c["d"]
    gsum = lambda a: np.asarray(a).reshape(T, c["H"] // G, G, d).sum(axis=2)
    for n in ("dq", "dk"):
        _check(n, np64(gr[n]), gsum(r[n]), None if ru is None else gsum(ru[n]), tol, cu_h)
    for n in ("dv", "dg", "dbeta"):
        _check(n, np64(gr[n]), r[n], None if ru is None else ru[n], tol, cu_h)
    if h0 is not None:
        if c["h0"] == "broadcast":
            report("dh0", np64(gr["dh0"]), r["dh0"].sum(axis=0), tol)
        else:
            _check("dh0", np64(gr["dh0"]), r["dh0"], None if ru is None else ru["dh0"], tol,
                   cu_h, states=True)
