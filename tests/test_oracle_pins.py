"""Pins of the fp64 oracle against facts fixed by the pages and by mathematics (CPU only).

Each test is chosen so that a plausible mistake in the oracle (a dropped term, a sign, an
index, a transposed operand, decay applied after instead of before the correction, reading the
state before instead of after the update) fails at least one of them:

* a hand-worked two-token example (tests/golden/hand_worked_d2.txt);
* closed forms: beta = 0 (pure decay), g = 0 / beta = 1 / orthonormal keys (exact overwrite),
  one token (the matrix form of the rule);
* invariants: chunked form == token form (C = 1, 16, 64), packed == unpacked, resume, boundary
  isolation, superposition in (v, h0), rotation invariance, the state-norm bound, the affine
  form of a segment (the exact split);
* the backward against central finite differences, the beta = 0 special case, and the sum of
  gradients at a shared initial state;
* the truncation plan's rule and its provable error bound;
* the optional q/k L2 normalisation: its closed form, its backward against central differences,
  scale invariance of the normalised forward, and the normalised backward against central
  differences.
"""
import os

import numpy as np
import pytest

from gdn_inputs import make_inputs

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _args(inp):
    return [inp[x] for x in ("q", "k", "v", "g", "beta")]


def _rel(a, b):
    return float(np.linalg.norm(np.ravel(a - b)) / max(np.linalg.norm(np.ravel(b)), 1e-300))


# --------------------------------------------------------------------------- golden example
def _load_golden(name):
    vals = {}
    with open(os.path.join(GOLDEN, name)) as f:
        for line in f:
            line = line.strip()
            if not line or line.startswith("#"):
                continue
            parts = line.split()
            vals[parts[0]] = np.array([float(x) for x in parts[1:]])
    return vals


def test_hand_worked_example(oracle_mod):
    gv = _load_golden("hand_worked_d2.txt")
    T, H, d = 2, 1, 2
    q = gv["q"].reshape(T, H, d)
    k = gv["k"].reshape(T, H, d)
    v = gv["v"].reshape(T, H, d)
    g = gv["g"].reshape(T, H)
    beta = gv["beta"].reshape(T, H)
    h0 = gv["h0"].reshape(1, H, d, d)
    cu = np.array([0, 2], np.int32)
    o_ref = gv["o"].reshape(T, H, d)
    ht_ref = gv["ht"].reshape(1, H, d, d)
    o, ht = oracle_mod.fwd_recurrent(q, k, v, g, beta, cu, h0=h0)
    np.testing.assert_allclose(o, o_ref, rtol=0, atol=1e-14)
    np.testing.assert_allclose(ht, ht_ref, rtol=0, atol=1e-14)
    for C in (1, 2, 64):
        o2, ht2 = oracle_mod.fwd_chunked(q, k, v, g, beta, cu, h0=h0, chunk=C)
        np.testing.assert_allclose(o2, o_ref, rtol=0, atol=1e-14)
        np.testing.assert_allclose(ht2, ht_ref, rtol=0, atol=1e-14)


# --------------------------------------------------------------------------- closed forms
@pytest.mark.parametrize("form", ["recurrent", "chunked"])
def test_beta_zero_is_pure_decay(oracle_mod, form):
    """beta = 0: S_t = exp(sum_{s<=t} g_s) h0 and o_t = exp(sum g) h0^T q_t."""
    inp = make_inputs([150, 70], H=2, dk=8, dv=5, dtype="f32", seed=3, h0_scale=1.0)
    inp["beta"] = np.zeros_like(inp["beta"])
    cu = inp["cu_seqlens"]
    fn = oracle_mod.fwd_recurrent if form == "recurrent" else oracle_mod.fwd_chunked
    o, ht = fn(*_args(inp), cu, h0=inp["h0"])
    g = inp["g"].astype(np.float64)
    h0 = inp["h0"].astype(np.float64)
    for n in range(2):
        a, b = cu[n], cu[n + 1]
        decay = np.exp(np.cumsum(g[a:b], axis=0))  # [len, H]
        for h in range(2):
            o_ref = decay[:, h, None] * (inp["q"][a:b, h].astype(np.float64) @ h0[n, h])
            np.testing.assert_allclose(o[a:b, h], o_ref, rtol=1e-12, atol=1e-14)
            np.testing.assert_allclose(ht[n, h], decay[-1, h] * h0[n, h], rtol=1e-12,
                                       atol=1e-14)


@pytest.mark.parametrize("form", ["recurrent", "chunked"])
def test_exact_overwrite_with_orthonormal_keys(oracle_mod, form):
    """g = 0, beta = 1, orthonormal keys, h0 = 0: S_t = sum_{j<=t} k_j v_j^T, so a query equal
    to a stored key returns its value; writing a key again overwrites its value."""
    rng = np.random.default_rng(5)
    d, dv, T = 12, 7, 10
    basis, _ = np.linalg.qr(rng.standard_normal((d, d)))
    keys = basis.T[:8]  # 8 orthonormal rows
    k = np.zeros((T, 1, d))
    k[:8, 0] = keys
    k[8, 0] = keys[2]  # rewrite key 2
    k[9, 0] = keys[5]  # rewrite key 5
    v = rng.standard_normal((T, 1, dv))
    q = np.zeros((T, 1, d))
    for t in range(T):
        q[t, 0] = keys[(3 * t + 1) % 8]
    g = np.zeros((T, 1))
    beta = np.ones((T, 1))
    cu = np.array([0, T], np.int32)
    fn = oracle_mod.fwd_recurrent if form == "recurrent" else oracle_mod.fwd_chunked
    o, ht = fn(q, k, v, g, beta, cu)
    stored = {}
    for t in range(T):
        j = {8: 2, 9: 5}.get(t, t)
        stored[j] = v[t, 0]
        want = stored.get((3 * t + 1) % 8, np.zeros(dv))
        np.testing.assert_allclose(o[t, 0], want, atol=1e-12)
    S_ref = sum(np.outer(keys[j], stored[j]) for j in stored)
    np.testing.assert_allclose(ht[0, 0], S_ref, atol=1e-12)


def test_one_token_matrix_form(oracle_mod):
    """T = 1: S_1 = alpha (I - beta k k^T) h0 + beta k v^T and o = S_1^T q, with the (I - beta k
    k^T) matrix built explicitly (the form the rule is stated in)."""
    rng = np.random.default_rng(11)
    dk, dv, H = 6, 4, 3
    q = rng.standard_normal((1, H, dk))
    k = rng.standard_normal((1, H, dk))
    v = rng.standard_normal((1, H, dv))
    g = -rng.random((1, H))
    beta = rng.random((1, H)) * 1.5
    h0 = rng.standard_normal((1, H, dk, dv))
    cu = np.array([0, 1], np.int32)
    o, ht = oracle_mod.fwd_recurrent(q, k, v, g, beta, cu, h0=h0, scale=0.7)
    for h in range(H):
        kk = k[0, h][:, None]
        S1 = np.exp(g[0, h]) * (np.eye(dk) - beta[0, h] * kk @ kk.T) @ h0[0, h] \
            + beta[0, h] * kk @ v[0, h][None, :]
        np.testing.assert_allclose(ht[0, h], S1, rtol=1e-13, atol=1e-13)
        np.testing.assert_allclose(o[0, h], 0.7 * S1.T @ q[0, h], rtol=1e-13, atol=1e-13)


def test_matrix_form_iterated(oracle_mod):
    """Several tokens: iterate the explicit matrix form and compare states and outputs."""
    inp = make_inputs([37], H=2, dk=5, dv=3, dtype="f32", seed=8, h0_scale=1.0)
    o, ht = oracle_mod.fwd_recurrent(*_args(inp), inp["cu_seqlens"], h0=inp["h0"])
    for h in range(2):
        S = inp["h0"][0, h].astype(np.float64)
        for t in range(37):
            kk = inp["k"][t, h].astype(np.float64)[:, None]
            a = np.exp(float(inp["g"][t, h]))
            b = float(inp["beta"][t, h])
            S = a * (np.eye(5) - b * kk @ kk.T) @ S + b * kk @ inp["v"][t, h][None, :]
            np.testing.assert_allclose(o[t, h], S.T @ inp["q"][t, h], rtol=1e-12, atol=1e-13)
        np.testing.assert_allclose(ht[0, h], S, rtol=1e-12, atol=1e-13)


# --------------------------------------------------------------------------- invariants
@pytest.mark.parametrize("C", [1, 16, 64])
def test_chunked_equals_recurrent(oracle_mod, C):
    lens = [1, 63, 64, 65, 127, 0, 200]
    inp = make_inputs(lens, H=2, dk=16, dv=12, dtype="f32", seed=21, h0_scale=0.3)
    o1, h1 = oracle_mod.fwd_recurrent(*_args(inp), inp["cu_seqlens"], h0=inp["h0"])
    o2, h2 = oracle_mod.fwd_chunked(*_args(inp), inp["cu_seqlens"], h0=inp["h0"], chunk=C)
    assert _rel(o2, o1) < 1e-12 and _rel(h2, h1) < 1e-12


def test_chunked_equals_recurrent_d128(oracle_mod):
    inp = make_inputs([130], H=1, dk=128, dv=128, dtype="bf16", seed=22)
    o1, h1 = oracle_mod.fwd_recurrent(*_args(inp), inp["cu_seqlens"])
    o2, h2 = oracle_mod.fwd_chunked(*_args(inp), inp["cu_seqlens"])
    assert _rel(o2, o1) < 1e-12 and _rel(h2, h1) < 1e-12


def test_chunked_intermediates_consistent(oracle_mod):
    """The exposed chunk intermediates satisfy their defining identities: (I + A) Tm = I with
    A rebuilt from k, beta, gamma; gamma is the within-chunk cumsum; Delta = U - W h."""
    inp = make_inputs([100], H=1, dk=8, dv=4, dtype="f32", seed=2, h0_scale=1.0)
    cu = inp["cu_seqlens"]
    o, ht, it = oracle_mod.fwd_chunked(*_args(inp), cu, h0=inp["h0"], intermediates=True)
    k = inp["k"][:, 0].astype(np.float64)
    b = inp["beta"][:, 0].astype(np.float64)
    g = inp["g"][:, 0].astype(np.float64)
    for c, (a, e) in enumerate([(0, 64), (64, 100)]):
        n = e - a
        gam = np.cumsum(g[a:e])
        np.testing.assert_allclose(it["gamma"][a:e, 0], gam, rtol=1e-13, atol=1e-13)
        A = np.zeros((n, n))
        for r in range(n):
            for i in range(r):
                A[r, i] = b[a + r] * np.exp(gam[r] - gam[i]) * (k[a + r] @ k[a + i])
        Tm = it["tm"][c, 0, :n, :n]
        np.testing.assert_allclose((np.eye(n) + A) @ Tm, np.eye(n), atol=1e-12)
        dl = it["u"][c, 0, :n] - it["w"][c, 0, :n] @ it["hc"][c, 0]
        np.testing.assert_allclose(it["delta"][a:e, 0], dl, atol=1e-12)


def test_packed_equals_unpacked_bitwise(oracle_mod):
    """Packed documents with state resets give exactly the per-document results."""
    lens = [40, 0, 129, 64]
    inp = make_inputs(lens, H=2, dk=8, dv=8, dtype="f32", seed=4, h0_scale=0.5)
    cu = inp["cu_seqlens"]
    o, ht = oracle_mod.fwd_recurrent(*_args(inp), cu, h0=inp["h0"])
    for n in range(len(lens)):
        a, b = cu[n], cu[n + 1]
        sub = [x[a:b] for x in _args(inp)]
        o1, h1 = oracle_mod.fwd_recurrent(*sub, np.array([0, b - a], np.int32),
                                          h0=inp["h0"][n:n + 1])
        assert np.array_equal(o1, o[a:b]) and np.array_equal(h1[0], ht[n])


def test_boundary_isolation(oracle_mod):
    """Perturbing every input of document A leaves document B bitwise unchanged."""
    inp = make_inputs([90, 77], H=2, dk=8, dv=6, dtype="f32", seed=9)
    cu = inp["cu_seqlens"]
    o, ht = oracle_mod.fwd_chunked(*_args(inp), cu)
    rng = np.random.default_rng(0)
    pert = {x: inp[x].copy() for x in ("q", "k", "v", "g", "beta")}
    for x in pert:
        pert[x][:90] += rng.standard_normal(pert[x][:90].shape).astype(np.float32)
    o2, ht2 = oracle_mod.fwd_chunked(*[pert[x] for x in ("q", "k", "v", "g", "beta")], cu)
    assert np.array_equal(o[90:], o2[90:]) and np.array_equal(ht[1], ht2[1])
    assert not np.allclose(o[:90], o2[:90])


def test_resume_equals_single_call(oracle_mod):
    """Running [0, T1) then [T1, T) with h0 = the first call's final state equals one call."""
    inp = make_inputs([173], H=2, dk=8, dv=8, dtype="f32", seed=12, h0_scale=0.4)
    args = _args(inp)
    o, ht = oracle_mod.fwd_recurrent(*args, inp["cu_seqlens"], h0=inp["h0"])
    T1 = 100
    oa, ha = oracle_mod.fwd_chunked(*[x[:T1] for x in args], np.array([0, T1], np.int32),
                                    h0=inp["h0"])
    ob, hb = oracle_mod.fwd_chunked(*[x[T1:] for x in args], np.array([0, 173 - T1], np.int32),
                                    h0=ha)
    assert _rel(np.concatenate([oa, ob]), o) < 1e-12 and _rel(hb, ht) < 1e-12


def test_superposition_in_v_and_h0(oracle_mod):
    """With q, k, g, beta fixed, (o, ht) is linear in (v, h0) jointly."""
    i1 = make_inputs([80], H=1, dk=8, dv=8, dtype="f32", seed=31, h0_scale=1.0)
    i2 = make_inputs([80], H=1, dk=8, dv=8, dtype="f32", seed=32, h0_scale=1.0)
    cu = i1["cu_seqlens"]
    base = [i1["q"], i1["k"]]
    rest = [i1["g"], i1["beta"]]
    oa, ha = oracle_mod.fwd_recurrent(*base, i1["v"], *rest, cu, h0=i1["h0"])
    ob, hb = oracle_mod.fwd_recurrent(*base, i2["v"], *rest, cu, h0=i2["h0"])
    vc = 2.0 * i1["v"].astype(np.float64) - 3.0 * i2["v"].astype(np.float64)
    hc = 2.0 * i1["h0"].astype(np.float64) - 3.0 * i2["h0"].astype(np.float64)
    oc, hcc = oracle_mod.fwd_recurrent(*base, vc, *rest, cu, h0=hc)
    assert _rel(oc, 2 * oa - 3 * ob) < 1e-12 and _rel(hcc, 2 * ha - 3 * hb) < 1e-12


def test_rotation_invariance(oracle_mod):
    """Rotating q, k and the key side of h0 by one orthogonal R leaves o unchanged and maps the
    final state to R ht."""
    inp = make_inputs([70], H=1, dk=8, dv=5, dtype="f32", seed=13, h0_scale=1.0)
    R, _ = np.linalg.qr(np.random.default_rng(1).standard_normal((8, 8)))
    o, ht = oracle_mod.fwd_recurrent(*_args(inp), inp["cu_seqlens"], h0=inp["h0"])
    qr = inp["q"].astype(np.float64) @ R.T
    kr = inp["k"].astype(np.float64) @ R.T
    h0r = np.einsum("ij,nhjv->nhiv", R, inp["h0"].astype(np.float64))
    o2, ht2 = oracle_mod.fwd_recurrent(qr, kr, inp["v"], inp["g"], inp["beta"],
                                       inp["cu_seqlens"], h0=h0r)
    assert _rel(o2, o) < 1e-12
    assert _rel(ht2, np.einsum("ij,nhjv->nhiv", R, ht)) < 1e-12


def test_state_norm_bound(oracle_mod):
    """With unit keys and beta in [0, 1]: ||S_t||_2 <= alpha_t ||S_{t-1}||_2 + beta_t ||v_t||."""
    inp = make_inputs([60], H=1, dk=6, dv=4, dtype="f32", seed=14, h0_scale=1.0)
    args = _args(inp)
    prev = np.linalg.norm(inp["h0"][0, 0].astype(np.float64), 2)
    h0 = inp["h0"]
    for t in range(60):
        _, ht = oracle_mod.fwd_recurrent(*[x[t:t + 1] for x in args], np.array([0, 1], np.int32),
                                         h0=h0)
        cur = np.linalg.norm(ht[0, 0], 2)
        bound = np.exp(float(inp["g"][t, 0])) * prev + float(inp["beta"][t, 0]) * \
            np.linalg.norm(inp["v"][t, 0].astype(np.float64))
        assert cur <= bound * (1 + 1e-12)
        prev, h0 = cur, ht


def test_segment_is_affine_in_its_start_state(oracle_mod):
    """S_end = M S_start + B with M = prod_t alpha_t (I - beta_t k_t k_t^T) (the exact split)."""
    inp = make_inputs([50], H=1, dk=6, dv=4, dtype="f32", seed=15, h0_scale=1.0)
    args = _args(inp)
    cu = inp["cu_seqlens"]
    _, B = oracle_mod.fwd_recurrent(*args, cu)
    M = np.eye(6)
    for t in range(50):
        kk = inp["k"][t, 0].astype(np.float64)[:, None]
        M = np.exp(float(inp["g"][t, 0])) * (np.eye(6) - inp["beta"][t, 0] * kk @ kk.T) @ M
    _, ht = oracle_mod.fwd_recurrent(*args, cu, h0=inp["h0"])
    np.testing.assert_allclose(ht[0, 0], M @ inp["h0"][0, 0] + B[0, 0], rtol=1e-12, atol=1e-13)


def test_scale_is_linear(oracle_mod):
    inp = make_inputs([40], H=1, dk=8, dv=8, dtype="f32", seed=16)
    o1, h1 = oracle_mod.fwd_chunked(*_args(inp), inp["cu_seqlens"], scale=1.0)
    o2, h2 = oracle_mod.fwd_chunked(*_args(inp), inp["cu_seqlens"], scale=0.125)
    assert _rel(o2, 0.125 * o1) < 1e-14 and np.array_equal(h1, h2)


# --------------------------------------------------------------------------- backward
def _loss(oracle_mod, args, cu, h0, dout, dht):
    o, ht = oracle_mod.fwd_recurrent(*args, cu, h0=h0)
    return float(np.sum(o * dout) + np.sum(ht * dht))


def test_backward_matches_finite_differences(oracle_mod):
    """Central differences of L = <o, dO> + <ht, dht> in fp64, for every input."""
    lens = [5, 0, 9]
    inp = make_inputs(lens, H=2, dk=4, dv=3, dtype="f32", seed=17, h0_scale=0.7)
    cu = inp["cu_seqlens"]
    args = [x.astype(np.float64) for x in _args(inp)]
    h0 = inp["h0"].astype(np.float64)
    rng = np.random.default_rng(3)
    dout = rng.standard_normal((14, 2, 3))
    dht = rng.standard_normal((3, 2, 4, 3))
    gr = oracle_mod.bwd(*args, cu, dout, h0=h0, dht=dht)
    names = ["dq", "dk", "dv", "dg", "dbeta"]
    eps = 1e-6
    for ai, name in enumerate(names):
        x = args[ai]
        num = np.zeros_like(x)
        for idx in np.ndindex(x.shape):
            xp = [a.copy() for a in args]
            xm = [a.copy() for a in args]
            xp[ai][idx] += eps
            xm[ai][idx] -= eps
            num[idx] = (_loss(oracle_mod, xp, cu, h0, dout, dht)
                        - _loss(oracle_mod, xm, cu, h0, dout, dht)) / (2 * eps)
        np.testing.assert_allclose(gr[name], num, rtol=1e-6, atol=1e-7, err_msg=name)
    num = np.zeros_like(h0)
    for idx in np.ndindex(h0.shape):
        hp, hm = h0.copy(), h0.copy()
        hp[idx] += eps
        hm[idx] -= eps
        num[idx] = (_loss(oracle_mod, args, cu, hp, dout, dht)
                    - _loss(oracle_mod, args, cu, hm, dout, dht)) / (2 * eps)
    np.testing.assert_allclose(gr["dh0"], num, rtol=1e-6, atol=1e-7, err_msg="dh0")


def test_backward_long_sequence_checkpoints(oracle_mod):
    """A sequence over several 64-token checkpoint blocks: spot-check with finite differences."""
    inp = make_inputs([150], H=1, dk=4, dv=3, dtype="f32", seed=18, h0_scale=0.5)
    cu = inp["cu_seqlens"]
    args = [x.astype(np.float64) for x in _args(inp)]
    h0 = inp["h0"].astype(np.float64)
    rng = np.random.default_rng(4)
    dout = rng.standard_normal((150, 1, 3))
    dht = rng.standard_normal((1, 1, 4, 3))
    gr = oracle_mod.bwd(*args, cu, dout, h0=h0, dht=dht)
    eps = 1e-6
    for ai, name in enumerate(["dq", "dk", "dv", "dg", "dbeta"]):
        for t in (0, 63, 64, 65, 128, 149):
            idx = (t, 0) + ((1,) if args[ai].ndim == 3 else ())
            xp = [a.copy() for a in args]
            xm = [a.copy() for a in args]
            xp[ai][idx] += eps
            xm[ai][idx] -= eps
            num = (_loss(oracle_mod, xp, cu, h0, dout, dht)
                   - _loss(oracle_mod, xm, cu, h0, dout, dht)) / (2 * eps)
            assert abs(gr[name][idx] - num) <= 1e-6 * max(1.0, abs(num)), (name, t)


def test_backward_beta_zero_gives_zero_dv(oracle_mod):
    inp = make_inputs([30], H=1, dk=4, dv=4, dtype="f32", seed=19, h0_scale=1.0)
    inp["beta"] = np.zeros_like(inp["beta"])
    dout = np.random.default_rng(5).standard_normal((30, 1, 4))
    gr = oracle_mod.bwd(*_args(inp), inp["cu_seqlens"], dout, h0=inp["h0"])
    assert np.all(gr["dv"] == 0.0)


def test_shared_state_gradient_is_sum_over_branches(oracle_mod):
    """A prefix's final state feeding several branches receives the sum of their dh0
    ("Backward through P"): checked against finite differences through prefix + branches."""
    pre = make_inputs([20], H=1, dk=4, dv=3, dtype="f32", seed=40)
    br = make_inputs([7, 11, 5], H=1, dk=4, dv=3, dtype="f32", seed=41)
    rng = np.random.default_rng(6)
    dout_b = rng.standard_normal((23, 1, 3))
    pa = [x.astype(np.float64) for x in _args(pre)]
    ba = [x.astype(np.float64) for x in _args(br)]

    def total_loss(v_pre):
        _, hp = oracle_mod.fwd_recurrent(pa[0], pa[1], v_pre, pa[3], pa[4],
                                         pre["cu_seqlens"])
        ob, _ = oracle_mod.fwd_recurrent(*ba, br["cu_seqlens"], h0=hp[0])
        return float(np.sum(ob * dout_b))

    _, hp = oracle_mod.fwd_recurrent(*pa, pre["cu_seqlens"])
    gb = oracle_mod.bwd(*ba, br["cu_seqlens"], dout_b, h0=hp[0])
    dh_shared = gb["dh0"].sum(axis=0, keepdims=True)
    gp = oracle_mod.bwd(*pa, pre["cu_seqlens"], np.zeros((20, 1, 3)), dht=dh_shared)
    eps = 1e-6
    for idx in [(0, 0, 0), (7, 0, 1), (19, 0, 2)]:
        vp, vm = pa[2].copy(), pa[2].copy()
        vp[idx] += eps
        vm[idx] -= eps
        num = (total_loss(vp) - total_loss(vm)) / (2 * eps)
        assert abs(gp["dv"][idx] - num) <= 1e-7 * max(1.0, abs(num))


# --------------------------------------------------------------------------- truncation
def test_segment_length_latency_model(oracle_mod):
    # 32K tokens, 8 heads, 256 CUs: 3*sqrt(8*512/256) = 12 -> nearest power of two 16
    assert oracle_mod.segment_chunks(8, 512, 1, 256) == 16
    # small problems hit the floor of 4 chunks
    assert oracle_mod.segment_chunks(1, 4, 1, 256) == 4
    # 3*sqrt(16*1024/256) = 24 -> log2 = 4.58 -> 32
    assert oracle_mod.segment_chunks(16, 1024, 1, 256) == 32
    # batch x heads fills the machine: no split
    assert oracle_mod.segment_chunks(8, 512, 32, 256) == 0
    # forced length wins
    assert oracle_mod.segment_chunks(8, 512, 1, 256, forced=5) == 5


def test_plan_rule(oracle_mod):
    """Every warmup window is the shortest run of whole preceding chunks whose gate sum is
    below the threshold, or reaches the sequence start."""
    lens = [64 * 40 + 17, 64 * 3, 64 * 25]
    inp = make_inputs(lens, H=3, dk=4, dv=4, dtype="f32", seed=23)
    cu = inp["cu_seqlens"]
    p = oracle_mod.plan(inp["g"], cu, H=3, P=256, seg_chunks=4)
    g = inp["g"].astype(np.float64)
    assert len(p["seq"]) == 11 + 1 + 7
    for s in range(len(p["seq"])):
        n, c0 = p["seq"][s], p["c0"][s]
        for h in range(3):
            w = p["warm"][s, h]
            assert 0 <= w <= c0
            tot = g[cu[n] + 64 * w: cu[n] + 64 * c0, h].sum()
            if c0 > 0 and w > 0:
                assert tot < -10.0
                shorter = g[cu[n] + 64 * (w + 1): cu[n] + 64 * c0, h].sum()
                assert not shorter < -10.0
            elif c0 > 0:
                assert not g[cu[n] + 64: cu[n] + 64 * c0, h].sum() < -10.0


def test_truncation_error_bound(oracle_mod):
    """Truncated-history outputs differ from exact ones by at most
    ||q_t|| * exp(sum of g from the window start to t) * ||S_exact(window start)||_2, because each
    token's factor alpha (I - beta k k^T) has spectral norm <= alpha when 0 <= beta ||k||^2 <= 2."""
    inp = make_inputs([64 * 24 + 5], H=2, dk=16, dv=8, dtype="f32", seed=24, h0_scale=1.0)
    cu = inp["cu_seqlens"]
    args = _args(inp)
    o, ht, it = oracle_mod.fwd_chunked(*args, cu, h0=inp["h0"], intermediates=True)
    p = oracle_mod.plan(inp["g"], cu, H=2, P=256, seg_chunks=4)
    ot, htt = oracle_mod.fwd_truncated(*args, cu, p, h0=inp["h0"])
    g = inp["g"].astype(np.float64)
    q = inp["q"].astype(np.float64)
    n_trunc = 0
    for s in range(len(p["seq"])):
        for h in range(2):
            w, c0, c1 = p["warm"][s, h], p["c0"][s], min(p["c1"][s] * 64, cu[1])
            if w == 0:  # window reached the sequence start: exact
                np.testing.assert_allclose(ot[64 * c0:c1, h], o[64 * c0:c1, h], rtol=1e-10,
                                           atol=1e-12)
                continue
            n_trunc += 1
            sw = np.linalg.norm(it["hc"][w, h], 2)
            for t in range(64 * c0, c1):
                decay = np.exp(g[64 * w:t + 1, h].sum())
                assert decay < np.exp(-10.0)
                err = np.linalg.norm(ot[t, h] - o[t, h])
                assert err <= np.linalg.norm(q[t, h]) * decay * sw * (1 + 1e-9) + 1e-15
    assert n_trunc > 0
    assert np.linalg.norm(htt - ht) <= np.exp(-10.0) * np.linalg.norm(ht)


# --------------------------------------------------------------------------- q/k L2 normalisation
def test_l2norm_closed_form(oracle_mod):
    """y = x / sqrt(|x|^2 + eps): same direction, |y|^2 = s / (s + eps); exactly unit for eps = 0;
    a row of zeros stays zero."""
    rng = np.random.default_rng(41)
    x = rng.standard_normal((7, 3, 16)) * rng.uniform(0.01, 5.0, (7, 3, 1))
    x[2, 1] = 0.0
    s = np.sum(x * x, axis=-1)
    for eps in (0.0, 1e-6, 0.3):
        if eps == 0.0:
            x0 = x.copy()
            x0[2, 1] = 1.0  # 0 / 0 is not defined
            y = oracle_mod.l2norm(x0, eps=0.0)
            np.testing.assert_allclose(np.linalg.norm(y, axis=-1), 1.0, rtol=1e-14)
            continue
        y = oracle_mod.l2norm(x, eps=eps)
        np.testing.assert_allclose(np.sum(y * y, axis=-1), s / (s + eps), rtol=1e-13, atol=1e-300)
        cosv = np.sum(x * y, axis=-1) / np.maximum(np.linalg.norm(x, axis=-1) *
                                                   np.linalg.norm(y, axis=-1), 1e-300)
        np.testing.assert_allclose(cosv[s > 0], 1.0, rtol=1e-13)
        assert np.all(y[2, 1] == 0.0)


def test_l2norm_backward_finite_differences(oracle_mod):
    """The normalisation's backward against central differences of <l2norm(x), dy>."""
    rng = np.random.default_rng(42)
    x = rng.standard_normal((4, 2, 6)) * 0.7
    dy = rng.standard_normal(x.shape)
    for eps_n in (1e-6, 0.25):
        dx = oracle_mod.l2norm_bwd(x, dy, eps=eps_n)
        num = np.zeros_like(x)
        h = 1e-6
        for idx in np.ndindex(x.shape):
            xp, xm = x.copy(), x.copy()
            xp[idx] += h
            xm[idx] -= h
            num[idx] = (np.sum(oracle_mod.l2norm(xp, eps=eps_n) * dy)
                        - np.sum(oracle_mod.l2norm(xm, eps=eps_n) * dy)) / (2 * h)
        np.testing.assert_allclose(dx, num, rtol=1e-6, atol=1e-8)


def test_qk_l2norm_forward_is_scale_invariant(oracle_mod):
    """With the normalisation, scaling any (token, head) row of q or k by a positive factor leaves
    o and ht unchanged (up to the eps term); without it, the same scaling changes them."""
    inp = make_inputs([37, 0, 70], H=2, dk=16, dv=16, dtype="f32", seed=43, h0_scale=0.5)
    rng = np.random.default_rng(44)
    args = _args(inp)
    fq = rng.uniform(0.5, 4.0, inp["q"].shape[:2] + (1,))
    fk = rng.uniform(0.5, 4.0, inp["k"].shape[:2] + (1,))
    scaled = [args[0] * fq, args[1] * fk] + args[2:]
    cu = inp["cu_seqlens"]
    o1, h1 = oracle_mod.fwd_recurrent(*args, cu, h0=inp["h0"], qk_l2norm=True)
    o2, h2 = oracle_mod.fwd_recurrent(*scaled, cu, h0=inp["h0"], qk_l2norm=True)
    assert _rel(o2, o1) < 1e-5 and _rel(h2, h1) < 1e-5
    o3, _ = oracle_mod.fwd_recurrent(*scaled, cu, h0=inp["h0"])
    assert _rel(o3, o1) > 0.1
    # and the inputs' own rows are already near unit length, so normalising them changes little
    o0, _ = oracle_mod.fwd_recurrent(*args, cu, h0=inp["h0"])
    assert _rel(o0, o1) < 1e-5


def test_qk_l2norm_backward_matches_finite_differences(oracle_mod):
    """Central differences of L = <o, dO> + <ht, dht> through the normalisation, for q and k
    with rows far from unit length."""
    lens = [6, 9]
    inp = make_inputs(lens, H=2, dk=4, dv=3, dtype="f32", seed=45, h0_scale=0.5)
    cu = inp["cu_seqlens"]
    rng = np.random.default_rng(46)
    args = [x.astype(np.float64) for x in _args(inp)]
    args[0] = args[0] * rng.uniform(0.3, 3.0, args[0].shape[:2] + (1,))
    args[1] = args[1] * rng.uniform(0.3, 3.0, args[1].shape[:2] + (1,))
    h0 = inp["h0"].astype(np.float64)
    dout = rng.standard_normal((15, 2, 3))
    dht = rng.standard_normal((2, 2, 4, 3))
    gr = oracle_mod.bwd(*args, cu, dout, h0=h0, dht=dht, qk_l2norm=True)

    def loss(a):
        o, ht = oracle_mod.fwd_recurrent(*a, cu, h0=h0, qk_l2norm=True)
        return float(np.sum(o * dout) + np.sum(ht * dht))

    h = 1e-6
    for ai, name in ((0, "dq"), (1, "dk"), (3, "dg")):
        num = np.zeros_like(args[ai])
        for idx in np.ndindex(args[ai].shape):
            ap = [a.copy() for a in args]
            am = [a.copy() for a in args]
            ap[ai][idx] += h
            am[ai][idx] -= h
            num[idx] = (loss(ap) - loss(am)) / (2 * h)
        np.testing.assert_allclose(gr[name], num, rtol=1e-6, atol=1e-7, err_msg=name)
