"""GPU parity of the backward against the fp64 oracle's hand-derived token backward
(gfx950 only; marked ``gpu``).  Tolerances as for the forward: relative L2 <= 1e-4 for fp32
inputs and <= 5e-3 for bf16 inputs, per gradient."""
import numpy as np
import pytest

from gdn_inputs import make_inputs, workload
from gpu_util import args_of, np64, report, to_dev, tol_for

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")

NAMES = ("dq", "dk", "dv", "dg", "dbeta")


@pytest.fixture(scope="module")
def gdn():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import linear_attention_recurrence_prefill_amd as m

    m.load_library()
    return m


def _oargs(inp, heads=None):
    out = []
    for x in ("q", "k", "v", "g", "beta"):
        a = inp[x]
        out.append(np.ascontiguousarray(a[:, heads]) if heads is not None else a)
    return out


def _check_bwd(gdn, oracle_mod, inp, label, dht_scale=0.0, scale=1.0, heads=None, **kw):
    d = to_dev(inp)
    rng = np.random.default_rng(123)
    dout = inp.get("dout")
    if dout is None:
        dout = rng.standard_normal(inp["v"].shape).astype(np.float32)
        if inp["dtype"] == "bf16":
            from gdn_inputs import bf16_round
            dout = bf16_round(dout)
    tdt = torch.bfloat16 if inp["dtype"] == "bf16" else torch.float32
    dout_d = torch.from_numpy(np.ascontiguousarray(dout)).cuda().to(tdt)
    N = len(inp["cu_seqlens"]) - 1
    T, H, D = inp["q"].shape
    dht = None
    dht_d = None
    if dht_scale:
        dht = (dht_scale * rng.standard_normal((N, H, D, D))).astype(np.float32)
        dht_d = torch.from_numpy(dht).cuda()
    gr = gdn.chunk_bwd(*args_of(d), d["cu_seqlens"], dout_d, d["h0"], dht_d, scale=scale, **kw)
    torch.cuda.synchronize()
    sel = heads if heads is not None else slice(None)
    h0 = inp["h0"]
    ref = oracle_mod.bwd(*_oargs(inp, heads), inp["cu_seqlens"],
                         np.ascontiguousarray(dout[:, sel]),
                         h0=None if h0 is None else np.ascontiguousarray(h0[:, sel]),
                         dht=None if dht is None else np.ascontiguousarray(dht[:, sel]),
                         scale=scale)
    tol = tol_for(inp["dtype"])
    print(f"[{label}]", flush=True)
    cu = inp["cu_seqlens"]
    for name in NAMES:
        report(name, np64(gr[name])[:, sel], ref[name], tol, cu=cu)
    if gr["dh0"] is not None:
        report("dh0", np64(gr["dh0"])[:, sel], ref["dh0"], tol, cu=cu, states=True)
    return gr, ref


@pytest.mark.parametrize("dtype,d", [("f32", 64), ("f32", 128), ("bf16", 64), ("bf16", 128)])
def test_bwd_ragged_with_h0_and_dht(gdn, oracle_mod, dtype, d):
    inp = make_inputs([1, 63, 64, 65, 130, 0, 200], H=2, dk=d, dv=d, dtype=dtype, seed=91,
                      h0_scale=0.5)
    _check_bwd(gdn, oracle_mod, inp, f"bwd ragged {dtype} d={d}", dht_scale=0.3)


def test_bwd_tiny_fp32(gdn, oracle_mod):
    inp = workload("tiny")
    _check_bwd(gdn, oracle_mod, inp, "bwd tiny fp32")


def test_bwd_scale(gdn, oracle_mod):
    inp = make_inputs([257], H=2, dk=128, dv=128, dtype="bf16", seed=92)
    _check_bwd(gdn, oracle_mod, inp, "bwd scale", scale=0.0883883)


@pytest.fixture(scope="module")
def train65k(oracle_mod):
    """The training workload on the GPU and the oracle's gradients for all 8 heads (computed once
    for the tests below)."""
    inp = workload("train")
    ref = oracle_mod.bwd(*_oargs(inp), inp["cu_seqlens"], inp["dout"])
    return inp, ref


def _report_train(gr, inp, ref, label):
    print(f"[{label}]", flush=True)
    cu = inp["cu_seqlens"]
    for name in NAMES:
        report(name, np64(gr[name]), ref[name], 5e-3, cu=cu)
    report("dh0", np64(gr["dh0"]), ref["dh0"], 5e-3, cu=cu, states=True)


def test_train_65k_forward_and_backward(gdn, oracle_mod, train65k):
    """The training workload: 65536 tokens packed from documents of U{4096..16384} tokens, H=8,
    d=128, bf16, dO ~ N(0, 1) ("How to Speed Up GDN Kernels for Qwen Models", section "What it
    adds up to": the backward at 16K-256K tokens).  The forward's o and final states, then every
    gradient, on all 8 heads, per (document, head) and per 4096-token block.  Both calls get the
    host copy of cu_seqlens, as the benchmark's do: the exact split then takes the shortest
    segment length (not below the latency model's 16) whose last pass fits one round of 256
    workgroups, 35 chunks for these documents."""
    inp, ref = train65k
    d = to_dev(inp)
    cu_h = inp["cu_seqlens"]
    plan = gdn.chunk_fwd_plan(d["g"], d["cu_seqlens"], 8, 128, torch.bfloat16, mode="exact",
                              num_slots=256, cu_seqlens_host=cu_h)
    chunks = (np.diff(cu_h) + 63) // 64
    assert plan["L"] == 35 and len(plan["seq"]) == int(((chunks + 34) // 35).sum()) <= 32
    o, ht = gdn.chunk_fwd(*args_of(d), d["cu_seqlens"], None, num_slots=256, cu_seqlens_host=cu_h)
    torch.cuda.synchronize()
    o_ref, ht_ref = oracle_mod.fwd_recurrent(*_oargs(inp), inp["cu_seqlens"])
    print("[train 65K forward]", flush=True)
    report("o", np64(o), o_ref, 5e-3, cu=inp["cu_seqlens"])
    report("ht", np64(ht), ht_ref, 5e-3, cu=inp["cu_seqlens"], states=True)
    del o, ht, o_ref, ht_ref
    gr = gdn.chunk_bwd(*args_of(d), d["cu_seqlens"], d["dout"], num_slots=256,
                       cu_seqlens_host=cu_h)
    torch.cuda.synchronize()
    _report_train(gr, inp, ref, "bwd train 65K, all 8 heads")


def test_train_65k_backward_truncate(gdn, train65k):
    """The truncate mode's backward on the training workload (warmup windows of e^-10 on both
    passes instead of the exact split's extra passes), against the oracle's exact gradients on all
    8 heads: the dropped terms are below the bf16 tolerance."""
    inp, ref = train65k
    d = to_dev(inp)
    gr = gdn.chunk_bwd(*args_of(d), d["cu_seqlens"], d["dout"], num_slots=256,
                       cu_seqlens_host=inp["cu_seqlens"], mode="truncate")
    torch.cuda.synchronize()
    _report_train(gr, inp, ref, "bwd train 65K truncate, all 8 heads")


def test_bwd_shared_initial_state_sums_branches(gdn, oracle_mod):
    """One initial state shared by every sequence (stride 0): dh0 is the sum over sequences of
    their per-sequence gradients ("Backward through P")."""
    inp = make_inputs([300, 77, 129], H=2, dk=128, dv=128, dtype="bf16", seed=93, h0_scale=0.5,
                      n_h0=1)
    d = to_dev(inp)
    rng = np.random.default_rng(7)
    from gdn_inputs import bf16_round
    dout = bf16_round(rng.standard_normal(inp["v"].shape).astype(np.float32))
    dout_d = torch.from_numpy(dout).cuda().to(torch.bfloat16)
    shared = d["h0"][0].contiguous()
    gr = gdn.chunk_bwd(*args_of(d), d["cu_seqlens"], dout_d, shared)
    torch.cuda.synchronize()
    assert tuple(gr["dh0"].shape) == (2, 128, 128)
    ref = oracle_mod.bwd(*_oargs(inp), inp["cu_seqlens"], dout, h0=inp["h0"][0])
    report("dh0 (summed)", np64(gr["dh0"]), ref["dh0"].sum(axis=0), 5e-3)
    for name in NAMES:
        report(name, np64(gr[name]), ref[name], 5e-3, cu=inp["cu_seqlens"])


def test_bwd_deterministic(gdn):
    inp = make_inputs([500, 200], H=2, dk=128, dv=128, dtype="bf16", seed=94, h0_scale=0.3,
                      with_dout=True)
    d = to_dev(inp)
    g1 = gdn.chunk_bwd(*args_of(d), d["cu_seqlens"], d["dout"], d["h0"])
    for _ in range(5):
        g2 = gdn.chunk_bwd(*args_of(d), d["cu_seqlens"], d["dout"], d["h0"])
        for name in NAMES + ("dh0",):
            assert torch.equal(g1[name], g2[name]), name


@pytest.mark.parametrize("seg,slots,mode", [(2, 0, "exact"), (0, 1, "exact"), (2, 0, "truncate")])
def test_bwd_recompute_split_and_unsplit(gdn, oracle_mod, seg, slots, mode):
    """The backward split into 2-chunk segments (several units per sequence, h0 and a nonzero
    dht), through the exact split or with the truncate mode's warmup windows (about three chunks
    here, so windows that stop inside a sequence and windows that reach its start or end), and
    run unsplit (one workgroup slot: num_seqs * H >= P): all match the oracle."""
    inp = make_inputs([700, 333, 0, 1000, 64], H=2, dk=128, dv=128, dtype="bf16", seed=95,
                      h0_scale=0.5)
    d = to_dev(inp)
    rng = np.random.default_rng(11)
    from gdn_inputs import bf16_round
    dout = bf16_round(rng.standard_normal(inp["v"].shape).astype(np.float32))
    N, H, D = 5, 2, 128
    dht = (0.3 * rng.standard_normal((N, H, D, D))).astype(np.float32)
    gr = gdn.chunk_bwd(*args_of(d), d["cu_seqlens"], torch.from_numpy(dout).cuda().to(torch.bfloat16),
                       d["h0"], torch.from_numpy(dht).cuda(), seg_chunks=seg, num_slots=slots,
                       mode=mode)
    torch.cuda.synchronize()
    ref = oracle_mod.bwd(*_oargs(inp), inp["cu_seqlens"], dout, h0=inp["h0"], dht=dht)
    print(f"[bwd recompute seg={seg} slots={slots} {mode}]", flush=True)
    for name in NAMES:
        report(name, np64(gr[name]), ref[name], 5e-3, cu=inp["cu_seqlens"])
    report("dh0", np64(gr["dh0"]), ref["dh0"], 5e-3, cu=inp["cu_seqlens"], states=True)


def test_bwd_truncate_unbounded_windows_equal_unsplit(gdn):
    """With a threshold no window reaches, every unit's recompute starts at its sequence's start
    (from h0) and its reverse chain at the sequence's end (from dht): each unit then repeats the
    unsplit backward's arithmetic on its chunks, so the gradients are bitwise those of the exact
    backward run unsplit."""
    inp = make_inputs([700, 333, 0, 1000, 64], H=2, dk=128, dv=128, dtype="bf16", seed=96,
                      h0_scale=0.5, with_dout=True)
    d = to_dev(inp)
    rng = np.random.default_rng(12)
    dht = torch.from_numpy((0.3 * rng.standard_normal((5, 2, 128, 128))).astype(np.float32)).cuda()
    a = gdn.chunk_bwd(*args_of(d), d["cu_seqlens"], d["dout"], d["h0"], dht, num_slots=1)
    b = gdn.chunk_bwd(*args_of(d), d["cu_seqlens"], d["dout"], d["h0"], dht, seg_chunks=2,
                      num_slots=0, mode="truncate", trunc_log_threshold=-1e30)
    torch.cuda.synchronize()
    for name in NAMES + ("dh0",):
        assert torch.equal(a[name], b[name]), name


def test_fork_backward_through_shared_prefix(gdn, oracle_mod):
    """Shared-prefix fork, backward ("Musings on long-context fine-tuning", section "Backward
    through P"): a prefix runs once and its final state starts every branch.  On the GPU the
    branches' backward with that shared initial state gives dh0 summed over the branches; it is
    the prefix's dht, and the prefix's backward with its own dO and that dht gives the prefix's
    gradients.  Reference: the oracle's backward of each concatenated prefix + branch with dO zero
    on the prefix, summed over the branches on the prefix's tokens, plus the oracle's backward of
    the prefix alone with its own dO; the branch tokens' gradients come from the same
    concatenations."""
    P, lens, H, D = 300, [150, 97, 220], 2, 128
    pre = make_inputs([P], H=H, dk=D, dv=D, dtype="bf16", seed=301, with_dout=True)
    br = make_inputs(lens, H=H, dk=D, dv=D, dtype="bf16", seed=302, with_dout=True)
    dp, db = to_dev(pre), to_dev(br)
    _, ht = gdn.chunk_fwd(*args_of(dp), dp["cu_seqlens"], None)
    shared = ht[0].contiguous()
    gb = gdn.chunk_bwd(*args_of(db), db["cu_seqlens"], db["dout"], shared)
    gp = gdn.chunk_bwd(*args_of(dp), dp["cu_seqlens"], dp["dout"], None,
                       gb["dh0"].unsqueeze(0).contiguous())
    torch.cuda.synchronize()

    names = ("q", "k", "v", "g", "beta")
    ref_p = oracle_mod.bwd(*[pre[x] for x in names], pre["cu_seqlens"], pre["dout"])
    ref_b = {n: np.zeros(br[n[1:]].shape) for n in NAMES}  # dq -> q's shape, ...
    ref_p = {n: np.array(ref_p[n], dtype=np.float64) for n in NAMES}
    cu = br["cu_seqlens"]
    for i in range(len(lens)):
        s0, s1 = int(cu[i]), int(cu[i + 1])
        cat = [np.concatenate([pre[x], br[x][s0:s1]]) for x in names]
        dout = np.concatenate([np.zeros_like(pre["dout"]), br["dout"][s0:s1]])
        r = oracle_mod.bwd(*cat, np.array([0, P + s1 - s0], dtype=np.int32), dout)
        for n in NAMES:
            ref_p[n] += r[n][:P]
            ref_b[n][s0:s1] = r[n][P:]
    print("[fork backward]", flush=True)
    for n in NAMES:
        report(f"prefix {n}", np64(gp[n]), ref_p[n], 5e-3, cu=pre["cu_seqlens"])
    for n in NAMES:
        report(f"branch {n}", np64(gb[n]), ref_b[n], 5e-3, cu=br["cu_seqlens"])
