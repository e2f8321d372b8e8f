"""GPU parity of the forward against the fp64 oracle (gfx950 only; marked ``gpu``).

Tolerances: relative L2 <= 1e-4 for fp32 inputs, <= 5e-3 for bf16 inputs (fp32 state), on the
outputs and on the final states.
"""
import numpy as np
import pytest

from gdn_inputs import make_inputs, workload
from gpu_util import args_of, np64, rel_l2, report, to_dev, tol_for

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")


@pytest.fixture(scope="module")
def gdn():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import linear_attention_recurrence_prefill_amd as m

    m.load_library()
    return m


def _oracle_args(inp):
    return [inp[x] for x in ("q", "k", "v", "g", "beta")]


def _check_fwd(gdn, oracle_mod, inp, label, **kw):
    d = to_dev(inp)
    o, ht = gdn.chunk_fwd(*args_of(d), d["cu_seqlens"], d["h0"], **kw)
    torch.cuda.synchronize()
    o_ref, ht_ref = oracle_mod.fwd_recurrent(*_oracle_args(inp), inp["cu_seqlens"], h0=inp["h0"],
                                             scale=kw.get("scale", 1.0))
    tol = tol_for(inp["dtype"])
    print(f"[{label}]", flush=True)
    report("o", np64(o), o_ref, tol, cu=inp["cu_seqlens"])
    report("ht", np64(ht), ht_ref, tol, cu=inp["cu_seqlens"], states=True)
    return o, ht


def test_tiny_fp32(gdn, oracle_mod):
    """1 x 256 tokens, H=2, d=64, fp32."""
    _check_fwd(gdn, oracle_mod, workload("tiny"), "tiny fp32")


@pytest.mark.parametrize("dtype,d", [("f32", 64), ("bf16", 64), ("f32", 128), ("bf16", 128)])
def test_ragged_documents_with_h0(gdn, oracle_mod, dtype, d):
    """Documents of 1, 63, 64, 65, 127, 0 and 200 tokens, nonzero initial states."""
    inp = make_inputs([1, 63, 64, 65, 127, 0, 200], H=3, dk=d, dv=d, dtype=dtype, seed=77,
                      h0_scale=0.5)
    _check_fwd(gdn, oracle_mod, inp, f"ragged {dtype} d={d}")


def test_scale(gdn, oracle_mod):
    inp = make_inputs([300], H=2, dk=128, dv=128, dtype="bf16", seed=78)
    _check_fwd(gdn, oracle_mod, inp, "scale", scale=0.0883883)


def test_packed_8k(gdn, oracle_mod):
    """8192 tokens packed from documents of U{256..2048} tokens, H=8, d=128, bf16."""
    _check_fwd(gdn, oracle_mod, workload("packed"), "packed 8K bf16")


def test_long_32k_exact(gdn, oracle_mod):
    """One 32768-token sequence, H=8, d=128, bf16, exact mode."""
    _check_fwd(gdn, oracle_mod, workload("long"), "long 32K exact")


def test_exact_split_forced_segments(gdn, oracle_mod):
    """Exact mode split into 2-chunk units (bf16, d=128) over ragged documents with nonzero
    initial states, scale 0.7 and weak decay (g ~ -1e-4), so that each unit's transition matrix
    carries the state into the next: the three passes (every unit's affine map, the maps
    composed along each document, every unit rerun from its true start) against the oracle."""
    lengths = [1, 63, 64, 65, 700, 0, 1500, 129]
    inp = make_inputs(lengths, H=3, dk=128, dv=128, dtype="bf16", seed=91, h0_scale=0.5,
                      g_mu=-9.0)
    d = to_dev(inp)
    plan = gdn.chunk_fwd_plan(d["g"], d["cu_seqlens"], 3, 128, torch.bfloat16, mode="exact",
                              seg_chunks=2, cu_seqlens_host=inp["cu_seqlens"])
    assert plan["L"] == 2
    assert len(plan["seq"]) == sum(max(1, ((n + 63) // 64 + 1) // 2) for n in lengths)
    assert np.array_equal(plan["warm"], np.repeat(plan["c0"][:, None], 3, axis=1))
    _check_fwd(gdn, oracle_mod, inp, "exact split L=2", seg_chunks=2, scale=0.7,
               cu_seqlens_host=inp["cu_seqlens"])


def test_exact_split_broadcast_h0_without_host_cu(gdn, oracle_mod):
    """The split with one initial state shared by every document (stride 0) and no host copy
    of cu_seqlens (the unit count is then a bound; the surplus workgroups find no unit)."""
    inp = make_inputs([900, 400, 1300], H=2, dk=128, dv=128, dtype="bf16", seed=92,
                      h0_scale=1.0, n_h0=1, g_mu=-6.0)
    inp["h0"] = inp["h0"][0]  # [H, D, D]: one state for every document
    _check_fwd(gdn, oracle_mod, inp, "exact split broadcast h0", seg_chunks=3)


def test_exact_split_equals_unsplit(gdn, oracle_mod):
    """The same exact forward split (latency model) and unsplit (num_slots = 1: num_seqs * H is
    not below P) agree with each other and with the oracle."""
    inp = make_inputs([2000, 3100], H=4, dk=128, dv=128, dtype="bf16", seed=93, h0_scale=0.5,
                      g_mu=-7.0)
    o_s, ht_s = _check_fwd(gdn, oracle_mod, inp, "exact split (latency model)",
                           cu_seqlens_host=inp["cu_seqlens"])
    o_u, ht_u = _check_fwd(gdn, oracle_mod, inp, "exact unsplit", num_slots=1)
    # two results each within 5e-3 of the oracle are within 1e-2 of each other (their bf16
    # roundings differ: the split rounds the transition's state fragments, not the chain's)
    report("o split vs unsplit", np64(o_s), np64(o_u), 1e-2)
    report("ht split vs unsplit", np64(ht_s), np64(ht_u), 1e-2)


def test_long_32k_truncate(gdn, oracle_mod):
    """The same sequence in truncate mode: the plan equals the oracle's, and the result is within
    tolerance of both the oracle's truncated and exact results."""
    inp = workload("long")
    d = to_dev(inp)
    H = 8
    plan = gdn.chunk_fwd_plan(d["g"], d["cu_seqlens"], H, 128, torch.bfloat16, mode="truncate",
                              num_slots=256, cu_seqlens_host=inp["cu_seqlens"])
    ref_plan = oracle_mod.plan(inp["g"], inp["cu_seqlens"], H, P=256)
    assert plan["L"] == 16
    for key in ("seq", "c0", "c1", "warm"):
        assert np.array_equal(plan[key], ref_plan[key]), key
    o, ht = gdn.chunk_fwd(*args_of(d), d["cu_seqlens"], None, mode="truncate", num_slots=256,
                          cu_seqlens_host=inp["cu_seqlens"])
    torch.cuda.synchronize()
    o_t, ht_t = oracle_mod.fwd_truncated(*_oracle_args(inp), inp["cu_seqlens"], ref_plan)
    o_e, ht_e = oracle_mod.fwd_recurrent(*_oracle_args(inp), inp["cu_seqlens"])
    print("[long 32K truncate]", flush=True)
    print(f"  oracle truncated vs exact: o {rel_l2(o_t, o_e):.2e}  ht {rel_l2(ht_t, ht_e):.2e}")
    cu = inp["cu_seqlens"]
    report("o vs oracle-trunc", np64(o), o_t, 5e-3, cu=cu)
    report("ht vs oracle-trunc", np64(ht), ht_t, 5e-3, cu=cu, states=True)
    report("o vs oracle-exact", np64(o), o_e, 5e-3, cu=cu)
    report("ht vs oracle-exact", np64(ht), ht_e, 5e-3, cu=cu, states=True)


def test_truncate_forced_segments_fp32(gdn, oracle_mod):
    """fp32, forced 4-chunk segments over several documents: GPU follows the oracle's plan."""
    inp = make_inputs([64 * 30 + 7, 64 * 9, 100], H=2, dk=64, dv=64, dtype="f32", seed=79,
                      h0_scale=0.3)
    d = to_dev(inp)
    plan = gdn.chunk_fwd_plan(d["g"], d["cu_seqlens"], 2, 64, torch.float32, mode="truncate",
                              seg_chunks=4, cu_seqlens_host=inp["cu_seqlens"])
    ref_plan = oracle_mod.plan(inp["g"], inp["cu_seqlens"], 2, P=256, seg_chunks=4)
    for key in ("seq", "c0", "c1", "warm"):
        assert np.array_equal(plan[key], ref_plan[key]), key
    o, ht = gdn.chunk_fwd(*args_of(d), d["cu_seqlens"], d["h0"], mode="truncate",
                          seg_chunks=4, cu_seqlens_host=inp["cu_seqlens"])
    o_t, ht_t = oracle_mod.fwd_truncated(*_oracle_args(inp), inp["cu_seqlens"], ref_plan,
                                         h0=inp["h0"])
    cu = inp["cu_seqlens"]
    report("o vs oracle-trunc", np64(o), o_t, 1e-4, cu=cu)
    report("ht vs oracle-trunc", np64(ht), ht_t, 1e-4, cu=cu, states=True)


@pytest.fixture(scope="module")
def fork_case(oracle_mod):
    """The shared-prefix fork workload ("Musings on long-context fine-tuning", section "Sharing
    the repeated work"): a 65536-token prefix, then 80 branches of U{1024..4096} tokens whose
    initial state is the prefix's final state; H=16, d=128, bf16.  With the oracle's prefix
    state (all 16 heads)."""
    w = workload("fork")
    pre = w["prefix"]
    _, ht_pr = oracle_mod.fwd_recurrent(*_oracle_args(pre), pre["cu_seqlens"])
    return w, ht_pr


def test_fork_shared_prefix(gdn, oracle_mod, fork_case):
    """The prefix runs once; its final state, broadcast (stride 0), starts all 80 branches in
    one packed call.  Every head of the prefix's final state and of the branches' outputs and
    final states against the oracle (which starts the branches from its own prefix state)."""
    w, ht_pr = fork_case
    pre, br = w["prefix"], w["branches"]
    dp, db = to_dev(pre), to_dev(br)
    _, ht_p = gdn.chunk_fwd(*args_of(dp), dp["cu_seqlens"], None)
    o_b, ht_b = gdn.chunk_fwd(*args_of(db), db["cu_seqlens"], ht_p[0].contiguous())
    torch.cuda.synchronize()
    o_br, ht_br = oracle_mod.fwd_recurrent(*_oracle_args(br), br["cu_seqlens"], h0=ht_pr[0])
    print("[fork, all 16 heads]", flush=True)
    report("prefix ht", np64(ht_p), ht_pr, 5e-3, cu=pre["cu_seqlens"], states=True)
    report("branch o", np64(o_b), o_br, 5e-3, cu=br["cu_seqlens"])
    report("branch ht", np64(ht_b), ht_br, 5e-3, cu=br["cu_seqlens"], states=True)


def test_fork_backward_full_size(gdn, oracle_mod, fork_case):
    """Backward of the fork workload at full size ("Musings on long-context fine-tuning",
    section "Backward through P"), every head: the branches' backward from the shared prefix
    state gives dh0 summed over the 80 branches; that sum is the prefix's dht, and the prefix's
    backward with its own dO gives the prefix's gradients.  The oracle takes the same two steps
    with its own backward (its per-branch dh0 summed in fp64); that a shared state's gradient is
    the sum over the branches is pinned on the CPU against the oracle's backward of every
    concatenated prefix + branch (test_oracle_pins), and on the GPU at small size
    (test_fork_backward_through_shared_prefix)."""
    from gdn_inputs import bf16_round

    w, ht_pr = fork_case
    pre, br = w["prefix"], w["branches"]
    rng = np.random.Generator(np.random.PCG64(4003))
    dout_p = bf16_round(rng.standard_normal(pre["v"].shape).astype(np.float32))
    dout_b = bf16_round(rng.standard_normal(br["v"].shape).astype(np.float32))
    dp, db = to_dev(pre), to_dev(br)
    _, ht_p = gdn.chunk_fwd(*args_of(dp), dp["cu_seqlens"], None)
    shared = ht_p[0].contiguous()
    gb = gdn.chunk_bwd(*args_of(db), db["cu_seqlens"],
                       torch.from_numpy(dout_b).cuda().to(torch.bfloat16), shared)
    gp = gdn.chunk_bwd(*args_of(dp), dp["cu_seqlens"],
                       torch.from_numpy(dout_p).cuda().to(torch.bfloat16), None,
                       gb["dh0"].unsqueeze(0).contiguous())
    torch.cuda.synchronize()
    rb = oracle_mod.bwd(*_oracle_args(br), br["cu_seqlens"], dout_b, h0=ht_pr[0])
    dht_ref = rb["dh0"].sum(axis=0)
    rp = oracle_mod.bwd(*_oracle_args(pre), pre["cu_seqlens"], dout_p, dht=dht_ref[None])
    print("[fork backward, all 16 heads]", flush=True)
    report("dh0 summed over branches", np64(gb["dh0"]), dht_ref, 5e-3)
    for n in ("dq", "dk", "dv", "dg", "dbeta"):
        report(f"branch {n}", np64(gb[n]), rb[n], 5e-3, cu=br["cu_seqlens"])
    for n in ("dq", "dk", "dv", "dg", "dbeta"):
        report(f"prefix {n}", np64(gp[n]), rp[n], 5e-3, cu=pre["cu_seqlens"])
    report("prefix dh0", np64(gp["dh0"]), rp["dh0"], 5e-3)


def test_broadcast_h0_equals_explicit_copies(gdn):
    inp = make_inputs([100, 64, 300], H=2, dk=128, dv=128, dtype="bf16", seed=80, h0_scale=1.0,
                      n_h0=1)
    d = to_dev(inp)
    shared = d["h0"][0].contiguous()
    o1, ht1 = gdn.chunk_fwd(*args_of(d), d["cu_seqlens"], shared)
    o2, ht2 = gdn.chunk_fwd(*args_of(d), d["cu_seqlens"], shared.expand(3, -1, -1, -1).contiguous())
    assert torch.equal(o1, o2) and torch.equal(ht1, ht2)


def test_boundary_isolation(gdn):
    """Perturbing document A leaves document B bitwise unchanged."""
    inp = make_inputs([200, 150], H=2, dk=128, dv=128, dtype="bf16", seed=81)
    d = to_dev(inp)
    o1, ht1 = gdn.chunk_fwd(*args_of(d), d["cu_seqlens"])
    for name in ("q", "k", "v", "beta"):
        d[name][:200] = d[name][:200].flip(0)
    d["g"][:200] *= 3.0
    o2, ht2 = gdn.chunk_fwd(*args_of(d), d["cu_seqlens"])
    assert torch.equal(o1[200:], o2[200:]) and torch.equal(ht1[1], ht2[1])
    assert not torch.equal(o1[:200], o2[:200])


def test_resume_equals_single_call(gdn):
    """Resuming at a chunk boundary from the first call's final state: bitwise equal to one call
    when every call runs each sequence as one chain (num_slots = 1), and equal up to rounding
    when the exact mode splits the calls differently."""
    inp = make_inputs([640], H=2, dk=128, dv=128, dtype="bf16", seed=82, h0_scale=0.2)
    d = to_dev(inp)
    T1 = 384
    a = [x[:T1].contiguous() for x in args_of(d)]
    b = [x[T1:].contiguous() for x in args_of(d)]
    cu1 = torch.tensor([0, T1], dtype=torch.int32, device="cuda")
    cu2 = torch.tensor([0, 640 - T1], dtype=torch.int32, device="cuda")
    for kw in (dict(num_slots=1), dict()):
        o, ht = gdn.chunk_fwd(*args_of(d), d["cu_seqlens"], d["h0"], **kw)
        oa, ha = gdn.chunk_fwd(*a, cu1, d["h0"], **kw)
        ob, hb = gdn.chunk_fwd(*b, cu2, ha, **kw)
        if kw:
            assert torch.equal(torch.cat([oa, ob]), o) and torch.equal(hb, ht)
        else:
            report("resumed o", np64(torch.cat([oa, ob])), np64(o), 5e-3)
            report("resumed ht", np64(hb), np64(ht), 5e-3)


def test_empty_sequences_keep_h0(gdn):
    inp = make_inputs([0, 70, 0], H=2, dk=64, dv=64, dtype="f32", seed=83, h0_scale=1.0)
    d = to_dev(inp)
    o, ht = gdn.chunk_fwd(*args_of(d), d["cu_seqlens"], d["h0"])
    assert torch.equal(ht[0], d["h0"][0]) and torch.equal(ht[2], d["h0"][2])


def test_deterministic_repeat(gdn):
    """Repeated launches give bitwise identical results (no races in the LDS pipeline)."""
    inp = workload("packed")
    d = to_dev(inp)
    o1, ht1 = gdn.chunk_fwd(*args_of(d), d["cu_seqlens"])
    for _ in range(20):
        o2, ht2 = gdn.chunk_fwd(*args_of(d), d["cu_seqlens"])
        assert torch.equal(o1, o2) and torch.equal(ht1, ht2)


@pytest.mark.parametrize("dtype,d", [("f32", 64), ("bf16", 128)])
def test_intermediates_per_step(gdn, oracle_mod, dtype, d):
    """Each step of the chunked form against the oracle's intermediates: gate cumsum (a1),
    the triangular inverse (a2, a3), W and U (a4), chunk-start states and Delta (a5)."""
    inp = make_inputs([130, 64, 1], H=2, dk=d, dv=d, dtype=dtype, seed=84, h0_scale=0.5)
    dd = to_dev(inp)
    o, ht, it = gdn.chunk_fwd_intermediates(*args_of(dd), dd["cu_seqlens"], dd["h0"])
    torch.cuda.synchronize()
    _, _, ref = oracle_mod.fwd_chunked(*_oracle_args(inp), inp["cu_seqlens"], h0=inp["h0"],
                                       intermediates=True)
    tol = tol_for(dtype)
    print(f"[intermediates {dtype} d={d}]", flush=True)
    report("gamma", np64(it["gamma"]), ref["gamma"], 1e-5)
    report("tmat", np64(it["tmat"]), ref["tm"], 1e-5)
    for name, key in (("w", "w"), ("u", "u"), ("hc", "hc"), ("delta", "delta")):
        report(name, np64(it[name]), ref[key], tol)
