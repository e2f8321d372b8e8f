"""GPU parity of the single-token decode step (gdn_decode_step) against the fp64 oracle's token
recurrence: one step on B states is the recurrence over B one-token sequences started from those
states (gfx950 only; marked ``gpu``).  Tolerances as for the forward: relative L2 <= 1e-4 for
fp32 inputs and <= 5e-3 for bf16 inputs, on o and on the updated state."""
import numpy as np
import pytest

from gdn_inputs import make_inputs
from gpu_util import args_of, np64, report, to_dev, tol_for

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")


@pytest.fixture(scope="module")
def gdn():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import linear_attention_recurrence_prefill_amd as m

    m.load_library()
    return m


@pytest.mark.parametrize("dtype,d", [("f32", 64), ("f32", 128), ("bf16", 64), ("bf16", 128)])
def test_decode_one_step(gdn, oracle_mod, dtype, d):
    B, H = 7, 3
    inp = make_inputs([1] * B, H=H, dk=d, dv=d, dtype=dtype, seed=201, h0_scale=0.5)
    dv = to_dev(inp)
    state = dv["h0"].clone()
    o = gdn.decode_step(*args_of(dv), state, scale=0.7)
    torch.cuda.synchronize()
    o_ref, s_ref = oracle_mod.fwd_recurrent(*[inp[x] for x in ("q", "k", "v", "g", "beta")],
                                            inp["cu_seqlens"], h0=inp["h0"], scale=0.7)
    tol = tol_for(dtype)
    print(f"[decode {dtype} d={d}]", flush=True)
    report("o", np64(o), o_ref, tol)
    report("state", np64(state), s_ref, tol)


def test_decode_steps_equal_recurrence(gdn, oracle_mod):
    """Twenty steps on five bf16 states equal the oracle's recurrence over twenty tokens."""
    B, H, D, S = 5, 2, 128, 20
    inp = make_inputs([S] * B, H=H, dk=D, dv=D, dtype="bf16", seed=202, h0_scale=0.5)
    dv = to_dev(inp)
    state = dv["h0"].clone()
    outs = []
    for s in range(S):
        step = [dv[x].view(B, S, *dv[x].shape[1:])[:, s].contiguous()
                for x in ("q", "k", "v", "g", "beta")]
        outs.append(gdn.decode_step(*step, state))
    torch.cuda.synchronize()
    o = torch.stack(outs, dim=1).reshape(B * S, H, D)
    o_ref, s_ref = oracle_mod.fwd_recurrent(*[inp[x] for x in ("q", "k", "v", "g", "beta")],
                                            inp["cu_seqlens"], h0=inp["h0"])
    print("[decode 20 steps]", flush=True)
    report("o", np64(o), o_ref, 5e-3)
    report("state", np64(state), s_ref, 5e-3)


def test_decode_continues_prefill(gdn, oracle_mod):
    """Prefill of n tokens (chunked forward, exact) then one decode step from its final state
    matches the oracle's recurrence over n + 1 tokens: the last token's output and the state."""
    B, H, D, n = 3, 4, 128, 300
    inp = make_inputs([n + 1] * B, H=H, dk=D, dv=D, dtype="bf16", seed=203)
    dv = to_dev(inp)
    T = B * (n + 1)
    rows = torch.arange(T, device="cuda").view(B, n + 1)
    pre = {x: dv[x][rows[:, :n].reshape(-1)].contiguous() for x in ("q", "k", "v", "g", "beta")}
    cu_pre = torch.arange(0, B * n + 1, n, dtype=torch.int32, device="cuda")
    _, ht = gdn.chunk_fwd(*[pre[x] for x in ("q", "k", "v", "g", "beta")], cu_pre, None)
    last = {x: dv[x][rows[:, n]].contiguous() for x in ("q", "k", "v", "g", "beta")}
    state = ht.contiguous()
    o = gdn.decode_step(*[last[x] for x in ("q", "k", "v", "g", "beta")], state)
    torch.cuda.synchronize()
    o_ref, s_ref = oracle_mod.fwd_recurrent(*[inp[x] for x in ("q", "k", "v", "g", "beta")],
                                            inp["cu_seqlens"])
    last_rows = np.arange(B) * (n + 1) + n
    print("[prefill + decode]", flush=True)
    report("o (last token)", np64(o), o_ref[last_rows], 5e-3)
    report("state", np64(state), s_ref, 5e-3)


def test_decode_rejects_bad_shapes(gdn):
    q = torch.zeros(2, 2, 96, device="cuda", dtype=torch.bfloat16)
    with pytest.raises(ValueError):
        gdn.decode_step(q, q, q, torch.zeros(2, 2, device="cuda"),
                        torch.zeros(2, 2, device="cuda", dtype=torch.bfloat16),
                        torch.zeros(2, 2, 96, 97, device="cuda"))


@pytest.mark.parametrize("dtype,d,G,norm", [("bf16", 128, 4, True), ("bf16", 128, 1, True),
                                            ("bf16", 128, 2, False), ("f32", 64, 2, True)])
def test_decode_grouped_heads_and_l2norm(gdn, oracle_mod, dtype, d, G, norm):
    """Grouped heads (q, k with H / G heads) and the in-kernel q/k L2 normalisation: one step
    against the oracle run on q, k repeated per value head (normalised first when asked)."""
    from gdn_inputs import scale_qk_rows

    B, H = 6, 8
    inp = make_inputs([1] * B, H=H, dk=d, dv=d, dtype=dtype, seed=204, h0_scale=0.5)
    inp = scale_qk_rows(inp, seed=205)
    tdt = torch.bfloat16 if dtype == "bf16" else torch.float32
    qg = np.ascontiguousarray(inp["q"][:, ::G])
    kg = np.ascontiguousarray(inp["k"][:, ::G])
    dev = lambda a, t=None: (torch.from_numpy(np.ascontiguousarray(a)).cuda().to(t)
                             if t is not None else torch.from_numpy(np.ascontiguousarray(a)).cuda())
    state = dev(inp["h0"]).clone()
    o = gdn.decode_step(dev(qg, tdt), dev(kg, tdt), dev(inp["v"], tdt), dev(inp["g"]),
                        dev(inp["beta"], tdt), state, scale=0.7, qk_l2norm=norm)
    torch.cuda.synchronize()
    o_ref, s_ref = oracle_mod.fwd_recurrent(np.repeat(qg, G, axis=1), np.repeat(kg, G, axis=1),
                                            inp["v"], inp["g"], inp["beta"], inp["cu_seqlens"],
                                            h0=inp["h0"], scale=0.7, qk_l2norm=norm)
    tol = tol_for(dtype)
    print(f"[decode {dtype} d={d} G={G} l2norm={norm}]", flush=True)
    report("o", np64(o), o_ref, tol)
    report("state", np64(state), s_ref, tol)


def test_decode_continues_normalised_prefill(gdn, oracle_mod):
    """A prefill with q and k normalised in the kernels, then one normalised decode step, equals
    the oracle's normalised recurrence over n + 1 tokens."""
    from gdn_inputs import scale_qk_rows

    B, H, D, n = 3, 4, 128, 200
    inp = scale_qk_rows(make_inputs([n + 1] * B, H=H, dk=D, dv=D, dtype="bf16", seed=206), 207)
    dv = to_dev(inp)
    T = B * (n + 1)
    rows = torch.arange(T, device="cuda").view(B, n + 1)
    pre = {x: dv[x][rows[:, :n].reshape(-1)].contiguous() for x in ("q", "k", "v", "g", "beta")}
    cu_pre = torch.arange(0, B * n + 1, n, dtype=torch.int32, device="cuda")
    _, ht = gdn.chunk_fwd(*[pre[x] for x in ("q", "k", "v", "g", "beta")], cu_pre, None,
                          qk_l2norm=True)
    last = {x: dv[x][rows[:, n]].contiguous() for x in ("q", "k", "v", "g", "beta")}
    state = ht.contiguous()
    o = gdn.decode_step(*[last[x] for x in ("q", "k", "v", "g", "beta")], state, qk_l2norm=True)
    torch.cuda.synchronize()
    o_ref, s_ref = oracle_mod.fwd_recurrent(*[inp[x] for x in ("q", "k", "v", "g", "beta")],
                                            inp["cu_seqlens"], qk_l2norm=True)
    last_rows = np.arange(B) * (n + 1) + n
    print("[normalised prefill + decode]", flush=True)
    report("o (last token)", np64(o), o_ref[last_rows], 5e-3)
    report("state", np64(state), s_ref, 5e-3)
