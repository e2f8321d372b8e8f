"""Grouped heads (num_k_heads < num_heads): q and k carry Hk heads and value head h reads key head
h // (H // Hk), the layout "How to Speed Up GDN Kernels for Qwen Models" (section "Using it, and
the fine print") lists, where value heads are a multiple of key heads.  The reference is the
fp64 oracle run on q and k repeated to one copy per value head; the gradients of a key head are
the sums over its value heads (gfx950 only; marked ``gpu``)."""
import numpy as np
import pytest

from gdn_inputs import make_inputs
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


def _grouped(inp, G):
    """Inputs with Hk = H // G key heads: q and k keep every G-th head; the oracle's copy repeats
    each key head G times."""
    gi = dict(inp)
    for x in ("q", "k"):
        gi[x] = np.ascontiguousarray(inp[x][:, ::G])
    ref = dict(gi)
    for x in ("q", "k"):
        ref[x] = np.ascontiguousarray(np.repeat(gi[x], G, axis=1))
    return gi, ref


def _dev(a, dtype):
    t = torch.from_numpy(np.ascontiguousarray(a)).cuda()
    return t.to(dtype) if dtype is not None else t


def _args(gi, tdt):
    return [_dev(gi[x], tdt if x != "g" else None) for x in NAMES]


@pytest.mark.parametrize("dtype,d,G,mode,seg", [
    ("bf16", 128, 2, "exact", 0), ("bf16", 128, 4, "truncate", 2), ("bf16", 128, 2, "exact", 2),
    ("bf16", 64, 2, "exact", 0), ("f32", 128, 4, "exact", 0)])
def test_grouped_forward(gdn, oracle_mod, dtype, d, G, mode, seg):
    inp = make_inputs([300, 65, 0, 700], H=8, dk=d, dv=d, dtype=dtype, seed=401, h0_scale=0.5)
    gi, ref = _grouped(inp, G)
    tdt = torch.bfloat16 if dtype == "bf16" else torch.float32
    o, ht = gdn.chunk_fwd(*_args(gi, tdt), _dev(inp["cu_seqlens"], None), _dev(inp["h0"], None),
                          mode=mode, seg_chunks=seg, num_slots=256, scale=0.5)
    torch.cuda.synchronize()
    if mode == "exact":
        o_ref, ht_ref = oracle_mod.fwd_recurrent(*[ref[x] for x in NAMES], inp["cu_seqlens"],
                                                 h0=inp["h0"], scale=0.5)
    else:
        plan = oracle_mod.plan(inp["g"], inp["cu_seqlens"], 8, P=256, seg_chunks=seg)
        o_ref, ht_ref = oracle_mod.fwd_truncated(*[ref[x] for x in NAMES], inp["cu_seqlens"],
                                                 plan, h0=inp["h0"], scale=0.5)
    print(f"[grouped fwd {dtype} d={d} G={G} {mode} seg={seg}]", flush=True)
    report("o", np64(o), o_ref, tol_for(dtype), cu=inp["cu_seqlens"])
    report("ht", np64(ht), ht_ref, tol_for(dtype), cu=inp["cu_seqlens"], states=True)


def test_grouped_forward_equals_repeated_heads(gdn):
    """The grouped call and an ungrouped call on q, k repeated per value head run the same
    arithmetic on the same values: outputs and final states are bitwise equal."""
    inp = make_inputs([1000, 333], H=8, dk=128, dv=128, dtype="bf16", seed=402)
    gi, ref = _grouped(inp, 4)
    cu = _dev(inp["cu_seqlens"], None)
    for mode in ("exact", "truncate"):
        a = gdn.chunk_fwd(*_args(gi, torch.bfloat16), cu, None, mode=mode)
        b = gdn.chunk_fwd(*_args(ref, torch.bfloat16), cu, None, mode=mode)
        torch.cuda.synchronize()
        assert torch.equal(a[0], b[0]) and torch.equal(a[1], b[1]), mode


@pytest.mark.parametrize("dtype,d,G", [("bf16", 128, 2), ("bf16", 128, 4), ("bf16", 64, 2),
                                     ("f32", 64, 2), ("f32", 128, 4)])
def test_grouped_backward(gdn, oracle_mod, dtype, d, G):
    inp = make_inputs([300, 65, 0, 260], H=4, dk=d, dv=d, dtype=dtype, seed=403, h0_scale=0.5,
                      with_dout=True)
    gi, ref = _grouped(inp, G)
    tdt = torch.bfloat16 if dtype == "bf16" else torch.float32
    gr = gdn.chunk_bwd(*_args(gi, tdt), _dev(inp["cu_seqlens"], None), _dev(inp["dout"], tdt),
                       _dev(inp["h0"], None))
    torch.cuda.synchronize()
    r = oracle_mod.bwd(*[ref[x] for x in NAMES], inp["cu_seqlens"], inp["dout"], h0=inp["h0"])
    T, H = inp["g"].shape
    tol = tol_for(dtype)
    print(f"[grouped bwd {dtype} d={d} G={G}]", flush=True)
    for n in ("dq", "dk"):
        summed = np.asarray(r[n]).reshape(T, H // G, G, d).sum(axis=2)
        assert tuple(gr[n].shape) == (T, H // G, d)
        report(n, np64(gr[n]), summed, tol, cu=inp["cu_seqlens"])
    for n in ("dv", "dg", "dbeta"):
        report(n, np64(gr[n]), r[n], tol, cu=inp["cu_seqlens"])
    report("dh0", np64(gr["dh0"]), r["dh0"], tol, cu=inp["cu_seqlens"], states=True)


@pytest.mark.parametrize("mode", ["truncate", "exact"])
def test_grouped_many_heads_normalised(gdn, oracle_mod, mode):
    """A Qwen-style layer shape: 32 value heads over 4 key heads (groups of 8), q and k
    normalised in the kernels, 8192 tokens in three documents, bf16 d = 128."""
    from gdn_inputs import scale_qk_rows

    G = 8
    inp = scale_qk_rows(make_inputs([4096, 2500, 1596], H=32, dk=128, dv=128, dtype="bf16",
                                    seed=404, h0_scale=0.5), seed=405)
    gi, ref = _grouped(inp, G)
    o, ht = gdn.chunk_fwd(*_args(gi, torch.bfloat16), _dev(inp["cu_seqlens"], None),
                          _dev(inp["h0"], None), mode=mode, num_slots=256,
                          cu_seqlens_host=inp["cu_seqlens"], qk_l2norm=True)
    torch.cuda.synchronize()
    if mode == "exact":
        o_ref, ht_ref = oracle_mod.fwd_recurrent(*[ref[x] for x in NAMES], inp["cu_seqlens"],
                                                 h0=inp["h0"], qk_l2norm=True)
    else:
        plan = oracle_mod.plan(inp["g"], inp["cu_seqlens"], 32, P=256)
        o_ref, ht_ref = oracle_mod.fwd_truncated(*[ref[x] for x in NAMES], inp["cu_seqlens"],
                                                 plan, h0=inp["h0"], qk_l2norm=True)
    print(f"[grouped 32/4 heads, normalised, {mode}]", flush=True)
    report("o", np64(o), o_ref, 5e-3, cu=inp["cu_seqlens"])
    report("ht", np64(ht), ht_ref, 5e-3, cu=inp["cu_seqlens"], states=True)
