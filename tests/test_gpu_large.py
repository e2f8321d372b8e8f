"""A large batch in the range of the pages' training runs ("How to Speed Up GDN Kernels for Qwen
Models", section "What it adds up to": backward at 16K-256K total tokens with 32 heads): 131072
tokens packed from documents of U{4096..16384} tokens, 32 heads, d = 128, bf16; forward in both
modes and the backward.  The inputs are drawn on the GPU (seeded; the recipe of gdn_inputs.py) and
the oracle checks three of the 32 heads on every document (a sample: the oracle's cost grows with
the heads it runs; every head of the five workloads of record is compared in the other tests)."""
import numpy as np
import pytest

from gdn_inputs import lengths_until
from gpu_util import np64, report

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")

HEADS = [0, 17, 31]


@pytest.fixture(scope="module")
def gdn():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import linear_attention_recurrence_prefill_amd as m

    m.load_library()
    return m


@pytest.fixture(scope="module")
def large():
    rng = np.random.Generator(np.random.PCG64(5005))
    lengths = lengths_until(rng, 4096, 16384, 131072)
    T, H, D = sum(lengths), 32, 128
    gen = torch.Generator(device="cuda").manual_seed(5006)
    q = torch.nn.functional.normalize(torch.randn(T, H, D, device="cuda", generator=gen), dim=-1)
    k = torch.nn.functional.normalize(torch.randn(T, H, D, device="cuda", generator=gen), dim=-1)
    d = dict(q=q.to(torch.bfloat16), k=k.to(torch.bfloat16),
             v=torch.randn(T, H, D, device="cuda", generator=gen).to(torch.bfloat16),
             g=-torch.nn.functional.softplus(torch.randn(T, H, device="cuda", generator=gen) - 3.0),
             beta=torch.sigmoid(torch.randn(T, H, device="cuda", generator=gen)).to(torch.bfloat16),
             dout=torch.randn(T, H, D, device="cuda", generator=gen).to(torch.bfloat16))
    d["g"] = d["g"].contiguous()
    del q, k
    cu = np.concatenate([[0], np.cumsum(lengths)]).astype(np.int32)
    d["cu"] = torch.from_numpy(cu).cuda()
    # the sampled heads on the host, exactly the device's bf16 values
    host = {n: np.ascontiguousarray(d[n][:, HEADS].float().cpu().numpy()) for n in
            ("q", "k", "v", "g", "beta", "dout")}
    return d, host, cu


def _args(d):
    return [d[x] for x in ("q", "k", "v", "g", "beta")]


def _oargs(host):
    return [host[x] for x in ("q", "k", "v", "g", "beta")]


def test_large_forward_both_modes(gdn, oracle_mod, large):
    d, host, cu = large
    o_ref, ht_ref = oracle_mod.fwd_recurrent(*_oargs(host), cu)
    for mode in ("exact", "truncate"):
        o, ht = gdn.chunk_fwd(*_args(d), d["cu"], None, mode=mode, cu_seqlens_host=cu)
        torch.cuda.synchronize()
        print(f"[131072 tokens x 32 heads, {mode}; heads {HEADS}]", flush=True)
        assert bool(torch.isfinite(o).all())
        report("o", np64(o[:, HEADS]), o_ref, 5e-3, cu=cu)
        report("ht", np64(ht[:, HEADS]), ht_ref, 5e-3, cu=cu, states=True)
        del o, ht


def test_large_backward(gdn, oracle_mod, large):
    d, host, cu = large
    gr = gdn.chunk_bwd(*_args(d), d["cu"], d["dout"], cu_seqlens_host=cu)
    torch.cuda.synchronize()
    ref = oracle_mod.bwd(*_oargs(host), cu, host["dout"])
    print(f"[131072 tokens x 32 heads, backward; heads {HEADS}]", flush=True)
    for n in ("dq", "dk", "dv", "dg", "dbeta"):
        assert bool(torch.isfinite(gr[n]).all()), n
        report(n, np64(gr[n][:, HEADS]), ref[n], 5e-3, cu=cu)
    report("dh0", np64(gr["dh0"][:, HEADS]), ref["dh0"], 5e-3, cu=cu, states=True)
