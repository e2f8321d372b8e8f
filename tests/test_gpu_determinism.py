"""Run-to-run determinism under repetition ("How to Speed Up GDN Kernels for Qwen Models",
section "Using it, and the fine print": the kernel is run a thousand times in a loop against a
reference): 1000 launches of the benchmarked forward (32768 tokens, 8 heads, d = 128, bf16,
truncate mode, the bench's launch configuration) and 200 of the exact split are bitwise equal to
the first launch; so are 20 backward calls on the 65536-token training workload.  Every kernel
reduces in a fixed order, so any difference would be a race (gfx950 only; marked ``gpu``)."""
import numpy as np
import pytest

from gdn_inputs import workload
from gpu_util import args_of, to_dev

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")


@pytest.fixture(scope="module")
def gdn():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import linear_attention_recurrence_prefill_amd as m

    m.load_library()
    return m


@pytest.mark.parametrize("mode,runs", [("truncate", 1000), ("exact", 200)])
def test_forward_bitwise_repeatable(gdn, mode, runs):
    inp = workload("long")
    d = to_dev(inp)
    cu_h = inp["cu_seqlens"]
    o1, ht1 = gdn.chunk_fwd(*args_of(d), d["cu_seqlens"], None, mode=mode, num_slots=256,
                            cu_seqlens_host=cu_h)
    o2, ht2 = torch.empty_like(o1), torch.empty_like(ht1)
    bad = torch.zeros((), dtype=torch.int64, device="cuda")
    print(f"[determinism {mode} x{runs}]", flush=True)
    for _ in range(runs):
        gdn.chunk_fwd(*args_of(d), d["cu_seqlens"], None, mode=mode, num_slots=256,
                      cu_seqlens_host=cu_h, out=o2, final_state=ht2)
        bad += (o2 != o1).any().to(torch.int64) + (ht2 != ht1).any().to(torch.int64)
    torch.cuda.synchronize()
    assert int(bad) == 0, f"{int(bad)} differing launches"


def test_backward_bitwise_repeatable(gdn):
    inp = workload("train")
    d = to_dev(inp)
    rng = np.random.default_rng(7)
    dout = torch.from_numpy(rng.standard_normal(inp["v"].shape).astype(np.float32)).cuda()
    dout = dout.to(torch.bfloat16)
    g1 = gdn.chunk_bwd(*args_of(d), d["cu_seqlens"], dout, None)
    print("[determinism backward x20]", flush=True)
    for _ in range(20):
        g2 = gdn.chunk_bwd(*args_of(d), d["cu_seqlens"], dout, None)
        for name in ("dq", "dk", "dv", "dg", "dbeta"):
            assert torch.equal(g1[name], g2[name]), name
