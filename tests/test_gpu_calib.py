"""The calibration kernels behind bench.py's measured peaks: the stream copy copies every byte
(full spans and a ragged tail), and the MFMA loop writes finite, repeatable sums (gfx950 only;
marked ``gpu``)."""
import pytest

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")


@pytest.fixture(scope="module")
def gdn():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import linear_attention_recurrence_prefill_amd as m

    m.load_library()
    return m


@pytest.mark.parametrize("n16", [1, 1023, 1024, 4096 * 16 + 77, (1 << 22) + 5])
def test_calib_copy_copies_every_byte(gdn, n16):
    print(f"[calib copy {n16} x 16 B]", flush=True)
    src = torch.randint(-2**31, 2**31 - 1, (n16 * 4,), dtype=torch.int32, device="cuda")
    dst = torch.zeros_like(src)
    gdn.calib_copy(src, dst)
    torch.cuda.synchronize()
    assert torch.equal(src, dst)


def test_calib_mfma_finite_and_repeatable(gdn):
    out = torch.empty(8 * 256 * 64, dtype=torch.float32, device="cuda")
    flops = gdn.calib_mfma_bf16(out, 2, 10)
    torch.cuda.synchronize()
    a = out[: 2 * 256 * 64].clone()
    assert flops == 2 * 256 * 10 * 4 * 32768
    assert torch.isfinite(a).all() and (a != 0).any()
    gdn.calib_mfma_bf16(out, 2, 10)
    torch.cuda.synchronize()
    assert torch.equal(a, out[: 2 * 256 * 64])
    # every wave computes the same values
    w = a.view(2 * 256, 64)
    assert torch.equal(w, w[:1].expand_as(w))
