"""The calibration kernels the bench reports the layer against (measurement support, not part of
the layer), through the C ABI: the matrix-core loop returns finite per-wavefront sums and the
flop count of its launch; the copy kernel reproduces its source bit for bit, ragged lengths
included."""
import pytest
import torch

pytestmark = pytest.mark.gpu

moe = pytest.importorskip("top_routing_grouped_router_amd")


@pytest.fixture(scope="module", autouse=True)
def _need_gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    torch.cuda.set_device(0)


def banner(msg):
    print(f"[case] {msg}", flush=True)


@pytest.mark.parametrize("mx", [False, True], ids=["bf16", "mxfp8"])
@pytest.mark.parametrize("iters", [1, 37, 400])
def test_mfma_loop(iters, mx):
    banner(f"mfma loop iters={iters} mx={mx}")
    run = moe.calibrate_mfma_mxfp8 if mx else moe.calibrate_mfma_bf16
    out, flops = run(iters)
    torch.cuda.synchronize()
    waves = out.numel()
    assert waves == torch.cuda.get_device_properties(0).multi_processor_count * 8
    assert flops == waves * iters * 8 * 2 * 32 * 32 * (64 if mx else 16)
    assert torch.isfinite(out).all()
    # the operands are fixed per lane, so every round adds the same products: the sums grow
    # linearly with the rounds (up to fp32 rounding)
    out2, _ = run(2 * iters)
    torch.cuda.synchronize()
    assert torch.allclose(out2, 2 * out, rtol=1e-3, atol=1e-3 * float(out.abs().max()))
    assert float(out.abs().max()) > 0


@pytest.mark.parametrize("nbytes", [16, 4096 + 48, (8 << 20) + 16 * 7, 256 << 20])
def test_copy_bitexact(nbytes):
    banner(f"copy {nbytes} bytes")
    g = torch.Generator(device="cuda").manual_seed(nbytes)
    src = torch.randint(0, 256, (nbytes,), dtype=torch.uint8, device="cuda", generator=g)
    dst = torch.zeros_like(src)
    moe.calibrate_copy(src, dst)
    torch.cuda.synchronize()
    assert torch.equal(src, dst)
