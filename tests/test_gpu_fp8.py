"""GPU parity of the FP8 (E4M3) path: zg_quantize_fp8 codes bit for bit
against the oracle's quantizer (the decision is taken in fp32 on both
sides), and zg_linear_fp8 against the oracle's fp64 product of the decoded
operands, at the bf16 output bar (the E4M3 products are exact in fp32; only
the fp32 accumulation and the final bf16 rounding differ).  The error of
FP8 against the unquantized bf16 product is measured and bounded loosely:
it is the format's, not the kernel's."""

import sys

import numpy as np
import pytest

from global_attention_zg_amd import inputs
from oracle import zg_oracle as orc
from tests import zg_cases as zc

pytestmark = pytest.mark.gpu

torch = pytest.importorskip("torch")


@pytest.fixture(autouse=True)
def _gpu(request):
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    print(f"\n[case] {request.node.nodeid}", file=sys.stderr, flush=True)
    yield
    torch.cuda.synchronize()


def _binding():
    from global_attention_zg_amd import binding
    return binding


def test_quantize_codes_bit_exact():
    bd = _binding()
    rng = np.random.default_rng(700)
    n = 1 << 16
    x = (rng.standard_normal(n) * np.exp2(rng.uniform(-14, 10, n))).astype(np.float32)
    x[:16] = [0.0, -0.0, 1.0625, 1.1875, 464.0, 1e6, -1e6, 2.0**-10, 1.5 * 2.0**-9, 448.0,
              -448.0, 2.0**-6, 2.0**-9, 3.0e-5, -3.0e-5, 0.5]
    bits = (x.view(np.uint32) >> 16).astype(np.uint16)  # truncate to bf16: exact inputs
    xb = orc.bf16_bits_to_f64(bits).astype(np.float32)
    for scale in (1.0, 3.7, 2.0**-5):
        got = bd.zg_quantize_fp8(zc.to_dev(bits, torch), scale).cpu().numpy()
        want, _ = orc.quantize_e4m3(xb, scale)
        bad = np.nonzero(got != want)[0]
        assert bad.size == 0, (scale, bad[:5], got[bad[:5]], want[bad[:5]], xb[bad[:5]])


def fp8_case(tag, M, N, K):
    x = zc.bits((tag, 0, inputs.T_X), (M, K))
    w = inputs.scaled_normal_bf16_bits((tag, 0, inputs.T_W), N * K, K ** -0.5).reshape(N, K)
    return x, w


# per-tensor scales: the values' largest magnitudes land near 2^8 (x ~ N(0,1),
# w ~ N(0, 1/K))
def scales(K):
    return 32.0, 32.0 * np.sqrt(K)


@pytest.mark.parametrize("M,N,K", [(1, 256, 128), (300, 512, 256), (1000, 1024, 4096),
                                   (2048, 4096, 4096)])
def test_linear_fp8_matches_oracle(M, N, K):
    bd = _binding()
    x, w = fp8_case(710 + M, M, N, K)
    sx, sw = scales(K)
    xq = bd.zg_quantize_fp8(zc.to_dev(x, torch), sx)
    wq = bd.zg_quantize_fp8(zc.to_dev(w, torch), sw)
    y = bd.zg_linear_fp8(xq, wq, 1.0 / (sx * sw))
    torch.cuda.synchronize()
    _, xv = orc.quantize_e4m3(zc.f64(x).astype(np.float32), sx)
    _, wv = orc.quantize_e4m3(zc.f64(w).astype(np.float32), sw)
    ref = orc.linear(xv, wv) / (sx * sw)
    got = y.float().cpu().numpy().astype(np.float64)
    zc.compare(got, ref, f"fp8 {M}x{N}x{K}")
    # the format's own error against the unquantized product (not a parity bar)
    exact = orc.linear(zc.f64(x), zc.f64(w))
    rel = float(np.sqrt(np.sum((got - exact) ** 2) / np.sum(exact ** 2)))
    print(f"fp8 {M}x{N}x{K}: rel-RMS vs unquantized {rel:.4f}", file=sys.stderr)
    assert rel < 0.1


def test_linear_fp8_deterministic_and_rows():
    bd = _binding()
    M, N, K = 300, 256, 512
    x, w = fp8_case(720, M, N, K)
    xq = bd.zg_quantize_fp8(zc.to_dev(x, torch), 32.0)
    wq = bd.zg_quantize_fp8(zc.to_dev(w, torch), 512.0)
    big = torch.full((M + 40, N), float("nan"), dtype=torch.bfloat16, device="cuda")
    bd.zg_linear_fp8(xq, wq, 1.0 / (32.0 * 512.0), out=big[:M])
    y2 = bd.zg_linear_fp8(xq, wq, 1.0 / (32.0 * 512.0))
    torch.cuda.synchronize()
    assert torch.isnan(big[M:]).all()
    assert torch.equal(big[:M].view(torch.int16), y2.view(torch.int16))
