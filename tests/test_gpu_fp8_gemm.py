"""FP8 (E4M3) GEMMs against the oracle: per-token activation and per-tensor weight codes bit-exact,
the scaled product against the oracle's float64 product of the same codes (the kernel adds only its
fp32 accumulation and the bf16 rounding of the output: rel-L2 <= 1e-2, the bf16 bar), and against
the exact product of the original values within the E4M3 bound: each operand carries ~2.4 % RMS
relative rounding, so a dot product of random-sign terms carries ~3.4 %; the bound is one E4M3 unit
roundoff, 2^-4."""
import numpy as np
import pytest
import torch

import wan_inputs as wi
from oracle import quant as OQ
from oracle import wan_oracle as WO
from tests.gpu_util import case, dev, host, rel_l2, require_gpu
from video_diffusion_transformer_step_amd import _lib as L

pytestmark = pytest.mark.gpu

TOL_CODES = 1e-2
TOL_EXACT = 2.0 ** -4


def _rows_quant(xd):
    codes = torch.empty(xd.shape, dtype=torch.uint8, device="cuda")
    scales = torch.empty(xd.shape[0], dtype=torch.float32, device="cuda")
    L.quantize_rows_e4m3(xd, codes, scales)
    return codes, scales


def _tensor_quant(wd):
    codes = torch.empty(wd.shape, dtype=torch.uint8, device="cuda")
    scale = torch.empty(1, dtype=torch.float32, device="cuda")
    ws = torch.empty(256, dtype=torch.uint8, device="cuda")
    L.quantize_tensor_e4m3(wd, codes, scale, ws)
    return codes, scale


@pytest.mark.parametrize("rows,cols", [(300, 1536), (7, 8960), (1, 256)])
def test_quantize_rows_and_tensor_bit_exact(rows, cols):
    require_gpu()
    case(f"e4m3 quantize rows={rows} cols={cols}")
    rng = np.random.default_rng(rows + cols)
    x = wi.bf16_round((rng.standard_normal((rows, cols)) * rng.uniform(0.01, 20, (rows, 1))).astype(np.float32))
    if rows > 2:
        x[2] = 0.0
    codes, scales = _rows_quant(dev(x, torch.bfloat16))
    rc, rs = OQ.quant_rows_e4m3(x)
    assert np.array_equal(codes.cpu().numpy(), rc)
    assert np.array_equal(scales.cpu().numpy().view(np.uint32), rs.view(np.uint32))
    wc, wsc = _tensor_quant(dev(x, torch.bfloat16))
    ec, es = OQ.quant_tensor_e4m3(x)
    assert np.array_equal(wc.cpu().numpy(), ec)
    assert wsc.cpu().numpy().view(np.uint32)[0] == np.float32(es).view(np.uint32)


def _check_gemm(xr, w, bias, act, got):
    """Rows xr of the input and the device result's same rows got against the oracle."""
    xc, xs = OQ.quant_rows_e4m3(xr)  # per-token codes: the sampled rows suffice
    wc, wsc = OQ.quant_tensor_e4m3(w)
    ref_codes = OQ.gemm_e4m3(xc, xs, wc, wsc, bias)
    exact = xr.astype(np.float64) @ w.astype(np.float64).T + bias
    if act == 1:
        ref_codes, exact = WO.gelu(ref_codes), WO.gelu(exact)
    e1, e2 = rel_l2(got, ref_codes), rel_l2(got, exact)
    print(f"[e4m3 gemm] rel-L2 vs codes {e1:.2e}, vs exact {e2:.4f}", flush=True)
    assert e1 <= TOL_CODES, e1
    assert e2 <= TOL_EXACT, e2


@pytest.mark.parametrize("M,N,K,act", [(300, 640, 1536, 0), (257, 260, 768, 1), (1, 256, 256, 0)])
def test_gemm_e4m3_small(M, N, K, act):
    """Every element at sizes with ragged row and column tiles (256 x 256 tiles)."""
    require_gpu()
    case(f"e4m3 gemm M={M} N={N} K={K} act={act}")
    rng = np.random.default_rng(M + N + K)
    x = wi.bf16_round(rng.standard_normal((M, K)).astype(np.float32))
    w = wi.bf16_round((rng.standard_normal((N, K)) * 0.02).astype(np.float32))
    bias = (rng.standard_normal(N) * 0.02).astype(np.float32)
    xc, xs = _rows_quant(dev(x, torch.bfloat16))
    wc, wsc = _tensor_quant(dev(w, torch.bfloat16))
    y = torch.empty((M, N), dtype=torch.bfloat16, device="cuda")
    L.gemm_e4m3(L.pack_weight(xc), xs, L.pack_weight(wc), wsc, y, K, bias=dev(bias), act=act)
    _check_gemm(x, w, bias, act, host(y))


@pytest.mark.parametrize("N,K,act", [(8960, 1536, 1), (1536, 8960, 0)], ids=["ffn1-gelu", "ffn2"])
def test_gemm_e4m3_ffn_shapes(N, K, act):
    """The 1.3B-shaped FFN products at 32760 rows, sampled rows checked."""
    require_gpu()
    M = 32760
    case(f"e4m3 gemm full size M={M} N={N} K={K}")
    g = torch.Generator(device="cuda")
    g.manual_seed(N + K)
    xd = torch.randn((M, K), generator=g, device="cuda").to(torch.bfloat16)
    wd = (torch.randn((N, K), generator=g, device="cuda") * 0.02).to(torch.bfloat16)
    bias = torch.randn(N, generator=g, device="cuda") * 0.02
    xc, xs = _rows_quant(xd)
    wc, wsc = _tensor_quant(wd)
    y = torch.empty((M, N), dtype=torch.bfloat16, device="cuda")
    L.gemm_e4m3(L.pack_weight(xc), xs, L.pack_weight(wc), wsc, y, K, bias=bias, act=act)
    rows = np.unique(np.concatenate([[0, 255, 256, M - 1], np.random.default_rng(5).choice(M, 28, replace=False)]))
    rt = torch.from_numpy(rows).cuda()
    _check_gemm(host(xd[rt]).astype(np.float32), host(wd).astype(np.float32), host(bias), act, host(y[rt]))
