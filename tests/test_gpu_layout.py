"""HIP layout kernels and the CFG + Euler kernel against the oracle (bit-exact / <= 1 ulp)."""
import numpy as np
import pytest
import torch

import oracle
from tests.gpu_util import case, dev, host, require_gpu, ulp_diff_f32
from video_diffusion_transformer_step_amd import _lib as L

pytestmark = pytest.mark.gpu

SHAPES = [
    (1, 16, 2, 8, 8),        # tiny image-to-video latent
    (2, 3, 3, 6, 10),        # ragged: 45 tokens per row, odd channel count
    (1, 16, 21, 60, 104),    # 480p x 81 frames latent (32760 tokens)
    (1, 48, 31, 44, 80),     # TI2V-5B-shaped latent (27280 tokens)
]


def _rand(shape, seed):
    return np.random.default_rng(seed).standard_normal(shape).astype(np.float32)


@pytest.mark.parametrize("shape", SHAPES, ids=lambda s: "x".join(map(str, s)))
def test_patchify_bit_exact(shape):
    require_gpu()
    case(f"patchify {shape}")
    x = _rand(shape, 1)
    B, C, T, H, W = shape
    S = T * (H // 2) * (W // 2)
    xd = dev(x)
    p = torch.empty((B, S, 4 * C), dtype=torch.float32, device="cuda")
    L.patchify(xd, p)
    ref = oracle.patchify(x).astype(np.float32)
    got = p.cpu().numpy()
    assert np.array_equal(got.view(np.uint32), ref.view(np.uint32))
    # unpatchify: exact inverse on the GPU
    back = torch.empty_like(xd)
    L.unpatchify(p, back)
    assert np.array_equal(back.cpu().numpy().view(np.uint32), x.view(np.uint32))
    ref_back = oracle.unpatchify(ref.astype(np.float64), C, T, H, W).astype(np.float32)
    assert np.array_equal(ref_back.view(np.uint32), x.view(np.uint32))


@pytest.mark.parametrize("shape,known", [
    ((1, 16, 2, 8, 8), None),
    ((2, 16, 21, 60, 104), None),
    ((1, 48, 31, 44, 80), None),
    ((1, 16, 3, 4, 6), [1, 0, 0, 0, 0, 0, 0, 0, 1]),
    ((2, 5, 4, 2, 4), [0, 1, 0, 0, 0, 1, 0, 0, 0, 1, 1, 0, 1]),
], ids=["tiny", "480p-B2", "ti2v", "first+last", "ragged-multi"])
def test_i2v_input_bit_exact(shape, known):
    require_gpu()
    case(f"i2v_input {shape} known={known}")
    x_t, z = _rand(shape, 2), _rand(shape, 3)
    B, C, T, H, W = shape
    out = torch.empty((B, 2 * C + 4, T, H, W), dtype=torch.float32, device="cuda")
    L.build_i2v_input(dev(x_t), dev(z), out, known)
    ref = oracle.build_i2v_input(x_t, z, known).astype(np.float32)
    assert np.array_equal(out.cpu().numpy().view(np.uint32), ref.view(np.uint32))


@pytest.mark.parametrize("n", [1, 7, 4096 + 3, 16 * 21 * 60 * 104, 48 * 31 * 44 * 80])
@pytest.mark.parametrize("cfg", [False, True])
def test_cfg_euler_within_one_ulp(n, cfg):
    require_gpu()
    case(f"euler n={n} cfg={cfg}")
    x, vc, vu = _rand(n, 4), _rand(n, 5), _rand(n, 6)
    s, dt = np.float32(5.0), np.float32(-0.25)
    xd = dev(x)
    L.fm_euler_step(xd, dev(vc), dev(vu) if cfg else None, float(s), float(dt))
    ref = oracle.cfg_euler(x.astype(np.float64), vc, vu if cfg else None, float(s), float(dt))
    got = xd.cpu().numpy()
    if cfg:
        # v = v_u + s (v_c - v_u) rounds twice in fp32 before the final fma; bound the result by
        # the error of the fp32-rounded v: |dt| * |err(v)| in ulps of x, plus the final rounding.
        v32 = np.float32(vu) + np.float32(s) * (np.float32(vc) - np.float32(vu))
        bound = np.abs(np.float64(dt)) * (np.abs(v32.astype(np.float64) - (vu + 5.0 * (vc.astype(np.float64) - vu)))
                                          + 2 * np.spacing(np.abs(v32)).astype(np.float64))
        err = np.abs(got.astype(np.float64) - ref)
        assert np.all(err <= bound + np.spacing(np.abs(ref).astype(np.float32)).astype(np.float64)), err.max()
    else:
        # a single fma of fp32 operands: the correctly rounded x + dt v, up to fp64 double rounding
        assert ulp_diff_f32(got, ref.astype(np.float32)).max() <= 1


def test_euler_special_cases():
    """s = 0 gives the unconditional velocity, s = 1 the conditional one (bit for bit)."""
    require_gpu()
    case("euler special cases")
    n = 1000
    x, vc, vu = _rand(n, 7), _rand(n, 8), _rand(n, 9)
    a, b = dev(x), dev(x)
    L.fm_euler_step(a, dev(vc), dev(vu), 0.0, -0.1)
    L.fm_euler_step(b, dev(vu), None, 7.0, -0.1)
    assert torch.equal(a, b)
    a, b = dev(x), dev(x)
    L.fm_euler_step(a, dev(vc), dev(vu), 1.0, -0.1)
    L.fm_euler_step(b, dev(vc), None, 1.0, -0.1)
    # fma(1, vc - vu, vu) can differ from vc by the rounding of vc - vu
    assert np.abs(host(a) - host(b)).max() <= 1e-6


def test_fm_straight_line_on_gpu():
    """Exact-velocity Euler steps along the straight path land on the endpoint (fp32)."""
    require_gpu()
    case("straight line")
    x0, x1 = _rand(4096, 10), _rand(4096, 11)
    v = dev(x1 - x0)
    for N in (1, 4, 25):
        xd = dev(x0)
        for _ in range(N):
            L.fm_euler_step(xd, v, None, 1.0, 1.0 / N)
        # fp32 accumulation over N steps: each step rounds once
        assert np.abs(host(xd) - x1.astype(np.float64)).max() <= N * 4e-7 * 8


def _panels_reference(w):
    """The K-panel layout wan.h defines, written out: element (n, k) at ((k / 32) * Np + n) * 32 + k % 32
    with Np = N rounded up to 256 and zero rows past N."""
    N, K = w.shape
    Np = (N + 255) // 256 * 256
    p = np.zeros((K // 32, Np, 32), dtype=w.dtype)
    for j in range(K // 32):
        p[j, :N, :] = w[:, 32 * j:32 * j + 32]
    return p.reshape(-1)


@pytest.mark.parametrize("N,K,dtype", [(260, 96, torch.bfloat16), (1, 32, torch.float32), (512, 256, torch.uint8),
                                       (1536, 8960, torch.bfloat16), (300, 288, torch.uint8)],
                         ids=lambda v: str(v).replace("torch.", ""))
def test_pack_weight_bit_exact(N, K, dtype):
    """wan_pack_weight against the layout definition, bit for bit (ragged rows, all three element sizes,
    the 1.3B block's FFN2 weight)."""
    require_gpu()
    case(f"pack_weight N={N} K={K} {dtype}")
    g = torch.Generator(device="cuda")
    g.manual_seed(N * 7 + K)
    if dtype == torch.uint8:
        w = torch.randint(0, 256, (N, K), generator=g, device="cuda", dtype=torch.int32).to(torch.uint8)
        raw = host(w)
    else:
        w = torch.randn((N, K), generator=g, device="cuda").to(dtype)
        raw = host(w.view(torch.int16 if dtype == torch.bfloat16 else torch.int32))
    got = L.pack_weight(w)
    torch.cuda.synchronize()
    got_raw = host(got if dtype == torch.uint8 else got.view(torch.int16 if dtype == torch.bfloat16 else torch.int32))
    assert got.numel() == L.lib().wan_pack_weight_bytes(w.element_size(), N, K) // w.element_size()
    np.testing.assert_array_equal(got_raw, _panels_reference(raw))
