"""Single HIP entry points against the oracle: attention (with 3D RoPE), patch embedding,
timestep embedding, context MLP, cross-attention K/V and head."""
import numpy as np
import pytest
import torch

import oracle
import wan_inputs as wi
from tests.gpu_util import case, dev, host, rel_l2, require_gpu
from video_diffusion_transformer_step_amd import _lib as L
from video_diffusion_transformer_step_amd import runtime as R

pytestmark = pytest.mark.gpu

TOL = {"f32": 1e-4, "bf16": 1e-2}


def _tdt(dtype):
    return torch.bfloat16 if dtype == "bf16" else torch.float32


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
@pytest.mark.parametrize("hd", [64, 128])
@pytest.mark.parametrize("grid,B,H", [((3, 6, 10), 1, 2), ((2, 4, 4), 2, 3), ((1, 1, 1), 1, 1),
                                      ((5, 7, 9), 1, 2)],
                         ids=["180tok", "32tok-B2", "1tok", "315tok"])
def test_attention_rope_small(dtype, hd, grid, B, H):
    """Full attention with RoPE at sizes spanning several 64-key tiles and 128-query tiles with
    ragged tails, every output element compared."""
    require_gpu()
    case(f"attention dtype={dtype} hd={hd} grid={grid} B={B} H={H}")
    S = grid[0] * grid[1] * grid[2]
    rng = np.random.default_rng(hd + S)
    q, k, v = (rng.standard_normal((B, S, H, hd)).astype(np.float32) for _ in range(3))
    if dtype == "bf16":
        q, k, v = wi.bf16_round(q), wi.bf16_round(k), wi.bf16_round(v)
    td = _tdt(dtype)
    qd, kd, vd = dev(q, td), dev(k, td), dev(v, td)
    o = torch.empty_like(qd)
    ws = torch.empty(L.attention_ws_bytes(L.dtype_code(td), grid, B, H, hd), dtype=torch.uint8, device="cuda")
    L.attention_fwd(qd, kd, vd, grid, o, ws)
    got = host(o)
    for b in range(B):
        ref = oracle.self_attention_rope_only(q[b], k[b], v[b], grid)
        assert rel_l2(got[b], ref) <= TOL[dtype] * (0.1 if dtype == "f32" else 1.0), rel_l2(got[b], ref)


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_patch_embed(dtype):
    require_gpu()
    c = wi.get_config("tiny").replace(dtype=dtype)
    case(f"patch_embed {dtype}")
    mw = wi.make_model_weights(c, seed=1)
    x_t, z = wi.make_latents(c, seed=1)
    x_in = oracle.build_i2v_input(x_t, z)
    p = oracle.patchify(x_in).astype(np.float32)
    cfg = R.cfg_of(c)
    out = torch.empty((1, c.S, c.dim), dtype=torch.float32, device="cuda")
    ws = torch.empty(max(L.patch_embed_ws_bytes(cfg, c.S, c.in_channels), 16), dtype=torch.uint8, device="cuda")
    L.patch_embed(cfg, dev(p), c.in_channels, dev(mw["w_pe"], _tdt(dtype)), dev(mw["b_pe"]), out, ws)
    ref = oracle.patch_embed(p, mw["w_pe"], mw["b_pe"])
    # bf16 mode rounds the patch vectors to bf16 before the product
    assert rel_l2(host(out), ref) <= TOL[dtype]


@pytest.mark.timeout(600)
@pytest.mark.parametrize("name", ["t2v-1.3b", "i2v-14b", "ti2v-5b"])
def test_patch_embed_full_size(name):
    """The patch embedding at the workloads' real shapes ("图解 Wan2.1 I2V" §5.1): K = 4 C_in = 64 / 144 / 400
    channels per patch vector, N = dim = 1536 / 5120 / 3072, M = B S = 32760 / 65520 / 54560 rows, the
    shapes that take the 256-row tiles with a partial last K step.  Patch vectors ~N(0,1) fp32 (rounded to
    bf16 inside, like the weights); sampled rows against the oracle's exact product."""
    require_gpu()
    c = wi.get_config(name)
    K, M = 4 * c.in_channels, c.B * c.S
    case(f"patch_embed full size {name}: M={M} K={K} N={c.dim}")
    mw = wi.make_model_weights(c, seed=8)
    p = wi.normal(8, c, "x_block", (M, K), quantize=False)
    cfg = R.cfg_of(c)
    out = torch.empty((M, c.dim), dtype=torch.float32, device="cuda")
    ws = torch.empty(max(L.patch_embed_ws_bytes(cfg, M, c.in_channels), 16), dtype=torch.uint8, device="cuda")
    L.patch_embed(cfg, dev(p), c.in_channels, dev(mw["w_pe"], torch.bfloat16), dev(mw["b_pe"]), out, ws)
    got = host(out)
    rows = np.unique(np.concatenate([wi.sample_rows(c.replace(B=1, T=c.T * c.B), 200, seed=8), [M - 1]]))
    ref = oracle.patch_embed(p[rows], mw["w_pe"], mw["b_pe"])
    e = rel_l2(got[rows], ref)
    print(f"[patch_embed {name}] rel-L2 {e:.3e} on {len(rows)} rows", flush=True)
    assert np.isfinite(got).all()
    assert e <= TOL["bf16"]


@pytest.mark.parametrize("cfg_name,dtype", [("tiny", "f32"), ("tiny", "bf16"), ("t2v-1.3b", "bf16"), ("ti2v-5b", "bf16")])
def test_time_embed(cfg_name, dtype):
    require_gpu()
    c = wi.get_config(cfg_name).replace(dtype=dtype)
    case(f"time_embed {cfg_name} {dtype}")
    mw = wi.make_model_weights(c, seed=2)
    model = R.DeviceModel(mw, dtype)
    cfg = R.cfg_of(c)
    ts = [0.5, 0.125] if c.B > 1 else [0.5]
    B = len(ts)
    e = torch.empty((B, c.dim), dtype=torch.float32, device="cuda")
    e0 = torch.empty((B, 6, c.dim), dtype=torch.float32, device="cuda")
    L.time_embed(cfg, c.freq_dim, model.tw, ts, e, e0)
    ge, ge0 = host(e), host(e0)
    for b, t in enumerate(ts):
        re, re0 = oracle.time_embed(t, mw, c.freq_dim)
        assert rel_l2(ge[b], re) <= TOL[dtype] * 0.1, rel_l2(ge[b], re)
        assert rel_l2(ge0[b], re0) <= TOL[dtype] * 0.1, rel_l2(ge0[b], re0)


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_time_embed_max_batch(dtype):
    """The largest batch wan_time_embed takes (B = 4) with the schedule's end points t = 1 and t = 0
    among the rows; each row against the oracle."""
    require_gpu()
    c = wi.get_config("tiny").replace(dtype=dtype)
    case(f"time_embed B=4 {dtype}")
    mw = wi.make_model_weights(c, seed=4)
    model = R.DeviceModel(mw, dtype)
    ts = [1.0, 0.75, 0.0, 0.3]
    e = torch.empty((4, c.dim), dtype=torch.float32, device="cuda")
    e0 = torch.empty((4, 6, c.dim), dtype=torch.float32, device="cuda")
    L.time_embed(R.cfg_of(c), c.freq_dim, model.tw, ts, e, e0)
    ge, ge0 = host(e), host(e0)
    for b, t in enumerate(ts):
        re, re0 = oracle.time_embed(t, mw, c.freq_dim)
        assert rel_l2(ge[b], re) <= TOL[dtype] * 0.1, (t, rel_l2(ge[b], re))
        assert rel_l2(ge0[b], re0) <= TOL[dtype] * 0.1, (t, rel_l2(ge0[b], re0))


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_context_embed_and_cross_kv(dtype):
    require_gpu()
    c = wi.get_config("tiny").replace(dtype=dtype, img_len=9, img_dim=32)
    case(f"context_embed + cross_kv {dtype}")
    mw = wi.make_model_weights(c, seed=3)
    bw = wi.make_block_weights(c, 0, seed=3)
    txt, img = wi.make_contexts(c, seed=3)
    model = R.DeviceModel(mw, dtype)
    t_emb, i_emb = R.embed_contexts(c, model, txt, img, c.B)
    ref_t = oracle.context_embed(txt[0], mw["wtx1"], mw["btx1"], mw["wtx2"], mw["btx2"])
    ref_i = oracle.context_embed(img, mw["wim1"], mw["bim1"], mw["wim2"], mw["bim2"])
    assert rel_l2(host(t_emb)[0], ref_t) <= TOL[dtype]
    assert rel_l2(host(i_emb)[0], ref_i) <= TOL[dtype]
    blk = R.DeviceBlock(bw, dtype)
    (kc,) = R.cross_kv_all(c, [blk], t_emb, i_emb, c.B)
    # K [B, L, dim]; V^T [B, H, hd, Lpad] zero-padded
    te, ie = host(t_emb)[0], host(i_emb)[0]
    k_ref, v_ref = oracle.cross_kv(te, bw["wck"], bw["bck"], bw["wcv"], bw["bcv"])
    es = 2 if dtype == "bf16" else 4
    td = _tdt(dtype)
    k_got = kc.bufs[0].view(td).float().cpu().numpy().reshape(c.text_len, c.dim)
    Lp = 64
    vt_got = kc.bufs[1].view(td).float().cpu().numpy().reshape(c.heads, c.head_dim, Lp)
    assert rel_l2(k_got, k_ref) <= TOL[dtype]
    if dtype == "bf16":  # bf16 V^T stores keys permuted within 16-key groups (bits 2 and 3 swapped)
        pos = np.arange(Lp)
        key = (pos & ~12) | ((pos & 4) << 1) | ((pos & 8) >> 1)
        unperm = np.empty_like(vt_got)
        unperm[:, :, key] = vt_got
        vt_got = unperm
    v_from_t = vt_got[:, :, :c.text_len].transpose(2, 0, 1).reshape(c.text_len, c.dim)
    assert rel_l2(v_from_t, v_ref) <= TOL[dtype]
    assert np.all(vt_got[:, :, c.text_len:] == 0.0)
    ki_ref, vi_ref = oracle.cross_kv(ie, bw["wki"], bw["bki"], bw["wvi"], bw["bvi"])
    ki_got = kc.bufs[2].view(td).float().cpu().numpy().reshape(c.img_len, c.dim)
    assert rel_l2(ki_got, ki_ref) <= TOL[dtype]
    del es


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_head(dtype):
    require_gpu()
    c = wi.get_config("tiny").replace(dtype=dtype)
    case(f"head {dtype}")
    mw = wi.make_model_weights(c, seed=4)
    model = R.DeviceModel(mw, dtype)
    rng = np.random.default_rng(4)
    B = 2
    x = rng.standard_normal((B, c.S, c.dim)).astype(np.float32)
    e = (0.1 * rng.standard_normal((B, c.dim))).astype(np.float32)
    cfg = R.cfg_of(c)
    out = torch.empty((B, c.S, 4 * c.out_channels), dtype=torch.float32, device="cuda")
    ws = torch.empty(L.head_ws_bytes(cfg, B * c.S), dtype=torch.uint8, device="cuda")
    L.head_fwd(cfg, model.hw, c.out_channels, B, c.S, dev(x), dev(e), out, ws)
    ref = oracle.head_fwd(x, e, mw)
    assert rel_l2(host(out), ref) <= TOL[dtype]


@pytest.mark.timeout(900)
def test_attention_720p_stress_sampled_rows():
    """75600-token self-attention with 3D RoPE (40 heads x 128, q/k/v ~N(0,1) bf16) checked on sampled
    query rows: the oracle rotates every key and evaluates those rows' softmax over all keys."""
    require_gpu()
    c = wi.get_config("attn-720p")
    case("attention 720p stress (75600 tokens)")
    q, k, v = wi.make_attention_qkv(c, seed=3)
    td = torch.bfloat16
    qd, kd, vd = dev(q, td), dev(k, td), dev(v, td)
    o = torch.empty_like(qd)
    ws = torch.empty(L.attention_ws_bytes(L.WAN_BF16, c.grid, c.B, c.heads, c.head_dim), dtype=torch.uint8,
                     device="cuda")
    L.attention_fwd(qd, kd, vd, c.grid, o, ws)
    rows = wi.sample_rows(c, 24, seed=3)
    got = o[0, torch.from_numpy(rows).cuda()].float().cpu().numpy()
    del qd, kd, vd, o, ws
    ref = oracle.self_attention_rope_only(q[0], k[0], v[0], c.grid, rows=rows)
    err = rel_l2(got, ref)
    print(f"[attn-720p] sampled-row rel-L2 {err:.3e}")
    assert err <= TOL["bf16"]


@pytest.mark.parametrize("kind,a_word,b_word,a,b", [(0, 0x3F003F00, 0x3FC03FC0, 0.5, 1.5),
                                                    (1, 0x30303030, 0x3C3C3C3C, 0.5, 1.5)],
                         ids=["bf16", "e4m3"])
def test_mfma_peak_probe_sums(kind, a_word, b_word, a, b):
    """The register-only MFMA probe did all its instructions: every lane's accumulator sum is
    64 * K * iters * a * b (bf16 0.5 = 0x3F00, 1.5 = 0x3FC0; E4M3 0.5 = 0x30, 1.5 = 0x3C)."""
    require_gpu()
    case(f"mfma probe kind {kind}")
    cus, khz = L.device_info()
    assert cus > 0 and khz > 0
    blocks, iters = 3, 5
    out = torch.full((blocks * 256,), -1.0, dtype=torch.float32, device="cuda")
    flop = L.mfma_peak_probe(kind, a_word, b_word, blocks, iters, out)
    assert flop == blocks * 16 * iters * L.MFMA_PROBE_FLOP[kind]
    expect = 64.0 * L.MFMA_PROBE_K[kind] * iters * a * b
    got = host(out)
    assert np.all(got == expect), (got.min(), got.max(), expect)


def test_mfma_peak_probe_hashed_operands():
    """Kind 2 (bf16 on hashed operands, a measurement aid): every lane's sum is finite, the same seed
    gives the same sums, and another seed gives other sums."""
    require_gpu()
    case("mfma probe kind 2")
    blocks, iters = 3, 5
    out = torch.full((blocks * 256,), float("nan"), dtype=torch.float32, device="cuda")
    flop = L.mfma_peak_probe(2, 0x9E3779B9, 0x7F4A7C15, blocks, iters, out)
    assert flop == blocks * 16 * iters * L.MFMA_PROBE_FLOP[2]
    first = host(out).copy()
    L.mfma_peak_probe(2, 0x9E3779B9, 0x7F4A7C15, blocks, iters, out)
    second = host(out).copy()
    L.mfma_peak_probe(2, 0x12345678, 0x7F4A7C15, blocks, iters, out)
    third = host(out)
    assert np.all(np.isfinite(first)) and np.array_equal(first, second) and not np.array_equal(first, third)
