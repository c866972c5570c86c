"""Each branch of wan_dit_block_fwd against the oracle on its own ("图解 Wan2.1 I2V" §5.3-§5.5).

The gated branches are a few per cent of the block's update, so x_out and dx alone cannot see a
broken self-attention.  Here every branch output is compared directly:
  * self-attention: the layer output y = o W_o^T + b_o that the cached entry point stores
    (WAN_ATTN_CACHE_STORE) against the oracle block's recorded y;
  * cross-attention: the block with gate1 = gate2 = 0, whose update is exactly the cross branch;
  * FFN: the block with gate1 = 0 and W_co = b_co = 0, whose update is exactly gate2 * FFN.
Full outputs at small sizes, sampled query rows at the workload sizes.  Quantised paths hold y to
the bound derived for their products."""
import numpy as np
import pytest
import torch

import oracle
import wan_inputs as wi
from tests.gpu_util import case, dev, host, rel_l2, require_gpu
from tests.test_gpu_block import SMALL, _inputs
from video_diffusion_transformer_step_amd import _lib as L
from video_diffusion_transformer_step_amd import runtime as R

pytestmark = pytest.mark.gpu

TOL = {"f32": 1e-4, "bf16": 1e-2}
# One E4M3 rounding (unit roundoff 2^-4) bounds the quantised attention's output error (INT8 Q.K adds
# < 1 %, see test_gpu_fp8.py); y = o W_o^T + b_o in bf16 keeps that relative error.
FP8_ATTN_Y = 2.0 ** -4
# With the E4M3 products as well, y passes three E4M3-bounded steps in sequence (the Q/K/V product, the
# quantised attention, the O product): their bounds add.
FP8_ALL_Y = 3 * 2.0 ** -4
# The FFN branch under E4M3 products chains two of them (FFN1's error enters FFN2's input).
FP8_ALL_FFN = 2 * 2.0 ** -4


def _off(e0, bw, which):
    """Switch branches off by the pages' own switches: "self" gate1 = 0, "ffn" gate2 = 0 (e0 chunk and
    block bias both zero, so the sum is exactly 0), "cross" W_co = b_co = 0."""
    e0 = e0.copy()
    bw = dict(bw)
    mb = bw["mod_bias"].copy()
    for name, chunk in (("self", 2), ("ffn", 5)):
        if name in which:
            e0[:, chunk] = 0.0
            mb[chunk] = 0.0
    bw["mod_bias"] = mb
    if "cross" in which:
        bw["wco"] = np.zeros_like(bw["wco"])
        bw["bco"] = np.zeros_like(bw["bco"])
    return e0, bw


def _kv(c, bw, t_emb, i_emb):
    kv = []
    for b in range(c.B):
        kt, vt = oracle.cross_kv(t_emb[b], bw["wck"], bw["bck"], bw["wcv"], bw["bcv"])
        ki = vi = None
        if i_emb is not None:
            ki, vi = oracle.cross_kv(i_emb[b], bw["wki"], bw["bki"], bw["wvi"], bw["bvi"])
        kv.append((kt, vt, ki, vi))
    return kv


def _oracle(c, x, e0, bw, kv, rows, store_y=False):
    """(x_out rows, y rows or None) of the oracle block."""
    cache = None
    if store_y:
        cache = {"mode": "store", "y": np.zeros((c.B, c.S if rows is None else len(rows), c.dim))}
    out = oracle.block_fwd(x, e0, bw, kv, c.grid, c.heads, rows=rows, ln_eps=c.ln_eps, rms_eps=c.rms_eps,
                           theta=c.rope_theta, attn_cache=cache)
    return out, None if cache is None else cache["y"]


def _gpu(c, x, e0, bw, t_emb, i_emb, store_y=False, fp8_attn=False, fp8_gemm=False):
    """(x_out, y or None) of the HIP block on the host."""
    td = torch.bfloat16 if c.dtype == "bf16" else torch.float32
    blk = R.DeviceBlock(bw, c.dtype)
    if fp8_gemm:
        blk.enable_e4m3()
    (kc,) = R.cross_kv_all(c, [blk], dev(t_emb, td), None if i_emb is None else dev(i_emb, td), c.B)
    cfg = R.cfg_of(c, fp8_attn=fp8_attn, fp8_gemm=fp8_gemm)
    ws = torch.empty(L.block_ws_bytes(cfg, c.grid, c.B), dtype=torch.uint8, device="cuda")
    xd = dev(x)
    if store_y:
        y = torch.zeros((c.B, c.S, c.dim), dtype=torch.float32, device="cuda")
        L.dit_block_fwd(cfg, blk.bw, c.grid, c.B, xd, dev(e0), kc.kv, ws, attn_y=y,
                        attn_mode=L.WAN_ATTN_CACHE_STORE)
        return host(xd), host(y)
    L.dit_block_fwd(cfg, blk.bw, c.grid, c.B, xd, dev(e0), kc.kv, ws)
    return host(xd), None


def _rows(a, rows):
    return a if rows is None else a[:, rows]


def _branch_refs(c, x, e0, bw, t_emb, i_emb, rows):
    """The oracle's three branch outputs on the rows: y, the cross update, the gated FFN update."""
    kv = _kv(c, bw, t_emb, i_emb)
    xr = _rows(x, rows)
    full, y = _oracle(c, x, e0, bw, kv, rows, store_y=True)
    e0c, bwc = _off(e0, bw, ("self", "ffn"))
    cross, _ = _oracle(c, x, e0c, bwc, kv, rows)
    e0f, bwf = _off(e0, bw, ("self", "cross"))
    ffn, _ = _oracle(c, x, e0f, bwf, kv, rows)
    return {"dx": full - xr, "y": y, "cross": cross - xr, "ffn": ffn - xr}


def _check_branches(c, x, e0, bw, t_emb, i_emb, rows, ref, tol_y, tol_ffn, tol_cross, fp8_attn=False,
                    fp8_gemm=False, label=""):
    xr = _rows(x, rows)
    got, y = _gpu(c, x, e0, bw, t_emb, i_emb, store_y=True, fp8_attn=fp8_attn, fp8_gemm=fp8_gemm)
    e_y = rel_l2(_rows(y, rows), ref["y"])
    e0c, bwc = _off(e0, bw, ("self", "ffn"))
    gc, _ = _gpu(c, x, e0c, bwc, t_emb, i_emb, fp8_attn=fp8_attn, fp8_gemm=fp8_gemm)
    e_c = rel_l2(_rows(gc, rows) - xr, ref["cross"])
    e0f, bwf = _off(e0, bw, ("self", "cross"))
    gf, _ = _gpu(c, x, e0f, bwf, t_emb, i_emb, fp8_attn=fp8_attn, fp8_gemm=fp8_gemm)
    e_f = rel_l2(_rows(gf, rows) - xr, ref["ffn"])
    e_dx = rel_l2(_rows(got, rows) - xr, ref["dx"])
    print(f"[branches {c.name} {c.dtype} S={c.S} B={c.B} dim={c.dim}{label}] rel-L2 self-attention y={e_y:.3e} cross={e_c:.3e} ffn={e_f:.3e} "
          f"dx={e_dx:.3e}", flush=True)
    assert e_y <= tol_y and e_c <= tol_cross and e_f <= tol_ffn
    return e_dx


@pytest.mark.parametrize("name,over", SMALL, ids=["tiny", "tiny-dual", "tiny-bf16", "tiny-180tok-B2",
                                                   "bf16-hd128-ragged", "bf16-45tok-B3"])
def test_branches_small_full(name, over):
    """Every element of each branch output, at the small block configurations."""
    require_gpu()
    c = wi.get_config(name).replace(**over)
    case(f"branches {c.name} {over}")
    x, e0, t_emb, i_emb, bw = _inputs(c)
    ref = _branch_refs(c, x, e0, bw, t_emb, i_emb, None)
    t = TOL[c.dtype]
    _check_branches(c, x, e0, bw, t_emb, i_emb, None, ref, t, t, t)


def test_branches_small_fp8():
    """The quantised paths' branch outputs at 180 tokens, hd 128, two rows, dual-stream cross-attention:
    y within its derived E4M3 bound; the cross branch is bf16 on every path; the FFN branch is bf16
    under WAN_FLAG_FP8_ATTN and two chained E4M3 products under WAN_FLAG_FP8_GEMM."""
    require_gpu()
    c = wi.get_config("tiny").replace(dtype="bf16", T=3, H=12, W=20, B=2, dim=256, heads=2, head_dim=128,
                                      ffn_dim=768, text_len=70, img_len=9, img_dim=32)
    case(f"branches fp8 {c.name} S={c.S}")
    x, e0, t_emb, i_emb, bw = _inputs(c)
    ref = _branch_refs(c, x, e0, bw, t_emb, i_emb, None)
    t = TOL["bf16"]
    _check_branches(c, x, e0, bw, t_emb, i_emb, None, ref, FP8_ATTN_Y, t, t, fp8_attn=True, label=" fp8 attention")
    _check_branches(c, x, e0, bw, t_emb, i_emb, None, ref, FP8_ALL_Y, FP8_ALL_FFN, t, fp8_attn=True,
                    fp8_gemm=True, label=" fp8 attention + e4m3 products")


@pytest.mark.timeout(600)
def test_branches_hd64_async_copy_products():
    """Head dim 64 on the large-row product path: B = 2 rows of 4096 tokens (4 frames of 32 x 32
    patches), dim 640 = 10 heads of 64.  The Q/K/V product then runs the asynchronous-copy kernel, whose
    waves' 128 columns span two heads, so the epilogue's gains, RoPE and row sums of squares cross a
    head boundary inside a wave tile, and batch row 1 exercises the position decode m % S.  Sampled
    rows of every branch at the bf16 bar."""
    require_gpu()
    c = wi.get_config("tiny").replace(dtype="bf16", T=4, H=64, W=64, B=2, dim=640, heads=10, head_dim=64,
                                      ffn_dim=1280, text_len=64)
    case(f"branches hd64 async-copy products {c.name} S={c.S} B={c.B}")
    rows = wi.sample_rows(c, 24, seed=11)
    x, e0, t_emb, i_emb, bw = _inputs(c, seed=11)
    ref = _branch_refs(c, x, e0, bw, t_emb, i_emb, rows)
    t = TOL["bf16"]
    _check_branches(c, x, e0, bw, t_emb, i_emb, rows, ref, t, t, t)


DEGENERATE = [
    # one row of patches (Hp = 1: every height-segment rotation is the identity), 5 frames, two rows
    ("hp1", {"dtype": "bf16", "T": 5, "H": 2, "W": 40, "B": 2, "dim": 256, "heads": 2, "head_dim": 128,
             "ffn_dim": 512, "text_len": 32}, None),
    # a single frame (T = 1: every time-segment rotation is the identity) large enough for the
    # asynchronous-copy products: B = 2 rows of 64 x 32 patches = 4096 product rows
    ("image-async-copy", {"dtype": "bf16", "T": 1, "H": 128, "W": 64, "B": 2, "dim": 512, "heads": 4,
                          "head_dim": 128, "ffn_dim": 1024, "text_len": 64}, 24),
]


@pytest.mark.timeout(600)
@pytest.mark.parametrize("label,over,n_rows", DEGENERATE, ids=[d[0] for d in DEGENERATE])
def test_branches_degenerate_grids(label, over, n_rows):
    """Grids where an axis of the 3D RoPE has a single position, through the Q/K/V epilogue's rotation
    table: every branch at the bf16 bar (all rows, or sampled rows for the larger grid)."""
    require_gpu()
    c = wi.get_config("tiny").replace(**over)
    case(f"branches degenerate grid {label} {c.grid} S={c.S} B={c.B}")
    rows = None if n_rows is None else wi.sample_rows(c, n_rows, seed=12)
    x, e0, t_emb, i_emb, bw = _inputs(c, seed=12)
    ref = _branch_refs(c, x, e0, bw, t_emb, i_emb, rows)
    t = TOL["bf16"]
    _check_branches(c, x, e0, bw, t_emb, i_emb, rows, ref, t, t, t)


@pytest.mark.timeout(900)
@pytest.mark.parametrize("name", ["t2v-1.3b", "ti2v-5b", pytest.param("i2v-14b", marks=pytest.mark.slow)])
def test_branches_full_size(name):
    """Workload-size blocks, sampled query rows: the self-attention layer output y at 32760 (27280) tokens
    with the real RoPE grid, the cross branch (text, or image + text for the 14B-shaped block) and the
    gated FFN branch, each against the oracle at the bf16 bar."""
    require_gpu()
    c = wi.get_config(name)
    case(f"branches full size {c.name}")
    rows = wi.sample_rows(c, {"t2v-1.3b": 64, "ti2v-5b": 32, "i2v-14b": 24}[name], seed=6)
    x, e0, t_emb, i_emb, bw = _inputs(c, seed=6)
    ref = _branch_refs(c, x, e0, bw, t_emb, i_emb, rows)
    t = TOL["bf16"]
    _check_branches(c, x, e0, bw, t_emb, i_emb, rows, ref, t, t, t)


@pytest.mark.timeout(900)
def test_branches_full_size_fp8():
    """The 32760-token 1.3B-shaped block on both quantised paths, sampled rows: y held to its derived
    E4M3 bound, the FFN branch to two chained E4M3 products, dx to the bf16 bar plus the self-attention
    branch's share of dx times its bound."""
    require_gpu()
    c = wi.get_config("t2v-1.3b")
    case(f"branches full size fp8 {c.name}")
    rows = wi.sample_rows(c, 48, seed=7)
    x, e0, t_emb, i_emb, bw = _inputs(c, seed=7)
    ref = _branch_refs(c, x, e0, bw, t_emb, i_emb, rows)
    gate1 = np.stack([e0[b, 2] + bw["mod_bias"][2] for b in range(c.B)])[:, None, :]
    share = np.linalg.norm(gate1 * ref["y"]) / np.linalg.norm(ref["dx"])
    t = TOL["bf16"]
    e_dx = _check_branches(c, x, e0, bw, t_emb, i_emb, rows, ref, FP8_ATTN_Y, t, t, fp8_attn=True,
                           label=" fp8 attention")
    print(f"  self-attention share of dx {share:.3e}; dx bound {t + FP8_ATTN_Y * share:.3e}", flush=True)
    assert e_dx <= t + FP8_ATTN_Y * share
    _check_branches(c, x, e0, bw, t_emb, i_emb, rows, ref, FP8_ALL_Y, FP8_ALL_FFN, t, fp8_attn=True, fp8_gemm=True,
                    label=" fp8 attention + e4m3 products")
