"""Host-side checks of the C ABI (no GPU): libwan.so loads, exports every function that
include/wan.h declares, and rejects bad arguments before enqueueing anything."""
import ctypes as C
import os
import re

import pytest

from video_diffusion_transformer_step_amd import _lib as L

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "wan.h")
FAKE = 0x10000  # aligned, non-null, never dereferenced: every call below fails validation first


@pytest.fixture(scope="module")
def lib():
    if not os.path.exists(L.LIB_PATH):
        from video_diffusion_transformer_step_amd.build import build
        build()
    return L.lib()


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(wan_[a-z0-9_]+)\s*\(", text)))


def test_header_declares_the_boundary():
    names = declared_functions()
    for required in ("wan_patchify", "wan_dit_block_fwd", "wan_fm_euler_step", "wan_unpatchify",
                     "wan_build_i2v_input", "wan_attention_fwd", "wan_time_embed", "wan_head_fwd"):
        assert required in names


def test_every_declared_symbol_is_exported(lib):
    for name in declared_functions():
        assert hasattr(lib, name), name
    assert set(declared_functions()) == set(L._SIGS), "binding and header disagree"


def _cfg(**kw):
    base = dict(dim=128, heads=2, head_dim=64, ffn_dim=512, text_len=16, img_len=0, dtype=L.WAN_F32)
    base.update(kw)
    return L.block_cfg(**base)


def _err(lib):
    return lib.wan_last_error().decode()


def test_layout_validation(lib):
    bad = L.LatentShape(1, 16, 2, 7, 8)  # odd H
    assert lib.wan_patchify(FAKE, bad, FAKE, None) == L.WAN_EINVAL
    assert "even" in _err(lib)
    ok = L.LatentShape(1, 16, 2, 8, 8)
    assert lib.wan_patchify(None, ok, FAKE, None) == L.WAN_EINVAL
    assert lib.wan_unpatchify(FAKE, ok, FAKE + 4, None) == L.WAN_EINVAL  # misaligned
    assert "aligned" in _err(lib)
    assert lib.wan_build_i2v_input(FAKE, FAKE, None, L.LatentShape(1, 16, 65, 8, 8), FAKE, None) \
        == L.WAN_EUNSUPPORTED
    assert lib.wan_build_i2v_input(FAKE, FAKE, None, L.LatentShape(0, 16, 2, 8, 8), FAKE, None) == L.WAN_EINVAL
    assert lib.wan_fm_euler_step(FAKE, None, None, 1.0, -0.1, 10, None) == L.WAN_EINVAL
    assert lib.wan_fm_euler_step(FAKE, FAKE, None, 1.0, -0.1, -1, None) == L.WAN_EINVAL


def test_block_validation(lib):
    g = L.Grid(2, 4, 4)
    kv = L.CrossKV(FAKE, FAKE, None, None)
    w = L.BlockWeights(*([FAKE] * 17))
    ws_need = lib.wan_dit_block_workspace_bytes(C.byref(_cfg()), g, 1)
    assert ws_need > 0
    assert lib.wan_dit_block_workspace_bytes(C.byref(_cfg(dtype=L.WAN_BF16)), g, 1) < ws_need
    for cfg, code in [(_cfg(dim=130), L.WAN_EINVAL),               # dim != heads * head_dim
                      (_cfg(head_dim=96, dim=192), L.WAN_EUNSUPPORTED),
                      (_cfg(dtype=7), L.WAN_EINVAL),
                      (_cfg(text_len=0), L.WAN_EINVAL),
                      (_cfg(ffn_dim=500), L.WAN_EINVAL),
                      (_cfg(dim=8192, heads=64, head_dim=128), L.WAN_EUNSUPPORTED)]:
        assert lib.wan_dit_block_fwd(C.byref(cfg), C.byref(w), g, 1, FAKE, FAKE, C.byref(kv), FAKE, ws_need,
                                     None) == code, _err(lib)
    c = _cfg()
    c.flags = L.WAN_FLAG_FP8_ATTN  # the quantised self-attention needs bf16 and head_dim 128
    assert lib.wan_dit_block_fwd(C.byref(c), C.byref(w), g, 1, FAKE, FAKE, C.byref(kv), FAKE, ws_need,
                                 None) == L.WAN_EUNSUPPORTED
    c.flags = 4  # unknown bit
    assert lib.wan_dit_block_fwd(C.byref(c), C.byref(w), g, 1, FAKE, FAKE, C.byref(kv), FAKE, ws_need,
                                 None) == L.WAN_EUNSUPPORTED
    b16 = _cfg(dtype=L.WAN_BF16, dim=256, heads=2, head_dim=128)
    plain = lib.wan_dit_block_workspace_bytes(C.byref(b16), g, 1)
    b16.flags = L.WAN_FLAG_FP8_ATTN
    assert lib.wan_dit_block_workspace_bytes(C.byref(b16), g, 1) > plain  # room for the codes
    # too small a workspace
    assert lib.wan_dit_block_fwd(C.byref(_cfg()), C.byref(w), g, 1, FAKE, FAKE, C.byref(kv), FAKE, ws_need - 1,
                                 None) == L.WAN_EWORKSPACE
    # bad grid / batch / missing weight / missing image K/V when img_len > 0
    assert lib.wan_dit_block_fwd(C.byref(_cfg()), C.byref(w), L.Grid(0, 4, 4), 1, FAKE, FAKE, C.byref(kv), FAKE,
                                 ws_need, None) == L.WAN_EINVAL
    assert lib.wan_dit_block_fwd(C.byref(_cfg()), C.byref(w), g, 0, FAKE, FAKE, C.byref(kv), FAKE, ws_need,
                                 None) == L.WAN_EINVAL
    w2 = L.BlockWeights(*([FAKE] * 17))
    w2.w1 = None
    assert lib.wan_dit_block_fwd(C.byref(_cfg()), C.byref(w2), g, 1, FAKE, FAKE, C.byref(kv), FAKE, ws_need,
                                 None) == L.WAN_EINVAL
    assert "w1" in _err(lib)
    assert lib.wan_dit_block_fwd(C.byref(_cfg(img_len=4)), C.byref(w), g, 1, FAKE, FAKE, C.byref(kv), FAKE,
                                 ws_need * 2, None) == L.WAN_EINVAL
    # the attention-cache entry: mode outside 0..2, or a cache mode without the y buffer
    blk = lib.wan_dit_block_fwd_cached
    assert blk(C.byref(_cfg()), C.byref(w), g, 1, FAKE, FAKE, C.byref(kv), FAKE, 3, FAKE, ws_need,
               None) == L.WAN_EINVAL
    assert "attn_mode" in _err(lib)
    for mode in (L.WAN_ATTN_CACHE_STORE, L.WAN_ATTN_CACHE_REUSE):
        assert blk(C.byref(_cfg()), C.byref(w), g, 1, FAKE, FAKE, C.byref(kv), None, mode, FAKE, ws_need,
                   None) == L.WAN_EINVAL
        assert "attn_y" in _err(lib)
    # the other checks still run behind a valid mode
    assert blk(C.byref(_cfg()), C.byref(w), g, 1, FAKE, FAKE, C.byref(kv), FAKE, L.WAN_ATTN_CACHE_REUSE, FAKE,
               ws_need - 1, None) == L.WAN_EWORKSPACE


def test_block_noalloc_validation(lib):
    """wan_dit_block_fwd_noalloc rejects a block whose workspace exceeds its static scratch, and bad
    arguments, on the host before touching the device (so these calls need no GPU)."""
    m = re.search(r"#define WAN_NOALLOC_SCRATCH_BYTES \(\(size_t\)(\d+) << (\d+)\)", open(HEADER).read())
    assert m and int(m.group(1)) << int(m.group(2)) == L.NOALLOC_SCRATCH_BYTES
    kv = L.CrossKV(FAKE, FAKE, None, None)
    w = L.BlockWeights(*([FAKE] * 17))
    big = _cfg(dtype=L.WAN_BF16, dim=1536, heads=12, head_dim=128, ffn_dim=8960)
    g = L.Grid(21, 30, 52)  # 32760 tokens: about 1.1 GB of workspace
    assert lib.wan_dit_block_workspace_bytes(C.byref(big), g, 1) > L.NOALLOC_SCRATCH_BYTES
    assert lib.wan_dit_block_fwd_noalloc(C.byref(big), C.byref(w), g, 1, FAKE, FAKE, C.byref(kv), None) \
        == L.WAN_EWORKSPACE
    assert "scratch" in _err(lib)
    assert lib.wan_dit_block_fwd_noalloc(C.byref(_cfg(dim=130)), C.byref(w), L.Grid(2, 4, 4), 1, FAKE, FAKE,
                                         C.byref(kv), None) == L.WAN_EINVAL
    assert lib.wan_dit_block_fwd_noalloc(C.byref(_cfg()), C.byref(w), L.Grid(0, 4, 4), 1, FAKE, FAKE, C.byref(kv),
                                         None) == L.WAN_EINVAL
    assert lib.wan_dit_block_fwd_noalloc(C.byref(_cfg()), C.byref(w), L.Grid(2, 4, 4), 0, FAKE, FAKE, C.byref(kv),
                                         None) == L.WAN_EINVAL


def test_other_entry_validation(lib):
    cfg = _cfg()
    tw = L.TimeWeights(*([FAKE] * 6))
    t = (C.c_float * 5)(0.5, 0.5, 0.5, 0.5, 0.5)
    assert lib.wan_time_embed(C.byref(cfg), 256, C.byref(tw), t, 5, FAKE, FAKE, None) == L.WAN_EUNSUPPORTED
    assert lib.wan_time_embed(C.byref(cfg), 260, C.byref(tw), t, 1, FAKE, FAKE, None) == L.WAN_EINVAL
    assert lib.wan_patch_embed(C.byref(cfg), FAKE, 32, 3, FAKE, None, FAKE, None, 0, None) == L.WAN_EUNSUPPORTED
    bcfg = _cfg(dtype=L.WAN_BF16)
    need = lib.wan_patch_embed_workspace_bytes(C.byref(bcfg), 32, 36)
    assert need >= 32 * 144 * 2
    assert lib.wan_patch_embed(C.byref(bcfg), FAKE, 32, 36, FAKE, None, FAKE, FAKE, need - 1, None) \
        == L.WAN_EWORKSPACE
    hw = L.HeadWeights(FAKE, FAKE, None)
    assert lib.wan_head_fwd(C.byref(cfg), C.byref(hw), 16, 1, 32, FAKE, FAKE, FAKE, FAKE, 0, None) \
        == L.WAN_EWORKSPACE
    assert lib.wan_attention_fwd(L.WAN_BF16, FAKE, FAKE, FAKE, L.Grid(2, 4, 4), 1, 2, 80, 10000.0, FAKE, FAKE,
                                 1 << 30, None) == L.WAN_EUNSUPPORTED
    need = lib.wan_attention_workspace_bytes(L.WAN_BF16, L.Grid(2, 4, 4), 1, 2, 64)
    assert lib.wan_attention_fwd(L.WAN_BF16, FAKE, FAKE, FAKE, L.Grid(2, 4, 4), 1, 2, 64, 10000.0, FAKE, FAKE,
                                 need - 1, None) == L.WAN_EWORKSPACE
    kvw = L.CrossKVWeights(FAKE, None, None, None)
    out = L.CrossKV(FAKE, FAKE, None, None)
    assert lib.wan_cross_kv_fwd(C.byref(_cfg(img_len=3)), C.byref(kvw), FAKE, FAKE, 1, C.byref(out), FAKE,
                                1 << 20, None) == L.WAN_EINVAL
    assert lib.wan_context_embed(C.byref(cfg), FAKE, 16, 60, FAKE, None, FAKE, None, FAKE, FAKE, 1 << 20,
                                 None) == L.WAN_EINVAL


def test_weight_panel_sizes_and_validation(lib):
    """K panels of 32 with N rounded up to 256 rows (the layout wan.h defines for the block's matrices)."""
    assert lib.wan_pack_weight_bytes(2, 1536, 8960) == 1536 * 8960 * 2
    assert lib.wan_pack_weight_bytes(2, 260, 768) == 512 * 768 * 2
    assert lib.wan_pack_weight_bytes(1, 1, 256) == 256 * 256
    assert lib.wan_pack_weight_bytes(4, 300, 32) == 512 * 32 * 4
    for bad in ((3, 256, 256), (2, 0, 256), (2, 256, 0), (2, 256, 48), (1, -1, 64)):
        assert lib.wan_pack_weight_bytes(*bad) == 0, bad
    assert lib.wan_pack_weight(2, FAKE, 256, 48, FAKE, None) == L.WAN_EINVAL
    assert lib.wan_pack_weight(3, FAKE, 256, 64, FAKE, None) == L.WAN_EINVAL
    assert lib.wan_pack_weight(2, None, 256, 64, FAKE, None) == L.WAN_EINVAL
    assert lib.wan_pack_weight(2, FAKE, 256, 64, FAKE + 8, None) == L.WAN_EINVAL
    # E4M3 product: K % 256, and the panels must stay below 2 GiB
    assert lib.wan_gemm_e4m3(FAKE, FAKE, FAKE, FAKE, 64, 256, 384, None, 0, FAKE, 256, None) == L.WAN_EUNSUPPORTED
    assert lib.wan_gemm_e4m3(FAKE, FAKE, FAKE, FAKE, 64, 1 << 17, 1 << 17, None, 0, FAKE, 1 << 17, None) \
        == L.WAN_EUNSUPPORTED
    assert lib.wan_gemm_e4m3(FAKE, FAKE, FAKE, FAKE, 1 << 17, 256, 1 << 14, None, 0, FAKE, 256, None) \
        == L.WAN_EUNSUPPORTED
    assert lib.wan_gemm_e4m3(FAKE, FAKE, FAKE, FAKE, 64, 256, 256, None, 0, FAKE, 255, None) == L.WAN_EINVAL


def test_ring_attention_validation(lib):
    need = lib.wan_attention_partial_workspace_bytes(L.WAN_BF16, 1, 50, 100, 2, 64)
    assert need == 2 * 64 * 128 * 2  # V^T of 100 keys padded to 128; too few keys to split
    # two query tiles against 4096 keys leave the chip idle: the workspace adds key-split parts
    vt = 2 * 64 * 4096 * 2
    assert lib.wan_attention_partial_workspace_bytes(L.WAN_BF16, 1, 300, 4096, 2, 64) > vt
    assert lib.wan_attention_partial_workspace_bytes(L.WAN_BF16, 1, 300, 0, 2, 64) == 0
    args = lambda **kw: dict(dict(dt=L.WAN_BF16, B=1, Sq=50, Sk=100, H=2, hd=64, lse=FAKE, ws=need), **kw)

    def part(a):
        return lib.wan_attention_partial_fwd(a["dt"], FAKE, FAKE, FAKE, a["B"], a["Sq"], a["Sk"], a["H"], a["hd"],
                                             FAKE, a["lse"], FAKE, a["ws"], None)
    assert part(args(hd=96)) == L.WAN_EUNSUPPORTED
    assert part(args(Sk=0)) == L.WAN_EINVAL
    assert part(args(dt=3)) == L.WAN_EINVAL
    assert part(args(lse=FAKE + 2)) == L.WAN_EINVAL           # misaligned lse
    assert part(args(ws=need - 1)) == L.WAN_EWORKSPACE

    def merge(n, lse_ptr=FAKE, hd=64):
        op = (C.c_void_p * max(n, 1))(*([FAKE] * max(n, 1)))
        lp = (C.c_void_p * max(n, 1))(*([lse_ptr] * max(n, 1)))
        return lib.wan_attention_lse_merge(L.WAN_BF16, n, op, lp, 1, 50, 2, hd, FAKE, None, None)
    assert merge(0) == L.WAN_EINVAL
    assert merge(17) == L.WAN_EINVAL
    assert merge(2, hd=96) == L.WAN_EUNSUPPORTED
    assert merge(2, lse_ptr=FAKE + 1) == L.WAN_EINVAL
    assert "lse_parts" in _err(lib)


def test_device_probe_validation(lib):
    assert lib.wan_device_info(None, None) == L.WAN_EINVAL
    for kind, blocks, iters, out in ((3, 1, 1, FAKE), (-1, 1, 1, FAKE), (0, 0, 1, FAKE), (1, 1, 0, FAKE),
                                     (0, 1 << 21, 1, FAKE), (0, 1, 1 << 21, FAKE), (0, 1, 1, None),
                                     (1, 1, 1, FAKE + 2)):
        assert lib.wan_mfma_peak_probe(kind, 0, 0, blocks, iters, out, None) == L.WAN_EINVAL, (kind, blocks, iters)
    assert "aligned" in _err(lib)


def test_status_strings(lib):
    assert lib.wan_status_string(L.WAN_EWORKSPACE) == b"WAN_EWORKSPACE"
    assert lib.wan_status_string(0) == b"WAN_OK"


def test_cross_kv_buffer_sizes(lib):
    c = _cfg(dtype=L.WAN_BF16, text_len=512, img_len=257, dim=5120, heads=40, head_dim=128)
    assert lib.wan_cross_kv_buffer_bytes(C.byref(c), 2, 0) == 2 * 512 * 5120 * 2
    assert lib.wan_cross_kv_buffer_bytes(C.byref(c), 2, 1) == 2 * 5120 * 512 * 2
    assert lib.wan_cross_kv_buffer_bytes(C.byref(c), 2, 3) == 2 * 5120 * 320 * 2  # 257 -> 320 (64-padded)


def test_missing_library_fails_loudly():
    """Without libwan.so the binding raises; nothing falls back to another implementation."""
    import subprocess
    import sys
    code = ("import video_diffusion_transformer_step_amd._lib as L\n"
            "L.LIB_PATH = '/nonexistent/libwan.so'\n"
            "L._lib = None\n"
            "try:\n"
            "    L.lib()\n"
            "except RuntimeError as e:\n"
            "    print('raised:', e)\n"
            "else:\n"
            "    raise SystemExit('no error')\n")
    r = subprocess.run([sys.executable, "-c", code], cwd=ROOT, capture_output=True, text=True, timeout=120)
    assert r.returncode == 0, r.stderr
    assert "raised:" in r.stdout and "libwan.so" in r.stdout
