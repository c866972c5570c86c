"""wan_dit_block_fwd_noalloc (the block with its scratch in a static device array) against
wan_dit_block_fwd with a caller workspace: the same kernels on the same inputs, so the outputs must be
bitwise equal.  Two calls in a row, the second on a smaller input (the scratch then holds the first
call's data), in bf16 and fp32, with and without the image stream."""
import numpy as np
import pytest
import torch

import wan_inputs as wi
from tests.gpu_util import case, dev, host, require_gpu
from tests.test_gpu_block import _inputs
from video_diffusion_transformer_step_amd import _lib as L
from video_diffusion_transformer_step_amd import runtime as R

pytestmark = pytest.mark.gpu


def _both(c, seed):
    """(noalloc output, workspace-entry output) of one block on the host."""
    x, e0, t_emb, i_emb, bw = _inputs(c, seed=seed)
    td = torch.bfloat16 if c.dtype == "bf16" else torch.float32
    blk = R.DeviceBlock(bw, c.dtype)
    (kc,) = R.cross_kv_all(c, [blk], dev(t_emb, td), None if i_emb is None else dev(i_emb, td), c.B)
    cfg = R.cfg_of(c)
    need = L.block_ws_bytes(cfg, c.grid, c.B)
    assert need <= L.NOALLOC_SCRATCH_BYTES
    e0d = dev(e0)
    xa = dev(x)
    L.dit_block_fwd_noalloc(cfg, blk.bw, c.grid, c.B, xa, e0d, kc.kv)
    xb = dev(x)
    ws = torch.full((need,), 0xFF, dtype=torch.uint8, device="cuda")
    L.dit_block_fwd(cfg, blk.bw, c.grid, c.B, xb, e0d, kc.kv, ws)
    return host(xa), host(xb), x


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
def test_noalloc_matches_workspace_entry_two_calls(dtype):
    require_gpu()
    big = wi.get_config("tiny").replace(dtype=dtype, T=3, H=12, W=20, B=2, dim=256, heads=2, head_dim=128,
                                        ffn_dim=640, text_len=70, img_len=9, img_dim=32)
    small = wi.get_config("tiny").replace(dtype=dtype, T=2, H=6, W=10, B=1, img_len=0)
    for c, seed in ((big, 21), (small, 22)):
        case(f"noalloc block {dtype} S={c.S} B={c.B} dim={c.dim} img_len={c.img_len}")
        a, b, x = _both(c, seed)
        assert np.isfinite(a).all()
        assert not np.array_equal(a, x)  # the block ran
        assert np.array_equal(a, b), float(np.abs(a - b).max())


def test_noalloc_rejects_a_block_beyond_its_scratch():
    require_gpu()
    c = wi.get_config("t2v-1.3b")
    cfg = R.cfg_of(c)
    assert L.block_ws_bytes(cfg, c.grid, c.B) > L.NOALLOC_SCRATCH_BYTES
    x = torch.zeros((c.B, c.S, c.dim), dtype=torch.float32, device="cuda")
    e0 = torch.zeros((c.B, 6, c.dim), dtype=torch.float32, device="cuda")
    w = L.BlockWeights(*([x.data_ptr()] * 17))
    kv = L.CrossKV(x.data_ptr(), x.data_ptr(), None, None)
    with pytest.raises(L.WanError) as err:
        L.dit_block_fwd_noalloc(cfg, w, c.grid, c.B, x, e0, kv)
    assert err.value.code == L.WAN_EWORKSPACE
    torch.cuda.synchronize()
    assert not bool(x.any())  # nothing was enqueued
