"""Wan2.2's two-expert sampling (a high-noise and a low-noise DiT, switched at t_moe) against the
oracle: the expert sequence exactly, the latent after every step within the uncached sampler's
tolerances (fp32 1e-4, bf16 1e-2)."""
import numpy as np
import pytest

import oracle
import wan_inputs as wi
from tests.gpu_util import case, dev, host, rel_l2, require_gpu
from video_diffusion_transformer_step_amd import runtime as R

pytestmark = pytest.mark.gpu

TOL = {"f32": 1e-4, "bf16": 1e-2}


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_sample_two_expert_small(dtype):
    """Tiny I2V config, two CFG rows, 2 blocks per expert, 4 steps from t = 1 with t_moe = 1/2
    (t = 1, 3/4 on the high-noise expert; the boundary t = 1/2 and t = 1/4 on the low-noise one)."""
    require_gpu()
    c = wi.get_config("tiny").replace(dtype=dtype, B=2, img_len=5, img_dim=32)
    case(f"two-expert sampling tiny {dtype}")
    steps, layers, t_moe = 4, 2, 0.5
    ws = [(wi.make_model_weights(c, seed=s), [wi.make_block_weights(c, i, seed=s) for i in range(layers)])
          for s in (3, 77)]
    x_t, z = wi.make_latents(c, seed=3)
    txt, img = wi.make_contexts(c, seed=3)
    experts = []
    for mw, bws in ws:
        model = R.DeviceModel(mw, c.dtype)
        blocks = [R.DeviceBlock(w, c.dtype) for w in bws]
        t_emb, i_emb = R.embed_contexts(c, model, txt, img, c.B)
        experts.append((model, blocks, R.cross_kv_all(c, blocks, t_emb, i_emb, c.B)))
    buf = R.alloc_step(c, c.B)
    xg = dev(x_t)
    used = R.sample_two_expert(c, experts, xg, dev(z), steps, c.guidance, buf, c.B, t_moe)
    got = host(xg)
    ref, _, ref_used = oracle.sample_two_expert(x_t, z, steps, c.guidance, ws, t_moe, txt, img, c.heads,
                                                ln_eps=c.ln_eps, rms_eps=c.rms_eps, theta=c.rope_theta,
                                                freq_dim=c.freq_dim, out_channels=c.out_channels)
    assert used == ref_used == [0, 0, 1, 1]
    e = rel_l2(got, ref)
    one, _ = oracle.sample(x_t, z, steps, c.guidance, ws[0][0], ws[0][1], txt, img, c.heads, ln_eps=c.ln_eps,
                           rms_eps=c.rms_eps, theta=c.rope_theta, freq_dim=c.freq_dim, out_channels=c.out_channels)
    x0 = np.asarray(x_t, np.float64)
    moved = rel_l2(ref - x0, one - x0)
    print(f"[two-expert {dtype}] rel-L2 vs oracle {e:.3e}; two experts vs the first alone (update) {moved:.3e}",
          flush=True)
    assert e <= TOL[dtype]
    assert moved > 5 * TOL[dtype]
