"""A whole denoise step through the C ABI -- [I2V input] -> patchify -> patch embedding ->
timestep embedding -> blocks -> head -> unpatchify -> CFG + Euler -- against the oracle."""
import numpy as np
import pytest
import torch

import oracle
import wan_inputs as wi
from tests.gpu_util import case, dev, host, rel_l2, require_gpu
from video_diffusion_transformer_step_amd import runtime as R

pytestmark = pytest.mark.gpu

TOL = {"f32": 1e-4, "bf16": 1e-2}


def _run(c, layers, steps, seed=0, t0=None, dt=None):
    mw = wi.make_model_weights(c, seed=seed)
    bws = [wi.make_block_weights(c, i, seed=seed) for i in range(layers)]
    x_t, z = wi.make_latents(c, seed=seed)
    txt, img = wi.make_contexts(c, seed=seed)
    t0 = c.t if t0 is None else t0
    explicit_dt = dt is not None
    dt = -t0 / steps if dt is None else dt
    # GPU
    model = R.DeviceModel(mw, c.dtype)
    blocks = [R.DeviceBlock(w, c.dtype) for w in bws]
    t_emb, i_emb = R.embed_contexts(c, model, txt, img, c.B)
    caches = R.cross_kv_all(c, blocks, t_emb, i_emb, c.B)
    buf = R.alloc_step(c, c.B)
    xg = dev(x_t)
    zg = dev(z) if z is not None else None
    gpu_traj = []
    v0 = None
    for k in range(steps):
        R.denoise_step(c, model, blocks, caches, xg, zg, t0 + k * dt, dt, c.guidance, buf, c.B)
        gpu_traj.append(host(xg))
        if k == 0:
            v0 = host(buf.v)
    # oracle
    if explicit_dt:
        # one step of the given size: v = DiT(x_in, t0), x <- x + dt * CFG(v)
        x_in1 = x_t if z is None else oracle.build_i2v_input(x_t, z)
        v = oracle.dit_fwd(np.repeat(x_in1, c.B, axis=0), t0, mw, bws, txt, img, c.heads, ln_eps=c.ln_eps,
                           rms_eps=c.rms_eps, theta=c.rope_theta, freq_dim=c.freq_dim,
                           out_channels=c.out_channels)
        traj = [oracle.cfg_euler(x_t, v[0:1], v[1:2] if c.B > 1 else None, c.guidance, dt)]
    else:
        x_fin, traj = oracle.sample(x_t, z, steps, c.guidance, mw, bws, txt, img, c.heads, t0=t0,
                                    ln_eps=c.ln_eps, rms_eps=c.rms_eps, theta=c.rope_theta,
                                    freq_dim=c.freq_dim, out_channels=c.out_channels)
    # the DiT's per-row velocity at the first step (both sides start from x_t)
    x_in = x_t if z is None else oracle.build_i2v_input(x_t, z)
    v0_ref = oracle.dit_fwd(np.repeat(x_in, c.B, axis=0), t0, mw, bws, txt, img, c.heads, ln_eps=c.ln_eps,
                            rms_eps=c.rms_eps, theta=c.rope_theta, freq_dim=c.freq_dim,
                            out_channels=c.out_channels)
    for b in range(c.B):
        e_v = rel_l2(v0[b], v0_ref[b])
        print(f"[{c.name}] step 0 row {b}: rel-L2 v={e_v:.3e}")
        assert e_v <= TOL[c.dtype]
    return x_t, gpu_traj, traj


def _check(c, x_t, gpu_traj, traj):
    for k, (g, o) in enumerate(zip(gpu_traj, traj)):
        e_x = rel_l2(g, o)
        print(f"[{c.name}] step {k}: rel-L2 x={e_x:.3e}")
        assert e_x <= TOL[c.dtype]
    if c.B == 1:
        # without guidance the first step's update is dt * v: it inherits v's tolerance.  (With
        # guidance s the update mixes (1 - s) v_u + s v_c, which scales the per-row error of v by up
        # to |1 - s| + s; the rows of v are checked individually above instead.)
        g0, o0 = gpu_traj[0], traj[0]
        assert rel_l2(g0 - x_t, o0 - x_t) <= TOL[c.dtype]


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_step_tiny_i2v(dtype):
    """Tiny image-to-video block config: one block, one Euler step (t = 0.5, dt = -0.1)."""
    require_gpu()
    c = wi.get_config("tiny").replace(dtype=dtype)
    case(f"step tiny {dtype}")
    x_t, gt, ot = _run(c, layers=1, steps=1, t0=c.t, dt=c.dt)
    _check(c, x_t, gt, ot)


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_step_cfg_two_rows(dtype):
    """Classifier-free guidance: two rows (conditional / unconditional text), shared latent,
    dual-stream cross-attention, 2 blocks, 3 Euler steps from t = 1."""
    require_gpu()
    c = wi.get_config("tiny").replace(dtype=dtype, B=2, img_len=9, img_dim=32, T=3, H=8, W=12, guidance=5.0)
    case(f"step CFG {dtype}")
    x_t, gt, ot = _run(c, layers=2, steps=3, t0=1.0)
    _check(c, x_t, gt, ot)


TI2V_LAYERS = 30  # "Wan2.2 TI2V-5B" §2.2: the 5B model's block count


@pytest.fixture(scope="module")
def ti2v_model():
    """The TI2V-5B-shaped model with all 30 blocks (dim 3072, 24 x 128 heads, FFN 14336, 512 text tokens
    of dim 4096, 48-channel latent, 100-channel input): host weights in float64 for the oracle and the same
    values resident on the device.  Shared by the reduced-latent chain and the teacher-forced full-size
    checks, which differ only in the latent's T, H, W."""
    c = wi.get_config("ti2v-5b")
    case(f"TI2V-shaped model: drawing {TI2V_LAYERS} blocks")
    mw = wi.make_model_weights(c, seed=0)
    bws32 = wi.make_blocks_weights(c, TI2V_LAYERS, seed=0)
    model = R.DeviceModel(mw, c.dtype)
    blocks = []
    bws = []
    for w in bws32:
        blocks.append(R.DeviceBlock(w, c.dtype))
        bws.append({k: np.asarray(v, np.float64) for k, v in w.items()})
    del bws32
    torch.cuda.synchronize()
    case("TI2V-shaped model resident")
    return mw, bws, model, blocks


@pytest.mark.timeout(900)
def test_step_ti2v_shaped_reduced_chain(ti2v_model):
    """All 30 TI2V-5B-shaped blocks (48-channel latent, 100-channel input, dim 3072, 24 x 128 heads,
    FFN 14336, 512 text tokens, CFG batch 2, guidance 5, 4 Euler steps from t = 1) on a 32-token latent
    [48, 2, 8, 8], so the oracle runs the whole chain.
      * every step's latent against the oracle's sampler (rel-L2 <= 1e-2);
      * every step's per-row velocities (conditional, unconditional) against the oracle's DiT evaluated
        at the GPU's own latent of that step (teacher-forced, rel-L2 <= 1e-2 each);
      * every step's update dt * (v_u + s (v_c - v_u)) against the same: with per-row errors <= e, the
        combination's error is at most e (|1 - s| |v_u| + s |v_c|), so the bound relative to the
        combination is e (|1 - s| |v_u| + s |v_c|) / |v_u + s (v_c - v_u)|."""
    require_gpu()
    c = wi.get_config("ti2v-5b").replace(T=2, H=8, W=8)
    mw, bws, model, blocks = ti2v_model
    case(f"step TI2V-shaped reduced chain, {TI2V_LAYERS} blocks")
    x_t, z = wi.make_latents(c, seed=0)
    txt, img = wi.make_contexts(c, seed=0)
    t_emb, i_emb = R.embed_contexts(c, model, txt, img, c.B)
    caches = R.cross_kv_all(c, blocks, t_emb, i_emb, c.B)
    buf = R.alloc_step(c, c.B)
    xg, zg = dev(x_t), dev(z)
    steps, dt = c.steps, -1.0 / c.steps
    gpu_x, gpu_v = [np.asarray(x_t, np.float64)], []
    for k in range(steps):
        R.denoise_step(c, model, blocks, caches, xg, zg, 1.0 + k * dt, dt, c.guidance, buf, c.B)
        gpu_v.append(host(buf.v))
        gpu_x.append(host(xg))
    kw = dict(ln_eps=c.ln_eps, rms_eps=c.rms_eps, theta=c.rope_theta, freq_dim=c.freq_dim,
              out_channels=c.out_channels)
    case("oracle: the 30-block chain, 4 steps")
    _, traj = oracle.sample(x_t, z, steps, c.guidance, mw, bws, txt, img, c.heads, t0=1.0, **kw)
    s = c.guidance
    for k in range(steps):
        e_x = rel_l2(gpu_x[k + 1], traj[k])
        case(f"oracle: DiT at the GPU's step-{k} latent")
        v = oracle.dit_fwd(np.repeat(oracle.build_i2v_input(gpu_x[k], z), c.B, axis=0), 1.0 + k * dt, mw, bws, txt,
                           img, c.heads, **kw)
        e_vc, e_vu = rel_l2(gpu_v[k][0], v[0]), rel_l2(gpu_v[k][1], v[1])
        v_cfg = oracle.cfg_combine(v[0], v[1], s)
        bound = TOL[c.dtype] * (abs(1 - s) * np.linalg.norm(v[1]) + s * np.linalg.norm(v[0])) / np.linalg.norm(v_cfg)
        e_u = rel_l2(gpu_x[k + 1] - gpu_x[k], dt * v_cfg)
        print(f"[{c.name} x{TI2V_LAYERS}] step {k}: rel-L2 x={e_x:.3e} v_c={e_vc:.3e} v_u={e_vu:.3e} "
              f"update={e_u:.3e} (bound {bound:.3e})", flush=True)
        assert e_x <= TOL[c.dtype] and e_vc <= TOL[c.dtype] and e_vu <= TOL[c.dtype]
        assert e_u <= bound


@pytest.mark.timeout(900)
def test_step_ti2v_teacher_forced_full_size(ti2v_model):
    """The full TI2V-5B-shaped sampling run on the GPU (latent [48, 31, 44, 80] -> 27280 tokens, CFG batch 2,
    30 blocks, 4 Euler steps from t = 1).  Blocks 0, 15 and 29 of steps 0 and 3 are checked teacher-forced:
    the oracle runs each of them from the GPU's own block input (x, e0 and the embedded text the GPU
    holds at that point), on sampled query rows, so errors do not compound over the chain."""
    require_gpu()
    c = wi.get_config("ti2v-5b")
    mw, bws, model, blocks = ti2v_model
    case(f"step TI2V full size: S={c.S}, B={c.B}, {TI2V_LAYERS} blocks, 4 steps")
    x_t, z = wi.make_latents(c, seed=0)
    txt, img = wi.make_contexts(c, seed=0)
    t_emb, i_emb = R.embed_contexts(c, model, txt, img, c.B)
    caches = R.cross_kv_all(c, blocks, t_emb, i_emb, c.B)
    buf = R.alloc_step(c, c.B)
    xg, zg = dev(x_t), dev(z)
    steps, dt = c.steps, -1.0 / c.steps
    rows = wi.sample_rows(c, 32, seed=11)
    taps = {}
    for k in range(steps):
        tap = {i: [] for i in (0, 15, 29)} if k in (0, 3) else None
        R.denoise_step(c, model, blocks, caches, xg, zg, 1.0 + k * dt, dt, c.guidance, buf, c.B, tap=tap)
        if tap is not None:
            for i, lst in tap.items():
                d = lst[0]
                taps[(k, i)] = {"x_in": host(d["x_in"]), "e0": host(d["e0"]), "x_out": host(d["x_out"])[:, rows]}
            del tap
    assert np.isfinite(host(xg)).all()
    t_emb_h = host(t_emb)
    kv = {}
    for (k, i), d in sorted(taps.items()):
        case(f"oracle: step {k} block {i}, {len(rows)} rows")
        if i not in kv:
            kv[i] = [oracle.cross_kv(t_emb_h[b], bws[i]["wck"], bws[i]["bck"], bws[i]["wcv"], bws[i]["bcv"]) + (None, None)
                     for b in range(c.B)]
        ref = oracle.block_fwd(d["x_in"], d["e0"], bws[i], kv[i], c.grid, c.heads, rows=rows, ln_eps=c.ln_eps,
                               rms_eps=c.rms_eps, theta=c.rope_theta)
        xin = d["x_in"][:, rows]
        e_x, e_dx = rel_l2(d["x_out"], ref), rel_l2(d["x_out"] - xin, ref - xin)
        print(f"[{c.name} teacher-forced] step {k} block {i}: rel-L2 x_out={e_x:.3e} dx={e_dx:.3e}", flush=True)
        assert e_x <= TOL[c.dtype] and e_dx <= TOL[c.dtype]


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_step_graph_replays_match_eager(dtype):
    """A captured step (runtime.StepGraph, CFG pair, I2V) replayed three times, with eager library work,
    a torch copy and a synchronisation between the replays: every replay equals the eager step bit for
    bit (same kernels, same inputs)."""
    require_gpu()
    c = wi.get_config("tiny").replace(dtype=dtype, B=2, img_len=5, img_dim=32, guidance=5.0)
    case(f"step graph replays {dtype}")
    mw = wi.make_model_weights(c, seed=9)
    bws = [wi.make_block_weights(c, i, seed=9) for i in range(2)]
    x_t, z = wi.make_latents(c, seed=9)
    txt, img = wi.make_contexts(c, seed=9)
    model = R.DeviceModel(mw, c.dtype)
    blocks = [R.DeviceBlock(w, c.dtype) for w in bws]
    t_emb, i_emb = R.embed_contexts(c, model, txt, img, c.B)
    caches = R.cross_kv_all(c, blocks, t_emb, i_emb, c.B)
    zg = dev(z)
    x0 = dev(x_t)
    # eager reference, on its own buffers
    buf_e = R.alloc_step(c, c.B)
    x_e = x0.clone()
    R.denoise_step(c, model, blocks, caches, x_e, zg, 0.75, -0.25, c.guidance, buf_e, c.B)
    ref = host(x_e)
    # captured step
    buf_g = R.alloc_step(c, c.B)
    x_g = x0.clone()
    g = R.StepGraph(c, model, blocks, caches, x_g, zg, 0.75, -0.25, c.guidance, buf_g, c.B)
    assert np.array_equal(host(x_g), x_t.astype(np.float32))  # capturing ran nothing
    for r in range(3):
        x_g.copy_(x0)
        g.replay()
        got = host(x_g)
        assert np.array_equal(got, ref), (r, float(np.abs(got - ref).max()))
        # eager work between replays, on the eager buffers
        x_e.copy_(x0)
        R.denoise_step(c, model, blocks, caches, x_e, zg, 0.5, -0.25, c.guidance, buf_e, c.B)
        torch.cuda.synchronize()
