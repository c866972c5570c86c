"""Quantised (INT8 Q.K / FP8 P.V) attention against the oracle.

* Quantisers: codes and scales bit-exact against oracle/quant.py (float32 decisions on both sides).
* Attention: against the plain float64 softmax attention of the original bf16 inputs, within a
  bound derived from the code precisions.  Per-element relative rounding errors are, in RMS: INT8 Q
  and K codes ~0.7 % and ~0.9 % of an element (scale/sqrt(12) against amax/127), i.e. ~0.011 on a
  unit-variance score; E4M3 for V and for P ~2.4 % each (half a step of 2^-3 over sqrt(3), averaged
  over mantissas).  The output error is then ~sqrt(0.024^2 + 0.024^2 + 0.011^2) ~= 0.036 of the
  output; the bound is one E4M3 unit roundoff, 2^-4 = 0.0625.  With the codes decoded exactly, the
  only remaining error is P's rounding (~0.026 measured); that comparison is held to the largest RMS
  relative E4M3 rounding error, 2^-4 / sqrt(3) ~= 0.036 (uniform error at the bottom of a binade).
* LSE: the score error (~0.011 RMS per score, averaged over keys) moves the log-sum-exp by about that
  much; bound 0.05 absolute.
"""
import numpy as np
import pytest
import torch

import oracle
import wan_inputs as wi
from oracle import quant as OQ
from tests.gpu_util import case, dev, host, rel_l2, require_gpu
from video_diffusion_transformer_step_amd import _lib as L

pytestmark = pytest.mark.gpu

TOL_OUT = 2.0 ** -4
TOL_DEQ = 2.0 ** -4 / 3 ** 0.5
TOL_LSE = 0.05


def _pos_to_key():
    """Position p of a 64-key E4M3 V^T tile -> key index (layout documented in wan.h)."""
    m = np.empty(64, np.int64)
    for h in range(2):
        for kb in range(2):
            for r in range(16):
                m[h * 32 + kb * 16 + r] = kb * 32 + (r // 4) * 8 + h * 4 + r % 4
    return m


def _inputs(rng, B, Sq, Sk, H, hd):
    q = wi.bf16_round(rng.standard_normal((B, Sq, H, hd)).astype(np.float32))
    k = wi.bf16_round(rng.standard_normal((B, Sk, H, hd)).astype(np.float32))
    v = wi.bf16_round(rng.standard_normal((B, Sk, H, hd)).astype(np.float32))
    return q, k, v


def _run(q, k, v):
    B, Sq, H, hd = q.shape
    Sk = k.shape[1]
    qd, kd, vd = (dev(a, torch.bfloat16) for a in (q, k, v))
    codes = L.Q8Codes(B, Sq, Sk, H, hd)
    ws = torch.empty(L.attention_q8_quantize_ws_bytes(B, Sk, H, hd), dtype=torch.uint8, device="cuda")
    L.attention_q8_quantize(qd, kd, vd, codes, ws)
    o = torch.empty_like(qd)
    lse = torch.empty((B, H, Sq), dtype=torch.float32, device="cuda")
    L.attention_q8_fwd(codes, o, lse)
    torch.cuda.synchronize()
    return codes, o, lse


def _expected_v8t(v):
    codes, scales = OQ.quant_v_e4m3(v)  # codes [B, S, H, d]
    B, S, H, d = v.shape
    pad = -(-S // 128) * 128
    vt = np.zeros((B, H, d, pad), np.uint8)
    vt[:, :, :, :S] = codes.transpose(0, 2, 3, 1)
    p2k = _pos_to_key()
    out = np.empty_like(vt)
    for t in range(pad // 64):
        out[..., t * 64:(t + 1) * 64] = vt[..., t * 64 + p2k]
    return out, scales


@pytest.mark.parametrize("Sq,Sk", [(300, 300), (70, 130), (1, 17)])
def test_quantize_bit_exact(Sq, Sk):
    require_gpu()
    B, H, hd = 2, 3, 128
    case(f"q8 quantize B={B} Sq={Sq} Sk={Sk} H={H}")
    rng = np.random.default_rng(Sq + Sk)
    q, k, v = _inputs(rng, B, Sq, Sk, H, hd)
    q[1, 0, 2] = 0.0  # an all-zero (token, head) group
    k[0, :, 1] = wi.bf16_round(k[0, :, 1] * 10.0)  # still exactly what the device holds
    v[1, :, 0, 7] = 0.0  # an all-zero V channel
    codes, _, _ = _run(q, k, v)
    q8, sq = OQ.quant_q_int8(q)
    k8, sk = OQ.quant_k_int8(k)
    v8t, sv = _expected_v8t(v)
    assert np.array_equal(codes.q8.cpu().numpy(), q8)
    assert np.array_equal(codes.sq.cpu().numpy().view(np.uint32), sq.view(np.uint32))
    assert np.array_equal(codes.k8.cpu().numpy(), k8)
    assert np.array_equal(codes.sk.cpu().numpy().view(np.uint32), sk.view(np.uint32))
    got = codes.v8t.cpu().numpy()
    assert np.array_equal(got, v8t), int((got != v8t).sum())
    assert np.array_equal(codes.sv.cpu().numpy().view(np.uint32), sv.view(np.uint32))


def _check_attention(q, k, v, o, lse, rows, report=None):
    B, _, H, _ = q.shape
    q8, sq = OQ.quant_q_int8(q[:, rows])  # per-token groups: the sampled rows suffice
    k8, sk = OQ.quant_k_int8(k)
    v8, sv = OQ.quant_v_e4m3(v)
    kb = np.repeat(sk, 64, axis=2)[:, :, :k.shape[1]]  # [B, H, Sk]
    worst = [0.0, 0.0, 0.0]
    for b in range(B):
        for h in range(H):
            ref, ref_lse = oracle.attention_lse(q[b, rows, h], k[b, :, h], v[b, :, h])
            e = rel_l2(o[b, rows, h], ref)
            # the same attention on the decoded codes: only P's rounding remains
            qd = q8[b, :, h].astype(np.float64) * sq[b, h][:, None]
            kd = k8[b, :, h].astype(np.float64) * kb[b, h][:, None]
            vd = OQ.e4m3_decode(v8[b, :, h]) * sv[b, h][None, :]
            deq = oracle.attention(qd, kd, vd)
            e2 = rel_l2(o[b, rows, h], deq)
            el = float(np.max(np.abs(lse[b, h, rows] - ref_lse)))
            worst = [max(worst[0], e), max(worst[1], e2), max(worst[2], el)]
            assert e <= TOL_OUT, (b, h, e)
            assert e2 <= TOL_DEQ, (b, h, e2)
            assert el <= TOL_LSE, (b, h, el)
    print(f"[fp8 attention] rel-L2 vs exact {worst[0]:.4f}, vs decoded codes {worst[1]:.4f}, lse {worst[2]:.4f}",
          flush=True)


@pytest.mark.parametrize("Sq,Sk", [(300, 300), (257, 70), (33, 1000)])
def test_attention_q8_small(Sq, Sk):
    """Every element at sizes spanning several tiles with ragged tails on both sides."""
    require_gpu()
    B, H, hd = 2, 2, 128
    case(f"q8 attention B={B} Sq={Sq} Sk={Sk} H={H}")
    rng = np.random.default_rng(7 * Sq + Sk)
    q, k, v = _inputs(rng, B, Sq, Sk, H, hd)
    _, o, lse = _run(q, k, v)
    _check_attention(q, k, v, host(o), host(lse), np.arange(Sq))


def test_attention_q8_sharp_drifting_scores():
    """Sharp, drifting rows: q and k scaled by 4 and each key's norm growing x1 to x4 along 2000 keys,
    so scores reach hundreds and the running maximum moves on many tiles.  At such scores the INT8
    codes' ~1 % error per product is an absolute score error near 0.5, beyond any fixed bound against
    the exact result; against attention over the decoded codes only P's E4M3 rounding remains, which
    does not depend on the scores' size.  So o is held to TOL_DEQ and lse to TOL_LSE against the
    decoded codes, every element."""
    require_gpu()
    B, Sq, Sk, H, hd = 1, 300, 2000, 2, 128
    case(f"q8 attention sharp drifting scores Sq={Sq} Sk={Sk}")
    rng = np.random.default_rng(77)
    q = wi.bf16_round((4.0 * rng.standard_normal((B, Sq, H, hd))).astype(np.float32))
    grow = (1.0 + 3.0 * np.arange(Sk) / (Sk - 1))[None, :, None, None]
    k = wi.bf16_round((4.0 * rng.standard_normal((B, Sk, H, hd)) * grow).astype(np.float32))
    v = wi.bf16_round(rng.standard_normal((B, Sk, H, hd)).astype(np.float32))
    _, o, lse = _run(q, k, v)
    got, got_lse = host(o), host(lse)
    assert np.isfinite(got).all() and np.isfinite(got_lse).all()
    q8, sq = OQ.quant_q_int8(q)
    k8, sk = OQ.quant_k_int8(k)
    v8, sv = OQ.quant_v_e4m3(v)
    kb = np.repeat(sk, 64, axis=2)[:, :, :Sk]
    worst = [0.0, 0.0]
    for h in range(H):
        qd = q8[0, :, h].astype(np.float64) * sq[0, h][:, None]
        kd = k8[0, :, h].astype(np.float64) * kb[0, h][:, None]
        vd = OQ.e4m3_decode(v8[0, :, h]) * sv[0, h][None, :]
        ref, ref_lse = oracle.attention_lse(qd, kd, vd)
        e = rel_l2(got[0, :, h], ref)
        el = float(np.max(np.abs(got_lse[0, h] - ref_lse)))
        worst = [max(worst[0], e), max(worst[1], el)]
        assert e <= TOL_DEQ, (h, e)
        assert el <= TOL_LSE, (h, el)
    print(f"[fp8 attention sharp] rel-L2 vs decoded codes {worst[0]:.4f}, lse {worst[1]:.4f}", flush=True)


def test_attention_q8_special():
    """An all-zero query attends uniformly (scale 0); an all-zero key block gives those keys score 0."""
    require_gpu()
    B, S, H, hd = 1, 200, 1, 128
    case("q8 attention special cases")
    rng = np.random.default_rng(11)
    q, k, v = _inputs(rng, B, S, S, H, hd)
    q[0, 5] = 0.0
    k[0, 64:128] = 0.0
    _, o, lse = _run(q, k, v)
    got = host(o)
    assert rel_l2(got[0, 5, 0], v[0, :, 0].mean(0)) <= TOL_OUT
    _check_attention(q, k, v, got, host(lse), np.arange(S))


def test_attention_q8_full_size():
    """The 1.3B-shaped self-attention (32760 tokens, 12 heads x 128), sampled query rows."""
    require_gpu()
    B, S, H, hd = 1, 32760, 12, 128
    case(f"q8 attention full size S={S} H={H}")
    rng = np.random.default_rng(21)
    q, k, v = _inputs(rng, B, S, S, H, hd)
    _, o, lse = _run(q, k, v)
    rows = np.unique(np.concatenate([[0, S - 1, 255, 256], np.random.default_rng(22).choice(S, 24, replace=False)]))
    _check_attention(q, k, v, host(o), host(lse), rows)
