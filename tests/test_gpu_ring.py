"""Sequence-sharded (ring) attention pieces against the oracle: attention of all queries to one
key/value chunk with its log-sum-exp, and the merge of chunk results, at small ragged sizes
(every element) and at the shapes one GPU of a sharded 32760-token step would run (sampled rows).

Tolerances: o to the dtype's rel-L2 bound (bf16 1e-2, fp32 1e-4); lse to rel-L2 1e-4 and max
absolute error 1e-3 in both dtypes.  The lse bound follows from the arithmetic: scores are fp32
dot products of exactly representable inputs (bf16 products are exact in fp32), the normaliser is
an fp32 sum of fp32 exponentials, so its log is good to ~1e-5 absolute for these magnitudes; 1e-3
leaves two orders of margin and still catches a base-2 log (off by a factor 1.44), a dropped
max (off by the max) or a dropped 1/sqrt(hd) scale."""
import numpy as np
import pytest
import torch

import oracle
import wan_inputs as wi
from tests.gpu_util import case, dev, host, rel_l2, require_gpu
from video_diffusion_transformer_step_amd import _lib as L

pytestmark = pytest.mark.gpu

TOL = {"f32": 1e-4, "bf16": 1e-2}
LSE_ABS = 1e-3


def _tdt(dtype):
    return torch.bfloat16 if dtype == "bf16" else torch.float32


def _qkv(rng, B, Sq, Sk, H, hd, dtype):
    q = rng.standard_normal((B, Sq, H, hd)).astype(np.float32)
    k = rng.standard_normal((B, Sk, H, hd)).astype(np.float32)
    v = rng.standard_normal((B, Sk, H, hd)).astype(np.float32)
    if dtype == "bf16":
        q, k, v = wi.bf16_round(q), wi.bf16_round(k), wi.bf16_round(v)
    return q, k, v


def _vt_bytes(qd, kd):
    B, _, H, hd = qd.shape
    return B * H * hd * (-(-kd.shape[1] // 64) * 64) * qd.element_size()


def _partial(qd, kd, vd, want_lse=True, unsplit=False):
    """The chunk attention with the workspace the library asks for (key splits where the grid would
    leave compute units idle), or, with unsplit, a workspace holding only V^T."""
    B, Sq, H, hd = qd.shape
    o = torch.empty_like(qd)
    lse = torch.empty((B, H, Sq), dtype=torch.float32, device="cuda") if want_lse else None
    n = _vt_bytes(qd, kd) if unsplit else L.attention_partial_ws_bytes(L.dtype_code(qd.dtype), B, Sq, kd.shape[1], H, hd)
    ws = torch.empty(n, dtype=torch.uint8, device="cuda")
    L.attention_partial_fwd(qd, kd, vd, o, lse, ws)
    return o, lse


def _check_rows(got_o, got_lse, q, k, v, rows, dtype):
    """got_o [B, Sq, H, hd], got_lse [B, H, Sq] against the oracle for query rows `rows`."""
    B, _, H, _ = q.shape
    for b in range(B):
        for h in range(H):
            ref_o, ref_lse = oracle.attention_lse(q[b, rows, h], k[b, :, h], v[b, :, h])
            e = rel_l2(got_o[b, rows, h], ref_o)
            assert e <= TOL[dtype], (b, h, e)
            gl = got_lse[b, h, rows]
            assert rel_l2(gl, ref_lse) <= 1e-4, (b, h)
            assert np.max(np.abs(gl - ref_lse)) <= LSE_ABS, (b, h, np.max(np.abs(gl - ref_lse)))


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
@pytest.mark.parametrize("hd", [64, 128])
def test_chunks_merge_small(dtype, hd):
    """Queries against three ragged key chunks (17, 128 and 155 keys: under one tile, two whole
    tiles, a ragged tail), each chunk's (o, lse) checked, then merged and checked against
    attention over all 300 keys -- every element."""
    require_gpu()
    B, S, H = 2, 300, 2
    case(f"ring chunks dtype={dtype} hd={hd} B={B} S={S} H={H}")
    rng = np.random.default_rng(500 + hd)
    q, k, v = _qkv(rng, B, S, S, H, hd, dtype)
    td = _tdt(dtype)
    qd = dev(q, td)
    cuts = (0, 17, 145, 300)
    parts, lses = [], []
    rows = np.arange(S)
    for lo, hi in zip(cuts[:-1], cuts[1:]):
        kd, vd = dev(k[:, lo:hi], td), dev(v[:, lo:hi], td)
        o, lse = _partial(qd, kd, vd)
        _check_rows(host(o), host(lse), q, k[:, lo:hi], v[:, lo:hi], rows, dtype)
        parts.append(o)
        lses.append(lse)
    out = torch.empty_like(qd)
    out_lse = torch.empty_like(lses[0])
    L.attention_lse_merge(parts, lses, out, out_lse)
    _check_rows(host(out), host(out_lse), q, k, v, rows, dtype)
    # without the lse output the chunk result is the same attention
    o2, _ = _partial(qd, dev(k[:, 17:145], td), dev(v[:, 17:145], td), want_lse=False)
    assert torch.equal(o2, parts[1])


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
@pytest.mark.parametrize("hd", [64, 128])
def test_partial_key_splits_small(dtype, hd):
    """A grid of one or two query tiles against 3000 keys: the library splits the keys (the last
    split ragged) and merges; every element of o and lse against the oracle, with and without the lse
    output, and against the unsplit call (V^T-only workspace)."""
    require_gpu()
    B, Sq, Sk, H = 1, 200, 3000, 2
    case(f"partial key splits dtype={dtype} hd={hd} Sq={Sq} Sk={Sk}")
    rng = np.random.default_rng(900 + hd)
    q, k, v = _qkv(rng, B, Sq, Sk, H, hd, dtype)
    td = _tdt(dtype)
    qd, kd, vd = dev(q, td), dev(k, td), dev(v, td)
    assert L.attention_partial_ws_bytes(L.dtype_code(td), B, Sq, Sk, H, hd) > _vt_bytes(qd, kd)  # split taken
    o, lse = _partial(qd, kd, vd)
    rows = np.arange(Sq)
    _check_rows(host(o), host(lse), q, k, v, rows, dtype)
    o2, _ = _partial(qd, kd, vd, want_lse=False)
    assert torch.equal(o2, o)
    o1, lse1 = _partial(qd, kd, vd, unsplit=True)
    _check_rows(host(o1), host(lse1), q, k, v, rows, dtype)
    assert rel_l2(host(o), host(o1)) <= TOL[dtype]


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
@pytest.mark.parametrize("hd", [64, 128])
def test_attention_sharp_drifting_scores(dtype, hd):
    """Sharp, drifting softmax rows: q and k scaled by 4 and each key's norm growing along the
    sequence (x1 to x4), so scores reach hundreds and the row maximum keeps rising from tile to tile.
    The running maximum then moves (O and l rescaled, weights recomputed) on many tiles rather than on
    the first only.  Every element of o and lse against the oracle, unsplit and with key splits."""
    require_gpu()
    B, Sq, Sk, H = 1, 300, 2000, 2
    case(f"sharp drifting scores dtype={dtype} hd={hd}")
    rng = np.random.default_rng(1200 + hd)
    q = 4.0 * rng.standard_normal((B, Sq, H, hd)).astype(np.float32)
    grow = (1.0 + 3.0 * np.arange(Sk) / (Sk - 1)).astype(np.float32)[None, :, None, None]
    k = (4.0 * rng.standard_normal((B, Sk, H, hd)) * grow).astype(np.float32)
    v = rng.standard_normal((B, Sk, H, hd)).astype(np.float32)
    if dtype == "bf16":
        q, k, v = wi.bf16_round(q), wi.bf16_round(k), wi.bf16_round(v)
    td = _tdt(dtype)
    qd, kd, vd = dev(q, td), dev(k, td), dev(v, td)
    rows = np.arange(Sq)
    for unsplit in (True, False):
        o, lse = _partial(qd, kd, vd, unsplit=unsplit)
        _check_rows(host(o), host(lse), q, k, v, rows, dtype)


def test_merge_single_part_is_identity():
    """One part merges to itself (weights exp(lse - lse) = 1)."""
    require_gpu()
    case("ring merge single part")
    rng = np.random.default_rng(7)
    q, k, v = _qkv(rng, 1, 130, 70, 3, 64, "f32")
    o, lse = _partial(dev(q), dev(k), dev(v))
    out = torch.empty_like(o)
    out_lse = torch.empty_like(lse)
    L.attention_lse_merge([o], [lse], out, out_lse)
    assert torch.allclose(out, o, rtol=1e-6, atol=1e-7)
    assert torch.allclose(out_lse, lse, rtol=1e-7, atol=1e-6)


def _sample_rows(S, R, seed):
    rng = np.random.default_rng(seed)
    return np.unique(np.concatenate([[0, S - 1, S // 2], rng.choice(S, R, replace=False)]))


def test_ulysses_shard_shape():
    """One GPU's share under head sharding of the 14B-shaped step (40 heads over 8 GPUs = 5 heads)
    at the full 32760 tokens: one chunk holding all keys, sampled query rows."""
    require_gpu()
    B, S, H, hd = 1, 32760, 5, 128
    case(f"ring ulysses shard B={B} S={S} H={H} hd={hd}")
    rng = np.random.default_rng(31)
    q, k, v = _qkv(rng, B, S, S, H, hd, "bf16")
    o, lse = _partial(dev(q, torch.bfloat16), dev(k, torch.bfloat16), dev(v, torch.bfloat16))
    rows = _sample_rows(S, 48, 32)
    _check_rows(host(o), host(lse), q, k, v, rows, "bf16")


def test_ring_shard_pair_shape():
    """One GPU's step under sequence sharding of the 1.3B-shaped step over 8 GPUs: 4095 local
    queries against two visiting 4095-token key/value shards (12 heads x 128), merged; sampled
    rows against attention over the 8190 keys."""
    require_gpu()
    B, Sq, H, hd = 1, 4095, 12, 128
    case(f"ring shard pair B={B} Sq={Sq} H={H} hd={hd}")
    rng = np.random.default_rng(41)
    q, k, v = _qkv(rng, B, Sq, 2 * Sq, H, hd, "bf16")
    qd = dev(q, torch.bfloat16)
    parts, lses = [], []
    for lo in (0, Sq):
        o, lse = _partial(qd, dev(k[:, lo:lo + Sq], torch.bfloat16), dev(v[:, lo:lo + Sq], torch.bfloat16))
        parts.append(o)
        lses.append(lse)
    out = torch.empty_like(qd)
    out_lse = torch.empty_like(lses[0])
    L.attention_lse_merge(parts, lses, out, out_lse)
    rows = _sample_rows(Sq, 32, 42)
    _check_rows(host(out), host(out_lse), q, k, v, rows, "bf16")
