"""Pins of the quantised-attention oracle (oracle/quant.py), no GPU.

The E4M3 encoder is checked against PyTorch's float8_e4m3fn conversion (an independent
implementation of the OCP format) over every code and over dense sweeps with ties, and against the
format's defining values; the INT8 and per-group scale definitions against their invariants.
Planted mistakes (a wrong exponent bias, ties away from zero, a 1/128 scale, a different key-block
size) must each fail one of these pins."""
import numpy as np
import pytest
import torch

from oracle import quant as Q


def _torch_e4m3(x):
    return torch.from_numpy(np.asarray(x, np.float32)).to(torch.float8_e4m3fn).view(torch.uint8).numpy()


def pin_e4m3_defining_values(q):
    # OCP E4M3: bias 7, subnormals m * 2^-9, largest finite 1.75 * 2^8 = 448, no infinities
    assert q.e4m3_decode(0x38) == 1.0 and q.e4m3_decode(0xB8) == -1.0
    assert q.e4m3_decode(0x7E) == 448.0 and np.isnan(q.e4m3_decode(0x7F))
    assert q.e4m3_decode(0x01) == 2.0 ** -9 and q.e4m3_decode(0x08) == 2.0 ** -6
    assert q.e4m3_decode(0x07) == 7 * 2.0 ** -9


def pin_e4m3_matches_library(q):
    # every finite code round-trips, and agrees with an independent conversion
    codes = np.array([c for c in range(256) if (c & 0x7F) != 0x7F], dtype=np.uint8)
    vals = q.e4m3_decode(codes)
    assert np.array_equal(q.e4m3_encode(vals)[vals != 0], codes[vals != 0])
    rng = np.random.default_rng(3)
    x = np.concatenate([rng.uniform(-448, 448, 20000), rng.uniform(-1, 1, 20000) * 2.0 ** rng.integers(-12, 1, 20000),
                        np.array([464.0, -464.0, 460.0, 1.0625, 17.0, 19.0, 2 ** -10, 3 * 2 ** -11])])
    grid = np.sort(np.unique(np.abs(vals[np.isfinite(vals)])))
    mids = (grid[:-1] + grid[1:]) / 2  # every tie between neighbours
    x = np.concatenate([x, mids, -mids]).astype(np.float32)
    assert np.array_equal(q.e4m3_encode(x), _torch_e4m3(x))


def pin_int8_group(q):
    rng = np.random.default_rng(4)
    x = (rng.standard_normal(128) * 3).astype(np.float32)
    c, s = q.int8_group(x)
    i = int(np.argmax(np.abs(x)))
    assert abs(int(c[i])) == 127 and np.sign(c[i]) == np.sign(x[i])
    assert s == np.float32(np.max(np.abs(x)) / np.float32(127))
    assert np.all(np.abs(x - c.astype(np.float64) * s) <= s * (0.5 + 1e-5))
    c0, s0 = q.int8_group(np.zeros(7, np.float32))
    assert s0 == 0 and not c0.any()
    # half-way cases go to the even integer: amax 127 makes the scale 1
    c1, _ = q.int8_group(np.array([127.0, 2.5, -3.5, 0.5], np.float32))
    assert c1.tolist() == [127, 2, -4, 0]


def pin_k_blocks(q):
    rng = np.random.default_rng(5)
    k = rng.standard_normal((1, 130, 2, 8)).astype(np.float32)
    codes, scales = q.quant_k_int8(k)
    assert scales.shape == (1, 2, 3)
    k2 = k.copy()
    k2[0, 70, 1, 3] = 1e3  # a spike in block 1 of head 1 changes that block only
    codes2, scales2 = q.quant_k_int8(k2)
    assert np.array_equal(codes2[0, :64], codes[0, :64]) and np.array_equal(codes2[0, 128:], codes[0, 128:])
    assert np.array_equal(codes2[0, 64:128, 0], codes[0, 64:128, 0])
    assert scales2[0, 1, 1] == np.float32(np.float32(1e3) / np.float32(127))
    for t in range(3):  # each block's largest magnitude maps to +-127
        blk = codes[0, t * 64:(t + 1) * 64, 0]
        assert np.max(np.abs(blk.astype(int))) == 127


def pin_v_channels(q):
    rng = np.random.default_rng(6)
    v = (rng.standard_normal((2, 50, 3, 16)) * rng.uniform(0.1, 5, 16)).astype(np.float32)
    v[1, :, 2, 5] = 0.0  # an all-zero channel
    codes, scales = q.quant_v_e4m3(v)
    deq = q.e4m3_decode(codes) * scales[:, None, :, :]
    amax = np.abs(v).max(axis=1)
    assert np.allclose(np.abs(q.e4m3_decode(codes)).max(axis=1)[amax > 0], 448.0)
    assert scales[1, 2, 5] == 0 and not codes[1, :, 2, 5].any()
    # relative error within half an E4M3 step (2^-4) for normal codes; subnormals within 2^-10 * scale
    err = np.abs(deq - v)
    bound = np.maximum(np.abs(v) * 2.0 ** -4, 2.0 ** -10 * scales[:, None, :, :]) * (1 + 1e-6)
    assert np.all(err <= bound)


def pin_rows_and_tensor(q):
    rng = np.random.default_rng(7)
    x = (rng.standard_normal((5, 96)) * rng.uniform(0.01, 10, (5, 1))).astype(np.float32)
    x[2] = 0.0
    codes, scales = q.quant_rows_e4m3(x)
    assert scales[2] == 0 and not codes[2].any()
    for m in (0, 1, 3, 4):  # each row's largest magnitude maps to +-448, independently of the others
        assert np.max(np.abs(q.e4m3_decode(codes[m]))) == 448.0
        assert scales[m] == np.float32(np.max(np.abs(x[m])) / np.float32(448))
    c2, s2 = q.quant_rows_e4m3(x[[4, 0]])
    assert np.array_equal(c2[1], codes[0]) and s2[1] == scales[0]
    w = rng.standard_normal((7, 96)).astype(np.float32)
    wc, ws = q.quant_tensor_e4m3(w)
    assert np.max(np.abs(q.e4m3_decode(wc))) == 448.0 and ws == np.float32(np.abs(w).max() / np.float32(448))
    # the scaled product of exactly representable codes is the plain product
    y = q.gemm_e4m3(codes, scales, wc, ws)
    ref = (q.e4m3_decode(codes) * scales[:, None].astype(np.float64)) @ (q.e4m3_decode(wc) * float(ws)).T
    assert np.allclose(y, ref, rtol=1e-12, atol=0)
    # and approximates x w^T within the E4M3 rounding of both operands
    exact = x.astype(np.float64) @ w.astype(np.float64).T
    rows = [0, 1, 3, 4]
    rel = np.linalg.norm(y[rows] - exact[rows]) / np.linalg.norm(exact[rows])
    assert rel < 2.0 ** -4, rel


PINS = [pin_e4m3_defining_values, pin_e4m3_matches_library, pin_int8_group, pin_k_blocks, pin_v_channels,
        pin_rows_and_tensor]


@pytest.mark.parametrize("pin", PINS, ids=lambda p: p.__name__)
def test_quant_pin(pin):
    pin(Q)


# ---- planted mistakes --------------------------------------------------------------------------
class _Mutant:
    """The oracle module with one function replaced."""

    def __init__(self, **over):
        self.__dict__.update({k: getattr(Q, k) for k in Q.__all__})
        self.__dict__.update(over)


def _values_bias8():
    vals = Q.e4m3_values().copy()
    return vals / 2.0  # exponent bias 8 instead of 7


def _mutant_bias8():
    vals = _values_bias8()

    def dec(codes):
        c = np.asarray(codes).astype(np.int64) & 0xFF
        mag = vals[c & 0x7F]
        return np.where(c & 0x80, -mag, mag)

    def enc(x):
        return Q.e4m3_encode(np.asarray(x, np.float64) * 2.0)
    return _Mutant(e4m3_decode=dec, e4m3_encode=enc)


def _mutant_ties_away():
    def enc(x):
        # nearest value, but exact ties go to the larger magnitude instead of the even code
        x = np.asarray(x, np.float64)
        grid = Q.e4m3_values().copy()
        grid[127] = 480.0
        a = np.abs(x)
        hi = np.clip(np.searchsorted(grid, a, side="left"), 0, 127)
        lo = np.clip(hi - 1, 0, 127)
        pick = np.where(a - grid[lo] < grid[hi] - a, lo, hi)
        return (pick | (np.signbit(x).astype(np.int64) << 7)).astype(np.uint8)
    return _Mutant(e4m3_encode=enc)


def _mutant_scale_128():
    def grp(x):
        x = np.asarray(x, np.float32)
        amax = np.float32(np.max(np.abs(x))) if x.size else np.float32(0)
        if amax == 0:
            return np.zeros(x.shape, np.int8), np.float32(0)
        return np.clip(np.rint(x * (np.float32(128) / amax)), -127, 127).astype(np.int8), amax / np.float32(128)
    m = _Mutant(int8_group=grp)
    return m


def _mutant_block_128():
    def qk(k):
        k = np.asarray(k, np.float32)
        B, S, H, _ = k.shape
        nb = -(-S // 64)
        codes = np.empty(k.shape, np.int8)
        scales = np.empty((B, H, nb), np.float32)
        for b in range(B):
            for h in range(H):
                for t in range(nb):
                    lo = (t // 2) * 128
                    sl = slice(lo, min(S, lo + 128))
                    c, s = Q.int8_group(k[b, sl, h])
                    own = slice(t * 64, min(S, (t + 1) * 64))
                    codes[b, own, h] = c[own.start - lo:own.stop - lo]
                    scales[b, h, t] = s
        return codes, scales
    return _Mutant(quant_k_int8=qk)


MUTANTS = {"e4m3_bias_8": _mutant_bias8, "e4m3_ties_away": _mutant_ties_away,
           "int8_scale_128": _mutant_scale_128, "k_block_128": _mutant_block_128}


@pytest.mark.parametrize("name", sorted(MUTANTS))
def test_quant_mutant_caught(name):
    m = MUTANTS[name]()
    caught = []
    for pin in PINS:
        try:
            pin(m)
        except AssertionError:
            caught.append(pin.__name__)
        except Exception as exc:  # a crash on a planted mistake also counts
            caught.append(f"{pin.__name__}({type(exc).__name__})")
    assert caught, name
