"""Helpers shared by the GPU parity tests (device transfer, error metrics)."""
from __future__ import annotations

import numpy as np
import pytest
import torch


def require_gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU visible")


def dev(a, dtype=torch.float32):
    return torch.from_numpy(np.ascontiguousarray(a, dtype=np.float32)).cuda().to(dtype).contiguous()


def host(t) -> np.ndarray:
    torch.cuda.synchronize()
    return t.detach().float().cpu().numpy().astype(np.float64)


def rel_l2(got, ref) -> float:
    got, ref = np.asarray(got, np.float64), np.asarray(ref, np.float64)
    den = np.linalg.norm(ref)
    return float(np.linalg.norm(got - ref) / (den if den > 0 else 1.0))


def ulp_diff_f32(a, b) -> np.ndarray:
    """|a - b| in units of float32 ulps (ordered-integer distance)."""
    ai = np.asarray(a, np.float32).view(np.int32).astype(np.int64)
    bi = np.asarray(b, np.float32).view(np.int32).astype(np.int64)
    ai = np.where(ai < 0, -(ai & 0x7FFFFFFF), ai)
    bi = np.where(bi < 0, -(bi & 0x7FFFFFFF), bi)
    return np.abs(ai - bi)


def case(msg: str):
    """Print (and flush) what the next GPU step runs, so a fault names its case."""
    print(f"[gpu case] {msg}", flush=True)
