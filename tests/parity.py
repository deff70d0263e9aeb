"""Comparison helpers shared by the GPU parity tests."""
from __future__ import annotations

import numpy as np

# bf16 attention gate: |gpu - ref| <= ATOL + RTOL * |ref| for every element
ATOL = 2e-2
RTOL = 1e-2


def close_stats(gpu: np.ndarray, ref: np.ndarray) -> dict:
    diff = np.abs(gpu - ref)
    big = np.abs(ref) >= 1e-1
    return {
        "max_abs": float(diff.max()) if diff.size else 0.0,
        "rel_l2": float(np.linalg.norm(gpu - ref) / max(np.linalg.norm(ref), 1e-300)) if diff.size else 0.0,
        "max_rel_big": float((diff[big] / np.abs(ref[big])).max()) if big.any() else 0.0,
        "n": int(diff.size),
    }


def assert_attention_close(gpu, ref, atol=ATOL, rtol=RTOL, rel_l2=None, label=""):
    gpu = np.asarray(gpu, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    assert gpu.shape == ref.shape, (gpu.shape, ref.shape)
    assert np.all(np.isfinite(gpu)), f"{label}: non-finite GPU output"
    st = close_stats(gpu, ref)
    bad = np.abs(gpu - ref) > atol + rtol * np.abs(ref)
    assert not bad.any(), f"{label}: {int(bad.sum())} elements outside the gate; {st}"
    # the max-abs half of the bar on its own (the elementwise form above lets an element
    # with |ref| near 1 be off by atol + rtol)
    assert st["max_abs"] <= atol, f"{label}: max-abs {st['max_abs']} > {atol}; {st}"
    if rel_l2 is not None:
        assert st["rel_l2"] <= rel_l2, f"{label}: rel-L2 {st['rel_l2']} > {rel_l2}; {st}"
    return st


def pool_bits(t) -> np.ndarray:
    """Raw bit patterns of a device pool as a numpy array (uint16 for bf16, uint32 for fp32)."""
    import torch
    if t.dtype == torch.bfloat16:
        return t.view(torch.int16).cpu().numpy().view(np.uint16)
    return t.view(torch.int32).cpu().numpy().view(np.uint32)


def oracle_bits(pool: np.ndarray) -> np.ndarray:
    return pool if pool.dtype == np.uint16 else pool.view(np.uint32)
