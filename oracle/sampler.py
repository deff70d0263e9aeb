"""Plain CPU oracle of the temperature sampler.

TEST INFRASTRUCTURE ONLY. Imported by tests/; never by the library, with which it shares
no code.

Source: [P3] "Nano-vLLM 代码解析", section 4.3 采样器: a row's logits are divided by its
temperature, turned into probabilities by a softmax, each probability is divided by an
independent Exp(1) draw clamped below at 1e-10, and the index of the largest quotient is the
sampled token ([P1] SamplingParams requires temperature > 1e-10).

The random draws are those the kernel is specified to use: Philox4x64-10 (Salmon et al.,
"Parallel random numbers: as easy as 1, 2, 3", SC 2011), key (seed, 0), counter
(i // 8, row, offset, 0); element i takes 32 bits of word (i % 8) // 2 (low half for even
i, high half for odd i); its top 23 bits b give u = (b + 0.5) / 2^23 and E = -log(u).

``sample`` follows the pages literally in fp64 (softmax, then the quotient); ``scores``
gives the fp64 log of the quotient up to a per-row constant, l / T - log(max(E, 1e-10)),
which the tests use to decide near-ties.

Pins (tests/test_sampler.py): ``philox4x64_10`` equals numpy's Philox bit generator; the
empirical frequencies of many draws match softmax(l / T); a tiny temperature returns the
argmax of the logits; ``sample`` and the argmax of ``scores`` agree.
"""
from __future__ import annotations

import numpy as np

M0 = np.uint64(0xD2E7470EE14C6C93)
M1 = np.uint64(0xCA5A826395121157)
W0 = 0x9E3779B97F4A7C15
W1 = 0xBB67AE8584CAA73B
_MASK32 = np.uint64(0xFFFFFFFF)
_MASK64 = (1 << 64) - 1


def _mulhilo64(a, b):
    """Full 64 x 64 -> 128-bit product of uint64 arrays, as (hi, lo), via 32-bit limbs."""
    a = np.asarray(a, dtype=np.uint64)
    b = np.asarray(b, dtype=np.uint64)
    s32 = np.uint64(32)
    a_lo, a_hi = a & _MASK32, a >> s32
    b_lo, b_hi = b & _MASK32, b >> s32
    ll = a_lo * b_lo
    lh = a_lo * b_hi
    hl = a_hi * b_lo
    hh = a_hi * b_hi
    mid = (ll >> s32) + (lh & _MASK32) + (hl & _MASK32)          # < 3 * 2^32, no overflow
    lo = (ll & _MASK32) | ((mid & _MASK32) << s32)
    hi = hh + (lh >> s32) + (hl >> s32) + (mid >> s32)
    return hi, lo


def philox4x64_10(ctr, key):
    """Philox4x64 with 10 rounds. ``ctr``: 4 uint64 arrays (or ints), ``key``: 2 ints.
    Returns the 4 output words as uint64 arrays."""
    with np.errstate(over="ignore"):
        c = [np.asarray(x, dtype=np.uint64) for x in ctr]
        k0, k1 = int(key[0]) & _MASK64, int(key[1]) & _MASK64
        for _ in range(10):
            hi0, lo0 = _mulhilo64(M0, c[0])
            hi1, lo1 = _mulhilo64(M1, c[2])
            c = [hi1 ^ c[1] ^ np.uint64(k0), lo1, hi0 ^ c[3] ^ np.uint64(k1), lo0]
            k0 = (k0 + W0) & _MASK64
            k1 = (k1 + W1) & _MASK64
    return c


def exp_draws(num_rows: int, vocab: int, seed: int, offset: int) -> np.ndarray:
    """E[r, i] ~ Exp(1) as specified above, fp64 [num_rows, vocab]."""
    groups = -(-vocab // 8)
    out = np.empty((num_rows, groups * 8))
    rows_per_pass = max(1, (1 << 20) // groups)
    for r0 in range(0, num_rows, rows_per_pass):
        r1 = min(num_rows, r0 + rows_per_pass)
        g = np.broadcast_to(np.arange(groups, dtype=np.uint64), (r1 - r0, groups))
        r = np.broadcast_to(np.arange(r0, r1, dtype=np.uint64)[:, None], (r1 - r0, groups))
        w = philox4x64_10([g, r, np.full_like(g, offset), np.zeros_like(g)], (seed, 0))
        words = np.stack(w, axis=-1)                              # [rows, groups, 4]
        halves = np.stack([words & _MASK32, words >> np.uint64(32)], axis=-1)  # [.., 4, 2]
        bits = halves.reshape(r1 - r0, groups * 8)               # element 8g + 2w + half
        u = ((bits >> np.uint64(9)).astype(np.float64) + 0.5) / 2.0 ** 23
        out[r0:r1] = -np.log(u)
    return out[:, :vocab]


def _to_f64(logits) -> np.ndarray:
    a = np.asarray(logits)
    if a.dtype == np.uint16:                       # bf16 bit patterns
        return (a.astype(np.uint32) << np.uint32(16)).view(np.float32).astype(np.float64)
    return a.astype(np.float64)


def sample(logits, temperatures, seed: int, offset: int = 0) -> np.ndarray:
    """The pages' sampler in fp64: argmax of softmax(l / T) / max(E, 1e-10) per row."""
    l = _to_f64(logits)
    T = np.asarray(temperatures, dtype=np.float64)
    z = l / T[:, None]
    z = z - z.max(axis=1, keepdims=True)
    p = np.exp(z)
    p /= p.sum(axis=1, keepdims=True)
    E = np.maximum(exp_draws(l.shape[0], l.shape[1], seed, offset), 1e-10)
    return np.argmax(p / E, axis=1).astype(np.int64)


def scores(logits, temperatures, seed: int, offset: int = 0) -> np.ndarray:
    """log of the quotient up to a per-row constant: l / T - log(max(E, 1e-10)), fp64."""
    l = _to_f64(logits)
    T = np.asarray(temperatures, dtype=np.float64)
    E = np.maximum(exp_draws(l.shape[0], l.shape[1], seed, offset), 1e-10)
    return l / T[:, None] - np.log(E)
