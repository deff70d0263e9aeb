"""GPU parity of pkv_sample (temperature sampling) against the fp64 sampler oracle.

The kernel decides in fp32, the oracle in fp64 with the same Philox draws. Where two
candidates' scores differ by less than fp32 rounding either is a correct sample, so every
row checks that the GPU's token is a maximiser of the fp64 score within that rounding
bound, and the rows as a whole must agree exactly almost always (near-ties are rare).
"""
from __future__ import annotations

import numpy as np
import pytest
import torch

from oracle.sampler import sample, scores
from paged_kv_cache_225_amd import _binding as B
from workloads import bf16_round_bits

pytestmark = pytest.mark.gpu

VOCAB = 151936  # Qwen3 vocabulary


def _logits(rng, rows, vocab, dtype, scale=3.0):
    x = (rng.standard_normal((rows, vocab)) * scale).astype(np.float32)
    if dtype == "bf16":
        bits = bf16_round_bits(x)
        t = torch.from_numpy(bits.view(np.int16)).cuda().view(torch.bfloat16)
        return bits, t
    return x, torch.from_numpy(x).cuda()


def _run(logits_t, temps, seed, offset):
    rows, vocab = logits_t.shape
    tokens = torch.empty(rows, dtype=torch.int32, device="cuda")
    ws = torch.empty(B.pkv_sample_workspace_bytes(rows, vocab), dtype=torch.uint8, device="cuda")
    B.pkv_sample(tokens, logits_t, torch.from_numpy(temps.astype(np.float32)).cuda(), seed, offset,
                 workspace=ws)
    torch.cuda.synchronize()
    return tokens.cpu().numpy().astype(np.int64)


def _check(host_logits, got, temps, seed, offset, min_exact):
    s = scores(host_logits, temps.astype(np.float32).astype(np.float64), seed, offset)
    ref = s.argmax(axis=1)
    best = s.max(axis=1)
    tol = 2e-6 * (1.0 + np.abs(s).max(axis=1))       # fp32 rounding of l / T and the logs
    picked = s[np.arange(len(got)), got]
    assert np.all(got >= 0) and np.all(got < s.shape[1])
    assert np.all(picked >= best - tol), (picked - best, tol)
    exact = float((got == ref).mean())
    assert exact >= min_exact, exact
    return exact


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_sampler_qwen3_vocab_batch64(dtype):
    rng = np.random.Generator(np.random.PCG64(31))
    host, dev = _logits(rng, 64, VOCAB, dtype)
    temps = rng.choice([0.1, 0.6, 1.0, 1.5], size=64)
    got = _run(dev, temps, seed=1234, offset=7)
    ex = _check(host, got, temps, 1234, 7, min_exact=0.95)
    print(f"{dtype}: exact agreement {ex:.3f}", flush=True)
    # same seed and offset: the same tokens; another offset: fresh draws
    assert np.array_equal(_run(dev, temps, 1234, 7), got)
    assert not np.array_equal(_run(dev, temps, 1234, 8), got)


@pytest.mark.parametrize("rows,vocab", [(1, 1), (3, 7), (2, 2048), (2, 2049), (5, 8191),
                                        (1, 100000), (300, 4096), (4, 1001)])
def test_sampler_edge_shapes(rows, vocab):
    rng = np.random.Generator(np.random.PCG64(rows * 7 + vocab))
    host, dev = _logits(rng, rows, vocab, "f32")
    temps = rng.uniform(0.3, 1.2, size=rows)
    got = _run(dev, temps, seed=99, offset=0)
    _check(host, got, temps, 99, 0, min_exact=0.9 if rows >= 10 else 1.0)


def test_sampler_reads_only_vocab_columns_of_a_padded_row():
    rng = np.random.Generator(np.random.PCG64(3))
    rows, vocab, stride = 4, 1000, 1024
    x = (rng.standard_normal((rows, stride)) * 2).astype(np.float32)
    x[:, vocab:] = 1e30                               # padding that would always win
    dev = torch.from_numpy(x).cuda()[:, :vocab]
    temps = np.full(rows, 0.8)
    got = _run(dev, temps, 5, 1)
    _check(x[:, :vocab], got, temps, 5, 1, min_exact=1.0)


def test_sampler_distribution_on_gpu():
    p = np.array([0.5, 0.3, 0.15, 0.05])
    T = 0.7
    n = 8192
    logits = np.tile((np.log(p) * T + 2.0).astype(np.float32), (n, 1))
    got = _run(torch.from_numpy(logits).cuda(), np.full(n, T), seed=2024, offset=0)
    freq = np.bincount(got, minlength=4) / n
    sigma = np.sqrt(p * (1 - p) / n)
    assert np.all(np.abs(freq - p) < 5 * sigma), (freq, p)
    # the oracle, same draws: identical tokens row for row
    assert np.array_equal(got, sample(logits, np.full(n, T), 2024, 0))
