"""The sampler oracle pinned (CPU): its Philox against numpy's Philox bit generator, its
draws against the distribution the pages' sampler defines, the small-temperature limit;
plus the ABI's argument checks."""
from __future__ import annotations

import ctypes

import numpy as np
import pytest

from oracle.sampler import exp_draws, philox4x64_10, sample, scores
from paged_kv_cache_225_amd import _binding as B


def test_philox_matches_numpy_bit_generator():
    # numpy's Philox is Philox4x64-10; random_raw advances the counter by one before each
    # block, so its first block is the function at counter + 1
    rng = np.random.Generator(np.random.PCG64(5))
    for _ in range(20):
        key = [int(x) for x in rng.integers(0, 2**62, size=2)]
        ctr = [int(x) for x in rng.integers(0, 2**62, size=4)]
        got = [int(x) for x in np.random.Philox(counter=ctr, key=key).random_raw(8)]
        c1 = [ctr[0] + 1] + ctr[1:]
        c2 = [ctr[0] + 2] + ctr[1:]
        want = [int(x) for x in philox4x64_10(c1, key)] + [int(x) for x in philox4x64_10(c2, key)]
        assert got == want
    # the 128-bit products hold at the top of the range too (exact big-integer check)
    mask = (1 << 64) - 1
    for a in (0, 1, 2**32 - 1, 2**32, 2**63, mask):
        from oracle.sampler import _mulhilo64, M0
        hi, lo = _mulhilo64(M0, np.uint64(a))
        assert (int(hi) << 64) | int(lo) == int(M0) * a


def test_exponential_draws_are_exp1():
    E = exp_draws(8, 50000, seed=11, offset=3)
    assert E.min() > 0 and np.isfinite(E).all()
    # Exp(1): mean 1, variance 1, P(E > 1) = 1/e
    assert abs(E.mean() - 1) < 0.01 and abs(E.var() - 1) < 0.03
    assert abs((E > 1).mean() - np.exp(-1)) < 0.005
    # rows, seeds and offsets give different draws
    assert not np.array_equal(exp_draws(1, 64, 11, 3), exp_draws(1, 64, 11, 4))
    assert not np.array_equal(exp_draws(2, 64, 11, 3)[0], exp_draws(2, 64, 11, 3)[1])
    assert not np.array_equal(exp_draws(1, 64, 11, 3), exp_draws(1, 64, 12, 3))


def test_sampler_draws_follow_softmax_of_tempered_logits():
    p = np.array([0.5, 0.3, 0.15, 0.05])
    T = 0.7
    logits = np.log(p) * T + 2.0               # softmax(logits / T) = p
    n = 40000
    toks = sample(np.tile(logits, (n, 1)), np.full(n, T), seed=2024, offset=0)
    freq = np.bincount(toks, minlength=4) / n
    sigma = np.sqrt(p * (1 - p) / n)
    assert np.all(np.abs(freq - p) < 5 * sigma), (freq, p)


def test_tiny_temperature_is_argmax():
    rng = np.random.Generator(np.random.PCG64(8))
    logits = rng.permutation(1000).reshape(4, 250) * 0.01
    toks = sample(logits, np.full(4, 1e-6), seed=1, offset=0)
    assert np.array_equal(toks, logits.argmax(axis=1))


def test_quotient_and_log_score_forms_agree():
    rng = np.random.Generator(np.random.PCG64(9))
    logits = rng.standard_normal((16, 3000)) * 3
    T = rng.uniform(0.2, 1.5, size=16)
    assert np.array_equal(sample(logits, T, 77, 5), scores(logits, T, 77, 5).argmax(axis=1))


FAKE = ctypes.c_void_p(0x1000)


def test_sample_argument_validation():
    lib = B.load_library()
    ws = B.pkv_sample_workspace_bytes(4, 1000)
    assert ws > 0 and B.pkv_sample_workspace_bytes(0, 10) == 0
    ok = dict(tokens=FAKE, logits=FAKE, stride=1000, rows=4, vocab=1000, dt=B.PKV_F32, temps=FAKE,
              ws=FAKE, ws_bytes=ws)

    def rc(**kw):
        a = dict(ok, **kw)
        return lib.pkv_sample(a["tokens"], a["logits"], a["stride"], a["rows"], a["vocab"], a["dt"],
                              a["temps"], 1, 0, a["ws"], a["ws_bytes"], None)
    assert rc(rows=0) == 0
    assert rc(tokens=None) == -1 and rc(temps=None) == -1
    assert rc(stride=999) == -1                      # row shorter than the vocabulary
    assert rc(dt=7) == -2 and rc(rows=70000) == -2
    assert rc(ws_bytes=ws - 1) == -3 and rc(ws=None) == -3


# ------------------------------------------------------------------ planted mistakes
def _sampler_pins():
    fails = 0
    for t in (test_sampler_draws_follow_softmax_of_tempered_logits, test_tiny_temperature_is_argmax,
              test_exponential_draws_are_exp1):
        try:
            t()
        except AssertionError:
            fails += 1
    return fails


@pytest.mark.parametrize("kind", ["temperature_multiplies", "multiplies_by_draw", "uniform_not_exp",
                                  "no_softmax_temperature"])
def test_planted_mistake_in_the_sampler_oracle_is_caught(kind, monkeypatch):
    import oracle.sampler as OS
    assert _sampler_pins() == 0
    real_draws, real_sample = OS.exp_draws, OS.sample

    def sample(logits, temperatures, seed, offset=0):
        l = OS._to_f64(logits)
        T = np.asarray(temperatures, dtype=np.float64)
        z = l * T[:, None] if kind == "temperature_multiplies" else (
            l if kind == "no_softmax_temperature" else l / T[:, None])
        p = np.exp(z - z.max(axis=1, keepdims=True))
        p /= p.sum(axis=1, keepdims=True)
        E = np.maximum(OS.exp_draws(l.shape[0], l.shape[1], seed, offset), 1e-10)
        return np.argmax(p * E if kind == "multiplies_by_draw" else p / E, axis=1)

    def exp_draws(num_rows, vocab, seed, offset):
        E = real_draws(num_rows, vocab, seed, offset)
        return np.exp(-E) if kind == "uniform_not_exp" else E   # u instead of -log(u)

    monkeypatch.setattr(OS, "exp_draws", exp_draws)
    monkeypatch.setitem(globals(), "exp_draws", exp_draws)
    monkeypatch.setitem(globals(), "sample", sample)
    assert _sampler_pins() >= 1, kind
