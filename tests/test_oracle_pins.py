"""Pins for the CPU oracle: it is checked against things other than itself.

* the pages' worked example (tests/golden/),
* pure-Python brute force that reads the generator's logical K/V directly
  (no pool, no slots, no gather), with math.exp / math.fsum,
* closed forms, torch's float64 SDPA as a library routine,
* invariants: block permutation, prefix cache = recompute, softmax rows sum
  to 1, GQA = MHA with replicated kv heads, decode = prefill with one query,
  NaN-poisoned free slots, the exactness of the split-K combine formula,
* scatter invariants.

A final group plants plausible mistakes in copies of the oracle and checks
that at least one pin fails for each.
"""
from __future__ import annotations

import json
import math
import os
import struct

import numpy as np
import pytest
import torch

import oracle as O
import oracle.paged_attention as OP
from workloads import make_decode, make_prefill
from tests.oracle_pipeline import run_workload, setup_pools, run_step, step_metadata

GOLD = os.path.join(os.path.dirname(__file__), "golden")


# ---------------------------------------------------------------- helpers
def _py_float(bits_or_val, dtype):
    if dtype == "bf16":
        return struct.unpack("<f", struct.pack("<I", int(bits_or_val) << 16))[0]
    return float(bits_or_val)


def brute_force(w):
    """Pure-Python attention over the generator's logical K/V (no paging at all)."""
    Hq, Hkv, D = w.num_heads, w.num_kv_heads, w.head_dim
    G = Hq // Hkv
    rows = []
    qi = 0
    for b in range(w.num_seqs):
        K, V = w.seq_kv_logical(b)
        n = int(w.seq_lens[b])
        start = int(w.num_cached[b])
        Kf = [[[_py_float(K[j, g, d], w.dtype) for d in range(D)] for g in range(Hkv)] for j in range(n)]
        Vf = [[[_py_float(V[j, g, d], w.dtype) for d in range(D)] for g in range(Hkv)] for j in range(n)]
        for i in range(n - start):
            pos = start + i
            row = []
            for h in range(Hq):
                g = h // G
                qv = [_py_float(w.q[qi, h, d], w.dtype) for d in range(D)]
                s = [w.scale * math.fsum(qv[d] * Kf[j][g][d] for d in range(D)) for j in range(pos + 1)]
                m = max(s)
                e = [math.exp(x - m) for x in s]
                l = math.fsum(e)
                row.append([math.fsum(e[j] * Vf[j][g][d] for j in range(pos + 1)) / l for d in range(D)])
            rows.append(row)
            qi += 1
    return np.asarray(rows, dtype=np.float64).reshape(-1, Hq, D)


def tiny_workloads():
    return [
        make_decode(1, [1, 5, 9, 13], Hq=4, Hkv=2, D=8, dtype="f32", bs=4),
        make_decode(2, [3, 17, 8], Hq=2, Hkv=1, D=4, dtype="bf16", bs=8),
        make_decode(3, [40, 1], Hq=3, Hkv=3, D=5, dtype="f32", bs=256),
        make_prefill(4, [5, 3, 7], Hq=4, Hkv=2, D=8, dtype="bf16", bs=4),
        make_prefill(5, [3, 6], cached=[9, 2], Hq=2, Hkv=1, D=6, dtype="f32", bs=4),
        make_prefill(6, [4, 2, 5], cached=[8, 8, 8], Hq=4, Hkv=2, D=4, dtype="bf16", bs=4,
                     shared_blocks=[2, 2, 1], n_prefix_blocks=2),
        make_decode(7, [9, 12, 30], Hq=4, Hkv=2, D=4, dtype="bf16", bs=4,
                    shared_blocks=[2, 0, 2], n_prefix_blocks=3),
    ]


def logical_f64(w, b):
    K, V = w.seq_kv_logical(b)
    return O.to_f64(K, w.dtype), O.to_f64(V, w.dtype)


# ---------------------------------------------------------------- golden
def test_worked_example_prefill_metadata():
    g = json.load(open(os.path.join(GOLD, "worked_example_metadata.json")))
    p = g["prefill"]
    md = O.prefill_metadata(p["seq_lens"], p["num_cached"], p["block_tables"], g["block_size"])
    for k, v in p["expect"].items():
        np.testing.assert_array_equal(md[k], v, err_msg=k)


def test_worked_example_decode_metadata():
    g = json.load(open(os.path.join(GOLD, "worked_example_metadata.json")))
    d = g["decode"]
    md = O.decode_metadata(d["seq_lens"], d["block_tables"], g["block_size"])
    for k, v in d["expect"].items():
        np.testing.assert_array_equal(md[k], v, err_msg=k)


def test_cu_seqlens_example():
    g = json.load(open(os.path.join(GOLD, "cu_seqlens_example.json")))
    lens = g["seq_lens"]
    tables = [[i] for i in range(len(lens))]
    md = O.prefill_metadata(lens, [0] * len(lens), tables, 256)
    np.testing.assert_array_equal(md["cu_seqlens_q"], g["expect"]["cu_seqlens_q"])
    np.testing.assert_array_equal(md["cu_seqlens_k"], g["expect"]["cu_seqlens_q"])


def test_prefill_metadata_unaligned_prefix_and_padding():
    # a cached prefix ending mid-block: slots start mid-block, tables padded with -1
    md = O.prefill_metadata([10, 3], [6, 0], [[7, 2, 9], [4]], 4)
    np.testing.assert_array_equal(md["slot_mapping"], [2 * 4 + 2, 2 * 4 + 3, 9 * 4, 9 * 4 + 1, 16, 17, 18])
    np.testing.assert_array_equal(md["cu_seqlens_q"], [0, 4, 7])
    np.testing.assert_array_equal(md["cu_seqlens_k"], [0, 10, 13])
    np.testing.assert_array_equal(md["block_tables"], [[7, 2, 9], [4, -1, -1]])


def test_decode_metadata_block_boundaries():
    # len 4 -> last slot of block 0; len 5 -> first slot of the second block
    md = O.decode_metadata([4, 5, 1], [[3], [3, 6], [0]], 4)
    np.testing.assert_array_equal(md["slot_mapping"], [15, 24, 0])
    with pytest.raises(ValueError):
        O.decode_metadata([5], [[3]], 4)        # table too short for the newest token


# ---------------------------------------------------------------- brute force
@pytest.mark.parametrize("idx", range(7))
def test_oracle_matches_brute_force(idx):
    w = tiny_workloads()[idx]
    out, _, _, _ = run_workload(w)
    ref = brute_force(w)
    assert out.shape == ref.shape
    assert np.max(np.abs(out - ref)) <= 1e-12


def packed_kv(w):
    """The workload's logical K/V rows packed sequence after sequence, and cu_seqlens_k."""
    ks, vs = zip(*(w.seq_kv_logical(b) for b in range(w.num_seqs)))
    cu_k = np.concatenate([[0], np.cumsum(w.seq_lens)]).astype(np.int64)
    return np.concatenate(ks), np.concatenate(vs), cu_k


@pytest.mark.parametrize("idx", [3, 4, 5])
def test_packed_prefill_matches_brute_force(idx):
    w = tiny_workloads()[idx]
    k, v, cu_k = packed_kv(w)
    cu_q = np.concatenate([[0], np.cumsum(w.q_lens)]).astype(np.int64)
    out = O.attn_prefill_varlen(w.q, k, v, w.dtype, cu_q, cu_k, w.scale)
    ref = brute_force(w)
    assert out.shape == ref.shape
    assert np.max(np.abs(out - ref)) <= 1e-12


def test_packed_prefill_equals_paged_prefill():
    w = make_prefill(22, [5, 0, 9, 3], cached=[8, 3, 0, 13], Hq=4, Hkv=2, D=8, dtype="bf16",
                     bs=4, shared_blocks=[2, 0, 0, 2], n_prefix_blocks=2)
    out, md, _, _ = run_workload(w)
    k, v, cu_k = packed_kv(w)
    packed = O.attn_prefill_varlen(w.q, k, v, w.dtype, md["cu_seqlens_q"], cu_k, w.scale)
    np.testing.assert_array_equal(out, packed)


# ---------------------------------------------------------------- closed forms
def test_single_key_returns_that_value_row():
    w = make_decode(11, [1, 1, 1], Hq=4, Hkv=2, D=16, dtype="bf16", bs=8)
    out, _, _, _ = run_workload(w)
    for b in range(3):
        _, V = logical_f64(w, b)
        np.testing.assert_array_equal(out[b], np.repeat(V[0], 2, axis=0))


@pytest.mark.parametrize("kind", ["decode", "prefill"])
def test_equal_keys_give_mean_of_visible_values(kind):
    if kind == "decode":
        w = make_decode(12, [6, 11], Hq=4, Hkv=2, D=8, dtype="f32", bs=4)
    else:
        w = make_prefill(12, [5, 4], cached=[0, 3], Hq=4, Hkv=2, D=8, dtype="f32", bs=4)
    w.priv_k[:] = w.priv_k[0]
    out, _, _, _ = run_workload(w)
    qi = 0
    for b in range(w.num_seqs):
        _, V = logical_f64(w, b)
        for i in range(int(w.q_lens[b])):
            pos = int(w.num_cached[b]) + i
            mean = V[:pos + 1].mean(axis=0)
            np.testing.assert_allclose(out[qi], np.repeat(mean, 2, axis=0), rtol=0, atol=1e-13)
            qi += 1


def test_constant_values_give_that_constant():
    w = make_prefill(13, [7, 2], cached=[2, 5], Hq=2, Hkv=1, D=4, dtype="f32", bs=4)
    c = np.array([[0.5, -1.25, 3.0, 7.75]], dtype=np.float32)
    w.priv_v[:] = c
    out, _, _, _ = run_workload(w)
    np.testing.assert_allclose(out, np.broadcast_to(c.astype(np.float64), out.shape), atol=1e-14, rtol=0)


def test_zero_query_gives_mean():
    w = make_decode(14, [9, 3], Hq=2, Hkv=2, D=4, dtype="bf16", bs=4)
    w.q[:] = 0
    out, _, _, _ = run_workload(w)
    for b in range(2):
        _, V = logical_f64(w, b)
        np.testing.assert_allclose(out[b], V.mean(axis=0), atol=1e-14, rtol=0)


def test_dominant_logit_selects_its_value_row():
    w = make_decode(15, [12], Hq=1, Hkv=1, D=8, dtype="f32", bs=4)
    w.q[:] = 0
    w.q[0, 0, 0] = 1.0
    w.priv_k[:] = 0
    star = 5
    w.priv_k[star, 0, 0] = np.float32(60.0 / w.scale)     # logit margin 60
    out, _, _, _ = run_workload(w)
    _, V = logical_f64(w, 0)
    np.testing.assert_allclose(out[0, 0], V[star, 0], rtol=0, atol=1e-20 * (1 + np.abs(V).max()) + 1e-24)


# ---------------------------------------------------------------- library routine
@pytest.mark.parametrize("cached", [0, 6, 9])
def test_matches_torch_sdpa_fp64(cached):
    Lq = 7
    w = make_prefill(16 + cached, [Lq], cached=[cached], Hq=4, Hkv=2, D=8, dtype="bf16", bs=4)
    out, _, _, _ = run_workload(w)
    K, V = logical_f64(w, 0)
    q = torch.from_numpy(O.to_f64(w.q, "bf16")).permute(1, 0, 2)[None]    # [1, Hq, Lq, D]
    k = torch.from_numpy(K).permute(1, 0, 2)[None]
    v = torch.from_numpy(V).permute(1, 0, 2)[None]
    Lk = cached + Lq
    if cached == 0:
        ref = torch.nn.functional.scaled_dot_product_attention(q, k, v, is_causal=True, scale=w.scale,
                                                               enable_gqa=True)
    else:
        # bottom-right alignment, written as an explicit boolean mask
        mask = torch.ones(Lq, Lk, dtype=torch.bool).tril(diagonal=Lk - Lq)
        ref = torch.nn.functional.scaled_dot_product_attention(q, k, v, attn_mask=mask, scale=w.scale,
                                                               enable_gqa=True)
    ref = ref[0].permute(1, 0, 2).numpy()
    assert np.max(np.abs(out - ref)) <= 1e-12


# ---------------------------------------------------------------- invariants
@pytest.mark.parametrize("idx", [0, 3, 5, 6])
def test_block_permutation_invariance(idx):
    w = tiny_workloads()[idx]
    out, md, kc, vc = run_workload(w)
    rng = np.random.default_rng(99)
    pi = rng.permutation(w.num_blocks)
    kc2, vc2 = np.empty_like(kc), np.empty_like(vc)
    kc2[pi] = kc
    vc2[pi] = vc
    tables = np.where(md["block_tables"] >= 0, pi[np.maximum(md["block_tables"], 0)], -1)
    if w.kind == "decode":
        out2 = O.paged_attn_decode(w.q, kc2, vc2, w.dtype, tables, md["context_lens"], w.scale, w.block_size)
    else:
        out2 = O.paged_attn_prefill_varlen(w.q, kc2, vc2, w.dtype, tables, md["cu_seqlens_q"],
                                           md["cu_seqlens_k"], w.scale, w.block_size)
    np.testing.assert_array_equal(out, out2)


def test_prefix_cache_hit_equals_full_recompute():
    w = make_prefill(21, [5, 7, 3], cached=[8, 8, 8], Hq=4, Hkv=2, D=8, dtype="bf16", bs=4,
                     shared_blocks=[2, 2, 2], n_prefix_blocks=2)
    out, md, kc, vc = run_workload(w)
    rng = np.random.default_rng(5)
    qi = 0
    for b in range(w.num_seqs):
        Ls, Lk = int(w.q_lens[b]), int(w.seq_lens[b])
        extra = rng.standard_normal((Lk - Ls, 4, 8)).astype(np.float32)
        from workloads import bf16_round_bits
        q_full = np.concatenate([bf16_round_bits(extra), w.q[qi:qi + Ls]])
        full = O.paged_attn_prefill_varlen(q_full, kc, vc, "bf16", md["block_tables"][b:b + 1],
                                           [0, Lk], [0, Lk], w.scale, w.block_size)
        np.testing.assert_allclose(out[qi:qi + Ls], full[Lk - Ls:], rtol=0, atol=1e-14)
        qi += Ls


def test_softmax_rows_sum_to_one_and_mask_is_exact():
    rng = np.random.default_rng(3)
    q = rng.standard_normal((6, 4, 8))
    K = rng.standard_normal((10, 2, 8)) * 3
    pos = np.array([0, 3, 4, 7, 9, 9])
    P = O.softmax_probs(q, K, None, pos, 0.7)
    assert np.all(np.abs(P.sum(axis=2) - 1.0) <= 1e-14)
    for i, p in enumerate(pos):
        assert np.all(P[:, i, p + 1:] == 0.0)
        assert np.all(P[:, i, :p + 1] > 0.0)


def test_gqa_equals_mha_with_replicated_kv_heads():
    rng = np.random.default_rng(4)
    q = rng.standard_normal((5, 6, 8))
    K = rng.standard_normal((9, 2, 8))
    V = rng.standard_normal((9, 2, 8))
    pos = np.arange(4, 9)
    a = O.attend(q, K, V, pos, 0.3)
    b = O.attend(q, np.repeat(K, 3, axis=1), np.repeat(V, 3, axis=1), pos, 0.3)
    np.testing.assert_array_equal(a, b)


def test_decode_equals_prefill_with_one_query():
    w = make_decode(22, [5, 9, 16, 1], Hq=4, Hkv=2, D=8, dtype="bf16", bs=4)
    out, md, kc, vc = run_workload(w)
    cu_q = np.arange(w.num_seqs + 1, dtype=np.int32)
    cu_k = np.concatenate([[0], np.cumsum(md["context_lens"])]).astype(np.int32)
    out2 = O.paged_attn_prefill_varlen(w.q, kc, vc, "bf16", md["block_tables"], cu_q, cu_k,
                                       w.scale, w.block_size)
    np.testing.assert_array_equal(out, out2)


@pytest.mark.parametrize("idx", [0, 1, 3, 6])
def test_nan_poisoned_free_slots_do_not_leak(idx):
    w = tiny_workloads()[idx]
    a, _, _, _ = run_workload(w)
    b, _, _, _ = run_workload(w, fill=0)
    assert np.all(np.isfinite(a))
    np.testing.assert_array_equal(a, b)


def test_context_len_zero_row_is_zero():
    w = make_decode(23, [5, 6], Hq=2, Hkv=1, D=4, dtype="f32", bs=4)
    kc, vc = setup_pools(w)
    md = step_metadata(w)
    ctx = md["context_lens"].copy()
    ctx[1] = 0
    out = O.paged_attn_decode(w.q, kc, vc, "f32", md["block_tables"], ctx, w.scale, 4)
    assert np.all(out[1] == 0)


def test_split_softmax_combine_is_exact():
    """(m, l, o) partials over any key partition combine to the unsplit result."""
    rng = np.random.default_rng(6)
    s = rng.standard_normal(300) * 4
    V = rng.standard_normal((300, 16))
    ref = (np.exp(s - s.max()) @ V) / np.exp(s - s.max()).sum()
    for cuts in ([0, 300], [0, 64, 128, 192, 256, 300], [0, 1, 299, 300], [0, 17, 256, 300]):
        parts = []
        for a, b in zip(cuts[:-1], cuts[1:]):
            m = s[a:b].max()
            e = np.exp(s[a:b] - m)
            parts.append((m, e.sum(), e @ V[a:b]))
        M = max(p[0] for p in parts)
        L = sum(np.exp(p[0] - M) * p[1] for p in parts)
        o = sum(np.exp(p[0] - M) * p[2] for p in parts) / L
        assert np.max(np.abs(o - ref)) <= 1e-12


# ---------------------------------------------------------------- scatter
def test_scatter_roundtrip_and_untouched_slots():
    w = make_prefill(31, [6, 9, 1], cached=[3, 0, 4], Hq=4, Hkv=2, D=8, dtype="bf16", bs=4)
    out, md, kc, vc = run_workload(w)
    for b in range(w.num_seqs):
        K, V = w.seq_kv_logical(b)
        n = int(w.seq_lens[b])
        j = np.arange(n)
        t = np.asarray(w.block_tables[b])
        np.testing.assert_array_equal(kc[t[j // 4], j % 4], K)
        np.testing.assert_array_equal(vc[t[j // 4], j % 4], V)
    written = int(w.seq_lens.sum())
    poison_rows = np.all(kc.reshape(-1, 16) == w.poison_bits(), axis=1)
    assert int((~poison_rows).sum()) == written


def test_scatter_skips_minus_one_and_rejects_duplicates():
    kc = np.zeros((2, 4, 1, 2), dtype=np.float32)
    vc = np.zeros_like(kc)
    key = np.arange(6, dtype=np.float32).reshape(3, 1, 2) + 1
    O.store_kvcache(key, -key, kc, vc, np.array([5, -1, 0], dtype=np.int32))
    flat = kc.reshape(-1, 2)
    np.testing.assert_array_equal(flat[5], key[0, 0])
    np.testing.assert_array_equal(flat[0], key[2, 0])
    assert np.count_nonzero(flat.any(axis=1)) == 2
    with pytest.raises(ValueError):
        O.store_kvcache(key, key, kc, vc, np.array([1, 1, -1], dtype=np.int32))


def test_scatter_strided_key_view():
    # keys taken from a wider fused-qkv-like buffer: token stride > Hkv*D
    buf = np.arange(3 * 10, dtype=np.float32).reshape(3, 10)
    key = buf[:, 2:6].reshape(3, 2, 2)
    kc = np.zeros((1, 4, 2, 2), dtype=np.float32)
    vc = np.zeros_like(kc)
    O.store_kvcache(key, key, kc, vc, np.array([3, 0, 1], dtype=np.int32))
    np.testing.assert_array_equal(kc.reshape(4, 4)[3], buf[0, 2:6])
    np.testing.assert_array_equal(kc.reshape(4, 4)[1], buf[2, 2:6])


# ---------------------------------------------------------------- planted mistakes
def _mutant_attend_factory(kind):
    def softmax_probs(q_rows, K, V, q_positions, scale):
        nq, Hq, _ = q_rows.shape
        nk, Hkv, _ = K.shape
        G = Hq // Hkv
        P = np.zeros((Hq, nq, nk))
        visible = np.arange(nk)[None, :] <= np.asarray(q_positions)[:, None]
        for h in range(Hq):
            g = h % Hkv if kind == "gqa_modulo" else h // G
            sc = 1.0 if kind == "no_scale" else scale
            S = sc * (q_rows[:, h, :] @ K[:, g, :].T)
            S = np.where(visible, S, -np.inf)
            w = np.exp(S - S.max(axis=1, keepdims=True))
            P[h] = w / w.sum(axis=1, keepdims=True)
        return P
    return softmax_probs


def _pin_battery():
    """Run the cheap pins; return the number that fail."""
    fails = 0
    for t in (test_worked_example_prefill_metadata, test_worked_example_decode_metadata):
        try:
            t()
        except AssertionError:
            fails += 1
    for w in tiny_workloads()[:5]:
        try:
            out, _, _, _ = run_workload(w)
            if not np.max(np.abs(out - brute_force(w))) <= 1e-12:
                fails += 1
        except (ValueError, IndexError):
            fails += 1
    try:
        test_matches_torch_sdpa_fp64(6)
    except (AssertionError, ValueError, IndexError):
        fails += 1
    return fails


MUTANTS = {
    "slot_off_by_one": ("slot_of", lambda t, pos, bs: int(t[pos // bs]) * bs + (pos + 1) % bs),
    "slot_block_stride_wrong": ("slot_of", lambda t, pos, bs: int(t[pos // bs]) * (bs + 1) + pos % bs),
    "gqa_modulo": ("softmax_probs", _mutant_attend_factory("gqa_modulo")),
    "no_scale": ("softmax_probs", _mutant_attend_factory("no_scale")),
}


@pytest.mark.parametrize("name", sorted(MUTANTS) + ["top_left_causal", "decode_drops_newest"])
def test_planted_mistake_is_caught(name, monkeypatch):
    if name in MUTANTS:
        attr, fn = MUTANTS[name]
        monkeypatch.setattr(OP, attr, fn)
    elif name == "top_left_causal":
        real = OP.attend
        monkeypatch.setattr(OP, "attend",
                            lambda q, K, V, pos, s: real(q, K, V, np.asarray(pos) - (np.asarray(pos)[0]
                                                         if len(pos) > 1 else 0), s))
    elif name == "decode_drops_newest":
        real = OP.attend
        monkeypatch.setattr(OP, "attend",
                            lambda q, K, V, pos, s: real(q, K[:-1], V[:-1], np.asarray(pos) - 1, s)
                            if len(pos) == 1 and len(K) > 1 else real(q, K, V, pos, s))
    assert _pin_battery() >= 1
