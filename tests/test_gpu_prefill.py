"""GPU parity of paged_attn_prefill_varlen (bf16 MFMA) against the fp64 oracle."""
from __future__ import annotations

import numpy as np
import pytest
import torch

import oracle as O
from paged_kv_cache_225_amd import _binding as B
from paged_kv_cache_225_amd.harness import DeviceStep
from tests.oracle_pipeline import run_workload
from tests.parity import assert_attention_close
from workloads import make_config, make_decode, make_prefill

pytestmark = pytest.mark.gpu


def gpu_run(w, **kw):
    ds = DeviceStep(w, **kw)
    ds.step()
    torch.cuda.synchronize()
    return ds


def check(w, **kw):
    ds = gpu_run(w, **kw)
    ref, _, _, _ = run_workload(w)
    return ds, assert_attention_close(ds.out_f64(), ref, rel_l2=1e-2, label=w.name)


SMALL = [
    # (D, Hq, Hkv, bs, q_lens, cached, shared_blocks, n_prefix_blocks)
    (128, 16, 8, 256, [1, 63, 64, 65, 200], [0, 0, 0, 0, 0], None, 0),
    (128, 16, 8, 256, [100, 37, 1], [300, 1, 999], None, 0),                 # unaligned prefixes
    (128, 16, 8, 16, [129, 70, 3], [32, 48, 16], [2, 3, 1], 3),              # shared prefix, bs 16
    (64, 8, 8, 64, [90, 130], [64, 0], None, 0),                             # G = 1, D = 64
    (128, 32, 8, 32, [77, 150], [40, 0], None, 0),                           # G = 4
    (64, 16, 2, 256, [65, 10], [7, 500], None, 0),                           # G = 8
]


@pytest.mark.parametrize("case", range(len(SMALL)))
def test_prefill_small_cases(case):
    D, Hq, Hkv, bs, ql, cached, shared, npb = SMALL[case]
    w = make_prefill(300 + case, ql, cached=cached, Hq=Hq, Hkv=Hkv, D=D, dtype="bf16", bs=bs,
                     shared_blocks=shared, n_prefix_blocks=npb, name=f"small{case}")
    check(w)


@pytest.mark.parametrize("cfg", [3, 4])
def test_prefill_configs_full(cfg):
    w = make_config(cfg)
    _, st = check(w)
    print(f"config {cfg}: {st}", flush=True)


# Long prefixes: a few hundred key tiles per unit (hundreds of grid planes), tables of
# hundreds of blocks (block 16), a one-query row over 16000 cached keys, and a sequence with
# no prefix beside them.
LONG = [
    # (D, Hq, Hkv, bs, q_lens, cached)
    (128, 16, 8, 256, [300, 1, 64], [12000, 16000, 0]),
    (128, 16, 8, 16, [130, 2], [7000, 8191]),
    (64, 16, 2, 64, [200, 65], [9999, 4096]),
]


@pytest.mark.parametrize("case", range(len(LONG)))
def test_prefill_long_prefixes(case):
    D, Hq, Hkv, bs, ql, cached = LONG[case]
    print(f"case {case}: D {D} Hq {Hq} Hkv {Hkv} bs {bs} q {ql} cached {cached}", flush=True)
    w = make_prefill(320 + case, ql, cached=cached, Hq=Hq, Hkv=Hkv, D=D, dtype="bf16", bs=bs,
                     name=f"long{case}")
    check(w)


def test_prefill_peaked_logits():
    check(make_config(3, q_mult=4.0))


def test_prefill_nan_poison_equals_zero_fill_bitwise():
    w = make_prefill(310, [70, 300, 1], cached=[0, 129, 40], Hq=16, Hkv=8, D=128, bs=256)
    a = gpu_run(w).out.clone()
    b = gpu_run(w, fill=0.0).out.clone()
    assert torch.equal(a.view(torch.int16), b.view(torch.int16))
    assert bool(torch.isfinite(a.float()).all())


def test_prefill_block_permutation_bitwise():
    w = make_prefill(311, [200, 333], cached=[256, 17], Hq=16, Hkv=8, D=128, bs=256,
                     shared_blocks=[1, 0], n_prefix_blocks=1)
    a = gpu_run(w).out.clone()
    pi = np.random.default_rng(2).permutation(w.num_blocks).astype(np.int32)
    w.block_tables = [pi[t] for t in w.block_tables]
    w.prefix_block_ids = pi[w.prefix_block_ids]
    b = gpu_run(w).out.clone()
    assert torch.equal(a.view(torch.int16), b.view(torch.int16))


def test_prefix_hit_matches_full_recompute_on_gpu():
    """Suffix rows of a cached-prefix prefill equal the last rows of a full prefill."""
    w = make_prefill(312, [150, 64], cached=[512, 512], Hq=16, Hkv=8, D=128, bs=256,
                     shared_blocks=[2, 2], n_prefix_blocks=2)
    ds = gpu_run(w)
    rng = np.random.default_rng(3)
    from workloads import bf16_round_bits
    qi = 0
    for b in range(w.num_seqs):
        Ls, Lk = int(w.q_lens[b]), int(w.seq_lens[b])
        q_full = np.concatenate([bf16_round_bits(rng.standard_normal((Lk - Ls, 16, 128)).astype(np.float32)),
                                 w.q[qi:qi + Ls]])
        qt = torch.from_numpy(q_full.view(np.int16)).cuda().view(torch.bfloat16)
        out = torch.empty_like(qt)
        cu = torch.tensor([0, Lk], dtype=torch.int32, device="cuda")
        B.paged_attn_prefill_varlen(out, qt, ds.k_cache, ds.v_cache, ds.block_tables[b:b + 1], cu, cu,
                                    Lk, Lk, w.scale)
        torch.cuda.synchronize()
        suffix = out.float().cpu().numpy()[Lk - Ls:]
        assert_attention_close(suffix, ds.out_f64()[qi:qi + Ls], label="recompute")
        qi += Ls


def test_decode_equals_one_query_prefill_across_entry_points():
    w = make_decode(313, [300, 1, 777, 256], Hq=16, Hkv=8, D=128, dtype="bf16", bs=256)
    ds = gpu_run(w)
    cu_q = torch.arange(w.num_seqs + 1, dtype=torch.int32, device="cuda")
    cu_k = torch.from_numpy(np.concatenate([[0], np.cumsum(w.seq_lens)]).astype(np.int32)).cuda()
    out = torch.empty_like(ds.q)
    B.paged_attn_prefill_varlen(out, ds.q, ds.k_cache, ds.v_cache, ds.block_tables, cu_q, cu_k, 1,
                                int(w.seq_lens.max()), w.scale)
    torch.cuda.synchronize()
    ref, _, _, _ = run_workload(w)
    assert_attention_close(out.float().cpu().numpy(), ref, label="prefill Lq=1")
    assert_attention_close(out.float().cpu().numpy(), ds.out_f64(), atol=4e-2, rtol=2e-2, label="cross")


def test_prefill_empty_sequences_in_batch():
    w = make_prefill(314, [0, 90, 0, 5], cached=[10, 0, 0, 300], Hq=16, Hkv=8, D=128, bs=256)
    check(w)


def test_prefill_invalid_block_id_poisons_only_rows_that_reach_it():
    # seq 0: bad third block (keys 512..639) - rows 0..511 never reach it, rows 512..639 do;
    # seq 1: bad cached-prefix block - every row attends it; seq 2 untouched.
    w = make_prefill(312, [640, 300, 200], cached=[0, 256, 40], Hq=16, Hkv=8, D=128, bs=256)
    ds = DeviceStep(w)
    ds.store()
    ds.block_tables[0, 2] = w.num_blocks + 3      # out of range: must not be read
    ds.block_tables[1, 0] = -7
    ds.attend()
    torch.cuda.synchronize()
    out = ds.out_f64()
    ref, _, _, _ = run_workload(w)
    assert np.all(np.isnan(out[512:640]))
    assert np.all(np.isnan(out[640:940]))
    keep = np.r_[0:512, 940:1140]
    assert_attention_close(out[keep], ref[keep], rel_l2=1e-2, label="unaffected rows")


def test_prefill_invalid_block_id_past_the_first_table_window():
    # blocks of 64 keys: a 4500-key sequence has 71 table columns, more than the 64 a tile
    # lookup holds at once, so the lookup reloads past column 63. Column 66 (keys 4224..4287)
    # is bad: rows from 4224 on reach it; the 64-row query tile holding row 4224 (rows
    # 4180..4243, tiles counted back from the last row) may be poisoned too; earlier rows
    # and the other sequence must match the oracle.
    w = make_prefill(315, [4500, 90], cached=[0, 70], Hq=16, Hkv=8, D=128, bs=64)
    ds = DeviceStep(w)
    ds.store()
    ds.block_tables[0, 66] = w.num_blocks + 5
    ds.attend()
    torch.cuda.synchronize()
    out = ds.out_f64()
    ref, _, _, _ = run_workload(w)
    assert np.all(np.isnan(out[4224:4500]))
    keep = np.r_[0:4180, 4500:4590]
    assert_attention_close(out[keep], ref[keep], rel_l2=1e-2, label="rows that do not reach it")


def test_prefill_loose_max_seqlen_k_is_bitwise_identical():
    # a larger max_seqlen_k only adds planes of empty workgroups to the launch
    w = make_prefill(313, [333, 0, 64, 17, 900], cached=[40, 5, 0, 300, 100], Hq=16, Hkv=8,
                     D=128, bs=64)
    ds = gpu_run(w)
    a = ds.out.clone()
    ds.out.view(torch.int16).fill_(0x7FC0)
    B.paged_attn_prefill_varlen(ds.out, ds.q, ds.k_cache, ds.v_cache, ds.block_tables,
                                ds.cu_seqlens_q, ds.cu_seqlens_k, ds.max_seqlen_q,
                                ds.max_seqlen_k + 777, w.scale)
    torch.cuda.synchronize()
    assert torch.equal(a.view(torch.int16), ds.out.view(torch.int16))
    ref, _, _, _ = run_workload(w)
    assert_attention_close(ds.out_f64(), ref, rel_l2=1e-2, label="loose bound")


def test_chunked_prefill_workload_full():
    # the benchmarked chunked-prefill workload at full size: resident prefixes cut anywhere,
    # so each chunk's store starts inside a block and every query row sits at Lk - Lq + i
    from workloads import make_chunked_prefill
    w = make_chunked_prefill()
    assert (w.num_cached % w.block_size != 0).all()
    ds = gpu_run(w)
    ref, _, kc, vc = run_workload(w)
    assert_attention_close(ds.out_f64(), ref, rel_l2=1e-2, label=w.name)
    # the mid-block store leaves both pools bit-identical to the oracle's scatter
    from tests.parity import oracle_bits, pool_bits
    assert np.array_equal(pool_bits(ds.k_cache), oracle_bits(kc))
    assert np.array_equal(pool_bits(ds.v_cache), oracle_bits(vc))
