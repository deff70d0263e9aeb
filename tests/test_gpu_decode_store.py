"""GPU parity of paged_attn_decode_store (the decode step with its store fused in) against
the fp64 oracle, which runs the step as store_kvcache followed by decode attention."""
from __future__ import annotations

import numpy as np
import pytest
import torch

from paged_kv_cache_225_amd import _binding as B
from paged_kv_cache_225_amd.harness import DeviceStep
from tests.oracle_pipeline import run_workload
from tests.parity import assert_attention_close
from tests.test_gpu_decode import SMALL
from workloads import make_config, make_decode

pytestmark = pytest.mark.gpu


def _bits(t):
    return t.view(torch.int16) if t.dtype == torch.bfloat16 else t.view(torch.int32)


def check_fused(w, partition_size=0, seqs=None):
    ds = DeviceStep(w, partition_size=partition_size)
    ds.step_fused()
    torch.cuda.synchronize()
    ref, _, _, _ = run_workload(w, seqs=seqs)
    out = ds.out_f64()
    if seqs is not None:
        out, ref = out[seqs], ref[seqs]
    atol = 1e-4 if w.dtype == "f32" else 2e-2
    l2 = 1e-5 if w.dtype == "f32" else 1e-2
    st = assert_attention_close(out, ref, atol=atol, rel_l2=l2, label=w.name + " fused")
    # the store half: the caches end bit for bit as after store_kvcache + paged_attn_decode
    sep = DeviceStep(w, partition_size=partition_size)
    sep.step()
    torch.cuda.synchronize()
    assert torch.equal(_bits(ds.k_cache), _bits(sep.k_cache))
    assert torch.equal(_bits(ds.v_cache), _bits(sep.v_cache))
    return ds, sep, st


@pytest.mark.parametrize("case", range(len(SMALL)))
def test_decode_store_small_cases(case):
    dtype, D, Hq, Hkv, bs, ctx, part = SMALL[case]
    w = make_decode(100 + case, ctx, Hq=Hq, Hkv=Hkv, D=D, dtype=dtype, bs=bs, name=f"small{case}")
    check_fused(w, partition_size=part)


def test_decode_store_config_full():
    w = make_config(2)
    ds, sep, st = check_fused(w)
    print(f"config 2 fused: {st}", flush=True)
    # same step as the two separate calls, up to rounding
    assert_attention_close(ds.out_f64(), sep.out_f64(), label="fused vs separate")
    first = ds.out.clone()
    ds.step_fused()
    torch.cuda.synchronize()
    assert torch.equal(first.view(torch.int16), ds.out.view(torch.int16)), "not deterministic"


def test_decode_store_large_config_full():
    """The fused step on all 512 rows of the large decode workload against the oracle, and
    the pools bit for bit against the separate store."""
    w = make_config(5)
    print("config 5 fused: GPU and oracle steps", flush=True)
    _, _, st = check_fused(w)
    print(f"config 5 fused, all {w.num_seqs} seqs: {st}", flush=True)


def test_decode_store_padding_rows_skip_store_and_give_zero():
    """Graph-style padding: a row with context length 0 and slot -1 reads and writes nothing."""
    w = make_decode(210, [600, 5, 2000], Hq=16, Hkv=8, D=128, dtype="bf16", bs=256)
    ds = DeviceStep(w)
    pad_slot = int(ds.slot_mapping[1].item())
    before_k = ds.k_cache.view(-1, w.num_kv_heads, w.head_dim)[pad_slot].clone()
    ds.context_lens[1] = 0
    ds.slot_mapping[1] = -1
    ds.step_fused()
    torch.cuda.synchronize()
    out = ds.out_f64()
    assert np.all(out[1] == 0)
    after_k = ds.k_cache.view(-1, w.num_kv_heads, w.head_dim)[pad_slot]
    assert torch.equal(before_k.view(torch.int16), after_k.view(torch.int16))
    ref, _, _, _ = run_workload(w, seqs=[0, 2])
    assert_attention_close(out[[0, 2]], ref[[0, 2]], label="padding, other rows")


def test_decode_store_strided_token_rows():
    """key/value as views into a wider per-token buffer (as a fused qkv projection gives)."""
    w = make_decode(211, [300, 1, 1500, 64], Hq=16, Hkv=8, D=128, dtype="bf16", bs=256)
    ds = DeviceStep(w)
    row = w.num_kv_heads * w.head_dim
    wide = torch.zeros(w.num_seqs, 3 * row, dtype=ds.new_k.dtype, device=ds.new_k.device)
    wide[:, row:2 * row] = ds.new_k.reshape(w.num_seqs, row)
    wide[:, 2 * row:] = ds.new_v.reshape(w.num_seqs, row)
    ds.new_k = wide[:, row:2 * row].view(w.num_seqs, w.num_kv_heads, w.head_dim)
    ds.new_v = wide[:, 2 * row:].view(w.num_seqs, w.num_kv_heads, w.head_dim)
    ds.step_fused()
    torch.cuda.synchronize()
    ref, _, _, _ = run_workload(w)
    assert_attention_close(ds.out_f64(), ref, label="strided rows")


def test_decode_store_misaligned_rows_are_rejected():
    w = make_decode(212, [300, 40], Hq=16, Hkv=8, D=128, dtype="bf16", bs=256)
    ds = DeviceStep(w)
    row = w.num_kv_heads * w.head_dim
    flat = torch.zeros(w.num_seqs * row + 1, dtype=ds.new_k.dtype, device=ds.new_k.device)
    bad = flat[1:].view(w.num_seqs, w.num_kv_heads, w.head_dim)   # 2-byte offset
    with pytest.raises(B.PagedKVError):
        B.paged_attn_decode_store(ds.out, ds.q, bad, ds.new_v, ds.slot_mapping, ds.k_cache,
                                  ds.v_cache, ds.block_tables, ds.context_lens, w.scale,
                                  workspace=ds.workspace)
