"""paged_attn_decode_noalloc (the decode call for callers that cannot allocate: its partials
live in the library's per-GPU scratch array) against paged_attn_decode with a caller-owned
workspace: two calls in a row, the second on fewer sequences, each bitwise equal to the
workspace call and within the bf16 gate of the fp64 oracle."""
from __future__ import annotations

import numpy as np
import pytest
import torch

from paged_kv_cache_225_amd import _binding as B
from paged_kv_cache_225_amd.harness import DeviceStep
from tests.oracle_pipeline import run_workload
from tests.parity import assert_attention_close
from workloads import make_config

pytestmark = pytest.mark.gpu


def _bits(t):
    return t.view(torch.int16) if t.dtype == torch.bfloat16 else t.view(torch.int32)


def test_noalloc_decode_matches_the_workspace_call_on_two_calls():
    w = make_config(2)
    ds = DeviceStep(w)
    ds.store()
    torch.cuda.synchronize()
    ref, _, _, _ = run_workload(w)
    for n in (64, 16):  # the second call is smaller
        print(f"noalloc decode: {n} sequences", flush=True)
        args = (ds.q[:n], ds.k_cache, ds.v_cache, ds.block_tables[:n], ds.context_lens[:n],
                w.scale)
        want = torch.full_like(ds.out[:n], float("nan"))
        B.paged_attn_decode(want, *args, workspace=ds.workspace)
        got = torch.full_like(ds.out[:n], float("nan"))
        B.paged_attn_decode_noalloc(got, *args)
        torch.cuda.synchronize()
        assert torch.equal(_bits(got), _bits(want)), n
        assert_attention_close(got.double().cpu().numpy(), ref[:n], rel_l2=1e-2,
                               label=f"noalloc {n}")


def test_noalloc_decode_fp32_and_streamed_rows():
    w = make_config(1)
    ds = DeviceStep(w)
    ds.store()
    ref, _, _, _ = run_workload(w)
    zeros = torch.zeros(w.num_seqs, dtype=torch.int32, device=ds.q.device)
    for ksf in (None, zeros):
        got = torch.full_like(ds.out, float("nan"))
        B.paged_attn_decode_noalloc(got, ds.q, ds.k_cache, ds.v_cache, ds.block_tables,
                                    ds.context_lens, w.scale, kv_stream_from=ksf)
        torch.cuda.synchronize()
        assert_attention_close(got.double().cpu().numpy(), ref, atol=1e-4, rel_l2=1e-5,
                               label="noalloc fp32")


def test_noalloc_decode_rejects_calls_beyond_its_scratch():
    # 2048 sequences of 16 x 256 keys need ~290 MB of partials: refused before any launch
    w = make_config(2)
    ds = DeviceStep(w)
    need = B.paged_attn_decode_workspace_bytes(2048, w.num_heads, w.head_dim, 16, 256, 0)
    assert need > B.PKV_DECODE_NOALLOC_SCRATCH_BYTES
    q = torch.zeros(2048, w.num_heads, w.head_dim, dtype=ds.q.dtype, device=ds.q.device)
    tables = torch.zeros(2048, 16, dtype=torch.int32, device=ds.q.device)
    ctx = torch.ones(2048, dtype=torch.int32, device=ds.q.device)
    with pytest.raises(B.PagedKVError) as e:
        B.paged_attn_decode_noalloc(torch.empty_like(q), q, ds.k_cache, ds.v_cache, tables, ctx,
                                    w.scale)
    assert e.value.status == -3
