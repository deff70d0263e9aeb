"""Child process of tests/test_gpu_checks.py: the device calls with PKV_DEBUG set.

The environment variable is read once per process, so these calls run here, apart from the
test runner. Each case prints a line; any failure raises (non-zero exit status). Valid calls
must compute as usual (checked against the fp64 oracle); calls whose metadata breaks a
precondition must return PKV_ERR_PRECONDITION and leave their outputs untouched; a decode
graph recorded in this mode (the checks are skipped while the stream records) must replay
correctly.
"""
from __future__ import annotations

import os
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

import numpy as np  # noqa: E402
import torch  # noqa: E402

from paged_kv_cache_225_amd import _binding as B  # noqa: E402
from paged_kv_cache_225_amd.harness import DeviceStep, GraphDecodeStep  # noqa: E402
from tests.oracle_pipeline import run_workload  # noqa: E402
from tests.parity import assert_attention_close  # noqa: E402
from workloads import make_config, make_decode, make_prefill  # noqa: E402


def expect_precondition(label, fn, *tensors):
    before = [t.clone() for t in tensors]
    try:
        fn()
    except B.PagedKVError as e:
        assert e.status == B.PKV_ERR_PRECONDITION, (label, e.status)
    else:
        raise AssertionError(f"{label}: the call did not report the violation")
    torch.cuda.synchronize()
    for a, b in zip(before, tensors):
        assert torch.equal(a.view(torch.uint8), b.view(torch.uint8)), f"{label}: output written"
    print(f"debug mode: {label}: rejected, outputs untouched", flush=True)


def main():
    assert os.environ.get("PKV_DEBUG") == "1"
    torch.cuda.set_device(0)
    w = make_config(1)
    ref, _, _, _ = run_workload(w)

    ds = DeviceStep(w)
    ds.step_fused()
    torch.cuda.synchronize()
    assert_attention_close(ds.out_f64(), ref, atol=1e-4, rel_l2=1e-5, label="fused decode")
    print("debug mode: valid fused decode computed", flush=True)

    ds = DeviceStep(w)
    ds.step()
    torch.cuda.synchronize()
    assert_attention_close(ds.out_f64(), ref, atol=1e-4, rel_l2=1e-5, label="decode")
    print("debug mode: valid store + decode computed", flush=True)

    # a context length past the tables' capacity
    ctx = ds.context_lens.clone()
    ctx[1] = ds.block_tables.shape[1] * w.block_size + 1
    ds.out.fill_(7.0)
    expect_precondition(
        "decode, context past capacity",
        lambda: B.paged_attn_decode(ds.out, ds.q, ds.k_cache, ds.v_cache, ds.block_tables, ctx,
                                    w.scale, workspace=ds.workspace), ds.out)
    # a block id out of range in a column the call reads
    bt = ds.block_tables.clone()
    bt[0, 0] = w.num_blocks
    expect_precondition(
        "decode, block id out of range",
        lambda: B.paged_attn_decode(ds.out, ds.q, ds.k_cache, ds.v_cache, bt, ds.context_lens,
                                    w.scale, workspace=ds.workspace), ds.out)
    # the fused store's slot pointing at another sequence's key
    slots = ds.slot_mapping.clone()
    slots[0] = slots[1] - 1
    expect_precondition(
        "decode_store, slot not the newest position's",
        lambda: B.paged_attn_decode_store(ds.out, ds.q, ds.new_k, ds.new_v, slots, ds.k_cache,
                                          ds.v_cache, ds.block_tables, ds.context_lens, w.scale,
                                          workspace=ds.workspace), ds.out, ds.k_cache, ds.v_cache)
    # a store with a duplicated slot
    dup = torch.stack([ds.slot_mapping[0], ds.slot_mapping[0]])
    expect_precondition(
        "store_kvcache, duplicate slot",
        lambda: B.store_kvcache(ds.new_k, ds.new_v, ds.k_cache, ds.v_cache, dup), ds.k_cache,
        ds.v_cache)

    # prefill: a valid call computes; Lk < Lq is rejected
    wp = make_prefill(7, [70, 129, 5], cached=[0, 256, 300], Hq=16, Hkv=8, D=128, bs=256)
    refp, _, _, _ = run_workload(wp)
    dp = DeviceStep(wp)
    dp.step()
    torch.cuda.synchronize()
    assert_attention_close(dp.out_f64(), refp, label="prefill")
    print("debug mode: valid prefill computed", flush=True)
    cu_k = dp.cu_seqlens_k.clone()
    cu_k[1:] -= 60  # sequence 0 keeps 10 keys for 70 queries
    dp.out.fill_(3.0)
    expect_precondition(
        "prefill, Lk < Lq",
        lambda: B.paged_attn_prefill_varlen(dp.out, dp.q, dp.k_cache, dp.v_cache,
                                            dp.block_tables, dp.cu_seqlens_q, cu_k,
                                            dp.max_seqlen_q, dp.max_seqlen_k, wp.scale), dp.out)

    # shared-prefix decode: valid groups compute; a member outside the batch and a member
    # holding another block in the group's column are rejected before any launch
    rng = np.random.default_rng(41)
    ctx = rng.integers(3 * 64 + 1, 6 * 64, size=24)
    shared = np.minimum(rng.integers(0, 4, size=24), (ctx - 1) // 64)
    wx = make_decode(42, ctx, Hq=16, Hkv=8, D=128, dtype="bf16", bs=64, shared_blocks=shared,
                     n_prefix_blocks=3, name="debug prefix")
    refx, _, _, _ = run_workload(wx)
    dx = DeviceStep(wx)
    dx.store()
    pf = dx.prefix_setup()
    dx.attend_prefix()
    torch.cuda.synchronize()
    assert_attention_close(dx.out_f64(), refx, rel_l2=1e-2, label="prefix decode")
    print("debug mode: valid shared-prefix decode computed", flush=True)
    mem = pf["group_members"].clone()
    mem[0] = wx.num_seqs
    dx.out.fill_(5.0)
    expect_precondition(
        "decode_prefix, member outside the batch",
        lambda: B.paged_attn_decode_prefix(dx.out, dx.q, dx.k_cache, dx.v_cache, dx.block_tables,
                                           dx.context_lens, wx.scale, pf["shared_cols"],
                                           pf["group_ptr"], mem, pf["group_col"],
                                           pf["max_group_size"], workspace=dx.pfx_workspace),
        dx.out)
    g = int(np.argmax(np.diff(pf["group_ptr"].cpu().numpy())))
    e = int(pf["group_ptr"][g]) + 1
    bt = dx.block_tables.clone()
    bt[int(pf["group_members"][e]), int(pf["group_col"][g])] += 1
    expect_precondition(
        "decode_prefix, member holding another block",
        lambda: B.paged_attn_decode_prefix(dx.out, dx.q, dx.k_cache, dx.v_cache, bt,
                                           dx.context_lens, wx.scale, pf["shared_cols"],
                                           pf["group_ptr"], pf["group_members"], pf["group_col"],
                                           pf["max_group_size"], workspace=dx.pfx_workspace),
        dx.out)

    # graphs record with the checks skipped and replay correctly
    ds = DeviceStep(w, table_width=4)
    st = GraphDecodeStep(ds, 2)
    st.load([1, 0])
    st.launch(2)
    torch.cuda.synchronize()
    assert_attention_close(st.out.double().cpu().numpy(), ref[[1, 0]], atol=1e-4, rel_l2=1e-5,
                           label="graph replay")
    st.graphs.close()
    print("debug mode: graph recorded and replayed", flush=True)
    print("debug mode: ok", flush=True)


if __name__ == "__main__":
    main()
