"""GPU parity of decode steps replayed from captured HIP graphs (pkv_decode_graphs_*).

One pool holds the resident tokens of a batch of sequences; the graphs are recorded once
over static buffers of max_batch rows. Each step copies a seeded subset of the sequences
into the first B rows, pads the rest of its bucket (context 0, slot -1), replays, and is
checked against the fp64 oracle and, bit for bit, against an eager paged_attn_decode_store
on the same padded buffers. Replays are repeated with eager work and synchronisations
between them, and the pool must end bit-identical to the one the separate store produces.
"""
from __future__ import annotations

import numpy as np
import pytest
import torch

from paged_kv_cache_225_amd import _binding as B
from paged_kv_cache_225_amd.harness import DeviceStep, GraphDecodeStep, LayeredGraphDecodeStep
from tests.oracle_pipeline import run_workload
from tests.parity import assert_attention_close
from workloads import another_layer, make_config, make_decode

pytestmark = pytest.mark.gpu

W = 16  # static table width: 4096 tokens / 256


def _bits(t):
    return t.view(torch.int16) if t.dtype == torch.bfloat16 else t.view(torch.int32)


def _run_steps(w, max_batch, batches, seed):
    ds = DeviceStep(w, table_width=W)
    st = GraphDecodeStep(ds, max_batch)
    ref, _, _, _ = run_workload(w)
    atol = 1e-4 if w.dtype == "f32" else 2e-2
    l2 = 1e-5 if w.dtype == "f32" else 1e-2
    rng = np.random.Generator(np.random.PCG64(seed))
    stream = torch.cuda.current_stream()
    for b in batches:
        seqs = rng.choice(w.num_seqs, size=b, replace=False)
        st.load(seqs)
        bucket = st.graphs.bucket(b)
        assert bucket >= b and bucket in st.graphs.buckets
        st.out.fill_(float("nan"))
        st.graphs.launch(b, stream)
        torch.cuda.synchronize()
        got = st.out[:b].double().cpu().numpy()
        print(f"graph step batch {b} -> bucket {bucket}", flush=True)
        assert_attention_close(got, ref[seqs], atol=atol, rel_l2=l2, label=f"graph batch {b}")
        pad = st.out[b:bucket]
        assert torch.equal(pad, torch.zeros_like(pad)), "padded rows must be zero"
        # the same call eagerly on the same padded buffers: bit for bit
        first = st.out[:bucket].clone()
        eager = torch.empty_like(st.out)
        st.eager(b, out=eager, stream=stream)
        torch.cuda.synchronize()
        assert torch.equal(_bits(eager[:bucket]), _bits(first)), "graph != eager"
        # replays with eager work and synchronisations in between
        for r in range(3):
            st.out.fill_(float("nan"))
            junk = torch.randn(256, 256, device=ds.q.device)
            junk = junk @ junk
            torch.cuda.synchronize()
            st.graphs.launch(b, stream)
            torch.cuda.synchronize()
            assert torch.equal(_bits(st.out[:bucket]), _bits(first)), f"replay {r} differs"
    return ds, st


def test_graph_buckets_follow_the_engine_list():
    w = make_decode(7, [5, 9], Hq=4, Hkv=2, D=64, dtype="f32")
    ds = DeviceStep(w, table_width=W)
    for max_batch, want in [(1, [1]), (6, [1, 2, 4, 6]), (16, [1, 2, 4, 8, 16]),
                            (50, [1, 2, 4, 8, 16, 32, 48, 50]),
                            (512, [1, 2, 4, 8] + list(range(16, 513, 16)))]:
        st = GraphDecodeStep(ds, max_batch)
        assert st.graphs.buckets == want
        assert st.graphs.bucket(1) == 1
        assert st.graphs.bucket(max_batch) == max_batch
        with pytest.raises(B.PagedKVError):
            st.graphs.bucket(max_batch + 1)
        with pytest.raises(B.PagedKVError):
            st.graphs.launch(0)
        st.graphs.close()


def test_graph_decode_qwen3_shapes():
    # 64 sequences, the bench workload's head shapes, lengths mixing edge cases and U[256, 4096]
    rng = np.random.Generator(np.random.PCG64(2024))
    ctx = np.concatenate([[1, 2, 255, 256, 257, 4096, 4095, 513],
                          rng.integers(256, 4096, size=56, endpoint=True)])
    w = make_decode(31, ctx, Hq=16, Hkv=8, D=128, dtype="bf16", name="graph64")
    ds, st = _run_steps(w, 64, [1, 3, 13, 16, 48, 64], seed=5)
    # every sequence's newest token went through the fused store at least once (batch 64):
    # the pool matches the one store_kvcache of all the step's tokens produces
    sep = DeviceStep(w, table_width=W)
    sep.store()
    torch.cuda.synchronize()
    assert torch.equal(_bits(ds.k_cache), _bits(sep.k_cache))
    assert torch.equal(_bits(ds.v_cache), _bits(sep.v_cache))


def test_graph_decode_tiny_fp32():
    w = make_config(1)
    _run_steps(w, 2, [1, 2, 1], seed=9)


def test_graph_decode_lengths_change_between_replays():
    # the same recorded graph serves different context lengths: everything that depends on
    # the data is computed on the device at replay time
    w = make_decode(41, [4096, 300, 17, 2000, 1, 777, 3000, 64], Hq=16, Hkv=8, D=128,
                    dtype="bf16", name="graph8")
    ds = DeviceStep(w, table_width=W)
    st = GraphDecodeStep(ds, 8)
    ref, _, _, _ = run_workload(w)
    for seqs in ([0, 1, 2, 3, 4, 5, 6, 7], [7, 6, 5, 4, 3, 2, 1, 0], [3, 1, 4, 0, 5, 7, 2, 6]):
        st.load(seqs)
        st.launch(8)
        torch.cuda.synchronize()
        assert_attention_close(st.out.double().cpu().numpy(), ref[seqs], label=f"rows {seqs}")


def test_graph_recorded_with_streaming_loads():
    """Graphs recorded with a per-row kv_stream_from buffer (every K/V row streamed) replay
    correctly: the replay matches the oracle and equals, bit for bit, the eager call made
    with the buffer or with no streaming at all (the loads never change the arithmetic)."""
    w = make_config(2)
    ds = DeviceStep(w, table_width=W)
    st = GraphDecodeStep(ds, 64, kv_stream_from=0)
    ref, _, _, _ = run_workload(w)
    stream = torch.cuda.current_stream()
    seqs = np.random.Generator(np.random.PCG64(9)).choice(w.num_seqs, size=40, replace=False)
    st.load(seqs)
    bucket = st.graphs.bucket(40)
    st.out.fill_(float("nan"))
    st.graphs.launch(40, stream)
    torch.cuda.synchronize()
    assert_attention_close(st.out[:40].double().cpu().numpy(), ref[seqs], label="streaming graph")
    first = st.out[:bucket].clone()
    for ksf in (None, "graph"):
        eager = torch.empty_like(st.out)
        st.eager(40, out=eager, stream=stream, kv_stream_from=ksf)
        torch.cuda.synchronize()
        assert torch.equal(_bits(eager[:bucket]), _bits(first)), ksf
    st.graphs.close()


def _layered_workloads(n_layers):
    rng = np.random.Generator(np.random.PCG64(606))
    ctx = np.concatenate([[1, 256, 257, 4096], rng.integers(2, 4096, size=20, endpoint=True)])
    w0 = make_decode(61, ctx, Hq=16, Hkv=8, D=128, dtype="bf16", name="layers24")
    return [w0] + [another_layer(w0, 700 + l) for l in range(1, n_layers)]


def test_layered_graph_decode_matches_the_oracle_per_layer():
    """A graph recording a three-layer decode step (one paged_attn_decode_store per layer, each
    layer its own pool and rows over shared metadata) replays every layer's output to the
    fp64 oracle of that layer, equals the eager layer-by-layer calls bit for bit, and leaves
    each layer's pool as store_kvcache of that layer's new tokens does."""
    ws = _layered_workloads(3)
    layers = [DeviceStep(w, table_width=W) for w in ws]
    st = LayeredGraphDecodeStep(layers, 24)
    refs = [run_workload(w)[0] for w in ws]
    stream = torch.cuda.current_stream()
    rng = np.random.Generator(np.random.PCG64(8))
    for b in (5, 16, 24):
        seqs = rng.choice(ws[0].num_seqs, size=b, replace=False)
        st.load(seqs)
        bucket = st.graphs.bucket(b)
        for o in st.out:
            o.fill_(float("nan"))
        st.launch(b, stream)
        torch.cuda.synchronize()
        print(f"layered graph batch {b} -> bucket {bucket}", flush=True)
        for l, ref in enumerate(refs):
            assert_attention_close(st.out[l][:b].double().cpu().numpy(), ref[seqs],
                                   label=f"layer {l} batch {b}")
        first = [o[:bucket].clone() for o in st.out]
        eager = [torch.empty_like(o) for o in st.out]
        st.eager(b, out=eager, stream=stream)
        torch.cuda.synchronize()
        for l in range(len(ws)):
            assert torch.equal(_bits(eager[l][:bucket]), _bits(first[l])), f"layer {l}"
    # the batch-24 step stored every sequence's newest token into every layer's pool
    for l, w in enumerate(ws):
        sep = DeviceStep(w, table_width=W)
        sep.store()
        torch.cuda.synchronize()
        assert torch.equal(_bits(layers[l].k_cache), _bits(sep.k_cache)), f"layer {l} K"
        assert torch.equal(_bits(layers[l].v_cache), _bits(sep.v_cache)), f"layer {l} V"
    st.graphs.close()


def test_layered_graph_of_a_whole_model_depth():
    """28 layers (a Qwen3-0.6B forward's attention calls) in one graph per bucket: replicas of
    one layer's pool and rows give identical outputs in every layer, the replay equals the
    eager calls, and layer 0 matches the oracle."""
    w = _layered_workloads(1)[0]
    ds = DeviceStep(w, table_width=W)
    layers = [ds] + [ds.replica() for _ in range(27)]
    st = LayeredGraphDecodeStep(layers, 24)
    ref = run_workload(w)[0]
    stream = torch.cuda.current_stream()
    seqs = np.random.Generator(np.random.PCG64(12)).choice(w.num_seqs, size=13, replace=False)
    st.load(seqs)
    for o in st.out:
        o.fill_(float("nan"))
    st.launch(13, stream)
    torch.cuda.synchronize()
    assert_attention_close(st.out[0][:13].double().cpu().numpy(), ref[seqs], label="layer 0")
    bucket = st.graphs.bucket(13)
    for l in range(1, 28):
        assert torch.equal(_bits(st.out[l][:bucket]), _bits(st.out[0][:bucket])), f"layer {l}"
    first = [o[:bucket].clone() for o in st.out]
    eager = [torch.empty_like(o) for o in st.out]
    st.eager(13, out=eager, stream=stream)
    torch.cuda.synchronize()
    for l in range(28):
        assert torch.equal(_bits(eager[l][:bucket]), _bits(first[l])), f"layer {l}"
    st.graphs.close()


def test_layered_graph_with_streaming_loads():
    """The layered recording with a per-row kv_stream_from buffer (every K/V row streamed, as
    the bench's 28-layer leg uses it): each layer matches its oracle and equals, bit for
    bit, the eager layer-by-layer calls made with the same buffer."""
    ws = _layered_workloads(2)
    layers = [DeviceStep(w, table_width=W) for w in ws]
    st = LayeredGraphDecodeStep(layers, 24, kv_stream_from=0)
    refs = [run_workload(w)[0] for w in ws]
    stream = torch.cuda.current_stream()
    seqs = np.random.Generator(np.random.PCG64(21)).choice(ws[0].num_seqs, size=11, replace=False)
    st.load(seqs)
    bucket = st.graphs.bucket(11)
    st.launch(11, stream)
    torch.cuda.synchronize()
    for l, ref in enumerate(refs):
        assert_attention_close(st.out[l][:11].double().cpu().numpy(), ref[seqs],
                               label=f"streamed layer {l}")
    first = [o[:bucket].clone() for o in st.out]
    eager = [torch.empty_like(o) for o in st.out]
    st.eager(11, out=eager, stream=stream)
    torch.cuda.synchronize()
    for l in range(len(ws)):
        assert torch.equal(_bits(eager[l][:bucket]), _bits(first[l])), f"layer {l}"
    st.graphs.close()
