"""Device-side driver of one engine step, built only on the library's entry points.

``DeviceStep(w)`` takes a seeded workload (see the ``workloads`` package), allocates the
paged pool on the GPU poisoned with NaN (as the engine's ``torch.empty`` pool holds
arbitrary bits), makes the resident tokens resident with the library's own metadata and
``store_kvcache``, and prepares the step's inputs. ``step()`` then runs the hot path:
``store_kvcache`` of the new tokens followed by ``paged_attn_decode`` or
``paged_attn_prefill_varlen``; ``step_fused()`` runs a decode step as one
``paged_attn_decode_store`` call. Host metadata is built by the library's host calls.
``GraphDecodeStep`` replays decode steps of any subset of a ``DeviceStep``'s sequences from
the library's recorded graphs, the way the engine's run_model does (static buffers, padded
rows, the smallest bucket that fits). ``LayeredGraphDecodeStep`` does the same for a model
of several attention layers (one ``DeviceStep`` per layer over the same metadata), one
recorded graph covering every layer's call.
"""
from __future__ import annotations

import copy

import numpy as np
import torch

from . import _binding as B


def _to_device(raw: np.ndarray, dtype: str, device) -> torch.Tensor:
    if dtype == "bf16":
        return torch.from_numpy(np.ascontiguousarray(raw).view(np.int16)).to(device).view(torch.bfloat16)
    return torch.from_numpy(np.ascontiguousarray(raw, dtype=np.float32)).to(device)


def _i32(a, device) -> torch.Tensor:
    return torch.from_numpy(np.ascontiguousarray(a, dtype=np.int32)).to(device)


def poison_fill_(t: torch.Tensor) -> torch.Tensor:
    if t.dtype == torch.bfloat16:
        t.view(torch.int16).fill_(0x7FC0)
    else:
        t.view(torch.int32).fill_(0x7FC00000)
    return t


class DeviceStep:
    def __init__(self, w, device="cuda", fill=None, partition_size=0, table_width=None,
                 kv_stream_from=None):
        self.w = w
        self.device = torch.device(device)
        self.partition_size = partition_size
        self.kv_stream_spec = kv_stream_from
        tdt = torch.bfloat16 if w.dtype == "bf16" else torch.float32
        shape = (w.num_blocks, w.block_size, w.num_kv_heads, w.head_dim)
        self.k_cache = torch.empty(shape, dtype=tdt, device=self.device)
        self.v_cache = torch.empty(shape, dtype=tdt, device=self.device)
        if fill is None:
            poison_fill_(self.k_cache)
            poison_fill_(self.v_cache)
        else:
            self.k_cache.fill_(fill)
            self.v_cache.fill_(fill)
        self._make_resident()
        self.table_width = w.max_table_len() if table_width is None else table_width
        self._prepare_step()

    # resident tokens: the common prefix once, then each sequence's private resident range
    def _make_resident(self):
        w = self.w
        segs_cached, segs_sched, segs_tables, ks, vs = [], [], [], [], []
        n_pre = len(w.prefix_block_ids) * w.block_size
        if n_pre:
            segs_cached.append(0)
            segs_sched.append(n_pre)
            segs_tables.append(w.prefix_block_ids)
            ks.append(w.prefix_k)
            vs.append(w.prefix_v)
        for b, lo, hi in w.resident_segments():
            segs_cached.append(lo)
            segs_sched.append(hi - lo)
            segs_tables.append(w.block_tables[b])
            k, v = w.seq_token_rows(b, lo, hi)
            ks.append(k)
            vs.append(v)
        if not ks:
            return
        md = B.pkv_prefill_metadata(segs_cached, segs_sched, segs_tables, w.block_size)
        k = _to_device(np.concatenate(ks), w.dtype, self.device)
        v = _to_device(np.concatenate(vs), w.dtype, self.device)
        B.store_kvcache(k, v, self.k_cache, self.v_cache, _i32(md["slot_mapping"], self.device))
        torch.cuda.synchronize(self.device)

    def _prepare_step(self):
        w, dev = self.w, self.device
        if w.kind == "decode":
            md = B.pkv_decode_metadata(w.seq_lens, w.block_tables, w.block_size, self.table_width)
            self.context_lens = _i32(md["context_lens"], dev)
        else:
            md = B.pkv_prefill_metadata(w.num_cached, w.q_lens, w.block_tables, w.block_size,
                                        self.table_width)
            self.cu_seqlens_q = _i32(md["cu_seqlens_q"], dev)
            self.cu_seqlens_k = _i32(md["cu_seqlens_k"], dev)
            self.max_seqlen_q = md["max_seqlen_q"]
            self.max_seqlen_k = md["max_seqlen_k"]
        self.md = md
        self.slot_mapping = _i32(md["slot_mapping"], dev)
        self.block_tables = _i32(md["block_tables"].reshape(w.num_seqs, -1), dev)
        nk, nv = w.new_tokens()
        self.new_k = _to_device(nk, w.dtype, dev)
        self.new_v = _to_device(nv, w.dtype, dev)
        self.q = _to_device(w.q, w.dtype, dev)
        self.out = torch.empty_like(self.q)
        self.kv_stream_from = self._stream_from(self.kv_stream_spec)
        if w.kind == "decode":
            nbytes = B.paged_attn_decode_workspace_bytes(w.num_seqs, w.num_heads, w.head_dim,
                                                         self.block_tables.shape[1], w.block_size,
                                                         self.partition_size)
            self.workspace = torch.empty(max(nbytes, 1), dtype=torch.uint8, device=dev)

    def _stream_from(self, spec):
        """The decode calls' kv_stream_from: None (every K/V row read with ordinary loads), an
        int (the same first streamed table column for every sequence), "shared" (each
        sequence's count of leading blocks shared with other sequences, as a block manager's
        reference counts give it) or a per-sequence array."""
        if spec is None:
            return None
        if isinstance(spec, str):
            assert spec == "shared", spec
            arr = np.asarray(self.w.shared_blocks, dtype=np.int32)
        elif np.isscalar(spec):
            arr = np.full(self.w.num_seqs, int(spec), dtype=np.int32)
        else:
            arr = np.asarray(spec, dtype=np.int32)
        return _i32(arr, self.device)

    def store(self, stream=None):
        B.store_kvcache(self.new_k, self.new_v, self.k_cache, self.v_cache, self.slot_mapping,
                        stream=stream)

    def attend(self, stream=None):
        w = self.w
        if w.kind == "decode":
            B.paged_attn_decode(self.out, self.q, self.k_cache, self.v_cache, self.block_tables,
                                self.context_lens, w.scale, workspace=self.workspace,
                                partition_size=self.partition_size,
                                kv_stream_from=self.kv_stream_from, stream=stream)
        else:
            B.paged_attn_prefill_varlen(self.out, self.q, self.k_cache, self.v_cache,
                                        self.block_tables, self.cu_seqlens_q, self.cu_seqlens_k,
                                        self.max_seqlen_q, self.max_seqlen_k, w.scale, stream=stream)

    def prefix_setup(self, shared_cols=None):
        """Decode only: the shared-prefix groups of the step's tables for
        paged_attn_decode_prefix (shared_cols: each sequence's count of shared leading
        columns; default the workload's shared blocks) and a workspace for it."""
        w = self.w
        sc = np.asarray(w.shared_blocks if shared_cols is None else shared_cols, dtype=np.int32)
        ptr, mem, col, largest = B.prefix_groups(self.block_tables.cpu().numpy(), sc)
        self.pfx = {"shared_cols": _i32(sc, self.device), "group_ptr": _i32(ptr, self.device),
                    "group_members": _i32(mem if len(mem) else np.zeros(1, np.int32), self.device),
                    "group_col": _i32(col, self.device), "max_group_size": largest,
                    "num_groups": len(col)}
        nbytes = B.paged_attn_decode_prefix_workspace_bytes(
            w.num_seqs, w.num_heads, w.head_dim, self.block_tables.shape[1], w.block_size,
            self.partition_size)
        self.pfx_workspace = torch.empty(max(nbytes, 1), dtype=torch.uint8, device=self.device)
        return self.pfx

    def attend_prefix(self, stream=None):
        """The step's decode attention through paged_attn_decode_prefix (prefix_setup first)."""
        p = self.pfx
        B.paged_attn_decode_prefix(self.out, self.q, self.k_cache, self.v_cache,
                                   self.block_tables, self.context_lens, self.w.scale,
                                   p["shared_cols"], p["group_ptr"], p["group_members"],
                                   p["group_col"], p["max_group_size"],
                                   workspace=self.pfx_workspace,
                                   partition_size=self.partition_size, stream=stream)
        return self.out

    def step(self, stream=None):
        self.store(stream)
        self.attend(stream)
        return self.out

    def step_fused(self, stream=None):
        """Decode only: the same step through paged_attn_decode_store (one call)."""
        w = self.w
        assert w.kind == "decode"
        B.paged_attn_decode_store(self.out, self.q, self.new_k, self.new_v, self.slot_mapping,
                                  self.k_cache, self.v_cache, self.block_tables,
                                  self.context_lens, w.scale, workspace=self.workspace,
                                  partition_size=self.partition_size,
                                  kv_stream_from=self.kv_stream_from, stream=stream)
        return self.out

    def replica(self) -> "DeviceStep":
        """Another layer over the same step: its own pool and rows, device copies of these
        (same metadata tensors, shared)."""
        r = copy.copy(self)
        for name in ("k_cache", "v_cache", "q", "new_k", "new_v", "out"):
            setattr(r, name, getattr(self, name).clone())
        return r

    def out_f64(self) -> np.ndarray:
        o = self.out.float().cpu().numpy() if self.out.dtype == torch.bfloat16 else self.out.cpu().numpy()
        return o.astype(np.float64)


class GraphDecodeStep:
    """Static buffers of max_batch rows over a DeviceStep's pool, with the library's decode
    graphs recorded over them (``pkv_decode_graphs_*``). ``load(seqs)`` copies those
    sequences' step inputs into the first rows and pads the rest of the bucket;
    ``launch(batch)`` replays the bucket's graph."""

    def __init__(self, ds: DeviceStep, max_batch: int, width: int = None,
                 kv_stream_from=None):
        w = ds.w
        assert w.kind == "decode"
        self.ds = ds
        width = ds.block_tables.shape[1] if width is None else width
        assert width >= ds.block_tables.shape[1]
        dev = ds.q.device
        Hq, D = ds.q.shape[1:]
        Hkv = ds.new_k.shape[1]
        self.out = torch.zeros(max_batch, Hq, D, dtype=ds.q.dtype, device=dev)
        self.q = torch.zeros_like(self.out)
        self.key = torch.zeros(max_batch, Hkv, D, dtype=ds.q.dtype, device=dev)
        self.value = torch.zeros_like(self.key)
        self.slots = torch.full((max_batch,), -1, dtype=torch.int32, device=dev)
        self.ctx = torch.zeros(max_batch, dtype=torch.int32, device=dev)
        # rows of padded sequences are never read; an out-of-range id makes that visible
        self.tables = torch.full((max_batch, width), 1 << 30, dtype=torch.int32, device=dev)
        nbytes = B.paged_attn_decode_workspace_bytes(max_batch, w.num_heads, w.head_dim, width,
                                                     w.block_size, ds.partition_size)
        self.workspace = torch.empty(nbytes, dtype=torch.uint8, device=dev)
        # per-row first streamed table column, a static buffer the graphs read at replay
        self.stream_from = None
        if kv_stream_from is not None:
            self.stream_from = torch.full((max_batch,), int(kv_stream_from), dtype=torch.int32,
                                          device=dev)
        self.graphs = B.DecodeGraphs(self.out, self.q, self.key, self.value, self.slots,
                                     ds.k_cache, ds.v_cache, self.tables, self.ctx, w.scale,
                                     self.workspace, ds.partition_size, self.stream_from)

    def load(self, seqs):
        ds, n = self.ds, len(seqs)
        idx = torch.as_tensor(np.asarray(seqs), dtype=torch.long, device=ds.q.device)
        self.q[:n] = ds.q[idx]
        self.key[:n] = ds.new_k[idx]
        self.value[:n] = ds.new_v[idx]
        self.slots[:n] = ds.slot_mapping[idx]
        self.ctx[:n] = ds.context_lens[idx]
        self.tables[:n, :ds.block_tables.shape[1]] = ds.block_tables[idx]
        self.graphs.pad(n)

    def launch(self, batch, stream=None):
        self.graphs.launch(batch, stream)
        return self.out[:batch]

    def eager(self, batch, out=None, stream=None, kv_stream_from="graph"):
        """The recorded call, made eagerly on the same padded buffers (bucket rows)."""
        n = self.graphs.bucket(batch)
        out = self.out if out is None else out
        ds = self.ds
        if isinstance(kv_stream_from, str):  # "graph": the recorded calls' buffer
            kv_stream_from = None if self.stream_from is None else self.stream_from[:n]
        B.paged_attn_decode_store(out[:n], self.q[:n], self.key[:n], self.value[:n],
                                  self.slots[:n], ds.k_cache, ds.v_cache, self.tables[:n],
                                  self.ctx[:n], ds.w.scale, workspace=self.workspace,
                                  partition_size=ds.partition_size,
                                  kv_stream_from=kv_stream_from, stream=stream)
        return out[:batch]


class LayeredGraphDecodeStep:
    """Static buffers of max_batch rows for each of several layers, with the library's decode
    graphs recorded over all of them (``pkv_decode_graphs_create_layers``): one replay runs
    every layer's paged_attn_decode_store in order. ``layers`` are DeviceSteps of one step
    (same sequences, lengths and block tables; each its own pool and rows); the metadata
    buffers are shared by the layers, as the engine's one Context is."""

    def __init__(self, layers, max_batch: int, width: int = None, kv_stream_from=None):
        ds0 = layers[0]
        w = ds0.w
        assert w.kind == "decode"
        for ds in layers[1:]:
            assert torch.equal(ds.block_tables, ds0.block_tables)
            assert torch.equal(ds.context_lens, ds0.context_lens)
            assert torch.equal(ds.slot_mapping, ds0.slot_mapping)
        self.layers = layers
        width = ds0.block_tables.shape[1] if width is None else width
        assert width >= ds0.block_tables.shape[1]
        dev = ds0.q.device
        Hq, D = ds0.q.shape[1:]
        Hkv = ds0.new_k.shape[1]
        dt = ds0.q.dtype
        self.out = [torch.zeros(max_batch, Hq, D, dtype=dt, device=dev) for _ in layers]
        self.q = [torch.zeros(max_batch, Hq, D, dtype=dt, device=dev) for _ in layers]
        self.key = [torch.zeros(max_batch, Hkv, D, dtype=dt, device=dev) for _ in layers]
        self.value = [torch.zeros(max_batch, Hkv, D, dtype=dt, device=dev) for _ in layers]
        self.slots = torch.full((max_batch,), -1, dtype=torch.int32, device=dev)
        self.ctx = torch.zeros(max_batch, dtype=torch.int32, device=dev)
        self.tables = torch.full((max_batch, width), 1 << 30, dtype=torch.int32, device=dev)
        nbytes = B.paged_attn_decode_workspace_bytes(max_batch, w.num_heads, w.head_dim, width,
                                                     w.block_size, ds0.partition_size)
        self.workspace = torch.empty(nbytes, dtype=torch.uint8, device=dev)
        self.stream_from = None
        if kv_stream_from is not None:
            self.stream_from = torch.full((max_batch,), int(kv_stream_from), dtype=torch.int32,
                                          device=dev)
        self.graphs = B.DecodeGraphs(self.out, self.q, self.key, self.value, self.slots,
                                     [ds.k_cache for ds in layers],
                                     [ds.v_cache for ds in layers], self.tables, self.ctx,
                                     w.scale, self.workspace, ds0.partition_size,
                                     self.stream_from)

    def load(self, seqs):
        ds0, n = self.layers[0], len(seqs)
        idx = torch.as_tensor(np.asarray(seqs), dtype=torch.long, device=ds0.q.device)
        for l, ds in enumerate(self.layers):
            self.q[l][:n] = ds.q[idx]
            self.key[l][:n] = ds.new_k[idx]
            self.value[l][:n] = ds.new_v[idx]
        self.slots[:n] = ds0.slot_mapping[idx]
        self.ctx[:n] = ds0.context_lens[idx]
        self.tables[:n, :ds0.block_tables.shape[1]] = ds0.block_tables[idx]
        self.graphs.pad(n)

    def launch(self, batch, stream=None):
        self.graphs.launch(batch, stream)
        return [o[:batch] for o in self.out]

    def eager(self, batch, out=None, stream=None):
        """The recorded calls, made eagerly, layer by layer, on the same padded buffers."""
        n = self.graphs.bucket(batch)
        out = self.out if out is None else out
        ksf = None if self.stream_from is None else self.stream_from[:n]
        for l, ds in enumerate(self.layers):
            B.paged_attn_decode_store(out[l][:n], self.q[l][:n], self.key[l][:n],
                                      self.value[l][:n], self.slots[:n], ds.k_cache,
                                      ds.v_cache, self.tables[:n], self.ctx[:n], ds.w.scale,
                                      workspace=self.workspace,
                                      partition_size=ds.partition_size, kv_stream_from=ksf,
                                      stream=stream)
        return [o[:batch] for o in out]
