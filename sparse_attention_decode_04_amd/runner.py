"""Device plumbing around the four C-ABI calls.

DeviceRows uploads one workload (a RowsInputs from inputs.py) to the current
HIP device, allocates every output and workspace with torch, builds the two
row tables and runs the decode path as the four library calls in order on one
stream. It performs no arithmetic of its own.

Row wiring: indexer row r reads q/weights row r and writes its 512 indices at
512*r; sparse row r reads indices at 512*r with width min(kv_len, 512) and
writes q/out row r. A subset of rows can be selected (for one-row launches);
selected rows keep their original q_row and offsets.
"""
from __future__ import annotations

import numpy as np
import torch

from . import ds_rows as ds
from .inputs import HEAD_DIM, HEADS, TOP_K, RowsInputs


def to_device(a: np.ndarray, device) -> torch.Tensor:
    a = np.ascontiguousarray(a)
    if a.dtype == np.uint16:
        a = a.view(np.int16)
    return torch.from_numpy(a).to(device)


def pooled(arrays, device):
    """One device allocation holding every array (row after row) and a view
    of each: a cache pool, as a server keeps a layer's cached rows."""
    flat = [np.ascontiguousarray(a).view(np.int16) if a.dtype == np.uint16 else np.ascontiguousarray(a)
            for a in arrays]
    pool = torch.from_numpy(np.concatenate([a.reshape(-1) for a in flat])).to(device)
    views, at = [], 0
    for a in flat:
        views.append(pool[at: at + a.size].view(a.shape))
        at += a.size
    return pool, views


class DeviceInputs:
    """Device copies of a workload's inputs (shared by any number of runs).
    Every row's KV rows sit in one allocation (the per-row tensors are views
    into it); each row's indexer keys are an allocation of their own."""

    def __init__(self, inp: RowsInputs, device="cuda"):
        self.inp = inp
        self.device = device
        self.idx_q = to_device(inp.idx_q, device)
        self.idx_w = to_device(inp.idx_w, device)
        self.keys = [to_device(k, device) for k in inp.idx_keys]
        self.attn_q = to_device(inp.attn_q, device)
        self.sinks = to_device(inp.sinks, device)
        self.kv_pool, self.kv = pooled(inp.kv, device)

    def clone(self) -> "DeviceInputs":
        """An independent device copy (new allocations, same values)."""
        c = DeviceInputs.__new__(DeviceInputs)
        c.inp, c.device = self.inp, self.device
        c.idx_q, c.idx_w, c.attn_q, c.sinks = (self.idx_q.clone(), self.idx_w.clone(), self.attn_q.clone(),
                                               self.sinks.clone())
        c.keys = [k.clone() for k in self.keys]
        c.kv_pool = self.kv_pool.clone()
        c.kv = [c.kv_pool[k.storage_offset() - self.kv_pool.storage_offset():][:k.numel()].view(k.shape)
                for k in self.kv]
        return c


class DeviceRows:
    def __init__(self, dev: DeviceInputs, rows=None, width=None):
        inp = dev.inp
        self.dev = dev
        self.rows = list(range(inp.rows)) if rows is None else list(rows)
        R_all = inp.rows
        sel = self.rows
        kv_len = [inp.kv_len[r] for r in sel]
        self.width = [min(n, TOP_K) for n in kv_len] if width is None else list(width)
        self.itab = ds.indexer_rows(
            kv_len, [inp.start_pos[r] for r in sel], [inp.offset[r] for r in sel], sel,
            [TOP_K * r for r in sel], keys=[dev.keys[r] for r in sel])
        self.stab = ds.sparse_rows(
            kv_len, self.width, [TOP_K * r for r in sel], sel, kv=[dev.kv[r] for r in sel])
        d = dev.device
        self.scores = torch.empty(ds.scores_elems(self.itab), dtype=torch.float32, device=d)
        self.topk_ws = torch.empty(max(1, ds.topk_workspace_bytes(self.itab)), dtype=torch.uint8, device=d)
        self.fused_ws = torch.empty(ds.indexer_topk_workspace_bytes(self.itab), dtype=torch.uint8, device=d)
        self.indices = torch.full((R_all * TOP_K,), -7, dtype=torch.int32, device=d)
        self.gathered = torch.empty(ds.gathered_elems(self.stab), dtype=torch.int16, device=d)
        self.mask = torch.empty(ds.mask_elems(self.stab), dtype=torch.int16, device=d)
        self.invalid = torch.full((len(self.rows),), 7, dtype=torch.int32, device=d)
        self.attn_ws = torch.empty(ds.attn_workspace_bytes(self.stab), dtype=torch.uint8, device=d)
        self.out = torch.zeros(R_all * HEADS * HEAD_DIM, dtype=torch.float32, device=d)
        self.scale = inp.scale

    # the four calls
    def indexer_score(self, stream=None):
        ds.indexer_score(self.itab, self.dev.idx_q, self.dev.idx_w, self.scores, stream)

    def topk(self, stream=None):
        ds.topk(self.itab, self.scores, self.topk_ws, self.indices, stream)

    def indexer_topk(self, stream=None):
        ds.indexer_topk(self.itab, self.dev.idx_q, self.dev.idx_w, self.scores, self.fused_ws, self.indices, stream)

    def indexer_candidates(self, stream=None):
        ds.indexer_candidates(self.itab, self.dev.idx_q, self.dev.idx_w, self.scores, self.fused_ws, stream)

    def indexer_topk_attn(self, stream=None):
        ds.indexer_topk_attn(self.itab, self.stab, self.dev.idx_q, self.dev.idx_w, self.scores, self.fused_ws,
                             self.indices, self.dev.attn_q, self.dev.sinks, self.scale, self.attn_ws, self.out,
                             stream)

    def gather(self, stream=None):
        ds.gather(self.stab, self.indices, self.gathered, self.mask, self.invalid, stream)

    def sparse_attn(self, stream=None):
        ds.sparse_attn(self.stab, self.dev.attn_q, self.dev.sinks, self.gathered, self.mask, self.invalid,
                       self.scale, self.attn_ws, self.out, stream)

    def sparse_attn_direct(self, stream=None):
        ds.sparse_attn_direct(self.stab, self.dev.attn_q, self.dev.sinks, self.indices, self.scale,
                              self.attn_ws, self.out, stream)

    def step(self, stream=None):
        """The four calls: indexer, top-k, gather, attention on the gathered rows."""
        self.indexer_score(stream)
        self.topk(stream)
        self.gather(stream)
        self.sparse_attn(stream)

    def step_direct(self, stream=None):
        """Indexer, top-k, then attention reading the selected KV rows directly
        (gather fused into the attention call; no gathered operand written)."""
        self.indexer_score(stream)
        self.topk(stream)
        self.sparse_attn_direct(stream)

    def step_fused(self, stream=None):
        """Indexer with the first top-k stage fused in (one call for score and
        top-512), then attention reading the selected KV rows directly."""
        self.indexer_topk(stream)
        self.sparse_attn_direct(stream)

    def step_one(self, stream=None):
        """The decode core in one call (ds_rows_indexer_topk_attn): the fused
        indexer, then the final top-k level inside the attention's
        workgroups, then the combine."""
        self.indexer_topk_attn(stream)

    # host copies, per selected row
    def results(self) -> list[dict]:
        torch.cuda.synchronize()
        inp = self.dev.inp
        scores = self.scores.cpu().numpy()
        stride = scores.size // len(self.rows)
        idx = self.indices.cpu().numpy()
        gathered = self.gathered.cpu().numpy().view(np.uint16)
        mask = self.mask.cpu().numpy().view(np.uint16)
        invalid = self.invalid.cpu().numpy().view(np.uint32)
        out = self.out.cpu().numpy().reshape(inp.rows, HEADS, HEAD_DIM)
        res, base = [], 0
        for i, r in enumerate(self.rows):
            w = self.width[i]
            res.append(dict(
                row=r,
                scores=scores[i * stride: i * stride + inp.kv_len[r]],
                indices=idx[TOP_K * r: TOP_K * (r + 1)],
                gathered=gathered[base * HEAD_DIM:(base + w) * HEAD_DIM].reshape(w, HEAD_DIM),
                mask=mask[base: base + w],
                invalid=int(invalid[i]),
                out=out[r],
            ))
            base += w
        return res


class DeviceCompressor:
    """One compressor workload (a CompressorInputs from inputs.py) on the
    current HIP device: inputs, per-row states (fresh copies of the
    workload's states) and a bf16 output. `copies` > 1
    keeps several independent state sets, for timing without reusing one
    row's state between calls."""

    def __init__(self, inp, device="cuda", rows=None, copies=1):
        self.inp = inp
        self.rows = list(range(inp.rows)) if rows is None else list(rows)
        self.kv = to_device(inp.kv[self.rows], device)
        self.score = to_device(inp.score[self.rows], device)
        self.ape = to_device(inp.ape, device)
        self.norm = to_device(inp.norm, device)
        self.out = torch.zeros(len(self.rows), inp.head_dim, dtype=torch.int16, device=device)
        self.states = []
        for _ in range(copies):
            kvs = [to_device(inp.kv_state[r], device) for r in self.rows]
            scs = [to_device(inp.score_state[r], device) for r in self.rows]
            self.states.append((kvs, scs))
        self.tables = [ds.compressor_rows([inp.start_pos[r] for r in self.rows], kvs, scs)
                       for kvs, scs in self.states]

    def run(self, copy=0, stream=None):
        inp = self.inp
        ds.compressor(self.tables[copy], inp.ratio, inp.head_dim, inp.eps, self.kv, self.score, self.ape,
                      self.norm, self.out, stream)

    def results(self, copy=0):
        torch.cuda.synchronize()
        kvs, scs = self.states[copy]
        out = self.out.cpu().numpy().view(np.uint16)
        return ([k.cpu().numpy() for k in kvs], [s.cpu().numpy() for s in scs], [out[i] for i in range(len(self.rows))])


class DeviceMultiQuery:
    """A multi-query indexer workload (MultiQueryInputs from inputs.py) on the
    current HIP device: keys, queries, weights and the scores buffer
    [rows * query_len, max kv_len]. `rows` selects a subset (each keeps its
    own queries)."""

    def __init__(self, inp, device="cuda", rows=None):
        self.inp = inp
        self.rows = list(range(inp.rows)) if rows is None else list(rows)
        Q = inp.query_len
        self.q = to_device(inp.idx_q, device)
        self.w = to_device(inp.idx_w, device)
        self.keys = [to_device(inp.idx_keys[r], device) for r in self.rows]
        kv = [inp.kv_len[r] for r in self.rows]
        self.table = ds.indexer_rows(kv, [inp.start_pos[r] for r in self.rows], [0] * len(self.rows),
                                     [Q * r for r in self.rows], [TOP_K * i for i in range(len(self.rows))],
                                     keys=self.keys)
        self.scores = torch.empty(ds.indexer_mq_scores_elems(self.table, Q), dtype=torch.float32, device=device)

    def run(self, stream=None):
        ds.indexer_score_mq(self.table, self.inp.query_len, self.q, self.w, self.scores, stream)

    def results(self):
        """scores[i][t] = float32 [kv_len] of selected row i, query t."""
        torch.cuda.synchronize()
        Q = self.inp.query_len
        s = self.scores.cpu().numpy().reshape(len(self.rows) * Q, -1)
        return [[s[i * Q + t, : self.inp.kv_len[r]] for t in range(Q)] for i, r in enumerate(self.rows)]
