"""ctypes binding of libds_rows.so (include/ds_rows.h).

Argument marshalling only: every step of the decode path runs in the HIP
library. Device buffers are torch tensors on the current HIP device; the
binding passes their addresses, capacities and torch's current stream. It
raises DsRowsError with the library's message on any failed call, and
load() raises if the library has not been built: there is no fallback.
"""
from __future__ import annotations

import ctypes
import os
from ctypes import c_float, c_int32, c_size_t, c_uint32, c_uint64, c_void_p

import torch

ROWS_MAX = 8
HEADS = 64
INDEXER_DIM = 128
HEAD_DIM = 512
TOP_K = 512

LIB_PATH = os.path.join(os.path.dirname(os.path.abspath(__file__)), "libds_rows.so")

FUNCTIONS = (
    "ds_rows_scores_elems", "ds_rows_topk_workspace_bytes", "ds_rows_gathered_elems",
    "ds_rows_mask_elems", "ds_rows_attn_workspace_bytes", "ds_rows_indexer_score",
    "ds_rows_topk", "ds_rows_gather", "ds_rows_sparse_attn", "ds_rows_sparse_attn_direct",
    "ds_rows_last_error", "ds_rows_version", "ds_rows_indexer_topk_workspace_bytes", "ds_rows_indexer_topk",
    "ds_rows_indexer_candidates", "ds_rows_compressor_state_elems", "ds_rows_compressor",
    "ds_rows_indexer_mq_scores_elems", "ds_rows_indexer_score_mq", "ds_rows_indexer_topk_attn",
    "ds_rows_indexer_topk_attn_noalloc", "ds_rows_time_next_indexer", "ds_rows_wall_clock_khz",
)


class DsRowsError(RuntimeError):
    pass


class IndexerRows(ctypes.Structure):
    """ds_indexer_rows"""
    _fields_ = [
        ("rows", c_uint32),
        ("kv_len", c_uint32 * ROWS_MAX),
        ("start_pos", c_uint32 * ROWS_MAX),
        ("offset", c_int32 * ROWS_MAX),
        ("q_row", c_uint32 * ROWS_MAX),
        ("output_offset", c_uint32 * ROWS_MAX),
        ("keys", c_void_p * ROWS_MAX),
        ("keys_elems", c_uint64 * ROWS_MAX),
    ]


class SparseRows(ctypes.Structure):
    """ds_sparse_rows"""
    _fields_ = [
        ("rows", c_uint32),
        ("kv_len", c_uint32 * ROWS_MAX),
        ("width", c_uint32 * ROWS_MAX),
        ("index_offset", c_uint32 * ROWS_MAX),
        ("q_row", c_uint32 * ROWS_MAX),
        ("kv", c_void_p * ROWS_MAX),
        ("kv_elems", c_uint64 * ROWS_MAX),
    ]


class CompressorRows(ctypes.Structure):
    """ds_compressor_rows"""
    _fields_ = [
        ("rows", c_uint32),
        ("start_pos", c_uint32 * ROWS_MAX),
        ("kv_state", c_void_p * ROWS_MAX),
        ("score_state", c_void_p * ROWS_MAX),
        ("kv_state_elems", c_uint64 * ROWS_MAX),
        ("score_state_elems", c_uint64 * ROWS_MAX),
    ]


_lib = None


def load(path: str = LIB_PATH) -> ctypes.CDLL:
    """Load the HIP library once. Raises if it is missing."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(path):
        raise DsRowsError(f"{path} is not built; run python -m sparse_attention_decode_04_amd.build")
    lib = ctypes.CDLL(path)
    P = ctypes.POINTER
    lib.ds_rows_scores_elems.argtypes = [P(IndexerRows)]
    lib.ds_rows_topk_workspace_bytes.argtypes = [P(IndexerRows)]
    lib.ds_rows_gathered_elems.argtypes = [P(SparseRows)]
    lib.ds_rows_mask_elems.argtypes = [P(SparseRows)]
    lib.ds_rows_attn_workspace_bytes.argtypes = [P(SparseRows)]
    lib.ds_rows_indexer_topk_workspace_bytes.argtypes = [P(IndexerRows)]
    for f in ("ds_rows_scores_elems", "ds_rows_topk_workspace_bytes", "ds_rows_gathered_elems",
              "ds_rows_mask_elems", "ds_rows_attn_workspace_bytes", "ds_rows_indexer_topk_workspace_bytes"):
        getattr(lib, f).restype = c_size_t
    lib.ds_rows_indexer_score.argtypes = [P(IndexerRows), c_void_p, c_size_t, c_void_p, c_size_t,
                                          c_void_p, c_size_t, c_void_p]
    lib.ds_rows_topk.argtypes = [P(IndexerRows), c_void_p, c_size_t, c_void_p, c_size_t,
                                 c_void_p, c_size_t, c_void_p]
    lib.ds_rows_gather.argtypes = [P(SparseRows), c_void_p, c_size_t, c_void_p, c_size_t,
                                   c_void_p, c_size_t, c_void_p, c_size_t, c_void_p]
    lib.ds_rows_sparse_attn.argtypes = [P(SparseRows), c_void_p, c_size_t, c_void_p, c_size_t,
                                        c_void_p, c_size_t, c_void_p, c_size_t, c_void_p, c_size_t, c_float,
                                        c_void_p, c_size_t, c_void_p, c_size_t, c_void_p]
    lib.ds_rows_sparse_attn_direct.argtypes = [P(SparseRows), c_void_p, c_size_t, c_void_p, c_size_t,
                                               c_void_p, c_size_t, c_float, c_void_p, c_size_t,
                                               c_void_p, c_size_t, c_void_p]
    lib.ds_rows_indexer_topk.argtypes = [P(IndexerRows), c_void_p, c_size_t, c_void_p, c_size_t,
                                         c_void_p, c_size_t, c_void_p, c_size_t, c_void_p, c_size_t, c_void_p]
    lib.ds_rows_indexer_candidates.argtypes = [P(IndexerRows), c_void_p, c_size_t, c_void_p, c_size_t,
                                               c_void_p, c_size_t, c_void_p, c_size_t, c_void_p]
    lib.ds_rows_indexer_topk_attn.argtypes = [P(IndexerRows), P(SparseRows), c_void_p, c_size_t, c_void_p, c_size_t,
                                              c_void_p, c_size_t, c_void_p, c_size_t, c_void_p, c_size_t,
                                              c_void_p, c_size_t, c_void_p, c_size_t, c_float,
                                              c_void_p, c_size_t, c_void_p, c_size_t, c_void_p]
    lib.ds_rows_indexer_topk_attn_noalloc.argtypes = [P(IndexerRows), P(SparseRows), c_void_p, c_size_t,
                                                      c_void_p, c_size_t, c_void_p, c_size_t, c_void_p, c_size_t,
                                                      c_void_p, c_size_t, c_void_p, c_size_t, c_float,
                                                      c_void_p, c_size_t, c_void_p]
    lib.ds_rows_indexer_mq_scores_elems.argtypes = [P(IndexerRows), c_uint32]
    lib.ds_rows_indexer_mq_scores_elems.restype = c_size_t
    lib.ds_rows_indexer_score_mq.argtypes = [P(IndexerRows), c_uint32, c_void_p, c_size_t, c_void_p, c_size_t,
                                             c_void_p, c_size_t, c_void_p]
    lib.ds_rows_compressor_state_elems.argtypes = [c_uint32, c_uint32]
    lib.ds_rows_compressor_state_elems.restype = c_size_t
    lib.ds_rows_compressor.argtypes = [P(CompressorRows), c_uint32, c_uint32, c_float,
                                       c_void_p, c_size_t, c_void_p, c_size_t, c_void_p, c_size_t,
                                       c_void_p, c_size_t, c_void_p, c_size_t, c_void_p]
    for f in ("ds_rows_indexer_score", "ds_rows_topk", "ds_rows_gather", "ds_rows_sparse_attn",
              "ds_rows_sparse_attn_direct", "ds_rows_indexer_topk", "ds_rows_indexer_candidates",
              "ds_rows_compressor", "ds_rows_indexer_score_mq", "ds_rows_indexer_topk_attn",
              "ds_rows_indexer_topk_attn_noalloc"):
        getattr(lib, f).restype = ctypes.c_int
    lib.ds_rows_time_next_indexer.argtypes = [c_void_p, c_size_t]
    lib.ds_rows_time_next_indexer.restype = ctypes.c_int
    lib.ds_rows_wall_clock_khz.argtypes = [ctypes.POINTER(ctypes.c_int)]
    lib.ds_rows_wall_clock_khz.restype = ctypes.c_int
    lib.ds_rows_last_error.restype = ctypes.c_char_p
    lib.ds_rows_version.restype = ctypes.c_char_p
    _lib = lib
    return lib


def last_error() -> str:
    return load().ds_rows_last_error().decode()


def _check(status: int):
    if status != 0:
        raise DsRowsError(f"status {status}: {last_error()}")


def _arr(ctype, values, n=ROWS_MAX):
    a = (ctype * n)()
    for i, v in enumerate(values):
        a[i] = v
    return a


def indexer_rows(kv_len, start_pos, offset, q_row, output_offset, keys=None, keys_elems=None) -> IndexerRows:
    """Build a ds_indexer_rows table. `keys` are device tensors (or raw
    addresses); capacities default to each tensor's element count."""
    t = IndexerRows()
    t.rows = len(kv_len)
    t.kv_len = _arr(c_uint32, kv_len)
    t.start_pos = _arr(c_uint32, start_pos)
    t.offset = _arr(c_int32, offset)
    t.q_row = _arr(c_uint32, q_row)
    t.output_offset = _arr(c_uint32, output_offset)
    keys = keys or []
    t.keys = _arr(c_void_p, [_addr(k) for k in keys])
    if keys_elems is None:
        keys_elems = [k.numel() if isinstance(k, torch.Tensor) else 0 for k in keys]
    t.keys_elems = _arr(c_uint64, keys_elems)
    return t


def sparse_rows(kv_len, width, index_offset, q_row, kv=None, kv_elems=None) -> SparseRows:
    """Build a ds_sparse_rows table."""
    t = SparseRows()
    t.rows = len(kv_len)
    t.kv_len = _arr(c_uint32, kv_len)
    t.width = _arr(c_uint32, width)
    t.index_offset = _arr(c_uint32, index_offset)
    t.q_row = _arr(c_uint32, q_row)
    kv = kv or []
    t.kv = _arr(c_void_p, [_addr(k) for k in kv])
    if kv_elems is None:
        kv_elems = [k.numel() if isinstance(k, torch.Tensor) else 0 for k in kv]
    t.kv_elems = _arr(c_uint64, kv_elems)
    return t


def compressor_rows(start_pos, kv_state=None, score_state=None, kv_state_elems=None,
                    score_state_elems=None) -> CompressorRows:
    """Build a ds_compressor_rows table from per-row device state tensors."""
    t = CompressorRows()
    t.rows = len(start_pos)
    t.start_pos = _arr(c_uint32, start_pos)
    kv_state = kv_state or []
    score_state = score_state or []
    t.kv_state = _arr(c_void_p, [_addr(k) for k in kv_state])
    t.score_state = _arr(c_void_p, [_addr(k) for k in score_state])
    if kv_state_elems is None:
        kv_state_elems = [k.numel() if isinstance(k, torch.Tensor) else 0 for k in kv_state]
    if score_state_elems is None:
        score_state_elems = [k.numel() if isinstance(k, torch.Tensor) else 0 for k in score_state]
    t.kv_state_elems = _arr(c_uint64, kv_state_elems)
    t.score_state_elems = _arr(c_uint64, score_state_elems)
    return t


def _addr(x):
    if x is None:
        return None
    if isinstance(x, int):
        return x
    if not isinstance(x, torch.Tensor):
        raise TypeError(f"expected a device tensor, got {type(x)}")
    if not x.is_cuda:
        raise ValueError("buffers must be device tensors on the HIP device")
    if not x.is_contiguous():
        raise ValueError("buffers must be contiguous")
    return x.data_ptr()


def _dev(x, itemsize=None):
    """(address, element capacity) of a device tensor."""
    if x is None:
        return None, 0
    a = _addr(x)
    if itemsize is not None and x.element_size() != itemsize:
        raise ValueError(f"expected {itemsize}-byte elements, got {x.dtype}")
    return a, x.numel()


def _stream(stream):
    if stream is None:
        return c_void_p(torch.cuda.current_stream().cuda_stream)
    if isinstance(stream, torch.cuda.Stream):
        return c_void_p(stream.cuda_stream)
    return c_void_p(stream)


def scores_elems(t: IndexerRows) -> int:
    return load().ds_rows_scores_elems(ctypes.byref(t))


def topk_workspace_bytes(t: IndexerRows) -> int:
    return load().ds_rows_topk_workspace_bytes(ctypes.byref(t))


def indexer_topk_workspace_bytes(t: IndexerRows) -> int:
    return load().ds_rows_indexer_topk_workspace_bytes(ctypes.byref(t))


def gathered_elems(t: SparseRows) -> int:
    return load().ds_rows_gathered_elems(ctypes.byref(t))


def mask_elems(t: SparseRows) -> int:
    return load().ds_rows_mask_elems(ctypes.byref(t))


def attn_workspace_bytes(t: SparseRows) -> int:
    return load().ds_rows_attn_workspace_bytes(ctypes.byref(t))


def indexer_score(t: IndexerRows, q, weights, scores, stream=None):
    qa, qn = _dev(q, 2)
    wa, wn = _dev(weights, 4)
    sa, sn = _dev(scores, 4)
    _check(load().ds_rows_indexer_score(ctypes.byref(t), qa, qn, wa, wn, sa, sn, _stream(stream)))


def topk(t: IndexerRows, scores, workspace, indices, stream=None):
    sa, sn = _dev(scores, 4)
    wa = _addr(workspace) if workspace is not None else None
    wb = workspace.numel() * workspace.element_size() if workspace is not None else 0
    ia, inn = _dev(indices, 4)
    _check(load().ds_rows_topk(ctypes.byref(t), sa, sn, wa, wb, ia, inn, _stream(stream)))


def indexer_topk(t: IndexerRows, q, weights, scores, workspace, indices, stream=None):
    qa, qn = _dev(q, 2)
    wa, wn = _dev(weights, 4)
    sa, sn = _dev(scores, 4)
    ka = _addr(workspace)
    kb = workspace.numel() * workspace.element_size()
    ia, inn = _dev(indices, 4)
    _check(load().ds_rows_indexer_topk(ctypes.byref(t), qa, qn, wa, wn, sa, sn, ka, kb, ia, inn, _stream(stream)))


def indexer_topk_attn(it: IndexerRows, st: SparseRows, idx_q, weights, scores, idx_workspace, indices,
                      q, sinks, scale, attn_workspace, out, stream=None):
    qa, qn = _dev(idx_q, 2)
    wa, wn = _dev(weights, 4)
    sa, sn = _dev(scores, 4)
    ka = _addr(idx_workspace)
    kb = idx_workspace.numel() * idx_workspace.element_size()
    ia, inn = _dev(indices, 4)
    aqa, aqn = _dev(q, 2)
    ska, skn = _dev(sinks, 4)
    awa = _addr(attn_workspace)
    awb = attn_workspace.numel() * attn_workspace.element_size()
    oa, on = _dev(out, 4)
    _check(load().ds_rows_indexer_topk_attn(ctypes.byref(it), ctypes.byref(st), qa, qn, wa, wn, sa, sn, ka, kb,
                                            ia, inn, aqa, aqn, ska, skn, float(scale), awa, awb, oa, on,
                                            _stream(stream)))


def indexer_topk_attn_noalloc(it: IndexerRows, st: SparseRows, idx_q, weights, scores, indices,
                              q, sinks, scale, out, stream=None):
    """ds_rows_indexer_topk_attn with the library's own device scratch array
    in place of the two workspaces."""
    qa, qn = _dev(idx_q, 2)
    wa, wn = _dev(weights, 4)
    sa, sn = _dev(scores, 4)
    ia, inn = _dev(indices, 4)
    aqa, aqn = _dev(q, 2)
    ska, skn = _dev(sinks, 4)
    oa, on = _dev(out, 4)
    _check(load().ds_rows_indexer_topk_attn_noalloc(ctypes.byref(it), ctypes.byref(st), qa, qn, wa, wn, sa, sn,
                                                    ia, inn, aqa, aqn, ska, skn, float(scale), oa, on,
                                                    _stream(stream)))


def indexer_candidates(t: IndexerRows, q, weights, scores, workspace, stream=None):
    qa, qn = _dev(q, 2)
    wa, wn = _dev(weights, 4)
    sa, sn = _dev(scores, 4)
    ka = _addr(workspace)
    kb = workspace.numel() * workspace.element_size()
    _check(load().ds_rows_indexer_candidates(ctypes.byref(t), qa, qn, wa, wn, sa, sn, ka, kb, _stream(stream)))


def gather(t: SparseRows, indices, gathered, mask, invalid, stream=None):
    ia, inn = _dev(indices, 4)
    ga, gn = _dev(gathered, 2)
    ma, mn = _dev(mask, 2)
    va, vn = _dev(invalid, 4)
    _check(load().ds_rows_gather(ctypes.byref(t), ia, inn, ga, gn, ma, mn, va, vn, _stream(stream)))


def sparse_attn(t: SparseRows, q, sinks, gathered, mask, invalid, scale, workspace, out, stream=None):
    qa, qn = _dev(q, 2)
    sa, sn = _dev(sinks, 4)
    ga, gn = _dev(gathered, 2)
    ma, mn = _dev(mask, 2)
    va, vn = _dev(invalid, 4)
    wa = _addr(workspace)
    wb = workspace.numel() * workspace.element_size()
    oa, on = _dev(out, 4)
    _check(load().ds_rows_sparse_attn(ctypes.byref(t), qa, qn, sa, sn, ga, gn, ma, mn, va, vn, float(scale),
                                      wa, wb, oa, on, _stream(stream)))


def sparse_attn_direct(t: SparseRows, q, sinks, indices, scale, workspace, out, stream=None):
    qa, qn = _dev(q, 2)
    sa, sn = _dev(sinks, 4)
    ia, inn = _dev(indices, 4)
    wa = _addr(workspace)
    wb = workspace.numel() * workspace.element_size()
    oa, on = _dev(out, 4)
    _check(load().ds_rows_sparse_attn_direct(ctypes.byref(t), qa, qn, sa, sn, ia, inn, float(scale),
                                             wa, wb, oa, on, _stream(stream)))


def indexer_mq_scores_elems(t: IndexerRows, query_len: int) -> int:
    return load().ds_rows_indexer_mq_scores_elems(ctypes.byref(t), int(query_len))


def indexer_score_mq(t: IndexerRows, query_len, q, weights, scores, stream=None):
    qa, qn = _dev(q, 2)
    wa, wn = _dev(weights, 4)
    sa, sn = _dev(scores, 4)
    _check(load().ds_rows_indexer_score_mq(ctypes.byref(t), int(query_len), qa, qn, wa, wn, sa, sn,
                                           _stream(stream)))


def compressor_state_elems(ratio: int, head_dim: int) -> int:
    return load().ds_rows_compressor_state_elems(ratio, head_dim)


def compressor(t: CompressorRows, ratio, head_dim, eps, kv, score, ape, norm, out, stream=None):
    ka, kn = _dev(kv, 4)
    sa, sn = _dev(score, 4)
    aa, an = _dev(ape, 4)
    na, nn = _dev(norm, 4)
    oa, on = _dev(out, 2)
    _check(load().ds_rows_compressor(ctypes.byref(t), int(ratio), int(head_dim), float(eps), ka, kn, sa, sn,
                                     aa, an, na, nn, oa, on, _stream(stream)))


TIMER_STAMPS_PER_WG = 8


def time_next_indexer(stamps):
    """Arm the calling thread's next indexer launch to write its workgroups'
    wall-clock stamps into `stamps` (a zero-filled int64 device tensor of at
    least 8 entries per workgroup: [start, end of wave 0..3, unused x 3])."""
    addr, n = _dev(stamps, 8)
    _check(load().ds_rows_time_next_indexer(addr, n))


def wall_clock_khz() -> int:
    """Frequency of the device wall clock the timing stamps count, in kHz."""
    v = ctypes.c_int(0)
    _check(load().ds_rows_wall_clock_khz(ctypes.byref(v)))
    return v.value


def indexer_span_ticks(stamps) -> int:
    """Smallest start to largest end (wall-clock ticks) of a timed launch's
    stamps (host copy, int64 [..., 8]; workgroups that wrote none are 0)."""
    import numpy as np
    a = np.asarray(stamps).reshape(-1, TIMER_STAMPS_PER_WG)
    starts = a[:, 0][a[:, 0] > 0]
    ends = a[:, 1:5][a[:, 1:5] > 0]
    return int(ends.max() - starts.min())


def version() -> str:
    return load().ds_rows_version().decode()
