"""Seeded synthetic inputs for the multi-row sparse-attention decode core.

This module is shared by the CPU oracle's tests, the GPU parity tests and the
benchmark. It only draws random numbers and encodes them as bf16 bit patterns;
it holds none of the decode method's arithmetic (no score, selection, gather or
attention step lives here).

Workloads (one "row" is one independent decode request):

  config 0: 1 row, kv_len 1024
  config 1: 8 rows, ragged kv_len drawn uniformly from [600, 8192]
  config 2: 8 rows, kv_len 32768 each (the throughput shape)
  config 3: 8 rows, kv_len {1, 37, 511, 512, 513, 4096, 65536, 131072},
            indexer q/keys drawn from {-1, 0, 1} (heavy score ties)
  config 4: 1 row, kv_len 1048576 (long context)

Per row the indexer query is [64 heads, 128] bf16 and the indexer keys are
[kv_len, 128] bf16, both integer-valued (uniform in [-4, 4], or {-1, 0, 1} for
config 3); the head weights are integers uniform in [-2, 2] stored as f32.
The attention query is [64 heads, 512] bf16 ~ N(0, 1), the shared key/value
cache is [kv_len, 512] bf16 ~ N(0, 1) (keys equal values), and the learned
per-head sink logits are one f32 [64] vector ~ N(0, 1) shared by all rows.

Generation order is fixed so any consumer can regenerate the same bytes:
  rng = numpy Generator(PCG64(20260000 + config_id))
  [config 1 only: kv_len per row] -> indexer q [R,64,128] -> weights [R,64]
  -> for each row: indexer keys [n_r,128] -> attention q [R,64,512]
  -> sinks [64] -> for each row: kv [n_r,512]
Large per-row arrays are drawn in chunks of 65536 rows.
"""
from __future__ import annotations

from dataclasses import dataclass, field

import numpy as np

HEADS = 64
INDEXER_DIM = 128
HEAD_DIM = 512
TOP_K = 512
RATIO = 4
CHUNK_ROWS = 65536
SEED_BASE = 20260000

CONFIG_NAMES = {
    0: "1 row x 1024 keys",
    1: "8 rows x ragged U[600,8192] keys",
    2: "8 rows x 32768 keys",
    3: "8 rows x {1,37,511,512,513,4096,65536,131072} keys, ternary indexer entries",
    4: "1 row x 1048576 keys",
}


def f32_to_bf16_bits(x: np.ndarray) -> np.ndarray:
    """Round float32 values to bfloat16 (round to nearest, ties to even) and
    return the 16-bit patterns as uint16. Inputs here are finite."""
    u = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32)
    rounded = u + np.uint32(0x7FFF) + ((u >> np.uint32(16)) & np.uint32(1))
    return (rounded >> np.uint32(16)).astype(np.uint16)


def int_to_bf16_bits(x: np.ndarray) -> np.ndarray:
    """Encode small integers (|x| <= 256, exactly representable) as bf16 bits."""
    return f32_to_bf16_bits(np.asarray(x, dtype=np.float32))


@dataclass
class RowsInputs:
    """Host copies of one workload. Arrays of bf16 values are uint16 bit
    patterns; everything is C-contiguous."""

    config_id: int
    kv_len: list[int]
    start_pos: list[int]
    offset: list[int]
    idx_q: np.ndarray            # uint16 [R, 64, 128]
    idx_w: np.ndarray            # float32 [R, 64]
    idx_keys: list[np.ndarray]   # uint16 [n_r, 128] per row
    attn_q: np.ndarray           # uint16 [R, 64, 512]
    sinks: np.ndarray            # float32 [64]
    kv: list[np.ndarray]         # uint16 [n_r, 512] per row
    scale: float = float(np.float32(1.0 / np.sqrt(HEAD_DIM)))  # the f32 value both sides use
    extra: dict = field(default_factory=dict)

    @property
    def rows(self) -> int:
        return len(self.kv_len)

    @property
    def width(self) -> list[int]:
        return [min(n, TOP_K) for n in self.kv_len]


def config_kv_lens(config_id: int, rng: np.random.Generator | None = None) -> list[int]:
    if config_id == 0:
        return [1024]
    if config_id == 1:
        assert rng is not None
        return [int(v) for v in rng.integers(600, 8192, size=8, endpoint=True)]
    if config_id == 2:
        return [32768] * 8
    if config_id == 3:
        return [1, 37, 511, 512, 513, 4096, 65536, 131072]
    if config_id == 4:
        return [1048576]
    raise ValueError(f"unknown config {config_id}")


def _int_rows(rng, n, cols, lo, hi):
    out = np.empty((n, cols), dtype=np.uint16)
    for s in range(0, n, CHUNK_ROWS):
        e = min(n, s + CHUNK_ROWS)
        out[s:e] = int_to_bf16_bits(rng.integers(lo, hi, size=(e - s, cols), endpoint=True))
    return out


def _normal_rows(rng, n, cols):
    out = np.empty((n, cols), dtype=np.uint16)
    for s in range(0, n, CHUNK_ROWS):
        e = min(n, s + CHUNK_ROWS)
        out[s:e] = f32_to_bf16_bits(rng.standard_normal((e - s, cols), dtype=np.float32))
    return out


def make_config(config_id: int, seed: int | None = None) -> RowsInputs:
    """Generate workload `config_id` with the fixed generation order."""
    rng = np.random.Generator(np.random.PCG64(SEED_BASE + config_id if seed is None else seed))
    kv_len = config_kv_lens(config_id, rng)
    return make_rows(rng, kv_len, ternary=(config_id == 3), config_id=config_id)


def make_rows(rng: np.random.Generator, kv_len: list[int], ternary: bool = False,
              config_id: int = -1, start_pos: list[int] | None = None,
              offset: list[int] | None = None) -> RowsInputs:
    """Generate rows with the given key counts, in the fixed order.

    start_pos defaults to 4 * kv_len - 1 (every cached compressed key is
    causally visible) and offset to 0."""
    R = len(kv_len)
    lo, hi = (-1, 1) if ternary else (-4, 4)
    idx_q = _int_rows(rng, R * HEADS, INDEXER_DIM, lo, hi).reshape(R, HEADS, INDEXER_DIM)
    idx_w = rng.integers(-2, 2, size=(R, HEADS), endpoint=True).astype(np.float32)
    idx_keys = [_int_rows(rng, n, INDEXER_DIM, lo, hi) for n in kv_len]
    attn_q = _normal_rows(rng, R * HEADS, HEAD_DIM).reshape(R, HEADS, HEAD_DIM)
    sinks = rng.standard_normal(HEADS, dtype=np.float32)
    kv = [_normal_rows(rng, n, HEAD_DIM) for n in kv_len]
    if start_pos is None:
        start_pos = [RATIO * n - 1 for n in kv_len]
    if offset is None:
        offset = [0] * R
    return RowsInputs(config_id, list(kv_len), list(start_pos), list(offset),
                      idx_q, idx_w, idx_keys, attn_q, sinks, kv)


def small_rows(seed: int, kv_len: list[int], ternary: bool = False, **kw) -> RowsInputs:
    """Convenience for tests: the same recipe at arbitrary small sizes."""
    return make_rows(np.random.Generator(np.random.PCG64(seed)), kv_len, ternary=ternary, **kw)


# ---------------------------------------------------------------------------
# Learned KV compressor, one decode token per row
# ---------------------------------------------------------------------------
# Shapes: coff = 2 for ratio 4 (overlapping windows) and 1 otherwise; the
# token's projected value and score are [coff * head_dim] f32, the position
# embedding [ratio, coff * head_dim] f32, the RMS scale [head_dim] f32 and
# each row's two recurrent states [coff * ratio, coff * head_dim] f32.
# Values, scores, embeddings and states ~ N(0, 1); the RMS scale ~ U[0.5, 1.5];
# epsilon 1e-6. The pages give no weights, so all are synthetic.
# Generation order: rng = Generator(PCG64(seed)) -> kv [R,P] -> score [R,P]
# -> ape [ratio,P] -> norm [head_dim] -> kv_state [R,S,P] -> score_state [R,S,P]
# -> [default positions].

COMPRESSOR_SEED_BASE = 20261000
COMPRESSOR_SHAPES = ((4, 128), (4, 512), (128, 512))


@dataclass
class CompressorInputs:
    ratio: int
    head_dim: int
    start_pos: list[int]
    kv: np.ndarray             # float32 [R, P]
    score: np.ndarray          # float32 [R, P]
    ape: np.ndarray            # float32 [ratio, P]
    norm: np.ndarray           # float32 [head_dim]
    kv_state: np.ndarray       # float32 [R, S, P]
    score_state: np.ndarray    # float32 [R, S, P]
    eps: float = 1e-6

    @property
    def rows(self) -> int:
        return len(self.start_pos)


def make_compressor(seed: int, rows: int, ratio: int, head_dim: int,
                    start_pos: list[int] | None = None) -> CompressorInputs:
    """Seeded compressor inputs. start_pos defaults to positions that end a
    block for every row (ratio * k - 1, k uniform in [1, 4096])."""
    if (ratio, head_dim) not in COMPRESSOR_SHAPES:
        raise ValueError(f"unsupported compressor shape ({ratio},{head_dim})")
    coff = 2 if ratio == 4 else 1
    P, S = coff * head_dim, coff * ratio
    rng = np.random.Generator(np.random.PCG64(seed))
    kv = rng.standard_normal((rows, P), dtype=np.float32)
    score = rng.standard_normal((rows, P), dtype=np.float32)
    ape = rng.standard_normal((ratio, P), dtype=np.float32)
    norm = rng.uniform(0.5, 1.5, size=head_dim).astype(np.float32)
    kv_state = rng.standard_normal((rows, S, P), dtype=np.float32)
    score_state = rng.standard_normal((rows, S, P), dtype=np.float32)
    if start_pos is None:
        start_pos = [ratio * int(k) - 1 for k in rng.integers(1, 4096, size=rows, endpoint=True)]
    return CompressorInputs(ratio, head_dim, list(start_pos), kv, score, ape, norm, kv_state, score_state)


def compressor_workload(ratio: int, head_dim: int) -> CompressorInputs:
    """The measured compressor workload of a shape: 8 rows, every row's token
    ends a block (the step that pools and normalises)."""
    return make_compressor(COMPRESSOR_SEED_BASE + ratio * 1000 + head_dim, 8, ratio, head_dim)


# ---------------------------------------------------------------------------
# Multi-query indexer (several consecutive queries per row)
# ---------------------------------------------------------------------------
# Row r's Q queries are q/weights rows r*Q .. r*Q + Q - 1 ([R*Q, 64, 128]
# bf16 and [R*Q, 64] f32), integer-valued as in the single-query workloads;
# keys [n_r, 128] per row. Query t of row r sits at position start_pos + t;
# start_pos defaults to max(0, 4 * n_r - Q), so the last query sees every key
# (rows of fewer than Q / 4 keys need Q <= 4 * n_r).
# Generation order: rng = Generator(PCG64(seed)) -> q -> weights -> keys per row.

MQ_SEED_BASE = 20262000


@dataclass
class MultiQueryInputs:
    query_len: int
    kv_len: list[int]
    start_pos: list[int]
    idx_q: np.ndarray            # uint16 [R*Q, 64, 128]
    idx_w: np.ndarray            # float32 [R*Q, 64]
    idx_keys: list[np.ndarray]   # uint16 [n_r, 128] per row

    @property
    def rows(self) -> int:
        return len(self.kv_len)


def make_mq(seed: int, kv_len: list[int], query_len: int, ternary: bool = False,
            start_pos: list[int] | None = None) -> MultiQueryInputs:
    rng = np.random.Generator(np.random.PCG64(seed))
    R, Q = len(kv_len), query_len
    lo, hi = (-1, 1) if ternary else (-4, 4)
    idx_q = _int_rows(rng, R * Q * HEADS, INDEXER_DIM, lo, hi).reshape(R * Q, HEADS, INDEXER_DIM)
    idx_w = rng.integers(-2, 2, size=(R * Q, HEADS), endpoint=True).astype(np.float32)
    idx_keys = [_int_rows(rng, n, INDEXER_DIM, lo, hi) for n in kv_len]
    if start_pos is None:
        start_pos = [max(0, RATIO * n - Q) for n in kv_len]
    return MultiQueryInputs(Q, list(kv_len), list(start_pos), idx_q, idx_w, idx_keys)


def mq_workload(query_len: int = 8) -> MultiQueryInputs:
    """The measured multi-query workload: 8 rows x 32768 keys, query_len
    queries per row."""
    return make_mq(MQ_SEED_BASE + query_len, [32768] * 8, query_len)


# ---------------------------------------------------------------------------
# Score distributions that defeat the fused indexer's per-wave candidates
# ---------------------------------------------------------------------------
# Used to time the one-call step's exact reselection path on the throughput
# shape (8 rows x 32768 keys):
#   "ties":   every indexer key is zero, so every score is 0 (the top 512 are
#             the lowest indices, all in the first waves);
#   "sorted": each query is one-hot on feature 0 with unit head weights and
#             key j holds bf16(4 j / kv_len) in feature 0 (zeros elsewhere),
#             so scores never decrease with the position and the top 512 sit
#             in the last waves (bf16 rounding leaves runs of equal scores).
# Everything else is the config-2 recipe (same seed and order).
FALLBACK_KINDS = ("ties", "sorted")


def fallback_workload(kind: str) -> RowsInputs:
    inp = make_config(2)
    if kind == "ties":
        for k in inp.idx_keys:
            k[:] = 0
    elif kind == "sorted":
        inp.idx_q[:] = 0
        inp.idx_q[:, :, 0] = int_to_bf16_bits(np.ones(1))[0]
        inp.idx_w[:] = 1.0
        for k in inp.idx_keys:
            n = k.shape[0]
            k[:] = 0
            k[:, 0] = f32_to_bf16_bits(np.arange(n, dtype=np.float32) * np.float32(4.0 / n))
    else:
        raise ValueError(kind)
    inp.extra["fallback"] = kind
    return inp
