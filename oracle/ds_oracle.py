"""CPU oracle for the multi-row sparse-attention decode core.

TEST INFRASTRUCTURE ONLY. Only the test suite, the package smoke check and the
benchmark's CPU-baseline leg may import or run this module. The product path
(the HIP library and its Python binding) never calls it and shares no code
with it.

Plain, slow and obviously correct: every step is written from its definition
on the source pages, in float64 (integers where the step is integer work),
with library primitives (a matmul, a sort) used only as whole steps. Rows are
independent, so the multi-row oracle is a loop over rows.

Sources (docs.rs source views of the Rust crate mlx-native):
  [shader 0.18] "mlx-native 0.18.0 src/shaders/deepseek_rows.metal"
  [host 0.21]   "mlx-native 0.21.0 src/ops/deepseek_rows.rs"
Each function names the kernel or dispatch function on those pages whose
computation it restates.

Readings taken where the pages are silent or loose (each is listed again in the
design notes):
  * ReLU is IEEE maxNum(d, 0): a NaN dot product contributes 0, as the pages'
    float `max` does. Any score that ends non-finite is excluded (-inf).
  * Scores are the exact float64 sum rounded once to float32. For the
    integer-valued workloads every partial sum is an integer below 2^24, so
    this equals any fp32 summation order; for other inputs the fp32 result of
    a particular order is not pinned.
  * Top-k output is in rank order (best first), -1 after the last selected key.
  * Attention output is float32 [64, 512] (the pages store bf16).
  * A head is zeroed when its row is invalid, any of its query elements or its
    sink is non-finite, a live logit is non-finite, or the softmax denominator
    is not in (0, inf); remaining non-finite output elements are zeroed.
"""
from __future__ import annotations

import numpy as np

HEADS = 64
INDEXER_DIM = 128
HEAD_DIM = 512
TOP_K = 512
RATIO = 4


def bf16_bits_to_f64(bits: np.ndarray) -> np.ndarray:
    """Decode bfloat16 bit patterns (uint16) to float64 values."""
    u = np.asarray(bits, dtype=np.uint16).astype(np.uint32) << np.uint32(16)
    return u.view(np.float32).astype(np.float64)


def valid_count(kv_len: int, start_pos: int, ratio: int = RATIO) -> int:
    """Causally visible compressed keys of a query at absolute position
    `start_pos`: min(kv_len, floor((start_pos + 1) / ratio)).
    [shader 0.18] deepseek_indexer_score_mma_rows_bf16 / _topk_block_ / _finalize_."""
    return min(int(kv_len), (int(start_pos) + 1) // ratio)


def indexer_scores_f64(q_bits: np.ndarray, w: np.ndarray, key_bits: np.ndarray) -> np.ndarray:
    """Lightning-indexer score of every key before masking, in float64:
        s[j] = sum_h w[h] * maxNum(0, sum_d q[h, d] * k[j, d]).
    [shader 0.18] deepseek_indexer_score_mma_rows_bf16 (head tiles, ReLU,
    head-weight epilogue)."""
    q = bf16_bits_to_f64(q_bits)            # [H, Di]
    k = bf16_bits_to_f64(key_bits)          # [n, Di]
    w = np.asarray(w, dtype=np.float64)     # [H]
    if np.isfinite(q).all() and np.isfinite(k).all():
        dots = k @ q.T                      # [n, H]; exact for integer-valued inputs
    else:
        # No BLAS here: some BLAS kernels skip zero operands, which would hide
        # inf * 0 = NaN. einsum without optimisation multiplies every pair.
        dots = np.einsum("jd,hd->jh", k, q, optimize=False)
    relu = np.fmax(dots, 0.0)               # maxNum: NaN -> 0
    with np.errstate(invalid="ignore", over="ignore"):
        return (relu * w[None, :]).sum(axis=1)


def indexer_scores(q_bits: np.ndarray, w: np.ndarray, key_bits: np.ndarray,
                   start_pos: int, ratio: int = RATIO) -> np.ndarray:
    """float32 scores of one row: the float64 score rounded to float32, and
    -inf for keys at or beyond the causal limit or with a non-finite score.
    [shader 0.18] deepseek_indexer_score_mma_rows_bf16 (final store)."""
    s64 = indexer_scores_f64(q_bits, w, key_bits)
    n = s64.shape[0]
    with np.errstate(over="ignore", invalid="ignore"):
        s32 = s64.astype(np.float32)
    s32[~np.isfinite(s32)] = -np.inf
    s32[valid_count(n, start_pos, ratio):] = -np.inf
    return s32


def topk_select(scores: np.ndarray, valid: int, offset: int = 0, k: int = TOP_K) -> np.ndarray:
    """Deterministic causal top-k of one row as int32 [k].

    Candidates are keys j < valid with a finite score. They are ranked by
    score, higher first, and on equal score (by value, so -0 equals +0) the
    lower index first; the first min(k, #candidates) are emitted as j + offset
    in rank order and the remaining slots are -1.
    [shader 0.18] index_rows_better (the order), deepseek_indexer_topk_block_/
    _merge_/_finalize_rows_i32 (block sort, merge tree, finalize)."""
    scores = np.asarray(scores, dtype=np.float32)
    cand = np.arange(min(int(valid), scores.shape[0]), dtype=np.int64)
    cand = cand[np.isfinite(scores[cand])]
    # lexsort: last key is primary -> score descending, then index ascending.
    order = np.lexsort((cand, -scores[cand].astype(np.float64)))
    chosen = cand[order[:k]]
    out = np.full(k, -1, dtype=np.int32)
    out[: chosen.shape[0]] = (chosen + int(offset)).astype(np.int32)
    return out


def gather_row(kv_bits: np.ndarray, indices: np.ndarray, kv_len: int):
    """Gather the selected rows of one row's shared KV.

    For slot t with index i = indices[t]:
      i == -1            sentinel: zero row, masked out of the softmax;
      i < -1 or i >= n   bad index: zero row, the row is invalid;
      otherwise          the bf16 bits of kv[i], with every non-finite element
                         replaced by +0 and the row marked invalid.
    Returns (gathered uint16 [w, 512], sentinel bool [w], slot_bad bool [w],
    row_invalid bool).
    [shader 0.18] deepseek_sparse_attention_gather_rows_bf16."""
    indices = np.asarray(indices, dtype=np.int64)
    w = indices.shape[0]
    gathered = np.zeros((w, kv_bits.shape[1]), dtype=np.uint16)
    sentinel = np.zeros(w, dtype=bool)
    slot_bad = np.zeros(w, dtype=bool)
    for t in range(w):
        i = int(indices[t])
        if i == -1:
            sentinel[t] = True
            continue
        if i < -1 or i >= kv_len:
            slot_bad[t] = True
            continue
        row = kv_bits[i]
        finite = (row & np.uint16(0x7F80)) != np.uint16(0x7F80)
        gathered[t] = np.where(finite, row, np.uint16(0))
        slot_bad[t] = not bool(finite.all())
    return gathered, sentinel, slot_bad, bool(slot_bad.any())


def sink_softmax(logits: np.ndarray, sink: float):
    """Softmax over the live logits plus one learned sink logit that carries
    no value: m = max(sink, max l), Z = e^(sink-m) + sum e^(l-m),
    p_t = e^(l_t-m)/Z, p_sink = e^(sink-m)/Z. Returns (p, p_sink, Z, m).
    [shader 0.18] deepseek_sparse_attention_reduce_rows_bf16 (max, then
    denominator including the sink)."""
    logits = np.asarray(logits, dtype=np.float64)
    m = max(float(sink), float(logits.max()) if logits.size else -np.inf)
    e = np.exp(logits - m)
    e_sink = np.exp(float(sink) - m)
    Z = e_sink + e.sum()
    return e / Z, e_sink / Z, Z, m


def sparse_attention_row(q_bits: np.ndarray, sinks: np.ndarray, gathered_bits: np.ndarray,
                         sentinel: np.ndarray, row_invalid: bool, scale: float) -> np.ndarray:
    """Sparse MQA attention of one row over its gathered KV (keys equal
    values) with a learned per-head sink, float64, returned as float32 [H, 512]:
        l[h, t] = scale * q[h] . G[t]   for live (non-sentinel) slots t
        out[h]  = sum_t p[h, t] * G[t]  with p from sink_softmax(l[h], sink[h]).
    Fail-closed zeroing as described in the module docstring.
    [shader 0.18] deepseek_sparse_attention_score_rows_bf16 (logit and bad
    inputs), deepseek_sparse_attention_reduce_rows_bf16 (softmax, weighted sum,
    zeroing), deepseek_sparse_attention_sanitize_rows_bf16 (row/head zeroing);
    [host 0.21] dispatch_deepseek_sparse_attention_flash_rows (keys = values,
    one sink vector for all rows)."""
    Q = bf16_bits_to_f64(q_bits)                      # [H, D]
    G = bf16_bits_to_f64(gathered_bits)               # [w, D]
    live = ~np.asarray(sentinel, dtype=bool)
    Gl = G[live]
    H, D = Q.shape
    out = np.zeros((H, D), dtype=np.float64)
    if row_invalid:
        return out.astype(np.float32)
    for h in range(H):
        sink = float(sinks[h])
        if not np.isfinite(sink) or not np.isfinite(Q[h]).all():
            continue
        logits = float(scale) * (Gl @ Q[h])
        if not np.isfinite(logits).all():
            continue
        p, _, Z, _ = sink_softmax(logits, sink)
        if not (Z > 0.0 and np.isfinite(Z)):
            continue
        o = p @ Gl
        o[~np.isfinite(o)] = 0.0
        out[h] = o
    return out.astype(np.float32)


def decode_row(idx_q, idx_w, idx_keys, start_pos, offset, attn_q, sinks, kv, kv_len, width, scale):
    """One row through the whole path: indexer score -> top-512 -> gather of
    the first `width` selected indices -> sparse attention with sink.
    Returns a dict with every intermediate the GPU path exposes."""
    scores = indexer_scores(idx_q, idx_w, idx_keys, start_pos)
    idx = topk_select(scores, valid_count(idx_keys.shape[0], start_pos), offset)
    gathered, sentinel, slot_bad, invalid = gather_row(kv, idx[:width], kv_len)
    out = sparse_attention_row(attn_q, sinks, gathered, sentinel, invalid, scale)
    return dict(scores=scores, indices=idx, gathered=gathered, sentinel=sentinel,
                slot_bad=slot_bad, invalid=invalid, out=out)


def decode_rows(inp) -> list[dict]:
    """Every row of a workload (an object with the fields of the seeded input
    generator's RowsInputs), row by row."""
    res = []
    for r in range(len(inp.kv_len)):
        res.append(decode_row(inp.idx_q[r], inp.idx_w[r], inp.idx_keys[r], inp.start_pos[r],
                              inp.offset[r], inp.attn_q[r], inp.sinks, inp.kv[r],
                              inp.kv_len[r], min(inp.kv_len[r], TOP_K), inp.scale))
    return res


# ---------------------------------------------------------------------------
# Learned KV compressor, one decode token per row
# ---------------------------------------------------------------------------
#
# [shader 0.18] deepseek_compressor_rows_bf16 and [host 0.21]
# dispatch_deepseek_compressor_rows. Each row owns a recurrent state of two
# f32 tensors (values and scores) of coff * ratio rows by coff * head_dim
# features, coff = 2 for ratio 4 (windows overlap by one block) and 1
# otherwise. The decode token is written into the state; when it completes a
# block of `ratio` positions the row emits one compressed vector: per feature,
# a softmax over the window's scores weights the window's values, the result
# is rounded to bf16, RMS-normalised with a learned scale and stored as bf16.
#
# Readings (also in the design notes):
#   * The state is f32 on the pages, so the state update is done in f32: the
#     value is copied (non-finite -> 0) and the score is the f32 sum of the
#     input score and the position embedding (NaN when either the sum or the
#     value is not finite).
#   * Pooling and normalisation are computed in float64. The pooled value is
#     rounded to bf16 (round to nearest even) straight from float64; the
#     normalised value likewise.
#   * The sum of squares is invalid when it exceeds the f32 range (the pages
#     keep it in f32); outputs beyond the bf16 range are not special-cased.
#   * A row that emits nothing writes zeros.

COMPRESSOR_SHAPES = ((4, 128), (4, 512), (128, 512))
FLT_MAX = float(np.finfo(np.float32).max)


def bf16_round_bits(x: np.ndarray) -> np.ndarray:
    """bfloat16 bit patterns of float64 values, rounded to nearest with ties
    to even directly from the float64 value (one rounding). bf16 keeps f32's
    exponent range and 8 significant bits; values beyond its largest finite
    value after rounding become +-inf; NaN becomes the canonical quiet NaN."""
    x = np.asarray(x, dtype=np.float64)
    out = np.zeros(x.shape, dtype=np.uint16)
    flat = x.reshape(-1)
    res = out.reshape(-1)
    bf16_max = (2.0 - 2.0 ** -7) * 2.0 ** 127
    for i, v in enumerate(flat):
        if np.isnan(v):
            res[i] = 0x7FC0
            continue
        if np.isinf(v):
            res[i] = 0xFF80 if v < 0 else 0x7F80
            continue
        if v == 0.0:
            res[i] = 0x8000 if np.signbit(v) else 0
            continue
        _, e = np.frexp(v)                      # |v| = m * 2^e, 0.5 <= m < 1
        ulp = 2.0 ** max(int(e) - 8, -133)      # 8 significant bits; subnormal spacing 2^-133
        r = float(np.round(v / ulp)) * ulp      # np.round rounds half to even
        if abs(r) > bf16_max:
            res[i] = 0xFF80 if r < 0 else 0x7F80
            continue
        res[i] = np.uint16(np.array(r, dtype=np.float32).view(np.uint32) >> np.uint32(16))
    return out


def compressor_dims(ratio: int, head_dim: int):
    """(coff, projected features, state rows) of a supported (ratio, head_dim);
    [host 0.21] dispatch_deepseek_compressor_rows accepts (4,128), (4,512) and
    (128,512)."""
    if (int(ratio), int(head_dim)) not in COMPRESSOR_SHAPES:
        raise ValueError(f"unsupported compressor shape ({ratio},{head_dim})")
    coff = 2 if ratio == 4 else 1
    return coff, coff * head_dim, coff * ratio


def compressor_row(kv, score, ape, norm, kv_state, score_state, start_pos: int,
                   ratio: int, head_dim: int, eps: float):
    """One decode token at absolute position `start_pos` (> 0) of one row.

    kv, score: f32 [coff*head_dim]; ape: f32 [ratio, coff*head_dim];
    norm: f32 [head_dim]; kv_state, score_state: f32 [coff*ratio,
    coff*head_dim] (not modified). Returns (new kv_state, new score_state,
    output bf16 bits [head_dim]).
    [shader 0.18] deepseek_compressor_rows_bf16 (token write, window pooling,
    RMS normalisation, fail-closed zeroing, overlap shift)."""
    coff, proj, _ = compressor_dims(ratio, head_dim)
    overlap = ratio == 4
    kv = np.asarray(kv, dtype=np.float32)
    score = np.asarray(score, dtype=np.float32)
    ape = np.asarray(ape, dtype=np.float32)
    norm64 = np.asarray(norm, dtype=np.float32).astype(np.float64)
    kvs = np.array(kv_state, dtype=np.float32, copy=True)
    scs = np.array(score_state, dtype=np.float32, copy=True)

    # Write the token into its slot of the current block.
    token = int(start_pos) % ratio
    slot = (ratio if overlap else 0) + token
    with np.errstate(over="ignore", invalid="ignore"):
        s = score + ape[token]                  # f32 addition
    kvs[slot] = np.where(np.isfinite(kv), kv, np.float32(0.0))
    scs[slot] = np.where(np.isfinite(s) & np.isfinite(kv), s, np.float32(np.nan))

    out = np.zeros(head_dim, dtype=np.uint16)
    if (int(start_pos) + 1) % ratio != 0:
        return kvs, scs, out

    # The window of feature f: the previous block's rows at feature f and the
    # current block's rows at feature head_dim + f (overlap), or the current
    # block's rows at feature f.
    window = 2 * ratio if overlap else ratio
    f = np.arange(head_dim)
    S = np.empty((window, head_dim), dtype=np.float64)
    V = np.empty((window, head_dim), dtype=np.float64)
    for item in range(window):
        feat = f + head_dim if (overlap and item >= ratio) else f
        S[item] = scs[item, feat]
        V[item] = kvs[item, feat]
    bad = (np.isnan(S) | (S == np.inf) | ~np.isfinite(V)).any(axis=0)
    with np.errstate(over="ignore", invalid="ignore", divide="ignore"):
        m = S.max(axis=0)
        wts = np.exp(S - m[None, :])
        pooled = (wts * V).sum(axis=0) / wts.sum(axis=0)
    finite = np.isfinite(pooled)
    c = bf16_bits_to_f64(bf16_round_bits(np.where(finite, pooled, 0.0)))
    bad |= ~finite | ~np.isfinite(norm64)
    total = float((c * c).sum())
    invalid = bool(bad.any()) or not (total <= FLT_MAX)
    if not invalid:
        rms = 1.0 / np.sqrt(total / head_dim + float(eps))
        invalid = not np.isfinite(rms)
    if not invalid:
        normalized = c * rms * norm64
        invalid = not np.isfinite(normalized).all()
    if not invalid:
        out = bf16_round_bits(normalized)

    if overlap:
        # The current block becomes the previous one.
        kvs[:ratio] = kvs[ratio:2 * ratio]
        scs[:ratio] = scs[ratio:2 * ratio]
    return kvs, scs, out


def compressor_rows(inp):
    """Every row of a compressor workload (an object with the fields of the
    seeded generator's CompressorInputs), row by row. Returns (kv_states,
    score_states, outputs) as lists."""
    kvs, scs, outs = [], [], []
    for r in range(len(inp.start_pos)):
        a, b, o = compressor_row(inp.kv[r], inp.score[r], inp.ape, inp.norm, inp.kv_state[r],
                                 inp.score_state[r], inp.start_pos[r], inp.ratio, inp.head_dim, inp.eps)
        kvs.append(a)
        scs.append(b)
        outs.append(o)
    return kvs, scs, outs


# ---------------------------------------------------------------------------
# Multi-query indexer
# ---------------------------------------------------------------------------

def indexer_scores_mq(q_bits: np.ndarray, w: np.ndarray, key_bits: np.ndarray,
                      start_pos: int, ratio: int = RATIO) -> np.ndarray:
    """float32 scores [Q, n] of Q consecutive queries of one row against the
    row's keys: query t is at absolute position start_pos + t, so its causal
    limit is min(n, (start_pos + t + 1) // ratio); otherwise as
    indexer_scores. [shader 0.18] deepseek_indexer_score_mma_rows_bf16 (its
    query loop over a group's rows, each with its own causal count)."""
    Q = q_bits.shape[0]
    return np.stack([indexer_scores(q_bits[t], w[t], key_bits, int(start_pos) + t, ratio) for t in range(Q)])
