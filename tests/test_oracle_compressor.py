"""Pins of the compressor oracle to facts outside itself (CPU only).

The learned KV compressor rows step (docs.rs "mlx-native 0.18.0
src/shaders/deepseek_rows.metal", kernel deepseek_compressor_rows_bf16;
"mlx-native 0.21.0 src/ops/deepseek_rows.rs", dispatch_deepseek_compressor_rows):
a decode token is written into its row's recurrent state and, when it ends a
block of `ratio` positions, a softmax over the window's scores pools the
window's values per feature and the pooled vector is RMS-normalised.

Each test checks the oracle against a closed form, torch's own softmax and
RMS norm, a whole-sequence definition written independently of the oracle's
state bookkeeping, or a hand-computed rounding, so that a wrong window half, a
missing position embedding, a skipped shift or a dropped fail-closed rule
fails at least one of them.
"""
import numpy as np
import pytest
import torch
import torch.nn.functional as F

from oracle import ds_oracle as O
from sparse_attention_decode_04_amd import inputs as I

SHAPES = [(4, 128), (4, 512), (128, 512)]


def ulp_diff(a_bits, b_bits):
    """Distance in bf16 units in the last place (same-sign finite values)."""
    a = np.asarray(a_bits, np.int32)
    b = np.asarray(b_bits, np.int32)
    sa = np.where(a & 0x8000, -(a & 0x7FFF), a)
    sb = np.where(b & 0x8000, -(b & 0x7FFF), b)
    return np.abs(sa - sb)


# ------------------------------------------------------------ bf16 rounding

def test_bf16_round_hand_cases():
    one = 1.0
    ulp1 = 2.0 ** -7                      # spacing of bf16 in [1, 2)
    cases = [
        (one, 0x3F80),
        (one + ulp1, 0x3F81),
        (one + ulp1 / 2, 0x3F80),           # tie -> even (0x3F80)
        (one + 3 * ulp1 / 2, 0x3F82),       # tie -> even (0x3F82)
        (one + ulp1 / 2 + 2.0 ** -30, 0x3F81),   # just above the tie (not representable in f32's 24 bits)
        (-2.0, 0xC000),
        (0.0, 0x0000),
        (-0.0, 0x8000),
        (2.0 ** -133, 0x0001),              # smallest bf16 subnormal
        (2.0 ** -134, 0x0000),              # tie between 0 and it -> even (0)
        (3 * 2.0 ** -134, 0x0002),          # tie between 1 and 2 subnormal units -> 2
        ((2 - 2.0 ** -7) * 2.0 ** 127, 0x7F7F),   # largest finite
        ((2 - 2.0 ** -8) * 2.0 ** 127, 0x7F80),   # tie above the largest -> even (inf)
        (np.inf, 0x7F80),
        (-np.inf, 0xFF80),
    ]
    got = O.bf16_round_bits(np.array([c[0] for c in cases]))
    assert [int(v) for v in got] == [c[1] for c in cases]
    assert O.bf16_round_bits(np.array([np.nan]))[0] & 0x7FFF > 0x7F80


def test_bf16_round_matches_torch_on_f32_values():
    # Values exactly representable in f32: one rounding either way.
    x = (np.random.default_rng(5).standard_normal(20000) * 1e3).astype(np.float32)
    ref = torch.from_numpy(x).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    np.testing.assert_array_equal(O.bf16_round_bits(x.astype(np.float64)), ref)


# ----------------------------------------------------------------- helpers

def expected_block(prev_s, prev_v, cur_s, cur_v, norm, eps, head_dim, overlap):
    """Output of one block from its window, with torch's softmax and RMS norm:
    overlap -> window = previous block at features [0, hd) and current block
    at [hd, 2hd); otherwise the current block at [0, hd)."""
    if overlap:
        S = torch.cat([torch.from_numpy(prev_s[:, :head_dim]), torch.from_numpy(cur_s[:, head_dim:])])
        V = torch.cat([torch.from_numpy(prev_v[:, :head_dim]), torch.from_numpy(cur_v[:, head_dim:])])
    else:
        S, V = torch.from_numpy(cur_s), torch.from_numpy(cur_v)
    S, V = S.double(), V.double()
    pooled = (torch.softmax(S, dim=0) * V).sum(dim=0).numpy()
    c = O.bf16_bits_to_f64(O.bf16_round_bits(pooled))
    normed = F.rms_norm(torch.from_numpy(c), (head_dim,), weight=torch.from_numpy(norm.astype(np.float64)),
                        eps=eps).numpy()
    return O.bf16_round_bits(normed)


def run_sequence(ratio, head_dim, blocks, seed):
    """Drive the oracle over `blocks` whole blocks of tokens starting at a
    block boundary, from a state whose previous-block rows hold a known block
    and whose current-block rows hold NaN (never read before overwritten).
    Returns the token arrays and the oracle's emissions."""
    coff, P, Srows = O.compressor_dims(ratio, head_dim)
    rng = np.random.default_rng(seed)
    overlap = ratio == 4
    T = (blocks + 1) * ratio                       # block -1 (history) + `blocks`
    kv = rng.standard_normal((T, P)).astype(np.float32)
    sc = rng.standard_normal((T, P)).astype(np.float32)
    ape = rng.standard_normal((ratio, P)).astype(np.float32)
    norm = rng.uniform(0.5, 1.5, head_dim).astype(np.float32)
    eps = 1e-6
    p0 = ratio * 7                                  # first position of block 0
    pos = p0 - ratio + np.arange(T)                 # absolute positions of the tokens
    stored = sc + ape[pos % ratio]                  # f32 sums, what the state keeps
    kvs = np.full((Srows, P), np.nan, np.float32)
    scs = np.full((Srows, P), np.nan, np.float32)
    if overlap:
        kvs[:ratio] = kv[:ratio]
        scs[:ratio] = stored[:ratio]
    outs = {}
    for t in range(ratio, T):
        kvs, scs, out = O.compressor_row(kv[t], sc[t], ape, norm, kvs, scs, int(pos[t]), ratio, head_dim, eps)
        outs[int(pos[t])] = out
    return dict(kv=kv, stored=stored, norm=norm, eps=eps, pos=pos, outs=outs, kvs=kvs, scs=scs)


# -------------------------------------------------------------- sequence pin

@pytest.mark.parametrize("ratio,head_dim", SHAPES)
def test_sequence_matches_window_definition(ratio, head_dim):
    blocks = 3 if ratio == 4 else 2
    r = run_sequence(ratio, head_dim, blocks, seed=ratio + head_dim)
    overlap = ratio == 4
    for b in range(blocks):
        cur = slice((b + 1) * ratio, (b + 2) * ratio)
        prev = slice(b * ratio, (b + 1) * ratio)
        exp = expected_block(r["stored"][prev].astype(np.float64), r["kv"][prev].astype(np.float64),
                             r["stored"][cur].astype(np.float64), r["kv"][cur].astype(np.float64),
                             r["norm"], r["eps"], head_dim, overlap)
        end = int(r["pos"][cur][-1])
        got = r["outs"][end]
        assert ulp_diff(got, exp).max() <= 1, (ratio, head_dim, b)
        assert np.mean(got == exp) >= 0.99
        # every other position of the block emits zeros
        for p in r["pos"][cur][:-1]:
            assert not r["outs"][int(p)].any()
    # the state at the end holds the last block (and, with overlap, a copy of
    # it as the previous block)
    last = slice(blocks * ratio, (blocks + 1) * ratio)
    if overlap:
        np.testing.assert_array_equal(r["kvs"][:ratio], r["kv"][last])
        np.testing.assert_array_equal(r["kvs"][ratio:], r["kv"][last])
        np.testing.assert_array_equal(r["scs"][:ratio], r["stored"][last])
    else:
        np.testing.assert_array_equal(r["kvs"], r["kv"][last])
        np.testing.assert_array_equal(r["scs"], r["stored"][last])


# ------------------------------------------------------------- closed forms

@pytest.mark.parametrize("a", [0.75, 2.0 ** -10])
@pytest.mark.parametrize("ratio,head_dim", SHAPES)
def test_equal_scores_pool_to_the_mean(ratio, head_dim, a):
    # All window scores equal -> pooled = mean of the window's values. The
    # values are a + d with d summing to zero over the window -> every pooled
    # value is a, so out = bf16(a / sqrt(a^2 + eps) * norm). At a = 2^-10,
    # a^2 is close to eps = 1e-6, so a dropped epsilon shows.
    coff, P, Srows = O.compressor_dims(ratio, head_dim)
    rng = np.random.default_rng(3)
    kvs = np.full((Srows, P), a, np.float32)
    d = (a * rng.integers(-3, 3, size=(Srows // 2 if Srows > 1 else 1, P), endpoint=True)).astype(np.float32)
    kvs[0::2][: d.shape[0]] += d
    kvs[1::2][: d.shape[0]] -= d
    scs = np.zeros((Srows, P), np.float32)
    ape = np.zeros((ratio, P), np.float32)
    norm = rng.uniform(0.5, 1.5, head_dim).astype(np.float32)
    start = 2 * ratio - 1
    slot = (ratio if ratio == 4 else 0) + start % ratio
    kv_in = kvs[slot].copy()                       # rewrite the slot with its own value
    _, _, out = O.compressor_row(kv_in, np.zeros(P, np.float32), ape, norm, kvs, scs, start, ratio, head_dim, 1e-6)
    exp = O.bf16_round_bits(a / np.sqrt(a * a + 1e-6) * norm.astype(np.float64))
    assert ulp_diff(out, exp).max() <= 1
    assert np.mean(out == exp) >= 0.99


@pytest.mark.parametrize("ratio,head_dim", SHAPES)
def test_single_live_item_passes_its_value(ratio, head_dim):
    # Every window score -inf but one item per feature -> pooled = that value.
    coff, P, Srows = O.compressor_dims(ratio, head_dim)
    rng = np.random.default_rng(4)
    kvs = rng.standard_normal((Srows, P)).astype(np.float32)
    scs = np.full((Srows, P), -np.inf, np.float32)
    window = 2 * ratio if ratio == 4 else ratio
    pick = rng.integers(0, window, size=head_dim)
    f = np.arange(head_dim)
    feat = np.where((ratio == 4) & (pick >= ratio), head_dim + f, f)
    scs[pick, feat] = rng.standard_normal(head_dim).astype(np.float32)
    start = 3 * ratio - 1
    slot = (ratio if ratio == 4 else 0) + start % ratio
    ape = np.zeros((ratio, P), np.float32)
    norm = np.ones(head_dim, np.float32)
    # The token rewrites its slot with the state's own contents, except that
    # a token score must be finite (a non-finite one is stored as NaN): its
    # dead features get -1e30, whose weight exp(-1e30 - s) is exactly 0.
    s_in = np.where(np.isfinite(scs[slot]), scs[slot], np.float32(-1e30))
    _, _, out = O.compressor_row(kvs[slot].copy(), s_in, ape, norm, kvs, scs, start, ratio, head_dim, 1e-6)
    c = O.bf16_bits_to_f64(O.bf16_round_bits(kvs[pick, feat].astype(np.float64)))
    exp = O.bf16_round_bits(c / np.sqrt(np.mean(c * c) + 1e-6))
    assert ulp_diff(out, exp).max() <= 1


# --------------------------------------------------------------- schedule

@pytest.mark.parametrize("ratio,head_dim", SHAPES)
def test_non_final_positions_write_the_slot_only(ratio, head_dim):
    inp = I.make_compressor(21, 1, ratio, head_dim, start_pos=[5 * ratio + 1])
    kvs, scs, out = O.compressor_row(inp.kv[0], inp.score[0], inp.ape, inp.norm, inp.kv_state[0],
                                     inp.score_state[0], inp.start_pos[0], ratio, head_dim, inp.eps)
    assert not out.any()
    slot = (ratio if ratio == 4 else 0) + 1
    others = np.ones(kvs.shape[0], bool)
    others[slot] = False
    np.testing.assert_array_equal(kvs[others], inp.kv_state[0][others])
    np.testing.assert_array_equal(scs[others], inp.score_state[0][others])
    np.testing.assert_array_equal(kvs[slot], inp.kv[0])
    np.testing.assert_array_equal(scs[slot], inp.score[0] + inp.ape[1])


def test_overlap_shift_after_emission():
    inp = I.make_compressor(22, 1, 4, 128, start_pos=[4 * 9 + 3])
    kvs, scs, out = O.compressor_row(inp.kv[0], inp.score[0], inp.ape, inp.norm, inp.kv_state[0],
                                     inp.score_state[0], inp.start_pos[0], 4, 128, inp.eps)
    assert out.any()
    np.testing.assert_array_equal(kvs[:4], kvs[4:])
    np.testing.assert_array_equal(scs[:4], scs[4:])
    np.testing.assert_array_equal(kvs[:3], inp.kv_state[0][4:7])
    np.testing.assert_array_equal(kvs[3], inp.kv[0])


# ------------------------------------------------------------ fail-closed

def emit_case(mutate, ratio=4, head_dim=128):
    inp = I.make_compressor(23, 1, ratio, head_dim, start_pos=[ratio * 11 - 1])
    kv, sc = inp.kv[0].copy(), inp.score[0].copy()
    kvs, scs, norm = inp.kv_state[0].copy(), inp.score_state[0].copy(), inp.norm.copy()
    mutate(kv, sc, kvs, scs, norm)
    return O.compressor_row(kv, sc, inp.ape, norm, kvs, scs, inp.start_pos[0], ratio, head_dim, inp.eps)


def test_fail_closed_rules():
    hd = 128
    # NaN window score (previous block, first half) -> zeros
    assert not emit_case(lambda kv, sc, kvs, scs, n: scs.__setitem__((0, 5), np.nan))[2].any()
    # +inf window score -> zeros
    assert not emit_case(lambda kv, sc, kvs, scs, n: scs.__setitem__((1, 7), np.inf))[2].any()
    # non-finite window value -> zeros
    assert not emit_case(lambda kv, sc, kvs, scs, n: kvs.__setitem__((5, hd + 3), np.inf))[2].any()
    # non-finite token value -> slot value 0, slot score NaN; in the window
    # (second half of the current block) -> zeros
    kvs, scs, out = emit_case(lambda kv, sc, kvs, scs, n: kv.__setitem__(hd + 9, np.nan))
    assert not out.any() and kvs[7, hd + 9] == 0 and np.isnan(scs[7, hd + 9])
    # ... in the first half it is outside this window (this block's output
    # stands) but, shifted into the previous-block rows, inside the next one
    kvs, scs, out = emit_case(lambda kv, sc, kvs, scs, n: kv.__setitem__(9, np.nan))
    assert out.any() and kvs[3, 9] == 0 and np.isnan(scs[3, 9])
    # non-finite RMS scale -> zeros
    assert not emit_case(lambda kv, sc, kvs, scs, n: n.__setitem__(0, np.inf))[2].any()
    # -inf window score: excluded from the softmax, not an error
    assert emit_case(lambda kv, sc, kvs, scs, n: scs.__setitem__((2, 4), -np.inf))[2].any()
    # NaN outside the window (previous block, second half) is never read
    ref = emit_case(lambda *a: None)[2]
    got = emit_case(lambda kv, sc, kvs, scs, n: scs.__setitem__((0, hd + 1), np.nan))[2]
    np.testing.assert_array_equal(got, ref)
    # a -inf token score is stored as NaN (only state rows can hold -inf) -> zeros
    kvs, scs, out = emit_case(lambda kv, sc, kvs, scs, n: sc.__setitem__(hd + 2, -np.inf))
    assert not out.any() and np.isnan(scs[7, hd + 2])


def test_rows_are_independent():
    inp = I.make_compressor(24, 3, 4, 512, start_pos=[7, 8, 11])
    kvs, scs, outs = O.compressor_rows(inp)
    for r in range(3):
        a, b, o = O.compressor_row(inp.kv[r], inp.score[r], inp.ape, inp.norm, inp.kv_state[r],
                                   inp.score_state[r], inp.start_pos[r], 4, 512, inp.eps)
        np.testing.assert_array_equal(o, outs[r])
    assert outs[0].any() and not outs[1].any() and outs[2].any()
