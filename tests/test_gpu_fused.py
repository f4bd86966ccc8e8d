"""GPU parity of the fused score + top-512 call (ds_rows_indexer_topk).

The fused call keeps, per 256-key wave of the indexer, only the wave's best
keys (with ties at its threshold, the lowest indices) plus a floor, selects
from those candidates, and selects again from the scores when a floor shows
that the candidates may miss a key of the top 512. Its scores and indices must
equal the oracle exactly and the separate calls (ds_rows_indexer_score +
ds_rows_topk) bit for bit: on the workloads, on heavy ties and scores sorted
by position (the tie-aware candidates hold the top 512), and on inputs whose
best keys all belong to one wave, which must take the in-call reselection. The first top-k stage on the pages keeps each block's best
512 (docs.rs "mlx-native 0.18.0 src/shaders/deepseek_rows.metal",
deepseek_indexer_topk_block_rows_i32); the selected set and its order are
unique, so any correct staging gives these results.
"""
import numpy as np
import pytest
import torch

from oracle import ds_oracle as O
from sparse_attention_decode_04_amd import ds_rows as ds
from sparse_attention_decode_04_amd import inputs as I
from sparse_attention_decode_04_amd.runner import DeviceInputs, DeviceRows

pytestmark = pytest.mark.gpu

MAX_ABS = 1e-2
MEAN_ABS = 1e-3


def say(*a):
    print(*a, flush=True)


@pytest.fixture(scope="module", autouse=True)
def gpu():
    assert torch.cuda.is_available(), "no HIP device"
    ds.load()
    yield


def one_wave_holds_the_top(seed, kv_len):
    """Inputs whose 256 best scores belong to the keys that one wave of the
    fused indexer scores. The kernel deals 16-key tiles round robin over a
    row's 4 x ceil(n / 1024) waves, so its first wave takes tiles 0, S, 2S, ...
    (S = 4 ceil(n / 1024)); that wave writes at most 32 of its keys, all of
    them in the row's top 512, so its floor lies above the 512th key and the
    row must be selected again from its scores. Scores are 256 * a + b for
    key entries a (feature 0) and b (feature 1), exact integers."""
    inp = I.small_rows(seed, kv_len)
    inp.idx_q[:] = 0
    inp.idx_w[:] = 0
    inp.idx_q[:, 0, 0] = I.int_to_bf16_bits(np.array(256))
    inp.idx_q[:, 0, 1] = I.int_to_bf16_bits(np.array(1))
    inp.idx_w[:, 0] = 1.0
    for k in inp.idx_keys:
        n = k.shape[0]
        j = np.arange(n)
        wave0 = (j // 16) % (4 * -(-n // 1024)) == 0
        assert wave0.sum() == 256
        a = (j // 256) % 150
        b = j % 256
        a[wave0] = 200
        b[wave0] = np.arange(256)
        k[:] = 0
        k[:, 0] = I.int_to_bf16_bits(a)
        k[:, 1] = I.int_to_bf16_bits(b)
    return inp


def fused_and_separate(dev, rows=None):
    fused = DeviceRows(dev, rows=rows)
    fused.indexer_topk()
    sep = DeviceRows(dev, rows=rows)
    sep.indexer_score()
    sep.topk()
    return fused.results(), sep.results()


def check_scores_indices(got, sep, inp, label):
    for r in range(len(got)):
        exp = O.indexer_scores(inp.idx_q[r], inp.idx_w[r], inp.idx_keys[r], inp.start_pos[r])
        np.testing.assert_array_equal(got[r]["scores"], exp, err_msg=f"{label} row {r} scores")
        idx = O.topk_select(exp, O.valid_count(inp.kv_len[r], inp.start_pos[r]), inp.offset[r])
        np.testing.assert_array_equal(got[r]["indices"], idx, err_msg=f"{label} row {r} indices")
        assert np.array_equal(got[r]["scores"].view(np.uint32), sep[r]["scores"].view(np.uint32)), (label, r)
        assert np.array_equal(got[r]["indices"], sep[r]["indices"]), (label, r)


@pytest.mark.parametrize("cid", [0, 1, 2, 3, 4])
def test_fused_config_parity(cid):
    say(f"generating config {cid}: {I.CONFIG_NAMES[cid]}")
    inp = I.make_config(cid)
    dev = DeviceInputs(inp)
    say(f"config {cid}: fused score + top-k against the oracle and the separate calls")
    got, sep = fused_and_separate(dev)
    check_scores_indices(got, sep, inp, f"config {cid}")
    # the whole fused step: same attention output bits as the separate calls
    say(f"config {cid}: fused step vs three-call step")
    a = DeviceRows(dev)
    a.step_fused()
    b = DeviceRows(dev)
    b.step_direct()
    ra, rb = a.results(), b.results()
    for r in range(inp.rows):
        assert np.array_equal(ra[r]["out"].view(np.uint32), rb[r]["out"].view(np.uint32)), (cid, r)
    if cid in (0, 1, 2):
        orc = O.decode_rows(inp) if cid != 2 else None
        if orc is not None:
            for r in range(inp.rows):
                err = np.abs(ra[r]["out"].astype(np.float64) - orc[r]["out"].astype(np.float64))
                assert err.max() <= MAX_ABS and err.mean() <= MEAN_ABS, (cid, r)


def test_fused_multi_row_equals_single_row():
    inp = I.make_config(3)
    dev = DeviceInputs(inp)
    say("config 3: fused multi-row vs one-row calls")
    multi = DeviceRows(dev)
    multi.indexer_topk()
    m = multi.results()
    for r in range(inp.rows):
        one = DeviceRows(dev, rows=[r])
        one.indexer_topk()
        o = one.results()[0]
        assert np.array_equal(m[r]["indices"], o["indices"]), r
        assert np.array_equal(m[r]["scores"].view(np.uint32), o["scores"].view(np.uint32)), r


def test_fused_ties_across_blocks():
    # every score 0: each wave keeps its 32 lowest-index keys and a floor at
    # its best unwritten one; the floors stay below the 512th key, so the
    # candidates give the answer (every row long enough for the fused stage;
    # the 131072-key row takes two selection levels)
    kv_len = [17000, 20000, 131072]
    inp = I.small_rows(7, kv_len)
    for k in inp.idx_keys:
        k[:] = 0
    say("fused: all-zero keys", kv_len)
    got, sep = fused_and_separate(DeviceInputs(inp))
    check_scores_indices(got, sep, inp, "ties")
    for r in range(len(kv_len)):
        np.testing.assert_array_equal(got[r]["indices"], np.arange(512))


def sorted_scores(seed, kv_len, sign):
    """Inputs whose score is sign * j for key j (ReLU of an exact dot product
    256 * (j // 256) + j % 256, times a head weight of +-1)."""
    inp = I.small_rows(seed, kv_len)
    inp.idx_q[:] = 0
    inp.idx_w[:] = 0
    inp.idx_q[:, 0, 0] = I.int_to_bf16_bits(np.array(256))
    inp.idx_q[:, 0, 1] = I.int_to_bf16_bits(np.array(1))
    inp.idx_w[:, 0] = sign
    for k in inp.idx_keys:
        j = np.arange(k.shape[0])
        k[:] = 0
        k[:, 0] = I.int_to_bf16_bits(j // 256)
        k[:, 1] = I.int_to_bf16_bits(j % 256)
    return inp


@pytest.mark.parametrize("sign", [1.0, -1.0])
def test_fused_sorted_scores(sign):
    # ascending: the top 512 are the last keys; descending: the first keys.
    kv_len = [16384, 40000, 65536]
    inp = sorted_scores(13, kv_len, sign)
    say("fused: scores sorted by position, sign", sign, kv_len)
    got, sep = fused_and_separate(DeviceInputs(inp))
    check_scores_indices(got, sep, inp, f"sorted {sign}")
    for r, n in enumerate(kv_len):
        exp = np.arange(n - 1, n - 513, -1) if sign > 0 else np.arange(512)
        np.testing.assert_array_equal(got[r]["indices"], exp)


def test_fused_one_wave_holding_the_top_is_selected_again():
    kv_len = [17000, 20000, 40000]
    inp = one_wave_holds_the_top(15, kv_len)
    say("fused: the 256 best keys of each row in one indexer wave", kv_len)
    got, sep = fused_and_separate(DeviceInputs(inp))
    check_scores_indices(got, sep, inp, "one wave")
    for r, n in enumerate(kv_len):
        j = np.arange(n)
        wave0 = j[(j // 16) % (4 * -(-n // 1024)) == 0]
        np.testing.assert_array_equal(got[r]["indices"][:256], wave0[::-1])


def test_fused_causal_offset_and_non_finite():
    kv_len = [5000, 300, 20000, 9000, 64]
    start_pos = [4 * 1000 + 2, 2, 4 * 20000 - 1, 4 * 8192 + 1, 4 * 64 - 1]
    offset = [0, 0, 12345, 3, 0]
    inp = I.small_rows(31, kv_len, start_pos=start_pos, offset=offset)
    keys = inp.idx_keys[4]
    keys[3, 5] = 0x7FC0
    keys[4, 9] = 0x7F80
    keys[6, :] = 0x7F80
    say("fused: causal limits, offsets, non-finite keys")
    got, sep = fused_and_separate(DeviceInputs(inp))
    check_scores_indices(got, sep, inp, "causal")
    assert np.all(got[1]["indices"] == -1)


def test_fused_long_rows_causal_offset_and_non_finite():
    # every row has at least 16384 visible keys, so the call keeps the fused
    # stage: causal limits inside the cache, offsets, non-finite keys
    kv_len = [40000, 20000, 70000]
    start_pos = [4 * 17000 + 2, 4 * 20000 - 1, 4 * 66000 + 3]
    offset = [7, 0, 100000]
    inp = I.small_rows(33, kv_len, start_pos=start_pos, offset=offset)
    keys = inp.idx_keys[1]
    keys[3, 5] = 0x7FC0
    keys[4, 9] = 0x7F80
    keys[6, :] = 0x7F80
    say("fused: long rows, causal limits, offsets, non-finite keys")
    got, sep = fused_and_separate(DeviceInputs(inp))
    check_scores_indices(got, sep, inp, "long causal")


def test_short_row_takes_the_separate_kernels():
    # a row under 16384 visible keys sends the whole call through the
    # separate score and top-k kernels: same results
    kv_len = [600, 40000]
    inp = I.small_rows(34, kv_len)
    say("fused call with a short row")
    got, sep = fused_and_separate(DeviceInputs(inp))
    check_scores_indices(got, sep, inp, "short row")
