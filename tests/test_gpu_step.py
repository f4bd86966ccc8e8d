"""GPU parity of the one-call decode core (ds_rows_indexer_topk_attn).

The call must give the scores, indices and attention output of
ds_rows_indexer_topk followed by ds_rows_sparse_attn_direct bit for bit,
whether the final top-k level runs inside the attention's workgroups (from the
fused indexer's candidates when every row has at least 16384 visible keys and
at most 65536 keys, from the scores when every row has at most 16384 visible
keys, or over lists when every row reaches its final level in the same later
pass) or the two calls run as they are; on the small workloads the output is
also checked against the oracle. Sources: docs.rs "mlx-native 0.18.0
src/shaders/deepseek_rows.metal" (deepseek_indexer_topk_finalize_rows_i32,
deepseek_sparse_attention_score_rows_bf16) and "mlx-native 0.21.0
src/ops/deepseek_rows.rs" (the rows dispatches run back to back). The selected
set, its order and the attention's arithmetic are the same code either way, so
equality is exact.
"""
import numpy as np
import pytest
import torch

from oracle import ds_oracle as O
from sparse_attention_decode_04_amd import inputs as I
from sparse_attention_decode_04_amd import ds_rows as ds
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


def one_and_two(dev, rows=None, width=None):
    one = DeviceRows(dev, rows=rows, width=width)
    one.step_one()
    two = DeviceRows(dev, rows=rows, width=width)
    two.step_fused()
    return one.results(), two.results()


def check_equal(a, b, label):
    for r in range(len(a)):
        assert np.array_equal(a[r]["scores"].view(np.uint32), b[r]["scores"].view(np.uint32)), (label, r, "scores")
        assert np.array_equal(a[r]["indices"], b[r]["indices"]), (label, r, "indices")
        assert np.array_equal(a[r]["out"].view(np.uint32), b[r]["out"].view(np.uint32)), (label, r, "out")


@pytest.mark.parametrize("cid", [0, 1, 2, 3, 4])
def test_step_config_parity(cid):
    say(f"generating config {cid}: {I.CONFIG_NAMES[cid]}")
    inp = I.make_config(cid)
    dev = DeviceInputs(inp)
    say(f"config {cid}: one call vs indexer_topk + sparse_attn_direct")
    a, b = one_and_two(dev)
    check_equal(a, b, f"config {cid}")
    if cid in (0, 1):
        orc = O.decode_rows(inp)
        for r in range(inp.rows):
            np.testing.assert_array_equal(a[r]["indices"], orc[r]["indices"], err_msg=f"config {cid} row {r}")
            err = np.abs(a[r]["out"].astype(np.float64) - orc[r]["out"].astype(np.float64))
            assert err.max() <= MAX_ABS and err.mean() <= MEAN_ABS, (cid, r, err.max(), err.mean())


def test_step_ties_inside_the_kernel():
    # all-zero indexer keys: every wave keeps its lowest-index ties, and its
    # floor (its best unwritten tie) stays below the 512th candidate
    kv_len = [17000, 20000, 40000]
    inp = I.small_rows(41, kv_len)
    for k in inp.idx_keys:
        k[:] = 0
    say("one call: all-zero keys", kv_len)
    a, b = one_and_two(DeviceInputs(inp))
    check_equal(a, b, "ties")
    for r in range(len(kv_len)):
        np.testing.assert_array_equal(a[r]["indices"], np.arange(512))


def test_step_one_wave_holding_the_top_is_selected_again_inside_the_kernel():
    # the 256 best keys of each row belong to one indexer wave: its floor lies
    # above the 512th candidate and each workgroup selects its row again from
    # the scores (the one-call path's reselection)
    from test_gpu_fused import one_wave_holds_the_top
    kv_len = [17000, 20000, 40000]
    inp = one_wave_holds_the_top(47, kv_len)
    say("one call: the 256 best keys of each row in one indexer wave", kv_len)
    a, b = one_and_two(DeviceInputs(inp))
    check_equal(a, b, "one wave")
    for r in range(len(kv_len)):
        exp = O.topk_select(O.indexer_scores(inp.idx_q[r], inp.idx_w[r], inp.idx_keys[r], inp.start_pos[r]),
                            kv_len[r])
        np.testing.assert_array_equal(a[r]["indices"], exp)


@pytest.mark.parametrize("sign", [1.0, -1.0])
def test_step_sorted_scores_inside_the_kernel(sign):
    kv_len = [16384, 40000, 65536]
    inp = I.small_rows(43, kv_len)
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
    say("one call: scores sorted by position, sign", sign)
    a, b = one_and_two(DeviceInputs(inp))
    check_equal(a, b, f"sorted {sign}")
    for r, n in enumerate(kv_len):
        exp = np.arange(n - 1, n - 513, -1) if sign > 0 else np.arange(512)
        np.testing.assert_array_equal(a[r]["indices"], exp)


def test_step_widths_below_512_write_every_index():
    # the attention reads the first `width` selected slots; all 512 indices
    # are still written
    kv_len = [20000, 30000, 17000]
    inp = I.small_rows(45, kv_len)
    dev = DeviceInputs(inp)
    width = [300, 512, 1]
    say("one call: widths", width)
    a, b = one_and_two(dev, width=width)
    check_equal(a, b, "widths")
    for r in range(len(kv_len)):
        assert np.all(a[r]["indices"] != -7), r


def test_step_rows_past_65536_keys_take_the_two_calls():
    kv_len = [70000, 20000]
    inp = I.small_rows(47, kv_len)
    say("one call with a 70000-key row")
    a, b = one_and_two(DeviceInputs(inp))
    check_equal(a, b, "long row")


def test_step_rows_past_65536_keys_final_level_inside_the_kernel():
    # both rows need a second selection pass, which is then every row's final
    # level: it runs inside the attention's workgroups
    kv_len = [70000, 90000]
    inp = I.small_rows(51, kv_len)
    say("one call with two rows past 65536 keys")
    a, b = one_and_two(DeviceInputs(inp))
    check_equal(a, b, "long rows, same final pass")
    orc = O.decode_rows(inp)
    for r in range(len(kv_len)):
        np.testing.assert_array_equal(a[r]["indices"], orc[r]["indices"], err_msg=f"long row {r}")
        err = np.abs(a[r]["out"].astype(np.float64) - orc[r]["out"].astype(np.float64))
        assert err.max() <= MAX_ABS and err.mean() <= MEAN_ABS, (r, err.max(), err.mean())


def test_step_short_row_takes_the_two_calls():
    kv_len = [600, 40000]
    inp = I.small_rows(48, kv_len)
    say("one call with a short row")
    a, b = one_and_two(DeviceInputs(inp))
    check_equal(a, b, "short row")


def test_step_short_rows_select_from_scores_inside_the_kernel():
    # every row's visible scores fit one selection chunk (at most 16384): the
    # one level from the scores runs inside the attention's workgroups. Causal
    # limits inside the cache (one row with nothing visible), offsets (a row
    # whose indices pass its cache, which the attention zeroes), widths below
    # 512 and non-finite indexer keys.
    kv_len = [5000, 300, 20000, 9000, 64]
    start_pos = [4 * 1000 + 2, 2, 4 * 16384 - 1, 4 * 8192 + 1, 4 * 64 - 1]
    offset = [0, 0, 12345, 3, 0]
    inp = I.small_rows(49, kv_len, start_pos=start_pos, offset=offset)
    keys = inp.idx_keys[3]
    keys[3, 5] = 0x7FC0
    keys[6, :] = 0x7F80
    dev = DeviceInputs(inp)
    width = [512, 300, 200, 1, 64]
    say("one call, short rows: causal limits, offsets, widths, non-finite keys")
    a, b = one_and_two(dev, width=width)
    check_equal(a, b, "short rows")
    for r in range(len(kv_len)):
        assert np.all(a[r]["indices"] != -7), r
    assert np.all(a[1]["indices"] == -1)
    orc = O.decode_rows(inp)
    for r in (0, 4):
        np.testing.assert_array_equal(a[r]["indices"], orc[r]["indices"], err_msg=f"short row {r}")


def test_step_rows_independent_and_non_finite_kv():
    # rows of a multi-row call equal one-row calls; a non-finite element in a
    # selected KV row zeroes that row's output in both forms
    kv_len = [20000, 33000, 18000]
    inp = I.small_rows(49, kv_len)
    dev = DeviceInputs(inp)
    probe = DeviceRows(dev)
    probe.step_one()
    res = probe.results()
    assert all(x["indices"].min() >= 0 for x in res)       # offsets 0, every slot selected
    kv0 = dev.kv[0].view(-1, 512)
    kv2 = dev.kv[2].view(-1, 512)
    kv0[int(res[0]["indices"][5]), 17] = 0x7FC0            # bf16 NaN
    kv2[int(res[2]["indices"][300]), 3] = 0x7F80           # bf16 +inf
    say("one call: non-finite selected KV rows, multi vs single rows")
    a, b = one_and_two(dev)
    check_equal(a, b, "non-finite kv")
    assert not a[0]["out"].any() and not a[2]["out"].any() and a[1]["out"].any()
    for r in range(len(kv_len)):
        one = DeviceRows(dev, rows=[r])
        one.step_one()
        o = one.results()[0]
        assert np.array_equal(o["indices"], a[r]["indices"]), r
        assert np.array_equal(o["out"].view(np.uint32), a[r]["out"].view(np.uint32)), r


def test_step_graph_replay_matches_eager():
    inp = I.make_config(3)
    dev = DeviceInputs(inp)
    eager = DeviceRows(dev)
    eager.step_one()
    ref = eager.results()
    g_run = DeviceRows(dev)
    g_run.step_one()                                   # warm-up before capture
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        g_run.step_one()
    say("one call: graph replays vs eager")
    for rep in range(3):
        g_run.out.zero_()
        g_run.indices.fill_(-7)
        graph.replay()
        torch.cuda.synchronize()
        got = g_run.results()
        check_equal(got, ref, f"replay {rep}")
        eager.step_one()
        torch.cuda.synchronize()


def test_step_permuted_row_subsets_match_full_launch():
    """Row tables whose entries are not in row order: entry i of a launch
    holds row sel[i] with that row's own q_row, offsets and buffers, so table
    index, q_row, index/output offsets and the grid's row index all differ.
    Every entry must give its row's results of the full launch bit for bit,
    on the one-call path and on the four-call path (gather kernel)."""
    kv_len = [20000, 33000, 18000, 24000, 40000]
    inp = I.small_rows(51, kv_len)
    dev = DeviceInputs(inp)
    full = DeviceRows(dev)
    full.step_one()
    ref = full.results()
    four = DeviceRows(dev)
    four.step()
    ref4 = four.results()
    for sel in ([4, 1, 3], [2, 0], [3, 4, 0, 2, 1]):
        say(f"one call and four calls: rows {sel}")
        sub = DeviceRows(dev, rows=sel)
        sub.step_one()
        got = sub.results()
        for i, r in enumerate(sel):
            assert np.array_equal(got[i]["scores"].view(np.uint32), ref[r]["scores"].view(np.uint32)), (sel, r)
            assert np.array_equal(got[i]["indices"], ref[r]["indices"]), (sel, r)
            assert np.array_equal(got[i]["out"].view(np.uint32), ref[r]["out"].view(np.uint32)), (sel, r)
        sub4 = DeviceRows(dev, rows=sel)
        sub4.step()
        got4 = sub4.results()
        for i, r in enumerate(sel):
            assert np.array_equal(got4[i]["gathered"], ref4[r]["gathered"]), (sel, r)
            assert np.array_equal(got4[i]["out"].view(np.uint32), ref4[r]["out"].view(np.uint32)), (sel, r)


@pytest.mark.parametrize("cid", [0, 1, 2, 3])
def test_timed_indexer_launch_changes_nothing(cid):
    """ds_rows_time_next_indexer: the armed step's indexer writes a start and
    four wave ends per workgroup (ends after starts, a span below a second),
    the outputs are those of an unarmed step bit for bit, the arm is used up
    by that launch, and a buffer too small for the grid is refused before
    anything is enqueued."""
    inp = I.make_config(cid)
    say(f"config {cid}: timed indexer launch")
    run = DeviceRows(DeviceInputs(inp))
    run.step_one()
    torch.cuda.synchronize()
    ref_out, ref_idx, ref_sc = run.out.clone(), run.indices.clone(), run.scores.clone()
    run.out.zero_()
    run.indices.fill_(-7)
    # The grid the header states: 1024-key blocks on a (blocks, rows) grid
    # with the fused stage (every row has 16384 visible keys or more), else
    # the largest power of two from 1024 down to 64 that gives the call at
    # least 256 blocks, on that grid or, when it would be more than twice
    # the blocks, one workgroup per block.
    visible = [min(n, (sp + 1) // 4) for n, sp in zip(inp.kv_len, inp.start_pos)]
    block = 1024
    if min(visible) < 16384:
        while block > 64 and sum(-(-n // block) for n in inp.kv_len) < 256:
            block //= 2
    blocks = sum(-(-n // block) for n in inp.kv_len)
    wgs = -(-max(inp.kv_len) // block) * inp.rows
    if min(visible) < 16384 and wgs > 2 * blocks:
        wgs = blocks   # the plain kernel's compact grid: one workgroup per block
    stamps = torch.zeros(wgs * ds.TIMER_STAMPS_PER_WG, dtype=torch.int64, device="cuda")
    ds.time_next_indexer(stamps)
    run.step_one()
    torch.cuda.synchronize()
    st = stamps.cpu().numpy().reshape(wgs, ds.TIMER_STAMPS_PER_WG)
    assert (st[:, 0] > 0).all()                       # every workgroup started
    assert (st[:, 1:5] >= st[:, :1]).all()            # ends after starts
    assert (st[:, 5:] == 0).all()
    span = ds.indexer_span_ticks(st)
    assert 0 < span < 10 ** 8, span                   # below a second at 100 MHz
    assert torch.equal(run.out, ref_out)
    assert torch.equal(run.indices, ref_idx)
    assert torch.equal(run.scores, ref_sc)
    # The arm was used up: a later step writes no stamps.
    stamps.zero_()
    run.step_one()
    torch.cuda.synchronize()
    assert int(stamps.abs().sum()) == 0
    # Too small for the grid: refused, outputs untouched, the arm stays.
    small = torch.zeros(ds.TIMER_STAMPS_PER_WG, dtype=torch.int64, device="cuda")
    ds.time_next_indexer(small)
    if wgs > 1:
        run.out.zero_()
        with pytest.raises(ds.DsRowsError, match="indexer timing buffer"):
            run.step_one()
        torch.cuda.synchronize()
        assert int(run.out.abs().sum()) == 0 and int(small.abs().sum()) == 0
        ds.time_next_indexer(stamps)   # replace the arm for the next call
        run.step_one()
        torch.cuda.synchronize()
