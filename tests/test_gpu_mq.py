"""GPU parity of the multi-query indexer (ds_rows_indexer_score_mq) against
the CPU oracle, and of each query's top-512 selected from its scores with
ds_rows_topk on the expanded row table.

Source: docs.rs "mlx-native 0.18.0 src/shaders/deepseek_rows.metal", kernel
deepseek_indexer_score_mma_rows_bf16 (query loop with a causal count per
query row). The inputs are integer-valued, so every score is an exact
integer below 2^24 and must match the oracle bit for bit; indices are exact.
"""
import numpy as np
import pytest
import torch

from oracle import ds_oracle as O
from sparse_attention_decode_04_amd import ds_rows as ds
from sparse_attention_decode_04_amd import inputs as I
from sparse_attention_decode_04_amd.runner import DeviceMultiQuery

pytestmark = pytest.mark.gpu


def say(*a):
    print(*a, flush=True)


@pytest.fixture(scope="module", autouse=True)
def gpu():
    assert torch.cuda.is_available(), "no HIP device"
    ds.load()
    yield


def oracle_row(inp, r):
    Q = inp.query_len
    return O.indexer_scores_mq(inp.idx_q[Q * r:Q * r + Q], inp.idx_w[Q * r:Q * r + Q], inp.idx_keys[r],
                               inp.start_pos[r])


def check_rows(inp, got, rows=None):
    rows = range(inp.rows) if rows is None else rows
    for i, r in enumerate(rows):
        exp = oracle_row(inp, r)
        for t in range(inp.query_len):
            np.testing.assert_array_equal(got[i][t], exp[t], err_msg=f"row {r} query {t}")


@pytest.mark.parametrize("Q", [1, 2, 3, 4, 5, 8])
def test_ragged_rows(Q):
    kv_len = [1 if Q <= 4 else 2, 63, 64, 65, 700, 2000, 4096, 513]
    inp = I.make_mq(300 + Q, kv_len, Q)
    say(f"multi-query indexer: Q={Q}, kv_len {kv_len}")
    dev = DeviceMultiQuery(inp)
    dev.run()
    check_rows(inp, dev.results())


def test_non_finite_keys_and_queries():
    # NaN and infinite key and query elements: a NaN dot product contributes
    # 0 through the ReLU (maxNum), an infinite one makes the score non-finite
    # (-inf), as the oracle computes it
    kv_len = [300, 130]
    Q = 3
    inp = I.make_mq(405, kv_len, Q)
    k0 = inp.idx_keys[0]
    k0[3, 5] = 0x7FC0     # NaN
    k0[4, 9] = 0x7F80     # +inf
    k0[5, 2] = 0xFF80     # -inf
    k0[6, :] = 0x7F80     # a whole row of +inf
    k0[7, 0] = 0x7F80     # +inf and -inf in one row
    k0[7, 1] = 0xFF80
    inp.idx_q[Q * 1 + 2, 10, 3] = 0x7FC0    # NaN in a query of row 1
    say("multi-query indexer: non-finite keys and queries")
    dev = DeviceMultiQuery(inp)
    dev.run()
    check_rows(inp, dev.results())


def test_per_query_causal_limits_and_ternary_keys():
    # start positions well inside the cache: each query hides a different
    # number of keys; ternary entries give many zero and tied scores
    kv_len = [3000, 777, 128]
    Q = 8
    start_pos = [4 * 1000 + 1, 4 * 500 + 3, 17]
    inp = I.make_mq(401, kv_len, Q, ternary=True, start_pos=start_pos)
    say("multi-query indexer: causal limits per query", start_pos)
    dev = DeviceMultiQuery(inp)
    dev.run()
    got = dev.results()
    check_rows(inp, got)
    for i, r in enumerate(range(inp.rows)):
        for t in range(Q):
            vis = O.valid_count(kv_len[r], start_pos[r] + t)
            assert np.all(np.isneginf(got[i][t][vis:])), (r, t)


def test_query_len_one_equals_single_query_indexer():
    kv_len = [5000, 1234]
    inp = I.make_mq(402, kv_len, 1)
    dev = DeviceMultiQuery(inp)
    dev.run()
    mq = dev.results()
    scores = torch.empty(ds.scores_elems(dev.table), dtype=torch.float32, device="cuda")
    ds.indexer_score(dev.table, dev.q, dev.w, scores)
    single = scores.cpu().numpy().reshape(len(kv_len), -1)
    for r, n in enumerate(kv_len):
        assert np.array_equal(mq[r][0].view(np.uint32), single[r, :n].view(np.uint32)), r


def test_rows_independent():
    inp = I.make_mq(403, [900, 64, 3000], 6)
    multi = DeviceMultiQuery(inp)
    multi.run()
    m = multi.results()
    for r in range(inp.rows):
        one = DeviceMultiQuery(inp, rows=[r])
        one.run()
        o = one.results()[0]
        for t in range(inp.query_len):
            assert np.array_equal(o[t].view(np.uint32), m[r][t].view(np.uint32)), (r, t)


@pytest.mark.parametrize("R,Q", [(1, 8), (2, 4)])
def test_topk_per_query_on_expanded_table(R, Q):
    kv_len = [20000, 9000][:R]
    start_pos = [4 * 20000 - 30, 4 * 9000 - Q][:R]
    inp = I.make_mq(404 + Q, kv_len, Q, start_pos=start_pos)
    dev = DeviceMultiQuery(inp)
    dev.run()
    # entry e = r*Q + t: the row's keys at position start_pos + t
    E = R * Q
    kv = [kv_len[e // Q] for e in range(E)]
    sp = [start_pos[e // Q] + e % Q for e in range(E)]
    table = ds.indexer_rows(kv, sp, [0] * E, [0] * E, [512 * e for e in range(E)],
                            keys=[dev.keys[e // Q] for e in range(E)])
    assert ds.scores_elems(table) == dev.scores.numel()
    ws = torch.empty(max(ds.topk_workspace_bytes(table), 1), dtype=torch.uint8, device="cuda")
    idx = torch.empty(512 * E, dtype=torch.int32, device="cuda")
    ds.topk(table, dev.scores, ws, idx)
    got = idx.cpu().numpy().reshape(E, 512)
    say(f"multi-query top-k: {R} rows x {Q} queries")
    for r in range(R):
        exp = oracle_row(inp, r)
        for t in range(Q):
            want = O.topk_select(exp[t], O.valid_count(kv_len[r], start_pos[r] + t), 0)
            np.testing.assert_array_equal(got[r * Q + t], want, err_msg=f"row {r} query {t}")


def test_full_workload_two_rows():
    # 8 rows x 32768 keys x 8 queries (the measured shape); the oracle checks
    # rows 0 and 7 in full, every query
    inp = I.mq_workload(8)
    say("multi-query indexer: 8 x 32768 x 8 queries")
    dev = DeviceMultiQuery(inp)
    dev.run()
    got = dev.results()
    check_rows(inp, [got[0], got[7]], rows=[0, 7])
