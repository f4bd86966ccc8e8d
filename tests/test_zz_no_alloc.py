"""ds_rows_indexer_topk_attn_noalloc (workspaces in the library's own device
scratch array) against ds_rows_indexer_topk_attn (caller workspaces), through
the C ABI: two calls in a row, the second on a smaller input than the first,
each equal to the existing entry point's scores, indices and output bit for
bit (and so to the oracle wherever that entry point is), plus the rejection
of a call whose workspaces exceed the array."""
import numpy as np
import pytest
import torch

from oracle import ds_oracle as O
from sparse_attention_decode_04_amd import ds_rows as ds
from sparse_attention_decode_04_amd import inputs as I
from sparse_attention_decode_04_amd.runner import DeviceInputs, DeviceRows

pytestmark = pytest.mark.gpu


def say(*a):
    print(*a, flush=True)


def noalloc_step(run):
    d = run.dev
    run.scores.fill_(float("nan"))
    run.indices.fill_(-7)
    run.out.fill_(float("nan"))
    ds.indexer_topk_attn_noalloc(run.itab, run.stab, d.idx_q, d.idx_w, run.scores, run.indices, d.attn_q,
                                 d.sinks, d.inp.scale, run.out)


def same_bits(a, b, label):
    for k in ("scores", "indices", "out"):
        assert np.array_equal(np.ascontiguousarray(a[k]).view(np.uint8),
                              np.ascontiguousarray(b[k]).view(np.uint8)), f"{label}: {k}"


@pytest.fixture(scope="module", autouse=True)
def gpu():
    assert torch.cuda.is_available(), "no HIP device"
    ds.load()
    yield


def test_noalloc_equals_one_call_twice_second_smaller():
    # first call: 8 rows x 32768 keys (fused indexer, final selection inside
    # the attention); second call: 3 shorter rows (separate score and top-k
    # kernels) in the same scratch array, which still holds the first call's
    # contents
    for seed, kv_len in ((61, [32768] * 8), (62, [17000, 700, 5000])):
        say(f"no-alloc vs one call: kv_len {kv_len}")
        inp = I.small_rows(seed, kv_len)
        dev = DeviceInputs(inp)
        ref = DeviceRows(dev)
        ref.step_one()
        want = ref.results()
        got_run = DeviceRows(dev)
        noalloc_step(got_run)
        got = got_run.results()
        for r in range(inp.rows):
            same_bits(got[r], want[r], f"kv_len {kv_len} row {r}")
        if len(kv_len) == 3:
            orc = O.decode_rows(inp)
            for r in range(inp.rows):
                np.testing.assert_array_equal(got[r]["indices"], orc[r]["indices"])
                err = np.abs(got[r]["out"].astype(np.float64) - orc[r]["out"])
                assert err.max() <= 1e-2 and err.mean() <= 1e-3, (r, err.max(), err.mean())


def test_noalloc_rejects_work_beyond_the_array():
    # 8 rows of 2M keys need ~28 MB of workspace: rejected from the tables
    # alone, before any operand is looked at or anything is enqueued
    small = I.small_rows(63, [1024])
    dev = DeviceInputs(small)
    run = DeviceRows(dev)
    big = [2_000_000] * 8
    it = ds.indexer_rows(big, [4 * n - 1 for n in big], [0] * 8, list(range(8)), [512 * r for r in range(8)],
                         keys=[dev.keys[0]] * 8)
    st = ds.sparse_rows(big, [512] * 8, [512 * r for r in range(8)], list(range(8)), kv=[dev.kv[0]] * 8)
    with pytest.raises(ds.DsRowsError, match="no-alloc scratch array holds"):
        ds.indexer_topk_attn_noalloc(it, st, dev.idx_q, dev.idx_w, run.scores, run.indices, dev.attn_q,
                                     dev.sinks, small.scale, run.out)
