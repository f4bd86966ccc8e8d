"""GPU parity of the HIP path against the CPU oracle (MI355X, gfx950).

Every test runs the library through its C ABI (via the ctypes binding) on
seeded synthetic inputs and compares each step's output with the oracle:
  indexer scores   exact (integer-valued inputs make every f32 score exact)
  top-k indices    exact, in rank order
  gathered rows    bit for bit; mask (0, or -inf for a sentinel) and the
                   per-row invalid flag exact
  attention out    max-abs <= 1e-2 and mean-abs <= 1e-3 against the oracle's
                   float64 result rounded to f32
and checks that each row of a multi-row launch equals a one-row launch on
that row bit for bit (docs.rs "mlx-native 0.21.0 src/ops/deepseek_rows.rs",
module documentation of the rows dispatches).
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

_cache = {}


def say(*a):
    print(*a, flush=True)


@pytest.fixture(scope="module", autouse=True)
def gpu():
    assert torch.cuda.is_available(), "no HIP device"
    ds.load()
    say("library:", ds.version(), "device:", torch.cuda.get_device_name(0))
    yield
    _cache.clear()


def config(cid):
    if cid not in _cache:
        say(f"generating config {cid}: {I.CONFIG_NAMES[cid]}")
        inp = I.make_config(cid)
        say(f"oracle for config {cid}")
        _cache.clear()
        _cache[cid] = (inp, O.decode_rows(inp), DeviceInputs(inp))
    return _cache[cid]


def mask_expected(orc):
    m = np.zeros(orc["sentinel"].shape[0], np.uint16)
    m[orc["sentinel"]] = 0xFF80
    return m


def check_row(got, orc, label, scores=True, gathered=True):
    if scores:
        np.testing.assert_array_equal(got["scores"], orc["scores"], err_msg=f"{label} scores")
    np.testing.assert_array_equal(got["indices"], orc["indices"], err_msg=f"{label} indices")
    if gathered:
        np.testing.assert_array_equal(got["gathered"], orc["gathered"], err_msg=f"{label} gathered")
        np.testing.assert_array_equal(got["mask"], mask_expected(orc), err_msg=f"{label} mask")
        assert got["invalid"] == int(bool(orc["slot_bad"].any())), f"{label} invalid flag"
    err = np.abs(got["out"].astype(np.float64) - orc["out"].astype(np.float64))
    say(f"  {label}: out max-abs {err.max():.3e} mean-abs {err.mean():.3e}")
    assert err.max() <= MAX_ABS and err.mean() <= MEAN_ABS, label


def bitwise_equal(a, b, label):
    for k in ("scores", "indices", "gathered", "mask"):
        assert np.array_equal(np.ascontiguousarray(a[k]).view(np.uint8),
                              np.ascontiguousarray(b[k]).view(np.uint8)), f"{label} {k}"
    assert a["invalid"] == b["invalid"], f"{label} invalid"
    assert np.array_equal(a["out"].view(np.uint32), b["out"].view(np.uint32)), f"{label} out"


@pytest.mark.parametrize("cid", [0, 1, 2, 3, 4])
def test_config_parity(cid):
    inp, orc, dev = config(cid)
    say(f"config {cid}: multi-row launch, rows={inp.rows}, gather + attention")
    run = DeviceRows(dev)
    run.step()
    got = run.results()
    for r in range(inp.rows):
        check_row(got[r], orc[r], f"config {cid} row {r} (kv_len {inp.kv_len[r]})")
    # the direct attention (gather fused in) on the same indices: same output bits
    say(f"config {cid}: direct attention")
    direct = DeviceRows(dev)
    direct.step_direct()
    got_d = direct.results()
    for r in range(inp.rows):
        check_row(got_d[r], orc[r], f"config {cid} row {r} direct", gathered=False)
        assert np.array_equal(got_d[r]["out"].view(np.uint32), got[r]["out"].view(np.uint32)), r


@pytest.mark.parametrize("cid", [1, 3])
def test_multi_row_equals_single_row_bitwise(cid):
    inp, _, dev = config(cid)
    say(f"config {cid}: multi-row vs single-row launches")
    multi = DeviceRows(dev)
    multi.step()
    m = multi.results()
    multi_d = DeviceRows(dev)
    multi_d.step_direct()
    md = multi_d.results()
    for r in range(inp.rows):
        one = DeviceRows(dev, rows=[r])
        one.step()
        bitwise_equal(m[r], one.results()[0], f"config {cid} row {r}")
        one_d = DeviceRows(dev, rows=[r])
        one_d.step_direct()
        assert np.array_equal(md[r]["out"].view(np.uint32), one_d.results()[0]["out"].view(np.uint32)), r


def test_repeated_steps_are_deterministic():
    inp, _, dev = config(1)
    say("config 1: two steps on the same buffers")
    run = DeviceRows(dev)
    run.step()
    a = run.results()
    run.step()
    b = run.results()
    for r in range(inp.rows):
        bitwise_equal(a[r], b[r], f"repeat row {r}")


def test_causal_limit_and_offset():
    # visible < kv_len, nothing visible, and a nonzero offset across chunks
    kv_len = [5000, 300, 20000, 9000]
    start_pos = [4 * 1000 + 2, 2, 4 * 20000 - 1, 4 * 8192 + 1]
    offset = [0, 0, 12345, 3]
    inp = I.small_rows(31, kv_len, start_pos=start_pos, offset=offset)
    say("causal/offset case", kv_len, start_pos, offset)
    dev = DeviceInputs(inp)
    run = DeviceRows(dev)
    run.step()
    got = run.results()
    orc = O.decode_rows(inp)
    for r in range(len(kv_len)):
        # rows with a nonzero offset emit indices past kv_len: the gather
        # flags them bad and the row's attention output is zero
        check_row(got[r], orc[r], f"causal row {r}")
    assert np.all(got[1]["indices"] == -1)
    assert np.all(got[2]["out"] == 0)


def test_all_equal_scores_take_lowest_indices():
    kv_len = [600, 20000, 131072]
    inp = I.small_rows(7, kv_len)
    for k in inp.idx_keys:
        k[:] = 0
    say("all-zero keys", kv_len)
    run = DeviceRows(DeviceInputs(inp))
    run.step()
    got = run.results()
    for r, n in enumerate(kv_len):
        assert np.all(got[r]["scores"] == 0)
        np.testing.assert_array_equal(got[r]["indices"], np.arange(512))
    orc = O.decode_rows(inp)
    for r in range(len(kv_len)):
        check_row(got[r], orc[r], f"tie row {r}")


def test_non_finite_indexer_keys():
    inp = I.small_rows(9, [64])
    q = inp.idx_q[0]
    keys = inp.idx_keys[0]
    keys[3, 5] = 0x7FC0    # NaN
    keys[4, 9] = 0x7F80    # +inf
    keys[5, 2] = 0xFF80    # -inf
    keys[6, :] = 0x7F80
    say("non-finite indexer keys")
    run = DeviceRows(DeviceInputs(inp))
    run.indexer_score()
    run.topk()
    got = run.results()[0]
    exp = O.indexer_scores(q, inp.idx_w[0], keys, inp.start_pos[0])
    np.testing.assert_array_equal(got["scores"], exp)
    np.testing.assert_array_equal(got["indices"], O.topk_select(exp, 64))


def test_fail_closed_injections():
    kv_len = [900, 1000, 700, 800, 950]
    inp = I.small_rows(17, kv_len)
    inp.attn_q[3, 7, 100] = 0x7FC0          # NaN in row 3, head 7 query
    inp.sinks[11] = np.inf                  # sink of head 11 (shared by every row)
    dev = DeviceInputs(inp)
    run = DeviceRows(dev)
    run.indexer_score()
    run.topk()
    torch.cuda.synchronize()
    idx = run.indices.cpu().numpy().reshape(-1, 512)[: len(kv_len)].copy()
    idx[0, [5, 100]] = -1                   # sentinels: excluded
    idx[1, 7] = kv_len[1]                   # bad index: row 1 zeroed
    idx[4, 487] = -5                        # bad index deep in the last chunk: row 4 zeroed
    nan_row = int(idx[2, 3])
    inp.kv[2][nan_row, 17] = 0x7FC0         # non-finite KV element: row 2 zeroed
    dev.kv[2][nan_row, 17] = torch.tensor(0x7FC0, dtype=torch.int16)
    run.indices[: idx.size] = torch.from_numpy(idx.reshape(-1)).cuda()
    say("fail-closed injections, direct attention")
    run.sparse_attn_direct()
    got_d = [g["out"].copy() for g in run.results()]
    say("fail-closed injections, gather + attention")
    run.out.zero_()
    run.gather()
    run.sparse_attn()
    got = run.results()
    for r in range(len(kv_len)):
        assert np.array_equal(got_d[r].view(np.uint32), got[r]["out"].view(np.uint32)), r
    for r in range(len(kv_len)):
        g, sent, bad, inv = O.gather_row(inp.kv[r], idx[r], kv_len[r])
        out = O.sparse_attention_row(inp.attn_q[r], inp.sinks, g, sent, inv, inp.scale)
        orc = dict(indices=idx[r], gathered=g, sentinel=sent, slot_bad=bad, out=out)
        got[r]["indices"] = idx[r]
        check_row(got[r], orc, f"inject row {r}", scores=False)
    assert [g["invalid"] for g in got] == [0, 1, 1, 0, 1]
    # bad slots keep mask 0 (only sentinels are -inf), as the pages' gather writes it
    assert got[1]["mask"][7] == 0 and got[4]["mask"][487] == 0 and got[0]["mask"][5] == 0xFF80
    assert np.all(got[1]["out"] == 0) and np.all(got[2]["out"] == 0) and np.all(got[4]["out"] == 0)
    assert np.all(got[3]["out"][7] == 0) and np.all(got[0]["out"][11] == 0)
    assert np.all(np.abs(got[0]["out"][10]) > 0)


def test_widths_other_than_512():
    rng = np.random.default_rng(5)
    kv_len = [3000, 5000, 40]
    width = [100, 700, 40]
    inp = I.small_rows(23, kv_len)
    idx = np.full(3 * 1024, -7, np.int32)
    offs = [0, 1024, 2048]
    rows_idx = []
    for r in range(3):
        sel = rng.choice(kv_len[r], size=width[r], replace=False).astype(np.int32)
        sel[rng.random(width[r]) < 0.05] = -1
        idx[offs[r]: offs[r] + width[r]] = sel
        rows_idx.append(sel)
    dev = DeviceInputs(inp)
    t = ds.sparse_rows(kv_len, width, offs, [0, 1, 2], kv=dev.kv)
    d_idx = torch.from_numpy(idx).cuda()
    gathered = torch.empty(ds.gathered_elems(t), dtype=torch.int16, device="cuda")
    mask = torch.empty(ds.mask_elems(t), dtype=torch.int16, device="cuda")
    invalid = torch.full((3,), 5, dtype=torch.int32, device="cuda")
    # The workspace starts as NaN bytes: the rows of 2 and 1 chunks have room
    # for 11 like the widest, and nothing left in that room may reach an output.
    ws = torch.full((ds.attn_workspace_bytes(t),), 0xFF, dtype=torch.uint8, device="cuda")
    out = torch.zeros(3 * 64 * 512, dtype=torch.float32, device="cuda")
    say("widths", width, "direct")
    ds.sparse_attn_direct(t, dev.attn_q, dev.sinks, d_idx, inp.scale, ws, out)
    torch.cuda.synchronize()
    o_direct = out.cpu().numpy().reshape(3, 64, 512).copy()
    out.zero_()
    ws.fill_(0xFF)
    say("widths", width, "gather + attention")
    ds.gather(t, d_idx, gathered, mask, invalid)
    ds.sparse_attn(t, dev.attn_q, dev.sinks, gathered, mask, invalid, inp.scale, ws, out)
    torch.cuda.synchronize()
    g_all = gathered.cpu().numpy().view(np.uint16).reshape(-1, 512)
    m_all = mask.cpu().numpy().view(np.uint16)
    v_all = invalid.cpu().numpy()
    o_all = out.cpu().numpy().reshape(3, 64, 512)
    assert np.array_equal(o_all.view(np.uint32), o_direct.view(np.uint32))
    base = 0
    for r in range(3):
        g, sent, bad, inv = O.gather_row(inp.kv[r], rows_idx[r], kv_len[r])
        o = O.sparse_attention_row(inp.attn_q[r], inp.sinks, g, sent, inv, inp.scale)
        got = dict(indices=rows_idx[r], gathered=g_all[base: base + width[r]],
                   mask=m_all[base: base + width[r]], invalid=int(v_all[r]), out=o_all[r])
        check_row(got, dict(indices=rows_idx[r], gathered=g, sentinel=sent, slot_bad=bad, out=o),
                  f"width {width[r]}", scores=False)
        base += width[r]


@pytest.mark.parametrize("ternary", [False, True])
@pytest.mark.parametrize("longest", [4096, 4097, 8192, 8193, 16384, 16385])
def test_first_level_sizes_at_their_edges(longest, ternary):
    # The first top-k level takes 4, 8, 16 or 32 score slots per thread by the
    # call's longest row (at most 4096, 8192, 16384 keys, or more): each edge
    # from both sides, with a shorter row and a row past 512 beside it, through
    # the four calls and the one call; ternary keys give heavy ties.
    kv_len = [longest, 700, longest - 1500]
    inp = I.small_rows(50 + longest % 97 + 7 * ternary, kv_len, ternary=ternary)
    say("first-level size edge", kv_len, "ternary" if ternary else "integer")
    orc = O.decode_rows(inp)
    dev = DeviceInputs(inp)
    run = DeviceRows(dev)
    run.step()
    got = run.results()
    for r in range(inp.rows):
        check_row(got[r], orc[r], f"edge {longest} row {r}")
    one = DeviceRows(dev)
    one.step_one()
    got1 = one.results()
    for r in range(inp.rows):
        check_row(got1[r], orc[r], f"edge {longest} row {r} one call", gathered=False)


@pytest.mark.parametrize("kv_len", [(1000, 20000), (20000,) * 8, (1000, 70000, 32768, 32769), (3000, 131072),
                                    (700, 200000)])
def test_topk_banks_hold_every_first_level_chunk(kv_len):
    # ds_rows_topk over scores split into chunks of 16384 (a longest row of at
    # most 8 x 16384) or 32768: the list banks the workspace query sizes hold
    # every chunk's list. The workspace is exactly that size, followed by a
    # canary that must come back untouched; the indices are the oracle's.
    rows = len(kv_len)
    rng = np.random.default_rng(sum(kv_len))
    sp = [4 * n - 1 for n in kv_len]
    table = ds.indexer_rows(list(kv_len), sp, [0] * rows, list(range(rows)), [512 * r for r in range(rows)])
    stride = max(kv_len)
    scores = np.full((rows, stride), -np.inf, np.float32)
    for r, n in enumerate(kv_len):
        scores[r, :n] = rng.standard_normal(n).astype(np.float32)
    need = ds.topk_workspace_bytes(table)
    canary = 1 << 16
    ws = torch.full((need + canary,), 0x5A, dtype=torch.uint8, device="cuda")
    idx = torch.full((512 * rows,), -7, dtype=torch.int32, device="cuda")
    say("top-k banks", kv_len, "workspace", need)
    ds.topk(table, torch.from_numpy(scores.reshape(-1)).cuda(), ws[:max(need, 1)], idx)
    torch.cuda.synchronize()
    assert bool((ws[need:] == 0x5A).all()), "the selection wrote past its workspace"
    got = idx.cpu().numpy().reshape(rows, 512)
    for r, n in enumerate(kv_len):
        want = O.topk_select(scores[r], O.valid_count(n, sp[r]), 0)
        np.testing.assert_array_equal(got[r], want, err_msg=f"row {r} ({n} keys)")
