"""GPU parity of ds_rows_compressor (learned KV compressor, one decode token
per row) against the CPU oracle.

Source: docs.rs "mlx-native 0.18.0 src/shaders/deepseek_rows.metal", kernel
deepseek_compressor_rows_bf16, and "mlx-native 0.21.0 src/ops/deepseek_rows.rs",
dispatch_deepseek_compressor_rows.

Bar. The state update is a copy and one f32 addition, so both states must
match the oracle bit for bit. The output is bf16: the kernel pools in f32
with the hardware exponential, the oracle in float64, so the pooled value can
land on the other side of a bf16 rounding boundary (one bf16 unit in the last
place), and the final bf16 rounding of the normalised value can differ by one
more unit; the sum of squares and the RMS scale move by far less than one
unit. Where the window's weighted sum cancels to a small value, the f32 error
is small in absolute terms (about 2^-24 times the magnitude of the terms, a
few 1e-7 for these inputs, times the RMS scale) but not relative to the tiny
result. Hence: every output element within 2 bf16 ulps of the oracle or
within 2^-12 absolute (outputs have RMS ~1, where a bf16 ulp is 2^-7 to
2^-8), at least 99% identical, and zero rows (no emission, fail-closed)
exactly zero. Rows of a multi-row call equal one-row calls bit for bit.
"""
import numpy as np
import pytest
import torch

from oracle import ds_oracle as O
from sparse_attention_decode_04_amd import ds_rows as ds
from sparse_attention_decode_04_amd import inputs as I
from sparse_attention_decode_04_amd.runner import DeviceCompressor

pytestmark = pytest.mark.gpu

SHAPES = [(4, 128), (4, 512), (128, 512)]


def say(*a):
    print(*a, flush=True)


@pytest.fixture(scope="module", autouse=True)
def gpu():
    assert torch.cuda.is_available(), "no HIP device"
    ds.load()
    yield


def ulp_diff(a_bits, b_bits):
    a = np.asarray(a_bits, np.int32)
    b = np.asarray(b_bits, np.int32)
    sa = np.where(a & 0x8000, -(a & 0x7FFF), a)
    sb = np.where(b & 0x8000, -(b & 0x7FFF), b)
    return np.abs(sa - sb)


ABS_TOL = 2.0 ** -12


def close(got_bits, exp_bits):
    """Elementwise: within 2 bf16 ulps, or within ABS_TOL absolute."""
    d = ulp_diff(got_bits, exp_bits)
    a = np.abs(O.bf16_bits_to_f64(got_bits) - O.bf16_bits_to_f64(exp_bits))
    return (d <= 2) | (a <= ABS_TOL)


def check_against_oracle(inp, got, label):
    kvs, scs, outs = got
    ekv, esc, eout = O.compressor_rows(inp)
    for r in range(inp.rows):
        assert np.array_equal(kvs[r].view(np.uint32), ekv[r].view(np.uint32)), (label, r, "kv_state")
        assert np.array_equal(scs[r].view(np.uint32), esc[r].view(np.uint32)), (label, r, "score_state")
        if not eout[r].any():
            assert not outs[r].any(), (label, r, "expected a zero row")
            continue
        ok = close(outs[r], eout[r])
        assert ok.all(), (label, r, np.nonzero(~ok)[0][:8], outs[r][~ok][:8], eout[r][~ok][:8])
        assert np.mean(outs[r] == eout[r]) >= 0.99, (label, r)


@pytest.mark.parametrize("ratio,head_dim", SHAPES)
def test_workload_parity(ratio, head_dim):
    inp = I.compressor_workload(ratio, head_dim)
    say(f"compressor ({ratio},{head_dim}): 8 rows, every token ends a block")
    dev = DeviceCompressor(inp)
    dev.run()
    check_against_oracle(inp, dev.results(), f"({ratio},{head_dim})")


@pytest.mark.parametrize("ratio,head_dim", SHAPES)
def test_mixed_positions_and_row_independence(ratio, head_dim):
    # rows that end a block and rows that do not, in one call; each row must
    # equal a one-row call on it
    pos = [ratio - 1, ratio, 2 * ratio + 1, 3 * ratio - 1, 5 * ratio + 2, 1, 77 * ratio - 1, 9 * ratio - 2]
    inp = I.make_compressor(41 + ratio + head_dim, 8, ratio, head_dim, start_pos=pos)
    say(f"compressor ({ratio},{head_dim}): mixed positions {pos}")
    multi = DeviceCompressor(inp)
    multi.run()
    got = multi.results()
    check_against_oracle(inp, got, f"mixed ({ratio},{head_dim})")
    for r in range(inp.rows):
        one = DeviceCompressor(inp, rows=[r])
        one.run()
        k1, s1, o1 = one.results()
        assert np.array_equal(o1[0], got[2][r]), r
        assert np.array_equal(k1[0].view(np.uint32), got[0][r].view(np.uint32)), r
        assert np.array_equal(s1[0].view(np.uint32), got[1][r].view(np.uint32)), r


@pytest.mark.parametrize("ratio,head_dim", SHAPES)
def test_decode_sequence(ratio, head_dim):
    # Consecutive tokens on the device state against the oracle stepped the
    # same way: two block ends per row (the state and the overlap shift
    # carried from call to call).
    rows = 3
    steps = 2 * ratio + 1
    base = I.make_compressor(51 + ratio, rows, ratio, head_dim, start_pos=[ratio * 5 + r for r in range(rows)])
    rng = np.random.default_rng(52 + ratio)
    dev = DeviceCompressor(base)
    ekv = [base.kv_state[r].copy() for r in range(rows)]
    esc = [base.score_state[r].copy() for r in range(rows)]
    say(f"compressor ({ratio},{head_dim}): {steps} consecutive tokens on {rows} rows")
    emitted = 0
    for t in range(steps):
        pos = [p + t for p in base.start_pos]
        kv = rng.standard_normal(base.kv.shape).astype(np.float32)
        sc = rng.standard_normal(base.score.shape).astype(np.float32)
        dev.kv.copy_(torch.from_numpy(kv))
        dev.score.copy_(torch.from_numpy(sc))
        dev.tables = [ds.compressor_rows(pos, *dev.states[0])]
        dev.run()
        out = dev.out.cpu().numpy().view(np.uint16)
        for r in range(rows):
            ekv[r], esc[r], eo = O.compressor_row(kv[r], sc[r], base.ape, base.norm, ekv[r], esc[r], pos[r],
                                                  ratio, head_dim, base.eps)
            if eo.any():
                emitted += 1
                assert close(out[r], eo).all() and np.mean(out[r] == eo) >= 0.99, (t, r)
            else:
                assert not out[r].any(), (t, r)
    assert emitted >= 2 * rows - 1
    kvs, scs, _ = dev.results()
    for r in range(rows):
        assert np.array_equal(kvs[r].view(np.uint32), ekv[r].view(np.uint32)), r
        assert np.array_equal(scs[r].view(np.uint32), esc[r].view(np.uint32)), r


@pytest.mark.parametrize("ratio,head_dim", SHAPES)
def test_fail_closed(ratio, head_dim):
    inp = I.compressor_workload(ratio, head_dim)
    hd = head_dim
    # row 1: NaN window score; row 2: +inf window score; row 3: non-finite
    # window value; row 4: non-finite token value inside the window;
    # row 5: NaN outside the window (overlap only: previous block, second
    # half) -> not zeroed; row 6: -inf window score -> not zeroed
    inp.score_state[1][1, 3] = np.nan
    inp.score_state[2][2, 5] = np.inf
    inp.kv_state[3][0, 7] = np.inf
    if ratio == 4:
        inp.kv[4][hd + 9] = np.nan
        inp.score_state[5][0, hd + 1] = np.nan
    else:
        inp.kv[4][9] = np.nan
    inp.score_state[6][3, 11] = -np.inf
    say(f"compressor ({ratio},{head_dim}): fail-closed injections")
    dev = DeviceCompressor(inp)
    dev.run()
    got = dev.results()
    check_against_oracle(inp, got, "fail-closed")
    outs = got[2]
    for r in (1, 2, 3, 4):
        assert not outs[r].any(), r
    assert outs[0].any() and outs[6].any() and outs[7].any()
    if ratio == 4:
        assert outs[5].any()
    # a non-finite RMS scale element zeroes every emitting row
    inp2 = I.compressor_workload(ratio, head_dim)
    inp2.norm[17] = np.nan
    dev2 = DeviceCompressor(inp2)
    dev2.run()
    assert not any(o.any() for o in dev2.results()[2])


def test_graph_replay_matches_eager():
    # The benchmark times this call through HIP graph replays: each replay
    # must give what the same eager call gives (state carried forward on two
    # identical state sets, one driven by the graph and one eagerly).
    inp = I.compressor_workload(128, 512)
    dev = DeviceCompressor(inp, copies=2)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    warm = DeviceCompressor(inp)
    warm.run()                                   # capture needs a warmed-up stream
    torch.cuda.synchronize()
    with torch.cuda.graph(graph):
        dev.run(0)
    say("compressor: graph replays vs eager calls")
    for rep in range(3):
        graph.replay()
        torch.cuda.synchronize()
        g = dev.results(0)
        dev.run(1)
        e = dev.results(1)
        for r in range(inp.rows):
            assert np.array_equal(g[2][r], e[2][r]), (rep, r)
            assert np.array_equal(g[0][r].view(np.uint32), e[0][r].view(np.uint32)), (rep, r)
            assert np.array_equal(g[1][r].view(np.uint32), e[1][r].view(np.uint32)), (rep, r)
