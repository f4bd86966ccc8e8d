"""The C ABI on the CPU: the library loads, exports every symbol the header
declares, the binding's struct layouts match the C compiler's, the size
queries are right, and every argument check fires before anything is
enqueued (so these calls use fake, never-dereferenced device addresses and
never reach a launch).

The checked conditions are those the host dispatch code on docs.rs
"mlx-native 0.21.0 src/ops/deepseek_rows.rs" requires of its rows dispatches;
the messages are this library's own.
"""
import ctypes
import os
import re
import subprocess
import tempfile

import pytest

from sparse_attention_decode_04_amd import ds_rows as ds

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "ds_rows.h")
FAKE = 0x100000            # never dereferenced: every call below fails its checks
BIG = 1 << 40
INVALID = 1
DEVICE = 3


@pytest.fixture(scope="module")
def lib():
    # These tests hand fake device addresses to calls that must fail their
    # argument checks. Never run them where a GPU could execute a launch.
    import torch
    if torch.cuda.is_available():
        pytest.skip("fake-address argument-check tests run only on hosts without a GPU")
    if not os.path.exists(ds.LIB_PATH):
        from sparse_attention_decode_04_amd import build
        build.build()
    return ds.load()


def header_functions():
    text = open(HEADER).read()
    return sorted(set(re.findall(r"^\s*(?:ds_status|size_t|const char \*)\s*(ds_rows_\w+)\s*\(", text, re.M)))


def test_exports_every_declared_symbol(lib):
    names = header_functions()
    assert len(names) == 23
    assert set(names) == set(ds.FUNCTIONS)
    out = subprocess.run(["nm", "-D", "--defined-only", ds.LIB_PATH], capture_output=True, text=True).stdout
    exported = set(re.findall(r" T (ds_rows_\w+)", out))
    assert set(names) <= exported
    for n in names:
        assert getattr(lib, n) is not None
    assert ds.version().startswith("ds_rows")


def test_struct_layout_matches_c_compiler():
    src = r"""
#include <stdio.h>
#include <stddef.h>
#include "ds_rows.h"
#define F(T, f) printf(#T "." #f " %zu\n", offsetof(T, f))
int main(void) {
  printf("ds_indexer_rows %zu\n", sizeof(ds_indexer_rows));
  F(ds_indexer_rows, kv_len); F(ds_indexer_rows, start_pos); F(ds_indexer_rows, offset);
  F(ds_indexer_rows, q_row); F(ds_indexer_rows, output_offset); F(ds_indexer_rows, keys);
  F(ds_indexer_rows, keys_elems);
  printf("ds_sparse_rows %zu\n", sizeof(ds_sparse_rows));
  F(ds_sparse_rows, kv_len); F(ds_sparse_rows, width); F(ds_sparse_rows, index_offset);
  F(ds_sparse_rows, q_row); F(ds_sparse_rows, kv); F(ds_sparse_rows, kv_elems);
  printf("ds_compressor_rows %zu\n", sizeof(ds_compressor_rows));
  F(ds_compressor_rows, start_pos); F(ds_compressor_rows, kv_state); F(ds_compressor_rows, score_state);
  F(ds_compressor_rows, kv_state_elems); F(ds_compressor_rows, score_state_elems);
  return 0;
}
"""
    with tempfile.TemporaryDirectory() as d:
        c = os.path.join(d, "layout.c")
        open(c, "w").write(src)
        exe = os.path.join(d, "layout")
        subprocess.run(["gcc", "-I", os.path.join(ROOT, "include"), c, "-o", exe], check=True)
        lines = subprocess.run([exe], capture_output=True, text=True, check=True).stdout.split("\n")
    got = dict(l.rsplit(" ", 1) for l in lines if l)
    assert int(got["ds_indexer_rows"]) == ctypes.sizeof(ds.IndexerRows)
    assert int(got["ds_sparse_rows"]) == ctypes.sizeof(ds.SparseRows)
    assert int(got["ds_compressor_rows"]) == ctypes.sizeof(ds.CompressorRows)
    for (T, C) in (("ds_indexer_rows", ds.IndexerRows), ("ds_sparse_rows", ds.SparseRows),
                   ("ds_compressor_rows", ds.CompressorRows)):
        for name, _ in C._fields_[1:]:
            assert int(got[f"{T}.{name}"]) == getattr(C, name).offset, (T, name)


# ------------------------------------------------------------------ helpers

def itab(kv_len=(100,), start_pos=None, offset=None, q_row=None, out_off=None, keys_elems=None):
    R = len(kv_len)
    start_pos = [4 * n - 1 for n in kv_len] if start_pos is None else start_pos
    offset = [0] * R if offset is None else offset
    q_row = list(range(R)) if q_row is None else q_row
    out_off = [512 * r for r in range(R)] if out_off is None else out_off
    keys_elems = [BIG] * R if keys_elems is None else keys_elems
    return ds.indexer_rows(kv_len, start_pos, offset, q_row, out_off, keys=[FAKE] * R, keys_elems=keys_elems)


def stab(kv_len=(100,), width=None, index_offset=None, q_row=None, kv_elems=None):
    R = len(kv_len)
    width = [min(n, 512) for n in kv_len] if width is None else width
    index_offset = [512 * r for r in range(R)] if index_offset is None else index_offset
    q_row = list(range(R)) if q_row is None else q_row
    kv_elems = [BIG] * R if kv_elems is None else kv_elems
    return ds.sparse_rows(kv_len, width, index_offset, q_row, kv=[FAKE] * R, kv_elems=kv_elems)


def call_score(lib, t, q=BIG, w=BIG, s=BIG, qp=FAKE):
    return lib.ds_rows_indexer_score(ctypes.byref(t), qp, q, FAKE, w, FAKE, s, None)


def call_topk(lib, t, s=BIG, ws=BIG, idx=BIG):
    return lib.ds_rows_topk(ctypes.byref(t), FAKE, s, FAKE, ws, FAKE, idx, None)


def call_fused(lib, t, q=BIG, w=BIG, s=BIG, ws=BIG, idx=BIG, wsp=FAKE):
    return lib.ds_rows_indexer_topk(ctypes.byref(t), FAKE, q, FAKE, w, FAKE, s, wsp, ws, FAKE, idx, None)


def call_gather(lib, t, idx=BIG, g=BIG, m=BIG, inv=BIG, invp=FAKE):
    return lib.ds_rows_gather(ctypes.byref(t), FAKE, idx, FAKE, g, FAKE, m, invp, inv, None)


def call_attn(lib, t, scale=0.0441941738, q=BIG, sinks=64, g=BIG, m=BIG, inv=BIG, ws=BIG, out=BIG, invp=FAKE):
    return lib.ds_rows_sparse_attn(ctypes.byref(t), FAKE, q, FAKE, sinks, FAKE, g, FAKE, m, invp, inv,
                                   ctypes.c_float(scale), FAKE, ws, FAKE, out, None)


def call_direct(lib, t, scale=0.0441941738, q=BIG, sinks=64, idx=BIG, ws=BIG, out=BIG):
    return lib.ds_rows_sparse_attn_direct(ctypes.byref(t), FAKE, q, FAKE, sinks, FAKE, idx,
                                          ctypes.c_float(scale), FAKE, ws, FAKE, out, None)


def expect_invalid(status, *fragments):
    assert status == INVALID
    msg = ds.last_error()
    assert msg.startswith("ds_rows: ")
    for f in fragments:
        assert f in msg, msg


# -------------------------------------------------------------------- sizes

def test_size_queries(lib):
    t = itab((1000, 70000, 32768, 32769))
    assert ds.scores_elems(t) == 4 * 70000
    # top-k lists: rows longer than one chunk need the banks. The call's
    # longest row (70000 <= 8 x 16384) sets chunks of 16384 scores: 5, 2 and 3
    # chunks of 512 keys for the rows of 70000, 32768 and 32769 keys
    assert ds.topk_workspace_bytes(t) == 2 * 8 * 512 * (5 + 2 + 3)
    assert ds.topk_workspace_bytes(itab((1000, 32768))) == 2 * 8 * 512 * 2
    assert ds.topk_workspace_bytes(itab((1000, 16384))) == 0      # one chunk per row
    # beyond 8 x 16384 scores in a row, chunks of 32768: 200000 -> 7 chunks
    assert ds.topk_workspace_bytes(itab((1000, 200000))) == 2 * 8 * 512 * 7
    # fused: 128 candidate keys and four u64 floors per 1024-key block, every
    # row with room for the widest row's blocks (here the 70000-key row's 69;
    # each region 256-byte aligned), plus two list banks for rows whose
    # candidates exceed one 8192-key chunk (rows over 65536 keys): here the
    # 70000-key row, 69 blocks -> 8832 candidates -> 2 chunks of 512
    room = 69
    floors = -(-4 * room * 4 * 8 // 256) * 256
    assert ds.indexer_topk_workspace_bytes(t) == 4 * room * 128 * 8 + floors + 2 * 2 * 512 * 8
    big = itab((200000,))
    nb = 196
    cand = -(-nb * 128 * 8 // 256) * 256
    floors = -(-nb * 4 * 8 // 256) * 256
    chunks = -(-nb * 128 // 8192)
    assert ds.indexer_topk_workspace_bytes(big) == cand + floors + 2 * chunks * 512 * 8
    # the size covers both of the call's paths: a lone 1000-key row (which
    # takes the separate score and top-k kernels) still gets the fused
    # stage's candidates (one block: 1 KiB) and floors (32 B -> 256)
    assert ds.indexer_topk_workspace_bytes(itab((1000,))) == 1024 + 256
    s = stab((1000, 37, 1), width=(512, 37, 1))
    assert ds.gathered_elems(s) == (512 + 37 + 1) * 512
    assert ds.mask_elems(s) == 512 + 37 + 1
    chunks = 3 * 8                              # every row has room for the call's most chunks (512 slots: 8)
    stat_bytes = 64 * chunks * 16               # f32x4 statistics per (chunk, head)
    part_bytes = chunks * 64 * 512 * 4          # f32 output of each chunk
    up = lambda x: (x + 255) // 256 * 256
    assert ds.attn_workspace_bytes(s) == up(stat_bytes) + up(part_bytes)
    assert ds.scores_elems(itab((0,))) == 0            # invalid table -> 0



def test_noalloc_capacity_matches_the_header(lib):
    # ds_rows.h states what the no-alloc array (DS_NOALLOC_SCRATCH_BYTES =
    # 16 MiB) holds: both workspaces (the indexer's rounded up to 256 bytes)
    # for 8 rows of 897024 keys or one row of 13.59 million, at width 512.
    cap = 16 << 20
    def need(rows, n):
        it = itab((n,) * rows)
        st = stab((n,) * rows)
        return -(-ds.indexer_topk_workspace_bytes(it) // 256) * 256 + ds.attn_workspace_bytes(st)
    assert need(8, 897024) <= cap < need(8, 897024 + 1024)
    assert need(1, 13591552) <= cap < need(1, 13591552 + 1024)

# ------------------------------------------------------- indexer-row checks

@pytest.mark.parametrize("rows", [0, 9])
def test_rows_out_of_range(lib, rows):
    t = itab((10,) * 8)
    t.rows = rows
    msg = f"row table has rows = {rows}; a call takes 1 to 8 rows"
    expect_invalid(call_score(lib, t), msg)
    expect_invalid(call_topk(lib, t), msg)
    s = stab((10,) * 8)
    s.rows = rows
    expect_invalid(call_gather(lib, s), msg)
    expect_invalid(call_attn(lib, s), msg)


def test_indexer_row_checks(lib):
    expect_invalid(call_score(lib, itab((10, 0))), "indexer row 1: kv_len is 0")
    expect_invalid(call_score(lib, itab((10,), start_pos=[4 * 11 - 1])), "makes 11 keys visible but kv_len is only 10")
    expect_invalid(call_score(lib, itab((10,), start_pos=[0xFFFFFFFF])), "must be at most 2^32 - 2")
    expect_invalid(call_score(lib, itab((10,), offset=[-1])), "offset -1 is negative")
    expect_invalid(call_score(lib, itab((10,), offset=[2 ** 31 - 9])), "does not fit in int32")
    # offset + causal - 1 == INT32_MAX is allowed, one more is not
    assert ds.scores_elems(itab((10,), offset=[2 ** 31 - 9])) == 0
    assert ds.scores_elems(itab((10,), offset=[2 ** 31 - 10])) == 10
    # no visible key: any offset is fine
    assert ds.scores_elems(itab((10,), start_pos=[2], offset=[2 ** 31 - 1])) == 10
    expect_invalid(call_topk(lib, itab((10, 10), out_off=[0, 511])), "rows 0 and 1: their 512-index output ranges")
    expect_invalid(call_topk(lib, itab((10, 10, 10), out_off=[1024, 3000, 1100])), "rows 0 and 2")
    assert ds.scores_elems(itab((10, 10), out_off=[512, 0])) == 20


def test_kv_len_limit(lib):
    # The selection kernels address a row's 8-byte keys with 32-bit byte
    # offsets: kv_len must stay below 2^30, in every indexer entry point.
    top = 2 ** 30 - 1
    assert ds.scores_elems(itab((top,))) == top
    for n in (2 ** 30, 2 ** 32 - 1):
        t = itab((10, n))
        assert ds.scores_elems(t) == 0
        assert "indexer row 1: kv_len %d is above DS_KV_LEN_MAX = 2^30 - 1" % n in ds.last_error()
        expect_invalid(call_score(lib, t), "is above DS_KV_LEN_MAX")
        expect_invalid(call_topk(lib, t), "is above DS_KV_LEN_MAX")
        expect_invalid(call_fused(lib, t), "is above DS_KV_LEN_MAX")
        expect_invalid(call_mq(lib, itab((n,), start_pos=[8]), 2), "is above DS_KV_LEN_MAX")


def test_valid_call_without_a_device_enqueues_nothing(lib):
    # Arguments that pass every check reach the device check, which fails on
    # a host without a HIP device: DS_ERR_DEVICE, and no launch is attempted.
    t = itab((100,))
    assert call_score(lib, t) == DEVICE
    assert "HIP device" in ds.last_error()
    assert call_gather(lib, stab((100,))) == DEVICE


def test_fused_indexer_topk_checks(lib):
    t = itab((100, 50), q_row=[3, 0])
    need = ds.indexer_topk_workspace_bytes(t)
    expect_invalid(call_fused(lib, t, q=4 * 64 * 128 - 1), "indexer q holds")
    expect_invalid(call_fused(lib, t, w=4 * 64 - 1), "indexer weights holds")
    expect_invalid(call_fused(lib, t, s=2 * 100 - 1), "indexer scores holds")
    expect_invalid(call_fused(lib, t, ws=need - 1), "indexer top-k workspace holds")
    expect_invalid(call_fused(lib, t, wsp=None), "indexer top-k workspace must not be null")
    expect_invalid(call_fused(lib, itab((10, 10), out_off=[0, 1024]), idx=1535), "indexer output holds")
    expect_invalid(call_fused(lib, itab((10, 0))), "indexer row 1: kv_len is 0")
    expect_invalid(call_fused(lib, itab((10,), keys_elems=[10 * 128 - 1])), "indexer kv holds")
    expect_invalid(lib.ds_rows_indexer_candidates(ctypes.byref(t), FAKE, BIG, FAKE, BIG, FAKE, BIG, FAKE, need - 1,
                                                  None), "indexer top-k workspace holds")


def test_indexer_capacity_checks(lib):
    t = itab((100, 50), q_row=[3, 0])
    expect_invalid(call_score(lib, t, q=4 * 64 * 128 - 1), "indexer q holds")
    expect_invalid(call_score(lib, t, w=4 * 64 - 1), "indexer weights holds")
    expect_invalid(call_score(lib, t, s=2 * 100 - 1), "indexer scores holds")
    expect_invalid(call_score(lib, itab((100,), keys_elems=[100 * 128 - 1])), "indexer kv holds")
    expect_invalid(call_score(lib, t, qp=None), "must not be null")
    big = itab((40000,))
    expect_invalid(call_topk(lib, big, ws=ds.topk_workspace_bytes(big) - 1), "top-k scratch holds")
    expect_invalid(call_topk(lib, itab((10, 10), out_off=[0, 1024]), idx=1535), "indexer output holds")


# -------------------------------------------------------- sparse-row checks

def test_sparse_row_checks(lib):
    expect_invalid(call_gather(lib, stab((10, 0), width=(10, 1))), "sparse row 1: kv_len is 0")
    expect_invalid(call_gather(lib, stab((10, 10), width=(10, 0))), "sparse row 1: width is 0")
    expect_invalid(call_attn(lib, stab((10, 10), q_row=[2, 2])), "sparse rows 0 and 1 both use q_row 2")
    expect_invalid(call_attn(lib, stab((10, 10, 10), q_row=[4, 1, 4])), "sparse rows 0 and 2 both use q_row 4")
    expect_invalid(call_gather(lib, stab((10,), kv_elems=[10 * 512 - 1])), "kv holds")
    for bad in (float("nan"), float("inf"), 0.0, -1.0):
        expect_invalid(call_attn(lib, stab((10,)), scale=bad), "is not a finite value above 0")
    s = stab((10,))
    s.rows = 9
    expect_invalid(call_direct(lib, s), "row table has rows = 9")


def test_sparse_capacity_checks(lib):
    t = stab((600, 30), width=(512, 30), index_offset=(0, 4000), q_row=(1, 5))
    expect_invalid(call_gather(lib, t, idx=4029), "indices holds")
    expect_invalid(call_gather(lib, t, g=542 * 512 - 1), "gathered_kv holds")
    expect_invalid(call_gather(lib, t, m=541), "mask holds")
    expect_invalid(call_gather(lib, t, inv=1), "invalid holds 1 elements, needs 2")
    expect_invalid(call_gather(lib, t, invp=None), "invalid must not be null")
    expect_invalid(call_attn(lib, t, inv=1), "invalid holds 1 elements, needs 2")
    expect_invalid(call_attn(lib, t, invp=None), "invalid must not be null")
    expect_invalid(call_attn(lib, t, q=6 * 64 * 512 - 1), "q holds")
    expect_invalid(call_attn(lib, t, out=6 * 64 * 512 - 1), "output holds")
    expect_invalid(call_attn(lib, t, sinks=63), "sinks holds")
    expect_invalid(call_attn(lib, t, ws=ds.attn_workspace_bytes(t) - 1), "attention workspace holds")
    # the direct variant checks the KV capacities and indices like the gather
    expect_invalid(call_direct(lib, t, idx=4029), "indices holds")
    expect_invalid(call_direct(lib, stab((10,), kv_elems=[10 * 512 - 1])), "kv holds")
    expect_invalid(call_direct(lib, t, ws=ds.attn_workspace_bytes(t) - 1), "attention workspace holds")
    expect_invalid(call_direct(lib, t, scale=float("nan")), "scale nan is not a finite value above 0")
    expect_invalid(call_direct(lib, stab((10, 10), q_row=[1, 1])), "both use q_row 1")


def call_step(lib, it, st, q=BIG, w=BIG, s=BIG, ws=BIG, idx=BIG, aq=BIG, sinks=64, scale=0.0441941738, aws=BIG,
              out=BIG):
    return lib.ds_rows_indexer_topk_attn(ctypes.byref(it), ctypes.byref(st), FAKE, q, FAKE, w, FAKE, s, FAKE, ws,
                                         FAKE, idx, FAKE, aq, FAKE, sinks, ctypes.c_float(scale), FAKE, aws,
                                         FAKE, out, None)


def test_indexer_topk_attn_checks(lib):
    # the two tables must describe the same rows: count, width <= 512 and the
    # attention's index_offset equal to the indexer's output_offset
    it = itab((20000, 30000), out_off=(0, 512), q_row=(0, 1))
    st = stab((20000, 30000), width=(512, 512), index_offset=(0, 512), q_row=(0, 1))
    expect_invalid(call_step(lib, it, stab((20000,), width=(512,))), "the indexer table has 2 rows but the sparse table 1")
    expect_invalid(call_step(lib, it, stab((20000, 30000), width=(512, 513), index_offset=(0, 512), q_row=(0, 1))),
                   "sparse row 1: width 513 is above the 512 selected slots")
    expect_invalid(call_step(lib, it, stab((20000, 30000), width=(512, 512), index_offset=(0, 1024), q_row=(0, 1))),
                   "sparse row 1: index_offset 1024 differs from the indexer row's output_offset 512")
    # and the checks of both calls
    expect_invalid(call_step(lib, it, st, ws=ds.indexer_topk_workspace_bytes(it) - 1), "indexer top-k workspace holds")
    expect_invalid(call_step(lib, it, st, idx=1023), "indexer output holds")
    expect_invalid(call_step(lib, it, st, aws=ds.attn_workspace_bytes(st) - 1), "attention workspace holds")
    expect_invalid(call_step(lib, it, st, scale=float("inf")), "scale inf is not a finite value above 0")
    expect_invalid(call_step(lib, it, stab((20000, 30000), width=(512, 512), index_offset=(0, 512), q_row=(0, 1),
                                          kv_elems=[20000 * 512, 30000 * 512 - 1])), "kv holds")
    expect_invalid(call_step(lib, itab((20000, 30000), out_off=(0, 512), q_row=(0, 1), keys_elems=[1, 1]), st),
                   "kv holds")


def test_binding_rejects_host_tensors():
    import torch
    t = itab((10,))
    with pytest.raises(ValueError):
        ds.indexer_score(t, torch.zeros(64 * 128, dtype=torch.int16), torch.zeros(64),
                         torch.zeros(10))


# ---------------------------------------------------------------- compressor
# The conditions dispatch_deepseek_compressor_rows ("mlx-native 0.21.0
# src/ops/deepseek_rows.rs") requires: rows, supported shapes, epsilon,
# positions, state capacities, disjoint states, operand capacities.

def ctab(start_pos=(7,), ratio=4, head_dim=128, state_elems=None, kv_addr=None, sc_addr=None):
    R = len(start_pos)
    n = ds.compressor_state_elems(ratio, head_dim)
    stride = 0x1000000
    kv_addr = [FAKE + 2 * r * stride for r in range(R)] if kv_addr is None else kv_addr
    sc_addr = [FAKE + (2 * r + 1) * stride for r in range(R)] if sc_addr is None else sc_addr
    se = [n] * R if state_elems is None else state_elems
    return ds.compressor_rows(list(start_pos), kv_addr, sc_addr, se, se)


def call_comp(lib, t, ratio=4, head_dim=128, eps=1e-6, kv=BIG, score=BIG, ape=BIG, norm=BIG, out=BIG, outp=FAKE):
    return lib.ds_rows_compressor(ctypes.byref(t), ratio, head_dim, ctypes.c_float(eps), FAKE, kv, FAKE, score,
                                  FAKE, ape, FAKE, norm, outp, out, None)


def test_compressor_sizes(lib):
    assert ds.compressor_state_elems(4, 128) == 8 * 256
    assert ds.compressor_state_elems(4, 512) == 8 * 1024
    assert ds.compressor_state_elems(128, 512) == 128 * 512
    assert ds.compressor_state_elems(128, 128) == 0
    assert "compressor shape (ratio 128, head_dim 128) is unsupported" in ds.last_error()


def test_compressor_checks(lib):
    expect_invalid(call_comp(lib, ctab(), ratio=4, head_dim=256), "shape (ratio 4, head_dim 256) is unsupported")
    expect_invalid(call_comp(lib, ctab(), ratio=128, head_dim=128), "(ratio 128, head_dim 128)")
    for bad in (0.0, -1e-6, float("nan"), float("inf")):
        expect_invalid(call_comp(lib, ctab(), eps=bad), "compressor epsilon")
        assert "is not a finite value above 0" in ds.last_error()
    expect_invalid(call_comp(lib, ctab((7, 0))), "compressor row 1: start_pos 0 is outside [1, 2^32 - 2]")
    expect_invalid(call_comp(lib, ctab((0xFFFFFFFF,))), "start_pos 4294967295 is outside")
    t = ctab()
    t.rows = 9
    expect_invalid(call_comp(lib, t), "rows = 9")
    t.rows = 0
    expect_invalid(call_comp(lib, t), "rows = 0")
    expect_invalid(call_comp(lib, ctab(state_elems=[2047])), "kv_state holds 2047 elements, needs 2048")
    t = ctab()
    t.score_state_elems[0] = 100
    expect_invalid(call_comp(lib, t), "score_state holds")
    # states of different rows, or a row's two states, must not overlap
    expect_invalid(call_comp(lib, ctab((7, 11), kv_addr=[FAKE, FAKE + 4096],
                                       sc_addr=[FAKE + 0x1000000, FAKE + 0x2000000])),
                   "compressor state buffers 0 and 1 share memory")
    expect_invalid(call_comp(lib, ctab((7,), kv_addr=[FAKE], sc_addr=[FAKE + 2048 * 4 - 4])),
                   "state buffers 0 and 1 share memory")
    call_comp(lib, ctab((7,), kv_addr=[FAKE], sc_addr=[FAKE + 2048 * 4]), kv=0)   # adjacent is fine...
    assert "share memory" not in ds.last_error()                                   # ...it fails on kv
    t2 = ctab((7, 11))
    expect_invalid(call_comp(lib, t2, kv=2 * 256 - 1), "kv holds 511")
    expect_invalid(call_comp(lib, t2, score=2 * 256 - 1), "score holds")
    expect_invalid(call_comp(lib, t2, ape=4 * 256 - 1), "ape holds")
    expect_invalid(call_comp(lib, t2, norm=127), "norm holds")
    expect_invalid(call_comp(lib, t2, out=2 * 128 - 1), "output holds")
    expect_invalid(call_comp(lib, t2, outp=None), "output must not be null")
    t3 = ctab((127,), ratio=128, head_dim=512)
    expect_invalid(call_comp(lib, t3, ratio=128, head_dim=512, ape=128 * 512 - 1), "ape holds")


# ------------------------------------------------------- multi-query indexer

def call_mq(lib, t, Q, q=BIG, w=BIG, s=BIG):
    return lib.ds_rows_indexer_score_mq(ctypes.byref(t), Q, FAKE, q, FAKE, w, FAKE, s, None)


def test_mq_sizes_and_checks(lib):
    t = itab((100, 50), start_pos=[4 * 100 - 8, 4 * 50 - 8], q_row=[3, 0])
    assert ds.indexer_mq_scores_elems(t, 8) == 2 * 8 * 100
    assert ds.indexer_mq_scores_elems(t, 9) == 0
    assert "query_len 9 is outside [1, 8]" in ds.last_error()
    expect_invalid(call_mq(lib, t, 0), "query_len 0 is outside [1, 8]")
    # the last query (start_pos + 7) must still fit the cache
    expect_invalid(call_mq(lib, itab((100,), start_pos=[4 * 100 - 4]), 8),
                   "makes 101 keys visible but kv_len is only 100")
    expect_invalid(call_mq(lib, itab((100,), start_pos=[0xFFFFFFFF - 3]), 4), "is past 2^32 - 2")
    # queries q_row .. q_row + 7: max q_row 3 -> 11 query rows
    expect_invalid(call_mq(lib, t, 8, q=11 * 64 * 128 - 1), "indexer q holds")
    expect_invalid(call_mq(lib, t, 8, w=11 * 64 - 1), "indexer weights holds")
    expect_invalid(call_mq(lib, t, 8, s=2 * 8 * 100 - 1), "indexer scores holds")
    expect_invalid(call_mq(lib, itab((100,), start_pos=[392], keys_elems=[100 * 128 - 1]), 8), "indexer kv holds")
    # overlapping output offsets do not matter to the scores
    u = itab((10, 10), start_pos=[32, 32], out_off=[0, 0])
    expect_invalid(call_mq(lib, u, 8, s=2 * 8 * 10 - 1), "indexer scores holds")


def test_indexer_timer_needs_a_buffer(lib):
    """ds_rows_time_next_indexer only arms the next indexer launch (no device
    work): a null stamp buffer is an argument error in the library's words."""
    expect_invalid(lib.ds_rows_time_next_indexer(None, 0), "indexer timing stamps")
