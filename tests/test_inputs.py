"""The seeded input generator: determinism, shapes and value recipes (CPU)."""
import numpy as np
import torch

from sparse_attention_decode_04_amd import inputs as I


def test_bf16_rounding_matches_torch():
    x = np.random.default_rng(3).standard_normal(1 << 16).astype(np.float32) * 37
    ref = torch.from_numpy(x).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    np.testing.assert_array_equal(I.f32_to_bf16_bits(x), ref)


def test_config0_recipe_and_determinism():
    a = I.make_config(0)
    b = I.make_config(0)
    assert a.kv_len == [1024] and a.start_pos == [4095] and a.offset == [0]
    for f in ("idx_q", "idx_w", "attn_q", "sinks"):
        np.testing.assert_array_equal(getattr(a, f), getattr(b, f))
    np.testing.assert_array_equal(a.idx_keys[0], b.idx_keys[0])
    np.testing.assert_array_equal(a.kv[0], b.kv[0])
    assert a.idx_q.shape == (1, 64, 128) and a.idx_keys[0].shape == (1024, 128)
    assert a.attn_q.shape == (1, 64, 512) and a.kv[0].shape == (1024, 512)
    qv = torch.from_numpy(a.idx_q.view(np.int16)).view(torch.bfloat16).float().numpy()
    assert np.all(qv == np.round(qv)) and qv.min() == -4 and qv.max() == 4
    assert set(np.unique(a.idx_w)) <= {-2, -1, 0, 1, 2}
    kv = torch.from_numpy(a.kv[0].view(np.int16)).view(torch.bfloat16).float().numpy()
    assert abs(kv.mean()) < 0.01 and abs(kv.std() - 1) < 0.01
    assert a.scale == float(np.float32(1 / np.sqrt(512)))


def test_config1_ragged_and_config3_ternary():
    c1 = I.make_config(1)
    assert len(c1.kv_len) == 8 and all(600 <= n <= 8192 for n in c1.kv_len)
    assert len(set(c1.kv_len)) > 1
    c3 = I.small_rows(9, [33, 70], ternary=True)
    v = torch.from_numpy(c3.idx_keys[1].view(np.int16)).view(torch.bfloat16).float().numpy()
    assert set(np.unique(v)) == {-1.0, 0.0, 1.0}
    assert I.config_kv_lens(3) == [1, 37, 511, 512, 513, 4096, 65536, 131072]
