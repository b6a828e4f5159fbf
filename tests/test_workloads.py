"""The seeded input generators: determinism, row-range slicing, shard layout, documents."""
import numpy as np

import workloads as W


def test_rows_regenerate_exactly():
    cfg = W.WORKLOADS["qwen_8k"]
    full = W.gen_rows(cfg, "k", 0, 9000)
    part = W.gen_rows(cfg, "k", 4000, 8200)
    np.testing.assert_array_equal(full[4000:8200], part)
    np.testing.assert_array_equal(W.gen_rows(cfg, "k", 4000, 8200), part)


def test_f32_amplitude_and_bits():
    cfg = W.WORKLOADS["tiny_f32"]
    q = W.gen_global(cfg, "q")
    assert q.dtype == np.uint32 and q.shape == (512, 4, 64)
    x = W.bits_to_f64(q, "f32")
    assert 0.4 < x.std() < 0.6
    do = W.bits_to_f64(W.gen_global(cfg, "do"), "f32")
    assert 0.9 < do.std() < 1.1


def test_bf16_is_round_to_nearest_even():
    x = np.array([1.0, 1.00390625, 1.005859375, -2.0, 3.0e-3], dtype=np.float32)
    bits = W.to_bf16_bits(x)
    # 1 + 2^-8 is a tie between 1 and 1 + 2^-7: even mantissa -> 1.0
    assert bits[1] == 0x3F80
    # 1 + 1.5 * 2^-8 rounds up to 1 + 2^-7
    assert bits[2] == 0x3F81
    np.testing.assert_array_equal(W.bits_to_f64(bits[[0, 3]], "bf16"), [1.0, -2.0])


def test_shards_are_contiguous_chunks():
    g = np.arange(8 * 2 * 1).reshape(8, 2, 1)
    sh = W.shards_of(g, 4)
    assert [s[0, 0, 0] for s in sh] == [0, 4, 8, 12]
    np.testing.assert_array_equal(W.head_slice(g, 2, 1), g[:, 1:2])


def test_documents_cover_the_sequence():
    cfg = W.WORKLOADS["packed_96k"]
    cu = W.cu_seqlens_for(cfg)
    assert cu[0] == 0 and cu[-1] == cfg.s and (np.diff(cu) >= 1).all()
    np.testing.assert_array_equal(cu, W.cu_seqlens_for(cfg))
    lens = np.diff(cu)[:-1]
    assert 2000 < lens.mean() < 20000


def test_packed_seed0_instance():
    """The seed-0 packed 96K instance: 11 documents, the last truncated, about a fifth of
    the dense-causal pair count."""
    cu = W.cu_seqlens_for(W.WORKLOADS["packed_96k"])
    assert list(cu) == [0, 4080, 10198, 10317, 10331, 13633, 23412, 27454, 31986, 48886, 85230, 98304]
    lens = np.diff(cu).astype(np.int64)
    assert int((lens ** 2).sum()) == 1974925326


def test_config_shapes():
    c = W.WORKLOADS["qwen_64k"]
    assert (c.s, c.Hq_l, c.Hkv_l, c.G, c.d) == (65536, 8, 2, 4, 128)
    c = W.WORKLOADS["upipe_256k"]
    assert (c.s, c.Hq_l, c.Hkv_l, c.G) == (262144, 8, 1, 8)
