"""Seeded generator: determinism, prefix consistency across chunks, planted scaling."""
import numpy as np

import workloads as W


def test_generator_is_deterministic_and_prefix_consistent():
    w = W.C3_7B_CHUNK_128K.scaled(h_q=4, h_kv=1, chunks=((4096, 1024),))
    k1, v1 = W.make_keys_values(w, 9000, seed=0)
    k2, v2 = W.make_keys_values(w, 5120, seed=0)
    assert np.array_equal(k1[:5120], k2) and np.array_equal(v1[:5120], v2)
    k3, _ = W.make_keys_values(w, 5120, seed=1)
    assert not np.array_equal(k2, k3)
    a = W.make(w, 0, seed=0)
    b = W.make(w, 0, seed=0)
    assert all(np.array_equal(a[x], b[x]) for x in ("q", "k", "v", "positions"))
    assert a["positions"][0] == 4096 and a["positions"][-1] == 5119 and a["n_k"] == 5120


def test_sinks_and_periodic_rows_are_scaled_exactly():
    w = W.C3_7B_CHUNK_128K.scaled(h_q=4, h_kv=1)
    base = W.C3_7B_CHUNK_128K.scaled(h_q=4, h_kv=1, sinks=False, periodic=False)
    k, _ = W.make_keys_values(w, 8200, seed=0)
    k0, _ = W.make_keys_values(base, 8200, seed=0)
    f, f0 = W.bf16_bits_to_f32(k), W.bf16_bits_to_f32(k0)
    assert np.array_equal(f[:4], 8 * f0[:4])
    assert np.array_equal(f[4096], 4 * f0[4096]) and np.array_equal(f[8192], 4 * f0[8192])
    assert np.array_equal(f[4:4096], f0[4:4096]) and np.array_equal(f[0 + 5000], f0[5000])


def test_sample_blocks_cover_first_mid_last():
    pairs = W.sample_blocks(32768, 2, seed=0)
    for h in range(2):
        bs = [b for hh, b in pairs if hh == h]
        assert {0, 1, 256, 511} <= set(bs)
