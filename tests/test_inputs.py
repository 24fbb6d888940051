"""Seeded generators: bf16 rounding, reproducibility, mask recipe."""
import numpy as np

import lsh_inputs as I


def test_bf16_round_to_nearest_even_bit_patterns():
    # (float32 bits, expected bf16 bits), worked by hand:
    cases = [
        (0x3F800000, 0x3F80),  # 1.0 exact
        (0x3F808000, 0x3F80),  # halfway, lower bf16 even -> round down
        (0x3F818000, 0x3F82),  # halfway, lower bf16 odd -> round up to even
        (0x3F808001, 0x3F81),  # just above halfway -> up
        (0x3F807FFF, 0x3F80),  # just below halfway -> down
        (0xBF808000, 0xBF80),  # negative halfway, even
        (0xBF818000, 0xBF82),  # negative halfway, odd
        (0x7F7FFFFF, 0x7F80),  # max float rounds to +inf in bf16
        (0x00000000, 0x0000),
        (0x80000000, 0x8000),
        (0x3FFFFFFF, 0x4000),  # carry into the exponent
    ]
    f = np.array([c[0] for c in cases], dtype=np.uint32).view(np.float32)
    got = I.bf16_bits(f)
    assert got.tolist() == [c[1] for c in cases]


def test_bf16_values_exact_and_nearest():
    x = I.standard_normal_f32((4096,), 1, 0)
    b = I.bf16_bits(x)
    y = I.bf16_bits_to_f32(b)
    # y is a bf16 value: low 16 bits zero
    assert np.all((y.view(np.uint32) & 0xFFFF) == 0)
    # nearest: neighbouring bf16 values are no closer
    up = I.bf16_bits_to_f32(b + 1)
    dn = I.bf16_bits_to_f32(b - 1)
    err = np.abs(y.astype(np.float64) - x)
    assert np.all(err <= np.abs(up.astype(np.float64) - x))
    assert np.all(err <= np.abs(dn.astype(np.float64) - x))


def test_seeded_reproducible_and_independent():
    w = I.WORKLOADS[1]
    q1, k1, v1 = I.make_qkv(w, seed=0, Sq=8, Skv=8)
    q2, k2, v2 = I.make_qkv(w, seed=0, Sq=8, Skv=8)
    assert np.array_equal(q1.values, q2.values) and np.array_equal(v1.values, v2.values)
    assert not np.array_equal(q1.values, k1.values)
    q3, _, _ = I.make_qkv(w, seed=1, Sq=8, Skv=8)
    assert not np.array_equal(q1.values, q3.values)


def test_bf16_workload_tensor():
    w = I.WORKLOADS[4]
    q, k, v = I.make_qkv(w, seed=0, Sq=16, Skv=16)
    assert q.bits.dtype == np.uint16 and q.bits.shape == (1, 16, 40, 128)
    assert np.array_equal(I.bf16_bits_to_f32(q.bits), q.values)


def test_block_mask_recipe():
    mask, dens = I.make_block_mask(1, 40, 256, 256, seed=0)
    assert mask.shape == (1, 40, 256, 256) and mask.dtype == np.uint8
    assert set(np.unique(mask)) <= {0, 1}
    for h in range(40):
        m = mask[0, h]
        assert np.all(np.diag(m) == 1), "diagonal kept"
        n = int(m.sum())
        assert abs(n / 65536 - dens[h]) < 1e-12
        assert 0.1 - 1e-6 <= dens[h] <= 0.6 + 1e-6
    assert dens.std() > 0.05, "densities vary across heads"
    mask2, dens2 = I.make_block_mask(1, 40, 256, 256, seed=0)
    assert np.array_equal(mask, mask2) and np.array_equal(dens, dens2)


def test_sample_rows_has_tail_tile():
    rows = I.sample_rows(56160, 300, seed=0)
    assert rows[0] == 0 and rows[-1] == 56159
    assert set(range(56064, 56160)) <= set(rows.tolist())
    assert np.all(np.diff(rows) > 0)
    assert rows.size >= 300
