"""The seeded input generator: determinism, block independence, bf16 rounding."""
import numpy as np

from synthetic import inputs as S


def test_normal_is_deterministic_and_thread_independent(monkeypatch):
    a = S.normal_f32(123, (5, 0), (3, S.BLOCK + 17))
    monkeypatch.setattr(S, "_threads", lambda: 1)
    b = S.normal_f32(123, (5, 0), (3, S.BLOCK + 17))
    assert np.array_equal(a, b)
    c = S.normal_f32(123, (5, 1), (3, S.BLOCK + 17))
    assert not np.array_equal(a, c)


def test_normal_moments():
    x = S.normal_f32(7, (1, 0), (1 << 20,), std=0.5)
    assert abs(x.mean()) < 3e-3 and abs(x.std() - 0.5) < 3e-3


def test_bf16_rounding_ties_to_even():
    # 1 + 2^-8 lies halfway between 1 and 1 + 2^-7: ties to even -> 1.0
    x = np.array([1 + 2 ** -8, 1 + 3 * 2 ** -8, -(1 + 2 ** -8), 1 + 2 ** -8 + 2 ** -20], dtype=np.float32)
    got = S.bf16_bits_to_f32(S.f32_to_bf16_bits(x))
    assert got.tolist() == [1.0, 1 + 2 ** -6, -1.0, 1 + 2 ** -7]


def test_bf16_rounding_error_bound():
    x = np.random.default_rng(0).standard_normal(1 << 18).astype(np.float32)
    y = S.bf16_bits_to_f32(S.f32_to_bf16_bits(x))
    assert np.all(np.abs(y - x) <= np.abs(x) * 2.0 ** -8)


def test_scaled_rows_and_plant_are_exact():
    w = S.DECODE_LONG
    T = 4096
    rows = S.scaled_rows(w, T)
    assert rows.shape == (w.B, int(round(0.01 * T)))
    k = S.normal_bf16(1, (0, 0), (w.B, 2, T, 8))
    k0 = k.copy()
    S.scale_key_rows_bf16(k, rows, 8.0)
    f0, f1 = S.bf16_bits_to_f32(k0), S.bf16_bits_to_f32(k)
    for b in range(w.B):
        assert np.array_equal(f1[b][:, rows[b]], 8.0 * f0[b][:, rows[b]])
        mask = np.ones(T, bool)
        mask[rows[b]] = False
        assert np.array_equal(f1[b][:, mask], f0[b][:, mask])
    q = S.normal_bf16(2, (0, 0), (1, 8, 8))
    kk = S.normal_bf16(3, (0, 0), (1, 2, 64, 8))
    S.plant_query_row_bf16(kk, q, 17, 4.0)
    assert np.array_equal(S.bf16_bits_to_f32(kk[0, 1, 17]), 4.0 * S.bf16_bits_to_f32(q[0, 4]))


def test_identity_alpha_is_fp32():
    assert S.IDENTITY_ALPHA[1] == float(np.float32(1 / 35))
    assert S.IDENTITY_ALPHA[0] == 0.0
