"""CPU pins of the fp64 oracle (closed forms, library routines, exact
arithmetic), plus mutation tests showing that plausible mistakes fail them."""
import json
import os

import numpy as np
import pytest

import oracle as O
from synthetic import inputs as S
from tests import oracle_checks as C

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "page_constants.json")


# ------------------------------------------------------------- page constants

def test_page_constants():
    g = json.load(open(GOLDEN))
    assert O.LAMBDA == g["lambda"]["value"] == 35.0
    a1, a2, b1, b2 = S.IDENTITY_ALPHA
    assert a1 == b1 == g["alpha_init"]["alpha_1"]
    # alpha_2 = 1/lambda held in fp32: lambda * alpha_2 rounds to exactly 1 in fp32
    assert np.float32(np.float32(g["lambda"]["value"]) * np.float32(a2)) == np.float32(g["alpha_init"]["alpha_2_times_lambda"])
    assert len(S.IDENTITY_ALPHA) == g["scalars_per_layer"]["value"]


def test_fl32_inverse_lambda_facts():
    """fl32(1/35) = 0x3CEA0EA1; 35 * fl32(1/35) = 1 + 5.6e-9 in fp64 (rounds to 1 in fp32);
    a bf16 alpha would not give the identity (35 * bf16(1/35) != 1)."""
    inv = np.float32(1.0 / 35.0)
    assert inv.view(np.uint32) == 0x3CEA0EA1
    prod = 35.0 * float(inv)
    assert 0 < prod - 1.0 < 6e-9
    assert np.float32(prod) == np.float32(1.0)
    inv_bf16 = float(S.bf16_bits_to_f32(S.f32_to_bf16_bits(np.array([inv])))[0])
    assert abs(35.0 * inv_bf16 - 1.0) > 1e-4


# ------------------------------------------------------------- compose pins

@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_compose_identity_init(dtype):
    C.check_compose_identity(O.compose, dtype)


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_compose_mirror(dtype):
    C.check_compose_mirror(O.compose, dtype)


def test_compose_integer_closed_form():
    C.check_compose_integer_closed_form(O.compose)


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_compose_kv_weights(dtype):
    C.check_compose_kv_weights(O.compose_kv, dtype)


def test_compose_backward_finite_differences():
    C.check_compose_backward_finite_differences(O.compose_backward, O.compose_kv)


def test_compose_backward_identity_init():
    C.check_compose_backward_identity_init(O.compose_backward)


@pytest.mark.parametrize("kind", ["no_lambda", "swapped_grad", "v_uses_k_weights", "sign"])
def test_compose_backward_mutants_fail_a_pin(kind):
    def f(gk, gv, k1, ki, v1, vi, alpha, lam=35.0):
        g = O.compose_backward(gk, gv, k1, ki, v1, vi, alpha, lam)
        aK1, aK2, aV1, aV2 = alpha
        if kind == "no_lambda":
            g["dalpha"] = tuple(x / lam for x in g["dalpha"])
        elif kind == "swapped_grad":
            g["dk1"], g["dki"] = g["dki"], g["dk1"]
        elif kind == "v_uses_k_weights":
            g["dv1"] = lam * aK1 * O.to_f64(gv)
        elif kind == "sign":
            g["dalpha"] = (-g["dalpha"][0],) + tuple(g["dalpha"][1:])
        return g
    with pytest.raises(AssertionError):
        C.check_compose_backward_finite_differences(f, O.compose_kv)


def test_compose_magnitude_bounds():
    k1, ki = C._pair("f32", seed=5)
    a1, a2 = 0.031, -0.047
    assert np.all(O.compose_magnitude(k1, ki, a1, a2) >= np.abs(O.compose(k1, ki, a1, a2)))
    same = np.sign(k1) == -np.sign(ki)   # a1 > 0 > a2: these terms add with equal sign
    assert np.allclose(O.compose_magnitude(k1, ki, a1, a2)[same], np.abs(O.compose(k1, ki, a1, a2))[same],
                       rtol=1e-15, atol=0)


def test_bf16_nearest_matches_bit_rounding():
    """For fp32 inputs, fp64->bf16 rounding equals the bit-level fp32->bf16 RNE."""
    r = np.random.default_rng(7)
    x = np.concatenate([r.standard_normal(100000).astype(np.float32),
                        # exact midpoints between bf16 neighbours: ties go to even
                        S.bf16_bits_to_f32(np.arange(0x3F80, 0x3FA0, dtype=np.uint16)) * np.float32(1 + 2 ** -8)])
    want = S.bf16_bits_to_f32(S.f32_to_bf16_bits(x)).astype(np.float64)
    assert np.array_equal(O.bf16_nearest(x.astype(np.float64)), want)


def test_to_f64_bf16_widening():
    bits = np.array([0x3F80, 0xBF80, 0x4049, 0x0000, 0x8000, 0x7F7F], dtype=np.uint16)
    got = O.to_f64(bits)
    assert got[0] == 1.0 and got[1] == -1.0 and got[3] == 0.0
    assert got[2] == 3.140625
    assert got[5] == float(np.finfo(np.float32).max) - float(2 ** 104) * (2 ** 16 - 1) or got[5] > 3e38


# ------------------------------------------------------------- decode pins

@pytest.mark.parametrize("check", C.DECODE_CHECKS, ids=lambda f: f.__name__)
def test_decode_pins(check):
    check(O.decode_attention)


def test_decode_heads_subset():
    q, k, v = C._qkv(2, 4, 2, 20, 8, 9)
    full, lfull = O.decode_attention(q, k, v)
    sub, lsub = O.decode_attention(q, k, v, heads=[(1, 3), (0, 0)])
    # a 1-row product may round differently from a 2-row one inside BLAS
    assert np.allclose(sub[1, 3], full[1, 3], rtol=0, atol=1e-15)
    assert np.allclose(sub[0, 0], full[0, 0], rtol=0, atol=1e-15)
    assert np.isnan(sub[0, 1]).all()


def test_decode_bf16_inputs_widen_exactly():
    q, k, v = C._qkv(1, 4, 1, 30, 8, 10)
    kb = S.f32_to_bf16_bits(k.astype(np.float32))
    vb = S.f32_to_bf16_bits(v.astype(np.float32))
    o1, l1 = O.decode_attention(q, kb, vb)
    o2, l2 = O.decode_attention(q, S.bf16_bits_to_f32(kb), S.bf16_bits_to_f32(vb))
    assert np.array_equal(o1, o2) and np.array_equal(l1, l2)


def test_decode_key_block_streaming(monkeypatch):
    """Streaming over key blocks (memory only) gives the single-block result."""
    from oracle import yoco_oracle as Y
    q, k, v = C._qkv(1, 8, 2, 300, 16, 8)
    o1, l1 = O.decode_attention(q, k, v)
    monkeypatch.setattr(Y, "KEY_BLOCK", 7)
    o2, l2 = O.decode_attention(q, k, v)
    assert np.allclose(o1, o2, rtol=0, atol=1e-14) and np.allclose(l1, l2, rtol=0, atol=1e-13)


# ------------------------------------------------------------- prefill pins

@pytest.mark.parametrize("check", C.PREFILL_CHECKS, ids=lambda f: f.__name__)
def test_prefill_pins(check):
    check(O.causal_prefill)


def test_prefill_row_is_decode():
    C.check_prefill_row_is_decode(O.causal_prefill, O.decode_attention)


def test_prefill_row_subset():
    q, k, v = C._prefill_inputs(1, 20, 4, 2, 25, 8, 48)
    full, lf = O.causal_prefill(q, k, v, 3)
    sub, ls = O.causal_prefill(q, k, v, 3, rows=[0, 19, 7])
    for r in (0, 7, 19):
        assert np.allclose(sub[:, r], full[:, r], rtol=0, atol=1e-14)
        assert np.allclose(ls[:, :, r], lf[:, :, r], rtol=0, atol=1e-14)
    assert np.isnan(sub[:, 1]).all()


def test_prefill_rejects_overflowing_chunk():
    q, k, v = C._prefill_inputs(1, 8, 2, 1, 10, 8, 49)
    with pytest.raises(ValueError):
        O.causal_prefill(q, k, v, 3)


# ------------------------------------------------------------- mutation tests
# Plausible mistakes, planted in small copies of the definitions (CPU only).

def _mut_compose(kind):
    def f(x1, xi, a1, a2, lam=35.0):
        x1, xi = O.to_f64(x1), O.to_f64(xi)
        if kind == "no_lambda":
            return a1 * x1 + a2 * xi
        if kind == "swapped_weights":
            return lam * (a2 * x1 + a1 * xi)
        if kind == "minus":
            return lam * (a1 * x1 - a2 * xi)
        if kind == "lambda_outside_second":
            return lam * a1 * x1 + a2 * xi
        raise AssertionError(kind)
    return f


def _mut_compose_kv(kind):
    def f(k1, ki, v1, vi, alpha, lam=35.0):
        aK1, aK2, aV1, aV2 = alpha
        if kind == "v_uses_k_weights":
            return O.compose(k1, ki, aK1, aK2, lam), O.compose(v1, vi, aK1, aK2, lam)
        if kind == "swapped_pairs":
            return O.compose(k1, ki, aK1, aV1, lam), O.compose(v1, vi, aK2, aV2, lam)
        raise AssertionError(kind)
    return f


def _mut_decode(kind):
    def f(q, k, v, seq_lens=None, scale=None):
        q, k64, v64 = O.to_f64(q), O.to_f64(k), O.to_f64(v)
        B, Hq, D = q.shape
        Hkv, T = k.shape[1], k.shape[2]
        G = Hq // Hkv
        o = np.empty((B, Hq, D))
        lse = np.empty((B, Hq))
        for b in range(B):
            n = T if seq_lens is None else int(seq_lens[b])
            if kind == "drop_last_row":
                n = max(1, n - 1)
            for h in range(Hq):
                g = h % Hkv if kind == "gqa_modulo" else h // G
                sc = 1.0 / D if kind == "scale_1_over_D" else 1.0 / np.sqrt(D)
                s = sc * (k64[b, g, :n] @ q[b, h])
                if kind == "no_scale":
                    s = k64[b, g, :n] @ q[b, h]
                m = s.max()
                p = np.exp(s - m)
                o[b, h] = p @ v64[b, g, :n] / p.sum()
                lse[b, h] = (m + np.log(p.sum())) / (np.log(2) if kind == "lse_log2" else 1.0)
                if kind == "lse_without_max":
                    lse[b, h] = np.log(p.sum())
        return o, lse
    return f


def _mut_prefill(kind):
    def f(q, k, v, p0, scale=None, rows=None):
        q = O.to_f64(q)
        B, C_, Hq, D = q.shape
        G = Hq // k.shape[1]
        o = np.empty((B, C_, Hq, D))
        lse = np.empty((B, Hq, C_))
        for b in range(B):
            for c in range(C_):
                pos = c if kind == "ignore_p0" else p0 + c
                n = pos if kind == "exclusive_diagonal" else pos + 1
                n = max(n, 1) if kind != "exclusive_diagonal" else n
                for h in range(Hq):
                    if n == 0:
                        o[b, c, h] = 0.0
                        lse[b, h, c] = -np.inf
                        continue
                    kk, vv = O.to_f64(k[b, h // G, :n]), O.to_f64(v[b, h // G, :n])
                    s = kk @ q[b, c, h] / np.sqrt(D)
                    p = np.exp(s - s.max())
                    o[b, c, h] = p @ vv / p.sum()
                    lse[b, h, c] = s.max() + np.log(p.sum())
        return o, lse
    return f


COMPOSE_CHECKS = [lambda f: C.check_compose_identity(f, "f32"), lambda f: C.check_compose_mirror(f, "f32"),
                  C.check_compose_integer_closed_form]


@pytest.mark.parametrize("kind", ["no_lambda", "swapped_weights", "minus", "lambda_outside_second"])
def test_compose_mutants_fail_a_pin(kind):
    f = _mut_compose(kind)
    failed = 0
    for chk in COMPOSE_CHECKS:
        try:
            chk(f)
        except AssertionError:
            failed += 1
    assert failed >= 1


@pytest.mark.parametrize("kind", ["v_uses_k_weights", "swapped_pairs"])
def test_compose_kv_mutants_fail_a_pin(kind):
    with pytest.raises(AssertionError):
        C.check_compose_kv_weights(_mut_compose_kv(kind), "f32")


@pytest.mark.parametrize("kind", ["gqa_modulo", "scale_1_over_D", "no_scale", "drop_last_row", "lse_log2",
                                  "lse_without_max"])
def test_decode_mutants_fail_a_pin(kind):
    f = _mut_decode(kind)
    failed = 0
    for chk in C.DECODE_CHECKS:
        try:
            chk(f)
        except AssertionError:
            failed += 1
    assert failed >= 1


def test_decode_unmutated_copy_passes():
    """The mutation harness itself is sound: the unbroken copy passes every check."""
    f = _mut_decode("none")
    for chk in C.DECODE_CHECKS:
        chk(f)


@pytest.mark.parametrize("kind", ["exclusive_diagonal", "ignore_p0"])
def test_prefill_mutants_fail_a_pin(kind):
    f = _mut_prefill(kind)
    failed = 0
    for chk in C.PREFILL_CHECKS:
        try:
            chk(f)
        except (AssertionError, FloatingPointError):
            failed += 1
    assert failed >= 1


def test_prefill_unmutated_copy_passes():
    f = _mut_prefill("none")
    for chk in C.PREFILL_CHECKS:
        chk(f)


def test_self_decode_pins():
    for chk in C.SELF_DECODE_CHECKS:
        chk(O.self_attn_decode)


def test_self_decode_default_lambda_and_lengths():
    """lambda defaults to 35; seq_lens None means every row; lengths outside [1, T] are rejected."""
    q, k, v, new = C._self_inputs(1, 2, 1, 6, 8, 44)
    inv = S.fl32(1 / 35)
    o, _, kn, _ = O.self_attn_decode(q, k, v, new, (0.0, inv, 0.0, inv))
    assert np.allclose(kn, new["ki"], rtol=1e-8, atol=0)
    o2, _, _, _ = O.self_attn_decode(q, k, v, new, (0.0, inv, 0.0, inv), seq_lens=np.array([6]))
    assert np.array_equal(o, o2)
    with pytest.raises(ValueError):
        O.self_attn_decode(q, k, v, new, (0.0, inv, 0.0, inv), seq_lens=np.array([7]))


def _mut_self_decode(kind):
    def f(q, k, v, new, alpha, seq_lens=None, scale=None, lam=35.0):
        aK1, aK2, aV1, aV2 = alpha
        if kind == "sources_swapped":
            new = {"k1": new["ki"], "ki": new["k1"], "v1": new["vi"], "vi": new["v1"]}
        if kind == "v_uses_k_weights":
            aV1, aV2 = aK1, aK2
        kn = lam * (aK1 * O.to_f64(new["k1"]) + aK2 * O.to_f64(new["ki"]))
        vn = lam * (aV1 * O.to_f64(new["v1"]) + aV2 * O.to_f64(new["vi"]))
        B, Hq, D = q.shape
        Hkv, T = k.shape[1], k.shape[2]
        G = Hq // Hkv
        o, lse = np.empty((B, Hq, D)), np.empty((B, Hq))
        for b in range(B):
            n = T if seq_lens is None else int(seq_lens[b])
            for h in range(Hq):
                g = h // G
                if kind == "new_row_from_cache":
                    keys, vals = O.to_f64(k[b, g, :n]), O.to_f64(v[b, g, :n])
                elif kind == "appended_after_n":
                    keys = np.concatenate([O.to_f64(k[b, g, :n]), kn[b, g][None]])
                    vals = np.concatenate([O.to_f64(v[b, g, :n]), vn[b, g][None]])
                else:
                    keys = np.concatenate([O.to_f64(k[b, g, :n - 1]), kn[b, g][None]])
                    vals = np.concatenate([O.to_f64(v[b, g, :n - 1]), vn[b, g][None]])
                s = keys @ O.to_f64(q[b, h]) / np.sqrt(D)
                m = s.max()
                p = np.exp(s - m)
                o[b, h] = p @ vals / p.sum()
                lse[b, h] = m + np.log(p.sum())
        return o, lse, kn, vn
    return f


@pytest.mark.parametrize("kind", ["sources_swapped", "v_uses_k_weights", "new_row_from_cache", "appended_after_n"])
def test_self_decode_mutants_fail_a_pin(kind):
    f = _mut_self_decode(kind)
    failed = 0
    for chk in C.SELF_DECODE_CHECKS:
        try:
            chk(f)
        except AssertionError:
            failed += 1
    assert failed >= 1


def test_self_decode_unmutated_copy_passes():
    f = _mut_self_decode("none")
    for chk in C.SELF_DECODE_CHECKS:
        chk(f)
