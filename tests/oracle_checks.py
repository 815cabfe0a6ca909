"""Pins for the fp64 oracle: checks against closed forms, library routines and
exact arithmetic, written as functions of the implementation under test.

Each check raises AssertionError when the implementation disagrees with what
the pages and the mathematics fix. The oracle must pass all of them; the
mutation tests run the same checks on deliberately broken variants (a dropped
lambda, swapped weights, a wrong GQA map, a wrong scale, an off-by-one mask,
a log2 lse) and require that some check fails for each.

Sources: YOCO++ technical summary, section 2 (KV composition equations;
key technical innovations items 2-3: lambda = 35, initialisation
alpha_1 = 0, alpha_2 = 1/lambda); YOCO summary, abstract (cross-decoder
reuses the global cache; end to end it works as a decoder-only Transformer
does; early exit leaves the output unchanged).
"""
from __future__ import annotations

from decimal import Decimal, getcontext

import numpy as np
import torch

from synthetic import inputs as S

LAM = 35.0
INV_LAM32 = S.fl32(1.0 / LAM)


def _rng(seed):
    return np.random.default_rng(seed)


def _f64(x):
    x = np.asarray(x)
    if x.dtype == np.uint16:
        return S.bf16_bits_to_f32(x).astype(np.float64)
    return x.astype(np.float64)


# ----------------------------------------------------------------- compose

def _pair(dtype, shape=(2, 19, 3, 64), seed=11):
    r = _rng(seed)
    a = r.standard_normal(shape).astype(np.float32)
    b = r.standard_normal(shape).astype(np.float32)
    if dtype == "bf16":
        return S.f32_to_bf16_bits(a), S.f32_to_bf16_bits(b)
    return a, b


def check_compose_identity(compose_fn, dtype="f32"):
    """Init alpha_1 = 0, alpha_2 = fl32(1/35): stored K'_i must equal K_i exactly."""
    k1, ki = _pair(dtype)
    r = np.asarray(compose_fn(k1, ki, 0.0, INV_LAM32), dtype=np.float64)
    want = _f64(ki)
    # fp64 value is K_i * 35 * fl32(1/35) = K_i * (1 + 5.6e-9): below half an
    # fp32 ulp, so the stored value rounds back to K_i.
    nz = want != 0
    assert np.all(np.abs(r[nz] / want[nz] - 1.0) < 1e-8)
    if dtype == "f32":
        assert np.array_equal(r.astype(np.float32), ki)
    else:
        assert np.array_equal(S.f32_to_bf16_bits(r.astype(np.float32)), ki)


def check_compose_mirror(compose_fn, dtype="f32"):
    """alpha_1 = fl32(1/35), alpha_2 = 0 stores layer 1's tensor."""
    k1, ki = _pair(dtype, seed=12)
    r = np.asarray(compose_fn(k1, ki, INV_LAM32, 0.0), dtype=np.float64)
    if dtype == "f32":
        assert np.array_equal(r.astype(np.float32), k1)
    else:
        assert np.array_equal(S.f32_to_bf16_bits(r.astype(np.float32)), k1)


def check_compose_integer_closed_form(compose_fn):
    """lam = 2, a1 = 1.5, a2 = -0.25 on small integers: exactly 3*X1 - 0.5*Xi."""
    r = _rng(13)
    x1 = r.integers(-8, 9, size=(1, 7, 2, 8)).astype(np.float32)
    xi = r.integers(-8, 9, size=(1, 7, 2, 8)).astype(np.float32)
    got = np.asarray(compose_fn(x1, xi, 1.5, -0.25, 2.0), dtype=np.float64)
    assert np.array_equal(got, 3.0 * x1.astype(np.float64) - 0.5 * xi.astype(np.float64))
    # and with the page's lambda: 35 * (0.5 * X1 + 0.25 * Xi) = 17.5 X1 + 8.75 Xi exactly
    got = np.asarray(compose_fn(x1, xi, 0.5, 0.25), dtype=np.float64)
    assert np.array_equal(got, 17.5 * x1.astype(np.float64) + 8.75 * xi.astype(np.float64))


def check_compose_kv_weights(compose_kv_fn, dtype="f32"):
    """Key weights act on K, value weights on V: K identity + V mirror in one call."""
    k1, ki = _pair(dtype, seed=14)
    v1, vi = _pair(dtype, seed=15)
    ident, mirror = (0.0, INV_LAM32), (INV_LAM32, 0.0)
    for ka, kw in ((ident, ki), (mirror, k1)):
        for va, vw in ((ident, vi), (mirror, v1)):
            kp, vp = compose_kv_fn(k1, ki, v1, vi, ka + va)
            if dtype == "f32":
                assert np.array_equal(np.asarray(kp).astype(np.float32), kw)
                assert np.array_equal(np.asarray(vp).astype(np.float32), vw)
            else:
                assert np.array_equal(S.f32_to_bf16_bits(np.asarray(kp).astype(np.float32)), kw)
                assert np.array_equal(S.f32_to_bf16_bits(np.asarray(vp).astype(np.float32)), vw)


# ----------------------------------------------------------------- compose backward

def _loss(compose_kv_fn, gk, gv, k1, ki, v1, vi, alpha, lam=35.0):
    kp, vp = compose_kv_fn(k1, ki, v1, vi, alpha, lam)
    return float(np.sum(gk * kp) + np.sum(gv * vp))


def check_compose_backward_finite_differences(backward_fn, compose_kv_fn):
    """The composition is linear in the weights and in the sources, so central
    differences of L = <gk, K'> + <gv, V'> give the exact gradient up to rounding."""
    r = _rng(16)
    shp = (2, 5, 3, 8)
    gk, gv, k1, ki, v1, vi = (r.standard_normal(shp) for _ in range(6))
    alpha = (0.013, -0.021, 0.034, 0.007)
    g = backward_fn(gk, gv, k1, ki, v1, vi, alpha)
    h = 0.5
    for idx in range(4):
        ap, am = list(alpha), list(alpha)
        ap[idx] += h
        am[idx] -= h
        fd = (_loss(compose_kv_fn, gk, gv, k1, ki, v1, vi, ap) - _loss(compose_kv_fn, gk, gv, k1, ki, v1, vi, am)) / (2 * h)
        assert abs(g["dalpha"][idx] - fd) <= 1e-10 * max(1.0, abs(fd))
    for name, arr in (("dk1", k1), ("dki", ki), ("dv1", v1), ("dvi", vi)):
        for flat in (0, 37, arr.size - 1):
            pert = np.zeros(arr.size)
            pert[flat] = h
            pert = pert.reshape(arr.shape)
            args = dict(k1=k1, ki=ki, v1=v1, vi=vi)
            key = {"dk1": "k1", "dki": "ki", "dv1": "v1", "dvi": "vi"}[name]
            lp = _loss(compose_kv_fn, gk, gv, **{**args, key: arr + pert}, alpha=alpha)
            lm = _loss(compose_kv_fn, gk, gv, **{**args, key: arr - pert}, alpha=alpha)
            fd = (lp - lm) / (2 * h)
            assert abs(g[name].reshape(-1)[flat] - fd) <= 1e-10 * max(1.0, abs(fd))


def check_compose_backward_identity_init(backward_fn):
    """At a1 = 0 the layer-1 tensors get no gradient; a2 = fl32(1/35) passes gk through."""
    r = _rng(17)
    gk, gv, k1, ki, v1, vi = (r.standard_normal((1, 4, 2, 8)) for _ in range(6))
    g = backward_fn(gk, gv, k1, ki, v1, vi, S.IDENTITY_ALPHA)
    assert np.array_equal(g["dk1"], np.zeros_like(gk)) and np.array_equal(g["dv1"], np.zeros_like(gv))
    assert np.allclose(g["dki"], gk, rtol=1e-8, atol=0) and np.allclose(g["dvi"], gv, rtol=1e-8, atol=0)


# ----------------------------------------------------------------- decode

def _qkv(B, Hq, Hkv, T, D, seed):
    r = _rng(seed)
    q = r.standard_normal((B, Hq, D))
    k = r.standard_normal((B, Hkv, T, D))
    v = r.standard_normal((B, Hkv, T, D))
    return q, k, v


def check_decode_identical_keys(decode_fn):
    """All keys equal: weights are uniform, o = mean_t V, lse = s + ln T."""
    B, Hq, Hkv, T, D = 2, 4, 2, 37, 8
    q, k, v = _qkv(B, Hq, Hkv, T, D, 21)
    k[:] = k[:, :, :1, :]
    o, lse = decode_fn(q, k, v)
    G = Hq // Hkv
    for b in range(B):
        for h in range(Hq):
            g = h // G
            assert np.allclose(o[b, h], v[b, g].mean(axis=0), rtol=0, atol=1e-13)
            s = (q[b, h] @ k[b, g, 0]) / np.sqrt(D)
            assert abs(lse[b, h] - (s + np.log(T))) < 1e-12


def check_decode_single_token(decode_fn):
    """T = 1: o = V[0] exactly, lse = the single score."""
    q, k, v = _qkv(2, 4, 1, 1, 16, 22)
    o, lse = decode_fn(q, k, v)
    for b in range(2):
        for h in range(4):
            assert np.array_equal(o[b, h], v[b, 0, 0])
            assert abs(lse[b, h] - q[b, h] @ k[b, 0, 0] / 4.0) < 1e-13


def check_decode_constant_values(decode_fn):
    """All value rows equal c: o = c whatever the keys."""
    q, k, v = _qkv(1, 8, 2, 50, 8, 23)
    k *= 5.0
    v[:] = v[:, :, :1, :]
    o, _ = decode_fn(q, k, v)
    for h in range(8):
        assert np.allclose(o[0, h], v[0, h // 4, 0], rtol=0, atol=1e-13)


def sdpa_reference(q, k, v, seq_lens=None):
    """torch fp64 scaled_dot_product_attention on CPU (library routine), GQA by
    repeat_interleave, one query per sequence."""
    B, Hq, D = q.shape
    G = Hq // k.shape[1]
    o = np.empty((B, Hq, D))
    lse = np.empty((B, Hq))
    for b in range(B):
        n = k.shape[2] if seq_lens is None else int(seq_lens[b])
        kk = torch.from_numpy(np.ascontiguousarray(k[b, :, :n])).repeat_interleave(G, dim=0)
        vv = torch.from_numpy(np.ascontiguousarray(v[b, :, :n])).repeat_interleave(G, dim=0)
        qq = torch.from_numpy(np.ascontiguousarray(q[b]))[:, None, :]
        ob = torch.nn.functional.scaled_dot_product_attention(qq, kk, vv)
        o[b] = ob[:, 0].numpy()
        sc = (qq @ kk.transpose(1, 2))[:, 0, :] / np.sqrt(D)
        lse[b] = torch.logsumexp(sc, dim=-1).numpy()
    return o, lse


def check_decode_vs_sdpa(decode_fn):
    """Tiny shapes against torch's fp64 SDPA (with GQA via repeat_interleave)."""
    for (B, Hq, Hkv, T, D, seed) in [(1, 4, 1, 5, 2, 31), (2, 8, 2, 64, 8, 32), (3, 6, 3, 33, 64, 33),
                                     (1, 2, 2, 17, 8, 34)]:
        q, k, v = _qkv(B, Hq, Hkv, T, D, seed)
        k[:, 1 % Hkv] *= 3.0  # make kv heads clearly different
        o, lse = decode_fn(q, k, v)
        o_ref, lse_ref = sdpa_reference(q, k, v)
        assert np.allclose(o, o_ref, rtol=0, atol=1e-12)
        assert np.allclose(lse, lse_ref, rtol=0, atol=1e-12)


def check_decode_seq_lens(decode_fn):
    """Rows at or beyond seq_lens[b] never matter (fill them with garbage)."""
    q, k, v = _qkv(3, 4, 2, 40, 8, 35)
    lens = np.array([40, 1, 23])
    k2, v2 = k.copy(), v.copy()
    for b, n in enumerate(lens):
        k2[b, :, n:] = 1e3
        v2[b, :, n:] = -7e2
    o, lse = decode_fn(q, k2, v2, seq_lens=lens)
    o_ref, lse_ref = sdpa_reference(q, k, v, seq_lens=lens)
    assert np.allclose(o, o_ref, rtol=0, atol=1e-12)
    assert np.allclose(lse, lse_ref, rtol=0, atol=1e-12)


def check_decode_decimal(decode_fn):
    """T = 3, D = 2 against a 50-digit Decimal evaluation of the definition."""
    getcontext().prec = 50
    r = _rng(36)
    q = np.round(r.standard_normal((1, 2, 2)), 3)
    k = np.round(r.standard_normal((1, 1, 3, 2)) * 2, 3)
    v = np.round(r.standard_normal((1, 1, 3, 2)), 3)
    o, lse = decode_fn(q, k, v)
    sc = Decimal(1) / Decimal(2).sqrt()
    for h in range(2):
        qs = [Decimal(repr(float(x))) for x in q[0, h]]
        s = [sc * sum(qs[d] * Decimal(repr(float(k[0, 0, t, d]))) for d in range(2)) for t in range(3)]
        e = [x.exp() for x in s]
        tot = sum(e)
        for d in range(2):
            od = sum(e[t] * Decimal(repr(float(v[0, 0, t, d]))) for t in range(3)) / tot
            assert abs(Decimal(repr(float(o[0, h, d]))) - od) < Decimal("1e-14")
        assert abs(Decimal(repr(float(lse[0, h]))) - tot.ln()) < Decimal("1e-14")


def check_decode_planted_row(decode_fn):
    """A key row equal to 4*q (score 4|q|^2/sqrt(D)) takes nearly all the weight."""
    B, Hq, Hkv, T, D = 1, 4, 1, 4096, 128
    q, k, v = _qkv(B, Hq, Hkv, T, D, 37)
    t_star = 1234
    k[0, 0, t_star] = 4.0 * q[0, 0]
    o, _ = decode_fn(q, k, v)
    assert np.max(np.abs(o[0, 0] - v[0, 0, t_star])) < 1e-6


DECODE_CHECKS = [check_decode_identical_keys, check_decode_single_token, check_decode_constant_values,
                 check_decode_vs_sdpa, check_decode_seq_lens, check_decode_decimal, check_decode_planted_row]


# ----------------------------------------------------------------- self-decoder decode step

def _self_inputs(B, Hq, Hkv, T, D, seed):
    """Random cache and query; the new token's four source rows are small integers."""
    r = _rng(seed)
    q = r.standard_normal((B, Hq, D))
    k = r.standard_normal((B, Hkv, T, D))
    v = r.standard_normal((B, Hkv, T, D))
    new = {name: r.integers(-8, 9, (B, Hkv, D)).astype(np.float64) for name in ("k1", "ki", "v1", "vi")}
    return q, k, v, new


def check_self_decode_single_row(fn):
    """n = 1: only the new row is attended. With lambda = 4 and weights
    (1/4, 0) for K, (0, 1/4) for V: K' = K_1 and V' = V_i exactly, so o is V_i's
    new row and lse = <q, K_1's new row> / sqrt(D)."""
    q, k, v, new = _self_inputs(2, 4, 2, 5, 16, 41)
    k[:] = 1e3
    v[:] = -1e3
    o, lse, kn, vn = fn(q, k, v, new, (0.25, 0.0, 0.0, 0.25), seq_lens=np.array([1, 1]), lam=4.0)
    assert np.array_equal(kn, new["k1"]) and np.array_equal(vn, new["vi"])
    for b in range(2):
        for h in range(4):
            assert np.array_equal(o[b, h], new["vi"][b, h // 2])
            assert abs(lse[b, h] - q[b, h] @ new["k1"][b, h // 2] / 4.0) < 1e-12


def check_self_decode_reduces_to_decode(fn):
    """With K' = K_i and V' = V_i (lambda = 4, weights (0, 1/4)) the step is
    torch's fp64 SDPA over a cache whose row n - 1 holds the new K_i, V_i; what
    the cache itself holds at rows >= n - 1 is never read."""
    q, k, v, new = _self_inputs(3, 8, 2, 30, 8, 42)
    lens = np.array([30, 7, 12])
    k_ref, v_ref = k.copy(), v.copy()
    for b, n in enumerate(lens):
        k_ref[b, :, n - 1] = new["ki"][b]
        v_ref[b, :, n - 1] = new["vi"][b]
        k[b, :, n - 1:] = 5e2
        v[b, :, n - 1:] = -3e2
    o, lse, _, _ = fn(q, k, v, new, (0.0, 0.25, 0.0, 0.25), seq_lens=lens, lam=4.0)
    o_ref, lse_ref = sdpa_reference(q, k_ref, v_ref, seq_lens=lens)
    assert np.allclose(o, o_ref, rtol=0, atol=1e-12)
    assert np.allclose(lse, lse_ref, rtol=0, atol=1e-12)


def check_self_decode_vs_sdpa(fn):
    """lambda = 4 and weights (1/2, 1/4, -1/4, 3/4) on integer source rows, so
    that K' = 2 K_1 + K_i and V' = -V_1 + 3 V_i exactly: torch's fp64 SDPA over
    the cache rows followed by that row."""
    q, k, v, new = _self_inputs(2, 4, 1, 9, 8, 43)
    lens = np.array([9, 4])
    k_ref, v_ref = k.copy(), v.copy()
    for b, n in enumerate(lens):
        k_ref[b, :, n - 1] = 2 * new["k1"][b] + new["ki"][b]
        v_ref[b, :, n - 1] = -new["v1"][b] + 3 * new["vi"][b]
    o, lse, kn, vn = fn(q, k, v, new, (0.5, 0.25, -0.25, 0.75), seq_lens=lens, lam=4.0)
    assert np.array_equal(kn, 2 * new["k1"] + new["ki"]) and np.array_equal(vn, -new["v1"] + 3 * new["vi"])
    o_ref, lse_ref = sdpa_reference(q, k_ref, v_ref, seq_lens=lens)
    assert np.allclose(o, o_ref, rtol=0, atol=1e-12)
    assert np.allclose(lse, lse_ref, rtol=0, atol=1e-12)


SELF_DECODE_CHECKS = [check_self_decode_single_row, check_self_decode_reduces_to_decode, check_self_decode_vs_sdpa]


# ----------------------------------------------------------------- prefill

def sdpa_causal_reference(q, k, v, p0):
    """torch fp64 SDPA with an explicit causal mask at offset p0 (library routine)."""
    B, C, Hq, D = q.shape
    G = Hq // k.shape[1]
    n = p0 + C
    o = np.empty((B, C, Hq, D))
    for b in range(B):
        kk = torch.from_numpy(np.ascontiguousarray(k[b, :, :n])).repeat_interleave(G, dim=0)
        vv = torch.from_numpy(np.ascontiguousarray(v[b, :, :n])).repeat_interleave(G, dim=0)
        qq = torch.from_numpy(np.ascontiguousarray(q[b].transpose(1, 0, 2)))   # [Hq, C, D]
        mask = torch.arange(n)[None, :] <= (p0 + torch.arange(C))[:, None]
        if p0 == 0:
            ob = torch.nn.functional.scaled_dot_product_attention(qq, kk, vv, is_causal=True)
        else:
            ob = torch.nn.functional.scaled_dot_product_attention(qq, kk, vv, attn_mask=mask)
        o[b] = ob.numpy().transpose(1, 0, 2)
    return o


def _prefill_inputs(B, C, Hq, Hkv, Tcap, D, seed):
    r = _rng(seed)
    return (r.standard_normal((B, C, Hq, D)), r.standard_normal((B, Hkv, Tcap, D)),
            r.standard_normal((B, Hkv, Tcap, D)))


def check_prefill_first_row(prefill_fn):
    """p0 = 0: the first query sees only row 0, so o = V[0] exactly."""
    q, k, v = _prefill_inputs(2, 9, 4, 2, 9, 16, 41)
    o, lse = prefill_fn(q, k, v, 0)
    for b in range(2):
        for h in range(4):
            assert np.array_equal(o[b, 0, h], v[b, h // 2, 0])


def check_prefill_vs_sdpa(prefill_fn):
    for (B, C, Hq, Hkv, Tcap, D, p0, seed) in [(1, 16, 4, 1, 16, 8, 0, 42), (2, 7, 4, 2, 30, 8, 11, 43),
                                               (1, 33, 8, 2, 40, 64, 0, 44), (1, 5, 2, 1, 12, 2, 7, 45)]:
        q, k, v = _prefill_inputs(B, C, Hq, Hkv, Tcap, D, seed)
        o, _ = prefill_fn(q, k, v, p0)
        assert np.allclose(o, sdpa_causal_reference(q, k, v, p0), rtol=0, atol=1e-12)


def check_prefill_row_is_decode(prefill_fn, decode_fn):
    """Row at position p equals a decode over the first p+1 rows (and the last
    row of the chunk equals decode at T = p0 + C: early exit changes nothing)."""
    B, C, Hq, Hkv, D, p0 = 2, 12, 4, 2, 8, 5
    q, k, v = _prefill_inputs(B, C, Hq, Hkv, p0 + C + 3, D, 46)
    o, lse = prefill_fn(q, k, v, p0)
    for c in range(C):
        od, ld = decode_fn(q[:, c], k, v, seq_lens=np.full(B, p0 + c + 1))
        assert np.allclose(o[:, c], od, rtol=0, atol=1e-13)
        assert np.allclose(lse[:, :, c], ld, rtol=0, atol=1e-13)


def check_prefill_chunk_independence(prefill_fn):
    """Chunking only partitions query rows: one call over all rows equals the
    concatenation of chunked calls."""
    B, T, Hq, Hkv, D = 1, 24, 4, 1, 8
    q, k, v = _prefill_inputs(B, T, Hq, Hkv, T, D, 47)
    full, full_lse = prefill_fn(q, k, v, 0)
    for c0 in range(0, T, 7):
        c1 = min(T, c0 + 7)
        part, part_lse = prefill_fn(q[:, c0:c1], k, v, c0)
        assert np.allclose(part, full[:, c0:c1], rtol=0, atol=1e-13)
        assert np.allclose(part_lse, full_lse[:, :, c0:c1], rtol=0, atol=1e-13)


PREFILL_CHECKS = [check_prefill_first_row, check_prefill_vs_sdpa, check_prefill_chunk_independence]
