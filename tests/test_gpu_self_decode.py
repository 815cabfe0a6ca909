"""GPU parity of the self-decoder decode step (yoco_self_attn_decode) against
the fp64 oracle.

Bars: the row written into the cache within the compose bars (bf16: one ulp
of the exact value plus 1e-6 of the summed terms; fp32: 1e-6 of the summed
terms) and bit for bit what yoco_compose_kv writes; every other cache row
untouched. The output within the decode bars (fp32 caches: per (b, h) row
1e-5 ||o_ref||_inf; bf16: each row within 1e-3 of its rms, lse within 1e-4,
as derived in tests/bars.py, and the stated 1e-2 absolute) plus the first-order
effect of storing the new row rounded: the oracle attends over the exactly
composed row, the kernel (like any later step) over the stored one, and when
that row carries most of the softmax weight its bf16 rounding alone moves the
output by up to p_new * ulp(V'_new)."""
import numpy as np
import pytest
import torch

import cross_layer_shared_amd as Y
import oracle as O
from synthetic import inputs as S
from tests import bars
from tests.gpu_util import bf16_to_f64, bf16_ulp, dev, host, rowwise_rel, say

pytestmark = pytest.mark.gpu


def _f64(x):
    return bf16_to_f64(x) if x.dtype == np.uint16 else x.astype(np.float64)


def _case(B, T, Hq, Hkv, D, dtype, seed, layer=4):
    w = S.Workload("self", seed, B=B, T=T, Hq=Hq, Hkv=Hkv, D=D, dtype=dtype)
    k, v = S.cache_kv(w)
    q = S.queries(w, layer=layer)
    new = {n: x[:, 0] for n, x in S.compose_sources(w, layer=layer, n=1).items()}   # [B, Hkv, D]
    return w, q, k, v, new, S.alphas(w.seed, layer)


def _step(q, k, v, new, alpha, seq_lens=None, splits=0, in_place=False):
    """One fused step on the GPU; returns out, lse and the caches after the step."""
    kd, vd = dev(k), dev(v)
    qd = dev(q)
    B, Hq, D = q.shape
    sl = None if seq_lens is None else torch.tensor(seq_lens, dtype=torch.int32, device="cuda")
    if in_place:
        # the new token's raw K_i, V_i already sit in the cache row; compose them there
        T = k.shape[2]
        for b in range(B):
            n = T if seq_lens is None else seq_lens[b]
            kd[b, :, n - 1] = dev(new["ki"][b])
            vd[b, :, n - 1] = dev(new["vi"][b])
        srcs = (dev(new["k1"]), Y.head_major(kd), dev(new["v1"]), Y.head_major(vd))
    else:
        srcs = tuple(dev(new[n]) for n in ("k1", "ki", "v1", "vi"))
    out = torch.empty((B, Hq, D), dtype=torch.float32, device="cuda")
    lse = torch.empty((B, Hq), dtype=torch.float32, device="cuda")
    Y.yoco_self_attn_decode(qd, *srcs, kd, vd, alpha, out, lse, seq_lens=sl, num_splits=splits)
    torch.cuda.synchronize()
    return host(out).astype(np.float64), host(lse).astype(np.float64), host(kd), host(vd)


def _row_bounds(new, alpha, dtype):
    """Exact composed rows and the compose bars on their stored values."""
    out = []
    for x1, xi, a1, a2 in ((new["k1"], new["ki"], alpha[0], alpha[1]), (new["v1"], new["vi"], alpha[2], alpha[3])):
        ref = O.compose(x1, xi, a1, a2)
        bar = 1e-6 * O.compose_magnitude(x1, xi, a1, a2) + (bf16_ulp(ref) if dtype == "bf16" else 0.0)
        out += [ref, bar]
    return out


def _rounding_slack(q, o_ref, lse_ref, appended, dtype):
    """How far the output may move because each appended row is attended as
    stored rather than exact, to first order, with a margin of 2:
    |do| <= p_r (|dV_r| + |V_r - o| |ds_r|),  |dlse| <= p_r |ds_r|,
    p_r = exp(s_r - lse), |ds_r| <= scale sum_d |q_d| |dK_r,d|."""
    B, Hq, D = q.shape
    q64 = _f64(q)
    scale = 1.0 / np.sqrt(D)
    so, sl = np.zeros_like(o_ref), np.zeros_like(lse_ref)
    for new, alpha in appended:
        kn, bk, vn, bv = _row_bounds(new, alpha, dtype)
        G = Hq // kn.shape[1]
        kn, bk, vn, bv = (np.repeat(x, G, axis=1) for x in (kn, bk, vn, bv))     # per query head
        p = np.exp(scale * np.sum(q64 * kn, axis=-1) - lse_ref)
        ds = scale * np.sum(np.abs(q64) * bk, axis=-1)
        so += p[..., None] * (bv + np.abs(vn - o_ref) * ds[..., None])
        sl += p * ds
    return 2.0 * so, 2.0 * sl


def _check_output(o, lse, o_ref, lse_ref, dtype, slack):
    so, sl = slack
    err = np.abs(o - o_ref)
    say(f"  max|o-ref| {err.max():.3e}  row-rel {rowwise_rel(o, o_ref):.3e}  max|lse-ref| "
        f"{np.max(np.abs(lse - lse_ref)):.3e}  max rounding slack {so.max():.3e}")
    if dtype == "f32":
        bar = 1e-5 * np.max(np.abs(o_ref), axis=-1, keepdims=True) + so
        assert np.all(err <= bar)
        assert np.all(np.abs(lse - lse_ref) <= 1e-5 * np.maximum(1.0, np.abs(lse_ref)) + sl)
    else:
        # the decode bars (tests/bars.py) plus the slack of the rounded new row
        bar = bars.DECODE_REL * bars.row_rms(o_ref)[..., None] + bars.O_FLOOR + so
        assert np.all(err <= bar) and np.all(err <= bars.STATED_ATOL + so)
        assert np.all(np.abs(lse - lse_ref) <= bars.DECODE_LSE + sl)


def _check_rows(k0, v0, k1, v1, new, alpha, seq_lens, dtype):
    """Row n-1 of each sequence holds the composed row (compose bar); all else is unchanged."""
    B, Hkv, T, D = k0.shape
    lens = [T] * B if seq_lens is None else list(seq_lens)
    for before, after, a1, a2, x1, xi in ((k0, k1, alpha[0], alpha[1], new["k1"], new["ki"]),
                                          (v0, v1, alpha[2], alpha[3], new["v1"], new["vi"])):
        mask = np.ones((B, Hkv, T), dtype=bool)
        for b, n in enumerate(lens):
            mask[b, :, n - 1] = False
        assert np.array_equal(before[mask], after[mask])
        ref = O.compose(x1, xi, a1, a2)                       # [B, Hkv, D]
        mag = O.compose_magnitude(x1, xi, a1, a2)
        got = np.stack([_f64(after[b, :, n - 1]) for b, n in enumerate(lens)])
        err = np.abs(got - ref)
        bound = 1e-6 * mag + (bf16_ulp(ref) if dtype == "bf16" else 0.0)
        assert np.all(err <= np.maximum(bound, 1e-30 if dtype == "f32" else 0.0))


@pytest.mark.parametrize("dtype,D", [("bf16", 128), ("bf16", 64), ("f32", 64)])
@pytest.mark.parametrize("splits", [1, 3, 0])
def test_against_oracle(dtype, D, splits):
    w, q, k, v, new, alpha = _case(3, 900, 8, 2, D, dtype, 60 + D)
    lens = [900, 1, 457]
    o, lse, k1, v1 = _step(q, k, v, new, alpha, lens, splits)
    o_ref, lse_ref, _, _ = O.self_attn_decode(q, k, v, new, alpha, seq_lens=np.array(lens))
    _check_output(o, lse, o_ref, lse_ref, dtype, _rounding_slack(q, o_ref, lse_ref, [(new, alpha)], dtype))
    _check_rows(k, v, k1, v1, new, alpha, lens, dtype)


@pytest.mark.parametrize("G", [1, 2, 8, 16])
@pytest.mark.parametrize("dtype,D", [("bf16", 128), ("bf16", 64), ("f32", 64)])
def test_group_sizes(G, dtype, D):
    """Every GQA group size: the new row's score is folded with the query slice
    of its own head whatever order the lane holds the heads in."""
    w, q, k, v, new, alpha = _case(2, 300, 2 * G, 2, D, dtype, 70 + G + D)
    lens = [300, 129]
    o, lse, k1, v1 = _step(q, k, v, new, alpha, lens, 3)
    o_ref, lse_ref, _, _ = O.self_attn_decode(q, k, v, new, alpha, seq_lens=np.array(lens))
    _check_output(o, lse, o_ref, lse_ref, dtype, _rounding_slack(q, o_ref, lse_ref, [(new, alpha)], dtype))
    _check_rows(k, v, k1, v1, new, alpha, lens, dtype)


@pytest.mark.parametrize("dtype,D", [("bf16", 128), ("f32", 64)])
def test_written_row_is_the_compose_kernels(dtype, D):
    """All sequences full (n = T): the fused step writes at row T-1 exactly what
    yoco_compose_kv writes there, and its output matches compose-then-decode up to
    the fp32 summation order of that one row."""
    w, q, k, v, new, alpha = _case(2, 333, 8, 2, D, dtype, 70 + D)
    o, lse, k1, v1 = _step(q, k, v, new, alpha)
    kd, vd = dev(k), dev(v)
    src = {n: dev(x[:, None]) for n, x in new.items()}             # [B, 1, Hkv, D]
    Y.yoco_compose_kv(src["k1"], src["ki"], src["v1"], src["vi"], kd, vd, w.T - 1, alpha)
    out = torch.empty((w.B, w.Hq, w.D), dtype=torch.float32, device="cuda")
    lse_b = torch.empty((w.B, w.Hq), dtype=torch.float32, device="cuda")
    Y.yoco_cross_attn_decode(dev(q), kd, vd, out, lse_b)
    torch.cuda.synchronize()
    assert np.array_equal(host(kd), k1) and np.array_equal(host(vd), v1)
    ob = host(out).astype(np.float64)
    assert rowwise_rel(o, ob) <= 1e-5
    assert np.max(np.abs(lse - host(lse_b))) <= 1e-5


@pytest.mark.parametrize("splits", [1, 4])
def test_single_row_sequence_returns_the_new_value(splits):
    """n = 1: the softmax has one term, so o is the stored V' row exactly."""
    w, q, k, v, new, alpha = _case(2, 64, 8, 2, 128, "bf16", 75)
    o, lse, _, v1 = _step(q, k, v, new, alpha, [1, 1], splits)
    for b in range(2):
        for h in range(8):
            assert np.array_equal(o[b, h], bf16_to_f64(v1[b, h // 4, 0]))
    _, lse_ref, _, _ = O.self_attn_decode(q, k, v, new, alpha, seq_lens=np.array([1, 1]))
    assert np.max(np.abs(lse - lse_ref)) <= 1e-2


@pytest.mark.parametrize("dtype,D", [("bf16", 128), ("f32", 64)])
def test_in_place_compose_of_the_cache_row(dtype, D):
    """The raw K_i, V_i written into the cache row itself and composed in place
    give the same bits as separate one-token sources."""
    w, q, k, v, new, alpha = _case(2, 500, 8, 2, D, dtype, 80 + D)
    lens = [500, 77]
    a = _step(q, k, v, new, alpha, lens)
    b = _step(q, k, v, new, alpha, lens, in_place=True)
    for x, y in zip(a, b):
        assert np.array_equal(x, y)


def test_layer_one_keeps_its_row():
    """Layer 1 (no composition): with the initialisation weights and K_1 = K_i the
    written row is the raw row bit for bit."""
    w, q, k, v, new, _ = _case(2, 256, 16, 4, 128, "bf16", 85)
    new = {"k1": new["k1"], "ki": new["k1"], "v1": new["v1"], "vi": new["v1"]}
    _, _, k1, v1 = _step(q, k, v, new, S.IDENTITY_ALPHA)
    assert np.array_equal(k1[:, :, -1], new["k1"]) and np.array_equal(v1[:, :, -1], new["v1"])


def test_three_consecutive_steps():
    """Three decode steps on one cache (n = 100, 101, 102): each step reads the rows
    the earlier steps appended. The oracle carries its own exactly composed rows."""
    w = S.Workload("self3", 90, B=2, T=256, Hq=8, Hkv=2, D=128, dtype="bf16")
    k, v = S.cache_kv(w)
    kd, vd = dev(k), dev(v)
    k_ref, v_ref = _f64(k), _f64(v)
    appended = []
    for step, n in enumerate((100, 101, 102)):
        layer = 10 + step
        q = S.queries(w, layer=layer)
        new = {nm: x[:, 0] for nm, x in S.compose_sources(w, layer=layer, n=1).items()}
        alpha = S.alphas(w.seed, 3)
        sl = torch.tensor([n, n], dtype=torch.int32, device="cuda")
        out = torch.empty((w.B, w.Hq, w.D), dtype=torch.float32, device="cuda")
        lse = torch.empty((w.B, w.Hq), dtype=torch.float32, device="cuda")
        Y.yoco_self_attn_decode(dev(q), *(dev(new[nm]) for nm in ("k1", "ki", "v1", "vi")), kd, vd, alpha, out,
                                lse, seq_lens=sl)
        torch.cuda.synchronize()
        o_ref, lse_ref, kn, vn = O.self_attn_decode(q, k_ref, v_ref, new, alpha, seq_lens=np.array([n, n]))
        k_ref[:, :, n - 1], v_ref[:, :, n - 1] = kn, vn
        appended.append((new, alpha))
        _check_output(host(out).astype(np.float64), host(lse).astype(np.float64), o_ref, lse_ref, "bf16",
                      _rounding_slack(q, o_ref, lse_ref, appended, "bf16"))


def test_mid_context_shape():
    """The mid-context decode shape (B=8, T=4096, 32/8 heads, D=128), automatic
    split count, sequences of mixed lengths."""
    w, q, k, v, new, alpha = _case(8, 4096, 32, 8, 128, "bf16", 2)
    lens = [4096, 4095, 3000, 2049, 1024, 513, 17, 1]
    o, lse, k1, v1 = _step(q, k, v, new, alpha, lens)
    o_ref, lse_ref, _, _ = O.self_attn_decode(q, k, v, new, alpha, seq_lens=np.array(lens))
    _check_output(o, lse, o_ref, lse_ref, "bf16", _rounding_slack(q, o_ref, lse_ref, [(new, alpha)], "bf16"))
    _check_rows(k, v, k1, v1, new, alpha, lens, "bf16")


@pytest.mark.parametrize("dtype,D", [("bf16", 128), ("f32", 64)])
def test_long_splits(dtype, D):
    """Splits longer than 1024 rows (one register set, 8 wavefronts per workgroup)."""
    w, q, k, v, new, alpha = _case(2, 3000, 8, 2, D, dtype, 95 + D)
    lens = [3000, 1800]
    for splits in (1, 2):
        o, lse, k1, v1 = _step(q, k, v, new, alpha, lens, splits)
        o_ref, lse_ref, _, _ = O.self_attn_decode(q, k, v, new, alpha, seq_lens=np.array(lens))
        _check_output(o, lse, o_ref, lse_ref, dtype, _rounding_slack(q, o_ref, lse_ref, [(new, alpha)], dtype))
        _check_rows(k, v, k1, v1, new, alpha, lens, dtype)
