"""The compose-on-read decode (the comparator that caches raw K_i, V_i and
K_1, V_1): bit-for-bit equal to compose-then-decode, and within the decode bar
of the fp64 oracle over the exactly composed cache."""
import numpy as np
import pytest
import torch

import cross_layer_shared_amd as Y
import oracle as O
from synthetic import inputs as S
from tests import bars
from tests.gpu_util import dev, host, host_bits, say

pytestmark = pytest.mark.gpu


def _raw_caches(w, layer):
    """Layer 1's and layer i's K, V as head-major caches [B, Hkv, T, D]."""
    src = S.compose_sources(w, layer=layer)
    return {k: np.ascontiguousarray(v.transpose(0, 2, 1, 3)) for k, v in src.items()}


def _run(w, layer, alpha, splits):
    raw = _raw_caches(w, layer)
    q = S.queries(w, layer=layer + 100)
    d = {k: dev(v) for k, v in raw.items()}
    qd = dev(q)
    B, Hq, D = q.shape
    out_a = torch.empty((B, Hq, D), dtype=torch.float32, device="cuda")
    lse_a = torch.empty((B, Hq), dtype=torch.float32, device="cuda")
    Y.yoco_cross_attn_decode_compose_on_read(qd, d["k1"], d["ki"], d["v1"], d["vi"], alpha, out_a, lse_a,
                                             num_splits=splits)
    # reference path on the GPU: compose into a cache, then decode
    kc, vc = torch.empty_like(d["ki"]), torch.empty_like(d["vi"])
    Y.yoco_compose_kv(Y.head_major(d["k1"]), Y.head_major(d["ki"]), Y.head_major(d["v1"]), Y.head_major(d["vi"]),
                      kc, vc, 0, alpha, B=w.B, n=w.T, Hkv=w.Hkv, D=w.D, dtype=0 if w.dtype == "f32" else 1)
    out_b = torch.empty_like(out_a)
    lse_b = torch.empty_like(lse_a)
    Y.yoco_cross_attn_decode(qd, kc, vc, out_b, lse_b, num_splits=splits)
    torch.cuda.synchronize()
    return raw, q, host(out_a), host(lse_a), host(out_b), host(lse_b)


@pytest.mark.parametrize("dtype,D", [("bf16", 128), ("bf16", 64), ("f32", 64)])
@pytest.mark.parametrize("which", ["random", "identity", "mirror"])
@pytest.mark.parametrize("splits", [1, 3, 0])
def test_bitwise_equal_to_compose_then_decode(dtype, D, which, splits):
    w = S.Workload("cor", 80 + D, B=2, T=777, Hq=8, Hkv=2, D=D, dtype=dtype)
    inv = S.fl32(1 / 35)
    alpha = {"random": S.alphas(w.seed, 3), "identity": S.IDENTITY_ALPHA, "mirror": (inv, 0.0, inv, 0.0)}[which]
    _, _, oa, la, ob, lb = _run(w, 3, alpha, splits)
    assert np.array_equal(oa, ob) and np.array_equal(la, lb)


@pytest.mark.parametrize("G", [1, 2, 8, 16])
@pytest.mark.parametrize("dtype,D", [("bf16", 128), ("f32", 64)])
def test_group_sizes_bitwise(G, dtype, D):
    w = S.Workload("cor_g", 85 + G + D, B=2, T=333, Hq=2 * G, Hkv=2, D=D, dtype=dtype)
    _, _, oa, la, ob, lb = _run(w, 5, S.alphas(w.seed, 5), 3)
    assert np.array_equal(oa, ob) and np.array_equal(la, lb)


@pytest.mark.parametrize("dtype,D,tol", [("bf16", 128, 1e-2), ("f32", 64, 1e-5)])
def test_against_oracle_over_exact_composition(dtype, D, tol):
    w = S.Workload("cor2", 90, B=2, T=1500, Hq=8, Hkv=2, D=D, dtype=dtype)
    alpha = S.alphas(w.seed, 5)
    raw, q, oa, la, _, _ = _run(w, 5, alpha, 0)
    kp, vp = O.compose_kv(raw["k1"], raw["ki"], raw["v1"], raw["vi"], alpha)
    o_ref, lse_ref = O.decode_attention(q, kp, vp)
    err = np.max(np.abs(oa - o_ref))
    say(f"  max|o-ref| {err:.3e}  max|lse-ref| {np.max(np.abs(la - lse_ref)):.3e}")
    if dtype == "f32":
        assert np.max(np.max(np.abs(oa - o_ref), axis=-1) / np.max(np.abs(o_ref), axis=-1)) <= tol
    else:
        assert err <= tol and np.max(np.abs(la - lse_ref)) <= tol
        # against the oracle over the composed values as stored (rounded to bf16 by the compose kernel,
        # whose arithmetic the decode repeats row by row): the decode bars
        d = {k: dev(v) for k, v in raw.items()}
        kc, vc = torch.empty_like(d["ki"]), torch.empty_like(d["vi"])
        Y.yoco_compose_kv(Y.head_major(d["k1"]), Y.head_major(d["ki"]), Y.head_major(d["v1"]),
                          Y.head_major(d["vi"]), kc, vc, 0, alpha, B=w.B, n=w.T, Hkv=w.Hkv, D=w.D, dtype=1)
        torch.cuda.synchronize()
        o_st, lse_st = O.decode_attention(q, host_bits(kc), host_bits(vc))
        r = bars.decode_bf16(oa, la, o_st, lse_st)
        say("  over the stored composition: " + bars.report(r))
        assert r["ok"], r


def test_mid_context_shape():
    """The mid-context decode shape (B=8, T=4096, 32/8 heads, D=128), automatic split count."""
    w = S.Workload("cor3", 2, B=8, T=4096, Hq=32, Hkv=8, D=128, dtype="bf16")
    _, _, oa, la, ob, lb = _run(w, 8, S.alphas(w.seed, 8), 0)
    assert np.array_equal(oa, ob) and np.array_equal(la, lb)


@pytest.mark.parametrize("splits", [1, 2])
def test_long_splits_bitwise(splits):
    """Splits longer than 1024 rows: one register set, 8 wavefronts per workgroup."""
    w = S.Workload("cor4", 97, B=2, T=3000, Hq=8, Hkv=2, D=128, dtype="bf16")
    _, _, oa, la, ob, lb = _run(w, 4, S.alphas(w.seed, 4), splits)
    assert np.array_equal(oa, ob) and np.array_equal(la, lb)
