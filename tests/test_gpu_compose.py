"""GPU parity of yoco_compose_kv against the fp64 oracle.

Bar: fp32 caches within 1e-6 of the exact value relative to the size of the
summed terms, lambda*(|a1 X1| + |a2 Xi|) (cancellation-aware); bf16 caches
within one bf16 ulp of the exact value plus that fp32 term; the YOCO
initialisation (and the mirror case) bit for bit."""
import numpy as np
import pytest
import torch

import cross_layer_shared_amd as Y
import oracle as O
from synthetic import inputs as S
from tests.gpu_util import bf16_to_f64, bf16_ulp, dev, host, say

pytestmark = pytest.mark.gpu


def _check_against_oracle(x1, xi, a1, a2, got, dtype):
    ref = O.compose(x1, xi, a1, a2)
    mag = O.compose_magnitude(x1, xi, a1, a2)
    g = got.astype(np.float64) if dtype == "f32" else bf16_to_f64(got)
    err = np.abs(g - ref)
    if dtype == "f32":
        rel = np.where(mag > 0, err / np.where(mag > 0, mag, 1.0), err)
        say(f"  compose fp32 max cancellation-aware rel err {rel.max():.3e}")
        assert rel.max() <= 1e-6
    else:
        bound = bf16_ulp(ref) + 1e-6 * mag
        say(f"  compose bf16 max err/bound {np.max(err / bound):.3f}; "
            f"bitwise == RNE(exact): {np.mean(g == O.bf16_nearest(ref)):.6f}")
        assert np.all(err <= bound)


def _cache(B, Hkv, T, D, dtype, fill=0.0):
    td = torch.float32 if dtype == "f32" else torch.bfloat16
    return torch.full((B, Hkv, T, D), fill, dtype=td, device="cuda")


def _slice_rows(c, t0, n):
    return host(c[:, :, t0:t0 + n].transpose(1, 2).contiguous())   # -> [B, n, Hkv, D]


def test_compose_tiny_fp32_stack():
    w = S.TINY_FP32_STACK
    src = S.compose_sources(w, layer=2)
    alpha = S.alphas(w.seed, 2)
    kc, vc = _cache(1, 1, w.T, w.D, "f32"), _cache(1, 1, w.T, w.D, "f32")
    d = {k: dev(v) for k, v in src.items()}
    Y.yoco_compose_kv(d["k1"], d["ki"], d["v1"], d["vi"], kc, vc, 0, alpha)
    torch.cuda.synchronize()
    _check_against_oracle(src["k1"], src["ki"], alpha[0], alpha[1], _slice_rows(kc, 0, w.T), "f32")
    _check_against_oracle(src["v1"], src["vi"], alpha[2], alpha[3], _slice_rows(vc, 0, w.T), "f32")


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_compose_identity_init_bitwise(dtype):
    """alpha = (0, fl32(1/35)): the cache holds K_i, V_i bit for bit (YOCO++ at init = YOCO)."""
    w = S.Workload("id", 11, B=2, T=77, Hq=4, Hkv=2, D=128 if dtype == "bf16" else 64, dtype=dtype)
    src = S.compose_sources(w, layer=3)
    kc, vc = _cache(2, 2, 80, w.D, dtype), _cache(2, 2, 80, w.D, dtype)
    d = {k: dev(v) for k, v in src.items()}
    Y.yoco_compose_kv(d["k1"], d["ki"], d["v1"], d["vi"], kc, vc, 3, S.IDENTITY_ALPHA)
    torch.cuda.synchronize()
    assert np.array_equal(_slice_rows(kc, 3, 77), src["ki"])
    assert np.array_equal(_slice_rows(vc, 3, 77), src["vi"])


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_compose_mirror_bitwise(dtype):
    w = S.Workload("mirror", 12, B=1, T=50, Hq=2, Hkv=2, D=64, dtype=dtype)
    src = S.compose_sources(w, layer=2)
    inv = S.fl32(1 / 35)
    kc, vc = _cache(1, 2, 50, 64, dtype), _cache(1, 2, 50, 64, dtype)
    d = {k: dev(v) for k, v in src.items()}
    Y.yoco_compose_kv(d["k1"], d["ki"], d["v1"], d["vi"], kc, vc, 0, (inv, 0.0, 0.0, inv))
    torch.cuda.synchronize()
    assert np.array_equal(_slice_rows(kc, 0, 50), src["k1"])
    assert np.array_equal(_slice_rows(vc, 0, 50), src["vi"])


@pytest.mark.parametrize("dtype,D", [("bf16", 128), ("bf16", 64), ("f32", 64), ("f32", 128)])
def test_compose_ragged_strided(dtype, D):
    """Strided source views, an offset t0, a ragged n; rows outside [t0, t0+n) keep their sentinel."""
    B, n, Hkv, T, t0 = 2, 301, 3, 320, 7
    w = S.Workload("ragged", 13, B=B, T=n, Hq=Hkv, Hkv=Hkv, D=D, dtype=dtype)
    src = S.compose_sources(w, layer=4)
    alpha = S.alphas(w.seed, 4)
    # views into wider buffers: [B, n, Hkv, 2D] -> [..., :D]
    d = {}
    for k, v in src.items():
        wide = torch.zeros((B, n, Hkv, 2 * D), dtype=torch.float32 if dtype == "f32" else torch.bfloat16,
                           device="cuda")
        wide[..., :D] = dev(v)
        d[k] = wide[..., :D]
    sentinel = 3.5
    kc, vc = _cache(B, Hkv, T, D, dtype, sentinel), _cache(B, Hkv, T, D, dtype, sentinel)
    Y.yoco_compose_kv(d["k1"], d["ki"], d["v1"], d["vi"], kc, vc, t0, alpha)
    torch.cuda.synchronize()
    _check_against_oracle(src["k1"], src["ki"], alpha[0], alpha[1], _slice_rows(kc, t0, n), dtype)
    _check_against_oracle(src["v1"], src["vi"], alpha[2], alpha[3], _slice_rows(vc, t0, n), dtype)
    for c in (kc, vc):
        assert torch.all(c[:, :, :t0] == sentinel) and torch.all(c[:, :, t0 + n:] == sentinel)


def test_compose_in_place():
    """K_i / V_i aliasing their cache exactly (t0 = 0) is allowed."""
    B, n, Hkv, D = 1, 64, 2, 128
    w = S.Workload("inplace", 14, B=B, T=n, Hq=2, Hkv=Hkv, D=D, dtype="bf16")
    src = S.compose_sources(w, layer=2)
    alpha = S.alphas(w.seed, 2)
    k1, v1 = dev(src["k1"]), dev(src["v1"])
    kc = dev(src["ki"]).transpose(1, 2).contiguous()   # [B, Hkv, n, D]
    vc = dev(src["vi"]).transpose(1, 2).contiguous()
    Y.yoco_compose_kv(k1, Y.head_major(kc), v1, Y.head_major(vc), kc, vc, 0, alpha, B=B, n=n, Hkv=Hkv, D=D,
                      dtype=1)
    torch.cuda.synchronize()
    _check_against_oracle(src["k1"], src["ki"], alpha[0], alpha[1], _slice_rows(kc, 0, n), "bf16")
    _check_against_oracle(src["v1"], src["vi"], alpha[2], alpha[3], _slice_rows(vc, 0, n), "bf16")


def test_compose_decode_append_row():
    """n = 1: the decode step's new token composed into row T-1 of a B=8 cache."""
    w = S.DECODE_MID
    src = S.compose_sources(w, layer=16, n=1)
    alpha = S.alphas(w.seed, 16)
    kc, vc = _cache(w.B, w.Hkv, 64, w.D, "bf16", 1.0), _cache(w.B, w.Hkv, 64, w.D, "bf16", 1.0)
    d = {k: dev(v) for k, v in src.items()}
    Y.yoco_compose_kv(d["k1"], d["ki"], d["v1"], d["vi"], kc, vc, 63, alpha)
    torch.cuda.synchronize()
    _check_against_oracle(src["k1"], src["ki"], alpha[0], alpha[1], _slice_rows(kc, 63, 1), "bf16")
    _check_against_oracle(src["v1"], src["vi"], alpha[2], alpha[3], _slice_rows(vc, 63, 1), "bf16")
    assert torch.all(kc[:, :, :63] == 1.0)


def test_compose_full_prefill_layer():
    """One full self-decoder layer of the 32K-token prefill workload (every element checked)."""
    w = S.PREFILL_CHUNKED
    layer = 2
    src = S.compose_sources(w, layer=layer)
    alpha = S.alphas(w.seed, layer)
    kc, vc = _cache(w.B, w.Hkv, w.T, w.D, "bf16"), _cache(w.B, w.Hkv, w.T, w.D, "bf16")
    d = {k: dev(v) for k, v in src.items()}
    say(f"  compose full layer {layer}: B={w.B} n={w.T} Hkv={w.Hkv} D={w.D}")
    Y.yoco_compose_kv(d["k1"], d["ki"], d["v1"], d["vi"], kc, vc, 0, alpha)
    torch.cuda.synchronize()
    _check_against_oracle(src["k1"], src["ki"], alpha[0], alpha[1], _slice_rows(kc, 0, w.T), "bf16")
    _check_against_oracle(src["v1"], src["vi"], alpha[2], alpha[3], _slice_rows(vc, 0, w.T), "bf16")
