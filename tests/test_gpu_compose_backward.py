"""GPU parity of the composition backward (yoco_compose_kv_backward) with the
fp64 oracle. Bars: each fp32 gradient element within 1e-6 of the exact value,
relative to the size of its terms (|previous value| + |lambda a g|); each
weight gradient within 1e-5 of lambda * sum |g x| (the size of its terms)."""
import numpy as np
import pytest
import torch

import cross_layer_shared_amd as Y
import oracle as O
from synthetic import inputs as S
from tests.gpu_util import dev, host, say

pytestmark = pytest.mark.gpu


def _case(w, layer, t0, Tc, alpha, seed_pre=3):
    src = S.compose_sources(w, layer=layer)
    B, n, Hkv, D = w.B, w.T, w.Hkv, w.D
    # upstream gradients in the cache layout [B, Hkv, Tc, D], rows [t0, t0+n) used
    gk = S.normal_f32(w.seed, (40, 0), (B, Hkv, Tc, D))
    gv = S.normal_f32(w.seed, (41, 0), (B, Hkv, Tc, D))
    if w.dtype == "bf16":
        gk, gv = S.f32_to_bf16_bits(gk), S.f32_to_bf16_bits(gv)
    pre_k = S.normal_f32(w.seed, (42, seed_pre), (B, n, Hkv, D))
    pre_v = S.normal_f32(w.seed, (43, seed_pre), (B, n, Hkv, D))
    d = {k: dev(v) for k, v in src.items()}
    dk1, dv1 = dev(pre_k), dev(pre_v)
    dki = torch.full((B, n, Hkv, D), 7.0, dtype=torch.float32, device="cuda")
    dvi = torch.full_like(dki, 7.0)
    dalpha = torch.zeros(4, dtype=torch.float32, device="cuda")
    Y.yoco_compose_kv_backward(dev(gk), dev(gv), t0, d["k1"], d["ki"], d["v1"], d["vi"], dk1, dki, dv1, dvi, alpha,
                               dalpha)
    torch.cuda.synchronize()
    # oracle, on the gradient rows transposed to the source layout
    gk_t = O.to_f64(gk)[:, :, t0:t0 + n].transpose(0, 2, 1, 3)
    gv_t = O.to_f64(gv)[:, :, t0:t0 + n].transpose(0, 2, 1, 3)
    ref = O.compose_backward(gk_t, gv_t, src["k1"], src["ki"], src["v1"], src["vi"], alpha)
    lam = 35.0
    got = {"dk1": host(dk1), "dki": host(dki), "dv1": host(dv1), "dvi": host(dvi)}
    size = {"dk1": np.abs(pre_k) + np.abs(ref["dk1"]), "dki": np.abs(ref["dki"]),
            "dv1": np.abs(pre_v) + np.abs(ref["dv1"]), "dvi": np.abs(ref["dvi"])}
    want = {"dk1": pre_k + ref["dk1"], "dki": ref["dki"], "dv1": pre_v + ref["dv1"], "dvi": ref["dvi"]}
    for k in got:
        err = np.abs(got[k] - want[k])
        rel = np.max(err / np.maximum(size[k], 1e-30))
        say(f"  {k}: max err/size {rel:.3e}")
        assert rel <= 1e-6
    da = host(dalpha).astype(np.float64)
    mags = [lam * np.sum(np.abs(gk_t * O.to_f64(src["k1"]))), lam * np.sum(np.abs(gk_t * O.to_f64(src["ki"]))),
            lam * np.sum(np.abs(gv_t * O.to_f64(src["v1"]))), lam * np.sum(np.abs(gv_t * O.to_f64(src["vi"])))]
    for i in range(4):
        say(f"  dalpha[{i}] {da[i]:.6e} ref {ref['dalpha'][i]:.6e} rel-to-size {abs(da[i] - ref['dalpha'][i]) / mags[i]:.2e}")
        assert abs(da[i] - ref["dalpha"][i]) <= 1e-5 * mags[i]


@pytest.mark.parametrize("dtype,D", [("bf16", 128), ("bf16", 64), ("f32", 64), ("f32", 128)])
def test_backward_small(dtype, D):
    w = S.Workload("bwd", 60 + D, B=2, T=301, Hq=6, Hkv=3, D=D, dtype=dtype)
    _case(w, 4, 5, 320, S.alphas(w.seed, 4))


def test_backward_identity_init():
    """At initialisation layer 1's gradients stay as they were and dK_i = gk."""
    w = S.Workload("bwd_id", 66, B=1, T=100, Hq=2, Hkv=2, D=128, dtype="bf16")
    _case(w, 2, 0, 100, S.IDENTITY_ALPHA)


def test_backward_full_prefill_layer():
    """One self-decoder layer of the 32K-token workload: [1, 32768, 8, 128] bf16."""
    _case(S.PREFILL_CHUNKED, 3, 0, S.PREFILL_CHUNKED.T, S.alphas(S.PREFILL_CHUNKED.seed, 3))


@pytest.mark.parametrize("dtype,D,n", [("f32", 64, 1), ("bf16", 64, 3), ("bf16", 128, 1)])
def test_backward_single_rows(dtype, D, n):
    """Fewer positions than one workgroup covers: most threads have no element."""
    w = S.Workload("bwd_tiny", 67 + n, B=1, T=n, Hq=2, Hkv=1, D=D, dtype=dtype)
    _case(w, 5, 2, n + 4, S.alphas(w.seed, 5))
