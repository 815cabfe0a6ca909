"""The prefill pipeline with YOCO's early exit: the self-decoder half composes
the middle layer's K', V' for every prompt row, and the cross-decoder half runs
only for the last token (one decode call per cross layer) instead of a full
causal prefill. The early exit must not change the output: the decode of the
last token equals the last row of the full causal prefill.

Bars: the decode and the prefill's last row each against the fp64 oracle over
the stored (bf16-rounded) composed cache, within their bars (tests/bars.py),
and within the prefill bar of each other; both also within the stated 1e-2
absolute of the oracle over the exactly composed cache (the whole pipeline,
compose rounding included)."""
import numpy as np
import pytest
import torch

import cross_layer_shared_amd as Y
import oracle as O
from synthetic import inputs as S
from tests import bars
from tests.gpu_util import dev, host, host_bits, say

pytestmark = pytest.mark.gpu

ATOL = 1e-2


def _pipeline(w, layer, chunk):
    """Compose layer `layer`'s K', V' for all rows, then (a) the causal prefill of
    the last chunk and (b) the decode of the last token over the composed cache."""
    src = S.compose_sources(w, layer=layer)                     # token-major [B, T, Hkv, D]
    alpha = S.alphas(w.seed, layer)
    d = {k: dev(v) for k, v in src.items()}
    kc = torch.empty((w.B, w.Hkv, w.T, w.D), dtype=torch.bfloat16, device="cuda")
    vc = torch.empty_like(kc)
    Y.yoco_compose_kv(d["k1"], d["ki"], d["v1"], d["vi"], kc, vc, 0, alpha)
    q = S.queries(w, layer=layer + 50, std=w.notes.get("q_std", 1.0), rows=chunk)   # the prompt's last chunk
    qd = dev(q)
    p0 = w.T - chunk
    out_pf = torch.empty((w.B, chunk, w.Hq, w.D), dtype=torch.float32, device="cuda")
    lse_pf = torch.empty((w.B, w.Hq, chunk), dtype=torch.float32, device="cuda")
    Y.yoco_cross_attn_prefill(qd, kc, vc, p0, out_pf, lse_pf)
    out_dec = torch.empty((w.B, w.Hq, w.D), dtype=torch.float32, device="cuda")
    lse_dec = torch.empty((w.B, w.Hq), dtype=torch.float32, device="cuda")
    Y.yoco_cross_attn_decode(qd[:, -1].contiguous(), kc, vc, out_dec, lse_dec)
    torch.cuda.synchronize()
    k_ref, v_ref = O.compose_kv(src["k1"], src["ki"], src["v1"], src["vi"], alpha)
    k_ref, v_ref = k_ref.transpose(0, 2, 1, 3), v_ref.transpose(0, 2, 1, 3)          # head-major, exact
    exact = O.decode_attention(q[:, -1], k_ref, v_ref)
    kb, vb = host_bits(kc), host_bits(vc)                                          # the stored cache
    o_ref, lse_ref = O.decode_attention(q[:, -1], kb, vb)
    _, lse2_ref = O.decode_attention(bars.doubled(q[:, -1]), kb, vb)
    return (host(out_pf)[:, -1].astype(np.float64), host(lse_pf)[:, :, -1].astype(np.float64),
            host(out_dec).astype(np.float64), host(lse_dec).astype(np.float64), (o_ref, lse_ref, lse2_ref), exact)


def _check(o_pf, l_pf, o_dec, l_dec, ref, exact):
    o_ref, l_ref, l2_ref = ref
    r_pf = bars.prefill_bf16(o_pf, l_pf, o_ref, l_ref, l2_ref)
    r_dec = bars.decode_bf16(o_dec, l_dec, o_ref, l_ref)
    r_pair = bars.prefill_bf16(o_pf, l_pf, o_dec, l_dec, l2_ref)
    say(f"  prefill: {bars.report(r_pf)}\n  decode: {bars.report(r_dec)}\n  prefill vs decode: {bars.report(r_pair)}")
    assert r_pf["ok"] and r_dec["ok"] and r_pair["ok"]
    o_x, l_x = exact
    e = max(np.max(np.abs(o_pf - o_x)), np.max(np.abs(o_dec - o_x)))
    le = max(np.max(np.abs(l_pf - l_x)), np.max(np.abs(l_dec - l_x)))
    say(f"  against the exactly composed cache: max|o| {e:.3e}  max|lse| {le:.3e}")
    assert e <= ATOL and le <= ATOL


@pytest.mark.parametrize("B,T,Hq,Hkv,chunk", [(2, 1536, 8, 2, 512), (1, 1000, 16, 4, 232)])
def test_early_exit_small(B, T, Hq, Hkv, chunk):
    w = S.Workload("early_exit", 95 + T, B=B, T=T, Hq=Hq, Hkv=Hkv, D=128, dtype="bf16")
    _check(*_pipeline(w, 3, chunk))


def test_early_exit_32k_prefill_workload():
    """The 32K-token prefill workload (1 sequence, 32/8 heads, D=128, chunk 4096),
    cache composed from its layer-16 and layer-1 sources."""
    w = S.PREFILL_CHUNKED
    _check(*_pipeline(w, w.self_layers, w.chunk))
