"""Caches in the token-major layout [B, Tcap, Hkv, D] (rows of one kv head
Hkv * D elements apart, the layout a fused QKV projection writes), passed
through the element strides of the ABI, with spare capacity Tcap > T.

Each entry point must give, on such a view, the same result as the fp64
oracle on the same values (the decode, compose and prefill bars), and the
same bits as on a head-major copy of the cache (the arithmetic does not
depend on where a row lives)."""
import numpy as np
import pytest
import torch

import cross_layer_shared_amd as Y
import oracle as O
from synthetic import inputs as S
from tests import bars
from tests.gpu_util import dev, host, rowwise_rel, say
from tests.test_gpu_self_decode import _check_output, _rounding_slack

pytestmark = pytest.mark.gpu


def _token_major(x: np.ndarray, Tcap: int) -> np.ndarray:
    """[B, Hkv, T, D] -> [B, Tcap, Hkv, D] (rows past T hold garbage)."""
    B, H, T, D = x.shape
    out = np.full((B, Tcap, H, D), 0x7F7F if x.dtype == np.uint16 else 3.0e3, dtype=x.dtype)
    out[:, :T] = x.transpose(0, 2, 1, 3)
    return out


def _view(t: torch.Tensor) -> Y.Tensor4:
    return Y.token_major(t)


def _check(o, lse, o_ref, lse_ref, dtype):
    err = np.max(np.abs(o - o_ref))
    say(f"  max|o-ref| {err:.3e}  row-rel {rowwise_rel(o, o_ref):.3e}")
    if dtype == "f32":
        assert rowwise_rel(o, o_ref) <= 1e-5
        assert np.max(np.abs(lse - lse_ref) / np.maximum(1.0, np.abs(lse_ref))) <= 1e-5
    else:
        r = bars.decode_bf16(o, lse, o_ref, lse_ref)
        say("  " + bars.report(r))
        assert r["ok"], r


def _decode(q, kc, vc, Hkv, T, splits, seq_lens=None):
    B, Hq, D = q.shape
    out = torch.empty((B, Hq, D), dtype=torch.float32, device="cuda")
    lse = torch.empty((B, Hq), dtype=torch.float32, device="cuda")
    sl = None if seq_lens is None else torch.tensor(seq_lens, dtype=torch.int32, device="cuda")
    Y.yoco_cross_attn_decode(q, kc, vc, out, lse, seq_lens=sl, T=T, num_splits=splits, Hkv=Hkv)
    torch.cuda.synchronize()
    return host(out).astype(np.float64), host(lse).astype(np.float64)


@pytest.mark.parametrize("dtype,D,Hq,Hkv", [("bf16", 128, 32, 8), ("bf16", 64, 8, 2), ("f32", 64, 4, 1)])
@pytest.mark.parametrize("splits", [1, 3, 0])
def test_decode_token_major(dtype, D, Hq, Hkv, splits):
    w = S.Workload("strided", 110 + D + Hq, B=3, T=1000, Hq=Hq, Hkv=Hkv, D=D, dtype=dtype)
    k, v = S.cache_kv(w)
    q = S.queries(w)
    lens = [1000, 3, 517]
    kt, vt = dev(_token_major(k, 1040)), dev(_token_major(v, 1040))
    o, lse = _decode(dev(q), _view(kt), _view(vt), Hkv, w.T, splits, lens)
    o_ref, lse_ref = O.decode_attention(q, k, v, seq_lens=np.array(lens))
    _check(o, lse, o_ref, lse_ref, dtype)
    o_hm, lse_hm = _decode(dev(q), dev(k), dev(v), Hkv, w.T, splits, lens)
    assert np.array_equal(o, o_hm) and np.array_equal(lse, lse_hm)


def test_prefill_token_major():
    w = S.Workload("strided_pf", 120, B=2, T=700, Hq=16, Hkv=4, D=128, dtype="bf16")
    k, v = S.cache_kv(w)
    C, p0 = 300, 400
    q = S.queries(w, rows=C)
    kt, vt = dev(_token_major(k, 760)), dev(_token_major(v, 760))
    out = torch.empty((w.B, C, w.Hq, w.D), dtype=torch.float32, device="cuda")
    lse = torch.empty((w.B, w.Hq, C), dtype=torch.float32, device="cuda")
    Y.yoco_cross_attn_prefill(dev(q), _view(kt), _view(vt), p0, out, lse, Hkv=w.Hkv)
    out_hm = torch.empty_like(out)
    lse_hm = torch.empty_like(lse)
    Y.yoco_cross_attn_prefill(dev(q), dev(k), dev(v), p0, out_hm, lse_hm)
    torch.cuda.synchronize()
    rows = [0, 1, 63, 64, 150, C - 1]
    o_ref, lse_ref = O.causal_prefill(q, k, v, p0, rows=rows)
    _, lse2_ref = O.causal_prefill(bars.doubled(q), k, v, p0, rows=rows)
    o = host(out).astype(np.float64)
    r = bars.prefill_bf16(o[:, rows], host(lse)[:, :, rows], o_ref[:, rows], lse_ref[:, :, rows],
                          lse2_ref[:, :, rows])
    say("  " + bars.report(r))
    assert r["ok"], r
    assert np.array_equal(host(out), host(out_hm)) and np.array_equal(host(lse), host(lse_hm))


def test_compose_on_read_over_projection_layout():
    """The raw K_1, K_i, V_1, V_i as a QKV projection writes them, [B, T, Hkv, D]."""
    w = S.Workload("strided_cor", 125, B=2, T=900, Hq=8, Hkv=2, D=128, dtype="bf16")
    src = S.compose_sources(w, layer=6)            # token-major [B, T, Hkv, D]
    alpha = S.alphas(w.seed, 6)
    q = S.queries(w, layer=7)
    d = {n: dev(x) for n, x in src.items()}
    out = torch.empty((w.B, w.Hq, w.D), dtype=torch.float32, device="cuda")
    lse = torch.empty((w.B, w.Hq), dtype=torch.float32, device="cuda")
    Y.yoco_cross_attn_decode_compose_on_read(dev(q), *(Y.token_major(d[n]) for n in ("k1", "ki", "v1", "vi")), alpha,
                                             out, lse, T=w.T, Hkv=w.Hkv)
    torch.cuda.synchronize()
    o, l = host(out).astype(np.float64), host(lse).astype(np.float64)
    # over the exactly composed cache (compose rounding included): the stated 1e-2
    kp, vp = O.compose_kv(src["k1"], src["ki"], src["v1"], src["vi"], alpha)
    o_x, lse_x = O.decode_attention(q, kp.transpose(0, 2, 1, 3), vp.transpose(0, 2, 1, 3))
    assert np.max(np.abs(o - o_x)) <= bars.STATED_ATOL and np.max(np.abs(l - lse_x)) <= bars.STATED_ATOL
    # over the composition as the compose kernel stores it (the same arithmetic per row): the decode bars
    kc = torch.empty((w.B, w.Hkv, w.T, w.D), dtype=torch.bfloat16, device="cuda")
    vc = torch.empty_like(kc)
    Y.yoco_compose_kv(d["k1"], d["ki"], d["v1"], d["vi"], kc, vc, 0, alpha)
    torch.cuda.synchronize()
    o_ref, lse_ref = O.decode_attention(q, host(kc), host(vc))
    _check(o, l, o_ref, lse_ref, "bf16")


def test_self_decoder_step_token_major():
    w = S.Workload("strided_self", 130, B=2, T=600, Hq=8, Hkv=2, D=128, dtype="bf16")
    k, v = S.cache_kv(w)
    q = S.queries(w, layer=3)
    new = {n: x[:, 0] for n, x in S.compose_sources(w, layer=3, n=1).items()}
    alpha = S.alphas(w.seed, 3)
    lens = [600, 250]
    kt, vt = dev(_token_major(k, 640)), dev(_token_major(v, 640))
    out = torch.empty((w.B, w.Hq, w.D), dtype=torch.float32, device="cuda")
    lse = torch.empty((w.B, w.Hq), dtype=torch.float32, device="cuda")
    sl = torch.tensor(lens, dtype=torch.int32, device="cuda")
    Y.yoco_self_attn_decode(dev(q), *(dev(new[n]) for n in ("k1", "ki", "v1", "vi")), _view(kt), _view(vt), alpha,
                            out, lse, seq_lens=sl, T=w.T, Hkv=w.Hkv)
    # the same step on head-major copies gives the same bits, in the output and in the written rows
    kh, vh = dev(k), dev(v)
    out_hm, lse_hm = torch.empty_like(out), torch.empty_like(lse)
    Y.yoco_self_attn_decode(dev(q), *(dev(new[n]) for n in ("k1", "ki", "v1", "vi")), kh, vh, alpha, out_hm, lse_hm,
                            seq_lens=sl)
    torch.cuda.synchronize()
    assert np.array_equal(host(out), host(out_hm)) and np.array_equal(host(lse), host(lse_hm))
    kt_h, kh_h = host(kt), host(kh)
    for b, n in enumerate(lens):
        assert np.array_equal(kt_h[b, n - 1], kh_h[b, :, n - 1])
    o_ref, lse_ref, _, _ = O.self_attn_decode(q, k, v, new, alpha, seq_lens=np.array(lens))
    _check_output(host(out).astype(np.float64), host(lse).astype(np.float64), o_ref, lse_ref, "bf16",
                  _rounding_slack(q, o_ref, lse_ref, [(new, alpha)], "bf16"))
