"""GPU parity of the causal chunked prefill (bf16 MFMA) against the fp64 oracle.

Bar: bf16 inputs with fp32 accumulation within 1e-2 absolute on unit-scale
outputs (and on lse); the first row of a chunk at p0 = 0 is V[0] exactly."""
import numpy as np
import pytest
import torch

import cross_layer_shared_amd as Y
import oracle as O
from synthetic import inputs as S
from tests.gpu_util import dev, host, say

pytestmark = pytest.mark.gpu

ATOL = 1e-2


def _prefill(q, kc, vc, p0, out_dtype=torch.float32):
    B, C, Hq, D = q.shape
    out = torch.empty((B, C, Hq, D), dtype=out_dtype, device="cuda")
    lse = torch.empty((B, Hq, C), dtype=torch.float32, device="cuda")
    Y.yoco_cross_attn_prefill(q, kc, vc, p0, out, lse)
    torch.cuda.synchronize()
    o = host(out)
    o = o.astype(np.float64) if out_dtype == torch.float32 else O.to_f64(o)
    return o, host(lse).astype(np.float64)


def _inputs(B, C, Hq, Hkv, Tcap, seed, D=128):
    w = S.Workload("pf", seed, B=B, T=Tcap, Hq=Hq, Hkv=Hkv, D=D, dtype="bf16")
    k, v = S.cache_kv(w)
    q = S.queries(w, rows=C)
    return q, k, v


def _compare(o, lse, o_ref, lse_ref, rows=None, out_bf16=False):
    if rows is not None:
        o, o_ref, lse, lse_ref = o[:, rows], o_ref[:, rows], lse[:, :, rows], lse_ref[:, :, rows]
    err = np.max(np.abs(o - o_ref))
    lerr = np.max(np.abs(lse - lse_ref))
    say(f"  max|o-ref| {err:.3e}  /rms {err / np.sqrt(np.mean(o_ref ** 2)):.3e}  max|lse-ref| {lerr:.3e}")
    assert np.isfinite(o).all()
    # a bf16 output adds its own rounding (half a bf16 ulp, up to ~2e-2 for |o| near 4)
    tol = ATOL + (np.abs(o_ref) * 2.0 ** -8 if out_bf16 else 0.0)
    assert np.all(np.abs(o - o_ref) <= tol)
    assert lerr <= ATOL


@pytest.mark.parametrize("Hq,Hkv", [(8, 2), (4, 2), (2, 2), (16, 2), (32, 2)])
@pytest.mark.parametrize("C,p0", [(1, 0), (33, 0), (100, 5), (64, 64), (129, 300)])
def test_small_shapes(Hq, Hkv, C, p0):
    q, k, v = _inputs(2, C, Hq, Hkv, p0 + C + 7, 50 + C + p0 + Hq)
    o, lse = _prefill(dev(q), dev(k), dev(v), p0)
    o_ref, lse_ref = O.causal_prefill(q, k, v, p0)
    _compare(o, lse, o_ref, lse_ref)


@pytest.mark.parametrize("Hq,Hkv", [(8, 2), (32, 4), (4, 4), (32, 2)])
@pytest.mark.parametrize("C,p0", [(1, 0), (100, 5), (300, 500)])
def test_head_dim_64(Hq, Hkv, C, p0):
    """D = 64 (the head size of a TinyLlama-configured model): group sizes 4, 8,
    1 and 16, ragged chunks, several 128-key tiles."""
    q, k, v = _inputs(2, C, Hq, Hkv, p0 + C + 7, 80 + C + p0 + Hq, D=64)
    o, lse = _prefill(dev(q), dev(k), dev(v), p0)
    o_ref, lse_ref = O.causal_prefill(q, k, v, p0)
    _compare(o, lse, o_ref, lse_ref)


def test_head_dim_64_bf16_output():
    q, k, v = _inputs(1, 200, 8, 2, 260, 61, D=64)
    o, lse = _prefill(dev(q), dev(k), dev(v), 50, out_dtype=torch.bfloat16)
    o_ref, lse_ref = O.causal_prefill(q, k, v, 50)
    _compare(o, lse, o_ref, lse_ref, out_bf16=True)


def test_bf16_output():
    q, k, v = _inputs(1, 200, 8, 2, 260, 60)
    o, lse = _prefill(dev(q), dev(k), dev(v), 60, out_dtype=torch.bfloat16)
    o_ref, lse_ref = O.causal_prefill(q, k, v, 60)
    _compare(o, lse, o_ref, lse_ref, out_bf16=True)


def test_first_row_is_value_row():
    """At p0 = 0 the first query sees only row 0: o = V[0] bit for bit (fp32 out)."""
    q, k, v = _inputs(2, 70, 8, 2, 70, 61)
    o, _ = _prefill(dev(q), dev(k), dev(v), 0)
    for h in range(8):
        assert np.array_equal(o[:, 0, h], O.to_f64(v[:, h // 4, 0]))


def test_rows_equal_decode_and_early_exit():
    """Row at position p equals a decode over the first p+1 rows; the chunk's last
    row equals the decode at T = p0 + C (early exit leaves the output unchanged)."""
    B, C, Hq, Hkv, p0 = 2, 96, 8, 2, 40
    q, k, v = _inputs(B, C, Hq, Hkv, p0 + C, 62)
    qd, kd, vd = dev(q), dev(k), dev(v)
    o, lse = _prefill(qd, kd, vd, p0)
    for c in (0, 1, 31, 32, 63, 64, C - 1):
        out = torch.empty((B, Hq, 128), dtype=torch.float32, device="cuda")
        l = torch.empty((B, Hq), dtype=torch.float32, device="cuda")
        Y.yoco_cross_attn_decode(qd[:, c].contiguous(), kd, vd, out, l, T=p0 + c + 1, num_splits=2)
        torch.cuda.synchronize()
        assert np.max(np.abs(o[:, c] - host(out))) <= ATOL
        assert np.max(np.abs(lse[:, :, c] - host(l))) <= ATOL


def test_chunking_only_partitions_rows():
    """One call over all rows and chunked calls give the same rows (within the bar)."""
    B, T, Hq, Hkv = 1, 300, 8, 2
    q, k, v = _inputs(B, T, Hq, Hkv, T, 63)
    qd, kd, vd = dev(q), dev(k), dev(v)
    full, full_lse = _prefill(qd, kd, vd, 0)
    for c0, c1 in ((0, 100), (100, 164), (164, 300)):
        part, part_lse = _prefill(qd[:, c0:c1].contiguous(), kd, vd, c0)
        assert np.max(np.abs(part - full[:, c0:c1])) <= ATOL
        assert np.max(np.abs(part_lse - full_lse[:, :, c0:c1])) <= ATOL


def test_full_chunked_prefill_workload():
    """T=32768 in 8 chunks of 4096, 32/8 heads, D=128; >= 512 sampled rows,
    including the first and last row of every chunk."""
    w = S.PREFILL_CHUNKED
    k, v = S.cache_kv(w)
    q = S.queries(w, rows=w.T)
    kd, vd, qd = dev(k), dev(v), dev(q)
    out = torch.empty((w.B, w.T, w.Hq, w.D), dtype=torch.float32, device="cuda")
    lses = []
    for c0 in range(0, w.T, w.chunk):
        say(f"  chunk p0={c0}")
        l = torch.empty((w.B, w.Hq, w.chunk), dtype=torch.float32, device="cuda")
        Y.yoco_cross_attn_prefill(qd[:, c0:c0 + w.chunk], kd, vd, c0, out[:, c0:c0 + w.chunk], l)
        lses.append(l)
    torch.cuda.synchronize()
    o = host(out).astype(np.float64)
    lse = np.concatenate([host(l) for l in lses], axis=2).astype(np.float64)
    assert np.isfinite(o).all() and np.isfinite(lse).all()
    r = np.random.default_rng(4)
    rows = set(r.choice(w.T, 496, replace=False).tolist())
    for c0 in range(0, w.T, w.chunk):
        rows |= {c0, c0 + w.chunk - 1}
    rows = sorted(rows)
    say(f"  {len(rows)} sampled rows")
    o_ref, lse_ref = O.causal_prefill(q, k, v, 0, rows=rows)
    _compare(o, lse, o_ref, lse_ref, rows=rows)


@pytest.mark.parametrize("case", range(12))
def test_random_shapes(case):
    """Seeded random shapes: batch 1-3, 1-4 kv heads, group sizes 1-8, D = 64 or
    128, chunks of 1-300 rows at offsets 0-400 in caches with spare rows, so
    tile counts, ragged query blocks and both wavefront schedules (staggered
    at D = 128, in step at D = 64) vary together."""
    r = np.random.default_rng(1000 + case)
    B = int(r.integers(1, 4))
    Hkv = int(r.choice([1, 2, 4]))
    G = int(r.choice([1, 2, 4, 8]))
    D = int(r.choice([64, 128]))
    C = int(r.integers(1, 301))
    p0 = int(r.integers(0, 401))
    spare = int(r.integers(0, 21))
    say(f"  B={B} Hkv={Hkv} G={G} D={D} C={C} p0={p0} spare={spare}")
    q, k, v = _inputs(B, C, Hkv * G, Hkv, p0 + C + spare, 2000 + case, D=D)
    o, lse = _prefill(dev(q), dev(k), dev(v), p0)
    o_ref, lse_ref = O.causal_prefill(q, k, v, p0)
    _compare(o, lse, o_ref, lse_ref)
