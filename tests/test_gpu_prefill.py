"""GPU parity of the causal chunked prefill (bf16 MFMA) against the fp64 oracle.

Bar (derived in tests/bars.py from the bf16 rounding of the probabilities):
every output row within 2e-2 of its rms, lse within 8 standard deviations of
that rounding's effect (at most 2^-8) plus 1e-4, besides the stated 1e-2
absolute; the first row of a chunk at p0 = 0 is V[0] exactly."""
import numpy as np
import pytest
import torch

import cross_layer_shared_amd as Y
import oracle as O
from synthetic import inputs as S
from tests import bars
from tests.gpu_util import dev, host, say

pytestmark = pytest.mark.gpu


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


def _oracle(q, k, v, p0, rows=None):
    """The oracle's o and lse, and its lse for the doubled query (sum of squared weights)."""
    o_ref, lse_ref = O.causal_prefill(q, k, v, p0, rows=rows)
    _, lse2_ref = O.causal_prefill(bars.doubled(q), k, v, p0, rows=rows)
    return o_ref, lse_ref, lse2_ref


def _compare(o, lse, ref, rows=None, out_bf16=False):
    o_ref, lse_ref, lse2_ref = ref
    if rows is not None:
        o, o_ref = o[:, rows], o_ref[:, rows]
        lse, lse_ref, lse2_ref = lse[:, :, rows], lse_ref[:, :, rows], lse2_ref[:, :, rows]
    assert np.isfinite(o).all()
    r = bars.prefill_bf16(o, lse, o_ref, lse_ref, lse2_ref, out_bf16=out_bf16)
    say("  " + bars.report(r))
    assert r["ok"], r


@pytest.mark.parametrize("Hq,Hkv", [(8, 2), (4, 2), (2, 2), (16, 2), (32, 2)])
@pytest.mark.parametrize("C,p0", [(1, 0), (33, 0), (100, 5), (64, 64), (129, 300)])
def test_small_shapes(Hq, Hkv, C, p0):
    q, k, v = _inputs(2, C, Hq, Hkv, p0 + C + 7, 50 + C + p0 + Hq)
    o, lse = _prefill(dev(q), dev(k), dev(v), p0)
    _compare(o, lse, _oracle(q, k, v, p0))


@pytest.mark.parametrize("Hq,Hkv", [(8, 2), (32, 4), (4, 4), (32, 2)])
@pytest.mark.parametrize("C,p0", [(1, 0), (100, 5), (300, 500)])
def test_head_dim_64(Hq, Hkv, C, p0):
    """D = 64 (the head size of a TinyLlama-configured model): group sizes 4, 8,
    1 and 16, ragged chunks, several 128-key tiles."""
    q, k, v = _inputs(2, C, Hq, Hkv, p0 + C + 7, 80 + C + p0 + Hq, D=64)
    o, lse = _prefill(dev(q), dev(k), dev(v), p0)
    _compare(o, lse, _oracle(q, k, v, p0))


def test_head_dim_64_bf16_output():
    q, k, v = _inputs(1, 200, 8, 2, 260, 61, D=64)
    o, lse = _prefill(dev(q), dev(k), dev(v), 50, out_dtype=torch.bfloat16)
    _compare(o, lse, _oracle(q, k, v, 50), out_bf16=True)


def test_bf16_output():
    q, k, v = _inputs(1, 200, 8, 2, 260, 60)
    o, lse = _prefill(dev(q), dev(k), dev(v), 60, out_dtype=torch.bfloat16)
    _compare(o, lse, _oracle(q, k, v, 60), out_bf16=True)


def test_first_row_is_value_row():
    """At p0 = 0 the first query sees only row 0: o = V[0] bit for bit (fp32 out)."""
    q, k, v = _inputs(2, 70, 8, 2, 70, 61)
    o, _ = _prefill(dev(q), dev(k), dev(v), 0)
    for h in range(8):
        assert np.array_equal(o[:, 0, h], O.to_f64(v[:, h // 4, 0]))


def test_rows_equal_decode_and_early_exit():
    """Row at position p equals a decode over the first p+1 rows; the chunk's last
    row equals the decode at T = p0 + C (early exit leaves the output unchanged).
    Each is within its bar of the oracle, and the two within the prefill bar of
    each other (the decode keeps its probabilities in fp32)."""
    B, C, Hq, Hkv, p0 = 2, 96, 8, 2, 40
    q, k, v = _inputs(B, C, Hq, Hkv, p0 + C, 62)
    qd, kd, vd = dev(q), dev(k), dev(v)
    o, lse = _prefill(qd, kd, vd, p0)
    ref = _oracle(q, k, v, p0)
    for c in (0, 1, 31, 32, 63, 64, C - 1):
        out = torch.empty((B, Hq, 128), dtype=torch.float32, device="cuda")
        l = torch.empty((B, Hq), dtype=torch.float32, device="cuda")
        Y.yoco_cross_attn_decode(qd[:, c].contiguous(), kd, vd, out, l, T=p0 + c + 1, num_splits=2)
        torch.cuda.synchronize()
        od, ld = host(out).astype(np.float64), host(l).astype(np.float64)
        rd = bars.decode_bf16(od, ld, ref[0][:, c], ref[1][:, :, c])
        assert rd["ok"], rd
        rp = bars.prefill_bf16(o[:, c], lse[:, :, c], od, ld, ref[2][:, :, c])
        say(f"  row {c}: decode vs oracle {bars.report(rd)}; prefill vs decode {bars.report(rp)}")
        assert rp["ok"], rp


def test_chunking_only_partitions_rows():
    """One call over all rows and chunked calls give the same rows: each within the
    bar of the oracle, and within twice the output bar of each other."""
    B, T, Hq, Hkv = 1, 300, 8, 2
    q, k, v = _inputs(B, T, Hq, Hkv, T, 63)
    qd, kd, vd = dev(q), dev(k), dev(v)
    full, full_lse = _prefill(qd, kd, vd, 0)
    _compare(full, full_lse, _oracle(q, k, v, 0))
    for c0, c1 in ((0, 100), (100, 164), (164, 300)):
        part, part_lse = _prefill(qd[:, c0:c1].contiguous(), kd, vd, c0)
        _compare(part, part_lse, _oracle(q[:, c0:c1], k, v, c0))
        assert np.max(bars.normalised_errors(part, full[:, c0:c1])) <= 2 * bars.PREFILL_REL


def test_full_chunked_prefill_workload():
    """T=32768 in 8 chunks of 4096, 32/8 heads, D=128; 768 distinct sampled rows,
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
    # 768 distinct rows: every chunk's first and last row and a seeded sample of the others
    ends = sorted({c0 for c0 in range(0, w.T, w.chunk)} | {c0 + w.chunk - 1 for c0 in range(0, w.T, w.chunk)})
    others = np.setdiff1d(np.arange(w.T), ends)
    r = np.random.default_rng(4)
    rows = sorted(set(ends) | set(r.choice(others, 768 - len(ends), replace=False).tolist()))
    assert len(rows) == 768
    say(f"  {len(rows)} sampled rows")
    _compare(o, lse, _oracle(q, k, v, 0, rows=rows), rows=rows)


@pytest.mark.parametrize("D,Hq,Hkv", [(128, 8, 2), (128, 4, 2), (128, 4, 4), (64, 8, 2)])
def test_reference_moves_differ_between_queries(D, Hq, Hkv):
    """Key rows scaled by 4 to 32 (exact powers of two) before and inside the
    chunk make each query's running maximum jump several times, by amounts and
    at steps that differ between the queries of one wavefront (the sign of
    each query's product with a scaled row is its own), so the lazy rescale of
    the numerator and the normaliser runs with a separate factor per query.
    The other cases rarely move the reference after its first value."""
    B, p0, C = 1, 700, 300
    w = S.Workload("pf_moves", 77, B=B, T=p0 + C, Hq=Hq, Hkv=Hkv, D=D, dtype="bf16")
    k, v = S.cache_kv(w)
    for f, rows in [(4, [90, 400]), (8, [250, 760]), (16, [520, 880]), (32, [690, 950])]:
        S.scale_key_rows_bf16(k, np.array([rows]), float(f))
    q = S.queries(w, rows=C)
    o, lse = _prefill(dev(q), dev(k), dev(v), p0)
    _compare(o, lse, _oracle(q, k, v, p0))


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
    _compare(o, lse, _oracle(q, k, v, p0))
