"""GPU parity of the split-K decode (yoco_cross_attn_decode, its split pass and
merge) against the fp64 oracle.

Bar: fp32 caches within 1e-5 (per (b, h) row: ||o - o_ref||_inf <= 1e-5 ||o_ref||_inf,
lse within 1e-5 relative); bf16 caches with fp32 accumulation: every output
row within 1e-3 of its rms and lse within 1e-4 absolute, besides the stated
1e-2 absolute (the derivation is in tests/bars.py)."""
import numpy as np
import pytest
import torch

import cross_layer_shared_amd as Y
import oracle as O
from synthetic import inputs as S
from tests import bars
from tests.gpu_util import dev, host, rowwise_rel, say

pytestmark = pytest.mark.gpu

BF16_ATOL = 1e-2
F32_RTOL = 1e-5


def _decode(q, k, v, splits=0, seq_lens=None, T=None):
    B, Hq, D = q.shape
    out = torch.empty((B, Hq, D), dtype=torch.float32, device="cuda")
    lse = torch.empty((B, Hq), dtype=torch.float32, device="cuda")
    sl = None if seq_lens is None else torch.tensor(seq_lens, dtype=torch.int32, device="cuda")
    Y.yoco_cross_attn_decode(q, k, v, out, lse, seq_lens=sl, T=T, num_splits=splits)
    torch.cuda.synchronize()
    return host(out).astype(np.float64), host(lse).astype(np.float64)


def _compare(o, lse, o_ref, lse_ref, dtype, mask=None):
    if mask is not None:
        o, lse, o_ref, lse_ref = o[mask], lse[mask], o_ref[mask], lse_ref[mask]
    if dtype == "f32":
        say(f"  row-rel {rowwise_rel(o, o_ref):.3e}  max|lse-ref| {np.max(np.abs(lse - lse_ref)):.3e}")
        assert rowwise_rel(o, o_ref) <= F32_RTOL
        assert np.max(np.abs(lse - lse_ref) / np.maximum(1.0, np.abs(lse_ref))) <= F32_RTOL
    else:
        r = bars.decode_bf16(o, lse, o_ref, lse_ref)
        say("  " + bars.report(r))
        assert r["ok"], r


def _inputs(B, T, Hq, Hkv, D, dtype, seed, q_std=1.0):
    w = S.Workload("case", seed, B=B, T=T, Hq=Hq, Hkv=Hkv, D=D, dtype=dtype)
    k, v = S.cache_kv(w)
    q = S.queries(w, std=q_std)
    return q, k, v


# ------------------------------------------------------------- tiny fp32 stack

@pytest.mark.parametrize("splits", [1, 2, 7, 0])
def test_tiny_fp32_stack_end_to_end(splits):
    """Compose layer 2 of a 4-layer stack, then one decode query per cross layer
    (layers 3 and 4) over the shared K'_2, V'_2."""
    w = S.TINY_FP32_STACK
    src = S.compose_sources(w, layer=2)
    alpha = S.alphas(w.seed, 2)
    kc = torch.zeros((1, 1, w.T, w.D), dtype=torch.float32, device="cuda")
    vc = torch.zeros_like(kc)
    d = {k: dev(x) for k, x in src.items()}
    Y.yoco_compose_kv(d["k1"], d["ki"], d["v1"], d["vi"], kc, vc, 0, alpha)
    k_ref, v_ref = O.compose_kv(src["k1"], src["ki"], src["v1"], src["vi"], alpha)
    k_ref, v_ref = k_ref.transpose(0, 2, 1, 3), v_ref.transpose(0, 2, 1, 3)   # -> [B, Hkv, T, D]
    # The oracle attends over the exact composed cache; the GPU over its fp32
    # rounding, which moves the result by far less than the 1e-5 bar.
    for layer in (3, 4):
        q = S.queries(w, layer=layer)
        o, lse = _decode(dev(q), kc, vc, splits)
        o_ref, lse_ref = O.decode_attention(q, k_ref, v_ref)
        _compare(o, lse, o_ref, lse_ref, "f32")


def test_yoco_plus_plus_at_init_equals_yoco():
    """Decode over compose(identity init) equals decode over the raw K_i, V_i bit for bit."""
    w = S.TINY_FP32_STACK
    src = S.compose_sources(w, layer=2)
    kc = torch.zeros((1, 1, w.T, w.D), dtype=torch.float32, device="cuda")
    vc = torch.zeros_like(kc)
    d = {k: dev(x) for k, x in src.items()}
    Y.yoco_compose_kv(d["k1"], d["ki"], d["v1"], d["vi"], kc, vc, 0, S.IDENTITY_ALPHA)
    raw_k = d["ki"].transpose(1, 2).contiguous()
    raw_v = d["vi"].transpose(1, 2).contiguous()
    q = dev(S.queries(w, layer=3))
    o1, l1 = _decode(q, kc, vc)
    o2, l2 = _decode(q, raw_k, raw_v)
    assert np.array_equal(o1, o2) and np.array_equal(l1, l2)


# ------------------------------------------------------------- shapes, tails, splits

@pytest.mark.parametrize("T", [1, 63, 65, 1000, 4097])
@pytest.mark.parametrize("splits", [1, 2, 7, 0])
def test_bf16_tails_and_splits(T, splits):
    q, k, v = _inputs(2, T, 8, 2, 128, "bf16", 20 + T)
    if splits > T:   # more splits than rows: rejected before anything is enqueued
        with pytest.raises(Y.YocoError) as e:
            _decode(dev(q), dev(k), dev(v), splits)
        assert e.value.status == 1   # YOCO_ERR_INVALID_ARG
        return
    o, lse = _decode(dev(q), dev(k), dev(v), splits)
    o_ref, lse_ref = O.decode_attention(q, k, v)
    _compare(o, lse, o_ref, lse_ref, "bf16")


@pytest.mark.parametrize("G", [1, 2, 4, 8, 16])
@pytest.mark.parametrize("D,dtype", [(64, "bf16"), (128, "bf16"), (64, "f32"), (128, "f32")])
def test_group_sizes_and_head_dims(G, D, dtype):
    Hkv = 2
    q, k, v = _inputs(2, 777, G * Hkv, Hkv, D, dtype, 30 + G + D)
    o, lse = _decode(dev(q), dev(k), dev(v), 3)
    o_ref, lse_ref = O.decode_attention(q, k, v)
    _compare(o, lse, o_ref, lse_ref, dtype)


@pytest.mark.parametrize("case", range(12))
def test_random_shapes(case):
    """Seeded random shapes: batch 1-4, 1-4 kv heads, group sizes 1-16, D = 64
    or 128, bf16 or fp32 caches, 1-3000 rows, automatic or explicit split
    counts, and per-sequence lengths on every other case."""
    r = np.random.default_rng(3000 + case)
    B = int(r.integers(1, 5))
    Hkv = int(r.integers(1, 5))
    G = int(r.choice([1, 2, 4, 8, 16]))
    D = int(r.choice([64, 128]))
    dtype = str(r.choice(["bf16", "f32"]))
    T = int(r.integers(1, 3001))
    splits = 0 if case % 3 == 0 else int(r.integers(1, min(T, 16) + 1))
    lens = [int(x) for x in r.integers(1, T + 1, size=B)] if case % 2 else None
    say(f"  B={B} Hkv={Hkv} G={G} D={D} {dtype} T={T} splits={splits} lens={lens}")
    q, k, v = _inputs(B, T, G * Hkv, Hkv, D, dtype, 4000 + case)
    o, lse = _decode(dev(q), dev(k), dev(v), splits, seq_lens=lens)
    o_ref, lse_ref = O.decode_attention(q, k, v, seq_lens=None if lens is None else np.array(lens))
    _compare(o, lse, o_ref, lse_ref, dtype)


@pytest.mark.parametrize("splits", [1, 5, 0])
def test_ragged_seq_lens(splits):
    """Per-sequence lengths (clamped to [1, T] on the device); rows past a length never matter."""
    B, T = 5, 1500
    q, k, v = _inputs(B, T, 8, 2, 128, "bf16", 40)
    lens = [1500, 1, 700, 1499, 2000]           # the last is clamped to T
    o, lse = _decode(dev(q), dev(k), dev(v), splits, seq_lens=lens)
    o_ref, lse_ref = O.decode_attention(q, k, v, seq_lens=np.minimum(lens, T))
    _compare(o, lse, o_ref, lse_ref, "bf16")


def test_gqa_equals_mha_on_repeated_kv():
    q, k, v = _inputs(2, 300, 8, 2, 128, "bf16", 41)
    o1, l1 = _decode(dev(q), dev(k), dev(v), 4)
    k4, v4 = np.repeat(k, 4, axis=1), np.repeat(v, 4, axis=1)
    o2, l2 = _decode(dev(q), dev(k4), dev(v4), 4)
    assert np.max(np.abs(o1 - o2)) <= 1e-6 and np.max(np.abs(l1 - l2)) <= 1e-6


def test_row_permutation_invariance():
    q, k, v = _inputs(1, 999, 4, 1, 128, "bf16", 42)
    perm = np.random.default_rng(0).permutation(999)
    o1, l1 = _decode(dev(q), dev(k), dev(v), 5)
    o2, l2 = _decode(dev(q), dev(np.ascontiguousarray(k[:, :, perm])), dev(np.ascontiguousarray(v[:, :, perm])), 5)
    assert np.max(np.abs(o1 - o2)) <= 1e-5 and np.max(np.abs(l1 - l2)) <= 1e-5


def test_split_pass_and_merge_entry_points():
    """The split pass alone writes per-split (o_s, lse_s) equal to the oracle over
    each split's rows; the merge of those equals the full decode."""
    B, T, Hq, Hkv, D, S_ = 2, 1000, 8, 2, 128, 4
    q, k, v = _inputs(B, T, Hq, Hkv, D, "bf16", 43)
    ws = Y.decode_workspace(B, T, Hq, Hkv, D, S_)
    qd, kd, vd = dev(q), dev(k), dev(v)
    Y.yoco_cross_attn_decode_partial(qd, kd, vd, ws, S_)
    torch.cuda.synchronize()
    rows = B * Hq * S_
    o_off = (B * Hkv * 4 + 15) // 16 * 4           # counters first, in float32 units
    part_o = host(ws[o_off: o_off + rows * D]).reshape(B, Hq, S_, D)
    part_l = host(ws[o_off + rows * D: o_off + rows * D + rows]).reshape(B, Hq, S_)
    rps = 256                                    # ceil(1000/4) = 250 rounded up to 16
    for s in range(S_):
        t0, t1 = s * rps, min(T, (s + 1) * rps)
        o_ref, l_ref = O.decode_attention(q, k[:, :, t0:t1], v[:, :, t0:t1])
        _compare(part_o[:, :, s].astype(np.float64), part_l[:, :, s].astype(np.float64), o_ref, l_ref, "bf16")
    out = torch.empty((B, Hq, D), dtype=torch.float32, device="cuda")
    lse = torch.empty((B, Hq), dtype=torch.float32, device="cuda")
    Y.yoco_decode_merge(ws, B, Hq, Hkv, D, S_, out, lse)
    torch.cuda.synchronize()
    o_ref, l_ref = O.decode_attention(q, k, v)
    _compare(host(out).astype(np.float64), host(lse).astype(np.float64), o_ref, l_ref, "bf16")


def test_fused_merge_reuses_one_workspace():
    """One zero-filled workspace serves successive calls whose T and split count
    change: the counters lead the workspace and every call leaves them at zero."""
    B, Hq, Hkv, D = 3, 8, 2, 128
    ws = Y.decode_workspace(B, 3000, Hq, Hkv, D, 32)
    o_off = (B * Hkv * 4 + 15) // 16 * 4
    for i, (T, S_) in enumerate([(3000, 32), (1000, 7), (3000, 0), (64, 4), (2500, 19), (2500, 19)]):
        q, k, v = _inputs(B, T, Hq, Hkv, D, "bf16", 70 + i)
        out = torch.empty((B, Hq, D), dtype=torch.float32, device="cuda")
        lse = torch.empty((B, Hq), dtype=torch.float32, device="cuda")
        Y.yoco_cross_attn_decode(dev(q), dev(k), dev(v), out, lse, num_splits=S_, workspace=ws)
        torch.cuda.synchronize()
        assert torch.all(ws[:o_off].view(torch.int32) == 0)
        o_ref, lse_ref = O.decode_attention(q, k, v)
        _compare(host(out).astype(np.float64), host(lse).astype(np.float64), o_ref, lse_ref, "bf16")


def test_workspace_reused_for_more_counters_after_rezeroing():
    """A call with one (sequence, kv head) leaves its partials right after its
    single counter; before a call with 64 counters reuses the workspace, the
    bytes between the two counter sections are zeroed, as the header asks."""
    ws = Y.decode_workspace(8, 4096, 32, 8, 128, 32)
    small = _inputs(1, 4096, 4, 1, 128, "bf16", 77)
    big = _inputs(8, 4096, 32, 8, 128, "bf16", 78)
    for (q, k, v), S_, rezero in ((small, 32, None), (big, 32, (1, 64)), (small, 8, None), (big, 4, (1, 64))):
        if rezero is not None:
            ws[rezero[0]:rezero[1]].zero_()
        B, Hq = q.shape[0], q.shape[1]
        out = torch.empty((B, Hq, 128), dtype=torch.float32, device="cuda")
        lse = torch.empty((B, Hq), dtype=torch.float32, device="cuda")
        Y.yoco_cross_attn_decode(dev(q), dev(k), dev(v), out, lse, num_splits=S_, workspace=ws)
        torch.cuda.synchronize()
        assert torch.all(ws[:B * k.shape[1]].view(torch.int32) == 0)
        o_ref, lse_ref = O.decode_attention(q, k, v)
        _compare(host(out).astype(np.float64), host(lse).astype(np.float64), o_ref, lse_ref, "bf16")


def test_binding_default_workspace_follows_the_counters():
    """Without a workspace argument the binding keeps one per (device, stream) and
    zeroes the counters a larger call adds; sizes grow and shrink on one stream."""
    for i, (B, Hkv, S_) in enumerate([(1, 1, 16), (4, 2, 8), (2, 2, 32), (8, 8, 4), (1, 1, 64), (8, 8, 0)]):
        q, k, v = _inputs(B, 2000, 4 * Hkv, Hkv, 128, "bf16", 120 + i)
        o, lse = _decode(dev(q), dev(k), dev(v), S_)
        o_ref, lse_ref = O.decode_attention(q, k, v)
        _compare(o, lse, o_ref, lse_ref, "bf16")


def test_concurrent_streams_with_their_own_workspaces():
    """Decodes enqueued on four streams at once, each with its own workspace:
    their fused merges count tickets independently, and every result equals the
    same call made alone."""
    B, Hq, Hkv, D, T, splits = 4, 16, 4, 128, 2048, 8
    cases = [_inputs(B, T, Hq, Hkv, D, "bf16", 90 + i) for i in range(4)]
    qs = [(dev(q), dev(k), dev(v)) for q, k, v in cases]
    alone = []
    for q, k, v in qs:
        o, l = _decode(q, k, v, splits)
        alone.append((o, l))
    streams = [torch.cuda.Stream() for _ in qs]
    wss = [Y.decode_workspace(B, T, Hq, Hkv, D, splits) for _ in qs]
    outs = [torch.empty((B, Hq, D), dtype=torch.float32, device="cuda") for _ in qs]
    lses = [torch.empty((B, Hq), dtype=torch.float32, device="cuda") for _ in qs]
    torch.cuda.synchronize()
    for rep in range(3):
        for (q, k, v), s, ws, o, l in zip(qs, streams, wss, outs, lses):
            Y.yoco_cross_attn_decode(q, k, v, o, l, num_splits=splits, workspace=ws, stream=s)
        torch.cuda.synchronize()
        for (o_a, l_a), o, l in zip(alone, outs, lses):
            assert np.array_equal(host(o).astype(np.float64), o_a) and np.array_equal(host(l).astype(np.float64), l_a)
    for (q, k, v), (o_a, l_a) in zip(cases, alone):
        o_ref, lse_ref = O.decode_attention(q, k, v)
        _compare(o_a, l_a, o_ref, lse_ref, "bf16")


def test_identical_keys_give_mean_value():
    q, k, v = _inputs(1, 2048, 4, 1, 128, "bf16", 44)
    k[:] = k[:, :, :1]
    o, _ = _decode(dev(q), dev(k), dev(v))
    mean = O.to_f64(v)[0, 0].mean(axis=0)
    assert np.max(np.abs(o[0] - mean[None, :])) <= 1e-4


# ------------------------------------------------------------- full-size workloads

def test_decode_mid_context_full():
    """B=8, T=4096, 32/8 heads, D=128: all 16 cross layers over the same cache, all heads checked."""
    w = S.DECODE_MID
    k, v = S.cache_kv(w)
    kd, vd = dev(k), dev(v)
    for layer in range(w.layers):
        q = S.queries(w, layer=layer, std=w.notes["q_std"])
        o, lse = _decode(dev(q), kd, vd)
        o_ref, lse_ref = O.decode_attention(q, k, v)
        say(f"  layer {layer}:")
        _compare(o, lse, o_ref, lse_ref, "bf16")


@pytest.mark.slow
def test_decode_long_context_full():
    """B=4, T=131072, 32/8 heads, 1% of key rows scaled x8 (peaked softmax); all 128 heads."""
    w = S.DECODE_LONG
    k, v = S.cache_kv(w)
    S.scale_key_rows_bf16(k, S.scaled_rows(w), w.notes["scale"])
    q = S.queries(w)
    o, lse = _decode(dev(q), dev(k), dev(v))
    o_ref, lse_ref = O.decode_attention(q, k, v)          # every (sequence, head)
    _compare(o, lse, o_ref, lse_ref, "bf16")


@pytest.mark.slow
def test_decode_million_token_planted_row():
    """B=1, T=2^20, 16/4 heads: one key row = 4*q at a seeded position dominates its head."""
    w = S.DECODE_MILLION
    k, v = S.cache_kv(w)
    q = S.queries(w)
    t_star = S.planted_position(w)
    S.plant_query_row_bf16(k, q, t_star, w.notes["plant_scale"])
    o, lse = _decode(dev(q), dev(k), dev(v))
    G = w.G
    o_ref, lse_ref = O.decode_attention(q, k, v)          # all 16 heads
    _compare(o, lse, o_ref, lse_ref, "bf16")
    for g in range(w.Hkv):
        planted = O.to_f64(v[0, g, t_star])
        say(f"  head {g * G}: max|o - V[t*]| = {np.max(np.abs(o[0, g * G] - planted)):.3e}")
        assert np.max(np.abs(o[0, g * G] - planted)) <= BF16_ATOL
