"""The allocation-free decode (yoco_cross_attn_decode_noalloc, partials and
merge counters in the library's per-GPU scratch array) against the decode
that takes a workspace (yoco_cross_attn_decode): the same kernels, so the
results must agree bit for bit, and both must meet the oracle's bars. Calls
come in a row on one GPU, the second with a smaller input than the first,
then larger ones again (the scratch array keeps what the last call left)."""
import numpy as np
import pytest
import torch

import cross_layer_shared_amd as Y
import oracle as O
from synthetic import inputs as S
from tests import bars
from tests.gpu_util import dev, host, rowwise_rel, say

pytestmark = pytest.mark.gpu


def _pair(B, T, Hq, Hkv, D, dtype, seed, splits, lens=None):
    w = S.Workload("noalloc", seed, B=B, T=T, Hq=Hq, Hkv=Hkv, D=D, dtype=dtype)
    k, v = S.cache_kv(w)
    q = S.queries(w)
    qd, kd, vd = dev(q), dev(k), dev(v)
    sl = None if lens is None else torch.tensor(lens, dtype=torch.int32, device="cuda")
    o_ws = torch.empty((B, Hq, D), dtype=torch.float32, device="cuda")
    l_ws = torch.empty((B, Hq), dtype=torch.float32, device="cuda")
    o_na, l_na = torch.empty_like(o_ws), torch.empty_like(l_ws)
    Y.yoco_cross_attn_decode(qd, kd, vd, o_ws, l_ws, seq_lens=sl, num_splits=splits)
    Y.yoco_cross_attn_decode_noalloc(qd, kd, vd, o_na, l_na, seq_lens=sl, num_splits=splits)
    torch.cuda.synchronize()
    return q, k, v, host(o_ws), host(l_ws), host(o_na), host(l_na)


def _check(q, k, v, o_ws, l_ws, o_na, l_na, dtype, lens=None):
    assert np.array_equal(o_na, o_ws) and np.array_equal(l_na, l_ws)
    o_ref, lse_ref = O.decode_attention(q, k, v, seq_lens=None if lens is None else np.array(lens))
    o, l = o_na.astype(np.float64), l_na.astype(np.float64)
    if dtype == "f32":
        assert rowwise_rel(o, o_ref) <= 1e-5
        assert np.max(np.abs(l - lse_ref) / np.maximum(1.0, np.abs(lse_ref))) <= 1e-5
    else:
        r = bars.decode_bf16(o, l, o_ref, lse_ref)
        say("  " + bars.report(r))
        assert r["ok"], r


# (B, T, Hq, Hkv, D, dtype, seed, splits, lens): the mid-context decode, then smaller
# calls (fewer sequences and kv heads, other split counts, ragged lengths, fp32),
# then larger ones again
CALLS = [
    (8, 4096, 32, 8, 128, "bf16", 300, 0, None),
    (2, 1000, 8, 2, 64, "bf16", 301, 7, [1000, 333]),
    (1, 300, 4, 1, 64, "f32", 302, 3, None),
    (4, 2048, 16, 4, 128, "bf16", 303, 16, None),
    (8, 4096, 32, 8, 128, "bf16", 304, 0, None),
]


def test_noalloc_equals_workspace_decode_on_consecutive_calls():
    for B, T, Hq, Hkv, D, dtype, seed, splits, lens in CALLS:
        say(f"  B={B} T={T} Hq={Hq} Hkv={Hkv} D={D} {dtype} splits={splits} lens={lens}")
        res = _pair(B, T, Hq, Hkv, D, dtype, seed, splits, lens)
        _check(*res, dtype, lens)


def test_noalloc_two_calls_in_a_row_second_smaller():
    """Back to back on one stream with no synchronisation between them."""
    first = (8, 4096, 32, 8, 128, 310)
    second = (2, 777, 8, 2, 128, 311)
    outs = []
    for B, T, Hq, Hkv, D, seed in (first, second):
        w = S.Workload("noalloc2", seed, B=B, T=T, Hq=Hq, Hkv=Hkv, D=D, dtype="bf16")
        k, v = S.cache_kv(w)
        q = S.queries(w)
        qd, kd, vd = dev(q), dev(k), dev(v)
        o = torch.empty((B, Hq, D), dtype=torch.float32, device="cuda")
        l = torch.empty((B, Hq), dtype=torch.float32, device="cuda")
        Y.yoco_cross_attn_decode_noalloc(qd, kd, vd, o, l)
        outs.append((q, k, v, qd, kd, vd, o, l))
    torch.cuda.synchronize()
    for q, k, v, qd, kd, vd, o, l in outs:
        o_ws, l_ws = torch.empty_like(o), torch.empty_like(l)
        Y.yoco_cross_attn_decode(qd, kd, vd, o_ws, l_ws)
        torch.cuda.synchronize()
        _check(q, k, v, host(o_ws), host(l_ws), host(o), host(l), "bf16")


def test_noalloc_rejects_calls_beyond_the_scratch_array():
    q = torch.empty((64, 64, 128), dtype=torch.bfloat16, device="cuda")
    kc = torch.empty((64, 64, 64, 128), dtype=torch.bfloat16, device="cuda")
    out = torch.empty((64, 64, 128), dtype=torch.float32, device="cuda")
    with pytest.raises(Y.YocoError) as e:   # 64 * 64 * 16 * 129 * 4 bytes of partials > 8 MiB
        Y.yoco_cross_attn_decode_noalloc(q, kc, kc, out, num_splits=16)
    assert e.value.status == 4 and "scratch" in str(e.value)
