"""Plain fp64 CPU oracle for cross-layer KV sharing (YOCO and YOCO++).

TEST INFRASTRUCTURE. Only the tests, the smoke check and the CPU-baseline
leg of the benchmark import this module. The product path (the HIP library
and its Python binding) never calls it, and this module imports nothing from
the product: it shares no code, constant or helper with the HIP kernels.

Every function is the plain definition of what the method computes, in
float64, on the exact values the GPU receives (bf16 bit patterns are widened
exactly). There is no tiling, no online softmax and no split of the key
axis: attention materialises the full score vector of a query and runs the
two-pass softmax. Loops over key blocks exist only to widen stored values
to fp64 without holding a whole 1M-token cache in fp64 at once.

Sources:
  [YOCO++] "YOCO++: Enhancing YOCO with KV Residual Connections for Efficient
           LLM Inference" (gist.science technical summary), section 2
           (methodology, core mechanism: the K'_i / V'_i equations and the
           reuse of the middle layer's composed KVs by the upper half),
           "key technical innovations" items 1-3 (cache the composed KVs;
           lambda > 1, set to 35; initialisation alpha_{i,1} = 0,
           alpha_{i,2} = 1/lambda), section 3 (decode reads one KV set).
  [YOCO]   "You Only Cache Once: Decoder-Decoder Architectures for Language
           Models" (shd-paper.top summary), abstract and method details: the
           cross-decoder reuses the global KV cache through cross-attention
           and end to end the model works as a decoder-only Transformer does.

Readings where the pages are silent (each is listed with its reason in the
design notes of the repository):
  * alpha holds four scalars per lower-half layer ([YOCO++] section 3 counts
    4 learnable weights per layer); lambda is a fixed constant.
  * Attention is scaled dot-product softmax attention with scale 1/sqrt(D)
    ([YOCO] abstract: end to end the model works as a decoder-only Transformer does).
  * Grouped-query heads: query head h reads kv head floor(h / (Hq/Hkv)).
  * A decode query attends to every cache row [0, T), which includes the
    current token, whose composed KV the self-decoder has just written.
  * Causal prefill: the query at absolute position p attends to rows [0, p]
    inclusive; the chunk only partitions query rows.
  * lse is the natural-log log-sum-exp of the scaled scores.
  * A self-decoder decode step (the lower half keeps L/2 caches, [YOCO++]
    section 3) composes the new token's K'_i, V'_i, which become the last
    row n - 1 of that layer's sequence, and attends over all n rows.
"""
from __future__ import annotations

import numpy as np

LAMBDA = 35.0          # [YOCO++] key technical innovations, item 2
KEY_BLOCK = 1 << 16    # rows widened to fp64 at a time (memory bound only)


def to_f64(x) -> np.ndarray:
    """Exact fp64 value of an input array (uint16 is read as bf16 bit patterns)."""
    x = np.asarray(x)
    if x.dtype == np.uint16:
        return (x.astype(np.uint32) << np.uint32(16)).view(np.float32).astype(np.float64)
    return x.astype(np.float64)


def bf16_nearest(x) -> np.ndarray:
    """Nearest bf16 value (ties to even) of fp64 values, returned as fp64.

    Rounds once, directly from fp64 (8 significant bits), for reporting how
    many stored bf16 results equal the correctly rounded exact value."""
    x = np.asarray(x, dtype=np.float64)
    m, e = np.frexp(x)                   # x = m * 2**e, 0.5 <= |m| < 1
    r = np.rint(np.ldexp(m, 8))          # 8 significant bits, half-to-even
    return np.ldexp(r, e - 8)


# ---------------------------------------------------------------------------
# O1. Composition of the cached KVs ([YOCO++] section 2, KV composition).
# ---------------------------------------------------------------------------

def compose(x1, xi, a1: float, a2: float, lam: float = LAMBDA) -> np.ndarray:
    """X'_i = lam * (a1 * X_1 + a2 * X_i), elementwise, in fp64.

    ``x1`` is layer 1's K (or V), ``xi`` layer i's; a1, a2 are that layer's
    two residual weights for K (or for V)."""
    return float(lam) * (float(a1) * to_f64(x1) + float(a2) * to_f64(xi))


def compose_kv(k1, ki, v1, vi, alpha, lam: float = LAMBDA):
    """Both equations of the composition for one layer.

    ``alpha`` = (aK1, aK2, aV1, aV2): the key weights act on K_1, K_i and the
    value weights on V_1, V_i."""
    aK1, aK2, aV1, aV2 = alpha
    return compose(k1, ki, aK1, aK2, lam), compose(v1, vi, aV1, aV2, lam)


def compose_magnitude(x1, xi, a1: float, a2: float, lam: float = LAMBDA) -> np.ndarray:
    """lam * (|a1 X_1| + |a2 X_i|): the size of the terms being summed.

    Rounding errors of any evaluation order scale with this, not with
    |X'_i|, which can cancel to zero."""
    return float(lam) * (np.abs(float(a1) * to_f64(x1)) + np.abs(float(a2) * to_f64(xi)))


def compose_backward(gk, gv, k1, ki, v1, vi, alpha, lam: float = LAMBDA) -> dict:
    """Gradients of one layer's composition, given the upstream gradients
    gk = dL/dK'_i and gv = dL/dV'_i (same layout as the sources).

    [YOCO++] section 2: the four residual weights are learnable and lambda is a
    fixed scale. K'_i = lam (aK1 K_1 + aK2 K_i) is linear in every input, so
      dL/dK_1 = lam aK1 gk,   dL/dK_i = lam aK2 gk,
      dL/daK1 = lam <gk, K_1>,  dL/daK2 = lam <gk, K_i>,
    and likewise for V. Returns fp64 arrays dk1, dki, dv1, dvi and the tuple
    dalpha = (daK1, daK2, daV1, daV2)."""
    aK1, aK2, aV1, aV2 = (float(a) for a in alpha)
    lam = float(lam)
    gk64, gv64 = to_f64(gk), to_f64(gv)
    return {
        "dk1": lam * aK1 * gk64, "dki": lam * aK2 * gk64,
        "dv1": lam * aV1 * gv64, "dvi": lam * aV2 * gv64,
        "dalpha": (lam * float(np.sum(gk64 * to_f64(k1))), lam * float(np.sum(gk64 * to_f64(ki))),
                   lam * float(np.sum(gv64 * to_f64(v1))), lam * float(np.sum(gv64 * to_f64(vi)))),
    }


# ---------------------------------------------------------------------------
# O2. Decode attention over the shared cache ([YOCO] cross-decoder;
#     [YOCO++] section 2: every upper-half layer reads K'_{L/2}, V'_{L/2}).
# ---------------------------------------------------------------------------

def _scores(q64: np.ndarray, k_bg, n: int, scale: float) -> np.ndarray:
    """s[j, t] = scale * <q_j, k_t> for t in [0, n); q64 is [G, D]."""
    out = np.empty((q64.shape[0], n), dtype=np.float64)
    for t0 in range(0, n, KEY_BLOCK):
        t1 = min(n, t0 + KEY_BLOCK)
        out[:, t0:t1] = q64 @ to_f64(k_bg[t0:t1]).T
    return out * scale


def _weighted_values(p: np.ndarray, v_bg, n: int) -> np.ndarray:
    """sum_t p[j, t] * v_t for t in [0, n); p is [G, n]."""
    acc = np.zeros((p.shape[0], v_bg.shape[-1]), dtype=np.float64)
    for t0 in range(0, n, KEY_BLOCK):
        t1 = min(n, t0 + KEY_BLOCK)
        acc += p[:, t0:t1] @ to_f64(v_bg[t0:t1])
    return acc


def softmax_attend(q64: np.ndarray, k_bg, v_bg, n: int, scale: float):
    """Softmax attention of queries q64 [G, D] over the first n rows.

    Two passes over a materialised score vector: m = max_t s_t,
    l = sum_t exp(s_t - m), o = sum_t exp(s_t - m) v_t / l, lse = m + ln l."""
    s = _scores(q64, k_bg, n, scale)
    m = s.max(axis=1, keepdims=True)
    p = np.exp(s - m)
    l = p.sum(axis=1, keepdims=True)
    o = _weighted_values(p, v_bg, n) / l
    lse = (m + np.log(l))[:, 0]
    return o, lse


def decode_attention(q, k, v, seq_lens=None, scale: float | None = None, heads=None):
    """One new query per sequence against the shared cache.

    q: [B, Hq, D]; k, v: [B, Hkv, T, D] (head-major cache); seq_lens: per
    sequence number of valid rows (None: all T). Returns o [B, Hq, D] and
    lse [B, Hq] in fp64. ``heads`` optionally restricts the computation to a
    list of (b, h) pairs (other entries are left NaN)."""
    q = np.asarray(q)
    B, Hq, D = q.shape
    Hkv, T = k.shape[1], k.shape[2]
    if Hq % Hkv:
        raise ValueError("Hq must be a multiple of Hkv")
    G = Hq // Hkv
    scale = 1.0 / np.sqrt(D) if scale is None else float(scale)
    q64 = to_f64(q)
    o = np.full((B, Hq, D), np.nan)
    lse = np.full((B, Hq), np.nan)
    want = None if heads is None else {(int(b), int(h)) for b, h in heads}
    for b in range(B):
        n = T if seq_lens is None else int(seq_lens[b])
        if not 1 <= n <= T:
            raise ValueError("seq_lens must lie in [1, T]")
        for g in range(Hkv):
            hs = [h for h in range(g * G, (g + 1) * G) if want is None or (b, h) in want]
            if not hs:
                continue
            ob, lb = softmax_attend(q64[b, hs], k[b, g], v[b, g], n, scale)
            o[b, hs], lse[b, hs] = ob, lb
    return o, lse


def self_attn_decode(q, k_cache, v_cache, new_rows: dict, alpha, seq_lens=None, scale: float | None = None,
                     lam: float = LAMBDA):
    """One decode step of a lower-half (self-decoder) layer i.

    [YOCO++] section 2: layer i caches its composed K'_i, V'_i; section 3: the
    lower half keeps L/2 such caches, so each self-decoder layer attends over
    its own. The new token's K'_i, V'_i are composed from its K_1, K_i, V_1,
    V_i (``new_rows`` = {"k1", "ki", "v1", "vi"}, each [B, Hkv, D]) and become
    row n - 1 of the sequence; the query attends over cache rows [0, n - 1)
    followed by that row, n = seq_lens[b] (all T when None). Whatever the
    cache holds at rows >= n - 1 is never read. Returns o [B, Hq, D],
    lse [B, Hq] and the exact composed rows k_new, v_new [B, Hkv, D] (fp64)."""
    q = np.asarray(q)
    B, Hq, D = q.shape
    Hkv, T = k_cache.shape[1], k_cache.shape[2]
    if Hq % Hkv:
        raise ValueError("Hq must be a multiple of Hkv")
    G = Hq // Hkv
    scale = 1.0 / np.sqrt(D) if scale is None else float(scale)
    k_new, v_new = compose_kv(new_rows["k1"], new_rows["ki"], new_rows["v1"], new_rows["vi"], alpha, lam)
    q64 = to_f64(q)
    o = np.empty((B, Hq, D))
    lse = np.empty((B, Hq))
    for b in range(B):
        n = T if seq_lens is None else int(seq_lens[b])
        if not 1 <= n <= T:
            raise ValueError("seq_lens must lie in [1, T]")
        for g in range(Hkv):
            keys = np.concatenate([to_f64(k_cache[b, g, :n - 1]), k_new[b, g][None]])
            vals = np.concatenate([to_f64(v_cache[b, g, :n - 1]), v_new[b, g][None]])
            hs = slice(g * G, (g + 1) * G)
            o[b, hs], lse[b, hs] = softmax_attend(q64[b, hs], keys, vals, n, scale)
    return o, lse, k_new, v_new


# ---------------------------------------------------------------------------
# O3. Causal prefill of the cross-decoder over the global cache ([YOCO]
#     abstract: end to end the model works as a decoder-only Transformer does,
#     so attention is causal).
# ---------------------------------------------------------------------------

def causal_prefill(q, k, v, p0: int, scale: float | None = None, rows=None, row_block: int = 64):
    """Query chunk at absolute positions [p0, p0 + C) over the cache.

    q: [B, C, Hq, D]; k, v: [B, Hkv, Tcap, D]. The query at position p
    attends to cache rows [0, p] inclusive. Returns o [B, C, Hq, D] and
    lse [B, Hq, C] (fp64). ``rows`` restricts evaluation to the listed chunk
    rows (the others stay NaN). Each query row is the decode definition over
    its own prefix: masked rows get score -inf and weight exp(-inf) = 0."""
    q = np.asarray(q)
    B, C, Hq, D = q.shape
    Hkv = k.shape[1]
    G = Hq // Hkv
    scale = 1.0 / np.sqrt(D) if scale is None else float(scale)
    if p0 < 0 or p0 + C > k.shape[2]:
        raise ValueError("p0 + C exceeds the cache")
    rows = np.arange(C) if rows is None else np.unique(np.asarray(rows, dtype=np.int64))
    o = np.full((B, C, Hq, D), np.nan)
    lse = np.full((B, Hq, C), np.nan)
    for b in range(B):
        for g in range(Hkv):
            for i0 in range(0, rows.size, row_block):
                rs = rows[i0:i0 + row_block]
                n = p0 + int(rs.max()) + 1                 # keys any of these rows can see
                qg = to_f64(q[b][rs][:, g * G:(g + 1) * G, :]).reshape(-1, D)   # [(r, j), D]
                s = _scores(qg, k[b, g], n, scale)           # [(r, j), n]
                pos = np.repeat(p0 + rs, G)[:, None]         # absolute position of each query
                s = np.where(np.arange(n)[None, :] <= pos, s, -np.inf)
                m = s.max(axis=1, keepdims=True)
                p = np.exp(s - m)
                l = p.sum(axis=1, keepdims=True)
                ob = _weighted_values(p, v[b, g], n) / l
                lb = (m + np.log(l))[:, 0]
                o[b, rs, g * G:(g + 1) * G, :] = ob.reshape(rs.size, G, D)
                lse[b, g * G:(g + 1) * G][:, rs] = lb.reshape(rs.size, G).T
    return o, lse
