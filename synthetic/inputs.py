"""Seeded synthetic inputs for the cross-layer KV-sharing hot path.

This module draws inputs only: it holds none of the method's arithmetic
(no composition, no attention). Both the fp64 oracle side and the HIP side
take their inputs from here, so that the two see the very same rounded
values.

Seeding. Every workload has a base seed (``0x594F434F`` + its index) and
every tensor a fixed stream id. A tensor is drawn in blocks of ``BLOCK``
elements; block ``i`` of stream ``s`` (layer ``l``) uses the generator
``PCG64(SeedSequence(seed, spawn_key=(s, l, i)))``. The blocks are
independent, so they are drawn on a thread pool and the result does not
depend on the number of threads.

bf16. Values are drawn as fp32 and rounded to bf16 with round-to-nearest,
ties-to-even, on the fp32 bit pattern. bf16 tensors are handed around as
``uint16`` bit patterns.
"""
from __future__ import annotations

import math
import os
from concurrent.futures import ThreadPoolExecutor
from dataclasses import dataclass, field

import numpy as np

SEED_BASE = 0x594F434F
BLOCK = 1 << 20

# Stream ids, in the fixed order: alpha, K_1, K_i, V_1, V_i, Q, structure.
S_ALPHA, S_K1, S_KI, S_V1, S_VI, S_Q, S_STRUCT = range(7)
# Extra streams for tensors that are drawn directly as cache contents.
S_KCACHE, S_VCACHE = 7, 8

LAMBDA = 35.0


def _threads() -> int:
    try:
        n = len(os.sched_getaffinity(0))
    except AttributeError:  # pragma: no cover
        n = os.cpu_count() or 1
    return max(1, min(16, n))


def _gen(seed: int, *key: int) -> np.random.Generator:
    return np.random.Generator(np.random.PCG64(np.random.SeedSequence(seed, spawn_key=tuple(key))))


def normal_f32(seed: int, key: tuple, shape, std: float = 1.0) -> np.ndarray:
    """iid N(0, std^2) fp32 samples of ``shape``, drawn block-wise."""
    n = int(np.prod(shape))
    out = np.empty(n, dtype=np.float32)
    nblocks = (n + BLOCK - 1) // BLOCK
    s = np.float32(std)

    def fill(i: int) -> None:
        seg = out[i * BLOCK: min(n, (i + 1) * BLOCK)]
        _gen(seed, *key, i).standard_normal(out=seg, dtype=np.float32)
        if std != 1.0:
            np.multiply(seg, s, out=seg)

    if nblocks == 1:
        fill(0)
    else:
        with ThreadPoolExecutor(_threads()) as ex:
            list(ex.map(fill, range(nblocks)))
    return out.reshape(shape)


def uniform_f32(seed: int, key: tuple, shape, lo: float, hi: float) -> np.ndarray:
    g = _gen(seed, *key, 0)
    return g.uniform(lo, hi, size=shape).astype(np.float32)


def f32_to_bf16_bits(x: np.ndarray) -> np.ndarray:
    """Round fp32 to bf16 (nearest, ties to even); returns uint16 bit patterns."""
    x = np.ascontiguousarray(x, dtype=np.float32)
    b = x.view(np.uint32)
    out = np.empty(b.shape, dtype=np.uint16)
    step = 1 << 24
    flat_b, flat_o = b.reshape(-1), out.reshape(-1)

    def work(i: int) -> None:
        seg = flat_b[i: i + step]
        r = seg + np.uint32(0x7FFF) + ((seg >> np.uint32(16)) & np.uint32(1))
        flat_o[i: i + step] = (r >> np.uint32(16)).astype(np.uint16)

    starts = range(0, flat_b.size, step)
    if flat_b.size <= step:
        for i in starts:
            work(i)
    else:
        with ThreadPoolExecutor(_threads()) as ex:
            list(ex.map(work, starts))
    return out


def bf16_bits_to_f32(bits: np.ndarray) -> np.ndarray:
    """Exact widening of bf16 bit patterns to fp32."""
    return (np.asarray(bits, dtype=np.uint16).astype(np.uint32) << np.uint32(16)).view(np.float32)


def normal_bf16(seed: int, key: tuple, shape, std: float = 1.0) -> np.ndarray:
    return f32_to_bf16_bits(normal_f32(seed, key, shape, std))


def fl32(x: float) -> float:
    """The fp32 value nearest to ``x`` (as a Python float)."""
    return float(np.float32(x))


# The initialisation that makes YOCO++ start as YOCO: alpha_1 = 0, alpha_2 = 1/lambda,
# held in fp32 exactly as it is passed across the C ABI.
IDENTITY_ALPHA = (0.0, fl32(1.0 / LAMBDA), 0.0, fl32(1.0 / LAMBDA))


# ---------------------------------------------------------------------------
# Workloads. Shapes follow the long-context settings the pages describe; the
# cache is head-major [B, Hkv, T, D]; sources are token-major [B, n, Hkv, D].
# ---------------------------------------------------------------------------

@dataclass(frozen=True)
class Workload:
    name: str
    index: int
    B: int
    T: int
    Hq: int
    Hkv: int
    D: int
    dtype: str  # "f32" or "bf16"
    layers: int = 1          # cross-decoder layers reading the shared cache
    self_layers: int = 0     # self-decoder layers (compose sources)
    chunk: int = 0           # prefill query chunk
    notes: dict = field(default_factory=dict)

    @property
    def seed(self) -> int:
        return SEED_BASE + self.index

    @property
    def G(self) -> int:
        return self.Hq // self.Hkv


TINY_FP32_STACK = Workload("tiny_fp32_stack", 1, B=1, T=256, Hq=4, Hkv=1, D=64, dtype="f32",
                           layers=2, self_layers=2)
DECODE_MID = Workload("decode_mid_context", 2, B=8, T=4096, Hq=32, Hkv=8, D=128, dtype="bf16",
                      layers=16, notes={"q_std": 128 ** -0.25})
DECODE_LONG = Workload("decode_long_context", 3, B=4, T=131072, Hq=32, Hkv=8, D=128, dtype="bf16",
                       notes={"scaled_row_fraction": 0.01, "scale": 8.0})
PREFILL_CHUNKED = Workload("prefill_chunked", 4, B=1, T=32768, Hq=32, Hkv=8, D=128, dtype="bf16",
                           self_layers=16, chunk=4096)
DECODE_MILLION = Workload("decode_million_token", 5, B=1, T=1 << 20, Hq=16, Hkv=4, D=128, dtype="bf16",
                          notes={"plant_scale": 4.0})

WORKLOADS = {w.name: w for w in (TINY_FP32_STACK, DECODE_MID, DECODE_LONG, PREFILL_CHUNKED, DECODE_MILLION)}


def alphas(seed: int, layer: int, lo: float = -0.05, hi: float = 0.05) -> tuple:
    """Four fp32 residual weights (aK1, aK2, aV1, aV2) for one self-decoder layer."""
    a = uniform_f32(seed, (S_ALPHA, layer), (4,), lo, hi)
    return tuple(float(v) for v in a)


def _cast(x32: np.ndarray, dtype: str) -> np.ndarray:
    return x32 if dtype == "f32" else f32_to_bf16_bits(x32)


def compose_sources(w: Workload, layer: int, n: int | None = None, B: int | None = None) -> dict:
    """K_1, K_i, V_1, V_i (token-major [B, n, Hkv, D]) for self-decoder layer ``layer``.

    K_1/V_1 belong to layer 1 and do not depend on ``layer``."""
    n = w.T if n is None else n
    B = w.B if B is None else B
    shp = (B, n, w.Hkv, w.D)
    return {
        "k1": _cast(normal_f32(w.seed, (S_K1, 1), shp), w.dtype),
        "ki": _cast(normal_f32(w.seed, (S_KI, layer), shp), w.dtype),
        "v1": _cast(normal_f32(w.seed, (S_V1, 1), shp), w.dtype),
        "vi": _cast(normal_f32(w.seed, (S_VI, layer), shp), w.dtype),
    }


def layer_source(w: Workload, which: str, layer: int, n: int | None = None) -> np.ndarray:
    """One token-major source tensor (``which`` in k/v) of one self-decoder layer."""
    n = w.T if n is None else n
    sid = {"k": S_KI, "v": S_VI}[which] if layer != 1 else {"k": S_K1, "v": S_V1}[which]
    return _cast(normal_f32(w.seed, (sid, layer), (w.B, n, w.Hkv, w.D)), w.dtype)


def cache_kv(w: Workload, T: int | None = None) -> tuple:
    """A shared cache K', V' ([B, Hkv, T, D]) drawn directly as iid N(0, 1)."""
    T = w.T if T is None else T
    shp = (w.B, w.Hkv, T, w.D)
    return (_cast(normal_f32(w.seed, (S_KCACHE, 0), shp), w.dtype),
            _cast(normal_f32(w.seed, (S_VCACHE, 0), shp), w.dtype))


def queries(w: Workload, layer: int = 0, std: float = 1.0, rows: int | None = None) -> np.ndarray:
    """Decode queries [B, Hq, D] (``rows`` None) or prefill queries [B, rows, Hq, D]."""
    shp = (w.B, w.Hq, w.D) if rows is None else (w.B, rows, w.Hq, w.D)
    return _cast(normal_f32(w.seed, (S_Q, layer), shp, std), w.dtype)


def scaled_rows(w: Workload, T: int | None = None) -> np.ndarray:
    """Per sequence, the sorted token rows whose keys are scaled (round(frac*T) rows)."""
    T = w.T if T is None else T
    cnt = int(round(w.notes["scaled_row_fraction"] * T))
    g = _gen(w.seed, S_STRUCT, 0)
    return np.stack([np.sort(g.permutation(T)[:cnt]) for _ in range(w.B)])


def scale_key_rows_bf16(k_bits: np.ndarray, rows: np.ndarray, factor: float) -> None:
    """Multiply the listed key rows (all kv heads) by a power of two, in place.

    A power-of-two factor only moves the bf16 exponent, so the scaled values
    stay exact (no overflow for N(0,1) samples)."""
    e = int(round(math.log2(factor)))
    assert 2.0 ** e == factor
    for b in range(k_bits.shape[0]):
        sel = k_bits[b][:, rows[b], :]
        nz = (sel & 0x7F80) != 0  # leave zeros / subnormals untouched
        sel = np.where(nz, sel + np.uint16(e << 7), sel).astype(np.uint16)
        k_bits[b][:, rows[b], :] = sel


def planted_position(w: Workload, T: int | None = None) -> int:
    T = w.T if T is None else T
    return int(_gen(w.seed, S_STRUCT, 1).integers(0, T))


def plant_query_row_bf16(k_bits: np.ndarray, q_bits: np.ndarray, t_star: int, factor: float) -> None:
    """Set K[b, g, t*, :] = factor * q[b, g*G, :] (power-of-two factor, exact in bf16)."""
    e = int(round(math.log2(factor)))
    assert 2.0 ** e == factor
    B, Hkv = k_bits.shape[0], k_bits.shape[1]
    G = q_bits.shape[1] // Hkv
    for b in range(B):
        for g in range(Hkv):
            qrow = q_bits[b, g * G].astype(np.uint16)
            nz = (qrow & 0x7F80) != 0
            k_bits[b, g, t_star] = np.where(nz, qrow + np.uint16(e << 7), qrow).astype(np.uint16)
