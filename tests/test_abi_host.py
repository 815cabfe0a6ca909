"""Host-side tests of the C ABI: the library loads, exports every function that
include/yoco.h declares, and rejects bad arguments before any launch (these
calls never reach the GPU, so they run on a CPU-only host)."""
import ctypes
import os
import re
import subprocess

import pytest

import cross_layer_shared_amd as Y
from cross_layer_shared_amd.binding import Tensor4

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "yoco.h")

OK, INVALID, UNSUPPORTED, ALIGN, WORKSPACE, LAUNCH = range(6)
F32, BF16 = 0, 1
BASE = 0x7F0000000000          # fake, 16-byte aligned device addresses (never dereferenced)


@pytest.fixture(scope="module")
def lib():
    return Y.load_library()


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(yoco_[a-z_0-9]+)\s*\(", text)))


def test_header_declares_the_boundary():
    names = declared_functions()
    for n in ("yoco_compose_kv", "yoco_cross_attn_decode", "yoco_cross_attn_prefill", "yoco_decode_merge",
              "yoco_cross_attn_decode_partial", "yoco_decode_workspace_size", "yoco_decode_num_splits"):
        assert n in names
    assert set(names) == set(Y.EXPORTED)


def test_library_exports_every_declared_symbol(lib):
    out = subprocess.run(["nm", "-D", "--defined-only", Y.LIB_PATH], capture_output=True, text=True, check=True).stdout
    exported = set(re.findall(r"\bT (yoco_\w+)", out))
    for name in declared_functions():
        assert name in exported, name
        assert hasattr(lib, name)


def test_version_and_status_strings(lib):
    assert Y.yoco_version() == 100
    assert Y.yoco_status_string(OK) == "ok"
    assert "workspace" in Y.yoco_status_string(WORKSPACE)
    assert Y.yoco_status_string(99) == "unknown status"


def t4(addr=BASE, sb=8 * 256 * 128, sh=256 * 128, st=128, rows=256):
    return Tensor4(addr, sb, sh, st, rows)


def src4(addr, n=256, Hkv=8, D=128, B=1):
    # token-major [B, n, Hkv, D]
    return Tensor4(addr, n * Hkv * D, D, Hkv * D, n)


def compose(lib, **kw):
    a = dict(k1=src4(BASE), ki=src4(BASE + (1 << 24)), v1=src4(BASE + (2 << 24)), vi=src4(BASE + (3 << 24)),
             kc=t4(BASE + (4 << 24)), vc=t4(BASE + (5 << 24)), t0=0, B=1, n=256, Hkv=8, D=128, lam=35.0,
             a=(0.01, 0.02, 0.03, 0.04), dt=BF16)
    a.update(kw)
    return lib.yoco_compose_kv(a["k1"], a["ki"], a["v1"], a["vi"], a["kc"], a["vc"], a["t0"], a["B"], a["n"],
                               a["Hkv"], a["D"], a["lam"], *a["a"], a["dt"], None)


@pytest.mark.parametrize("kw,status", [
    (dict(B=0), INVALID), (dict(n=0), INVALID), (dict(t0=-1), INVALID), (dict(dt=7), INVALID),
    (dict(D=60), UNSUPPORTED), (dict(D=2048), UNSUPPORTED),
    (dict(k1=src4(0)), INVALID), (dict(kc=t4(0)), INVALID),
    (dict(ki=src4(BASE + 8)), ALIGN), (dict(vc=t4(st=132)), ALIGN),
    (dict(kc=t4(BASE + (4 << 24), rows=100)), INVALID), (dict(t0=1), INVALID),
    (dict(lam=float("inf")), INVALID), (dict(a=(0.0, float("nan"), 0.0, 0.0)), INVALID),
    # a source overlapping a destination without aliasing it exactly
    (dict(ki=src4(BASE + (4 << 24) + 4096)), INVALID),
    # the same source buffer as the cache but at t0 > 0 is a partial overlap
    (dict(ki=t4(BASE + (4 << 24)), kc=t4(BASE + (4 << 24), rows=300), t0=16), INVALID),
    (dict(vc=t4(BASE + (4 << 24))), INVALID),
    # 2^31 16-byte vectors in one call: beyond the kernel's 32-bit index
    (dict(n=1 << 21, Hkv=64), UNSUPPORTED),
])
def test_compose_rejects(lib, kw, status):
    assert compose(lib, **kw) == status
    assert Y.yoco_last_error() != ""


def decode(lib, **kw):
    a = dict(q=BASE, k=t4(BASE + (1 << 28), rows=4096, sb=8 * 4096 * 128, sh=4096 * 128),
             v=t4(BASE + (2 << 28), rows=4096, sb=8 * 4096 * 128, sh=4096 * 128), sl=None, B=8, T=4096, Hq=32,
             Hkv=8, D=128, scale=0.0, out=BASE + (3 << 28), lse=None, ws=BASE + (4 << 28), wsb=1 << 30, S=0,
             dt=BF16)
    a.update(kw)
    return lib.yoco_cross_attn_decode(a["q"], a["k"], a["v"], a["sl"], a["B"], a["T"], a["Hq"], a["Hkv"], a["D"],
                                      a["scale"], a["out"], a["lse"], a["ws"], a["wsb"], a["S"], a["dt"], None)


@pytest.mark.parametrize("kw,status", [
    (dict(B=0), INVALID), (dict(T=0), INVALID), (dict(Hq=30), INVALID), (dict(dt=3), INVALID),
    (dict(D=96), UNSUPPORTED), (dict(Hq=256), UNSUPPORTED), (dict(q=None), INVALID), (dict(q=BASE + 4), ALIGN),
    (dict(out=None), INVALID), (dict(out=BASE + (3 << 28) + 8), ALIGN), (dict(lse=BASE + 2), ALIGN),
    (dict(T=5000), INVALID), (dict(S=-1), INVALID), (dict(S=5000), INVALID),
    (dict(ws=None), WORKSPACE), (dict(wsb=1000), WORKSPACE), (dict(ws=BASE + 8), ALIGN),
    (dict(sl=BASE + 2), ALIGN), (dict(scale=float("inf")), INVALID),
    # one head's rows must span less than 2 GiB (32-bit row offsets)
    (dict(k=t4(BASE + (1 << 28), rows=1 << 23, sb=0, sh=0, st=128), v=t4(BASE + (1 << 40), rows=1 << 23, sb=0, sh=0),
          T=1 << 23, B=1, S=1), UNSUPPORTED),
    (dict(v=t4(BASE + (2 << 28), rows=4096, sb=0, sh=0, st=128 * 4096)), UNSUPPORTED),
])
def test_decode_rejects(lib, kw, status):
    assert decode(lib, **kw) == status
    assert Y.yoco_last_error() != ""


def test_partial_and_merge_reject(lib):
    k = t4(BASE + (1 << 28), rows=4096)
    assert lib.yoco_cross_attn_decode_partial(BASE, k, k, None, 1, 4096, 4, 1, 128, 0.0, BASE, 1 << 30, 1, BF16,
                                              None) == INVALID
    assert lib.yoco_decode_merge(BASE, 1 << 30, 1, 4, 1, 96, 4, BASE, None, None) == UNSUPPORTED
    assert lib.yoco_decode_merge(BASE, 100, 1, 4, 1, 128, 4, BASE, None, None) == WORKSPACE
    assert lib.yoco_decode_merge(BASE, 1 << 30, 1, 4, 1, 128, 1, BASE, None, None) == INVALID
    assert lib.yoco_decode_merge(BASE, 1 << 30, 1, 4, 3, 128, 4, BASE, None, None) == INVALID
    assert lib.yoco_decode_merge(None, 1 << 30, 1, 4, 1, 128, 4, BASE, None, None) == WORKSPACE


def test_compose_on_read_rejects(lib):
    k = t4(BASE + (1 << 28), rows=4096, sb=8 * 4096 * 128, sh=4096 * 128)

    def call(**kw):
        a = dict(q=BASE, k1=k, ki=k, v1=k, vi=k, B=8, T=4096, lam=35.0, a=(0.0, 0.02, 0.01, 0.03), ws=BASE + (4 << 28))
        a.update(kw)
        return lib.yoco_cross_attn_decode_compose_on_read(a["q"], a["k1"], a["ki"], a["v1"], a["vi"], None, a["B"],
                                                          a["T"], 32, 8, 128, a["lam"], *a["a"], 0.0,
                                                          BASE + (3 << 28), None, a["ws"], 1 << 30, 0, BF16, None)
    assert call(k1=t4(0, rows=4096)) == INVALID
    assert call(v1=t4(BASE + 8, rows=4096)) == ALIGN
    assert call(k1=t4(BASE, rows=100)) == INVALID
    assert call(lam=float("nan")) == INVALID
    assert call(ws=None) == WORKSPACE
    assert call(T=0) == INVALID


def test_self_attn_decode_rejects(lib):
    kc = t4(BASE + (1 << 28), rows=4096, sb=8 * 4096 * 128, sh=4096 * 128)
    vc = t4(BASE + (2 << 28), rows=4096, sb=8 * 4096 * 128, sh=4096 * 128)
    one = t4(BASE + (5 << 28), sb=8 * 128, sh=128, st=0, rows=1)      # [B, Hkv, D] one-token rows

    def call(**kw):
        a = dict(q=BASE, k1=one, ki=one, v1=one, vi=one, kc=kc, vc=vc, B=8, T=4096, lam=35.0,
                 a=(0.0, 0.02, 0.01, 0.03), ws=BASE + (4 << 28))
        a.update(kw)
        return lib.yoco_self_attn_decode(a["q"], a["k1"], a["ki"], a["v1"], a["vi"], a["kc"], a["vc"], None, a["B"],
                                         a["T"], 32, 8, 128, a["lam"], *a["a"], 0.0, BASE + (3 << 28), None, a["ws"],
                                         1 << 30, 0, BF16, None)
    assert call(k1=t4(0, st=0, rows=1)) == INVALID                                  # null source
    assert call(v1=t4(BASE + (5 << 28) + 8, sb=8 * 128, sh=128, st=0, rows=1)) == ALIGN
    assert call(ki=t4(BASE + (6 << 28), rows=100)) == INVALID                       # too few rows, stride_t != 0
    # a source inside a cache without being the same view, or inside the other cache
    assert call(ki=t4(BASE + (1 << 28) + 4096 * 128 * 2, rows=4096, sb=8 * 4096 * 128, sh=4096 * 128)) == INVALID
    assert call(vi=t4(BASE + (1 << 28), sb=8 * 128, sh=128, st=0, rows=1)) == INVALID
    assert call(vc=kc) == INVALID                                                   # caches overlap
    assert call(lam=float("inf")) == INVALID
    assert call(ws=None) == WORKSPACE
    assert call(T=0) == INVALID


def test_compose_backward_rejects(lib):
    src = [src4(BASE + (i << 24)) for i in range(4)]
    gk, gv = t4(BASE + (4 << 24)), t4(BASE + (5 << 24))
    g32 = [Tensor4(BASE + ((6 + i) << 24), 256 * 8 * 128, 128, 8 * 128, 256) for i in range(4)]

    def call(**kw):
        a = dict(gk=gk, gv=gv, t0=0, src=src, g=g32, B=1, n=256, D=128, lam=35.0, dalpha=BASE + (12 << 24),
                 ws=BASE + (13 << 24), wsb=1 << 20, dt=BF16)
        a.update(kw)
        return lib.yoco_compose_kv_backward(a["gk"], a["gv"], a["t0"], *a["src"], *a["g"], a["B"], a["n"], 8,
                                            a["D"], a["lam"], 0.01, 0.02, 0.03, 0.04, a["dalpha"], a["ws"],
                                            a["wsb"], a["dt"], None)
    assert call(n=0) == INVALID
    assert call(D=60) == UNSUPPORTED
    assert call(dalpha=None) == INVALID
    assert call(ws=None) == WORKSPACE
    assert call(wsb=16) == WORKSPACE
    assert call(g=[g32[0], g32[0], g32[2], g32[3]]) == INVALID          # two outputs overlap
    assert call(g=[Tensor4(src[0].ptr, 256 * 8 * 128, 128, 8 * 128, 256)] + g32[1:]) == INVALID   # output over input
    assert call(gk=t4(BASE + (4 << 24), rows=100)) == INVALID
    assert call(lam=float("inf")) == INVALID
    assert call(n=1 << 23) == UNSUPPORTED      # 2^31 four-element vectors: beyond the 32-bit index
    # one fp32 partial per weight per workgroup of 256 threads x 4 four-element vectors
    assert Y.yoco_compose_backward_workspace_size(1, 256, 8, 128, BF16) == ((256 * 8 * 32 + 1023) // 1024) * 16
    assert Y.yoco_compose_backward_workspace_size(1, 3, 1, 64, F32) == 16


def prefill(lib, **kw):
    a = dict(q=BASE, k=t4(BASE + (1 << 28), rows=8192, sb=8 * 8192 * 128, sh=8192 * 128),
             v=t4(BASE + (2 << 28), rows=8192, sb=8 * 8192 * 128, sh=8192 * 128), B=1, C=4096, p0=4096, Hq=32,
             Hkv=8, D=128, scale=0.0, out=BASE + (3 << 28), odt=F32, lse=None, dt=BF16)
    a.update(kw)
    return lib.yoco_cross_attn_prefill(a["q"], a["k"], a["v"], a["B"], a["C"], a["p0"], a["Hq"], a["Hkv"], a["D"],
                                       a["scale"], a["out"], a["odt"], a["lse"], a["dt"], None)


@pytest.mark.parametrize("kw,status", [
    (dict(C=0), INVALID), (dict(p0=-1), INVALID), (dict(p0=4097), INVALID), (dict(Hq=33), INVALID),
    (dict(dt=F32), UNSUPPORTED), (dict(D=96), UNSUPPORTED), (dict(Hq=8 * 32), UNSUPPORTED), (dict(odt=9), INVALID),
    (dict(q=BASE + 2), ALIGN), (dict(out=None), INVALID), (dict(lse=BASE + 1), ALIGN),
    (dict(k=t4(BASE + 8, rows=8192)), ALIGN),
])
def test_prefill_rejects(lib, kw, status):
    assert prefill(lib, **kw) == status
    assert Y.yoco_last_error() != ""


def test_prefill_rejects_row_strides_past_its_32_bit_step_offsets(lib):
    """The prefill addresses the 64 rows of a step with 32-bit byte offsets
    from a per-step base, so a cache row stride of 2^24 elements or more is
    refused."""
    big = t4(BASE + (1 << 28), rows=8192, sb=0, sh=0, st=1 << 24)
    assert prefill(lib, B=1, Hq=4, Hkv=1, k=big) == UNSUPPORTED
    assert "stride_t" in Y.yoco_last_error()
    assert prefill(lib, B=1, Hq=4, Hkv=1, v=big) == UNSUPPORTED


def test_split_heuristic_and_workspace():
    # launch shapes measured best on MI355X for the three decode workloads
    assert Y.yoco_decode_num_splits(8, 4096, 32, 8, 128) == 4
    assert Y.yoco_decode_num_splits(4, 131072, 32, 8, 128) == 8
    assert Y.yoco_decode_num_splits(1, 1 << 20, 16, 4, 128) == 64
    assert Y.yoco_decode_num_splits(1, 256, 4, 1, 64) == 1
    assert Y.yoco_decode_num_splits(0, 256, 4, 1, 64) == 0
    # [B, Hkv] u32 counters + [B, Hq, S, D] f32 + [B, Hq, S] f32, sections 16-byte aligned
    assert Y.yoco_decode_workspace_size(8, 4096, 32, 8, 128, 16) == 8 * 8 * 4 + 8 * 32 * 16 * 129 * 4
    assert Y.yoco_decode_workspace_size(1, 100, 3, 1, 64, 3) == 16 + 3 * 3 * 64 * 4 + 48
    assert Y.yoco_decode_workspace_size(1, 256, 4, 1, 64, 1) == 0
    for B, T, Hq, Hkv in [(3, 5, 4, 1), (1, 4097, 8, 2), (2, 100000, 16, 4)]:
        s = Y.yoco_decode_num_splits(B, T, Hq, Hkv, 128)
        assert 1 <= s <= T


def test_binding_fails_loudly_without_library(tmp_path):
    from cross_layer_shared_amd import binding
    with pytest.raises(RuntimeError):
        binding.load_library.__wrapped__(str(tmp_path / "missing.so")) if hasattr(binding.load_library, "__wrapped__") \
            else _load_missing(binding, str(tmp_path / "missing.so"))


def _load_missing(binding, path):
    saved = binding._lib
    binding._lib = None
    try:
        binding.load_library(path)
    finally:
        binding._lib = saved


# ----------------------------------------------------------------- bandwidth probes

CEILING_HEADER = os.path.join(ROOT, "include", "yoco_ceiling.h")


def test_ceiling_library_exports_every_declared_symbol():
    from cross_layer_shared_amd import ceiling as C
    text = re.sub(r"/\*.*?\*/", "", open(CEILING_HEADER).read(), flags=re.S)
    names = sorted(set(re.findall(r"\b(yoco_ceiling_[a-z_0-9]+)\s*\(", text)))
    assert set(names) == set(C.CEILING_EXPORTED)
    out = subprocess.run(["nm", "-D", "--defined-only", C.CEILING_LIB_PATH], capture_output=True, text=True,
                         check=True).stdout
    exported = set(re.findall(r"\bT (yoco_\w+)", out))
    for n in names:
        assert n in exported, n
    assert not any(n.startswith("yoco_") and not n.startswith("yoco_ceiling_") for n in exported)


def test_ceiling_probes_reject_bad_arguments():
    from cross_layer_shared_amd import ceiling as C
    lib = C.load_ceiling_library()
    sink = BASE + (1 << 30)
    cases = [
        (lib.yoco_ceiling_read(None, 1 << 20, 256, 512, 4, 1, sink, None), INVALID),
        (lib.yoco_ceiling_read(BASE + 8, 1 << 20, 256, 512, 4, 1, sink, None), ALIGN),
        (lib.yoco_ceiling_read(BASE, 1000, 256, 512, 4, 1, sink, None), INVALID),
        (lib.yoco_ceiling_read(BASE, 1 << 20, -1, 512, 4, 1, sink, None), INVALID),
        (lib.yoco_ceiling_read(BASE, 1 << 20, 256, 100, 4, 1, sink, None), INVALID),
        (lib.yoco_ceiling_read(BASE, 1 << 20, 256, 2048, 4, 1, sink, None), INVALID),
        (lib.yoco_ceiling_read(BASE, 1 << 20, 256, 512, 4, 1, sink + 2, None), ALIGN),
        (lib.yoco_ceiling_read(BASE, 1 << 20, 256, 512, 3, 1, sink, None), INVALID),
        (lib.yoco_ceiling_read(BASE, 1 << 20, 256, 512, 32, 1, sink, None), INVALID),
        (lib.yoco_ceiling_read_blocks(None, 1 << 20, 256, 512, 8, sink, None), INVALID),
        (lib.yoco_ceiling_read_blocks(BASE + 8, 1 << 20, 256, 512, 8, sink, None), ALIGN),
        (lib.yoco_ceiling_read_blocks(BASE, 1000, 256, 512, 8, sink, None), INVALID),
        (lib.yoco_ceiling_read_blocks(BASE, 1 << 20, 0, 512, 8, sink, None), INVALID),
        (lib.yoco_ceiling_read_blocks(BASE, 1 << 20, 256, 100, 8, sink, None), INVALID),
        (lib.yoco_ceiling_read_blocks(BASE, 1 << 20, 256, 512, 5, sink, None), INVALID),
    ]
    bufs = [BASE + (i << 24) for i in range(6)]
    cases += [
        (lib.yoco_ceiling_read4_write2(*bufs[:5], None, 1 << 20, 512, 1, None), INVALID),
        (lib.yoco_ceiling_read4_write2(*bufs[:5], bufs[5] + 4, 1 << 20, 512, 1, None), ALIGN),
        (lib.yoco_ceiling_read4_write2(*bufs, 0, 512, 1, None), INVALID),
        (lib.yoco_ceiling_read4_write2(*bufs, 1 << 20, 32, 1, None), INVALID),
        (lib.yoco_ceiling_read4_write2(*bufs[:4], bufs[0], bufs[5], 1 << 20, 512, 1, None), INVALID),   # e aliases a
        (lib.yoco_ceiling_read4_write2(*bufs[:5], bufs[4] + 16, 1 << 20, 512, 1, None), INVALID),       # e, f overlap
        (lib.yoco_ceiling_read4_write2(*bufs, 1 << 20, 512, 3, None), INVALID),
    ]
    cases += [
        (lib.yoco_ceiling_mfma_bf16(None, 1 << 20, 256, 16, sink, None), INVALID),
        (lib.yoco_ceiling_mfma_bf16(BASE, 1 << 20, 256, 16, None, None), INVALID),
        (lib.yoco_ceiling_mfma_bf16(BASE + 8, 1 << 20, 256, 16, sink, None), ALIGN),
        (lib.yoco_ceiling_mfma_bf16(BASE, 1 << 20, 256, 16, sink + 2, None), ALIGN),
        (lib.yoco_ceiling_mfma_bf16(BASE, 0, 256, 16, sink, None), INVALID),
        (lib.yoco_ceiling_mfma_bf16(BASE, 24, 256, 16, sink, None), INVALID),
        (lib.yoco_ceiling_mfma_bf16(BASE, 240, 256, 16, sink, None), INVALID),
        (lib.yoco_ceiling_mfma_bf16(BASE, 1 << 20, 0, 16, sink, None), INVALID),
        (lib.yoco_ceiling_mfma_bf16(BASE, 1 << 20, 65537, 16, sink, None), INVALID),
        (lib.yoco_ceiling_mfma_bf16(BASE, 1 << 20, 256, 0, sink, None), INVALID),
        (lib.yoco_ceiling_mfma_bf16(BASE, 1 << 20, 256, (1 << 24) + 1, sink, None), INVALID),
    ]
    for got, want in cases:
        assert got == want
        assert lib.yoco_ceiling_last_error().decode()


def test_noalloc_decode_rejects_before_any_launch(lib):
    """The allocation-free decode checks its arguments like the workspace decode,
    and rejects calls whose partials or counters exceed its scratch array."""
    def call(B=8, T=4096, Hq=32, Hkv=8, D=128, S=0, q=BASE, out=BASE + (1 << 30), dt=BF16):
        k = t4(BASE + (2 << 30), sb=Hkv * T * D, sh=T * D, st=D, rows=T)
        v = t4(BASE + (3 << 30), sb=Hkv * T * D, sh=T * D, st=D, rows=T)
        return lib.yoco_cross_attn_decode_noalloc(q, k, v, None, B, T, Hq, Hkv, D, 0.0, out, None, S, dt, None)
    assert call(B=0) == INVALID
    assert call(q=0) == INVALID
    assert call(out=BASE + 4) == ALIGN
    assert call(D=96) == UNSUPPORTED
    assert call(S=-1) == INVALID
    assert call(T=100, S=101) == INVALID
    assert call(B=64, Hq=64, Hkv=64, T=64, S=16) == WORKSPACE            # partials beyond 8 MiB
    assert "scratch" in Y.yoco_last_error()
    assert call(B=4096, Hq=8, Hkv=8, T=64, S=2) == WORKSPACE             # 32768 counters > 16384
    assert "counters" in Y.yoco_last_error()


def test_overlapping_rows_and_aliased_destinations_are_rejected(lib):
    """A cache read row by row needs stride_t >= D (stride 0 would read one row,
    or nothing through the decode's row-bounded buffer); a tensor the library
    writes must give every element an address of its own."""
    # decode and prefill caches: stride_t 0 or below D
    for st in (0, 64):
        bad = t4(BASE + (1 << 28), rows=4096, sb=8 * 4096 * 128, sh=4096 * 128, st=st)
        assert decode(lib, k=bad) == INVALID and "stride_t" in Y.yoco_last_error()
        assert decode(lib, v=bad) == INVALID
        badp = t4(BASE + (1 << 28), rows=8192, sb=8 * 8192 * 128, sh=8192 * 128, st=st)
        assert prefill(lib, k=badp) == INVALID
    # compose destinations: heads or sequences sharing memory
    assert compose(lib, kc=t4(BASE + (4 << 24), sh=0)) == INVALID
    assert "address" in Y.yoco_last_error()
    assert compose(lib, vc=t4(BASE + (5 << 24), st=64)) == INVALID
    assert compose(lib, B=2, kc=t4(BASE + (4 << 24), sb=0, rows=256), k1=src4(BASE, B=2), ki=src4(BASE + (1 << 24), B=2),
                   v1=src4(BASE + (2 << 24), B=2), vi=src4(BASE + (3 << 24), B=2)) == INVALID


def test_self_decode_and_backward_destinations_must_not_alias(lib):
    kc = t4(BASE + (1 << 28), rows=4096, sb=8 * 4096 * 128, sh=0)        # all kv heads on one memory
    vc = t4(BASE + (2 << 28), rows=4096, sb=8 * 4096 * 128, sh=4096 * 128)
    one = t4(BASE + (5 << 28), sb=8 * 128, sh=128, st=0, rows=1)
    st = lib.yoco_self_attn_decode(BASE, one, one, one, one, kc, vc, None, 8, 4096, 32, 8, 128, 35.0, 0.0, 0.02, 0.01,
                                   0.03, 0.0, BASE + (3 << 28), None, BASE + (4 << 28), 1 << 30, 0, BF16, None)
    assert st == INVALID
    src = [src4(BASE + (i << 24)) for i in range(4)]
    gk, gv = t4(BASE + (4 << 24)), t4(BASE + (5 << 24))
    g32 = [Tensor4(BASE + ((6 + i) << 24), 256 * 8 * 128, 128, 8 * 128, 256) for i in range(4)]
    g32[1] = Tensor4(BASE + (7 << 24), 256 * 8 * 128, 0, 8 * 128, 256)   # dki: kv heads alias
    st = lib.yoco_compose_kv_backward(gk, gv, 0, *src, *g32, 1, 256, 8, 128, 35.0, 0.01, 0.02, 0.03, 0.04,
                                      BASE + (12 << 24), BASE + (13 << 24), 1 << 20, BF16, None)
    assert st == INVALID
