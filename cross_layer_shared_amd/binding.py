"""Python binding of libyoco.so: argument marshalling only.

Every function has the name of its C entry point and takes torch tensors,
from which it reads device pointers, sizes and element strides; all
arithmetic runs in the HIP kernels behind the C ABI. There is no fallback:
if the library is missing or a call fails, an exception is raised.
"""
from __future__ import annotations

import ctypes
import math
import os

import torch

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libyoco.so")

YOCO_OK, YOCO_ERR_INVALID_ARG, YOCO_ERR_UNSUPPORTED, YOCO_ERR_ALIGNMENT, YOCO_ERR_WORKSPACE, YOCO_ERR_LAUNCH = range(6)
YOCO_F32, YOCO_BF16 = 0, 1

EXPORTED = ("yoco_compose_kv", "yoco_compose_backward_workspace_size", "yoco_compose_kv_backward", "yoco_decode_num_splits", "yoco_decode_workspace_size", "yoco_cross_attn_decode",
            "yoco_cross_attn_decode_noalloc", "yoco_cross_attn_decode_compose_on_read", "yoco_self_attn_decode", "yoco_cross_attn_decode_partial", "yoco_decode_merge", "yoco_cross_attn_prefill", "yoco_status_string",
            "yoco_last_error", "yoco_version")


class YocoError(RuntimeError):
    def __init__(self, status: int, msg: str):
        super().__init__(f"{msg} (status {status})")
        self.status = status


class Tensor4(ctypes.Structure):
    _fields_ = [("ptr", ctypes.c_void_p), ("stride_b", ctypes.c_int64), ("stride_h", ctypes.c_int64),
                ("stride_t", ctypes.c_int64), ("rows", ctypes.c_int64)]


_lib = None


def load_library(path: str = LIB_PATH) -> ctypes.CDLL:
    """Load libyoco.so once; raises if it has not been built."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(path):
        raise RuntimeError(f"{path} is missing: build it with `python -m cross_layer_shared_amd.build`")
    lib = ctypes.CDLL(path)
    T4, i, f, vp, sz, st = Tensor4, ctypes.c_int, ctypes.c_float, ctypes.c_void_p, ctypes.c_size_t, ctypes.c_int
    lib.yoco_compose_kv.argtypes = [T4, T4, T4, T4, T4, T4, i, i, i, i, i, f, f, f, f, f, i, vp]
    lib.yoco_compose_kv.restype = st
    lib.yoco_compose_backward_workspace_size.argtypes = [i, i, i, i, i]
    lib.yoco_compose_backward_workspace_size.restype = sz
    lib.yoco_compose_kv_backward.argtypes = [T4, T4, i, T4, T4, T4, T4, T4, T4, T4, T4, i, i, i, i, f, f, f, f, f, vp,
                                             vp, sz, i, vp]
    lib.yoco_compose_kv_backward.restype = st
    lib.yoco_decode_num_splits.argtypes = [i, i, i, i, i]
    lib.yoco_decode_num_splits.restype = i
    lib.yoco_decode_workspace_size.argtypes = [i, i, i, i, i, i]
    lib.yoco_decode_workspace_size.restype = sz
    lib.yoco_cross_attn_decode.argtypes = [vp, T4, T4, vp, i, i, i, i, i, f, vp, vp, vp, sz, i, i, vp]
    lib.yoco_cross_attn_decode.restype = st
    lib.yoco_cross_attn_decode_noalloc.argtypes = [vp, T4, T4, vp, i, i, i, i, i, f, vp, vp, i, i, vp]
    lib.yoco_cross_attn_decode_noalloc.restype = st
    lib.yoco_cross_attn_decode_compose_on_read.argtypes = [vp, T4, T4, T4, T4, vp, i, i, i, i, i, f, f, f, f, f, f,
                                                           vp, vp, vp, sz, i, i, vp]
    lib.yoco_cross_attn_decode_compose_on_read.restype = st
    lib.yoco_self_attn_decode.argtypes = [vp, T4, T4, T4, T4, T4, T4, vp, i, i, i, i, i, f, f, f, f, f, f, vp, vp,
                                          vp, sz, i, i, vp]
    lib.yoco_self_attn_decode.restype = st
    lib.yoco_cross_attn_decode_partial.argtypes = [vp, T4, T4, vp, i, i, i, i, i, f, vp, sz, i, i, vp]
    lib.yoco_cross_attn_decode_partial.restype = st
    lib.yoco_decode_merge.argtypes = [vp, sz, i, i, i, i, i, vp, vp, vp]
    lib.yoco_decode_merge.restype = st
    lib.yoco_cross_attn_prefill.argtypes = [vp, T4, T4, i, i, i, i, i, i, f, vp, i, vp, i, vp]
    lib.yoco_cross_attn_prefill.restype = st
    lib.yoco_status_string.argtypes = [i]
    lib.yoco_status_string.restype = ctypes.c_char_p
    lib.yoco_last_error.argtypes = []
    lib.yoco_last_error.restype = ctypes.c_char_p
    lib.yoco_version.argtypes = []
    lib.yoco_version.restype = i
    _lib = lib
    return lib


def _check(status: int) -> None:
    if status != YOCO_OK:
        lib = load_library()
        raise YocoError(status, lib.yoco_last_error().decode() or lib.yoco_status_string(status).decode())


def _dtype_code(t: torch.Tensor) -> int:
    if t.dtype == torch.bfloat16:
        return YOCO_BF16
    if t.dtype == torch.float32:
        return YOCO_F32
    raise TypeError(f"unsupported dtype {t.dtype}")


def _stream(stream) -> int | None:
    if stream is None:
        return torch.cuda.current_stream().cuda_stream
    return getattr(stream, "cuda_stream", stream)


def _need_contiguous(**tensors) -> None:
    for name, t in tensors.items():
        if t is not None and not t.is_contiguous():
            raise ValueError(f"{name} must be a contiguous tensor")


def _ptr(t: torch.Tensor | None) -> int | None:
    return None if t is None else t.data_ptr()


def _bytes(t: torch.Tensor | None) -> int:
    return 0 if t is None else t.numel() * t.element_size()


def token_major(t: torch.Tensor) -> Tensor4:
    """[B, n, H, D] (D contiguous) -> Tensor4 with t as the token axis."""
    if t.dim() != 4 or t.stride(3) != 1:
        raise ValueError("expected a [B, n, H, D] tensor with a contiguous last axis")
    return Tensor4(t.data_ptr(), t.stride(0), t.stride(2), t.stride(1), t.shape[1])


def head_major(t: torch.Tensor) -> Tensor4:
    """[B, H, T, D] (D contiguous) -> Tensor4."""
    if t.dim() != 4 or t.stride(3) != 1:
        raise ValueError("expected a [B, H, T, D] tensor with a contiguous last axis")
    return Tensor4(t.data_ptr(), t.stride(0), t.stride(1), t.stride(2), t.shape[2])


def _as_t4(x) -> Tensor4:
    return x if isinstance(x, Tensor4) else head_major(x)


def _heads(cache, Hkv: int | None) -> int:
    """KV head count: given explicitly, or axis 1 of a head-major [B, Hkv, T, D] tensor."""
    if Hkv is not None:
        return int(Hkv)
    if isinstance(cache, Tensor4):
        raise ValueError("pass Hkv with a Tensor4 cache view")
    return cache.shape[1]


# ----------------------------------------------------------------- entry points

def yoco_compose_kv(k1, ki, v1, vi, k_cache, v_cache, t0: int, alpha, lam: float = 35.0, stream=None,
                    B: int | None = None, n: int | None = None, Hkv: int | None = None, D: int | None = None,
                    dtype: int | None = None) -> None:
    """Compose one layer's K', V' into cache rows [t0, t0+n).

    Sources are [B, n, Hkv, D] tensors (token-major) or Tensor4; caches are
    [B, Hkv, T, D] tensors (head-major) or Tensor4. alpha = (aK1, aK2, aV1, aV2)."""
    lib = load_library()
    ref = k1 if isinstance(k1, torch.Tensor) else None
    if ref is not None:
        B, n, Hkv, D = ref.shape
        dtype = _dtype_code(ref)
    srcs = [x if isinstance(x, Tensor4) else token_major(x) for x in (k1, ki, v1, vi)]
    aK1, aK2, aV1, aV2 = (float(a) for a in alpha)
    _check(lib.yoco_compose_kv(*srcs, _as_t4(k_cache), _as_t4(v_cache), int(t0), int(B), int(n), int(Hkv), int(D),
                               float(lam), aK1, aK2, aV1, aV2, int(dtype), _stream(stream)))


def yoco_compose_backward_workspace_size(B: int, n: int, Hkv: int, D: int, dtype: int) -> int:
    return load_library().yoco_compose_backward_workspace_size(B, n, Hkv, D, dtype)


def yoco_compose_kv_backward(gk, gv, t0: int, k1, ki, v1, vi, dk1, dki, dv1, dvi, alpha, dalpha, lam: float = 35.0,
                             workspace=None, stream=None) -> None:
    """Gradients of one layer's composition. gk, gv: cache-shaped [B, Hkv, T, D] upstream
    gradients (rows [t0, t0+n)); sources and the fp32 gradients [B, n, Hkv, D] token-major
    (or Tensor4); dk1, dv1 accumulate, dki, dvi are written; dalpha: fp32 [4] on the device."""
    lib = load_library()
    B, n, Hkv, D = k1.shape
    dtype = _dtype_code(k1)
    if workspace is None:
        workspace = _cached_workspace("compose_backward", yoco_compose_backward_workspace_size(B, n, Hkv, D, dtype),
                                      k1.device, stream)
    srcs = [token_major(x) for x in (k1, ki, v1, vi)]
    grads = [token_major(x) for x in (dk1, dki, dv1, dvi)]
    aK1, aK2, aV1, aV2 = (float(a) for a in alpha)
    _need_contiguous(dalpha=dalpha)
    _check(lib.yoco_compose_kv_backward(_as_t4(gk), _as_t4(gv), int(t0), *srcs, *grads, B, n, Hkv, D, float(lam),
                                        aK1, aK2, aV1, aV2, dalpha.data_ptr(), workspace.data_ptr(),
                                        workspace.numel() * workspace.element_size(), dtype, _stream(stream)))


def yoco_decode_num_splits(B: int, T: int, Hq: int, Hkv: int, D: int) -> int:
    return load_library().yoco_decode_num_splits(B, T, Hq, Hkv, D)


def yoco_decode_workspace_size(B: int, T: int, Hq: int, Hkv: int, D: int, num_splits: int = 0) -> int:
    return load_library().yoco_decode_workspace_size(B, T, Hq, Hkv, D, num_splits)


def decode_workspace(B, T, Hq, Hkv, D, num_splits=0, device="cuda") -> torch.Tensor:
    """A zero-filled workspace (its counter section must start at zero)."""
    nbytes = max(16, yoco_decode_workspace_size(B, T, Hq, Hkv, D, num_splits))
    return torch.zeros(math.ceil(nbytes / 16) * 4, dtype=torch.float32, device=device)


def _torch_stream(stream, device):
    """The torch stream object for a binding `stream` argument (None: the current one)."""
    if stream is None:
        return torch.cuda.current_stream(device)
    if isinstance(stream, torch.cuda.Stream):
        return stream
    return torch.cuda.ExternalStream(int(stream), device=device)


# Workspaces the binding keeps for calls that pass none: one per (device, stream,
# kind), so that calls on one stream (which run in order) share it and calls on
# different streams never do. An entry is [tensor, counters]: `counters` is the
# B * Hkv of the last decode that used it, whose counter section that call left
# at zero.
_WORKSPACES: dict = {}


def _cached_workspace(kind: str, nbytes: int, device, stream, counters: int = 0) -> torch.Tensor | None:
    """The binding's own workspace of at least nbytes for a call on (device, stream).

    Allocated zero-filled (on the call's stream) the first time and whenever a
    call needs more bytes than the one held; otherwise reused without any
    allocation. For the decode (kind "decode"), when this call has more merge
    counters than the last one, the bytes between the two counter sections
    (which held the last call's partials) are zeroed first on the call's stream.
    Pass a workspace explicitly under HIP graph capture."""
    if nbytes == 0:                          # no workspace used: the held one keeps its state
        return None
    ts = _torch_stream(stream, device)
    key = (torch.device(device).index, ts.cuda_stream, kind)
    entry = _WORKSPACES.get(key)
    with torch.cuda.stream(ts):
        if entry is None or entry[0].numel() * 4 < nbytes:
            entry = [torch.zeros(math.ceil(max(16, nbytes) / 16) * 4, dtype=torch.float32, device=device), 0]
            _WORKSPACES[key] = entry
        elif counters > entry[1]:
            entry[0][entry[1]:counters].zero_()     # 4-byte counters: one float32 slot each
        entry[1] = max(counters, 0)
    return entry[0]


def _decode_workspace_for(B, T, Hq, Hkv, D, num_splits, device, stream) -> torch.Tensor | None:
    nbytes = yoco_decode_workspace_size(B, T, Hq, Hkv, D, num_splits)
    return _cached_workspace("decode", nbytes, device, stream, counters=B * Hkv)


def yoco_cross_attn_decode(q, k_cache, v_cache, out, lse=None, seq_lens=None, T: int | None = None,
                           num_splits: int = 0, workspace: torch.Tensor | None = None, scale: float = 0.0,
                           stream=None, Hkv: int | None = None) -> None:
    """q [B, Hq, D]; caches [B, Hkv, T, D]; out [B, Hq, D] fp32; lse [B, Hq] fp32."""
    lib = load_library()
    _need_contiguous(q=q, out=out, lse=lse, seq_lens=seq_lens)
    B, Hq, D = q.shape
    kc, vc = _as_t4(k_cache), _as_t4(v_cache)
    Hkv = _heads(k_cache, Hkv)
    T = kc.rows if T is None else T
    if workspace is None:
        workspace = _decode_workspace_for(B, T, Hq, Hkv, D, num_splits, q.device, stream)
    _check(lib.yoco_cross_attn_decode(q.data_ptr(), kc, vc, _ptr(seq_lens), B, T, Hq, Hkv, D, float(scale),
                                      out.data_ptr(), _ptr(lse), _ptr(workspace), _bytes(workspace), int(num_splits),
                                      _dtype_code(q), _stream(stream)))


def yoco_cross_attn_decode_noalloc(q, k_cache, v_cache, out, lse=None, seq_lens=None, T: int | None = None,
                                   num_splits: int = 0, scale: float = 0.0, stream=None,
                                   Hkv: int | None = None) -> None:
    """yoco_cross_attn_decode without a workspace: the partials and merge counters
    live in the library's per-GPU scratch array (no allocation anywhere)."""
    lib = load_library()
    _need_contiguous(q=q, out=out, lse=lse, seq_lens=seq_lens)
    B, Hq, D = q.shape
    kc, vc = _as_t4(k_cache), _as_t4(v_cache)
    Hkv = _heads(k_cache, Hkv)
    T = kc.rows if T is None else T
    _check(lib.yoco_cross_attn_decode_noalloc(q.data_ptr(), kc, vc, _ptr(seq_lens), B, T, Hq, Hkv, D, float(scale),
                                              out.data_ptr(), _ptr(lse), int(num_splits), _dtype_code(q),
                                              _stream(stream)))


def yoco_cross_attn_decode_compose_on_read(q, k1_cache, ki_cache, v1_cache, vi_cache, alpha, out, lse=None,
                                           lam: float = 35.0, seq_lens=None, T: int | None = None,
                                           num_splits: int = 0, workspace: torch.Tensor | None = None,
                                           scale: float = 0.0, stream=None, Hkv: int | None = None) -> None:
    """Decode over raw caches of layer 1 and layer i, composing K', V' per row on read."""
    lib = load_library()
    _need_contiguous(q=q, out=out, lse=lse, seq_lens=seq_lens)
    B, Hq, D = q.shape
    k1, ki, v1, vi = (_as_t4(x) for x in (k1_cache, ki_cache, v1_cache, vi_cache))
    Hkv = _heads(ki_cache, Hkv)
    T = ki.rows if T is None else T
    if workspace is None:
        workspace = _decode_workspace_for(B, T, Hq, Hkv, D, num_splits, q.device, stream)
    aK1, aK2, aV1, aV2 = (float(a) for a in alpha)
    _check(lib.yoco_cross_attn_decode_compose_on_read(
        q.data_ptr(), k1, ki, v1, vi, _ptr(seq_lens), B, T, Hq, Hkv, D, float(lam), aK1, aK2, aV1, aV2, float(scale),
        out.data_ptr(), _ptr(lse), _ptr(workspace), _bytes(workspace),
        int(num_splits), _dtype_code(q), _stream(stream)))


def one_token(t: torch.Tensor) -> Tensor4:
    """[B, H, D] (D contiguous), the rows of one token -> Tensor4 with stride_t = 0."""
    if t.dim() != 3 or t.stride(2) != 1:
        raise ValueError("expected a [B, H, D] tensor with a contiguous last axis")
    return Tensor4(t.data_ptr(), t.stride(0), t.stride(1), 0, 1)


def _source_t4(x) -> Tensor4:
    if isinstance(x, Tensor4):
        return x
    return one_token(x) if x.dim() == 3 else head_major(x)


def yoco_self_attn_decode(q, k1_new, ki_new, v1_new, vi_new, k_cache, v_cache, alpha, out, lse=None,
                          lam: float = 35.0, seq_lens=None, T: int | None = None, num_splits: int = 0,
                          workspace: torch.Tensor | None = None, scale: float = 0.0, stream=None,
                          Hkv: int | None = None) -> None:
    """Self-decoder decode step of layer i: compose the new token's K', V' (sources [B, Hkv, D]
    one-token tensors, [B, Hkv, T, D] caches read at row seq_len-1, or Tensor4), write them at
    row seq_len-1 of k_cache, v_cache [B, Hkv, T, D] and attend over rows [0, seq_len)."""
    lib = load_library()
    _need_contiguous(q=q, out=out, lse=lse, seq_lens=seq_lens)
    B, Hq, D = q.shape
    srcs = [_source_t4(x) for x in (k1_new, ki_new, v1_new, vi_new)]
    kc, vc = _as_t4(k_cache), _as_t4(v_cache)
    Hkv = _heads(k_cache, Hkv)
    T = kc.rows if T is None else T
    if workspace is None:
        workspace = _decode_workspace_for(B, T, Hq, Hkv, D, num_splits, q.device, stream)
    aK1, aK2, aV1, aV2 = (float(a) for a in alpha)
    _check(lib.yoco_self_attn_decode(
        q.data_ptr(), *srcs, kc, vc, _ptr(seq_lens), B, T, Hq, Hkv, D, float(lam), aK1, aK2, aV1, aV2,
        float(scale), out.data_ptr(), _ptr(lse), _ptr(workspace), _bytes(workspace),
        int(num_splits), _dtype_code(q), _stream(stream)))


def yoco_cross_attn_decode_partial(q, k_cache, v_cache, workspace, num_splits: int, seq_lens=None,
                                   T: int | None = None, scale: float = 0.0, stream=None,
                                   Hkv: int | None = None) -> None:
    lib = load_library()
    _need_contiguous(q=q, workspace=workspace, seq_lens=seq_lens)
    B, Hq, D = q.shape
    kc, vc = _as_t4(k_cache), _as_t4(v_cache)
    Hkv = _heads(k_cache, Hkv)
    T = kc.rows if T is None else T
    _check(lib.yoco_cross_attn_decode_partial(q.data_ptr(), kc, vc, _ptr(seq_lens), B, T, Hq, Hkv, D, float(scale),
                                              workspace.data_ptr(), workspace.numel() * workspace.element_size(),
                                              int(num_splits), _dtype_code(q), _stream(stream)))


def yoco_decode_merge(workspace, B: int, Hq: int, Hkv: int, D: int, num_splits: int, out, lse=None,
                      stream=None) -> None:
    lib = load_library()
    _need_contiguous(workspace=workspace, out=out, lse=lse)
    _check(lib.yoco_decode_merge(workspace.data_ptr(), workspace.numel() * workspace.element_size(), B, Hq, Hkv, D,
                                 int(num_splits), out.data_ptr(), _ptr(lse), _stream(stream)))


def yoco_cross_attn_prefill(q, k_cache, v_cache, p0: int, out, lse=None, scale: float = 0.0, stream=None,
                            Hkv: int | None = None) -> None:
    """q [B, C, Hq, D] bf16; caches [B, Hkv, Tcap, D] bf16; out [B, C, Hq, D] fp32 or bf16; lse [B, Hq, C]."""
    lib = load_library()
    B, C, Hq, D = q.shape
    # a chunk sliced out of a [B, T, Hq, D] tensor is row-contiguous per sequence
    # but not across sequences when B > 1; the kernel needs [B, C, Hq, D] dense
    _need_contiguous(q=q, out=out, lse=lse)
    kc, vc = _as_t4(k_cache), _as_t4(v_cache)
    Hkv = _heads(k_cache, Hkv)
    _check(lib.yoco_cross_attn_prefill(q.data_ptr(), kc, vc, B, C, int(p0), Hq, Hkv, D, float(scale), out.data_ptr(),
                                       _dtype_code(out), _ptr(lse), _dtype_code(q), _stream(stream)))


def yoco_version() -> int:
    return load_library().yoco_version()


def yoco_last_error() -> str:
    return load_library().yoco_last_error().decode()


def yoco_status_string(status: int) -> str:
    return load_library().yoco_status_string(status).decode()
