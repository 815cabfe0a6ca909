"""Cross-layer KV sharing (YOCO / YOCO++) hot path for AMD MI355X (gfx950).

The compute runs in hand-written HIP kernels inside ``libyoco.so``; this
package only builds that library and marshals torch tensors across its C ABI.
"""
from .binding import (  # noqa: F401
    EXPORTED,
    LIB_PATH,
    Tensor4,
    YocoError,
    decode_workspace,
    head_major,
    load_library,
    one_token,
    token_major,
    yoco_compose_backward_workspace_size,
    yoco_compose_kv,
    yoco_compose_kv_backward,
    yoco_cross_attn_decode,
    yoco_cross_attn_decode_compose_on_read,
    yoco_cross_attn_decode_noalloc,
    yoco_cross_attn_decode_partial,
    yoco_cross_attn_prefill,
    yoco_decode_merge,
    yoco_decode_num_splits,
    yoco_decode_workspace_size,
    yoco_last_error,
    yoco_self_attn_decode,
    yoco_status_string,
    yoco_version,
)
