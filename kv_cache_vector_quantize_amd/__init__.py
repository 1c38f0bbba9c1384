"""MI355X (gfx950) online KV-vector quantization, decode attention from
packed codes (contiguous or paged caches), inner-product top-k over codes and
dequantization.  The compute runs in libtq.so (hand-written HIP kernels behind
a C ABI, declared in include/tq.h); this package is a thin ctypes binding."""
from ._lib import (  # noqa: F401
    EXPORTS,
    LIB_PATH,
    TQ_BF16,
    TQ_F16,
    TQ_F32,
    TQ_LAYOUT_ROW,
    TQ_KERNEL_DECODE_SPLIT,
    TQ_KERNEL_DEQUANTIZE,
    TQ_KERNEL_QUANTIZE,
    TQ_KERNEL_TOPK,
    TQ_LAYOUT_TILE32,
    Codebook,
    Codes,
    TQError,
    lib,
    tq_attn_decode,
    tq_attn_decode_paged,
    tq_attn_decode_paged_workspace,
    tq_attn_decode_workspace,
    tq_codebook_solver_limits,
    tq_codebook_values,
    tq_dequantize,
    tq_ip_topk,
    tq_ip_topk_workspace,
    tq_profile_enable,
    tq_profile_read,
    tq_quantize_kv,
    tq_quantize_kv_paged,
)
