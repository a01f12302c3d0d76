"""Softmax-gated token-pool KV compression for AMD Instinct MI355X (gfx950).

The compute lives in ``libkvc.so`` (HIP kernels behind the C ABI in
``include/kvc.h``); ``kvc`` is its ctypes binding.  Importing the package does
not load the library; the first call does and fails loudly if it is missing.
"""
from .kvc import (ITEM_DTYPE, KvcError, PLAN_DTYPE, PLAN_SENTINEL, PreparedCall, items_to_device,
                  kvc_c128_online_decode,
                  kvc_c128_online_decode_layers, kvc_c128_online_decode_quant,
                  kvc_c128_online_prefill, kvc_c128_online_prefill_fused,
                  kvc_c128_online_prefill_quant, kvc_c128_plan_prefill,
                  kvc_c128_fused_capacity, kvc_c128_plan_prefill_fused, kvc_compress_decode_ring,
                  kvc_compress_decode_ring_layers, kvc_compress_decode_ring_paged, kvc_compress_prefill,
                  kvc_compress_prefill_paged,
                  kvc_diag_convert, kvc_plan_pool_prefill, kvc_seed_tail_ring,
                  plans_to_device, prepare)

__all__ = ["ITEM_DTYPE", "KvcError", "PLAN_DTYPE", "PLAN_SENTINEL", "PreparedCall", "items_to_device",
           "kvc_c128_online_decode",
           "kvc_c128_online_decode_layers", "kvc_c128_online_decode_quant",
           "kvc_c128_online_prefill", "kvc_c128_online_prefill_fused",
           "kvc_c128_online_prefill_quant", "kvc_c128_plan_prefill",
           "kvc_c128_fused_capacity", "kvc_c128_plan_prefill_fused", "kvc_compress_decode_ring", "kvc_compress_decode_ring_layers",
           "kvc_compress_decode_ring_paged",
           "kvc_compress_prefill", "kvc_compress_prefill_paged",
           "kvc_diag_convert", "kvc_plan_pool_prefill", "kvc_seed_tail_ring",
           "plans_to_device", "prepare"]
