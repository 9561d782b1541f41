"""Block-quantized (ggml Q4_0 / Q4_K / Q6_K) weight products on MI355X.

The compute lives in ``libgq.so`` (HIP kernels for gfx950 behind the C ABI of
``include/gq.h``); :mod:`._binding` is a thin ctypes layer with the same entry
point names that marshals torch tensors (device memory, streams) into it.

The binding is loaded on first use, so ``block_quantized_weight_q4_amd.synth``
(the seeded input generator) can be imported without the library.
"""
__all__ = [
    "gq_abi_version", "gq_block_info", "gq_dequant", "gq_matvec", "gq_matvec_id",
    "gq_matvec_id_workspace", "gq_matvec_id_check", "gq_matmul", "gq_route_topk", "gq_matvec_glu",
    "gq_matvec_id_glu", "gq_matvec_id_noalloc", "gq_route_topk_plan", "gq_route_matvec_id_glu", "GqError", "TYPES", "lib_path",
]


def __getattr__(name):
    if name in __all__:
        from . import _binding
        return getattr(_binding, name)
    raise AttributeError(name)
