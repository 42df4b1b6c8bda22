"""Multi-scale deformable attention on MI355X (gfx950): a C-ABI HIP library
(``libmsda.so``, declared in ``include/msda.h``) and its thin Python binding.

The binding (and with it torch and the library) is loaded on first use, so the
seeded workload generators in ``workloads`` import without a GPU.
"""
__all__ = ["msda_forward", "msda_backward", "msda_backward_noalloc", "ms_deformable_attention", "MSDeformableAttention",
           "msda_producer_forward", "msda_fused_forward", "msda_producer_backward", "MSDAProducer",
           "load_library"]


def __getattr__(name):
    if name in __all__:
        from . import binding
        return getattr(binding, name)
    raise AttributeError(name)
