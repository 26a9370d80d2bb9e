"""etc-moe: an event-tensor Mixture-of-Experts layer for AMD MI355X (gfx950).

One persistent HIP kernel runs RMSNorm, the router, top-k and softmax, per-expert
counts with an exclusive-scan permutation, SwiGLU expert GEMM tiles on bf16 MFMA and
a weighted combine; event counters in global memory release each tile once its true
dependencies are met.  The same mechanism runs a split-K GEMM.

The compute lives in ``libetc_moe.so`` behind the C ABI of ``include/etc_moe.h``;
``moe_layer_scheduling_amd.binding`` marshals torch tensors into it.  The library is
loaded on first use and a missing or stale build raises ``EtcLibraryError`` -- there
is no CPU fallback.
"""

from . import synth  # noqa: F401  (pure-Python input generator, no GPU needed)

_BINDING_NAMES = {
    "moe_layer", "splitk_gemm", "MoEWorkspace", "SplitKWorkspace", "load_library",
    "EtcError", "EtcLibraryError", "library_path", "default_workers", "Workspace",
}


def __getattr__(name):
    if name in _BINDING_NAMES:
        from . import binding

        return getattr(binding, name)
    raise AttributeError(name)
