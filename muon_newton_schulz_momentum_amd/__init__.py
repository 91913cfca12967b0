"""libmuon: a Muon optimizer step (FP32 momentum -> BF16 -> batched symmetric
Newton–Schulz -> FP32 apply with decoupled weight decay) on one AMD Instinct MI355X.

The compute path is the C-ABI library libmuon.so (hand-written HIP for gfx950), declared
in include/muon.h.  `muon_newton_schulz_momentum_amd.binding` is its ctypes binding
(argument marshalling only) and `harness` builds torch-owned tensors around it.
Importing the package itself loads nothing native; importing `binding` fails loudly when
the shared library has not been built.
"""

__all__ = ["workloads", "binding", "harness", "build"]


def __getattr__(name):
    if name in __all__:
        import importlib
        return importlib.import_module(f"{__name__}.{name}")
    raise AttributeError(name)
