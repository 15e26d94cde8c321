"""negacyclic_ntt_amd -- batched RNS negacyclic NTT, pointwise products, Galois
automorphisms and the hybrid rotation key-switch on AMD Instinct MI355X (gfx950).

The arithmetic runs in hand-written HIP kernels behind a C ABI
(``include/negacyclic_ntt.h``); this package is a thin ctypes binding that takes
torch tensors for device memory and streams.  ``inputs`` and ``workloads`` are
pure-Python helpers (seeded synthetic data and workload shapes).
"""
from . import inputs, workloads  # noqa: F401  (pure Python, no GPU needed)


def __getattr__(name):
    # The binding loads the shared library on first use, so that importing the
    # package (e.g. for `inputs`) does not require a GPU or a built library.
    if name.startswith("__") or name in ("binding", "build"):
        raise AttributeError(name)
    import importlib
    return getattr(importlib.import_module(__name__ + ".binding"), name)
