"""sparse_autodiff_mesh_amd: locality-aware per-element forward-mode AD of
mesh energies with GPU sparse assembly on AMD Instinct MI355X (gfx950).

The compute path is liblad.so (HIP kernels + C ABI in include/lad.h); the
`binding` module is its ctypes front end.  Submodules are imported on
demand: `inputs` (seeded synthetic grids) needs neither the library nor a GPU.
"""
__all__ = ["binding", "inputs", "build"]


def __getattr__(name):
    if name in __all__:
        import importlib
        return importlib.import_module(f"{__name__}.{name}")
    raise AttributeError(name)
