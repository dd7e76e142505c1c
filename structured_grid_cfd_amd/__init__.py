"""structured_grid_cfd_amd -- structured-grid stencil sweeps on AMD MI355X.

Hand-written HIP kernels for gfx950 behind the C ABI of ``libsgc.so``
(declared in ``include/sgc.h``): ``stencil_diffuse2d``, ``field_pack``,
``field_unpack`` and ``flux_diff3d``.  The Python layer in :mod:`.binding`
only marshals torch device tensors and streams into those calls.

Importing the package loads nothing; :mod:`.binding` loads the library on
first use and raises if it has not been built.
"""
__all__ = ["binding", "inputs"]
