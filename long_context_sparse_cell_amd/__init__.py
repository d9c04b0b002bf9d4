"""FS-L (FreeSolo-Linear) two-branch sparse attention for MI355X (gfx950).

The compute lives in a C-ABI HIP library (libfsl.so, declared in include/fsl.h);
``long_context_sparse_cell_amd.fsl`` is its thin Python binding and
``long_context_sparse_cell_amd.synth`` draws the seeded synthetic inputs.
Importing the package loads nothing; the binding loads the library on first use
and raises if it is missing.
"""
