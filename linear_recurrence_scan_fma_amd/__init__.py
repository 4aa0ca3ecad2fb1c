"""Linear-recurrence scan engine for AMD MI355X (gfx950).

The compute lives in a C-ABI shared library (``liblrs.so``) built from the
hand-written HIP sources in ``csrc/``; this package only marshals arguments
into it (see :mod:`.binding`).  Importing the package does not load the
library; the first call does, and fails loudly if it is not built.
"""
