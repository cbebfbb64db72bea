"""Nano-batched decoder-layer step for MI355X (gfx950).

The compute path is a HIP library (``libnf.so``) behind a C ABI declared in
``include/nf.h``; :mod:`intra_operation_overlap_amd.binding` marshals
arguments to it.  :mod:`intra_operation_overlap_amd.workload` draws seeded
synthetic inputs.  Importing this package does not load the library.
"""
