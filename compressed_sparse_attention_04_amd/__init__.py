"""MI355X (gfx950) compressed sparse attention (CSA) and heavily compressed
attention (HCA) for one layer on one GPU.

The compute path is the HIP library ``libcsa.so`` behind the C ABI declared
in ``include/csa.h``; :mod:`.binding` marshals torch tensors into it.
"""
