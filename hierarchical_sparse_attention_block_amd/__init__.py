"""MI355X (gfx950) two-level sparse-attention decode: block filtering on
per-block key max/min bounds, label-channel token selection inside the kept
blocks, and exact attention over the kept tokens, as one C-ABI HIP library
(``libhsab.so``) with a thin ctypes binding (``hsab``)."""
