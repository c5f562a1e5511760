"""MI355X-native HiKVP knowledge-injected attention.

The compute path is the C-ABI library libatlaskv.so (hand-written HIP kernels
for gfx950); `hierarchical_kv_pruning_amd.atlaskv` is its thin ctypes binding.
Importing the package itself loads nothing.
"""
