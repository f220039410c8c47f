"""MI355X-native sparse paged decode step (gfx950 HIP kernels behind a C ABI).

Importing the package loads nothing; the HIP library is loaded on first use by
``adaptive_sparse_paged_amd.lib`` and every operation fails loudly when it is
missing.
"""
