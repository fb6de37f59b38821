"""libmambamix: the selective-SSM mixer core as a C-ABI HIP library for gfx950 (MI355X)."""
