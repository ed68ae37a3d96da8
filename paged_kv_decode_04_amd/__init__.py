"""paged_kv_decode_04_amd: paged-KV decode attention and the paged KV append on AMD MI355X (gfx950).

The compute path is the HIP library ``libpkv.so`` (hand-written gfx950 kernels behind the C ABI in
``include/pkv.h``).  ``paged_kv_decode_04_amd.pkv`` is its thin Python binding (argument marshalling only; PyTorch
supplies device memory and streams).  ``paged_kv_decode_04_amd.workloads`` holds the seeded input generators.

Importing this package loads nothing; the binding loads ``libpkv.so`` on first use and raises if it is missing.
"""
__all__ = ["pkv", "workloads"]
__version__ = "0.1.0"
