"""MI355X-native (gfx950) Mamba2 SSD selective-state-space scan.

The scan runs in libssd.so (HIP kernels behind a C ABI, include/ssd.h); this package is
its Python binding (``api``), the build script (``build``) and the seeded synthetic
input generators (``inputs``).
"""
from .api import (ssd_abi_version, ssd_build_chunk_metadata, ssd_chunk_metadata_count,
                  ssd_prefill, ssd_prefill_workspace_size, ssd_state_update,
                  ssd_status_string)

__all__ = ["ssd_abi_version", "ssd_build_chunk_metadata", "ssd_chunk_metadata_count",
           "ssd_prefill", "ssd_prefill_workspace_size", "ssd_state_update",
           "ssd_status_string"]
