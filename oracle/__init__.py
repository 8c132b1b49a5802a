"""fp64 CPU oracle for the SSD scan path -- test infrastructure only (see ssd_oracle)."""
from .ssd_oracle import (block_indices, chunk_metadata, conv1d_prefill, conv1d_update,
                         group_of_head, scan_decode, scan_prefill, transform_dt)

__all__ = ["block_indices", "chunk_metadata", "conv1d_prefill", "conv1d_update",
           "group_of_head", "scan_decode", "scan_prefill", "transform_dt"]
