"""fp64 CPU oracle for the SSD scan path -- test infrastructure only (see ssd_oracle)."""
from .ssd_oracle import (chunk_metadata, group_of_head, scan_decode, scan_prefill,
                         transform_dt)

__all__ = ["chunk_metadata", "group_of_head", "scan_decode", "scan_prefill", "transform_dt"]
