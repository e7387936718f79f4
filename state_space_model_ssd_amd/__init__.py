"""Mamba-2 SSD chunked-scan forward on AMD Instinct MI355X (gfx950).

The compute path is the HIP library libssd_hip.so (C ABI: include/ssd.h);
`binding` marshals torch tensors into it.  Importing the package does not
load the library; the first call does, and raises if it is not built.
"""
from .binding import (ssd_fwd, ssd_fwd_seq_idx, load_library, workspace_size,  # noqa: F401
                      workspace_layout, intermediates, make_problem, config_supported,
                      SsdError, STAGES, STAGE_ALL)
