"""MI355X-native Mamba-2 SSD chunked scan (forward, recompute backward, state moments).

The computation lives in the HIP library built from ``csrc/`` (C ABI in
``include/ssd.h``); :mod:`mamba_ssd_chunked_amd.ssd` is its thin ctypes binding
and :mod:`mamba_ssd_chunked_amd.inputs` draws the seeded synthetic inputs.
"""
from .ssd import (SSD_BF16, SSD_F32, SSD_OP_BWD, SSD_OP_FWD, SSD_OP_MOMENTS,  # noqa: F401
                  SSD_OP_MOMENTS_BWD, SsdError, backward, dims_of, forward, load_library,
                  make_dims, ssd_bwd, ssd_dims, ssd_fwd, ssd_last_error, ssd_state_moments,
                  ssd_state_moments_bwd, ssd_workspace_size, state_moments, state_moments_bwd,
                  workspace)
