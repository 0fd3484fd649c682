"""MI355X (gfx950) library for the Gated DeltaNet recurrent-state update.

Entry points (same names as the C ABI in include/gdn.h): gdn_decode_step,
gdn_spec_decode, gdn_copy_state_blocks, gdn_chunk_prefill, gdn_replay_decode,
gdn_replay_flush, gdn_replay_rollback, and the Mamba2 variant gdn_mamba2_decode_step,
gdn_mamba2_replay_decode, gdn_mamba2_replay_flush, gdn_mamba2_replay_rollback.
The kernels live in libgdn.so, built in-tree by
``python -m gated_deltanet_state_gdn_amd.build``; importing this package does
not need the library, calling an entry point does (and raises if it is
missing).
"""
from ._binding import (  # noqa: F401
    EXPORTS, GDN_BF16, GDN_EINVAL, GDN_ELAUNCH, GDN_EUNSUPPORTED, GDN_F16, GDN_F32, GDN_OK, GdnError, LIB_PATH, Ring,
    dtype_code, gdn_chunk_prefill, gdn_copy_state_blocks, gdn_chunk_prefill_workspace_bytes, gdn_decode_step, gdn_last_error,
    gdn_replay_decode, gdn_replay_decode_noalloc, gdn_replay_flush, gdn_replay_rollback, gdn_replay_workspace_bytes, gdn_spec_decode,
    gdn_status_string, lib, make_state_table, new_ring, state_refs_bytes, M2Ring, new_m2_ring,
    gdn_mamba2_decode_step, gdn_mamba2_replay_decode, gdn_mamba2_replay_flush, gdn_mamba2_replay_rollback,
)
