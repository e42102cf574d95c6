"""MI355X (gfx950) Gated DeltaNet streaming core.

The library ``libgdn_stream.so`` (hand-written HIP kernels behind the C ABI in
``include/gdn_stream.h``) does all the work; ``binding`` only marshals torch
tensors into that ABI.  Build it with ``python -m gated_deltanet_streaming_amd.build``.
"""
from .binding import (GdnError, Stream, gdn_chunk_bidir, gdn_chunk_forward, gdn_chunk_reverse,
                      gdn_last_error, gdn_profile, gdn_profile_read, gdn_state_get, gdn_state_set,
                      gdn_stream_destroy, gdn_stream_init, library_path, load_library)

__all__ = ["GdnError", "Stream", "gdn_chunk_bidir", "gdn_chunk_forward", "gdn_chunk_reverse",
           "gdn_last_error", "gdn_profile", "gdn_profile_read", "gdn_state_get", "gdn_state_set",
           "gdn_stream_destroy", "gdn_stream_init", "library_path", "load_library"]
