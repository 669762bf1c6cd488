"""DART chunk state memories and state-memory attention on AMD MI355X (gfx950).

The computation runs in hand-written HIP kernels behind a C ABI
(``include/dart.h``, ``libdart.so``); ``state_memory_attention_amd.dart`` is
its Python binding.  The library is loaded on first use and every call raises
if it is missing: there is no fallback path.
"""
from .dart import (  # noqa: F401
    DART_BF16, DART_F32, DART_PATH_AUTO, DART_PATH_GENERAL, DartError, abi_version,
    dart_chunk_states, dart_chunk_states_bwd, dart_decode_state_update, dart_sma_bwd,
    dart_sma_decode, dart_sma_decode_noalloc, dart_sma_fwd,
    dart_chunk_rms, dart_chunk_states_rms, dart_decode_state_update_rms, dart_ssd_fwd, dart_sma_decode_rms, dart_sma_fwd_rms,
    dart_sma_bwd_rms,
    decode_workspace_bytes, num_chunks, score_dtype, set_path,
)
