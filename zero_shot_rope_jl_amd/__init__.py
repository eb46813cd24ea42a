"""Python binding of libjetlong.so, the gfx950 Jet-Long bifocal RoPE attention
library ("Jet-Long: Efficient Long-Context Extension with Dynamic Bifocal
RoPE", §3).

The functions carry the C ABI's names and only marshal arguments: shapes,
dtypes, device pointers and the current HIP stream are read from torch
tensors and passed to the library, which does every step of the computation
in its own kernels.  There is no fallback: if the library is missing the
import fails, and a non-OK return code raises :class:`JetLongError`.
"""
from .binding import (  # noqa: F401
    JL_BF16, JL_F32, JL_OK, JL_EINVAL, JL_EUNSUPPORTED, JL_EHIP, JL_ESPACE,
    JetLongError, lib, lib_path, jl_version, jl_last_error, jl_schedule,
    jl_bifocal_prefill, jl_bifocal_prefill_workspace, jl_bifocal_prefill_chunk, jl_bifocal_decode,
    jl_bifocal_prefill_unfused, jl_bifocal_prefill_unfused_workspace, alloc_prefill_unfused_workspace,
    jl_bifocal_prefill_chunk_paged, jl_bifocal_decode_rkc, RotatedKeyCache, JLRotatedKeys,
    jl_bifocal_decode_paged, jl_fi_table, jl_fi_table_fill_host, alloc_fi_table, jl_bifocal_prefill_fi,
    jl_bifocal_decode_fi, jl_rope_interleaved_to_half,
    jl_bifocal_decode_workspace, jl_table_fill_host, alloc_table, alloc_prefill_workspace,
    alloc_decode_workspace, jl_bifocal_decode_unfused, jl_bifocal_decode_unfused_workspace,
    alloc_decode_unfused_workspace, jl_device_info, jl_bifocal_decode_noalloc,
    jl_bifocal_prefill_chunk_workspace, ChunkState, alloc_chunk_state,
)
