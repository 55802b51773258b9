"""FlashAttention forward (and backward) for MI355X (gfx950).

The hot path is the HIP library ``libfa.so`` (C ABI in ``include/fa.h``);
this package only marshals arguments to it (``fa_fwd``, ``fa_fwd_f32``,
``fa_fwd_fp8``, ``fa_bwd``, ``fa_decode_paged``, ``fa_status_string``) and
offers ``attention()``, ``attention_fp8()``, ``attention_backward()`` and
``decode_paged()``, which allocate the outputs with torch and call the
library. The standard (materializing) baseline is in
``io_aware_tiled_09_amd.standard`` (libfa_std.so). Seeded synthetic inputs live in ``io_aware_tiled_09_amd.inputs``.
"""
from ._binding import (EXPORTS, FA_OK, FAError, LIB_PATH, attention, attention_backward,
                       attention_fp8, decode_paged, fa_bwd, fa_bwd_noalloc,
                       fa_bwd_noalloc_max_rows, fa_decode_paged,
                       fa_decode_workspace_bytes, fa_fwd, fa_fwd_f32, fa_fwd_fp8,
                       fa_fwd_grid, fa_status_string, fa_tile_cols, fa_tile_rows, load)

__all__ = ["attention", "attention_backward", "attention_fp8", "decode_paged", "fa_fwd",
           "fa_fwd_f32", "fa_fwd_fp8", "fa_bwd", "fa_bwd_noalloc", "fa_bwd_noalloc_max_rows",
           "fa_decode_paged", "fa_decode_workspace_bytes",
           "fa_status_string", "fa_tile_rows", "fa_tile_cols", "fa_fwd_grid", "FAError", "FA_OK",
           "EXPORTS",
           "LIB_PATH", "load"]
