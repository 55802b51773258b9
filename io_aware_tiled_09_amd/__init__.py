"""FlashAttention forward for MI355X (gfx950).

The hot path is the HIP library ``libfa.so`` (C ABI in ``include/fa.h``);
this package only marshals arguments to it (``fa_fwd``, ``fa_fwd_f32``,
``fa_status_string``) and offers ``attention()``, which allocates the outputs
with torch and calls ``fa_fwd``. Seeded synthetic inputs live in
``io_aware_tiled_09_amd.inputs``.
"""
from ._binding import (EXPORTS, FA_OK, FAError, LIB_PATH, attention, fa_fwd, fa_fwd_f32,
                       fa_status_string, fa_tile_cols, fa_tile_rows, load)

__all__ = ["attention", "fa_fwd", "fa_fwd_f32", "fa_status_string", "fa_tile_rows",
           "fa_tile_cols", "FAError", "FA_OK", "EXPORTS", "LIB_PATH", "load"]
