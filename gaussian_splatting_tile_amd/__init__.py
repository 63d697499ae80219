"""MI355X-native tile-based 3D Gaussian Splatting rasterizer (forward + backward).

The compute path is libgs.so (HIP kernels for gfx950 behind the C ABI in
include/gs.h); this package is its thin torch binding. The library is loaded
on first use; every entry point raises ImportError if it has not been built
(there is no fallback path).
"""
from ._lib import EXPORTS, GsError, LIB_PATH
from .rasterizer import (appearance_bwd, appearance_fwd, appearance_params, BinBuffers, Rasterizer, Scene, bin_and_sort, bin_and_sort_async, camera, chunk_words, ckpt_rows, part_bytes,
                         composite_bwd, composite_fwd, constants, preprocess, preprocess_bwd, tile_ranges,
                         tile_ranges_async, tiles_xy, version, ViewBatch, ViewStack, preprocess_views,
                         bin_and_sort_views_async, scheduled_forward)

__all__ = ["appearance_bwd", "appearance_fwd", "appearance_params", "EXPORTS", "GsError", "LIB_PATH", "BinBuffers", "Rasterizer", "Scene", "bin_and_sort",
           "bin_and_sort_async", "camera", "chunk_words", "ckpt_rows", "part_bytes", "composite_bwd", "composite_fwd", "constants", "preprocess",
           "preprocess_bwd",
           "tile_ranges", "tile_ranges_async", "tiles_xy", "version", "ViewBatch", "ViewStack",
           "preprocess_views", "bin_and_sort_views_async", "scheduled_forward"]
