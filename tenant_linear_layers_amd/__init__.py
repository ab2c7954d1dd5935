"""BitDelta multi-tenant linear layer for MI355X (gfx950).

The path lives in libbitdelta.so (HIP kernels behind the C ABI of
include/bitdelta.h); this package is the build script and a thin ctypes
binding with the same names.
"""

from .bitdelta import (  # noqa: F401
    ALPHA_PER_MATRIX,
    ALPHA_PER_ROW,
    CACHE_ABSENT,
    CACHE_FULL,
    CACHE_HIT,
    CACHE_LOAD,
    CACHE_LOADING,
    CACHE_QUEUED,
    CACHE_RESIDENT,
    EXPORTS,
    LIB_PATH,
    MAX_VARIANTS,
    BitDeltaError,
    DeltaCache,
    compress,
    compress_noalloc,
    compress_workspace_size,
    delta_layout,
    delta_views,
    lib,
    linear,
    linear_multi,
    monosoup_merge,
    monosoup_workspace_size,
    probe_decode_loads,
    probe_mfma_bf16,
    probe_stream_read,
    Router,
    ratio_to_f32_bits,
    reconstruct,
    status_string,
)
from .deltafile import delta_blob, load_delta, read_delta_header, save_delta  # noqa: F401
