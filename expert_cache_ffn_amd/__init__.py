"""expert_cache_ffn_amd: one expert-cached MoE layer forward on MI355X (gfx950).

The compute lives in libecf.so (HIP kernels + host C++ behind the C ABI in
include/ecf.h).  This package is the thin Python face of that ABI:
  _lib   -- ctypes wrappers, one per C entry point, same names;
  layer  -- torch conveniences (device buffers, workspace, argument structs);
  build  -- compiles libecf.so in-tree with hipcc for gfx950.
Importing the package does not load the library; the first call does, and
fails loudly if the library has not been built.
"""
from ._lib import (  # noqa: F401
    ECF_OK, ECF_EINVAL, ECF_ENOSPC, ECF_EHIP, ECF_EUNSUPPORTED, ECF_ESTATE,
    ECF_F32, ECF_BF16, ECF_MXFP4,
    ECF_Q_AUTO, ECF_Q_ALL_GPU, ECF_Q_ALL_HOST, ECF_Q_FIXED,
    ECF_PATH_AUTO, ECF_PATH_DECODE, ECF_PATH_PREFILL,
    EcfError, Shape, LayerArgs, StepStats, CacheStats, BwProfile, EXPORTS,
    lib, make_shape,
    ecf_expert_bytes, ecf_expert_layout, ecf_workspace_bytes, qstar_split,
    ecf_cache_create, ecf_cache_destroy, expert_cache_lookup, expert_cache_evict,
    ecf_cache_available, ecf_cache_slot_of, ecf_cache_get_stats, ecf_cache_resize,
    prefetch_layer, moe_layer_forward, moe_layer_forward_noalloc, ecf_noalloc_scratch_bytes,
    ecf_host_experts, ecf_bandwidth_profile,
    ecf_profile_enable, ecf_profile_get_all, ecf_profile_reset, ecf_stream_read, ecf_mfma_rate,
)
