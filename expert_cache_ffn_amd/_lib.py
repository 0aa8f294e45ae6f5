"""ctypes binding of libecf (include/ecf.h): argument marshalling only.

Every function here forwards to the C call of the same name; none computes any
part of the layer.  The library must have been built in-tree
(expert_cache_ffn_amd/libecf.so, see build.py); loading fails loudly if not.
"""
from __future__ import annotations

import ctypes
import os
from ctypes import POINTER, Structure, c_char_p, c_double, c_int32, c_int64, c_size_t, c_void_p

HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(HERE, "libecf.so")

ECF_OK, ECF_EINVAL, ECF_ENOSPC, ECF_EHIP, ECF_EUNSUPPORTED, ECF_ESTATE = 0, -1, -2, -3, -4, -5
ECF_F32, ECF_BF16, ECF_MXFP4 = 0, 1, 2
ECF_Q_AUTO, ECF_Q_ALL_GPU, ECF_Q_ALL_HOST, ECF_Q_FIXED = 0, 1, 2, 3
ECF_PATH_AUTO, ECF_PATH_DECODE, ECF_PATH_PREFILL = 0, 1, 2
DTYPES = {"f32": ECF_F32, "bf16": ECF_BF16, "mxfp4": ECF_MXFP4}

# every symbol include/ecf.h declares
EXPORTS = [
    "ecf_last_error", "ecf_expert_bytes", "ecf_expert_layout", "ecf_workspace_bytes", "qstar_split",
    "ecf_cache_create", "ecf_cache_destroy", "expert_cache_lookup", "expert_cache_evict",
    "ecf_cache_available", "ecf_cache_slot_of", "ecf_cache_get_stats", "ecf_cache_resize",
    "prefetch_layer", "moe_layer_forward", "moe_layer_forward_noalloc", "ecf_noalloc_scratch_bytes",
    "ecf_host_experts", "ecf_bandwidth_profile", "ecf_profile_enable",
    "ecf_profile_get", "ecf_profile_reset", "ecf_stream_read", "ecf_mfma_rate",
]


class EcfError(RuntimeError):
    def __init__(self, code: int, msg: str):
        super().__init__(f"libecf error {code}: {msg}")
        self.code = code


class Shape(Structure):
    _fields_ = [("hidden", c_int32), ("inter", c_int32), ("n_experts", c_int32), ("top_k", c_int32),
                ("w_dtype", c_int32), ("a_dtype", c_int32), ("renorm_topk", c_int32)]


class CacheStats(Structure):
    _fields_ = [(n, c_int64) for n in ("lookups", "hits", "misses", "inserts", "evictions", "dropped")]

    def as_dict(self):
        return {n: getattr(self, n) for n, _ in self._fields_}


class StepStats(Structure):
    _fields_ = [("n_unique", c_int32), ("hits", c_int32), ("misses", c_int32), ("q", c_int32),
                ("host", c_int32), ("path", c_int32), ("bytes_h2d", c_int64), ("bytes_host", c_int64),
                ("ms_wait_route", c_double), ("ms_host_ffn", c_double)]

    def as_dict(self):
        return {n: getattr(self, n) for n, _ in self._fields_}


class BwProfile(Structure):
    _fields_ = [(n, c_double) for n in ("b_p", "b_cpu", "b_read", "b_p_conc", "b_cpu_conc", "b_h")] + \
        [("host_threads", c_int32)]

    def as_dict(self):
        return {n: getattr(self, n) for n, _ in self._fields_}


class LayerArgs(Structure):
    _fields_ = [
        ("shape", Shape), ("layer", c_int32),
        ("d_router_w", c_void_p), ("d_router_logits", c_void_p),
        ("d_expert_ptrs", c_void_p), ("cache", c_void_p),
        ("b_p", c_double), ("b_h", c_double), ("q_mode", c_int32), ("q_fixed", c_int32), ("path", c_int32),
        ("d_ws", c_void_p), ("ws_bytes", c_size_t), ("stream", c_void_p), ("copy_stream", c_void_p),
        ("d_residual", c_void_p), ("d_out_act", c_void_p),
        ("d_topk_idx", c_void_p), ("d_topk_gate", c_void_p), ("d_counts", c_void_p), ("d_perm", c_void_p),
        ("d_logits", c_void_p),
    ]


_lib = None


def lib():
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(f"{LIB_PATH} is missing: build it first (python -m expert_cache_ffn_amd.build "
                               "or __graft_entry__.build())")
        L = ctypes.CDLL(LIB_PATH)
        L.ecf_last_error.restype = c_char_p
        L.ecf_expert_bytes.argtypes, L.ecf_expert_bytes.restype = [POINTER(Shape)], c_size_t
        L.ecf_expert_layout.argtypes, L.ecf_expert_layout.restype = [POINTER(Shape), POINTER(c_size_t)], c_int32
        L.ecf_workspace_bytes.argtypes, L.ecf_workspace_bytes.restype = [POINTER(Shape), c_int32], c_size_t
        L.qstar_split.argtypes, L.qstar_split.restype = [c_int32, c_double, c_double], c_int32
        L.ecf_cache_create.argtypes = [c_int32, c_int32, c_int32, c_int32, c_size_t, c_void_p, c_void_p, c_int32,
                                       POINTER(c_void_p)]
        L.ecf_cache_create.restype = c_int32
        L.ecf_cache_destroy.argtypes, L.ecf_cache_destroy.restype = [c_void_p], None
        L.expert_cache_lookup.argtypes = [c_void_p, c_int32, POINTER(c_int32), c_int32, POINTER(c_int32)]
        L.expert_cache_lookup.restype = c_int32
        L.expert_cache_evict.argtypes = [c_void_p, c_int32, POINTER(c_int32), c_int32, POINTER(c_int32),
                                         POINTER(c_int32)]
        L.expert_cache_evict.restype = c_int32
        L.ecf_cache_available.argtypes, L.ecf_cache_available.restype = [c_void_p], c_int32
        L.ecf_cache_slot_of.argtypes, L.ecf_cache_slot_of.restype = [c_void_p, c_int32, c_int32], c_int32
        L.ecf_cache_get_stats.argtypes = [c_void_p, POINTER(CacheStats)]
        L.ecf_cache_get_stats.restype = c_int32
        L.ecf_cache_resize.argtypes, L.ecf_cache_resize.restype = [c_void_p, c_int32], c_int32
        L.prefetch_layer.argtypes = [c_void_p, c_int32, c_size_t, c_void_p, c_void_p, POINTER(c_int32),
                                     POINTER(c_int32)]
        L.prefetch_layer.restype = c_int32
        L.moe_layer_forward.argtypes = [POINTER(LayerArgs), c_void_p, c_int32, c_void_p, POINTER(StepStats)]
        L.moe_layer_forward.restype = c_int32
        L.moe_layer_forward_noalloc.argtypes = [POINTER(LayerArgs), c_void_p, c_int32, c_void_p,
                                                POINTER(StepStats)]
        L.moe_layer_forward_noalloc.restype = c_int32
        L.ecf_noalloc_scratch_bytes.argtypes, L.ecf_noalloc_scratch_bytes.restype = [], c_size_t
        L.ecf_host_experts.argtypes = [POINTER(Shape), c_int32, c_void_p, c_void_p, c_void_p, c_void_p, c_int32,
                                       c_void_p, c_int32]
        L.ecf_host_experts.restype = c_int32
        L.ecf_bandwidth_profile.argtypes = [POINTER(Shape), c_int32, c_void_p, c_int32, c_void_p, c_size_t,
                                            c_void_p, c_double, POINTER(BwProfile)]
        L.ecf_bandwidth_profile.restype = c_int32
        L.ecf_profile_enable.argtypes, L.ecf_profile_enable.restype = [c_int32], c_int32
        L.ecf_profile_get.argtypes = [c_int32, POINTER(c_char_p), POINTER(c_int64), POINTER(c_double)]
        L.ecf_profile_get.restype = c_int32
        L.ecf_profile_reset.argtypes, L.ecf_profile_reset.restype = [], c_int32
        L.ecf_stream_read.argtypes = [c_void_p, c_size_t, c_void_p, c_void_p]
        L.ecf_stream_read.restype = c_int32
        L.ecf_mfma_rate.argtypes = [c_int32, c_int32, c_void_p, c_void_p, POINTER(c_double)]
        L.ecf_mfma_rate.restype = c_int32
        _lib = L
    return _lib


def _check(rc: int) -> int:
    if rc < 0:
        raise EcfError(rc, lib().ecf_last_error().decode())
    return rc


def _i32(seq):
    seq = [int(v) for v in seq]
    return (c_int32 * max(1, len(seq)))(*seq), len(seq)


# ---- same-named wrappers -------------------------------------------------------------

def make_shape(hidden, inter, n_experts, top_k, w_dtype="bf16", a_dtype="bf16", renorm_topk=1) -> Shape:
    return Shape(hidden, inter, n_experts, top_k, DTYPES[w_dtype] if isinstance(w_dtype, str) else w_dtype,
                 DTYPES[a_dtype] if isinstance(a_dtype, str) else a_dtype, int(renorm_topk))


def ecf_expert_bytes(shape: Shape) -> int:
    n = lib().ecf_expert_bytes(ctypes.byref(shape))
    if n == 0:
        raise EcfError(ECF_EINVAL, lib().ecf_last_error().decode())
    return n


def ecf_expert_layout(shape: Shape):
    arr = (c_size_t * 6)()
    _check(lib().ecf_expert_layout(ctypes.byref(shape), arr))
    return list(arr)


def ecf_workspace_bytes(shape: Shape, max_tokens: int) -> int:
    n = lib().ecf_workspace_bytes(ctypes.byref(shape), int(max_tokens))
    if n == 0:
        raise EcfError(ECF_EINVAL, lib().ecf_last_error().decode())
    return n


def qstar_split(m: int, b_p: float, b_h: float) -> int:
    return _check(lib().qstar_split(int(m), float(b_p), float(b_h)))


def ecf_cache_create(n_layers, n_experts, n_slots, max_slots, slot_bytes, d_slots, h_pool_ptrs=None,
                     host_threads=0):
    """h_pool_ptrs: sequence of n_layers*n_experts host addresses (ints) or None."""
    out = c_void_p()
    pool = None
    if h_pool_ptrs is not None:
        pool = (c_void_p * len(h_pool_ptrs))(*[int(p) for p in h_pool_ptrs])
    _check(lib().ecf_cache_create(int(n_layers), int(n_experts), int(n_slots), int(max_slots), int(slot_bytes),
                                  c_void_p(int(d_slots)) if d_slots else None, pool, int(host_threads),
                                  ctypes.byref(out)))
    return out.value


def ecf_cache_destroy(cache):
    lib().ecf_cache_destroy(c_void_p(cache))


def expert_cache_lookup(cache, layer, experts):
    arr, n = _i32(experts)
    slots = (c_int32 * max(1, n))()
    _check(lib().expert_cache_lookup(c_void_p(cache), int(layer), arr, n, slots))
    return list(slots)[:n]


def expert_cache_evict(cache, layer, experts):
    arr, n = _i32(experts)
    slots = (c_int32 * max(1, n))()
    victims = (c_int32 * max(1, n))()
    _check(lib().expert_cache_evict(c_void_p(cache), int(layer), arr, n, slots, victims))
    return list(slots)[:n], list(victims)[:n]


def ecf_cache_available(cache) -> int:
    return _check(lib().ecf_cache_available(c_void_p(cache)))


def ecf_cache_slot_of(cache, layer, expert) -> int:
    return lib().ecf_cache_slot_of(c_void_p(cache), int(layer), int(expert))


def ecf_cache_get_stats(cache) -> dict:
    st = CacheStats()
    _check(lib().ecf_cache_get_stats(c_void_p(cache), ctypes.byref(st)))
    return st.as_dict()


def ecf_cache_resize(cache, n_slots):
    _check(lib().ecf_cache_resize(c_void_p(cache), int(n_slots)))


def prefetch_layer(cache, layer, blob_bytes, copy_stream=0, done_event=0):
    """Returns (experts copied, experts that did not fit)."""
    nc, nm = c_int32(), c_int32()
    _check(lib().prefetch_layer(c_void_p(cache), int(layer), int(blob_bytes),
                                c_void_p(int(copy_stream)) if copy_stream else None,
                                c_void_p(int(done_event)) if done_event else None, ctypes.byref(nc),
                                ctypes.byref(nm)))
    return nc.value, nm.value


def moe_layer_forward(args: LayerArgs, d_x, n_tokens, d_out, want_stats=True):
    st = StepStats()
    _check(lib().moe_layer_forward(ctypes.byref(args), c_void_p(int(d_x)) if d_x else None, int(n_tokens),
                                   c_void_p(int(d_out)) if d_out else None,
                                   ctypes.byref(st) if want_stats else None))
    return st.as_dict() if want_stats else None


def moe_layer_forward_noalloc(args: LayerArgs, d_x, n_tokens, d_out, want_stats=True):
    st = StepStats()
    _check(lib().moe_layer_forward_noalloc(ctypes.byref(args), c_void_p(int(d_x)) if d_x else None,
                                           int(n_tokens), c_void_p(int(d_out)) if d_out else None,
                                           ctypes.byref(st) if want_stats else None))
    return st.as_dict() if want_stats else None


def ecf_noalloc_scratch_bytes() -> int:
    return int(lib().ecf_noalloc_scratch_bytes())


def ecf_host_experts(shape: Shape, blob_ptrs, rows_per_job, x_ptr, n_tokens, y_ptr, n_threads=0):
    """blob_ptrs: host addresses, rows_per_job: list of lists of flat rows."""
    n = len(blob_ptrs)
    blobs = (c_void_p * max(1, n))(*[int(p) for p in blob_ptrs])
    counts, _ = _i32([len(r) for r in rows_per_job])
    flat, _ = _i32([f for r in rows_per_job for f in r])
    _check(lib().ecf_host_experts(ctypes.byref(shape), n, blobs, counts, flat, c_void_p(int(x_ptr)),
                                  int(n_tokens), c_void_p(int(y_ptr)), int(n_threads)))


def ecf_bandwidth_profile(shape: Shape, blob_ptrs, d_buf, d_buf_bytes, copy_stream=0, seconds=2.0,
                          host_threads=0) -> dict:
    arr = (c_void_p * max(1, len(blob_ptrs)))(*[int(p) for p in blob_ptrs])
    out = BwProfile()
    _check(lib().ecf_bandwidth_profile(ctypes.byref(shape), len(blob_ptrs), arr, int(host_threads),
                                       int(d_buf) or None, int(d_buf_bytes), int(copy_stream) or None,
                                       float(seconds), ctypes.byref(out)))
    return out.as_dict()


def ecf_profile_enable(on: bool):
    _check(lib().ecf_profile_enable(1 if on else 0))


def ecf_profile_get_all() -> dict:
    out, i = {}, 0
    while True:
        name, n, ms = c_char_p(), c_int64(), c_double()
        rc = lib().ecf_profile_get(i, ctypes.byref(name), ctypes.byref(n), ctypes.byref(ms))
        if rc == ECF_EINVAL:
            break
        _check(rc)
        out[name.value.decode()] = (n.value, ms.value)
        i += 1
    return out


def ecf_stream_read(d_buf, nbytes, d_sink, stream=0):
    return _check(lib().ecf_stream_read(int(d_buf) or None, int(nbytes), int(d_sink) or None, int(stream) or None))


def ecf_mfma_rate(iters, blocks_per_cu, d_sink, stream=0):
    """Enqueue the MFMA-rate measurement kernel; returns the flop it performs."""
    flop = c_double(0.0)
    _check(lib().ecf_mfma_rate(int(iters), int(blocks_per_cu), int(d_sink) or None, int(stream) or None,
                               ctypes.byref(flop)))
    return flop.value


def ecf_profile_reset():
    _check(lib().ecf_profile_reset())
