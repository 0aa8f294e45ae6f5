/*
 * ecf.h -- C ABI of libecf, one expert-cached Mixture-of-Experts layer on an
 * AMD Instinct MI355X (gfx950).
 *
 * The layer: router softmax/top-k, token->expert permutation, SwiGLU expert
 * FFNs (fp32, bf16 or MXFP4 weights) and the gate-weighted combine.  Experts
 * either all sit in device memory, or live in a pinned host pool (the source
 * of truth) with a fixed pool of device slots in front of it, one LRU shared
 * by all layers.  On a miss, the bandwidth-adaptive q* split copies about
 * m * B_P / B_H of the m missed experts into slots and computes the rest on
 * host cores; the two partial sums are added.
 *
 * Sources (page title, section), quoted nowhere, restated here:
 *  [TF]  techfeed summary of "Meet FreeToken: An Edge-Native MoE Serving
 *        Engine ..." (MarkTechPost), section "FreeToken's three core
 *        mechanisms": "Bandwidth-adaptive execution (q* policy)" and
 *        "Semantic-aware caching".
 *  [PL]  FreeToken paper explainer (ta-paperlens), sections "Design: two-tier
 *        expert memory" and "Prefill: full-layer double buffer and semantic
 *        anchors".
 *  [LE]  leadeas blog on FreeToken, section "Using VRAM as a cache --
 *        bandwidth-adaptive CPU-GPU co-execution".
 *
 * Conventions for every call:
 *  - Pointers prefixed d_ are device memory, h_ are host memory.  Every
 *    buffer is owned by the caller; the library keeps no pointer beyond a
 *    call except the slot base inside an ecf_cache and the host pool table
 *    the caller hands to ecf_cache_create.
 *  - Streams and events are hipStream_t / hipEvent_t passed as void*.
 *    NULL means the default stream.
 *  - Return value: ECF_OK (0) or a negative ECF_* code; the thread-local
 *    ecf_last_error() explains the last failure.  No C++ exception crosses
 *    the ABI.  Kernel faults are asynchronous and surface at the next
 *    synchronising call as ECF_EHIP.
 *  - The library never allocates device memory on a forward call; it uses
 *    the caller's workspace.  A cache owns a small pinned host staging area
 *    and a host thread pool, both allocated once at ecf_cache_create.
 */
#ifndef ECF_H
#define ECF_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* ---- status codes ----------------------------------------------------------- */
#define ECF_OK 0
#define ECF_EINVAL (-1)       /* bad argument (shape, NULL, out of range) */
#define ECF_ENOSPC (-2)       /* not enough cache slots / buffer too small */
#define ECF_EHIP (-3)         /* a HIP runtime call failed */
#define ECF_EUNSUPPORTED (-4) /* valid but not implemented combination */
#define ECF_ESTATE (-5)       /* call out of order (e.g. evict without lookup) */

/* Message for the last failure on the calling thread ("" if none). */
const char *ecf_last_error(void);

/* ---- shapes and expert blobs ------------------------------------------------- */
typedef enum { ECF_F32 = 0, ECF_BF16 = 1, ECF_MXFP4 = 2 } ecf_dtype;

typedef struct {
    int32_t hidden;      /* d: model width; multiple of 256 */
    int32_t inter;       /* I: expert intermediate width; multiple of 64 (of 128 for
                            the prefill path) */
    int32_t n_experts;   /* E: routed experts per layer, 1..1024 */
    int32_t top_k;       /* k: experts per token, 1..min(E, 32) */
    int32_t w_dtype;     /* expert weight encoding, ecf_dtype */
    int32_t a_dtype;     /* activation and router-weight encoding: ECF_F32 or ECF_BF16
                            (must be ECF_BF16 for ECF_BF16 / ECF_MXFP4 weights) */
    int32_t renorm_topk; /* 1: gates = softmax over the k selected logits;
                            0: gates = full softmax over E, read at the selected */
} ecf_shape;

/*
 * One expert slot blob holds every tensor needed to evaluate one (layer,
 * expert) pair [PL "Design: two-tier expert memory"], each section starting
 * at a 256-byte boundary:
 *   W_gate [I][d], W_up [I][d], W_down [d][I]   (row-major, reduction dim contiguous)
 * and, for ECF_MXFP4, the E8M0 scales S_gate [I][d/32], S_up [I][d/32],
 * S_down [d][I/32].  MXFP4 element 2i is the low nibble of byte i (OCP MX v1.0
 * E2M1); 32 consecutive elements along the reduction dim share one scale.
 * ecf_expert_layout writes the byte offsets of the six sections (the last
 * three are 0 for non-MXFP4).
 */
size_t ecf_expert_bytes(const ecf_shape *shape);
int ecf_expert_layout(const ecf_shape *shape, size_t offsets_out[6]);

/* Device workspace bytes a forward call needs for up to max_tokens tokens
 * (0 for an invalid shape or max_tokens * top_k above 2^26). */
size_t ecf_workspace_bytes(const ecf_shape *shape, int32_t max_tokens);

/* ---- q* split [TF "Bandwidth-adaptive execution (q* policy)"] ----------------
 * PCIe copies and CPU expert execution read the same host memory: with PCIe
 * drawing b_p of the host bandwidth b_h, the CPU has b_h - b_p left.  Of m
 * missed experts, copying q takes q/b_p and computing m-q on the CPU takes
 * (m-q)/(b_h-b_p) (per expert size); the real balance is q = m*b_p/b_h.
 * Returns the integer q in [0, m] with the smaller of the two makespans at
 * floor/ceil of m*b_p/b_h (equal makespans, within relative 1e-12, take the
 * larger q).  b_p <= 0 -> 0; b_p >= b_h -> m.  Returns ECF_EINVAL (< 0) for
 * m < 0, b_h <= 0 or NaN arguments.  Pure function, thread-safe.
 */
int32_t qstar_split(int32_t m, double b_p, double b_h);

/* ---- the shared expert cache [TF "Semantic-aware caching"; PL "Design: two-tier
 *      expert memory"] -------------------------------------------------------------
 * Host-side metadata of one LRU over (layer, expert) pairs, shared by all
 * layers, in front of n_slots device slots of slot_bytes each, at
 * d_slots + slot * slot_bytes (caller-owned, room for max_slots slots).
 * h_pool[layer * n_experts + expert] is the pinned host blob of that pair
 * (the source of truth; entries may alias), or h_pool may be NULL if the
 * caller never asks the library to copy or host-compute experts.
 * host_threads sizes the pool of CPU threads that evaluate host-assigned
 * experts (0 = min(16, hardware threads)).  A cache is not thread-safe: one
 * caller thread per cache.
 */
typedef struct ecf_cache ecf_cache;

typedef struct {
    int64_t lookups, hits, misses, inserts, evictions, dropped;
} ecf_cache_stats;

int ecf_cache_create(int32_t n_layers, int32_t n_experts, int32_t n_slots, int32_t max_slots,
                     size_t slot_bytes, void *d_slots, const void *const *h_pool,
                     int32_t host_threads, ecf_cache **out);
void ecf_cache_destroy(ecf_cache *cache);

/*
 * Start a layer-step of `layer` and look up experts[0..n) (distinct, in the
 * order the caller wants them touched; the forward call uses ascending id).
 * slots[i] = the resident slot, or -1 on a miss.  Hits become most recently
 * used, in the given order, and are pinned for the rest of this layer-step.
 */
int expert_cache_lookup(ecf_cache *cache, int32_t layer, const int32_t *experts, int32_t n,
                        int32_t *slots);

/*
 * Bind experts[0..n) (missed, distinct) of the current layer-step's layer to
 * slots: the lowest free slot, else the least recently used entry not pinned
 * by this layer-step (which is evicted).  slots[i] receives the slot;
 * victims (nullable) receives the evicted pair as layer * n_experts + expert,
 * or -1 when a free slot was used.  New entries become most recently used and
 * are pinned.  The caller must then copy the experts' blobs into their slots
 * before any kernel reads them.  ECF_ENOSPC, with no change made, if fewer
 * than n slots can be had; ECF_ESTATE if no layer-step is open or `layer`
 * differs from it; ECF_EINVAL if an expert is already resident.
 */
int expert_cache_evict(ecf_cache *cache, int32_t layer, const int32_t *experts, int32_t n,
                       int32_t *slots, int32_t *victims);

/* Slots a bind could take now: free ones, plus resident entries neither pinned
 * by the open layer-step nor held by a pending prefetch. */
int32_t ecf_cache_available(const ecf_cache *cache);
/* Resident slot of (layer, expert) or -1; does not touch the LRU order. */
int32_t ecf_cache_slot_of(const ecf_cache *cache, int32_t layer, int32_t expert);
int ecf_cache_get_stats(const ecf_cache *cache, ecf_cache_stats *out);

/*
 * Elastic resize at a safe point (between forward calls) [PL "Design: two-tier
 * expert memory": the host pool stays the source of truth, so the cache may
 * shrink or grow at any time without changing results].  Entries in slots
 * >= n_slots are dropped; growing adds free slots, up to max_slots.
 */
int ecf_cache_resize(ecf_cache *cache, int32_t n_slots);

/* ---- prefill layer prefetch [PL "Prefill: full-layer double buffer and semantic
 *      anchors": layer l+1 streams into the same slot pool while layer l computes,
 *      and what is left of it afterwards warms the decode cache] -------------------
 * Queue the copy of every expert of `layer` into the cache's slots, on
 * copy_stream, before that layer's routing is known.  In ascending expert id,
 * an entry already resident becomes most recently used, and a missing one is
 * bound like a miss (lowest free slot, else the least recently used entry
 * neither pinned nor held) and becomes most recently used; its host blob
 * (blob_bytes <= the slot size, from the cache's host pool) is copied into the
 * slot.  Runs of consecutive slots fed by consecutive host blobs (slot size ==
 * blob_bytes) go as one copy, so a layer stored contiguously on the host
 * streams as a few large copies.  Copies into a slot taken from another entry
 * wait first for the kernels of the last cache-mode forward call (call this
 * before the forward call of the layer now computing, then the two overlap).
 * The layer's entries are then held: no bind evicts them until the forward
 * call of `layer`, which waits on device for these copies and ends the hold.
 * If the layer does not fit, the experts that do are placed (ascending id)
 * and the rest, *n_missing of them, are reserved: a later prefetch places at
 * most the available slots less every pending reserve, so the forward calls of
 * the held layers, taken in prefetch order, can still fill their missing
 * experts on demand.  *n_copied receives the
 * experts copied (both outputs nullable).  done_event (nullable) is recorded
 * on copy_stream after the copies.  A second prefetch of a pending layer adds
 * nothing.  Asynchronous; returns once queued.  ECF_EINVAL for bad arguments
 * or a cache without a host pool; ECF_EHIP on a HIP failure (the cache's
 * contents are then undefined).
 */
int prefetch_layer(ecf_cache *cache, int32_t layer, size_t blob_bytes, void *copy_stream,
                   void *done_event, int32_t *n_copied, int32_t *n_missing);

/* ---- one layer forward --------------------------------------------------------- */
enum { ECF_Q_AUTO = 0, ECF_Q_ALL_GPU = 1, ECF_Q_ALL_HOST = 2, ECF_Q_FIXED = 3 };
enum { ECF_PATH_AUTO = 0, ECF_PATH_DECODE = 1, ECF_PATH_PREFILL = 2 };

typedef struct {
    int32_t n_unique;  /* experts routed to by at least one token */
    int32_t hits;      /* of those, resident in a slot */
    int32_t misses;    /* m */
    int32_t q;         /* misses copied into slots */
    int32_t host;      /* misses computed on the host (m - q) */
    int32_t path;      /* ECF_PATH_DECODE or ECF_PATH_PREFILL */
    int64_t bytes_h2d;  /* expert bytes copied host->device */
    int64_t bytes_host; /* expert bytes read by host threads */
    double ms_wait_route; /* host time blocked on the routing readback */
    double ms_host_ffn;   /* host time spent in host experts */
} ecf_step_stats;

typedef struct {
    ecf_shape shape;
    int32_t layer;               /* layer id (cache key) */
    /* routing input: exactly one of the two */
    const void *d_router_w;      /* [E][d] in a_dtype: logits = x . W_r^T in fp64, rounded to fp32 */
    const float *d_router_logits;/* [T][E] fp32, given directly */
    /* expert placement: exactly one of the two */
    const uint64_t *d_expert_ptrs; /* [E] device addresses of resident blobs (all experts resident) */
    ecf_cache *cache;              /* expert cache (blobs from the cache's host pool) */
    /* q* policy (cache mode) */
    double b_p, b_h;             /* bandwidth figures for qstar_split (any unit, same for both) */
    int32_t q_mode;              /* ECF_Q_*: AUTO uses qstar_split; the others are for tests */
    int32_t q_fixed;             /* q for ECF_Q_FIXED (clamped to [0, m]) */
    int32_t path;                /* ECF_PATH_*: AUTO takes the decode GEMVs in cache mode, for
                                    fp32 weights and, for bf16 / MXFP4, while T <= 64 or
                                    I % 128 != 0; the prefill grouped GEMM otherwise (bf16 /
                                    MXFP4; it needs I % 128 == 0 and x and one expert blob
                                    each under 4 GiB, else ECF_EUNSUPPORTED).  In cache mode
                                    PREFILL copies every miss into a slot and computes none
                                    on the host (the GEMM rounds h to bf16, the host experts
                                    do not, so a split would change the output); q_mode is
                                    then ignored and too few slots for the misses is
                                    ECF_ENOSPC */
    /* buffers */
    void *d_ws;                  /* workspace, >= ecf_workspace_bytes(shape, T) bytes, 256-B aligned */
    size_t ws_bytes;
    void *stream;                /* compute stream */
    void *copy_stream;           /* cache mode: stream for slot fills (NULL = stream) */
    const float *d_residual;     /* optional [T][d] fp32 added to the output (may equal d_out) */
    void *d_out_act;             /* optional [T][d] copy of the output in a_dtype (next layer input) */
    /* optional debug outputs (device, nullable) */
    int32_t *d_topk_idx;         /* [T][k] selected experts, logit descending, ties -> lower id */
    float *d_topk_gate;          /* [T][k] gates */
    int32_t *d_counts;           /* [E] rows per expert */
    int32_t *d_perm;             /* [T*k] row r of the expert-sorted order -> flat (t*k + j) */
    float *d_logits;             /* [T][E] router logits (router-weight mode only) */
} ecf_layer_args;

/*
 * out[t][:] = residual[t][:] + sum_{j=0..k-1} gate[t][j] * FFN_{idx[t][j]}(x[t])
 * with FFN_e(v) = W_down[e] . (silu(W_gate[e] . v) * (W_up[e] . v)), x [T][d]
 * in a_dtype (16-byte aligned, else ECF_EINVAL), out [T][d] fp32.  All-resident mode is fully asynchronous on
 * args->stream.  Cache mode blocks the calling thread once on the routing
 * readback (the q* decision is taken on the host from the step's miss count
 * [TF "Bandwidth-adaptive execution (q* policy)"]), queues the kernels of the
 * hits, then those of the copied misses behind their copies, computes
 * host-assigned experts on the cache's host threads, and returns with the rest
 * queued.  A cache-mode call opens and closes its own layer-step (its pins end
 * when it returns), ends the hold of a pending prefetch of its layer, and must
 * use one compute stream for all calls on a cache.
 * n_tokens == 0 is a no-op; n_tokens * top_k above 2^26 is ECF_EINVAL (row
 * indices are 32-bit).  stats (nullable) receives the step's figures.
 */
int moe_layer_forward(const ecf_layer_args *args, const void *d_x, int32_t n_tokens, float *d_out,
                      ecf_step_stats *stats);

/*
 * Allocation-free variant of moe_layer_forward, for callers that cannot
 * allocate device memory or call anything that does: code under HIP graph
 * capture, tight serving loops, harnesses that forbid allocation.
 * Same arguments and results as moe_layer_forward in all-resident mode, except
 * that args->d_ws and args->ws_bytes are ignored: the workspace is a device
 * array inside the library, ecf_noalloc_scratch_bytes() bytes (32 MiB) per GPU,
 * held until the process ends.  The call allocates nothing and records no
 * profiling events.  ECF_ENOSPC if ecf_workspace_bytes(shape, n_tokens)
 * exceeds that size (about 230 tokens of a d 4096 / E 256 / I 1024 / top-6
 * layer); ECF_EUNSUPPORTED in cache mode (args->cache non-NULL).  Every call on
 * one GPU shares that GPU's array (the current device's at the call), and the
 * array keeps the last call's contents: calls that overlap on one GPU (other
 * streams or threads) race and must be serialised by the caller.
 */
int moe_layer_forward_noalloc(const ecf_layer_args *args, const void *d_x, int32_t n_tokens,
                              float *d_out, ecf_step_stats *stats);
/* Bytes of the per-GPU array moe_layer_forward_noalloc uses as its workspace. */
size_t ecf_noalloc_scratch_bytes(void);

/*
 * The host half of the split on its own: y[f][:] = FFN_e(x[f / k]) for the rows
 * f listed per expert, evaluated by n_threads host threads (0 = default) the
 * same way a forward call evaluates host-assigned experts [TF "Bandwidth-
 * adaptive execution (q* policy)": missed experts not copied run on the CPU
 * straight from host memory].  h_blobs[i] is the host blob of job i (fp32, bf16
 * or MXFP4 weights), rows of job i are rows[sum(n_rows[<i]) .. + n_rows[i]];
 * h_x [T][d] in a_dtype, h_y [T*k][d] fp32 (only listed rows written).  No
 * GPU is touched.  ECF_EINVAL for negative counts, a row outside [0, T*k),
 * NULL arrays with n_jobs > 0, or n_tokens * top_k above 2^26.
 */
int ecf_host_experts(const ecf_shape *shape, int32_t n_jobs, const void *const *h_blobs,
                     const int32_t *n_rows, const int32_t *rows, const void *h_x, int32_t n_tokens,
                     float *h_y, int32_t n_threads);

/* ---- bandwidth profiler for the split [TF "FreeToken's three core mechanisms" /
 *      "Bandwidth-adaptive execution (q* policy)": the split ratio is measured on
 *      the machine the engine runs on] -----------------------------------------------
 * Measures, for about `seconds` in total:
 *   b_p         pinned host -> device copies of whole expert blobs on copy_stream
 *               (NULL = the null stream), alone;
 *   b_cpu       expert weight bytes per second the host expert threads consume
 *               (the forward pass's own host FFN, one routed row per expert), alone;
 *   b_read      a plain streaming read of the blobs by the same threads;
 *   b_p_conc, b_cpu_conc   the copy and host-expert rates while both run;
 *   b_h         b_p_conc + b_cpu_conc: the host bandwidth the two share.
 * All in GB/s (1e9 B/s).  Pass (b_p_conc, b_h) as (b_p, b_h) to qstar_split or
 * ecf_layer_args.  h_blobs: n_blobs pinned host expert blobs of `shape` (fp32 or
 * bf16 or MXFP4 weights), read only.  d_buf: device scratch of
 * d_buf_bytes >= one blob (ECF_ENOSPC otherwise), overwritten.  host_threads 0 =
 * min(16, hardware threads).  Allocates its thread pool; blocks until done.
 * ECF_EINVAL for NULL pointers, n_blobs < 1 or seconds <= 0; ECF_EHIP on a HIP
 * failure.
 */
typedef struct {
    double b_p, b_cpu, b_read, b_p_conc, b_cpu_conc, b_h;
    int32_t host_threads;
} ecf_bw_profile;

int ecf_bandwidth_profile(const ecf_shape *shape, int32_t n_blobs, const void *const *h_blobs,
                          int32_t host_threads, void *d_buf, size_t d_buf_bytes, void *copy_stream,
                          double seconds, ecf_bw_profile *out);

/* ---- measurement hooks ------------------------------------------------------------- */
/* When enabled, every kernel launch is bracketed by HIP events on its stream
 * and its duration is accumulated per kernel name (adds event overhead). */
int ecf_profile_enable(int32_t on);
/* Kernel name i (0-based) with its launch count and summed milliseconds;
 * ECF_EINVAL when i is past the last name.  Synchronises the device. */
int ecf_profile_get(int32_t i, const char **name, int64_t *launches, double *total_ms);
int ecf_profile_reset(void);

/*
 * One plain streaming read of bytes (a multiple of 16) at d_buf (16-byte
 * aligned): two blocks per CU, each reading one contiguous chunk front to back,
 * 16 bytes per lane and load, as a yardstick for the HBM bandwidth the
 * layer's kernels reach; *d_sink ^= the XOR of every 32-bit word read (the
 * caller zeroes it first if it wants the value).  Asynchronous on stream (NULL =
 * null stream); the caller times it.  ECF_EINVAL for bad pointers or sizes.
 */
int ecf_stream_read(const void *d_buf, size_t bytes, uint32_t *d_sink, void *stream);

/* Measurement: enqueue on `stream` a kernel that runs only bf16 MFMAs
 * (v_mfma_f32_32x32x16_bf16, 32x32x16 per instruction) from registers on
 * every compute unit: blocks_per_cu blocks of 4 waves each, `iters` rounds of
 * eight independent MFMAs per wave, on pseudo-random operands that change
 * from one MFMA to the next.  *flop receives the flop it performs (host
 * value, known at enqueue); timing it with events around the launch gives
 * the MFMA rate the GPU sustains under that load, the yardstick for the
 * grouped GEMMs' MFMA fraction (MI355X datasheet: 2.5 PFLOP/s dense bf16).
 * d_sink: one device float, written only in a case that cannot occur.
 * ECF_EINVAL if iters <= 0, blocks_per_cu is outside 1..8, or a pointer is
 * NULL. */
int ecf_mfma_rate(int32_t iters, int32_t blocks_per_cu, float *d_sink, void *stream, double *flop);

#ifdef __cplusplus
}
#endif
#endif /* ECF_H */
