/*
 * eo.h — MoE expert-layer forward over a device-resident LRU expert cache,
 * backed by an expert pool in pinned host memory, on one AMD MI355X (gfx950).
 *
 * The method (FreeToken, "Efficient Edge-Native MoE Serving with
 * Bandwidth-Adaptive Execution"; zhichai.net article, section 2):
 *   route -> look up the expert cache -> plan the misses -> fill over PCIe or
 *   execute on the host cores -> grouped SwiGLU expert FFN -> weighted combine.
 * Decode (Decode paragraph): of the m cache misses of a layer call,
 * q* = m * B_P / B_H are filled over PCIe into the cache, the rest run on the
 * host cores from host memory; B_P and B_H are measured on the machine.
 * Cache (LRU paragraph): one global LRU over all layers' experts.
 * Prefill (Prefill paragraph): whole layers stream over PCIe with double
 * buffering; layer l+1's experts are copied while layer l computes.
 *
 * Conventions for every call:
 *   - Returns eo_status; never throws. On failure eo_last_error() holds a
 *     message (thread-local, valid until the next call on that thread).
 *   - "device" pointers are HIP device memory owned by the caller; "host"
 *     pointers are ordinary host memory owned by the caller unless stated.
 *   - `stream` is a hipStream_t passed as void* (NULL = the null stream).
 *     Step calls are asynchronous and ordered on that stream; results in
 *     caller buffers are valid once the stream has reached that point.
 *   - Asynchronous device errors surface at the next call or at eo_sync() as
 *     EO_ERR_HIP.
 *   - An engine is used from one host thread at a time. Calls that touch the
 *     device make the engine's device (cfg->device) current on the calling
 *     thread; a stream passed in must belong to that device.
 *   - Debugging: with EO_DEBUG_SYNC=1 in the environment at eo_create, the step
 *     calls wait for the device after every stage (route, lookup and plan,
 *     fill, expert FFN, host-execute, combine; per layer in eo_decode_step and
 *     eo_prefill) and report an asynchronous device error as EO_ERR_HIP naming
 *     the stage and layer. Results are the same as without it.
 *   - Tracing: every step call, each layer of eo_decode_step and eo_prefill,
 *     the host's wait for a plan and the host-core routine are named trace
 *     ranges (roctx: "eo.decode_step", "eo.decode.layer", "eo.wait_plan",
 *     "eo.host_routine", "eo.prefill", ...), which a profiler that records
 *     markers shows beside the kernels (rocprofv3 --marker-trace).
 * Tensor layouts are row-major. Activations are bf16 (act_bf16 = 1) or fp32.
 */
#ifndef EO_H
#define EO_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
    EO_OK = 0,
    EO_ERR_INVALID_ARG = -1,
    EO_ERR_OOM = -2,
    EO_ERR_HIP = -3,
    EO_ERR_STATE = -4,
    EO_ERR_UNSUPPORTED = -5
} eo_status;

/* Expert weight storage formats (juejin.cn overview, section 5: MXFP4, NVFP4,
 * FP8 and BF16; fp32 for small test models). Packed expert block, hidden H,
 * intermediate I; W13 = [W_gate; W_up] (2I rows of H), W2 = W_down (H rows of
 * I); quantisation blocks run along rows; two fp4 codes per byte, the even
 * element in the low nibble:
 *   FP32 : W13 f32 | W2 f32
 *   BF16 : W13 bf16 | W2 bf16
 *   MXFP4: W13 e2m1 | W2 e2m1 | W13 e8m0 per 32 | W2 e8m0 per 32
 *   NVFP4: W13 e2m1 | W2 e2m1 | W13 e4m3 per 16 | W2 e4m3 per 16 | f32 g_gate, g_up, g_down
 *   FP8  : W13 e4m3fn | W2 e4m3fn | f32 scale per W13 row | f32 scale per W2 row
 * Values: MXFP4 e2m1 * 2^(e8m0-127); NVFP4 (e2m1 * e4m3) * g; FP8 e4m3 * s_row. */
typedef enum { EO_W_FP32 = 0, EO_W_BF16 = 1, EO_W_MXFP4 = 2, EO_W_NVFP4 = 3, EO_W_FP8 = 4 } eo_wfmt;

typedef struct {
    int32_t layers;         /* MoE layers L */
    int32_t experts;        /* routed experts per layer E (<= 1024) */
    int32_t top_k;          /* experts per token k (<= 16, <= E) */
    int32_t hidden;         /* H, multiple of 128 */
    int32_t inter;          /* I, multiple of 64 */
    int32_t shared_experts; /* 0 or 1 always-on shared expert per layer (device-resident) */
    int32_t wfmt;           /* eo_wfmt */
    int32_t act_bf16;       /* 1: activations bf16 (needs wfmt != FP32); 0: fp32 (needs wfmt == FP32) */
    int64_t cache_slots;    /* C: device expert-cache capacity in experts (>= 0) */
    int32_t max_tokens;     /* largest T of any step call */
    int32_t host_threads;   /* host-core expert routine threads; 0 = hardware threads - 1, at most 15 */
    int32_t device;         /* HIP device ordinal */
} eo_config;

typedef struct eo_engine eo_engine;

/* Largest E for which plans are reported (eo_plan_host arrays). */
#define EO_MAX_EXPERTS 1024

/* Plan of the last lookup call (zhichai.net article, section 2, Decode
 * paragraph). Lists hold the experts of `layer`. */
typedef struct {
    int32_t layer;
    int32_t m;          /* misses */
    int32_t q;          /* misses the bandwidth split sends to PCIe */
    int32_t q_fill;     /* of those, filled (q clamped by free capacity C - hits) */
    int32_t n_hit, n_host, n_evict, pad_;
    int64_t clock;      /* lookup calls so far (the LRU clock) */
    int64_t credit;     /* split remainder after this call, 0 <= credit < B_H */
    int32_t hit_expert[EO_MAX_EXPERTS], hit_slot[EO_MAX_EXPERTS];   /* expert id ascending */
    int32_t fill_expert[EO_MAX_EXPERTS], fill_slot[EO_MAX_EXPERTS]; /* rank order */
    int32_t host_expert[EO_MAX_EXPERTS];                              /* rank order */
    int32_t evicted_key[EO_MAX_EXPERTS];                              /* key = layer*E + expert */
} eo_plan_host;

typedef struct {
    int64_t lookups, hits, misses, fills, host_experts;
    int64_t pcie_bytes;  /* bytes copied host->device by fills and prefill streaming */
    int64_t host_bytes;  /* expert bytes read by the host-core routine */
    int64_t prefill_layers;
    int64_t device_expert_bytes;  /* expert weight bytes the device FFN reads, once per expert
                                     and layer call: (hits + fills + shared) * expert size for
                                     lookups, the whole layer (+ shared) for prefill layers */
    int64_t host_wait_ns;     /* host time spent waiting for device plans */
    int64_t host_routine_ns;  /* host time spent in the host-core expert routine */
} eo_stats;

/* Create an engine on cfg->device: allocates the pinned host expert pool
 * (L*E blocks, each padded to 4 KiB), C device cache slots, the shared experts,
 * router copies, plan buffers, a copy stream and the host thread pool. Pool
 * contents are undefined until written; shared experts and routers start
 * zeroed, the cache empty, B_P = B_H = 1.
 * Errors: INVALID_ARG (shape limits above), UNSUPPORTED (format / activation
 * combination), OOM (pinned or device allocation failed), HIP. */
eo_status eo_create(const eo_config* cfg, eo_engine** out);

/* Frees everything the engine owns; waits for its outstanding work. */
eo_status eo_destroy(eo_engine* e);

/* Host address and size of one pool entry (pinned memory owned by the
 * engine, valid until eo_destroy). The caller writes the packed expert block
 * there before the first forward call that may need it. */
eo_status eo_pool_expert(eo_engine* e, int32_t layer, int32_t expert, void** host_ptr,
                         uint64_t* bytes);

/* Copy one layer's shared-expert block (host bytes, `bytes` must equal the
 * expert block size) to its device home. Synchronous. */
eo_status eo_set_shared_expert(eo_engine* e, int32_t layer, const void* host_block,
                               uint64_t bytes);

/* Copy router weights R_l, fp32 [E, H] host, to the device. Synchronous. */
eo_status eo_set_router(eo_engine* e, int32_t layer, const float* host_w);

/* Measure B_P (one expert host->device copy into a cache slot, made the way
 * fills are made: by the fill kernel, or by hipMemcpyAsync under EO_FILL_SDMA=1)
 * and B_H (the
 * host-core expert routine over one expert at T = 1, with the engine's thread
 * count), each the median of several timed runs over different experts,
 * floored to integer MB/s, and use them for the miss split (zhichai.net
 * article, section 2, Decode paragraph: measured on the machine with real
 * tensor shapes). Overwrites cache slot 0's bytes; resets the cache to empty
 * and the split credit to 0. Either output pointer may be NULL. */
eo_status eo_measure_bandwidth(eo_engine* e, uint32_t* bp_mbps, uint32_t* bh_mbps);

/* The same probes while serving (B_P and B_H change at run time on a shared
 * machine; the split is re-derived from the next lookup on): the copy goes to a
 * scratch buffer, the cache, clock and stamps are kept and the credit is
 * clamped below the new B_H, as eo_set_bandwidth does. Call between steps
 * (EO_ERR_STATE with a pending lookup plan). Either output pointer may be NULL. */
eo_status eo_remeasure_bandwidth(eo_engine* e, uint32_t* bp_mbps, uint32_t* bh_mbps);

/* Set B_P and B_H (MB/s, both > 0) directly; clips the credit below B_H. */
eo_status eo_set_bandwidth(eo_engine* e, uint32_t bp_mbps, uint32_t bh_mbps);

/* ---- step calls (stream-ordered; x, ids, w, y are device pointers) ---- */
/* T, the tokens of a call, is 1 .. max_tokens: an empty batch (T = 0) or a
 * larger one returns EO_ERR_INVALID_ARG before anything is launched, and the
 * cache, the LRU clock, the credit and the statistics stay as they were. */

/* Route, the first stage of a layer (explainer on papers.ananclaw.com, section
 * 4, engineering path: softmax top-k routing, the expert count and the shared
 * expert are the axes on which MoE architectures differ; zhichai.net article,
 * section 2, LRU paragraph: which experts a token routes to is what the cache
 * sees). Router: z = x . R_l^T in fp32 (64 strided fused multiply-add chains,
 * then an xor butterfly), top-k by (z desc, id asc), w = softmax over the k
 * selected.
 * forced_ids (device [T,k] or NULL): take these ids in this order (routing
 * trace replay) and return the softmax of z at them. ids: int32 [T,k];
 * w: fp32 [T,k]. */
eo_status eo_route(eo_engine* e, int32_t layer, const void* x, int32_t T,
                   const int32_t* forced_ids, int32_t* ids, float* w, void* stream);

/* eo_route without any device allocation, for callers that cannot allocate
 * device memory (code under HIP graph capture, tight serving loops, harnesses
 * that forbid hipMalloc). Same arguments, results and errors as eo_route; its
 * kernels keep their scratch (logits [T,E] fp32 and, for the chain-interleaved
 * kernel, x rearranged as [T,H] bf16) in a fixed 16 MiB device array per GPU,
 * held until the process ends, instead of the engine's buffers. The call
 * allocates nothing and launches kernels only. EO_ERR_INVALID_ARG when
 * T * 4 * E (+ T * 2 * H when H % 512 == 0, E % 32 == 0, T >= 32 and
 * activations are bf16) exceeds 16 MiB. Calls that overlap on one GPU (other
 * streams, other engines on the same device) share the array and race: order
 * them on one stream. */
eo_status eo_route_noalloc(eo_engine* e, int32_t layer, const void* x, int32_t T,
                           const int32_t* forced_ids, int32_t* ids, float* w, void* stream);

/* Look up the cache and plan the misses (zhichai.net article, section 2:
 * Decode paragraph, most routed experts hit the device LRU cache and the m
 * misses are split q* = m*B_P/B_H to PCIe, the rest to the host cores; LRU
 * paragraph, one global LRU over all layers). Cache lookup, LRU update and miss
 * plan for the distinct experts in ids [T,k] (one LRU clock tick). Runs on the device; the plan is kept by the
 * engine for eo_fill / eo_host_execute / eo_expert_ffn_combine and returned by
 * eo_last_plan. Split: q = min(m, floor((c + m*B_P)/B_H)),
 * c <- min(c + m*B_P - q*B_H, B_H - 1), q_fill = min(q, C - hits); misses
 * ranked by (tokens desc, id asc); victims by (stamp asc, key asc) among slots
 * not touched by this call; freed and empty slots go to fills in slot order;
 * host-executed misses are not inserted. */
eo_status eo_lookup_plan(eo_engine* e, int32_t layer, const int32_t* ids, int32_t T,
                         void* stream);

/* Queue the last plan's fills (pinned pool -> cache slot, zhichai.net article,
 * section 2, Decode paragraph) on `stream`: a kernel reads the fill list from
 * device memory and copies each expert block over PCIe from the pool's
 * device-visible mapping, so the call does not wait for the plan on the host.
 * (Environment EO_FILL_SDMA=1 at engine creation: hipMemcpyAsync per expert on
 * the engine's copy stream instead, after a host wait for the plan.)
 * EO_ERR_STATE without a pending plan. Fills are counted in eo_stats when the
 * host reads the plan. */
eo_status eo_fill(eo_engine* e, void* stream);

/* Host-execute (zhichai.net article, section 2, Decode paragraph: the misses
 * not filled run in place on the host cores, reading their weights from host
 * memory at B_H). Run the last plan's host-list experts on the host cores for
 * the tokens routed to them (x device [T,H], ids [T,k], w [T,k] as passed to
 * the lookup; copied to the host after a wait on `stream` unless the engine
 * already mirrored them) and stage their weighted sum for the next
 * eo_expert_ffn_combine. Waits on the host for the plan and blocks while the
 * host routine runs. EO_ERR_STATE without a pending plan. */
eo_status eo_host_execute(eo_engine* e, const void* x, const int32_t* ids, const float* w,
                          void* stream);

/* Grouped expert FFN and combine (zhichai.net article, section 2, Decode
 * paragraph: hits and filled experts are served from device memory; Prefill
 * paragraph: expert compute of a layer on the device). Device part of the
 * layer for the last plan: permute tokens by expert,
 * grouped SwiGLU FFN on the resident experts (decode: dequant-GEMV), the
 * shared expert, and the weighted combine plus any staged host results:
 * y fp32 [T,H] = sum_j w[t,j] * FFN_{e_j}(x_t) + FFN_shared(x_t).
 * No residual. Consumes the plan. x [T,H] and y device, 16-byte aligned; ids
 * and w as passed to the lookup. EO_ERR_STATE without a pending plan or when
 * `layer` is not the plan's. For T > 1 the environment switch EO_GEMM_PATH,
 * read at each call, selects the grouped GEMM kernel that the tests compare:
 * 3 (the default; bf16 weights load in 128-byte rows), 2 (one three-stage
 * ring), 1 (register-staged tiles) or 0 (plain 128 x 128 tiles); all are held
 * to the same bar against the oracle, and paths 3 and 2 give the same bits. */
eo_status eo_expert_ffn_combine(eo_engine* e, int32_t layer, const void* x, const int32_t* ids,
                                const float* w, float* y, void* stream);

/* One MoE layer in the method's order, route -> look up -> plan -> fill or
 * host-execute -> grouped FFN -> combine (zhichai.net article, section 2,
 * Decode paragraph): all of the above for one layer, y fp32 [T,H] (no
 * residual). x device [T,H] in the activation dtype, 16-byte aligned;
 * forced_ids device [T,k] or NULL as for eo_route. */
eo_status eo_moe_layer(eo_engine* e, int32_t layer, const void* x, float* y, int32_t T,
                       const int32_t* forced_ids, void* stream);

/* Decode (zhichai.net article, section 2, Decode paragraph: per token, each
 * layer's routed experts are served from the LRU cache, and its misses are
 * filled or run on the host by the q* split; LRU paragraph: consecutive tokens
 * reuse experts, which is what the cache keeps). One decode step through all
 * layers, in place. x_inout [T,H] (activation
 * dtype) is the residual stream r: layer l takes u_l = r_l / sqrt(mean(r_l^2)
 * + 1e-6) per token (stored in the activation dtype; a parameter-free RMS
 * normalisation, as in pre-norm transformer blocks) and r_{l+1} = r_l + y_l(u_l)
 * (stored in the activation dtype). forced_ids: device [L, T, k] or NULL.
 * One token with bf16 activations runs three kernels per layer and no host wait
 * between layers other than the plan readback for the host-list experts:
 * layer entry + plan (one launch); the fills and the expert GEMV (one launch:
 * 64 workgroups copy the fills, the gate/up bytes of each filled expert first,
 * while the others run the gate/up rows, a filled expert's once its bytes are
 * in, and, on a layer with fills, the down rows of the experts resident before
 * it once their gate/up rows are done); the down GEMV (the filled experts' rows
 * after a layer with fills, else all). Should one of these bounded waits run
 * out (1 s; EO_TEST_FILL_WAIT_TICKS=n at engine creation sets it to n ticks of
 * the device's 100 MHz clock, for tests of this path), the next one-token plan
 * returns EO_ERR_HIP and changes nothing.
 * The results
 * do not depend on which kernels run; the environment switches EO_ENTRY_PLAN=0
 * (entry and plan as two launches), EO_PLAN1=0 (the general plan kernel for
 * one token), EO_FUSED_ENTRY=0 (separate norm, router and top-k kernels, read
 * at engine creation), EO_GEMV_FAST=0 (the generic GEMV, read at engine
 * creation) and EO_FILL_GEMV=0 (fill kernel and gate/up GEMV as two launches,
 * read at engine creation; also the case while timing is enabled, so that the
 * kernel times stay those of each kernel alone) select the alternatives that the
 * tests compare. */
eo_status eo_decode_step(eo_engine* e, void* x_inout, int32_t T, const int32_t* forced_ids,
                         void* stream);

/* Prefill of T tokens (T <= max_tokens) through all layers, in place (the
 * same residual stream and normalisation as eo_decode_step), with full-layer
 * double-buffered streaming of each layer's E experts from the pool (zhichai.net
 * article, section 2, Prefill paragraph); the cache is not updated. flags:
 * EO_PREFILL_DOUBLE_BUFFER overlaps layer l+1's copy with layer l's compute
 * (0: serialised, the ablation); EO_PREFILL_SKIP_RESIDENT streams only the
 * experts that are not resident in the cache and reads the resident ones from
 * their slots (waits for `stream` once to read the residency). Other bits:
 * EO_ERR_INVALID_ARG. */
#define EO_PREFILL_DOUBLE_BUFFER 1
#define EO_PREFILL_SKIP_RESIDENT 2
eo_status eo_prefill(eo_engine* e, void* x_inout, int32_t T, int32_t flags, void* stream);

/* Optional per-layer capture for tests, device buffers written by
 * eo_decode_step / eo_prefill (NULL disables): x_in [L, T, H] layer inputs u_l
 * (activation dtype), y [L, T, H] fp32 MoE outputs, ids [L, T, k], w [L, T, k].
 * Capacity is given in tokens per layer. */
eo_status eo_set_capture(eo_engine* e, void* x_in, float* y, int32_t* ids, float* w,
                         int32_t tokens_per_layer);

/* Elastic cache resize (zhichai.net article, section 2, the elastic VRAM
 * paragraph: the expert cache is a run-time quantity, rebuilt at scheduler safe
 * points without restarting the engine or reloading weights from the pool).
 * Call between steps (no pending lookup plan: EO_ERR_STATE otherwise); waits for
 * the device. New capacity `slots` in [0, 8192]. If more experts are resident
 * than `slots`, the least recently used are evicted in (stamp asc, key asc)
 * order; survivors in slots below the new capacity stay, the others move, in
 * ascending old slot order, to the lowest empty slots (device-to-device
 * copies). Stamps, clock and credit are kept. The slot memory is reallocated at
 * the new size (the old block is freed after the copies; both exist during the
 * call); on EO_ERR_OOM the engine is unchanged. n_evicted / n_moved may be NULL. */
eo_status eo_resize_cache(eo_engine* e, int64_t slots, int64_t* n_evicted, int64_t* n_moved);

/* Static placement, for the placement-policy comparison (zhichai.net article,
 * section 2, LRU paragraph: one routing trace replayed under the global LRU,
 * under a placement fixed from prefill routing and under a routing-blind static
 * split). Between steps: the n keys (host array, key = layer*E + expert,
 * distinct, n <= cache slots) are copied from the pool into slots 0..n-1 (stamp
 * 0; other slots empty) and the cache is frozen: lookups still count and stamp
 * hits and run the credit split, but fill and evict nothing, so every miss runs
 * on the host. Synchronous. eo_clear_static_placement returns to the LRU from
 * the current residency. EO_ERR_STATE with a pending lookup plan. */
eo_status eo_set_static_placement(eo_engine* e, const int32_t* keys, int32_t n);
eo_status eo_clear_static_placement(eo_engine* e);

/* ---- introspection ---- */
/* Slot table and counters (host buffers of C entries each). Synchronous. */
eo_status eo_cache_snapshot(eo_engine* e, int32_t* slot_key, int64_t* slot_stamp, int64_t* clock,
                            int64_t* credit);
/* The last lookup's plan. Synchronous. */
eo_status eo_last_plan(eo_engine* e, eo_plan_host* out);
/* Dequantise one pool expert with the device decoder: out_host fp32
 * [W_gate (I*H) | W_up (I*H) | W_down (H*I)]. Synchronous. */
eo_status eo_dequant(eo_engine* e, int32_t layer, int32_t expert, float* out_host);
/* The same expert decoded through the weight decoders of one family of expert
 * kernels, element by element, each value multiplied by the factors that family
 * applies outside its decode (row scale, NVFP4 global scale) in the same order:
 * EO_DECODER_GEMM the grouped GEMM's tile decode (scaled converts),
 * EO_DECODER_GEMV the decode GEMV's, EO_DECODER_SCALAR the scalar decoders of
 * eo_dequant. Formats as eo_wfmt (juejin.cn overview, section 5); values as
 * defined there. Synchronous; out_host as for eo_dequant; INVALID_ARG for an
 * unknown decoder. */
#define EO_DECODER_SCALAR 0
#define EO_DECODER_GEMM 1
#define EO_DECODER_GEMV 2
eo_status eo_dequant_with(eo_engine* e, int32_t layer, int32_t expert, int32_t decoder,
                          float* out_host);
/* Counters since eo_create (host memory). With EO_LOG=1 in the environment at
 * eo_create the engine prints its configuration and allocations to stderr;
 * EO_LOG=2 also prints one line per lookup plan. */
eo_status eo_stats_get(eo_engine* e, eo_stats* out);
/* Device time of the expert FFN and fill kernels since the last reset, from HIP
 * start/stop events attached to each kernel launch on the compute stream while
 * timing is enabled (hipExtLaunchKernel: the events take the kernel's own start
 * and end; they are created without a system-scope fence so that they do not
 * slow the kernels they time): ms[0] decode GEMV gate/up kernel, ms[1] decode
 * GEMV down kernel, ms[2] grouped GEMM gate/up (+SwiGLU) kernel, ms[3] grouped
 * GEMM down kernel, ms[4] fill kernel (totals); launches[0] decode GEMV pairs,
 * launches[1] grouped GEMM pairs, launches[2] fill kernels. Either pointer may
 * be NULL; reset != 0 clears after reading. Synchronises on the events. */
eo_status eo_kernel_times(eo_engine* e, double* ms /*[5]*/, int64_t* launches /*[3]*/,
                          int32_t reset);
/* Prefill streaming, copy against compute (zhichai.net article, section 2,
 * Prefill paragraph: the next layer's weights cross PCIe while the current
 * layer computes). While timing is enabled, eo_prefill stamps each layer's
 * copies on the copy stream (from when the copy stream reaches them, after any
 * wait for the staging buffer to be free) and each layer's kernels on the
 * compute stream (from when the layer's weights are in): ms[0] the summed copy
 * time, ms[1] the summed compute time; layers[0] / layers[1] the layers stamped
 * on each. With double buffering the chunk takes about max(ms[0], ms[1]),
 * without it about their sum. Either pointer may be NULL; reset != 0 clears
 * after reading. Synchronises on the events. */
eo_status eo_stream_times(eo_engine* e, double* ms /*[2]*/, int64_t* layers /*[2]*/,
                          int32_t reset);
/* Plan sizes of each lookup, recorded on the host when it reads the plan
 * (zhichai.net article, section 2, Decode paragraph: per layer call, hits are
 * served from the device, q* misses filled over PCIe, the rest run on the host;
 * the three lanes bound the call). eo_set_plan_log(e, 1) clears the log and
 * starts recording, 0 stops. eo_get_plan_log copies the first min(n, cap)
 * entries, each int32 {layer, hits, fills, host experts} in call order, to out
 * (host [cap][4]; NULL with cap 0 only counts) and stores the number recorded
 * in *n (may be NULL). */
eo_status eo_set_plan_log(eo_engine* e, int32_t enable);
eo_status eo_get_plan_log(eo_engine* e, int32_t* out, int64_t cap, int64_t* n);
/* Enable (1) or disable (0) the per-launch timing events behind eo_kernel_times
 * and eo_stream_times. While enabled, a decode step launches the fill kernel
 * and the gate/up GEMV apart, so that each is timed alone. */
eo_status eo_set_timing(eo_engine* e, int32_t enable);
/* Size in bytes of one packed expert block (unpadded). */
uint64_t eo_expert_bytes(int32_t hidden, int32_t inter, int32_t wfmt);
/* Wait for the engine's streams and the device; report async HIP errors. */
eo_status eo_sync(eo_engine* e);
const char* eo_last_error(void);

#ifdef __cplusplus
}
#endif
#endif /* EO_H */
