// Internal declarations shared by the engine and its kernels (not installed).
#pragma once

#include <hip/hip_runtime.h>

#include <atomic>
#include <cstdint>
#include <string>
#include <vector>

#include "../../include/eo.h"
#include "eo_host.h"

namespace eo {

// ---------------------------------------------------------------- plan
// Device-side plan of one lookup call. The lists hold experts of `layer`.
struct DevPlan {
    int32_t seq;  // written last; the host polls the mirror's copy
    int32_t layer, T, k;
    int32_t m, q, q_fill, n_hit, n_host, n_evict, n_res, pad;
    int64_t clock, credit;
    int32_t e2slot[kMaxE];  // slot of each routed resident expert (hit or fill), else -1
    int32_t count[kMaxE];   // tokens routed to each expert
    int32_t hit_e[kMaxE], hit_slot[kMaxE];
    int32_t fill_e[kMaxE], fill_slot[kMaxE];
    int32_t host_e[kMaxE];
    int32_t evict_key[kMaxE];
    int32_t tok_slot[kMaxK];  // one-token plans: slot of the token's j-th expert, -1 if not resident
};

// Residency state in device memory.
struct DevState {
    int64_t clock, credit;
    int32_t bp, bh;  // MB/s
    int32_t seq;
    int32_t frozen;  // static placement: lookups fill and evict nothing
    int32_t ticket;  // workgroups done in the fused entry + plan launch (0 between launches)
    int32_t sync_err;  // a fill + gate/up launch gave up waiting for its fills: the next
                       // one-token plan reports the error and clears it
    // fill workgroups of the fill + gate/up launch that have copied what gate/up
    // reads of the r-th filled expert; every plan sets them to 0 for the launch
    // that follows it
    uint32_t fill_ready[kMaxK];
};

// ---------------------------------------------------------------- launches
// Router (fixed-order fp32 logits, top-k, softmax).
// Rt: R interleaved per chain ([E][H/256][64][4] fp32) and xT: scratch for x
// interleaved the same way ([T][H/512][64][8] bf16); both optional (then the
// direct kernel runs).
hipError_t launch_route(const void* x, int act_bf16, const float* R, const float* Rt, int T,
                        int E, int H, int k, const int32_t* forced, int32_t* ids, float* w,
                        float* z_scratch, uint16_t* xT, hipStream_t s);

// True when launch_route takes the chain-interleaved kernel (then it needs Rt
// and the xT scratch of T * H bf16).
bool route_chains_ok(int T, int E, int H, int act_bf16);

// Layer entry of one token in the stacked decode step (bf16 activations):
// r_out = bf16(r_in + sum_j parts[j] + y_host) (r_in copied when there are no
// parts), u = bf16(r_out / sqrt(mean(r_out^2) + 1e-6)), z[e] = router logit of
// u in the fixed chain order from the chain-interleaved router Rt.
// y_out (optional) receives the summed parts. r_out must not alias r_in when
// parts are given. Needs entry_ok(E, H, act_bf16).
struct EntryArgs {
    const uint16_t* r_in;
    uint16_t* r_out;
    const float* parts;  // [nparts][H] or null
    int nparts;
    const float* y_host;  // [H] or null (device-visible)
    float* y_out;         // [H] or null
    uint16_t* u;          // [H]
    const float* Rt;
    float* z;  // [E]
    int E, H;
};
bool entry_ok(int E, int H, int act_bf16);
hipError_t launch_entry(const EntryArgs& a, hipStream_t s);

// Lookup + LRU + miss plan, single workgroup; writes plan to d_plan and a
// mirror (header, lists, ids, w and, when x_mirror != null, x) to host memory.
// With rt.z (one token only), the kernel first selects the token's experts
// from the logits z [E] (forced ids if given) and writes them to rt.ids_out /
// rt.w_out; ids and w are then ignored.
struct PlanRoute {
    const float* z;
    const int32_t* forced;
    int32_t* ids_out;
    float* w_out;
};
hipError_t launch_plan(int layer, const int32_t* ids, const float* w, const void* x,
                       size_t x_bytes, int T, int k, int E, int64_t C, int32_t* slot_key,
                       int64_t* slot_stamp, int32_t* key2slot, DevState* st, DevPlan* d_plan,
                       DevPlan* h_plan, int32_t* h_ids, float* h_w, void* h_x, hipStream_t s,
                       PlanRoute rt = PlanRoute{nullptr, nullptr, nullptr, nullptr});
// Layer entry and the one-token plan in one launch (E/4 workgroups; the last
// to finish plans). rt.z must be a.z; x of the plan is a.u.
bool entry_plan_ok(int T, int k, int E, int H, int64_t C, int act_bf16);
hipError_t launch_entry_plan(const EntryArgs& a, int layer, int k, int64_t C, int32_t* slot_key,
                             int64_t* slot_stamp, int32_t* key2slot, DevState* st,
                             DevPlan* d_plan, DevPlan* h_plan, int32_t* h_ids, float* h_w,
                             void* h_x, hipStream_t s, PlanRoute rt);

// Fill: copy the plan's q_fill experts from the layer's pool (device-visible
// pointer to pinned host memory, E * S_pad bytes) into their slots. Reads the
// fill list from d_plan; no host synchronisation.
hipError_t launch_fill(const DevPlan* plan, const uint8_t* pool_layer_dev, uint8_t* slots,
                       uint64_t S, uint64_t S_pad, hipStream_t s, hipEvent_t ev_start = nullptr,
                       hipEvent_t ev_stop = nullptr);

// One expert block from host (device-visible address) to device with the fill
// kernel's copy (the B_P probe).
hipError_t launch_copy_expert(const uint8_t* src_dev, uint8_t* dst, uint64_t S, hipStream_t s);

// Permute: group the (token, k) pairs whose expert is resident by expert,
// stable in pair order; the shared expert (when present) is group E holding
// every token. Produces offsets [E+2], tile offsets and perm_pair; the grouped
// GEMM gathers each permuted row's input row through perm_pair itself.
struct PermuteBufs {
    int32_t* counts;     // [E+1]
    int32_t* offsets;    // [E+2]
    int32_t* tile_off;   // [E+2], tiles of kTileM rows per group
    int32_t* perm_pair;  // [P_max], pair index t*k+j (shared rows: T*k + t)
    int32_t* chunk_cnt;  // [nchunks, E]
};
hipError_t launch_permute(const int32_t* ids, const int32_t* e2slot, int all_resident, int T,
                          int k, int E, int has_shared, PermuteBufs b, hipStream_t s);

// Grouped SwiGLU FFN (GEMM path). Weight base of group g: shared_w for g == E,
// else (e2slot ? slots + e2slot[g]*stride : slots + g*stride).
struct GroupW {
    const uint8_t* slots;
    const int32_t* e2slot;  // null: group g lives at slots + g*stride
    uint64_t stride;
    const uint8_t* shared_w;
    const uint8_t* const* gbase = nullptr;  // when set: group g (< E) lives at gbase[g]
};
hipError_t launch_ffn_gemm(int fmt, const Layout& lay, GroupW gw, int E, int has_shared, int H,
                           int I, int P_max, const int32_t* offsets, const int32_t* tile_off,
                           const void* x /*[T, H] layer input*/, void* h_buf,
                           const int32_t* perm_pair,
                           const int32_t* ids, const float* w, int k, int T, void* o_pairs,
                           hipStream_t s,
                           hipEvent_t* ev /*[4]: start/stop of each kernel, entries may be null*/);

// Combine: y[t] = sum_j (resident) o_pairs[t*k+j] + o_pairs[T*k+t] (shared)
// + y_host[t] (if given). Optional residual: x_out = act(x + y).
hipError_t launch_combine(const void* o_pairs, const int32_t* ids, const int32_t* e2slot,
                          int all_resident, int has_shared, const float* y_host, int T, int k,
                          int H, float* y, void* x_res, int act_bf16, hipStream_t s, int E);

// Decode GEMV path (T == 1): phase A gate/up -> h, phase B down with weights.
// When the host already knows the plan and the routing of the token it passes
// each slot's weight base (null: host-executed) and routing weight directly.
struct GemvExperts {
    int valid;
    const uint8_t* base[kMaxK + 1];
    float w[kMaxK + 1];
};
// Without ex, a one-token plan's weight bases come from plan->tok_slot (one
// load) rather than from ids and e2slot.
hipError_t launch_ffn_gemv(int fmt, const Layout& lay, GroupW gw, const DevPlan* plan,
                           const int32_t* ids, const float* w, int k, int E, int has_shared,
                           int H, int I, const void* x, int act_bf16, float* h_buf,
                           float* y_parts, hipStream_t s,
                           hipEvent_t* ev /*[4]: start/stop of each kernel, entries may be null*/,
                           int allow_fast, const GemvExperts* ex /*may be null*/);
// One-token decode, fill and GEMV with the copies overlapped: one launch whose
// first kFillBlocks workgroups copy the plan's fills from the layer's pool into
// their slots (slots: gw.slots, writable; as launch_fill) while the others run
// gate/up for every expert slot, those of a filled expert once the bytes gate/up
// reads are in (st->fill_ready[r], which the plan set to 0, reaching
// kFillBlocks; a wait bounded by wait_ticks of the device's 100 MHz clock that
// sets st->sync_err when it runs out); on a layer call with fills the same
// launch also runs the down rows of the slots resident before the call, once
// their gate/up rows are counted in `counters`; then the down kernel (the
// filled experts' down rows on such a call, every slot's otherwise). The same
// arithmetic as launch_fill followed by launch_ffn_gemv.
// hipErrorNotSupported (nothing launched) where the tuned one-token GEMV does
// not apply (activations not bf16, fp32 weights, untuned shapes).
hipError_t launch_fill_gemv(int fmt, const Layout& lay, GroupW gw, uint8_t* slots,
                            const DevPlan* plan, const uint8_t* pool_layer_dev, uint64_t S,
                            uint64_t S_pad,
                            const int32_t* ids, const float* w, int k, int E, int has_shared,
                            int H, int I, const void* x, int act_bf16, float* h_buf,
                            float* y_parts, DevState* st, uint32_t* counters,
                            uint64_t wait_ticks, hipStream_t s);
// Bytes of the counters launch_fill_gemv takes (device memory, zero before the
// first launch; each launch leaves them zero).
size_t fill_gemv_counter_bytes();
// Sum of the GEMV partials (k + shared rows of [H]) plus host results; with
// x_res, x_res = act(x_in + y) (x_in null: in place).
hipError_t launch_gemv_reduce(const float* y_parts, int nparts, const float* y_host, int H,
                              float* y, void* x_res, int act_bf16, hipStream_t s,
                              const void* x_in = nullptr);

// u [T,H] = RMS-normalised rows of r (activation dtype, 16-byte aligned rows).
hipError_t launch_rmsnorm(const void* r, void* u, int T, int H, int act_bf16, hipStream_t s);

// Debug dequant of one expert block to fp32 (device decoder).
hipError_t launch_dequant(int fmt, const Layout& lay, const uint8_t* blk, int H, int I, float* out,
                          hipStream_t s);
// The same through the decoders of the grouped GEMM (dec 1) or the decode GEMV
// (dec 2), with the factors each applies outside its decode.
hipError_t launch_dequant_dec(int dec, int fmt, const Layout& lay, const uint8_t* blk, int H,
                              int I, float* out, hipStream_t s);

constexpr int kTileM = 128;  // grouped GEMM tile rows

}  // namespace eo
