// Expert-cache lookup, global LRU update and miss plan (one workgroup).
//
// zhichai.net article, section 2: the Decode paragraph has most routed experts
// hit a device-resident LRU expert cache and splits the m misses of a step
// by the measured bandwidths, q* = m * B_P / B_H filled over PCIe and the rest
// executed on the host; the LRU paragraph makes the cache one global LRU over
// all layers. Integer rules (exactly reproducible):
//   clock += 1 per call; hits get stamp = clock;
//   q = min(m, floor((c + m*B_P)/B_H)), c <- min(c + m*B_P - q*B_H, B_H - 1);
//   q_fill = min(q, C - hits) (0 under a static placement); misses ranked by
//   (tokens desc, id asc), the
//   first q_fill filled, the rest host-executed and not inserted;
//   evict max(0, q_fill - empty) slots not touched this call in
//   (stamp asc, key asc) order; empty + freed slots, ascending, go to the
//   fills in rank order.
// The slot table is staged in LDS for the call (C <= kMaxSlotsLds) and
// written back; key2slot (L*E entries) stays in global memory, each entry
// touched by one thread only.
#include <algorithm>

#include "dev_common.h"
#include "eo_internal.h"
#include "route_dev.h"
#include "entry_dev.h"

namespace eo {

namespace {

constexpr int kThreads = 1024;
constexpr int kMaxSlotsLds = 8192;
constexpr int kMaxSlotsPerThread = kMaxSlotsLds / kThreads;

__device__ __forceinline__ uint64_t wave_min_u64(uint64_t v) {
#pragma unroll
    for (int s = 32; s >= 1; s >>= 1) {
        uint32_t lo = __shfl_xor((uint32_t)v, s, 64);
        uint32_t hi = __shfl_xor((uint32_t)(v >> 32), s, 64);
        uint64_t o = ((uint64_t)hi << 32) | lo;
        v = o < v ? o : v;
    }
    return v;
}

__device__ __forceinline__ int wave_sum_i32(int v) {
#pragma unroll
    for (int s = 32; s >= 1; s >>= 1) v += __shfl_xor(v, s, 64);
    return v;
}

// Block-wide sum; every thread gets the total.
__device__ int block_sum(int v, int* red) {
    v = wave_sum_i32(v);
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    __syncthreads();
    if (lane == 0) red[wave] = v;
    __syncthreads();
    int tot = 0;
    for (int i = 0; i < kThreads / 64; ++i) tot += red[i];
    return tot;
}

// Block-wide exclusive prefix of v in thread order; returns (prefix, total).
__device__ int2 block_scan(int v, int* red) {
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    int incl = v;
#pragma unroll
    for (int s = 1; s < 64; s <<= 1) {
        int o = __shfl_up(incl, s, 64);
        if (lane >= s) incl += o;
    }
    __syncthreads();
    if (lane == 63) red[wave] = incl;
    __syncthreads();
    int base = 0, tot = 0;
    for (int i = 0; i < kThreads / 64; ++i) {
        if (i < wave) base += red[i];
        tot += red[i];
    }
    return make_int2(base + incl - v, tot);
}

// Block-wide exclusive prefix of a 64-bit v in thread order (fields packed in
// v must not carry into each other); returns the prefix, *total gets the sum.
__device__ uint64_t block_scan64(uint64_t v, uint64_t* red, uint64_t* total) {
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    uint64_t incl = v;
#pragma unroll
    for (int s = 1; s < 64; s <<= 1) {
        uint32_t lo = __shfl_up((uint32_t)incl, s, 64);
        uint32_t hi = __shfl_up((uint32_t)(incl >> 32), s, 64);
        if (lane >= s) incl += ((uint64_t)hi << 32) | lo;
    }
    __syncthreads();
    if (lane == 63) red[wave] = incl;
    __syncthreads();
    uint64_t base = 0, tot = 0;
    for (int i = 0; i < kThreads / 64; ++i) {
        if (i < wave) base += red[i];
        tot += red[i];
    }
    *total = tot;
    return base + incl - v;
}

__device__ uint64_t block_min_u64(uint64_t v, uint64_t* red) {
    v = wave_min_u64(v);
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    __syncthreads();
    if (lane == 0) red[wave] = v;
    __syncthreads();
    uint64_t m = ~0ull;
    for (int i = 0; i < kThreads / 64; ++i) m = red[i] < m ? red[i] : m;
    return m;
}

__global__ __launch_bounds__(kThreads) void k_plan(
    int layer, const int32_t* ids, const float* w, const uint8_t* __restrict__ x, int x_bytes,
    int T, int k, int E, int C, int32_t* __restrict__ g_slot_key,
    int64_t* __restrict__ g_slot_stamp, int32_t* __restrict__ key2slot,
    DevState* __restrict__ st, DevPlan* __restrict__ dp, DevPlan* __restrict__ hp,
    int32_t* __restrict__ h_ids, float* __restrict__ h_w, uint8_t* __restrict__ h_x,
    PlanRoute rt) {
    extern __shared__ int64_t smem64[];
    int64_t* s_stamp = smem64;                    // [C]
    int32_t* s_key = (int32_t*)(smem64 + C);      // [C]
    __shared__ int cnt[kMaxE];
    __shared__ int kind[kMaxE];  // 0 unrouted, 1 hit, 2 miss
    __shared__ int slot_of[kMaxE];
    __shared__ int red[kThreads / 64];
    __shared__ uint64_t red64[kThreads / 64];
    __shared__ int s_err;
    __shared__ long long s_clock, s_credit;
    __shared__ int s_m, s_h, s_q, s_qfill;
    __shared__ int fill_e[kMaxE];

    __shared__ int32_t s_ids[kMaxK];
    __shared__ float s_w[kMaxK];

    __shared__ int s_vslot;

    __shared__ int s_miss[kMaxE];
    __shared__ long long s_credit0;
    __shared__ int s_bp, s_bh, s_seq0, s_frozen;

    const int tid = threadIdx.x;
    // slot table into LDS (every load of a thread issued before its first
    // store), the empty slots of this thread counted on the way; the residency
    // counters
    int my_empty = 0;
    {
        int32_t kr[kMaxSlotsPerThread];
        int64_t sr[kMaxSlotsPerThread];
#pragma unroll
        for (int i = 0; i < kMaxSlotsPerThread; ++i) {
            const int sl = tid + i * kThreads;
            if (sl < C) {
                kr[i] = g_slot_key[sl];
                sr[i] = g_slot_stamp[sl];
            }
        }
        if (tid == 0) {
            s_clock = st->clock;
            s_credit0 = st->credit;
            s_bp = st->bp;
            s_bh = st->bh;
            s_seq0 = st->seq;
            s_frozen = st->frozen;
        }
        // one token: the first wavefront selects its experts from the logits
        // while the table loads are in flight
        if (rt.z && tid < 64) topk_token(rt.z, E, k, rt.forced, s_ids, s_w);
#pragma unroll
        for (int i = 0; i < kMaxSlotsPerThread; ++i) {
            const int sl = tid + i * kThreads;
            if (sl < C) {
                s_key[sl] = kr[i];
                s_stamp[sl] = sr[i];
                my_empty += kr[i] < 0;
            }
        }
    }
    for (int e = tid; e < E; e += kThreads) cnt[e] = 0;
    if (tid == 0) s_err = 0;
    __syncthreads();
    if (rt.z) {
        if (tid < k) {
            rt.ids_out[tid] = s_ids[tid];
            rt.w_out[tid] = s_w[tid];
        }
        ids = s_ids;
        w = s_w;
    }

    // token counts per expert; ids must be in range and distinct per token
    for (int p = tid; p < T * k; p += kThreads) {
        int e = ids[p];
        if (e < 0 || e >= E) {
            s_err = 1;
            continue;
        }
        int t = p / k, j = p - t * k;
        for (int jj = 0; jj < j; ++jj)
            if (ids[t * k + jj] == e) s_err = 2;
        atomicAdd(&cnt[e], 1);
    }
    __syncthreads();
    if (s_err) {
        if (tid < kMaxK) dp->tok_slot[tid] = -1;  // nothing resident for this token
        if (tid == 0) {
            int seq = s_seq0 + 1;
            st->seq = seq;
            for (int i = 0; i < kMaxK; ++i) st->fill_ready[i] = 0;  // for the launch after the plan
            dp->pad = s_err;
            hp->pad = s_err;
            dp->seq = seq;
            __threadfence_system();
            __hip_atomic_store(&hp->seq, seq, __ATOMIC_RELEASE, __HIP_MEMORY_SCOPE_SYSTEM);
        }
        return;
    }
    const int64_t clock = s_clock + 1;

    // hits and misses (E <= kThreads: one expert per thread)
    const int my_e = tid < E ? tid : -1;
    int kd = 0, sl = -1;
    if (my_e >= 0 && cnt[my_e] > 0) {
        int s = key2slot[layer * E + my_e];
        if (s >= 0) {
            kd = 1;
            sl = s;
            s_stamp[s] = clock;
        } else {
            kd = 2;
        }
    }
    if (my_e >= 0) {
        kind[my_e] = kd;
        slot_of[my_e] = sl;
    }
    // one scan: hit index (bits 0-15), miss index (16-31), empty slots (32-)
    uint64_t tot;
    const uint64_t pre = block_scan64((uint64_t)(kd == 1) | ((uint64_t)(kd == 2) << 16) |
                                          ((uint64_t)my_empty << 32),
                                      red64, &tot);
    const int n_hit0 = (int)(tot & 0xFFFF), m = (int)((tot >> 16) & 0xFFFF);
    const int empty = (int)(tot >> 32);
    if (kd == 1) {
        const int hi = (int)(pre & 0xFFFF);
        dp->hit_e[hi] = hp->hit_e[hi] = my_e;
        dp->hit_slot[hi] = hp->hit_slot[hi] = sl;
    } else if (kd == 2) {
        s_miss[(pre >> 16) & 0xFFFF] = my_e;
    }
    if (tid == 0) {
        s_h = n_hit0;
        s_m = m;
        long long c = s_credit0, bp = s_bp, bh = s_bh;
        long long q = (c + (long long)m * bp) / bh;
        if (q > m) q = m;
        long long c2 = c + (long long)m * bp - q * bh;
        if (c2 > bh - 1) c2 = bh - 1;
        s_credit = c2;
        s_q = (int)q;
        int room = s_frozen ? 0 : C - n_hit0;  // a static placement takes no fills
        s_qfill = (int)(q < room ? q : room);
    }
    __syncthreads();
    const int q_fill = s_qfill;

    // rank misses by (count desc, id asc) within the list of misses
    if (kd == 2) {
        const int c0 = cnt[my_e];
        int r = 0;
        for (int j = 0; j < m; ++j) {
            const int e2 = s_miss[j], c2 = cnt[e2];
            r += (c2 > c0 || (c2 == c0 && e2 < my_e));
        }
        if (r < q_fill) {
            fill_e[r] = my_e;
            dp->fill_e[r] = hp->fill_e[r] = my_e;
        } else {
            dp->host_e[r - q_fill] = hp->host_e[r - q_fill] = my_e;
        }
    }

    // victims among occupied slots not touched this call (stamp < clock)
    int need = q_fill - empty;
    int n_ev = 0;
    for (int r = 0; r < need; ++r, ++n_ev) {
        uint64_t best = ~0ull;
        int best_slot = -1;
        for (int s = tid; s < C; s += kThreads) {
            if (s_key[s] >= 0 && s_stamp[s] < clock) {
                uint64_t v = ((uint64_t)s_stamp[s] << 24) | (uint64_t)s_key[s];
                if (v < best) {
                    best = v;
                    best_slot = s;
                }
            }
        }
        const uint64_t mine = best;
        best = block_min_u64(best, red64);
        if (best == ~0ull) break;  // unreachable: q_fill <= C - hits
        // keys are unique among occupied slots: one thread holds the victim
        if (mine == best) s_vslot = best_slot;
        __syncthreads();
        if (tid == 0) {
            const int vkey = (int)(best & 0xFFFFFFull);
            dp->evict_key[r] = hp->evict_key[r] = vkey;
            key2slot[vkey] = -1;
            s_key[s_vslot] = -1;  // refilled below: every freed slot takes a fill
        }
        __syncthreads();
    }

    // empty slots in ascending order go to the fills in rank order
    const int per = (C + kThreads - 1) / kThreads;
    const int s_lo = min(C, tid * per), s_hi = min(C, s_lo + per);
    int range_empty = 0;
    if (q_fill > 0)  // block-uniform
        for (int s = s_lo; s < s_hi; ++s) range_empty += (s_key[s] < 0);
    int r = q_fill > 0 ? block_scan(range_empty, red).x : 0;
    for (int s = s_lo; s < s_hi && r < q_fill; ++s) {
        if (s_key[s] < 0) {
            int e = fill_e[r];
            int key = layer * E + e;
            s_key[s] = key;
            s_stamp[s] = clock;
            g_slot_key[s] = key;
            g_slot_stamp[s] = clock;
            key2slot[key] = s;
            slot_of[e] = s;
            dp->fill_slot[r] = hp->fill_slot[r] = s;
            ++r;
        }
    }
    // write-back of the rest of the table: only hit stamps changed (evicted
    // slots are all refilled above)
    for (int e = tid; e < E; e += kThreads)
        if (kind[e] == 1) g_slot_stamp[slot_of[e]] = clock;
    __syncthreads();

    for (int e = tid; e < E; e += kThreads) {
        dp->e2slot[e] = slot_of[e];
        dp->count[e] = cnt[e];
    }
    if (T == 1 && tid < k) dp->tok_slot[tid] = slot_of[ids[tid]];
    const int n_hit = s_h, n_host = s_m - q_fill, n_evict = n_ev;
    if (tid == 0) {
        dp->pad = 0;
        dp->layer = layer;
        dp->T = T;
        dp->k = k;
        dp->m = s_m;
        dp->q = s_q;
        dp->q_fill = q_fill;
        dp->n_hit = n_hit;
        dp->n_host = n_host;
        dp->n_evict = n_evict;
        dp->clock = clock;
        dp->credit = s_credit;
        st->clock = clock;
        st->credit = s_credit;
    }
    __syncthreads();  // dp lists complete (same workgroup)

    // host mirror: lists were written alongside the device copy; add ids, w, x
    if (h_ids && h_w) {
        for (int p = tid; p < T * k; p += kThreads) {
            h_ids[p] = ids[p];
            h_w[p] = w[p];
        }
    }
    if (h_x && n_host > 0) {
        const uint4* xs = (const uint4*)x;
        uint4* xd = (uint4*)h_x;
        for (int i = tid; i < x_bytes / 16; i += kThreads) xd[i] = xs[i];
    }
    if (tid == 0) {
        hp->pad = 0;
        hp->layer = layer;
        hp->T = T;
        hp->k = k;
        hp->m = s_m;
        hp->q = s_q;
        hp->q_fill = q_fill;
        hp->n_hit = n_hit;
        hp->n_host = n_host;
        hp->n_evict = n_evict;
        hp->clock = clock;
        hp->credit = s_credit;
    }
    __syncthreads();
    if (tid == 0) {
        int seq = s_seq0 + 1;
        st->seq = seq;
        for (int i = 0; i < kMaxK; ++i) st->fill_ready[i] = 0;  // for the launch after the plan
        dp->seq = seq;
        __threadfence_system();
        __hip_atomic_store(&hp->seq, seq, __ATOMIC_RELEASE, __HIP_MEMORY_SCOPE_SYSTEM);
    }
}

// ---------------------------------------------------------------- one token
// The same rules for a single token (T = 1, every decode step). The token's k
// experts are lanes of the first wavefront, which takes every decision with
// ballots and shuffles and no workgroup barrier; the other wavefronts only
// stage the slot table in LDS (needed when something is filled) and help with
// the host mirror. With one token every routed expert has count 1, so misses
// rank by expert id, and hits are listed in expert-id order.
constexpr int kThreads1 = 256;

__device__ __forceinline__ uint64_t wave_min_u64_1(uint64_t v) {
#pragma unroll
    for (int s = 32; s >= 1; s >>= 1) {
        uint32_t lo = __shfl_xor((uint32_t)v, s, 64);
        uint32_t hi = __shfl_xor((uint32_t)(v >> 32), s, 64);
        uint64_t o = ((uint64_t)hi << 32) | lo;
        v = o < v ? o : v;
    }
    return v;
}

// floor(a / b) for 0 <= a < 2^52 and b > 0, exactly: the double quotient is
// within one of it, and the integer products correct it.
__device__ __forceinline__ long long div_floor_small(long long a, long long b) {
    long long q = (long long)((double)a / (double)b);
    if (q * b > a)
        --q;
    else if ((q + 1) * b <= a)
        ++q;
    return q;
}

// The one-token plan for one workgroup of kThreads1 threads; smem64 holds
// 12*C bytes of LDS. x_lds != null: the token's row is taken from these LDS
// floats (bf16 values) instead of from x.
__device__ __forceinline__ void plan1_body(
    int64_t* smem64, int layer, const int32_t* ids_in, const float* w_in,
    const uint8_t* __restrict__ x, int x_bytes, int k, int E, int C,
    int32_t* __restrict__ g_slot_key, int64_t* __restrict__ g_slot_stamp,
    int32_t* __restrict__ key2slot, DevState* __restrict__ st, DevPlan* __restrict__ dp,
    DevPlan* __restrict__ hp, int32_t* __restrict__ h_ids, float* __restrict__ h_w,
    uint8_t* __restrict__ h_x, PlanRoute rt, const float* x_lds = nullptr) {
    int64_t* s_stamp = smem64;                // [C]
    int32_t* s_key = (int32_t*)(smem64 + C);  // [C]
    __shared__ int32_t s_ids[kMaxK];
    __shared__ float s_w[kMaxK];
    __shared__ int32_t s_fill_slot[kMaxK];
    __shared__ int32_t s_k2s[kMaxE];  // this layer's row of key2slot
    __shared__ int s_err, s_nhost, s_qfill, s_empty;
    __shared__ long long s_clock0, s_credit0;
    __shared__ int s_bp, s_bh, s_seq0, s_frozen;
    __shared__ int red[kThreads1 / 64];
    __shared__ uint64_t red64[2][kThreads1 / 64];
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    // after the load, each thread owns a contiguous range of slots (empty-slot
    // order is by index)
    const int per = (C + kThreads1 - 1) / kThreads1;
    const int s_lo = min(C, tid * per), s_hi = min(C, s_lo + per);

    // wavefronts 1.. load the slot table into LDS (coalesced, in batches whose
    // loads are all issued before their stores, empty slots counted on the
    // way) while wavefront 0 loads the state and this layer's key2slot row and
    // takes the token's experts; no wavefront's loads queue behind another's
    if (tid == 0) s_empty = 0;
    if (tid < kMaxK) s_fill_slot[tid] = -1;
    int my_empty = 0;
    constexpr int kB = 16, kLoaders = kThreads1 - 64, kRowPer = kMaxE / 64;
    if (wave == 0) {
        // unconditional loads (indexes clamped into the row): no load waits
        // for the one before it
        int32_t k2[kRowPer];
#pragma unroll
        for (int i = 0; i < kRowPer; ++i) k2[i] = key2slot[layer * E + min(lane + 64 * i, E - 1)];
        long long c0 = 0, c1 = 0;
        int v0 = 0, v1 = 0, v2 = 0, v3 = 0, v4 = 0;
        if (lane == 0) {
            c0 = st->clock;
            c1 = st->credit;
            v0 = st->bp;
            v1 = st->bh;
            v2 = st->seq;
            v3 = st->frozen;
            v4 = st->sync_err;
        }
        if (rt.z) {
            topk_token<true>(rt.z, E, k, rt.forced, s_ids, s_w);
        } else if (lane < k) {
            s_ids[lane] = ids_in[lane];
            s_w[lane] = w_in ? w_in[lane] : 0.0f;
        }
#pragma unroll
        for (int i = 0; i < kRowPer; ++i)
            if (lane + 64 * i < E) s_k2s[lane + 64 * i] = k2[i];
        if (lane == 0) {
            s_clock0 = c0;
            s_credit0 = c1;
            s_bp = v0;
            s_bh = v1;
            s_seq0 = v2;
            s_frozen = v3;
            s_err = v4 ? 3 : 0;
        }
    } else {
        const int lt = tid - 64;
        for (int b0 = 0; b0 * kLoaders < C; b0 += kB) {
            int32_t kr[kB];
            int64_t sr[kB];
#pragma unroll
            for (int i = 0; i < kB; ++i) {  // unconditional (clamped): all in flight at once
                const int sl = min(lt + kLoaders * (b0 + i), C - 1);
                kr[i] = g_slot_key[sl];
                sr[i] = g_slot_stamp[sl];
            }
#pragma unroll
            for (int i = 0; i < kB; ++i) {
                const int sl = lt + kLoaders * (b0 + i);
                if (sl < C) {
                    s_key[sl] = kr[i];
                    s_stamp[sl] = sr[i];
                    my_empty += kr[i] < 0;
                }
            }
        }
    }
    __syncthreads();
    if (my_empty) atomicAdd(&s_empty, my_empty);

    // the decisions, in the first wavefront (lane j holds the token's j-th expert)
    const bool act = wave == 0 && lane < k;
    const int e = act ? s_ids[lane] : -1;
    const int key = layer * E + e;
    int slot = -1, rank = 0;
    bool hit = false, miss = false;
    long long q = 0, c2 = 0;
    int m = 0, n_hit = 0;
    const int64_t clock = s_clock0 + 1;
    if (wave == 0) {
        const bool bad = act && (e < 0 || e >= E);
        // other lanes' experts are read across the wavefront (no LDS round trips)
        bool dup = false;
        for (int jj = 0; jj < k; ++jj) dup |= jj < lane && __builtin_amdgcn_readlane(e, jj) == e;
        dup = dup && act && !bad;
        const uint64_t mbad = __ballot(bad), mdup = __ballot(dup);
        const bool late = s_err == 3;  // the previous call's decode launch lost its fills
        if (late || (mbad | mdup)) {
            if (lane == 0) s_err = late ? 3 : mbad ? 1 : 2;
        } else {
            slot = act ? s_k2s[e] : -1;
            hit = act && slot >= 0;
            miss = act && slot < 0;
            const uint64_t mh = __ballot(hit), mm = __ballot(miss);
            n_hit = __popcll(mh);
            m = __popcll(mm);
            for (int jj = 0; jj < k; ++jj)  // rank among the hits (or misses) by expert id
                rank += ((hit ? (mh >> jj) : (mm >> jj)) & 1) &&
                        __builtin_amdgcn_readlane(e, jj) < e;
            if (lane == 0) {  // the split (integer credit)
                const long long c = s_credit0, bp = s_bp, bh = s_bh;
                q = div_floor_small(c + (long long)m * bp, bh);
                if (q > m) q = m;
                c2 = c + (long long)m * bp - q * bh;
                if (c2 > bh - 1) c2 = bh - 1;
                s_qfill = s_frozen ? 0 : (int)min(q, (long long)(C - n_hit));
            }
            q = __shfl(q, 0, 64);
            c2 = __shfl(c2, 0, 64);
            if (hit) {
                s_stamp[slot] = clock;  // touched: not evictable in this call
                g_slot_stamp[slot] = clock;
                dp->hit_e[rank] = hp->hit_e[rank] = e;
                dp->hit_slot[rank] = hp->hit_slot[rank] = slot;
            }
        }
    }
    __syncthreads();
    if (s_err) {
        if (tid < kMaxK) dp->tok_slot[tid] = -1;
        if (tid == 0) {
            const int seq = s_seq0 + 1;
            st->seq = seq;
            for (int i = 0; i < kMaxK; ++i) st->fill_ready[i] = 0;  // for the launch after the plan
            if (s_err == 3) st->sync_err = 0;
            dp->pad = s_err;
            hp->pad = s_err;
            dp->seq = seq;
            __threadfence_system();
            __hip_atomic_store(&hp->seq, seq, __ATOMIC_RELEASE, __HIP_MEMORY_SCOPE_SYSTEM);
        }
        return;
    }
    const int q_fill = s_qfill;
    int n_ev = 0;
    if (q_fill > 0) {  // block-uniform
        // victims (stamp asc, key asc) among occupied slots not touched in
        // this call, one per missing empty slot: each thread keeps the oldest
        // of its slots (tid, tid + 256, ...; read four at a time), one
        // workgroup minimum per victim, and only the owner of the victim looks
        // at its slots again
        const int n_vic = q_fill - s_empty;  // workgroup-uniform
        uint64_t mine = ~0ull;
        int mine_slot = -1;
        auto oldest = [&]() {
            mine = ~0ull;
            for (int s0 = tid; s0 < C; s0 += 4 * kThreads1) {
                int32_t kk[4];
                int64_t ss[4];
#pragma unroll
                for (int u = 0; u < 4; ++u) {
                    const int sl = min(s0 + u * kThreads1, C - 1);
                    kk[u] = s_key[sl];
                    ss[u] = s_stamp[sl];
                }
#pragma unroll
                for (int u = 0; u < 4; ++u) {
                    const int sl = s0 + u * kThreads1;
                    if (sl < C && kk[u] >= 0 && ss[u] < clock) {
                        const uint64_t v = ((uint64_t)ss[u] << 24) | (uint64_t)kk[u];
                        if (v < mine) {
                            mine = v;
                            mine_slot = sl;
                        }
                    }
                }
            }
        };
        if (n_vic > 0) oldest();
        for (int r = 0; r < n_vic; ++r) {
            uint64_t best = wave_min_u64_1(mine);
            if (lane == 0) red64[r & 1][wave] = best;  // two buffers: one barrier per round
            __syncthreads();
            best = red64[r & 1][0];
#pragma unroll
            for (int i = 1; i < kThreads1 / 64; ++i)
                best = red64[r & 1][i] < best ? red64[r & 1][i] : best;
            if (best == ~0ull) break;  // no candidate (cannot happen on a consistent table)
            if (mine == best) {        // exactly one thread: keys are unique
                const int vkey = (int)(best & 0xFFFFFFull);
                dp->evict_key[r] = hp->evict_key[r] = vkey;
                key2slot[vkey] = -1;
                s_key[mine_slot] = -1;  // refilled below
                s_fill_slot[r] = mine_slot;
                if (r + 1 < n_vic) oldest();
            }
            ++n_ev;
        }
        __syncthreads();
        // empty and freed slots in ascending order go to the fills in rank order
        if (s_empty == 0) {  // no empty slot: the freed ones, sorted
            if (tid == 0)
                for (int i = 1; i < n_ev; ++i)
                    for (int j = i; j > 0 && s_fill_slot[j - 1] > s_fill_slot[j]; --j) {
                        const int t = s_fill_slot[j];
                        s_fill_slot[j] = s_fill_slot[j - 1];
                        s_fill_slot[j - 1] = t;
                    }
            __syncthreads();
        } else {
            int mine_empty = 0;
            for (int sl = s_lo; sl < s_hi; ++sl) mine_empty += s_key[sl] < 0;
            int incl = mine_empty;
#pragma unroll
            for (int s = 1; s < 64; s <<= 1) {
                const int o = __shfl_up(incl, s, 64);
                if (lane >= s) incl += o;
            }
            if (lane == 63) red[wave] = incl;
            __syncthreads();
            int r0 = incl - mine_empty;
            for (int i = 0; i < wave; ++i) r0 += red[i];
            for (int sl = s_lo; sl < s_hi && r0 < q_fill; ++sl)
                if (s_key[sl] < 0) s_fill_slot[r0++] = sl;
            __syncthreads();
        }
        if (miss && rank < q_fill && s_fill_slot[rank] >= 0) {
            const int sl = s_fill_slot[rank];
            g_slot_key[sl] = key;
            g_slot_stamp[sl] = clock;
            key2slot[key] = sl;
            dp->fill_e[rank] = hp->fill_e[rank] = e;
            dp->fill_slot[rank] = hp->fill_slot[rank] = sl;
        }
    }
    if (miss && rank >= q_fill) dp->host_e[rank - q_fill] = hp->host_e[rank - q_fill] = e;
    if (act) {
        dp->tok_slot[lane] = hit ? slot : (rank < q_fill ? s_fill_slot[rank] : -1);
        if (rt.z) {
            rt.ids_out[lane] = e;
            rt.w_out[lane] = s_w[lane];
        }
        if (h_ids && h_w) {
            h_ids[lane] = e;
            h_w[lane] = s_w[lane];
        }
    }
    if (tid == 0) {
        const int n_host = m - q_fill;
        s_nhost = n_host;
        dp->pad = 0;
        dp->layer = hp->layer = layer;
        dp->T = hp->T = 1;
        dp->k = hp->k = k;
        dp->m = hp->m = m;
        dp->q = hp->q = (int)q;
        dp->q_fill = hp->q_fill = q_fill;
        dp->n_hit = hp->n_hit = n_hit;
        dp->n_host = hp->n_host = n_host;
        dp->n_evict = hp->n_evict = n_ev;
        dp->clock = hp->clock = clock;
        dp->credit = hp->credit = c2;
        st->clock = clock;
        st->credit = c2;
        hp->pad = 0;
    }
    __syncthreads();
    if (h_x && s_nhost > 0) {
        uint4* xd = (uint4*)h_x;
        if (x_lds) {  // 8 bf16 values held as floats -> 16 bytes of bf16
            for (int i = tid; i < x_bytes / 16; i += kThreads1) {
                const float* f = x_lds + 8 * i;
                uint32_t wd[4];
#pragma unroll
                for (int q = 0; q < 4; ++q)
                    wd[q] = (__float_as_uint(f[2 * q]) >> 16) |
                            (__float_as_uint(f[2 * q + 1]) & 0xFFFF0000u);
                xd[i] = make_uint4(wd[0], wd[1], wd[2], wd[3]);
            }
        } else {
            const uint4* xs = (const uint4*)x;
            for (int i = tid; i < x_bytes / 16; i += kThreads1) xd[i] = xs[i];
        }
    }
    __syncthreads();
    if (tid == 0) {
        const int seq = s_seq0 + 1;
        st->seq = seq;
        for (int i = 0; i < kMaxK; ++i) st->fill_ready[i] = 0;  // for the launch after the plan
        dp->seq = seq;
        __threadfence_system();
        __hip_atomic_store(&hp->seq, seq, __ATOMIC_RELEASE, __HIP_MEMORY_SCOPE_SYSTEM);
    }
}

__global__ __launch_bounds__(kThreads1) void k_plan1(
    int layer, const int32_t* ids_in, const float* w_in, const uint8_t* __restrict__ x,
    int x_bytes, int k, int E, int C, int32_t* __restrict__ g_slot_key,
    int64_t* __restrict__ g_slot_stamp, int32_t* __restrict__ key2slot,
    DevState* __restrict__ st, DevPlan* __restrict__ dp, DevPlan* __restrict__ hp,
    int32_t* __restrict__ h_ids, float* __restrict__ h_w, uint8_t* __restrict__ h_x,
    PlanRoute rt) {
    extern __shared__ int64_t smem64[];
    plan1_body(smem64, layer, ids_in, w_in, x, x_bytes, k, E, C, g_slot_key, g_slot_stamp,
               key2slot, st, dp, hp, h_ids, h_w, h_x, rt);
}

// LDS of the fused kernel: the plan's slot table, then the entry's row of H floats.
__host__ __device__ constexpr size_t entry_plan_row_off(int C) { return (12 * (size_t)C + 15) / 16 * 16; }
__host__ __device__ constexpr size_t entry_plan_lds(int C, int H) {
    return entry_plan_row_off(C) + 4 * (size_t)H;
}
// dynamic LDS limit of the fused kernel (its static LDS is under 16 KB)
constexpr size_t kMaxLdsBytes = 144 * 1024;

// Layer entry and one-token plan in one launch. Every workgroup runs the
// entry (residual, norm, its experts' logits); the last one to finish, found
// with a ticket counter, runs the plan on the complete logit vector. No
// workgroup waits for another, and the last one resets the counter for the
// next launch. The logits are the only data one workgroup of the launch reads
// from another: they are stored and read at device scope, and each workgroup's
// stores have completed before it takes its ticket, so no cache writeback or
// invalidate is needed. The plan takes the token's row from its own LDS copy.
__global__ __launch_bounds__(kThreads1) void k_entry_plan1(
    EntryArgs ea, int layer, int k, int C, int32_t* __restrict__ g_slot_key,
    int64_t* __restrict__ g_slot_stamp, int32_t* __restrict__ key2slot,
    DevState* __restrict__ st, DevPlan* __restrict__ dp, DevPlan* __restrict__ hp,
    int32_t* __restrict__ h_ids, float* __restrict__ h_w, uint8_t* __restrict__ h_x,
    PlanRoute rt) {
    extern __shared__ int64_t smem64[];
    __shared__ int s_last;
    float* s_u = (float*)((uint8_t*)smem64 + entry_plan_row_off(C));
    entry_body(ea, s_u);
    __atomic_signal_fence(__ATOMIC_SEQ_CST);  // the logit store stays above the wait
    __builtin_amdgcn_s_waitcnt(0x0F70);       // vmcnt(0): this wavefront's logit store has completed
    __syncthreads();
    if (threadIdx.x == 0) s_last = atomicAdd(&st->ticket, 1) == (int)gridDim.x - 1;
    __syncthreads();
    if (!s_last) return;
    if (threadIdx.x == 0) st->ticket = 0;
    plan1_body(smem64, layer, nullptr, nullptr, nullptr, ea.H * 2, k, ea.E, C, g_slot_key,
               g_slot_stamp, key2slot, st, dp, hp, h_ids, h_w, h_x, rt, s_u);
}

}  // namespace

int plan_max_slots() { return kMaxSlotsLds; }

hipError_t launch_plan(int layer, const int32_t* ids, const float* w, const void* x,
                       size_t x_bytes, int T, int k, int E, int64_t C, int32_t* slot_key,
                       int64_t* slot_stamp, int32_t* key2slot, DevState* st, DevPlan* d_plan,
                       DevPlan* h_plan, int32_t* h_ids, float* h_w, void* h_x, hipStream_t s,
                       PlanRoute rt) {
    if (rt.z && T != 1) return hipErrorInvalidValue;
    static bool attr_set = false;
    size_t lds = 12 * (size_t)C;
    if (!attr_set) {
        hipError_t e = hipFuncSetAttribute((const void*)k_plan,
                                           hipFuncAttributeMaxDynamicSharedMemorySize,
                                           12 * kMaxSlotsLds);
        if (e == hipSuccess)
            e = hipFuncSetAttribute((const void*)k_plan1, hipFuncAttributeMaxDynamicSharedMemorySize,
                                    12 * kMaxSlotsLds);
        if (e != hipSuccess) return e;
        attr_set = true;
    }
    // EO_PLAN1=0 sends one-token lookups to the general kernel (tests compare them)
    const char* p1 = getenv("EO_PLAN1");
    if (T == 1 && k <= 64 && !(p1 && p1[0] == '0')) {
        k_plan1<<<1, kThreads1, lds, s>>>(layer, ids, w, (const uint8_t*)x, (int)x_bytes, k, E,
                                          (int)C, slot_key, slot_stamp, key2slot, st, d_plan,
                                          h_plan, h_ids, h_w, (uint8_t*)h_x, rt);
        return hipGetLastError();
    }
    k_plan<<<1, kThreads, lds, s>>>(layer, ids, w, (const uint8_t*)x, (int)x_bytes, T, k, E,
                                    (int)C, slot_key, slot_stamp, key2slot, st, d_plan, h_plan,
                                    h_ids, h_w, (uint8_t*)h_x, rt);
    return hipGetLastError();
}

bool entry_plan_ok(int T, int k, int E, int H, int64_t C, int act_bf16) {
    return T == 1 && k <= 64 && C <= kMaxSlotsLds && entry_ok(E, H, act_bf16) &&
           entry_plan_lds((int)C, H) <= kMaxLdsBytes;
}

hipError_t launch_entry_plan(const EntryArgs& a, int layer, int k, int64_t C, int32_t* slot_key,
                             int64_t* slot_stamp, int32_t* key2slot, DevState* st,
                             DevPlan* d_plan, DevPlan* h_plan, int32_t* h_ids, float* h_w,
                             void* h_x, hipStream_t s, PlanRoute rt) {
    if (!rt.z || rt.z != a.z || !entry_plan_ok(1, k, a.E, a.H, C, 1)) return hipErrorInvalidValue;
    static bool attr_set = false;
    if (!attr_set) {
        hipError_t e = hipFuncSetAttribute((const void*)k_entry_plan1,
                                           hipFuncAttributeMaxDynamicSharedMemorySize,
                                           (int)kMaxLdsBytes);
        if (e != hipSuccess) return e;
        attr_set = true;
    }
    const size_t lds = entry_plan_lds((int)C, a.H);
    k_entry_plan1<<<a.E / 4, kThreads1, lds, s>>>(a, layer, k, (int)C, slot_key, slot_stamp,
                                                   key2slot, st, d_plan, h_plan, h_ids, h_w,
                                                   (uint8_t*)h_x, rt);
    return hipGetLastError();
}

}  // namespace eo
