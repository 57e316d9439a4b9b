// Engine and C ABI: the MoE expert-layer forward over a device-resident global
// LRU expert cache backed by a pinned host expert pool (FreeToken; zhichai.net
// article, section 2: Prefill, Decode and LRU paragraphs).
//
// Per layer call: route -> lookup/plan (device) -> fills by a kernel that reads
// the fill list from device memory and the pool over PCIe (hipMemcpyAsync on
// the copy stream under EO_FILL_SDMA=1) -> device FFN on the hits and fills ->
// host-core FFN on the host list (the host reads the plan from mapped memory),
// overlapped with the device -> combine. Prefill streams whole layers into two
// staging buffers. Trace ranges (roctx) name each step call, each layer of a
// decode step or prefill, the plan wait and the host routine.
#include <algorithm>
#include <chrono>
#include <cstdio>
#include <cstdlib>
#include <cstring>
#include <mutex>
#include <string>
#include <thread>
#include <vector>

#include <immintrin.h>

#include <rocprofiler-sdk-roctx/roctx.h>

#include "eo_internal.h"

namespace eo {

// A trace range for the scope (roctx: shown by profilers that record markers,
// a no-op call otherwise).
struct TraceRange {
    explicit TraceRange(const char* name) { roctxRangePushA(name); }
    ~TraceRange() { roctxRangePop(); }
    TraceRange(const TraceRange&) = delete;
    TraceRange& operator=(const TraceRange&) = delete;
};
int plan_max_slots();
}

using namespace eo;

namespace {

thread_local std::string g_err;

eo_status fail(eo_status s, const std::string& msg) {
    g_err = msg;
    return s;
}

#define HIPCHK(expr)                                                                       \
    do {                                                                                   \
        hipError_t e_ = (expr);                                                            \
        if (e_ != hipSuccess)                                                              \
            return fail(EO_ERR_HIP, std::string(#expr) + ": " + hipGetErrorString(e_));   \
    } while (0)

#define EOCHK(expr)                          \
    do {                                     \
        eo_status s_ = (expr);               \
        if (s_ != EO_OK) return s_;          \
    } while (0)

uint64_t round_up(uint64_t v, uint64_t a) { return (v + a - 1) / a * a; }

struct TimedSet {  // start/stop events stamped on each kernel of a pair
    hipEvent_t ev[4];
};

}  // namespace


struct eo_engine {
    eo_config cfg{};
    Layout lay;
    uint64_t S = 0, S_pad = 0;
    int L = 0, E = 0, k = 0, H = 0, I = 0, shared = 0, fmt = 0, act_bf16 = 0;
    int64_t C = 0;
    int act_size = 4;

    std::vector<uint8_t*> pool;      // per layer, E * S_pad pinned bytes
    std::vector<uint8_t*> pool_dev;  // the same, as device-visible addresses
    bool fill_sdma = false;          // EO_FILL_SDMA=1: fills by hipMemcpyAsync (ablation)
    bool fill_gemv = true;  // EO_FILL_GEMV=0: decode fills and gate/up in separate launches
    // longest wait of a filled expert's gate/up rows for its bytes: 1 s of the
    // device's 100 MHz clock (EO_TEST_FILL_WAIT_TICKS sets it, for the test of
    // the path where the wait runs out)
    uint64_t fill_wait_ticks = 100000000ull;
    uint32_t* d_fill_counters = nullptr;  // counters of the fill + GEMV launch (zero between)
    uint8_t* d_slots = nullptr;
    uint8_t* d_shared = nullptr;
    float* d_router = nullptr;
    float* d_router_t = nullptr;  // chain-interleaved layout [L][E][H/256][64][4]
    uint16_t* d_xt = nullptr;     // [max_tokens][64][H/64] bf16 scratch
    int32_t* d_slot_key = nullptr;
    int64_t* d_slot_stamp = nullptr;
    int32_t* d_key2slot = nullptr;
    DevState* d_state = nullptr;
    DevPlan* d_plan = nullptr;
    DevPlan* h_plan = nullptr;  // mapped, coherent
    DevPlan* h_plan_dev = nullptr;
    int32_t* h_ids = nullptr;
    int32_t* h_ids_dev = nullptr;
    float* h_w = nullptr;
    float* h_w_dev = nullptr;
    uint8_t* h_x = nullptr;
    uint8_t* h_x_dev = nullptr;

    int32_t* d_ids = nullptr;
    float* d_w = nullptr;
    float* d_z = nullptr;
    float* d_y = nullptr;
    void* d_u = nullptr;  // [max_tokens, H] layer input (RMS-normalised residual)
    uint16_t* d_r = nullptr;  // [2, H] residual stream of the one-token decode step
    bool fused_entry = true;  // EO_FUSED_ENTRY=0: separate norm / router / top-k kernels
    float* d_hgemv = nullptr;
    float* d_yparts = nullptr;
    float* d_yhost = nullptr;
    float* h_yhost = nullptr;      // mapped, coherent
    float* h_yhost_dev = nullptr;
    std::vector<float> xf;  // host fp32 copy of x for the host routine
    std::vector<float> host_scratch;

    // grouped-FFN buffers, sized for gemm_T tokens
    int gemm_T = 0;
    PermuteBufs pb{};
    void* d_hbuf = nullptr;
    float* d_opairs = nullptr;

    uint8_t* d_staging[2] = {nullptr, nullptr};
    const uint8_t** d_gbase = nullptr;  // [L][E] weight bases of a resident-aware prefill
    size_t gbase_n = 0;
    hipStream_t copy_stream = nullptr;
    hipEvent_t ev_fill = nullptr, ev_copy[2] = {nullptr, nullptr}, ev_comp[2] = {nullptr, nullptr};
    hipEvent_t ev_start = nullptr;

    ThreadPool* tp = nullptr;
    uint32_t bp = 1, bh = 1;

    // plan bookkeeping
    bool plan_pending = false, plan_ready = false, host_staged = false, mirrored = false;
    int plan_seq = 0, plan_layer = -1, plan_T = 0;
    eo_plan_host last_plan{};

    eo_stats stats{};

    uint8_t* scratch = nullptr;  // this device's copy of the file-scope scratch array

    bool plan_log_on = false;
    std::vector<int32_t> plan_log;  // {layer, hits, fills, host experts} per lookup

    bool debug_sync = false;  // EO_DEBUG_SYNC=1: wait for the device after every stage
    int log_level = 0;        // EO_LOG: 1 configuration, 2 + one line per plan
    bool timing = false;
    int gemv_fast = 1;  // EO_GEMV_FAST=0 selects the generic decode GEMV kernels
    std::vector<TimedSet> gemv_ev, gemm_ev, fill_ev, free_ev;
    double kms[5] = {0, 0, 0, 0, 0};  // gemv gate/up, gemv down, gemm1, gemm2, fill
    int64_t gemv_n = 0, gemm_n = 0, fill_n = 0;
    // prefill: one layer's copies on the copy stream / its kernels on the compute stream
    std::vector<TimedSet> copy_ev, comp_ev;
    double sms[2] = {0, 0};
    int64_t copy_n = 0, comp_n = 0;

    void* cap_x = nullptr;
    float* cap_y = nullptr;
    int32_t* cap_ids = nullptr;
    float* cap_w = nullptr;
    int cap_T = 0;
};

// Device scratch of the allocation-free entry point (eo_route_noalloc): one
// copy per GPU, held until the process ends. Host code never passes the
// array's name to a kernel or a copy (on the host it is a stand-in, not a
// device address); it uses the per-device address taken once below.
constexpr size_t kScratchBytes = 16u << 20;
static __device__ __align__(256) uint8_t scratch[kScratchBytes];

namespace {

constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
uint8_t* g_scratch_ptr[kMaxDevices] = {};

// The scratch array's address on `device` (which must be current), looked up
// once per device.
eo_status scratch_on_device(int device, uint8_t** out) {
    if (device < 0 || device >= kMaxDevices) return fail(EO_ERR_UNSUPPORTED, "device ordinal above 63");
    std::lock_guard<std::mutex> lk(g_scratch_mu);
    if (!g_scratch_ptr[device]) {
        void* p = nullptr;
        hipError_t he = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
        if (he != hipSuccess || !p)
            return fail(EO_ERR_HIP, std::string("hipGetSymbolAddress(scratch): ") + hipGetErrorString(he));
        g_scratch_ptr[device] = (uint8_t*)p;
    }
    *out = g_scratch_ptr[device];
    return EO_OK;
}

eo_status get_set(eo_engine* e, TimedSet* p) {
    if (!e->free_ev.empty()) {
        *p = e->free_ev.back();
        e->free_ev.pop_back();
        return EO_OK;
    }
    // timing only: no system-scope fence at record time, so the cache writeback
    // and invalidation it implies do not slow the kernels being timed
    for (int i = 0; i < 4; ++i)
        HIPCHK(hipEventCreateWithFlags(&p->ev[i], hipEventDisableSystemFence));
    return EO_OK;
}

eo_status harvest_times(eo_engine* e) {
    for (auto* v : {&e->gemv_ev, &e->gemm_ev}) {
        const int base = v == &e->gemv_ev ? 0 : 2;
        for (auto& p : *v) {
            HIPCHK(hipEventSynchronize(p.ev[3]));
            float m0 = 0, m1 = 0;
            HIPCHK(hipEventElapsedTime(&m0, p.ev[0], p.ev[1]));
            HIPCHK(hipEventElapsedTime(&m1, p.ev[2], p.ev[3]));
            e->kms[base] += m0;
            e->kms[base + 1] += m1;
            (base == 0 ? e->gemv_n : e->gemm_n) += 1;
            e->free_ev.push_back(p);
        }
        v->clear();
    }
    for (auto* v : {&e->fill_ev, &e->copy_ev, &e->comp_ev}) {
        double& acc = v == &e->fill_ev ? e->kms[4] : e->sms[v == &e->copy_ev ? 0 : 1];
        int64_t& n = v == &e->fill_ev ? e->fill_n : v == &e->copy_ev ? e->copy_n : e->comp_n;
        for (auto& p : *v) {
            HIPCHK(hipEventSynchronize(p.ev[1]));
            float m0 = 0;
            HIPCHK(hipEventElapsedTime(&m0, p.ev[0], p.ev[1]));
            acc += m0;
            n += 1;
            e->free_ev.push_back(p);
        }
        v->clear();
    }
    return EO_OK;
}

eo_status check_layer(eo_engine* e, int layer) {
    if (!e) return fail(EO_ERR_INVALID_ARG, "null engine");
    if (layer < 0 || layer >= e->L) return fail(EO_ERR_INVALID_ARG, "layer out of range");
    return EO_OK;
}

eo_status check_T(eo_engine* e, int T) {
    if (T < 1 || T > e->cfg.max_tokens) return fail(EO_ERR_INVALID_ARG, "T out of range [1, max_tokens]");
    return EO_OK;
}

bool aligned16(const void* p) { return ((uintptr_t)p & 15u) == 0; }

// Debug mode (EO_DEBUG_SYNC=1 at engine creation): after each stage, wait for
// the stream and report an asynchronous device error with the stage's name.
// The kernels and their order are the same, so the results are too.
eo_status stage_done(eo_engine* e, hipStream_t s, const char* stage, int layer) {
    if (!e->debug_sync) return EO_OK;
    hipError_t he = hipStreamSynchronize(s);
    if (he == hipSuccess) he = hipGetLastError();
    if (he != hipSuccess)
        return fail(EO_ERR_HIP, std::string(stage) + " (layer " + std::to_string(layer) + "): " +
                                    hipGetErrorString(he));
    return EO_OK;
}

// Grow the grouped-FFN buffers to hold T tokens.
eo_status ensure_gemm(eo_engine* e, int T, hipStream_t s) {
    if (T <= e->gemm_T) return EO_OK;
    HIPCHK(hipStreamSynchronize(s));
    auto fr = [](void* p) { if (p) (void)hipFree(p); };
    fr(e->pb.counts); fr(e->pb.offsets); fr(e->pb.tile_off); fr(e->pb.perm_pair);
    fr(e->pb.chunk_cnt); fr(e->d_hbuf); fr(e->d_opairs);
    e->pb = PermuteBufs{};
    e->d_hbuf = nullptr;
    e->d_opairs = nullptr;
    e->gemm_T = 0;
    const size_t P = (size_t)T * e->k + T;
    const size_t nchunks = ((size_t)T * e->k + 1023) / 1024 + 1;
    HIPCHK(hipMalloc(&e->pb.counts, sizeof(int32_t) * (e->E + 2)));
    HIPCHK(hipMalloc(&e->pb.offsets, sizeof(int32_t) * (e->E + 2)));
    HIPCHK(hipMalloc(&e->pb.tile_off, sizeof(int32_t) * (e->E + 2)));
    HIPCHK(hipMalloc(&e->pb.perm_pair, sizeof(int32_t) * P));
    HIPCHK(hipMalloc(&e->pb.chunk_cnt, sizeof(int32_t) * nchunks * e->E));
    HIPCHK(hipMalloc(&e->d_hbuf, sizeof(float) * P * e->I));
    HIPCHK(hipMalloc(&e->d_opairs, sizeof(float) * P * e->H));
    e->gemm_T = T;
    return EO_OK;
}

// Spin on the mapped plan mirror until the device has written this call's plan.
eo_status wait_plan(eo_engine* e) {
    if (!e->plan_pending) return fail(EO_ERR_STATE, "no pending plan (call eo_lookup_plan first)");
    if (e->plan_ready) return EO_OK;
    TraceRange trace_range("eo.wait_plan");
    auto t0 = std::chrono::steady_clock::now();
    struct WaitTimer {  // host time spent in this wait, on every way out
        eo_engine* e;
        std::chrono::steady_clock::time_point t0;
        ~WaitTimer() {
            e->stats.host_wait_ns += std::chrono::duration_cast<std::chrono::nanoseconds>(
                                         std::chrono::steady_clock::now() - t0).count();
        }
    } wait_timer{e, t0};
    uint64_t spins = 0;
    while (__atomic_load_n(&e->h_plan->seq, __ATOMIC_ACQUIRE) != e->plan_seq) {
        _mm_pause();
        if ((++spins & 0xFFFF) == 0) {
            hipError_t he = hipGetLastError();
            if (he != hipSuccess) {
                e->plan_pending = false;
                return fail(EO_ERR_HIP, std::string("device error while waiting for plan: ") +
                                            hipGetErrorString(he));
            }
            if (std::chrono::steady_clock::now() - t0 > std::chrono::seconds(20)) {
                e->plan_pending = false;
                return fail(EO_ERR_HIP, "timed out waiting for the device plan");
            }
        }
    }
    const DevPlan* hp = e->h_plan;
    if (hp->pad != 0) {
        e->plan_pending = false;
        if (hp->pad == 3)
            return fail(EO_ERR_HIP, "the previous decode launch gave up waiting for its fills");
        return fail(EO_ERR_INVALID_ARG, hp->pad == 1 ? "expert id out of range in ids"
                                                     : "expert id repeated within a token");
    }
    eo_plan_host& p = e->last_plan;
    p.layer = hp->layer;
    p.m = hp->m;
    p.q = hp->q;
    p.q_fill = hp->q_fill;
    p.n_hit = hp->n_hit;
    p.n_host = hp->n_host;
    p.n_evict = hp->n_evict;
    p.clock = hp->clock;
    p.credit = hp->credit;
    std::memcpy(p.hit_expert, hp->hit_e, sizeof(int32_t) * p.n_hit);
    std::memcpy(p.hit_slot, hp->hit_slot, sizeof(int32_t) * p.n_hit);
    std::memcpy(p.fill_expert, hp->fill_e, sizeof(int32_t) * p.q_fill);
    std::memcpy(p.fill_slot, hp->fill_slot, sizeof(int32_t) * p.q_fill);
    std::memcpy(p.host_expert, hp->host_e, sizeof(int32_t) * p.n_host);
    std::memcpy(p.evicted_key, hp->evict_key, sizeof(int32_t) * p.n_evict);
    e->stats.lookups += 1;
    e->stats.hits += p.n_hit;
    e->stats.misses += p.m;
    e->stats.fills += p.q_fill;
    e->stats.pcie_bytes += (int64_t)p.q_fill * (int64_t)e->S;
    e->stats.device_expert_bytes += (int64_t)(p.n_hit + p.q_fill + e->shared) * (int64_t)e->S;
    if (e->log_level >= 2)
        std::fprintf(stderr, "eo: plan layer %d clock %lld: %d hits, %d misses, q %d, %d fills, %d host, %d evicted, credit %lld\n",
                     p.layer, (long long)p.clock, p.n_hit, p.m, p.q, p.q_fill, p.n_host, p.n_evict,
                     (long long)p.credit);
    if (e->plan_log_on) e->plan_log.insert(e->plan_log.end(), {p.layer, p.n_hit, p.q_fill, p.n_host});
    e->plan_ready = true;
    return EO_OK;
}

// ea != null: the layer entry runs in the same launch (one token; x is ea->u)
eo_status do_plan(eo_engine* e, int layer, const int32_t* ids, const float* w, const void* x,
                  int T, hipStream_t s, PlanRoute rt = PlanRoute{nullptr, nullptr, nullptr, nullptr},
                  const EntryArgs* ea = nullptr) {
    const size_t xb = (size_t)T * e->H * e->act_size;
    hipError_t he =
        ea ? launch_entry_plan(*ea, layer, e->k, e->C, e->d_slot_key, e->d_slot_stamp,
                               e->d_key2slot, e->d_state, e->d_plan, e->h_plan_dev,
                               w ? e->h_ids_dev : nullptr, w ? e->h_w_dev : nullptr,
                               x ? e->h_x_dev : nullptr, s, rt)
           : launch_plan(layer, ids, w ? w : nullptr, x, xb, T, e->k, e->E, e->C,
                         e->d_slot_key, e->d_slot_stamp, e->d_key2slot, e->d_state, e->d_plan,
                         e->h_plan_dev, w ? e->h_ids_dev : nullptr, w ? e->h_w_dev : nullptr,
                         x ? e->h_x_dev : nullptr, s, rt);
    if (he != hipSuccess) return fail(EO_ERR_HIP, std::string("plan launch: ") + hipGetErrorString(he));
    e->plan_seq += 1;
    e->plan_pending = true;
    e->plan_ready = false;
    e->host_staged = false;
    e->mirrored = (w != nullptr && x != nullptr);
    e->plan_layer = layer;
    e->plan_T = T;
    return EO_OK;
}

// Fills of the pending plan, queued on s behind the plan kernel: the fill kernel
// reads the fill list from device memory, so nothing waits for the host.
eo_status do_fill(eo_engine* e, hipStream_t s) {
    if (!e->plan_pending) return fail(EO_ERR_STATE, "no pending plan (call eo_lookup_plan first)");
    if (e->C == 0) return EO_OK;
    if (!e->fill_sdma) {
        TimedSet ts{};
        if (e->timing) EOCHK(get_set(e, &ts));
        hipError_t he = launch_fill(e->d_plan, e->pool_dev[e->plan_layer], e->d_slots, e->S,
                                    e->S_pad, s, ts.ev[0], ts.ev[1]);
        if (he != hipSuccess) return fail(EO_ERR_HIP, std::string("fill: ") + hipGetErrorString(he));
        if (e->timing) e->fill_ev.push_back(ts);
        return EO_OK;
    }
    EOCHK(wait_plan(e));
    const eo_plan_host& p = e->last_plan;
    if (p.q_fill == 0) return EO_OK;
    uint8_t* base = e->pool[p.layer];
    for (int r = 0; r < p.q_fill; ++r) {
        HIPCHK(hipMemcpyAsync(e->d_slots + (uint64_t)p.fill_slot[r] * e->S_pad,
                              base + (uint64_t)p.fill_expert[r] * e->S_pad, e->S,
                              hipMemcpyHostToDevice, e->copy_stream));
    }
    HIPCHK(hipEventRecord(e->ev_fill, e->copy_stream));
    HIPCHK(hipStreamWaitEvent(s, e->ev_fill, 0));
    return EO_OK;
}

eo_status do_host(eo_engine* e, const void* x, const int32_t* ids, const float* w, hipStream_t s) {
    EOCHK(wait_plan(e));
    const eo_plan_host& p = e->last_plan;
    if (p.n_host == 0) return EO_OK;
    const int T = e->plan_T, k = e->k, H = e->H;
    const int32_t* hids;
    const float* hw;
    const uint8_t* hx;
    if (e->mirrored) {
        hids = e->h_ids;
        hw = e->h_w;
        hx = e->h_x;
    } else {
        HIPCHK(hipMemcpyAsync(e->h_ids, ids, sizeof(int32_t) * T * k, hipMemcpyDeviceToHost, s));
        HIPCHK(hipMemcpyAsync(e->h_w, w, sizeof(float) * T * k, hipMemcpyDeviceToHost, s));
        HIPCHK(hipMemcpyAsync(e->h_x, x, (size_t)T * H * e->act_size, hipMemcpyDeviceToHost, s));
        HIPCHK(hipStreamSynchronize(s));
        hids = e->h_ids;
        hw = e->h_w;
        hx = e->h_x;
    }
    e->xf.resize((size_t)T * H);
    if (e->act_bf16) {
        const uint16_t* xb = (const uint16_t*)hx;
        for (size_t i = 0; i < (size_t)T * H; ++i) {
            uint32_t u = (uint32_t)xb[i] << 16;
            std::memcpy(&e->xf[i], &u, 4);
        }
    } else {
        std::memcpy(e->xf.data(), hx, sizeof(float) * T * H);
    }
    std::vector<const uint8_t*> table(e->E, nullptr);
    for (int i = 0; i < p.n_host; ++i)
        table[p.host_expert[i]] = e->pool[p.layer] + (uint64_t)p.host_expert[i] * e->S_pad;
    std::memset(e->h_yhost, 0, sizeof(float) * T * H);
    HostJob jb;
    jb.fmt = e->fmt;
    jb.lay = e->lay;
    jb.H = H;
    jb.I = e->I;
    jb.T = T;
    jb.k = k;
    jb.x = e->xf.data();
    jb.xb = e->act_bf16 ? (const uint16_t*)hx : nullptr;
    jb.ids = hids;
    jb.w = hw;
    jb.experts = table.data();
    jb.y = e->h_yhost;
    const auto th0 = std::chrono::steady_clock::now();
    TraceRange trace_range("eo.host_routine");
    host_ffn(e->tp, jb, e->host_scratch);
    e->stats.host_routine_ns += std::chrono::duration_cast<std::chrono::nanoseconds>(
                                    std::chrono::steady_clock::now() - th0).count();
    // one token: the combine reads the mapped host result directly
    if (T > 1)
        HIPCHK(hipMemcpyAsync(e->d_yhost, e->h_yhost, sizeof(float) * T * H, hipMemcpyHostToDevice, s));
    e->host_staged = true;
    e->stats.host_experts += p.n_host;
    e->stats.host_bytes += (int64_t)p.n_host * (int64_t)e->S;
    return EO_OK;
}

GroupW slots_gw(eo_engine* e, int layer) {
    GroupW gw;
    gw.slots = e->d_slots;
    gw.e2slot = e->d_plan->e2slot;
    gw.stride = e->S_pad;
    gw.shared_w = e->shared ? e->d_shared + (uint64_t)layer * e->S_pad : nullptr;
    return gw;
}

// Device FFN part for the current plan; T == 1 uses the GEMV path.
eo_status do_ffn_device(eo_engine* e, int layer, const void* x, const int32_t* ids, const float* w,
                        hipStream_t s) {
    const int T = e->plan_T;
    GroupW gw = slots_gw(e, layer);
    TimedSet ts{};
    if (e->timing) EOCHK(get_set(e, &ts));
    hipEvent_t* ev = e->timing ? ts.ev : nullptr;
    hipEvent_t none[4] = {nullptr, nullptr, nullptr, nullptr};
    hipError_t he;
    if (T == 1) {
        // the host holds the plan and (mirrored) the token's ids and weights:
        // hand the kernels their weight pointers instead of device lookups
        GemvExperts gx{};
        if (e->mirrored && e->plan_ready) {
            const eo_plan_host& p = e->last_plan;
            gx.valid = 1;
            for (int j = 0; j < e->k; ++j) {
                const int ex = e->h_ids[j];
                int slot = -1;
                for (int i = 0; i < p.n_hit && slot < 0; ++i)
                    if (p.hit_expert[i] == ex) slot = p.hit_slot[i];
                for (int i = 0; i < p.q_fill && slot < 0; ++i)
                    if (p.fill_expert[i] == ex) slot = p.fill_slot[i];
                gx.base[j] = slot < 0 ? nullptr : e->d_slots + (uint64_t)slot * e->S_pad;
                gx.w[j] = e->h_w[j];
            }
            gx.base[e->k] = gw.shared_w;
            gx.w[e->k] = 1.0f;
        }
        he = launch_ffn_gemv(e->fmt, e->lay, gw, e->d_plan, ids, w, e->k, e->E, e->shared, e->H,
                             e->I, x, e->act_bf16, e->d_hgemv, e->d_yparts, s, ev ? ev : none,
                             e->gemv_fast, gx.valid ? &gx : nullptr);
        if (e->timing) e->gemv_ev.push_back(ts);
    } else {
        EOCHK(ensure_gemm(e, T, s));
        he = launch_permute(ids, e->d_plan->e2slot, 0, T, e->k, e->E, e->shared, e->pb, s);
        if (he == hipSuccess)
            he = launch_ffn_gemm(e->fmt, e->lay, gw, e->E, e->shared, e->H, e->I,
                                 T * e->k + T, e->pb.offsets, e->pb.tile_off, x,
                                 e->d_hbuf, e->pb.perm_pair, ids, w, e->k, T, e->d_opairs, s,
                                 ev ? ev : none);
        if (e->timing) e->gemm_ev.push_back(ts);
    }
    if (he != hipSuccess) return fail(EO_ERR_HIP, std::string("ffn launch: ") + hipGetErrorString(he));
    return EO_OK;
}

// One-token decode: the fills and the expert GEMV, in one launch that copies
// the fills while the other experts' gate/up rows run (then the down kernel),
// unless timing is on (the kernels are then timed apart), fills go by
// hipMemcpyAsync, the cache is empty of slots or the tuned GEMV does not apply.
eo_status do_fill_gemv(eo_engine* e, int layer, const int32_t* ids, const float* w,
                       hipStream_t s) {
    if (!e->plan_pending) return fail(EO_ERR_STATE, "no pending plan (call eo_lookup_plan first)");
    if (e->fill_gemv && e->gemv_fast && !e->timing && !e->fill_sdma && e->C > 0 &&
        e->plan_T == 1) {
        hipError_t he = launch_fill_gemv(e->fmt, e->lay, slots_gw(e, layer), e->d_slots, e->d_plan,
                                         e->pool_dev[e->plan_layer], e->S, e->S_pad, ids, w, e->k,
                                         e->E, e->shared, e->H, e->I, e->d_u, e->act_bf16,
                                         e->d_hgemv, e->d_yparts, e->d_state,
                                         e->d_fill_counters, e->fill_wait_ticks, s);
        if (he == hipSuccess) return EO_OK;
        if (he != hipErrorNotSupported)
            return fail(EO_ERR_HIP, std::string("fill and GEMV: ") + hipGetErrorString(he));
    }
    EOCHK(do_fill(e, s));
    return do_ffn_device(e, layer, e->d_u, ids, w, s);
}

eo_status do_combine(eo_engine* e, const int32_t* ids, float* y, void* x_res, hipStream_t s) {
    const int T = e->plan_T;
    const float* yh = e->host_staged ? (T == 1 ? e->h_yhost_dev : e->d_yhost) : nullptr;
    hipError_t he;
    if (T == 1)
        he = launch_gemv_reduce(e->d_yparts, e->k + e->shared, yh, e->H, y, x_res, e->act_bf16, s);
    else
        he = launch_combine(e->d_opairs, ids, e->d_plan->e2slot, 0, e->shared, yh, T, e->k, e->H,
                            y, x_res, e->act_bf16, s, e->E);
    if (he != hipSuccess) return fail(EO_ERR_HIP, std::string("combine: ") + hipGetErrorString(he));
    e->plan_pending = false;
    e->plan_ready = false;
    e->host_staged = false;
    return EO_OK;
}

// One full layer through the cache. x_res != null applies the residual in place.
eo_status moe_layer_impl(eo_engine* e, int layer, const void* x, float* y, int T,
                         const int32_t* forced, int32_t* ids, float* w, void* x_res,
                         hipStream_t s) {
    const size_t roff = (size_t)layer * e->E * e->H;
    hipError_t he = launch_route(x, e->act_bf16, e->d_router + roff, e->d_router_t + roff, T,
                                 e->E, e->H, e->k, forced, ids, w, e->d_z, e->d_xt, s);
    if (he != hipSuccess) return fail(EO_ERR_HIP, std::string("route: ") + hipGetErrorString(he));
    EOCHK(stage_done(e, s, "route", layer));
    EOCHK(do_plan(e, layer, ids, w, x, T, s));
    EOCHK(stage_done(e, s, "lookup and plan", layer));
    EOCHK(do_fill(e, s));
    EOCHK(stage_done(e, s, "fill", layer));
    EOCHK(do_ffn_device(e, layer, x, ids, w, s));
    EOCHK(stage_done(e, s, "expert FFN", layer));
    EOCHK(do_host(e, x, ids, w, s));
    EOCHK(stage_done(e, s, "host-execute", layer));
    EOCHK(do_combine(e, ids, y, x_res, s));
    return stage_done(e, s, "combine", layer);
}

// One token through all layers with the fused layer entry: per layer, one
// kernel applies the previous layer's result to the residual stream,
// normalises and computes the logits; the plan kernel selects the experts,
// then fill, GEMV and host execution as in moe_layer_impl. The previous
// layer's partial outputs are summed by the next entry (the last layer's by a
// final reduce into x_inout). The stream ping-pongs between two rows of d_r.
eo_status decode_one_token(eo_engine* e, uint16_t* x_inout, const int32_t* forced_ids,
                           hipStream_t s) {
    const int H = e->H, k = e->k, nparts = e->k + e->shared;
    const bool cap = e->cap_y && 1 <= e->cap_T;
    // EO_ENTRY_PLAN=0 keeps the entry and the plan in separate launches (tests compare them)
    const char* ep = std::getenv("EO_ENTRY_PLAN");
    const bool fuse_plan = !(ep && ep[0] == '0') &&
                           entry_plan_ok(1, k, e->E, H, e->C, e->act_bf16);
    const float* prev_host = nullptr;
    for (int l = 0; l < e->L; ++l) {
        TraceRange trace_range("eo.decode.layer");
        int32_t* ids = e->d_ids;
        float* w = e->d_w;
        EntryArgs a;
        a.r_in = l == 0 ? x_inout : e->d_r + (size_t)((l - 1) & 1) * H;
        a.r_out = e->d_r + (size_t)(l & 1) * H;
        a.parts = l > 0 ? e->d_yparts : nullptr;
        a.nparts = l > 0 ? nparts : 0;
        a.y_host = prev_host;
        a.y_out = (cap && l > 0) ? e->cap_y + (size_t)(l - 1) * e->cap_T * H : nullptr;
        a.u = (uint16_t*)e->d_u;
        a.Rt = e->d_router_t + (size_t)l * e->E * H;
        a.z = e->d_z;
        a.E = e->E;
        a.H = H;
        if (cap) {
            ids = e->cap_ids + (size_t)l * e->cap_T * k;
            w = e->cap_w + (size_t)l * e->cap_T * k;
        }
        PlanRoute rt{e->d_z, forced_ids ? forced_ids + (size_t)l * k : nullptr, ids, w};
        if (fuse_plan) {
            EOCHK(do_plan(e, l, ids, w, e->d_u, 1, s, rt, &a));
        } else {
            hipError_t he = launch_entry(a, s);
            if (he != hipSuccess)
                return fail(EO_ERR_HIP, std::string("layer entry: ") + hipGetErrorString(he));
            EOCHK(do_plan(e, l, ids, w, e->d_u, 1, s, rt));
        }
        EOCHK(stage_done(e, s, "layer entry and plan", l));
        if (cap)  // u is not changed by the plan
            HIPCHK(hipMemcpyAsync((uint8_t*)e->cap_x + (size_t)l * e->cap_T * H * 2, e->d_u,
                                  (size_t)H * 2, hipMemcpyDeviceToDevice, s));
        EOCHK(do_fill_gemv(e, l, ids, w, s));
        EOCHK(stage_done(e, s, "fill and expert GEMV", l));
        EOCHK(do_host(e, e->d_u, ids, w, s));
        EOCHK(stage_done(e, s, "host-execute", l));
        prev_host = e->host_staged ? e->h_yhost_dev : nullptr;
        // the plan is consumed here; its outputs are summed by the next entry
        e->plan_pending = false;
        e->plan_ready = false;
        e->host_staged = false;
    }
    float* y_last = cap ? e->cap_y + (size_t)(e->L - 1) * e->cap_T * H : nullptr;
    hipError_t he = launch_gemv_reduce(e->d_yparts, nparts, prev_host, H, y_last, x_inout, 1, s,
                                       e->d_r + (size_t)((e->L - 1) & 1) * H);
    if (he != hipSuccess) return fail(EO_ERR_HIP, std::string("combine: ") + hipGetErrorString(he));
    return stage_done(e, s, "final combine", e->L - 1);
}

eo_status reset_cache(eo_engine* e) {
    if (e->C > 0) {
        std::vector<int32_t> keys(e->C, -1);
        HIPCHK(hipMemcpy(e->d_slot_key, keys.data(), sizeof(int32_t) * e->C, hipMemcpyHostToDevice));
        HIPCHK(hipMemset(e->d_slot_stamp, 0, sizeof(int64_t) * e->C));
    }
    std::vector<int32_t> k2s((size_t)e->L * e->E, -1);
    HIPCHK(hipMemcpy(e->d_key2slot, k2s.data(), sizeof(int32_t) * k2s.size(), hipMemcpyHostToDevice));
    DevState st{};
    HIPCHK(hipMemcpy(&st, e->d_state, sizeof(DevState), hipMemcpyDeviceToHost));
    st.clock = 0;
    st.credit = 0;
    st.bp = (int32_t)e->bp;
    st.bh = (int32_t)e->bh;
    st.frozen = 0;
    HIPCHK(hipMemcpy(e->d_state, &st, sizeof(DevState), hipMemcpyHostToDevice));
    return EO_OK;
}

void destroy_all(eo_engine* e) {
    if (!e) return;
    (void)hipSetDevice(e->cfg.device);
    (void)hipDeviceSynchronize();
    for (auto p : e->pool)
        if (p) (void)hipHostFree(p);
    auto fr = [](void* p) { if (p) (void)hipFree(p); };
    auto fh = [](void* p) { if (p) (void)hipHostFree(p); };
    fr(e->d_slots); fr(e->d_shared); fr(e->d_router); fr(e->d_router_t); fr(e->d_xt);
    fr(e->d_slot_key); fr(e->d_slot_stamp);
    fr(e->d_key2slot); fr(e->d_state); fr(e->d_fill_counters); fr(e->d_plan); fr(e->d_ids); fr(e->d_w); fr(e->d_z);
    fr(e->d_y); fr(e->d_u); fr(e->d_r); fr(e->d_hgemv); fr(e->d_yparts); fr(e->d_yhost);
    fr(e->pb.counts); fr(e->pb.offsets); fr(e->pb.tile_off); fr(e->pb.perm_pair);
    fr(e->pb.chunk_cnt); fr(e->d_hbuf); fr(e->d_opairs);
    fr(e->d_staging[0]); fr(e->d_staging[1]); fr((void*)e->d_gbase);
    fh(e->h_plan); fh(e->h_ids); fh(e->h_w); fh(e->h_x); fh(e->h_yhost);
    if (e->copy_stream) (void)hipStreamDestroy(e->copy_stream);
    for (hipEvent_t ev : {e->ev_fill, e->ev_copy[0], e->ev_copy[1], e->ev_comp[0], e->ev_comp[1],
                          e->ev_start})
        if (ev) (void)hipEventDestroy(ev);
    for (auto* v : {&e->gemv_ev, &e->gemm_ev, &e->fill_ev, &e->copy_ev, &e->comp_ev, &e->free_ev})
        for (auto& p : *v)
            for (hipEvent_t ev : p.ev) (void)hipEventDestroy(ev);
    if (e->tp) threadpool_destroy(e->tp);
    delete e;
}

template <typename T>
eo_status dmalloc(T** p, size_t bytes) {
    if (bytes == 0) bytes = 16;
    hipError_t he = hipMalloc((void**)p, bytes);
    if (he != hipSuccess) {
        *p = nullptr;
        (void)hipGetLastError();
        return fail(he == hipErrorOutOfMemory ? EO_ERR_OOM : EO_ERR_HIP,
                    std::string("hipMalloc: ") + hipGetErrorString(he));
    }
    return EO_OK;
}

template <typename T>
eo_status hmalloc(T** p, size_t bytes, unsigned flags) {
    if (bytes == 0) bytes = 16;
    hipError_t he = hipHostMalloc((void**)p, bytes, flags);
    if (he != hipSuccess) {
        *p = nullptr;
        (void)hipGetLastError();
        return fail(EO_ERR_OOM, std::string("hipHostMalloc: ") + hipGetErrorString(he));
    }
    return EO_OK;
}

eo_status create_impl(const eo_config* cfg, eo_engine* e) {
    e->cfg = *cfg;
    e->L = cfg->layers;
    e->E = cfg->experts;
    e->k = cfg->top_k;
    e->H = cfg->hidden;
    e->I = cfg->inter;
    e->shared = cfg->shared_experts;
    e->fmt = cfg->wfmt;
    e->act_bf16 = cfg->act_bf16;
    e->C = cfg->cache_slots;
    e->act_size = e->act_bf16 ? 2 : 4;
    e->lay = layout_of(e->H, e->I, e->fmt);
    e->S = e->lay.bytes;
    e->S_pad = round_up(e->S, kPoolAlign);
    HIPCHK(hipSetDevice(cfg->device));

    e->pool.assign(e->L, nullptr);
    e->pool_dev.assign(e->L, nullptr);
    for (int l = 0; l < e->L; ++l) {
        if (hmalloc(&e->pool[l], e->E * e->S_pad, hipHostMallocDefault) != EO_OK)
            return fail(EO_ERR_OOM, g_err + " (pool layer " + std::to_string(l) + " of " +
                                        std::to_string(e->L) + ", " +
                                        std::to_string((double)l * e->E * e->S_pad / 1e9) +
                                        " GB already pinned, " +
                                        std::to_string((double)e->E * e->S_pad / 1e9) +
                                        " GB per layer)");
        HIPCHK(hipHostGetDevicePointer((void**)&e->pool_dev[l], e->pool[l], 0));
    }
    EOCHK(dmalloc(&e->d_slots, e->C * e->S_pad));
    if (e->shared) {
        EOCHK(dmalloc(&e->d_shared, (size_t)e->L * e->S_pad));
        HIPCHK(hipMemset(e->d_shared, 0, (size_t)e->L * e->S_pad));
    }
    EOCHK(dmalloc(&e->d_router, sizeof(float) * e->L * e->E * e->H));
    HIPCHK(hipMemset(e->d_router, 0, sizeof(float) * e->L * e->E * e->H));
    EOCHK(dmalloc(&e->d_router_t, sizeof(float) * e->L * e->E * e->H));
    HIPCHK(hipMemset(e->d_router_t, 0, sizeof(float) * e->L * e->E * e->H));
    if (e->act_bf16 && cfg->max_tokens >= 32 && e->H % 512 == 0)
        EOCHK(dmalloc(&e->d_xt, sizeof(uint16_t) * (size_t)cfg->max_tokens * e->H));
    EOCHK(dmalloc(&e->d_slot_key, sizeof(int32_t) * e->C));
    EOCHK(dmalloc(&e->d_slot_stamp, sizeof(int64_t) * e->C));
    EOCHK(dmalloc(&e->d_key2slot, sizeof(int32_t) * e->L * e->E));
    EOCHK(dmalloc(&e->d_state, sizeof(DevState)));
    HIPCHK(hipMemset(e->d_state, 0, sizeof(DevState)));
    EOCHK(dmalloc(&e->d_fill_counters, fill_gemv_counter_bytes()));
    HIPCHK(hipMemset(e->d_fill_counters, 0, fill_gemv_counter_bytes()));
    EOCHK(dmalloc(&e->d_plan, sizeof(DevPlan)));
    HIPCHK(hipMemset(e->d_plan, 0, sizeof(DevPlan)));
    const unsigned mflags = hipHostMallocMapped | hipHostMallocCoherent;
    const int Tm = cfg->max_tokens;
    EOCHK(hmalloc(&e->h_plan, sizeof(DevPlan), mflags));
    std::memset(e->h_plan, 0, sizeof(DevPlan));
    EOCHK(hmalloc(&e->h_ids, sizeof(int32_t) * Tm * e->k, mflags));
    EOCHK(hmalloc(&e->h_w, sizeof(float) * Tm * e->k, mflags));
    EOCHK(hmalloc(&e->h_x, (size_t)e->act_size * Tm * e->H, mflags));
    HIPCHK(hipHostGetDevicePointer((void**)&e->h_plan_dev, e->h_plan, 0));
    HIPCHK(hipHostGetDevicePointer((void**)&e->h_ids_dev, e->h_ids, 0));
    HIPCHK(hipHostGetDevicePointer((void**)&e->h_w_dev, e->h_w, 0));
    HIPCHK(hipHostGetDevicePointer((void**)&e->h_x_dev, e->h_x, 0));
    EOCHK(dmalloc(&e->d_ids, sizeof(int32_t) * Tm * e->k));
    EOCHK(dmalloc(&e->d_w, sizeof(float) * Tm * e->k));
    EOCHK(dmalloc(&e->d_z, sizeof(float) * Tm * e->E));
    EOCHK(dmalloc(&e->d_y, sizeof(float) * Tm * e->H));
    EOCHK(dmalloc(&e->d_u, (size_t)e->act_size * Tm * e->H));
    EOCHK(dmalloc(&e->d_r, sizeof(uint16_t) * 2 * e->H));
    EOCHK(dmalloc(&e->d_hgemv, sizeof(float) * (e->k + 1) * e->I));
    EOCHK(dmalloc(&e->d_yparts, sizeof(float) * (e->k + 1) * e->H));
    EOCHK(dmalloc(&e->d_yhost, sizeof(float) * Tm * e->H));
    EOCHK(hmalloc(&e->h_yhost, sizeof(float) * Tm * e->H, mflags));
    HIPCHK(hipHostGetDevicePointer((void**)&e->h_yhost_dev, e->h_yhost, 0));
    HIPCHK(hipStreamCreateWithFlags(&e->copy_stream, hipStreamNonBlocking));
    HIPCHK(hipEventCreateWithFlags(&e->ev_fill, hipEventDisableTiming));
    HIPCHK(hipEventCreateWithFlags(&e->ev_start, hipEventDisableTiming));
    for (int i = 0; i < 2; ++i) {
        HIPCHK(hipEventCreateWithFlags(&e->ev_copy[i], hipEventDisableTiming));
        HIPCHK(hipEventCreateWithFlags(&e->ev_comp[i], hipEventDisableTiming));
    }
    int nt = cfg->host_threads;
    // leave one hardware thread for the engine's own orchestration and the runtime
    if (nt <= 0) nt = std::max(1, std::min(15, (int)std::thread::hardware_concurrency() - 1));
    e->tp = threadpool_create(nt);
    if (const char* v = std::getenv("EO_GEMV_FAST")) e->gemv_fast = std::atoi(v) != 0;
    if (const char* v = std::getenv("EO_FILL_SDMA")) e->fill_sdma = std::atoi(v) != 0;
    if (const char* v = std::getenv("EO_FILL_GEMV")) e->fill_gemv = std::atoi(v) != 0;
    if (const char* v = std::getenv("EO_TEST_FILL_WAIT_TICKS")) e->fill_wait_ticks = std::strtoull(v, nullptr, 10);
    if (const char* v = std::getenv("EO_FUSED_ENTRY")) e->fused_entry = std::atoi(v) != 0;
    if (const char* v = std::getenv("EO_DEBUG_SYNC")) e->debug_sync = std::atoi(v) != 0;
    if (const char* v = std::getenv("EO_LOG")) e->log_level = std::atoi(v);
    if (e->log_level >= 1)
        std::fprintf(stderr,
                     "eo: engine on device %d: %d layers x %d experts (top-%d, H %d, I %d, format %d, "
                     "shared %d), expert %llu bytes (%llu padded); pool %.2f GB pinned, cache %lld "
                     "slots (%.2f GB), max tokens %d, host threads %d\n",
                     cfg->device, e->L, e->E, e->k, e->H, e->I, e->fmt, e->shared,
                     (unsigned long long)e->S, (unsigned long long)e->S_pad,
                     (double)e->L * e->E * e->S_pad / 1e9, (long long)e->C,
                     (double)e->C * e->S_pad / 1e9, cfg->max_tokens, threadpool_size(e->tp));
    e->bp = e->bh = 1;
    EOCHK(scratch_on_device(cfg->device, &e->scratch));
    EOCHK(reset_cache(e));
    HIPCHK(hipDeviceSynchronize());
    return EO_OK;
}

}  // namespace

// ====================================================================== C ABI
extern "C" {

const char* eo_last_error(void) { return g_err.c_str(); }

uint64_t eo_expert_bytes(int32_t hidden, int32_t inter, int32_t wfmt) {
    if (hidden <= 0 || inter <= 0 || wfmt < 0 || wfmt > 4) return 0;
    return layout_of(hidden, inter, wfmt).bytes;
}

eo_status eo_create(const eo_config* cfg, eo_engine** out) {
    if (!cfg || !out) return fail(EO_ERR_INVALID_ARG, "null argument");
    *out = nullptr;
    const eo_config& c = *cfg;
    if (c.layers < 1 || c.experts < 1 || c.experts > EO_MAX_EXPERTS || c.top_k < 1 ||
        c.top_k > kMaxK || c.top_k > c.experts)
        return fail(EO_ERR_INVALID_ARG, "layers >= 1, 1 <= experts <= 1024, 1 <= top_k <= min(16, experts)");
    if (c.hidden < 128 || c.hidden % 128 || c.inter < 64 || c.inter % 64)
        return fail(EO_ERR_INVALID_ARG, "hidden must be a multiple of 128, inter a multiple of 64");
    if (c.shared_experts != 0 && c.shared_experts != 1)
        return fail(EO_ERR_INVALID_ARG, "shared_experts must be 0 or 1");
    if (c.wfmt < EO_W_FP32 || c.wfmt > EO_W_FP8) return fail(EO_ERR_INVALID_ARG, "unknown wfmt");
    if ((c.wfmt == EO_W_FP32) != (c.act_bf16 == 0))
        return fail(EO_ERR_UNSUPPORTED, "fp32 weights need fp32 activations; other formats need bf16 activations");
    if (c.cache_slots < 0 || c.cache_slots > plan_max_slots())
        return fail(EO_ERR_INVALID_ARG, "cache_slots out of range [0, 8192]");
    if ((int64_t)c.layers * c.experts >= (1 << 24))
        return fail(EO_ERR_INVALID_ARG, "layers * experts must be below 2^24");
    if (c.max_tokens < 1) return fail(EO_ERR_INVALID_ARG, "max_tokens >= 1");
    int ndev = 0;
    if (hipGetDeviceCount(&ndev) != hipSuccess || c.device < 0 || c.device >= ndev)
        return fail(EO_ERR_INVALID_ARG, "no such HIP device");
    eo_engine* e = new eo_engine();
    eo_status s = create_impl(cfg, e);
    if (s != EO_OK) {
        std::string msg = g_err;
        destroy_all(e);
        g_err = msg;
        return s;
    }
    *out = e;
    return EO_OK;
}

eo_status eo_destroy(eo_engine* e) {
    destroy_all(e);
    return EO_OK;
}

eo_status eo_pool_expert(eo_engine* e, int32_t layer, int32_t expert, void** host_ptr,
                         uint64_t* bytes) {
    EOCHK(check_layer(e, layer));
    if (expert < 0 || expert >= e->E || !host_ptr) return fail(EO_ERR_INVALID_ARG, "bad expert");
    *host_ptr = e->pool[layer] + (uint64_t)expert * e->S_pad;
    if (bytes) *bytes = e->S;
    return EO_OK;
}

eo_status eo_set_shared_expert(eo_engine* e, int32_t layer, const void* host_block, uint64_t bytes) {
    EOCHK(check_layer(e, layer));
    if (!e->shared) return fail(EO_ERR_STATE, "engine has no shared expert");
    if (!host_block || bytes != e->S) return fail(EO_ERR_INVALID_ARG, "block size mismatch");
    HIPCHK(hipSetDevice(e->cfg.device));
    HIPCHK(hipMemcpy(e->d_shared + (uint64_t)layer * e->S_pad, host_block, bytes, hipMemcpyHostToDevice));
    return EO_OK;
}

eo_status eo_set_router(eo_engine* e, int32_t layer, const float* host_w) {
    EOCHK(check_layer(e, layer));
    if (!host_w) return fail(EO_ERR_INVALID_ARG, "null router");
    HIPCHK(hipSetDevice(e->cfg.device));
    HIPCHK(hipMemcpy(e->d_router + (size_t)layer * e->E * e->H, host_w,
                     sizeof(float) * e->E * e->H, hipMemcpyHostToDevice));
    // chain-interleaved copy for the many-token router kernel (which reads it only
    // when H % 512 == 0); shapes its layout does not cover are left zero
    std::vector<float> rt((size_t)e->E * e->H);
    if (router_chain_layout(host_w, e->E, e->H, rt.data()))
        HIPCHK(hipMemcpy(e->d_router_t + (size_t)layer * e->E * e->H, rt.data(),
                         sizeof(float) * e->E * e->H, hipMemcpyHostToDevice));
    return EO_OK;
}

eo_status eo_set_bandwidth(eo_engine* e, uint32_t bp_mbps, uint32_t bh_mbps) {
    if (!e) return fail(EO_ERR_INVALID_ARG, "null engine");
    if (bp_mbps == 0 || bh_mbps == 0 || bp_mbps > 0x7FFFFFFFu || bh_mbps > 0x7FFFFFFFu)
        return fail(EO_ERR_INVALID_ARG, "bandwidths must be in [1, 2^31)");
    HIPCHK(hipSetDevice(e->cfg.device));
    HIPCHK(hipDeviceSynchronize());
    DevState st{};
    HIPCHK(hipMemcpy(&st, e->d_state, sizeof(DevState), hipMemcpyDeviceToHost));
    st.bp = (int32_t)bp_mbps;
    st.bh = (int32_t)bh_mbps;
    if (st.credit > (int64_t)bh_mbps - 1) st.credit = (int64_t)bh_mbps - 1;
    HIPCHK(hipMemcpy(e->d_state, &st, sizeof(DevState), hipMemcpyHostToDevice));
    e->bp = bp_mbps;
    e->bh = bh_mbps;
    return EO_OK;
}

// B_P and B_H probes. keep_cache: copy into a scratch buffer and keep the
// cache, clock and (clamped) credit; else copy into slot 0 and reset the cache.
static eo_status measure_impl(eo_engine* e, bool keep_cache, uint32_t* bp_out, uint32_t* bh_out) {
    if (!e) return fail(EO_ERR_INVALID_ARG, "null engine");
    if (keep_cache && e->plan_pending)
        return fail(EO_ERR_STATE, "a lookup plan is pending: re-measure between steps");
    HIPCHK(hipSetDevice(e->cfg.device));
    HIPCHK(hipDeviceSynchronize());
    uint8_t* dst = e->d_slots;
    uint8_t* tmp = nullptr;
    if (e->C == 0 || keep_cache) {
        EOCHK(dmalloc(&tmp, e->S));
        dst = tmp;
    }
    const int reps = 9, warm = 2;
    const int n_exp = e->L * e->E;
    hipEvent_t a, b;
    HIPCHK(hipEventCreate(&a));
    HIPCHK(hipEventCreate(&b));
    std::vector<double> tp, th;
    for (int r = 0; r < reps + warm; ++r) {
        int id = (r * 7919) % n_exp;
        const uint64_t off = (uint64_t)(id % e->E) * e->S_pad;
        HIPCHK(hipEventRecord(a, e->copy_stream));
        if (e->fill_sdma)
            HIPCHK(hipMemcpyAsync(dst, e->pool[id / e->E] + off, e->S, hipMemcpyHostToDevice,
                                  e->copy_stream));
        else  // the way fills are made: the fill kernel's copy over the pool's mapping
            HIPCHK(launch_copy_expert(e->pool_dev[id / e->E] + off, dst, e->S, e->copy_stream));
        HIPCHK(hipEventRecord(b, e->copy_stream));
        HIPCHK(hipEventSynchronize(b));
        float ms = 0;
        HIPCHK(hipEventElapsedTime(&ms, a, b));
        if (r >= warm) tp.push_back(ms * 1e-3);
    }
    (void)hipEventDestroy(a);
    (void)hipEventDestroy(b);
    if (tmp) (void)hipFree(tmp);
    // host routine over one expert at T = 1
    // x = 0.01 (as stored in the activation dtype: bf16 0x3C24 = 0.010009765625)
    std::vector<float> x(e->H, e->act_bf16 ? 0.010009765625f : 0.01f), y(e->H);
    std::vector<uint16_t> xb(e->H, 0x3C24);
    std::vector<const uint8_t*> table(e->E, nullptr);
    int32_t ids[kMaxK];
    float w[kMaxK];
    for (int j = 0; j < e->k; ++j) {
        ids[j] = j;
        w[j] = j == 0 ? 1.0f : 0.0f;
    }
    for (int r = 0; r < reps + warm; ++r) {
        int id = (r * 104729 + 17) % n_exp;
        const int le = id % e->E;
        std::fill(table.begin(), table.end(), nullptr);
        // route the single token to expert `le` (slot 0), other slots to non-host experts
        ids[0] = le;
        for (int j = 1; j < e->k; ++j) ids[j] = (le + j) % e->E;
        table[le] = e->pool[id / e->E] + (uint64_t)le * e->S_pad;
        HostJob jb;
        jb.fmt = e->fmt;
        jb.lay = e->lay;
        jb.H = e->H;
        jb.I = e->I;
        jb.T = 1;
        jb.k = e->k;
        jb.x = x.data();
        jb.xb = e->act_bf16 ? xb.data() : nullptr;
        jb.ids = ids;
        jb.w = w;
        jb.experts = table.data();
        std::fill(y.begin(), y.end(), 0.0f);
        jb.y = y.data();
        auto t0 = std::chrono::steady_clock::now();
        host_ffn(e->tp, jb, e->host_scratch);
        double dt = std::chrono::duration<double>(std::chrono::steady_clock::now() - t0).count();
        if (r >= warm) th.push_back(dt);
    }
    std::sort(tp.begin(), tp.end());
    std::sort(th.begin(), th.end());
    double bp = (double)e->S / tp[tp.size() / 2] / 1e6, bh = (double)e->S / th[th.size() / 2] / 1e6;
    uint32_t bpi = (uint32_t)std::max(1.0, std::min(2e9, bp));
    uint32_t bhi = (uint32_t)std::max(1.0, std::min(2e9, bh));
    if (keep_cache) {
        EOCHK(eo_set_bandwidth(e, bpi, bhi));
    } else {
        e->bp = bpi;
        e->bh = bhi;
        EOCHK(reset_cache(e));
    }
    if (bp_out) *bp_out = bpi;
    if (bh_out) *bh_out = bhi;
    return EO_OK;
}

eo_status eo_measure_bandwidth(eo_engine* e, uint32_t* bp_out, uint32_t* bh_out) {
    TraceRange trace_range("eo.measure_bandwidth");
    return measure_impl(e, false, bp_out, bh_out);
}

eo_status eo_remeasure_bandwidth(eo_engine* e, uint32_t* bp_out, uint32_t* bh_out) {
    TraceRange trace_range("eo.remeasure_bandwidth");
    return measure_impl(e, true, bp_out, bh_out);
}

eo_status eo_route(eo_engine* e, int32_t layer, const void* x, int32_t T, const int32_t* forced_ids,
                   int32_t* ids, float* w, void* stream) {
    EOCHK(check_layer(e, layer));
    EOCHK(check_T(e, T));
    if (!x || !ids || !w) return fail(EO_ERR_INVALID_ARG, "null pointer");
    HIPCHK(hipSetDevice(e->cfg.device));
    const size_t roff = (size_t)layer * e->E * e->H;
    hipError_t he = launch_route(x, e->act_bf16, e->d_router + roff, e->d_router_t + roff, T, e->E,
                                 e->H, e->k, forced_ids, ids, w, e->d_z, e->d_xt,
                                 (hipStream_t)stream);
    if (he != hipSuccess) return fail(EO_ERR_HIP, std::string("route: ") + hipGetErrorString(he));
    return EO_OK;
}

eo_status eo_route_noalloc(eo_engine* e, int32_t layer, const void* x, int32_t T,
                           const int32_t* forced_ids, int32_t* ids, float* w, void* stream) {
    EOCHK(check_layer(e, layer));
    EOCHK(check_T(e, T));
    if (!x || !ids || !w) return fail(EO_ERR_INVALID_ARG, "null pointer");
    if (!e->scratch) return fail(EO_ERR_STATE, "no scratch address on this engine's device");
    HIPCHK(hipSetDevice(e->cfg.device));
    // logits [T, E] fp32 at the start, then (chain-interleaved kernel) x as
    // [T][H/512][64][8] bf16 at the next 256-byte boundary
    const bool chains = route_chains_ok(T, e->E, e->H, e->act_bf16);
    const uint64_t z_bytes = round_up((uint64_t)T * e->E * 4, 256);
    const uint64_t need = z_bytes + (chains ? (uint64_t)T * e->H * 2 : 0);
    if (need > kScratchBytes)
        return fail(EO_ERR_INVALID_ARG, "T * (4 E + 2 H) bytes exceed the 16 MiB scratch of eo_route_noalloc");
    const size_t roff = (size_t)layer * e->E * e->H;
    hipError_t he = launch_route(x, e->act_bf16, e->d_router + roff, e->d_router_t + roff, T, e->E,
                                 e->H, e->k, forced_ids, ids, w, (float*)e->scratch,
                                 chains ? (uint16_t*)(e->scratch + z_bytes) : nullptr,
                                 (hipStream_t)stream);
    if (he != hipSuccess) return fail(EO_ERR_HIP, std::string("route: ") + hipGetErrorString(he));
    return EO_OK;
}

eo_status eo_lookup_plan(eo_engine* e, int32_t layer, const int32_t* ids, int32_t T, void* stream) {
    EOCHK(check_layer(e, layer));
    EOCHK(check_T(e, T));
    if (!ids) return fail(EO_ERR_INVALID_ARG, "null ids");
    HIPCHK(hipSetDevice(e->cfg.device));
    return do_plan(e, layer, ids, nullptr, nullptr, T, (hipStream_t)stream);
}

eo_status eo_fill(eo_engine* e, void* stream) {
    if (!e) return fail(EO_ERR_INVALID_ARG, "null engine");
    HIPCHK(hipSetDevice(e->cfg.device));
    return do_fill(e, (hipStream_t)stream);
}

eo_status eo_host_execute(eo_engine* e, const void* x, const int32_t* ids, const float* w,
                          void* stream) {
    if (!e || !x || !ids || !w) return fail(EO_ERR_INVALID_ARG, "null argument");
    HIPCHK(hipSetDevice(e->cfg.device));
    return do_host(e, x, ids, w, (hipStream_t)stream);
}

eo_status eo_expert_ffn_combine(eo_engine* e, int32_t layer, const void* x, const int32_t* ids,
                                const float* w, float* y, void* stream) {
    EOCHK(check_layer(e, layer));
    if (!x || !ids || !w || !y) return fail(EO_ERR_INVALID_ARG, "null argument");
    EOCHK(wait_plan(e));
    if (layer != e->plan_layer) return fail(EO_ERR_STATE, "layer differs from the pending plan's");
    if (!aligned16(x) || !aligned16(y)) return fail(EO_ERR_INVALID_ARG, "x and y must be 16-byte aligned");
    HIPCHK(hipSetDevice(e->cfg.device));
    hipStream_t s = (hipStream_t)stream;
    EOCHK(do_ffn_device(e, layer, x, ids, w, s));
    return do_combine(e, ids, y, nullptr, s);
}

eo_status eo_moe_layer(eo_engine* e, int32_t layer, const void* x, float* y, int32_t T,
                       const int32_t* forced_ids, void* stream) {
    TraceRange trace_range("eo.moe_layer");
    EOCHK(check_layer(e, layer));
    EOCHK(check_T(e, T));
    if (!x || !y) return fail(EO_ERR_INVALID_ARG, "null argument");
    if (!aligned16(x) || !aligned16(y)) return fail(EO_ERR_INVALID_ARG, "x and y must be 16-byte aligned");
    HIPCHK(hipSetDevice(e->cfg.device));
    EOCHK(moe_layer_impl(e, layer, x, y, T, forced_ids, e->d_ids, e->d_w, nullptr,
                         (hipStream_t)stream));
    if (e->timing) EOCHK(harvest_times(e));
    return EO_OK;
}

eo_status eo_decode_step(eo_engine* e, void* x_inout, int32_t T, const int32_t* forced_ids,
                         void* stream) {
    TraceRange trace_range("eo.decode_step");
    if (!e || !x_inout) return fail(EO_ERR_INVALID_ARG, "null argument");
    EOCHK(check_T(e, T));
    if (!aligned16(x_inout)) return fail(EO_ERR_INVALID_ARG, "x must be 16-byte aligned");
    HIPCHK(hipSetDevice(e->cfg.device));
    hipStream_t s = (hipStream_t)stream;
    if (T == 1 && e->fused_entry && entry_ok(e->E, e->H, e->act_bf16)) {
        EOCHK(decode_one_token(e, (uint16_t*)x_inout, forced_ids, s));
        if (e->timing) EOCHK(harvest_times(e));
        return EO_OK;
    }
    const size_t xb = (size_t)T * e->H * e->act_size;
    const bool cap = e->cap_y && T <= e->cap_T;
    for (int l = 0; l < e->L; ++l) {
        const int32_t* forced = forced_ids ? forced_ids + (size_t)l * T * e->k : nullptr;
        int32_t* ids = e->d_ids;
        float* w = e->d_w;
        float* y = e->d_y;
        hipError_t he = launch_rmsnorm(x_inout, e->d_u, T, e->H, e->act_bf16, s);
        if (he != hipSuccess) return fail(EO_ERR_HIP, std::string("rmsnorm: ") + hipGetErrorString(he));
        if (cap) {
            HIPCHK(hipMemcpyAsync((uint8_t*)e->cap_x + (size_t)l * e->cap_T * e->H * e->act_size,
                                  e->d_u, xb, hipMemcpyDeviceToDevice, s));
            ids = e->cap_ids + (size_t)l * e->cap_T * e->k;
            w = e->cap_w + (size_t)l * e->cap_T * e->k;
            y = e->cap_y + (size_t)l * e->cap_T * e->H;
        }
        EOCHK(moe_layer_impl(e, l, e->d_u, y, T, forced, ids, w, x_inout, s));
    }
    if (e->timing) EOCHK(harvest_times(e));
    return EO_OK;
}

eo_status eo_prefill(eo_engine* e, void* x_inout, int32_t T, int32_t flags, void* stream) {
    TraceRange trace_range("eo.prefill");
    if (!e || !x_inout) return fail(EO_ERR_INVALID_ARG, "null argument");
    EOCHK(check_T(e, T));
    if (!aligned16(x_inout)) return fail(EO_ERR_INVALID_ARG, "x must be 16-byte aligned");
    if (flags & ~(EO_PREFILL_DOUBLE_BUFFER | EO_PREFILL_SKIP_RESIDENT))
        return fail(EO_ERR_INVALID_ARG, "unknown prefill flags");
    const bool double_buffer = flags & EO_PREFILL_DOUBLE_BUFFER;
    const bool skip = (flags & EO_PREFILL_SKIP_RESIDENT) && e->C > 0;
    hipStream_t s = (hipStream_t)stream;
    HIPCHK(hipSetDevice(e->cfg.device));
    const uint64_t layer_bytes = (uint64_t)e->E * e->S_pad;
    for (int i = 0; i < 2; ++i)
        if (!e->d_staging[i]) EOCHK(dmalloc(&e->d_staging[i], layer_bytes));
    EOCHK(ensure_gemm(e, T, s));
    const size_t xb = (size_t)T * e->H * e->act_size;
    const bool cap = e->cap_y && T <= e->cap_T;
    // Resident-aware streaming: experts resident in the cache are read from
    // their slots, only the others are streamed; prefill does not change the
    // cache, so the residency read once here holds for the whole call.
    std::vector<int32_t> k2s;
    if (skip) {
        HIPCHK(hipStreamSynchronize(s));
        k2s.resize((size_t)e->L * e->E);
        HIPCHK(hipMemcpy(k2s.data(), e->d_key2slot, sizeof(int32_t) * k2s.size(), hipMemcpyDeviceToHost));
        std::vector<const uint8_t*> gb(k2s.size());
        for (int l = 0; l < e->L; ++l)
            for (int g = 0; g < e->E; ++g) {
                const int32_t sl = k2s[(size_t)l * e->E + g];
                gb[(size_t)l * e->E + g] = sl >= 0 ? e->d_slots + (uint64_t)sl * e->S_pad
                                                   : e->d_staging[l & 1] + (uint64_t)g * e->S_pad;
            }
        if (e->gbase_n < gb.size()) {
            if (e->d_gbase) (void)hipFree(e->d_gbase);
            e->d_gbase = nullptr;
            e->gbase_n = 0;
            EOCHK(dmalloc(&e->d_gbase, sizeof(const uint8_t*) * gb.size()));
            e->gbase_n = gb.size();
        }
        HIPCHK(hipMemcpy(e->d_gbase, gb.data(), sizeof(const uint8_t*) * gb.size(), hipMemcpyHostToDevice));
    }
    int64_t streamed = 0;
    // layer l's experts into staging buffer `buf` on the copy stream (runs of
    // consecutive non-resident experts when skipping)
    auto copy_layer_bytes = [&](int l, int buf) -> eo_status {
        if (!skip) {
            HIPCHK(hipMemcpyAsync(e->d_staging[buf], e->pool[l], layer_bytes, hipMemcpyHostToDevice,
                                  e->copy_stream));
            streamed += (int64_t)layer_bytes;
            return EO_OK;
        }
        for (int g = 0; g < e->E;) {
            if (k2s[(size_t)l * e->E + g] >= 0) {
                ++g;
                continue;
            }
            int g1 = g;
            while (g1 < e->E && k2s[(size_t)l * e->E + g1] < 0) ++g1;
            const uint64_t off = (uint64_t)g * e->S_pad, n = (uint64_t)(g1 - g) * e->S_pad;
            HIPCHK(hipMemcpyAsync(e->d_staging[buf] + off, e->pool[l] + off, n, hipMemcpyHostToDevice,
                                  e->copy_stream));
            streamed += (int64_t)n;
            g = g1;
        }
        return EO_OK;
    };
    // the same between two timing events on the copy stream when timing is on
    auto copy_layer = [&](int l, int buf) -> eo_status {
        TimedSet ts{};
        if (e->timing) {
            EOCHK(get_set(e, &ts));
            HIPCHK(hipEventRecord(ts.ev[0], e->copy_stream));
        }
        EOCHK(copy_layer_bytes(l, buf));
        if (e->timing) {
            HIPCHK(hipEventRecord(ts.ev[1], e->copy_stream));
            e->copy_ev.push_back(ts);
        }
        return EO_OK;
    };
    // the first copy must not overwrite staging still read by earlier work on s
    HIPCHK(hipEventRecord(e->ev_start, s));
    HIPCHK(hipStreamWaitEvent(e->copy_stream, e->ev_start, 0));
    EOCHK(copy_layer(0, 0));
    HIPCHK(hipEventRecord(e->ev_copy[0], e->copy_stream));
    for (int l = 0; l < e->L; ++l) {
        TraceRange trace_range("eo.prefill.layer");
        const int b = l & 1, nb = b ^ 1;
        HIPCHK(hipStreamWaitEvent(s, e->ev_copy[b], 0));
        TimedSet tc{};  // this layer's kernels, once its weights are in
        if (e->timing) {
            EOCHK(get_set(e, &tc));
            HIPCHK(hipEventRecord(tc.ev[0], s));
        }
        if (double_buffer && l + 1 < e->L) {
            // buffer nb was last read by layer l-1's compute
            if (l >= 1) HIPCHK(hipStreamWaitEvent(e->copy_stream, e->ev_comp[nb], 0));
            EOCHK(copy_layer(l + 1, nb));
            HIPCHK(hipEventRecord(e->ev_copy[nb], e->copy_stream));
        }
        int32_t* ids = e->d_ids;
        float* w = e->d_w;
        float* y = nullptr;
        hipError_t he = launch_rmsnorm(x_inout, e->d_u, T, e->H, e->act_bf16, s);
        if (he != hipSuccess) return fail(EO_ERR_HIP, std::string("rmsnorm: ") + hipGetErrorString(he));
        if (cap) {
            HIPCHK(hipMemcpyAsync((uint8_t*)e->cap_x + (size_t)l * e->cap_T * e->H * e->act_size,
                                  e->d_u, xb, hipMemcpyDeviceToDevice, s));
            ids = e->cap_ids + (size_t)l * e->cap_T * e->k;
            w = e->cap_w + (size_t)l * e->cap_T * e->k;
            y = e->cap_y + (size_t)l * e->cap_T * e->H;
        }
        const size_t roff = (size_t)l * e->E * e->H;
        he = launch_route(e->d_u, e->act_bf16, e->d_router + roff, e->d_router_t + roff, T, e->E,
                          e->H, e->k, nullptr, ids, w, e->d_z, e->d_xt, s);
        if (he == hipSuccess)
            he = launch_permute(ids, nullptr, 1, T, e->k, e->E, e->shared, e->pb, s);
        TimedSet ts{};
        if (e->timing) EOCHK(get_set(e, &ts));
        hipEvent_t none[4] = {nullptr, nullptr, nullptr, nullptr};
        if (he == hipSuccess) {
            GroupW gw;
            gw.slots = e->d_staging[b];
            gw.e2slot = nullptr;
            gw.stride = e->S_pad;
            gw.shared_w = e->shared ? e->d_shared + (uint64_t)l * e->S_pad : nullptr;
            gw.gbase = skip ? e->d_gbase + (size_t)l * e->E : nullptr;
            he = launch_ffn_gemm(e->fmt, e->lay, gw, e->E, e->shared, e->H, e->I, T * e->k + T,
                                 e->pb.offsets, e->pb.tile_off, e->d_u, e->d_hbuf,
                                 e->pb.perm_pair, ids, w, e->k, T, e->d_opairs, s,
                                 e->timing ? ts.ev : none);
        }
        if (e->timing) e->gemm_ev.push_back(ts);
        if (he == hipSuccess)
            he = launch_combine(e->d_opairs, ids, nullptr, 1, e->shared, nullptr, T, e->k, e->H, y,
                                x_inout, e->act_bf16, s, e->E);
        if (he != hipSuccess) return fail(EO_ERR_HIP, std::string("prefill layer: ") + hipGetErrorString(he));
        EOCHK(stage_done(e, s, "prefill layer (norm, route, permute, grouped FFN, combine)", l));
        if (e->timing) {
            HIPCHK(hipEventRecord(tc.ev[1], s));
            e->comp_ev.push_back(tc);
        }
        HIPCHK(hipEventRecord(e->ev_comp[b], s));
        if (!double_buffer && l + 1 < e->L) {
            HIPCHK(hipStreamWaitEvent(e->copy_stream, e->ev_comp[b], 0));
            EOCHK(copy_layer(l + 1, nb));
            HIPCHK(hipEventRecord(e->ev_copy[nb], e->copy_stream));
        }
    }
    e->stats.prefill_layers += e->L;
    e->stats.device_expert_bytes += (int64_t)e->L * (e->E + e->shared) * (int64_t)e->S;
    e->stats.pcie_bytes += streamed;
    if (e->timing) EOCHK(harvest_times(e));
    return EO_OK;
}

eo_status eo_set_capture(eo_engine* e, void* x_in, float* y, int32_t* ids, float* w,
                         int32_t tokens_per_layer) {
    if (!e) return fail(EO_ERR_INVALID_ARG, "null engine");
    if (y && (!x_in || !ids || !w || tokens_per_layer < 1))
        return fail(EO_ERR_INVALID_ARG, "capture needs all four buffers and a capacity");
    e->cap_x = x_in;
    e->cap_y = y;
    e->cap_ids = ids;
    e->cap_w = w;
    e->cap_T = y ? tokens_per_layer : 0;
    return EO_OK;
}

eo_status eo_resize_cache(eo_engine* e, int64_t slots, int64_t* n_evicted, int64_t* n_moved) {
    TraceRange trace_range("eo.resize_cache");
    if (!e) return fail(EO_ERR_INVALID_ARG, "null engine");
    if (slots < 0 || slots > plan_max_slots())
        return fail(EO_ERR_INVALID_ARG, "slots out of range [0, 8192]");
    if (e->plan_pending) return fail(EO_ERR_STATE, "a lookup plan is pending: resize between steps");
    HIPCHK(hipSetDevice(e->cfg.device));
    HIPCHK(hipDeviceSynchronize());
    const int64_t C = e->C, Cn = slots;
    std::vector<int32_t> key(C);
    std::vector<int64_t> stamp(C);
    if (C) {
        HIPCHK(hipMemcpy(key.data(), e->d_slot_key, sizeof(int32_t) * C, hipMemcpyDeviceToHost));
        HIPCHK(hipMemcpy(stamp.data(), e->d_slot_stamp, sizeof(int64_t) * C, hipMemcpyDeviceToHost));
    }
    // least recently used first: (stamp asc, key asc)
    std::vector<int64_t> occ;
    for (int64_t i = 0; i < C; ++i)
        if (key[i] >= 0) occ.push_back(i);
    std::sort(occ.begin(), occ.end(), [&](int64_t a, int64_t b) {
        return stamp[a] != stamp[b] ? stamp[a] < stamp[b] : key[a] < key[b];
    });
    const int64_t excess = std::max<int64_t>(0, (int64_t)occ.size() - Cn);
    std::vector<int32_t> nkey(Cn, -1);
    std::vector<int64_t> nstamp(Cn, 0);
    std::vector<char> evict(C, 0);
    for (int64_t i = 0; i < excess; ++i) evict[occ[i]] = 1;
    std::vector<std::pair<int64_t, int64_t>> moves;  // (old slot, new slot)
    std::vector<int64_t> movers;
    for (int64_t i = 0; i < C; ++i) {
        if (key[i] < 0 || evict[i]) continue;
        if (i < Cn) {
            nkey[i] = key[i];
            nstamp[i] = stamp[i];
        } else {
            movers.push_back(i);
        }
    }
    int64_t hole = 0;
    for (int64_t src : movers) {  // ascending old slot -> ascending holes below Cn
        while (nkey[hole] >= 0) ++hole;
        nkey[hole] = key[src];
        nstamp[hole] = stamp[src];
        moves.push_back({src, hole});
    }
    // new device storage first, so that a failed allocation leaves the engine as it was
    uint8_t* nslots = nullptr;
    int32_t* nd_key = nullptr;
    int64_t* nd_stamp = nullptr;
    eo_status st = dmalloc(&nslots, (uint64_t)Cn * e->S_pad);
    if (st == EO_OK) st = dmalloc(&nd_key, sizeof(int32_t) * std::max<int64_t>(Cn, 1));
    if (st == EO_OK) st = dmalloc(&nd_stamp, sizeof(int64_t) * std::max<int64_t>(Cn, 1));
    if (st != EO_OK) {
        if (nslots) (void)hipFree(nslots);
        if (nd_key) (void)hipFree(nd_key);
        return st;
    }
    std::vector<int32_t> k2s((size_t)e->L * e->E);
    HIPCHK(hipMemcpy(k2s.data(), e->d_key2slot, sizeof(int32_t) * k2s.size(), hipMemcpyDeviceToHost));
    for (int64_t i = 0; i < Cn; ++i) {
        if (nkey[i] < 0) continue;
        int64_t src = i;  // where this block lives now
        for (auto& m : moves)
            if (m.second == i) src = m.first;
        HIPCHK(hipMemcpy(nslots + (uint64_t)i * e->S_pad, e->d_slots + (uint64_t)src * e->S_pad, e->S,
                         hipMemcpyDeviceToDevice));
        k2s[nkey[i]] = (int32_t)i;
    }
    for (int64_t i = 0; i < C; ++i)
        if (evict[i]) k2s[key[i]] = -1;
    if (Cn) {
        HIPCHK(hipMemcpy(nd_key, nkey.data(), sizeof(int32_t) * Cn, hipMemcpyHostToDevice));
        HIPCHK(hipMemcpy(nd_stamp, nstamp.data(), sizeof(int64_t) * Cn, hipMemcpyHostToDevice));
    }
    HIPCHK(hipMemcpy(e->d_key2slot, k2s.data(), sizeof(int32_t) * k2s.size(), hipMemcpyHostToDevice));
    HIPCHK(hipDeviceSynchronize());
    (void)hipFree(e->d_slots);
    (void)hipFree(e->d_slot_key);
    (void)hipFree(e->d_slot_stamp);
    e->d_slots = nslots;
    e->d_slot_key = nd_key;
    e->d_slot_stamp = nd_stamp;
    e->C = Cn;
    e->cfg.cache_slots = Cn;
    if (n_evicted) *n_evicted = excess;
    if (n_moved) *n_moved = (int64_t)moves.size();
    return EO_OK;
}

eo_status eo_set_static_placement(eo_engine* e, const int32_t* keys, int32_t n) {
    if (!e) return fail(EO_ERR_INVALID_ARG, "null engine");
    if (n < 0 || n > e->C || (n > 0 && !keys))
        return fail(EO_ERR_INVALID_ARG, "0 <= n <= cache slots keys required");
    if (e->plan_pending) return fail(EO_ERR_STATE, "a lookup plan is pending: place between steps");
    const int64_t nk = (int64_t)e->L * e->E;
    std::vector<int32_t> k2s(nk, -1);
    for (int32_t i = 0; i < n; ++i) {
        if (keys[i] < 0 || keys[i] >= nk) return fail(EO_ERR_INVALID_ARG, "key out of range");
        if (k2s[keys[i]] >= 0) return fail(EO_ERR_INVALID_ARG, "repeated key");
        k2s[keys[i]] = i;
    }
    HIPCHK(hipSetDevice(e->cfg.device));
    HIPCHK(hipDeviceSynchronize());
    for (int32_t i = 0; i < n; ++i)
        HIPCHK(hipMemcpyAsync(e->d_slots + (uint64_t)i * e->S_pad,
                              e->pool[keys[i] / e->E] + (uint64_t)(keys[i] % e->E) * e->S_pad, e->S,
                              hipMemcpyHostToDevice, e->copy_stream));
    std::vector<int32_t> skey(e->C, -1);
    for (int32_t i = 0; i < n; ++i) skey[i] = keys[i];
    if (e->C) {
        HIPCHK(hipMemcpy(e->d_slot_key, skey.data(), sizeof(int32_t) * e->C, hipMemcpyHostToDevice));
        HIPCHK(hipMemset(e->d_slot_stamp, 0, sizeof(int64_t) * e->C));
    }
    HIPCHK(hipMemcpy(e->d_key2slot, k2s.data(), sizeof(int32_t) * nk, hipMemcpyHostToDevice));
    DevState st{};
    HIPCHK(hipMemcpy(&st, e->d_state, sizeof(DevState), hipMemcpyDeviceToHost));
    st.frozen = 1;
    HIPCHK(hipMemcpy(e->d_state, &st, sizeof(DevState), hipMemcpyHostToDevice));
    HIPCHK(hipStreamSynchronize(e->copy_stream));
    e->stats.pcie_bytes += (int64_t)n * (int64_t)e->S;
    return EO_OK;
}

eo_status eo_clear_static_placement(eo_engine* e) {
    if (!e) return fail(EO_ERR_INVALID_ARG, "null engine");
    if (e->plan_pending) return fail(EO_ERR_STATE, "a lookup plan is pending");
    HIPCHK(hipSetDevice(e->cfg.device));
    HIPCHK(hipDeviceSynchronize());
    DevState st{};
    HIPCHK(hipMemcpy(&st, e->d_state, sizeof(DevState), hipMemcpyDeviceToHost));
    st.frozen = 0;
    HIPCHK(hipMemcpy(e->d_state, &st, sizeof(DevState), hipMemcpyHostToDevice));
    return EO_OK;
}

eo_status eo_cache_snapshot(eo_engine* e, int32_t* slot_key, int64_t* slot_stamp, int64_t* clock,
                            int64_t* credit) {
    if (!e) return fail(EO_ERR_INVALID_ARG, "null engine");
    HIPCHK(hipSetDevice(e->cfg.device));
    HIPCHK(hipDeviceSynchronize());
    if (slot_key && e->C) HIPCHK(hipMemcpy(slot_key, e->d_slot_key, sizeof(int32_t) * e->C, hipMemcpyDeviceToHost));
    if (slot_stamp && e->C)
        HIPCHK(hipMemcpy(slot_stamp, e->d_slot_stamp, sizeof(int64_t) * e->C, hipMemcpyDeviceToHost));
    DevState st{};
    HIPCHK(hipMemcpy(&st, e->d_state, sizeof(DevState), hipMemcpyDeviceToHost));
    if (clock) *clock = st.clock;
    if (credit) *credit = st.credit;
    return EO_OK;
}

eo_status eo_last_plan(eo_engine* e, eo_plan_host* out) {
    if (!e || !out) return fail(EO_ERR_INVALID_ARG, "null argument");
    if (e->plan_pending && !e->plan_ready) EOCHK(wait_plan(e));
    *out = e->last_plan;
    return EO_OK;
}

static eo_status dequant_impl(eo_engine* e, int32_t layer, int32_t expert, int32_t decoder,
                              float* out_host) {
    EOCHK(check_layer(e, layer));
    if (expert < 0 || expert >= e->E || !out_host) return fail(EO_ERR_INVALID_ARG, "bad expert");
    if (decoder < EO_DECODER_SCALAR || decoder > EO_DECODER_GEMV)
        return fail(EO_ERR_INVALID_ARG, "unknown decoder");
    HIPCHK(hipSetDevice(e->cfg.device));
    uint8_t* blk = nullptr;
    float* out = nullptr;
    const size_t n = 3ull * e->H * e->I;
    EOCHK(dmalloc(&blk, e->S_pad));
    eo_status st = dmalloc(&out, sizeof(float) * n);
    if (st != EO_OK) {
        (void)hipFree(blk);
        return st;
    }
    hipError_t he = hipMemcpy(blk, e->pool[layer] + (uint64_t)expert * e->S_pad, e->S, hipMemcpyHostToDevice);
    if (he == hipSuccess)
        he = decoder == EO_DECODER_SCALAR
                 ? launch_dequant(e->fmt, e->lay, blk, e->H, e->I, out, nullptr)
                 : launch_dequant_dec(decoder, e->fmt, e->lay, blk, e->H, e->I, out, nullptr);
    if (he == hipSuccess) he = hipMemcpy(out_host, out, sizeof(float) * n, hipMemcpyDeviceToHost);
    (void)hipFree(blk);
    (void)hipFree(out);
    if (he != hipSuccess) return fail(EO_ERR_HIP, std::string("dequant: ") + hipGetErrorString(he));
    return EO_OK;
}

eo_status eo_dequant(eo_engine* e, int32_t layer, int32_t expert, float* out_host) {
    return dequant_impl(e, layer, expert, EO_DECODER_SCALAR, out_host);
}

eo_status eo_dequant_with(eo_engine* e, int32_t layer, int32_t expert, int32_t decoder,
                          float* out_host) {
    return dequant_impl(e, layer, expert, decoder, out_host);
}

eo_status eo_stats_get(eo_engine* e, eo_stats* out) {
    if (!e || !out) return fail(EO_ERR_INVALID_ARG, "null argument");
    *out = e->stats;
    return EO_OK;
}

eo_status eo_set_plan_log(eo_engine* e, int32_t enable) {
    if (!e) return fail(EO_ERR_INVALID_ARG, "null engine");
    e->plan_log_on = enable != 0;
    if (e->plan_log_on) e->plan_log.clear();
    return EO_OK;
}

eo_status eo_get_plan_log(eo_engine* e, int32_t* out, int64_t cap, int64_t* n) {
    if (!e) return fail(EO_ERR_INVALID_ARG, "null engine");
    if (cap < 0 || (cap > 0 && !out)) return fail(EO_ERR_INVALID_ARG, "out must hold cap entries");
    const int64_t have = (int64_t)e->plan_log.size() / 4;
    if (out && cap > 0)
        std::memcpy(out, e->plan_log.data(), sizeof(int32_t) * 4 * std::min(have, cap));
    if (n) *n = have;
    return EO_OK;
}

eo_status eo_set_timing(eo_engine* e, int32_t enable) {
    if (!e) return fail(EO_ERR_INVALID_ARG, "null engine");
    e->timing = enable != 0;
    return EO_OK;
}

eo_status eo_kernel_times(eo_engine* e, double* ms, int64_t* launches, int32_t reset) {
    if (!e) return fail(EO_ERR_INVALID_ARG, "null engine");
    EOCHK(harvest_times(e));
    if (ms)
        for (int i = 0; i < 5; ++i) ms[i] = e->kms[i];
    if (launches) {
        launches[0] = e->gemv_n;
        launches[1] = e->gemm_n;
        launches[2] = e->fill_n;
    }
    if (reset) {
        for (double& v : e->kms) v = 0;
        e->gemv_n = e->gemm_n = e->fill_n = 0;
    }
    return EO_OK;
}

eo_status eo_stream_times(eo_engine* e, double* ms, int64_t* layers, int32_t reset) {
    if (!e) return fail(EO_ERR_INVALID_ARG, "null engine");
    EOCHK(harvest_times(e));
    if (ms) {
        ms[0] = e->sms[0];
        ms[1] = e->sms[1];
    }
    if (layers) {
        layers[0] = e->copy_n;
        layers[1] = e->comp_n;
    }
    if (reset) {
        e->sms[0] = e->sms[1] = 0;
        e->copy_n = e->comp_n = 0;
    }
    return EO_OK;
}

eo_status eo_sync(eo_engine* e) {
    if (!e) return fail(EO_ERR_INVALID_ARG, "null engine");
    HIPCHK(hipSetDevice(e->cfg.device));
    HIPCHK(hipStreamSynchronize(e->copy_stream));
    HIPCHK(hipDeviceSynchronize());
    HIPCHK(hipGetLastError());
    return EO_OK;
}

}  // extern "C"
