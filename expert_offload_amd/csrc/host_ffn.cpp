// Host-core expert routine: runs a missed expert's SwiGLU FFN on the CPU,
// reading its packed block straight from the pinned host pool.
//
// zhichai.net article, section 2, Decode paragraph: misses that the bandwidth
// split does not send over PCIe are executed in place on the host cores, so
// host memory bandwidth (B_H) is put to use instead of sitting idle. The
// routine is fp32 on the host (decoding the block's format in-line) and is
// spread over a pool of threads: phase 1 over the gate/up rows of every host
// expert, phase 2 over the output rows, where each token's host pairs are summed
// in slot order j.
#include <immintrin.h>

#include <algorithm>
#include <atomic>
#include <cmath>
#include <condition_variable>
#include <cstdlib>
#include <cstring>
#include <functional>
#include <memory>
#include <mutex>
#include <thread>

#include "eo_host.h"

namespace eo {

// ------------------------------------------------------------ thread pool
class ThreadPool {
  public:
    explicit ThreadPool(int n) : n_(std::max(1, n)) {
        // every worker starts from generation 0, the value before any run(): a
        // worker that is scheduled late must still take part in run() #1
        for (int i = 1; i < n_; ++i) workers_.emplace_back([this] { loop(0); });
    }
    ~ThreadPool() {
        {
            std::lock_guard<std::mutex> lk(mu_);
            stop_ = true;
            gen_.fetch_add(1, std::memory_order_release);
        }
        cv_.notify_all();
        for (auto& t : workers_) t.join();
    }
    int size() const { return n_; }

    // Run fn(task) for task in [0, ntasks) on all threads (the caller included).
    void run(int ntasks, const std::function<void(int)>& fn) {
        if (ntasks <= 0) return;
        if (n_ == 1 || ntasks == 1) {
            for (int i = 0; i < ntasks; ++i) fn(i);
            return;
        }
        fn_ = &fn;
        ntasks_ = ntasks;
        next_.store(0, std::memory_order_relaxed);
        done_.store(0, std::memory_order_relaxed);
        {
            std::lock_guard<std::mutex> lk(mu_);
            gen_.fetch_add(1, std::memory_order_release);
        }
        cv_.notify_all();
        work();
        while (done_.load(std::memory_order_acquire) < n_ - 1) _mm_pause();
    }

  private:
    void work() {
        for (;;) {
            int i = next_.fetch_add(1, std::memory_order_relaxed);
            if (i >= ntasks_) break;
            (*fn_)(i);
        }
    }
    void loop(uint64_t seen) {
        for (;;) {
            // spin briefly for low dispatch latency, then sleep
            int spins = 0;
            while (gen_.load(std::memory_order_acquire) == seen && spins < 200000) {
                _mm_pause();
                ++spins;
            }
            if (gen_.load(std::memory_order_acquire) == seen) {
                std::unique_lock<std::mutex> lk(mu_);
                cv_.wait(lk, [&] { return gen_.load(std::memory_order_acquire) != seen; });
            }
            seen = gen_.load(std::memory_order_acquire);
            if (stop_) return;
            work();
            done_.fetch_add(1, std::memory_order_acq_rel);
        }
    }

    int n_;
    std::vector<std::thread> workers_;
    std::mutex mu_;
    std::condition_variable cv_;
    std::atomic<uint64_t> gen_{0};
    std::atomic<int> next_{0}, done_{0};
    const std::function<void(int)>* fn_ = nullptr;
    int ntasks_ = 0;
    bool stop_ = false;
};

ThreadPool* threadpool_create(int n) { return new ThreadPool(n); }
void threadpool_destroy(ThreadPool* p) { delete p; }
int threadpool_size(ThreadPool* p) { return p->size(); }
void threadpool_run(ThreadPool* p, int ntasks, const std::function<void(int)>& fn) {
    p->run(ntasks, fn);
}

// ------------------------------------------------------------ decoding
namespace {

float e2m1_val(uint32_t c) {
    static const float t[8] = {0.f, 0.5f, 1.f, 1.5f, 2.f, 3.f, 4.f, 6.f};
    float v = t[c & 7];
    return (c & 8) ? -v : v;
}
float e4m3_val(uint32_t c) {
    uint32_t e = (c >> 3) & 15, m = c & 7;
    float v;
    if (e == 15 && m == 7) v = NAN;
    else if (e == 0) v = std::ldexp((float)m, -9);
    else v = std::ldexp(1.0f + m / 8.0f, (int)e - 7);
    return (c & 0x80) ? -v : v;
}
float e8m0_val(uint32_t c) { return c == 0xFF ? NAN : std::ldexp(1.0f, (int)c - 127); }

// Decode row `row` (K elements) of a matrix section into out (fp32).
void decode_row(int fmt, const uint8_t* data, const uint8_t* scal, float gscale, int row, int K,
                float* out) {
    switch (fmt) {
    case EO_W_FP32: std::memcpy(out, (const float*)data + (size_t)row * K, sizeof(float) * K); break;
    case EO_W_BF16: {
        const uint16_t* p = (const uint16_t*)data + (size_t)row * K;
        int i = 0;
        for (; i + 8 <= K; i += 8) {
            __m128i b = _mm_loadu_si128((const __m128i*)(p + i));
            __m256i w = _mm256_slli_epi32(_mm256_cvtepu16_epi32(b), 16);
            _mm256_storeu_ps(out + i, _mm256_castsi256_ps(w));
        }
        for (; i < K; ++i) {
            uint32_t u = (uint32_t)p[i] << 16;
            std::memcpy(out + i, &u, 4);
        }
        break;
    }
    case EO_W_FP8: {
        const uint8_t* p = data + (size_t)row * K;
        float s = ((const float*)scal)[row];
        for (int i = 0; i < K; ++i) out[i] = e4m3_val(p[i]) * s;
        break;
    }
    case EO_W_MXFP4: {
        const uint8_t* p = data + (size_t)row * (K / 2);
        const uint8_t* sp = scal + (size_t)row * (K / 32);
        for (int b = 0; b < K / 32; ++b) {
            float s = e8m0_val(sp[b]);
            for (int i = 0; i < 16; ++i) {
                uint32_t byte = p[b * 16 + i];
                out[b * 32 + 2 * i] = e2m1_val(byte & 0xF) * s;
                out[b * 32 + 2 * i + 1] = e2m1_val(byte >> 4) * s;
            }
        }
        break;
    }
    case EO_W_NVFP4: {
        const uint8_t* p = data + (size_t)row * (K / 2);
        const uint8_t* sp = scal + (size_t)row * (K / 16);
        for (int b = 0; b < K / 16; ++b) {
            float s = e4m3_val(sp[b]);
            for (int i = 0; i < 8; ++i) {
                uint32_t byte = p[b * 8 + i];
                out[b * 16 + 2 * i] = (e2m1_val(byte & 0xF) * s) * gscale;
                out[b * 16 + 2 * i + 1] = (e2m1_val(byte >> 4) * s) * gscale;
            }
        }
        break;
    }
    }
}

inline float hsum256(__m256 v) {
    __m128 lo = _mm256_castps256_ps128(v), hi = _mm256_extractf128_ps(v, 1);
    __m128 s = _mm_add_ps(lo, hi);
    s = _mm_add_ps(s, _mm_movehl_ps(s, s));
    s = _mm_add_ss(s, _mm_shuffle_ps(s, s, 1));
    return _mm_cvtss_f32(s);
}

float dot(const float* a, const float* b, int K) {
    __m256 s0 = _mm256_setzero_ps(), s1 = _mm256_setzero_ps();
    int i = 0;
    for (; i + 16 <= K; i += 16) {
        s0 = _mm256_fmadd_ps(_mm256_loadu_ps(a + i), _mm256_loadu_ps(b + i), s0);
        s1 = _mm256_fmadd_ps(_mm256_loadu_ps(a + i + 8), _mm256_loadu_ps(b + i + 8), s1);
    }
    float s = hsum256(_mm256_add_ps(s0, s1));
    for (; i < K; ++i) s += a[i] * b[i];
    return s;
}

// bf16 row (raw) dot fp32 vector, no staging.
float dot_bf16(const uint16_t* w, const float* x, int K) {
    __m256 s0 = _mm256_setzero_ps(), s1 = _mm256_setzero_ps();
    int i = 0;
    for (; i + 16 <= K; i += 16) {
        __m256i b = _mm256_loadu_si256((const __m256i*)(w + i));
        __m256 lo = _mm256_castsi256_ps(
            _mm256_slli_epi32(_mm256_cvtepu16_epi32(_mm256_castsi256_si128(b)), 16));
        __m256 hi = _mm256_castsi256_ps(
            _mm256_slli_epi32(_mm256_cvtepu16_epi32(_mm256_extracti128_si256(b, 1)), 16));
        s0 = _mm256_fmadd_ps(lo, _mm256_loadu_ps(x + i), s0);
        s1 = _mm256_fmadd_ps(hi, _mm256_loadu_ps(x + i + 8), s1);
    }
    float s = hsum256(_mm256_add_ps(s0, s1));
    for (; i < K; ++i) {
        uint32_t u = (uint32_t)w[i] << 16;
        float f;
        std::memcpy(&f, &u, 4);
        s += f * x[i];
    }
    return s;
}

// ---------------------------------------------------------- AVX-512 BF16
// bf16 weights against bf16 activations with the bf16 pair dot product
// (vdpbf16ps: 32 products per instruction, fp32 accumulation). Used when the
// CPU has AVX512_BF16; the SwiGLU output h is rounded to bf16 (nearest even)
// before the down projection, as on the device.
#define EO_AVX512BF16 __attribute__((target("avx512f,avx512bw,avx512vl,avx512bf16")))

EO_AVX512BF16 inline __m512bh as_bh(__m512i v) { return (__m512bh)v; }

// Two rows of K (K % 128 == 0) against one vector.
EO_AVX512BF16 void dot2_bf16_avx512(const uint16_t* a, const uint16_t* b, const uint16_t* x,
                                    int K, float* ra, float* rb) {
    __m512 a0 = _mm512_setzero_ps(), a1 = _mm512_setzero_ps();
    __m512 b0 = _mm512_setzero_ps(), b1 = _mm512_setzero_ps();
    for (int i = 0; i < K; i += 64) {
        __m512i x0 = _mm512_loadu_si512(x + i), x1 = _mm512_loadu_si512(x + i + 32);
        a0 = _mm512_dpbf16_ps(a0, as_bh(_mm512_loadu_si512(a + i)), as_bh(x0));
        a1 = _mm512_dpbf16_ps(a1, as_bh(_mm512_loadu_si512(a + i + 32)), as_bh(x1));
        b0 = _mm512_dpbf16_ps(b0, as_bh(_mm512_loadu_si512(b + i)), as_bh(x0));
        b1 = _mm512_dpbf16_ps(b1, as_bh(_mm512_loadu_si512(b + i + 32)), as_bh(x1));
    }
    *ra = _mm512_reduce_add_ps(_mm512_add_ps(a0, a1));
    *rb = _mm512_reduce_add_ps(_mm512_add_ps(b0, b1));
}

// Four rows (stride ld, K % 64 == 0) against one vector.
EO_AVX512BF16 void dot4_bf16_avx512(const uint16_t* a, size_t ld, const uint16_t* x, int K,
                                    float* out) {
    __m512 s0 = _mm512_setzero_ps(), s1 = _mm512_setzero_ps();
    __m512 s2 = _mm512_setzero_ps(), s3 = _mm512_setzero_ps();
    for (int i = 0; i < K; i += 32) {
        __m512bh xv = as_bh(_mm512_loadu_si512(x + i));
        s0 = _mm512_dpbf16_ps(s0, as_bh(_mm512_loadu_si512(a + i)), xv);
        s1 = _mm512_dpbf16_ps(s1, as_bh(_mm512_loadu_si512(a + ld + i)), xv);
        s2 = _mm512_dpbf16_ps(s2, as_bh(_mm512_loadu_si512(a + 2 * ld + i)), xv);
        s3 = _mm512_dpbf16_ps(s3, as_bh(_mm512_loadu_si512(a + 3 * ld + i)), xv);
    }
    out[0] = _mm512_reduce_add_ps(s0);
    out[1] = _mm512_reduce_add_ps(s1);
    out[2] = _mm512_reduce_add_ps(s2);
    out[3] = _mm512_reduce_add_ps(s3);
}

// fp4 weights (MXFP4 / NVFP4) against bf16 activations on the same pair dot
// product: 32 codes (16 bytes, even element in the low nibble) become 32 bf16
// by widening each byte to a dword whose low word is its low nibble and whose
// high word is its high nibble, and looking both up in a 16-entry table of the
// e2m1 values (vpermw). One vdpbf16ps then gives 16 fp32 partial sums of a
// 32-code group, lane l holding codes 2l and 2l+1; the group's block scales
// multiply those partials (MXFP4: one e8m0 scale per 32 codes; NVFP4: one
// e4m3 scale per 16 codes, lanes 0-7 and 8-15). Every weight is exact in bf16.
alignas(64) const uint16_t kE2m1Bf16[32] = {
    0x0000, 0x3F00, 0x3F80, 0x3FC0, 0x4000, 0x4040, 0x4080, 0x40C0,   // 0 0.5 1 1.5 2 3 4 6
    0x8000, 0xBF00, 0xBF80, 0xBFC0, 0xC000, 0xC040, 0xC080, 0xC0C0};  // the same, negative

// Block-scale codes as fp32: e8m0 (MXFP4) and e4m3 (NVFP4), all 256 codes.
const float* scale_table(int fmt) {
    static const std::vector<float> e8m0 = [] {
        std::vector<float> t(256);
        for (int c = 0; c < 256; ++c) t[c] = e8m0_val(c);
        return t;
    }();
    static const std::vector<float> e4m3 = [] {
        std::vector<float> t(256);
        for (int c = 0; c < 256; ++c) t[c] = e4m3_val(c);
        return t;
    }();
    return fmt == EO_W_MXFP4 ? e8m0.data() : e4m3.data();
}

EO_AVX512BF16 inline __m512i fp4x32_bf16(const uint8_t* p, __m512i lut) {
    const __m512i d = _mm512_cvtepu8_epi32(_mm_loadu_si128((const __m128i*)p));
    const __m512i idx = _mm512_or_si512(
        _mm512_and_si512(d, _mm512_set1_epi32(0xF)),
        _mm512_slli_epi32(_mm512_and_si512(d, _mm512_set1_epi32(0xF0)), 12));
    return _mm512_permutexvar_epi16(idx, lut);
}

// NR fp4 rows of K codes (K % 32 == 0; row r's codes at rows[r], its block
// scale codes at scal[r]) against the bf16 vector x, block scales applied.
template <int FMT, int NR>
EO_AVX512BF16 void dot_fp4_avx512(const uint8_t* const (&rows)[NR],
                                  const uint8_t* const (&scal)[NR], const uint16_t* x, int K,
                                  const float* st, float (&out)[NR]) {
    const __m512i lut = _mm512_load_si512(kE2m1Bf16);
    __m512 acc[NR];
    for (int r = 0; r < NR; ++r) acc[r] = _mm512_setzero_ps();
    for (int g = 0; g < K / 32; ++g) {
        const __m512bh xv = as_bh(_mm512_loadu_si512(x + 32 * g));
        for (int r = 0; r < NR; ++r) {
            const __m512 p = _mm512_dpbf16_ps(_mm512_setzero_ps(),
                                              as_bh(fp4x32_bf16(rows[r] + 16 * g, lut)), xv);
            __m512 sv;
            if (FMT == EO_W_MXFP4)
                sv = _mm512_set1_ps(st[scal[r][g]]);
            else
                sv = _mm512_mask_mov_ps(_mm512_set1_ps(st[scal[r][2 * g]]), (__mmask16)0xFF00,
                                        _mm512_set1_ps(st[scal[r][2 * g + 1]]));
            acc[r] = _mm512_fmadd_ps(p, sv, acc[r]);
        }
    }
    for (int r = 0; r < NR; ++r) out[r] = _mm512_reduce_add_ps(acc[r]);
}

// fp8 (e4m3fn) weights on the same pair dot product: a code's 7 magnitude bits
// shifted left by 7 are the fp16 encoding of value / 256 (exponent bias 15
// against 7; e4m3 subnormals land on fp16 subnormals), so 32 codes become bf16
// through fp16 -> fp32 -> bf16, every step exact; the dot is scaled by 256 and
// the row scale afterwards. (0x7F / 0xFF, e4m3fn's NaN, is never stored.)
EO_AVX512BF16 inline __m512i fp8x32_bf16(const uint8_t* p) {
    const __m512i w = _mm512_cvtepu8_epi16(_mm256_loadu_si256((const __m256i*)p));
    const __m512i h = _mm512_or_si512(
        _mm512_slli_epi16(_mm512_and_si512(w, _mm512_set1_epi16(0x7F)), 7),
        _mm512_slli_epi16(_mm512_and_si512(w, _mm512_set1_epi16(0x80)), 8));
    const __m512 lo = _mm512_cvtph_ps(_mm512_castsi512_si256(h));
    const __m512 hi = _mm512_cvtph_ps(_mm512_extracti64x4_epi64(h, 1));
    return (__m512i)_mm512_cvtne2ps_pbh(hi, lo);
}

// NR fp8 rows of K codes (K % 32 == 0) against the bf16 vector x, times 256
// (the row scales are the caller's).
template <int NR>
EO_AVX512BF16 void dot_fp8_avx512(const uint8_t* const (&rows)[NR], const uint16_t* x, int K,
                                  float (&out)[NR]) {
    __m512 acc[NR];
    for (int r = 0; r < NR; ++r) acc[r] = _mm512_setzero_ps();
    for (int g = 0; g < K / 32; ++g) {
        const __m512bh xv = as_bh(_mm512_loadu_si512(x + 32 * g));
        for (int r = 0; r < NR; ++r)
            acc[r] = _mm512_dpbf16_ps(acc[r], as_bh(fp8x32_bf16(rows[r] + 32 * g)), xv);
    }
    for (int r = 0; r < NR; ++r) out[r] = _mm512_reduce_add_ps(acc[r]) * 256.0f;
}

uint16_t bf16_rne(float f) {
    uint32_t u;
    std::memcpy(&u, &f, 4);
    u += 0x7FFFu + ((u >> 16) & 1u);
    return (uint16_t)(u >> 16);
}

bool cpu_has_avx512bf16() {
    static const bool ok = [] {
        if (const char* v = std::getenv("EO_HOST_ISA"))
            if (!std::strcmp(v, "avx2")) return false;
        return __builtin_cpu_supports("avx512bf16") != 0;
    }();
    return ok;
}

}  // namespace

bool host_ffn_uses_avx512bf16() { return cpu_has_avx512bf16(); }

namespace {
EO_AVX512BF16 void decode_codes_avx512(int fmt, const uint8_t* codes, uint16_t* out) {
    const __m512i v = fmt == EO_W_FP8 ? fp8x32_bf16(codes)
                                      : fp4x32_bf16(codes, _mm512_load_si512(kE2m1Bf16));
    _mm512_storeu_si512(out, v);
}
}  // namespace

bool host_decode_codes(int fmt, const uint8_t* codes, uint16_t* out) {
    if (!cpu_has_avx512bf16() || (fmt != EO_W_FP8 && fmt != EO_W_MXFP4 && fmt != EO_W_NVFP4))
        return false;
    decode_codes_avx512(fmt, codes, out);
    return true;
}

void host_ffn(ThreadPool* pool, const HostJob& jb, std::vector<float>& scratch) {
    const int H = jb.H, I = jb.I, T = jb.T, k = jb.k;
    // host experts and their pairs
    std::vector<int> exps;  // expert ids, ascending
    std::vector<int> slot_of(EO_MAX_EXPERTS, -1);
    for (int p = 0; p < T * k; ++p) {
        int e = jb.ids[p];
        if (e >= 0 && e < EO_MAX_EXPERTS && jb.experts[e] && slot_of[e] < 0) {
            slot_of[e] = 0;
            exps.push_back(e);
        }
    }
    if (exps.empty()) return;
    std::sort(exps.begin(), exps.end());
    const int ne = (int)exps.size();
    for (int i = 0; i < ne; ++i) slot_of[exps[i]] = i;
    // tokens per host expert
    std::vector<std::vector<int>> toks(ne);
    for (int t = 0; t < T; ++t)
        for (int j = 0; j < k; ++j) {
            int e = jb.ids[t * k + j];
            if (e >= 0 && e < EO_MAX_EXPERTS && jb.experts[e]) toks[slot_of[e]].push_back(t);
        }
    // h[i][t_idx][I]
    std::vector<size_t> hoff(ne + 1, 0);
    for (int i = 0; i < ne; ++i) hoff[i + 1] = hoff[i] + toks[i].size() * (size_t)I;
    if (scratch.size() < hoff[ne]) scratch.resize(hoff[ne]);
    float* h = scratch.data();
    const int fmt = jb.fmt;
    const Layout lay = jb.lay;

    auto gl = [&](const uint8_t* b, int t) -> float {
        return fmt == EO_W_NVFP4 ? ((const float*)(b + lay.gl))[t] : 1.0f;
    };

    constexpr int RB = 16;
    const int nb1_fp32 = (I + RB - 1) / RB;
    const bool fp4 = fmt == EO_W_MXFP4 || fmt == EO_W_NVFP4;
    const bool coded = fp4 || fmt == EO_W_FP8;  // weights decoded to bf16 in registers
    if ((fmt == EO_W_BF16 || coded) && jb.xb && H % 128 == 0 && I % 64 == 0 &&
        cpu_has_avx512bf16()) {
        // task sizes: two tasks per thread and expert in each phase, so that
        // every thread streams the same share (measured on the 16-core host:
        // smaller tasks cost dispatch, uneven counts leave threads idle)
        const int nth = threadpool_size(pool);
        const int RB1 = std::max(4, (I + 2 * nth - 1) / (2 * nth));
        const int nb1 = (I + RB1 - 1) / RB1;
        const int RB2 = 4 * std::max(1, (H + 8 * nth - 1) / (8 * nth));  // multiple of 4
        const int nb2 = (H + RB2 - 1) / RB2;
        // One pool run, pipelined over experts: gate/up rows of expert i (h_i,
        // bf16) and the down rows of expert i-1 (v_i = W_down h_i per token,
        // unweighted fp32) are queued alternately; a down task waits for its
        // expert's gate/up tasks, which were all handed out before it. The
        // weighted sum over each token's slots follows in slot order.
        std::vector<size_t> voff(ne + 1, 0);
        for (int i = 0; i < ne; ++i) voff[i + 1] = voff[i] + toks[i].size() * (size_t)H;
        const size_t vtot = voff[ne];
        const size_t hwords = (hoff[ne] + 1) / 2;
        if (scratch.size() < hwords + vtot) scratch.resize(hwords + vtot);
        uint16_t* hb = (uint16_t*)scratch.data();
        float* v = scratch.data() + hwords;
        // segments: (phase, expert) in queue order
        std::vector<std::pair<int, int>> seg;
        seg.push_back({1, 0});
        for (int i = 1; i < ne; ++i) {
            seg.push_back({1, i});
            seg.push_back({2, i - 1});
        }
        seg.push_back({2, ne - 1});
        std::vector<int> seg_start(seg.size() + 1, 0);
        for (size_t q = 0; q < seg.size(); ++q)
            seg_start[q + 1] = seg_start[q] + (seg[q].first == 1 ? nb1 : nb2);
        // fp4 rows: gate row r and up row I + r of W13 (K = H), or four rows of
        // W2 (K = I); NVFP4's per-tensor scales (gate, up, down) multiply the dots
        const int blk = fmt == EO_W_MXFP4 ? 32 : 16;
        const float* st = fp4 ? scale_table(fmt) : nullptr;
        auto fp4_gate_up = [&](const uint8_t* b, int r, const uint16_t* xt, float* g, float* u) {
            const uint8_t* d = b + lay.d13;
            if (fmt == EO_W_FP8) {
                const uint8_t* const rows[2] = {d + (size_t)r * H, d + (size_t)(I + r) * H};
                const float* rs = (const float*)(b + lay.s13);
                float o2[2];
                dot_fp8_avx512<2>(rows, xt, H, o2);
                *g = o2[0] * rs[r];
                *u = o2[1] * rs[I + r];
                return;
            }
            const uint8_t* sc = b + lay.s13;
            const uint8_t* const rows[2] = {d + (size_t)r * (H / 2), d + (size_t)(I + r) * (H / 2)};
            const uint8_t* const scs[2] = {sc + (size_t)r * (H / blk), sc + (size_t)(I + r) * (H / blk)};
            float o2[2];
            if (fmt == EO_W_MXFP4)
                dot_fp4_avx512<EO_W_MXFP4, 2>(rows, scs, xt, H, st, o2);
            else
                dot_fp4_avx512<EO_W_NVFP4, 2>(rows, scs, xt, H, st, o2);
            *g = o2[0] * gl(b, 0);
            *u = o2[1] * gl(b, 1);
        };
        auto fp4_down4 = [&](const uint8_t* b, int o, const uint16_t* ht, float* out) {
            const uint8_t* d = b + lay.d2;
            if (fmt == EO_W_FP8) {
                const uint8_t* const rows[4] = {d + (size_t)o * I, d + (size_t)(o + 1) * I,
                                                d + (size_t)(o + 2) * I, d + (size_t)(o + 3) * I};
                const float* rs = (const float*)(b + lay.s2);
                float o4[4];
                dot_fp8_avx512<4>(rows, ht, I, o4);
                for (int q = 0; q < 4; ++q) out[q] = o4[q] * rs[o + q];
                return;
            }
            const uint8_t* sc = b + lay.s2;
            const uint8_t* const rows[4] = {d + (size_t)o * (I / 2), d + (size_t)(o + 1) * (I / 2),
                                            d + (size_t)(o + 2) * (I / 2), d + (size_t)(o + 3) * (I / 2)};
            const uint8_t* const scs[4] = {sc + (size_t)o * (I / blk), sc + (size_t)(o + 1) * (I / blk),
                                           sc + (size_t)(o + 2) * (I / blk), sc + (size_t)(o + 3) * (I / blk)};
            float o4[4];
            if (fmt == EO_W_MXFP4)
                dot_fp4_avx512<EO_W_MXFP4, 4>(rows, scs, ht, I, st, o4);
            else
                dot_fp4_avx512<EO_W_NVFP4, 4>(rows, scs, ht, I, st, o4);
            const float g2 = gl(b, 2);
            for (int q = 0; q < 4; ++q) out[q] = o4[q] * g2;
        };
        std::unique_ptr<std::atomic<int>[]> done1(new std::atomic<int>[ne]);
        for (int i = 0; i < ne; ++i) done1[i].store(0, std::memory_order_relaxed);
        pool->run(seg_start.back(), [&](int task) {
            size_t q = 0;
            while (task >= seg_start[q + 1]) ++q;
            const int ph = seg[q].first, ei = seg[q].second, blk = task - seg_start[q];
            const uint8_t* b = jb.experts[exps[ei]];
            const size_t nt = toks[ei].size();
            if (ph == 1) {
                const uint16_t* W = (const uint16_t*)(b + lay.d13);
                for (int r = blk * RB1; r < std::min(I, blk * RB1 + RB1); ++r)
                    for (size_t ti = 0; ti < nt; ++ti) {
                        float g, u;
                        const uint16_t* xt = jb.xb + (size_t)toks[ei][ti] * H;
                        if (coded)
                            fp4_gate_up(b, r, xt, &g, &u);
                        else
                            dot2_bf16_avx512(W + (size_t)r * H, W + (size_t)(I + r) * H, xt, H,
                                             &g, &u);
                        hb[hoff[ei] + ti * I + r] = bf16_rne(g / (1.0f + std::exp(-g)) * u);
                    }
                done1[ei].fetch_add(1, std::memory_order_release);
            } else {
                while (done1[ei].load(std::memory_order_acquire) < nb1) _mm_pause();
                const uint16_t* W2 = (const uint16_t*)(b + lay.d2);
                for (int o = blk * RB2; o < std::min(H, blk * RB2 + RB2); o += 4)  // H % 4 == 0
                    for (size_t ti = 0; ti < nt; ++ti) {
                        float out[4];
                        if (coded)
                            fp4_down4(b, o, hb + hoff[ei] + ti * I, out);
                        else
                            dot4_bf16_avx512(W2 + (size_t)o * I, I, hb + hoff[ei] + ti * I, I,
                                             out);
                        float* vo = v + voff[ei] + ti * H + o;
                        vo[0] = out[0];
                        vo[1] = out[1];
                        vo[2] = out[2];
                        vo[3] = out[3];
                    }
            }
        });
        // y[t] += sum over the token's host slots, in slot order, of w * v
        auto combine_rows = [&](int t) {
            float* yt = jb.y + (size_t)t * H;
            thread_local std::vector<float> a;
            a.assign(H, 0.0f);
            for (int j = 0; j < k; ++j) {
                int e = jb.ids[t * k + j];
                if (e < 0 || e >= EO_MAX_EXPERTS || !jb.experts[e]) continue;
                const int ei = slot_of[e];
                const std::vector<int>& tl = toks[ei];
                const size_t ti = std::lower_bound(tl.begin(), tl.end(), t) - tl.begin();
                const float* vt = v + voff[ei] + ti * H;
                const float wt = jb.w[t * k + j];
                for (int o = 0; o < H; ++o) a[o] += wt * vt[o];
            }
            for (int o = 0; o < H; ++o) yt[o] += a[o];
        };
        if (T == 1)
            combine_rows(0);
        else
            pool->run(T, combine_rows);
        return;
    }
    pool->run(ne * nb1_fp32, [&](int task) {
        const int ei = task / nb1_fp32, rb = task % nb1_fp32;
        const uint8_t* b = jb.experts[exps[ei]];
        thread_local std::vector<float> rg, ru;
        rg.resize(H);
        ru.resize(H);
        for (int r = rb * RB; r < std::min(I, rb * RB + RB); ++r) {
            const float* gr;
            const float* ur;
            if (fmt == EO_W_BF16) {
                gr = ur = nullptr;
            } else {
                decode_row(fmt, b + lay.d13, b + lay.s13, gl(b, 0), r, H, rg.data());
                decode_row(fmt, b + lay.d13, b + lay.s13, gl(b, 1), I + r, H, ru.data());
                gr = rg.data();
                ur = ru.data();
            }
            for (size_t ti = 0; ti < toks[ei].size(); ++ti) {
                const float* xt = jb.x + (size_t)toks[ei][ti] * H;
                float g, u;
                if (fmt == EO_W_BF16) {
                    const uint16_t* W = (const uint16_t*)(b + lay.d13);
                    g = dot_bf16(W + (size_t)r * H, xt, H);
                    u = dot_bf16(W + (size_t)(I + r) * H, xt, H);
                } else {
                    g = dot(gr, xt, H);
                    u = dot(ur, xt, H);
                }
                h[hoff[ei] + ti * I + r] = g / (1.0f + std::exp(-g)) * u;
            }
        }
    });

    const int nb2 = (H + RB - 1) / RB;
    pool->run(nb2, [&](int task) {
        thread_local std::vector<float> rd;
        rd.resize(I);
        for (int o = task * RB; o < std::min(H, task * RB + RB); ++o) {
            for (int t = 0; t < T; ++t) {
                float acc = 0.0f;
                for (int j = 0; j < k; ++j) {
                    int e = jb.ids[t * k + j];
                    if (e < 0 || e >= EO_MAX_EXPERTS || !jb.experts[e]) continue;
                    int ei = slot_of[e];
                    const uint8_t* b = jb.experts[e];
                    // position of t in toks[ei]
                    const std::vector<int>& tl = toks[ei];
                    int ti = (int)(std::lower_bound(tl.begin(), tl.end(), t) - tl.begin());
                    const float* ht = h + hoff[ei] + (size_t)ti * I;
                    float v;
                    if (fmt == EO_W_BF16) {
                        v = dot_bf16((const uint16_t*)(b + lay.d2) + (size_t)o * I, ht, I);
                    } else {
                        decode_row(fmt, b + lay.d2, b + lay.s2, gl(b, 2), o, I, rd.data());
                        v = dot(rd.data(), ht, I);
                    }
                    acc += jb.w[t * k + j] * v;
                }
                jb.y[(size_t)t * H + o] += acc;
            }
        }
    });
}

}  // namespace eo
