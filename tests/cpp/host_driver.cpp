// Test driver for the host-core expert routine and its thread pool (CPU only).
//   host_driver pool            : create a pool and run at once, many times
//   host_driver decode <fmt>    : the AVX512-BF16 route's weight decode of every code
//                                 (FP8: bytes 0..255; fp4: the 256 byte values, two codes
//                                 each), bf16 bit patterns as text, one per line
//   host_driver chains <E> <H> : the router's chain-interleaved layout, checked entry by entry
//   host_driver ffn <dir>       : read meta.txt, block.bin, x.bin, ids.bin, w.bin from <dir>,
//                                 run host_ffn with every routed expert on the host,
//                                 write y.bin (fp32 [T,H])
#include <atomic>
#include <chrono>
#include <cstdio>
#include <cstdlib>
#include <cstring>
#include <string>
#include <thread>
#include <unistd.h>
#include <vector>

#include "../../expert_offload_amd/csrc/eo_host.h"

static std::vector<char> slurp(const std::string& p) {
    FILE* f = fopen(p.c_str(), "rb");
    if (!f) { fprintf(stderr, "cannot open %s\n", p.c_str()); exit(2); }
    fseek(f, 0, SEEK_END);
    long n = ftell(f);
    fseek(f, 0, SEEK_SET);
    std::vector<char> b(n);
    if (fread(b.data(), 1, n, f) != (size_t)n) exit(2);
    fclose(f);
    return b;
}

int main(int argc, char** argv) {
    if (argc >= 2 && !strcmp(argv[1], "pool")) {
        for (int it = 0; it < 500; ++it) {
            eo::ThreadPool* p = eo::threadpool_create(8);
            std::atomic<int> sum{0};
            std::atomic<bool> done{false};
            std::thread wd([&] {
                auto t0 = std::chrono::steady_clock::now();
                while (!done) {
                    if (std::chrono::steady_clock::now() - t0 > std::chrono::seconds(10)) {
                        printf("DEADLOCK %d\n", it);
                        fflush(stdout);
                        _exit(3);
                    }
                    std::this_thread::sleep_for(std::chrono::milliseconds(2));
                }
            });
            eo::threadpool_run(p, 37, [&](int i) { sum += i; });
            eo::threadpool_run(p, 5, [&](int i) { sum += i; });
            done = true;
            wd.join();
            eo::threadpool_destroy(p);
            if (sum != 666 + 10) { printf("BAD SUM %d\n", (int)sum); return 4; }
        }
        printf("ok\n");
        return 0;
    }
    if (argc >= 3 && !strcmp(argv[1], "decode")) {
        const int fmt = atoi(argv[2]);
        uint8_t codes[256];
        for (int i = 0; i < 256; ++i) codes[i] = (uint8_t)i;
        const int step = fmt == 4 ? 32 : 16;  // bytes per call
        for (int b = 0; b < 256; b += step) {
            uint16_t out[32];
            if (!eo::host_decode_codes(fmt, codes + b, out)) return 3;
            for (int i = 0; i < 32; ++i) printf("%u\n", out[i]);
        }
        return 0;
    }
    if (argc >= 4 && !strcmp(argv[1], "chains")) {
        // the router's chain-interleaved layout for E experts of H: every entry
        // checked against R[e][i + 64 j]; shapes it does not cover must be refused
        // with the output untouched
        const int E = atoi(argv[2]), H = atoi(argv[3]);
        std::vector<float> R((size_t)E * H), out((size_t)E * H, -7.0f);
        for (size_t i = 0; i < R.size(); ++i) R[i] = (float)i;
        const bool ok = eo::router_chain_layout(R.data(), E, H, out.data());
        if (H % 256 != 0) {
            for (float v : out)
                if (v != -7.0f) { printf("refused shape written to\n"); return 1; }
            printf(ok ? "accepted\n" : "refused\n");
            return ok ? 1 : 0;
        }
        if (!ok) { printf("refused\n"); return 1; }
        for (int e = 0; e < E; ++e)
            for (int j = 0; j < H / 64; ++j)
                for (int i = 0; i < 64; ++i) {
                    const float got = out[(size_t)e * H + ((size_t)(j / 4) * 64 + i) * 4 + (j % 4)];
                    if (got != R[(size_t)e * H + i + 64 * j]) { printf("mismatch\n"); return 1; }
                }
        printf("ok\n");
        return 0;
    }
    if (argc >= 3 && !strcmp(argv[1], "ffn")) {
        std::string d = argv[2];
        int fmt, H, I, T, k, E, threads;
        FILE* m = fopen((d + "/meta.txt").c_str(), "r");
        if (!m || fscanf(m, "%d %d %d %d %d %d %d", &fmt, &H, &I, &T, &k, &E, &threads) != 7) return 2;
        fclose(m);
        std::vector<char> blocks = slurp(d + "/blocks.bin"), x = slurp(d + "/x.bin"),
                          ids = slurp(d + "/ids.bin"), w = slurp(d + "/w.bin");
        eo::Layout lay = eo::layout_of(H, I, fmt);
        std::vector<const uint8_t*> table(E);
        for (int e = 0; e < E; ++e) table[e] = (const uint8_t*)blocks.data() + (size_t)e * lay.bytes;
        std::vector<float> y((size_t)T * H, 0.0f), scratch;
        eo::ThreadPool* p = eo::threadpool_create(threads);
        eo::HostJob jb;
        jb.fmt = fmt; jb.lay = lay; jb.H = H; jb.I = I; jb.T = T; jb.k = k;
        jb.x = (const float*)x.data();
        // bf16 bits of x when every value is a bf16 value (the bf16 route needs them)
        std::vector<uint16_t> xb((size_t)T * H);
        bool exact = true;
        for (size_t i = 0; i < xb.size(); ++i) {
            uint32_t u;
            std::memcpy(&u, (const float*)x.data() + i, 4);
            exact = exact && (u & 0xFFFFu) == 0;
            xb[i] = (uint16_t)(u >> 16);
        }
        jb.xb = exact ? xb.data() : nullptr;
        jb.ids = (const int32_t*)ids.data();
        jb.w = (const float*)w.data();
        jb.experts = table.data();
        jb.y = y.data();
        eo::host_ffn(p, jb, scratch);
        eo::threadpool_destroy(p);
        FILE* o = fopen((d + "/y.bin").c_str(), "wb");
        fwrite(y.data(), sizeof(float), y.size(), o);
        fclose(o);
        return 0;
    }
    return 1;
}
