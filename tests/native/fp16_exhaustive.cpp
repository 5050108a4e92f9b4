// Exhaustive pin of the oracle's fp32 -> fp16 conversion against the host's
// F16C instruction (round to nearest even).  Test infrastructure: loads
// liboracle.so given on the command line, compares all 2^32 encodings.
#include <dlfcn.h>
#include <immintrin.h>

#include <atomic>
#include <cstdint>
#include <cstdio>
#include <cstring>
#include <thread>
#include <vector>

typedef uint16_t (*f2h_t)(float);

int main(int argc, char** argv) {
    if (argc < 2) return 2;
    void* h = dlopen(argv[1], RTLD_NOW);
    if (!h) { std::printf("dlopen failed\n"); return 2; }
    f2h_t f2h = reinterpret_cast<f2h_t>(dlsym(h, "oracle_float_to_half"));
    if (!f2h) return 2;
    const int nt = 8;
    std::atomic<uint64_t> bad{0};
    std::vector<std::thread> th;
    for (int t = 0; t < nt; ++t) {
        th.emplace_back([&, t] {
            const uint64_t lo = (uint64_t(1) << 32) * t / nt, hi = (uint64_t(1) << 32) * (t + 1) / nt;
            uint64_t local = 0;
            for (uint64_t b = lo; b < hi; ++b) {
                uint32_t u = static_cast<uint32_t>(b);
                float f;
                std::memcpy(&f, &u, 4);
                const uint16_t ref = static_cast<uint16_t>(_cvtss_sh(f, _MM_FROUND_TO_NEAREST_INT));
                if (f2h(f) != ref) {
                    if (local < 4) std::printf("mismatch %08x: oracle %04x f16c %04x\n", u, f2h(f), ref);
                    ++local;
                }
            }
            bad += local;
        });
    }
    for (auto& x : th) x.join();
    std::printf("mismatches %llu\n", static_cast<unsigned long long>(bad.load()));
    return bad.load() == 0 ? 0 : 1;
}
