// Drives the library's host-side code -- the table build (histogram -> DP split -> state
// allocation -> spread -> kernel tables, device-table images, container headers) and the
// host entry points of the C ABI that need no GPU (sh_table_from_histogram, sh_stats,
// sh_stats_batch, sh_tables_from_bytes, the size queries) -- on random and malformed
// inputs, for a build with AddressSanitizer and UndefinedBehaviorSanitizer.  The GPU
// launches are replaced by stubs that report a HIP error.  Test infrastructure: built and
// run by tests/test_sanitizers.py.
#include <cstdio>
#include <cstring>
#include <vector>

#include "../../entropy_coding_quantized_amd/csrc/codec_internal.hpp"

namespace shn {
sh_status launch_histogram(const HistArgs&, uint32_t, void*) { return SH_ERR_HIP; }
sh_status launch_build_tables(const BuildArgs&, void*) { return SH_ERR_HIP; }
sh_status launch_decode(const CodecArgs&, uint32_t, void*) { return SH_ERR_HIP; }
sh_status launch_decode_halves(const CodecArgs&, uint32_t, void*) { return SH_ERR_HIP; }
sh_status launch_decode_wide_halves(const CodecArgs&, uint32_t, void*) { return SH_ERR_HIP; }
sh_status launch_decode_matvec(const CodecArgs&, uint32_t, void*) { return SH_ERR_HIP; }
sh_status launch_decode_matvec_rows(const CodecArgs&, uint32_t, bool, void*) { return SH_ERR_HIP; }
sh_status launch_encode(const CodecArgs&, uint32_t, uint32_t, bool, void*, void*, void*, void*) {
    return SH_ERR_HIP;
}
}  // namespace shn

static uint64_t rng_state = 0x2545F4914F6CDD1Dull;
static uint64_t next_u64() {  // splitmix64
    uint64_t z = (rng_state += 0x9E3779B97F4A7C15ull);
    z = (z ^ (z >> 30)) * 0xBF58476D1CE4E5B9ull;
    z = (z ^ (z >> 27)) * 0x94D049BB133111EBull;
    return z ^ (z >> 31);
}
static uint32_t below(uint32_t m) { return (uint32_t)(next_u64() % m); }

int main() {
    int failures = 0;
    std::vector<uint32_t> dt(shn::kDTDwords);
    for (int trial = 0; trial < 400; ++trial) {
        uint64_t h[256] = {0};
        const uint32_t occupied = 1 + below(256);
        for (uint32_t i = 0; i < occupied; ++i) h[below(256)] += 1 + below(1u << below(20));
        if (below(20) == 0) std::memset(h, 0, sizeof(h));
        sh_params p{1 + below(256), 1 + below(12), 32 * (1 + below(512)), 32};
        sh_table t;
        const sh_status st = sh_table_from_histogram(h, &p, &t);
        if (st != SH_OK) {
            if (st != SH_ERR_UNSUPPORTED) ++failures;
            continue;
        }
        sh_stats_t s;
        if (sh_stats(&t, 1000, 5000, 900, &s) != SH_OK) ++failures;
        if (sh_stats_batch(&t, 1, nullptr, nullptr, nullptr, &s) != SH_OK) ++failures;
        if (t.n == 0) continue;
        shn::SlotTables slots;
        if (shn::derive_slots(t, &slots) != SH_OK) {
            ++failures;
            continue;
        }
        if (t.log2_L <= 8) {
            shn::make_device_table(t, &slots, p.chunk_symbols, p.streams, dt.data());
            sh_table back;
            int32_t ts = 0;
            if (sh_tables_from_bytes(dt.data(), 1, &back, &ts) != SH_OK || ts != SH_OK ||
                std::memcmp(back.lo, t.lo, sizeof(t.lo)) != 0)
                ++failures;
            // a device-table image with random bytes is refused, never read out of bounds
            std::vector<uint32_t> junk(dt);
            for (int k = 0; k < 8; ++k) junk[below(shn::kDTDwords)] = (uint32_t)next_u64();
            (void)sh_tables_from_bytes(junk.data(), 1, &back, &ts);
            (void)sh_encode_bound(below(1u << 30), &p);
            (void)sh_encode_workspace(below(1u << 30), &p);
        }
        // malformed tables are refused by every host entry point
        sh_table bad = t;
        bad.lo[below(bad.K + 1)] = (uint16_t)below(300);
        bad.freq[below(bad.K)] += (uint16_t)below(3);
        (void)sh_stats(&bad, 10, 10, 10, &s);
    }
    std::printf("host driver: %d failures\n", failures);
    return failures != 0;
}
