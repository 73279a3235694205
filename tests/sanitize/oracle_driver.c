/*
 * Drives every function of the CPU oracle on random and corrupted inputs, for a build with
 * AddressSanitizer and UndefinedBehaviorSanitizer (host code only).  Exits non-zero on any
 * failed round trip; the sanitizers abort on any out-of-bounds access or undefined
 * behaviour.  Test infrastructure: built and run by tests/test_sanitizers.py.
 */
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

#include "../../oracle/shannonic_oracle.h"

static uint64_t rng_state = 0x9E3779B97F4A7C15ull;
static uint64_t next_u64(void)
{ /* splitmix64 */
    uint64_t z = (rng_state += 0x9E3779B97F4A7C15ull);
    z = (z ^ (z >> 30)) * 0xBF58476D1CE4E5B9ull;
    z = (z ^ (z >> 27)) * 0x94D049BB133111EBull;
    return z ^ (z >> 31);
}
static uint32_t below(uint32_t m) { return (uint32_t)(next_u64() % m); }

/* a value near the centre with a random spread */
static int8_t draw(int spread)
{
    int v = (int)below(2 * (uint32_t)spread + 1) - spread;
    if (below(50) == 0) v = (int)below(256) - 128;
    if (v < -128) v = -128;
    if (v > 127) v = 127;
    return (int8_t)v;
}

int main(void)
{
    int failures = 0;
    static const int Ks[] = {1, 2, 3, 16, 64, 256};
    static const uint32_t Cs[] = {32, 96, 4096, 8192};
    static const uint32_t Ss[] = {1, 2, 8, 32};
    for (int trial = 0; trial < 120; trial++) {
        uint64_t n = below(5) == 0 ? below(40) : below(20000);
        int K = Ks[below(6)];
        int R = 1 + (int)below(12);
        uint32_t C = Cs[below(4)], S = Ss[below(4)];
        if (S > C) S = C;
        int spread = 1 + (int)below(80);
        int8_t* x = (int8_t*)malloc(n ? n : 1);
        for (uint64_t i = 0; i < n; i++) x[i] = draw(spread);
        uint64_t h[256];
        orc_histogram(x, n, h);
        uint16_t lo[257], f[256];
        int st = orc_build_table(h, K, R, lo, f);
        if (st == ORC_ERR_UNSUPPORTED) { /* more occupied ranges than states */
            free(x);
            continue;
        }
        if (st != ORC_OK) { printf("build %d\n", st); failures++; free(x); continue; }
        uint64_t cap = orc_container_bound(n, K, R, C, S);
        uint8_t* buf = (uint8_t*)malloc(cap);
        uint64_t bytes = 0, bits = 0;
        st = orc_encode(x, n, K, R, lo, f, C, S, buf, cap, &bytes, &bits);
        if (st != ORC_OK) { printf("encode %d\n", st); failures++; }
        int8_t* y = (int8_t*)malloc(n ? n : 1);
        if (st == ORC_OK) {
            st = orc_decode(buf, bytes, y, n);
            if (st != ORC_OK || memcmp(x, y, n) != 0) { printf("decode %d\n", st); failures++; }
            double s[ORC_N_STATS];
            if (orc_stats(h, K, R, lo, f, bits, bytes, n, s) != ORC_OK) failures++;
            /* corruptions: a flipped bit anywhere, a truncated container; only the status
             * matters here, the sanitizers watch every access */
            for (int c = 0; c < 20 && bytes > 0; c++) {
                uint8_t* bad = (uint8_t*)malloc(bytes);
                memcpy(bad, buf, bytes);
                uint64_t at = below((uint32_t)bytes);
                bad[at] ^= (uint8_t)(1u << below(8));
                (void)orc_decode(bad, bytes, y, n);
                (void)orc_decode(bad, at, y, n);
                free(bad);
            }
            /* an encode into a buffer too small */
            if (bytes > 8) (void)orc_encode(x, n, K, R, lo, f, C, S, buf, bytes / 2, &bytes, &bits);
        }
        if (n > 0 && n % 32 == 0) {
            int8_t a[32];
            int32_t yv[20000 / 32 + 1];
            for (int i = 0; i < 32; i++) a[i] = draw(100);
            memset(yv, 0, sizeof(yv));
            if (orc_matvec_i8(x, n, 32, a, yv) != ORC_OK) failures++;
        }
        free(x);
        free(y);
        free(buf);
    }
    /* the DP on small alphabets and the allocation, spread and tables at every size */
    for (int trial = 0; trial < 200; trial++) {
        int A = 1 + (int)below(14), K = 1 + (int)below((uint32_t)A);
        uint64_t h[256] = {0}, cost = 0;
        for (int v = 0; v < A; v++) h[v] = below(4) == 0 ? 0 : below(1000);
        uint16_t lo[257];
        if (orc_dp(h, A, K, lo, &cost) != ORC_OK) failures++;
        int R = 1 + (int)below(12);
        uint64_t cnt[64];
        int Kn = 1 + (int)below(64);
        for (int k = 0; k < Kn; k++) cnt[k] = below(3) == 0 ? 0 : below(100000);
        uint16_t f[64];
        if (orc_normalize(cnt, Kn, R, f) == ORC_OK) {
            uint64_t tot = 0;
            for (int k = 0; k < Kn; k++) tot += f[k];
            if (tot == ((uint64_t)1 << R)) {
                uint16_t rng_[4096], next[4096], enc[4096];
                uint8_t nb[4096];
                if (orc_slot_tables(f, Kn, R, rng_, nb, next, enc) != ORC_OK) failures++;
            }
        }
        (void)orc_lg(next_u64());
    }
    printf("oracle driver: %d failures\n", failures);
    return failures != 0;
}
