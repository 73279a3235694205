/*
 * Shannonic codec -- CPU ORACLE (test infrastructure only).
 *
 * Plain, slow, single-threaded C.  Only the test suite, the smoke check and the
 * benchmark's CPU-baseline leg may load it; the HIP library never does, and the two
 * share no code, header, table or constant.  See shannonic_oracle.c for the method,
 * the citations and the readings taken where the source pages are silent.
 */
#ifndef SHANNONIC_ORACLE_H
#define SHANNONIC_ORACLE_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* status codes (same meaning as the library's) */
#define ORC_OK 0
#define ORC_ERR_INVALID (-1)
#define ORC_ERR_UNSUPPORTED (-2)
#define ORC_ERR_SYMBOL (-3)
#define ORC_ERR_CORRUPT (-4)
#define ORC_ERR_SMALL (-5)

#define ORC_LG_FRAC 24   /* fractional bits of the fixed-point binary logarithm */
#define ORC_N_STATS 14   /* number of doubles written by orc_stats */

uint64_t orc_lg(uint64_t x);
void orc_histogram(const int8_t* x, uint64_t n, uint64_t* h256);
int orc_dp(const uint64_t* h, int A, int K, uint16_t* lo, uint64_t* cost);
int orc_normalize(const uint64_t* count, int K, int log2_L, uint16_t* freq);
int orc_build_table(const uint64_t* h256, int K, int log2_L, uint16_t* lo, uint16_t* freq);
int orc_spread(const uint16_t* freq, int K, int log2_L, uint16_t* slot_range);
int orc_slot_tables(const uint16_t* freq, int K, int log2_L, uint16_t* slot_range,
                    uint8_t* slot_nb, uint16_t* slot_next, uint16_t* enc_slot);
uint64_t orc_container_bound(uint64_t n, int K, int log2_L, uint32_t C, uint32_t S);
int orc_encode(const int8_t* x, uint64_t n, int K, int log2_L, const uint16_t* lo,
               const uint16_t* freq, uint32_t C, uint32_t S, uint8_t* out, uint64_t cap,
               uint64_t* out_bytes, uint64_t* payload_bits);
int orc_decode(const uint8_t* in, uint64_t nbytes, int8_t* y, uint64_t n);
int orc_stats(const uint64_t* h256, int K, int log2_L, const uint16_t* lo,
              const uint16_t* freq, uint64_t payload_bits, uint64_t container_bytes,
              uint64_t n, double* out);
/* The consumer of a decoded matrix in the fused decode: y[r] += sum_c w[r*cols + c] * a[c]
 * for every row r < n / cols, wrapping like int32 addition. */
int orc_matvec_i8(const int8_t* w, uint64_t n, uint32_t cols, const int8_t* a, int32_t* y);

#ifdef __cplusplus
}
#endif
#endif
