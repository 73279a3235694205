/*
 * Shannonic codec -- CPU ORACLE (test infrastructure only).
 *
 * A plain, slow, single-threaded C implementation of what the Shannonic codec
 * computes.  It is the correctness reference for the HIP library: only the test
 * suite, the smoke check and the benchmark's CPU-baseline leg may load it.  The
 * product path never calls it, and the two share no code, header, table or constant.
 *
 * Method: "Shannonic: Efficient Entropy-Optimal Compression for ML Workloads"
 * (MLSys 2026), as summarised in the talk notes, sections
 *   "Shannonic approach: range partition + ANS",
 *   "Theoretical basis: Theorem 1"                       (paper section 4),
 *   "Preprocessing: range selection by dynamic programming" (paper section 4.1),
 *   "Runtime encoding/decoding"                          (paper section 4.2, Algorithm 2),
 *   "Evaluation: compression ratio"                      (paper section 5).
 *
 * In short: a histogram of the 8-bit values is cut into K contiguous ranges by dynamic
 * programming; every value becomes (range index s, offset o); s is coded by a tabled
 * ANS (tANS) coder with L = 2^R states built from the range probabilities, o is
 * written as w_s = ceil(log2 |range s|) raw bits.
 *
 * Readings taken where the pages are silent (each one is restated where it is used):
 *   R1  values are offset-binary: u = x + 128, so ranges are contiguous in value.
 *   R2  the DP cost of a range is its ideal range-id cost plus its offset bits,
 *       evaluated in integers with a fixed-point base-2 logarithm (orc_lg, 24
 *       fractional bits, computed by repeated squaring) so that every
 *       implementation of the DP reaches the same partition, ties included.
 *   R3  frequencies: every occupied range starts at 1; the remaining states go one by
 *       one to the range with the largest gain in N_k * log2 f_k (smallest k on ties).
 *   R4  slot spread: Duda's "precise" spread, slots ordered by (2j+1)/(2 f_k).
 *   R5  bitstream: chunks of C symbols, S interleaved lanes (symbol i of a chunk goes
 *       to lane i mod S, step i div S), one tANS state per lane; each chunk is a
 *       little-endian LSB-first bit string of the lanes' initial states followed by
 *       the fields in (step, lane) order, padded with zeros to a whole number of size
 *       units (a unit is 2^u bytes, the smallest that lets every chunk's size fit 16
 *       bits; one byte at the pages' parameters).  Chunks follow each other byte by byte;
 *       the index holds every chunk's size in units and, every 64 chunks, a 32-bit offset.
 *       A field is the offset in its low w_s bits with the state bits above it.
 */
#include "shannonic_oracle.h"

#include <math.h>
#include <stdlib.h>
#include <string.h>

/* ------------------------------------------------------------------------------ */
/* small helpers                                                                   */
/* ------------------------------------------------------------------------------ */

/* floor(log2(x)) for x >= 1: position of the highest set bit */
static int floor_log2_u64(uint64_t x)
{
    int e = -1;
    while (x) {
        x >>= 1;
        e++;
    }
    return e;
}

/* ceil(log2(m)) for m >= 1: the smallest w with 2^w >= m (0 for m = 1) */
static int ceil_log2_u64(uint64_t m)
{
    int w = 0;
    while (((uint64_t)1 << w) < m) w++;
    return w;
}

/* ------------------------------------------------------------------------------ */
/* R2: fixed-point binary logarithm                                                */
/* ------------------------------------------------------------------------------ */

/*
 * orc_lg(x) ~= 2^24 * log2(x) for integer x >= 1 (0 for x = 0).
 *
 * The classic digit-by-digit method: write x = 2^e * m with m in [1, 2); each
 * fractional bit of log2(m) is 1 exactly when m^2 >= 2, in which case m^2 / 2
 * carries on, else m^2 does.  m is held as a Q1.63 fixed-point number and each
 * square is truncated back to 64 bits, so the result is a fixed function of x that
 * any implementation reproduces bit for bit.  It is never above the true value by
 * more than rounding of the last bit and never below it by more than 2^-24 + 2^-30
 * (checked against the math library in the tests).
 */
uint64_t orc_lg(uint64_t x)
{
    if (x == 0) return 0;
    int e = floor_log2_u64(x);
    uint64_t m = x << (63 - e); /* Q1.63, top bit set */
    uint64_t frac = 0;
    for (int b = 0; b < ORC_LG_FRAC; b++) {
        unsigned __int128 p = (unsigned __int128)m * m; /* Q2.126 */
        frac <<= 1;
        if (p >> 127) {
            frac |= 1;
            m = (uint64_t)(p >> 64);
        } else {
            m = (uint64_t)(p >> 63);
        }
    }
    return ((uint64_t)e << ORC_LG_FRAC) + frac;
}

/* ------------------------------------------------------------------------------ */
/* histogram (paper section 4.1): h[u] over the alphabet [0, 255], u = x + 128 (R1) */
/* ------------------------------------------------------------------------------ */

void orc_histogram(const int8_t* x, uint64_t n, uint64_t* h256)
{
    for (int u = 0; u < 256; u++) h256[u] = 0;
    for (uint64_t i = 0; i < n; i++) h256[(int)x[i] + 128]++;
}

/* ------------------------------------------------------------------------------ */
/* range selection by dynamic programming (paper section 4.1)                      */
/* ------------------------------------------------------------------------------ */

/*
 * Cost, in units of 2^-24 bit, of coding the N_R symbols whose values lie in
 * [j, i): each costs its ideal range-id length log2(N / N_R) plus the w = ceil(log2
 * (i - j)) raw offset bits.  This is the quantity the DP minimises (R2); summed over a
 * partition it is N * (H(P) + sum_k P_k w_k), Theorem 1 without the D_KL(P||Q) term,
 * which depends on all ranges jointly through the state allocation.
 */
static uint64_t range_cost(const uint64_t* h, int j, int i, uint64_t N)
{
    uint64_t NR = 0;
    for (int v = j; v < i; v++) NR += h[v];
    if (NR == 0) return 0;
    uint64_t w = (uint64_t)ceil_log2_u64((uint64_t)(i - j));
    return NR * (orc_lg(N) - orc_lg(NR)) + NR * (w << ORC_LG_FRAC);
}

/*
 * Split the alphabet [0, A) into exactly K contiguous, non-empty ranges minimising the
 * summed range_cost: C[i][k] = min over j < i of C[j][k-1] + Cost(j, i - 1) (the
 * notes' recurrence, with the range [j, i) written half-open), then backtrack from
 * C[A][K].  j is scanned upward and replaced only on a strictly smaller cost, so ties
 * keep the smallest j.  Ranges holding no symbols are allowed and cost nothing.
 * Writes lo[0..K] with lo[0] = 0 and lo[K] = A; range k is [lo[k], lo[k+1]).
 */
int orc_dp(const uint64_t* h, int A, int K, uint16_t* lo, uint64_t* cost)
{
    if (A < 1 || A > 256 || K < 1 || K > A) return ORC_ERR_INVALID;
    uint64_t N = 0;
    for (int v = 0; v < A; v++) N += h[v];
    if (N >= ((uint64_t)1 << 32)) return ORC_ERR_UNSUPPORTED;

    const uint64_t INF = UINT64_MAX;
    uint64_t* C = (uint64_t*)malloc(sizeof(uint64_t) * (size_t)(A + 1) * (size_t)(K + 1));
    int* back = (int*)malloc(sizeof(int) * (size_t)(A + 1) * (size_t)(K + 1));
    if (!C || !back) {
        free(C);
        free(back);
        return ORC_ERR_INVALID;
    }
#define CI(i, k) C[(size_t)(i) * (size_t)(K + 1) + (size_t)(k)]
#define BI(i, k) back[(size_t)(i) * (size_t)(K + 1) + (size_t)(k)]
    for (int i = 0; i <= A; i++)
        for (int k = 0; k <= K; k++) {
            CI(i, k) = INF;
            BI(i, k) = -1;
        }
    CI(0, 0) = 0;
    for (int k = 1; k <= K; k++) {
        for (int i = k; i <= A; i++) {
            for (int j = k - 1; j < i; j++) {
                if (CI(j, k - 1) == INF) continue;
                uint64_t c = CI(j, k - 1) + range_cost(h, j, i, N);
                if (c < CI(i, k)) {
                    CI(i, k) = c;
                    BI(i, k) = j;
                }
            }
        }
    }
    if (cost) *cost = CI(A, K);
    int i = A;
    lo[K] = (uint16_t)A;
    for (int k = K; k >= 1; k--) {
        int j = BI(i, k);
        lo[k - 1] = (uint16_t)j;
        i = j;
    }
#undef CI
#undef BI
    free(C);
    free(back);
    return ORC_OK;
}

/* ------------------------------------------------------------------------------ */
/* state allocation (R3): q_k = f_k / L from the range probabilities p_k = N_k / N   */
/* ------------------------------------------------------------------------------ */

/*
 * The notes only say the 128-entry table is built from p_k = N_k / N (paper section
 * 4.1).  Reading R3: give each occupied range one state, then hand the remaining
 * states out one at a time to the range whose count gains most, gain_k =
 * N_k * (log2(f_k + 1) - log2(f_k)), scanning k upward and keeping the first maximum.
 * Every step adds the largest available decrease of sum_k N_k * -log2(f_k / L), a
 * separable concave objective, so the result minimises D_KL(P || Q) -- the quantisation
 * loss Theorem 1 charges.  The logarithm is orc_lg (R2).  With no symbols at all every
 * frequency stays 0.
 */
int orc_normalize(const uint64_t* count, int K, int log2_L, uint16_t* freq)
{
    if (K < 1 || K > 4096 || log2_L < 1 || log2_L > 12) return ORC_ERR_INVALID;
    uint64_t L = (uint64_t)1 << log2_L;
    uint64_t used = 0;
    for (int k = 0; k < K; k++) {
        freq[k] = count[k] ? 1 : 0;
        used += freq[k];
    }
    if (used == 0) return ORC_OK;
    if (used > L) return ORC_ERR_UNSUPPORTED;
    for (; used < L; used++) {
        int best = -1;
        uint64_t best_gain = 0;
        for (int k = 0; k < K; k++) {
            if (!count[k]) continue;
            uint64_t gain = count[k] * (orc_lg((uint64_t)freq[k] + 1) - orc_lg(freq[k]));
            if (best < 0 || gain > best_gain) {
                best = k;
                best_gain = gain;
            }
        }
        freq[best]++;
    }
    return ORC_OK;
}

/* the whole offline step: DP over the 256 values, then the state allocation */
int orc_build_table(const uint64_t* h256, int K, int log2_L, uint16_t* lo, uint16_t* freq)
{
    if (K < 1 || K > 256 || log2_L < 1 || log2_L > 12) return ORC_ERR_INVALID;
    int st = orc_dp(h256, 256, K, lo, NULL);
    if (st != ORC_OK) return st;
    uint64_t count[256];
    for (int k = 0; k < K; k++) {
        count[k] = 0;
        for (int u = lo[k]; u < lo[k + 1]; u++) count[k] += h256[u];
    }
    return orc_normalize(count, K, log2_L, freq);
}

/* ------------------------------------------------------------------------------ */
/* R4: slot spread and the tANS tables                                             */
/* ------------------------------------------------------------------------------ */

typedef struct {
    int k;        /* range */
    uint64_t j;   /* occurrence index within the range */
    uint64_t fk;  /* frequency of the range */
} spread_key;

/* order by (2j+1)/(2 f_k), compared exactly by cross-multiplication; ties: smaller k */
static int spread_cmp(const void* pa, const void* pb)
{
    const spread_key* a = (const spread_key*)pa;
    const spread_key* b = (const spread_key*)pb;
    uint64_t lhs = (2 * a->j + 1) * b->fk;
    uint64_t rhs = (2 * b->j + 1) * a->fk;
    if (lhs < rhs) return -1;
    if (lhs > rhs) return 1;
    return (a->k > b->k) - (a->k < b->k);
}

/*
 * slot_range[i] = range owning tANS slot i, i in [0, L).  Reading R4 (the pages do not
 * say how symbols are laid out over the states): range k takes f_k slots at the
 * positions its keys (2j+1)/(2 f_k), j < f_k, fall in once all keys are sorted -- an
 * evenly spaced spread for every range.
 */
int orc_spread(const uint16_t* freq, int K, int log2_L, uint16_t* slot_range)
{
    if (K < 1 || K > 4096 || log2_L < 1 || log2_L > 12) return ORC_ERR_INVALID;
    uint64_t L = (uint64_t)1 << log2_L, total = 0;
    for (int k = 0; k < K; k++) total += freq[k];
    if (total != L) return ORC_ERR_INVALID;
    spread_key* keys = (spread_key*)malloc(sizeof(spread_key) * (size_t)L);
    if (!keys) return ORC_ERR_INVALID;
    uint64_t at = 0;
    for (int k = 0; k < K; k++)
        for (uint64_t j = 0; j < freq[k]; j++) {
            keys[at].k = k;
            keys[at].j = j;
            keys[at].fk = freq[k];
            at++;
        }
    qsort(keys, (size_t)L, sizeof(spread_key), spread_cmp);
    for (uint64_t i = 0; i < L; i++) slot_range[i] = (uint16_t)keys[i].k;
    free(keys);
    return ORC_OK;
}

/*
 * The decode and encode tables, from the tANS definition (paper section 4.2).
 * The state X lives in [L, 2L); slot i = X - L.  If slot i is the j-th slot (in slot
 * order) of range s, decoding from it yields s and the sub-state x_s = f_s + j in
 * [f_s, 2 f_s); the decoder then reads nb = R - floor(log2 x_s) bits b and moves to
 * X' = (x_s << nb) + b, i.e. slot slot_next[i] + b with slot_next[i] = (x_s << nb) - L.
 * The encoder inverts this: enc_slot[cum_s + j] = i, with cum_s = f_0 + ... + f_{s-1}.
 * (These are the pages' decTable and encTable; base, nb and start are derived where
 * they are used.)
 */
int orc_slot_tables(const uint16_t* freq, int K, int log2_L, uint16_t* slot_range,
                    uint8_t* slot_nb, uint16_t* slot_next, uint16_t* enc_slot)
{
    int st = orc_spread(freq, K, log2_L, slot_range);
    if (st != ORC_OK) return st;
    uint64_t L = (uint64_t)1 << log2_L;
    uint64_t* seen = (uint64_t*)calloc((size_t)K, sizeof(uint64_t));
    uint64_t* cum = (uint64_t*)calloc((size_t)K + 1, sizeof(uint64_t));
    if (!seen || !cum) {
        free(seen);
        free(cum);
        return ORC_ERR_INVALID;
    }
    for (int k = 0; k < K; k++) cum[k + 1] = cum[k] + freq[k];
    for (uint64_t i = 0; i < L; i++) {
        int s = slot_range[i];
        uint64_t j = seen[s]++;
        uint64_t xs = (uint64_t)freq[s] + j;
        int nb = log2_L - floor_log2_u64(xs);
        slot_nb[i] = (uint8_t)nb;
        slot_next[i] = (uint16_t)((xs << nb) - L);
        enc_slot[cum[s] + j] = (uint16_t)i;
    }
    free(seen);
    free(cum);
    return ORC_OK;
}

/* ------------------------------------------------------------------------------ */
/* R5: container                                                                   */
/* ------------------------------------------------------------------------------ */
/*
 * Byte layout (all integers little-endian):
 *   0   "SHN1"          magic
 *   4   u8  version     3
 *   5   u8  R           log2 of the number of tANS states L
 *   6   u16 K           number of ranges
 *   8   u64 n           number of symbols
 *   16  u32 C           symbols per chunk
 *   20  u32 S           interleaved lanes per chunk
 *   24  u32 n_chunks    ceil(n / C)
 *   28  u32 index_at    byte offset of the chunk index = header size
 *   32  u16 freq[K]     state counts f_k (sum L; all 0 only when n = 0)
 *   32+2K u8 lo[1..K-1] range starts (lo[0] = 0, lo[K] = 256 are implied)
 *   zero padding up to index_at = 4 * ceil((32 + 3K - 1) / 4)
 *   index_at: u32 goff[G + 1], G = ceil(n_chunks / 64): byte offset, from the payload
 *             start, of chunk 64g; goff[G] = the payload's size in bytes
 *             then u16 size[n_chunks], every chunk's size in units, then a zero u16 when
 *             n_chunks is odd
 *   payload: the chunks back to back (chunk c starts at goff[c / 64] plus the sizes of
 *            the chunks before it in its group of 64), then zero bytes up to a multiple
 *            of 4 bytes (the container's end)
 * The unit is 2^u bytes, u the smallest with ceil(B / 2^u) <= 65535 where B is the largest
 * chunk a valid stream can hold (chunk_bound_bytes of a whole chunk).
 */

static uint64_t header_bytes(int K) { return ((uint64_t)(32 + 3 * K - 1) + 3) / 4 * 4; }

static void put_u16(uint8_t* p, uint64_t v)
{
    p[0] = (uint8_t)v;
    p[1] = (uint8_t)(v >> 8);
}
static void put_u32(uint8_t* p, uint64_t v)
{
    for (int b = 0; b < 4; b++) p[b] = (uint8_t)(v >> (8 * b));
}
static void put_u64(uint8_t* p, uint64_t v)
{
    for (int b = 0; b < 8; b++) p[b] = (uint8_t)(v >> (8 * b));
}
static uint64_t get_le(const uint8_t* p, int bytes)
{
    uint64_t v = 0;
    for (int b = bytes - 1; b >= 0; b--) v = (v << 8) | p[b];
    return v;
}

/* bit b of the stream is bit (b mod 8) of byte b / 8; a value's bit 0 is written first */
static void write_bits(uint8_t* buf, uint64_t pos, uint64_t value, int len)
{
    for (int b = 0; b < len; b++)
        if ((value >> b) & 1) buf[(pos + (uint64_t)b) >> 3] |= (uint8_t)(1u << ((pos + (uint64_t)b) & 7));
}
static uint64_t read_bits(const uint8_t* buf, uint64_t pos, int len)
{
    uint64_t v = 0;
    for (int b = 0; b < len; b++)
        v |= (uint64_t)((buf[(pos + (uint64_t)b) >> 3] >> ((pos + (uint64_t)b) & 7)) & 1) << b;
    return v;
}

/* the largest chunk a valid stream can hold: every field at its longest, 8 + R bits */
static uint64_t chunk_bound_bits(uint64_t nc, int log2_L, uint32_t S)
{
    uint64_t lanes = nc < S ? nc : S;
    return lanes * (uint64_t)log2_L + nc * (uint64_t)(8 + log2_L);
}

/* log2 of the size unit in bytes: the smallest u with ceil(B / 2^u) <= 65535, B the bound
 * of a whole chunk in bytes */
static int unit_log2(uint32_t C, int log2_L, uint32_t S)
{
    uint64_t B = (chunk_bound_bits(C, log2_L, S) + 7) / 8;
    int u = 0;
    while ((B + ((uint64_t)1 << u) - 1) >> u > 65535) u++;
    return u;
}

/* bytes of the index: goff[G + 1] and size[n_chunks], padded to 4 bytes */
static uint64_t index_bytes(uint64_t nch)
{
    uint64_t groups = (nch + 63) / 64;
    return 4 * (groups + 1) + (2 * nch + 3) / 4 * 4;
}

uint64_t orc_container_bound(uint64_t n, int K, int log2_L, uint32_t C, uint32_t S)
{
    if (C == 0 || S == 0) return 0;
    uint64_t nch = (n + C - 1) / C;
    uint64_t unit = (uint64_t)1 << unit_log2(C, log2_L, S);
    uint64_t total = 0;
    for (uint64_t c = 0; c < nch; c++) {
        uint64_t nc = (c + 1 < nch) ? C : n - c * (uint64_t)C;
        total += (chunk_bound_bits(nc, log2_L, S) + 8 * unit - 1) / (8 * unit) * unit;
    }
    return header_bytes(K) + index_bytes(nch) + (total + 3) / 4 * 4;
}

/* range of value u: the k with lo[k] <= u < lo[k+1] */
static int range_of(const uint16_t* lo, int K, int u)
{
    for (int k = 0; k < K; k++)
        if (u >= lo[k] && u < lo[k + 1]) return k;
    return -1;
}

static int check_table(int K, int log2_L, const uint16_t* lo, const uint16_t* freq, uint64_t n)
{
    if (K < 1 || K > 256 || log2_L < 1 || log2_L > 12) return ORC_ERR_INVALID;
    if (lo[0] != 0 || lo[K] != 256) return ORC_ERR_INVALID;
    for (int k = 0; k < K; k++)
        if (lo[k + 1] <= lo[k]) return ORC_ERR_INVALID;
    uint64_t total = 0;
    for (int k = 0; k < K; k++) total += freq[k];
    if (total != ((uint64_t)1 << log2_L) && !(total == 0 && n == 0)) return ORC_ERR_INVALID;
    return ORC_OK;
}

/*
 * Encode n values into a container (paper section 4.2, Algorithm 2, with the chunk
 * layout of R5).  Per symbol, in constant time: s = rangeId[u]; the offset o = u -
 * base[s] goes out in w_s bits; then the k state bits that bring X into [f_s, 2 f_s);
 * then the state moves through encTable.  tANS encodes backwards, so each lane runs
 * from its last symbol to its first, starting in state L (slot 0); its final state is
 * the decoder's initial state.  The state bits of the first symbol it encodes (the lane's
 * last) are the low bits of L, all zero, so they are left out and the decoder implies
 * them: about H(P) bits less a lane.  The fields are then written in decoding order.
 * payload_bits receives the summed field lengths (initial states and padding excluded).
 */
int orc_encode(const int8_t* x, uint64_t n, int K, int log2_L, const uint16_t* lo,
               const uint16_t* freq, uint32_t C, uint32_t S, uint8_t* out, uint64_t cap,
               uint64_t* out_bytes, uint64_t* payload_bits)
{
    int st = check_table(K, log2_L, lo, freq, n);
    if (st != ORC_OK) return st;
    if (C == 0 || S == 0 || S > C) return ORC_ERR_INVALID;
    const uint64_t L = (uint64_t)1 << log2_L;
    const uint64_t nch = (n + C - 1) / C;
    if (nch > 0xFFFFFFFEull) return ORC_ERR_UNSUPPORTED;
    const uint64_t bound = orc_container_bound(n, K, log2_L, C, S);
    if (bound - header_bytes(K) - index_bytes(nch) > 0xFFFFFFFFull) return ORC_ERR_UNSUPPORTED;
    if (cap < header_bytes(K) + index_bytes(nch)) return ORC_ERR_SMALL;
    const int ul = unit_log2(C, log2_L, S);
    const uint64_t unit = (uint64_t)1 << ul;

    uint16_t slot_range[4096], slot_next[4096], enc_slot[4096];
    uint8_t slot_nb[4096];
    uint64_t cum[257];
    if (n > 0) {
        st = orc_slot_tables(freq, K, log2_L, slot_range, slot_nb, slot_next, enc_slot);
        if (st != ORC_OK) return st;
    }
    cum[0] = 0;
    for (int k = 0; k < K; k++) cum[k + 1] = cum[k] + freq[k];

    /* header */
    uint64_t hb = header_bytes(K);
    memset(out, 0, hb);
    out[0] = 'S';
    out[1] = 'H';
    out[2] = 'N';
    out[3] = '1';
    out[4] = 3;
    out[5] = (uint8_t)log2_L;
    put_u16(out + 6, (uint64_t)K);
    put_u64(out + 8, n);
    put_u32(out + 16, C);
    put_u32(out + 20, S);
    put_u32(out + 24, nch);
    put_u32(out + 28, hb);
    for (int k = 0; k < K; k++) put_u16(out + 32 + 2 * k, freq[k]);
    for (int k = 1; k < K; k++) out[32 + 2 * K + (k - 1)] = (uint8_t)lo[k];

    uint8_t* goff = out + hb;                      /* u32 per group of 64 chunks, + 1 */
    uint8_t* sizes = goff + 4 * ((nch + 63) / 64 + 1);  /* u16 per chunk */
    uint64_t payload_at = hb + index_bytes(nch);
    uint64_t off = 0, fields_total = 0;
    memset(goff, 0, index_bytes(nch));

    uint64_t* field = (uint64_t*)malloc(sizeof(uint64_t) * (size_t)(C ? C : 1));
    int* flen = (int*)malloc(sizeof(int) * (size_t)(C ? C : 1));
    uint64_t* init = (uint64_t*)malloc(sizeof(uint64_t) * (size_t)S);
    if (!field || !flen || !init) {
        free(field);
        free(flen);
        free(init);
        return ORC_ERR_INVALID;
    }
    st = ORC_OK;
    for (uint64_t c = 0; c < nch && st == ORC_OK; c++) {
        uint64_t first = c * (uint64_t)C;
        uint64_t nc = (c + 1 < nch) ? C : n - first;
        uint64_t lanes = nc < S ? nc : S;
        /* each lane, backwards over its own symbols */
        for (uint64_t l = 0; l < lanes && st == ORC_OK; l++) {
            uint64_t T = (nc - l + S - 1) / S;
            uint64_t X = L;
            for (uint64_t t = T; t-- > 0;) {
                uint64_t i = t * S + l;
                int u = (int)x[first + i] + 128;
                int s = range_of(lo, K, u);
                if (freq[s] == 0) {
                    st = ORC_ERR_SYMBOL;
                    break;
                }
                uint64_t o = (uint64_t)(u - lo[s]);
                int w = ceil_log2_u64((uint64_t)(lo[s + 1] - lo[s]));
                int k = 0;
                while ((X >> k) >= 2 * (uint64_t)freq[s]) k++;
                field[i] = o | ((X & (((uint64_t)1 << k) - 1)) << w);
                /* the lane's last value (encoded first, from X = L): its k state bits are
                 * the low bits of L, all zero, and the decoder implies them */
                flen[i] = t + 1 == T ? w : w + k;
                X = L + enc_slot[cum[s] + ((X >> k) - freq[s])];
            }
            init[l] = X - L;
        }
        if (st != ORC_OK) break;
        /* lay the chunk out in decoding order */
        uint64_t bits = lanes * (uint64_t)log2_L;
        for (uint64_t i = 0; i < nc; i++) bits += (uint64_t)flen[i];
        uint64_t units = (bits + 8 * unit - 1) / (8 * unit);
        uint64_t bytes = units * unit;
        if (payload_at + off + bytes > cap) {
            st = ORC_ERR_SMALL;
            break;
        }
        uint8_t* chunk = out + payload_at + off;
        memset(chunk, 0, bytes);
        uint64_t pos = 0;
        for (uint64_t l = 0; l < lanes; l++) {
            write_bits(chunk, pos, init[l], log2_L);
            pos += (uint64_t)log2_L;
        }
        for (uint64_t i = 0; i < nc; i++) { /* i = t*S + l runs in (step, lane) order */
            write_bits(chunk, pos, field[i], flen[i]);
            pos += (uint64_t)flen[i];
            fields_total += (uint64_t)flen[i];
        }
        if (c % 64 == 0) put_u32(goff + 4 * (c / 64), off);
        put_u16(sizes + 2 * c, units);
        off += bytes;
    }
    if (st == ORC_OK) {
        put_u32(goff + 4 * ((nch + 63) / 64), off);
        uint64_t padded = (off + 3) / 4 * 4;       /* the container ends on 4 bytes */
        if (payload_at + padded > cap) st = ORC_ERR_SMALL;
        else {
            memset(out + payload_at + off, 0, padded - off);
            off = padded;
        }
    }
    free(field);
    free(flen);
    free(init);
    if (st != ORC_OK) return st;
    if (out_bytes) *out_bytes = payload_at + off;
    if (payload_bits) *payload_bits = fields_total;
    return ORC_OK;
}

/*
 * Decode a container into n values (paper section 4.2): from state X, decTable[X]
 * gives the range s and the state bit count; the field's low w_s bits are the offset o
 * and x = base[s] + o.  A lane's last field is the offset alone (its state bits are
 * zero, implied).  A stream is valid only if the header is consistent, every offset lies
 * inside its range, every lane ends in slot 0 (the encoder's start state), every chunk's
 * bits end in its last size unit with zero padding after them, every group offset equals
 * the one before it plus the sizes of the group's chunks, and the container ends right
 * after the payload's zero padding to 4 bytes.
 */
int orc_decode(const uint8_t* in, uint64_t nbytes, int8_t* y, uint64_t n)
{
    if (nbytes < 32) return ORC_ERR_CORRUPT;
    if (in[0] != 'S' || in[1] != 'H' || in[2] != 'N' || in[3] != '1' || in[4] != 3)
        return ORC_ERR_CORRUPT;
    int R = in[5];
    int K = (int)get_le(in + 6, 2);
    uint64_t hn = get_le(in + 8, 8);
    uint64_t C = get_le(in + 16, 4), S = get_le(in + 20, 4), nch = get_le(in + 24, 4);
    uint64_t hb = get_le(in + 28, 4);
    if (hn != n) return ORC_ERR_INVALID;
    if (R < 1 || R > 12 || K < 1 || K > 256 || C == 0 || S == 0 || S > C) return ORC_ERR_CORRUPT;
    if (hb != header_bytes(K) || nch != (n + C - 1) / C) return ORC_ERR_CORRUPT;
    if (nbytes < hb + index_bytes(nch)) return ORC_ERR_CORRUPT;
    uint16_t lo[257], freq[256];
    lo[0] = 0;
    lo[K] = 256;
    for (int k = 0; k < K; k++) freq[k] = (uint16_t)get_le(in + 32 + 2 * k, 2);
    for (int k = 1; k < K; k++) lo[k] = in[32 + 2 * K + (k - 1)];
    for (uint64_t b = 32 + 3 * (uint64_t)K - 1; b < hb; b++)
        if (in[b]) return ORC_ERR_CORRUPT;
    if (check_table(K, R, lo, freq, n) != ORC_OK) return ORC_ERR_CORRUPT;

    const uint64_t L = (uint64_t)1 << R;
    uint16_t slot_range[4096], slot_next[4096], enc_slot[4096];
    uint8_t slot_nb[4096];
    if (n > 0 && orc_slot_tables(freq, K, R, slot_range, slot_nb, slot_next, enc_slot) != ORC_OK)
        return ORC_ERR_CORRUPT;

    const uint64_t groups = (nch + 63) / 64;
    const uint8_t* goff = in + hb;
    const uint8_t* sizes = goff + 4 * (groups + 1);
    const uint64_t unit = (uint64_t)1 << unit_log2((uint32_t)C, R, (uint32_t)S);
    uint64_t payload_at = hb + index_bytes(nch);
    if (get_le(goff, 4) != 0) return ORC_ERR_CORRUPT;
    for (uint64_t g = 0; g < groups; g++) {  /* every group offset follows from the sizes */
        uint64_t sum = 0;
        for (uint64_t c = 64 * g; c < nch && c < 64 * g + 64; c++) sum += unit * get_le(sizes + 2 * c, 2);
        if (get_le(goff + 4 * g, 4) + sum != get_le(goff + 4 * (g + 1), 4)) return ORC_ERR_CORRUPT;
    }
    if (nch % 2 && get_le(sizes + 2 * nch, 2) != 0) return ORC_ERR_CORRUPT;
    const uint64_t payload = get_le(goff + 4 * groups, 4);
    if (payload_at + (payload + 3) / 4 * 4 != nbytes) return ORC_ERR_CORRUPT;
    for (uint64_t b = payload_at + payload; b < nbytes; b++)
        if (in[b]) return ORC_ERR_CORRUPT;

    uint64_t* X = (uint64_t*)malloc(sizeof(uint64_t) * (size_t)S);
    if (!X) return ORC_ERR_INVALID;
    int st = ORC_OK;
    uint64_t a = 0;  /* the chunk's first byte */
    for (uint64_t c = 0; c < nch && st == ORC_OK; c++) {
        if (c % 64 == 0) a = get_le(goff + 4 * (c / 64), 4);
        const uint64_t units = get_le(sizes + 2 * c, 2);
        uint64_t b = a + unit * units;
        uint64_t first = c * C;
        uint64_t nc = (c + 1 < nch) ? C : n - first;
        uint64_t lanes = nc < S ? nc : S;
        if (units > (chunk_bound_bits(nc, R, (uint32_t)S) + 8 * unit - 1) / (8 * unit)) {
            st = ORC_ERR_CORRUPT;
            break;
        }
        const uint8_t* chunk = in + payload_at + a;
        uint64_t avail = 8 * (b - a), pos = 0;
        if (lanes * (uint64_t)R > avail) {
            st = ORC_ERR_CORRUPT;
            break;
        }
        for (uint64_t l = 0; l < lanes; l++) {
            X[l] = L + read_bits(chunk, pos, R);
            pos += (uint64_t)R;
        }
        for (uint64_t i = 0; i < nc; i++) { /* (step, lane) order */
            uint64_t l = i % S;
            uint64_t slot = X[l] - L;
            int s = slot_range[slot];
            int w = ceil_log2_u64((uint64_t)(lo[s + 1] - lo[s]));
            /* a lane's last field holds the offset only: its state bits are zero */
            int need = i + S >= nc ? w : w + slot_nb[slot];
            if (pos + (uint64_t)need > avail) {
                st = ORC_ERR_CORRUPT;
                break;
            }
            uint64_t v = read_bits(chunk, pos, need);
            pos += (uint64_t)need;
            uint64_t o = v & (((uint64_t)1 << w) - 1);
            if (o >= (uint64_t)(lo[s + 1] - lo[s])) {
                st = ORC_ERR_CORRUPT;
                break;
            }
            y[first + i] = (int8_t)((int)(lo[s] + o) - 128);
            X[l] = L + slot_next[slot] + (v >> w);
        }
        if (st != ORC_OK) break;
        for (uint64_t l = 0; l < lanes; l++)
            if (X[l] != L) st = ORC_ERR_CORRUPT;
        if ((pos + 8 * unit - 1) / (8 * unit) != units) st = ORC_ERR_CORRUPT;
        for (uint64_t p = pos; p < avail && st == ORC_OK; p++)
            if (read_bits(chunk, p, 1)) st = ORC_ERR_CORRUPT;
        a = b;
    }
    free(X);
    return st;
}

/* ------------------------------------------------------------------------------ */
/* statistics: Theorem 1 (paper section 4) and the section-5 efficiency metrics     */
/* ------------------------------------------------------------------------------ */

/*
 * out[0]  H(X)          entropy of the histogram, bits/symbol
 * out[1]  H(P)          entropy of the range probabilities P_k
 * out[2]  D_KL(P||Q)    with Q_k = f_k / L (the tANS quantisation loss)
 * out[3]  sum_k P_k w_k offset bits
 * out[4]  CL_Thm1       H(P) + D_KL(P||Q) + sum_k P_k w_k  (Theorem 1)
 * out[5]  H(p|P)        H(X) - H(P)
 * out[6]  D_KL(p||q)    plain tANS over the 256 values at L = 1024, frequencies by R3
 * out[7]  CL_tANS       H(X) + out[6]
 * out[8]  payload bits/symbol (field bits only)
 * out[9]  container bits/symbol (everything, header and index included)
 * out[10] CSR           container bytes / n
 * out[11] %diff of the payload rate = (rate - H) / H * 100 (paper section 5)
 * out[12] %diff of the container rate
 * out[13] %diff of CL_Thm1
 */
int orc_stats(const uint64_t* h256, int K, int log2_L, const uint16_t* lo,
              const uint16_t* freq, uint64_t payload_bits, uint64_t container_bytes,
              uint64_t n, double* out)
{
    int st = check_table(K, log2_L, lo, freq, n);
    if (st != ORC_OK) return st;
    for (int i = 0; i < ORC_N_STATS; i++) out[i] = 0.0;
    uint64_t N = 0;
    for (int u = 0; u < 256; u++) N += h256[u];
    if (N == 0) return ORC_OK;
    double dN = (double)N, L = (double)((uint64_t)1 << log2_L);
    double H = 0.0;
    for (int u = 0; u < 256; u++)
        if (h256[u]) {
            double p = (double)h256[u] / dN;
            H -= p * log2(p);
        }
    double HP = 0.0, dkl = 0.0, pw = 0.0;
    for (int k = 0; k < K; k++) {
        uint64_t Nk = 0;
        for (int u = lo[k]; u < lo[k + 1]; u++) Nk += h256[u];
        if (!Nk) continue;
        double P = (double)Nk / dN, Q = (double)freq[k] / L;
        HP -= P * log2(P);
        dkl += P * log2(P / Q);
        pw += P * (double)ceil_log2_u64((uint64_t)(lo[k + 1] - lo[k]));
    }
    uint16_t fref[256];
    double dkl_ref = 0.0;
    if (orc_normalize(h256, 256, 10, fref) == ORC_OK) {
        for (int u = 0; u < 256; u++)
            if (h256[u]) {
                double p = (double)h256[u] / dN;
                dkl_ref += p * log2(p / ((double)fref[u] / 1024.0));
            }
    }
    out[0] = H;
    out[1] = HP;
    out[2] = dkl;
    out[3] = pw;
    out[4] = HP + dkl + pw;
    out[5] = H - HP;
    out[6] = dkl_ref;
    out[7] = H + dkl_ref;
    if (n > 0) {
        out[8] = (double)payload_bits / (double)n;
        out[9] = 8.0 * (double)container_bytes / (double)n;
        out[10] = (double)container_bytes / (double)n;
    }
    if (H > 0.0) {
        out[11] = (out[8] - H) / H * 100.0;
        out[12] = (out[9] - H) / H * 100.0;
        out[13] = (out[4] - H) / H * 100.0;
    }
    return ORC_OK;
}

/* Decode fused into a consumer (Ecco summary page, section 3: entropy-coded data decoded
 * inside the kernel that uses it).  The oracle's side is the definition: the decoded
 * matrix (rows of cols values, row-major, as orc_decode writes the tensor) times the
 * vector, each row summed exactly in 64 bits and added to y[r] modulo 2^32. */
int orc_matvec_i8(const int8_t* w, uint64_t n, uint32_t cols, const int8_t* a, int32_t* y)
{
    if (cols == 0 || n % cols != 0) return ORC_ERR_INVALID;
    for (uint64_t r = 0; r < n / cols; ++r) {
        int64_t s = 0;
        for (uint32_t c = 0; c < cols; ++c) s += (int64_t)w[r * cols + c] * (int64_t)a[c];
        y[r] = (int32_t)((uint32_t)y[r] + (uint32_t)(uint64_t)s);
    }
    return ORC_OK;
}
