// Host side of the offline step: histogram -> DP range split -> tANS state allocation
// -> derived tables, plus the container header.
//
// Method: "Shannonic: Efficient Entropy-Optimal Compression for ML Workloads" (MLSys 2026),
// talk notes, "Preprocessing: range selection by dynamic programming" (paper section 4.1)
// and "Runtime encoding/decoding" (paper section 4.2).
//
// Everything here is integer arithmetic.  The DP cost uses a fixed-point base-2 logarithm
// with 24 fractional bits computed by repeated squaring (a defined function, so any
// implementation reaches the same partition, exact ties included); the pages do not fix
// the precision of the objective.
#include <cstring>
#include <algorithm>
#include <cmath>
#include <vector>

#include "codec_internal.hpp"

namespace shn {

// 2^24 * log2(x), digit by digit: with x = 2^e * m, m in [1, 2) kept in Q1.63, each
// fractional bit of log2 m is set exactly when m^2 >= 2; the square (halved when the bit
// is set) is truncated back to 64 bits and carries on.
uint64_t fixed_log2(uint64_t x) {
    if (x == 0) return 0;
    const int e = 63 - __builtin_clzll(x);
    uint64_t m = x << (63 - e);
    uint64_t frac = 0;
    for (int i = 0; i < kLgFrac; ++i) {
        const unsigned __int128 sq = (unsigned __int128)m * m;
        const uint64_t top = (uint64_t)(sq >> 127);
        frac = (frac << 1) | top;
        m = (uint64_t)(sq >> (63 + top));
    }
    return ((uint64_t)e << kLgFrac) | frac;
}

sh_status check_table(const sh_table& t, bool allow_empty) {
    if (t.K < 1 || t.K > 256 || t.log2_L < 1 || t.log2_L > (uint32_t)kMaxLog2LHost)
        return SH_ERR_INVALID_ARG;
    if (t.lo[0] != 0 || t.lo[t.K] != 256) return SH_ERR_INVALID_ARG;
    for (uint32_t k = 0; k < t.K; ++k)
        if (t.lo[k + 1] <= t.lo[k]) return SH_ERR_INVALID_ARG;
    uint64_t total = 0;
    for (uint32_t k = 0; k < t.K; ++k) total += t.freq[k];
    if (total == (1ull << t.log2_L)) return SH_OK;
    return (total == 0 && allow_empty) ? SH_OK : SH_ERR_INVALID_ARG;
}

// Exactly-K contiguous ranges over [0, 256) minimising the summed range cost
//   N_R * (log2 N - log2 N_R) + N_R * ceil(log2 width)     (units of 2^-24 bit)
// -- the ideal range-id code length plus the raw offset bits.  Recurrence
// C[i][k] = min_{j<i} C[j][k-1] + cost[j, i); the smallest j wins ties.
static void dp_split(const uint64_t* hist, uint32_t K, uint16_t* lo) {
    constexpr int A = 256;
    uint64_t prefix[A + 1];
    prefix[0] = 0;
    for (int v = 0; v < A; ++v) prefix[v + 1] = prefix[v] + hist[v];
    const uint64_t N = prefix[A];
    const uint64_t lgN = fixed_log2(N);

    // cost of [j, i) for all 0 <= j < i <= 256, row i holds j = 0..i-1
    std::vector<uint64_t> cost((size_t)(A + 1) * (A + 2) / 2);
    auto at = [](int j, int i) { return (size_t)i * (i - 1) / 2 + (size_t)j; };
    for (int i = 1; i <= A; ++i)
        for (int j = 0; j < i; ++j) {
            const uint64_t nr = prefix[i] - prefix[j];
            cost[at(j, i)] = nr ? nr * (lgN - fixed_log2(nr)) +
                                      nr * ((uint64_t)ceil_log2_u32((uint32_t)(i - j)) << kLgFrac)
                                : 0;
        }

    constexpr uint64_t INF = ~0ull;
    std::vector<uint64_t> prev(A + 1, INF), cur(A + 1, INF);
    std::vector<int16_t> arg((size_t)(K + 1) * (A + 1), -1);
    prev[0] = 0;
    for (uint32_t k = 1; k <= K; ++k) {
        std::fill(cur.begin(), cur.end(), INF);
        for (int i = (int)k; i <= A; ++i) {
            uint64_t best = INF;
            int bj = -1;
            for (int j = (int)k - 1; j < i; ++j) {
                if (prev[j] == INF) continue;
                const uint64_t c = prev[j] + cost[at(j, i)];
                if (c < best) {
                    best = c;
                    bj = j;
                }
            }
            cur[i] = best;
            arg[(size_t)k * (A + 1) + i] = (int16_t)bj;
        }
        std::swap(prev, cur);
    }
    int i = A;
    lo[K] = A;
    for (uint32_t k = K; k >= 1; --k) {
        i = arg[(size_t)k * (A + 1) + i];
        lo[k - 1] = (uint16_t)i;
    }
}

// State allocation: one state for each occupied range, then each remaining state to the
// range whose N_k * (log2(f_k + 1) - log2 f_k) is largest (first k on ties) -- the
// greedy optimum of sum_k N_k log2 f_k, i.e. the smallest D_KL(P || Q).
sh_status allocate_states(const uint64_t* count, uint32_t K, uint32_t L, uint16_t* f) {
    uint32_t used = 0;
    for (uint32_t k = 0; k < K; ++k) {
        f[k] = count[k] ? 1 : 0;
        used += f[k];
    }
    if (used == 0) return SH_OK;
    if (used > L) return SH_ERR_UNSUPPORTED;
    // log2(f + 1) - log2 f in fixed point, for every f up to the largest L: built once
    static const std::vector<uint64_t> gain_of = [] {
        std::vector<uint64_t> g((1u << kMaxLog2LHost) + 1, 0);
        for (uint32_t v = 1; v < g.size(); ++v) g[v] = fixed_log2(v + 1) - fixed_log2(v);
        return g;
    }();
    if (L > (1u << kMaxLog2LHost)) return SH_ERR_UNSUPPORTED;
    // The greedy steps take the L - used largest increments N_k * gain(f), f >= 1, in the
    // order (gain down, k up); a range's increments fall strictly with f.  So a start
    // close to the result can be finished greedily and then checked: the allocation is
    // the greedy one exactly when the last increment taken precedes the first one left.
    struct Item {
        uint64_t g;
        uint32_t k;
        bool operator<(const Item& o) const { return g < o.g || (g == o.g && k > o.k); }
    };
    // greedy increments from f up to L: a binary max-heap whose top is replaced in place
    Item heap[256];
    auto finish = [&](uint32_t total) {
        uint32_t n = 0;
        for (uint32_t k = 0; k < K; ++k)
            if (count[k]) heap[n++] = {count[k] * gain_of[f[k]], k};
        std::make_heap(heap, heap + n);
        for (; total < L; ++total) {
            const uint32_t k = heap[0].k;
            f[k]++;
            const Item v{count[k] * gain_of[f[k]], k};
            uint32_t i = 0;  // sift v down from the root
            while (true) {
                uint32_t c = 2 * i + 1;
                if (c >= n) break;
                if (c + 1 < n && heap[c] < heap[c + 1]) ++c;
                if (!(v < heap[c])) break;
                heap[i] = heap[c];
                i = c;
            }
            heap[i] = v;
        }
    };
    uint64_t N = 0;
    for (uint32_t k = 0; k < K; ++k) N += count[k];
    uint32_t total = 0;
    // the proportional share (at least one): rarely above the result.  Any start gives the
    // greedy result once the check below passes, so it is computed in floating point.
    const double scale = (double)(L - used) / (double)N;
    for (uint32_t k = 0; k < K; ++k)
        if (count[k]) {
            const double share = std::floor(scale * (double)count[k]);
            f[k] = (uint16_t)(share > 1 ? share : 1);
            total += f[k];
        }
    if (total > L) {
        for (uint32_t k = 0; k < K; ++k) f[k] = count[k] ? 1 : 0;
        total = used;
    }
    finish(total);
    bool have_last = false, have_next = false;
    Item last{0, 0}, next{0, 0};  // last increment taken, first increment left
    for (uint32_t k = 0; k < K; ++k) {
        if (!count[k]) continue;
        if (f[k] >= 2) {
            const Item t{count[k] * gain_of[f[k] - 1], k};
            if (!have_last || t < last) last = t;  // later in the order
            have_last = true;
        }
        if (f[k] < L) {
            const Item t{count[k] * gain_of[f[k]], k};
            if (!have_next || next < t) next = t;  // earlier in the order
            have_next = true;
        }
    }
    if (have_last && have_next && last < next) {  // the start overshot: greedy from one each
        for (uint32_t k = 0; k < K; ++k) f[k] = count[k] ? 1 : 0;
        finish(used);
    }
    return SH_OK;
}

sh_status table_from_histogram(const uint64_t* hist, uint32_t K, uint32_t log2_L, sh_table* out) {
    if (!hist || !out || K < 1 || K > 256 || log2_L < 1 || log2_L > (uint32_t)kMaxLog2LHost)
        return SH_ERR_INVALID_ARG;
    uint64_t N = 0;
    for (int u = 0; u < 256; ++u) N += hist[u];
    if (N >= (1ull << 32)) return SH_ERR_UNSUPPORTED;
    sh_table t;
    std::memset(&t, 0, sizeof(t));
    t.K = K;
    t.log2_L = log2_L;
    std::memcpy(t.hist, hist, sizeof(t.hist));
    t.n = N;
    dp_split(hist, K, t.lo);
    uint64_t count[256];
    for (uint32_t k = 0; k < K; ++k) {
        count[k] = 0;
        for (int u = t.lo[k]; u < t.lo[k + 1]; ++u) count[k] += hist[u];
    }
    const sh_status st = allocate_states(count, K, 1u << log2_L, t.freq);
    if (st != SH_OK) return st;
    *out = t;
    return SH_OK;
}

// Slot spread: range k's keys (2j+1)/(2 f_k), j < f_k, merged in increasing order (exact
// cross-multiplied comparison, smaller k first on equal keys); slot i takes the range of
// the i-th key.  Then the tANS tables: if slot i is range s's j-th slot, decoding it
// gives s and the sub-state x = f_s + j, reads nb = R - floor(log2 x) bits b and moves to
// slot (x << nb) - L + b; the encoder maps (s, j) back to slot i.
sh_status derive_slots(const sh_table& t, SlotTables* out) {
    const sh_status st = check_table(t, false);
    if (st != SH_OK) return st;
    const uint32_t K = t.K, R = t.log2_L, L = 1u << R;
    out->L = L;
    out->cum[0] = 0;
    for (uint32_t k = 0; k < K; ++k) out->cum[k + 1] = out->cum[k] + t.freq[k];
    uint32_t taken[256] = {0};
    for (uint32_t i = 0; i < L; ++i) {
        uint32_t best = K;
        for (uint32_t k = 0; k < K; ++k) {
            if (taken[k] >= t.freq[k]) continue;
            if (best == K) {
                best = k;
                continue;
            }
            // (2 taken[k] + 1) / f_k  <  (2 taken[best] + 1) / f_best ?
            const uint64_t lhs = (uint64_t)(2 * taken[k] + 1) * t.freq[best];
            const uint64_t rhs = (uint64_t)(2 * taken[best] + 1) * t.freq[k];
            if (lhs < rhs) best = k;
        }
        const uint32_t j = taken[best]++;
        const uint32_t x = t.freq[best] + j;
        const uint32_t nb = R - floor_log2_u32(x);
        out->range[i] = (uint16_t)best;
        out->nb[i] = (uint8_t)nb;
        out->next[i] = (uint16_t)((x << nb) - L);
        out->enc[out->cum[best] + j] = (uint16_t)i;
    }
    return SH_OK;
}

void write_header(const sh_table& t, uint64_t n, uint32_t C, uint32_t S, uint64_t n_chunks,
                  uint32_t* dwords) {
    uint8_t b[kMaxHeaderDwords * 4];
    std::memset(b, 0, sizeof(b));
    auto put = [&](uint32_t at, uint64_t v, int bytes) {
        for (int i = 0; i < bytes; ++i) b[at + i] = (uint8_t)(v >> (8 * i));
    };
    b[0] = 'S';
    b[1] = 'H';
    b[2] = 'N';
    b[3] = '1';
    b[4] = 3;  // version 3: byte-aligned chunks, u16 sizes (version 2: a lane's last field
               // without state bits)
    b[5] = (uint8_t)t.log2_L;
    put(6, t.K, 2);
    put(8, n, 8);
    put(16, C, 4);
    put(20, S, 4);
    put(24, n_chunks, 4);
    put(28, header_bytes(t.K), 4);
    for (uint32_t k = 0; k < t.K; ++k) put(kHeaderFixed + 2 * k, t.freq[k], 2);
    for (uint32_t k = 1; k < t.K; ++k) b[kHeaderFixed + 2 * t.K + k - 1] = (uint8_t)t.lo[k];
    std::memcpy(dwords, b, header_bytes(t.K));
}

}  // namespace shn

namespace shn {

// The kernels' forms of a table (see codec_internal.hpp for the packing).
void derive_kernel_tables(const sh_table& t, const SlotTables& st, uint32_t* dec, uint32_t* vt,
                          uint16_t* es) {
    const uint32_t K = t.K, R = t.log2_L, L = 1u << R;
    if (dec) {
        for (uint32_t i = 0; i < L; ++i) {
            const uint32_t s = st.range[i];
            const uint32_t width = t.lo[s + 1] - t.lo[s];
            const uint32_t w = ceil_log2_u32(width);
            dec[2 * i] = (w + st.nb[i]) | ((uint32_t)st.next[i] * 8u << 16);
            dec[2 * i + 1] = w | (((uint32_t)(t.lo[s] - 128) & 0xFFu) << 8) | ((width - 1) << 16);
        }
    }
    if (vt) {
        for (uint32_t s = 0; s < K; ++s) {
            const uint32_t f = t.freq[s];
            const uint32_t w = ceil_log2_u32(t.lo[s + 1] - t.lo[s]);
            int32_t bias = 0, start = -(int32_t)L;
            if (f > 0) {
                const uint32_t m = floor_log2_u32(f);
                bias = (int32_t)((R - m) << (R + 1)) - (int32_t)(f << (R - m));
                start = (int32_t)st.cum[s] - (int32_t)f;
            }
            for (uint32_t u = t.lo[s]; u < t.lo[s + 1]; ++u) {
                vt[2 * u] = (uint32_t)bias;
                vt[2 * u + 1] = (u - t.lo[s]) | (w << 8) | ((uint32_t)(start + (int32_t)kMaxLGpu) << 16) |
                                (f == 0 ? 0x8000u : 0u);
            }
        }
    }
    if (es)
        for (uint32_t i = 0; i < L; ++i) es[i] = st.enc[i];
}

uint32_t max_field_bits(const sh_table& t) {
    uint32_t w = 0;
    for (uint32_t k = 0; k < t.K; ++k) {
        const uint32_t wk = ceil_log2_u32(t.lo[k + 1] - t.lo[k]);
        w = wk > w ? wk : w;
    }
    return w + t.log2_L;
}

void make_device_table(const sh_table& t, const SlotTables* st, uint32_t C, uint32_t S,
                       uint32_t* dt) {
    std::memset(dt, 0, kDTBytes);
    dt[kDTK] = t.K;
    dt[kDTLog2L] = t.log2_L;
    dt[kDTL] = 1u << t.log2_L;
    dt[kDTStatus] = 0;
    std::memcpy(dt + kDTN, &t.n, 8);
    dt[kDTHdrDwords] = header_bytes(t.K) / 4;
    write_header(t, 0, C, S, 0, dt + kDTHdr);
    if (st)
        derive_kernel_tables(t, *st, dt + kDTDec, dt + kDTVt, reinterpret_cast<uint16_t*>(dt + kDTEs));
    else  // a table built from no values: every value is outside it
        for (uint32_t u = 0; u < 256; ++u) dt[kDTVt + 2 * u + 1] = 0x8000u;
    std::memcpy(dt + kDTLo, t.lo, sizeof(t.lo));
    std::memcpy(dt + kDTFreq, t.freq, sizeof(t.freq));
    std::memcpy(dt + kDTHist, t.hist, sizeof(t.hist));
}

}  // namespace shn
