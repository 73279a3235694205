// Histogram and table-build kernels of the Shannonic codec for gfx950 (CDNA4, wave64):
// the offline step of the Shannonic talk notes ("Preprocessing: range selection by dynamic
// programming", paper section 4.1) run on the GPU, so that tables never leave HBM.
#include <type_traits>

#include "device_common.hpp"

namespace shn {

// ------------------------------------------------------------------------------------
// histogram: h[u] = #{i : x[i] + 128 == u}   (paper section 4.1)
// ------------------------------------------------------------------------------------
constexpr int kHistBlock = 256;
constexpr int kHistCopies = 32;

__global__ void k_zero_u64(uint64_t* p, uint32_t count) {
    const uint32_t i = blockIdx.x * blockDim.x + threadIdx.x;
    if (i < count) p[i] = 0;
}

template <class H>
__global__ __launch_bounds__(kHistBlock) void k_histogram(const H a) {
    // 32 private copies per block, copy c of bin b at b * 32 + c: the 32 lanes of a half
    // wavefront hit 32 different banks even when every value is the same.
    __shared__ uint32_t h[256 * kHistCopies];
    for (int i = threadIdx.x; i < 256 * kHistCopies; i += kHistBlock) h[i] = 0;
    __syncthreads();
    const uint32_t block = blockIdx.x;
    const uint32_t seg = __builtin_amdgcn_readfirstlane(find_seg_index(a.segs, a.nseg, block, false));
    const uint8_t* x = a.segs[seg].x;
    const uint64_t n = a.segs[seg].n;
    const uint64_t lo = (uint64_t)(block - a.segs[seg].first_block) * a.block_bytes;
    const uint64_t hi = lo + a.block_bytes < n ? lo + a.block_bytes : n;
    const uint32_t copy = threadIdx.x & (kHistCopies - 1);
    auto count16 = [&](const v4u w) {
#pragma unroll
        for (int q = 0; q < 4; ++q) {
#pragma unroll
            for (int b = 0; b < 4; ++b) {
                const uint32_t u = ((w[q] >> (8 * b)) & 0xFF) ^ 0x80;
                atomicAdd(&h[u * kHistCopies + copy], 1u);
            }
        }
    };
    // 16-byte groups fully inside [lo, hi); x is 16-byte aligned and lo a multiple of 16.
    // Four loads per thread are in flight before their counts.
    const uint64_t g0 = lo / 16, g1 = hi / 16;
    uint64_t g = g0 + threadIdx.x;
    for (; g + 3 * kHistBlock < g1; g += 4 * kHistBlock) {
        v4u w[4];
#pragma unroll
        for (int r = 0; r < 4; ++r) w[r] = *reinterpret_cast<const v4u*>(x + 16 * (g + r * kHistBlock));
#pragma unroll
        for (int r = 0; r < 4; ++r) count16(w[r]);
    }
    for (; g < g1; g += kHistBlock) count16(*reinterpret_cast<const v4u*>(x + 16 * g));
    for (uint64_t i = g1 * 16 + threadIdx.x; i < hi; i += kHistBlock)  // tail < 16 values
        atomicAdd(&h[((uint32_t)x[i] ^ 0x80) * kHistCopies + copy], 1u);
    __syncthreads();
    for (int b = threadIdx.x; b < 256; b += kHistBlock) {
        uint64_t s = 0;
#pragma unroll 8
        for (int c = 0; c < kHistCopies; ++c) s += h[b * kHistCopies + c];
        if (s) atomicAdd((unsigned long long*)&a.hist[256 * seg + b], (unsigned long long)s);
    }
}

sh_status launch_histogram(const HistArgs& h, uint32_t nseg_zero, void* stream) {
    hipStream_t s = (hipStream_t)stream;
    const uint32_t words = 256 * nseg_zero;
    hipLaunchKernelGGL(k_zero_u64, dim3((words + 255) / 256), dim3(256), 0, s, h.hist, words);
    if (h.n_blocks > 0) {
        if (h.nseg <= 1)
            hipLaunchKernelGGL(k_histogram<HistArgsN<1>>, dim3(h.n_blocks), dim3(kHistBlock), 0, s,
                               hist_args<1>(h));
        else if (h.nseg <= 16)
            hipLaunchKernelGGL(k_histogram<HistArgsN<16>>, dim3(h.n_blocks), dim3(kHistBlock), 0,
                               s, hist_args<16>(h));
        else
            hipLaunchKernelGGL(k_histogram<HistArgs>, dim3(h.n_blocks), dim3(kHistBlock), 0, s, h);
    }
    return hipGetLastError() == hipSuccess ? SH_OK : SH_ERR_HIP;
}

// ------------------------------------------------------------------------------------
// table build on the GPU (paper section 4.1): one block per tensor
// ------------------------------------------------------------------------------------
// 2^24 * log2(x), digit by digit: with x = 2^e * m, m in [1, 2) kept in Q1.63, each
// fractional bit of log2 m is set exactly when m^2 >= 2; the square (halved when the bit
// is set) is truncated back to 64 bits and carries on.  The same function as the host's.
__device__ uint64_t dev_fixed_log2(uint64_t x) {
    if (x == 0) return 0;
    const int e = 63 - __builtin_clzll(x);
    uint64_t m = x << (63 - e);
    uint64_t frac = 0;
    for (int i = 0; i < kLgFrac; ++i) {
        const uint64_t hi = __umul64hi(m, m);
        const uint64_t lo = m * m;
        const uint64_t top = hi >> 63;
        frac = (frac << 1) | top;
        m = top ? hi : (hi << 1) | (lo >> 63);
    }
    return ((uint64_t)e << kLgFrac) | frac;
}

__device__ __forceinline__ uint32_t dev_ceil_log2(uint32_t m) { return m <= 1 ? 0 : 32 - __builtin_clz(m - 1); }
__device__ __forceinline__ uint32_t dev_floor_log2(uint32_t x) { return 31 - __builtin_clz(x); }

// Row i (1..256) of the cost triangle holds the ranges [j, i), j = 0..i-1, at i(i-1)/2 + j.
__device__ __forceinline__ void cost_pair(uint32_t idx, uint32_t& i, uint32_t& j) {
    uint32_t r = (uint32_t)((1.0f + sqrtf(1.0f + 8.0f * (float)idx)) * 0.5f);
    while (r * (r - 1) / 2 > idx) --r;
    while ((r + 1) * r / 2 <= idx) ++r;
    i = r;
    j = idx - r * (r - 1) / 2;
}

// Inclusive sum over a wavefront of a value held in every lane.
__device__ __forceinline__ uint32_t wave_sum(uint32_t v) {
    for (int d = 32; d >= 1; d >>= 1) v += __shfl_xor(v, d, 64);
    return v;
}

// Build, step 1 (every tensor, many blocks each): the cost factor of every range [j, i),
//   s(j, i) = log2 N - log2 N_R + ceil(log2 (i - j))   (fixed point, 2^-24 bit),
// so that the DP's cost N_R * (log2 N - log2 N_R) + N_R * ceil(log2 |R|) is N_R * s.
// Zero for an empty range (whose cost is 0 whatever s is).
constexpr uint32_t kCostBlocks = (kCostEntries + 255) / 256;

__global__ __launch_bounds__(256) void k_build_cost(const BuildArgs a) {
    __shared__ uint32_t prefix[257];
    __shared__ uint32_t wsum[4];
    __shared__ uint32_t lgN_s;
    const uint32_t tid = threadIdx.x, lane = tid & 63;
    const uint32_t seg = blockIdx.x / kCostBlocks, part = blockIdx.x % kCostBlocks;
    const uint64_t* hist = a.hist + 256ull * seg;
    // totals below 2^32 (checked by the caller), so 32-bit prefix sums are exact
    uint32_t incl = (uint32_t)hist[tid];
    for (int d = 1; d < 64; d <<= 1) {
        const uint32_t o = __shfl_up(incl, d, 64);
        if (lane >= (uint32_t)d) incl += o;
    }
    if (lane == 63) wsum[tid >> 6] = incl;
    __syncthreads();
    uint32_t before = 0;
    for (uint32_t w = 0; w < (tid >> 6); ++w) before += wsum[w];
    prefix[tid + 1] = before + incl;
    if (tid == 0) {
        prefix[0] = 0;
        lgN_s = (uint32_t)dev_fixed_log2(wsum[0] + wsum[1] + wsum[2] + wsum[3]);
    }
    __syncthreads();
    const uint32_t idx = part * 256 + tid;
    if (idx >= kCostEntries) return;
    uint32_t i, j;
    cost_pair(idx, i, j);
    const uint32_t nr = prefix[i] - prefix[j];
    a.scost[(uint64_t)seg * kCostEntries + idx] =
        nr ? lgN_s - (uint32_t)dev_fixed_log2(nr) + (dev_ceil_log2(i - j) << kLgFrac) : 0u;
}

// Build, step 2 (one block per tensor): the DP over the cost factors held in LDS, the
// state allocation, the spread and every derived table.
constexpr int kBuildBlock = 1024;

// floor(A / f) for A < 2^24, f >= 1: a float quotient through the hardware reciprocal (A
// is exact in a float and the product's relative error stays below 2^-21, so the quotient
// is at most 9 away), then a fixed number of one-step corrections with 64-bit products
__device__ __forceinline__ uint32_t small_div(uint32_t A, uint32_t f) {
    uint32_t q = (uint32_t)((float)A * __builtin_amdgcn_rcpf((float)f));
#pragma unroll
    for (int i = 0; i < 12; ++i)
        if (q > 0 && (uint64_t)q * f > A) --q;
#pragma unroll
    for (int i = 0; i < 12; ++i)
        if ((uint64_t)(q + 1) * f <= A) ++q;
    return q;
}

// DP work split: lane q < 1008 owns value i and the 37 j in [37 p, 37 p + 37), for the
// pieces p = 0 .. ceil(i / 37) - 1 of every i in [1, 256) (piece-major, so a wavefront
// mostly shares p and its reads of C[j] are broadcasts).  The lane keeps the 37 candidate
// costs N_[j,i) * s(j, i), which do not change between layers, in registers; slots with
// j >= i hold kInfCost.  Infeasible C entries hold kInfC.  s(j, i) < 40 * 2^24, so every
// real cost and every real C value (a sum of costs over a partition of at most N values) is
// below N * 2^29.33 <= 2^61.33: no sum wraps and every sum with an infinite part stays above
// every real one.  When N <= 2^27 the values also fit in 57 bits, and the DP runs on keys
// value << 6 | u (u = the slot of j): the smallest key is the smallest value with the
// smallest j, one 64-bit compare per candidate.
constexpr uint32_t kPiece = 37, kPieces = 7, kDpLanes = 1008;
// state allocation in LDS: at most kIncMax increments (8 bytes each) and their ranks
constexpr uint32_t kIncMax = 8192;
constexpr uint64_t kInfC = 1ull << 63, kInfCost = 3ull << 61;
__global__ __launch_bounds__(kBuildBlock) void k_build_tables(const BuildArgs a) {
    __shared__ __align__(16) uint32_t sc[kCostEntries];  // cost factors; the DP's choices after it
    __shared__ uint32_t prefix[257];
    __shared__ uint64_t cbuf[2][kPiece * kPieces];  // C[j][k-1] and C[j][k], kInfC past 255
    __shared__ uint64_t qbest[kPieces][256];        // per-piece minima of a layer
    __shared__ uint8_t qarg[kPieces][256];
    __shared__ uint64_t red_c[kBuildBlock / 64];
    __shared__ uint32_t red_j[kBuildBlock / 64];
    __shared__ uint32_t lo_s[257], freq_s[256], cum_s[257], range_of_u[256], count_s[256];

    __shared__ uint32_t f0_s[256], add_s[256], alloc_s[2];  // state allocation: start, taken, total and check
    __shared__ uint32_t status_s;
    const uint32_t tid = threadIdx.x, lane = tid & 63, seg = blockIdx.x;
    const uint32_t wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const uint64_t* hist = a.hist + 256ull * seg;
    uint32_t* dt = a.tables + (uint64_t)seg * kDTDwords;
    const uint32_t K = a.K, R = a.R, L = 1u << R;

    for (uint32_t i = tid; i < kDTDwords; i += kBuildBlock) dt[i] = 0;  // unused parts read 0
    {  // the cost factors into LDS: every thread's loads in flight together
        static_assert(kCostEntries % 4 == 0, "16-byte groups");
        constexpr uint32_t kGroups = kCostEntries / 4, kPer = (kGroups + kBuildBlock - 1) / kBuildBlock;
        const v4u* src = reinterpret_cast<const v4u*>(a.scost + (uint64_t)seg * kCostEntries);
        v4u* dst = reinterpret_cast<v4u*>(sc);
        v4u v[kPer];
#pragma unroll
        for (uint32_t r = 0; r < kPer; ++r) {
            const uint32_t i = tid + r * kBuildBlock;
            if (i < kGroups) v[r] = src[i];
        }
#pragma unroll
        for (uint32_t r = 0; r < kPer; ++r) {
            const uint32_t i = tid + r * kBuildBlock;
            if (i < kGroups) dst[i] = v[r];
        }
    }

    // prefix sums of the histogram, 64-bit to check that the total fits 32 bits
    uint64_t incl = 0;
    if (tid < 256) {
        incl = hist[tid];
        for (int d = 1; d < 64; d <<= 1) {
            const uint64_t o = __shfl_up(incl, d, 64);
            if (lane >= (uint32_t)d) incl += o;
        }
        if (lane == 63) red_c[wave] = incl;
    }
    lds_barrier();
    if (tid < 256) {
        uint64_t before = 0;
        for (uint32_t w = 0; w < wave; ++w) before += red_c[w];
        prefix[tid + 1] = (uint32_t)(before + incl);
    }
    if (tid == 0) {
        prefix[0] = 0;
        const uint64_t total = red_c[0] + red_c[1] + red_c[2] + red_c[3];
        status_s = total >= (1ull << 32) ? (uint32_t)SH_ERR_UNSUPPORTED : 0u;
    }
    lds_barrier();

    // ---- the DP: C[i][k] = min over k-1 <= j < i of C[j][k-1] + N_[j,i) * s(j, i) ----
    // Ties keep the smallest j.  C[j][k-1] is finite for every j >= k-1 once k >= 2.
    // Layer 1 has the single choice j = 0; the last layer needs i = 256 only, every
    // other layer i < 256 only.
    if (K == 1) {
        if (tid == 0) {
            lo_s[0] = 0;
            lo_s[1] = 256;
        }
    } else {
        const bool packed = prefix[256] <= (1u << 27);  // uniform
        for (uint32_t i = tid; i < kPiece * kPieces; i += kBuildBlock) {
            const uint64_t c1 = i >= 1 && i < 256 ? (uint64_t)prefix[i] * sc[i * (i - 1) / 2] : kInfC;
            cbuf[1][i] = packed && c1 != kInfC ? c1 << 6 : c1;
            cbuf[0][i] = kInfC;
        }
        // this lane's piece: p, then i = 37 p + 1 + (q - first lane of p)
        uint32_t p = 0, first = 0;
        while (p + 1 < kPieces && tid >= first + (255 - kPiece * p)) {
            first += 255 - kPiece * p;
            ++p;
        }
        const bool dp_lane = tid < kDpLanes;
        const uint32_t i = dp_lane ? kPiece * p + 1 + (tid - first) : 1;  // idle lanes: no j < i
        const uint32_t j0 = kPiece * p;
        uint64_t cost[kPiece];
        {
            const uint32_t row = i * (i - 1) / 2, pi = dp_lane ? prefix[i] : 0;
#pragma unroll
            for (uint32_t u = 0; u < kPiece; ++u) {
                const uint32_t j = j0 + u;
                const uint64_t c = dp_lane && j < i ? (uint64_t)(pi - prefix[j]) * sc[row + j] : kInfCost;
                cost[u] = packed ? (c == kInfCost ? c : c << 6) | u : c;
            }
        }
        lds_barrier();  // from here the cost factors' LDS holds the DP's choices
        auto layers = [&](auto packed_tag) {
            constexpr bool kPacked = decltype(packed_tag)::value;
            for (uint32_t k = 2; k < K; ++k) {
                const uint64_t* cp = cbuf[(k - 1) & 1] + j0;
                uint64_t best = ~0ull;
                uint32_t bu = 0;
                if constexpr (kPacked) {  // keys are distinct: any order, four running minima
                    uint64_t m[4] = {~0ull, ~0ull, ~0ull, ~0ull};
#pragma unroll
                    for (uint32_t u = 0; u < kPiece; ++u) {
                        const uint64_t c = cp[u] + cost[u];
                        m[u & 3] = c < m[u & 3] ? c : m[u & 3];
                    }
                    m[0] = m[1] < m[0] ? m[1] : m[0];
                    m[2] = m[3] < m[2] ? m[3] : m[2];
                    best = m[2] < m[0] ? m[2] : m[0];
                } else {
#pragma unroll
                    for (uint32_t u = 0; u < kPiece; ++u) {
                        const uint64_t c = cp[u] + cost[u];
                        if (c < best) {
                            best = c;
                            bu = u;
                        }
                    }
                }
                if (dp_lane) {
                    qbest[p][i] = kPacked ? best >> 6 : best;
                    qarg[p][i] = (uint8_t)(j0 + (kPacked ? (uint32_t)best & 63 : bu));
                }
                lds_barrier();
                if (tid < 256) {  // pieces in increasing j: the first minimum keeps the smallest j
                    const uint64_t inf = kPacked ? kInfC >> 6 : kInfC;
                    // every piece's entry is read at once; pieces past i (never written for
                    // this i) are left out by the predicate
                    uint64_t qb[kPieces];
                    uint32_t qa[kPieces];
#pragma unroll
                    for (uint32_t pp = 0; pp < kPieces; ++pp) {
                        qb[pp] = qbest[pp][tid];
                        qa[pp] = qarg[pp][tid];
                    }
                    uint64_t bb = qb[0];
                    uint32_t jj = qa[0];
#pragma unroll
                    for (uint32_t pp = 1; pp < kPieces; ++pp)
                        if (kPiece * pp < tid && qb[pp] < bb) {
                            bb = qb[pp];
                            jj = qa[pp];
                        }
                    bb = tid == 0 ? inf : (bb < inf ? bb : inf);
                    jj = tid == 0 ? 0u : jj;
                    cbuf[k & 1][tid] = kPacked && bb != inf ? bb << 6 : (bb == inf ? kInfC : bb);
                    reinterpret_cast<uint8_t*>(sc)[k * 256 + tid] = (uint8_t)jj;
                }
                lds_barrier();
            }
        };
        if (packed) layers(std::true_type{});
        else layers(std::false_type{});
        // layer K at i = 256
        {
            const uint64_t* cp = cbuf[(K - 1) & 1];
            const uint32_t j = K - 1 + tid;
            uint64_t c = ~0ull;
            if (j < 256) c = (uint64_t)(prefix[256] - prefix[j]) * sc[256 * 255 / 2 + j] +
                             (packed && cp[j] != kInfC ? cp[j] >> 6 : cp[j]);
            uint32_t bj = j;
            for (int d = 1; d < 64; d <<= 1) {  // lexicographic (cost, j) minimum
                const uint64_t oc = __shfl_xor(c, d, 64);
                const uint32_t oj = __shfl_xor(bj, d, 64);
                if (oc < c || (oc == c && oj < bj)) {
                    c = oc;
                    bj = oj;
                }
            }
            if (lane == 0) {
                red_c[wave] = c;
                red_j[wave] = bj;
            }
        }
        lds_barrier();
        const uint8_t* argl = reinterpret_cast<const uint8_t*>(sc);  // choices of layers 2 .. K-1
        if (tid == 0) {
            uint64_t c = red_c[0];
            uint32_t i = red_j[0];
            for (uint32_t w = 1; w < kBuildBlock / 64; ++w)
                if (red_c[w] < c || (red_c[w] == c && red_j[w] < i)) {
                    c = red_c[w];
                    i = red_j[w];
                }
            lo_s[K] = 256;
            lo_s[K - 1] = i;
            for (uint32_t k = K - 1; k >= 2; --k) {
                i = argl[k * 256 + i];
                lo_s[k - 1] = i;
            }
            lo_s[0] = 0;
        }
    }
    lds_barrier();
    for (uint32_t k = tid; k < K; k += kBuildBlock) count_s[k] = prefix[lo_s[k + 1]] - prefix[lo_s[k]];
    if (wave == 0) {
        uint32_t used = 0, wmax = 0;
        for (uint32_t k = lane; k < K; k += 64) {
            used += prefix[lo_s[k + 1]] != prefix[lo_s[k]] ? 1 : 0;
            const uint32_t w = dev_ceil_log2(lo_s[k + 1] - lo_s[k]);
            wmax = w > wmax ? w : wmax;
        }
        used = wave_sum(used);
        for (int d = 1; d < 64; d <<= 1) {
            const uint32_t o = __shfl_xor(wmax, d, 64);
            wmax = o > wmax ? o : wmax;
        }
        if (lane == 0) {
            // more occupied ranges than states, or a field longer than the GPU path takes
            if (used > L || wmax + R > kMaxFieldBitsGpu) status_s = (uint32_t)SH_ERR_UNSUPPORTED;
            red_j[0] = used;
            alloc_s[0] = 0;
        }
    }
    lds_barrier();

    // the histogram's copy for the table, loaded here so that it has arrived by the
    // barrier before the spread, which waits for every outstanding memory access
    const uint64_t h_mine = tid < 256 ? hist[tid] : 0;

    // ---- state allocation ----
    // One state per occupied range, then the remaining L - used states one at a time to
    // the range with the largest N_k * gain(f_k), the smallest k on ties; gain(f) =
    // log2(f + 1) - log2 f falls strictly with f.  Start from the proportional share (at
    // least one per occupied range); the greedy from there takes the L - total largest of
    // the increments N_k * gain(f), f >= f_start, in the order (gain down, k up), so every
    // candidate increment counts, by one binary search per other range, the increments
    // before it, and is taken when fewer than L - total are.  The result is the greedy
    // from one state per range when the last increment taken comes before the first one
    // left; otherwise the selection runs again from one state per range.
    const uint32_t used = red_j[0];
    const bool alloc_ok = used <= L && status_s == 0;
    if (tid < 256) {
        uint32_t f0 = 0;
        if (tid < K && count_s[tid] && alloc_ok) {
            const uint64_t share = (uint64_t)(L - used) * count_s[tid] / prefix[256];
            f0 = share > 1 ? (uint32_t)share : 1u;
        }
        f0_s[tid] = f0;
        add_s[tid] = 0;
        const uint32_t ws = wave_sum(f0);
        if (lane == 0) atomicAdd(&alloc_s[0], ws);
    }
    lds_barrier();
    uint32_t total = alloc_s[0];
    if (total > L) {  // the start overshot L: one state per range
        if (tid < 256) f0_s[tid] = tid < K && count_s[tid] && alloc_ok ? 1u : 0u;
        total = used;
        lds_barrier();
    }
    // the L - from largest increments beyond f0_s, counted in add_s.  Small cases hold the
    // increments and their ranks in LDS (over the cost factors, no longer needed) and split
    // the work per (increment, other range); others search the gain table per increment.
    uint64_t* inc = reinterpret_cast<uint64_t*>(sc);
    uint32_t* rank_of = reinterpret_cast<uint32_t*>(inc + kIncMax);
    // gain(f) = log2(f + 1) - log2 f in the DP's fixed point, for f = 0 .. L, after them
    uint32_t* gain_s = rank_of + kIncMax;
    static_assert(3 * kIncMax + kMaxLGpu + 1 <= kCostEntries, "gain table inside the cost area");
    for (uint32_t f = tid; f <= L; f += kBuildBlock)
        gain_s[f] = f == 0 ? 0u : (uint32_t)(dev_fixed_log2(f + 1) - dev_fixed_log2(f));
    lds_barrier();
    auto take = [&](uint32_t from) {
        const uint32_t Mp = L - from, n_inc = K * Mp;
        if (!alloc_ok || Mp == 0) return;
        // power-of-two strides: increment c = k << lm | t, pair q = c << lk | k2
        uint32_t lm = 0, lk = 0;
        while ((1u << lm) < Mp) ++lm;
        while ((1u << lk) < K) ++lk;
        const uint32_t n_slots = K << lm;
        if (n_inc <= kBuildBlock && K <= 256) {
            // one candidate per thread, c = k * Mp + t, keyed (g << 8) | (255 - k): g < 2^56
            // (counts < 2^32, gains <= 2^24), and a range's increments fall strictly, so
            // the keys are distinct and a larger key comes first in the order (g down, k up).
            // A candidate's rank is the number of larger keys; every lane reads the same
            // key in each round.
            const uint32_t c = tid, k = c < n_inc ? c / Mp : 0, t = c - k * Mp;
            bool valid = false;
            if (c < n_inc) {
                const uint32_t fk = f0_s[k];
                valid = count_s[k] && fk + t < L;
                inc[c] = valid ? ((uint64_t)count_s[k] * gain_s[fk + t]) << 8 | (255u - k) : 0ull;
            }
            lds_barrier();
            if (valid) {
                const uint64_t key = inc[c];
                uint32_t before = 0;
                uint32_t d = 0;
                for (; d + 8 <= n_inc; d += 8) {  // eight reads in flight
                    uint64_t v[8];
#pragma unroll
                    for (uint32_t r = 0; r < 8; ++r) v[r] = inc[d + r];
#pragma unroll
                    for (uint32_t r = 0; r < 8; ++r) before += v[r] > key ? 1u : 0u;
                }
                for (; d < n_inc; ++d) before += inc[d] > key ? 1u : 0u;
                if (before < Mp) atomicAdd(&add_s[k], 1u);
            }
        } else if (n_slots <= kIncMax && (n_slots << lk) <= 64 * kBuildBlock) {
            for (uint32_t c = tid; c < n_slots; c += kBuildBlock) {
                const uint32_t k = c >> lm, t = c & ((1u << lm) - 1);
                const uint32_t fk = f0_s[k];
                inc[c] = count_s[k] && t < Mp && fk + t < L ? (uint64_t)count_s[k] * gain_s[fk + t] : 0;
                rank_of[c] = t;
            }
            lds_barrier();
            for (uint32_t q = tid; q < (n_slots << lk); q += kBuildBlock) {
                const uint32_t c = q >> lk, k2 = q & ((1u << lk) - 1);
                const uint32_t k = c >> lm, t = c & ((1u << lm) - 1);
                if (k2 >= K || k2 == k || t >= Mp || !count_s[k2] || !count_s[k] || f0_s[k] + t >= L)
                    continue;
                const uint64_t g = inc[c];
                const uint64_t* row = inc + (k2 << lm);
                uint32_t lo = 0, hi = min(Mp, L - f0_s[k2]);  // increments of k2 before (g, k)
                while (lo < hi) {
                    const uint32_t mid = (lo + hi) >> 1;
                    const uint64_t g2 = row[mid];
                    if (g2 > g || (g2 == g && k2 < k)) lo = mid + 1;
                    else hi = mid;
                }
                if (lo) atomicAdd(&rank_of[c], lo);
            }
            lds_barrier();
            for (uint32_t c = tid; c < n_slots; c += kBuildBlock) {
                const uint32_t k = c >> lm, t = c & ((1u << lm) - 1);
                if (t < Mp && count_s[k] && f0_s[k] + t < L && rank_of[c] < Mp) atomicAdd(&add_s[k], 1u);
            }
        } else {
            for (uint32_t c = tid; c < n_inc; c += kBuildBlock) {
                const uint32_t k = c / Mp, t = c - k * Mp;
                const uint32_t fk = f0_s[k];
                if (!count_s[k] || fk + t >= L) continue;
                const uint64_t g = (uint64_t)count_s[k] * gain_s[fk + t];
                uint32_t rank = t;
                for (uint32_t k2 = 0; k2 < K && rank < Mp; ++k2) {
                    if (k2 == k || !count_s[k2]) continue;
                    const uint64_t c2 = count_s[k2];
                    const uint32_t f2 = f0_s[k2];
                    uint32_t lo = 0, hi = min(Mp, L - f2);  // increments of k2 before (g, k)
                    while (lo < hi) {
                        const uint32_t mid = (lo + hi) >> 1;
                        const uint64_t g2 = c2 * gain_s[f2 + mid];
                        if (g2 > g || (g2 == g && k2 < k)) lo = mid + 1;
                        else hi = mid;
                    }
                    rank += lo;
                }
                if (rank < Mp) atomicAdd(&add_s[k], 1u);
            }
        }
        lds_barrier();
    };
    take(total);
    if (wave == 0) {  // the check: lane l looks at ranges l, l + 64, l + 128, l + 192
        // is (g, k) later in the order than (g2, k2)?
        auto later = [](uint64_t g, uint32_t k, uint64_t g2, uint32_t k2) {
            return g < g2 || (g == g2 && k > k2);
        };
        uint64_t lg = 0, ng = 0;  // last increment taken, first one left
        uint32_t lk = 0xFFFFFFFFu, nk = 0xFFFFFFFFu;
        for (uint32_t k = lane; k < K; k += 64) {
            if (!count_s[k]) continue;
            const uint32_t f = f0_s[k] + add_s[k];
            if (f >= 2) {
                const uint64_t g = (uint64_t)count_s[k] * gain_s[f - 1];
                if (lk == 0xFFFFFFFFu || later(g, k, lg, lk)) {
                    lg = g;
                    lk = k;
                }
            }
            if (f < L) {
                const uint64_t g = (uint64_t)count_s[k] * gain_s[f];
                if (nk == 0xFFFFFFFFu || later(ng, nk, g, k)) {
                    ng = g;
                    nk = k;
                }
            }
        }
        for (int d = 1; d < 64; d <<= 1) {
            const uint64_t olg = __shfl_xor(lg, d, 64), ong = __shfl_xor(ng, d, 64);
            const uint32_t olk = __shfl_xor(lk, d, 64), onk = __shfl_xor(nk, d, 64);
            if (olk != 0xFFFFFFFFu && (lk == 0xFFFFFFFFu || later(olg, olk, lg, lk))) {
                lg = olg;
                lk = olk;
            }
            if (onk != 0xFFFFFFFFu && (nk == 0xFFFFFFFFu || later(ng, nk, ong, onk))) {
                ng = ong;
                nk = onk;
            }
        }
        if (lane == 0) alloc_s[1] = lk != 0xFFFFFFFFu && nk != 0xFFFFFFFFu && later(lg, lk, ng, nk);
    }
    lds_barrier();
    if (alloc_s[1]) {  // uniform
        if (tid < 256) {
            f0_s[tid] = tid < K && count_s[tid] && alloc_ok ? 1u : 0u;
            add_s[tid] = 0;
        }
        lds_barrier();
        take(used);
    }
    if (tid < K) freq_s[tid] = alloc_ok ? f0_s[tid] + add_s[tid] : 0u;
    if (!alloc_ok && tid == 0) status_s = (uint32_t)SH_ERR_UNSUPPORTED;
    lds_barrier();
    if (wave == 0) {  // cum_k = f_0 + ... + f_{k-1}; lane l sums ranges 4l .. 4l+3
        uint32_t v[4], sum = 0;
        for (uint32_t r = 0; r < 4; ++r) {
            const uint32_t k = 4 * lane + r;
            v[r] = k < K ? freq_s[k] : 0u;
            sum += v[r];
        }
        uint32_t incl = sum;
        for (int d = 1; d < 64; d <<= 1) {
            const uint32_t o = __shfl_up(incl, d, 64);
            if (lane >= (uint32_t)d) incl += o;
        }
        uint32_t c = incl - sum;
        for (uint32_t r = 0; r < 4; ++r) {
            const uint32_t k = 4 * lane + r;
            if (k < K) cum_s[k] = c;
            c += v[r];
        }
        if (lane == 63) cum_s[K] = incl;
    }
    __syncthreads();  // also orders the zeroing of the table before the writes below
    const bool ok = status_s == 0 && cum_s[K] == L;

    // slot spread: pair (k, j), j < f_k, goes to the slot equal to the number of pairs with
    // a smaller key (2j'+1)/(2 f_k'), or an equal key and a smaller range; then the tANS
    // tables of that slot: sub-state x = f_k + j, nb = R - floor(log2 x), next (x << nb) - L
    if (!ok)  // no usable table: every value is outside it
        for (uint32_t u = tid; u < 256; u += kBuildBlock) dt[kDTVt + 2 * u + 1] = 0x8000u;
    for (uint32_t p = tid; ok && p < L; p += kBuildBlock) {
        uint32_t k = 0, khi = K - 1;  // the range of slot p: the first k with cum_s[k + 1] > p
        while (k < khi) {
            const uint32_t mid = (k + khi) >> 1;
            if (cum_s[mid + 1] > p) khi = mid;
            else k = mid + 1;
        }
        const uint32_t j = p - cum_s[k], f = freq_s[k];
        uint32_t rank = 0;  // A = (2j + 1) f2 < 2L * L <= 2^23
        for (uint32_t k0 = 0; k0 < K; k0 += 4) {  // four ranges at a time, reads together
            uint32_t f2v[4];
#pragma unroll
            for (uint32_t r = 0; r < 4; ++r) f2v[r] = k0 + r < K ? freq_s[k0 + r] : 0u;
#pragma unroll
            for (uint32_t r = 0; r < 4; ++r) {
                const uint32_t k2 = k0 + r, f2 = f2v[r];
                if (f2 == 0) continue;  // a range without states takes no slot
                const uint32_t A = (2 * j + 1) * f2;  // >= 1
                const uint32_t odd_max = small_div(k2 < k ? A : A - 1, f);  // largest usable 2j'+1
                const uint32_t c = (odd_max + 1) >> 1;
                rank += c < f2 ? c : f2;
            }
        }
        const uint32_t x = f + j;
        const uint32_t nb = R - dev_floor_log2(x);
        const uint32_t next = (x << nb) - L;
        const uint32_t width = lo_s[k + 1] - lo_s[k];
        const uint32_t w = dev_ceil_log2(width);
        dt[kDTDec + 2 * rank] = (w + nb) | ((next * 8u) << 16);
        dt[kDTDec + 2 * rank + 1] = w | (((lo_s[k] - 128u) & 0xFFu) << 8) | ((width - 1) << 16);
        reinterpret_cast<uint16_t*>(dt + kDTEs)[cum_s[k] + j] = (uint16_t)rank;
    }
    for (uint32_t u = tid; u < 256; u += kBuildBlock) {  // the range of value u: lo_s[k] <= u < lo_s[k+1]
        uint32_t lo = 0, hi = K - 1;
        while (lo < hi) {
            const uint32_t mid = (lo + hi + 1) >> 1;
            if (lo_s[mid] <= u) lo = mid;
            else hi = mid - 1;
        }
        range_of_u[u] = lo;
    }
    lds_barrier();
    // encode entry of every value u
    for (uint32_t u = tid; ok && u < 256; u += kBuildBlock) {
        const uint32_t s = range_of_u[u];
        const uint32_t f = freq_s[s];
        const uint32_t w = dev_ceil_log2(lo_s[s + 1] - lo_s[s]);
        int32_t bias = 0, start = -(int32_t)L;
        if (f > 0) {
            const uint32_t m = dev_floor_log2(f);
            bias = (int32_t)((R - m) << (R + 1)) - (int32_t)(f << (R - m));
            start = (int32_t)cum_s[s] - (int32_t)f;
        }
        dt[kDTVt + 2 * u] = (uint32_t)bias;
        dt[kDTVt + 2 * u + 1] = (u - lo_s[s]) | (w << 8) | ((uint32_t)(start + (int32_t)kMaxLGpu) << 16) |
                                (f == 0 ? 0x8000u : 0u);
    }
    // canonical table, histogram and the header template (n and n_chunks left 0)
    uint16_t* lo16 = reinterpret_cast<uint16_t*>(dt + kDTLo);
    uint16_t* f16 = reinterpret_cast<uint16_t*>(dt + kDTFreq);
    for (uint32_t k = tid; k <= 256; k += kBuildBlock) lo16[k] = k <= K ? (uint16_t)lo_s[k] : 0;
    for (uint32_t k = tid; k < 256; k += kBuildBlock) f16[k] = k < K ? (uint16_t)freq_s[k] : 0;
    if (tid < 256) reinterpret_cast<uint64_t*>(dt + kDTHist)[tid] = h_mine;
    const uint32_t hbytes = (kHeaderFixed + 3 * K - 1 + 3) / 4 * 4;
    // header template: the fixed 32 bytes ("SHN1", version 3, log2 L, K, n = 0, C, S,
    // n_chunks = 0, header bytes), then freq[k] as u16 and lo[1..K-1] as bytes.  Every byte
    // is computed without branches (both table reads are made, one is kept), so that the
    // lanes of a wavefront do not serialise over the cases.
    for (uint32_t d = tid; d < kMaxHeaderDwords; d += kBuildBlock) {
        uint32_t word = 0;
        if (d < kHeaderFixed / 4) {
            word = d == 0 ? 0x314E4853u : d == 1 ? 3u | (R << 8) | ((K & 0xFFFFu) << 16)
                 : d == 4 ? a.C : d == 5 ? a.S : d == 7 ? hbytes : 0u;
        } else {
#pragma unroll
            for (uint32_t b = 0; b < 4; ++b) {
                const uint32_t at = 4 * d + b - kHeaderFixed;  // byte after the fixed part
                const uint32_t fi = (at >> 1) < 255 ? at >> 1 : 255u;
                const uint32_t li = at - 2 * K + 1 < 256 ? at - 2 * K + 1 : 0u;
                const uint32_t fv = (freq_s[fi] >> (8 * (at & 1))) & 0xFF, lv = lo_s[li] & 0xFF;
                const uint32_t byte = at < 2 * K ? fv : at < 3 * K - 1 ? lv : 0u;
                word |= byte << (8 * b);
            }
        }
        dt[kDTHdr + d] = 4 * d < hbytes ? word : 0;
    }
    if (tid == 0) {
        dt[kDTK] = K;
        dt[kDTLog2L] = R;
        dt[kDTL] = L;
        dt[kDTStatus] = ok || prefix[256] == 0 ? status_s : (uint32_t)SH_ERR_UNSUPPORTED;
        reinterpret_cast<uint64_t*>(dt + kDTN)[0] = prefix[256];
        dt[kDTHdrDwords] = hbytes / 4;
    }
}

sh_status launch_build_tables(const BuildArgs& b, void* stream) {
    if (b.nseg == 0) return SH_OK;
    hipStream_t s = (hipStream_t)stream;
    hipLaunchKernelGGL(k_build_cost, dim3(b.nseg * kCostBlocks), dim3(256), 0, s, b);
    hipLaunchKernelGGL(k_build_tables, dim3(b.nseg), dim3(kBuildBlock), 0, s, b);
    return hipGetLastError() == hipSuccess ? SH_OK : SH_ERR_HIP;
}

}  // namespace shn
