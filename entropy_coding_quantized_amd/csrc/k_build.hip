// Histogram and table-build kernels of the Shannonic codec for gfx950 (CDNA4, wave64):
// the offline step of the Shannonic talk notes ("Preprocessing: range selection by dynamic
// programming", paper section 4.1) run on the GPU, so that tables never leave HBM.
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
    const uint64_t lo = (uint64_t)(block - a.segs[seg].first_block) * kHistBytesPerBlock;
    const uint64_t hi = lo + kHistBytesPerBlock < n ? lo + kHistBytesPerBlock : n;
    const uint32_t copy = threadIdx.x & (kHistCopies - 1);
    // 16-byte groups fully inside [lo, hi); x is 16-byte aligned and lo a multiple of 16
    const uint64_t g0 = lo / 16, g1 = hi / 16;
    for (uint64_t g = g0 + threadIdx.x; g < g1; g += kHistBlock) {
        const v4u w = *reinterpret_cast<const v4u*>(x + 16 * g);
#pragma unroll
        for (int q = 0; q < 4; ++q) {
#pragma unroll
            for (int b = 0; b < 4; ++b) {
                const uint32_t u = ((w[q] >> (8 * b)) & 0xFF) ^ 0x80;
                atomicAdd(&h[u * kHistCopies + copy], 1u);
            }
        }
    }
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
constexpr uint64_t kInf = ~0ull;

// c_k(T) = #{f in [1, L) : N_k * gain(f) >= T}; gain(f) = log2(f+1) - log2(f) strictly
// decreases in f for f <= 256, so the count is a binary search.
__device__ __forceinline__ uint32_t items_at_least(uint32_t count, const uint32_t* gain,
                                                   uint32_t L, uint64_t T) {
    if (count == 0) return 0;
    uint32_t lo = 0, hi = L - 1;
    while (lo < hi) {
        const uint32_t mid = (lo + hi + 1) >> 1;
        if ((uint64_t)count * gain[mid] >= T) lo = mid;
        else hi = mid - 1;
    }
    return lo;
}

// floor(A / f) for A < 2^24, f >= 1: a correctly rounded float quotient, then corrected
__device__ __forceinline__ uint32_t small_div(uint32_t A, uint32_t f) {
    uint32_t q = (uint32_t)((float)A / (float)f);
    if (q * f > A) --q;
    else if ((q + 1) * f <= A) ++q;
    return q;
}

// DP work split of one layer: the i < 256 form four groups of 64 (one per lane), group g
// needing the j below 64 g + 64.  Work unit u (0..15) is group g = floor(sqrt(u)) and
// chunk c = u - g^2 of it: chunks c < 2g are the 32 j at 32c (all below every i of the group),
// chunk 2g the 64 j at 64g, where j < i per lane (a triangle, the same work as 32 full j).
// So all sixteen wavefronts get the same useful work; a diagonal chunk takes 64 passes
// for it, so the four of them are spread over the four SIMDs (wave w runs on SIMD w % 4).
__constant__ uint8_t kDpUnit[16] = {0, 3, 8, 15, 1, 2, 4, 5, 6, 7, 9, 10, 11, 12, 13, 14};
__global__ __launch_bounds__(kBuildBlock) void k_build_tables(const BuildArgs a) {
    __shared__ __align__(16) uint32_t sc[kCostEntries];  // cost factors; the DP's choices after it
    __shared__ uint32_t prefix[257];
    __shared__ uint64_t cbuf[2][256];              // C[i][k-1] and C[i][k], i < 256
    __shared__ uint64_t qbest[7][256];             // per j-chunk minima of a layer
    __shared__ uint8_t qarg[7][256];
    __shared__ uint64_t red_c[kBuildBlock / 64];
    __shared__ uint32_t red_j[kBuildBlock / 64];
    __shared__ uint32_t lo_s[257], freq_s[256], cum_s[257], range_of_u[256], count_s[256];
    __shared__ uint32_t lg_s[257], gain_s[256];
    __shared__ uint32_t g_at[64];                  // state allocation: G at the probes
    __shared__ uint64_t t_lo_s, t_hi_s;
    __shared__ uint32_t status_s;
    const uint32_t tid = threadIdx.x, lane = tid & 63, seg = blockIdx.x;
    const uint32_t wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const uint64_t* hist = a.hist + 256ull * seg;
    uint32_t* dt = a.tables + (uint64_t)seg * kDTDwords;
    uint8_t* arg = a.arg + (uint64_t)seg * kArgBytes;
    const uint32_t K = a.K, R = a.R, L = 1u << R;

    for (uint32_t i = tid; i < kDTDwords; i += kBuildBlock) dt[i] = 0;  // unused parts read 0
    {
        const v4u* src = reinterpret_cast<const v4u*>(a.scost + (uint64_t)seg * kCostEntries);
        v4u* dst = reinterpret_cast<v4u*>(sc);
#pragma unroll 3
        for (uint32_t i = tid; i < kCostEntries / 4; i += kBuildBlock) dst[i] = src[i];
    }
    if (tid < 257) lg_s[tid] = (uint32_t)dev_fixed_log2(tid);

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
    __syncthreads();
    if (tid < 256) {
        uint64_t before = 0;
        for (uint32_t w = 0; w < wave; ++w) before += red_c[w];
        prefix[tid + 1] = (uint32_t)(before + incl);
        gain_s[tid] = tid == 0 ? 0u : lg_s[tid + 1] - lg_s[tid];
    }
    if (tid == 0) {
        prefix[0] = 0;
        const uint64_t total = red_c[0] + red_c[1] + red_c[2] + red_c[3];
        status_s = total >= (1ull << 32) ? (uint32_t)SH_ERR_UNSUPPORTED : 0u;
    }
    __syncthreads();

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
        for (uint32_t i = tid; i < 256; i += kBuildBlock)
            cbuf[1][i] = i >= 1 ? (uint64_t)prefix[i] * sc[i * (i - 1) / 2] : kInf;
        __syncthreads();
        // work unit of this wavefront: the four diagonal units (0, 3, 8, 15) go to waves
        // 0-3, one per SIMD, the twelve others to waves 4-15
        const uint32_t unit = kDpUnit[wave];
        const uint32_t g = unit >= 9 ? 3 : unit >= 4 ? 2 : unit >= 1 ? 1 : 0;
        const uint32_t chunk = unit - g * g;
        const bool diag = chunk == 2 * g;
        const uint32_t ja = diag ? 64 * g : 32 * chunk, jb = diag ? 64 * g + 64 : 32 * chunk + 32;
        const uint32_t i = 64 * g + lane;
        const uint32_t row = i * (i - 1) / 2, pi = prefix[i];
        for (uint32_t k = 2; k < K; ++k) {
            const uint64_t* cp = cbuf[(k - 1) & 1];
            uint64_t best = kInf;
            uint32_t bj = 0;
            uint32_t j = max(k - 1, ja);
            if (!diag) {  // every j of the chunk lies below every i of the group
                for (; j + 4 <= jb; j += 4) {
#pragma unroll
                    for (uint32_t u = 0; u < 4; ++u) {
                        const uint64_t c = (uint64_t)(pi - prefix[j + u]) * sc[row + j + u] + cp[j + u];
                        if (c < best) {
                            best = c;
                            bj = j + u;
                        }
                    }
                }
                for (; j < jb; ++j) {
                    const uint64_t c = (uint64_t)(pi - prefix[j]) * sc[row + j] + cp[j];
                    if (c < best) {
                        best = c;
                        bj = j;
                    }
                }
            } else {  // j < i per lane
                for (; j + 4 <= jb; j += 4) {
#pragma unroll
                    for (uint32_t u = 0; u < 4; ++u) {
                        const uint64_t c = (uint64_t)(pi - prefix[j + u]) * sc[row + j + u] + cp[j + u];
                        if (j + u < i && c < best) {
                            best = c;
                            bj = j + u;
                        }
                    }
                }
                for (; j < jb; ++j) {
                    const uint64_t c = (uint64_t)(pi - prefix[j]) * sc[row + j] + cp[j];
                    if (j < i && c < best) {
                        best = c;
                        bj = j;
                    }
                }
            }
            qbest[chunk][i] = best;
            qarg[chunk][i] = (uint8_t)bj;
            __syncthreads();
            if (tid < 256) {  // chunks in increasing j: the first minimum keeps the smallest j
                uint64_t b = qbest[0][tid];
                uint32_t jj = qarg[0][tid];
                for (uint32_t cc = 1; cc <= 2 * (tid >> 6); ++cc)
                    if (qbest[cc][tid] < b) {
                        b = qbest[cc][tid];
                        jj = qarg[cc][tid];
                    }
                cbuf[k & 1][tid] = b;
                arg[k * 256 + tid] = (uint8_t)jj;
            }
            __syncthreads();
        }
        // layer K at i = 256
        {
            const uint64_t* cp = cbuf[(K - 1) & 1];
            const uint32_t j = K - 1 + tid;
            uint64_t c = kInf;
            if (j < 256) c = (uint64_t)(prefix[256] - prefix[j]) * sc[256 * 255 / 2 + j] + cp[j];
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
        __syncthreads();
        // the choices of layers 2 .. K-1 back from global memory (written by this block)
        uint8_t* argl = reinterpret_cast<uint8_t*>(sc);
        for (uint32_t d = 2 * 64 + tid; d < K * 64; d += kBuildBlock)
            reinterpret_cast<uint32_t*>(argl)[d] = reinterpret_cast<const uint32_t*>(arg)[d];
        __syncthreads();
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
    __syncthreads();
    for (uint32_t k = tid; k < K; k += kBuildBlock) count_s[k] = prefix[lo_s[k + 1]] - prefix[lo_s[k]];
    if (wave == 0) {
        uint32_t used = 0;
        for (uint32_t k = lane; k < K; k += 64) used += prefix[lo_s[k + 1]] != prefix[lo_s[k]] ? 1 : 0;
        used = wave_sum(used);
        if (lane == 0) {
            if (used > L) status_s = (uint32_t)SH_ERR_UNSUPPORTED;
            t_lo_s = 0;
            t_hi_s = 1ull << 57;  // above every N_k * gain(f)
            red_j[0] = used;
        }
        g_at[lane] = 0;
    }
    __syncthreads();

    // ---- state allocation ----
    // One state per occupied range, then the remaining M = L - used states one at a time to
    // the range with the largest N_k * gain(f_k), the smallest k on ties.  Each range's
    // gains fall strictly with f, so those M steps take the M largest items N_k * gain(f)
    // (f >= 1) in the order (value down, k up): find the value T of the M-th item, give
    // every range its items above T, and the items equal to T (at most one per range) to
    // the first ranges in k order.  T is found by a multiway search: per round, every
    // thread counts one range's items at or above one of nt probes, so the bracket
    // [t_lo, t_hi) with G(t_lo) >= M > G(t_hi) shrinks (nt + 1)-fold.
    const uint32_t used = red_j[0];
    const bool alloc_ok = used <= L && status_s == 0;
    const uint32_t M = alloc_ok && used > 0 ? L - used : 0;
    if (M > 0) {
        uint32_t kp = 16;
        while (kp < K) kp <<= 1;
        const uint32_t nt = kBuildBlock / kp;  // probes per round, at most 64
        const uint32_t kk = tid % kp, probe = tid / kp;
        while (true) {
            const uint64_t t_lo = t_lo_s, t_hi = t_hi_s;
            if (t_hi - t_lo <= 1) break;
            const uint64_t span = t_hi - t_lo;
            const uint64_t step = span / (nt + 1) + 1;
            if (tid < 64) g_at[tid] = 0;
            __syncthreads();
            const uint64_t T = t_lo + step * (probe + 1);
            if (kk < K && T < t_hi) {
                const uint32_t c = items_at_least(count_s[kk], gain_s, L, T);
                if (c) atomicAdd(&g_at[probe], c);
            }
            __syncthreads();
            if (wave == 0) {
                const uint64_t Tl = t_lo + step * (lane + 1);
                const bool probe_ok = lane < nt && Tl < t_hi;
                const uint64_t ge = __ballot(probe_ok && g_at[lane] >= M);
                const uint64_t lt = __ballot(probe_ok && g_at[lane] < M);
                if (lane == 0) {
                    // G falls with T: the probes at or above M form a prefix
                    if (ge) t_lo_s = t_lo + step * (63 - __builtin_clzll(ge) + 1);
                    if (lt) t_hi_s = t_lo + step * (__builtin_ctzll(lt) + 1);
                }
            }
            __syncthreads();
        }
    }
    if (wave == 0) {
        const uint64_t T = t_lo_s;
        uint32_t above = 0;
        for (uint32_t k = lane; k < K; k += 64) above += M ? items_at_least(count_s[k], gain_s, L, T + 1) : 0;
        const uint32_t r = M - wave_sum(above);  // items equal to T still to give
        uint32_t given = 0;                       // ties given to ranges below k
        for (uint32_t k0 = 0; k0 < K; k0 += 64) {
            const uint32_t k = k0 + lane;
            uint32_t f = 0;
            bool tie = false;
            if (k < K && count_s[k] && alloc_ok) {
                const uint32_t gt = M ? items_at_least(count_s[k], gain_s, L, T + 1) : 0;
                tie = M && items_at_least(count_s[k], gain_s, L, T) > gt;
                f = 1 + gt;
            }
            const uint64_t ties = __ballot(tie);
            const uint32_t rank = given + __builtin_amdgcn_mbcnt_hi(
                                              (uint32_t)(ties >> 32), __builtin_amdgcn_mbcnt_lo((uint32_t)ties, 0u));
            if (tie && rank < r) ++f;
            if (k < K) freq_s[k] = f;
            given += (uint32_t)__builtin_popcountll(ties);
        }
        if (!alloc_ok && lane == 0) status_s = (uint32_t)SH_ERR_UNSUPPORTED;
    }
    __syncthreads();
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
    __syncthreads();
    const bool ok = status_s == 0 && cum_s[K] == L;

    // slot spread: pair (k, j), j < f_k, goes to the slot equal to the number of pairs with
    // a smaller key (2j'+1)/(2 f_k'), or an equal key and a smaller range; then the tANS
    // tables of that slot: sub-state x = f_k + j, nb = R - floor(log2 x), next (x << nb) - L
    if (!ok)  // no usable table: every value is outside it
        for (uint32_t u = tid; u < 256; u += kBuildBlock) dt[kDTVt + 2 * u + 1] = 0x8000u;
    for (uint32_t p = tid; ok && p < L; p += kBuildBlock) {
        uint32_t k = 0;
        while (cum_s[k + 1] <= p) ++k;
        const uint32_t j = p - cum_s[k], f = freq_s[k];
        uint32_t rank = 0;
        for (uint32_t k2 = 0; k2 < K; ++k2) {
            const uint32_t f2 = freq_s[k2];
            if (!f2) continue;
            const uint32_t A = (2 * j + 1) * f2;
            const uint32_t odd_max = small_div(k2 < k ? A : A - 1, f);  // largest usable 2j'+1
            const uint32_t c = (odd_max + 1) >> 1;
            rank += c < f2 ? c : f2;
        }
        const uint32_t x = f + j;
        const uint32_t nb = R - dev_floor_log2(x);
        const uint32_t next = (x << nb) - L;
        const uint32_t width = lo_s[k + 1] - lo_s[k];
        const uint32_t w = dev_ceil_log2(width);
        dt[kDTDec + 2 * rank] = (w + nb) | ((next * 8u) << 16);
        dt[kDTDec + 2 * rank + 1] = w | (((lo_s[k] - 128u) & 0xFFu) << 8) | ((width - 1) << 16);
        reinterpret_cast<uint8_t*>(dt + kDTEs)[cum_s[k] + j] = (uint8_t)rank;
    }
    for (uint32_t k = tid; k < K; k += kBuildBlock)
        for (uint32_t u = lo_s[k]; u < lo_s[k + 1]; ++u) range_of_u[u] = k;
    __syncthreads();
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
        dt[kDTVt + 2 * u + 1] = (u - lo_s[s]) | (w << 8) | ((uint32_t)(start + 512) << 16) |
                                (f == 0 ? 0x8000u : 0u);
    }
    // canonical table, histogram and the header template (n and n_chunks left 0)
    uint16_t* lo16 = reinterpret_cast<uint16_t*>(dt + kDTLo);
    uint16_t* f16 = reinterpret_cast<uint16_t*>(dt + kDTFreq);
    for (uint32_t k = tid; k <= 256; k += kBuildBlock) lo16[k] = k <= K ? (uint16_t)lo_s[k] : 0;
    for (uint32_t k = tid; k < 256; k += kBuildBlock) f16[k] = k < K ? (uint16_t)freq_s[k] : 0;
    for (uint32_t u = tid; u < 256; u += kBuildBlock)
        reinterpret_cast<uint64_t*>(dt + kDTHist)[u] = hist[u];
    const uint32_t hbytes = (kHeaderFixed + 3 * K - 1 + 3) / 4 * 4;
    for (uint32_t d = tid; d < kMaxHeaderDwords; d += kBuildBlock) {
        uint32_t word = 0;
        for (uint32_t b = 0; b < 4; ++b) {
            const uint32_t at = 4 * d + b;
            uint32_t byte = 0;
            if (at < 4) byte = (uint32_t)"SHN1"[at];
            else if (at == 4) byte = 1;
            else if (at == 5) byte = R;
            else if (at < 8) byte = (K >> (8 * (at - 6))) & 0xFF;
            else if (at < 16) byte = 0;                                   // n
            else if (at < 20) byte = (a.C >> (8 * (at - 16))) & 0xFF;
            else if (at < 24) byte = (a.S >> (8 * (at - 20))) & 0xFF;
            else if (at < 28) byte = 0;                                   // n_chunks
            else if (at < 32) byte = (hbytes >> (8 * (at - 28))) & 0xFF;
            else if (at < kHeaderFixed + 2 * K) byte = (freq_s[(at - kHeaderFixed) >> 1] >> (8 * ((at - kHeaderFixed) & 1))) & 0xFF;
            else if (at < kHeaderFixed + 3 * K - 1) byte = lo_s[at - kHeaderFixed - 2 * K + 1] & 0xFF;
            word |= byte << (8 * b);
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
