// HIP kernels of the Shannonic codec for gfx950 (CDNA4, wave64).
//
// Method: "Shannonic: Efficient Entropy-Optimal Compression for ML Workloads" (MLSys 2026),
// talk notes, "Runtime encoding/decoding" (paper section 4.2, Algorithm 2): per value a
// range id through tANS plus raw offset bits, with table lookups, shifts, masks and adds
// only.  The chunked, lane-interleaved layout and everything about the GPU mapping are
// this library's own design; the pages give no GPU design.
//
// Mapping: one chunk of C values per half wavefront (32 lanes), one tANS state machine per
// lane.  At every step the 32 lanes of a chunk code 32 consecutive values, so their fields
// sit back to back in the bit stream; a 32-lane DPP prefix sum of the field lengths gives
// each lane its bit position.  Compressed words are staged through a per-chunk LDS ring
// fed by 128-bit loads; the decode table (<= 2 KB) lives in LDS.  No MFMA: there is no
// dense contraction.
#include <hip/hip_runtime.h>

#include "codec_internal.hpp"

namespace shn {

typedef __amdgpu_buffer_rsrc_t rsrc_t;
typedef unsigned int v4u __attribute__((ext_vector_type(4)));

// Raw buffer descriptor over [p, p + bytes): accesses past the end read 0 / are dropped.
__device__ __forceinline__ rsrc_t make_rsrc(const void* p, uint32_t bytes) {
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(p), (short)0, (int)bytes,
                                             0x00020000);
}

// Inclusive prefix sum within each 32-lane half of the wavefront (DPP row shifts, then
// the last lane of rows 0 and 2 added into rows 1 and 3).
__device__ __forceinline__ uint32_t scan32(uint32_t v) {
    v += (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x111, 0xF, 0xF, true);  // row_shr:1
    v += (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x112, 0xF, 0xF, true);  // row_shr:2
    v += (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x114, 0xF, 0xF, true);  // row_shr:4
    v += (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x118, 0xF, 0xF, true);  // row_shr:8
    v += (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x142, 0xA, 0xF, false); // row_bcast:15
    return v;
}

// Value of lane 31 of this lane's 32-lane half (ds_swizzle bit mode, or_mask = 31).
__device__ __forceinline__ uint32_t bcast31(uint32_t v) {
    return (uint32_t)__builtin_amdgcn_ds_swizzle((int)v, 0x3E0);
}

typedef const __attribute__((address_space(3))) uint32_t lds_u32;

// LDS byte offset of a __shared__ object
__device__ __forceinline__ uint32_t lds_offset(const void* p) {
    return (uint32_t)(uintptr_t)(const __attribute__((address_space(3))) void*)p;
}

// Record an error for the whole wavefront: one atomic from the first lane that has one,
// skipped when an error is already recorded (the first error wins).
__device__ __forceinline__ void report(int32_t* status, int32_t code, bool mine = true) {
    const uint64_t who = __builtin_amdgcn_ballot_w64(mine);
    if (!status || who == 0) return;
    const uint32_t lane = __builtin_amdgcn_mbcnt_hi(~0u, __builtin_amdgcn_mbcnt_lo(~0u, 0u));
    if (lane == (uint32_t)__builtin_ctzll(who) && __atomic_load_n(status, __ATOMIC_RELAXED) == 0)
        atomicCAS(status, 0, code);
}

// ------------------------------------------------------------------------------------
// segments: every launch covers one or more tensors; a block finds its tensor by a binary
// search over the descriptors' first blocks (uniform, so it runs on the scalar unit)
// ------------------------------------------------------------------------------------
__device__ __forceinline__ const SegDesc* find_seg(const SegDesc* segs, uint32_t nseg,
                                                    uint32_t block, bool compaction) {
    uint32_t lo = 0, hi = nseg;  // the last segment whose first block <= block
    while (hi - lo > 1) {
        const uint32_t mid = (lo + hi) >> 1;
        const uint32_t fb = compaction ? segs[mid].first_block_c : segs[mid].first_block;
        if (fb <= block) lo = mid;
        else hi = mid;
    }
    return &segs[lo];
}
__device__ __forceinline__ const SegDesc* codec_seg(const CodecArgs& a, uint32_t block,
                                                     bool compaction) {
    return a.nseg == 0 ? &a.one.seg : find_seg(a.many, a.nseg, block, compaction);
}

// ------------------------------------------------------------------------------------
// histogram: h[u] = #{i : x[i] + 128 == u}   (paper section 4.1)
// ------------------------------------------------------------------------------------
constexpr int kHistBlock = 256;
constexpr int kHistCopies = 32;
constexpr uint32_t kHistBytesPerBlock = 1u << 18;  // 256 KiB of values per block

__global__ void k_zero_u64(uint64_t* p, uint32_t count) {
    const uint32_t i = blockIdx.x * blockDim.x + threadIdx.x;
    if (i < count) p[i] = 0;
}

__global__ __launch_bounds__(kHistBlock) void k_histogram(const HistArgs a) {
    // 32 private copies per block, copy c of bin b at b * 32 + c: the 32 lanes of a half
    // wavefront hit 32 different banks even when every value is the same.
    __shared__ uint32_t h[256 * kHistCopies];
    for (int i = threadIdx.x; i < 256 * kHistCopies; i += kHistBlock) h[i] = 0;
    __syncthreads();
    const uint32_t block = blockIdx.x;
    const SegDesc* sg = find_seg(a.segs, a.nseg, block, false);
    const uint32_t seg = (uint32_t)(sg - a.segs);
    const uint8_t* x = sg->x;
    const uint64_t n = sg->n;
    const uint64_t lo = (uint64_t)(block - sg->first_block) * kHistBytesPerBlock;
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
    if (h.n_blocks > 0)
        hipLaunchKernelGGL(k_histogram, dim3(h.n_blocks), dim3(kHistBlock), 0, s, h);
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

__device__ __forceinline__ uint32_t header_bytes_dev(uint32_t K) { return (kHeaderFixed + 3 * K - 1 + 3) / 4 * 4; }
__device__ __forceinline__ uint32_t dev_ceil_log2(uint32_t m) { return m <= 1 ? 0 : 32 - __builtin_clz(m - 1); }
__device__ __forceinline__ uint32_t dev_floor_log2(uint32_t x) { return 31 - __builtin_clz(x); }

constexpr int kBuildBlock = 256;

__global__ __launch_bounds__(kBuildBlock) void k_build_tables(const BuildArgs a) {
    __shared__ uint64_t prefix[257];
    __shared__ uint64_t cprev[257], ccur[257];
    __shared__ uint64_t gain[257];
    __shared__ uint32_t lo_s[257], freq_s[256], cum_s[257], range_of_u[256];
    __shared__ uint64_t count_s[256];
    __shared__ uint64_t lgN_s;
    __shared__ uint32_t status_s;
    const uint32_t tid = threadIdx.x, seg = blockIdx.x;
    const uint64_t* hist = a.hist + 256 * (uint64_t)seg;
    uint32_t* dt = a.tables + (uint64_t)seg * kDTDwords;
    uint64_t* cost = a.cost + (uint64_t)seg * kCostEntries;
    uint16_t* arg = a.arg + (uint64_t)seg * 257 * 257;
    const uint32_t K = a.K, R = a.R, L = 1u << R;
    constexpr uint64_t INF = ~0ull;

    for (uint32_t i = tid; i < kDTDwords; i += kBuildBlock) dt[i] = 0;  // unused parts read 0
    if (tid == 0) {
        uint64_t acc = 0;
        prefix[0] = 0;
        for (int v = 0; v < 256; ++v) prefix[v + 1] = (acc += hist[v]);
        status_s = acc >= (1ull << 32) ? (uint32_t)SH_ERR_UNSUPPORTED : 0u;
        lgN_s = dev_fixed_log2(acc);
    }
    __syncthreads();
    const uint64_t lgN = lgN_s;

    // cost of [j, i) for every 0 <= j < i <= 256, row i holding j = 0..i-1:
    // N_R * (log2 N - log2 N_R) + N_R * ceil(log2 (i - j)), in units of 2^-24 bit
    for (uint32_t idx = tid; idx < kCostEntries; idx += kBuildBlock) {
        uint32_t i = (uint32_t)((1.0 + sqrt(1.0 + 8.0 * (double)idx)) * 0.5);
        while ((uint64_t)i * (i - 1) / 2 > idx) --i;
        while ((uint64_t)(i + 1) * i / 2 <= idx) ++i;
        const uint32_t j = idx - i * (i - 1) / 2;
        const uint64_t nr = prefix[i] - prefix[j];
        cost[idx] = nr ? nr * (lgN - dev_fixed_log2(nr)) + nr * ((uint64_t)dev_ceil_log2(i - j) << kLgFrac)
                       : 0;
    }
    for (uint32_t i = tid; i <= 256; i += kBuildBlock) cprev[i] = i == 0 ? 0 : INF;
    __syncthreads();

    // C[i][k] = min over j < i of C[j][k-1] + cost[j, i): the smallest j wins ties
    for (uint32_t k = 1; k <= K; ++k) {
        for (uint32_t i = tid; i <= 256; i += kBuildBlock) {
            uint64_t best = INF;
            uint32_t bj = 0;
            if (i >= k) {
                const uint64_t* row = cost + (uint64_t)i * (i - 1) / 2;
                for (uint32_t j = k - 1; j < i; ++j) {
                    if (cprev[j] == INF) continue;
                    const uint64_t c = cprev[j] + row[j];
                    if (c < best) {
                        best = c;
                        bj = j;
                    }
                }
            }
            ccur[i] = best;
            arg[k * 257 + i] = (uint16_t)bj;
        }
        __syncthreads();
        for (uint32_t i = tid; i <= 256; i += kBuildBlock) cprev[i] = ccur[i];
        __syncthreads();
    }

    if (tid == 0) {
        uint32_t i = 256;
        lo_s[K] = 256;
        for (uint32_t k = K; k >= 1; --k) {
            i = arg[k * 257 + i];
            lo_s[k - 1] = i;
        }
    }
    __syncthreads();
    for (uint32_t k = tid; k < K; k += kBuildBlock) count_s[k] = prefix[lo_s[k + 1]] - prefix[lo_s[k]];
    for (uint32_t f = tid; f <= L; f += kBuildBlock)
        gain[f] = f == 0 ? 0 : dev_fixed_log2(f + 1) - dev_fixed_log2(f);
    __syncthreads();

    // state allocation: one state per occupied range, then every remaining state to the
    // range with the largest N_k * (log2(f_k + 1) - log2 f_k), first k on ties
    if (tid == 0) {
        uint32_t used = 0;
        for (uint32_t k = 0; k < K; ++k) {
            freq_s[k] = count_s[k] ? 1 : 0;
            used += freq_s[k];
        }
        if (used > L) status_s = (uint32_t)SH_ERR_UNSUPPORTED;
        if (used > 0 && status_s == 0) {
            for (; used < L; ++used) {
                uint32_t best = K;
                uint64_t bg = 0;
                for (uint32_t k = 0; k < K; ++k) {
                    if (!count_s[k]) continue;
                    const uint64_t g = count_s[k] * gain[freq_s[k]];
                    if (best == K || g > bg) {
                        best = k;
                        bg = g;
                    }
                }
                freq_s[best]++;
            }
        }
        uint32_t c = 0;
        for (uint32_t k = 0; k < K; ++k) {
            cum_s[k] = c;
            c += freq_s[k];
        }
        cum_s[K] = c;
    }
    __syncthreads();
    const bool ok = status_s == 0 && cum_s[K] == L;

    // slot spread: pair (k, j), j < f_k, goes to the slot equal to the number of pairs with
    // a smaller key (2j'+1)/(2 f_k'), or an equal key and a smaller range; then the tANS
    // tables of that slot: sub-state x = f_k + j, nb = R - floor(log2 x), next (x << nb) - L
    if (!ok)  // no usable table: every value is outside it
        for (uint32_t u = tid; u < 256; u += kBuildBlock) dt[kDTVt + 2 * u + 1] = 0x80000000u;
    for (uint32_t p = tid; ok && p < L; p += kBuildBlock) {
        uint32_t k = 0;
        while (cum_s[k + 1] <= p) ++k;
        const uint32_t j = p - cum_s[k], f = freq_s[k];
        uint32_t rank = 0;
        for (uint32_t k2 = 0; k2 < K; ++k2) {
            const uint32_t f2 = freq_s[k2];
            if (!f2) continue;
            const uint32_t A = (2 * j + 1) * f2;
            const uint32_t odd_max = k2 < k ? A / f : (A - 1) / f;  // largest usable 2j'+1
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
                                (f == 0 ? 0x80000000u : 0u);
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
    hipLaunchKernelGGL(k_build_tables, dim3(b.nseg), dim3(kBuildBlock), 0, (hipStream_t)stream, b);
    return hipGetLastError() == hipSuccess ? SH_OK : SH_ERR_HIP;
}

// ------------------------------------------------------------------------------------
// decode
// ------------------------------------------------------------------------------------
constexpr uint32_t kRing = 256;               // compressed dwords resident per chunk
// each ring starts on a 2 KB boundary (so the wrapped word address is one and-or) and is
// followed by a copy of its dword 0, so a two-word read never wraps
constexpr uint32_t kRingStride = 512;
constexpr uint32_t kFill = 128;               // dwords per refill: 32 lanes x 16 bytes
// decode table in LDS, 8 bytes per slot (a random 8-byte LDS read costs less than half of
// a 16-byte one): e0 = need | maxo << 16 | base << 24, e1 = w | next << 16, where need =
// w_s + nb, maxo = |range| - 1, base = the range's first value as int8 bits and next = the
// LDS byte address of the entry reached with zero state bits
constexpr uint32_t kTabDwords = 512;

// 16 bytes of the chunk starting at dword d (dwords at or past cdw read as 0).
__device__ __forceinline__ v4u load_words(rsrc_t r, uint32_t chunk_byte, uint32_t d,
                                          uint32_t cdw) {
    if (d + 4 <= cdw)
        return __builtin_bit_cast(v4u, __builtin_amdgcn_raw_buffer_load_b128(
                                           r, (int)(chunk_byte + 4 * d), 0, 0));
    v4u v = {0, 0, 0, 0};
    for (uint32_t k = 0; k < 4; ++k)
        if (d + k < cdw)
            v[k] = __builtin_amdgcn_raw_buffer_load_b32(r, (int)(chunk_byte + 4 * (d + k)), 0, 0);
    return v;
}

typedef unsigned int v2u __attribute__((ext_vector_type(2)));

typedef const __attribute__((address_space(3))) v2u lds_v2u;

// Per-chunk decoder state of one half wavefront.
struct DecChain {
    uint32_t nc, cdw, cbyte, ring, ring_byte, lanes, pos, addr, res_hi, refill_at, err, vout;
    v4u pf;
};

constexpr int kDecBlock = 256;  // 4 wavefronts
// ILP chunks per lane: a wavefront decodes 2 * ILP chunks, lanes 32h..32h+31 take chunks
// 2k + h (k < ILP) of the wavefront's group.  ILP = 1 is the one launched: measured on
// MI355X, two independent chains per lane ran slower than twice as many wavefronts.
template <int ILP>
__global__ __launch_bounds__(kDecBlock) void k_decode(const CodecArgs a) {
    constexpr uint32_t kChunksPerWave = 2 * ILP;
    constexpr uint32_t kChunksPerBlock = kDecBlock / 64 * kChunksPerWave;
    __shared__ __align__(16) uint32_t sm[kTabDwords + kChunksPerBlock * kRingStride];
    const uint32_t tid = threadIdx.x, lane = tid & 63, li = lane & 31, hw = lane >> 5;
    const uint32_t block = __builtin_amdgcn_readfirstlane(blockIdx.x);
    const SegDesc* sg = codec_seg(a, block, false);
    const uint32_t bseg = block - sg->first_block;  // block within its segment
    // wavefront index within the segment, uniform so that descriptors stay scalar
    const uint32_t wid = __builtin_amdgcn_readfirstlane(bseg * (kDecBlock / 64) + (tid >> 6));
    const uint32_t wv = wid & (kDecBlock / 64 - 1);
    const uint32_t tab_byte = lds_offset(sm);
    const uint32_t* dec = sg->tab ? sg->tab + kDTDec : a.one.tab;
    const uint32_t* hdr = sg->tab ? sg->tab + kDTHdr : a.one.hdr;
    const uint32_t n_chunks = sg->n_chunks;
    const uint64_t n = sg->n;
    const uint32_t index_at = header_bytes_dev(a.K);
    const uint32_t payload_at = index_at + 4 * (n_chunks + 1);
    const uint64_t in_nbytes = sg->c_bytes;

    // rearrange the table's entries into the LDS form
    for (uint32_t i = tid; i < a.L; i += kDecBlock) {
        const uint32_t e0 = dec[2 * i], e1 = dec[2 * i + 1];
        sm[2 * i] = (e0 & 0xFFFF) | (e1 & 0x00FF0000u) | ((e1 & 0xFF00u) << 16);
        sm[2 * i + 1] = (e1 & 31) | ((tab_byte + (e0 >> 16)) << 16);
    }

    const rsrc_t rin = make_rsrc(sg->c, (uint32_t)in_nbytes);
    if (wid == 0) {
        // header and index ends: the container must belong to this table and fit in_nbytes
        // a device table that failed to build, or was built from no values, decodes nothing
        bool bad = sg->tab && (sg->tab[kDTStatus] != 0 ||
                               (n > 0 && (sg->tab[kDTN] | sg->tab[kDTN + 1]) == 0));
        for (uint32_t i = lane; i < index_at / 4; i += 64)
            bad |= __builtin_amdgcn_raw_buffer_load_b32(rin, (int)(4 * i), 0, 0) !=
                   header_dword(hdr, i, n, n_chunks);
        if (lane == 0) {
            const uint32_t first = __builtin_amdgcn_raw_buffer_load_b32(rin, (int)index_at, 0, 0);
            const uint32_t last = __builtin_amdgcn_raw_buffer_load_b32(
                rin, (int)(index_at + 4 * n_chunks), 0, 0);
            bad |= first != 0 || (uint64_t)payload_at + last > in_nbytes;
        }
        report(a.status, SH_ERR_CORRUPT_STREAM, bad);
    }

    // output: per-wavefront descriptor over the wavefront's chunks
    const uint32_t group = kChunksPerWave * wid;
    const uint64_t grp_first = (uint64_t)group * a.C;
    const uint64_t grp_len = grp_first < n ? n - grp_first : 0;
    const uint64_t grp_cap = (uint64_t)kChunksPerWave * a.C;
    const rsrc_t rout = make_rsrc(sg->x + (grp_first < n ? grp_first : 0),
                                  (uint32_t)(grp_len < grp_cap ? grp_len : grp_cap));

    DecChain ch[ILP];
#pragma unroll
    for (int k = 0; k < ILP; ++k) {
        DecChain& c = ch[k];
        const uint32_t slot = 2 * k + hw;
        const uint32_t chunk = group + slot;
        c.ring = kTabDwords + (wv * kChunksPerWave + slot) * kRingStride;
        c.ring_byte = tab_byte + 4 * c.ring;
        c.vout = slot * a.C + li;
        c.nc = 0;
        c.cdw = 0;
        c.cbyte = 0;
        c.err = 0;
        if (chunk < n_chunks) {
            const uint32_t o0 = __builtin_amdgcn_raw_buffer_load_b32(rin, (int)(index_at + 4 * chunk), 0, 0);
            const uint32_t o1 = __builtin_amdgcn_raw_buffer_load_b32(rin, (int)(index_at + 4 * chunk + 4), 0, 0);
            const uint64_t first = (uint64_t)chunk * a.C;
            const uint32_t m = (uint32_t)((n - first) < a.C ? (n - first) : a.C);
            const bool ok = o0 <= o1 && ((o0 | o1) & 3) == 0 &&
                            (o1 - o0) <= 4 * chunk_bound_dwords(m, a.R) &&
                            (uint64_t)payload_at + o1 <= in_nbytes;
            if (ok) {
                c.nc = m;
                c.cdw = (o1 - o0) >> 2;
                c.cbyte = payload_at + o0;
            } else {
                c.err = 1;
            }
        }
        c.lanes = c.nc < 32 ? c.nc : 32;
        // first two refills, plus the third in flight
        for (uint32_t b = 0; b < 2; ++b) {
            const uint32_t d = b * kFill + 4 * li;
            const v4u v = load_words(rin, c.cbyte, d, c.cdw);
            *reinterpret_cast<v4u*>(&sm[c.ring + d]) = v;
            if (b == 0 && li == 0) sm[c.ring + kRing] = v[0];
        }
        c.res_hi = 2 * kFill;  // dwords [res_hi - kRing, res_hi) are in the ring
        c.pf = load_words(rin, c.cbyte, c.res_hi + 4 * li, c.cdw);
        // refills are checked every other step; one is due once the next two steps could
        // read past res_hi (each advances at most 16 dwords): pos >> 5 >= res_hi - 33
        c.refill_at = c.res_hi < c.cdw ? (c.res_hi - 33) * 32 : 0xFFFFFFFFu;
    }
    __syncthreads();

    uint32_t nc_min = 0xFFFFFFFFu, nc_max = 0;
#pragma unroll
    for (int k = 0; k < ILP; ++k) {
        DecChain& c = ch[k];
        // initial slots: lane l's R bits at l * R
        c.addr = tab_byte;  // LDS byte address of the current slot's decode entry
        if (li < c.lanes) {
            const uint32_t p = li * a.R;
            const uint32_t bits = __builtin_amdgcn_alignbit(sm[c.ring + (p >> 5) + 1], sm[c.ring + (p >> 5)], p);
            c.addr = tab_byte + ((bits & (a.L - 1)) << 3);
        }
        c.pos = c.lanes * a.R;
        const uint32_t lo = __builtin_amdgcn_readlane(c.nc, 0), hi = __builtin_amdgcn_readlane(c.nc, 32);
        nc_min = nc_min < lo ? nc_min : lo;
        nc_min = nc_min < hi ? nc_min : hi;
        nc_max = nc_max > lo ? nc_max : lo;
        nc_max = nc_max > hi ? nc_max : hi;
    }
    const uint32_t full = nc_min >> 5;
    const uint32_t steps = (nc_max + 31) >> 5;
    uint64_t bad_offsets = 0;  // lanes that decoded an offset outside its range

    auto refill = [&](DecChain& c) {
        if (c.pos >= c.refill_at) {
            const uint32_t d = (c.res_hi + 4 * li) & (kRing - 1);
            *reinterpret_cast<v4u*>(&sm[c.ring + d]) = c.pf;
            if (d == 0) sm[c.ring + kRing] = c.pf[0];
            c.res_hi += kFill;
            c.refill_at = c.res_hi < c.cdw ? (c.res_hi - 33) * 32 : 0xFFFFFFFFu;
            c.pf = load_words(rin, c.cbyte, c.res_hi + 4 * li, c.cdw);
        }
    };

    // One step of every chain: each lane decodes one value per chain.  The entries for the
    // step were read at the end of the previous one, so the serial path per chain is
    // scan -> ring read -> bit extract -> next entry read; the chains go through these
    // phases side by side so that one chain's LDS waits overlap the other's work.
    auto full_step = [&](const v2u (&e)[ILP], v2u (&en)[ILP], uint32_t t) {
        uint32_t incl[ILP], start[ILP], w0[ILP], w1[ILP];
#pragma unroll
        for (int k = 0; k < ILP; ++k) {
            const uint32_t posm = ch[k].pos - e[k][0];   // bits 16.. of e0 and sums ignored
            incl[k] = scan32(e[k][0]);
            start[k] = posm + incl[k];                   // only bits 0..12 matter below
        }
#pragma unroll
        for (int k = 0; k < ILP; ++k) {
            const uint32_t rb = ((start[k] >> 3) & (4 * kRing - 4)) | ch[k].ring_byte;
            const lds_u32* rp = (const lds_u32*)(uintptr_t)rb;
            w0[k] = rp[0];
            w1[k] = rp[1];
        }
#pragma unroll
        for (int k = 0; k < ILP; ++k) {
            const uint32_t bits = __builtin_amdgcn_alignbit(w1[k], w0[k], start[k]);
            const uint32_t v = __builtin_amdgcn_ubfe(bits, 0, e[k][0]);   // the field (need bits)
            const uint32_t o = __builtin_amdgcn_ubfe(bits, 0, e[k][1]);   // its low w_s bits
            ch[k].addr = ((v >> (e[k][1] & 31)) << 3) + (e[k][1] >> 16);
            en[k] = *(lds_v2u*)(uintptr_t)ch[k].addr;
            bad_offsets |= __builtin_amdgcn_ballot_w64(o > ((e[k][0] >> 16) & 0xFF));
            __builtin_amdgcn_raw_buffer_store_b8((uint8_t)(o + (e[k][0] >> 24)), rout,
                                                 (int)ch[k].vout, (int)(t * 32), 0);
        }
#pragma unroll
        for (int k = 0; k < ILP; ++k) ch[k].pos += bcast31(incl[k]) & 0xFFFFu;
    };

    v2u e[ILP], e2[ILP];
#pragma unroll
    for (int k = 0; k < ILP; ++k) e[k] = *(lds_v2u*)(uintptr_t)ch[k].addr;
    uint32_t t = 0;
    for (; t + 2 <= full; t += 2) {  // two steps per trip, so the entries alternate registers
        full_step(e, e2, t);
        full_step(e2, e, t + 1);
#pragma unroll
        for (int k = 0; k < ILP; ++k) refill(ch[k]);
    }
    if (t < full) {
        full_step(e, e2, t);
#pragma unroll
        for (int k = 0; k < ILP; ++k) {
            e[k] = e2[k];
            refill(ch[k]);
        }
        ++t;
    }
    for (; t < steps; ++t) {  // chunks shorter than the others: lanes past n_c take no bits
#pragma unroll
        for (int k = 0; k < ILP; ++k) {
            DecChain& c = ch[k];
            const bool act = t * 32 + li < c.nc;
            v2u ek = e[k];
            if (!act) ek = v2u{0, 0};
            const uint32_t incl = scan32(ek[0]);
            const uint32_t start = c.pos - ek[0] + incl;
            const uint32_t rb = ((start >> 3) & (4 * kRing - 4)) | c.ring_byte;
            const lds_u32* rp = (const lds_u32*)(uintptr_t)rb;
            const uint32_t bits = __builtin_amdgcn_alignbit(rp[1], rp[0], start);
            const uint32_t v = __builtin_amdgcn_ubfe(bits, 0, ek[0]);
            const uint32_t o = __builtin_amdgcn_ubfe(bits, 0, ek[1]);
            if (act) {
                c.err |= o > ((ek[0] >> 16) & 0xFF);
                __builtin_amdgcn_raw_buffer_store_b8((uint8_t)(o + (ek[0] >> 24)), rout,
                                                     (int)c.vout, (int)(t * 32), 0);
                c.addr = ((v >> (ek[1] & 31)) << 3) + (ek[1] >> 16);
            }
            c.pos += bcast31(incl) & 0xFFFFu;
            e[k] = *(lds_v2u*)(uintptr_t)c.addr;
            refill(c);
        }
    }

    // a valid chunk leaves every lane in slot 0 and ends in its last word, zero-padded
    uint32_t err = 0;
#pragma unroll
    for (int k = 0; k < ILP; ++k) {
        DecChain& c = ch[k];
        err |= c.err;
        if (c.nc > 0) {
            if (li < c.lanes && c.addr != tab_byte) err = 1;
            if (((c.pos + 31) >> 5) != c.cdw) err = 1;
            else if ((c.pos & 31) && (sm[c.ring + ((c.pos >> 5) & (kRing - 1))] >> (c.pos & 31)) != 0)
                err = 1;
        }
    }
    report(a.status, SH_ERR_CORRUPT_STREAM, err != 0 || bad_offsets != 0);
}

sh_status launch_decode(const CodecArgs& a, uint32_t total_blocks, void* stream) {
    if (total_blocks == 0) return SH_OK;
    hipLaunchKernelGGL(k_decode<1>, dim3(total_blocks), dim3(kDecBlock), 0, (hipStream_t)stream, a);
    return hipGetLastError() == hipSuccess ? SH_OK : SH_ERR_HIP;
}

// ------------------------------------------------------------------------------------
// encode, kernel 1: every chunk into a worst-case slot of the workspace
// ------------------------------------------------------------------------------------
// tANS encodes backwards.  Each lane walks its values from the last step to the first;
// at every step the 32 fields of a chunk are placed right to left: the step's fields end
// where the later steps' fields begin, so a 32-lane prefix sum of the lengths gives every
// field's bit position.  Fields are OR-ed into a 256-dword LDS ring that is flushed to
// the chunk's slot 128 dwords at a time, highest first; the chunk ends up right-aligned
// in its slot with the lanes' final states (the decoder's initial states) in front.
constexpr int kEncBlock = 256;
constexpr uint32_t kERing = 256;
constexpr uint32_t kEncHalfDwords = 256 /* input tile, 32 steps x 32 lanes bytes */ + kERing;
constexpr uint32_t kVtDwords = 512 + 64;  // value table + encTable bytes

__device__ __forceinline__ void ring_or(uint32_t* sm, uint32_t ring, uint32_t pos,
                                        uint32_t field, uint32_t len) {
    if (len == 0) return;
    const uint64_t wide = (uint64_t)field << (pos & 31);
    const uint32_t d = pos >> 5;
    atomicOr(&sm[ring + (d & (kERing - 1))], (uint32_t)wide);
    if ((pos & 31) + len > 32) atomicOr(&sm[ring + ((d + 1) & (kERing - 1))], (uint32_t)(wide >> 32));
}

__global__ __launch_bounds__(kEncBlock) void k_encode_chunks(const CodecArgs a) {
    __shared__ __align__(16) uint32_t sm[kVtDwords + 8 * kEncHalfDwords];
    const uint32_t tid = threadIdx.x, lane = tid & 63, li = lane & 31, hw = lane >> 5;
    const uint32_t block = __builtin_amdgcn_readfirstlane(blockIdx.x);
    const SegDesc* sg = codec_seg(a, block, false);
    const uint32_t bseg = block - sg->first_block;
    const uint32_t wid = __builtin_amdgcn_readfirstlane(bseg * (kEncBlock / 64) + (tid >> 6));
    const uint32_t wv = wid & (kEncBlock / 64 - 1);
    const uint32_t* vt = sg->tab ? sg->tab + kDTVt : a.one.tab;
    const uint8_t* es_src = sg->tab ? reinterpret_cast<const uint8_t*>(sg->tab + kDTEs) : a.one.es;
    const uint32_t n_chunks = sg->n_chunks;
    const uint64_t n = sg->n;
    for (uint32_t i = tid; i < 512; i += kEncBlock) sm[i] = vt[i];
    for (uint32_t i = tid; i < 64; i += kEncBlock) {
        sm[512 + i] = (uint32_t)es_src[4 * i] | ((uint32_t)es_src[4 * i + 1] << 8) |
                      ((uint32_t)es_src[4 * i + 2] << 16) | ((uint32_t)es_src[4 * i + 3] << 24);
    }
    const uint8_t* es = reinterpret_cast<const uint8_t*>(&sm[512]);
    const uint32_t half = kVtDwords + (wv * 2 + hw) * kEncHalfDwords;
    const uint32_t tile = half;            // 256 dwords: bytes of 32 steps x 32 lanes
    const uint32_t ring = half + 256;      // 256 dwords
    for (uint32_t i = li; i < kERing; i += 32) sm[ring + i] = 0;

    const uint32_t pair = 2 * wid;
    const uint32_t chunk = pair + hw;
    const uint64_t pair_first = (uint64_t)pair * a.C;
    const uint64_t pair_len = pair_first < n ? n - pair_first : 0;
    const rsrc_t rin = make_rsrc(sg->x + (pair_first < n ? pair_first : 0),
                                 (uint32_t)(pair_len < 2ull * a.C ? pair_len : 2ull * a.C));
    const uint32_t slot0 = sg->slot_base + (pair < n_chunks ? pair : 0);
    const rsrc_t rslot = make_rsrc(a.slots + (uint64_t)slot0 * a.slot_dwords, 8u * a.slot_dwords);
    const uint32_t in_base = hw * a.C;          // byte offset of this chunk in rin
    const uint32_t slot_base = hw * a.slot_dwords * 4;
    uint32_t nc = 0;
    if (chunk < n_chunks) {
        const uint64_t first = (uint64_t)chunk * a.C;
        nc = (uint32_t)((n - first) < a.C ? (n - first) : a.C);
    }
    const uint32_t lanes = nc < 32 ? nc : 32;
    const uint32_t nc_lo = __builtin_amdgcn_readlane(nc, 0), nc_hi = __builtin_amdgcn_readlane(nc, 32);
    const uint32_t steps = ((nc_lo > nc_hi ? nc_lo : nc_hi) + 31) >> 5;
    const uint32_t L = a.L, R1 = a.R + 1;

    // 32 bytes of input tile tl for this lane (32 steps x 32 lanes = 1 KB per tile)
    auto load_tile = [&](uint32_t tl, v4u& p0, v4u& p1) {
        const uint32_t b = tl * 1024 + 32 * li;   // chunk-relative byte
        if (b + 32 <= nc) {
            p0 = __builtin_bit_cast(v4u, __builtin_amdgcn_raw_buffer_load_b128(rin, (int)(in_base + b), 0, 0));
            p1 = __builtin_bit_cast(v4u, __builtin_amdgcn_raw_buffer_load_b128(rin, (int)(in_base + b + 16), 0, 0));
        } else {
            p0 = v4u{0, 0, 0, 0};
            p1 = v4u{0, 0, 0, 0};
            for (uint32_t k = 0; k < 32; ++k)
                if (b + k < nc) {
                    const uint32_t byte = __builtin_amdgcn_raw_buffer_load_b8(rin, (int)(in_base + b + k), 0, 0);
                    if (k < 16) p0[k >> 2] |= byte << (8 * (k & 3));
                    else p1[(k - 16) >> 2] |= byte << (8 * (k & 3));
                }
        }
    };
    v4u p0, p1;
    if (steps > 0) load_tile((steps - 1) >> 5, p0, p1);
    __syncthreads();

    uint32_t X = L;
    uint32_t P = a.slot_dwords * 32;   // fields go below P, right to left
    uint32_t fmark = a.slot_dwords;    // dwords at or above fmark are in the slot
    uint32_t pay = 0, bad = sg->tab && sg->tab[kDTStatus] != 0 && nc > 0;

    auto flush_block = [&](uint32_t blk) {  // ring dwords [blk, blk + 128) -> slot
        uint32_t* r = &sm[ring + ((blk + 4 * li) & (kERing - 1))];
        const v4u v = *reinterpret_cast<v4u*>(r);
        *reinterpret_cast<v4u*>(r) = v4u{0, 0, 0, 0};
        __builtin_amdgcn_raw_buffer_store_b128(v, rslot, (int)(slot_base + 4 * (blk + 4 * li)), 0, 0);
    };

    for (uint32_t t = steps; t-- > 0;) {
        if ((t & 31) == 31 || t + 1 == steps) {  // entering tile t >> 5: stage it, fetch the next
            *reinterpret_cast<v4u*>(&sm[tile + 8 * li]) = p0;
            *reinterpret_cast<v4u*>(&sm[tile + 8 * li + 4]) = p1;
            if (t >= 32) load_tile((t >> 5) - 1, p0, p1);
        }
        const bool act = t * 32 + li < nc;
        const uint32_t u = (uint32_t)reinterpret_cast<const uint8_t*>(&sm[tile])[(t & 31) * 32 + li] ^ 0x80;
        const uint2 e = *reinterpret_cast<const uint2*>(&sm[2 * u]);
        const uint32_t k = (uint32_t)((int)X + (int)e.x) >> R1;
        const uint32_t w = (e.y >> 8) & 15;
        const uint32_t field = (e.y & 0xFF) | (__builtin_amdgcn_ubfe(X, 0, k) << w);
        uint32_t len = act ? w + k : 0;
        const uint32_t Xn = L + es[((e.y >> 16) & 0x3FF) - 512 + (X >> k)];
        if (act) {
            bad |= e.y >> 31;
            X = Xn;
        }
        const uint32_t incl = scan32(len);
        const uint32_t total = bcast31(incl);
        const uint32_t Pt = P - total;
        ring_or(sm, ring, Pt + incl - len, field, len);
        P = Pt;
        pay += total;
        if ((P >> 5) + 129 <= fmark) {  // dwords above P's word are final
            fmark -= 128;
            flush_block(fmark);
        }
    }
    // the lanes' final states, the decoder's initial states, in front of the fields
    const uint32_t Pi = P - lanes * a.R;
    if (li < lanes) ring_or(sm, ring, Pi + li * a.R, X - L, a.R);
    if (nc > 0) {
        while (fmark > (Pi >> 5)) {
            fmark -= 128;
            flush_block(fmark);
        }
    }
    if (chunk < n_chunks && li == 0) {
        a.meta[2 * (sg->slot_base + chunk)] = Pi;
        a.meta[2 * (sg->slot_base + chunk) + 1] = pay;
    }
    report(a.status, bad && sg->tab && sg->tab[kDTStatus] != 0 ? SH_ERR_UNSUPPORTED
                                                              : SH_ERR_SYMBOL_NOT_IN_TABLE,
           bad != 0);
}

// ------------------------------------------------------------------------------------
// encode, kernel 2: chunk index (exclusive scan of chunk sizes), header, totals
// ------------------------------------------------------------------------------------
constexpr int kScanBlock = 1024;

__global__ __launch_bounds__(kScanBlock) void k_encode_index(const CodecArgs a) {
    __shared__ uint32_t wsum[kScanBlock / 64];
    __shared__ unsigned long long bits_sum;
    const uint32_t tid = threadIdx.x, lane = tid & 63, wv = tid >> 6;
    const SegDesc* sg = a.nseg == 0 ? &a.one.seg : &a.many[blockIdx.x];
    const uint32_t n_chunks = sg->n_chunks;
    const uint32_t index_at = header_bytes_dev(a.K);
    const uint32_t* tmpl = sg->tab ? sg->tab + kDTHdr : a.one.hdr;
    const uint32_t* meta = a.meta + 2ull * sg->slot_base;
    uint32_t* index = reinterpret_cast<uint32_t*>(sg->c + index_at);
    uint32_t* hdr = reinterpret_cast<uint32_t*>(sg->c);
    for (uint32_t i = tid; i < index_at / 4; i += kScanBlock) hdr[i] = header_dword(tmpl, i, sg->n, n_chunks);
    if (tid == 0) bits_sum = 0;
    __syncthreads();
    uint32_t carry = 0;
    uint64_t my_bits = 0;
    for (uint32_t base = 0; base < n_chunks; base += kScanBlock) {
        const uint32_t c = base + tid;
        uint32_t bytes = 0;
        if (c < n_chunks) {
            const uint32_t start = meta[2 * c];
            bytes = 4 * ((a.slot_dwords * 32 - start + 31) >> 5);
            my_bits += meta[2 * c + 1];
        }
        // wavefront inclusive scan, then across the 16 wavefronts
        uint32_t v = bytes;
        for (int sh = 1; sh < 64; sh <<= 1) {
            const uint32_t o = __shfl_up(v, sh, 64);
            if (lane >= (uint32_t)sh) v += o;
        }
        if (lane == 63) wsum[wv] = v;
        __syncthreads();
        uint32_t before = 0, all = 0;
        for (uint32_t w = 0; w < kScanBlock / 64; ++w) {
            before += w < wv ? wsum[w] : 0;
            all += wsum[w];
        }
        if (c < n_chunks) index[c] = carry + before + v - bytes;
        carry += all;
        __syncthreads();
    }
    if (tid == 0) index[n_chunks] = carry;
    atomicAdd(&bits_sum, (unsigned long long)my_bits);
    __syncthreads();
    if (tid == 0 && sg->info) {
        sg->info->container_bytes = (uint64_t)index_at + 4ull * (n_chunks + 1) + carry;
        sg->info->payload_bits = bits_sum;
    }
}

// ------------------------------------------------------------------------------------
// encode, kernel 3: move every chunk from its slot to its place in the payload
// ------------------------------------------------------------------------------------
__global__ __launch_bounds__(256) void k_encode_compact(const CodecArgs a) {
    const uint32_t lane = threadIdx.x & 63;
    const uint32_t block = __builtin_amdgcn_readfirstlane(blockIdx.x);
    const SegDesc* sg = codec_seg(a, block, true);
    const uint32_t c = (block - sg->first_block_c) * 4 + (threadIdx.x >> 6);
    if (c >= sg->n_chunks) return;
    const uint32_t index_at = header_bytes_dev(a.K);
    const uint32_t payload_at = index_at + 4 * (sg->n_chunks + 1);
    const uint32_t slot = sg->slot_base + c;
    const uint32_t start = a.meta[2 * slot];
    const uint32_t ndw = (a.slot_dwords * 32 - start + 31) >> 5;
    const uint32_t off = reinterpret_cast<const uint32_t*>(sg->c + index_at)[c];
    const uint32_t* s = a.slots + (uint64_t)slot * a.slot_dwords;
    uint32_t* d = reinterpret_cast<uint32_t*>(sg->c + payload_at + off);
    const uint32_t s0 = start >> 5;
    for (uint32_t j = lane; j < ndw; j += 64) {
        const uint32_t lo = s[s0 + j];
        const uint32_t hi = s0 + j + 1 < a.slot_dwords ? s[s0 + j + 1] : 0;
        d[j] = __builtin_amdgcn_alignbit(hi, lo, start);
    }
}

sh_status launch_encode(const CodecArgs& a, uint32_t total_blocks, uint32_t total_blocks_c,
                        void* stream) {
    hipStream_t s = (hipStream_t)stream;
    if (total_blocks > 0)
        hipLaunchKernelGGL(k_encode_chunks, dim3(total_blocks), dim3(kEncBlock), 0, s, a);
    hipLaunchKernelGGL(k_encode_index, dim3(a.nseg ? a.nseg : 1), dim3(kScanBlock), 0, s, a);
    if (total_blocks_c > 0)
        hipLaunchKernelGGL(k_encode_compact, dim3(total_blocks_c), dim3(256), 0, s, a);
    return hipGetLastError() == hipSuccess ? SH_OK : SH_ERR_HIP;
}

}  // namespace shn
