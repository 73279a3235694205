// Encode kernels of the Shannonic codec for gfx950 (CDNA4, wave64): the inverse of the
// decode mapping ("Runtime encoding/decoding", paper section 4.2, Algorithm 2, of the
// Shannonic talk notes), run backwards per lane, then the chunk index and the compaction:
// one kernel for tensors of up to kPlaceMaxChunks chunks, two for longer ones.
#include <type_traits>

#include "device_common.hpp"

namespace shn {

// ------------------------------------------------------------------------------------
// encode, kernel 1: every chunk into a worst-case slot of the workspace
// ------------------------------------------------------------------------------------
// The decoder's mapping run backwards: one chunk per row of W lanes (a 16-lane DPP row, or a
// half wavefront), lane j of a row runs P adjacent streams, P j to P j + P - 1 (16 x 2 for
// chunks of 32 streams, 16 x 4 for 64, 16 x 8 for 128; 32 x 2 for launches of few chunks of
// 64 streams, which it gives twice the wavefronts), whose fields are adjacent in every
// step.  tANS encodes backwards, so each stream walks its values from the last step to the
// first and every step's fields are placed right to left: the step's fields end where the
// later steps' fields begin, and a W-lane prefix sum of the lanes' field lengths gives every
// lane's bit position.  A lane's fields are OR-ed, a pair at a time, into an LDS ring per
// chunk (128 dwords, 256 for 128 streams) that is flushed to the chunk's slot 64 dwords at a
// time, highest first; the chunk ends up right-aligned in its slot with the streams' final
// states (the decoder's initial states) in front.
constexpr uint32_t kEFlush = 64;                   // dwords per flush
// LDS (dynamic; the kernel's only LDS, so it starts at LDS byte 0): the value entries (two
// dwords per value, at a 2 KB boundary so that an entry's address is one AND-OR), the
// rings (one per chunk, each followed by its spill dword), the encTable (a dword per slot,
// holding the next state L + slot), the input tiles (u = x + 128 of kTileSteps steps of a
// chunk), then the block's two totals
constexpr uint32_t kEVtByte = 0;
constexpr uint32_t kERingsByte = kEVtByte + 256 * 8;                                 // 2 KB
template <int W, int P>
struct EncGeom {
    static_assert((W == 16 && (P == 2 || P == 4 || P == 8)) || (W == 32 && P == 2),
                  "16 x 2, 16 x 4, 16 x 8, 32 x 2");
    static constexpr uint32_t kS = W * P;                   // streams of a chunk
    static constexpr uint32_t kRowsPerWave = 64 / W;
    static constexpr uint32_t kBlock = kEncodeChunksPerBlock * W;  // threads: one row a chunk
    // The ring holds every dword not yet flushed.  After a flush check the fields reach no
    // lower than 64 dwords below the flush mark; checks come at least every other step, and
    // a step places at most kS fields of 16 bits, kS / 2 dwords; so the unflushed dwords span
    // at most 64 + kS dwords: 128 dwords (the ring exactly at 64 streams; the mark's own
    // dword, the lowest one's twin in the ring, is flushed and zero), 256 at 128 streams.
    static constexpr uint32_t kRingLog2 = kS == 128 ? 8 : 7;
    static constexpr uint32_t kRing = 1u << kRingLog2;
    static_assert(kEFlush + kS <= kRing, "two steps fit in the ring");
    // a ring's LDS: its kRing dwords, the spill dword (ring_or2), padding to 16 bytes
    static constexpr uint32_t kRingStride = kRing + 4;
    static constexpr uint32_t kTileSteps = kS == 128 ? 8 : 16;  // input steps staged at a time
    static constexpr uint32_t kTileBytes = kTileSteps * kS;
    static constexpr uint32_t kLaneStage = kTileBytes / W;   // bytes a lane stages
    static constexpr uint32_t kTileVecs = kLaneStage / 16;   // 16-byte loads a lane stages
    // The rows of a wavefront write their rings and read their tiles at similar offsets in
    // the same steps.  A row reads kS bytes of a tile step (kS / 4 banks) and ORs about kS x
    // 6.5 bits of fields a step into its ring (some kS / 5 dwords), so the tiles sit kS bytes
    // apart beyond their size and the ring origins kS / 4 dwords apart (ring dword (d + kS / 4
    // row) mod kRing holds slot dword d): the rows use different LDS banks.
    static constexpr uint32_t kTileStride = kTileBytes + kS;
    static constexpr uint32_t kRowTurn = kS / 4;            // ring dwords per row of the wavefront
    static constexpr uint32_t kEsByte = kERingsByte + kEncodeChunksPerBlock * kRingStride * 4;
    static_assert(kEsByte >= 4 * kMaxLGpu && kEsByte + 4 * kMaxLGpu < 32768,
                  "encTable addresses stay positive and below bit 15 of an entry");
    __host__ __device__ static constexpr uint32_t tiles_byte(uint32_t L) {
        return (kEsByte + 4 * L + 15) / 16 * 16;
    }
    __host__ __device__ static constexpr uint32_t lds_bytes(uint32_t L) {
        return tiles_byte(L) + kEncodeChunksPerBlock * kTileStride + 16;
    }
};

// container bytes of a chunk of the given bits: whole size units of 2^ulog bytes
__device__ __forceinline__ uint32_t chunk_bytes_of(uint32_t bits, uint32_t ulog) {
    return ((bits + (8u << ulog) - 1) >> (3 + ulog)) << ulog;
}

typedef __attribute__((address_space(3))) uint32_t lds_w32;
typedef const __attribute__((address_space(3))) uint16_t lds_r16;
typedef const __attribute__((address_space(3))) uint32_t lds_r32;
typedef unsigned int v2u_e __attribute__((ext_vector_type(2)));

// OR a pair of fields (at most 32 bits) into a ring of 2^kRingLog2 dwords at bit pos;
// ring_byte is the ring's LDS byte address.  A pair that reaches past the ring's last dword
// goes on into the spill dword after it, which holds bits of ring dword 0 until that dword is
// flushed (flush_block folds it in), so the second dword is always the first one's address
// plus 4, an instruction offset.  The second dword is OR-ed only by the lanes whose pair
// reaches into it: the pairs of a step share a few dwords, and same-address LDS atomics
// serialise.  The address is one v_bfe_u32 and one v_lshl_add_u32 (the compiler would
// split the extract, the scaling and the add into more operations).
template <uint32_t kRingLog2>
__device__ __forceinline__ void ring_or2(uint32_t ring_byte, uint32_t pos, uint32_t field) {
    const uint64_t wide = (uint64_t)field << (pos & 31);
    uint32_t a;
    asm("v_bfe_u32 %0, %1, 5, %2\n\tv_lshl_add_u32 %0, %0, 2, %3"
        : "=&v"(a) : "v"(pos), "i"(kRingLog2), "v"(ring_byte));
    lds_w32* a0 = (lds_w32*)(uintptr_t)a;
    __hip_atomic_fetch_or(a0, (uint32_t)wide, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP);
    if ((uint32_t)(wide >> 32))
        __hip_atomic_fetch_or(a0 + 1, (uint32_t)(wide >> 32), __ATOMIC_RELAXED,
                              __HIP_MEMORY_SCOPE_WORKGROUP);
}

// Inclusive prefix sum within each 16-lane row (DPP row shifts).
__device__ __forceinline__ uint32_t escan16(uint32_t v) {
    v += (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x111, 0xF, 0xF, true);  // row_shr:1
    v += (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x112, 0xF, 0xF, true);  // row_shr:2
    v += (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x114, 0xF, 0xF, true);  // row_shr:4
    v += (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x118, 0xF, 0xF, true);  // row_shr:8
    return v;
}
// Value of lane 15 of this lane's row (DPP row_newbcast:15).  The empty asm keeps the
// broadcast a v_mov_b32_dpp of its own: folded into the subtraction that uses it (as
// v_subrev_u32_dpp) the broadcast was measured on MI355X not to take effect, every lane
// subtracting its own value.
__device__ __forceinline__ uint32_t erow_last(uint32_t v) {
    uint32_t b = (uint32_t)__builtin_amdgcn_mov_dpp((int)v, 0x15F, 0xF, 0xF, true);
    asm volatile("" : "+v"(b));
    return b;
}

// Byte B of v times 8 (the LDS byte offset of value entry number byte B of v): one VOP2
// shift reading a byte of its operand, where the compiler would extract and scale in two.
template <int B>
__device__ __forceinline__ uint32_t byte_x8(uint32_t v) {
    static_assert(B >= 0 && B <= 3, "bytes 0..3");
    uint32_t r;
    if constexpr (B == 0)
        asm("v_lshlrev_b32_sdwa %0, 3, %1 dst_sel:DWORD dst_unused:UNUSED_PAD src0_sel:DWORD src1_sel:BYTE_0" : "=v"(r) : "v"(v));
    else if constexpr (B == 1)
        asm("v_lshlrev_b32_sdwa %0, 3, %1 dst_sel:DWORD dst_unused:UNUSED_PAD src0_sel:DWORD src1_sel:BYTE_1" : "=v"(r) : "v"(v));
    else if constexpr (B == 2)
        asm("v_lshlrev_b32_sdwa %0, 3, %1 dst_sel:DWORD dst_unused:UNUSED_PAD src0_sel:DWORD src1_sel:BYTE_2" : "=v"(r) : "v"(v));
    else
        asm("v_lshlrev_b32_sdwa %0, 3, %1 dst_sel:DWORD dst_unused:UNUSED_PAD src0_sel:DWORD src1_sel:BYTE_3" : "=v"(r) : "v"(v));
    return r;
}

// An encode entry in LDS, two dwords:
//   B = bias_s & 0xFFFFFF | w_s << 24: the state-bit count is bits R+1.. of X + B (the
//       bias's sign bits above bit 23 do not reach them)
//   A = o | (encTable byte address of range s's first slot, minus 4 f_s) << 16 |
//       (f_s == 0) << 31
struct EEnt {
    uint32_t B, A;
};

// A value's field, o | s << w (s: the state bits, o: the offset), in two VOP2 operations
// that read w from byte 3 of B and o from byte 0 of A (the compiler would extract both
// first).
__device__ __forceinline__ uint32_t field_of(uint32_t s, const EEnt& en) {
    uint32_t t, f;
    asm("v_lshlrev_b32_sdwa %0, %1, %2 dst_sel:DWORD dst_unused:UNUSED_PAD src0_sel:BYTE_3 src1_sel:DWORD"
        : "=v"(t) : "v"(en.B), "v"(s));
    asm("v_or_b32_sdwa %0, %1, %2 dst_sel:DWORD dst_unused:UNUSED_PAD src0_sel:DWORD src1_sel:BYTE_0"
        : "=v"(f) : "v"(t), "v"(en.A));
    return f;
}

template <class A, int W, int P>
__global__ __launch_bounds__(kEncodeChunksPerBlock * W) void k_encode_chunks(const A a) {
    using G = EncGeom<W, P>;
    constexpr uint32_t kBlock = G::kBlock, kRowsPerWave = G::kRowsPerWave;
    constexpr uint32_t kS = G::kS, kERing = G::kRing, kETileSteps = G::kTileSteps;
    constexpr uint32_t kEEsByte = G::kEsByte;
    using VT = std::conditional_t<P == 8, uint64_t, uint32_t>;  // a lane's P values, a byte each
    // the entry addresses below are formed with AND-OR, so the LDS block must start on a
    // 2 KB boundary (it is the kernel's only LDS, at byte 0)
    extern __shared__ __align__(2048) uint32_t esm[];
    const uint32_t tid = threadIdx.x, lane = tid & 63, j = lane % W, row = lane / W;
    const uint32_t block = __builtin_amdgcn_readfirstlane(blockIdx.x);
    const SegDesc* sg = codec_seg(a, block, false);
    const uint32_t bseg = block - sg->first_block;
    const uint32_t wid = __builtin_amdgcn_readfirstlane(bseg * (kBlock / 64) + (tid >> 6));
    const uint32_t rowi = (wid & (kBlock / 64 - 1)) * kRowsPerWave + row;  // row in the block
    const uint32_t n_chunks = sg->n_chunks;
    const uint64_t n = sg->n;
    const uint32_t L = a.h.L, R = a.h.R, R1 = a.h.R + 1;
    const uint32_t base = lds_offset(esm);  // 0: the only LDS of the kernel
    const uint32_t ring_byte = base + kERingsByte + 4 * G::kRingStride * rowi;
    const uint32_t tile_byte = base + G::tiles_byte(L) + G::kTileStride * rowi;
    const uint32_t vt_byte = base + kEVtByte, es_byte = base + kEEsByte;
    uint32_t* agg_s = reinterpret_cast<uint32_t*>(reinterpret_cast<uint8_t*>(esm) + G::tiles_byte(L) +
                                                  kEncodeChunksPerBlock * G::kTileStride);

    // the tables in their LDS form (device form: v0 = bias, v1 = o | w << 8 | (f == 0) << 15 |
    // (start + kMaxLGpu) << 16, start = cum - f; encTable entries are slots)
    const uint32_t* vt = sg->tab ? sg->tab + kDTVt : inline_tab(a);
    const uint16_t* es_src = sg->tab ? reinterpret_cast<const uint16_t*>(sg->tab + kDTEs)
                                    : inline_es(a);
    if (tid < 256) {
        const uint32_t v0 = vt[2 * tid], v1 = vt[2 * tid + 1];  // value tid
        const uint32_t start4 = es_byte + 4 * ((v1 >> 16) - kMaxLGpu);
        esm[kEVtByte / 4 + 2 * tid] = (v0 & 0xFFFFFFu) | (((v1 >> 8) & 15u) << 24);
        esm[kEVtByte / 4 + 2 * tid + 1] = (v1 & 0xFFu) | (start4 << 16) | ((v1 & 0x8000u) << 16);
    }
    for (uint32_t i = tid; i < L; i += kBlock) esm[kEEsByte / 4 + i] = L + es_src[i];
    for (uint32_t i = j; i < G::kRingStride; i += W) esm[kERingsByte / 4 + G::kRingStride * rowi + i] = 0;
    if (tid < 2) agg_s[tid] = 0;

    // the wavefront's chunks, one per row
    const uint32_t group = kRowsPerWave * wid;
    const uint32_t chunk = group + row;
    const uint64_t grp_first = (uint64_t)group * a.h.C;
    const uint64_t grp_len = grp_first < n ? n - grp_first : 0;
    const rsrc_t rin = make_rsrc(sg->x + (grp_first < n ? grp_first : 0),
                                 (uint32_t)(grp_len < kRowsPerWave * (uint64_t)a.h.C ? grp_len : kRowsPerWave * (uint64_t)a.h.C));
    const uint32_t slot0 = sg->slot_base + (group < n_chunks ? group : 0);
    const rsrc_t rslot = make_rsrc(a.h.slots + (uint64_t)slot0 * a.h.slot_dwords,
                                   4 * kRowsPerWave * a.h.slot_dwords);
    const uint32_t in_row = row * a.h.C;                   // byte of this row's chunk in rin
    const uint32_t slot_row = row * a.h.slot_dwords * 4;   // byte of its slot in rslot
    // a device table built for other parameters than the launch's, or one whose build
    // failed, is refused: its chunks are coded as empty (the workspace stays consistent for
    // the placement) and the call fails
    const bool mismatch = sg->tab && (sg->tab[kDTK] != a.h.K || sg->tab[kDTLog2L] != a.h.R);
    const bool unusable = sg->tab && sg->tab[kDTStatus] != 0;
    uint32_t nc = 0;
    if (chunk < n_chunks && !mismatch && !unusable) {
        const uint64_t first = (uint64_t)chunk * a.h.C;
        nc = (uint32_t)((n - first) < a.h.C ? (n - first) : a.h.C);
    }
    const uint32_t lanes = nc < kS ? nc : kS;
    uint32_t nc_min = 0xFFFFFFFFu, nc_max = 0;
#pragma unroll
    for (uint32_t k = 0; k < kRowsPerWave; ++k) {
        const uint32_t v = __builtin_amdgcn_readlane(nc, W * k);
        nc_min = nc_min < v ? nc_min : v;
        nc_max = nc_max > v ? nc_max : v;
    }
    const uint32_t steps = (nc_max + kS - 1) / kS;

    // Lane j stages bytes [kLaneStage j, kLaneStage (j + 1)) of tile T.  Past a short chunk's end lies the end of the wavefront's range (a
    // 16-byte load reaching past it reads 0 as a whole, so the lanes at the end read byte by
    // byte) or the next chunk, whose values go unused.
    constexpr uint32_t kLaneStage = G::kLaneStage;
    const uint32_t in_len = (uint32_t)(grp_len < kRowsPerWave * (uint64_t)a.h.C ? grp_len : kRowsPerWave * (uint64_t)a.h.C);
    auto load_tile = [&](uint32_t T, v4u* pv) {
        const uint32_t b = in_row + G::kTileBytes * T + kLaneStage * j;
        if (b + kLaneStage <= in_len) {
#pragma unroll
            for (uint32_t v = 0; v < G::kTileVecs; ++v)
                pv[v] = __builtin_bit_cast(v4u, __builtin_amdgcn_raw_buffer_load_b128(rin, (int)(b + 16 * v), 0, 0));
        } else {
#pragma unroll
            for (uint32_t v = 0; v < G::kTileVecs; ++v) pv[v] = v4u{0, 0, 0, 0};
            for (uint32_t k = 0; k < kLaneStage; ++k)
                if (b + k < in_len) {
                    const uint32_t byte = __builtin_amdgcn_raw_buffer_load_b8(rin, (int)(b + k), 0, 0);
                    pv[k >> 4][(k >> 2) & 3] |= byte << (8 * (k & 3));
                }
        }
    };
    v4u pv[G::kTileVecs];
#pragma unroll
    for (uint32_t v = 0; v < G::kTileVecs; ++v) pv[v] = v4u{0, 0, 0, 0};
    if (steps > 0) load_tile((steps - 1) / kETileSteps, pv);
    __syncthreads();

    // bit positions are kept turned by the row's ring origin: position p stands for slot bit
    // p - turn
    const uint32_t turn = 32 * G::kRowTurn * row;
    uint32_t fpos = a.h.slot_dwords * 32 + turn;  // fields go below fpos, right to left
    uint32_t fmark = a.h.slot_dwords;    // dwords at or above fmark are in the slot
    uint32_t flush_at = (fmark - kEFlush) * 32 + turn;  // once fpos is below this, flush a block
    uint32_t bad = 0;                    // entries OR-ed in: bit 31 marks a range without states

    auto flush_block = [&](uint32_t blk) {  // ring dwords [blk, blk + 64) -> slot, 16 lanes
        if (j >= kEFlush / 4) return;
        typedef __attribute__((address_space(3))) v4u lds_v4;
        const uint32_t idx = (blk + G::kRowTurn * row + 4 * j) & (kERing - 1);
        lds_v4* r = (lds_v4*)(uintptr_t)(ring_byte + 4 * idx);
        v4u v = *r;
        *r = v4u{0, 0, 0, 0};
        if (idx == 0) {  // ring dword 0 with the bits carried into the spill dword
            lds_w32* spill = (lds_w32*)(uintptr_t)(ring_byte + 4 * kERing);
            v[0] |= *spill;
            *spill = 0;
        }
        __builtin_amdgcn_raw_buffer_store_b128(v, rslot, (int)(slot_row + 4 * (blk + 4 * j)), 0, 0);
    };
    auto stage = [&]() {  // the tile in pv into LDS, as u = x + 128
        typedef __attribute__((address_space(3))) v4u lds_v4;
        const v4u flip = {0x80808080u, 0x80808080u, 0x80808080u, 0x80808080u};
#pragma unroll
        for (uint32_t v = 0; v < G::kTileVecs; ++v)
            *(lds_v4*)(uintptr_t)(tile_byte + kLaneStage * j + 16 * v) = pv[v] ^ flip;
    };
    auto vals_at = [&](uint32_t t) -> VT {  // u of the lane's P streams at step t (staged)
        const uint32_t at = tile_byte + kS * (t & (kETileSteps - 1)) + P * j;
        if constexpr (P == 2) return (uint32_t) * (lds_r16*)(uintptr_t)at;
        else if constexpr (P == 4) return *(lds_r32*)(uintptr_t)at;
        else return *(const __attribute__((address_space(3))) uint64_t*)(uintptr_t)at;
    };
    // the entry of byte i of vals (the table sits on a 2 KB boundary)
    auto entry_of = [&](VT vals, int i) {
        const uint32_t word = i < 4 ? (uint32_t)vals : (uint32_t)((uint64_t)vals >> 32);
        const uint32_t off = (i & 3) == 0 ? byte_x8<0>(word) : (i & 3) == 1 ? byte_x8<1>(word)
                           : (i & 3) == 2 ? byte_x8<2>(word) : byte_x8<3>(word);
        const v2u_e v = *(const __attribute__((address_space(3))) v2u_e*)(uintptr_t)(off | vt_byte);
        return EEnt{v[0], v[1]};
    };
    // step t2's values, staging its tile first when t2 is the tile's first step in this
    // (backward) order; the tile it replaces is no longer read
    auto fetch = [&](uint32_t t2) {
        if ((t2 & (kETileSteps - 1)) == kETileSteps - 1) {
            stage();
            if (t2 >= kETileSteps) load_tile(t2 / kETileSteps - 1, pv);
        }
        return vals_at(t2);
    };

    // Values are read two steps ahead and entries one step ahead, so the only LDS read on
    // the chain from one step to the next is the state-dependent encTable read.
    EEnt e[P];
    uint32_t X[P];
#pragma unroll
    for (int i = 0; i < P; ++i) {
        e[i] = EEnt{0, 0};
        X[i] = L;
    }
    VT u_n = 0;
    if (steps > 0) {
        stage();
        if (steps - 1 >= kETileSteps) load_tile((steps - 1) / kETileSteps - 1, pv);
        const VT u_c = vals_at(steps - 1);
        if (steps >= 2) u_n = fetch(steps - 2);
#pragma unroll
        for (int i = 0; i < P; ++i) e[i] = entry_of(u_c, i);
    }
    auto flush_due = [&]() {
        if (fpos < flush_at) {  // dwords from fpos's dword + 1 up are final
            fmark -= kEFlush;
            flush_at -= kEFlush * 32;
            flush_block(fmark);
        }
    };
    // one stream's step: the next state's encTable read goes out first
    auto code = [&](const EEnt& en, uint32_t x, uint32_t& xn, uint32_t& field, uint32_t& len) {
        const uint32_t k = __builtin_amdgcn_ubfe(x + en.B, R1, 5);
        const uint32_t addr = ((x >> k) << 2) + __builtin_amdgcn_ubfe(en.A, 16, 15);
        xn = *(lds_r32*)(uintptr_t)addr;
        field = field_of(__builtin_amdgcn_ubfe(x, 0, k), en);
        len = (en.B >> 24) + k;
    };
    // may_stage: false for a step whose t is known even (t - 2 is then never a tile's first
    // step in backward order, and for t = 0 the value read is a harmless, unused one)
    auto step = [&](uint32_t t, auto partial, auto may_stage) {
        VT u_nn;
        if constexpr (decltype(may_stage)::value) u_nn = t >= 2 ? fetch(t - 2) : VT(0);
        else u_nn = vals_at(t - 2);
        EEnt ne[P];
#pragma unroll
        for (int i = 0; i < P; ++i) ne[i] = entry_of(u_n, i);
        uint32_t Xn[P], f[P], l[P];
#pragma unroll
        for (int i = 0; i < P; ++i) code(e[i], X[i], Xn[i], f[i], l[i]);
        uint32_t flag = 0;
        if constexpr (decltype(partial)::value) {
#pragma unroll
            for (int i = 0; i < P; ++i) {
                const uint32_t si = t * kS + P * j + i;
                const bool act = si < nc;
                // a stream's last value, the first it encodes (from X = L): its state bits
                // are zero and are left out
                l[i] = act ? (si + kS >= nc ? e[i].B >> 24 : l[i]) : 0u;
                f[i] = act ? f[i] : 0u;
                flag |= act ? e[i].A : 0u;
                X[i] = act ? Xn[i] : X[i];
            }
        } else {
#pragma unroll
            for (int i = 0; i < P; ++i) {
                flag |= e[i].A;
                X[i] = Xn[i];
            }
        }
        bad |= flag;
        // the lane's fields, stream P j's lowest: pairs of at most 32 bits
        uint32_t fp[P / 2], lq[P / 2], lp = 0;
#pragma unroll
        for (int k = 0; k < P / 2; ++k) {
            fp[k] = f[2 * k] | (f[2 * k + 1] << l[2 * k]);
            lq[k] = l[2 * k] + l[2 * k + 1];
            lp += lq[k];
        }
        uint32_t at;
        if constexpr (W == 16) {
            const uint32_t incl = escan16(lp);
            fpos -= erow_last(incl);
            // the lane's position: the previous lane's inclusive sum above fpos (a DPP row
            // shift, zero for lane 0, in the add)
            at = fpos + (uint32_t)__builtin_amdgcn_update_dpp(0, (int)incl, 0x111, 0xF, 0xF, true);
        } else {  // a half wavefront: the row total from lane 31
            const uint32_t incl = scan32(lp);
            fpos -= bcast31(incl);
            at = fpos + incl - lp;
        }
#pragma unroll
        for (int k = 0; k < P / 2; ++k) {
            ring_or2<G::kRingLog2>(ring_byte, at, fp[k]);
            at += lq[k];
        }
#pragma unroll
        for (int i = 0; i < P; ++i) e[i] = ne[i];
        u_n = u_nn;
    };
    // steps where a stream of some row has no value (the tail of a short chunk) or has its
    // last value: every stream's last value lies at or after step nc / kS - 1
    uint32_t t_full = nc_min / kS;
    t_full = t_full > 0 ? t_full - 1 : 0;
    uint32_t t = steps;
    while (t > t_full) {
        step(--t, std::true_type{}, std::true_type{});
        flush_due();
    }
    if (t & 1) {
        step(--t, std::false_type{}, std::true_type{});
        flush_due();
    }
    // the waves on a SIMD take turns at the highest priority (take_turn)
    const uint32_t slot_id = wave_slot();
    while (t > 0) {
        take_turn(t / kPrioSteps, slot_id);
        const uint32_t stop = t > kPrioSteps ? t - kPrioSteps : 0;  // t and kPrioSteps even
        while (t > stop) {  // two steps per check: a step places at most kS / 2 dwords
            step(--t, std::false_type{}, std::true_type{});   // odd t
            step(--t, std::false_type{}, std::false_type{});  // even t
            flush_due();
        }
    }
    __builtin_amdgcn_s_setprio(0);
    const uint32_t top = a.h.slot_dwords * 32;
    const uint32_t pay = top + turn - fpos;  // field bits
    // the streams' final states, the decoder's initial states, in front of the fields.  A
    // valid encode never exceeds the chunk's bound; the span recorded for the placement is
    // clamped to it all the same, so that no table, however corrupt, moves the placement
    // outside the container's bound
    uint32_t Pi = fpos - turn - lanes * R;
    {
        const uint32_t most = (uint32_t)chunk_bound_bits(nc, R, kS);
        if (Pi > top || top - Pi > most) Pi = top - most;
    }
#pragma unroll
    for (int i = 0; i < P; i += 2) {  // two states (at most 22 bits) at a time
        const uint32_t s0 = P * j + i < lanes ? X[i] - L : 0u;
        const uint32_t s1 = P * j + i + 1 < lanes ? X[i + 1] - L : 0u;
        ring_or2<G::kRingLog2>(ring_byte, Pi + turn + (P * j + i) * R, s0 | (s1 << R));
    }
    while (fmark > (Pi >> 5)) {
        fmark -= kEFlush;
        flush_block(fmark);
    }
    const uint32_t ulog = size_unit_log2(a.h.C, R, kS);
    if (chunk < n_chunks && j == 0) {
        a.h.meta[2 * (sg->slot_base + chunk)] = Pi;
        a.h.meta[2 * (sg->slot_base + chunk) + 1] = pay;
        atomicAdd(&agg_s[0], chunk_bytes_of(top - Pi, ulog));
        atomicAdd(&agg_s[1], pay);
    }
    __syncthreads();
    if (tid < 2) a.h.agg[2 * block + tid] = agg_s[tid];
    bad &= 0x80000000u;
    if (mismatch) report(a.h.status, SH_ERR_INVALID_ARG, true);
    else if (unusable) report(a.h.status, SH_ERR_UNSUPPORTED, chunk < n_chunks);
    report(a.h.status, SH_ERR_SYMBOL_NOT_IN_TABLE, bad != 0);
}

// ------------------------------------------------------------------------------------
// a chunk from its workspace slot to the container: bytes [d0, d1) of the container take the
// slot's bits from start on, byte d0 + i bits [start + 8i, start + 8i + 8) (bits past the
// slot's end read 0).  Whole container dwords are stored as dwords, the partial ones at
// either end byte by byte: the neighbouring chunks own their other bytes.  The 64 lanes of a
// wavefront share the work.
// ------------------------------------------------------------------------------------
__device__ __forceinline__ void move_chunk(const uint32_t* src, uint32_t slot_dwords,
                                           uint32_t start, uint8_t* c, uint32_t d0, uint32_t d1,
                                           uint32_t lane) {
    typedef uint32_t v4u_d __attribute__((ext_vector_type(4), aligned(4)));  // dword aligned
    auto bits32 = [&](uint32_t bit) {  // 32 slot bits from bit on
        const uint32_t w = bit >> 5;
        const uint32_t lo = w < slot_dwords ? src[w] : 0u;
        const uint32_t hi = w + 1 < slot_dwords ? src[w + 1] : 0u;
        return __builtin_amdgcn_alignbit(hi, lo, bit);
    };
    const uint32_t q0 = (d0 + 3) >> 2, q1 = d1 >> 2;       // whole dwords [q0, q1)
    const uint32_t head_end = 4 * q0 < d1 ? 4 * q0 : d1;    // bytes [d0, head_end)
    const uint32_t tail_at = 4 * q1 > head_end ? 4 * q1 : head_end;  // bytes [tail_at, d1)
    uint32_t* cw = reinterpret_cast<uint32_t*>(c);
    // whole dwords four at a time: dword q0 + i takes the slot bits from sb0 + 32 i on, so
    // every lane's four come from five consecutive slot dwords and one shift
    const uint32_t sb0 = start + 8 * (4 * q0 - d0);
    const uint32_t w0 = sb0 >> 5, sh = sb0 & 31;
    for (uint32_t i = 4 * lane; q0 + i < q1; i += 256) {
        const uint32_t w = w0 + i;
        if (q0 + i + 4 <= q1 && w + 5 <= slot_dwords) {
            const v4u_d a = *reinterpret_cast<const v4u_d*>(src + w);
            const uint32_t e = src[w + 4];
            v4u_d o;
            o[0] = __builtin_amdgcn_alignbit(a[1], a[0], sh);
            o[1] = __builtin_amdgcn_alignbit(a[2], a[1], sh);
            o[2] = __builtin_amdgcn_alignbit(a[3], a[2], sh);
            o[3] = __builtin_amdgcn_alignbit(e, a[3], sh);
            *reinterpret_cast<v4u_d*>(cw + q0 + i) = o;
        } else {
            for (uint32_t k = 0; k < 4 && q0 + i + k < q1; ++k)
                cw[q0 + i + k] = bits32(sb0 + 32 * (i + k));
        }
    }
    if (lane < 3) {
        const uint32_t b = d0 + lane;
        if (b < head_end) c[b] = (uint8_t)bits32(start + 8 * (b - d0));
    } else if (lane < 6) {
        const uint32_t b = tail_at + lane - 3;
        if (b < d1) c[b] = (uint8_t)bits32(start + 8 * (b - d0));
    }
}

// ------------------------------------------------------------------------------------
// encode, kernel 2 of the long-tensor path: chunk index (exclusive scan of chunk sizes),
// header, totals
// ------------------------------------------------------------------------------------
constexpr int kScanBlock = 1024;

template <class A>
__global__ __launch_bounds__(kScanBlock) void k_encode_index(const A a) {
    __shared__ uint32_t wsum[kScanBlock / 64];
    __shared__ unsigned long long bits_sum;
    const uint32_t tid = threadIdx.x, lane = tid & 63, wv = tid >> 6;
    const SegDesc* sg = &a.segs[blockIdx.x];
    const uint32_t n_chunks = sg->n_chunks;
    const uint32_t index_at = header_bytes_dev(a.h.K);
    const uint32_t payload_at = index_at + (uint32_t)index_bytes_of(n_chunks);
    const uint32_t ulog = size_unit_log2(a.h.C, a.h.R, a.h.S);
    const uint32_t* tmpl = sg->tab ? sg->tab + kDTHdr : inline_hdr(a);
    uint32_t* meta = a.h.meta + 2ull * sg->slot_base;
    uint32_t* goff = reinterpret_cast<uint32_t*>(sg->c + index_at);
    uint16_t* sizes = reinterpret_cast<uint16_t*>(sg->c + index_at + sizes_rel_of(n_chunks));
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
            bytes = chunk_bytes_of(a.h.slot_dwords * 32 - meta[2 * c], ulog);
            my_bits += meta[2 * c + 1];
        }
        // wavefront inclusive scan, then across the 16 wavefronts
        const uint32_t v = scan64(bytes);
        if (lane == 63) wsum[wv] = v;
        __syncthreads();
        uint32_t before = 0, all = 0;
        for (uint32_t w = 0; w < kScanBlock / 64; ++w) {
            before += w < wv ? wsum[w] : 0;
            all += wsum[w];
        }
        if (c < n_chunks) {
            const uint32_t off = carry + before + v - bytes;
            meta[2 * c + 1] = off;  // the chunk's payload offset, for the compaction
            sizes[c] = (uint16_t)(bytes >> ulog);
            if (c % kGroupChunks == 0) goff[c / kGroupChunks] = off;
        }
        carry += all;
        __syncthreads();
    }
    if (tid == 0) {
        goff[n_groups_of(n_chunks)] = carry;
        if (n_chunks & 1) sizes[n_chunks] = 0;
    }
    atomicAdd(&bits_sum, (unsigned long long)my_bits);
    __syncthreads();
    if (tid == 0 && sg->info) {
        sg->info->container_bytes = (uint64_t)payload_at + (carry + 3) / 4 * 4;
        sg->info->payload_bits = bits_sum;
    }
}

// ------------------------------------------------------------------------------------
// encode, kernel 3 of the long-tensor path: move every chunk from its slot to its place in
// the payload
// ------------------------------------------------------------------------------------
template <class A>
__global__ __launch_bounds__(256) void k_encode_compact(const A a) {
    const uint32_t lane = threadIdx.x & 63;
    const uint32_t block = __builtin_amdgcn_readfirstlane(blockIdx.x);
    const SegDesc* sg = codec_seg(a, block, true);
    const uint32_t c = (block - sg->first_block_c) * 4 + (threadIdx.x >> 6);
    if (c >= sg->n_chunks) return;
    const uint32_t payload_at = header_bytes_dev(a.h.K) + (uint32_t)index_bytes_of(sg->n_chunks);
    const uint32_t slot = sg->slot_base + c;
    const uint32_t start = a.h.meta[2 * slot];
    const uint32_t off = a.h.meta[2 * slot + 1];  // written by the index kernel
    const uint32_t bytes = chunk_bytes_of(a.h.slot_dwords * 32 - start, size_unit_log2(a.h.C, a.h.R, a.h.S));
    // the last chunk also writes the zero bytes that end the payload on 4 bytes
    const uint32_t end = c + 1 == sg->n_chunks ? (off + bytes + 3) / 4 * 4 : off + bytes;
    move_chunk(a.h.slots + (uint64_t)slot * a.h.slot_dwords, a.h.slot_dwords, start, sg->c,
               payload_at + off, payload_at + end, lane);
}

// ------------------------------------------------------------------------------------
// encode, kernels 2 and 3 in one (segments of at most kPlaceMaxChunks chunks): every block
// finds the offset of its first chunk from the chunk kernel's per-block aggregates (the
// container bytes of 16 chunks each) and the sizes of at most 15 chunks after the last whole
// aggregate, writes its chunks' index entries and moves them into place; the segment's
// first block writes the header and its last block the index end and the totals.
// ------------------------------------------------------------------------------------
template <class A>
__global__ __launch_bounds__(256) void k_encode_place(const A a) {
    __shared__ uint32_t red_b[4];
    __shared__ unsigned long long red_f[4];
    const uint32_t tid = threadIdx.x, lane = tid & 63, wv = tid >> 6;
    const uint32_t block = __builtin_amdgcn_readfirstlane(blockIdx.x);
    const SegDesc* sg = codec_seg(a, block, true);
    const uint32_t n_chunks = sg->n_chunks;
    const uint32_t c0 = (block - sg->first_block_c) * 4;   // this block's first chunk
    const uint32_t index_at = header_bytes_dev(a.h.K);
    const uint32_t payload_at = index_at + (uint32_t)index_bytes_of(n_chunks);
    const uint32_t ulog = size_unit_log2(a.h.C, a.h.R, a.h.S);
    const uint32_t* meta = a.h.meta + 2ull * sg->slot_base;
    const uint32_t* agg = a.h.agg + 2ull * sg->first_block;  // the segment's chunk-kernel blocks
    uint32_t* goff = reinterpret_cast<uint32_t*>(sg->c + index_at);
    uint16_t* sizes = reinterpret_cast<uint16_t*>(sg->c + index_at + sizes_rel_of(n_chunks));
    const bool last = c0 + 4 >= n_chunks;
    auto chunk_bytes = [&](uint32_t ch) {
        return chunk_bytes_of(a.h.slot_dwords * 32 - meta[2 * ch], ulog);
    };

    // bytes of the chunk-kernel blocks before c0 (c0 / 16 of them); in the last block also
    // the field bits of all of them
    const uint32_t nb_before = c0 / kEncodeChunksPerBlock;
    const uint32_t nb_all = (n_chunks + kEncodeChunksPerBlock - 1) / kEncodeChunksPerBlock;
    uint32_t bytes = 0;
    uint64_t fbits = 0;
    for (uint32_t e = tid; e < (last ? nb_all : nb_before); e += 256) {
        if (e < nb_before) bytes += agg[2 * e];
        fbits += agg[2 * e + 1];
    }
    for (int sh = 32; sh >= 1; sh >>= 1) {
        bytes += __shfl_xor(bytes, sh, 64);
        fbits += __shfl_xor(fbits, sh, 64);
    }
    if (lane == 0) {
        red_b[wv] = bytes;
        red_f[wv] = fbits;
    }
    __syncthreads();
    uint32_t off = red_b[0] + red_b[1] + red_b[2] + red_b[3];
    // then the chunks from the last whole aggregate up to this wavefront's chunk (at most 15),
    // one per lane
    const uint32_t c = c0 + wv;
    {
        const uint32_t j = nb_before * kEncodeChunksPerBlock + lane;
        uint32_t part = j < c && j < n_chunks ? chunk_bytes(j) : 0u;
        for (int sh = 8; sh >= 1; sh >>= 1) part += __shfl_xor(part, sh, 64);
        off += __builtin_amdgcn_readfirstlane(part);
    }

    if (c0 == 0)
        for (uint32_t i = tid; i < index_at / 4; i += 256)
            reinterpret_cast<uint32_t*>(sg->c)[i] =
                header_dword(sg->tab ? sg->tab + kDTHdr : inline_hdr(a), i, sg->n, n_chunks);
    if (c < n_chunks) {
        const uint32_t slot = sg->slot_base + c;
        const uint32_t start = a.h.meta[2 * slot];
        const uint32_t bytes = chunk_bytes(c);
        if (lane == 0) {
            sizes[c] = (uint16_t)(bytes >> ulog);
            if (c % kGroupChunks == 0) goff[c / kGroupChunks] = off;
        }
        // the last chunk also writes the zero bytes that end the payload on 4 bytes
        const uint32_t end = c + 1 == n_chunks ? (off + bytes + 3) / 4 * 4 : off + bytes;
        move_chunk(a.h.slots + (uint64_t)slot * a.h.slot_dwords, a.h.slot_dwords, start, sg->c,
                   payload_at + off, payload_at + end, lane);
    }
    // the segment's end: the wavefront holding its last chunk (wavefront 0 of the only
    // block of an empty segment)
    if (last && lane == 0 && c == (n_chunks > 0 ? n_chunks - 1 : 0)) {
        const uint32_t total = n_chunks > 0 ? off + chunk_bytes(c) : 0;
        goff[n_groups_of(n_chunks)] = total;
        if (n_chunks & 1) sizes[n_chunks] = 0;
        if (sg->info) {
            sg->info->container_bytes = (uint64_t)payload_at + (total + 3) / 4 * 4;
            sg->info->payload_bits = red_f[0] + red_f[1] + red_f[2] + red_f[3];
        }
    }
}

// Launches of fewer chunks than this take half-wavefront rows for 64-stream chunks (the
// decoder's launch planner draws the same line for its row mappings).
constexpr uint64_t kEncodeFewChunks = 16384;

template <class K, int W, int P>
void launch_chunks(const K& k, uint32_t blocks, uint32_t L, hipStream_t s) {
    using G = EncGeom<W, P>;
    const uint32_t lds = G::lds_bytes(L);
    hipLaunchKernelGGL((k_encode_chunks<K, W, P>), dim3(blocks), dim3(G::kBlock), lds, s, k);
}

sh_status launch_encode(const CodecArgs& a, uint32_t total_blocks, uint32_t total_blocks_c,
                        bool place, void* stream, void* place_stream, void* ready,
                        void* placed) {
    if (a.S != kStreamsNarrow && a.S != kStreamsWide && a.S != kStreamsWidest)
        return SH_ERR_UNSUPPORTED;
    hipStream_t s = (hipStream_t)stream;
    hipError_t ev = hipSuccess;
    with_kernel_args(a, [&](const auto& k) {
        using K = std::decay_t<decltype(k)>;
        if (total_blocks > 0) {
            // 64-stream chunks of a launch too small to fill the GPU with 16-lane rows go to
            // half-wavefront rows (twice the wavefronts), as in the decoder
            const bool few = (uint64_t)total_blocks * kEncodeChunksPerBlock < kEncodeFewChunks;
            if (a.S == kStreamsWidest) launch_chunks<K, 16, 8>(k, total_blocks, a.L, s);
            else if (a.S == kStreamsWide && few) launch_chunks<K, 32, 2>(k, total_blocks, a.L, s);
            else if (a.S == kStreamsWide) launch_chunks<K, 16, 4>(k, total_blocks, a.L, s);
            else launch_chunks<K, 16, 2>(k, total_blocks, a.L, s);
        }
        if (place_stream) {
            ev = hipEventRecord((hipEvent_t)ready, s);
            if (ev == hipSuccess) ev = hipStreamWaitEvent((hipStream_t)place_stream, (hipEvent_t)ready, 0);
            if (ev != hipSuccess) return;
            s = (hipStream_t)place_stream;
        }
        if (place) {
            hipLaunchKernelGGL(k_encode_place<K>, dim3(total_blocks_c), dim3(256), 0, s, k);
            return;
        }
        hipLaunchKernelGGL(k_encode_index<K>, dim3(k.h.nseg), dim3(kScanBlock), 0, s, k);
        if (total_blocks_c > 0)
            hipLaunchKernelGGL(k_encode_compact<K>, dim3(total_blocks_c), dim3(256), 0, s, k);
    });
    if (ev == hipSuccess && place_stream) ev = hipEventRecord((hipEvent_t)placed, s);
    return hipGetLastError() == hipSuccess && ev == hipSuccess ? SH_OK : SH_ERR_HIP;
}

}  // namespace shn
