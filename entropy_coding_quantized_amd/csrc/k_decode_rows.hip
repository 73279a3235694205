// Decode kernel of the Shannonic codec for gfx950 (CDNA4, wave64): the decoder behind
// sh_decode and sh_decode_batch.
//
// Method: "Shannonic: Efficient Entropy-Optimal Compression for ML Workloads" (MLSys 2026),
// talk notes, "Runtime encoding/decoding" (paper section 4.2): from the state X the decode
// table gives the range s and the count of state bits; the offset o is read as w_s raw
// bits, the value is base[s] + o, and the state bits lead to the next state.  Table
// lookups, shifts, masks and adds only.  The container layout (chunks of C values, 32, 64 or
// 128 interleaved tANS streams per chunk, fields in (step, stream) order) and the GPU mapping
// below are this library's own design; the pages give no GPU design.
//
// Mapping: one chunk per row of W lanes, a 16-lane DPP row (W = 16) or a half wavefront
// (W = 32), so a wavefront decodes 64 / W chunks side by side.  Lane j of a row runs P
// adjacent streams, P j to P j + P - 1 (W P streams a chunk: 16 x 2 for chunks of 32
// streams, 16 x 4 or 32 x 2 for chunks of 64, 32 x 4 for 128), whose fields are adjacent in
// every step: one W-lane prefix sum (DPP) of the lanes' field lengths gives every lane's bit
// position, and one LDS read of two (P = 2) or three (P = 4) ring dwords brings all its
// fields.  Rows of 32 lanes give a launch with few chunks twice the wavefronts of rows of 16.
// Compressed words reach a per-chunk LDS ring through 128-bit loads; the decode table is
// staged in LDS as 8-byte entries (measured on MI355X: a random 8-byte LDS read costs 7
// clocks per wavefront and CU at full occupancy, a 16-byte one 12, a 12-byte one 20).  No
// MFMA: there is no dense contraction.
#include "device_common.hpp"

namespace shn {

namespace {

constexpr int kRowsBlock = 256;                    // 4 wavefronts, 256 / W rows = chunks
// Decoded bytes of kTileSteps steps of a chunk are gathered in an LDS tile and stored
// together: measured on MI355X, the 32-byte stores of single steps held the decode near
// 1.7 TB/s of output however short the rest of the step was.  The tiles of a block's rows
// sit 8 dwords more than a tile apart, so that the four rows of a wavefront write
// different LDS banks in the same step.  (Measured side by side on one GPU: 4-step tiles
// with 256-dword rings, 8-step tiles, 128-dword rings and a two-step write through a
// neighbour exchange all decode the model workload within 5% of each other; the simplest
// is kept.)
constexpr uint32_t kTileSteps = 4;
static_assert(kPrioSteps % kTileSteps == 0, "a turn covers whole tiles");

// Geometry of a row of W lanes that run P streams each.
template <int W, int P>
struct RowGeom {
    static_assert((W == 16 && (P == 2 || P == 4)) || (W == 32 && (P == 2 || P == 4)),
                  "16 x 2, 16 x 4, 32 x 2, 32 x 4");
    static constexpr uint32_t kS = W * P;                      // streams of a chunk
    static constexpr uint32_t kRowsPerWave = 64 / W;
    static constexpr uint32_t kRowsPerBlock = kRowsBlock / W;
    // compressed dwords resident per chunk: 256, 512 for chunks of 128 streams (whose steps
    // take up to 64 dwords)
    static constexpr uint32_t kRingLog2 = kS == 128 ? 9 : 8;
    static constexpr uint32_t kRing = 1u << kRingLog2;
    // a ring is followed by copies of its first dwords (a lane's read of two or three dwords
    // never wraps) and padding that keeps the next ring 16-byte aligned for the 128-bit writes
    static constexpr uint32_t kRingStride = kRing + 4;
    static constexpr uint32_t kRFill = kRing / 2;              // dwords per refill
    static constexpr uint32_t kFillVecs = kRFill / (4 * W);    // 16-byte loads a lane, a refill
    static constexpr uint32_t kTileDwords = kTileSteps * kS / 4;
    static constexpr uint32_t kTileStride = kTileDwords + 8;
    static constexpr uint32_t kWin = P == 2 ? 2 : 3;           // ring dwords a lane reads a step
    // Refills are checked every other step.  A step's fields take at most kS * 16 bits, kS / 2
    // dwords, and a lane reads up to kWin - 1 dwords past its first bit's dword; so once the
    // position is below (res_hi - kMargin) * 32 the next two steps read only dwords below
    // res_hi, and from there on a refill is due: the dwords it overwrites, those below
    // res_hi - kRFill, are all read, and the kS dwords two steps advance at most leave the
    // next refill for a later check.
    static constexpr uint32_t kMargin = kS + kWin - 1;
    static_assert(kMargin <= kRFill && kS < kRFill, "one refill a check, over read dwords only");
};

typedef unsigned int v2u __attribute__((ext_vector_type(2)));
typedef const __attribute__((address_space(3))) v2u lds_v2u;

// 16 bytes of the chunk starting at dword d (dwords at or past cdw read as 0); the rare
// lanes at the chunk's end fetch their dwords one by one.
__device__ __forceinline__ v4u load4(rsrc_t r, uint32_t chunk_byte, uint32_t d, uint32_t cdw) {
    const bool whole = d + 4 <= cdw;
    const v4u full = __builtin_bit_cast(v4u, __builtin_amdgcn_raw_buffer_load_b128(
                                                 r, whole ? (int)(chunk_byte + 4 * d) : 0, 0, 0));
    v4u part = {0, 0, 0, 0};
    if (!whole && d < cdw) {
        for (uint32_t k = 0; k < 4; ++k)
            if (d + k < cdw)
                part[k] = __builtin_amdgcn_raw_buffer_load_b32(r, (int)(chunk_byte + 4 * (d + k)), 0, 0);
    }
    return whole ? full : part;
}

// Inclusive prefix sum within each 16-lane row (DPP row shifts; lanes shifted in from
// outside the row read 0).
__device__ __forceinline__ uint32_t scan16(uint32_t v) {
    v += (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x111, 0xF, 0xF, true);  // row_shr:1
    v += (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x112, 0xF, 0xF, true);  // row_shr:2
    v += (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x114, 0xF, 0xF, true);  // row_shr:4
    v += (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x118, 0xF, 0xF, true);  // row_shr:8
    return v;
}
// ... within each row of W lanes
template <int W>
__device__ __forceinline__ uint32_t scan_row(uint32_t v) {
    if constexpr (W == 16) return scan16(v);
    else return scan32(v);
}

// The ring's dword index of a bit position, (pos >> 5) mod 2^kLog2, as one v_bfe_u32 (the
// compiler would split the extract and the scaling that follows it into three operations).
template <uint32_t kLog2>
__device__ __forceinline__ uint32_t ring_dword(uint32_t pos) {
    uint32_t d;
    asm("v_bfe_u32 %0, %1, 5, %2" : "=v"(d) : "v"(pos), "i"(kLog2));
    return d;
}

// Value of the last lane of this lane's row of W lanes: lane 15 of a 16-lane row (DPP
// row_newbcast:15), lane 31 of a half wavefront (ds_swizzle).
template <int W>
__device__ __forceinline__ uint32_t row_last(uint32_t v) {
    if constexpr (W == 16) return (uint32_t)__builtin_amdgcn_mov_dpp((int)v, 0x15F, 0xF, 0xF, true);
    else return bcast31(v);
}

// The decode entry of a state, 8 bytes in LDS:
//   A = need | base << 16 | maxo << 24: need = w_s + nb, the field's length (used as a
//       bit-field width or shift as it is: only bits 0..4 count); base = the range's first
//       value as int8 bits; maxo = |range| - 1, the largest valid offset
//   B = w_s | next << 16: next = LDS byte address of the entry reached with zero state bits
// A state is held as the LDS byte address of its entry.
struct Ent {
    uint32_t A, B;
};
__device__ __forceinline__ Ent read_ent(uint32_t addr) {
    const v2u v = *(lds_v2u*)(uintptr_t)addr;
    return Ent{v[0], v[1]};
}
__device__ __forceinline__ uint32_t need_of(const Ent& e) { return e.A & 0xFFu; }
__device__ __forceinline__ uint32_t base_of(const Ent& e) { return (e.A >> 16) & 0xFFu; }
__device__ __forceinline__ uint32_t maxo_of(const Ent& e) { return e.A >> 24; }
__device__ __forceinline__ uint32_t next_of(const Ent& e) { return e.B >> 16; }

// The fields of a lane's P streams from the bits at its first field's position: w[0..kWin)
// are the ring dwords from that position's dword on, n[i] holds field i's length in its bits
// 0..4 and n01 is the first two lengths' sum (fields are at most 16 bits, so two fit the low
// word whole, and a lane's P fields take at most 16 P bits).
template <int P>
__device__ __forceinline__ void split_fields(const uint32_t* w, uint32_t start, const uint32_t* n,
                                             uint32_t* f, uint32_t n01) {
    const uint32_t lo = __builtin_amdgcn_alignbit(w[1], w[0], start);
    f[0] = __builtin_amdgcn_ubfe(lo, 0, n[0]);
    f[1] = __builtin_amdgcn_ubfe(lo, n[0], n[1]);
    if constexpr (P == 4) {
        // fields 2 and 3 from the 64 bits at the position (hi:lo) shifted past the first two
        // (one 64-bit shift: n01 may be 32)
        const uint32_t hi = __builtin_amdgcn_alignbit(w[2], w[1], start);
        const uint32_t t2 = (uint32_t)((((uint64_t)hi << 32) | lo) >> n01);
        f[2] = __builtin_amdgcn_ubfe(t2, 0, n[2]);
        f[3] = __builtin_amdgcn_ubfe(t2, n[2], n[3]);
    }
}

// A decoded value's byte, the low byte of o + (A >> 16) (the range's first value in bits
// 16..23 of the entry word A), added straight into byte B of a packed dword: one VOP2 add
// with a byte destination.  byte0 zeroes the other bytes, put_byte keeps them.
__device__ __forceinline__ uint32_t byte0(uint32_t o, uint32_t A) {
    uint32_t x;
    asm("v_add_u32_sdwa %0, %1, %2 dst_sel:BYTE_0 dst_unused:UNUSED_PAD src0_sel:DWORD src1_sel:WORD_1"
        : "=v"(x) : "v"(o), "v"(A));
    return x;
}
template <int B>
__device__ __forceinline__ uint32_t put_byte(uint32_t x, uint32_t o, uint32_t A) {
    static_assert(B >= 1 && B <= 3, "bytes 1..3");
    if constexpr (B == 1)
        asm("v_add_u32_sdwa %0, %1, %2 dst_sel:BYTE_1 dst_unused:UNUSED_PRESERVE src0_sel:DWORD src1_sel:WORD_1"
            : "+v"(x) : "v"(o), "v"(A));
    else if constexpr (B == 2)
        asm("v_add_u32_sdwa %0, %1, %2 dst_sel:BYTE_2 dst_unused:UNUSED_PRESERVE src0_sel:DWORD src1_sel:WORD_1"
            : "+v"(x) : "v"(o), "v"(A));
    else
        asm("v_add_u32_sdwa %0, %1, %2 dst_sel:BYTE_3 dst_unused:UNUSED_PRESERVE src0_sel:DWORD src1_sel:WORD_1"
            : "+v"(x) : "v"(o), "v"(A));
    return x;
}

// Where the decoded values go.  RowBytes: to the output tensor, through the LDS tiles.
// RowMatvec: into y += W a for a row-major int8 matrix W of cols values a row (the
// container's values) and an int8 vector a of cols values staged in LDS, int32 sums; the
// values are never written.  Chunks and rows are multiples of the W P streams (C and cols),
// so a step's values are W P adjacent columns of one matrix row and lane j's P values are
// columns c .. c + P - 1: one dot product of the lane's packed bytes with P vector bytes
// (v_dot4_i32_i8) takes them.  A chunk row's sum of a matrix row goes to y with one atomic
// add by the row's last lane when the step reaches the matrix row's end, and at the chunk's
// end (a matrix row may span chunks).
struct RowBytes {
    static constexpr bool kBytes = true;
};
template <int W, int P>
struct RowMatvec {
    static constexpr bool kBytes = false;
    static constexpr uint32_t kS = W * P;
    int32_t acc;
    uint32_t a_cur;                // the vector bytes of this lane's columns in the step
    uint32_t abyte, abase, aend;   // LDS byte addresses, each + P j: the next step's
                                   // columns, column 0, column cols
    uint32_t mrow;                 // the matrix row of the step
    int32_t* y;
    __device__ __forceinline__ uint32_t read_vec(uint32_t addr) const {
        if constexpr (P == 4) return *(const __attribute__((address_space(3))) uint32_t*)(uintptr_t)addr;
        else return *(const __attribute__((address_space(3))) uint16_t*)(uintptr_t)addr;
    }
    // chunk: the chunk index in its tensor; vec_byte: the staged vector's LDS byte address
    __device__ __forceinline__ void init(uint32_t chunk, uint32_t C, uint32_t cols, uint32_t j,
                                         uint32_t vec_byte, int32_t* y_) {
        const uint32_t first = chunk * C;  // below 2^32: n is
        acc = 0;
        mrow = first / cols;
        abase = vec_byte + P * j;
        aend = abase + cols;
        abyte = abase + first % cols;
        y = y_;
        a_cur = read_vec(abyte);
    }
    // the row sums of the chunk rows whose lanes have mine set go to y
    __device__ __forceinline__ void flush(bool mine, uint32_t j) {
        const uint32_t tot = scan_row<W>((uint32_t)acc);
        if (mine) {
            if (j == W - 1 && tot != 0) atomicAdd(y + mrow, (int32_t)tot);
            acc = 0;
            ++mrow;
        }
    }
    // a step's packed values (byte i: stream P j + i, zero for streams without a value)
    __device__ __forceinline__ void put(uint32_t packed, uint32_t j) {
        acc = __builtin_amdgcn_sdot4((int)packed, (int)a_cur, acc, false);
        abyte += kS;
        const bool wrap = abyte == aend;
        if (wrap) abyte = abase;
        a_cur = read_vec(abyte);
        if (__builtin_amdgcn_ballot_w64(wrap) != 0) flush(wrap, j);
    }
    __device__ __forceinline__ void finish(uint32_t j) { flush(true, j); }
};

// One chunk row's decoder state (every lane of the row holds the same values, except the
// states).
template <int W, int P>
struct Row {
    uint32_t nc, cdw, cbyte, ring_byte, pos, res_hi, refill_at, vout;
    uint32_t end;      // bit position of the chunk's end (its first bit is at bit 0..24 of
                       // the chunk's first dword, the dword holding its first byte)
    uint32_t tile;     // LDS byte address of this lane's bytes in step 0 of the tile
    uint32_t s[P];     // states of streams P j .. P j + P - 1
    v4u pf[RowGeom<W, P>::kFillVecs]; // the next refill, in flight
};

template <class A, int W, int P, class Sink>
__global__ __launch_bounds__(kRowsBlock) void k_decode_rows(const A a) {
    using G = RowGeom<W, P>;
    constexpr uint32_t kS = G::kS, kRowsPerWave = G::kRowsPerWave, kFillVecs = G::kFillVecs;
    constexpr uint32_t kRRing = G::kRing, kRRingStride = G::kRingStride, kRFill = G::kRFill;
    extern __shared__ __align__(16) uint32_t dsm[];
    const uint32_t tid = threadIdx.x, lane = tid & 63, j = lane % W, row = lane / W;
    const uint32_t block = __builtin_amdgcn_readfirstlane(blockIdx.x);
    const SegDesc* sg = codec_seg(a, block, false);
    const uint32_t bseg = block - sg->first_block;
    const uint32_t wid = __builtin_amdgcn_readfirstlane(bseg * (kRowsBlock / 64) + (tid >> 6));
    const uint32_t wv = wid & (kRowsBlock / 64 - 1);
    const uint32_t L = a.h.L, R = a.h.R;
    const uint32_t tab_byte = lds_offset(dsm);
    const uint32_t rings = 2 * L;                   // dwords: the table takes L entries of 2
    const uint32_t* dec = sg->tab ? sg->tab + kDTDec : inline_tab(a);
    const uint32_t* hdr = sg->tab ? sg->tab + kDTHdr : inline_hdr(a);
    const uint32_t n_chunks = sg->n_chunks;
    const uint64_t n = sg->n;
    const uint32_t index_at = header_bytes_dev(a.h.K);
    const uint32_t payload_at = index_at + (uint32_t)index_bytes_of(n_chunks);
    const uint32_t ulog = size_unit_log2(a.h.C, R, kS);  // chunk sizes count units of 2^ulog bytes
    const uint64_t in_nbytes = sg->c_bytes;
    const rsrc_t rin = make_rsrc(sg->c, (uint32_t)in_nbytes);

    // loads that need nothing else go out first: this thread's table slot and the sizes of
    // the chunks of the wavefront's group of 64 (its chunks lie in one group)
    static_assert(kGroupChunks % kRowsPerWave == 0, "a wavefront's chunks lie in one group");
    const uint32_t group = kRowsPerWave * wid;      // the wavefront's first chunk
    const uint32_t chunk = group + row;
    const uint32_t ts = tid < L ? tid : L - 1;      // slot tid (more below when L > 256)
    const uint32_t te0 = dec[2 * ts], te1 = dec[2 * ts + 1];
    const GroupSpans gs = group_spans(rin, index_at, n_chunks, group / kGroupChunks, ulog);
    const uint32_t c_rel = lane_value(gs.rel, chunk % kGroupChunks);
    const uint32_t c_bytes = lane_value(gs.bytes, chunk % kGroupChunks);

    const uint64_t grp_first = (uint64_t)group * a.h.C;
    const uint64_t grp_len = grp_first < n ? n - grp_first : 0;
    const uint64_t grp_cap = (uint64_t)kRowsPerWave * a.h.C;
    const rsrc_t rout = make_rsrc(sg->x + (grp_first < n ? grp_first : 0),
                                  (uint32_t)(grp_len < grp_cap ? grp_len : grp_cap));

    Row<W, P> r;
    const uint32_t rowi = wv * kRowsPerWave + row;  // the row in the block
    r.ring_byte = tab_byte + 4 * (rings + rowi * kRRingStride);
    const uint32_t tile_base =
        tab_byte + 4 * (rings + G::kRowsPerBlock * kRRingStride + rowi * G::kTileStride);
    r.tile = tile_base + P * j;
    r.vout = row * a.h.C + P * j;
    r.nc = 0;
    r.cdw = 0;
    r.cbyte = 0;
    r.end = 0;
    uint32_t bit0 = 0;  // the chunk's first bit within its first dword
    uint32_t err = 0;
    if (chunk < n_chunks) {
        const uint64_t first = (uint64_t)chunk * a.h.C;
        const uint32_t m = (uint32_t)((n - first) < a.h.C ? (n - first) : a.h.C);
        const uint64_t at = (uint64_t)payload_at + gs.head + c_rel;  // the chunk's first byte
        const bool ok = gs.ok && (c_bytes >> ulog) <= chunk_bound_units(m, R, ulog, kS) &&
                        at + c_bytes <= in_nbytes;
        if (ok) {
            r.nc = m;
            bit0 = 8 * ((uint32_t)at & 3);
            r.cbyte = (uint32_t)at & ~3u;
            r.end = bit0 + 8 * c_bytes;
            r.cdw = (r.end + 31) >> 5;
        } else {
            err = 1;
        }
    }
    // the first two refills (the whole ring), and the third in flight
    constexpr uint32_t kLaneFill = 4 * kFillVecs;   // dwords a lane loads per refill
    v4u f0[kFillVecs], f1[kFillVecs];
#pragma unroll
    for (uint32_t v = 0; v < kFillVecs; ++v) {
        f0[v] = load4(rin, r.cbyte, kLaneFill * j + 4 * v, r.cdw);
        f1[v] = load4(rin, r.cbyte, kRFill + kLaneFill * j + 4 * v, r.cdw);
    }
    r.res_hi = 2 * kRFill;  // dwords [res_hi - kRRing, res_hi) are in the ring
#pragma unroll
    for (uint32_t v = 0; v < kFillVecs; ++v)
        r.pf[v] = load4(rin, r.cbyte, r.res_hi + kLaneFill * j + 4 * v, r.cdw);
    r.refill_at = r.res_hi < r.cdw ? (r.res_hi - G::kMargin) * 32 : 0xFFFFFFFFu;

    if (wid == 0) {
        // header and index ends: the container must belong to this table and fit in_nbytes;
        // a device table that failed to build, or was built from no values, decodes nothing
        constexpr int kHdrPerLane = (kMaxHeaderDwords + 63) / 64;
        const uint32_t hd = index_at / 4;
        uint32_t hv[kHdrPerLane], tv[kHdrPerLane];
#pragma unroll
        for (int k = 0; k < kHdrPerLane; ++k) {
            const uint32_t i = lane + 64 * k, jj = i < hd ? i : 0;
            hv[k] = __builtin_amdgcn_raw_buffer_load_b32(rin, (int)(4 * jj), 0, 0);
            tv[k] = hdr[jj];
        }
        const bool ends_ok = index_ends_ok(rin, index_at, payload_at, n_chunks, in_nbytes);
        bool bad = sg->tab && (sg->tab[kDTStatus] != 0 ||
                               (n > 0 && (sg->tab[kDTN] | sg->tab[kDTN + 1]) == 0));
        // a device table built for other parameters than the launch's
        report(a.h.status, SH_ERR_INVALID_ARG,
               sg->tab && (sg->tab[kDTK] != a.h.K || sg->tab[kDTLog2L] != a.h.R));
#pragma unroll
        for (int k = 0; k < kHdrPerLane; ++k) {
            const uint32_t i = lane + 64 * k;
            if (i < hd) bad |= hv[k] != header_dword_of(tv[k], i, n, n_chunks);
        }
        bad |= !ends_ok;
        report(a.h.status, SH_ERR_CORRUPT_STREAM, bad);
    }

    // the table's entries in the LDS form (device form: e0 = need | next slot * 8 << 16,
    // e1 = w | base << 8 | (|range| - 1) << 16)
    auto stage_entry = [&](uint32_t slot, uint32_t e0, uint32_t e1) {
        dsm[2 * slot] = (e0 & 0xFFu) | ((e1 & 0xFF00u) << 8) | ((e1 & 0xFF0000u) << 8);
        dsm[2 * slot + 1] = (e1 & 0xFFu) | ((tab_byte + (e0 >> 16)) << 16);
    };
    if (tid < L) stage_entry(tid, te0, te1);
    for (uint32_t slot = tid + kRowsBlock; slot < L; slot += kRowsBlock)
        stage_entry(slot, dec[2 * slot], dec[2 * slot + 1]);
    {
        uint32_t* rg = &dsm[rings + rowi * kRRingStride];
#pragma unroll
        for (uint32_t v = 0; v < kFillVecs; ++v) {
            *reinterpret_cast<v4u*>(&rg[kLaneFill * j + 4 * v]) = f0[v];
            *reinterpret_cast<v4u*>(&rg[kRFill + kLaneFill * j + 4 * v]) = f1[v];
        }
        if (j == 0) {
            rg[kRRing] = f0[0][0];
            rg[kRRing + 1] = f0[0][1];
        }
    }
    // the matrix-vector sink's vector, where the tiles would be: cols values (a multiple of
    // the chunk's streams, 16-byte aligned source)
    const uint32_t vec_dw = rings + G::kRowsPerBlock * kRRingStride;
    if constexpr (!Sink::kBytes) {
        const v4u* src = reinterpret_cast<const v4u*>(sg->vec);
        for (uint32_t i = tid; i < a.h.cols / 16; i += kRowsBlock)
            *reinterpret_cast<v4u*>(&dsm[vec_dw + 4 * i]) = src[i];
    }
    __syncthreads();
    Sink sink;
    if constexpr (!Sink::kBytes)
        sink.init(chunk, a.h.C, a.h.cols, j, tab_byte + 4 * vec_dw, reinterpret_cast<int32_t*>(sg->x));

    // initial slots: stream s's R bits at bit0 + s * R (at most 24 + 127 * 11 + 11 bits: within
    // the first ring words, no wrap)
    const uint32_t lanes = r.nc < kS ? r.nc : kS;
    auto init_state = [&](uint32_t s) {
        if (s >= lanes) return tab_byte;
        const uint32_t p = bit0 + s * R;
        const lds_u32* w = (const lds_u32*)(uintptr_t)(r.ring_byte + 4 * (p >> 5));
        const uint32_t bits = __builtin_amdgcn_alignbit(w[1], w[0], p);
        return tab_byte + ((bits & (L - 1)) << 3);
    };
#pragma unroll
    for (int i = 0; i < P; ++i) r.s[i] = init_state(P * j + i);
    r.pos = bit0 + lanes * R;

    // steps where every stream of the wavefront's chunks decodes a value that is not its
    // last (every stream's last value lies at or after step nc / kS - 1); the rest go
    // through the general step
    uint32_t nc_min = 0xFFFFFFFFu, nc_max = 0;
#pragma unroll
    for (uint32_t k = 0; k < kRowsPerWave; ++k) {
        const uint32_t v = __builtin_amdgcn_readlane(r.nc, W * k);
        nc_min = nc_min < v ? nc_min : v;
        nc_max = nc_max > v ? nc_max : v;
    }
    const uint32_t full = nc_min / kS > 0 ? nc_min / kS - 1 : 0;
    const uint32_t steps = (nc_max + kS - 1) / kS;
    uint64_t bad_offsets = 0;  // lanes that decoded an offset outside its range

    auto refill = [&]() {
        if (r.pos >= r.refill_at) {
            const uint32_t d = (r.res_hi + kLaneFill * j) & (kRRing - 1);
            typedef __attribute__((address_space(3))) v4u lds_w4;
            typedef __attribute__((address_space(3))) v2u lds_w2;
#pragma unroll
            for (uint32_t v = 0; v < kFillVecs; ++v)
                *(lds_w4*)(uintptr_t)(r.ring_byte + 4 * (d + 4 * v)) = r.pf[v];
            if (d == 0) *(lds_w2*)(uintptr_t)(r.ring_byte + 4 * kRRing) = v2u{r.pf[0][0], r.pf[0][1]};
            r.res_hi += kRFill;
            r.refill_at = r.res_hi < r.cdw ? (r.res_hi - G::kMargin) * 32 : 0xFFFFFFFFu;
#pragma unroll
            for (uint32_t v = 0; v < kFillVecs; ++v)
                r.pf[v] = load4(rin, r.cbyte, r.res_hi + kLaneFill * j + 4 * v, r.cdw);
        }
    };

    // One step: the lane's P fields are adjacent, stream P j's first.  The entries were read
    // at the end of the previous step, so the serial path is scan -> ring read -> bit
    // extract -> next entry read.  k is the step's place in the tile (a constant in the
    // unrolled loop, so the tile writes take their offset from the instruction).
    auto full_step = [&](const Ent* e, Ent* ne, uint32_t k) {
        uint32_t tot, nd[P], w[G::kWin], f[P], packed = 0;
        const uint32_t n01 = need_of(e[0]) + need_of(e[1]);
        if constexpr (P == 2) tot = n01;
        else tot = n01 + ((e[2].A + e[3].A) & 0xFFu);  // two needs of at most 16: no carry out
#pragma unroll
        for (int i = 0; i < P; ++i) nd[i] = e[i].A;  // bits 0..4: the need
        // the lane's first bit: the row's position plus the previous lane's inclusive sum
        // within its 16 lanes (one DPP add with a row shift, which reads zero for lane 0);
        // in a 32-lane row the upper 16 lanes then add lane 15's sum (row_bcast:15, rows 1
        // and 3 only).  The two adds are written out because the compiler makes four
        // operations of the masked broadcast; the s_nop gives the DPP source, written by
        // the scan just before, its two wait states.
        const uint32_t incl = scan16(tot);
        uint32_t start = r.pos;
        if constexpr (W == 16)
            start += (uint32_t)__builtin_amdgcn_update_dpp(0, (int)incl, 0x111, 0xF, 0xF, true);
        else
            asm("s_nop 1\n\tv_add_u32_dpp %0, %1, %0 row_shr:1 row_mask:0xf bank_mask:0xf bound_ctrl:1\n\t"
                "v_add_u32_dpp %0, %1, %0 row_bcast:15 row_mask:0xa bank_mask:0xf"
                : "+v"(start) : "v"(incl));
        const lds_u32* rp = (const lds_u32*)(uintptr_t)((ring_dword<G::kRingLog2>(start) << 2) + r.ring_byte);
#pragma unroll
        for (uint32_t i = 0; i < G::kWin; ++i) w[i] = rp[i];
        split_fields<P>(w, start, nd, f, n01);
#pragma unroll
        for (int i = 0; i < P; ++i) {
            const uint32_t o = __builtin_amdgcn_ubfe(f[i], 0, e[i].B);
            r.s[i] = ((f[i] >> (e[i].B & 31)) << 3) + next_of(e[i]);
            ne[i] = read_ent(r.s[i]);
            bad_offsets |= __builtin_amdgcn_ballot_w64(o > maxo_of(e[i]));
            if (i == 0) {
                packed = byte0(o, e[i].A);
            } else if (i == 1) {
                packed = put_byte<1>(packed, o, e[i].A);
            } else if (i == 2) {
                packed = put_byte<2>(packed, o, e[i].A);
            } else {
                packed = put_byte<3>(packed, o, e[i].A);
            }
        }
        // the lane's bytes into the tile, packed by the byte-destination adds above: one
        // 16-bit write for two, one dword for four (or into the consumer's sums)
        if constexpr (!Sink::kBytes) {
            sink.put(packed, j);
        } else if constexpr (P == 2) {
            typedef __attribute__((address_space(3))) uint16_t lds_w2b;
            *(lds_w2b*)(uintptr_t)(r.tile + kS * k) = (uint16_t)packed;
        } else {
            typedef __attribute__((address_space(3))) uint32_t lds_w4b;
            *(lds_w4b*)(uintptr_t)(r.tile + kS * k) = packed;
        }
        // the next step's position: the end of the row's last lane
        if constexpr (W == 16) r.pos += row_last<W>(incl);
        else r.pos = bcast31(start + tot);
    };
    // the tile of steps [t0, t0 + kTileSteps) to the output: lane j stores its share of
    // the row's kS * kTileSteps bytes (LDS operations of a wavefront complete in order, so
    // the row's writes are visible); a lane's share lies within one step
    constexpr uint32_t kLaneBytes = P * kTileSteps;
    auto flush_tile = [&](uint32_t t0) {
        const uint32_t at = row * a.h.C + kLaneBytes * j;
        if constexpr (kLaneBytes == 16) {
            const v4u w = *(const __attribute__((address_space(3))) v4u*)(uintptr_t)(tile_base + 16 * j);
            __builtin_amdgcn_raw_buffer_store_b128(w, rout, (int)at, (int)(t0 * kS), 0);
        } else {
            const v2u w = *(lds_v2u*)(uintptr_t)(tile_base + 8 * j);
            __builtin_amdgcn_raw_buffer_store_b64(w, rout, (int)at, (int)(t0 * kS), 0);
        }
    };
    static_assert(kS % kLaneBytes == 0, "a lane's share of a tile lies within one step");

    Ent ea[P], eb[P];
#pragma unroll
    for (int i = 0; i < P; ++i) ea[i] = read_ent(r.s[i]);
    uint32_t t = 0;
    // the waves on a SIMD take turns at the highest priority (take_turn)
    const uint32_t slot_id = wave_slot();
    const uint32_t full4 = full & ~(kTileSteps - 1);
    while (t < full4) {
        take_turn(t / kPrioSteps, slot_id);
        const uint32_t stop = full4 - t < kPrioSteps ? full4 : t + kPrioSteps;
        for (; t < stop; t += kTileSteps) {  // the entries alternate registers step by step
#pragma unroll
            for (uint32_t k = 0; k < kTileSteps; k += 2) {
                full_step(ea, eb, k);
                full_step(eb, ea, k + 1);
                refill();
            }
            if constexpr (Sink::kBytes) flush_tile(t);
        }
    }
    __builtin_amdgcn_s_setprio(0);
    // the full steps after the last whole tile (fewer than kTileSteps, the same for the
    // wavefront's rows), then their part of a tile: only the steps that hold a stream's last
    // value go through the general step
    static_assert(kTileSteps == 4, "up to three full steps after the last whole tile");
    if (t < full) {
        const uint32_t left = full - t;
        full_step(ea, eb, 0);
        if (left > 1) {
            full_step(eb, ea, 1);
            refill();
            if (left > 2) {
                full_step(ea, eb, 2);
#pragma unroll
                for (int i = 0; i < P; ++i) ea[i] = eb[i];
            }
        } else {
#pragma unroll
            for (int i = 0; i < P; ++i) ea[i] = eb[i];
        }
        refill();
        if (Sink::kBytes && kLaneBytes * j < left * kS) {
            const uint32_t at = row * a.h.C + kLaneBytes * j;
            if constexpr (kLaneBytes == 16) {
                const v4u w = *(const __attribute__((address_space(3))) v4u*)(uintptr_t)(tile_base + 16 * j);
                __builtin_amdgcn_raw_buffer_store_b128(w, rout, (int)at, (int)(t * kS), 0);
            } else {
                const v2u w = *(lds_v2u*)(uintptr_t)(tile_base + 8 * j);
                __builtin_amdgcn_raw_buffer_store_b64(w, rout, (int)at, (int)(t * kS), 0);
            }
        }
        t = full;
    }
    // the general step: a stream past its chunk's end has no field, and a stream at its
    // last value has the offset alone (its state bits are zero and implied)
    for (; t < steps; ++t) {
        uint32_t nd[P], w[G::kWin], f[P], tot = 0;
        bool act[P];
#pragma unroll
        for (int i = 0; i < P; ++i) {
            const uint32_t s = t * kS + P * j + i;
            act[i] = s < r.nc;
            const bool last = act[i] && s + kS >= r.nc;
            nd[i] = act[i] ? (last ? (ea[i].B & 31) : need_of(ea[i])) : 0;
            tot += nd[i];
        }
        const uint32_t incl = scan_row<W>(tot);
        const uint32_t start = r.pos - tot + incl;
        const lds_u32* rp = (const lds_u32*)(uintptr_t)((ring_dword<G::kRingLog2>(start) << 2) + r.ring_byte);
#pragma unroll
        for (uint32_t i = 0; i < G::kWin; ++i) w[i] = rp[i];
        split_fields<P>(w, start, nd, f, nd[0] + nd[1]);
        uint32_t pk = 0;  // the matrix-vector sink's packed values
#pragma unroll
        for (int i = 0; i < P; ++i) {
            const uint32_t o = __builtin_amdgcn_ubfe(f[i], 0, act[i] ? ea[i].B : 0u);
            if (act[i]) {
                err |= o > maxo_of(ea[i]);
                r.s[i] = ((f[i] >> (ea[i].B & 31)) << 3) + next_of(ea[i]);
                if constexpr (Sink::kBytes)
                    __builtin_amdgcn_raw_buffer_store_b8((uint8_t)(o + base_of(ea[i])), rout,
                                                         (int)(r.vout + i), (int)(t * kS), 0);
                else
                    pk |= ((o + base_of(ea[i])) & 0xFFu) << (8 * i);
            }
        }
        if constexpr (!Sink::kBytes) sink.put(pk, j);
        r.pos += row_last<W>(incl);
#pragma unroll
        for (int i = 0; i < P; ++i) ea[i] = read_ent(r.s[i]);
        refill();
    }

    // a valid chunk leaves every stream in slot 0 and ends in its last size unit, zero-padded
    // (a unit of at most 4 bytes never straddles a dword: chunks start on unit boundaries)
    if (r.nc > 0) {
#pragma unroll
        for (int i = 0; i < P; ++i)
            if (P * j + i < lanes && r.s[i] != tab_byte) err = 1;
        if (r.pos > r.end || r.end - r.pos >= (8u << ulog)) {
            err = 1;
        } else if (r.pos < r.end) {
            const lds_u32* w = (const lds_u32*)(uintptr_t)(r.ring_byte + 4 * ((r.pos >> 5) & (kRRing - 1)));
            const uint32_t gap = r.end - r.pos;
            const uint32_t pad = *w >> (r.pos & 31);
            if ((gap < 32 ? pad & ((1u << gap) - 1) : pad) != 0) err = 1;
        }
    }
    if constexpr (!Sink::kBytes) sink.finish(j);
    report(a.h.status, SH_ERR_CORRUPT_STREAM, err != 0 || bad_offsets != 0);
}

template <int W, int P>
uint32_t rows_lds_bytes(uint32_t L) {
    using G = RowGeom<W, P>;
    return 4 * (2 * L + G::kRowsPerBlock * (G::kRingStride + G::kTileStride));
}
// the matrix-vector form: the vector (cols bytes, 16-byte multiples) in place of the tiles
template <int W, int P>
uint32_t rows_matvec_lds_bytes(uint32_t L, uint32_t cols) {
    using G = RowGeom<W, P>;
    return 4 * (2 * L + G::kRowsPerBlock * G::kRingStride) + (cols + 15) / 16 * 16;
}

template <int W, int P, class Sink = RowBytes>
sh_status launch_rows(const CodecArgs& a, uint32_t total_blocks, void* stream) {
    if (total_blocks == 0) return SH_OK;
    const uint32_t lds = Sink::kBytes ? rows_lds_bytes<W, P>(a.L)
                                      : rows_matvec_lds_bytes<W, P>(a.L, a.cols);
    with_kernel_args(a, [&](const auto& k) {
        using K = std::decay_t<decltype(k)>;
        // the matrix-vector form takes device tables only
        if constexpr (Sink::kBytes || !std::is_same_v<K, KOne>)
            hipLaunchKernelGGL((k_decode_rows<K, W, P, Sink>), dim3(total_blocks),
                               dim3(kRowsBlock), lds, (hipStream_t)stream, k);
    });
    return hipGetLastError() == hipSuccess ? SH_OK : SH_ERR_HIP;
}

}  // namespace

sh_status launch_decode(const CodecArgs& a, uint32_t total_blocks, void* stream) {
    if (a.S == kStreamsNarrow) return launch_rows<16, 2>(a, total_blocks, stream);
    if (a.S == kStreamsWide) return launch_rows<16, 4>(a, total_blocks, stream);
    return SH_ERR_UNSUPPORTED;
}

sh_status launch_decode_wide_halves(const CodecArgs& a, uint32_t total_blocks, void* stream) {
    if (a.S == kStreamsWide) return launch_rows<32, 2>(a, total_blocks, stream);
    if (a.S == kStreamsWidest) return launch_rows<32, 4>(a, total_blocks, stream);
    return SH_ERR_UNSUPPORTED;
}

sh_status launch_decode_matvec_rows(const CodecArgs& a, uint32_t total_blocks, bool few,
                                    void* stream) {
    if (a.nseg == 0) return SH_ERR_INVALID_ARG;  // device tables only
    if (a.S == kStreamsWide && !few) return launch_rows<16, 4, RowMatvec<16, 4>>(a, total_blocks, stream);
    if (a.S == kStreamsWide) return launch_rows<32, 2, RowMatvec<32, 2>>(a, total_blocks, stream);
    if (a.S == kStreamsWidest) return launch_rows<32, 4, RowMatvec<32, 4>>(a, total_blocks, stream);
    return SH_ERR_UNSUPPORTED;
}

}  // namespace shn
