// Decode kernel of the Shannonic codec for gfx950 (CDNA4, wave64).
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
// dense contraction.  The same kernel either stores the decoded bytes or hands them to a
// consumer in registers (an int8 matrix-vector product, MatvecSink), so that the decoded
// tensor never reaches HBM.
#include <type_traits>

#include "device_common.hpp"

namespace shn {

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
constexpr uint32_t kRot = 32;  // ring turn of the odd half wavefront, dwords

// 16 bytes of the chunk starting at dword d (dwords at or past cdw read as 0).  The whole
// load is issued by every lane (from offset 0 where it would leave the chunk) and the rare
// lanes at the chunk's end fetch their dwords one by one into other registers, so nothing
// waits for the load here.
__device__ __forceinline__ v4u load_words(rsrc_t r, uint32_t chunk_byte, uint32_t d,
                                          uint32_t cdw) {
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

typedef unsigned int v2u __attribute__((ext_vector_type(2)));

typedef const __attribute__((address_space(3))) v2u lds_v2u;

// Per-chunk decoder state of one half wavefront.
struct DecChain {
    uint32_t nc, cdw, cbyte, ring, ring_byte, rot, lanes, pos, addr, res_hi, refill_at, err, vout;
    uint32_t bit0, end;  // the chunk's first bit in its first dword; its end (ring bits)
    v4u pf;
};

constexpr int kDecBlock = 256;  // 4 wavefronts

// Where the decoded values go.  Bytes: the decoded tensor, one byte per value
// (sh_decode); the kernel stores them itself.  Any other sink takes one value per lane,
// step and chain (put, or put_if in the steps where a chunk may already have ended);
// step_done follows every step and finish the last one.
struct Bytes {
    static constexpr bool kBytes = true;
    static constexpr uint32_t kLdsDwords = 0;
};

// MatvecSink: y[r] += sum_c W[r][c] a[c] over the decoded matrix W (row-major, cols values
// a row, cols a multiple of 32) without writing W (sh_decode_matvec_batch).  The 32 values
// of a chunk's step lie in one row; every lane keeps the products of its values in an int32
// and, where a row ends within the chunk or the chunk ends, the half wavefront's 32 sums go
// into y[r] with one atomic add, so rows split across chunks are summed exactly too.  The
// vector a (int8, at most kMaxMatvecCols values) is held in LDS.
// a * b + c for a, b sign-extended bytes: one 24-bit multiply-add (the compiler would
// otherwise pick a 64-bit multiply-add for the wrapping 32-bit sum)
__device__ __forceinline__ int32_t mad24(int32_t a, int32_t b, int32_t c) {
    int32_t d;
    asm volatile("v_mad_i32_i24 %0, %1, %2, %3" : "=v"(d) : "v"(a), "v"(b), "v"(c));
    return d;
}

template <bool kAligned>
struct MatvecSink {
    static constexpr bool kBytes = false;
    static constexpr uint32_t kLdsDwords = kMaxMatvecCols / 4;
    int32_t acc;
    int32_t xp, ap;           // the last step's value and vector entry, multiplied one step
                              // later so that nothing waits for the vector's LDS read
    uint32_t abyte;           // LDS byte address of a[c] for this lane's value of the step
    uint32_t cols;
    int32_t* y;
    // per half wavefront (wave-uniform copies of both): the step that ends the current row
    // (~0 once past the chunk), the row, and the chunk's steps; next = the earlier end
    uint32_t wrap[2], row[2], steps[2], next;
    // kAligned: rows start with every chunk (C a multiple of cols), so both halves end their
    // rows at the same steps, every cols / 32 steps from the chunk start
    uint32_t abase, row_mine;
    template <class A>
    __device__ __forceinline__ void init(const A& a, const SegDesc* sg, uint32_t group,
                                         uint32_t li, uint32_t hw, uint32_t n_chunks,
                                         uint32_t vec_byte) {
        cols = a.h.cols;
        y = reinterpret_cast<int32_t*>(sg->x);
        acc = 0;
        xp = 0;
        ap = 0;
        uint32_t col_mine = 0;
#pragma unroll
        for (int h = 0; h < 2; ++h) {
            const uint32_t chunk = group + h;
            const uint32_t first = chunk * a.h.C;  // below 2^32: n is
            const uint32_t col0 = first % cols;
            steps[h] = 0;
            if (chunk < n_chunks) {
                const uint32_t m = (uint32_t)(sg->n - first) < a.h.C ? (uint32_t)(sg->n - first) : a.h.C;
                steps[h] = m / 32;
            }
            wrap[h] = (cols - col0) / 32 - 1;
            if (wrap[h] >= steps[h]) wrap[h] = ~0u;
            row[h] = first / cols;
            if (h == (int)hw) col_mine = col0;
        }
        next = wrap[0] < wrap[1] ? wrap[0] : wrap[1];
        abyte = vec_byte + col_mine + li;
        abase = vec_byte + li;
        row_mine = hw ? row[1] : row[0];
        if (kAligned) next = cols / 32 - 1;
    }
    // the value: offset o plus the range's first value (e0's top byte, int8 bits); for a
    // valid offset the sum stays in [-128, 127]
    __device__ __forceinline__ void put(int, uint32_t o, uint32_t e0, uint32_t) {
        typedef const __attribute__((address_space(3))) int8_t lds_i8;
        acc = mad24(xp, ap, acc);
        xp = (int32_t)o + (int32_t)(int8_t)(uint8_t)(e0 >> 24);
        ap = *(lds_i8*)(uintptr_t)abyte;
    }
    __device__ __forceinline__ void put_if(int k, uint32_t o, uint32_t e0, uint32_t t, bool act) {
        acc = mad24(xp, ap, acc);
        xp = 0;
        ap = 0;
        if (act) put(k, o, e0, t);
    }
    // the sums of the half wavefronts whose row ended with step t go to y
    __device__ __forceinline__ void flush(bool end0, bool end1, uint32_t li, uint32_t hw) {
        acc = mad24(xp, ap, acc);
        xp = 0;
        const uint32_t tot = scan32((uint32_t)acc);  // lane 31 of a half: its sum
        if (hw ? end1 : end0) {
            if (li == 31 && tot != 0) atomicAdd(y + (hw ? row[1] : row[0]), (int32_t)tot);
            acc = 0;
        }
    }
    __device__ __forceinline__ void step_done(uint32_t t) {
        abyte += 32;
        if constexpr (kAligned) {
            // every lane's row ends here; a half whose chunk has ended holds 0 and adds
            // nothing (its row index may be past the tensor)
            if (__builtin_expect(t == next, 0)) {
                acc = mad24(xp, ap, acc);
                xp = 0;
                const uint32_t tot = scan32((uint32_t)acc);
                if ((__lane_id() & 31) == 31 && tot != 0) atomicAdd(y + row_mine, (int32_t)tot);
                acc = 0;
                ++row_mine;
                abyte = abase;
                next += cols / 32;
            }
            return;
        }
        if (__builtin_expect(t == next, 0)) {  // one scalar compare a step; the rest once a row
            const bool end0 = t == wrap[0], end1 = t == wrap[1];
            const uint32_t lane = __lane_id(), li = lane & 31, hw = lane >> 5;
            flush(end0, end1, li, hw);
            if (hw ? end1 : end0) abyte -= cols;
#pragma unroll
            for (int h = 0; h < 2; ++h)
                if (h == 0 ? end0 : end1) {
                    wrap[h] += cols / 32;
                    if (wrap[h] >= steps[h]) wrap[h] = ~0u;
                    ++row[h];
                }
            next = wrap[0] < wrap[1] ? wrap[0] : wrap[1];
        }
    }
    // a chunk that ends inside a row leaves a partial sum (the sums of ended rows are 0)
    __device__ __forceinline__ void finish() {
        const uint32_t lane = __lane_id();
        flush(true, true, lane & 31, lane >> 5);
    }
    // the vector into LDS at vec_byte (cols values, 16-byte aligned, a multiple of 32)
    template <class A>
    __device__ __forceinline__ static void stage(const A& a, const SegDesc* sg, uint32_t* vec,
                                                 uint32_t tid) {
        const uint32_t groups = a.h.cols / 16;
        const v4u* src = reinterpret_cast<const v4u*>(sg->vec);
        for (uint32_t i = tid; i < groups; i += kDecBlock) reinterpret_cast<v4u*>(vec)[i] = src[i];
    }
};
// ILP chunks per lane: a wavefront decodes 2 * ILP chunks, lanes 32h..32h+31 take chunks
// 2k + h (k < ILP) of the wavefront's group.  ILP = 1 is the one launched: measured on
// MI355X, two independent chains per lane ran slower than twice as many wavefronts.
template <int ILP, class Sink, class A>
__global__ __launch_bounds__(kDecBlock) void k_decode(const A a) {
    static_assert(Sink::kBytes || ILP == 1, "a consumer sink takes one chunk per half wavefront");
    constexpr uint32_t kChunksPerWave = 2 * ILP;
    static_assert(kGroupChunks % kChunksPerWave == 0, "a wavefront's chunks lie in one index group");
    constexpr uint32_t kChunksPerBlock = kDecBlock / 64 * kChunksPerWave;
    constexpr uint32_t kVecAt = kTabDwords + kChunksPerBlock * kRingStride;
    // the rings' wrapped addresses are formed with an and-or, which needs every ring on a
    // kRingStride boundary of the LDS address space: sm is the kernel's only LDS object
    __shared__ __align__(4 * kRingStride) uint32_t sm[kVecAt + Sink::kLdsDwords];
    const uint32_t tid = threadIdx.x, lane = tid & 63, li = lane & 31, hw = lane >> 5;
    const uint32_t block = __builtin_amdgcn_readfirstlane(blockIdx.x);
    const SegDesc* sg = codec_seg(a, block, false);
    const uint32_t bseg = block - sg->first_block;  // block within its segment
    // wavefront index within the segment, uniform so that descriptors stay scalar
    const uint32_t wid = __builtin_amdgcn_readfirstlane(bseg * (kDecBlock / 64) + (tid >> 6));
    const uint32_t wv = wid & (kDecBlock / 64 - 1);
    const uint32_t tab_byte = lds_offset(sm);
    const uint32_t* dec = sg->tab ? sg->tab + kDTDec : inline_tab(a);
    const uint32_t* hdr = sg->tab ? sg->tab + kDTHdr : inline_hdr(a);
    const uint32_t n_chunks = sg->n_chunks;
    const uint64_t n = sg->n;
    const uint32_t index_at = header_bytes_dev(a.h.K);
    const uint32_t payload_at = index_at + (uint32_t)index_bytes_of(n_chunks);
    const uint32_t ulog = size_unit_log2(a.h.C, a.h.R, kStreamsNarrow);  // units of 2^ulog bytes
    const uint64_t in_nbytes = sg->c_bytes;

    // The prologue's loads go out in two waves: first everything that needs nothing else
    // (the table slot of each thread and the chunk sizes of the wavefront's index group),
    // then, once the index is in, the chunk's first payload words; LDS is written only after
    // both waves are issued.
    const rsrc_t rin = make_rsrc(sg->c, (uint32_t)in_nbytes);
    const uint32_t group = kChunksPerWave * wid;
    // L <= 256 = kDecBlock: one slot per thread; threads past L repeat the last slot
    const uint32_t ts = tid < a.h.L ? tid : a.h.L - 1;
    const uint32_t te0 = dec[2 * ts], te1 = dec[2 * ts + 1];
    const GroupSpans gs = group_spans(rin, index_at, n_chunks, group / kGroupChunks, ulog);

    // output: per-wavefront descriptor over the wavefront's chunks
    const uint64_t grp_first = (uint64_t)group * a.h.C;
    const uint64_t grp_len = grp_first < n ? n - grp_first : 0;
    const uint64_t grp_cap = (uint64_t)kChunksPerWave * a.h.C;
    const rsrc_t rout = make_rsrc(sg->x + (grp_first < n ? grp_first : 0),
                                  (uint32_t)(grp_len < grp_cap ? grp_len : grp_cap));
    Sink sink;
    if constexpr (!Sink::kBytes) {
        sink.init(a, sg, group, li, hw, n_chunks, tab_byte + 4 * kVecAt);
        Sink::stage(a, sg, sm + kVecAt, tid);
    }

    DecChain ch[ILP];
    v4u fill0[ILP], fill1[ILP];
#pragma unroll
    for (int k = 0; k < ILP; ++k) {
        DecChain& c = ch[k];
        const uint32_t slot = 2 * k + hw;
        const uint32_t chunk = group + slot;
        c.ring = kTabDwords + (wv * kChunksPerWave + slot) * kRingStride;
        c.ring_byte = tab_byte + 4 * c.ring;
        // the odd half wavefront's ring is turned by kRot dwords, so that the two halves,
        // which read at similar offsets, do not read the same LDS banks
        c.rot = hw * kRot;
        c.vout = slot * a.h.C + li;
        c.nc = 0;
        c.cdw = 0;
        c.cbyte = 0;
        c.err = 0;
        c.bit0 = 0;
        c.end = 0;
        const uint32_t c_rel = lane_value(gs.rel, chunk % kGroupChunks);
        const uint32_t c_bytes = lane_value(gs.bytes, chunk % kGroupChunks);
        if (chunk < n_chunks) {
            const uint64_t first = (uint64_t)chunk * a.h.C;
            const uint32_t m = (uint32_t)((n - first) < a.h.C ? (n - first) : a.h.C);
            const uint64_t at = (uint64_t)payload_at + gs.head + c_rel;  // the chunk's first byte
            const bool ok = gs.ok && (c_bytes >> ulog) <= chunk_bound_units(m, a.h.R, ulog, kStreamsNarrow) &&
                            at + c_bytes <= in_nbytes;
            if (ok) {
                c.nc = m;
                c.bit0 = 8 * ((uint32_t)at & 3);
                c.cbyte = (uint32_t)at & ~3u;
                c.cdw = (c.bit0 + 8 * c_bytes + 31) >> 5;
                c.end = c.bit0 + 8 * c_bytes + 32 * c.rot;
            } else {
                c.err = 1;
            }
        }
        c.lanes = c.nc < 32 ? c.nc : 32;
        // the first two refills, plus the third in flight
        fill0[k] = load_words(rin, c.cbyte, 4 * li, c.cdw);
        fill1[k] = load_words(rin, c.cbyte, kFill + 4 * li, c.cdw);
        c.res_hi = 2 * kFill;  // dwords [res_hi - kRing, res_hi) are in the ring
        c.pf = load_words(rin, c.cbyte, c.res_hi + 4 * li, c.cdw);
        // refills are checked every other step; one is due once the next two steps could
        // read past res_hi (each advances at most 16 dwords): pos >> 5 >= res_hi - 33 + rot
        c.refill_at = c.res_hi < c.cdw ? (c.res_hi - 33 + c.rot) * 32 : 0xFFFFFFFFu;
    }

    if (wid == 0) {
        // header and index ends: the container must belong to this table and fit in_nbytes
        // a device table that failed to build, or was built from no values, decodes nothing
        // every load first (at most 200 header dwords: four per lane), then the compares
        constexpr int kHdrPerLane = (kMaxHeaderDwords + 63) / 64;
        const uint32_t hd = index_at / 4;
        uint32_t hv[kHdrPerLane], tv[kHdrPerLane];
#pragma unroll
        for (int r = 0; r < kHdrPerLane; ++r) {
            const uint32_t i = lane + 64 * r, j = i < hd ? i : 0;
            hv[r] = __builtin_amdgcn_raw_buffer_load_b32(rin, (int)(4 * j), 0, 0);
            tv[r] = hdr[j];
        }
        const bool ends_ok = index_ends_ok(rin, index_at, payload_at, n_chunks, in_nbytes);
        bool bad = sg->tab && (sg->tab[kDTStatus] != 0 ||
                               (n > 0 && (sg->tab[kDTN] | sg->tab[kDTN + 1]) == 0));
        // a device table built for other parameters than the launch's
        report(a.h.status, SH_ERR_INVALID_ARG,
               sg->tab && (sg->tab[kDTK] != a.h.K || sg->tab[kDTLog2L] != a.h.R));
#pragma unroll
        for (int r = 0; r < kHdrPerLane; ++r) {
            const uint32_t i = lane + 64 * r;
            if (i < hd) bad |= hv[r] != header_dword_of(tv[r], i, n, n_chunks);
        }
        bad |= !ends_ok;
        report(a.h.status, SH_ERR_CORRUPT_STREAM, bad);
    }

    // the table's entries in the LDS form
    sm[2 * ts] = (te0 & 0xFFFF) | (te1 & 0x00FF0000u) | ((te1 & 0xFF00u) << 16);
    sm[2 * ts + 1] = (te1 & 31) | ((tab_byte + (te0 >> 16)) << 16);
#pragma unroll
    for (int k = 0; k < ILP; ++k) {
        const DecChain& c = ch[k];
        const uint32_t d0 = (4 * li + c.rot) & (kRing - 1), d1 = (kFill + 4 * li + c.rot) & (kRing - 1);
        *reinterpret_cast<v4u*>(&sm[c.ring + d0]) = fill0[k];
        *reinterpret_cast<v4u*>(&sm[c.ring + d1]) = fill1[k];
        if (d0 == 0) sm[c.ring + kRing] = fill0[k][0];
        if (d1 == 0) sm[c.ring + kRing] = fill1[k][0];
    }
    __syncthreads();

    uint32_t nc_min = 0xFFFFFFFFu, nc_max = 0;
#pragma unroll
    for (int k = 0; k < ILP; ++k) {
        DecChain& c = ch[k];
        // initial slots: lane l's R bits at l * R
        c.addr = tab_byte;  // LDS byte address of the current slot's decode entry
        if (li < c.lanes) {
            const uint32_t p = c.bit0 + li * a.h.R;  // below 24 + 32 * 8 bits: no wrap
            const uint32_t bits = __builtin_amdgcn_alignbit(sm[c.ring + (p >> 5) + c.rot + 1],
                                                            sm[c.ring + (p >> 5) + c.rot], p);
            c.addr = tab_byte + ((bits & (a.h.L - 1)) << 3);
        }
        c.pos = c.bit0 + c.lanes * a.h.R + 32 * c.rot;  // ring bit position
        const uint32_t lo = __builtin_amdgcn_readlane(c.nc, 0), hi = __builtin_amdgcn_readlane(c.nc, 32);
        nc_min = nc_min < lo ? nc_min : lo;
        nc_min = nc_min < hi ? nc_min : hi;
        nc_max = nc_max > lo ? nc_max : lo;
        nc_max = nc_max > hi ? nc_max : hi;
    }
    // steps where every lane of the wavefront's chunks decodes a value that is not its
    // lane's last (every lane's last value lies at or after step nc / 32 - 1); the rest,
    // where lanes may be done or at their last value, go through the general step below
    const uint32_t full = (nc_min >> 5) > 0 ? (nc_min >> 5) - 1 : 0;
    const uint32_t steps = (nc_max + 31) >> 5;
    uint64_t bad_offsets = 0;  // lanes that decoded an offset outside its range

    auto refill = [&](DecChain& c) {
        if (c.pos >= c.refill_at) {
            const uint32_t d = (c.res_hi + 4 * li + c.rot) & (kRing - 1);
            *reinterpret_cast<v4u*>(&sm[c.ring + d]) = c.pf;
            if (d == 0) sm[c.ring + kRing] = c.pf[0];
            c.res_hi += kFill;
            c.refill_at = c.res_hi < c.cdw ? (c.res_hi - 33 + c.rot) * 32 : 0xFFFFFFFFu;
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
            const uint32_t o = __builtin_amdgcn_ubfe(bits, 0, e[k][1]);   // the low w_s bits
            // the nb = need - w_s state bits above them
            const uint32_t sb = __builtin_amdgcn_ubfe(bits, e[k][1], e[k][0] - e[k][1]);
            ch[k].addr = (sb << 3) + (e[k][1] >> 16);
            en[k] = *(lds_v2u*)(uintptr_t)ch[k].addr;
            // the sink's own LDS reads must not go out ahead of the chain's entry read
            if constexpr (!Sink::kBytes) __builtin_amdgcn_sched_barrier(0);
            bad_offsets |= __builtin_amdgcn_ballot_w64(o > ((e[k][0] >> 16) & 0xFF));
            if constexpr (Sink::kBytes)
                __builtin_amdgcn_raw_buffer_store_b8((uint8_t)(o + (e[k][0] >> 24)), rout,
                                                     (int)ch[k].vout, (int)(t * 32), 0);
            else
                sink.put(k, o, e[k][0], t);
        }
#pragma unroll
        for (int k = 0; k < ILP; ++k) ch[k].pos += bcast31(incl[k]) & 0xFFFFu;
        if constexpr (!Sink::kBytes) sink.step_done(t);
    };

    v2u e[ILP], e2[ILP];
#pragma unroll
    for (int k = 0; k < ILP; ++k) e[k] = *(lds_v2u*)(uintptr_t)ch[k].addr;
    uint32_t t = 0;
    // the waves on a SIMD take turns at the highest priority (take_turn)
    const uint32_t slot_id = wave_slot();
    const uint32_t full2 = full & ~1u;
    while (t < full2) {
        take_turn(t / kPrioSteps, slot_id);
        const uint32_t stop = full2 - t < kPrioSteps ? full2 : t + kPrioSteps;
        for (; t < stop; t += 2) {  // two steps per trip, so the entries alternate registers
            full_step(e, e2, t);
            full_step(e2, e, t + 1);
#pragma unroll
            for (int k = 0; k < ILP; ++k) refill(ch[k]);
        }
    }
    __builtin_amdgcn_s_setprio(0);
    if (t < full) {
        full_step(e, e2, t);
#pragma unroll
        for (int k = 0; k < ILP; ++k) {
            e[k] = e2[k];
            refill(ch[k]);
        }
        ++t;
    }
    for (; t < steps; ++t) {  // lanes past n_c: no bits; lanes at their last value: no state bits
#pragma unroll
        for (int k = 0; k < ILP; ++k) {
            DecChain& c = ch[k];
            const bool act = t * 32 + li < c.nc;
            v2u ek = e[k];
            if (!act) ek = v2u{0, 0};
            // a lane's last field is its offset alone: the state bits are implied zero, so
            // the field length becomes w (and the state-bit width need - w becomes 0)
            if (act && (t + 1) * 32 + li >= c.nc) ek[0] = (ek[0] & 0xFFFF0000u) | (ek[1] & 31u);
            const uint32_t incl = scan32(ek[0]);
            const uint32_t start = c.pos - ek[0] + incl;
            const uint32_t rb = ((start >> 3) & (4 * kRing - 4)) | c.ring_byte;
            const lds_u32* rp = (const lds_u32*)(uintptr_t)rb;
            const uint32_t bits = __builtin_amdgcn_alignbit(rp[1], rp[0], start);
            const uint32_t o = __builtin_amdgcn_ubfe(bits, 0, ek[1]);
            const uint32_t sb = __builtin_amdgcn_ubfe(bits, ek[1], ek[0] - ek[1]);
            if constexpr (!Sink::kBytes) sink.put_if(k, o, ek[0], t, act);
            if (act) {
                c.err |= o > ((ek[0] >> 16) & 0xFF);
                if constexpr (Sink::kBytes)
                    __builtin_amdgcn_raw_buffer_store_b8((uint8_t)(o + (ek[0] >> 24)), rout,
                                                         (int)c.vout, (int)(t * 32), 0);
                c.addr = (sb << 3) + (ek[1] >> 16);
            }
            c.pos += bcast31(incl) & 0xFFFFu;
            e[k] = *(lds_v2u*)(uintptr_t)c.addr;
            refill(c);
        }
        if constexpr (!Sink::kBytes) sink.step_done(t);
    }
    if constexpr (!Sink::kBytes) sink.finish();

    // a valid chunk leaves every lane in slot 0 and ends in its last size unit, zero-padded
    // (a unit of at most 4 bytes never straddles a dword: chunks start on unit boundaries)
    uint32_t err = 0;
#pragma unroll
    for (int k = 0; k < ILP; ++k) {
        DecChain& c = ch[k];
        err |= c.err;
        if (c.nc > 0) {
            if (li < c.lanes && c.addr != tab_byte) err = 1;
            if (c.pos > c.end || c.end - c.pos >= (8u << ulog)) {
                err = 1;
            } else if (c.pos < c.end) {
                const uint32_t gap = c.end - c.pos;
                const uint32_t pad = sm[c.ring + ((c.pos >> 5) & (kRing - 1))] >> (c.pos & 31);
                if ((gap < 32 ? pad & ((1u << gap) - 1) : pad) != 0) err = 1;
            }
        }
    }
    report(a.h.status, SH_ERR_CORRUPT_STREAM, err != 0 || bad_offsets != 0);
}

// The decode of launches with few chunks (sh_decode, sh_decode_batch): one chunk per
// 32-lane half wavefront twice the wavefronts of the row decoder for the same chunks,
// which is what a launch that cannot fill the GPU needs.  Tables of at most 256 states.
sh_status launch_decode_halves(const CodecArgs& a, uint32_t total_blocks, void* stream) {
    if (total_blocks == 0) return SH_OK;
    if (a.L > (uint32_t)kDecBlock || a.S != kStreamsNarrow) return SH_ERR_UNSUPPORTED;
    with_kernel_args(a, [&](const auto& k) {
        hipLaunchKernelGGL((k_decode<1, Bytes, std::decay_t<decltype(k)>>), dim3(total_blocks),
                           dim3(kDecBlock), 0, (hipStream_t)stream, k);
    });
    return hipGetLastError() == hipSuccess ? SH_OK : SH_ERR_HIP;
}

sh_status launch_decode_matvec(const CodecArgs& a, uint32_t total_blocks, void* stream) {
    if (total_blocks == 0) return SH_OK;
    if (a.nseg == 0) return SH_ERR_INVALID_ARG;  // device tables only
    if (a.S != kStreamsNarrow) return SH_ERR_UNSUPPORTED;
    with_kernel_args(a, [&](const auto& k) {
        using K = std::decay_t<decltype(k)>;
        if constexpr (!std::is_same_v<K, KOne>) {
            if (a.C % a.cols == 0)
                hipLaunchKernelGGL((k_decode<1, MatvecSink<true>, K>), dim3(total_blocks),
                                   dim3(kDecBlock), 0, (hipStream_t)stream, k);
            else
                hipLaunchKernelGGL((k_decode<1, MatvecSink<false>, K>), dim3(total_blocks),
                                   dim3(kDecBlock), 0, (hipStream_t)stream, k);
        }
    });
    return hipGetLastError() == hipSuccess ? SH_OK : SH_ERR_HIP;
}

}  // namespace shn
