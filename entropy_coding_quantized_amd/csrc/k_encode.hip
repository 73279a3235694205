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
// tANS encodes backwards.  Each lane walks its values from the last step to the first;
// at every step the 32 fields of a chunk are placed right to left: the step's fields end
// where the later steps' fields begin, so a 32-lane prefix sum of the lengths gives every
// field's bit position.  Fields are OR-ed into a 256-dword LDS ring that is flushed to
// the chunk's slot 128 dwords at a time, highest first; the chunk ends up right-aligned
// in its slot with the lanes' final states (the decoder's initial states) in front.
constexpr int kEncBlock = 256;
constexpr uint32_t kChunksPerBlockE = kEncBlock / 64 * 2;  // two chunks a wavefront
constexpr uint32_t kERing = 256;
// LDS (dynamic, sized by L; the kernel's only LDS, so it starts at LDS byte 0): eight 1 KB
// rings (one per half wavefront, 1 KB aligned), eight 1 KB input tiles (bytes of 32 steps x
// 32 lanes), the value table (512 dwords), the encTable slots (u16, L of them), then the
// block's two totals
constexpr uint32_t kTileBase = 8 * kERing;
constexpr uint32_t kVtBase = kTileBase + 8 * 256;
constexpr uint32_t kEsBase = kVtBase + 512;
__host__ __device__ constexpr uint32_t encode_lds_dwords(uint32_t L) { return kEsBase + (L + 1) / 2 + 2; }

// OR a field (zero above its length) into a ring at bit pos; ring_byte is the ring's LDS
// byte offset, a multiple of its 1 KB size.  The second dword is OR-ed only by the lanes
// whose field reaches into it: the 32 fields of a step share a few dwords, and same-address
// LDS atomics serialise.
__device__ __forceinline__ void ring_or(uint32_t* sm, uint32_t ring_byte, uint32_t pos,
                                        uint32_t field) {
    typedef __attribute__((address_space(3))) uint32_t lds_word;
    const uint64_t wide = (uint64_t)field << (pos & 31);
    const uint32_t b = pos >> 3;
    const uint32_t a0 = (b & 0x3FC) | ring_byte, a1 = ((b + 4) & 0x3FC) | ring_byte;
    (void)sm;  // the rings sit at LDS byte 0 of the block's only __shared__ array
    __hip_atomic_fetch_or((lds_word*)(uintptr_t)a0, (uint32_t)wide, __ATOMIC_RELAXED,
                          __HIP_MEMORY_SCOPE_WORKGROUP);
    if ((uint32_t)(wide >> 32))
        __hip_atomic_fetch_or((lds_word*)(uintptr_t)a1, (uint32_t)(wide >> 32), __ATOMIC_RELAXED,
                              __HIP_MEMORY_SCOPE_WORKGROUP);
}

// container bytes of a chunk of the given bits: whole size units of 2^ulog bytes
__device__ __forceinline__ uint32_t chunk_bytes_of(uint32_t bits, uint32_t ulog) {
    return ((bits + (8u << ulog) - 1) >> (3 + ulog)) << ulog;
}

template <class A>
__global__ __launch_bounds__(kEncBlock) void k_encode_chunks(const A a) {
    extern __shared__ __align__(16) uint32_t sm[];
    const uint32_t tid = threadIdx.x, lane = tid & 63, li = lane & 31, hw = lane >> 5;
    const uint32_t block = __builtin_amdgcn_readfirstlane(blockIdx.x);
    const SegDesc* sg = codec_seg(a, block, false);
    const uint32_t bseg = block - sg->first_block;
    const uint32_t wid = __builtin_amdgcn_readfirstlane(bseg * (kEncBlock / 64) + (tid >> 6));
    const uint32_t wv = wid & (kEncBlock / 64 - 1);
    const uint32_t* vt = sg->tab ? sg->tab + kDTVt : inline_tab(a);
    const uint16_t* es_src = sg->tab ? reinterpret_cast<const uint16_t*>(sg->tab + kDTEs)
                                    : inline_es(a);
    const uint32_t n_chunks = sg->n_chunks;
    const uint64_t n = sg->n;
    const uint32_t L = a.h.L, R1 = a.h.R + 1;
    uint32_t* agg_s = &sm[kEsBase + (L + 1) / 2];  // the block's container bytes and field bits
    for (uint32_t i = tid; i < 512; i += kEncBlock) sm[kVtBase + i] = vt[i];
    for (uint32_t i = tid; 2 * i < L; i += kEncBlock)
        sm[kEsBase + i] = (uint32_t)es_src[2 * i] | ((uint32_t)es_src[2 * i + 1] << 16);
    const uint16_t* es = reinterpret_cast<const uint16_t*>(&sm[kEsBase]);
    const uint32_t hi = wv * 2 + hw;       // this half wavefront's ring and tile
    const uint32_t tile = kTileBase + hi * 256;
    const uint32_t ring = hi * kERing;
    const uint32_t ring_byte = lds_offset(sm) + 4 * ring;  // 1 KB aligned
    for (uint32_t i = li; i < kERing; i += 32) sm[ring + i] = 0;

    const uint32_t pair = 2 * wid;
    const uint32_t chunk = pair + hw;
    const uint64_t pair_first = (uint64_t)pair * a.h.C;
    const uint64_t pair_len = pair_first < n ? n - pair_first : 0;
    const rsrc_t rin = make_rsrc(sg->x + (pair_first < n ? pair_first : 0),
                                 (uint32_t)(pair_len < 2ull * a.h.C ? pair_len : 2ull * a.h.C));
    const uint32_t slot0 = sg->slot_base + (pair < n_chunks ? pair : 0);
    const rsrc_t rslot = make_rsrc(a.h.slots + (uint64_t)slot0 * a.h.slot_dwords, 8u * a.h.slot_dwords);
    const uint32_t in_base = hw * a.h.C;          // byte offset of this chunk in rin
    const uint32_t slot_base = hw * a.h.slot_dwords * 4;
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
    const uint32_t lanes = nc < 32 ? nc : 32;
    const uint32_t nc_lo = __builtin_amdgcn_readlane(nc, 0), nc_hi = __builtin_amdgcn_readlane(nc, 32);
    const uint32_t steps = ((nc_lo > nc_hi ? nc_lo : nc_hi) + 31) >> 5;

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
    if (tid < 2) agg_s[tid] = 0;
    __syncthreads();

    uint32_t X = L;
    uint32_t P = a.h.slot_dwords * 32;   // fields go below P, right to left
    uint32_t fmark = a.h.slot_dwords;    // dwords at or above fmark are in the slot
    uint32_t flush_at = (fmark - 128) * 32;  // once P is below this, flush a block
    // every encode entry is OR-ed in; its bit 15 marks a value in a range without states
    uint32_t bad = 0;

    auto flush_block = [&](uint32_t blk) {  // ring dwords [blk, blk + 128) -> slot
        uint32_t* r = &sm[ring + ((blk + 4 * li) & (kERing - 1))];
        const v4u v = *reinterpret_cast<v4u*>(r);
        *reinterpret_cast<v4u*>(r) = v4u{0, 0, 0, 0};
        __builtin_amdgcn_raw_buffer_store_b128(v, rslot, (int)(slot_base + 4 * (blk + 4 * li)), 0, 0);
    };

    // Values are read two steps ahead and table entries one step ahead, so the only LDS
    // read on the chain from one step to the next is the state-dependent encTable read,
    // and no read waits for the previous step's ring writes.
    auto stage = [&]() {  // the tile in p0/p1 into LDS, as u = x + 128
        const v4u flip = {0x80808080u, 0x80808080u, 0x80808080u, 0x80808080u};
        *reinterpret_cast<v4u*>(&sm[tile + 8 * li]) = p0 ^ flip;
        *reinterpret_cast<v4u*>(&sm[tile + 8 * li + 4]) = p1 ^ flip;
    };
    auto value_at = [&](uint32_t t) {  // u of step t, from the staged tile t >> 5
        return (uint32_t)reinterpret_cast<const uint8_t*>(&sm[tile])[(t & 31) * 32 + li];
    };
    auto entry = [&](uint32_t u) {  // encode entry of value u
        return *reinterpret_cast<const uint2*>(&sm[kVtBase + 2 * u]);
    };
    // step t2's value, staging its tile first when t2 is the first step of a tile; the tile it
    // replaces is no longer read (the values of later steps are in registers)
    auto fetch = [&](uint32_t t2) {
        if ((t2 & 31) == 31) {
            stage();
            if (t2 >= 32) load_tile((t2 >> 5) - 1, p0, p1);
        }
        return value_at(t2);
    };
    uint2 e_c = {0, 0};
    uint32_t u_n = 0;
    if (steps > 0) {
        stage();
        if (steps - 1 >= 32) load_tile(((steps - 1) >> 5) - 1, p0, p1);
        const uint32_t u_c = value_at(steps - 1);
        if (steps >= 2) u_n = fetch(steps - 2);
        e_c = entry(u_c);
    }
    // A step's fields are placed one step late, so that the state update of step t, whose
    // encTable read is in flight, overlaps the placement of step t + 1's fields.
    uint32_t len_p = 0, field_p = 0;  // nothing to place before the first step
    auto place = [&]() {  // the carried fields, right to left below P
        const uint32_t incl = scan32(len_p);
        P -= bcast31_valu(incl);
        ring_or(sm, ring_byte, P + incl - len_p, field_p);
    };
    // Checked every other step: P then falls at most 48 dwords past flush_at before the
    // flush (two steps and the final placement), and the ring keeps 256.
    auto flush_due = [&]() {
        if (P < flush_at) {  // dwords from P's word + 129 up are final
            fmark -= 128;
            flush_at -= 128 * 32;
            flush_block(fmark);
        }
    };
    // may_stage: false for a step whose t is known even (t - 2 is then never a tile's first
    // step, and for t = 0 the value read is a harmless, unused byte of the tile)
    auto step = [&](uint32_t t, auto partial, auto may_stage) {
        uint32_t u_nn;
        if constexpr (decltype(may_stage)::value) u_nn = t >= 2 ? fetch(t - 2) : 0u;
        else u_nn = value_at(t - 2);
        const uint2 e_n = entry(u_n);
        const uint32_t k = (uint32_t)((int)X + (int)e_c.x) >> R1;
        const uint32_t sx = es[(e_c.y >> 16) - kMaxLGpu + (X >> k)];
        const uint32_t w = (e_c.y >> 8) & 15;
        uint32_t field = (e_c.y & 0xFF) | (__builtin_amdgcn_ubfe(X, 0, k) << w);
        uint32_t len = w + k;
        uint32_t flag = e_c.y;
        if constexpr (decltype(partial)::value) {
            const bool act = t * 32 + li < nc;
            // a lane's last value, the first it encodes (from X = L): its k state bits
            // are zero and are left out
            const bool last = (t + 1) * 32 + li >= nc;
            field = act ? field : 0u;
            len = act ? (last ? w : len) : 0u;
            flag = act ? flag : 0u;
        }
        bad |= flag;
        place();
        if constexpr (decltype(partial)::value) {
            X = t * 32 + li < nc ? L + sx : X;
        } else {
            X = L + sx;
        }
        len_p = len;
        field_p = field;
        e_c = e_n;
        u_n = u_nn;
    };
    // steps where a lane of either half has no value (the tail of a short chunk) or has its
    // last value first: every lane's last value lies at or after step nc / 32 - 1
    uint32_t t_full = (nc_lo < nc_hi ? nc_lo : nc_hi) >> 5;
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
        while (t > stop) {  // two steps per iteration: the carried values need no copies
            step(--t, std::false_type{}, std::true_type{});   // odd t
            step(--t, std::false_type{}, std::false_type{});  // even t
            flush_due();
        }
    }
    place();  // the first step's fields
    __builtin_amdgcn_s_setprio(0);
    const uint32_t pay = a.h.slot_dwords * 32 - P;  // field bits
    // the lanes' final states, the decoder's initial states, in front of the fields.  A
    // valid encode never exceeds the chunk's bound; the span recorded for the placement is
    // clamped to it all the same, so that no table, however corrupt, moves the placement
    // outside the container's bound
    uint32_t Pi = P - lanes * a.h.R;
    {
        const uint32_t top = a.h.slot_dwords * 32, most = (uint32_t)chunk_bound_bits(nc, a.h.R);
        if (Pi > top || top - Pi > most) Pi = top - most;
    }
    ring_or(sm, ring_byte, Pi + li * a.h.R, li < lanes ? X - L : 0u);
    if (nc > 0) {
        while (fmark > (Pi >> 5)) {
            fmark -= 128;
            flush_block(fmark);
        }
    }
    if (chunk < n_chunks && li == 0) {
        a.h.meta[2 * (sg->slot_base + chunk)] = Pi;
        a.h.meta[2 * (sg->slot_base + chunk) + 1] = pay;
        atomicAdd(&agg_s[0], chunk_bytes_of(a.h.slot_dwords * 32 - Pi, size_unit_log2(a.h.C, a.h.R)));
        atomicAdd(&agg_s[1], pay);
    }
    __syncthreads();
    if (tid < 2) a.h.agg[2 * block + tid] = agg_s[tid];
    bad &= 0x8000u;
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
    for (uint32_t q = q0 + lane; q < q1; q += 64) cw[q] = bits32(start + 8 * (4 * q - d0));
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
    const uint32_t ulog = size_unit_log2(a.h.C, a.h.R);
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
    const uint32_t bytes = chunk_bytes_of(a.h.slot_dwords * 32 - start, size_unit_log2(a.h.C, a.h.R));
    // the last chunk also writes the zero bytes that end the payload on 4 bytes
    const uint32_t end = c + 1 == sg->n_chunks ? (off + bytes + 3) / 4 * 4 : off + bytes;
    move_chunk(a.h.slots + (uint64_t)slot * a.h.slot_dwords, a.h.slot_dwords, start, sg->c,
               payload_at + off, payload_at + end, lane);
}

// ------------------------------------------------------------------------------------
// encode, kernels 2 and 3 in one (segments of at most kPlaceMaxChunks chunks): every block
// finds the offset of its first chunk from the chunk kernel's per-block aggregates (the
// container bytes of 8 chunks each) and the sizes of at most 4 chunks after the last whole
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
    const uint32_t ulog = size_unit_log2(a.h.C, a.h.R);
    const uint32_t* meta = a.h.meta + 2ull * sg->slot_base;
    const uint32_t* agg = a.h.agg + 2ull * sg->first_block;  // the segment's chunk-kernel blocks
    uint32_t* goff = reinterpret_cast<uint32_t*>(sg->c + index_at);
    uint16_t* sizes = reinterpret_cast<uint16_t*>(sg->c + index_at + sizes_rel_of(n_chunks));
    const bool last = c0 + 4 >= n_chunks;
    auto chunk_bytes = [&](uint32_t ch) {
        return chunk_bytes_of(a.h.slot_dwords * 32 - meta[2 * ch], ulog);
    };

    // bytes of the chunk-kernel blocks before c0 (c0 / 8 of them); in the last block also
    // the field bits of all of them
    const uint32_t nb_before = c0 / kChunksPerBlockE;
    const uint32_t nb_all = (n_chunks + kChunksPerBlockE - 1) / kChunksPerBlockE;
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
    // then the chunks from the last whole aggregate up to this wavefront's chunk
    const uint32_t c = c0 + wv;
    for (uint32_t j = nb_before * kChunksPerBlockE; j < c && j < n_chunks; ++j) off += chunk_bytes(j);

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

sh_status launch_encode(const CodecArgs& a, uint32_t total_blocks, uint32_t total_blocks_c,
                        bool place, void* stream) {
    hipStream_t s = (hipStream_t)stream;
    with_kernel_args(a, [&](const auto& k) {
        using K = std::decay_t<decltype(k)>;
        if (total_blocks > 0)
            hipLaunchKernelGGL(k_encode_chunks<K>, dim3(total_blocks), dim3(kEncBlock),
                               4 * encode_lds_dwords(a.L), s, k);
        if (place) {
            hipLaunchKernelGGL(k_encode_place<K>, dim3(total_blocks_c), dim3(256), 0, s, k);
            return;
        }
        hipLaunchKernelGGL(k_encode_index<K>, dim3(k.h.nseg), dim3(kScanBlock), 0, s, k);
        if (total_blocks_c > 0)
            hipLaunchKernelGGL(k_encode_compact<K>, dim3(total_blocks_c), dim3(256), 0, s, k);
    });
    return hipGetLastError() == hipSuccess ? SH_OK : SH_ERR_HIP;
}

}  // namespace shn
