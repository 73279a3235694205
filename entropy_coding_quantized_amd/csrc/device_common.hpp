// Device helpers shared by the HIP kernels of the Shannonic codec (gfx950, wave64).
#pragma once

#include <hip/hip_runtime.h>

#include <cstring>

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

// Inclusive prefix sum over the whole wavefront: scan32, then lane 31 added into rows 2
// and 3 (DPP row_bcast:31).
__device__ __forceinline__ uint32_t scan64(uint32_t v) {
    v = scan32(v);
    v += (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x143, 0xC, 0xF, false); // row_bcast:31
    return v;
}

// Value of lane 31 of this lane's 32-lane half (ds_swizzle bit mode, or_mask = 31).
__device__ __forceinline__ uint32_t bcast31(uint32_t v) {
    return (uint32_t)__builtin_amdgcn_ds_swizzle((int)v, 0x3E0);
}

// The same in VALU only: DPP row_newbcast:15 gives every row its own lane 15, then
// v_permlane16_swap moves rows 1 and 3 into rows 0 and 2.
__device__ __forceinline__ uint32_t bcast31_valu(uint32_t v) {
    const uint32_t r = (uint32_t)__builtin_amdgcn_mov_dpp((int)v, 0x15F, 0xF, 0xF, true);
    return __builtin_amdgcn_permlane16_swap(r, r, false, false)[1];
}

typedef const __attribute__((address_space(3))) uint32_t lds_u32;

// LDS byte offset of a __shared__ object
__device__ __forceinline__ uint32_t lds_offset(const void* p) {
    return (uint32_t)(uintptr_t)(const __attribute__((address_space(3))) void*)p;
}

// Workgroup barrier that orders LDS accesses only: global stores issued before it may still
// be in flight (__syncthreads would wait for them).
__device__ __forceinline__ void lds_barrier() {
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup", "local");
    __builtin_amdgcn_s_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup", "local");
}

// Waves that share a SIMD are issued oldest first, which over hundreds of dependent steps
// lets the oldest wave finish far ahead of the youngest while the launch waits for the
// youngest.  Kernels with long step loops let their waves take turns at the highest
// priority: in period p a wave's priority is set from (p + its slot on the SIMD) mod 4.
// Eight steps a turn measured slightly faster than 16 on launches of four wavefronts a SIMD
// (about 1.5% on a 134 M-value tensor's decode and encode) and the same on large launches.
constexpr uint32_t kPrioSteps = 8;  // steps per period (even, a multiple of the decode tile)
__device__ __forceinline__ uint32_t wave_slot() {
    return __builtin_amdgcn_s_getreg((3 << 11) | (0 << 6) | 4);  // HW_ID bits 0..3
}
__device__ __forceinline__ void take_turn(uint32_t period, uint32_t slot) {
    const uint32_t turn = (period + slot) & 3;
    if (turn == 0) __builtin_amdgcn_s_setprio(3);
    else if (turn == 1) __builtin_amdgcn_s_setprio(2);
    else if (turn == 2) __builtin_amdgcn_s_setprio(1);
    else __builtin_amdgcn_s_setprio(0);
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
__device__ __forceinline__ uint32_t find_seg_index(const SegDesc* segs, uint32_t nseg,
                                                    uint32_t block, bool compaction) {
    uint32_t lo = 0, hi = nseg;  // the last segment whose first block <= block
    while (hi - lo > 1) {
        const uint32_t mid = (lo + hi) >> 1;
        const uint32_t fb = compaction ? segs[mid].first_block_c : segs[mid].first_block;
        if (fb <= block) lo = mid;
        else hi = mid;
    }
    return lo;
}
__device__ __forceinline__ const SegDesc* find_seg(const SegDesc* segs, uint32_t nseg,
                                                    uint32_t block, bool compaction) {
    return &segs[find_seg_index(segs, nseg, block, compaction)];
}
template <class A>
__device__ __forceinline__ const SegDesc* codec_seg(const A& a, uint32_t block, bool compaction) {
    return find_seg(a.segs, a.h.nseg, block, compaction);
}

// the tables carried in the arguments (KOne), or none (KSegs: every segment has a device
// table); which a segment uses is decided by its tab pointer
__device__ __forceinline__ const uint32_t* inline_tab(const KOne& a) { return a.tab; }
__device__ __forceinline__ const uint32_t* inline_hdr(const KOne& a) { return a.hdr; }
__device__ __forceinline__ const uint16_t* inline_es(const KOne& a) { return a.es; }
template <int N>
__device__ __forceinline__ const uint32_t* inline_tab(const KSegs<N>&) { return nullptr; }
template <int N>
__device__ __forceinline__ const uint32_t* inline_hdr(const KSegs<N>&) { return nullptr; }
template <int N>
__device__ __forceinline__ const uint16_t* inline_es(const KSegs<N>&) { return nullptr; }

// ---- host side: the smallest argument block for a launch ----
inline KHead kernel_head(const CodecArgs& a) {
    return KHead{a.nseg ? a.nseg : 1, a.C, a.R, a.L, a.K, a.S, {a.slot_dwords}, a.status, a.slots,
                 a.meta, a.agg};
}
inline KOne kernel_one(const CodecArgs& a) {
    KOne k;
    k.h = kernel_head(a);
    k.segs[0] = a.one.seg;
    std::memcpy(k.hdr, a.one.hdr, sizeof(k.hdr));
    std::memcpy(k.tab, a.one.tab, sizeof(k.tab));
    std::memcpy(k.es, a.one.es, sizeof(k.es));
    return k;
}
template <int N>
inline KSegs<N> kernel_segs(const CodecArgs& a) {
    KSegs<N> k;
    k.h = kernel_head(a);
    std::memcpy(k.segs, a.many, sizeof(SegDesc) * a.nseg);
    return k;
}
// Calls f(args) with the smallest argument block that holds a.
template <class F>
inline void with_kernel_args(const CodecArgs& a, F&& f) {
    if (a.nseg == 0) f(kernel_one(a));
    else if (a.nseg <= 1) f(kernel_segs<1>(a));
    else if (a.nseg <= 4) f(kernel_segs<4>(a));
    else if (a.nseg <= 16) f(kernel_segs<16>(a));
    else f(kernel_segs<kMaxInlineSegs>(a));
}
template <int N>
inline HistArgsN<N> hist_args(const HistArgs& h) {
    HistArgsN<N> k;
    k.nseg = h.nseg;
    k.n_blocks = h.n_blocks;
    k.block_bytes = h.block_bytes;
    k.hist = h.hist;
    std::memcpy(k.segs, h.segs, sizeof(SegDesc) * h.nseg);
    return k;
}

__device__ __forceinline__ uint32_t header_bytes_dev(uint32_t K) {
    return (kHeaderFixed + 3 * K - 1 + 3) / 4 * 4;
}

// Where the chunks of one group of kGroupChunks (64) lie in a container (the chunk index of
// version 3): lane i of the wavefront gets chunk 64 g + i's first byte after the group's
// first chunk (rel) and its size in bytes (0 past the last chunk); head is the group's
// offset from the payload start.  ok: the next group's offset (the payload's size after the
// last group) is this one's plus the sizes of its chunks.  Every lane takes part.
struct GroupSpans {
    uint32_t head, rel, bytes;
    bool ok;
};
__device__ __forceinline__ GroupSpans group_spans(rsrc_t rin, uint32_t index_at, uint32_t n_chunks,
                                                  uint32_t g, uint32_t unit_log2) {
    const uint32_t lane = __builtin_amdgcn_mbcnt_hi(~0u, __builtin_amdgcn_mbcnt_lo(~0u, 0u));
    const uint32_t c = g * kGroupChunks + lane;
    const uint32_t sizes_at = index_at + sizes_rel_of(n_chunks);
    const uint32_t units = c < n_chunks
        ? (uint32_t)__builtin_amdgcn_raw_buffer_load_b16(rin, (int)(sizes_at + 2 * c), 0, 0) : 0u;
    const uint32_t head = __builtin_amdgcn_raw_buffer_load_b32(rin, (int)(index_at + 4 * g), 0, 0);
    const uint32_t next = __builtin_amdgcn_raw_buffer_load_b32(rin, (int)(index_at + 4 * g + 4), 0, 0);
    const uint32_t incl = scan64(units);  // at most 64 * 65535 units
    const uint32_t total = __builtin_amdgcn_readlane(incl, 63);
    GroupSpans s;
    s.head = head;
    s.rel = (incl - units) << unit_log2;
    s.bytes = units << unit_log2;
    s.ok = (uint64_t)head + ((uint64_t)total << unit_log2) == next;
    return s;
}

// The lane's value taken from lane src of the wavefront (ds_bpermute).
__device__ __forceinline__ uint32_t lane_value(uint32_t v, uint32_t src) {
    return (uint32_t)__builtin_amdgcn_ds_bpermute((int)(src << 2), (int)v);
}

// Checks of a version-3 index that no single chunk makes: the first group starts at 0, the
// payload ends within in_nbytes and is padded with zero bytes to 4, and an odd number of
// sizes is followed by a zero u16.  True when all hold.  Every lane takes part.
__device__ __forceinline__ bool index_ends_ok(rsrc_t rin, uint32_t index_at, uint32_t payload_at,
                                              uint32_t n_chunks, uint64_t in_nbytes) {
    const uint32_t first = __builtin_amdgcn_raw_buffer_load_b32(rin, (int)index_at, 0, 0);
    const uint32_t pay = __builtin_amdgcn_raw_buffer_load_b32(
        rin, (int)(index_at + 4 * n_groups_of(n_chunks)), 0, 0);
    const uint64_t end = (uint64_t)payload_at + ((uint64_t)pay + 3) / 4 * 4;
    bool ok = first == 0 && end <= in_nbytes;
    if (ok && (pay & 3)) {  // the pad bytes after the payload's last byte
        const uint32_t w = __builtin_amdgcn_raw_buffer_load_b32(
            rin, (int)(payload_at + (pay & ~3u)), 0, 0);
        ok = (w >> (8 * (pay & 3))) == 0;
    }
    if (n_chunks & 1) {
        const uint32_t pad = __builtin_amdgcn_raw_buffer_load_b16(
            rin, (int)(index_at + sizes_rel_of(n_chunks) + 2 * n_chunks), 0, 0);
        ok = ok && pad == 0;
    }
    return ok;
}

}  // namespace shn
