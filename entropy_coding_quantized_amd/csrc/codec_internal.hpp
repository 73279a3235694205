// Internal declarations shared by the host table builder, the HIP kernels and the C ABI
// of libshannonic.so.  Nothing here is exported.
#pragma once

#include <cstddef>
#include <cstdint>
#include <vector>

#include "../../include/shannonic.h"

#if defined(__HIP__)
#define SHN_HD __host__ __device__
#else
#define SHN_HD
#endif

namespace shn {

constexpr int kLgFrac = 24;            // fractional bits of the DP's fixed-point log2
// interleaved tANS streams per chunk on the GPU path: 32 (two a lane of a 16-lane row, or
// one a lane of a half wavefront), 64 (four a lane of a 16-lane row, or two a lane of a half
// wavefront) or 128 (four a lane of a half wavefront to decode, eight a lane of a 16-lane
// row to encode)
constexpr uint32_t kStreamsNarrow = 32, kStreamsWide = 64, kStreamsWidest = 128;
constexpr int kMaxLog2LHost = 12;      // host table build
// GPU path: L up to 2048 states (standard tANS sizes), tables held in LDS; the decoder
// takes two adjacent fields in one 32-bit window, so a table is usable on the GPU only when
// its longest field, the widest range's offset bits plus log2 L state bits, is at most 16
// bits (always at log2 L <= 8, and for K = 256, where every range is one value)
constexpr int kMaxLog2LGpu = 11;
constexpr uint32_t kMaxLGpu = 1u << kMaxLog2LGpu;
constexpr int kInlineMaxLog2L = 8;     // single-tensor calls carry their tables inline
constexpr uint32_t kMaxFieldBitsGpu = 16;
constexpr uint32_t kMaxChunk = 65536;  // GPU path
constexpr uint32_t kHeaderFixed = 32;  // bytes of the fixed part of the container header
constexpr uint32_t kMaxHeaderDwords = (kHeaderFixed + 3 * 256 - 1 + 3) / 4;  // 200

// ---- host table build (host_tables.cpp) --------------------------------------------
uint64_t fixed_log2(uint64_t x);
sh_status table_from_histogram(const uint64_t* hist, uint32_t K, uint32_t log2_L, sh_table* out);
sh_status check_table(const sh_table& t, bool allow_empty);

// Everything the kernels need, derived from a canonical table.
struct SlotTables {
    uint32_t L = 0;
    uint16_t range[4096];     // slot -> range
    uint8_t nb[4096];         // slot -> state bits read after it
    uint16_t next[4096];      // slot -> base of the next slot
    uint16_t enc[4096];       // cum_s + j -> slot of range s's j-th occurrence
    uint32_t cum[257];        // cum_s = f_0 + ... + f_{s-1}
};
sh_status derive_slots(const sh_table& t, SlotTables* out);

inline uint32_t ceil_log2_u32(uint32_t m) {
    uint32_t w = 0;
    while ((1u << w) < m) w++;
    return w;
}
inline uint32_t floor_log2_u32(uint32_t x) {
    uint32_t e = 0;
    while (x >> (e + 1)) e++;
    return e;
}

// ---- container geometry (version 3) ---------------------------------------------------
// Chunks follow each other byte by byte, each padded to a whole number of size units of
// 2^u bytes, u the smallest that lets the size of the largest chunk a valid stream holds
// fit 16 bits (u = 0 for C up to 34,937 at log2 L = 7; at most 2 on the GPU path).
// The index after the header: u32 goff[G + 1], G = ceil(n_chunks / 64) (the payload byte
// of chunk 64g; goff[G] = the payload's size), then u16 size[n_chunks] in units, then a
// zero u16 when n_chunks is odd.  The payload ends with zero bytes up to a multiple of 4.
constexpr uint32_t kGroupChunks = 64;
inline uint32_t header_bytes(uint32_t K) { return (kHeaderFixed + 3 * K - 1 + 3) / 4 * 4; }
inline uint64_t n_chunks_of(uint64_t n, uint32_t C) { return (n + C - 1) / C; }
// bits of the largest chunk of nc values a valid stream of S streams holds: the initial
// states and every field at 8 + R bits
SHN_HD inline uint64_t chunk_bound_bits(uint32_t nc, uint32_t R, uint32_t S) {
    const uint64_t lanes = nc < S ? nc : S;
    return lanes * R + (uint64_t)nc * (8 + R);
}
// ... in 32-bit words (the encoder's per-chunk workspace slots)
SHN_HD inline uint32_t chunk_bound_dwords(uint32_t nc, uint32_t R, uint32_t S) {
    return (uint32_t)((chunk_bound_bits(nc, R, S) + 31) / 32);
}
SHN_HD inline uint32_t size_unit_log2(uint32_t C, uint32_t R, uint32_t S) {
    const uint64_t most = (chunk_bound_bits(C, R, S) + 7) / 8;
    uint32_t u = 0;
    while (((most + (1ull << u) - 1) >> u) > 0xFFFFull) ++u;
    return u;
}
SHN_HD inline uint32_t chunk_bound_units(uint32_t nc, uint32_t R, uint32_t u, uint32_t S) {
    return (uint32_t)((chunk_bound_bits(nc, R, S) + (8ull << u) - 1) >> (3 + u));
}
SHN_HD inline uint32_t n_groups_of(uint32_t nch) { return (nch + kGroupChunks - 1) / kGroupChunks; }
// bytes of the index, and where its sizes start (relative to index_at)
SHN_HD inline uint64_t index_bytes_of(uint64_t nch) {
    return 4 * ((nch + kGroupChunks - 1) / kGroupChunks + 1) + (2 * nch + 3) / 4 * 4;
}
SHN_HD inline uint32_t sizes_rel_of(uint32_t nch) { return 4 * (n_groups_of(nch) + 1); }
void write_header(const sh_table& t, uint64_t n, uint32_t C, uint32_t S, uint64_t n_chunks,
                  uint32_t* dwords /* kMaxHeaderDwords */);

// ---- device-resident table --------------------------------------------------------------
// Everything the kernels need for one tensor, in device memory (dword offsets below).
// Written by the GPU table builder or uploaded from a host sh_table.
constexpr uint32_t kDTK = 0, kDTLog2L = 1, kDTL = 2, kDTStatus = 3, kDTN = 4 /* u64 */;
constexpr uint32_t kDTHdrDwords = 6;
constexpr uint32_t kDTHdr = 8;        // 200 dwords: container header with n = n_chunks = 0
constexpr uint32_t kDTLo = 208;       // 129 dwords: lo[257] as u16
constexpr uint32_t kDTFreq = 337;     // 128 dwords: freq[256] as u16
constexpr uint32_t kDTHist = 466;     // 512 dwords: hist[256] as u64 (8-byte aligned)
constexpr uint32_t kDTVt = 978;       // 512 dwords: encode entries, two per value
constexpr uint32_t kDTDec = 1490;     // 2 * kMaxLGpu dwords: decode entries, two per slot
constexpr uint32_t kDTEs = 5586;      // kMaxLGpu / 2 dwords: encode slots as u16
constexpr uint32_t kDTDwords = 6612;  // 26,448 bytes (16-byte multiple)
constexpr uint32_t kDTBytes = 4 * kDTDwords;

// header dwords that depend on the segment, not on the table: n (2, 3) and n_chunks (6)
// (template dword ti already read)
SHN_HD inline uint32_t header_dword_of(uint32_t ti, uint32_t i, uint64_t n, uint32_t nch) {
    return i == 2 ? (uint32_t)n : i == 3 ? (uint32_t)(n >> 32) : i == 6 ? nch : ti;
}
SHN_HD inline uint32_t header_dword(const uint32_t* tmpl, uint32_t i, uint64_t n, uint32_t nch) {
    return header_dword_of(tmpl[i], i, n, nch);
}

// Decode entry of a slot (kernel-argument / device-table form), two dwords:
//   e0 = need | (next slot * 8) << 16, need = w_s + nb <= 16
//   e1 = w_s | (int8 bits of the range base) << 8 | (|range| - 1) << 16
// Encode entry of a value u, two dwords:
//   v0 = bias_s (int32): the state-bit count is (X + bias_s) >> (R + 1)
//   v1 = o | w_s << 8 | (f_s == 0) << 15 | (start_s + kMaxLGpu) << 16, start_s = cum_s - f_s
void derive_kernel_tables(const sh_table& t, const SlotTables& st, uint32_t* dec,
                          uint32_t* vt, uint16_t* es);
// the longest field (offset bits of the widest range plus log2 L) of a table, in bits
uint32_t max_field_bits(const sh_table& t);
// st is null for a table built from no values
void make_device_table(const sh_table& t, const SlotTables* st, uint32_t C, uint32_t S,
                       uint32_t* dt /* kDTDwords */);

// ---- kernel arguments (kernels.hip) ------------------------------------------------------
// One tensor of a launch.
struct SegDesc {
    uint8_t* x;             // int8 values: encode input, decode output
    uint8_t* c;             // container: encode output, decode input
    uint64_t n;             // values
    uint64_t c_bytes;       // decode: readable bytes at c
    const uint32_t* tab;    // device table, or null: the tables inside CodecArgs
    union {
        sh_encode_info* info;   // encode: where to report (may be null)
        const int8_t* vec;      // decode into a matrix-vector product: the vector
    };
    uint32_t first_block;   // this segment's first block in the chunk kernels
    uint32_t first_block_c; // ... and in the compaction kernel
    uint32_t n_chunks;
    uint32_t slot_base;     // encode: first workspace slot
};

constexpr uint32_t kMaxInlineSegs = 48;  // descriptors carried in one launch's arguments

// A launch as the C ABI describes it (host side).  The launch functions pass the kernels
// the smallest argument block that holds it (KOne or KSegs<N> below): the cost of a
// launch on the host grows with the size of its arguments.
struct CodecArgs {
    uint32_t nseg;          // 0: a single segment with host-built tables (one), else many
    uint32_t C, R, L, K, S;
    union {
        uint32_t slot_dwords;   // encode: dwords per slot, a multiple of 128
        uint32_t cols;          // decode into a matrix-vector product: values per row
    };
    int32_t* status;
    uint32_t* slots;        // encode workspace
    uint32_t* meta;         // encode workspace: per slot {start bit, field bits}
    uint32_t* agg;          // encode workspace: per chunk-kernel block {bytes, field bits}
    union {
        struct {
            SegDesc seg;
            uint32_t hdr[kMaxHeaderDwords];
            uint32_t tab[2 * 256];  // decode entries (decode) or value entries (encode)
            uint16_t es[256];       // encode slots
        } one;
        SegDesc many[kMaxInlineSegs];  // each with a device table
    };
};

// ---- kernel argument blocks ----
struct KHead {
    uint32_t nseg, C, R, L, K, S;
    union {
        uint32_t slot_dwords;
        uint32_t cols;
    };
    int32_t* status;
    uint32_t* slots;
    uint32_t* meta;
    uint32_t* agg;
};
template <int N>
struct KSegs {  // N segments with device tables
    KHead h;
    SegDesc segs[N];
};
struct KOne {  // one segment with the tables in the arguments
    KHead h;
    SegDesc segs[1];
    uint32_t hdr[kMaxHeaderDwords];
    uint32_t tab[2 * 256];
    uint16_t es[256];
};

// values per histogram block: a power of two from 16 KB to 1 MB, so that a launch has about
// 512 blocks when it can.  Every block ends with 256 global atomic adds to the same 256
// counters, so fewer, larger blocks cost less: measured on MI355X, 134 M values took 59 us
// in 2048 blocks and 35 us in 512 (256 blocks: 45 us, too few to fill the GPU).
inline uint32_t hist_block_bytes(uint64_t total) {
    uint32_t b = 1u << 14;
    while (b < (1u << 20) && (uint64_t)b * 512 < total) b <<= 1;
    return b;
}

template <int N>
struct HistArgsN {
    uint32_t nseg;
    uint32_t n_blocks;
    uint32_t block_bytes;   // values per block (hist_block_bytes)
    uint64_t* hist;         // nseg x 256
    SegDesc segs[N];        // x, n and first_block of each segment
};
using HistArgs = HistArgsN<kMaxInlineSegs>;  // host side; launches pass the smallest N

struct BuildArgs {
    const uint64_t* hist;   // nseg x 256
    uint32_t* tables;       // nseg x kDTDwords
    uint32_t* scost;        // workspace: nseg x kCostEntries cost factors
    uint8_t* arg;           // workspace: nseg x kArgBytes, the DP's choice per (k, i < 256)
    uint32_t nseg, K, R, C, S;
};
constexpr uint32_t kCostEntries = 257 * 256 / 2;  // [j, i) for 0 <= j < i <= 256
constexpr uint32_t kArgBytes = 257 * 256;

sh_status launch_histogram(const HistArgs& h, uint32_t nseg_zero, void* stream);
sh_status launch_build_tables(const BuildArgs& b, void* stream);
// the decode behind sh_decode and sh_decode_batch (k_decode_rows.hip): one chunk per
// 16-lane row (two or four streams a lane), kDecodeChunksPerBlock chunks a block; and, for
// launches of few chunks of 64 streams and every launch of chunks of 128, one chunk per half
// wavefront (two or four streams a lane), kWideHalvesChunksPerBlock chunks a block
constexpr uint32_t kDecodeChunksPerBlock = 16;
sh_status launch_decode(const CodecArgs& a, uint32_t total_blocks, void* stream);
constexpr uint32_t kWideHalvesChunksPerBlock = 8;
sh_status launch_decode_wide_halves(const CodecArgs& a, uint32_t total_blocks, void* stream);
// decode into a matrix-vector product: the vector is staged in LDS, so rows are at most
// this many values long
constexpr uint32_t kMaxMatvecCols = 16384;
sh_status launch_decode_matvec(const CodecArgs& a, uint32_t total_blocks, void* stream);
// the matrix-vector decode of chunks of 64 or 128 streams (the row decoder with a consumer
// sink); few: a launch of fewer than 16,384 chunks (rows of 32 lanes)
sh_status launch_decode_matvec_rows(const CodecArgs& a, uint32_t total_blocks, bool few,
                                    void* stream);
// the encoder's chunk kernel: one chunk per row of 16 lanes (two, four or eight streams a
// lane) or, for launches of few chunks of 64 streams, of 32 lanes (two streams a lane); 16
// chunks a block
constexpr uint32_t kEncodeChunksPerBlock = 16;
// segments of at most this many chunks are indexed and compacted by one kernel
// (k_encode_place: each block sums the sizes of the chunks before its own, so the work
// grows with the square of the chunk count); longer ones take the index kernel first
constexpr uint32_t kPlaceMaxChunks = 16384;
// The chunk kernel runs on stream.  With place_stream non-null the placement kernels run
// there instead: ready (an event) is recorded on stream after the chunk kernel, place_stream
// waits for it, and placed is recorded on place_stream after the placement.
sh_status launch_encode(const CodecArgs& a, uint32_t total_blocks, uint32_t total_blocks_c,
                        bool place, void* stream, void* place_stream = nullptr,
                        void* ready = nullptr, void* placed = nullptr);

// encode workspace layout
inline uint32_t encode_slot_dwords(uint32_t C, uint32_t R, uint32_t S) {
    uint32_t d = chunk_bound_dwords(C, R, S) + 1;
    return (d + 127) / 128 * 128;
}

}  // namespace shn
