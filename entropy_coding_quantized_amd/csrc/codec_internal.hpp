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
constexpr int kLanes = 32;             // interleaved tANS lanes per chunk (a half wavefront)
constexpr int kMaxLog2LHost = 12;      // host table build
constexpr int kMaxLog2LGpu = 8;        // GPU path: a field is at most 8 + 8 = 16 bits
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

// ---- container geometry ------------------------------------------------------------
inline uint32_t header_bytes(uint32_t K) { return (kHeaderFixed + 3 * K - 1 + 3) / 4 * 4; }
inline uint64_t n_chunks_of(uint64_t n, uint32_t C) { return (n + C - 1) / C; }
// largest chunk a valid stream holds: every field at 8 + R bits, padded to 32-bit words
SHN_HD inline uint32_t chunk_bound_dwords(uint32_t nc, uint32_t R) {
    uint64_t lanes = nc < (uint32_t)kLanes ? nc : (uint32_t)kLanes;
    uint64_t bits = lanes * R + (uint64_t)nc * (8 + R);
    return (uint32_t)((bits + 31) / 32);
}
void write_header(const sh_table& t, uint64_t n, uint32_t C, uint32_t S, uint64_t n_chunks,
                  uint32_t* dwords /* kMaxHeaderDwords */);

// ---- kernel argument blocks (kernels.hip) ------------------------------------------
// Decode entry of a slot, two dwords:
//   e0 = need | (byte address of the next slot's entry) << 16, need = w_s + nb <= 16
//   e1 = w_s | (int8 bits of the range base) << 8 | (|range| - 1) << 16
// Encode entry of a value u, two dwords:
//   v0 = bias_s (int32): the state-bit count is (X + bias_s) >> (R + 1)
//   v1 = o | w_s << 8 | (start_s + 512) << 16 | (f_s == 0) << 31, start_s = cum_s - f_s
struct DecodeArgs {
    const uint8_t* in;
    int8_t* out;
    int32_t* status;
    uint64_t in_nbytes;
    uint64_t n;
    uint32_t payload_at;    // byte offset of the payload in the container
    uint32_t index_at;      // byte offset of the chunk index
    uint32_t C;
    uint32_t R;
    uint32_t L;
    uint32_t n_chunks;
    uint32_t hdr_dwords;
    uint32_t pad_;
    uint32_t hdr[kMaxHeaderDwords];
    uint32_t dec[2 * 256];
};

struct EncodeArgs {
    const int8_t* x;
    uint32_t* slots;        // workspace: n_chunks slots of slot_dwords
    uint32_t* meta;         // workspace: per chunk {start bit in slot, field bits}
    int32_t* status;
    uint64_t n;
    uint32_t C;
    uint32_t R;
    uint32_t L;
    uint32_t n_chunks;
    uint32_t slot_dwords;   // multiple of 128
    uint32_t pad_;
    uint32_t vt[2 * 256];
    uint8_t es[256];
};

struct IndexArgs {
    const uint32_t* meta;
    uint8_t* out;
    sh_encode_info* info;
    uint64_t n;
    uint32_t n_chunks;
    uint32_t slot_dwords;
    uint32_t index_at;
    uint32_t hdr_dwords;
    uint32_t hdr[kMaxHeaderDwords];
};

struct CompactArgs {
    const uint32_t* slots;
    const uint32_t* meta;
    uint8_t* out;
    uint32_t n_chunks;
    uint32_t slot_dwords;
    uint32_t index_at;
    uint32_t payload_at;
};

sh_status launch_histogram(const int8_t* d_x, uint64_t n, uint64_t* d_hist, void* stream);
sh_status launch_decode(const DecodeArgs& a, void* stream);
sh_status launch_encode(const EncodeArgs& e, const IndexArgs& ix, const CompactArgs& cp,
                        void* stream);

// encode workspace layout
inline uint32_t encode_slot_dwords(uint32_t C, uint32_t R) {
    uint32_t d = chunk_bound_dwords(C, R) + 1;
    return (d + 127) / 128 * 128;
}

}  // namespace shn
