// C ABI of libshannonic.so (declared in include/shannonic.h): argument checks, table
// derivation for the kernels, workspace layout, segment grouping and launches.
#include <hip/hip_runtime.h>

#include <algorithm>
#include <cmath>
#include <cstring>
#include <vector>

#include "codec_internal.hpp"

namespace shn {
sh_status allocate_states(const uint64_t* count, uint32_t K, uint32_t L, uint16_t* f);
// k_decode.hip: the decode of launches with few chunks, one chunk per 32-lane half
// wavefront, 8 chunks a block, tables of at most 256 states
sh_status launch_decode_halves(const CodecArgs& a, uint32_t total_blocks, void* stream);
}

using namespace shn;

namespace {

constexpr uint32_t kChunksPerBlock = 8;   // the half-wavefront decode kernels
// A decode launch of fewer chunks than this cannot fill the GPU with the row decoder's 4
// chunks a wavefront (the chunks' steps are serial, so the launch takes the steps of one
// chunk times the step's latency); below it chunks go one per half wavefront, twice the
// wavefronts: for chunks of 32 streams the half-wavefront decoder (measured on MI355X: 1,024
// chunks 20.4 against 26.2 us, 8,192 chunks 93.8 against 95.5 us; a 48-tensor model launch
// of 91,000 chunks 0.37 against 0.50 of 8 TB/s the other way), for chunks of 64 the row
// decoder's 32-lane rows (8,192 chunks: 76 against 81.6 us).  Chunks of 128 streams always
// take 32-lane rows (four streams a lane).
constexpr uint64_t kHalfDecodeMaxChunks = 16384;

// the decode of a launch group of total_chunks chunks: blocks per chunk count and launcher
struct DecodePath {
    uint32_t per_block;
    sh_status (*launch)(const CodecArgs&, uint32_t, void*);
};
DecodePath decode_path(uint64_t total_chunks, const sh_params* p) {
    if (p->streams == kStreamsWidest) return {kWideHalvesChunksPerBlock, launch_decode_wide_halves};
    if (total_chunks < kHalfDecodeMaxChunks) {
        if (p->streams == kStreamsWide) return {kWideHalvesChunksPerBlock, launch_decode_wide_halves};
        if (p->log2_L <= (uint32_t)kInlineMaxLog2L) return {kChunksPerBlock, launch_decode_halves};
    }
    return {kDecodeChunksPerBlock, launch_decode};
}
constexpr uint32_t kChunksPerBlockC = 4;  // compaction kernel

bool gpu_params_ok(const sh_params* p) {
    return p && p->K >= 1 && p->K <= 256 && p->log2_L >= 1 && p->log2_L <= (uint32_t)kMaxLog2LGpu &&
           (p->streams == kStreamsNarrow || p->streams == kStreamsWide ||
            p->streams == kStreamsWidest) &&
           p->chunk_symbols >= p->streams && p->chunk_symbols <= kMaxChunk &&
           p->chunk_symbols % p->streams == 0;
}

// INVALID_ARG for nonsense, UNSUPPORTED for valid parameters the GPU path does not take
sh_status check_params(const sh_params* p) {
    if (!p || p->K < 1 || p->K > 256 || p->log2_L < 1 || p->chunk_symbols == 0 || p->streams == 0)
        return SH_ERR_INVALID_ARG;
    return gpu_params_ok(p) ? SH_OK : SH_ERR_UNSUPPORTED;
}

bool aligned(const void* p, uintptr_t a) { return ((uintptr_t)p & (a - 1)) == 0; }

// the container's first payload byte: header, then the chunk index
uint64_t payload_at_of(uint64_t nch, const sh_params* p) {
    return header_bytes(p->K) + index_bytes_of(nch);
}

// container bytes at most: every chunk at its bound, in whole size units
uint64_t bound_of(uint64_t n, const sh_params* p) {
    const uint64_t nch = n_chunks_of(n, p->chunk_symbols);
    const uint32_t u = size_unit_log2(p->chunk_symbols, p->log2_L, p->streams);
    uint64_t payload = 0;
    if (nch > 0) {
        payload += ((uint64_t)chunk_bound_units(p->chunk_symbols, p->log2_L, u, p->streams) << u) *
                   (nch - 1);
        const uint64_t last = n - (nch - 1) * p->chunk_symbols;
        payload += (uint64_t)chunk_bound_units((uint32_t)last, p->log2_L, u, p->streams) << u;
    }
    return payload_at_of(nch, p) + (payload + 3) / 4 * 4;
}

uint32_t blocks_for(uint64_t nch, uint32_t per) { return (uint32_t)((nch + per - 1) / per); }

// slots a segment takes in the encode workspace: its chunks rounded up to a wavefront's four
uint64_t slots_for(uint64_t nch) { return (nch + 3) / 4 * 4; }

uint64_t align256(uint64_t v) { return (v + 255) / 256 * 256; }

// encode workspace for a group of segments: slots, then per-slot meta, then per-block
// aggregates of the chunk kernel (a block takes kEncodeChunksPerBlock chunks, so a group has
// at most total_slots / kEncodeChunksPerBlock + kMaxInlineSegs blocks)
struct EncLayout {
    uint64_t meta_at, agg_at, bytes;
    uint32_t slot_dwords;
};
EncLayout enc_layout(uint64_t total_slots, const sh_params* p) {
    EncLayout l;
    l.slot_dwords = encode_slot_dwords(p->chunk_symbols, p->log2_L, p->streams);
    l.meta_at = align256(total_slots * l.slot_dwords * 4);
    l.agg_at = l.meta_at + align256(8 * total_slots);
    l.bytes = l.agg_at + align256(8 * (total_slots / kEncodeChunksPerBlock + kMaxInlineSegs)) + 256;
    return l;
}

// compaction blocks of a segment: the one-kernel placement gives an empty segment a block
// of its own (it writes the header, the index end and the totals)
uint32_t place_blocks(uint64_t nch, bool place) {
    const uint32_t b = blocks_for(nch, kChunksPerBlockC);
    return place && b == 0 ? 1 : b;
}

// groups of at most kMaxInlineSegs segments: [begin, end)
std::vector<std::pair<uint32_t, uint32_t>> groups_of(uint32_t nseg) {
    std::vector<std::pair<uint32_t, uint32_t>> g;
    for (uint32_t b = 0; b < nseg; b += kMaxInlineSegs) g.push_back({b, std::min(nseg, b + kMaxInlineSegs)});
    return g;
}

// one launch group's workspace region: the largest group's layout (a multiple of 256 bytes)
uint64_t encode_group_ws(const uint64_t* n, uint32_t nseg, const sh_params* p) {
    uint64_t best = 256;
    for (auto [b, e] : groups_of(nseg)) {
        uint64_t slots = 0;
        for (uint32_t i = b; i < e; ++i) slots += slots_for(n_chunks_of(n[i], p->chunk_symbols));
        best = std::max(best, enc_layout(slots, p).bytes);
    }
    return best;
}

// the batch workspace: two group regions when the batch takes more than one launch group
// (with a placement stream, group g's placement reads region g mod 2 while group g + 1's
// chunk kernel writes the other), else one
uint64_t encode_batch_ws(const uint64_t* n, uint32_t nseg, const sh_params* p) {
    return encode_group_ws(n, nseg, p) * (nseg > kMaxInlineSegs ? 2 : 1);
}

void fill_codec_common(CodecArgs& a, const sh_params* p, int32_t* d_status) {
    a.C = p->chunk_symbols;
    a.R = p->log2_L;
    a.L = 1u << p->log2_L;
    a.K = p->K;
    a.S = p->streams;
    a.slot_dwords = encode_slot_dwords(p->chunk_symbols, p->log2_L, p->streams);
    a.status = d_status;
}

sh_status hip_ok(hipError_t e) { return e == hipSuccess ? SH_OK : SH_ERR_HIP; }

}  // namespace

extern "C" {

uint32_t sh_version(void) { return (1u << 16) | 3u; }

const char* sh_status_string(sh_status st) {
    switch (st) {
        case SH_OK: return "ok";
        case SH_ERR_INVALID_ARG: return "invalid argument";
        case SH_ERR_UNSUPPORTED: return "unsupported parameters";
        case SH_ERR_SYMBOL_NOT_IN_TABLE: return "value outside the table's occupied ranges";
        case SH_ERR_CORRUPT_STREAM: return "corrupt stream";
        case SH_ERR_BUFFER_TOO_SMALL: return "buffer too small";
        case SH_ERR_HIP: return "HIP runtime error";
        default: return "unknown status";
    }
}

sh_status sh_histogram(const int8_t* d_x, uint64_t n, uint64_t* d_hist, void* stream) {
    if (!d_hist || (n > 0 && !d_x)) return SH_ERR_INVALID_ARG;
    if (!aligned(d_x, 16) || !aligned(d_hist, 8)) return SH_ERR_INVALID_ARG;
    HistArgs h;
    std::memset(&h, 0, sizeof(h));
    h.nseg = 1;
    h.hist = d_hist;
    h.segs[0].x = (uint8_t*)d_x;
    h.segs[0].n = n;
    h.block_bytes = hist_block_bytes(n);
    h.n_blocks = (uint32_t)((n + h.block_bytes - 1) / h.block_bytes);
    return launch_histogram(h, 1, stream);
}

sh_status sh_table_from_histogram(const uint64_t* hist, const sh_params* params, sh_table* out) {
    if (!hist || !params || !out) return SH_ERR_INVALID_ARG;
    return table_from_histogram(hist, params->K, params->log2_L, out);
}

uint64_t sh_build_tables_workspace(void) {
    return align256(kDTBytes) + sh_build_tables_batch_workspace(1);
}

sh_status sh_build_tables(const int8_t* x, uint64_t n, int x_on_device, const sh_params* params,
                          void* d_ws, uint64_t ws_bytes, void* stream, sh_table* out) {
    if (!params || !out || (n > 0 && !x)) return SH_ERR_INVALID_ARG;
    if (!x_on_device) {
        uint64_t h[256] = {0};
        for (uint64_t i = 0; i < n; ++i) h[(uint8_t)x[i] ^ 0x80]++;
        return table_from_histogram(h, params->K, params->log2_L, out);
    }
    // on the GPU: histogram and the whole table build, then one copy back
    sh_status st = check_params(params);
    if (st != SH_OK) return st;
    if (!d_ws || !aligned(d_ws, 256)) return SH_ERR_INVALID_ARG;
    if (ws_bytes < sh_build_tables_workspace()) return SH_ERR_BUFFER_TOO_SMALL;
    uint8_t* dt = (uint8_t*)d_ws;
    uint8_t* ws = dt + align256(kDTBytes);
    st = sh_build_tables_batch(&x, &n, 1, params, dt, ws, sh_build_tables_batch_workspace(1), stream);
    if (st != SH_OK) return st;
    int32_t table_status = SH_OK;
    st = sh_tables_from_device(dt, 1, out, &table_status, stream);
    return st != SH_OK ? st : table_status;
}

// ---- device-resident tables ------------------------------------------------------------

uint64_t sh_device_table_bytes(void) { return kDTBytes; }

sh_status sh_table_to_device(const sh_table* table, const sh_params* params, void* d_table,
                             void* stream) {
    if (!table || !d_table || !aligned(d_table, 16)) return SH_ERR_INVALID_ARG;
    sh_status st = check_params(params);
    if (st != SH_OK) return st;
    if (table->K != params->K || table->log2_L != params->log2_L) return SH_ERR_INVALID_ARG;
    const bool empty = table->n == 0;
    if (check_table(*table, empty) != SH_OK) return SH_ERR_INVALID_ARG;
    if (max_field_bits(*table) > kMaxFieldBitsGpu) return SH_ERR_UNSUPPORTED;
    std::vector<uint32_t> dt(kDTDwords, 0);
    SlotTables slots;
    if (!empty && derive_slots(*table, &slots) != SH_OK) return SH_ERR_INVALID_ARG;
    make_device_table(*table, empty ? nullptr : &slots, params->chunk_symbols, params->streams,
                      dt.data());
    hipStream_t s = (hipStream_t)stream;
    if (hipMemcpyAsync(d_table, dt.data(), kDTBytes, hipMemcpyHostToDevice, s) != hipSuccess)
        return SH_ERR_HIP;
    return hip_ok(hipStreamSynchronize(s));
}

sh_status sh_tables_from_bytes(const void* tables, uint32_t count, sh_table* out,
                               int32_t* table_status) {
    if (count == 0) return SH_OK;
    if (!tables || !out || !table_status || !aligned(tables, 4)) return SH_ERR_INVALID_ARG;
    for (uint32_t i = 0; i < count; ++i) {
        const uint32_t* d = (const uint32_t*)tables + (size_t)kDTDwords * i;
        sh_table t;
        std::memset(&t, 0, sizeof(t));
        t.K = d[kDTK];
        t.log2_L = d[kDTLog2L];
        std::memcpy(&t.n, d + kDTN, 8);
        std::memcpy(t.lo, d + kDTLo, sizeof(t.lo));
        std::memcpy(t.freq, d + kDTFreq, sizeof(t.freq));
        std::memcpy(t.hist, d + kDTHist, sizeof(t.hist));
        table_status[i] = (int32_t)d[kDTStatus];
        if (table_status[i] == SH_OK && check_table(t, t.n == 0) != SH_OK)
            table_status[i] = SH_ERR_CORRUPT_STREAM;
        out[i] = t;
    }
    return SH_OK;
}

sh_status sh_tables_from_device(const void* d_tables, uint32_t count, sh_table* out,
                                int32_t* table_status, void* stream) {
    if (count == 0) return SH_OK;
    if (!d_tables || !out || !table_status) return SH_ERR_INVALID_ARG;
    std::vector<uint32_t> dt((size_t)kDTDwords * count, 0);
    hipStream_t s = (hipStream_t)stream;
    if (hipMemcpyAsync(dt.data(), d_tables, (size_t)kDTBytes * count, hipMemcpyDeviceToHost, s) !=
            hipSuccess ||
        hipStreamSynchronize(s) != hipSuccess)
        return SH_ERR_HIP;
    return sh_tables_from_bytes(dt.data(), count, out, table_status);
}

uint64_t sh_build_tables_batch_workspace(uint32_t nseg) {
    return align256(8ull * 256 * nseg) + align256(4ull * kCostEntries * nseg) +
           align256((uint64_t)kArgBytes * nseg);
}

sh_status sh_build_tables_batch(const int8_t* const* d_x, const uint64_t* n, uint32_t nseg,
                                const sh_params* params, void* d_tables, void* d_ws,
                                uint64_t ws_bytes, void* stream) {
    if (nseg == 0) return SH_OK;
    if (!d_x || !n || !d_tables || !d_ws || !aligned(d_tables, 16) || !aligned(d_ws, 256))
        return SH_ERR_INVALID_ARG;
    sh_status st = check_params(params);
    if (st != SH_OK) return st;
    if (ws_bytes < sh_build_tables_batch_workspace(nseg)) return SH_ERR_BUFFER_TOO_SMALL;
    for (uint32_t i = 0; i < nseg; ++i) {
        if (n[i] > 0 && (!d_x[i] || !aligned(d_x[i], 16))) return SH_ERR_INVALID_ARG;
        if (n[i] >= (1ull << 32)) return SH_ERR_UNSUPPORTED;
    }
    uint8_t* ws = (uint8_t*)d_ws;
    uint64_t* hist = (uint64_t*)ws;
    uint32_t* scost = (uint32_t*)(ws + align256(8ull * 256 * nseg));
    uint8_t* arg = ws + align256(8ull * 256 * nseg) + align256(4ull * kCostEntries * nseg);
    for (auto [b, e] : groups_of(nseg)) {
        HistArgs h;
        std::memset(&h, 0, sizeof(h));
        h.nseg = e - b;
        h.hist = hist + 256ull * b;
        uint64_t total = 0;
        for (uint32_t i = b; i < e; ++i) total += n[i];
        h.block_bytes = hist_block_bytes(total);
        uint32_t blocks = 0;
        for (uint32_t i = b; i < e; ++i) {
            SegDesc& sd = h.segs[i - b];
            sd.x = (uint8_t*)d_x[i];
            sd.n = n[i];
            sd.first_block = blocks;
            blocks += (uint32_t)((n[i] + h.block_bytes - 1) / h.block_bytes);
        }
        h.n_blocks = blocks;
        st = launch_histogram(h, e - b, stream);
        if (st != SH_OK) return st;
    }
    BuildArgs bd;
    bd.hist = hist;
    bd.tables = (uint32_t*)d_tables;
    bd.scost = scost;
    bd.arg = arg;
    bd.nseg = nseg;
    bd.K = params->K;
    bd.R = params->log2_L;
    bd.C = params->chunk_symbols;
    bd.S = params->streams;
    return launch_build_tables(bd, stream);
}

// ---- encode / decode -------------------------------------------------------------------

uint64_t sh_encode_bound(uint64_t n, const sh_params* params) {
    if (!gpu_params_ok(params)) return 0;
    return bound_of(n, params);
}

uint64_t sh_encode_workspace(uint64_t n, const sh_params* params) {
    if (!gpu_params_ok(params)) return 0;
    return encode_batch_ws(&n, 1, params);
}

sh_status sh_encode(const sh_table* table, const sh_params* params, const int8_t* d_x,
                    uint64_t n, uint8_t* d_out, uint64_t out_cap, void* d_ws, uint64_t ws_bytes,
                    sh_encode_info* d_info, int32_t* d_status, void* stream) {
    if (!table || !d_out || (n > 0 && !d_x)) return SH_ERR_INVALID_ARG;
    sh_status st = check_params(params);
    if (st != SH_OK) return st;
    if (table->K != params->K || table->log2_L != params->log2_L) return SH_ERR_INVALID_ARG;
    if (check_table(*table, n == 0) != SH_OK) return SH_ERR_INVALID_ARG;
    // the table travels in the launch's arguments: at most 256 states (larger tables go
    // through sh_table_to_device and the batch calls)
    if (params->log2_L > (uint32_t)kInlineMaxLog2L || max_field_bits(*table) > kMaxFieldBitsGpu)
        return SH_ERR_UNSUPPORTED;
    if (n >= (1ull << 32)) return SH_ERR_UNSUPPORTED;
    const uint64_t bound = bound_of(n, params);
    if (bound > 0xFFFFFFFFull) return SH_ERR_UNSUPPORTED;
    if (out_cap < bound) return SH_ERR_BUFFER_TOO_SMALL;
    const uint64_t nch = n_chunks_of(n, params->chunk_symbols);
    const EncLayout lay = enc_layout(slots_for(nch), params);
    if (!d_ws || ws_bytes < lay.bytes) return SH_ERR_BUFFER_TOO_SMALL;
    if (!aligned(d_x, 16) || !aligned(d_out, 4) || !aligned(d_ws, 256) ||
        !aligned(d_info, 8) || !aligned(d_status, 4))
        return SH_ERR_INVALID_ARG;

    CodecArgs a;
    std::memset(&a, 0, sizeof(a));
    fill_codec_common(a, params, d_status);
    a.nseg = 0;
    a.slots = (uint32_t*)d_ws;
    a.meta = (uint32_t*)((uint8_t*)d_ws + lay.meta_at);
    a.agg = (uint32_t*)((uint8_t*)d_ws + lay.agg_at);
    const bool place = nch <= kPlaceMaxChunks;
    if (n > 0) {
        SlotTables slots;
        if (derive_slots(*table, &slots) != SH_OK) return SH_ERR_INVALID_ARG;
        derive_kernel_tables(*table, slots, nullptr, a.one.tab, a.one.es);
    }
    write_header(*table, n, params->chunk_symbols, params->streams, nch, a.one.hdr);
    SegDesc& sd = a.one.seg;
    sd.x = (uint8_t*)d_x;
    sd.c = d_out;
    sd.n = n;
    sd.c_bytes = out_cap;
    sd.info = d_info;
    sd.n_chunks = (uint32_t)nch;
    return launch_encode(a, blocks_for(nch, kEncodeChunksPerBlock), place_blocks(nch, place), place,
                         stream);
}

sh_status sh_decode(const sh_table* table, const sh_params* params, const uint8_t* d_in,
                    uint64_t in_nbytes, int8_t* d_y, uint64_t n, int32_t* d_status,
                    void* stream) {
    if (!table || !d_in || (n > 0 && !d_y)) return SH_ERR_INVALID_ARG;
    sh_status st = check_params(params);
    if (st != SH_OK) return st;
    if (table->K != params->K || table->log2_L != params->log2_L) return SH_ERR_INVALID_ARG;
    if (check_table(*table, n == 0) != SH_OK) return SH_ERR_INVALID_ARG;
    if (params->log2_L > (uint32_t)kInlineMaxLog2L || max_field_bits(*table) > kMaxFieldBitsGpu)
        return SH_ERR_UNSUPPORTED;
    if (n >= (1ull << 32) || in_nbytes > 0xFFFFFFFFull) return SH_ERR_UNSUPPORTED;
    if (!aligned(d_in, 4) || !aligned(d_status, 4)) return SH_ERR_INVALID_ARG;
    const uint64_t nch = n_chunks_of(n, params->chunk_symbols);
    if (in_nbytes < payload_at_of(nch, params)) return SH_ERR_CORRUPT_STREAM;
    if (n == 0) return SH_OK;

    CodecArgs a;
    std::memset(&a, 0, sizeof(a));
    fill_codec_common(a, params, d_status);
    a.nseg = 0;
    SlotTables slots;
    if (derive_slots(*table, &slots) != SH_OK) return SH_ERR_INVALID_ARG;
    derive_kernel_tables(*table, slots, a.one.tab, nullptr, nullptr);
    write_header(*table, n, params->chunk_symbols, params->streams, nch, a.one.hdr);
    SegDesc& sd = a.one.seg;
    sd.x = (uint8_t*)d_y;
    sd.c = (uint8_t*)d_in;
    sd.n = n;
    sd.c_bytes = in_nbytes;
    sd.n_chunks = (uint32_t)nch;
    const DecodePath path = decode_path(nch, params);
    return path.launch(a, blocks_for(nch, path.per_block), stream);
}

uint64_t sh_encode_batch_workspace(const uint64_t* n, uint32_t nseg, const sh_params* params) {
    if (!n || !gpu_params_ok(params)) return 0;
    return encode_batch_ws(n, nseg, params);
}

sh_status sh_encode_batch(const void* d_tables, const int8_t* const* d_x, const uint64_t* n,
                          uint32_t nseg, const sh_params* params, uint8_t* const* d_out,
                          const uint64_t* out_cap, void* d_ws, uint64_t ws_bytes,
                          sh_encode_info* d_info, int32_t* d_status, void* stream,
                          void* place_stream) {
    if (nseg == 0) return SH_OK;
    if (!d_tables || !d_x || !n || !d_out || !out_cap || !aligned(d_tables, 16))
        return SH_ERR_INVALID_ARG;
    sh_status st = check_params(params);
    if (st != SH_OK) return st;
    const auto groups = groups_of(nseg);
    const bool overlap = place_stream != nullptr && place_stream != stream && groups.size() > 1;
    const uint64_t region = encode_group_ws(n, nseg, params);
    if (!d_ws || !aligned(d_ws, 256) || ws_bytes < region * (overlap ? 2 : 1))
        return SH_ERR_BUFFER_TOO_SMALL;
    if (!aligned(d_info, 8) || !aligned(d_status, 4)) return SH_ERR_INVALID_ARG;
    for (uint32_t i = 0; i < nseg; ++i) {
        if (!d_out[i] || !aligned(d_out[i], 4) || (n[i] > 0 && (!d_x[i] || !aligned(d_x[i], 16))))
            return SH_ERR_INVALID_ARG;
        if (n[i] >= (1ull << 32) || bound_of(n[i], params) > 0xFFFFFFFFull) return SH_ERR_UNSUPPORTED;
        if (out_cap[i] < bound_of(n[i], params)) return SH_ERR_BUFFER_TOO_SMALL;
    }
    // With overlap, group g's chunk kernel runs on stream in region g mod 2 and its
    // placement on place_stream once the chunk kernel is done, beside group g + 1's chunk
    // kernel; group g + 2's chunk kernel waits for group g's placement (it reuses the
    // region), and stream waits for the last placement before the call returns.
    std::vector<hipEvent_t> ready(overlap ? groups.size() : 0, nullptr);
    std::vector<hipEvent_t> placed(ready.size(), nullptr);
    auto release = [&]() {
        for (hipEvent_t ev : ready)
            if (ev) (void)hipEventDestroy(ev);
        for (hipEvent_t ev : placed)
            if (ev) (void)hipEventDestroy(ev);
    };
    for (size_t g = 0; g < ready.size(); ++g)
        if (hipEventCreateWithFlags(&ready[g], hipEventDisableTiming) != hipSuccess ||
            hipEventCreateWithFlags(&placed[g], hipEventDisableTiming) != hipSuccess) {
            release();
            return SH_ERR_HIP;
        }
    int last_placed = -1;
    for (size_t g = 0; g < groups.size(); ++g) {
        const auto [b, e] = groups[g];
        CodecArgs a;
        std::memset(&a, 0, sizeof(a));
        fill_codec_common(a, params, d_status);
        a.nseg = e - b;
        uint64_t slots = 0;
        uint32_t blocks = 0, blocks_c = 0;
        bool place = true;
        for (uint32_t i = b; i < e; ++i)
            place = place && n_chunks_of(n[i], params->chunk_symbols) <= kPlaceMaxChunks;
        for (uint32_t i = b; i < e; ++i) {
            SegDesc& sd = a.many[i - b];
            const uint64_t nch = n_chunks_of(n[i], params->chunk_symbols);
            sd.x = (uint8_t*)d_x[i];
            sd.c = d_out[i];
            sd.n = n[i];
            sd.c_bytes = out_cap[i];
            sd.tab = (const uint32_t*)((const uint8_t*)d_tables + (uint64_t)i * kDTBytes);
            sd.info = d_info ? d_info + i : nullptr;
            sd.first_block = blocks;
            sd.first_block_c = blocks_c;
            sd.n_chunks = (uint32_t)nch;
            sd.slot_base = (uint32_t)slots;
            blocks += blocks_for(nch, kEncodeChunksPerBlock);
            blocks_c += place_blocks(nch, place);
            slots += slots_for(nch);
        }
        const EncLayout lay = enc_layout(slots, params);
        uint8_t* ws = (uint8_t*)d_ws + (overlap ? (g & 1) * region : 0);
        a.slots = (uint32_t*)ws;
        a.meta = (uint32_t*)(ws + lay.meta_at);
        a.agg = (uint32_t*)(ws + lay.agg_at);
        if (overlap && g >= 2 &&
            hipStreamWaitEvent((hipStream_t)stream, placed[g - 2], 0) != hipSuccess) {
            st = SH_ERR_HIP;
            break;
        }
        st = overlap ? launch_encode(a, blocks, blocks_c, place, stream, place_stream, ready[g],
                                     placed[g])
                     : launch_encode(a, blocks, blocks_c, place, stream);
        if (st != SH_OK) break;
        last_placed = (int)g;
    }
    // stream takes up after the last placement queued, also when a later launch failed
    if (overlap && last_placed >= 0 &&
        hipStreamWaitEvent((hipStream_t)stream, placed[last_placed], 0) != hipSuccess &&
        st == SH_OK)
        st = SH_ERR_HIP;
    release();
    return st;
}

sh_status sh_decode_batch(const void* d_tables, const uint8_t* const* d_in,
                          const uint64_t* in_nbytes, int8_t* const* d_y, const uint64_t* n,
                          uint32_t nseg, const sh_params* params, int32_t* d_status,
                          void* stream) {
    if (nseg == 0) return SH_OK;
    if (!d_tables || !d_in || !in_nbytes || !d_y || !n || !aligned(d_tables, 16))
        return SH_ERR_INVALID_ARG;
    sh_status st = check_params(params);
    if (st != SH_OK) return st;
    if (!aligned(d_status, 4)) return SH_ERR_INVALID_ARG;
    for (uint32_t i = 0; i < nseg; ++i) {
        if (!d_in[i] || !aligned(d_in[i], 4) || (n[i] > 0 && !d_y[i])) return SH_ERR_INVALID_ARG;
        if (n[i] >= (1ull << 32) || in_nbytes[i] > 0xFFFFFFFFull) return SH_ERR_UNSUPPORTED;
        const uint64_t nch = n_chunks_of(n[i], params->chunk_symbols);
        if (in_nbytes[i] < payload_at_of(nch, params)) return SH_ERR_CORRUPT_STREAM;
    }
    for (auto [b, e] : groups_of(nseg)) {
        CodecArgs a;
        std::memset(&a, 0, sizeof(a));
        fill_codec_common(a, params, d_status);
        a.nseg = e - b;
        uint64_t total_chunks = 0;
        for (uint32_t i = b; i < e; ++i) total_chunks += n_chunks_of(n[i], params->chunk_symbols);
        const DecodePath path = decode_path(total_chunks, params);
        uint32_t blocks = 0;
        for (uint32_t i = b; i < e; ++i) {
            SegDesc& sd = a.many[i - b];
            const uint64_t nch = n_chunks_of(n[i], params->chunk_symbols);
            sd.x = (uint8_t*)d_y[i];
            sd.c = (uint8_t*)d_in[i];
            sd.n = n[i];
            sd.c_bytes = in_nbytes[i];
            sd.tab = (const uint32_t*)((const uint8_t*)d_tables + (uint64_t)i * kDTBytes);
            sd.first_block = blocks;
            sd.n_chunks = (uint32_t)nch;
            blocks += blocks_for(nch, path.per_block);
        }
        st = path.launch(a, blocks, stream);
        if (st != SH_OK) return st;
    }
    return SH_OK;
}

sh_status sh_decode_matvec_batch(const void* d_tables, const uint8_t* const* d_in,
                                 const uint64_t* in_nbytes, const int8_t* const* d_a,
                                 int32_t* const* d_y, const uint64_t* n, uint32_t cols,
                                 uint32_t nseg, const sh_params* params, int32_t* d_status,
                                 void* stream) {
    if (nseg == 0) return SH_OK;
    if (!d_tables || !d_in || !in_nbytes || !d_a || !d_y || !n || !aligned(d_tables, 16) ||
        cols == 0)
        return SH_ERR_INVALID_ARG;
    sh_status st = check_params(params);
    if (st != SH_OK) return st;
    // chunks of 32 streams: the half-wavefront kernel (one slot a thread: L <= 256); of 64 or
    // 128: the row decoder; a matrix row holds whole steps of the chunks' streams
    const bool narrow = params->streams == kStreamsNarrow;
    if (cols % params->streams != 0 || cols > kMaxMatvecCols) return SH_ERR_UNSUPPORTED;
    if (narrow && params->log2_L > (uint32_t)kInlineMaxLog2L) return SH_ERR_UNSUPPORTED;
    if (!aligned(d_status, 4)) return SH_ERR_INVALID_ARG;
    for (uint32_t i = 0; i < nseg; ++i) {
        if (!d_in[i] || !aligned(d_in[i], 4) || n[i] % cols != 0) return SH_ERR_INVALID_ARG;
        if (n[i] > 0 && (!d_a[i] || !d_y[i] || !aligned(d_a[i], 16) || !aligned(d_y[i], 4)))
            return SH_ERR_INVALID_ARG;
        if (n[i] >= (1ull << 32) || in_nbytes[i] > 0xFFFFFFFFull) return SH_ERR_UNSUPPORTED;
        const uint64_t nch = n_chunks_of(n[i], params->chunk_symbols);
        if (in_nbytes[i] < payload_at_of(nch, params)) return SH_ERR_CORRUPT_STREAM;
    }
    for (auto [b, e] : groups_of(nseg)) {
        CodecArgs a;
        std::memset(&a, 0, sizeof(a));
        fill_codec_common(a, params, d_status);
        a.cols = cols;
        a.nseg = e - b;
        uint64_t total_chunks = 0;
        for (uint32_t i = b; i < e; ++i) total_chunks += n_chunks_of(n[i], params->chunk_symbols);
        const uint32_t per_block = narrow ? kChunksPerBlock : decode_path(total_chunks, params).per_block;
        uint32_t blocks = 0;
        for (uint32_t i = b; i < e; ++i) {
            SegDesc& sd = a.many[i - b];
            const uint64_t nch = n_chunks_of(n[i], params->chunk_symbols);
            sd.x = (uint8_t*)d_y[i];
            sd.vec = d_a[i];
            sd.c = (uint8_t*)d_in[i];
            sd.n = n[i];
            sd.c_bytes = in_nbytes[i];
            sd.tab = (const uint32_t*)((const uint8_t*)d_tables + (uint64_t)i * kDTBytes);
            sd.first_block = blocks;
            sd.n_chunks = (uint32_t)nch;
            blocks += blocks_for(nch, per_block);
        }
        st = narrow ? launch_decode_matvec(a, blocks, stream)
                    : launch_decode_matvec_rows(a, blocks, total_chunks < kHalfDecodeMaxChunks, stream);
        if (st != SH_OK) return st;
    }
    return SH_OK;
}

uint64_t sh_decode_stream_staging(const uint64_t* in_nbytes, uint32_t nseg, uint32_t depth) {
    if (!in_nbytes || depth == 0) return 0;
    uint64_t most = 0;
    for (uint32_t i = 0; i < nseg; ++i) most = std::max(most, in_nbytes[i]);
    return (uint64_t)depth * align256(std::max<uint64_t>(most, 1));
}

sh_status sh_decode_stream(const void* d_tables, const uint8_t* const* h_in,
                           const uint64_t* in_nbytes, int8_t* const* d_y, const uint64_t* n,
                           uint32_t nseg, const sh_params* params, void* d_staging,
                           uint64_t staging_bytes, uint32_t depth, int32_t* d_status,
                           void* copy_stream, void* stream) {
    if (nseg == 0) return SH_OK;
    if (!d_tables || !h_in || !in_nbytes || !d_y || !n || !d_staging || depth == 0 ||
        !aligned(d_tables, 16) || !aligned(d_staging, 256) || !aligned(d_status, 4))
        return SH_ERR_INVALID_ARG;
    sh_status st = check_params(params);
    if (st != SH_OK) return st;
    const uint64_t slot_bytes = staging_bytes / depth / 256 * 256;
    for (uint32_t i = 0; i < nseg; ++i) {
        if (!h_in[i] || (n[i] > 0 && !d_y[i])) return SH_ERR_INVALID_ARG;
        if (n[i] >= (1ull << 32) || in_nbytes[i] > 0xFFFFFFFFull) return SH_ERR_UNSUPPORTED;
        if (in_nbytes[i] > slot_bytes) return SH_ERR_BUFFER_TOO_SMALL;
        const uint64_t nch = n_chunks_of(n[i], params->chunk_symbols);
        if (in_nbytes[i] < payload_at_of(nch, params)) return SH_ERR_CORRUPT_STREAM;
    }
    hipStream_t cs = (hipStream_t)copy_stream, ds = (hipStream_t)stream;
    std::vector<hipEvent_t> copied(depth, nullptr), freed(depth, nullptr);
    hipEvent_t start = nullptr;
    auto release = [&]() {
        for (hipEvent_t e : copied)
            if (e) (void)hipEventDestroy(e);
        for (hipEvent_t e : freed)
            if (e) (void)hipEventDestroy(e);
        if (start) (void)hipEventDestroy(start);
    };
    bool ok = hipEventCreateWithFlags(&start, hipEventDisableTiming) == hipSuccess;
    for (uint32_t s = 0; s < depth && ok; ++s)
        ok = hipEventCreateWithFlags(&copied[s], hipEventDisableTiming) == hipSuccess &&
             hipEventCreateWithFlags(&freed[s], hipEventDisableTiming) == hipSuccess;
    // the first copies wait for everything already queued on stream, which may still read
    // the staging area (an earlier call)
    ok = ok && hipEventRecord(start, ds) == hipSuccess && hipStreamWaitEvent(cs, start, 0) == hipSuccess;
    if (!ok) {
        release();
        return SH_ERR_HIP;
    }
    // groups of consecutive containers that fit one staging slot go up together and are
    // decoded by one launch; slot g % depth is reused once the decode that read it is done
    std::vector<const uint8_t*> ins;
    uint32_t i = 0;
    for (uint32_t g = 0; i < nseg && st == SH_OK; ++g) {
        const uint32_t slot = g % depth;
        uint8_t* base = (uint8_t*)d_staging + (uint64_t)slot * slot_bytes;
        uint32_t j = i;
        uint64_t used = 0;
        ins.clear();
        while (j < nseg && j - i < kMaxInlineSegs && align256(used) + in_nbytes[j] <= slot_bytes) {
            ins.push_back(base + align256(used));
            used = align256(used) + in_nbytes[j];
            ++j;
        }
        if (g >= depth && hipStreamWaitEvent(cs, freed[slot], 0) != hipSuccess) st = SH_ERR_HIP;
        for (uint32_t k = i; k < j && st == SH_OK; ++k)
            if (hipMemcpyAsync((void*)ins[k - i], h_in[k], in_nbytes[k], hipMemcpyHostToDevice, cs) !=
                hipSuccess)
                st = SH_ERR_HIP;
        if (st == SH_OK && (hipEventRecord(copied[slot], cs) != hipSuccess ||
                            hipStreamWaitEvent(ds, copied[slot], 0) != hipSuccess))
            st = SH_ERR_HIP;
        if (st == SH_OK)
            st = sh_decode_batch((const uint8_t*)d_tables + (uint64_t)i * kDTBytes, ins.data(),
                                 in_nbytes + i, d_y + i, n + i, j - i, params, d_status, stream);
        if (st == SH_OK && hipEventRecord(freed[slot], ds) != hipSuccess) st = SH_ERR_HIP;
        i = j;
    }
    release();  // events still pending are released once they complete
    return st;
}

sh_status sh_stats(const sh_table* table, uint64_t n, uint64_t payload_bits,
                   uint64_t container_bytes, sh_stats_t* out) {
    if (!table || !out) return SH_ERR_INVALID_ARG;
    if (check_table(*table, true) != SH_OK) return SH_ERR_INVALID_ARG;
    std::memset(out, 0, sizeof(*out));
    uint64_t N = 0;
    for (int u = 0; u < 256; ++u) N += table->hist[u];
    if (N == 0) return SH_OK;
    const double dN = (double)N, L = (double)(1u << table->log2_L);
    double H = 0, HP = 0, dkl = 0, pw = 0;
    for (int u = 0; u < 256; ++u)
        if (table->hist[u]) {
            const double p = table->hist[u] / dN;
            H -= p * std::log2(p);
        }
    for (uint32_t k = 0; k < table->K; ++k) {
        uint64_t nk = 0;
        for (uint32_t u = table->lo[k]; u < table->lo[k + 1]; ++u) nk += table->hist[u];
        if (!nk) continue;
        if (!table->freq[k]) return SH_ERR_INVALID_ARG;
        const double P = nk / dN, Q = table->freq[k] / L;
        HP -= P * std::log2(P);
        dkl += P * std::log2(P / Q);
        pw += P * ceil_log2_u32(table->lo[k + 1] - table->lo[k]);
    }
    uint16_t fref[256];
    double dref = 0;
    if (allocate_states(table->hist, 256, 1024, fref) == SH_OK)
        for (int u = 0; u < 256; ++u)
            if (table->hist[u]) {
                const double p = table->hist[u] / dN;
                dref += p * std::log2(p / (fref[u] / 1024.0));
            }
    out->H = H;
    out->H_P = HP;
    out->D_KL = dkl;
    out->sum_Pw = pw;
    out->cl_thm1 = HP + dkl + pw;
    out->H_p_given_P = H - HP;
    out->dkl_tans_ref = dref;
    out->cl_tans_ref = H + dref;
    if (n > 0) {
        out->payload_bps = (double)payload_bits / (double)n;
        out->container_bps = 8.0 * (double)container_bytes / (double)n;
        out->csr = (double)container_bytes / (double)n;
    }
    if (H > 0) {
        out->pct_payload_over_H = (out->payload_bps - H) / H * 100.0;
        out->pct_container_over_H = (out->container_bps - H) / H * 100.0;
        out->pct_thm1_over_H = (out->cl_thm1 - H) / H * 100.0;
    }
    return SH_OK;
}

sh_status sh_stats_batch(const sh_table* tables, uint32_t nseg, const uint64_t* n,
                         const uint64_t* payload_bits, const uint64_t* container_bytes,
                         sh_stats_t* out) {
    if (nseg == 0) return SH_OK;
    if (!tables || !out) return SH_ERR_INVALID_ARG;
    sh_status first = SH_OK;
    for (uint32_t i = 0; i < nseg; ++i) {
        const sh_status st = sh_stats(&tables[i], n ? n[i] : 0, payload_bits ? payload_bits[i] : 0,
                                      container_bytes ? container_bytes[i] : 0, &out[i]);
        if (st != SH_OK && first == SH_OK) first = st;
    }
    return first;
}

}  // extern "C"
