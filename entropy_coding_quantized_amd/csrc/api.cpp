// C ABI of libshannonic.so (declared in include/shannonic.h): argument checks, table
// derivation for the kernels, workspace layout and launches.
#include <hip/hip_runtime.h>

#include <cmath>
#include <cstring>
#include <vector>

#include "codec_internal.hpp"

namespace shn {
sh_status allocate_states(const uint64_t* count, uint32_t K, uint32_t L, uint16_t* f);
}

using namespace shn;

namespace {

bool gpu_params_ok(const sh_params* p) {
    return p && p->K >= 1 && p->K <= 256 && p->log2_L >= 1 && p->log2_L <= (uint32_t)kMaxLog2LGpu &&
           p->streams == (uint32_t)kLanes && p->chunk_symbols >= 32 &&
           p->chunk_symbols <= kMaxChunk && p->chunk_symbols % 32 == 0;
}

bool aligned(const void* p, uintptr_t a) { return ((uintptr_t)p & (a - 1)) == 0; }

// container bytes at most, or 0 when the parameters are unusable
uint64_t bound_of(uint64_t n, const sh_params* p) {
    const uint64_t nch = n_chunks_of(n, p->chunk_symbols);
    uint64_t total = header_bytes(p->K) + 4 * (nch + 1);
    if (nch > 0) {
        total += 4ull * chunk_bound_dwords(p->chunk_symbols, p->log2_L) * (nch - 1);
        const uint64_t last = n - (nch - 1) * p->chunk_symbols;
        total += 4ull * chunk_bound_dwords((uint32_t)last, p->log2_L);
    }
    return total;
}

struct EncLayout {
    uint64_t slots_at, meta_at, bytes;
    uint32_t slot_dwords;
};

EncLayout enc_layout(uint64_t n, const sh_params* p) {
    EncLayout l;
    const uint64_t nch = n_chunks_of(n, p->chunk_symbols);
    const uint64_t pairs = (nch + 1) / 2;
    l.slot_dwords = encode_slot_dwords(p->chunk_symbols, p->log2_L);
    l.slots_at = 0;
    l.meta_at = (2 * pairs * l.slot_dwords * 4 + 255) / 256 * 256;
    l.bytes = l.meta_at + (8 * nch + 255) / 256 * 256 + 256;
    return l;
}

}  // namespace

extern "C" {

uint32_t sh_version(void) { return (1u << 16) | 0u; }

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
    return launch_histogram(d_x, n, d_hist, stream);
}

sh_status sh_table_from_histogram(const uint64_t* hist, const sh_params* params, sh_table* out) {
    if (!hist || !params || !out) return SH_ERR_INVALID_ARG;
    return table_from_histogram(hist, params->K, params->log2_L, out);
}

uint64_t sh_build_tables_workspace(void) { return 256 * sizeof(uint64_t); }

sh_status sh_build_tables(const int8_t* x, uint64_t n, int x_on_device, const sh_params* params,
                          void* d_ws, uint64_t ws_bytes, void* stream, sh_table* out) {
    if (!params || !out || (n > 0 && !x)) return SH_ERR_INVALID_ARG;
    uint64_t h[256] = {0};
    if (x_on_device) {
        if (!d_ws || ws_bytes < sh_build_tables_workspace()) return SH_ERR_BUFFER_TOO_SMALL;
        uint64_t* d_hist = (uint64_t*)d_ws;
        sh_status st = sh_histogram(x, n, d_hist, stream);
        if (st != SH_OK) return st;
        if (hipMemcpyAsync(h, d_hist, sizeof(h), hipMemcpyDeviceToHost, (hipStream_t)stream) !=
                hipSuccess ||
            hipStreamSynchronize((hipStream_t)stream) != hipSuccess)
            return SH_ERR_HIP;
    } else {
        for (uint64_t i = 0; i < n; ++i) h[(uint8_t)x[i] ^ 0x80]++;
    }
    return table_from_histogram(h, params->K, params->log2_L, out);
}

uint64_t sh_encode_bound(uint64_t n, const sh_params* params) {
    if (!gpu_params_ok(params)) return 0;
    return bound_of(n, params);
}

uint64_t sh_encode_workspace(uint64_t n, const sh_params* params) {
    if (!gpu_params_ok(params)) return 0;
    return enc_layout(n, params).bytes;
}

sh_status sh_encode(const sh_table* table, const sh_params* params, const int8_t* d_x,
                    uint64_t n, uint8_t* d_out, uint64_t out_cap, void* d_ws, uint64_t ws_bytes,
                    sh_encode_info* d_info, int32_t* d_status, void* stream) {
    if (!table || !params || !d_out || (n > 0 && !d_x)) return SH_ERR_INVALID_ARG;
    if (params->K < 1 || params->K > 256 || params->log2_L < 1) return SH_ERR_INVALID_ARG;
    if (!gpu_params_ok(params)) return SH_ERR_UNSUPPORTED;
    if (table->K != params->K || table->log2_L != params->log2_L) return SH_ERR_INVALID_ARG;
    if (check_table(*table, n == 0) != SH_OK) return SH_ERR_INVALID_ARG;
    if (n >= (1ull << 32)) return SH_ERR_UNSUPPORTED;
    const uint64_t bound = bound_of(n, params);
    if (bound > 0xFFFFFFFFull) return SH_ERR_UNSUPPORTED;
    if (out_cap < bound) return SH_ERR_BUFFER_TOO_SMALL;
    const EncLayout lay = enc_layout(n, params);
    if (!d_ws || ws_bytes < lay.bytes) return SH_ERR_BUFFER_TOO_SMALL;
    if (!aligned(d_x, 16) || !aligned(d_out, 4) || !aligned(d_ws, 256) ||
        !aligned(d_info, 8) || !aligned(d_status, 4))
        return SH_ERR_INVALID_ARG;

    const uint32_t C = params->chunk_symbols, R = params->log2_L, L = 1u << R, K = params->K;
    const uint64_t nch = n_chunks_of(n, C);
    const uint32_t index_at = header_bytes(K);

    EncodeArgs e;
    std::memset(&e, 0, sizeof(e));
    if (n > 0) {
        SlotTables st;
        if (derive_slots(*table, &st) != SH_OK) return SH_ERR_INVALID_ARG;
        // value entries: bias_s, and o | w << 8 | (start_s + 512) << 16 | (f_s == 0) << 31
        for (uint32_t s = 0; s < K; ++s) {
            const uint32_t f = table->freq[s];
            const uint32_t width = table->lo[s + 1] - table->lo[s];
            const uint32_t w = ceil_log2_u32(width);
            int32_t bias = 0, start = -(int32_t)L;
            if (f > 0) {
                const uint32_t m = floor_log2_u32(f);
                bias = (int32_t)((R - m) << (R + 1)) - (int32_t)(f << (R - m));
                start = (int32_t)st.cum[s] - (int32_t)f;
            }
            for (uint32_t u = table->lo[s]; u < table->lo[s + 1]; ++u) {
                e.vt[2 * u] = (uint32_t)bias;
                e.vt[2 * u + 1] = (u - table->lo[s]) | (w << 8) | ((uint32_t)(start + 512) << 16) |
                                  (f == 0 ? 0x80000000u : 0u);
            }
        }
        for (uint32_t i = 0; i < L; ++i) e.es[i] = (uint8_t)st.enc[i];
    }
    e.x = d_x;
    e.slots = (uint32_t*)((uint8_t*)d_ws + lay.slots_at);
    e.meta = (uint32_t*)((uint8_t*)d_ws + lay.meta_at);
    e.status = d_status;
    e.n = n;
    e.C = C;
    e.R = R;
    e.L = L;
    e.n_chunks = (uint32_t)nch;
    e.slot_dwords = lay.slot_dwords;

    IndexArgs ix;
    std::memset(&ix, 0, sizeof(ix));
    ix.meta = e.meta;
    ix.out = d_out;
    ix.info = d_info;
    ix.n = n;
    ix.n_chunks = (uint32_t)nch;
    ix.slot_dwords = lay.slot_dwords;
    ix.index_at = index_at;
    ix.hdr_dwords = index_at / 4;
    write_header(*table, n, C, (uint32_t)kLanes, nch, ix.hdr);

    CompactArgs cp;
    cp.slots = e.slots;
    cp.meta = e.meta;
    cp.out = d_out;
    cp.n_chunks = (uint32_t)nch;
    cp.slot_dwords = lay.slot_dwords;
    cp.index_at = index_at;
    cp.payload_at = index_at + 4 * (uint32_t)(nch + 1);
    return launch_encode(e, ix, cp, stream);
}

sh_status sh_decode(const sh_table* table, const sh_params* params, const uint8_t* d_in,
                    uint64_t in_nbytes, int8_t* d_y, uint64_t n, int32_t* d_status,
                    void* stream) {
    if (!table || !params || !d_in || (n > 0 && !d_y)) return SH_ERR_INVALID_ARG;
    if (params->K < 1 || params->K > 256 || params->log2_L < 1) return SH_ERR_INVALID_ARG;
    if (!gpu_params_ok(params)) return SH_ERR_UNSUPPORTED;
    if (table->K != params->K || table->log2_L != params->log2_L) return SH_ERR_INVALID_ARG;
    if (check_table(*table, n == 0) != SH_OK) return SH_ERR_INVALID_ARG;
    if (n >= (1ull << 32) || in_nbytes > 0xFFFFFFFFull) return SH_ERR_UNSUPPORTED;
    if (!aligned(d_in, 4) || !aligned(d_status, 4)) return SH_ERR_INVALID_ARG;

    const uint32_t C = params->chunk_symbols, R = params->log2_L, L = 1u << R, K = params->K;
    const uint64_t nch = n_chunks_of(n, C);
    const uint32_t index_at = header_bytes(K);
    const uint64_t payload_at = index_at + 4 * (nch + 1);
    if (in_nbytes < payload_at) return SH_ERR_CORRUPT_STREAM;
    if (n == 0) return SH_OK;

    SlotTables st;
    if (derive_slots(*table, &st) != SH_OK) return SH_ERR_INVALID_ARG;
    DecodeArgs a;
    std::memset(&a, 0, sizeof(a));
    for (uint32_t i = 0; i < L; ++i) {
        const uint32_t s = st.range[i];
        const uint32_t width = table->lo[s + 1] - table->lo[s];
        const uint32_t w = ceil_log2_u32(width);
        a.dec[2 * i] = (w + st.nb[i]) | ((uint32_t)st.next[i] * 8u << 16);
        a.dec[2 * i + 1] = w | (((uint32_t)(table->lo[s] - 128) & 0xFFu) << 8) | ((width - 1) << 16);
    }
    write_header(*table, n, C, (uint32_t)kLanes, nch, a.hdr);
    a.hdr_dwords = index_at / 4;
    a.in = d_in;
    a.out = d_y;
    a.status = d_status;
    a.in_nbytes = in_nbytes;
    a.n = n;
    a.payload_at = (uint32_t)payload_at;
    a.index_at = index_at;
    a.C = C;
    a.R = R;
    a.L = L;
    a.n_chunks = (uint32_t)nch;
    return launch_decode(a, stream);
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

}  // extern "C"
