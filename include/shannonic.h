/*
 * shannonic.h -- C ABI of the MI355X (gfx950) Shannonic codec library, libshannonic.so.
 *
 * Method: "Shannonic: Efficient Entropy-Optimal Compression for ML Workloads" (MLSys 2026),
 * talk notes.  An offline step histograms an 8-bit tensor and splits the 256-value
 * alphabet into K contiguous ranges by dynamic programming ("Preprocessing: range
 * selection by dynamic programming", paper section 4.1).  Every value is then coded as
 * (range index s, offset o): s goes through a tabled-ANS coder with L = 2^log2_L states,
 * o is written as w_s = ceil(log2 |range s|) raw bits ("Runtime encoding/decoding", paper
 * section 4.2, Algorithm 2).  Theorem 1 (paper section 4) gives the expected rate.
 *
 * Conventions shared by every call:
 *   - Values are int8.  The coder works on u = x + 128 (offset binary, so ranges are
 *     contiguous in value).
 *   - Pointers named d_* are device (HBM) pointers; all others are host pointers.
 *   - stream is a hipStream_t (0 = the null stream).  Device work is enqueued on it and
 *     the call returns without waiting, except where a host result needs device data
 *     or a host buffer is copied (sh_build_tables with x_on_device != 0,
 *     sh_table_to_device and sh_tables_from_device wait for the stream).
 *   - The library allocates no device memory and keeps no global state: the caller owns
 *     every buffer, and sizes of the workspaces are exported.  Calls are thread-safe.
 *   - Argument errors are returned synchronously.  Errors found by the GPU (a corrupt
 *     stream, a value whose range holds no tANS state) are written to *d_status with an
 *     atomic compare-and-swap from 0, so the first error wins; the caller zeroes
 *     *d_status beforehand and reads it back when convenient.
 *
 * Container (the bytes sh_encode writes and sh_decode reads), all integers little-endian:
 *   0   "SHN1", u8 version = 3, u8 log2_L, u16 K
 *   8   u64 n              number of values
 *   16  u32 chunk_symbols  C
 *   20  u32 streams        S (interleaved tANS lanes per chunk)
 *   24  u32 n_chunks       ceil(n / C)
 *   28  u32 index_at       header size = 4 * ceil((32 + 3K - 1) / 4)
 *   32  u16 freq[K]        tANS state count of every range (sum L)
 *   32+2K u8 lo[1..K-1]    first value u of ranges 1..K-1 (range 0 starts at 0, the
 *                          last ends at 256); zero padding up to index_at
 *   index_at: u32 goff[G + 1], G = ceil(n_chunks / 64): the payload byte where chunk 64g
 *             starts; goff[G] = the payload's size in bytes.  Then u16 size[n_chunks],
 *             every chunk's size in units of 2^u bytes, u the smallest with
 *             ceil(B / 2^u) <= 65535 for B = ceil((min(S, C) log2_L + C (8 + log2_L)) / 8),
 *             the largest chunk a valid stream holds (u = 0 at the pages' parameters).
 *             Then a zero u16 when n_chunks is odd.  Chunk c starts at goff[c / 64] plus
 *             the sizes of the chunks before it in its group of 64.
 *   payload: the chunks back to back, then zero bytes up to a multiple of 4 (the
 *   container's end).  Chunk c holds values [c*C, c*C + n_c).  Value i of a chunk belongs
 *   to lane i mod S at step i div S.  The chunk is an LSB-first bit string (bit b is bit
 *   b mod 8 of byte b / 8): the initial tANS slot of each of its min(S, n_c) lanes in
 *   log2_L bits, in lane order, then every value's field in (step, lane) order, then zero
 *   bits up to a whole number of size units.  A field is the offset o in its low w_s bits
 *   and, above it, the nb state bits the decoder appends to the slot's base to reach the
 *   next state.  Every lane ends in slot 0.  A lane's last field is the offset alone: the
 *   encoder starts each lane in state L (slot 0), so the state bits of the last value are
 *   the low bits of L, all zero, and the decoder implies them.
 *   (Version 2 padded every chunk to 32-bit words with a u32 offset per chunk; version 1
 *   also wrote the last fields' state bits.  Both are framing choices: the pages fix what
 *   a chunk codes, not how chunks are laid out.)
 */
#ifndef SHANNONIC_H
#define SHANNONIC_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef int32_t sh_status;
#define SH_OK 0
#define SH_ERR_INVALID_ARG (-1)          /* a pointer, size or parameter is out of range   */
#define SH_ERR_UNSUPPORTED (-2)          /* valid, but outside what the GPU path handles    */
#define SH_ERR_SYMBOL_NOT_IN_TABLE (-3)  /* a value falls in a range with no tANS state     */
#define SH_ERR_CORRUPT_STREAM (-4)       /* the container is not a valid stream             */
#define SH_ERR_BUFFER_TOO_SMALL (-5)     /* output or workspace capacity below the bound    */
#define SH_ERR_HIP (-6)                  /* a HIP runtime call failed                       */

/* Codec parameters.  The GPU path supports 1 <= K <= 256, 1 <= log2_L <= 11 (tables with
 * fields of at most 16 bits, the widest range's offset bits plus log2_L; sh_encode and
 * sh_decode, which carry the table in their launch arguments, take log2_L <= 8),
 * streams 32, 64 or 128, and chunk_symbols a multiple of streams in [streams, 65536].  More
 * streams give a launch with few chunks more independent state machines at a framing cost
 * of about log2_L bits a stream and chunk; the fused matrix-vector decode takes 32.
 * The pages' configuration is K = 16, log2_L = 7 (530 B of codec state,
 * "Codec state footprint", paper section 4.1 and Appendix A). */
typedef struct {
    uint32_t K;
    uint32_t log2_L;
    uint32_t chunk_symbols;
    uint32_t streams;
} sh_params;

/* The canonical table of one tensor: a plain host struct, copyable and serialisable.
 * Everything the kernels use (rangeId, base, nb, start, bias, encTable, decTable) is
 * derived from lo[] and freq[] deterministically.  hist[] and n are kept for sh_stats. */
typedef struct {
    uint32_t K;
    uint32_t log2_L;
    uint16_t lo[257];    /* range k covers u in [lo[k], lo[k+1]); lo[0] = 0, lo[K] = 256 */
    uint16_t freq[256];  /* f_k, sum = L (all 0 only for an empty tensor)                  */
    uint64_t hist[256];  /* h[u] of the tensor the table was built from                    */
    uint64_t n;          /* sum of hist                                                   */
} sh_table;

/* Theorem-1 terms and the measured rates (paper sections 4 and 5), in bits/value. */
typedef struct {
    double H;                    /* H(X) of the histogram                              */
    double H_P;                  /* H(P) of the range probabilities P_k                */
    double D_KL;                 /* D_KL(P || Q), Q_k = f_k / L                         */
    double sum_Pw;               /* sum_k P_k w_k, offset bits                          */
    double cl_thm1;              /* H(P) + D_KL(P || Q) + sum_k P_k w_k                  */
    double H_p_given_P;          /* H(X) - H(P)                                         */
    double dkl_tans_ref;         /* D_KL(p || q) of plain tANS, 256 values, L = 1024     */
    double cl_tans_ref;          /* H(X) + dkl_tans_ref                                 */
    double payload_bps;          /* field bits / n                                      */
    double container_bps;        /* 8 * container bytes / n                             */
    double csr;                  /* container bytes / n                                 */
    double pct_payload_over_H;   /* (payload_bps - H) / H * 100                         */
    double pct_container_over_H; /* (container_bps - H) / H * 100                       */
    double pct_thm1_over_H;      /* (cl_thm1 - H) / H * 100                             */
} sh_stats_t;

/* What sh_encode reports, written to device memory. */
typedef struct {
    uint64_t container_bytes; /* bytes of the container written to d_out        */
    uint64_t payload_bits;    /* summed field bits (initial states and padding excluded) */
} sh_encode_info;

/* Library version (major << 16 | minor). */
uint32_t sh_version(void);

/* Static text for a status code. */
const char* sh_status_string(sh_status st);

/*
 * Histogram of n int8 values on the GPU (paper section 4.1: h[u] over [0, 255]).
 * d_x: device, n bytes.  d_hist: device, 256 uint64, overwritten (not accumulated).
 * Asynchronous on stream.
 */
sh_status sh_histogram(const int8_t* d_x, uint64_t n, uint64_t* d_hist, void* stream);

/*
 * The offline table build from a histogram, on the host (paper section 4.1): the
 * exactly-K-range DP split minimising the summed range-id and offset cost, then the
 * allocation of the L tANS states minimising D_KL(P || Q).  hist: host, 256 uint64 with
 * a total below 2^32.  Supports 1 <= K <= 256 and 1 <= log2_L <= 12.  Returns
 * SH_ERR_UNSUPPORTED when more ranges hold values than there are states.
 */
sh_status sh_table_from_histogram(const uint64_t* hist, const sh_params* params, sh_table* out);

/*
 * The table of one tensor: the offline step of "Preprocessing: range selection by dynamic
 * programming" (paper section 4.1) -- the histogram h[u], the exactly-K-range DP split, the
 * allocation of the L states, the spread and every derived entry.  x is device memory when
 * x_on_device != 0: the histogram and the whole table build run on the GPU (sh_build_tables_batch with one tensor; the table is
 * identical to sh_table_from_histogram's), x must be 16-byte aligned, params must be ones
 * the GPU path supports, d_ws must hold sh_build_tables_workspace() bytes (256-byte
 * aligned) and the call waits for the stream.  Otherwise x is host memory, counted and
 * built on the host (d_ws and stream unused).
 */
uint64_t sh_build_tables_workspace(void);
sh_status sh_build_tables(const int8_t* x, uint64_t n, int x_on_device, const sh_params* params,
                          void* d_ws, uint64_t ws_bytes, void* stream, sh_table* out);

/* Largest container sh_encode can produce for n values (every field at its maximum
 * length of 8 + log2_L bits), and the device workspace sh_encode needs.  0 on bad
 * parameters. */
uint64_t sh_encode_bound(uint64_t n, const sh_params* params);
uint64_t sh_encode_workspace(uint64_t n, const sh_params* params);

/*
 * Encode n int8 values (paper section 4.2, Algorithm 2) into a container.
 * d_x: device, n bytes.  d_out: device, out_cap >= sh_encode_bound(n, params) bytes.
 * d_ws: device workspace of ws_bytes >= sh_encode_workspace(n, params).
 * d_info: device sh_encode_info or NULL.  d_status: device int32 or NULL.
 * table->K and table->log2_L must equal params->K and params->log2_L.
 * A value in a range with f = 0 sets *d_status = SH_ERR_SYMBOL_NOT_IN_TABLE and the
 * container is then unusable.  Asynchronous on stream.
 */
sh_status sh_encode(const sh_table* table, const sh_params* params, const int8_t* d_x,
                    uint64_t n, uint8_t* d_out, uint64_t out_cap, void* d_ws, uint64_t ws_bytes,
                    sh_encode_info* d_info, int32_t* d_status, void* stream);

/*
 * Decode the container at d_in (device) into n int8 values (d_y, device): the decoder of
 * "Runtime encoding/decoding" (paper section 4.2) -- from the state X, decTable[X] gives the
 * range s and its state-bit count, the offset o is read in w_s raw bits, the value is
 * base[s] + o, and the state bits lead to the next state.  in_nbytes is
 * the number of readable bytes at d_in: at least the container's size (its chunk index
 * gives the payload's size), so the output buffer of sh_encode can be passed with its capacity and
 * no host round trip.  The container must have been written with this table and these
 * params; its header is checked on the GPU.  Any inconsistency -- header, chunk index, an offset outside its
 * range, a lane not ending in slot 0, bits past a chunk's end or non-zero padding, a
 * container end past in_nbytes -- sets
 * *d_status = SH_ERR_CORRUPT_STREAM (d_status may be NULL to skip reporting); d_y is
 * then unspecified, but no access leaves d_in[0, in_nbytes) or d_y[0, n).
 * Asynchronous on stream.
 */
sh_status sh_decode(const sh_table* table, const sh_params* params, const uint8_t* d_in,
                    uint64_t in_nbytes, int8_t* d_y, uint64_t n, int32_t* d_status,
                    void* stream);

/*
 * sh_encode for callers that cannot allocate device memory (code under HIP graph capture,
 * tight serving loops, harnesses that forbid allocation): the same arguments without the
 * workspace.  The workspace is a file-scope device array of
 * sh_encode_noalloc_scratch_bytes() (64 MiB) that the library holds on every GPU it runs on
 * until the process ends; its device address is taken on the first call on each device.
 * Tensors whose sh_encode_workspace() exceeds it are refused with SH_ERR_BUFFER_TOO_SMALL
 * (at K = 16, log2_L = 7: about 33 M values at 4,096 values a chunk, 34 M at 16,384).  The
 * call allocates nothing.  Every call on one GPU shares that GPU's array: calls that
 * overlap on one GPU (other streams, other host threads) race and must be serialised by
 * the caller.  Output, errors and asynchrony are sh_encode's.
 */
uint64_t sh_encode_noalloc_scratch_bytes(void);
sh_status sh_encode_noalloc(const sh_table* table, const sh_params* params, const int8_t* d_x,
                            uint64_t n, uint8_t* d_out, uint64_t out_cap,
                            sh_encode_info* d_info, int32_t* d_status, void* stream);

/* ---- device-resident tables and batches ---------------------------------------------
 *
 * A device table is the per-tensor state the kernels read, in device memory: the canonical
 * table (lo, freq, hist, n), its decode and encode entries and the container header that
 * goes with it.  It is sh_device_table_bytes() bytes, 16-byte aligned, and is written by
 * sh_build_tables_batch (on the GPU, nothing returns to the host) or by sh_table_to_device
 * (from a host sh_table).  Tables of a batch sit back to back: table i at
 * d_tables + i * sh_device_table_bytes().
 *
 * The batch calls take host arrays of nseg device pointers and sizes and cover all the
 * tensors in a few launches (tensors are grouped 48 to a launch), so a model's worth of
 * small tensors costs no more launches than one large one.
 */
uint64_t sh_device_table_bytes(void);

/*
 * The tables of "Preprocessing" (paper section 4.1) moved between host and device.
 * Upload a host table for params (K and log2_L must match) to d_table.  Waits for the
 * copy.  An empty table (n = 0) is accepted: it encodes and decodes only empty tensors.
 */
sh_status sh_table_to_device(const sh_table* table, const sh_params* params, void* d_table,
                             void* stream);

/*
 * Read count device tables (back to back at d_tables) into out[count] with one copy; waits
 * for the stream.  table_status[i] (host) gets the status the GPU table build recorded
 * for table i: SH_OK, or SH_ERR_UNSUPPORTED when more ranges hold values than there are
 * states or the tensor has 2^32 values or more (out[i] is then not a usable table), or
 * SH_ERR_CORRUPT_STREAM for bytes that do not form a table.  The call itself returns
 * SH_ERR_HIP if the copy fails, else SH_OK.
 */
sh_status sh_tables_from_device(const void* d_tables, uint32_t count, sh_table* out,
                                int32_t* table_status, void* stream);

/*
 * sh_tables_from_device for tables the caller has already copied to host memory (for
 * example with an asynchronous copy into pinned memory): tables points to count device-
 * table images, back to back, 4-byte aligned.  Host only; statuses as above.
 */
sh_status sh_tables_from_bytes(const void* tables, uint32_t count, sh_table* out,
                               int32_t* table_status);

/*
 * The offline table build of paper section 4.1, on the GPU, for nseg tensors: histogram,
 * the exactly-K-range DP split (same integer cost and tie rule as sh_table_from_histogram,
 * so the tables are identical), the state allocation, the spread and every derived entry.
 * d_x[i] (device, 16-byte aligned when n[i] > 0) holds n[i] < 2^32 values.  d_tables:
 * nseg device tables.  d_ws: device workspace, 256-byte aligned, of
 * sh_build_tables_batch_workspace(nseg) bytes.  Asynchronous on stream; a tensor whose
 * table cannot be built gets a status inside its table (see sh_tables_from_device), which
 * the batch encode and decode turn into errors.
 */
uint64_t sh_build_tables_batch_workspace(uint32_t nseg);
sh_status sh_build_tables_batch(const int8_t* const* d_x, const uint64_t* n, uint32_t nseg,
                                const sh_params* params, void* d_tables, void* d_ws,
                                uint64_t ws_bytes, void* stream);

/*
 * The encoder of "Runtime encoding/decoding" (paper section 4.2, Algorithm 2) for nseg
 * tensors with device tables (sh_encode, batched): tensor i (d_x[i], n[i] values) is
 * encoded with table i into d_out[i] (out_cap[i] >= sh_encode_bound(n[i]) bytes, 4-byte
 * aligned), and its sh_encode_info goes to d_info[i] (d_info may be NULL).  d_ws: device
 * workspace, 256-byte aligned, of sh_encode_batch_workspace(n, nseg, params) bytes, reused
 * by every launch of the batch.  Errors of any tensor go to the one *d_status: a value
 * outside its table (SH_ERR_SYMBOL_NOT_IN_TABLE), a table whose build failed
 * (SH_ERR_UNSUPPORTED), or a device table built for another K or log2_L than params
 * (SH_ERR_INVALID_ARG; that tensor's chunks are then coded empty).  Asynchronous on stream.
 * The batch is encoded in launches of up to 48 tensors, each a chunk kernel and then a
 * placement that moves the chunks to their offsets.  place_stream (may be NULL) is a second
 * stream of the caller's: when it is given, differs from stream and the batch takes more than
 * one launch, each launch's placement runs on it, beside the next launch's chunk kernel, and
 * the workspace holds two launch regions that the launches take in turn (the size
 * sh_encode_batch_workspace returns covers this; one region, half of it, suffices without
 * place_stream).  place_stream first waits for the work queued on stream before the call,
 * and stream waits for the last placement, so work queued on stream after the call sees
 * every container; work queued on place_stream after the call runs after the placements.
 * The call creates and releases its own events.
 */
uint64_t sh_encode_batch_workspace(const uint64_t* n, uint32_t nseg, const sh_params* params);
sh_status sh_encode_batch(const void* d_tables, const int8_t* const* d_x, const uint64_t* n,
                          uint32_t nseg, const sh_params* params, uint8_t* const* d_out,
                          const uint64_t* out_cap, void* d_ws, uint64_t ws_bytes,
                          sh_encode_info* d_info, int32_t* d_status, void* stream,
                          void* place_stream);

/*
 * The decoder of "Runtime encoding/decoding" (paper section 4.2) for nseg containers with
 * device tables (sh_decode, batched): container i (d_in[i], in_nbytes[i]
 * readable bytes) decodes into d_y[i] (n[i] values) with table i.  Every check of
 * sh_decode applies to every container; the first error of any goes to *d_status.
 * A device table built for another K or log2_L than params sets SH_ERR_INVALID_ARG.
 * A table that failed to build, or was built from no values, decodes no values.
 * Asynchronous on stream.
 */
sh_status sh_decode_batch(const void* d_tables, const uint8_t* const* d_in,
                          const uint64_t* in_nbytes, int8_t* const* d_y, const uint64_t* n,
                          uint32_t nseg, const sh_params* params, int32_t* d_status,
                          void* stream);

/*
 * Decode fused into its consumer: container i (as for sh_decode_batch, table i) holds a
 * row-major int8 matrix W of n[i] / cols rows and cols values a row, and the call adds
 * y[i][r] += sum_c W[r][c] * d_a[i][c] (int32, wrapping like int32 addition) for every
 * row r, without writing W anywhere: the decoded values go from the decoder's registers
 * into the products.  This is the use the Ecco summary page (section 3, the core technique,
 * and its discussion of GPU decoding pipelines) describes for entropy-coded caches,
 * decompression inside the kernels that consume the data, applied to this container with
 * a matrix-vector product as the consumer (an int8 weight matrix times an int8 activation
 * vector, or int8 keys times a query).
 * params->streams may be 32, 64 or 128: chunks of 32 streams go through the half-wavefront
 * decoder (log2_L <= 8), chunks of 64 or 128 through the row decoder, whose lanes take the
 * dot product of their packed values with the vector's bytes.
 * cols: a multiple of params->streams, at most 16384 (SH_ERR_UNSUPPORTED otherwise; 0 is
 * SH_ERR_INVALID_ARG); every n[i] a multiple of cols (SH_ERR_INVALID_ARG).  d_a[i]: device,
 * cols int8 values, 16-byte aligned; d_y[i]: device, n[i] / cols int32, 4-byte aligned, read
 * and written (zero it first for y = W a).  Rows may span chunks: each chunk adds its part
 * of a row with one atomic add per row (per half wavefront or row of lanes), so y[i] is exact
 * in any order.
 * Every check of sh_decode applies and the first error goes to *d_status; y[i] of a
 * container that fails them is unspecified.  Asynchronous on stream.
 */
sh_status sh_decode_matvec_batch(const void* d_tables, const uint8_t* const* d_in,
                                 const uint64_t* in_nbytes, const int8_t* const* d_a,
                                 int32_t* const* d_y, const uint64_t* n, uint32_t cols,
                                 uint32_t nseg, const sh_params* params, int32_t* d_status,
                                 void* stream);

/*
 * Streaming decode (the decoder of "Runtime encoding/decoding", paper section 4.2), for
 * tensors parked compressed in host memory: the data movement between memory tiers that
 * "Problem: data-movement bottleneck in ML workloads" (paper sections 1 and 2) names, here
 * a model's tensors streamed from host memory into HBM.  Container i (h_in[i], host,
 * in_nbytes[i] bytes, pinned for the copies to be asynchronous) is decoded with device
 * table i into d_y[i] (n[i] values).  Containers are copied to the device on copy_stream
 * into d_staging (256-byte aligned, staging_bytes), split into depth slots: groups of
 * consecutive containers that fit one slot go up together and are decoded by one launch
 * on stream, and a slot is refilled only after the decode that read it has finished, so
 * copies overlap decodes.  Every container must fit one slot (else
 * SH_ERR_BUFFER_TOO_SMALL); sh_decode_stream_staging gives the smallest staging size for
 * a depth.  The first copy waits for the work already queued on stream, so a staging area
 * may be reused by consecutive calls.  Checks and errors are sh_decode_batch's.
 * Asynchronous: the call only queues work on both streams (it creates and releases its own
 * events); synchronise stream.
 */
uint64_t sh_decode_stream_staging(const uint64_t* in_nbytes, uint32_t nseg, uint32_t depth);
sh_status sh_decode_stream(const void* d_tables, const uint8_t* const* h_in,
                           const uint64_t* in_nbytes, int8_t* const* d_y, const uint64_t* n,
                           uint32_t nseg, const sh_params* params, void* d_staging,
                           uint64_t staging_bytes, uint32_t depth, int32_t* d_status,
                           void* copy_stream, void* stream);

/*
 * Theorem-1 terms of a table and the measured rates of a container of n values, on the
 * host (paper section 4; %diff as in section 5).  The entropy terms use table->hist;
 * payload_bits and container_bytes come from sh_encode_info (pass n = 0 to get the table
 * terms only).
 */
sh_status sh_stats(const sh_table* table, uint64_t n, uint64_t payload_bits,
                   uint64_t container_bytes, sh_stats_t* out);

/*
 * sh_stats (Theorem 1, paper section 4; %diff of paper section 5) for nseg tables in one
 * call (a tensor with several tables, e.g. one per KV head).
 * tables: host array of nseg sh_table.  n, payload_bits, container_bytes: host arrays of
 * nseg values, or NULL for zeros.  out: host array of nseg sh_stats_t.  Returns the status
 * of the first table (in index order) that fails; every other entry is still filled.
 */
sh_status sh_stats_batch(const sh_table* tables, uint32_t nseg, const uint64_t* n,
                         const uint64_t* payload_bits, const uint64_t* container_bytes,
                         sh_stats_t* out);

#ifdef __cplusplus
}
#endif
#endif
