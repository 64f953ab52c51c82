/*
 * kvq.h -- C ABI of the layer-wise mixed-precision KV-cache library for
 * MI355X (gfx950).
 *
 * The library keeps a decode KV cache quantized at a static per-layer
 * (key bits, value bits) pair chosen offline -- K8V4, K4V2, K8V8 and the
 * like -- and runs split-KV decode attention straight from the packed
 * codes. Sources of each operation are named on its declaration; the pages
 * cited are: the KVTuner summary page (scime atlas), the "Mixed-precision
 * KV-cache quantization per-layer sensitivity" notes page, the TriAxialKV
 * notes page and the KVSplit Show HN thread.
 *
 * Conventions
 *  - All device buffers (cache, inputs, outputs, workspace, page tables) are
 *    owned by the caller. The library never allocates device memory and keeps
 *    no state between calls except the optional timer below.
 *  - Every call checks its host-side arguments first and returns a status
 *    (KVQ_OK = 0, negative on error; kvq_last_error() gives a message, per
 *    thread). Nothing throws or aborts across the ABI. Kernels run
 *    asynchronously on the given stream (a hipStream_t; NULL = the null
 *    stream).
 *  - Values that live on the device (sequence lengths, page ids) are checked
 *    before every write: a length past the planned capacity, or a page-table
 *    entry that is out of range or names a page of the wrong pool, makes the
 *    kernel skip that write, so no kernel writes outside the cache region of
 *    the layer it was given. Reads trust them: a decode over a bad page table
 *    reads whatever the ids point at.
 *  - fp16 data is passed as uint16_t bit patterns (IEEE binary16).
 *  - head_dim is 128 and the quantization group is 32 (elements of a group:
 *    32 tokens of one channel for per-channel keys, 32 channels of one token
 *    otherwise).
 */
#ifndef KVQ_H
#define KVQ_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define KVQ_MAX_LAYERS 256
#define KVQ_HEAD_DIM 128
#define KVQ_GROUP 32

/* status codes */
#define KVQ_OK 0
#define KVQ_ERR_INVALID_ARG (-1) /* a null pointer, a size out of range, a bad layer index */
#define KVQ_ERR_UNSUPPORTED (-2) /* a bit-width, axis or shape the library does not implement */
#define KVQ_ERR_CAPACITY (-3)    /* the request would exceed the planned cache capacity */
#define KVQ_ERR_WORKSPACE (-4)   /* the workspace is too small */
#define KVQ_ERR_HIP (-5)         /* a HIP runtime call failed (message has the HIP error) */

/* quantization axis */
#define KVQ_AXIS_CHANNEL 0 /* one scale/zero per channel per 32-token group (keys) */
#define KVQ_AXIS_TOKEN 1   /* one scale/zero per token per 32-channel group */

/* output dtypes */
#define KVQ_OUT_F16 0
#define KVQ_OUT_F32 1

typedef void *kvq_stream_t; /* a hipStream_t */

/* Cache geometry shared by all layers. */
typedef struct kvq_shape {
    int32_t num_q_heads;  /* Hq */
    int32_t num_kv_heads; /* Hkv; Hq must be a multiple, G = Hq / Hkv <= 16 */
    int32_t head_dim;     /* must be 128 */
    int32_t group_size;   /* must be 32 */
    int32_t max_batch;    /* requests the cache holds */
    int32_t max_tokens;   /* contiguous mode: token capacity of each request */
    int32_t page_tokens;  /* 0 = contiguous streams; 16 = paged INT2/INT4 pool */
    int32_t int2_pages;   /* paged: pages in the INT2 region (even) */
    int32_t int4_pages;   /* paged: pages in the INT4 region */
    int32_t reserved;
} kvq_shape;

/* One entry of the static per-layer map. Bits are 2, 4, 8 or 16 (16 = fp16
 * passthrough, i.e. a layer left unquantized). v_axis must be
 * KVQ_AXIS_TOKEN. */
typedef struct kvq_layer_cfg {
    int32_t k_bits;
    int32_t v_bits;
    int32_t k_axis;
    int32_t v_axis;
} kvq_layer_cfg;

/* Byte geometry of one layer, filled by kvq_plan_layers. */
typedef struct kvq_layer_plan {
    int32_t k_bits, v_bits, k_axis, v_axis;
    uint64_t offset;          /* start of the layer region in the cache buffer */
    uint64_t bytes;           /* size of the layer region */
    uint64_t record_bytes;    /* one 32-token group record */
    uint64_t groups_cap;      /* contiguous: records per stream */
    uint64_t stream_bytes;    /* contiguous: bytes per (request, KV head) stream */
    uint64_t tail_offset;     /* contiguous: tail record inside a stream */
    uint64_t int4_offset;     /* paged: start of the INT4 region (the pool split) */
    uint64_t int2_page_bytes; /* paged: one INT2 page, all KV heads */
    uint64_t int4_page_bytes; /* paged: one INT4 page, all KV heads */
} kvq_layer_plan;

/* Caller-owned, plain-old-data plan. */
typedef struct kvq_plan {
    kvq_shape shape;
    int32_t num_layers;
    int32_t reserved;
    uint64_t total_bytes; /* device bytes the cache buffer must have */
    double equiv_bits;    /* mean over layers of (k_bits + v_bits) / 2 */
    double int2_fraction; /* paged: int2_pages / (int2_pages + int4_pages) */
    kvq_layer_plan layers[KVQ_MAX_LAYERS];
} kvq_plan;

/* Paged-pool bookkeeping (device arrays, caller-owned). One page table per
 * request, shared by all layers (TriAxialKV page, "Facts": each request's
 * page table lists its INT2 pages before its INT4 pages). A page holds 16
 * tokens of every KV head. Page ids below shape.int2_pages are INT2 pages
 * (region at byte 0 of the layer, int2_page_bytes each); the others are INT4
 * pages (region at int4_offset, the pool split, int4_page_bytes each).
 * Entries 0 .. int2_len/16 - 1 hold the INT2 pages: a 32-token INT2 group
 * (keys per-channel, values per-token, 2 bits) takes an aligned pair, entry
 * 2i = its even id P and entry 2i+1 = P + 1. The next ceil(int4_len/16)
 * entries hold the INT4 pages (keys and values per-token, 4 bits), entry
 * int2_len/16 + t/16 holding INT4 token t. A request's tokens are its INT2
 * tokens, then its INT4 tokens. The appends check every entry they write
 * through (entry below max_pages_per_req; an INT2 pair id even and below
 * int2_pages; an INT4 id in [int2_pages, int2_pages + int4_pages)) and skip
 * the write otherwise; the decode passes read through the ids unchecked. */
typedef struct kvq_pages {
    const int32_t *page_table; /* [batch][max_pages_per_req] */
    int32_t max_pages_per_req;
    int32_t reserved;
    const int32_t *int2_len; /* [batch] tokens in INT2 page pairs, a multiple of 32 */
    const int32_t *int4_len; /* [batch] tokens in INT4 pages */
    const int32_t *int2_add; /* append only, nullable: [batch] how many of the new tokens
                                (the first ones, a multiple of 32) go to INT2 pages */
} kvq_pages;

/*
 * kvq_plan_layers -- turn the static per-layer (bK, bV) map into byte
 * offsets. Host only, pure, no HIP call.
 * The map is searched offline and applied as is, with no decision at run
 * time (notes page, "Facts": KVTuner's per-layer configuration is applied at
 * inference with no online decision overhead; KVTuner summary page,
 * "Approach"). Key and value bits are set separately (KVSplit thread:
 * separate key and value flags). A layer may be left at 16 bits, the way
 * vLLM excludes layers from KV quantization (notes page, "Facts").
 * Paged mode (shape.page_tokens = 16) needs every layer at
 * {2, 2, KVQ_AXIS_CHANNEL, KVQ_AXIS_TOKEN}: INT2 per-channel keys and
 * per-token values in the INT2 region; the INT4 region holds per-token keys
 * and values at 4 bits (TriAxialKV page, "Facts": quantizer and page-pool
 * bullets).
 *   shape, cfg[num_layers]: in; out: filled on success.
 *   Errors: INVALID_ARG (null, num_layers out of 1..KVQ_MAX_LAYERS, sizes
 *   <= 0), UNSUPPORTED (head_dim != 128, group_size != 32, bits not in
 *   {2,4,8,16}, v_axis != TOKEN, Hq not a multiple of Hkv or G > 16,
 *   page_tokens not 0 or 16, paged layer not K2V2).
 */
int kvq_plan_layers(const kvq_shape *shape, const kvq_layer_cfg *cfg, int32_t num_layers,
                    kvq_plan *out);

/*
 * kvq_quantize_append -- append n_new tokens to every request of one layer.
 * k_new, v_new: device fp16 [batch][Hkv][n_new][128].
 * Contiguous mode: seq_lens (device int32 [batch]) is each request's length
 * before the call. Every 32-token group that the new tokens complete is
 * quantized and packed (asymmetric min/max, group 32: TriAxialKV page,
 * "Facts", quantizer bullet; keys per-channel or per-token as planned, values
 * per-token); the tokens past the last full group are kept in fp16 in the
 * stream's tail record. The call does not advance seq_lens: the caller
 * does. A stream whose length would pass max_tokens is left unchanged.
 * Paged mode (pages != NULL, required for a paged plan; seq_lens is then
 * ignored): the first int2_add[r] new tokens of request r (a multiple of
 * 32; int2_add NULL = 0) are quantized as INT2 groups into the page pairs
 * that follow its int2_len[r] INT2 tokens; the others, each token on its
 * own, into INT4 page slots after its int4_len[r] INT4 tokens (TriAxialKV
 * page, "Facts": leftover INT2 tokens go through the INT4 per-token path).
 * The page table must already hold its state after the call (the new INT2
 * pairs at entries int2_len/16 .., the INT4 pages after all INT2 entries).
 * A request whose int2_len or int2_add is not a multiple of 32 is left
 * unchanged. The caller advances int2_len/int4_len.
 *   Errors: INVALID_ARG (null pointers, layer, batch, n_new out of range,
 *   pages given for a contiguous plan or missing for a paged one),
 *   CAPACITY (n_new > max_tokens, or > 16 * max_pages_per_req), HIP.
 */
int kvq_quantize_append(const kvq_plan *plan, int32_t layer, void *cache, const uint16_t *k_new,
                        const uint16_t *v_new, const int32_t *seq_lens, int32_t batch,
                        int32_t n_new, const kvq_pages *pages, kvq_stream_t stream);

/* Workspace bytes kvq_decode_attention needs (split partials:
 * batch * Hq * splits * (128 + 1) fp32). num_splits = 0 means the count the
 * library would choose. Returns 0 on invalid arguments. */
size_t kvq_decode_workspace_bytes(const kvq_plan *plan, int32_t batch, int32_t max_seq_len,
                                  int32_t num_splits);

/* The split count kvq_decode_attention uses for num_splits = 0. */
int32_t kvq_decode_num_splits(const kvq_plan *plan, int32_t layer, int32_t batch,
                              int32_t max_seq_len);

/*
 * kvq_decode_attention -- one decode step of one layer: softmax attention of
 * q (device fp16 [batch][Hq][128]) over every cached token of each request.
 * Split-KV flash decoding: each split reads its share of the packed groups,
 * dequantizes in registers and keeps a running max and sum; a second pass
 * merges the splits by log-sum-exp (TriAxialKV page, "Facts": flash-decoding
 * splits merged by online log-sum-exp). The fp16 tail is part of the last
 * split. Query head h uses KV head h / (Hq / Hkv).
 *   seq_lens: device [batch] tokens per request (contiguous mode);
 *   max_seq_len: host upper bound of seq_lens (sizes the grid, no sync);
 *   softmax_scale: score = scale * q.k (usually 1/sqrt(128));
 *   out: device [batch][Hq][128], fp16 or fp32 (out_dtype);
 *   lse_out: device fp32 [batch][Hq] natural-log log-sum-exp, nullable;
 *   workspace: device, at least kvq_decode_workspace_bytes(...);
 *   num_splits: 0 = automatic, else 1..1024.
 * A request with no tokens gets out = 0 and lse = -inf.
 * Paged mode (pages != NULL): lengths come from pages->int2_len/int4_len and
 * seq_lens is ignored; max_seq_len bounds int2_len + int4_len. Each split
 * reads either INT2 groups or INT4 page pairs of one request, never both
 * (TriAxialKV page, "Facts": INT2 pointers first give bitwidth-homogeneous
 * splits), so a paged decode uses at least 2 splits and at most 256 groups
 * of 32 tokens per split: num_splits >= 2 and
 * (ceil(max_seq_len/32) + num_splits - 2) / (num_splits - 1) <= 256.
 *   Errors: INVALID_ARG (including the split limits above), CAPACITY
 *   (max_seq_len > max_tokens, or > 16 * max_pages_per_req), WORKSPACE, HIP.
 */
int kvq_decode_attention(const kvq_plan *plan, int32_t layer, const void *cache,
                         const uint16_t *q, const int32_t *seq_lens, int32_t batch,
                         int32_t max_seq_len, float softmax_scale, void *out, int32_t out_dtype,
                         float *lse_out, void *workspace, size_t workspace_bytes,
                         int32_t num_splits, const kvq_pages *pages, kvq_stream_t stream);

/*
 * kvq_decode_attention_noalloc -- kvq_decode_attention for callers that
 * cannot allocate device memory (code under stream capture, tight serving
 * loops, harnesses that forbid allocation): the same result, from the same
 * kernels, with the split partials kept in a 16 MiB array of device memory
 * that the library holds (one per GPU, until the process ends) instead of a
 * caller-given workspace. It allocates nothing. Calls that overlap on one GPU
 * (running at the same time on different streams) share that array and race.
 *   Arguments as in kvq_decode_attention, without workspace and
 *   workspace_bytes.
 *   Errors: those of kvq_decode_attention, and WORKSPACE when the partials
 *   (kvq_decode_workspace_bytes(plan, batch, max_seq_len, num_splits)) would
 *   need more than 16 MiB.
 */
int kvq_decode_attention_noalloc(const kvq_plan *plan, int32_t layer, const void *cache,
                                 const uint16_t *q, const int32_t *seq_lens, int32_t batch,
                                 int32_t max_seq_len, float softmax_scale, void *out,
                                 int32_t out_dtype, float *lse_out, int32_t num_splits,
                                 const kvq_pages *pages, kvq_stream_t stream);

/*
 * kvq_append_decode_attention -- one decode step of one layer with its token
 * append fused in: the same result, in the cache and in out/lse_out, as
 * kvq_quantize_append with n_new = 1 followed by kvq_decode_attention with
 * every length one larger, in one split pass (plus the merge pass when
 * there are several splits). The workgroup whose split holds the new
 * token's place appends it before any wave reads that place: into the fp16
 * tail record, or, when it completes a 32-token group, by quantizing and
 * packing that group (TriAxialKV page, "Facts", quantizer bullet, as in
 * kvq_quantize_append); in a paged pool, into the request's INT4 page as a
 * per-token INT4 token (TriAxialKV page, "Facts": decoded tokens take the
 * INT4 per-token path). This saves the append launch of every decode step.
 *   k_new, v_new: device fp16 [batch][Hkv][1][128], the new token;
 *   seq_lens: device [batch] tokens per request BEFORE the append (the
 *     caller advances them afterwards, as with kvq_quantize_append); a
 *     stream at max_tokens is left unchanged and attended as it is;
 *   pages: NULL for a contiguous plan; for a paged plan, int4_len counts
 *     the INT4 tokens BEFORE the append (the caller advances it) and
 *     int2_add must be NULL; seq_lens is then ignored;
 *   max_seq_len: host bound of the lengths + 1 (at least 1);
 *   q, softmax_scale, out, out_dtype, lse_out, workspace, num_splits: as in
 *     kvq_decode_attention (workspace sized by kvq_decode_workspace_bytes
 *     with the same max_seq_len; a paged pool has its split limits).
 *   Errors: INVALID_ARG, CAPACITY (max_seq_len > capacity), WORKSPACE, HIP.
 */
int kvq_append_decode_attention(const kvq_plan *plan, int32_t layer, void *cache,
                                const uint16_t *k_new, const uint16_t *v_new, const uint16_t *q,
                                const int32_t *seq_lens, int32_t batch, int32_t max_seq_len,
                                float softmax_scale, void *out, int32_t out_dtype, float *lse_out,
                                void *workspace, size_t workspace_bytes, int32_t num_splits,
                                const kvq_pages *pages, kvq_stream_t stream);

/* Workspace bytes kvq_prefix_attention needs: 0 when it uses one split, else
 * batch * chunk * Hq * splits * (128 + 1) fp32. num_splits = 0 means the
 * count the library would choose. Returns 0 on invalid arguments too. */
size_t kvq_prefix_workspace_bytes(const kvq_plan *plan, int32_t batch, int32_t chunk,
                                  int32_t max_seq_len, int32_t num_splits);

/*
 * kvq_prefix_attention -- chunked prefill against a quantized cache: softmax
 * attention of a chunk of new query tokens over every token already cached
 * for the request (the prefix: packed groups and fp16 tail, as stored), with
 * no mask, since the whole prefix precedes the chunk. Its (out, lse) is the
 * prefix part of the chunk's attention; the chunk's own causal part (its
 * fp16 K and V, which kvq_quantize_append then stores) merges with it by
 * log-sum-exp: o = (e^lse_p o_p + e^lse_c o_c) / (e^lse_p + e^lse_c). Each
 * packed group is dequantized once per 256 query rows (fmaf(code, scale,
 * zero) as in kvq_dequantize: asymmetric groupwise codes, per-channel or
 * per-token keys, per-token values, KIVI and KVTuner summary pages) and
 * multiplied on the matrix cores; the prefix may be split as in flash
 * decoding (TriAxialKV page, "Facts": splits merged by online log-sum-exp).
 *   q: device fp16 [batch][chunk][Hq][128], the chunk's queries;
 *   chunk: query tokens a request (the same for every request), >= 0;
 *   seq_lens: device [batch] cached tokens per request (the prefix length);
 *   max_seq_len: host upper bound of seq_lens;
 *   out: device fp32 [batch][chunk][Hq][128];
 *   lse_out: device fp32 [batch][chunk][Hq] natural-log log-sum-exp,
 *     nullable; a request with an empty prefix gets out = 0, lse = -inf;
 *   workspace: device, kvq_prefix_workspace_bytes(...) bytes (may be NULL
 *     when that is 0); num_splits: 0 = automatic, else 1..1024;
 *   cache, q, out and workspace 16-byte aligned.
 * Query head h of a token uses KV head h / (Hq / Hkv).
 * Paged mode (pages != NULL, required for a paged plan; seq_lens ignored):
 * the prefix is each request's INT2 tokens then its INT4 tokens
 * (pages->int2_len, int4_len), as kvq_decode_attention reads them; any split
 * count is allowed.
 *   Errors: INVALID_ARG (batch * chunk * Hq > 2^26 included; pages given for a
 *   contiguous plan or missing for a paged one), CAPACITY (max_seq_len past the
 *   capacity), WORKSPACE, HIP.
 */
int kvq_prefix_attention(const kvq_plan *plan, int32_t layer, const void *cache,
                         const uint16_t *q, int32_t chunk, const int32_t *seq_lens,
                         int32_t batch, int32_t max_seq_len, float softmax_scale, float *out,
                         float *lse_out, void *workspace, size_t workspace_bytes,
                         int32_t num_splits, const kvq_pages *pages, kvq_stream_t stream);

/* Workspace bytes kvq_chunk_prefill_attention needs: batch * chunk * Hq *
 * (splits + 1) * (128 + 1) fp32 (the prefix splits' partials and the chunk's
 * own). num_splits = 0 means the count the library would choose. Returns 0 on
 * invalid arguments. */
size_t kvq_chunk_prefill_workspace_bytes(const kvq_plan *plan, int32_t batch, int32_t chunk,
                                         int32_t max_seq_len, int32_t num_splits);

/*
 * kvq_chunk_prefill_attention -- the whole attention of a prefill chunk that
 * follows a quantized cache: every query row (chunk token i, query head)
 * attends to the request's cached prefix as stored (packed groups and fp16
 * tail, no mask) and, causally, to the chunk's own fp16 tokens 0 .. i (the
 * chunk is quantized only when kvq_quantize_append later stores it). Three
 * launches: the prefix pass of kvq_prefix_attention, a causal pass over the
 * chunk's keys and values (matrix cores, fp16 operands), and the log-sum-exp
 * merge of the prefix splits and the chunk part (TriAxialKV page, "Facts":
 * partial attentions merged by online log-sum-exp). The result is softmax
 * attention over the union, one softmax.
 *   q: device fp16 [batch][chunk][Hq][128];
 *   k_chunk, v_chunk: device fp16 [batch][Hkv][chunk][128], the chunk's own
 *     keys and values;
 *   seq_lens, max_seq_len, softmax_scale: as in kvq_prefix_attention (a
 *     request with an empty prefix attends to its chunk only);
 *   out: device fp32 [batch][chunk][Hq][128]; lse_out: device fp32
 *     [batch][chunk][Hq], nullable;
 *   workspace: kvq_chunk_prefill_workspace_bytes(...) bytes (never 0 for a
 *     non-empty chunk); num_splits: 0 = automatic, else 1..1023 (prefix
 *     splits);
 *   cache, q, k_chunk, v_chunk, out and workspace 16-byte aligned;
 *   pages: as in kvq_prefix_attention (paged plans).
 *   Errors: INVALID_ARG, CAPACITY, WORKSPACE, HIP.
 */
int kvq_chunk_prefill_attention(const kvq_plan *plan, int32_t layer, const void *cache,
                                const uint16_t *q, const uint16_t *k_chunk,
                                const uint16_t *v_chunk, int32_t chunk, const int32_t *seq_lens,
                                int32_t batch, int32_t max_seq_len, float softmax_scale,
                                float *out, float *lse_out, void *workspace,
                                size_t workspace_bytes, int32_t num_splits,
                                const kvq_pages *pages, kvq_stream_t stream);

/*
 * kvq_dequantize -- the cache of one layer back in fp32, for checking:
 * k_out, v_out: device fp32 [batch][Hkv][max_seq_len][128]; token j of
 * request r is fmaf(code, scale, zero) for quantized tokens and the stored
 * fp16 value for tail tokens; rows at or past the request's length are not
 * written. The codes, scales and zero points are those of the asymmetric
 * groupwise quantizer (TriAxialKV page, "Facts", quantizer bullet: one
 * scale and zero point per group of 32, keys per-channel or per-token,
 * values per-token); a code maps back to code * scale + zero, taken as one
 * fused multiply-add (the pages give no dequantization formula; one
 * rounding makes this call exact and reproducible). Paged mode (pages != NULL; seq_lens ignored) lists each
 * request's INT2 tokens first, then its INT4 tokens.
 *   Errors: INVALID_ARG, CAPACITY, HIP.
 */
int kvq_dequantize(const kvq_plan *plan, int32_t layer, const void *cache,
                   const int32_t *seq_lens, int32_t batch, int32_t max_seq_len, float *k_out,
                   float *v_out, const kvq_pages *pages, kvq_stream_t stream);

/* Alignment: the kernels read the cache, k_new, v_new, q and the split
 * partials in the workspace, and write out, in 16-byte pieces (an fp16 out
 * in 8-byte pieces); a call given one of them not 16-byte aligned returns
 * INVALID_ARG. */

/* Message of the last failed call on this thread ("" if none). */
const char *kvq_last_error(void);

/*
 * Optional kernel timer (HIP events recorded around each kernel launch, on
 * the launch stream). kvq_timer_start(capacity) clears and arms it for up to
 * `capacity` launches per kind; kvq_timer_read(kind, ...) synchronizes the
 * recorded events and returns the summed milliseconds and the launch count
 * for a kind (0 = append, 1 = decode split pass, 2 = merge pass, 3 = prefix
 * split pass);
 * kvq_timer_stop() disarms it and frees the events.
 */
int kvq_timer_start(int32_t capacity);
int kvq_timer_read(int32_t kind, double *total_ms, int32_t *launches);
int kvq_timer_stop(void);

#ifdef __cplusplus
}
#endif

#endif /* KVQ_H */
