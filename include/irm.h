/*
 * irm.h - C ABI of the MLA position-independent KV path on MI355X (gfx950).
 *
 * The operations follow the Irminsul pages (arXiv:2605.05696):
 *   - an MLA KV row is a 512-wide position-free latent c_KV plus a 64-wide
 *     RoPE key slice k_r (gist.science summary, section 2.1; gentlecold.top
 *     article, section 4);
 *   - a registry hit stores (c_KV, k_r_base, p_src); placed at p_tgt it is
 *     reused with k_r = R(delta) k_r_base, delta = p_tgt - p_src, because
 *     R(delta) R(p_src) = R(p_tgt) (gist.science section 2.2; gentlecold.top
 *     sections 4 and 15);
 *   - segments are appended to the assembled cache in target order and
 *     positions below 32 are always freshly prefilled (gentlecold.top
 *     section 5 serve-path pseudocode and section 7; gist.science 2.2);
 *   - attention is the absorbed-matmul MLA form: score = q_lat . c_KV +
 *     q_rope . k_r, value = c_KV (gentlecold.top section 4).
 *
 * Conventions for every function:
 *   - Every call returns an irm_status; no exception crosses the ABI.  On a
 *     non-OK status irm_last_error() returns a message for the calling thread.
 *   - Validation errors are returned synchronously before any GPU work.
 *     Launch failures return IRM_EHIP; faults inside a kernel surface at the
 *     caller's next synchronisation of the stream.
 *   - "device" pointers are HIP device memory owned by the caller; "host"
 *     pointers are ordinary host memory.  The library never allocates device
 *     memory and never synchronises a stream.
 *   - `stream` is a hipStream_t passed as void* (NULL = the default stream).
 *   - bf16 tensors are IEEE bfloat16 bit patterns; all float->bf16 rounding
 *     on the GPU is round-to-nearest-even.
 *   - The KV pool is bf16 [pool_rows][576], row = [c_KV 512 | k_r 64]
 *     (1152 bytes, 16-byte aligned).
 */
#ifndef IRM_H
#define IRM_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  IRM_OK = 0,
  IRM_EINVAL = 1,       /* malformed argument or table entry */
  IRM_ERANGE = 2,       /* pool row, position or delta out of range */
  IRM_ELAYOUT = 3,      /* target positions not contiguous from 0 */
  IRM_ECARVEOUT = 4,    /* a registry (non-fresh) row below position 32 */
  IRM_EWORKSPACE = 5,   /* workspace missing or too small */
  IRM_EUNSUPPORTED = 6, /* shape the kernels do not support */
  IRM_EHIP = 7          /* HIP runtime error (launch, copy, device) */
} irm_status;

enum {
  IRM_D_LATENT = 512,   /* c_KV width */
  IRM_D_ROPE = 64,      /* k_r width: 32 interleaved pairs (2i, 2i+1) */
  IRM_ROW = 576,        /* pool / assembled row width in bf16 elements */
  IRM_CARVE_OUT = 32,   /* positions [0, 32) are never served from the registry */
  IRM_MAX_HEADS = 128
};

#define IRM_FRESH 1u    /* irm_chunk.flags: rows freshly prefilled at p_tgt */

/*
 * One chunk-table entry, built on the host.  Entries of a sequence are listed
 * in target order.  Row j (0 <= j < len) of the entry is assembled at
 * position p_tgt + j from pool row pool_row + j; its k_r is rotated by
 * delta = p_tgt - p_src (gentlecold.top section 5: one delta per segment).
 * A fresh entry (flags & IRM_FRESH) holds rows prefilled at p_tgt, is copied
 * verbatim and must have p_src == p_tgt.  An exact-prefix entry is a
 * non-fresh entry with p_src == p_tgt (delta 0, copied verbatim).
 * 20 bytes, no padding.
 */
typedef struct irm_chunk {
  uint32_t pool_row;
  uint32_t len;
  int32_t p_src;
  int32_t p_tgt;
  uint32_t flags;
} irm_chunk;

typedef struct irm_table irm_table; /* opaque; owned by the library */

/* Thread-local message for the last non-OK status of this thread ("" if none). */
const char* irm_last_error(void);

/*
 * Standard RoPE inverse frequencies for the 64-wide k_r slice:
 * inv_freq[i] = theta^(-2i/64), i = 0..31, in double precision.
 * The pages stress that the rotation must use the model's own rotary
 * frequencies (gentlecold.top section 11), so every entry point that rotates
 * takes the 32 frequencies themselves; this helper covers plain RoPE.
 * host out: inv_freq[32].  EINVAL if theta <= 1 or inv_freq is NULL.
 */
irm_status irm_rope_inv_freq(double theta, double* inv_freq);

/*
 * Standard RoPE inverse frequencies for a rotary slice of any even width:
 * inv_freq[i] = theta^(-2i/dim), i = 0 .. dim/2 - 1, in double precision
 * (for example the whole head_dim of a GQA/MHA key, which the comparison
 * path irm_gqa_rotate_gather turns; the pages insist that the rotation use
 * the model's own rotary frequencies: gentlecold.top article, section 11).
 * irm_rope_inv_freq(theta, f) equals irm_rope_inv_freq_dim(theta, 64, f).
 *   host out inv_freq[dim / 2].  EINVAL if theta <= 1 or not finite, dim odd,
 *   below 2 or above 4096, or inv_freq is NULL.
 */
irm_status irm_rope_inv_freq_dim(double theta, uint32_t dim, double* inv_freq);

/*
 * Validate a chunk table and build its device image in library-owned host
 * memory.  Makes no HIP call (usable without a GPU).
 *   host chunks[n_chunks]; host seq_first[n_seq + 1]: sequence s owns
 *   entries [seq_first[s], seq_first[s+1]); seq_first[0] == 0 and
 *   seq_first[n_seq] == n_chunks, nondecreasing.  An empty sequence is legal.
 *   pool_rows: rows in the pool this table will be used with (the kernels
 *   address at most 2^32 pool rows; larger values are treated as 2^32).
 * Checks, per entry in order, returning the first failure:
 *   unknown flag bits (EINVAL); len == 0 (EINVAL);
 *   pool_row + len > pool_rows (ERANGE);
 *   p_tgt != previous p_tgt + previous len, or != 0 for a sequence's first
 *   entry (ELAYOUT); p_tgt + len - 1 > INT32_MAX (ERANGE);
 *   fresh with p_src != p_tgt (EINVAL); non-fresh with p_tgt < 32 (ECARVEOUT);
 *   delta outside int32 (ERANGE).  Total rows over all sequences must stay
 *   below 2^31 (ERANGE).
 * Output row of (sequence s, position p) in every assembled buffer is
 * seq_base[s] + p, with seq_base the prefix sum of sequence lengths.
 * *out receives the handle; free it with irm_table_destroy.
 */
irm_status irm_table_create(const irm_chunk* chunks, uint32_t n_chunks,
                            const uint32_t* seq_first, uint32_t n_seq,
                            uint64_t pool_rows, irm_table** out);

/* Frees the handle.  The device buffer given to irm_table_upload stays the
 * caller's; destroy only after the stream is done with kernels using it. */
irm_status irm_table_destroy(irm_table* t);

/*
 * Sizes of a table (any pointer may be NULL):
 *   n_seq, n_chunks; total_rows = sum of lengths; max_seq_len;
 *   device_bytes = size of the device image irm_table_upload needs.
 */
irm_status irm_table_info(const irm_table* t, uint32_t* n_seq, uint32_t* n_chunks,
                          uint64_t* total_rows, uint32_t* max_seq_len,
                          size_t* device_bytes);

/*
 * How irm_rotate_gather works through a table (any pointer may be NULL):
 *   n_groups = work records (entries that start at the same pool row form a
 *   group, cut into records of at most 256 rows and 8 entries); n_items =
 *   one-wave work items of up to 8 rows; read_rows = pool rows one
 *   irm_rotate_gather call reads (each record's rows once, for all its
 *   entries; total_rows minus this is the chunk reuse the call exploits); host_bytes = bytes
 *   irm_table_upload copies to the device (the rest of device_bytes is
 *   written there by the table's own kernels).  Needs no GPU.
 */
irm_status irm_table_gather_stats(const irm_table* t, uint32_t* n_groups, uint64_t* n_items, uint64_t* read_rows,
                                  size_t* host_bytes);

/* host out seq_base[n_seq + 1]: first assembled row of each sequence. */
irm_status irm_table_seq_base(const irm_table* t, uint64_t* seq_base);

/*
 * Host-side expansion of the table, one value per assembled row (each array
 * host, [total_rows], any may be NULL): the pool row it is gathered from,
 * its delta (0 for fresh rows) and its fresh flag.  No HIP call.
 */
irm_status irm_table_expand_host(const irm_table* t, int64_t* pool_row, int32_t* delta,
                                 uint8_t* fresh);

/*
 * Copy the device image to dev_buf (device, dev_bytes >= device_bytes,
 * 256-byte aligned) on `stream` and compute, on the GPU in double precision,
 * cos and sin of delta * inv_freq[i] for every entry and pair (stored as
 * float).  host inv_freq[32].  The handle remembers dev_buf; every later call
 * taking this table reads it there, ordered after this call on the same
 * stream.  The host image stays valid until destroy, so the copy needs no
 * synchronisation by the caller.  EWORKSPACE if dev_bytes is too small.
 */
irm_status irm_table_upload(irm_table* t, const double* inv_freq, void* dev_buf,
                            size_t dev_bytes, void* stream);

/*
 * The device passes of irm_table_upload without its host-to-device copy: on
 * `stream`, rebuild the row map (one record per assembled row: pool row,
 * delta, entry) from the entries already in the uploaded device image, and
 * the per-entry cos/sin of delta * inv_freq[i] (as irm_table_set_rope), in
 * one kernel launch.
 * host inv_freq[32].  Requires an uploaded table (EINVAL otherwise); the
 * result is the same as that of irm_table_upload.  This is the per-batch
 * device work of a table whose image reached HBM by a copy made earlier or
 * on another stream.
 */
irm_status irm_table_prepare(irm_table* t, const double* inv_freq, void* stream);

/*
 * Recompute, on `stream`, the per-entry cos/sin of delta * inv_freq[i] of an
 * uploaded table (the trig pass irm_table_upload also runs), e.g. for another
 * model's rotary frequencies.  host inv_freq[32].  No host-to-device copy.
 */
irm_status irm_table_set_rope(irm_table* t, const double* inv_freq, void* stream);

/*
 * Device export of the gather map (device int64 pool_row[total_rows] and
 * int32 delta[total_rows], either may be NULL).  Requires an uploaded table.
 */
irm_status irm_table_gather_index(const irm_table* t, int64_t* pool_row, int32_t* delta,
                                  void* stream);

/*
 * Rotate-gather: assemble every sequence of the table into out_kv.
 *   device pool bf16 [pool_rows][576] (pool_rows >= the table's pool_rows);
 *   device out_kv bf16 [total_rows][576]: c_KV copied bit for bit; k_r
 *   copied bit for bit for fresh and delta == 0 rows, else R(delta) k_r_base
 *   computed in float and rounded to bf16;
 *   device kr_f32 optional float [total_rows][64]: the rotated k_r before
 *   rounding (NULL in production).
 * Buffers must not overlap.  Requires an uploaded table.  Entries that
 * start at the same pool row (a registry chunk several requests place) are
 * read from the pool once per call (once per 8 placements) and written to
 * every placement.
 */
irm_status irm_rotate_gather(const irm_table* t, const void* pool, uint64_t pool_rows,
                             void* out_kv, float* kr_f32, void* stream);

/*
 * Split-KV decode workspace size for a table, head count and split count
 * (n_splits == 0 picks the library default; the same rule is used by
 * irm_mla_decode).  *bytes receives the size (256-byte aligned pointer).
 */
irm_status irm_mla_decode_workspace(const irm_table* t, uint32_t n_heads, uint32_t n_splits,
                                    size_t* bytes);

/*
 * Absorbed MLA decode, one query token per sequence, over the cache the table
 * assembles, with k_r rotated on load (no assembled buffer is written).
 *   device q_latent bf16 [n_seq][n_heads][512]; device q_rope bf16
 *   [n_seq][n_heads][64] (already RoPE'd at the query position);
 *   device out bf16 [n_seq][n_heads][512]; device lse optional float
 *   [n_seq][n_heads] (natural-log sum of exp of the scaled scores);
 *   n_heads a multiple of 16, <= 128 (else EUNSUPPORTED); scale > 0 finite;
 *   n_splits: KV splits per sequence (0 = default); every sequence must hold
 *   at least one row (EINVAL).  At 64 or more heads (a multiple of 64), when
 *   the batch has more (sequence, split, 64-head block) triples than the
 *   device has compute units, one workgroup streams several consecutive
 *   splits as one softmax run, so the rounding order (not the result within
 *   float accuracy) depends on the device's compute-unit count; a given
 *   device, table and split count always give the same bits.
 *   device workspace of at least irm_mla_decode_workspace bytes (EWORKSPACE).
 * Each query attends to every row of its sequence.  Reused rows are turned
 * with the table's per-entry cos/sin (the values irm_rotate_gather applies,
 * from the last irm_table_upload / irm_table_set_rope on the stream) and
 * rounded to bf16 before the score product, so decoding the rotate-gather
 * output as fresh rows gives the same bits.
 */
irm_status irm_mla_decode(const void* q_latent, const void* q_rope, const irm_table* t,
                          const void* pool, uint64_t pool_rows, uint32_t n_heads,
                          uint32_t n_splits, float scale, void* out, float* lse,
                          void* workspace, size_t ws_bytes, void* stream);

/*
 * irm_mla_decode for callers that cannot allocate device memory (code under
 * HIP graph capture, tight serving loops, harnesses that forbid allocation):
 * the same computation, arguments and results as irm_mla_decode, without the
 * workspace arguments.  The split pass keeps its partial states in a device
 * array the library holds for each GPU until the process ends (64 MiB; its
 * device address is looked up on the first call on that GPU).  The call
 * allocates nothing: no hipMalloc, no hipFree, no allocating library call.
 *   Limit: n_seq * parts * n_heads * (512 + 2) * 4 bytes (each half rounded
 *   up to 256) must fit in 64 MiB, where parts is the number of partial
 *   states the split pass writes per sequence (n_splits, or fewer when one
 *   workgroup streams a run of splits); else EWORKSPACE, before any launch.
 *   The batched 64 x 8192 x 16-head and the 32 x 32768 x 128-head decodes fit.
 * Every call on a GPU shares that GPU's array: calls that may overlap on one
 * GPU (different streams without ordering between them) race and give wrong
 * results; order them on one stream.  No state carries over between calls
 * (every partial slot is written before it is read), so nothing needs
 * clearing.
 */
irm_status irm_mla_decode_noalloc(const void* q_latent, const void* q_rope, const irm_table* t,
                                  const void* pool, uint64_t pool_rows, uint32_t n_heads,
                                  uint32_t n_splits, float scale, void* out, float* lse, void* stream);

/*
 * Chunked tail-prefill for one sequence (the table must hold exactly one
 * sequence of N rows): n_q query tokens at positions q_pos0 .. q_pos0+n_q-1
 * attend causally (row t visible to query i iff t <= q_pos0 + i) over the
 * assembled cache, with k_r rotated on load (with the table's per-entry
 * cos/sin, as in irm_mla_decode).
 *   device q_latent bf16 [n_q][n_heads][512]; q_rope bf16 [n_q][n_heads][64];
 *   device out bf16 [n_q][n_heads][512]; lse optional float [n_q][n_heads].
 *   0 <= q_pos0, 1 <= n_q, q_pos0 + n_q <= N (ERANGE); n_heads a multiple of
 *   16, <= 128 (EUNSUPPORTED).
 */
irm_status irm_mla_prefill_tail(const void* q_latent, const void* q_rope, int32_t q_pos0,
                                uint32_t n_q, const irm_table* t, const void* pool,
                                uint64_t pool_rows, uint32_t n_heads, float scale,
                                void* out, float* lse, void* stream);

/*
 * GQA/MHA comparison path (the correction earlier position-independent
 * caching systems need; gist.science summary, section 1; gentlecold.top
 * article, sections 3-4): in GQA/MHA the position is folded into the full
 * key, so every reused row has the whole key of each KV head rotated by
 * delta (O(N d_K) per KV head), against MLA's 64-wide k_r slice.  Same chunk
 * table and deltas as irm_rotate_gather.
 *   Row layout: bf16 [K: n_kv_heads x head_dim | V: n_kv_heads x head_dim];
 *   device pool [pool_rows][2 * n_kv_heads * head_dim] (16-byte aligned);
 *   device out [total_rows][same width].  K is turned over the whole
 *   head_dim with the half-split pairing (element i with i + head_dim/2,
 *   angle delta * inv_freq[i], host inv_freq[head_dim/2], cos/sin in double
 *   per entry, the 2x2 rotation in float, RNE to bf16); fresh and delta-0
 *   rows and all of V are copied bit for bit.
 *   device ws[irm_gqa_workspace bytes] (16-byte aligned) holds the per-entry
 *   (cos, sin) table.  head_dim a multiple of 16 in [16, 256], n_kv_heads in
 *   [1, 256] (EUNSUPPORTED).
 */
irm_status irm_gqa_workspace(const irm_table* t, uint32_t head_dim, size_t* bytes);
irm_status irm_gqa_rotate_gather(const irm_table* t, const void* pool, uint64_t pool_rows, uint32_t n_kv_heads,
                                 uint32_t head_dim, const double* inv_freq, void* ws, size_t ws_bytes, void* out,
                                 void* stream);

/*
 * Chunked tail-prefill over an assembled cache (the output of
 * irm_rotate_gather for one sequence): the same causal absorbed MLA attention
 * as irm_mla_prefill_tail, with row r of kv at position r and no rotation
 * left to apply.  Assembling once and attending over the result serves every
 * query block from the same rotated rows, where irm_mla_prefill_tail turns
 * each row again for every block of four queries.
 *   device kv bf16 [kv_rows][576] (16-byte aligned); queries, out and lse as
 *   in irm_mla_prefill_tail; query i attends rows t <= q_pos0 + i.
 *   0 <= q_pos0, 1 <= n_q, q_pos0 + n_q <= kv_rows (ERANGE); kv_rows <= 2^32
 *   and n_heads a multiple of 16, <= 128 (EUNSUPPORTED).
 */
irm_status irm_mla_prefill_assembled(const void* q_latent, const void* q_rope, int32_t q_pos0,
                                     uint32_t n_q, const void* kv, uint64_t kv_rows, uint32_t n_heads,
                                     float scale, void* out, float* lse, void* stream);

/*
 * Non-absorbed MLA prefill, step 1: up-project the latent rows of an
 * assembled cache to a full key and value per head (gentlecold.top article,
 * section 4: key [W_UK c_KV, k_r], value from c_KV; section 13: a
 * non-absorbed model has to up-project c_KV at run time).
 *   device kv bf16 [kv_rows][576] (c_KV = the first 512; 16-byte aligned);
 *   device w_uk, w_uv bf16 [n_heads][128][512] (output feature, latent input;
 *   16-byte aligned); device out bf16 [n_heads][kv_rows][256] = per head and
 *   row [W_UK[h] c_KV | W_UV[h] c_KV] (16-byte aligned), float accumulation,
 *   RNE to bf16.  n_heads in [1, 128], kv_rows < 2^32 (EUNSUPPORTED).
 */
irm_status irm_mla_kv_upproj(const void* kv, uint64_t kv_rows, const void* w_uk, const void* w_uv,
                             uint32_t n_heads, void* out, void* stream);

/*
 * Non-absorbed MLA prefill, step 2: causal attention of every head with its
 * own key [k_nope (128) | k_r (64)] and value (128), k_r being the rotated
 * slice of the assembled row shared by all heads; score scale `scale`
 * (1/sqrt(192) for the 128 + 64 key).
 *   device q_nope bf16 [n_q][n_heads][128], q_rope bf16 [n_q][n_heads][64]
 *   (already RoPE'd at its position); kv as in irm_mla_kv_upproj (for k_r);
 *   kvh = that call's out; device out bf16 [n_q][n_heads][128]; lse float
 *   [n_q][n_heads] (natural log, optional).  Query i at q_pos0 + i attends
 *   rows t <= q_pos0 + i.  0 <= q_pos0, 1 <= n_q, q_pos0 + n_q <= kv_rows
 *   (ERANGE); n_heads in [1, 128], kv_rows < 2^32 (EUNSUPPORTED).
 */
irm_status irm_mla_prefill_nonabsorbed(const void* q_nope, const void* q_rope, int32_t q_pos0, uint32_t n_q,
                                       const void* kv, const void* kvh, uint64_t kv_rows, uint32_t n_heads,
                                       float scale, void* out, float* lse, void* stream);

/* ------------------------------------------------------------------------
 * Host chunk-table producer (no HIP call; usable without a GPU).
 *
 * The serve path of the pages splits a request's unmatched tail by
 * content-defined chunking (CDC), fingerprints every chunk with xxHash64 and
 * looks it up in a content registry: a hit at target position p is reused
 * with delta = p - p_src, a miss is prefilled and inserted as
 * (c_KV, k_r_base, p), and a segment starting below position 32 is always
 * prefilled (gentlecold.top article, section 5 pseudocode).  The chunker is a
 * rolling Gear hash over a 64-token window that cuts where its low 7 bits
 * meet the mask, chunks of about 128 tokens clamped to [32, 512]
 * (gentlecold.top section 6; gist.science summary, section 2.2).
 * ------------------------------------------------------------------------ */

/*
 * CDC parameters.  The Gear state is 64 bits: h = (h << 1) + gear(token)
 * mod 2^64, starting at 0 at the first token and rolling on across chunk
 * boundaries; gear(t) is the splitmix64 output for the state
 * seed + t * 0x9E3779B97F4A7C15 (the pages give no table; this one is ours).
 * A chunk ends after token i when it holds at least min_len tokens and
 * h & (2^mask_bits - 1) == 0, or when it holds max_len tokens; the last chunk
 * takes what remains.
 */
typedef struct irm_cdc_params {
  uint64_t seed;
  uint32_t mask_bits;       /* 1..63 */
  uint32_t min_len;         /* >= 1 */
  uint32_t max_len;         /* >= min_len */
  uint32_t fallback_window; /* 0: off; else the S1 fallback of irm_registry_assemble with windows of this many tokens */
} irm_cdc_params;

/* The values the pages fix: mask_bits 7, [min_len, max_len] = [32, 512]; seed 0;
 * S1 fallback off (the pages use 128-token windows when it is on). */
irm_status irm_cdc_params_default(irm_cdc_params* p);

/*
 * Chunk lengths of a token stream.
 *   host tokens[n] (token ids); host out lens[max_chunks]; *n_chunks receives
 *   the number of chunks (also when it exceeds max_chunks: ERANGE, nothing
 *   written).  EINVAL for bad parameters or NULL pointers.
 */
irm_status irm_cdc_split(const irm_cdc_params* p, const int32_t* tokens, uint64_t n, uint32_t* lens,
                         uint64_t max_chunks, uint64_t* n_chunks);

/* xxHash64 (per its specification) of host data[bytes] with the given seed. */
irm_status irm_xxh64(const void* data, uint64_t bytes, uint64_t seed, uint64_t* out);

/*
 * Content registry: fingerprint -> (pool_row, len, p_src), plus the counter
 * that allocates pool rows for freshly prefilled segments, starting at
 * first_free_row.  Host memory owned by the library; free with
 * irm_registry_destroy.  Not thread-safe: one call at a time per registry.
 */
typedef struct irm_registry irm_registry;
irm_status irm_registry_create(uint64_t first_free_row, irm_registry** out);
irm_status irm_registry_destroy(irm_registry* r);
irm_status irm_registry_info(const irm_registry* r, uint64_t* n_entries, uint64_t* next_free_row);

/*
 * Turn a batch of requests into one chunk table (the input of
 * irm_table_create).
 *   host tokens: the requests' token ids back to back; host tok_first[n_req+1]:
 *   request q owns tokens [tok_first[q], tok_first[q+1]) (tok_first[0] == 0,
 *   nondecreasing, each request < 2^31 tokens).
 *   host prefix_len[n_req], prefix_row[n_req] (either may be NULL = 0): the
 *   exact-prefix match of the request (a standard prefix cache, outside the
 *   method), already in the pool from row prefix_row; it is emitted as a
 *   fresh entry for its first min(prefix_len, 32) rows and an exact-prefix
 *   entry (delta 0) for the rest.
 *   The tail after the prefix is CDC-split with *p; each chunk at target
 *   position pos: pos < 32 -> fresh entry on newly allocated rows, not
 *   registered; fingerprint hit with the same length -> registry entry
 *   (pool_row, len, p_src) placed at pos; otherwise fresh entry on newly
 *   allocated rows, registered with p_src = pos (a stored entry of another
 *   length is replaced).  With p->fallback_window = W > 0 (the pages' S1
 *   fallback: gist.science section 2.2, gentlecold.top section 6), a missed
 *   chunk is re-split into W-token windows from its start and each is looked
 *   up: if none hits, the chunk is prefilled on consecutive rows and
 *   registered together with its windows; otherwise each window becomes its
 *   own entry (hit, or fresh rows registered as that window).  Fingerprint =
 *   xxHash64, seed 0, of the chunk's ids
 *   as 4-byte little-endian integers.  Requests are processed in order, so a
 *   chunk inserted by request q is a hit for request q+1.
 *   CDC and fingerprints run on n_threads host threads (0 = all cores).
 *   host out chunks[max_chunks], fingerprints[max_chunks] (optional; 0 for
 *   prefix entries), seq_first[n_req + 1]; *n_chunks = entries.  Every fresh
 *   entry's rows are the caller's to prefill at p_tgt.
 *   ERANGE with *n_chunks = the needed count (with the fallback on, an upper
 *   bound: every missed chunk counted as all its windows), and the registry
 *   unchanged, if max_chunks is too small or the allocation counter would
 *   pass 2^32 rows.
 */
irm_status irm_registry_assemble(irm_registry* r, const irm_cdc_params* p, const int32_t* tokens,
                                 const uint64_t* tok_first, uint32_t n_req, const uint32_t* prefix_len,
                                 const uint32_t* prefix_row, uint32_t n_threads, irm_chunk* chunks,
                                 uint64_t* fingerprints, uint32_t max_chunks, uint32_t* seq_first,
                                 uint32_t* n_chunks);

#ifdef __cplusplus
}
#endif

#endif /* IRM_H */
