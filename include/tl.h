/*
 * tl.h -- C ABI of the paged KV-cache write and paged attention library (libtl.so),
 * hand-written HIP kernels for AMD Instinct MI355X (gfx950).
 *
 * The operations are the two serving-graph ops of the page "How serving works in
 * Tlaloc" (section 1, the decoder graph; section 2, their lowering):
 *   KV_CACHE_WRITE   store each new token's key and value rows into a page pool at
 *                    the token's slot; slot -1 is never written;
 *   PAGED_ATTENTION  attend over the pages a per-sequence block table names, for a
 *                    decode entry (one new token per sequence) or a prefill entry
 *                    (right-aligned rows, causal length = position + 1), optionally
 *                    with a sliding window (section 3, "Sliding-window layers").
 * Arithmetic follows the same page's rule for these dots: f32 operands, f32
 * products and f32 sums (section 2, PAGED_ATTENTION bullet); stored bf16 or fp8
 * keys and values are widened to f32 exactly before use.
 *
 * Conventions for every entry point
 * ---------------------------------
 * - All array arguments are DEVICE pointers owned by the caller (e.g. torch CUDA
 *   tensors), contiguous, in the layouts stated below, and 16-byte aligned.  The
 *   library allocates nothing, keeps no state between calls and never
 *   synchronises: every call enqueues its kernels on `stream` (a hipStream_t; NULL
 *   is the default stream) and returns.
 * - Pools are updated in place at the addresses given (the pages donate the pool
 *   buffers to each execution so that the updated pool is written where it was
 *   read, section 3, "donation pairs").
 * - Each call returns TL_OK (0) or a negative tl_status.  Argument checks run on the
 *   host before anything is enqueued; on failure nothing is enqueued and
 *   tl_last_error() names the offending argument.  Contents of device arrays
 *   (slot ids, table entries, lengths, positions) are the caller's contract and
 *   are not read on the host, except when the environment variable TL_VALIDATE=1
 *   is set: then those arrays are copied to the host (a synchronising copy) and
 *   range-checked before launch.  Kernels never access memory outside the
 *   arrays described here, whatever the contents: an out-of-range slot is
 *   skipped by the write, an out-of-range table entry or length is clamped.
 * - Supported shapes: head_dim D in {64, 128}; page_size S a power of two with
 *   8 <= S <= 1024; num_pages * page_size < 2^31; G = num_q_heads / num_kv_heads
 *   in {1, 2, 4, 8}.  Other shapes return TL_ERR_UNSUPPORTED.
 *
 * Pool layout (one layer; K and V are separate arrays, "numBlocks pages of
 * blockSize tokens, for K and for V", section 3 manifest bullets):
 *   x        = 16 / bytes(dtype)  elements per 16-byte chunk (f32 4, bf16 8, fp8 and int8 16)
 *   k        [num_pages][num_kv_heads][head_dim / x][page_size][x]   of dtype
 *   v        [num_pages][num_kv_heads][page_size][head_dim]          of dtype
 *   k_scale  [num_pages][num_kv_heads][page_size]  f32  (TL_KV_FP8_E4M3, TL_KV_INT8; else NULL)
 *   v_scale  [num_pages][num_kv_heads][page_size]  f32  (TL_KV_FP8_E4M3, TL_KV_INT8; else NULL)
 * Slot s names page s / page_size, offset s % page_size.  Position j of sequence
 * b lives on page block_tables[b][j / page_size] at offset j % page_size.
 *
 * Stored encodings:
 *   TL_KV_F32       the f32 bits unchanged;
 *   TL_KV_BF16      round to nearest, ties to even (NaN kept quiet, sign kept);
 *   TL_KV_FP8_E4M3  OCP e4m3fn codes with one f32 scale per (token, kv head):
 *                   scale = f32(max_d |x_d| / 448) (1 for an all-zero row),
 *                   code_d = RNE_e4m3fn(clamp(f32(x_d / scale), -448, 448)),
 *                   both divisions IEEE f32 (section 6, FP8 and FP8 KV cache
 *                   paragraphs).  Value = code * scale.
 *   TL_KV_FP8_E4M3_UNSCALED  the pages' own fp8 KV (section 6, FP8 KV cache
 *                   paragraph): code_d = RNE_e4m3fn(clamp(x_d, -448, 448)), no
 *                   scale (k_scale and v_scale are not used and may be NULL); a value
 *                   beyond +-448 saturates.  Value = code.
 *   TL_KV_INT8      int8 codes with one f32 scale per (token, kv head), the pages'
 *                   int8 formula applied per row (section 6, "Int8 weights"; the
 *                   pages list int8 KV pools as not built): scale = f32(max_d |x_d|
 *                   / 127) (1 for an all-zero row), code_d = clamp(round_half_even(
 *                   f32(x_d / scale)), -127, 127), IEEE f32 divisions.  Value =
 *                   code * scale.
 */
#ifndef TL_H
#define TL_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  TL_OK = 0,
  TL_ERR_INVALID = -1,      /* an argument is null, negative, misaligned or inconsistent */
  TL_ERR_UNSUPPORTED = -2,  /* a shape or dtype outside the supported set above */
  TL_ERR_WORKSPACE = -3,    /* workspace missing or smaller than the *_workspace_size query */
  TL_ERR_HIP = -4,          /* a HIP runtime call failed (message in tl_last_error) */
  TL_ERR_NO_PAGES = -5      /* the page allocator refused a request (message names the holders) */
} tl_status;

typedef enum {
  TL_KV_F32 = 0,
  TL_KV_BF16 = 1,
  TL_KV_FP8_E4M3 = 2,
  TL_KV_FP8_E4M3_UNSCALED = 3,
  TL_KV_INT8 = 4
} tl_kv_dtype;

/* One layer's page pool.  The struct itself is a host object read during the call. */
typedef struct {
  void* k;         /* device, layout above */
  void* v;         /* device, layout above */
  float* k_scale;  /* device, TL_KV_FP8_E4M3 and TL_KV_INT8 only */
  float* v_scale;  /* device, TL_KV_FP8_E4M3 and TL_KV_INT8 only */
  int32_t dtype;   /* tl_kv_dtype */
  int32_t num_pages;
  int32_t page_size;
  int32_t num_kv_heads;
  int32_t head_dim;
} tl_kv_pool;

/*
 * KV_CACHE_WRITE ("How serving works in Tlaloc", section 1 decoder graph and
 * section 2 KV_CACHE_WRITE bullet: a scatter into the pool at the token's slot).
 *   k_new, v_new  [n_tokens][num_kv_heads][head_dim] f32
 *   slots         [n_tokens] int32; -1 = pad, never written (section 1, prefill
 *                 entries).  Slots of one call must be distinct (a repeated slot
 *                 is a caller error; which row lands is then unspecified).
 * n_tokens == 0 is a no-op.  Encodes per the pool dtype (see above).
 */
int tl_kv_cache_write(const tl_kv_pool* pool, const float* k_new, const float* v_new,
                      const int32_t* slots, int64_t n_tokens, void* stream);

/*
 * PAGED_ATTENTION, decode entry ("How serving works in Tlaloc", section 1: one new
 * token per sequence; section 2: gather the pages the block table names, f32 dots,
 * masked softmax; section 3: sliding window).  Split-K over the context, then a merge.
 *   q             [batch][num_q_heads][head_dim] f32, the new token's queries
 *   block_tables  [batch][max_blocks] int32 page ids; entries past ceil(len/S) may
 *                 be read (the row must hold max_blocks entries) but are never used
 *   seq_lens      [batch] int32, positions held INCLUDING the new token, whose
 *                 position is seq_lens[b]-1 (its K/V must already be written);
 *                 0 gives an all-zero output row
 *   window        <= 0: full causal attention; W > 0: keys p-W+1 .. p only
 *   scale         multiplies q.k (e.g. 1/sqrt(head_dim))
 *   out           [batch][num_q_heads][head_dim] f32
 *   workspace     device scratch of at least tl_paged_attn_decode_workspace_size(...)
 *                 bytes: a header of 524,304 bytes (16 bytes of work counters, then
 *                 one arrival counter per (sequence, head group) that the in-place
 *                 merge of the splits uses; the same bytes for every shape), then
 *                 partial softmax states.  The header must be zero before the first
 *                 use; every call leaves it at zero again, so the workspace can be
 *                 reused by later calls of any shape on the same stream without
 *                 clearing (the partial states need no initial value).  Two calls in
 *                 flight at once (on different streams) need separate workspaces.
 * Query head h reads kv head h / (num_q_heads / num_kv_heads).
 * Results depend only on each sequence's own inputs (no cross-sequence reductions),
 * so a sequence's output is the same bits in any batch.
 */
size_t tl_paged_attn_decode_workspace_size(const tl_kv_pool* pool, int32_t batch,
                                           int32_t num_q_heads, int32_t max_blocks);
int tl_paged_attn_decode(const tl_kv_pool* pool, const float* q, int32_t num_q_heads,
                         const int32_t* block_tables, int32_t max_blocks,
                         const int32_t* seq_lens, int32_t batch, int32_t window, float scale,
                         float* out, void* workspace, size_t workspace_bytes, void* stream);

/*
 * PAGED_ATTENTION decode that allocates nothing, for callers that cannot allocate
 * device memory or pass a workspace: code under HIP graph capture, tight serving
 * loops, harnesses that forbid hipMalloc.  Arguments, results and errors are those
 * of tl_paged_attn_decode (the same kernels, so the same bits), without the
 * workspace: the library keeps one static device array of TL_STATIC_SCRATCH_BYTES
 * (64 MiB) per device it runs on, held until the process ends.  The first call on a
 * device (with that device current) resolves the array's address and clears its
 * header with a kernel on `stream`; every call leaves the header at zero again.
 *   - A call whose tl_paged_attn_decode_workspace_size(...) exceeds
 *     TL_STATIC_SCRATCH_BYTES returns TL_ERR_WORKSPACE and enqueues nothing (64 MiB
 *     holds, e.g., 128 sequences x 64 query heads of 32K positions in fp8, or 64 x 32
 *     of 8K in bf16).
 *   - No hipMalloc, hipFree or other allocating call is made (TL_VALIDATE=1 aside,
 *     whose range checks copy index arrays to host memory as for every entry).
 *   - All calls on one device share the array: calls that overlap on one GPU (e.g.
 *     on two streams without ordering between them) race and give wrong results.
 */
#define TL_STATIC_SCRATCH_BYTES (64u << 20)
int tl_paged_attn_decode_static(const tl_kv_pool* pool, const float* q, int32_t num_q_heads,
                                const int32_t* block_tables, int32_t max_blocks, const int32_t* seq_lens,
                                int32_t batch, int32_t window, float scale, float* out, void* stream);

/*
 * PAGED_ATTENTION, prefill entry ("How serving works in Tlaloc", section 1: each
 * sequence has its own right-aligned row of the token axis, pads first; a token's
 * causal length is its position + 1; section 2 blockwise bullet: online softmax over
 * 2,048-key blocks from the first block a row can see to the block of its last
 * position; section 3: chunked prefill over cached history).  Each sequence's pages
 * are read once per query tile in the kernel, never gathered per token.
 *   q             [batch][tokens_per_row][num_q_heads][head_dim] f32
 *   positions     [batch][tokens_per_row] int32; -1 = pad (its output row is 0).
 *                 Every position's K/V (and all earlier visible ones) must already be
 *                 written, i.e. call tl_kv_cache_write for the chunk first.  Keys a
 *                 row's tokens cannot see (before a window, past the last position)
 *                 are never read; keys between the first one a row can see and the
 *                 row's last position must hold written (finite) K/V.
 *   out           [batch][tokens_per_row][num_q_heads][head_dim] f32 (every row written)
 *   workspace     may be NULL when tl_paged_attn_prefill_workspace_size(...) is 0
 */
size_t tl_paged_attn_prefill_workspace_size(const tl_kv_pool* pool, int32_t batch,
                                            int32_t tokens_per_row, int32_t num_q_heads,
                                            int32_t max_blocks);
int tl_paged_attn_prefill(const tl_kv_pool* pool, const float* q, int32_t num_q_heads,
                          const int32_t* block_tables, int32_t max_blocks,
                          const int32_t* positions, int32_t batch, int32_t tokens_per_row,
                          int32_t window, float scale, float* out, void* workspace,
                          size_t workspace_bytes, void* stream);

/*
 * PAGED_ATTENTION over a windowed pool whose tables are rings ("How serving works in
 * Tlaloc", section 3, windowed KV pool bullets: each sequence holds a ring of
 * ring_pages pages and logical block j of the sequence is on ring page j % ring_pages,
 * so position p overwrites position p - N, N = ring_pages * page_size; section 2, the
 * ring bullet: with ring = true the ring's N slots are scored, each masked by its
 * age).  The K/V of position p are written beforehand with tl_kv_cache_write at slot
 * ring_tables[b][(p / S) % ring_pages] * S + p % S (the windowed slot mapping).
 *   ring_tables   [batch][ring_pages] int32 page ids of each sequence's ring
 *   ring_pages    > 0, ring_pages * page_size < 2^30
 *   window        W > 0: the window; <= 0: none.  A row of causal length L (decode:
 *                 seq_lens[b]; prefill: position + 1) scores ring slot i when its age
 *                 (L - 1 - i) mod N is below min(W, L); that is the last min(W, N, L)
 *                 positions, each read from its ring slot as it stands.  The slot holds
 *                 the position its age names whenever every call writes at most
 *                 N - min(p0, W - 1) tokens starting at position p0 (section 3).
 *   seq_lens, positions: no upper bound (a ring has no end); other arguments, the
 *                 workspace rules and the results' batch invariance are those of the
 *                 full-table entries above.
 * With a ring of at least ceil(W / S) pages (decode) or ceil((W - 1 + n) / S) pages
 * (prefill calls of n tokens), the results are the same bits as the full-table entry
 * with window W over a pool holding the same K/V.
 */
size_t tl_paged_attn_decode_ring_workspace_size(const tl_kv_pool* pool, int32_t batch,
                                                int32_t num_q_heads, int32_t ring_pages,
                                                int32_t window);
int tl_paged_attn_decode_ring(const tl_kv_pool* pool, const float* q, int32_t num_q_heads,
                              const int32_t* ring_tables, int32_t ring_pages,
                              const int32_t* seq_lens, int32_t batch, int32_t window, float scale,
                              float* out, void* workspace, size_t workspace_bytes, void* stream);
int tl_paged_attn_prefill_ring(const tl_kv_pool* pool, const float* q, int32_t num_q_heads,
                               const int32_t* ring_tables, int32_t ring_pages,
                               const int32_t* positions, int32_t batch, int32_t tokens_per_row,
                               int32_t window, float scale, float* out, void* workspace,
                               size_t workspace_bytes, void* stream);

/*
 * SLOT_MAPPING and WINDOW_SLOT_MAPPING ("How serving works in Tlaloc", section 3: the
 * slot each new token's K/V is written at, an input of every entry beside the block
 * tables; with a windowed pool, logical block j of a sequence is on its ring's page
 * j % ringPages, so position p is written over position p - ringPages * page_size).
 * Fills the slots that tl_kv_cache_write takes, for a whole call:
 *   slots[b][t] = tables[b][j] * page_size + p % page_size,  p = positions[b][t],
 *                 j = p / page_size            (ring_pages == 0: block tables)
 *                 j = (p / page_size) % ring_pages   (ring_pages > 0: rings)
 * and -1 where p < 0 (a pad), where j >= width, or where the entry is not a page of
 * the pool ([0, num_pages)), so that the write skips those tokens.
 *   tables     [batch][width] int32 (device): block tables or ring tables; a ring
 *              occupies the first ring_pages entries of its row (ring_pages <= width)
 *   positions  [batch][tokens_per_row] int32 (device)
 *   slots      [batch][tokens_per_row] int32 (device, output)
 *   page_size  a power of two in [8, 1024]; num_pages * page_size < 2^31
 * With TL_VALIDATE=1, a live position past the table or naming an entry outside the
 * pool is an error instead (nothing enqueued).
 */
int tl_slot_mapping(const int32_t* tables, int32_t width, int32_t ring_pages, const int32_t* positions,
                    int32_t batch, int32_t tokens_per_row, int32_t page_size, int32_t num_pages, int32_t* slots,
                    void* stream);

/*
 * GATED_DELTA_RULE, decode step ("How serving works in Tlaloc", "Linear-attention
 * layers: the state pools"): a Gated DeltaNet layer keeps per sequence an f32
 * recurrent state [num_heads][128][128] in a pool indexed by the sequence's state
 * slot.  For each row b with slot s = state_slots[b] and each head h, with S the
 * state (S[i][j]: i over the key dimension, j over the value dimension):
 *     S = S * exp(g);  S += k (outer) beta (v - k^T S);  o = q^T S  (the updated S)
 * and S is written back to the pool in place.  A row at position 0 starts from zero
 * state (the slot's old contents are not read); slot -1 is a pad: nothing is read or
 * written and its output row is 0.  Rows of one call must hold distinct slots.
 *   state_pool   [num_slots][num_heads][128][128] f32 (device, updated in place)
 *   q, k, v      [batch][num_heads][128] f32;  g, beta [batch][num_heads] f32
 *                (g is the log decay; q, k, v are used as given)
 *   state_slots  [batch] int32;  positions [batch] int32 (the row's position)
 *   out          [batch][num_heads][128] f32
 * head_dim must be 128.  f32 operands, products and sums.
 */
int tl_gated_delta_rule_decode(float* state_pool, int32_t num_slots, int32_t num_heads,
                               int32_t head_dim, const float* q, const float* k, const float* v,
                               const float* g, const float* beta, const int32_t* state_slots,
                               const int32_t* positions, int32_t batch, float* out, void* stream);

/*
 * Host page allocator ("How serving works in Tlaloc": the runtime comparison table and
 * the backend bullets of section 3; prefix sharing: the KV-cache management page,
 * "Reuse identical causal prefixes" and the paragraph before it).  An opaque HOST
 * object, not thread-safe.  Sequences are named by int64 ids; `now` is the caller's
 * clock (any unit; idle_timeout in the same unit).
 * - tl_alloc_start: a new sequence, holding no pages (an id already started is refused).
 * - tl_alloc_append: room for n_tokens more positions.  Writes their slots (host
 *   int32 [n_tokens], for tl_kv_cache_write) and at most one page copy (host int32
 *   [1] each) that the caller must run with tl_kv_copy_pages BEFORE writing: a page
 *   shared with a forked sequence and only partly filled is copied before this
 *   sequence writes into it.  When pages run short, sequences idle past the timeout
 *   (last activity < now - idle_timeout) are reclaimed, least recently active first
 *   and only as many as needed, if they cover the shortage; otherwise the call returns
 *   TL_ERR_NO_PAGES, tl_last_error() names the sequences holding pages, the request
 *   changes nothing (its sequence keeps its pages) and counts as activity.  The lowest
 *   free page is always taken first.
 * - tl_alloc_fork: child shares parent's pages covering its first n_tokens positions
 *   (reference counted); tl_alloc_end: releases a sequence's pages (a page returns to
 *   the free list when no sequence holds it).
 * - tl_alloc_tables: block tables [n][max_blocks] (-1 past a sequence's pages) and
 *   lengths [n] of the given sequences, host arrays, for the attention entries.
 * - tl_kv_copy_pages: device copy of whole pages src_pages[i] -> dst_pages[i] (K, V
 *   and, for scaled pools, scales), n <= 65535; device int32 arrays.
 */
typedef struct tl_page_allocator tl_page_allocator;
tl_page_allocator* tl_alloc_create(int32_t num_pages, int32_t page_size, double idle_timeout);
void tl_alloc_destroy(tl_page_allocator* a);
int32_t tl_alloc_free_pages(const tl_page_allocator* a);
int tl_alloc_start(tl_page_allocator* a, int64_t seq, double now);
int tl_alloc_end(tl_page_allocator* a, int64_t seq);
int tl_alloc_fork(tl_page_allocator* a, int64_t parent, int64_t child, int64_t n_tokens, double now);
int tl_alloc_append(tl_page_allocator* a, int64_t seq, int32_t n_tokens, double now, int32_t* slots_out,
                    int32_t* copy_src, int32_t* copy_dst, int32_t* n_copies);
int tl_alloc_tables(const tl_page_allocator* a, const int64_t* seqs, int32_t n, int32_t max_blocks,
                    int32_t* tables, int32_t* lens);
int tl_kv_copy_pages(const tl_kv_pool* pool, const int32_t* src_pages, const int32_t* dst_pages,
                     int32_t n, void* stream);

/*
 * Copy sequence positions 0..length-1 out of the pool in logical order, as stored
 * (no decoding), so that a test can compare written/gathered KV byte for byte
 * ("How serving works in Tlaloc", section 2: the pages a block table names).
 *   block_table_row  [>= ceil(length / page_size)] int32 (device)
 *   k_out, v_out     [length][num_kv_heads][head_dim] of the pool dtype (device)
 *   k_scale_out, v_scale_out  [length][num_kv_heads] f32 (scaled pools only, else NULL)
 */
int tl_kv_gather(const tl_kv_pool* pool, const int32_t* block_table_row, int32_t length,
                 void* k_out, void* v_out, float* k_scale_out, float* v_scale_out,
                 void* stream);

/* Message of the last failing call on this thread ("" if none).  Owned by the library. */
const char* tl_last_error(void);

/* ABI version: 1. */
int tl_abi_version(void);

#ifdef __cplusplus
}
#endif

#endif /* TL_H */
