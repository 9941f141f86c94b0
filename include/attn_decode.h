/*
 * attn_decode.h -- single-query scaled-dot-product decode attention over an
 * fp16 KV cache, for AMD Instinct MI355X (gfx950).
 *
 * The operation is the one defined on the page "Developing Apple Metal
 * Kernels in Rust - A Deep Dive Through Attention", section "The MSL,
 * briefly" (kernels attention_qk_f16 and attention_pv_f16), computed in one
 * pass over the cache instead of the page's two dispatches:
 *
 *   s[h,p]   = (sum_i q[h,i] * k[p,h,i]) / sqrt(head_dim)   for p <= current_pos
 *   w[h,:]   = softmax over p <= current_pos of s[h,p]      (positions after
 *              current_pos are masked: weight 0, never read)
 *   out[h,d] = sum_p w[h,p] * v[p,h,d]
 *
 * Conventions shared by every entry point
 *  - Tensor pointers are DEVICE pointers on the current HIP device.  fp16
 *    means IEEE binary16 bits.  All tensors are dense and row-major
 *    (contiguous), as the page's layouts are.
 *  - Layouts (page section "The MSL, briefly"): Q and out [n_heads, head_dim];
 *    K and V caches [seq_len, n_heads, head_dim]; element (p,h,i) of the
 *    cache at (p*n_heads + h)*head_dim + i.  Batched forms put a leading
 *    [batch] dimension on every tensor: caches [batch, seq_len, n_heads,
 *    head_dim], Q/out [batch, n_heads, head_dim].
 *  - current_pos is the index of the newest cached token: positions
 *    p > current_pos are masked (the page's attention_qk_f16 writes -inf
 *    there).  current_pos >= seq_len masks nothing.  The number of positions
 *    read is L = min(current_pos, seq_len - 1) + 1.
 *  - Arithmetic: fp32 dot products and softmax state, output rounded to fp16
 *    to nearest even.  Same inputs and shapes give bit-identical results.
 *  - Ownership: the caller owns every buffer.  The library keeps no device
 *    memory and no state between calls.
 *  - Asynchrony: each call enqueues kernels on `stream` (a hipStream_t;
 *    NULL is the null stream) and returns without synchronising.  Inputs
 *    must stay valid until the work completes.  No call allocates memory or
 *    synchronises, so calls may be captured in a HIP graph.
 *  - Errors: arguments are checked on the host before any HIP call; a
 *    non-OK status means nothing was enqueued (ATTN_ERR_HIP: a launch was
 *    refused; work enqueued before it on the same call may have run).
 *    attn_last_error() gives the calling thread's detail text for its last
 *    non-OK return.
 *  - Outputs (out, scores_dump, workspace) must not overlap any input, except
 *    where an entry point says otherwise (the decode step writes one row of
 *    its caches; the row softmax may run in place).
 */
#ifndef ATTN_DECODE_H
#define ATTN_DECODE_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum attn_status {
    ATTN_OK = 0,
    ATTN_ERR_NULL = 1,        /* a required pointer is NULL                     */
    ATTN_ERR_DIM = 2,         /* a size is 0, head_dim > ATTN_MAX_HEAD_DIM,
                                 seq_len > 2^31, batch > 65535,
                                 batch*n_heads > 67108860, the cache is too
                                 large to index, or a launch would exceed the
                                 GPU's dispatch limit (2^32 - 1 work-items)   */
    ATTN_ERR_ALIGN = 3,       /* fp16 pointer not 2-byte aligned, fp32/uint32
                                 pointer not 4-byte aligned, workspace not
                                 16-byte aligned                                */
    ATTN_ERR_WORKSPACE = 4,   /* workspace NULL or smaller than required       */
    ATTN_ERR_HIP = 5          /* the HIP runtime refused a launch              */
} attn_status_t;

#define ATTN_MAX_HEAD_DIM 256u

/*
 * Bytes of device workspace that every call below needs for these sizes
 * (seq_len is the cache length, or the per-sequence capacity of a batch).
 * Depends only on the arguments.  Returns 0 for invalid sizes.
 * The workspace holds per-chunk partial softmax states; its content between
 * calls is meaningless and it needs no initialisation.
 */
size_t attn_decode_workspace_bytes(uint32_t batch, uint32_t n_heads, uint32_t head_dim,
                                   uint32_t seq_len);

/*
 * How a call with these sizes is carried out: the grid of its streaming
 * (split) launch, whether a merge (combine) launch follows, and how many
 * partial softmax states it leaves in the workspace.  For callers that
 * budget launches or graph nodes, and for checking that every plan's
 * partial states fit the workspace attn_decode_workspace_bytes sizes.
 * Host only: no HIP call is made and no device is needed.  The plan assumes
 * tensors aligned for 16-byte loads (as a caching allocator returns them);
 * with less aligned tensors a call may put fewer heads in a workgroup and
 * runs U = 4 without the wave bound.
 *   flags        which call is meant, ATTN_PLAN_* bits (0: attn_decode_f16,
 *                or attn_decode_f16_split with one host current_pos for the
 *                whole batch):
 *                DEVICE_POS attn_decode_f16_batched; PAGED attn_decode_f16_paged
 *                (seq_len = max_blocks * page_size); STEP the decode step
 *                (with DEVICE_POS or PAGED, its batched or paged form);
 *                FROM_SCORES attn_pv_f16.
 *   current_pos  the host current_pos of a single-sequence call; ignored
 *                with DEVICE_POS or PAGED, whose plans cover the capacity.
 *   info         written on ATTN_OK.
 * Errors: ATTN_ERR_NULL (info), ATTN_ERR_DIM (sizes as for the calls,
 * unknown flags, FROM_SCORES with other flags or batch != 1, a
 * single-sequence STEP with current_pos >= seq_len).
 * Not counted: the fill launch a score dump adds.
 */
#define ATTN_PLAN_DEVICE_POS 1u
#define ATTN_PLAN_PAGED 2u
#define ATTN_PLAN_STEP 4u
#define ATTN_PLAN_FROM_SCORES 8u

typedef struct attn_plan_info {
    uint32_t balanced;             /* 1: balanced grid (equal positions per
                                      workgroup across the batch); 0: chunked */
    uint32_t heads_per_workgroup;  /* heads one split workgroup reads together */
    uint64_t workgroups;           /* workgroups of the split launch          */
    uint32_t chunk;                /* chunked grid: positions per chunk (0 if
                                      balanced)                                */
    uint32_t chunks;               /* chunked grid: chunks per (sequence, head
                                      block) (0 if balanced)                   */
    uint32_t launches;             /* 1: the split launch writes out; 2: a
                                      combine launch follows.  For the
                                      one-call entry points; the split /
                                      combine pair is always two launches, its
                                      split writing partial states            */
    uint64_t partial_slots;        /* one past the highest partial state the
                                      split launch may write (0 with one
                                      launch)                                  */
    uint64_t workspace_slots;      /* partial states the workspace holds      */
    uint32_t unroll;               /* positions each row group of a split
                                      workgroup streams per block (2, 4, 8);
                                      calls that differ in it round their
                                      softmax differently                      */
    uint32_t max_waves;            /* waves per SIMD the split kernel was
                                      compiled for: 2 (its loads issued a
                                      block ahead), or 8 (no bound)            */
} attn_plan_info;

attn_status_t attn_decode_plan(uint32_t batch, uint32_t n_heads, uint32_t head_dim,
                               uint32_t seq_len, uint32_t current_pos, uint32_t flags,
                               attn_plan_info *info);

/*
 * One sequence.
 *   q            [n_heads, head_dim] fp16
 *   k_cache      [seq_len, n_heads, head_dim] fp16
 *   v_cache      [seq_len, n_heads, head_dim] fp16
 *   out          [n_heads, head_dim] fp16, written
 *   scores_dump  NULL, or [n_heads, seq_len] fp32, written: the scaled score
 *                (natural-log units) for p <= current_pos and -inf after it,
 *                as the page's attention_qk_f16 stores them.  For checking;
 *                it costs a write of the whole buffer.
 *   workspace    >= attn_decode_workspace_bytes(1, n_heads, head_dim, seq_len)
 *                bytes of device memory, 16-byte aligned.
 */
attn_status_t attn_decode_f16(const uint16_t *q, const uint16_t *k_cache,
                              const uint16_t *v_cache, uint16_t *out,
                              uint32_t n_heads, uint32_t head_dim, uint32_t seq_len,
                              uint32_t current_pos, float *scores_dump,
                              void *workspace, size_t workspace_bytes, void *stream);

/*
 * A batch of independent sequences sharing one cache capacity, each with
 * its own current_pos (a ragged batch).
 *   q            [batch, n_heads, head_dim] fp16
 *   k_cache      [batch, capacity, n_heads, head_dim] fp16
 *   v_cache      [batch, capacity, n_heads, head_dim] fp16
 *   out          [batch, n_heads, head_dim] fp16, written
 *   current_pos  DEVICE [batch] uint32; values >= capacity mask nothing.  Read
 *                by the kernels, so it may change between enqueued calls
 *                without a host synchronisation.
 *   scores_dump  NULL, or [batch, n_heads, capacity] fp32 (as above)
 *   workspace    >= attn_decode_workspace_bytes(batch, n_heads, head_dim, capacity)
 */
attn_status_t attn_decode_f16_batched(const uint16_t *q, const uint16_t *k_cache,
                                      const uint16_t *v_cache, uint16_t *out,
                                      const uint32_t *current_pos, uint32_t batch,
                                      uint32_t n_heads, uint32_t head_dim, uint32_t capacity,
                                      float *scores_dump, void *workspace,
                                      size_t workspace_bytes, void *stream);

/*
 * attn_decode_f16_batched with no workspace argument, for callers that
 * cannot allocate device memory: code under HIP graph capture, serving loops
 * and harnesses that forbid allocation.  The workspace is instead a fixed
 * array of ATTN_NOALLOC_SCRATCH_BYTES that the library holds on every GPU it
 * runs on, from the first call there until the process ends; the call
 * itself allocates nothing.  The caller still passes inputs and outputs.
 *   Errors: as attn_decode_f16_batched; ATTN_ERR_WORKSPACE when
 *   attn_decode_workspace_bytes(batch, n_heads, head_dim, capacity) exceeds
 *   ATTN_NOALLOC_SCRATCH_BYTES (checked on the host, nothing enqueued);
 *   ATTN_ERR_HIP when the array cannot be located on the current device;
 *   ATTN_ERR_DIM when `stream` belongs to another device than the current
 *   one (both checked before anything is enqueued).
 *   Nothing in the array needs to start at zero.
 * The array is per GPU and shared by every call on that GPU: calls that can
 * run at the same time on one GPU (enqueued on different streams, or graphs
 * replayed concurrently) race on it and give wrong results.  Keep such calls
 * on one stream.  `stream` must belong to the current device.
 */
#define ATTN_NOALLOC_SCRATCH_BYTES (32u << 20)

attn_status_t attn_decode_f16_batched_noalloc(const uint16_t *q, const uint16_t *k_cache,
                                              const uint16_t *v_cache, uint16_t *out,
                                              const uint32_t *current_pos, uint32_t batch,
                                              uint32_t n_heads, uint32_t head_dim,
                                              uint32_t capacity, float *scores_dump,
                                              void *stream);

/*
 * The same computation as the two calls above, split at its one internal
 * boundary, for callers that need to place work between the two launches
 * (timing the streaming kernel alone, or moving the partial states between
 * devices before merging).  attn_decode_f16_split streams the cache and
 * leaves one partial softmax state per (sequence, head, chunk) in the
 * workspace; attn_decode_f16_combine merges them into `out`.  Both take the
 * same sizes and the same current_pos arguments as the call they pair with;
 * between the two, the workspace belongs to the library.
 *   current_pos_dev  DEVICE [batch] uint32, or NULL: then every sequence uses
 *                    current_pos.
 * attn_decode_f16 is split + combine with current_pos_dev = NULL, batch = 1;
 * attn_decode_f16_batched is split + combine with the device array.
 */
attn_status_t attn_decode_f16_split(const uint16_t *q, const uint16_t *k_cache,
                                    const uint16_t *v_cache, const uint32_t *current_pos_dev,
                                    uint32_t current_pos, uint32_t batch, uint32_t n_heads,
                                    uint32_t head_dim, uint32_t seq_len, float *scores_dump,
                                    void *workspace, size_t workspace_bytes, void *stream);

attn_status_t attn_decode_f16_combine(uint16_t *out, const uint32_t *current_pos_dev,
                                      uint32_t current_pos, uint32_t batch, uint32_t n_heads,
                                      uint32_t head_dim, uint32_t seq_len,
                                      const void *workspace, size_t workspace_bytes,
                                      void *stream);

/*
 * A batch whose K/V caches live in a paged pool.  The page "Tutorial 16:
 * Writing Custom Metal Kernels" (section "7. Performance Impact") names paged
 * attention that reads pages directly instead of gathering them first; the
 * page "Developing Apple Metal Kernels in Rust - A Deep Dive Through
 * Attention" (section "setBuffer_offset_atIndex and unified memory") keeps
 * tensors as sub-regions of one pool handed out by a paged block allocator.
 * Each page holds page_size consecutive positions of one sequence in the
 * dense row layout, and a block table names the pages of each sequence:
 *   k_pool, v_pool  [num_blocks, page_size, n_heads, head_dim] fp16
 *   block_table     DEVICE [batch, max_blocks] uint32: position p of sequence
 *                   b is row p % page_size of page block_table[b][p / page_size].
 *                   Only entries for positions <= current_pos are read;
 *                   several sequences may share a page.  An entry >=
 *                   num_blocks is read as num_blocks - 1 (in bounds, output
 *                   meaningless); attn_paged_table_check finds such entries.
 *   current_pos     DEVICE [batch] uint32; capacity = max_blocks * page_size
 *   page_size       a power of two, 1..65536
 *   q, out          [batch, n_heads, head_dim] fp16; scores_dump NULL or
 *                   [batch, n_heads, capacity] fp32
 *   workspace       >= attn_decode_workspace_bytes(batch, n_heads, head_dim, capacity)
 * attn_decode_f16_paged_split is its first launch; attn_decode_f16_combine
 * (with current_pos_dev = current_pos and seq_len = capacity) is the second.
 */
attn_status_t attn_decode_f16_paged(const uint16_t *q, const uint16_t *k_pool,
                                    const uint16_t *v_pool, uint16_t *out,
                                    const uint32_t *block_table, const uint32_t *current_pos,
                                    uint32_t batch, uint32_t n_heads, uint32_t head_dim,
                                    uint32_t page_size, uint32_t max_blocks, uint32_t num_blocks,
                                    float *scores_dump, void *workspace, size_t workspace_bytes,
                                    void *stream);

attn_status_t attn_decode_f16_paged_split(const uint16_t *q, const uint16_t *k_pool,
                                          const uint16_t *v_pool, const uint32_t *block_table,
                                          const uint32_t *current_pos, uint32_t batch,
                                          uint32_t n_heads, uint32_t head_dim, uint32_t page_size,
                                          uint32_t max_blocks, uint32_t num_blocks,
                                          float *scores_dump, void *workspace,
                                          size_t workspace_bytes, void *stream);

/*
 * A check of a paged cache's block table, for callers that want to know
 * whether a paged call read a table entry that names no page of the pool
 * (such an entry is read as the last page: in bounds, output meaningless).
 * It enqueues two small launches on `stream` and writes, in device memory:
 *   result[0]  the number of entries a paged decode or decode step with these
 *              block_table and current_pos reads (block j of sequence b when
 *              j * page_size <= min(current_pos[b], capacity - 1)) that are
 *              >= num_blocks;
 *   result[1]  the lowest sequence index holding such an entry, or
 *              0xFFFFFFFF when there is none.
 * result: DEVICE uint32[2], written (no initialisation needed).  Other
 * arguments as attn_decode_f16_paged.  The check reads the table once; it is
 * not part of a decode call.
 * Errors: ATTN_ERR_NULL, ATTN_ERR_ALIGN (4-byte pointers), ATTN_ERR_DIM (as
 * the paged calls), ATTN_ERR_HIP.
 */
attn_status_t attn_paged_table_check(const uint32_t *block_table, const uint32_t *current_pos,
                                     uint32_t batch, uint32_t page_size, uint32_t max_blocks,
                                     uint32_t num_blocks, uint32_t *result, void *stream);

/*
 * The page's own two-dispatch form (section "The MSL, briefly": kernels
 * attention_qk_f16 then attention_pv_f16), for callers that need the score
 * row itself.  One sequence.
 *
 * attn_qk_f16 writes, for every head h and position p < seq_len, the scaled
 * score (sum_i q[h,i] k[p,h,i]) / sqrt(head_dim) accumulated in fp32 and
 * rounded to fp16 (nearest even), or -inf for p > current_pos; masked
 * positions are not read.
 *   scores  [n_heads, seq_len] fp16, written
 *
 * attn_pv_f16 takes such a score row (from attn_qk_f16 or any other source):
 * softmax over positions 0..current_pos, then the weighted sum of V.  Unlike
 * the page's kernel, which weighs every position of the row, positions after
 * current_pos are not read at all, and a stored score of -inf weighs exactly
 * nothing whatever V holds there.
 *   scores     [n_heads, seq_len] fp16; v_cache [seq_len, n_heads, head_dim]
 *   out        [n_heads, head_dim] fp16, written
 *   workspace  >= attn_decode_workspace_bytes(1, n_heads, head_dim, seq_len)
 */
attn_status_t attn_qk_f16(const uint16_t *q, const uint16_t *k_cache, uint16_t *scores,
                          uint32_t n_heads, uint32_t head_dim, uint32_t seq_len,
                          uint32_t current_pos, void *stream);

attn_status_t attn_pv_f16(const uint16_t *scores, const uint16_t *v_cache, uint16_t *out,
                          uint32_t n_heads, uint32_t head_dim, uint32_t seq_len,
                          uint32_t current_pos, void *workspace, size_t workspace_bytes,
                          void *stream);

/*
 * One decode step: rotary embedding of the new token's query and key, the
 * append of its key and value rows to the caches, and attention over the
 * cache including the new row: one launch when the plan gives each head
 * block of a sequence one chunk (short caches; attn_decode_plan reports it),
 * else two.  The rotation is the one the
 * page "Tutorial 16: Writing Custom Metal Kernels" describes (section "5.
 * Example: Fused RoPE Kernel": FastRoPE(dims, base, traditional) applied at
 * a per-sequence offset); the cache layout, current_pos and the attention
 * are those of the page "Developing Apple Metal Kernels in Rust - A Deep
 * Dive Through Attention" (section "The MSL, briefly").
 *
 * For each sequence, with pos = current_pos (single sequence) or
 * min(current_pos[b], capacity - 1) (batch):
 *   rot(x)[2 values of pair i] = 2D rotation by pos * rope_base^(-2i/rope_dims)
 *       of pair i, i < rope_dims/2; pair i is (i, i + rope_dims/2), or
 *       (2i, 2i+1) when rope_traditional != 0; values at index >= rope_dims
 *       are unchanged.  The rotated q and k_new are rounded to fp16 (nearest
 *       even), as a rotated tensor is stored.
 *   k_cache[pos] = rot(k_new), v_cache[pos] = v_new          (the append)
 *   out = attention of rot(q) over cache positions 0..pos, as attn_decode_f16
 * Rows before pos must already hold rotated keys.  Positions after pos are
 * neither read nor written.
 *   q, k_new, v_new   [n_heads, head_dim] fp16 (batch: [batch, n_heads, head_dim])
 *   k_cache, v_cache  [seq_len, n_heads, head_dim] fp16 (batch: [batch,
 *                     capacity, n_heads, head_dim]); row pos is written
 *   out               [n_heads, head_dim] fp16 (batch: [batch, n_heads, head_dim])
 *   current_pos       single: host value, must be < seq_len (ATTN_ERR_DIM
 *                     otherwise); batch: DEVICE [batch] uint32, values >=
 *                     capacity use slot capacity - 1
 *   rope_dims         even, <= head_dim; 0 rotates nothing (append + attend)
 *   rope_base         > 0 and finite (10000 on the page)
 *   workspace         >= attn_decode_workspace_bytes(batch, n_heads, head_dim, seq_len)
 * q, k_new, v_new and out must not overlap the caches or each other.
 * Arithmetic: angle and its reduction modulo pi/2 in fp64, cos/sin and the
 * rotation in fp32; the rest as attn_decode_f16.
 */
attn_status_t attn_decode_step_f16(const uint16_t *q, const uint16_t *k_new, const uint16_t *v_new,
                                   uint16_t *k_cache, uint16_t *v_cache, uint16_t *out,
                                   uint32_t n_heads, uint32_t head_dim, uint32_t seq_len,
                                   uint32_t current_pos, uint32_t rope_dims, double rope_base,
                                   int rope_traditional, void *workspace, size_t workspace_bytes,
                                   void *stream);

attn_status_t attn_decode_step_f16_batched(const uint16_t *q, const uint16_t *k_new,
                                           const uint16_t *v_new, uint16_t *k_cache,
                                           uint16_t *v_cache, uint16_t *out,
                                           const uint32_t *current_pos, uint32_t batch,
                                           uint32_t n_heads, uint32_t head_dim, uint32_t capacity,
                                           uint32_t rope_dims, double rope_base,
                                           int rope_traditional, void *workspace,
                                           size_t workspace_bytes, void *stream);

/*
 * The decode step on a paged cache (pool and block table as for
 * attn_decode_f16_paged): slot pos = min(current_pos[b], capacity - 1) of
 * sequence b is row pos % page_size of page block_table[b][pos / page_size];
 * the rotated key and the new value are written there, positions 0..pos-1
 * are read through the table, and the output is that of
 * attn_decode_step_f16_batched on the equivalent dense cache.  A table entry
 * >= num_blocks for slot pos means the new rows are not written (and reads
 * use the last page, as for attn_decode_f16_paged: the output is then
 * meaningless but every access stays in bounds).
 *   k_pool, v_pool  [num_blocks, page_size, n_heads, head_dim] fp16, written at slot pos
 *   capacity        max_blocks * page_size; workspace as for the batched step
 *                   with that capacity
 */
attn_status_t attn_decode_step_f16_paged(const uint16_t *q, const uint16_t *k_new,
                                         const uint16_t *v_new, uint16_t *k_pool, uint16_t *v_pool,
                                         uint16_t *out, const uint32_t *block_table,
                                         const uint32_t *current_pos, uint32_t batch,
                                         uint32_t n_heads, uint32_t head_dim, uint32_t page_size,
                                         uint32_t max_blocks, uint32_t num_blocks,
                                         uint32_t rope_dims, double rope_base, int rope_traditional,
                                         void *workspace, size_t workspace_bytes, void *stream);

/*
 * The rotation alone (the page's FastRoPE with one offset per batch entry):
 * row (b, h) of x turns at position positions[b], as rot() above, and is
 * rounded to fp16.
 *   x, out     [batch, n_heads, head_dim] fp16; out must not overlap x
 *   positions  DEVICE [batch] uint32, any value
 *   rope_dims, rope_base, rope_traditional  as for attn_decode_step_f16
 */
attn_status_t attn_rope_f16(const uint16_t *x, uint16_t *out, const uint32_t *positions,
                            uint32_t batch, uint32_t n_heads, uint32_t head_dim, uint32_t rope_dims,
                            double rope_base, int rope_traditional, void *stream);

/*
 * Softmax over the last dimension of an fp32 [rows, cols] tensor, the softmax
 * step on its own: the Foundry notes' fm_softmax (section "API Reference":
 * x [rows, cols] -> out [rows, cols]), computed max-shifted as the page
 * "Developing Apple Metal Kernels in Rust - A Deep Dive Through Attention"
 * does inside attention_pv_f16 (section "The MSL, briefly"):
 *   out[r,c] = exp(x[r,c] - m_r) / sum_c' exp(x[r,c'] - m_r),  m_r = max_c x[r,c]
 * A -inf entry gets exactly 0.  A row of -inf only, or a row holding a NaN,
 * gives NaN throughout, as the definition does.
 *   x, out     DEVICE [rows, cols] fp32, row-major, 4-byte aligned (16-byte
 *              aligned with cols % 4 == 0 takes 16-byte loads); out may be x
 *              itself (in place), otherwise they must not overlap
 *   workspace  >= attn_softmax_workspace_bytes(rows, cols) bytes, 16-byte
 *              aligned (per-chunk statistics for long rows; no initialisation)
 * Arithmetic: fp32; exp(t) as the hardware 2^(t log2 e); fixed reduction
 * order, so results are bitwise reproducible.  Returns ATTN_ERR_DIM for a
 * zero size or when rows * ceil(cols / 4096) exceeds 2^31 - 1.
 */
size_t attn_softmax_workspace_bytes(uint32_t rows, uint32_t cols);

attn_status_t attn_softmax_f32(const float *x, float *out, uint32_t rows, uint32_t cols,
                               void *workspace, size_t workspace_bytes, void *stream);

/* Static description of a status code. */
const char *attn_status_string(attn_status_t status);

/* Detail text of the calling thread's last non-OK return ("" if none). */
const char *attn_last_error(void);

#ifdef __cplusplus
}
#endif

#endif /* ATTN_DECODE_H */
