/*
 * kvc.h -- decode attention over a growing KV cache on AMD Instinct MI355X (gfx950).
 *
 * One new query per sequence attends every cached position of that sequence:
 *     out[b,h,:] = softmax(scale * q[b,h,:] . K[b,h,0:L_b,:]^T) . V[b,h,0:L_b,:]
 * where L_b counts the token appended in this step. Two cache layouts are served by one
 * kernel body: a contiguous [B, H, S_max, D] cache per layer, and a paged cache whose
 * sequences reach fixed 16-token physical blocks through per-sequence block tables.
 *
 * Pages cited (titles as printed, with their own section numbers):
 *   "LLM Inference Acceleration -- KV Cache" (大模型推理加速——KV Cache篇)
 *   "KV Cache Mechanism Explained" (KV缓存机制解析：优化大型语言模型推理性能)
 *   "From Neuron to GPT -- KV cache chapter" (键值缓存)
 *   "KV Cache and PagedAttention" (KV Cache与PagedAttention：大模型推理显存优化方案)
 *
 * General rules
 *   - Every call returns kvc_status. Nothing aborts and no C++ exception crosses this ABI.
 *   - Host-pool calls (kvc_pool_*, kvc_alloc ... kvc_check) touch host memory only, are not
 *     thread-safe for one pool (serialise calls per pool), and give the strong guarantee: a call
 *     that fails leaves the pool exactly as it was.
 *   - Device calls never allocate device memory. Every array they take is caller-owned device
 *     memory unless marked "host". They are stream-ordered on `stream` (a hipStream_t passed as
 *     void*; NULL is the default stream) and return once the work is queued. Arguments are
 *     validated on the host before anything is launched (KVC_E_INVALID / KVC_E_UNSUPPORTED, and
 *     nothing is queued); a launch failure reported by the runtime gives KVC_E_HIP. Faults
 *     inside kernels surface at the caller's next synchronisation.
 *   - Device arrays must be 16-byte aligned and densely packed in the stated layouts.
 *   - Kernels read device-side lengths and block ids defensively: lengths are clamped to
 *     [0, capacity] and a block id outside [0, num_blocks) makes that block contribute nothing,
 *     so malformed tables cannot make a kernel read outside the pools.
 */
#ifndef KVC_H
#define KVC_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum kvc_status {
  KVC_OK = 0,
  KVC_E_INVALID = -1,     /* bad argument (null pointer, bad size, misaligned, short buffer) */
  KVC_E_OOM = -2,         /* the block pool has no free block for the request */
  KVC_E_NOSEQ = -3,       /* the sequence id is not live */
  KVC_E_CAPACITY = -4,    /* a sequence would exceed max_blocks_per_seq blocks */
  KVC_E_UNSUPPORTED = -5, /* valid but not implemented combination (dtype, head_dim) */
  KVC_E_HIP = -6          /* the HIP runtime reported an error */
} kvc_status;

typedef enum kvc_dtype {
  KVC_F32 = 0,  /* IEEE binary32 */
  KVC_F16 = 1,  /* IEEE binary16 */
  KVC_E4M3 = 2, /* OCP fp8 e4m3 ("fn": bias 7, max 448, no inf, 0x7F/0xFF NaN); cache only */
  KVC_I8 = 3    /* two's-complement int8 codes in [-127, 127] with a scale; cache only */
} kvc_dtype;

#define KVC_BLOCK_SIZE 16

/* Human-readable name of a status code (static storage; never NULL). */
const char *kvc_status_str(kvc_status s);

/* ==================================================================================== *
 * Host-side block pool ("KV Cache and PagedAttention", sections 2.1, 2.2, 3.1, 3.3, 5.1;
 * "LLM Inference Acceleration -- KV Cache", section 6.1).
 *
 * The pool tracks, for num_blocks physical blocks of KVC_BLOCK_SIZE token slots, a reference
 * count per block, and per live sequence its length and block table (logical block i holds
 * tokens 16i .. 16i+15). One table per sequence serves every layer: each layer has its own
 * K/V pool arrays indexed by the same physical block ids. The pool never touches device
 * memory; device-side effects of its decisions are carried out by kvc_copy_blocks and
 * kvc_write_paged.
 *
 * Allocation is first fit: the first free block in pool order (section 3.1 chooses first fit).
 * Pool order is block id order, or a caller-given permutation (a shuffled pool).
 * Sequence ids are the lowest non-negative id not in use.
 * ==================================================================================== */
typedef struct kvc_pool kvc_pool; /* opaque */

typedef struct kvc_pool_stats {
  int32_t num_blocks;    /* physical blocks in the pool */
  int32_t used;          /* blocks with refcount > 0 */
  int32_t free_blocks;   /* blocks with refcount == 0 */
  int32_t shared;        /* blocks with refcount > 1 */
  int32_t num_seqs;      /* live sequences */
  int32_t reserved;
  int64_t cow_copies;    /* copy-on-write copies emitted since creation */
  int64_t tokens;        /* sum of live sequence lengths (shared prefixes counted per sequence) */
  int64_t slots_logical; /* sum over live sequences of 16 x table entries (dropped ones not counted) */
} kvc_pool_stats;

/* Create a pool. block_size must be KVC_BLOCK_SIZE. order: host int32[num_blocks], a
 * permutation of 0..num_blocks-1 giving the first-fit search order, or NULL for id order
 * (copied; the caller keeps ownership). On success *out owns the pool (kvc_pool_destroy). */
kvc_status kvc_pool_create(int32_t num_blocks, int32_t block_size, int32_t max_blocks_per_seq,
                           const int32_t *order, kvc_pool **out);
void kvc_pool_destroy(kvc_pool *pool);

/* New empty sequence (length 0, no blocks). *seq_out receives its id. */
kvc_status kvc_alloc(kvc_pool *pool, int32_t *seq_out);

/* Reserve n_tokens new token slots at the end of each listed sequence, in list order, all tokens
 * of seqs[0] first. For each token, at length L: if L % 16 == 0 a fresh block is taken (first
 * fit, refcount 1); otherwise, if the last block is shared (refcount > 1), copy-on-write takes a
 * fresh block, records the pair (old, new), drops one reference to the old block and repoints
 * the table (section 3.3); the token's slot is block*16 + L%16.
 *   seqs:        host int32[n_seqs] (a sequence may appear more than once)
 *   slots_out:   host int64[n_seqs * n_tokens]; slots_out[i*n_tokens + j] is token j of seqs[i]
 *   cow_src_out, cow_dst_out: host int32[cow_cap]; the copy pairs, in the order they arose.
 *                Copies must be carried out (kvc_copy_blocks) before the writes of this call.
 *   cow_cap:     must be >= n_seqs (each sequence copies at most once per call)
 *   n_cow_out:   host; receives the number of pairs
 * Errors: KVC_E_NOSEQ (a listed id is not live), KVC_E_CAPACITY (a table would exceed
 * max_blocks_per_seq), KVC_E_OOM (no free block), KVC_E_INVALID. On error nothing changes. */
kvc_status kvc_append(kvc_pool *pool, const int32_t *seqs, int32_t n_seqs, int32_t n_tokens,
                      int64_t *slots_out, int32_t *cow_src_out, int32_t *cow_dst_out,
                      int32_t cow_cap, int32_t *n_cow_out);

/* New sequence sharing all of parent's blocks: same length, same table, one more reference on
 * every block it holds (parallel sampling, section 5.1). *child_out receives its id. */
kvc_status kvc_fork(kvc_pool *pool, int32_t parent, int32_t *child_out);

/* End a sequence: one reference fewer on each block it holds; blocks reaching 0 become free
 * (their device contents are left as they are). */
kvc_status kvc_free(kvc_pool *pool, int32_t seq);

/* Rolling window in paged form ("KV Cache Mechanism Explained", section 8, item 2: keep only the
 * most recent WINDOW_SIZE tokens). For each listed sequence of length L, every block whose 16
 * positions all lie before max(0, L - window) is dropped: one reference released (a block that
 * reaches 0 is free) and its table entry set to -1. The length keeps counting every token, so
 * positions stay absolute and the table still needs ceil(L/16) <= max_blocks_per_seq entries;
 * dropped entries form a prefix of the table. Decode such a sequence with the window entry
 * points and the same window (they never read dropped entries).
 *   seqs:          host int32[n_seqs]
 *   window:        >= 0; 0 drops nothing
 *   n_dropped_out: host, may be NULL; receives the number of entries dropped
 * Errors: KVC_E_NOSEQ, KVC_E_INVALID (nothing changes). */
kvc_status kvc_slide(kvc_pool *pool, const int32_t *seqs, int32_t n_seqs, int32_t window,
                     int32_t *n_dropped_out);

/* Block tables and lengths of the listed sequences.
 *   tables_out: host int32[n_seqs][max_blocks_per_seq], unused (and dropped) entries are -1
 *   lens_out:   host int32[n_seqs] (may be NULL) */
kvc_status kvc_block_table(const kvc_pool *pool, const int32_t *seqs, int32_t n_seqs,
                           int32_t *tables_out, int32_t *lens_out);

kvc_status kvc_stats(const kvc_pool *pool, kvc_pool_stats *out);

/* Check the pool's invariants ("KV Cache and PagedAttention", section 6.2: leaks show up as
 * wrong reference counts): every refcount equals the number of table entries naming the block,
 * every table has exactly ceil(len/16) entries, within capacity, in range, without repeats,
 * except a prefix of entries dropped by kvc_slide (-1).
 * Returns KVC_OK or KVC_E_INVALID. */
kvc_status kvc_check(const kvc_pool *pool);

/* ==================================================================================== *
 * Device side: cache writes.
 * ==================================================================================== */

/* One layer of a paged cache (device pointers owned by the caller).
 *   k_pool, v_pool: [num_blocks][num_heads][16][head_dim] elements of kv_dtype
 *   k_scale, v_scale: float[num_blocks], one fp32 scale per block for K and for V, covering all
 *                     heads of the block (KVC_E4M3 and KVC_I8 only; NULL otherwise). The stored
 *                     value of code c in block p is e4m3(c) * scale[p], or c * scale[p]. */
typedef struct kvc_paged_layer {
  kvc_dtype kv_dtype;
  int32_t num_blocks;
  int32_t num_heads;
  int32_t head_dim; /* 64 or 128 */
  void *k_pool;
  void *v_pool;
  float *k_scale;
  float *v_scale;
} kvc_paged_layer;

/* Contiguous append ("LLM Inference Acceleration -- KV Cache", section 3.1: the new k/v are
 * stored at start_pos before attention reads the cache).
 *   k_cache, v_cache: [B][H][S_max][D] of dtype (KVC_F32 or KVC_F16)
 *   pos:   device int32[B], first position written for each sequence
 *   k_new, v_new: [B][n_tok][H][D] of dtype (token-major, as projections produce them)
 * Writes K[b,h,pos[b]+t,:] = k_new[b,t,h,:] for t < n_tok; positions outside [0, S_max) are
 * skipped. D is 64 or 128. */
kvc_status kvc_append_contig(void *k_cache, void *v_cache, kvc_dtype dtype, int32_t B, int32_t H,
                             int32_t S_max, int32_t D, const int32_t *pos, int32_t n_tok,
                             const void *k_new, const void *v_new, void *stream);

/* Carry out copy-on-write pairs ("KV Cache and PagedAttention", section 3.3, copy_block): for
 * each i < n, block dst[i] of K and V (and its fp8 scales) becomes a copy of block src[i].
 * src, dst: device int32[n]. All pairs are done in one launch. A pair naming a block outside
 * [0, num_blocks) is skipped. The dst blocks of one call must be distinct and no dst may be a src
 * (kvc_append's pairs satisfy both). */
kvc_status kvc_copy_blocks(const kvc_paged_layer *layer, const int32_t *src, const int32_t *dst,
                           int32_t n, void *stream);

/* Store new tokens' K and V at their slots (slot = block*16 + offset, from kvc_append).
 *   slots: device int64[n_tok]; k_new, v_new: [n_tok][H][D] of new_dtype
 *   f32/f16 pools: new_dtype must equal kv_dtype; a plain copy.
 *   e4m3 pools: new_dtype is KVC_F16 or KVC_F32; tokens are quantised one at a time in slot-array
 *     order with the per-block running-maximum rule: writing offset 0 starts the block afresh
 *     (scale 0); for a token x, s_new = fp32(max|x| / 448); if s_new exceeds the block's scale,
 *     codes already in offsets [0, off) are requantised as e4m3(fp32(fp32(e4m3(c) * old) /
 *     s_new)) and the scale becomes s_new; the token is stored as e4m3(fp32(x / scale)), rounded
 *     to nearest even and saturated to +-448 (signed zero while the scale is 0). ("KV Cache
 *     Mechanism Explained", section 8, item 3: fp8 e4m3 cache with a scaling factor.) All
 *     entries that target one block must be adjacent in `slots`; inputs must be finite.
 *   int8 pools ("KV Cache Mechanism Explained", section 8, item 3 names FP8/INT8 with a scaling
 *     factor max|x| / 127; "KV Cache and PagedAttention", section 7.2, 8-bit quantisation of
 *     blocks): the same rule with the int8 limit, s_new = fp32(max|x| / 127), codes
 *     rint(fp32(y / scale)) saturated to +-127 (never -128), ties to even, zero while the scale
 *     is 0.
 * Entries with a slot outside [0, 16*num_blocks) are skipped. */
kvc_status kvc_write_paged(const kvc_paged_layer *layer, const int64_t *slots, int32_t n_tok,
                           const void *k_new, const void *v_new, kvc_dtype new_dtype,
                           void *stream);

/* Compress blocks of a 16-bit (or fp32) layer into an 8-bit layer in one shot ("KV Cache
 * Mechanism Explained", section 6.1, item 1: compress the cache to 8 bits once it grows past a
 * threshold; "KV Cache and PagedAttention", section 7.2, item 1: compress inactive blocks with
 * 8-bit quantisation).
 *   src: layer with kv_dtype KVC_F16 or KVC_F32; dst: layer with kv_dtype KVC_E4M3 or KVC_I8,
 *     the same num_heads and head_dim, its own (non-overlapping) device memory.
 *   src_ids, dst_ids: device int32[n], block pairs; dst ids distinct; a pair with an id outside
 *     its pool is skipped.
 *   n_valid: device int32[n], slots of each source block that hold positions (clamped to
 *     [0, 16]; a sequence's last block may be partial), or null for 16 everywhere.
 * For each pair the destination block's K scale is fp32(max|K| / limit) over the valid slots of
 * every head (limit 448 for e4m3, 127 for int8), each valid value is stored as the code of
 * fp32(x / scale) (the write rule's encoding; signed zero while the scale is 0), the other slots
 * get code 0, and the same for V. Source values past n_valid take no part (they may hold
 * anything, NaN included). A NaN among the valid values makes the scale NaN (codes 0 for int8,
 * 0x7F for e4m3); an infinite one makes it +inf (finite values then get zero codes).
 * kvc_write_paged can then continue writing a compressed partial block with its running-maximum
 * rule. */
kvc_status kvc_compress_blocks(const kvc_paged_layer *src, const kvc_paged_layer *dst,
                               const int32_t *src_ids, const int32_t *dst_ids,
                               const int32_t *n_valid, int32_t n, void *stream);

/* ==================================================================================== *
 * Device side: decode attention.
 *
 * Pass 1 cuts the work of all (sequence, head) pairs -- H * sum_b ceil(L_b/16) tiles of 16
 * positions -- into equal contiguous chunks, one per wavefront of a grid sized to the GPU. Each
 * wavefront runs an online softmax (running max and running sum) over its chunk and either
 * writes the finished output row (when it saw the whole sequence-head) or a partial state
 * (max, sum, unnormalised output) to the workspace. Pass 2 combines the partial states of every
 * sequence-head that was split and zeroes the rows of empty sequences. Accumulation is fp32;
 * scores are never rounded below fp32 ("LLM Inference Acceleration -- KV Cache", section 3.1
 * takes the softmax in float).
 *
 * Common arguments
 *   q:        [B][H][D] of q_dtype (KVC_F32 or KVC_F16)
 *   ctx_lens: device int32[B], L_b = positions attended by sequence b (its new token included);
 *             clamped to [0, capacity]; L_b = 0 gives a zero output row
 *   max_ctx:  host upper bound of every L_b (sizes the grid; need not be tight)
 *   scale:    multiplies q.k (normally 1/sqrt(D)); finite
 *   out:      [B][H][D] of out_dtype (KVC_F32 or KVC_F16), rounded to nearest even
 *   workspace: device buffer of at least kvc_decode_workspace_bytes(B, H, D) bytes, 256-byte
 *             aligned, owned by the caller; no initialisation needed, contents overwritten.
 *             Calls that may overlap in time need different workspaces.
 * Supported: D in {64, 128}; B <= 4096; kv dtype f32/f16 (contiguous) and f32/f16/e4m3/int8
 * (paged; 8-bit codes are dequantised in-kernel with their block scales).
 * ==================================================================================== */
size_t kvc_decode_workspace_bytes(int32_t B, int32_t H, int32_t D);

/* Contiguous cache: k_cache, v_cache [B][H][S_max][D] of kv_dtype (capacity = S_max). */
kvc_status kvc_decode_attn_contig(const void *q, kvc_dtype q_dtype, const void *k_cache,
                                  const void *v_cache, kvc_dtype kv_dtype, const int32_t *ctx_lens,
                                  int32_t B, int32_t H, int32_t S_max, int32_t D, int32_t max_ctx,
                                  float scale, void *out, kvc_dtype out_dtype, void *workspace,
                                  size_t ws_bytes, void *stream);

/* Paged cache ("KV Cache and PagedAttention", section 3.2: gather each sequence's blocks
 * through its block table). block_tables: device int32[B][max_blocks_per_seq] (from
 * kvc_block_table); capacity = 16 * max_blocks_per_seq. H and D come from the layer. */
kvc_status kvc_decode_attn_paged(const void *q, kvc_dtype q_dtype, const kvc_paged_layer *layer,
                                 const int32_t *block_tables, int32_t max_blocks_per_seq,
                                 const int32_t *ctx_lens, int32_t B, int32_t max_ctx, float scale,
                                 void *out, kvc_dtype out_dtype, void *workspace, size_t ws_bytes,
                                 void *stream);

/* kvc_decode_attn_paged without a workspace argument, for callers that cannot allocate device
 * memory: code under HIP graph capture, tight serving loops, harnesses that forbid hipMalloc.
 * It allocates nothing: its workspace is a file-scope device array of this library
 * (8,667,648 bytes on each GPU it runs on, held until the process ends), looked up on the first
 * call on each device. The caller still passes q, the layer, tables, lengths and out; all other
 * arguments, layouts, results and errors are those of kvc_decode_attn_paged (the same kernels,
 * so the same output bit for bit). Limits: B <= 4096 and head_dim 64 or 128, else
 * KVC_E_INVALID / KVC_E_UNSUPPORTED before anything is queued; KVC_E_HIP if the runtime cannot
 * give the array's address. The array needs no initialisation and keeps the last call's
 * contents. Every call on one GPU shares that array: calls that may overlap in time (other
 * streams, other host threads) race and must be serialised, for example on one stream. */
kvc_status kvc_decode_attn_paged_noalloc(const void *q, kvc_dtype q_dtype,
                                         const kvc_paged_layer *layer, const int32_t *block_tables,
                                         int32_t max_blocks_per_seq, const int32_t *ctx_lens,
                                         int32_t B, int32_t max_ctx, float scale, void *out,
                                         kvc_dtype out_dtype, void *stream);

/* The two passes as separate launches, for callers that time or schedule them apart.
 * kvc_decode_attn_{contig,paged} == the matching *_partial call followed by kvc_decode_merge
 * on the same stream, workspace and out. Pass 1 leaves a record of its split in the workspace;
 * kvc_decode_merge must follow it with the same B, H, D and out before the workspace is reused.
 * The merges return KVC_E_INVALID when B times the query heads exceeds 2^31 - 1. */
kvc_status kvc_decode_partial_contig(const void *q, kvc_dtype q_dtype, const void *k_cache,
                                     const void *v_cache, kvc_dtype kv_dtype,
                                     const int32_t *ctx_lens, int32_t B, int32_t H, int32_t S_max,
                                     int32_t D, int32_t max_ctx, float scale, void *out,
                                     kvc_dtype out_dtype, void *workspace, size_t ws_bytes,
                                     void *stream);
kvc_status kvc_decode_partial_paged(const void *q, kvc_dtype q_dtype,
                                    const kvc_paged_layer *layer, const int32_t *block_tables,
                                    int32_t max_blocks_per_seq, const int32_t *ctx_lens, int32_t B,
                                    int32_t max_ctx, float scale, void *out, kvc_dtype out_dtype,
                                    void *workspace, size_t ws_bytes, void *stream);
kvc_status kvc_decode_merge(int32_t B, int32_t H, int32_t D, void *out, kvc_dtype out_dtype,
                            void *workspace, size_t ws_bytes, void *stream);

/* Whether pass 1 of a problem of these sizes leaves partial records for the merge, for callers
 * of the two-pass interface: *needed = 0 means pass 1 finishes every output row itself (few,
 * short sequence-heads run one workgroup each), so the merge launch can be skipped (it would
 * find nothing to do); 1 means the merge must follow. The one-shot calls make the same choice
 * internally. Host only: no device memory is read and nothing is queued; the answer depends on
 * the current device (its CU count and how many pass-1 wavefronts fit on a CU).
 *   paged:   1 for the paged entry points, 0 for the contiguous ones
 *   append:  1 for the kvc_append_decode_* (fused append) entry points, else 0
 *   q_dtype, kv_dtype, B, D, max_ctx, window: as passed to the pass-1 call (window 0: none)
 *   H, G:    K/V heads and query heads per K/V head (G = 1 for the multi-head calls)
 *   cap:     positions a sequence can hold: S_max (contiguous) or 16 * max_blocks_per_seq
 * Returns KVC_E_INVALID or KVC_E_UNSUPPORTED where the matching pass-1 call would for these
 * sizes and dtypes, KVC_E_INVALID if needed is null; it checks no pointer, layer or table width
 * (a paged call also rejects max_blocks_per_seq < 1, which this query does not see). B = 0
 * gives *needed = 0. */
kvc_status kvc_decode_merge_needed(int32_t paged, int32_t append, kvc_dtype q_dtype,
                                   kvc_dtype kv_dtype, int32_t B, int32_t H, int32_t G, int32_t D,
                                   int32_t cap, int32_t max_ctx, int32_t window,
                                   int32_t *needed);

/* Append and attend in one pass ("LLM Inference Acceleration -- KV Cache", section 3.1: each
 * decode step stores the new token's k/v in the cache and then attends over the whole cache,
 * itself included). Same arguments and result as the matching kvc_decode_* call, plus
 *   k_new, v_new: [B][H][D] of the cache's dtype (KVC_F32 or KVC_F16; e4m3 caches return
 *                 KVC_E_UNSUPPORTED, their block scale needs kvc_write_paged), 16-byte aligned
 * For every sequence with L_b >= 1 and every head, position L_b - 1 is the new token: its
 * scores and values are taken from k_new/v_new, and the row is stored into the cache --
 * contiguous: at [b][h][L_b-1]; paged: at offset (L_b-1) % 16 of block
 * block_tables[b][(L_b-1) / 16] (skipped if that id is outside [0, num_blocks)). Output and
 * cache contents equal those of kvc_write_paged / kvc_append_contig of the same rows followed
 * by the plain decode call, bit for bit; one read of the cache is saved. Paged callers run
 * kvc_append and kvc_block_table first, and kvc_copy_blocks for its copy-on-write pairs on the
 * same stream before this call, so that the written block belongs to this sequence alone.
 * k_cache and v_cache are written, so the contiguous variant takes them non-const. */
kvc_status kvc_append_decode_contig(const void *q, kvc_dtype q_dtype, void *k_cache,
                                    void *v_cache, kvc_dtype kv_dtype, const int32_t *ctx_lens,
                                    const void *k_new, const void *v_new, int32_t B, int32_t H,
                                    int32_t S_max, int32_t D, int32_t max_ctx, float scale,
                                    void *out, kvc_dtype out_dtype, void *workspace,
                                    size_t ws_bytes, void *stream);
kvc_status kvc_append_decode_paged(const void *q, kvc_dtype q_dtype, const kvc_paged_layer *layer,
                                   const int32_t *block_tables, int32_t max_blocks_per_seq,
                                   const int32_t *ctx_lens, const void *k_new, const void *v_new,
                                   int32_t B, int32_t max_ctx, float scale, void *out,
                                   kvc_dtype out_dtype, void *workspace, size_t ws_bytes,
                                   void *stream);
/* Pass 1 alone of the two calls above (the cache row is stored by pass 1); follow with
 * kvc_decode_merge exactly as for kvc_decode_partial_*. */
kvc_status kvc_append_decode_partial_contig(const void *q, kvc_dtype q_dtype, void *k_cache,
                                            void *v_cache, kvc_dtype kv_dtype,
                                            const int32_t *ctx_lens, const void *k_new,
                                            const void *v_new, int32_t B, int32_t H,
                                            int32_t S_max, int32_t D, int32_t max_ctx, float scale,
                                            void *out, kvc_dtype out_dtype, void *workspace,
                                            size_t ws_bytes, void *stream);
kvc_status kvc_append_decode_partial_paged(const void *q, kvc_dtype q_dtype,
                                           const kvc_paged_layer *layer,
                                           const int32_t *block_tables, int32_t max_blocks_per_seq,
                                           const int32_t *ctx_lens, const void *k_new,
                                           const void *v_new, int32_t B, int32_t max_ctx,
                                           float scale, void *out, kvc_dtype out_dtype,
                                           void *workspace, size_t ws_bytes, void *stream);

/* ==================================================================================== *
 * Shared key/value heads (MQA / GQA).
 *
 * "LLM Inference Acceleration -- KV Cache", section 6.2: with MQA all query heads share one
 * key/value head; with GQA the query heads form groups and each group shares one key/value
 * head. Here G consecutive query heads share each K/V head: query head hq (of H_kv * G) reads
 * K/V head hq / G. G = 1 is multi-head attention (results equal kvc_decode_*, bit for bit);
 * H_kv = 1 is MQA.
 *
 *   q, out:   [B][H_kv*G][D] (q_dtype, out_dtype as above)
 *   caches:   as for kvc_decode_* with H_kv heads (contiguous [B][H_kv][S_max][D]; paged: the
 *             layer's num_heads is H_kv)
 *   workspace: at least kvc_gqa_workspace_bytes(B, H_kv, G, D) bytes, otherwise as above
 *
 * With an fp16 q over an fp16 cache (or a paged e4m3 one) and G > 1, one wavefront serves gq
 * query heads of a group from each K/V tile it loads, on the matrix cores, gq being the largest
 * divisor of G up to 16; each K/V byte is then read from HBM G/gq times (once for G <= 16).
 * Other dtype combinations run one query head per wavefront (each K/V byte read G times).
 * kvc_append_decode_gqa_* below are the append-and-attend variants. */
size_t kvc_gqa_workspace_bytes(int32_t B, int32_t H_kv, int32_t G, int32_t D);

kvc_status kvc_decode_gqa_contig(const void *q, kvc_dtype q_dtype, int32_t G, const void *k_cache,
                                 const void *v_cache, kvc_dtype kv_dtype, const int32_t *ctx_lens,
                                 int32_t B, int32_t H_kv, int32_t S_max, int32_t D,
                                 int32_t max_ctx, float scale, void *out, kvc_dtype out_dtype,
                                 void *workspace, size_t ws_bytes, void *stream);
kvc_status kvc_decode_gqa_paged(const void *q, kvc_dtype q_dtype, int32_t G,
                                const kvc_paged_layer *layer, const int32_t *block_tables,
                                int32_t max_blocks_per_seq, const int32_t *ctx_lens, int32_t B,
                                int32_t max_ctx, float scale, void *out, kvc_dtype out_dtype,
                                void *workspace, size_t ws_bytes, void *stream);
/* The two passes of the calls above, as for kvc_decode_partial_* and kvc_decode_merge. */
kvc_status kvc_decode_gqa_partial_contig(const void *q, kvc_dtype q_dtype, int32_t G,
                                         const void *k_cache, const void *v_cache,
                                         kvc_dtype kv_dtype, const int32_t *ctx_lens, int32_t B,
                                         int32_t H_kv, int32_t S_max, int32_t D, int32_t max_ctx,
                                         float scale, void *out, kvc_dtype out_dtype,
                                         void *workspace, size_t ws_bytes, void *stream);
kvc_status kvc_decode_gqa_partial_paged(const void *q, kvc_dtype q_dtype, int32_t G,
                                        const kvc_paged_layer *layer, const int32_t *block_tables,
                                        int32_t max_blocks_per_seq, const int32_t *ctx_lens,
                                        int32_t B, int32_t max_ctx, float scale, void *out,
                                        kvc_dtype out_dtype, void *workspace, size_t ws_bytes,
                                        void *stream);
kvc_status kvc_decode_gqa_merge(int32_t B, int32_t H_kv, int32_t G, int32_t D, void *out,
                                kvc_dtype out_dtype, void *workspace, size_t ws_bytes,
                                void *stream);
/* Append and attend in one pass with shared K/V heads: the kvc_append_decode_* contract
 * (section 3.1 of "LLM Inference Acceleration -- KV Cache", as above) with G query heads per K/V
 * head as for kvc_decode_gqa_*. k_new, v_new: [B][H_kv][D], one row per sequence and K/V head,
 * of the cache's dtype (KVC_F32 or KVC_F16; 8-bit caches return KVC_E_UNSUPPORTED). Every query
 * head of a group scores the new row from k_new/v_new; the row is stored into the cache once.
 * Output and cache contents equal kvc_write_paged / kvc_append_contig of the same rows followed
 * by kvc_decode_gqa_*, bit for bit. The _partial forms are pass 1 alone; follow them with
 * kvc_decode_gqa_merge. */
kvc_status kvc_append_decode_gqa_contig(const void *q, kvc_dtype q_dtype, int32_t G,
                                        void *k_cache, void *v_cache, kvc_dtype kv_dtype,
                                        const int32_t *ctx_lens, const void *k_new,
                                        const void *v_new, int32_t B, int32_t H_kv, int32_t S_max,
                                        int32_t D, int32_t max_ctx, float scale, void *out,
                                        kvc_dtype out_dtype, void *workspace, size_t ws_bytes,
                                        void *stream);
kvc_status kvc_append_decode_gqa_paged(const void *q, kvc_dtype q_dtype, int32_t G,
                                       const kvc_paged_layer *layer, const int32_t *block_tables,
                                       int32_t max_blocks_per_seq, const int32_t *ctx_lens,
                                       const void *k_new, const void *v_new, int32_t B,
                                       int32_t max_ctx, float scale, void *out,
                                       kvc_dtype out_dtype, void *workspace, size_t ws_bytes,
                                       void *stream);
kvc_status kvc_append_decode_gqa_partial_contig(const void *q, kvc_dtype q_dtype, int32_t G,
                                                void *k_cache, void *v_cache, kvc_dtype kv_dtype,
                                                const int32_t *ctx_lens, const void *k_new,
                                                const void *v_new, int32_t B, int32_t H_kv,
                                                int32_t S_max, int32_t D, int32_t max_ctx,
                                                float scale, void *out, kvc_dtype out_dtype,
                                                void *workspace, size_t ws_bytes, void *stream);
kvc_status kvc_append_decode_gqa_partial_paged(const void *q, kvc_dtype q_dtype, int32_t G,
                                               const kvc_paged_layer *layer,
                                               const int32_t *block_tables,
                                               int32_t max_blocks_per_seq, const int32_t *ctx_lens,
                                               const void *k_new, const void *v_new, int32_t B,
                                               int32_t max_ctx, float scale, void *out,
                                               kvc_dtype out_dtype, void *workspace,
                                               size_t ws_bytes, void *stream);

/* ==================================================================================== *
 * Rolling window ("KV Cache Mechanism Explained", section 8, item 2: the cache keeps only the
 * most recent WINDOW_SIZE tokens).
 *
 * Sequence b attends positions max(0, L_b - window) .. L_b - 1 (the new token included), with
 * L_b = ctx_lens[b] clamped to the capacity as above; window >= 1 (KVC_E_INVALID otherwise). G
 * query heads share each K/V head exactly as for kvc_decode_gqa_* (G = 1: multi-head). All
 * other arguments, layouts and errors are those of kvc_decode_gqa_*; the workspace is sized by
 * kvc_gqa_workspace_bytes(B, H_kv, G, D).
 *   Paged: positions keep their absolute logical blocks (block b // 16 of the table); entries
 *     before block max(0, L_b - window) / 16 are never read, so a pool slid with kvc_slide and
 *     the same window decodes correctly.
 *   Contiguous: a window over the full-length cache [B][H_kv][S_max][D]. A cache that holds only
 *     the window can instead be a ring of W = S_max slots (position p stored at slot p % W,
 *     kvc_append_contig) decoded by kvc_decode_gqa_contig with ctx_lens min(L_b, W): attention
 *     does not depend on the order of positions. */
kvc_status kvc_decode_window_contig(const void *q, kvc_dtype q_dtype, int32_t G,
                                    const void *k_cache, const void *v_cache, kvc_dtype kv_dtype,
                                    const int32_t *ctx_lens, int32_t B, int32_t H_kv,
                                    int32_t S_max, int32_t D, int32_t max_ctx, int32_t window,
                                    float scale, void *out, kvc_dtype out_dtype, void *workspace,
                                    size_t ws_bytes, void *stream);
kvc_status kvc_decode_window_paged(const void *q, kvc_dtype q_dtype, int32_t G,
                                   const kvc_paged_layer *layer, const int32_t *block_tables,
                                   int32_t max_blocks_per_seq, const int32_t *ctx_lens, int32_t B,
                                   int32_t max_ctx, int32_t window, float scale, void *out,
                                   kvc_dtype out_dtype, void *workspace, size_t ws_bytes,
                                   void *stream);
/* Pass 1 alone of the two calls above; follow with kvc_decode_gqa_merge. */
kvc_status kvc_decode_window_partial_contig(const void *q, kvc_dtype q_dtype, int32_t G,
                                            const void *k_cache, const void *v_cache,
                                            kvc_dtype kv_dtype, const int32_t *ctx_lens,
                                            int32_t B, int32_t H_kv, int32_t S_max, int32_t D,
                                            int32_t max_ctx, int32_t window, float scale,
                                            void *out, kvc_dtype out_dtype, void *workspace,
                                            size_t ws_bytes, void *stream);
kvc_status kvc_decode_window_partial_paged(const void *q, kvc_dtype q_dtype, int32_t G,
                                           const kvc_paged_layer *layer,
                                           const int32_t *block_tables,
                                           int32_t max_blocks_per_seq, const int32_t *ctx_lens,
                                           int32_t B, int32_t max_ctx, int32_t window,
                                           float scale, void *out, kvc_dtype out_dtype,
                                           void *workspace, size_t ws_bytes, void *stream);

/* ==================================================================================== *
 * Chunked prefill: several new tokens per sequence attend with the causal mask ("LLM Inference
 * Acceleration -- KV Cache", section 3.1: a forward pass over seqlen > 1 tokens at start_pos uses
 * triu(-inf, start_pos + 1); "KV Cache and PagedAttention", section 5.3: FlashAttention tiles
 * within blocks, PagedAttention between blocks).
 *
 * Sequence b's chunk is rows q_start[b] .. q_start[b+1]-1 of q and out: its last
 * n_b = q_start[b+1] - q_start[b] positions, whose K/V are already in the cache (written with
 * kvc_append_contig / kvc_write_paged). L_b = ctx_lens[b] counts every position, the chunk
 * included. Row i of the chunk (position L_b - n_b + i) attends positions 0 .. L_b - n_b + i.
 * G query heads share each K/V head as for kvc_decode_gqa_* (G = 1: multi-head).
 *   q, out:    [total_q][H_kv*G][D] (q fp16; out fp16, rounded to nearest even, or fp32)
 *   q_start:   device int32[B+1], non-decreasing, q_start[B] <= total_q
 *   ctx_lens:  device int32[B], clamped to [0, capacity]; a chunk longer than L_b keeps its first
 *              L_b rows (the rest of out is not written)
 *   caches:    fp16 only, as for kvc_decode_* (contiguous [B][H_kv][S_max][D]; paged layer with
 *              H_kv heads and the block tables of the sequences)
 * D = 64 or 128. No workspace. Each workgroup of 4 wavefronts computes two tiles of 128 query
 * rows of one sequence (a long and a short one) to the end: no split across workgroups, no merge.
 * Errors: KVC_E_UNSUPPORTED (dtypes, D), KVC_E_INVALID (shapes, alignment, B > 4096); block ids
 * outside the pool skip their block. */
kvc_status kvc_prefill_contig(const void *q, kvc_dtype q_dtype, int32_t G, const void *k_cache,
                              const void *v_cache, kvc_dtype kv_dtype, const int32_t *q_start,
                              const int32_t *ctx_lens, int32_t B, int32_t H_kv, int32_t S_max,
                              int32_t D, int32_t total_q, float scale, void *out,
                              kvc_dtype out_dtype, void *stream);
kvc_status kvc_prefill_paged(const void *q, kvc_dtype q_dtype, int32_t G,
                             const kvc_paged_layer *layer, const int32_t *block_tables,
                             int32_t max_blocks_per_seq, const int32_t *q_start,
                             const int32_t *ctx_lens, int32_t B, int32_t total_q, float scale,
                             void *out, kvc_dtype out_dtype, void *stream);

/* ==================================================================================== *
 * Measurement: the read ceiling of an access pattern ("LLM Inference Acceleration -- KV Cache",
 * section 6.3: decode is bound by memory bandwidth, so its rate is compared with a pure read of
 * the same bytes in the same pattern).
 *
 * kvc_read_pieces reads n pieces of piece_bytes (1024, 2048, 4096 or 8192) bytes: piece i at
 * a + offsets[i] and, when b is not NULL, at b + offsets[i] as well (the K and V tiles of one
 * work-list entry). Wavefront w of a grid of P = waves_per_cu (1..32) x compute units reads
 * pieces w*C .. w*C + C - 1 (C = ceil(n / P)) in order, with 16-byte non-temporal loads, and
 * writes a checksum word to sink[w] (device uint32[sink_words], sink_words >= P; P <= 65536).
 * a, b: 16-byte aligned device memory; offsets: device int64[n], multiples of 16, each piece
 * inside the caller's buffers (the probe cannot check device arrays). Nothing else is computed;
 * the caller times the launch. */
kvc_status kvc_read_pieces(const void *a, const void *b, const int64_t *offsets, int32_t n,
                           int32_t piece_bytes, int32_t waves_per_cu, uint32_t *sink,
                           size_t sink_words, void *stream);

#ifdef __cplusplus
}
#endif

#endif /* KVC_H */
