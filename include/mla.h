/*
 * mla.h -- C ABI of libmla: MLA (multi-head latent attention) paged decode
 * for AMD Instinct MI355X (gfx950).
 *
 * What the library computes.  At one decode step every sequence b has one
 * query per head, q[b, h, 0:D] = [q_nope (D_v) | q_pe (64)], and a paged
 * cache of latent rows [kv_c (D_v = kv_lora_rank) | k_pe (64)], one row per
 * context position.  All H heads read the same row stream as a single-head K
 * (multi-query attention), and V is the first D_v columns of that same row
 * ("Triton と MLA" page, section データフロー / data flow: the cache is passed
 * to the decode kernel as a one-head K cache and its leading kv_lora_rank
 * slice as V).  Position t of sequence b lives in physical page
 * block_table[b][t / page_size], slot t % page_size ("vLLM 中 Attention
 * Kernel 如何并行处理多个请求", section 十一).  A decode query sees every
 * position, so there is no mask (same article, section 九).  Outputs:
 *
 *     s[t]      = scale * sum_d q[b,h,d] * K[t,d]        (d < D, t < n_b)
 *     lse[b,h]  = ln sum_t exp(s[t])                      (natural log)
 *     o[b,h,:]  = sum_t exp(s[t] - lse[b,h]) * K[t, 0:D_v]
 *
 * lse is always returned and is a natural logarithm ("Triton と MLA" page,
 * 設計動機: lse is returned for cross-shard merging and lse_base_on_e
 * defaults to true; "AttentionBackend" page, Limites et échecs: ln versus
 * log2 must not be mixed).  For an fp8 cache one per-layer scale k_scale
 * multiplies every element of K and V; for a bf16 cache k_scale is ignored
 * ("Triton と MLA" page, データフロー: k_scale = v_scale = the layer's
 * _k_scale, and the fp8 check is a no-op for bf16 caches).
 *
 * How it is computed.  Stage 1 splits each sequence's positions into
 * segments and runs an online softmax (running max, running sum, rescaled
 * accumulator; article section 七) over 32-position tiles of each segment.
 * Each segment yields a partial (o_s, lse_s); a sequence covered by a single
 * segment is written to o/lse directly.  Stage 2 merges the partials of the
 * other sequences with the log-sum-exp rule of article section 十二.  Both
 * stages run as HIP kernels on the caller's stream.
 *
 * Conventions for every function below.
 *   - Device pointers are HIP device addresses owned by the caller; the
 *     library never allocates, frees, copies to the host or synchronises.
 *   - Arguments are checked on the host before anything is enqueued; on any
 *     error the function returns a non-zero mla_status and enqueues nothing.
 *   - Table contents are not validated before a launch (that would need a
 *     device-to-host copy), but the kernels stay inside every buffer whatever
 *     they hold: a length in seq_lens is clamped to [0, max_blocks_per_seq *
 *     page_size] (a top-k length to [0, topk]); a block_table entry outside
 *     [0, num_blocks) and a top-k position outside [0, max_blocks_per_seq *
 *     page_size) read as all-zero cache rows.  The results of such a call
 *     are unspecified.  mla_check_inputs() checks host copies of the tables
 *     and names the first offending entry.
 *   - Entry points are re-entrant; concurrent calls must use distinct
 *     workspaces and outputs.
 */
#ifndef MLA_H_
#define MLA_H_

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum mla_status {
  MLA_OK = 0,
  MLA_ERR_NULL = 1,      /* a required pointer is NULL                                   */
  MLA_ERR_HEAD_SIZE = 2, /* head_size not 576 or 320, or kv_lora_rank != head_size - 64
                            ("Triton と MLA" page, 設計動機 and 境界と失敗: only these two
                            head sizes are accepted)                                    */
  MLA_ERR_PAGE_SIZE = 3, /* page_size not a positive multiple of 16, or the page_size
                            argument differs from shape->page_size ("AttentionBackend"
                            page, Limites et échecs: block sizes are multiples of 16)   */
  MLA_ERR_DTYPE = 4,     /* q not bf16 (an fp8 query is refused: "Triton と MLA" page,
                            境界と失敗), kv not bf16 / fp8 e4m3fn (per-tensor or
                            per-token scale) / per-token int8 / per-token int4, o not
                            bf16/fp32                                                    */
  MLA_ERR_SHAPE = 5,     /* batch < 1 or above MLA_MAX_BATCH, num_heads not a positive
                            multiple of 16 or above MLA_MAX_ROWS, num_blocks < 1 (empty
                            cache), max_blocks_per_seq < 1, a size whose byte count
                            overflows, or a launch grid beyond the HIP limit             */
  MLA_ERR_SPLITS = 6,    /* num_kv_splits < 1 or above MLA_MAX_KV_SPLITS, or an unknown
                            split mode                                                   */
  MLA_ERR_WORKSPACE = 7, /* workspace NULL or smaller than mla_workspace_size() for the
                            same shape, split mode and split count                       */
  MLA_ERR_LAUNCH = 8,    /* HIP reported an error when the kernels were enqueued        */
  MLA_ERR_ARGUMENT = 9,  /* a non-finite or non-positive scale / k_scale, num_cus < 1,
                            q_len outside [1, MLA_MAX_Q_LEN] or q_len x num_heads above
                            MLA_MAX_ROWS, topk < 1, or a misaligned pointer or query
                            stride                                                       */
  MLA_ERR_TABLE = 10,    /* mla_check_inputs: a length, block-table entry or top-k entry
                            out of range                                                 */
  MLA_ERR_SCRATCH = 11   /* mla_decode_noalloc: the split layout needs more workspace than
                            the built-in scratch holds (mla_noalloc_scratch_bytes())     */
} mla_status;

typedef enum mla_dtype {
  MLA_BF16 = 0,     /* bfloat16                                                       */
  MLA_FP8_E4M3 = 1, /* OCP fp8 e4m3fn: bias 7, max 448, no infinity (cache only)      */
  MLA_FP32 = 2,     /* float32 (output only)                                          */
  /* Cache only: fp8 e4m3fn codes with one scale per token, stored inline.  A
   * row is head_size code bytes followed by a MLA_PER_TOKEN_PAD-byte pad whose
   * first 4 bytes are the token's little-endian float32 scale (the other 12
   * are never read); value = code * scale, for K and V alike ("Triton と MLA"
   * page, 主要ファイル: in the per-token-head modes the cache's head_dim is
   * padded to hold an inline scale).  k_scale does not apply.  Rows start on
   * 16-byte boundaries (head_size + 16 is a multiple of 16). */
  MLA_FP8_E4M3_PER_TOKEN = 3,
  /* Cache only: as MLA_FP8_E4M3_PER_TOKEN with signed (two's-complement)
   * int8 codes; value = code * scale (the same page lists int8 among the
   * per-token-head modes). */
  MLA_INT8_PER_TOKEN = 4,
  /* Cache only: two signed (two's-complement) 4-bit codes per byte, element
   * 2i in the low nibble and 2i+1 in the high nibble of byte i; a row is
   * head_size / 2 code bytes followed by the MLA_PER_TOKEN_PAD-byte pad with
   * the token's float32 scale; value = code * scale (the same page lists
   * int4 among the per-token-head modes).  Rows start on 16-byte boundaries
   * (head_size / 2 + 16 is a multiple of 16). */
  MLA_INT4_PER_TOKEN = 5
} mla_dtype;

#define MLA_PER_TOKEN_PAD 16 /* bytes after the codes of a per-token cache row */

/* How stage 1 divides the positions of a batch among workgroups.
 *
 * MLA_SPLIT_PER_SEQUENCE -- the split-KV layout of the "Triton と MLA" page
 *   (num_kv_splits per request, workspace [B, S] partials): sequence b is cut
 *   into S segments of C_b = roundup(ceil(n_b / S), 32) positions; segment s
 *   covers [s*C_b, min((s+1)*C_b, n_b)) and may be empty.  With S == 1 every
 *   sequence is reduced by one workgroup in a fixed order: the result of a
 *   sequence does not depend on the rest of the batch and is bitwise
 *   reproducible (the page's batch-invariant mode forces one split), and no
 *   workspace is needed.  Any fixed S keeps the same property: a sequence's
 *   segments depend only on its own length and S, each is reduced in a fixed
 *   order and stage 2 merges them in a fixed order, so a caller that fixes S
 *   (rather than taking it from the batch's lengths) gets bitwise the same
 *   result for a sequence in any batch, with up to S workgroups per sequence.
 *
 * MLA_SPLIT_BALANCED -- the batch's 32-position tiles, sequence after
 *   sequence, are cut into S equal runs ("work units"), one per workgroup and
 *   head chunk, so that every workgroup does the same amount of work whatever
 *   the mix of lengths.  Each non-empty sequence is charged a few extra
 *   virtual tiles for the fixed cost of starting a segment (its query load
 *   and partial store), so a unit that also starts a new sequence streams
 *   correspondingly fewer tiles.  A unit may hold the end of one sequence and
 *   the start of the next.  Results are reproducible run to run for the same
 *   batch, but a sequence's rounding may depend on the other lengths.
 */
typedef enum mla_split_mode {
  MLA_SPLIT_PER_SEQUENCE = 0,
  MLA_SPLIT_BALANCED = 1
} mla_split_mode;

#define MLA_MAX_KV_SPLITS 65536
#define MLA_ROPE_DIM 64
#define MLA_MAX_Q_LEN 16 /* query tokens per sequence in multi-token decode */
#define MLA_MAX_ROWS 65536      /* query rows per sequence: num_heads x q_len */
#define MLA_MAX_BATCH (1 << 24) /* sequences per call */

/* Problem shape.  Layouts (all row-major, densely packed unless noted):
 *   q           [batch, num_heads, head_size]              q_dtype (bf16)
 *   kv_cache    [num_blocks, page_size, head_size]         kv_dtype; row =
 *               [kv_c (kv_lora_rank) | k_pe (64)]; per-token caches are
 *               [num_blocks, page_size, C + MLA_PER_TOKEN_PAD] bytes,
 *               C = head_size (fp8, int8 codes) or head_size / 2 (int4)
 *   block_table [batch, max_blocks_per_seq]                int32; entries at
 *               index >= ceil(seq_lens[b] / page_size) are never read
 *   seq_lens    [batch]                                    int32, >= 0
 *   o           [batch, num_heads, kv_lora_rank]           o_dtype
 *   lse         [batch, num_heads]                         float32
 */
typedef struct mla_shape {
  int32_t batch;              /* B >= 1                                     */
  int32_t num_heads;          /* H, a multiple of 16                        */
  int32_t head_size;          /* D: 576 or 320                              */
  int32_t kv_lora_rank;       /* D_v = D - 64: 512 or 256                   */
  int32_t page_size;          /* P, a multiple of 16                        */
  int32_t num_blocks;         /* pages in the pool, >= 1                    */
  int32_t max_blocks_per_seq; /* block_table row stride in entries, >= 1    */
  int32_t q_dtype;            /* mla_dtype: MLA_BF16                        */
  int32_t kv_dtype;           /* mla_dtype: MLA_BF16, MLA_FP8_E4M3,
                                 MLA_FP8_E4M3_PER_TOKEN, MLA_INT8_PER_TOKEN
                                 or MLA_INT4_PER_TOKEN */
  int32_t o_dtype;            /* mla_dtype: MLA_BF16 or MLA_FP32            */
} mla_shape;

/* The split count of the "Triton と MLA" page (主要ファイル,
 * _compute_num_kv_splits): one split per 512 positions of the longest
 * sequence, capped at twice the number of compute units.  Read as
 * clamp(ceil(max_seq_len / 512), 1, 2 * num_cus).  Pure host function;
 * returns 0 if num_cus < 1. */
int32_t mla_pages_split_count(int32_t max_seq_len, int32_t num_cus);

/* Choose a split mode and count for a batch, and the workspace it needs.
 *   max_seq_len    longest sequence in the batch (host-side metadata)
 *   total_seq_len  sum of the batch's lengths, or <= 0 if unknown (then
 *                  batch * max_seq_len is assumed)
 *   num_cus        compute units of the device (256 on MI355X)
 *   deterministic  non-zero: MLA_SPLIT_PER_SEQUENCE with one split (no
 *                  workspace, batch-invariant, see above)
 * Otherwise the balanced mode is chosen with enough units to fill the device.
 * The same function is meant to run when the workspace is reserved and when
 * decode is called, so the two always agree ("Triton と MLA" page, 境界と失敗:
 * stage 2 must see the split count stage 1 used).  Pure host function, no HIP
 * call.  Outputs may not be NULL. */
mla_status mla_plan(const mla_shape* shape, int32_t max_seq_len, int64_t total_seq_len,
                    int32_t num_cus, int32_t deterministic, int32_t* split_mode,
                    int32_t* num_kv_splits, size_t* workspace_bytes);

/* Bytes of device workspace mla_decode needs for this shape, split mode and
 * split count (0 when none is needed: per-sequence mode with one split).
 * Returns 0 as well for an invalid shape or mode; mla_decode rejects those.
 * Pure host function. */
size_t mla_workspace_size(const mla_shape* shape, int32_t split_mode, int32_t num_kv_splits);

/* Enqueue one MLA decode step on `hip_stream` (a hipStream_t, NULL for the
 * null stream) of the current HIP device.
 *   q, kv_cache, block_table, seq_lens   inputs, layouts as in mla_shape
 *   scale          softmax scale applied to q.K (e.g. 192^-0.5), finite > 0
 *   page_size      must equal shape->page_size
 *   k_scale        per-layer dequantisation scale of an MLA_FP8_E4M3 cache
 *                  (finite > 0); ignored for bf16 and per-token caches
 *   num_kv_splits, split_mode   as returned by mla_plan (or chosen freely)
 *   o, lse         outputs, every [b, h] entry is overwritten; a sequence
 *                  with seq_lens[b] == 0 gets o = 0 and lse = -inf
 *   workspace      device buffer of at least
 *                  mla_workspace_size(shape, split_mode, num_kv_splits) bytes
 *                  (may be NULL when that size is 0); contents on return are
 *                  unspecified
 * Returns MLA_OK once the kernels are enqueued; results are ready when the
 * stream reaches them.  Inputs are not modified. */
mla_status mla_decode(const mla_shape* shape, const void* q, const void* kv_cache,
                      const int32_t* block_table, const int32_t* seq_lens, float scale,
                      int32_t page_size, float k_scale, int32_t num_kv_splits,
                      int32_t split_mode, void* o, float* lse, void* workspace,
                      size_t workspace_bytes, void* hip_stream);

/* The two halves of mla_decode, for callers that time or schedule them
 * apart.  Same arguments, checks and ownership as mla_decode; issuing
 * mla_decode_stage1 then mla_decode_stage2 on one stream with the same
 * arguments is exactly mla_decode.
 *   stage1  the split-KV attention over every segment ("vLLM 中 Attention
 *           Kernel 如何并行处理多个请求", section 十二, the parallel segments):
 *           sequences covered by one segment get their final o/lse, the others
 *           leave (o_s, lse_s) partials in the workspace.
 *   stage2  the log-sum-exp merge of those partials into o/lse (same section,
 *           the second reduction kernel); enqueues nothing when the split
 *           layout produced no partials (per-sequence mode with one split). */
mla_status mla_decode_stage1(const mla_shape* shape, const void* q, const void* kv_cache,
                             const int32_t* block_table, const int32_t* seq_lens, float scale,
                             int32_t page_size, float k_scale, int32_t num_kv_splits,
                             int32_t split_mode, void* o, float* lse, void* workspace,
                             size_t workspace_bytes, void* hip_stream);
mla_status mla_decode_stage2(const mla_shape* shape, const void* q, const void* kv_cache,
                             const int32_t* block_table, const int32_t* seq_lens, float scale,
                             int32_t page_size, float k_scale, int32_t num_kv_splits,
                             int32_t split_mode, void* o, float* lse, void* workspace,
                             size_t workspace_bytes, void* hip_stream);

/* Multi-token decode (verification of q_len new positions per sequence,
 * "vLLM 中 Attention Kernel 如何并行处理多个请求", section 十).  Each sequence
 * has q_len query tokens; seq_lens[b] = n counts every key, the q_len new
 * positions included (their cache rows are written before the call), so the
 * context before them is n - q_len.  Query token i sits at absolute position
 * n - q_len + i and sees the keys at positions <= n - q_len + i: the whole
 * context and new positions 0..i (a rectangle plus a lower triangle).
 *
 * Layouts: q [batch, q_len, num_heads, head_size], o [batch, q_len, num_heads,
 * kv_lora_rank], lse [batch, q_len, num_heads]; shape->num_heads is H per
 * token.  Every other argument, check and ownership rule is that of the
 * corresponding single-token function, which is the case q_len = 1.  Plan
 * and size the workspace with the _mtp functions (the q_len x H rows share
 * one cache stream).  A query row that sees no key (seq_lens[b] < q_len, or
 * 0) gets o = 0 and lse = -inf.  q_len outside [1, MLA_MAX_Q_LEN] is
 * MLA_ERR_ARGUMENT. */
mla_status mla_plan_mtp(const mla_shape* shape, int32_t q_len, int32_t max_seq_len,
                        int64_t total_seq_len, int32_t num_cus, int32_t deterministic,
                        int32_t* split_mode, int32_t* num_kv_splits, size_t* workspace_bytes);
size_t mla_workspace_size_mtp(const mla_shape* shape, int32_t q_len, int32_t split_mode,
                              int32_t num_kv_splits);
mla_status mla_decode_mtp(const mla_shape* shape, int32_t q_len, const void* q,
                          const void* kv_cache, const int32_t* block_table,
                          const int32_t* seq_lens, float scale, int32_t page_size, float k_scale,
                          int32_t num_kv_splits, int32_t split_mode, void* o, float* lse,
                          void* workspace, size_t workspace_bytes, void* hip_stream);
mla_status mla_decode_mtp_stage1(const mla_shape* shape, int32_t q_len, const void* q,
                                 const void* kv_cache, const int32_t* block_table,
                                 const int32_t* seq_lens, float scale, int32_t page_size,
                                 float k_scale, int32_t num_kv_splits, int32_t split_mode,
                                 void* o, float* lse, void* workspace, size_t workspace_bytes,
                                 void* hip_stream);
mla_status mla_decode_mtp_stage2(const mla_shape* shape, int32_t q_len, const void* q,
                                 const void* kv_cache, const int32_t* block_table,
                                 const int32_t* seq_lens, float scale, int32_t page_size,
                                 float k_scale, int32_t num_kv_splits, int32_t split_mode,
                                 void* o, float* lse, void* workspace, size_t workspace_bytes,
                                 void* hip_stream);

/* The query as two separate parts, q_nope (the first kv_lora_rank columns of a
 * query row) and q_pe (the last 64), each with its own strides, read directly
 * by the decode kernel: no concatenated copy is made ("Triton と MLA" page,
 * データフロー: forward_mqa takes q either whole or as the tuple (q_nope,
 * q_pe) and joins the tuple on the last axis, in that order, before the
 * kernel).  Row r of sequence b (r = query token * num_heads + head) is
 *     [ q_nope + b * nope_seq_stride + r * nope_row_stride : kv_lora_rank elems
 *     | q_pe   + b * pe_seq_stride   + r * pe_row_stride   : 64 elems ]
 * Strides are in bf16 elements, non-negative multiples of 8 (each 16-byte
 * chunk is loaded aligned); both pointers are 16-byte aligned device
 * pointers owned by the caller. */
typedef struct mla_query {
  const void* q_nope;
  const void* q_pe;
  int64_t nope_seq_stride, nope_row_stride;
  int64_t pe_seq_stride, pe_row_stride;
} mla_query;

/* mla_decode_mtp (q_len = 1: mla_decode) with the query given as an
 * mla_query instead of one contiguous [B, q_len, H, head_size] tensor.  Every
 * other argument, check, layout and ownership rule is that of
 * mla_decode_mtp; a misaligned pointer or stride is MLA_ERR_ARGUMENT, a NULL
 * query or part MLA_ERR_NULL.  With q_nope = q, q_pe = q + kv_lora_rank and
 * strides (q_len * H * head_size, head_size) for both parts the call is
 * exactly mla_decode_mtp on q. */
mla_status mla_decode_split_q(const mla_shape* shape, int32_t q_len, const mla_query* q,
                              const void* kv_cache, const int32_t* block_table,
                              const int32_t* seq_lens, float scale, int32_t page_size,
                              float k_scale, int32_t num_kv_splits, int32_t split_mode, void* o,
                              float* lse, void* workspace, size_t workspace_bytes,
                              void* hip_stream);

/* Sparse (top-k) decode ("vLLM 中 Attention Kernel 如何并行处理多个请求",
 * section 十三): each sequence attends only to a selected list of its
 * positions, e.g. the top 2048, instead of all of them.  Request isolation is
 * unchanged: the selected logical positions go through the sequence's block
 * table to physical slots.  Sequence b attends to the cache rows of
 *     topk_indices[b * topk + e]   for e < topk_lens[b]
 * (logical positions, each < that sequence's length; a position listed twice
 * counts twice).  Everything else is as in mla_decode, with topk_lens[b] in
 * place of seq_lens[b] for the split plan (plan with max_seq_len = topk and
 * total_seq_len = sum of topk_lens; workspace from mla_workspace_size).
 *   topk_indices  [batch, topk] int32, device; entries and topk_lens[b] <= topk
 *                 are not validated (see the conventions above:
 *                 out-of-range values stay inside every buffer)
 *   topk_lens     [batch] int32, device; 0 gives o = 0, lse = -inf
 * The index-driven gather takes every cache dtype, head size and head count
 * mla_decode takes, for pools of at most 4 GB (else MLA_ERR_SHAPE); topk < 1
 * is MLA_ERR_ARGUMENT, NULL lists MLA_ERR_NULL. */
mla_status mla_decode_sparse(const mla_shape* shape, int32_t topk, const void* q,
                             const void* kv_cache, const int32_t* block_table,
                             const int32_t* topk_indices, const int32_t* topk_lens, float scale,
                             int32_t page_size, float k_scale, int32_t num_kv_splits,
                             int32_t split_mode, void* o, float* lse, void* workspace,
                             size_t workspace_bytes, void* hip_stream);
mla_status mla_decode_sparse_stage1(const mla_shape* shape, int32_t topk, const void* q,
                                    const void* kv_cache, const int32_t* block_table,
                                    const int32_t* topk_indices, const int32_t* topk_lens,
                                    float scale, int32_t page_size, float k_scale,
                                    int32_t num_kv_splits, int32_t split_mode, void* o,
                                    float* lse, void* workspace, size_t workspace_bytes,
                                    void* hip_stream);
mla_status mla_decode_sparse_stage2(const mla_shape* shape, int32_t topk, const void* q,
                                    const void* kv_cache, const int32_t* block_table,
                                    const int32_t* topk_indices, const int32_t* topk_lens,
                                    float scale, int32_t page_size, float k_scale,
                                    int32_t num_kv_splits, int32_t split_mode, void* o,
                                    float* lse, void* workspace, size_t workspace_bytes,
                                    void* hip_stream);

/* Allocation-free decode, for callers that cannot allocate device memory
 * (code under HIP graph capture, tight serving loops, harnesses that forbid
 * allocation): mla_decode_mtp (q_len = 1: mla_decode) without the workspace
 * arguments.  The stage-1 partials go to a scratch array built into the
 * library, one copy per device, of mla_noalloc_scratch_bytes() bytes
 * (64 MiB, held from the library's load until the process ends); the call
 * itself allocates nothing, synchronises nothing and enqueues the same
 * kernels as mla_decode_mtp with the same split plan, so its results are
 * bitwise those of mla_decode_mtp.  A split layout whose
 * mla_workspace_size_mtp() exceeds the scratch is refused with
 * MLA_ERR_SCRATCH before anything is enqueued (plan fewer units or use
 * mla_decode_mtp with a workspace).  The scratch needs no clearing: every
 * byte a call reads is written earlier in the same call.  All calls on one
 * device share its scratch: calls that may overlap in time on one device
 * (concurrent streams, or calls from several host threads) race and must be
 * serialised by the caller; calls in order on one stream are safe.  Every
 * other argument, check and ownership rule is that of mla_decode_mtp. */
mla_status mla_decode_noalloc(const mla_shape* shape, int32_t q_len, const void* q,
                              const void* kv_cache, const int32_t* block_table,
                              const int32_t* seq_lens, float scale, int32_t page_size,
                              float k_scale, int32_t num_kv_splits, int32_t split_mode, void* o,
                              float* lse, void* hip_stream);
/* Bytes of the built-in scratch of mla_decode_noalloc (pure host). */
size_t mla_noalloc_scratch_bytes(void);

/* Host-side check of the tables a decode call will read ("vLLM 中 Attention
 * Kernel 如何并行处理多个请求", section 十一: each request reaches the cache only
 * through its own block-table row, so a bad entry would read another
 * request's rows).  All pointers are HOST pointers (copies of the device
 * tables); nothing is enqueued.  Dense decode (topk_indices = topk_lens =
 * NULL): every seq_lens[b] must lie in [0, max_blocks_per_seq * page_size]
 * and the entries block_table[b][j], j < ceil(seq_lens[b] / page_size), in
 * [0, num_blocks).  Sparse decode (both lists given, seq_lens ignored):
 * topk_lens[b] in [0, topk], and every listed position e < topk_lens[b] in
 * [0, max_blocks_per_seq * page_size) with its page entry in [0, num_blocks).
 * Returns MLA_OK, MLA_ERR_TABLE with *bad_index (if not NULL) = the flat
 * index of the first offending element (into seq_lens / topk_lens for a
 * length, into block_table for a page, into topk_indices for a position),
 * or the shape / NULL / argument errors of the decode calls.  Multi-token
 * decode uses the same tables as dense decode. */
mla_status mla_check_inputs(const mla_shape* shape, const int32_t* block_table,
                            const int32_t* seq_lens, int32_t topk, const int32_t* topk_indices,
                            const int32_t* topk_lens, int64_t* bad_index);

/* Merge the results of a context-parallel decode ("Triton と MLA" page,
 * 設計動機: decode always returns lse because the context shards are merged
 * through it; "AttentionBackend" page, Limites et échecs: an lse taken in the
 * wrong base silently corrupts the merge, so the base is stated here).
 *
 * Each of num_shards shards has decoded the same rows (a row = one sequence
 * and query head, or one query token and head) over its own share of the
 * keys, e.g. the pages j % num_shards == shard of every sequence, each with
 * this library.  Per row:
 *   lse = ln sum_g e^lse_g,   o = sum_g e^(lse_g - lse) o_g;
 * a shard with lse_g = -inf (it held no key of the row) has weight 0 whatever
 * its o_g holds; a row with no live shard gets o = 0 and lse = -inf.
 *   o_parts    device, [num_shards][rows][d_v], parts_dtype MLA_BF16 or
 *              MLA_FP32, 16-byte aligned
 *   lse_parts  device, [num_shards][rows] float32, natural log
 *              (lse_base MLA_LSE_LN) or base 2 (MLA_LSE_LOG2)
 *   o          device, [rows][d_v], o_dtype MLA_BF16 or MLA_FP32, 16-byte
 *              aligned; lse device [rows] float32, natural log
 *   d_v        512 or 256 (kv_lora_rank); 1 <= rows <= MLA_MAX_MERGE_ROWS;
 *              1 <= num_shards <= MLA_MAX_SHARDS
 * Buffers are caller-owned and may not overlap the outputs; one kernel is
 * enqueued on hip_stream; nothing is allocated.  Errors (nothing enqueued):
 * MLA_ERR_NULL, MLA_ERR_ARGUMENT (shard count, base or alignment),
 * MLA_ERR_SHAPE (rows), MLA_ERR_HEAD_SIZE (d_v), MLA_ERR_DTYPE. */
typedef enum mla_lse_base { MLA_LSE_LN = 0, MLA_LSE_LOG2 = 1 } mla_lse_base;
#define MLA_MAX_SHARDS 65536
#define MLA_MAX_MERGE_ROWS ((int64_t)1 << 32)
mla_status mla_merge_shards(int32_t num_shards, int64_t rows, int32_t d_v, const void* o_parts,
                            int32_t parts_dtype, const float* lse_parts, int32_t lse_base,
                            void* o, int32_t o_dtype, float* lse, void* hip_stream);

/* Measurement aid: the next launch of stage `stage` (1: the attention pass
 * with its partials, 2: the merge) made by the calling thread, by any decode
 * entry point, records the kernel's own start into start_event and its end
 * into stop_event (hipEvent_t values created by the caller with timing
 * enabled; either may be NULL).  The setting then clears; a call that does
 * not launch that stage leaves it pending.  Unlike events recorded on the
 * stream between launches, these bracket the kernel alone.  Pure host;
 * MLA_ERR_ARGUMENT for another stage number. */
mla_status mla_time_next_launch(int32_t stage, void* start_event, void* stop_event);

/* A static, human-readable name for a status code (never NULL). */
const char* mla_status_string(int32_t status);

#ifdef __cplusplus
}
#endif

#endif /* MLA_H_ */
