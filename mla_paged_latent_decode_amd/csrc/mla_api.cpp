// Host side of libmla: argument checks, the split planner, workspace sizing
// and the C ABI of include/mla.h.  Everything here is plain host C++; the only
// GPU work is enqueued by mla::launch_decode (mla_kernels.hip).
#include <math.h>
#include <stdint.h>
#include <string.h>

#include "mla.h"
#include "mla_internal.h"

namespace mla {

static int64_t align_up(int64_t x, int64_t a) { return (x + a - 1) / a * a; }

WorkspaceLayout workspace_layout(int32_t batch, int32_t heads, int32_t d_v, int32_t split_mode,
                                 int32_t num_splits) {
  WorkspaceLayout w;
  if (batch < 1 || heads < 1 || d_v < 1 || num_splits < 1) return w;
  if (split_mode == MLA_SPLIT_PER_SEQUENCE) {
    if (num_splits == 1) return w;  // one segment per sequence: written directly
    w.slots = (int64_t)batch * num_splits;
  } else if (split_mode == MLA_SPLIT_BALANCED) {
    // slot of (unit u, sequence b) is u + b: both grow along the tile stream,
    // so u + b is distinct for every segment, and below U + B.
    w.slots = (int64_t)num_splits + batch;
  } else {
    return w;
  }
  const int64_t o_bytes = w.slots * heads * (int64_t)d_v * 2;
  const int64_t lse_off = align_up(o_bytes, 256);
  const int64_t seg_off = lse_off + align_up(w.slots * heads * 8, 256);
  const int64_t total = seg_off + align_up((int64_t)batch * 8, 256);
  w.o_bytes = (size_t)o_bytes;
  w.lse_offset = (size_t)lse_off;
  w.seg_offset = (size_t)seg_off;
  w.total = (size_t)total;
  return w;
}

thread_local LaunchTiming g_launch_timing[2];

HeadTiling head_tiling(int32_t heads) {
  HeadTiling t;
  t.heads_per_wave = heads % 32 == 0 ? 32 : 16;
  const int groups = heads / t.heads_per_wave;
  t.waves = groups % 4 == 0 ? 4 : (groups % 2 == 0 ? 2 : 1);
  t.head_chunks = groups / t.waves;
  return t;
}

// Per-token cache kind of a dtype: 0 none, 1 e4m3fn, 2 int8, 3 int4 codes.
static int per_token_kind(int32_t kv_dtype) {
  return kv_dtype == MLA_FP8_E4M3_PER_TOKEN ? 1
         : kv_dtype == MLA_INT8_PER_TOKEN   ? 2
         : kv_dtype == MLA_INT4_PER_TOKEN   ? 3
                                            : 0;
}

// Bytes of one cache row (one token).
static uint64_t kv_row_bytes(const mla_shape& s) {
  const int pt = per_token_kind(s.kv_dtype);
  if (pt) return (uint64_t)(pt == 3 ? s.head_size / 2 : s.head_size) + MLA_PER_TOKEN_PAD;
  return (uint64_t)s.head_size * (s.kv_dtype == MLA_BF16 ? 2 : 1);
}

// LDS bytes of one stage-1 workgroup (the same plan the kernel dispatch uses).
static int64_t stage1_lds(const mla_shape& s) {
  const HeadTiling t = head_tiling(s.num_heads);
  return stage1_lds_bytes(t.heads_per_wave, t.waves, s.head_size, s.kv_dtype != MLA_BF16,
                          per_token_kind(s.kv_dtype));
}

}  // namespace mla

using namespace mla;

static mla_status check_shape(const mla_shape* s) {
  if (!s) return MLA_ERR_NULL;
  if (!((s->head_size == 576 && s->kv_lora_rank == 512) ||
        (s->head_size == 320 && s->kv_lora_rank == 256)))
    return MLA_ERR_HEAD_SIZE;
  if (s->page_size <= 0 || s->page_size % 16 != 0) return MLA_ERR_PAGE_SIZE;
  if (s->q_dtype != MLA_BF16) return MLA_ERR_DTYPE;
  if (s->kv_dtype != MLA_BF16 && s->kv_dtype != MLA_FP8_E4M3 && !per_token_kind(s->kv_dtype))
    return MLA_ERR_DTYPE;
  if (s->o_dtype != MLA_BF16 && s->o_dtype != MLA_FP32) return MLA_ERR_DTYPE;
  if (s->batch < 1 || s->batch > MLA_MAX_BATCH || s->num_heads < 16 || s->num_heads % 16 != 0 ||
      s->num_heads > MLA_MAX_ROWS || s->num_blocks < 1 || s->max_blocks_per_seq < 1)
    return MLA_ERR_SHAPE;
  // byte counts of the biggest buffers must fit comfortably in 64 bits
  const double kv_bytes = (double)s->num_blocks * s->page_size * s->head_size * 2.0;
  const double q_bytes = (double)s->batch * s->num_heads * s->head_size * 2.0;
  const double bt = (double)s->batch * s->max_blocks_per_seq;
  if (kv_bytes > 4.0e18 || q_bytes > 4.0e18 || bt > 2.0e9) return MLA_ERR_SHAPE;
  return MLA_OK;
}

static bool aligned(const void* p, uintptr_t a) { return ((uintptr_t)p % a) == 0; }

// The row shape of a multi-token decode: q_len query tokens x H heads are the
// kernels' rows (row = token * H + head), so q [B, q_len, H, D] is q [B, rows, D].
static bool row_shape(const mla_shape* s, int32_t q_len, mla_shape* out) {
  if (!s || q_len < 1 || q_len > MLA_MAX_Q_LEN) return false;
  const int64_t rows = (int64_t)s->num_heads * q_len;
  if (rows > MLA_MAX_ROWS) return false;
  *out = *s;
  out->num_heads = (int32_t)rows;
  return true;
}

extern "C" {

int32_t mla_pages_split_count(int32_t max_seq_len, int32_t num_cus) {
  if (num_cus < 1) return 0;
  int64_t s = ((int64_t)max_seq_len + 511) / 512;
  if (s < 1) s = 1;
  if (s > 2 * (int64_t)num_cus) s = 2 * (int64_t)num_cus;
  return (int32_t)s;
}

size_t mla_workspace_size_mtp(const mla_shape* shape, int32_t q_len, int32_t split_mode,
                              int32_t num_kv_splits) {
  mla_shape rs;
  if (!row_shape(shape, q_len, &rs)) return 0;
  shape = &rs;
  if (check_shape(shape) != MLA_OK) return 0;
  if (num_kv_splits < 1 || num_kv_splits > MLA_MAX_KV_SPLITS) return 0;
  return workspace_layout(shape->batch, shape->num_heads, shape->kv_lora_rank, split_mode,
                          num_kv_splits)
      .total;
}

size_t mla_workspace_size(const mla_shape* shape, int32_t split_mode, int32_t num_kv_splits) {
  return mla_workspace_size_mtp(shape, 1, split_mode, num_kv_splits);
}

mla_status mla_plan_mtp(const mla_shape* shape, int32_t q_len, int32_t max_seq_len,
                        int64_t total_seq_len, int32_t num_cus, int32_t deterministic,
                        int32_t* split_mode, int32_t* num_kv_splits, size_t* workspace_bytes) {
  mla_status st = check_shape(shape);
  if (st != MLA_OK) return st;
  mla_shape rs;
  if (!row_shape(shape, q_len, &rs)) return MLA_ERR_ARGUMENT;
  shape = &rs;
  st = check_shape(shape);
  if (st != MLA_OK) return st;
  if (!split_mode || !num_kv_splits || !workspace_bytes) return MLA_ERR_NULL;
  if (num_cus < 1 || max_seq_len < 0) return MLA_ERR_ARGUMENT;
  if (deterministic) {
    *split_mode = MLA_SPLIT_PER_SEQUENCE;
    *num_kv_splits = 1;
    *workspace_bytes = 0;
    return MLA_OK;
  }
  const HeadTiling ht = head_tiling(shape->num_heads);
  int64_t per_cu = kLdsBytes / stage1_lds(*shape);
  if (per_cu < 1) per_cu = 1;
  if (per_cu > 4) per_cu = 4;
  // one workgroup per resident slot, each head chunk counting as its own
  int64_t units = num_cus * per_cu / ht.head_chunks;
  if (units < 1) units = 1;
  // keep at least 4 tiles (128 positions) per unit
  int64_t total = total_seq_len > 0 ? total_seq_len : (int64_t)shape->batch * max_seq_len;
  const int64_t tiles = total / kTile + shape->batch;
  const int64_t cap = (tiles + 3) / 4;
  if (units > cap) units = cap;
  if (units < 1) units = 1;
  if (units > MLA_MAX_KV_SPLITS) units = MLA_MAX_KV_SPLITS;
  *split_mode = MLA_SPLIT_BALANCED;
  *num_kv_splits = (int32_t)units;
  *workspace_bytes = mla_workspace_size(shape, MLA_SPLIT_BALANCED, (int32_t)units);
  return MLA_OK;
}

mla_status mla_plan(const mla_shape* shape, int32_t max_seq_len, int64_t total_seq_len,
                    int32_t num_cus, int32_t deterministic, int32_t* split_mode,
                    int32_t* num_kv_splits, size_t* workspace_bytes) {
  return mla_plan_mtp(shape, 1, max_seq_len, total_seq_len, num_cus, deterministic, split_mode,
                      num_kv_splits, workspace_bytes);
}

// The query of a call as two parts with strides (see mla_query in mla.h);
// a contiguous q [B, rows, D] is q_nope = q, q_pe = q + D_v, row stride D.
static mla_query contiguous_query(const mla_shape* s, int32_t q_len, const void* q) {
  mla_query x;
  memset(&x, 0, sizeof(x));
  if (!s || !q) return x;  // decode_stages reports the missing shape or query
  const int64_t rows = (int64_t)s->num_heads * q_len;
  x.q_nope = q;
  x.q_pe = reinterpret_cast<const uint16_t*>(q) + s->kv_lora_rank;
  x.nope_seq_stride = x.pe_seq_stride = rows * s->head_size;
  x.nope_row_stride = x.pe_row_stride = s->head_size;
  return x;
}

static bool query_ok(const mla_query* q) {
  // every 8-element (16-byte) chunk a lane loads must be aligned
  const int64_t st[4] = {q->nope_seq_stride, q->nope_row_stride, q->pe_seq_stride,
                         q->pe_row_stride};
  for (int64_t v : st)
    if (v < 0 || v % 8 != 0 || v > ((int64_t)1 << 40)) return false;
  return aligned(q->q_nope, 16) && aligned(q->q_pe, 16);
}

static mla_status decode_stages(const mla_shape* shape, int32_t q_len, const mla_query* qd,
                                const void* kv_cache,
                                const int32_t* block_table, const int32_t* seq_lens,
                                float scale, int32_t page_size, float k_scale,
                                int32_t num_kv_splits, int32_t split_mode, void* o, float* lse,
                                void* workspace, size_t workspace_bytes, void* hip_stream,
                                int stages, const int32_t* topk_idx = nullptr,
                                int32_t topk = 0, bool builtin_scratch = false) {
  mla_status st = check_shape(shape);
  if (st != MLA_OK) return st;
  mla_shape rs;
  if (!row_shape(shape, q_len, &rs)) return MLA_ERR_ARGUMENT;
  shape = &rs;
  st = check_shape(shape);
  if (st != MLA_OK) return st;
  if (!qd || !qd->q_nope || !qd->q_pe || !kv_cache || !block_table || !seq_lens || !o || !lse)
    return MLA_ERR_NULL;
  if (page_size != shape->page_size) return MLA_ERR_PAGE_SIZE;
  if (split_mode != MLA_SPLIT_PER_SEQUENCE && split_mode != MLA_SPLIT_BALANCED)
    return MLA_ERR_SPLITS;
  if (num_kv_splits < 1 || num_kv_splits > MLA_MAX_KV_SPLITS) return MLA_ERR_SPLITS;
  if (split_mode == MLA_SPLIT_PER_SEQUENCE &&
      (int64_t)shape->batch * num_kv_splits > (int64_t)1 << 27)
    return MLA_ERR_SPLITS;
  if (!(isfinite(scale) && scale > 0.f)) return MLA_ERR_ARGUMENT;
  const bool fp8 = shape->kv_dtype != MLA_BF16;
  const bool per_token = per_token_kind(shape->kv_dtype) != 0;
  if (fp8 && !per_token && !(isfinite(k_scale) && k_scale > 0.f)) return MLA_ERR_ARGUMENT;
  if (!query_ok(qd) || !aligned(kv_cache, 16) || !aligned(o, 16) || !aligned(lse, 4) ||
      !aligned(block_table, 4) || !aligned(seq_lens, 4))
    return MLA_ERR_ARGUMENT;
  const WorkspaceLayout wl = workspace_layout(shape->batch, shape->num_heads,
                                              shape->kv_lora_rank, split_mode, num_kv_splits);
  if (builtin_scratch && wl.total > 0) {
    // the built-in scratch of this device instead of a caller's workspace
    if (wl.total > kNoAllocScratchBytes) return MLA_ERR_SCRATCH;
    if (noalloc_scratch(&workspace) != 0) return MLA_ERR_LAUNCH;
    workspace_bytes = kNoAllocScratchBytes;
  }
  if (wl.total > 0) {
    if (!workspace || workspace_bytes < wl.total) return MLA_ERR_WORKSPACE;
    if (!aligned(workspace, 256)) return MLA_ERR_ARGUMENT;
  }

  DecodeArgs a;
  a.q_nope = qd->q_nope;
  a.q_pe = qd->q_pe;
  a.qn_seq = qd->nope_seq_stride;
  a.qn_row = qd->nope_row_stride;
  a.qp_seq = qd->pe_seq_stride;
  a.qp_row = qd->pe_row_stride;
  a.kv = kv_cache;
  a.block_table = block_table;
  a.seq_lens = seq_lens;
  a.o = o;
  a.lse = lse;
  a.ws_o = wl.total ? workspace : nullptr;
  a.ws_ls = wl.total ? reinterpret_cast<char*>(workspace) + wl.lse_offset : nullptr;
  a.ws_seg = wl.total ? reinterpret_cast<char*>(workspace) + wl.seg_offset : nullptr;
  a.batch = shape->batch;
  a.heads = shape->num_heads;  // rows: q_len tokens x heads
  a.q_len = q_len;
  a.head_size = shape->head_size;
  a.d_v = shape->kv_lora_rank;
  a.page_size = shape->page_size;
  a.bt_stride = shape->max_blocks_per_seq;
  a.kv_fp8 = fp8 ? 1 : 0;
  a.kv_pt = per_token_kind(shape->kv_dtype);
  a.o_f32 = shape->o_dtype == MLA_FP32 ? 1 : 0;
  a.split_mode = split_mode;
  a.num_splits = num_kv_splits;
  a.scale = scale;
  a.k_scale = k_scale;
  a.pool_bytes = (uint64_t)shape->num_blocks * shape->page_size * kv_row_bytes(*shape);
  a.num_blocks = shape->num_blocks;
  if (topk_idx) {
    a.topk_idx = topk_idx;
    a.topk_stride = topk;
  }
  const int rc = launch_decode(a, hip_stream, stages);
  return rc == 0 ? MLA_OK : rc == kGridTooLarge ? MLA_ERR_SHAPE : MLA_ERR_LAUNCH;
}

mla_status mla_decode(const mla_shape* shape, const void* q, const void* kv_cache,
                      const int32_t* block_table, const int32_t* seq_lens, float scale,
                      int32_t page_size, float k_scale, int32_t num_kv_splits,
                      int32_t split_mode, void* o, float* lse, void* workspace,
                      size_t workspace_bytes, void* hip_stream) {
  const mla_query qd = contiguous_query(shape, 1, q);
  return decode_stages(shape, 1, &qd, kv_cache, block_table, seq_lens, scale, page_size, k_scale,
                       num_kv_splits, split_mode, o, lse, workspace, workspace_bytes, hip_stream,
                       kBothStages);
}

mla_status mla_decode_mtp(const mla_shape* shape, int32_t q_len, const void* q,
                      const void* kv_cache, const int32_t* block_table, const int32_t* seq_lens,
                      float scale, int32_t page_size, float k_scale, int32_t num_kv_splits,
                      int32_t split_mode, void* o, float* lse, void* workspace,
                      size_t workspace_bytes, void* hip_stream) {
  const mla_query qd = contiguous_query(shape, q_len, q);
  return decode_stages(shape, q_len, &qd, kv_cache, block_table, seq_lens, scale, page_size, k_scale,
                       num_kv_splits, split_mode, o, lse, workspace, workspace_bytes, hip_stream,
                       kBothStages);
}

mla_status mla_decode_split_q(const mla_shape* shape, int32_t q_len, const mla_query* q,
                              const void* kv_cache, const int32_t* block_table,
                              const int32_t* seq_lens, float scale, int32_t page_size,
                              float k_scale, int32_t num_kv_splits, int32_t split_mode, void* o,
                              float* lse, void* workspace, size_t workspace_bytes,
                              void* hip_stream) {
  return decode_stages(shape, q_len, q, kv_cache, block_table, seq_lens, scale, page_size,
                       k_scale, num_kv_splits, split_mode, o, lse, workspace, workspace_bytes,
                       hip_stream, kBothStages);
}

mla_status mla_decode_noalloc(const mla_shape* shape, int32_t q_len, const void* q,
                              const void* kv_cache, const int32_t* block_table,
                              const int32_t* seq_lens, float scale, int32_t page_size,
                              float k_scale, int32_t num_kv_splits, int32_t split_mode, void* o,
                              float* lse, void* hip_stream) {
  const mla_query qd = contiguous_query(shape, q_len, q);
  return decode_stages(shape, q_len, &qd, kv_cache, block_table, seq_lens, scale, page_size,
                       k_scale, num_kv_splits, split_mode, o, lse, nullptr, 0, hip_stream,
                       kBothStages, nullptr, 0, true);
}

size_t mla_noalloc_scratch_bytes(void) { return kNoAllocScratchBytes; }

mla_status mla_time_next_launch(int32_t stage, void* start_event, void* stop_event) {
  if (stage != 1 && stage != 2) return MLA_ERR_ARGUMENT;
  g_launch_timing[stage - 1] = LaunchTiming{start_event, stop_event};
  return MLA_OK;
}

mla_status mla_decode_stage1(const mla_shape* shape, const void* q, const void* kv_cache,
                             const int32_t* block_table, const int32_t* seq_lens, float scale,
                             int32_t page_size, float k_scale, int32_t num_kv_splits,
                             int32_t split_mode, void* o, float* lse, void* workspace,
                             size_t workspace_bytes, void* hip_stream) {
  const mla_query qd = contiguous_query(shape, 1, q);
  return decode_stages(shape, 1, &qd, kv_cache, block_table, seq_lens, scale, page_size, k_scale,
                       num_kv_splits, split_mode, o, lse, workspace, workspace_bytes, hip_stream,
                       kStage1);
}

mla_status mla_decode_mtp_stage1(const mla_shape* shape, int32_t q_len, const void* q,
                      const void* kv_cache, const int32_t* block_table, const int32_t* seq_lens,
                      float scale, int32_t page_size, float k_scale, int32_t num_kv_splits,
                      int32_t split_mode, void* o, float* lse, void* workspace,
                      size_t workspace_bytes, void* hip_stream) {
  const mla_query qd = contiguous_query(shape, q_len, q);
  return decode_stages(shape, q_len, &qd, kv_cache, block_table, seq_lens, scale, page_size, k_scale,
                       num_kv_splits, split_mode, o, lse, workspace, workspace_bytes, hip_stream,
                       kStage1);
}

mla_status mla_decode_stage2(const mla_shape* shape, const void* q, const void* kv_cache,
                             const int32_t* block_table, const int32_t* seq_lens, float scale,
                             int32_t page_size, float k_scale, int32_t num_kv_splits,
                             int32_t split_mode, void* o, float* lse, void* workspace,
                             size_t workspace_bytes, void* hip_stream) {
  const mla_query qd = contiguous_query(shape, 1, q);
  return decode_stages(shape, 1, &qd, kv_cache, block_table, seq_lens, scale, page_size, k_scale,
                       num_kv_splits, split_mode, o, lse, workspace, workspace_bytes, hip_stream,
                       kStage2);
}

mla_status mla_decode_mtp_stage2(const mla_shape* shape, int32_t q_len, const void* q,
                      const void* kv_cache, const int32_t* block_table, const int32_t* seq_lens,
                      float scale, int32_t page_size, float k_scale, int32_t num_kv_splits,
                      int32_t split_mode, void* o, float* lse, void* workspace,
                      size_t workspace_bytes, void* hip_stream) {
  const mla_query qd = contiguous_query(shape, q_len, q);
  return decode_stages(shape, q_len, &qd, kv_cache, block_table, seq_lens, scale, page_size, k_scale,
                       num_kv_splits, split_mode, o, lse, workspace, workspace_bytes, hip_stream,
                       kStage2);
}

// Sparse (top-k) decode: checks of the configurations its gather is built for.
static mla_status check_sparse(const mla_shape* shape, int32_t topk, const int32_t* topk_indices,
                               const int32_t* topk_lens) {
  mla_status st = check_shape(shape);
  if (st != MLA_OK) return st;
  if (!topk_indices || !topk_lens) return MLA_ERR_NULL;
  if (topk < 1) return MLA_ERR_ARGUMENT;
  const uint64_t pool = (uint64_t)shape->num_blocks * shape->page_size * kv_row_bytes(*shape);
  if (pool + 65536 >= ((uint64_t)1 << 32)) return MLA_ERR_SHAPE;
  if (!aligned(topk_indices, 4)) return MLA_ERR_ARGUMENT;
  return MLA_OK;
}

#define MLA_SPARSE_ENTRY(NAME, STAGES)                                                          \
  mla_status NAME(const mla_shape* shape, int32_t topk, const void* q, const void* kv_cache,    \
                  const int32_t* block_table, const int32_t* topk_indices,                      \
                  const int32_t* topk_lens, float scale, int32_t page_size, float k_scale,      \
                  int32_t num_kv_splits, int32_t split_mode, void* o, float* lse,               \
                  void* workspace, size_t workspace_bytes, void* hip_stream) {                  \
    const mla_status st = check_sparse(shape, topk, topk_indices, topk_lens);                   \
    if (st != MLA_OK) return st;                                                                \
    const mla_query qd = contiguous_query(shape, 1, q);                                         \
    return decode_stages(shape, 1, &qd, kv_cache, block_table, topk_lens, scale, page_size,     \
                         k_scale, num_kv_splits, split_mode, o, lse, workspace,                 \
                         workspace_bytes, hip_stream, STAGES, topk_indices, topk);              \
  }
MLA_SPARSE_ENTRY(mla_decode_sparse, kBothStages)
MLA_SPARSE_ENTRY(mla_decode_sparse_stage1, kStage1)
MLA_SPARSE_ENTRY(mla_decode_sparse_stage2, kStage2)
#undef MLA_SPARSE_ENTRY

mla_status mla_check_inputs(const mla_shape* shape, const int32_t* block_table,
                            const int32_t* seq_lens, int32_t topk, const int32_t* topk_indices,
                            const int32_t* topk_lens, int64_t* bad_index) {
  if (bad_index) *bad_index = -1;
  const mla_status st = check_shape(shape);
  if (st != MLA_OK) return st;
  if (!block_table) return MLA_ERR_NULL;
  const bool sparse = topk_indices != nullptr || topk_lens != nullptr;
  if (sparse && (!topk_indices || !topk_lens)) return MLA_ERR_NULL;
  if (!sparse && !seq_lens) return MLA_ERR_NULL;
  if (sparse && topk < 1) return MLA_ERR_ARGUMENT;
  const int64_t W = shape->max_blocks_per_seq, P = shape->page_size;
  const int64_t cap = W * P;  // positions one table row can address
  auto bad = [&](int64_t i) {
    if (bad_index) *bad_index = i;
    return MLA_ERR_TABLE;
  };
  auto page_ok = [&](int64_t b, int64_t j) {
    const int32_t pg = block_table[b * W + j];
    return pg >= 0 && pg < shape->num_blocks;
  };
  for (int64_t b = 0; b < shape->batch; ++b) {
    if (!sparse) {
      // every page a sequence of n positions reads: table entries 0 .. ceil(n/P) - 1
      const int64_t n = seq_lens[b];
      if (n < 0 || n > cap) return bad(b);
      for (int64_t j = 0; j < (n + P - 1) / P; ++j)
        if (!page_ok(b, j)) return bad(b * W + j);
    } else {
      // every listed position, and the page it goes through
      const int64_t k = topk_lens[b];
      if (k < 0 || k > topk) return bad(b);
      for (int64_t e = 0; e < k; ++e) {
        const int64_t pos = topk_indices[b * topk + e];
        if (pos < 0 || pos >= cap || !page_ok(b, pos / P)) return bad(b * topk + e);
      }
    }
  }
  return MLA_OK;
}

mla_status mla_merge_shards(int32_t num_shards, int64_t rows, int32_t d_v, const void* o_parts,
                            int32_t parts_dtype, const float* lse_parts, int32_t lse_base,
                            void* o, int32_t o_dtype, float* lse, void* hip_stream) {
  if (!o_parts || !lse_parts || !o || !lse) return MLA_ERR_NULL;
  if (num_shards < 1 || num_shards > MLA_MAX_SHARDS) return MLA_ERR_ARGUMENT;
  if (rows < 1 || rows > MLA_MAX_MERGE_ROWS) return MLA_ERR_SHAPE;
  if (d_v != 512 && d_v != 256) return MLA_ERR_HEAD_SIZE;
  if ((parts_dtype != MLA_BF16 && parts_dtype != MLA_FP32) ||
      (o_dtype != MLA_BF16 && o_dtype != MLA_FP32))
    return MLA_ERR_DTYPE;
  if (lse_base != MLA_LSE_LN && lse_base != MLA_LSE_LOG2) return MLA_ERR_ARGUMENT;
  if (!aligned(o_parts, 16) || !aligned(o, 16) || !aligned(lse_parts, 4) || !aligned(lse, 4))
    return MLA_ERR_ARGUMENT;
  MergeArgs a;
  a.o_parts = o_parts;
  a.lse_parts = lse_parts;
  a.o = o;
  a.lse = lse;
  a.rows = rows;
  a.shards = num_shards;
  a.d_v = d_v;
  a.parts_f32 = parts_dtype == MLA_FP32 ? 1 : 0;
  a.o_f32 = o_dtype == MLA_FP32 ? 1 : 0;
  a.lse_log2 = lse_base == MLA_LSE_LOG2 ? 1 : 0;
  return launch_merge_shards(a, hip_stream) == 0 ? MLA_OK : MLA_ERR_LAUNCH;
}

const char* mla_status_string(int32_t status) {
  switch (status) {
    case MLA_OK: return "MLA_OK";
    case MLA_ERR_NULL: return "MLA_ERR_NULL: a required pointer is NULL";
    case MLA_ERR_HEAD_SIZE: return "MLA_ERR_HEAD_SIZE: head_size must be 576 or 320 with kv_lora_rank = head_size - 64";
    case MLA_ERR_PAGE_SIZE: return "MLA_ERR_PAGE_SIZE: page_size must be a positive multiple of 16 and match the shape";
    case MLA_ERR_DTYPE: return "MLA_ERR_DTYPE: q must be bf16, kv bf16, fp8 e4m3fn (per-tensor or per-token scale) or per-token int8 / int4, o bf16 or fp32";
    case MLA_ERR_SHAPE: return "MLA_ERR_SHAPE: batch, heads (multiple of 16), num_blocks or table width out of range";
    case MLA_ERR_SPLITS: return "MLA_ERR_SPLITS: num_kv_splits or split_mode out of range";
    case MLA_ERR_WORKSPACE: return "MLA_ERR_WORKSPACE: workspace missing or too small";
    case MLA_ERR_LAUNCH: return "MLA_ERR_LAUNCH: HIP kernel launch failed";
    case MLA_ERR_ARGUMENT: return "MLA_ERR_ARGUMENT: non-finite/non-positive scale or k_scale, num_cus < 1, q_len outside [1, MLA_MAX_Q_LEN], topk < 1, or a misaligned pointer or query stride";
    case MLA_ERR_TABLE: return "MLA_ERR_TABLE: a sequence length, block-table entry or top-k entry is out of range";
    case MLA_ERR_SCRATCH: return "MLA_ERR_SCRATCH: the split layout needs more than the built-in scratch of mla_decode_noalloc (mla_noalloc_scratch_bytes())";
    default: return "unknown mla_status";
  }
}

}  // extern "C"
