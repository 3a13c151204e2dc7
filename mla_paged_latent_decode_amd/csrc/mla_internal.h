// Internal interface between the host ABI (mla_api.cpp) and the HIP kernels
// (mla_kernels.hip).  Not installed; the public surface is include/mla.h.
#pragma once

#include <stddef.h>
#include <stdint.h>

namespace mla {

constexpr int kTile = 32;  // context positions per stage-1 tile

// Workspace layout (both split modes): `slots` partial results, each
//   ws_o  [slots][H][D_v]  fp16, the segment's normalised output o_s stored
//                          as o_s * 2^-e (e per row, see ws_ls)
//   ws_ls [slots][H][2]    float32 {lse_s (natural log), 2^e}
//   ws_seg [B][2]          int32 {first slot, partial count} of each sequence
//                          (balanced mode; written by stage 1 for stage 2)
// ws_ls and ws_seg each start at the next 256-byte boundary.
struct WorkspaceLayout {
  int64_t slots = 0;
  size_t o_bytes = 0;
  size_t lse_offset = 0;
  size_t seg_offset = 0;
  size_t total = 0;
};

WorkspaceLayout workspace_layout(int32_t batch, int32_t heads, int32_t d_v, int32_t split_mode,
                                 int32_t num_splits);

// How the heads of one sequence are spread over waves and workgroups.
struct HeadTiling {
  int heads_per_wave;   // 32 (32x32 MFMA tiles) or 16 (16x16 tiles)
  int waves;            // waves per workgroup, each owning heads_per_wave heads
  int head_chunks;      // workgroups per work unit along the head axis
};

HeadTiling head_tiling(int32_t heads);

// LDS plan of one stage-1 workgroup, shared by the planner (mla_api.cpp) and
// the kernel dispatch (mla_kernels.hip).  A bf16 cache streams straight into
// a ring of `ring_depth` bf16 tiles (32 positions x D).  An fp8 cache streams
// into two fp8 staging tiles and is widened to bf16 into a ring of 3 (32-head
// waves, 4 waves: software-pipelined loop) or 2 tiles.  With 32 heads per
// wave at D = 576 the last `qlds_steps` 16-wide k-steps of Q live in LDS
// (1 KB per step and wave), as many as the remaining LDS holds, up to 12.
constexpr int kLdsBytes = 160 * 1024;

// Per-token caches (rows of D fp8 or int8 codes + a 16-byte inline scale pad) run
// the plain fp8 loop with a ring of 2 and keep each tile's 32 scales in LDS:
// two staging slots of 2 x 256 B and a ring of 128 B slots.
constexpr int kPerTokenPad = 16;
// pt (per-token rows): 0 none, 1 e4m3fn codes, 2 int8 codes, 3 int4 codes
constexpr int stage1_code_bytes(int d, bool fp8, int pt) {
  return pt == 3 ? d / 2 : (fp8 ? d : 2 * d);
}
constexpr int stage1_ring_depth(int hpw, int waves, int d, bool fp8, int pt = 0) {
  if (pt) return 2;
  if (fp8) return (hpw == 32 && waves == 4) ? 3 : 2;
  if (d != 576) return 4;
  // 32-head waves at D = 576: three tiles, so that 12 of Q's 36 k-steps fit
  // in LDS and the score accumulators stay in VGPRs beside Q and O
  if (hpw == 32) return waves == 4 ? 3 : (waves == 2 ? 3 : 2);
  return waves == 4 ? 4 : 2;
}
constexpr int stage1_staging_bytes(int d, bool fp8, int pt) {
  return fp8 ? 2 * kTile * stage1_code_bytes(d, fp8, pt) : 0;
}
constexpr int stage1_scale_bytes(int hpw, int waves, int d, bool fp8, int pt) {
  // two staging slots of 2 x 256 B; per ring slot the 32 scales and their reciprocals
  return pt ? 2 * 512 + stage1_ring_depth(hpw, waves, d, fp8, pt) * 256 : 0;
}
constexpr int stage1_qlds_steps(int hpw, int waves, int d, bool fp8, int pt = 0) {
  if (!(hpw == 32 && d == 576)) return 0;
  const int room = (kLdsBytes - stage1_ring_depth(hpw, waves, d, fp8, pt) * kTile * d * 2 -
                    stage1_staging_bytes(d, fp8, pt) - stage1_scale_bytes(hpw, waves, d, fp8, pt)) /
                   (waves * 1024);
  return room < 12 ? room : 12;
}
constexpr int stage1_lds_bytes(int hpw, int waves, int d, bool fp8, int pt = 0) {
  return stage1_ring_depth(hpw, waves, d, fp8, pt) * kTile * d * 2 +
         stage1_staging_bytes(d, fp8, pt) +
         stage1_qlds_steps(hpw, waves, d, fp8, pt) * waves * 1024 +
         stage1_scale_bytes(hpw, waves, d, fp8, pt);
}

struct DecodeArgs {
  // query rows [q_nope | q_pe] of sequence b, row r (query token x heads +
  // head): q_nope + b * qn_seq + r * qn_row and q_pe + b * qp_seq + r * qp_row
  // (bf16 elements)
  const void* q_nope;
  const void* q_pe;
  int64_t qn_seq, qn_row, qp_seq, qp_row;
  const void* kv;
  const int32_t* block_table;
  const int32_t* seq_lens;
  void* o;
  float* lse;
  void* ws_o;
  void* ws_ls;
  void* ws_seg;
  int32_t batch;
  int32_t heads;  // rows: q_len query tokens x heads per token
  int32_t q_len;  // query tokens per sequence (1: plain decode)
  int32_t head_size;
  int32_t d_v;
  int32_t page_size;
  int32_t bt_stride;
  int32_t kv_fp8;
  int32_t kv_pt;  // per-token rows (codes + an inline fp32 scale): 1 e4m3fn, 2 int8, 3 int4
  int32_t o_f32;
  int32_t split_mode;
  int32_t num_splits;
  float scale;
  float k_scale;
  // sparse decode: top-k list [batch][topk_stride] of logical positions
  // (NULL for dense decode; seq_lens then holds the list lengths)
  const int32_t* topk_idx = nullptr;
  int32_t topk_stride = 0;
  uint64_t pool_bytes = 0;  // num_blocks * page_size * head_size * kv bytes
  int32_t num_blocks = 0;   // pages in the pool (page numbers outside read as zero rows)
};

enum Stages { kStage1 = 1, kStage2 = 2, kBothStages = 3 };

// Measurement aid (mla_time_next_launch): events (hipEvent_t) that the next
// launch of stage 1 / stage 2 made by this thread records its own start and
// end into; taken (and cleared) by that launch.  Null: a plain launch.
struct LaunchTiming {
  void* start = nullptr;
  void* stop = nullptr;
};
extern thread_local LaunchTiming g_launch_timing[2];

// Enqueues stage 1 and/or stage 2 (stage 2 only when the split layout needs
// a merge).  Returns 0 or a HIP error code.
// Enqueues the stages of a decode; 0, a HIP error code, or kGridTooLarge (nothing
// enqueued) when a launch grid would exceed what HIP accepts (kMaxGrid workgroups).
constexpr int kGridTooLarge = -1;
constexpr int64_t kMaxGrid = 0x7fffffff;
int launch_decode(const DecodeArgs& a, void* stream, int stages);

// Cross-shard merge (mla_merge.hip).
struct MergeArgs {
  const void* o_parts;     // [shards][rows][d_v]
  const float* lse_parts;  // [shards][rows]
  void* o;                 // [rows][d_v]
  float* lse;              // [rows]
  int64_t rows;
  int32_t shards, d_v;
  int32_t parts_f32, o_f32, lse_log2;
};

int launch_merge_shards(const MergeArgs& a, void* stream);

// Scratch of the allocation-free entry point (mla_noalloc.hip): a device
// array of kNoAllocScratchBytes per device; noalloc_scratch() returns the
// current device's copy (looked up once per device).  Returns 0 or a HIP
// error code.
constexpr size_t kNoAllocScratchBytes = (size_t)64 << 20;
int noalloc_scratch(void** ptr);

}  // namespace mla
