// Cross-shard merge of decode results (decode context parallelism).
//
// Each of G context shards has run the decode over its own share of every
// sequence's keys and returned, per (sequence, head) row, its normalised
// output o_g and its log-sum-exp lse_g.  The shards are combined through
// their LSE ("Triton と MLA" page, 設計動機: decode always returns lse
// because the shards of a context-parallel decode are merged with it; the
// same page and the "AttentionBackend" page, Limites et échecs: an lse read
// in the wrong base silently corrupts the merged denominator, so the base is
// an argument here):
//   lse = ln sum_g e^lse_g,   o = sum_g e^(lse_g - lse) o_g,
// a shard with lse_g = -inf (no keys) has weight 0 whatever its o_g holds,
// and a row that no shard saw gets o = 0, lse = -inf.
//
// On one GPU this is the whole of the merge; across GPUs the o_g and lse_g
// would first be gathered (or the rows exchanged all-to-all) over xGMI.
//
// The kernel is HBM-bound: every shard row is read once, the merged row
// written once.  One wave per row, D_v / 64 consecutive columns per lane,
// eight shards' rows in flight per lane.

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "mla_internal.h"

namespace mla {
namespace {

typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));

constexpr int kMergeBatch = 8;   // shard rows loaded before any is used
constexpr int kRowsPerBlock = 4; // one wave per row

struct MergeParams {
  const void* o_parts;  // [G][rows][DV], bf16 or fp32
  const float* lse_parts;  // [G][rows]
  void* o;              // [rows][DV], bf16 or fp32
  float* lse;           // [rows], natural log
  int64_t rows;
  int32_t shards;
  int32_t parts_f32, o_f32;
  float lse_to_ln;      // 1, or ln 2 for base-2 inputs
};

// C consecutive values of one shard row (C = 4 or 8) as fp32.
template <int C>
struct Chunk {
  f32x4 v[C / 4];
};

template <int C>
__device__ __forceinline__ Chunk<C> load_chunk(const void* base, int f32, size_t idx) {
  Chunk<C> c;
  if (f32) {
    const f32x4* s = reinterpret_cast<const f32x4*>(reinterpret_cast<const float*>(base) + idx);
#pragma unroll
    for (int k = 0; k < C / 4; ++k) c.v[k] = s[k];
  } else {
    const bf16x4* s = reinterpret_cast<const bf16x4*>(reinterpret_cast<const __bf16*>(base) + idx);
#pragma unroll
    for (int k = 0; k < C / 4; ++k) c.v[k] = __builtin_convertvector(s[k], f32x4);
  }
  return c;
}

template <int DV>
__global__ __launch_bounds__(64 * kRowsPerBlock) void mla_merge_shards_kernel(MergeParams p) {
  constexpr int C = DV / 64;  // columns per lane
  static_assert(C == 4 || C == 8, "D_v must be 256 or 512");
  const int64_t row = (int64_t)blockIdx.x * kRowsPerBlock + (threadIdx.x >> 6);
  if (row >= p.rows) return;
  const int lane = threadIdx.x & 63;
  const size_t col = (size_t)lane * C;

  float m = -INFINITY, tot = 0.f;
  f32x4 acc[C / 4];
#pragma unroll
  for (int k = 0; k < C / 4; ++k) acc[k] = f32x4{0.f, 0.f, 0.f, 0.f};

  for (int g0 = 0; g0 < p.shards; g0 += kMergeBatch) {
    float ls[kMergeBatch];
    Chunk<C> x[kMergeBatch];
#pragma unroll
    for (int i = 0; i < kMergeBatch; ++i) {
      const int g = g0 + i;
      if (g < p.shards) {
        ls[i] = p.lse_parts[(size_t)g * p.rows + row] * p.lse_to_ln;
        x[i] = load_chunk<C>(p.o_parts, p.parts_f32, ((size_t)g * p.rows + row) * DV + col);
      } else {
        ls[i] = -INFINITY;
      }
    }
    float mb = m;
#pragma unroll
    for (int i = 0; i < kMergeBatch; ++i) mb = fmaxf(mb, ls[i]);
    if (mb == -INFINITY) continue;  // no live shard yet
    const float r = m == -INFINITY ? 0.f : __expf(m - mb);
    tot *= r;
#pragma unroll
    for (int k = 0; k < C / 4; ++k) acc[k] *= r;
#pragma unroll
    for (int i = 0; i < kMergeBatch; ++i) {
      // a shard without keys adds nothing, not even a NaN from its o row
      if (ls[i] != -INFINITY) {
        const float w = __expf(ls[i] - mb);
        tot += w;
#pragma unroll
        for (int k = 0; k < C / 4; ++k) acc[k] += w * x[i].v[k];
      }
    }
    m = mb;
  }

  const bool any = tot > 0.f;
  const float inv = any ? 1.f / tot : 0.f;
  const size_t o_idx = (size_t)row * DV + col;
#pragma unroll
  for (int k = 0; k < C / 4; ++k) {
    const f32x4 v = acc[k] * inv;
    if (p.o_f32)
      *reinterpret_cast<f32x4*>(reinterpret_cast<float*>(p.o) + o_idx + 4 * k) = v;
    else
      *reinterpret_cast<bf16x4*>(reinterpret_cast<__bf16*>(p.o) + o_idx + 4 * k) =
          __builtin_convertvector(v, bf16x4);
  }
  if (lane == 0) p.lse[row] = any ? m + __logf(tot) : -INFINITY;
}

}  // namespace

int launch_merge_shards(const MergeArgs& a, void* stream) {
  hipStream_t st = reinterpret_cast<hipStream_t>(stream);
  MergeParams p;
  p.o_parts = a.o_parts;
  p.lse_parts = a.lse_parts;
  p.o = a.o;
  p.lse = a.lse;
  p.rows = a.rows;
  p.shards = a.shards;
  p.parts_f32 = a.parts_f32;
  p.o_f32 = a.o_f32;
  p.lse_to_ln = a.lse_log2 ? 0.6931471805599453f : 1.f;
  const int64_t blocks = (a.rows + kRowsPerBlock - 1) / kRowsPerBlock;
  if (a.d_v == 512)
    hipLaunchKernelGGL(mla_merge_shards_kernel<512>, dim3((uint32_t)blocks),
                       dim3(64 * kRowsPerBlock), 0, st, p);
  else
    hipLaunchKernelGGL(mla_merge_shards_kernel<256>, dim3((uint32_t)blocks),
                       dim3(64 * kRowsPerBlock), 0, st, p);
  return (int)hipGetLastError();
}

}  // namespace mla
