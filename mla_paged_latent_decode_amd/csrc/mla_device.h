// Device helpers of the stage-1 kernels of libmla: wrappers of gfx950
// instructions, the work-unit arithmetic of the split layouts, the LDS tile
// layout and the stage-1 parameter block.  Every translation unit that
// includes it gets its own internal copies.
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

#include <type_traits>

#include "mla_internal.h"

namespace mla {
namespace {

typedef int i32x4 __attribute__((ext_vector_type(4)));

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x8 __attribute__((ext_vector_type(8)));
typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
#define LDS_AS __attribute__((address_space(3)))

constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;
// Lazy rescale: the running max used for the exponentials is only moved when
// a tile's max exceeds it by more than kTau (log2 units), so p <= 2^kTau.
// The final result does not depend on this choice; it only saves rescales.
constexpr float kTau = 8.0f;

// Compile-time loop: f(std::integral_constant<int, i>) for i = 0 .. N-1.
template <int I, int N, typename F>
__device__ __forceinline__ void static_for_impl(F&& f) {
  if constexpr (I < N) {
    f(std::integral_constant<int, I>{});
    static_for_impl<I + 1, N>(f);
  }
}
template <int N, typename F>
__device__ __forceinline__ void static_for(F&& f) {
  static_for_impl<0, N>(f);
}

template <int VM>
__device__ __forceinline__ void wait_vmcnt() {
  static_assert(VM >= 0 && VM < 64, "vmcnt is a 6-bit counter");
  // simm16: vmcnt[3:0], expcnt[6:4] (7 = no wait), lgkmcnt[11:8] (0), vmcnt[5:4] at [15:14]
  __builtin_amdgcn_s_waitcnt((VM & 15) | (7 << 4) | (0 << 8) | ((VM >> 4) << 14));
}

__device__ __forceinline__ int uniform(int x) { return __builtin_amdgcn_readfirstlane(x); }
__device__ __forceinline__ int64_t uniform64(int64_t x) {
  const uint32_t lo = (uint32_t)__builtin_amdgcn_readfirstlane((int)(uint32_t)x);
  const uint32_t hi = (uint32_t)__builtin_amdgcn_readfirstlane((int)(uint32_t)((uint64_t)x >> 32));
  return (int64_t)(((uint64_t)hi << 32) | lo);
}

// A wave-uniform value the compiler must materialise in an SGPR at this
// point: per-lane addresses built from it are then formed right before
// their use instead of being hoisted out of the loop into long-lived VGPRs.
__device__ __forceinline__ int sgpr_here(int x) {
  asm volatile("" : "+s"(x));
  return x;
}

// A read of an MFMA accumulator element (held in an AGPR) that the compiler
// cannot reuse for a later read of the same element: a pass over all of a
// wave's accumulators then does not keep VGPR copies of all of them alive
// for the pass that follows (more than the VGPR file holds: spills).
__device__ __forceinline__ float acc_read(float a) {
  float v;
  asm volatile("v_accvgpr_read_b32 %0, %1" : "=v"(v) : "a"(a));
  return v;
}

// A per-lane value the compiler cannot see through or move out of a loop:
// what is derived from it is computed after this point, on every pass.
__device__ __forceinline__ int vgpr_here(int x) {
  asm volatile("" : "+v"(x));
  return x;
}

__device__ __forceinline__ float wave_max_xor(float x, int mask) {
  return fmaxf(x, __shfl_xor(x, mask, 64));
}

// v_permlane32_swap with both operands x returns {x, partner} in some order
// in every lane (partner = lane ^ 32), so max/sum of the pair is symmetric.
__device__ __forceinline__ float max_halves(float x) {
  auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
__device__ __forceinline__ float sum_halves(float x) {
  auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}

// Transposed LDS read (ds_read_b64_tr_b16) issued from inline asm.  Issued
// through the builtin, the compiler conservatively drains every in-flight
// tile load (vmcnt(0)) before it, which would serialise the HBM->LDS ring;
// from asm it does not, and the ring's own explicit waits + barrier already
// order these reads after the tile's loads.  The result may only be used
// after lds_wait<N>() on it (asm reads are invisible to the compiler's
// lgkmcnt tracking).
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
template <int OFF>
__device__ __forceinline__ u32x2 ds_read_tr16_asm(uint32_t addr) {
  static_assert(OFF >= 0 && OFF < 65536, "ds offset field is 16 bits");
  u32x2 r;
  asm volatile("ds_read_b64_tr_b16 %0, %1 offset:%2" : "=v"(r) : "v"(addr), "i"(OFF));
  return r;
}
// Wait until at most N LDS/SMEM operations are outstanding, then hand x
// back: the dependence makes every use of x come after the wait.
template <int N>
__device__ __forceinline__ void lds_wait(u32x4& x) {
  static_assert(N >= 0 && N < 16, "lgkmcnt is a 4-bit counter");
  asm volatile("s_waitcnt lgkmcnt(%1)" : "+v"(x) : "i"(N));
}

template <int N>
__device__ __forceinline__ void lds_wait(u32x2& x) {
  static_assert(N >= 0 && N < 16, "lgkmcnt is a 4-bit counter");
  asm volatile("s_waitcnt lgkmcnt(%1)" : "+v"(x) : "i"(N));
}
template <int N>
__device__ __forceinline__ void lds_wait(uint32_t& x) {
  static_assert(N >= 0 && N < 16, "lgkmcnt is a 4-bit counter");
  asm volatile("s_waitcnt lgkmcnt(%1)" : "+v"(x) : "i"(N));
}
// Plain LDS read / write from asm, for the fp8 widening step: the compiler
// would otherwise order them after every in-flight tile load (the loads
// write LDS), and it does not count them, so every use of a read comes after
// an explicit lds_wait.  The write clobbers memory so that no compiler LDS
// access moves across it.
__device__ __forceinline__ u32x2 ds_read_b64_asm(uint32_t addr) {
  u32x2 r;
  asm volatile("ds_read_b64 %0, %1" : "=v"(r) : "v"(addr));
  return r;
}
__device__ __forceinline__ void ds_write_b128_asm(uint32_t addr, u32x4 v) {
  asm volatile("ds_write_b128 %0, %1" : : "v"(addr), "v"(v) : "memory");
}
__device__ __forceinline__ uint32_t ds_read_b32_asm(uint32_t addr) {
  uint32_t r;
  asm volatile("ds_read_b32 %0, %1" : "=v"(r) : "v"(addr));
  return r;
}
__device__ __forceinline__ void ds_write_b32_asm(uint32_t addr, uint32_t v) {
  asm volatile("ds_write_b32 %0, %1" : : "v"(addr), "v"(v) : "memory");
}
__device__ __forceinline__ u32x4 ds_read_b128_asm(uint32_t addr) {
  u32x4 r;
  asm volatile("ds_read_b128 %0, %1" : "=v"(r) : "v"(addr));
  return r;
}

// Eight OCP e4m3fn values (one per byte, lowest byte first) to eight bf16.
// Every e4m3fn value is exactly representable in bf16, so the conversion
// (scale 1) is exact.
__device__ __forceinline__ u32x4 e4m3x8_to_bf16x8(u32x2 v) {
  u32x4 r;
  r[0] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(v[0], 1.0f, false));
  r[1] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(v[0], 1.0f, true));
  r[2] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(v[1], 1.0f, false));
  r[3] = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(v[1], 1.0f, true));
  return r;
}

// Eight signed int4 codes (element 2i in the low nibble of byte i, 2i+1 in
// its high nibble) to eight bf16: every value in [-8, 7] is exact in bf16.
// (Each code is moved to the top of the word as unsigned, then shifted back
// down as signed: an arithmetic shift sign-extends it.)
__device__ __forceinline__ u32x4 i4x8_to_bf16x8(uint32_t v) {
  u32x4 r;
#pragma unroll
  for (int k = 0; k < 4; ++k) {
    const f32x2 e = {(float)((int)(v << (28 - 8 * k)) >> 28),
                     (float)((int)(v << (24 - 8 * k)) >> 28)};
    r[k] = __builtin_bit_cast(uint32_t, __builtin_convertvector(e, bf16x2));
  }
  return r;
}

// Eight signed int8 codes (one per byte, lowest byte first) to eight bf16:
// every value in [-128, 127] is exact in bf16.
__device__ __forceinline__ u32x4 i8x8_to_bf16x8(u32x2 v) {
  u32x4 r;
#pragma unroll
  for (int w = 0; w < 2; ++w) {
    const uint32_t x = v[w];
    const f32x2 lo = {(float)((int)(x << 24) >> 24), (float)((int)(x << 16) >> 24)};
    const f32x2 hi = {(float)((int)(x << 8) >> 24), (float)((int)x >> 24)};
    r[2 * w] = __builtin_bit_cast(uint32_t, __builtin_convertvector(lo, bf16x2));
    r[2 * w + 1] = __builtin_bit_cast(uint32_t, __builtin_convertvector(hi, bf16x2));
  }
  return r;
}

// LDS reads of one P V^T pass of the pipelined loop: step s issues the two
// transposed V reads of step s+3, then waits for its own (issued three steps
// earlier, or before step 0) and runs its MFMA.  The lgkmcnt to wait for is
// the number of LDS reads issued after them (LDS operations complete in order).
template <int NST>
constexpr int pv_reads_after(int st) {
  int n = st >= 3 ? 0 : 2 * (2 - st);  // pre-issued reads of steps st+1 .. 2
  for (int s = st >= 3 ? st - 2 : 0; s <= st; ++s) n += s + 3 < NST ? 2 : 0;
  return n;
}

// Multiply an MFMA accumulator held in AGPRs by s in place.  The "+a"
// constraints keep the accumulator in the AGPR file, so this (rare) rescale
// costs no VGPRs beyond one temporary.
__device__ __forceinline__ void scale_acc4(float& x0, float& x1, float& x2, float& x3, float s) {
  float t;
  asm volatile(
      "v_accvgpr_read_b32 %4, %0\n\tv_mul_f32 %4, %4, %5\n\tv_accvgpr_write_b32 %0, %4\n\t"
      "v_accvgpr_read_b32 %4, %1\n\tv_mul_f32 %4, %4, %5\n\tv_accvgpr_write_b32 %1, %4\n\t"
      "v_accvgpr_read_b32 %4, %2\n\tv_mul_f32 %4, %4, %5\n\tv_accvgpr_write_b32 %2, %4\n\t"
      "v_accvgpr_read_b32 %4, %3\n\tv_mul_f32 %4, %4, %5\n\tv_accvgpr_write_b32 %3, %4"
      : "+a"(x0), "+a"(x1), "+a"(x2), "+a"(x3), "=&v"(t)
      : "v"(s));
}

template <int N>
__device__ __forceinline__ void scale_acc(float __attribute__((ext_vector_type(N))) & a, float s) {
#pragma unroll
  for (int i = 0; i < N; i += 4) {
    float x0 = a[i], x1 = a[i + 1], x2 = a[i + 2], x3 = a[i + 3];
    scale_acc4(x0, x1, x2, x3, s);
    a[i] = x0;
    a[i + 1] = x1;
    a[i + 2] = x2;
    a[i + 3] = x3;
  }
}

__device__ __forceinline__ void store_out4(void* o, int o_f32, size_t idx, f32x4 v) {
  if (o_f32) {
    *reinterpret_cast<f32x4*>(reinterpret_cast<float*>(o) + idx) = v;
  } else {
    bf16x4 b = __builtin_convertvector(v, bf16x4);
    *reinterpret_cast<bf16x4*>(reinterpret_cast<__bf16*>(o) + idx) = b;
  }
}


}  // namespace

// Kernel parameters of stage 1 (one definition for every translation unit
// built from this source, see the dispatch section).
struct Stage1Params {
  // The query rows: row r (= query token x heads + head) of sequence b is
  // [q_nope (D_v) | q_pe (64)], the two parts read from two base pointers
  // with their own sequence and row strides (in elements), so that a caller
  // holding them as separate tensors needs no concatenation.
  const __bf16* q_nope;
  const __bf16* q_pe;
  int64_t qn_seq, qn_row, qp_seq, qp_row;
  const uint8_t* kv;
  const int32_t* block_table;
  const int32_t* seq_lens;
  void* o;
  float* lse;
  _Float16* ws_o;  // partial outputs, fp16, each row scaled by a power of two
  f32x2* ws_ls;    // per partial row: {lse (natural log), that power of two}
  int32_t* ws_seg; // balanced mode, per sequence: {first slot, partial count or -1}
  int32_t batch, heads, page_size, bt_stride;
  int32_t o_f32, split_mode, num_splits, head_chunks;
  int32_t seg_cost;  // balanced mode: virtual tiles charged per sequence start
  // Memory safety: every length read from seq_lens is clamped to [0, len_cap]
  // (len_cap = bt_stride * page_size, or topk for sparse decode), so no read
  // goes past a block-table or index row; a page number outside
  // [0, num_blocks) reads as zero rows.
  int32_t len_cap;
  uint32_t num_blocks;
  // Multi-token decode: the rows are q_len query tokens x heads_per_token
  // heads (row = token * heads_per_token + head).  Token i of a sequence with
  // n keys sees positions t < n - q_len + 1 + i.  Plain decode: q_len = 1.
  int32_t q_len, heads_per_token;
  // Sparse (top-k) decode: sequence b attends to the cache rows of the
  // logical positions topk_idx[b * topk_stride + e], e < seq_lens[b] (the
  // split logic then counts list entries, not positions).  pool_bytes bounds
  // the one buffer resource over the whole cache (< 4 GB); page_shift is
  // log2(page_size) when that is a power of two, else -1.
  const int32_t* topk_idx;
  int32_t topk_stride, page_shift;
  uint32_t pool_bytes;
  float score_log2;  // scale * log2(e) (* k_scale for per-tensor fp8 caches)
  float out_scale;   // 1, or k_scale for per-tensor fp8 caches
};

namespace {


// ---------------------------------------------------------------- work units

// Split of sequence b in per-sequence mode: C_b = roundup(ceil(n / S), 32).
__device__ __forceinline__ int per_seq_chunk(int n, int S) {
  int c = (n + S - 1) / S;
  return (c + kTile - 1) / kTile * kTile;
}

// Unit that holds global tile x when TT tiles are cut into U runs
// [floor(u*TT/U), floor((u+1)*TT/U)).
__device__ __forceinline__ int unit_of_tile(int64_t x, int64_t TT, int U) {
  return (int)(((x + 1) * (int64_t)U - 1) / TT);
}

__device__ __forceinline__ int tiles_of(int n) { return (n + kTile - 1) / kTile; }

// Length of sequence b, clamped to [0, cap]: the kernels never read past the
// table (or index list) row a length implies, whatever seq_lens holds.
__device__ __forceinline__ int seq_len_at(const int32_t* seq_lens, int b, int cap) {
  const int n = seq_lens[b];
  return n < 0 ? 0 : (n > cap ? cap : n);
}

// Inclusive wave prefix sum.
__device__ __forceinline__ int wave_incl_scan(int x, int lane) {
#pragma unroll
  for (int d = 1; d < 64; d <<= 1) {
    int y = __shfl_up(x, d, 64);
    if (lane >= d) x += y;
  }
  return x;
}

// Balanced mode cuts a "cost stream" into equal runs: every non-empty
// sequence contributes SC virtual tiles (what starting a segment costs: the
// query load, the first tiles' latency and a partial's store) and then its
// 32-position tiles.  A unit that starts a sequence part-way through
// therefore streams fewer tiles, and units finish together.
__device__ __forceinline__ int cost_of(int n, int sc) { return n > 0 ? sc + tiles_of(n) : 0; }

__device__ __forceinline__ int64_t total_cost(const int32_t* seq_lens, int B, int sc, int cap,
                                              int lane) {
  int64_t tot = 0;
  for (int c0 = 0; c0 < B; c0 += 64) {
    int b = c0 + lane;
    int nt = b < B ? cost_of(seq_len_at(seq_lens, b, cap), sc) : 0;
    int s = wave_incl_scan(nt, lane);
    tot += __shfl(s, 63, 64);
  }
  return tot;
}

// LDS layout of a 32-position tile.  Block (th, kq), at (th * NKQ + kq) KB,
// holds positions 16*th .. 16*th+15 and the four 16-byte chunks c4 of d-group
// kq (d = 32*kq + 8*c4 + e).  Position t16 owns the 64 bytes of slots
// 4*t16 .. 4*t16+3, its chunk c4 at slot 4*t16 + (c4 ^ tile_swz(t16)), where
// tile_swz bit-reverses t16 / 4.  A 16-lane quarter of a QK^T read (fixed
// c4, t16 = 0..15) and each half-wave of a transposed V read (4 or 8
// positions x 2 or 4 chunks) touch 16 distinct 16-byte bank groups.  The
// copy that fills a block from the cache then has each quad of lanes read
// one row's 64 contiguous bytes, which the address unit takes about three
// times faster than one 16-byte chunk from each of four rows.
__device__ __forceinline__ int tile_swz(int t16) { return 2 * ((t16 >> 2) & 1) + ((t16 >> 3) & 1); }
__device__ __forceinline__ int tile_slot(int t16, int c4) {
  return 4 * t16 + (c4 ^ tile_swz(t16));
}

}  // namespace
}  // namespace mla
