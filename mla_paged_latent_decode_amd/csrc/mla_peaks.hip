// Measured-ceiling probes for MI355X (gfx950), built into libmla_peaks.so and
// called only by the benchmark (`bench.py --peaks`).  They are not part of the
// decode path.  Each probe isolates one resource the stage-1 decode kernel
// leans on and reports what the chip sustains for it:
//
//   mla_peak_stream   HBM -> LDS streaming with the decode's own load pattern:
//                     32-row tiles of 576-wide bf16 rows (36 KB), each tile
//                     half a 64-row page placed at a random page of a pool,
//                     copied by 16-byte buffer_load ... lds instructions into
//                     a ring of LDS tiles with one workgroup barrier per tile;
//                     optionally every wave also reads each tile back from LDS
//                     (the QK^T + PV operand traffic of one tile per wave).
//   mla_peak_mfma     a dependency-free loop of v_mfma_f32_32x32x16_bf16
//                     (the decode's contraction instruction) on every SIMD.
//   mla_peak_mfma_chain the same instruction on 1, 2, 4 or 8 accumulator
//                     chains: with one chain every MFMA takes the previous
//                     one's result as its accumulator (the decode's QK^T).
//   mla_peak_lds      ds_read_b128 from LDS by 4 or 8 waves per workgroup.
//   mla_peak_tileloop the stage-1 tile loop stripped to its resource use:
//                     per 36 KB tile and wave, 9 copies in the decode's
//                     pattern (ring of 3) spread over 68 MFMAs
//                     (v_mfma_f32_32x32x16_bf16, K and V operands read from
//                     the tile in LDS, 256 AGPR accumulators) and softmax-like
//                     VALU work on the scores; or the compute alone.  Run on
//                     the caller's page contents, it shows how the data (and
//                     the HBM streaming beside the MFMAs) sets the clock.
//
// Every probe records, per workgroup, the shader-clock cycles (s_memtime) and
// the 100 MHz constant-clock ticks (s_memrealtime) it ran for, so the caller
// can derive both the rate and the clock it ran at.
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
#define LDS_AS __attribute__((address_space(3)))

constexpr int kRow = 1152;            // bytes of one 576-wide bf16 row
constexpr int kTileRows = 32;
constexpr int kTileBytes = kTileRows * kRow;  // 36 KB
constexpr int kBlocks = kTileBytes / 1024;    // 36 blocks of 1 KB per tile

template <int VM>
__device__ __forceinline__ void wait_vmcnt() {
  __builtin_amdgcn_s_waitcnt((VM & 15) | (7 << 4) | (0 << 8) | ((VM >> 4) << 14));
}

__device__ __forceinline__ void stamp(uint64_t* out, uint64_t c0, uint64_t r0) {
  out[2 * blockIdx.x] = __builtin_amdgcn_s_memtime() - c0;
  out[2 * blockIdx.x + 1] = __builtin_amdgcn_s_memrealtime() - r0;
}

// Workgroup w streams tiles w * per_wg .. (w+1) * per_wg - 1; tile t is half
// `t & 1` of page pages[t >> 1] of a pool of 64-row pages.  W waves, NBUF
// LDS tiles, block j of a tile copied by wave j % W.  ROWS = true: each load
// instruction takes 64 bytes from each of 16 consecutive rows, each quad of
// lanes one row's 64 contiguous bytes in a row-dependent order (the decode's
// tile copies); false: 1 KB contiguous per instruction.  READ = true: each
// wave then reads the whole tile back with ds_read_b128.
template <int W, int NBUF, bool ROWS, bool READ>
__global__ __launch_bounds__(64 * W) void stream_probe(const uint8_t* __restrict__ pool,
                                                       const int32_t* __restrict__ pages,
                                                       int per_wg, uint64_t* cycles,
                                                       uint32_t* sink) {
  __shared__ __attribute__((aligned(1024))) uint8_t ring[NBUF * kTileBytes];
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  constexpr int LPW = (kBlocks + W - 1) / W;  // most blocks any wave copies per tile
  const bool full = kBlocks % W == 0 || wave < kBlocks % W;
  // per-lane source offset of a block: 16 rows x 64 B (row lane / 4, chunk
  // (lane % 4) ^ f(row)), or 1 KB contiguous
  const int voff = ROWS ? (lane >> 2) * kRow + 16 * ((lane & 3) ^ (2 * ((lane >> 4) & 1) +
                                                                   ((lane >> 5) & 1)))
                        : 16 * lane;
  const uint64_t c0 = __builtin_amdgcn_s_memtime();
  const uint64_t r0 = __builtin_amdgcn_s_memrealtime();
  const int t0 = blockIdx.x * per_wg;
  auto issue = [&](int i) {
    const int t = t0 + i;
    const int64_t page = pages[t >> 1];
    const uint8_t* base = pool + (page * 64 + (t & 1) * 32) * (int64_t)kRow;
    const __amdgpu_buffer_rsrc_t rs =
        __builtin_amdgcn_make_buffer_rsrc((void*)base, (short)0, kTileBytes, 0x00020000);
    uint8_t* dst = ring + (i % NBUF) * kTileBytes;
#pragma unroll
    for (int k = 0; k < LPW; ++k) {
      const int j = wave + k * W;
      if (j < kBlocks) {
        // block j: rows 16 * (j / 18) .., 64-byte column group j % 18 (ROWS),
        // or bytes 1024 j .. (contiguous)
        const int src = ROWS ? (j / 18) * 16 * kRow + (j % 18) * 64 : j * 1024;
        __builtin_amdgcn_raw_ptr_buffer_load_lds(rs, (LDS_AS void*)(dst + j * 1024), 16,
                                                 voff + src, 0, 0, 0);
      }
    }
  };
  uint32_t acc = 0;
#pragma unroll
  for (int i = 0; i < NBUF - 1; ++i)
    if (i < per_wg) issue(i);
  for (int i = 0; i < per_wg; ++i) {
    const int ahead = min(NBUF - 2, per_wg - 1 - i);
    if (ahead >= 2) {
      if (full) wait_vmcnt<2 * LPW>(); else wait_vmcnt<2 * (LPW - 1)>();
    } else if (ahead == 1) {
      if (full) wait_vmcnt<LPW>(); else wait_vmcnt<LPW - 1>();
    } else {
      wait_vmcnt<0>();
    }
    __builtin_amdgcn_s_barrier();
    if (i + NBUF - 1 < per_wg) issue(i + NBUF - 1);
    if constexpr (READ) {
      const LDS_AS uint8_t* t = (const LDS_AS uint8_t*)ring + (i % NBUF) * kTileBytes;
#pragma unroll 4
      for (int b = 0; b < kBlocks; ++b) {
        const u32x4 v = *reinterpret_cast<const LDS_AS u32x4*>(t + b * 1024 + 16 * lane);
        acc ^= v[0] ^ v[1] ^ v[2] ^ v[3];
      }
    }
  }
  wait_vmcnt<0>();
  __builtin_amdgcn_s_barrier();
  if (threadIdx.x == 0) stamp(cycles, c0, r0);
  if (acc == 0x9e3779b9u) sink[threadIdx.x] = acc;  // keep the LDS reads alive
}

// Each wave runs `iters` rounds of 8 independent 32x32x16 bf16 MFMAs.
__global__ __launch_bounds__(256) void mfma_probe(int iters, uint64_t* cycles, float* sink) {
  const uint64_t c0 = __builtin_amdgcn_s_memtime();
  const uint64_t r0 = __builtin_amdgcn_s_memrealtime();
  bf16x8 a, b;
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    a[i] = (__bf16)(0.001f * (threadIdx.x + i));
    b[i] = (__bf16)(0.002f * (i - 3));
  }
  f32x16 acc[8] = {};
  for (int it = 0; it < iters; ++it) {
#pragma unroll
    for (int c = 0; c < 8; ++c) acc[c] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, acc[c], 0, 0, 0);
  }
  __syncthreads();
  if (threadIdx.x == 0) stamp(cycles, c0, r0);
  float s = 0.f;
#pragma unroll
  for (int c = 0; c < 8; ++c) s += acc[c][c];
  if (s == 1234.5f) sink[threadIdx.x] = s;
}

// Each wave runs `iters` rounds of 8 v_mfma_f32_32x32x16_bf16 spread over CH
// accumulator chains (CH = 1: each MFMA depends on the one before it).
template <int CH>
__global__ __launch_bounds__(256) void mfma_chain_probe(int iters, uint64_t* cycles, float* sink) {
  static_assert(8 % CH == 0, "");
  const uint64_t c0 = __builtin_amdgcn_s_memtime();
  const uint64_t r0 = __builtin_amdgcn_s_memrealtime();
  bf16x8 a, b;
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    a[i] = (__bf16)(0.001f * (threadIdx.x + i));
    b[i] = (__bf16)(0.002f * (i - 3));
  }
  f32x16 acc[CH] = {};
  for (int it = 0; it < iters; ++it) {
#pragma unroll
    for (int r = 0; r < 8 / CH; ++r)
#pragma unroll
      for (int c = 0; c < CH; ++c)
        acc[c] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, acc[c], 0, 0, 0);
  }
  __syncthreads();
  if (threadIdx.x == 0) stamp(cycles, c0, r0);
  float s = 0.f;
#pragma unroll
  for (int c = 0; c < CH; ++c) s += acc[c][c];
  if (s == 1234.5f) sink[threadIdx.x] = s;
}

// W waves each read `iters` x 64 KB of LDS with ds_read_b128.
template <int W>
__global__ __launch_bounds__(64 * W) void lds_probe(int iters, uint64_t* cycles, uint32_t* sink) {
  __shared__ __attribute__((aligned(1024))) uint8_t buf[65536];
  for (int i = threadIdx.x; i < 65536 / 16; i += 64 * W)
    reinterpret_cast<u32x4*>(buf)[i] = u32x4{(uint32_t)i, 1u, 2u, 3u};
  __syncthreads();
  const int lane = threadIdx.x & 63;
  const uint64_t c0 = __builtin_amdgcn_s_memtime();
  const uint64_t r0 = __builtin_amdgcn_s_memrealtime();
  uint32_t acc = 0;
  for (int it = 0; it < iters; ++it) {
#pragma unroll 8
    for (int b = 0; b < 64; ++b) {
      const u32x4 v = *reinterpret_cast<const LDS_AS u32x4*>((const LDS_AS uint8_t*)buf +
                                                             b * 1024 + 16 * lane);
      acc ^= v[0] + v[3];
    }
  }
  __syncthreads();
  if (threadIdx.x == 0) stamp(cycles, c0, r0);
  if (acc == 0x9e3779b9u) sink[threadIdx.x] = acc;
}

// W waves each read `iters` x 32 KB of LDS with ds_read_b64_tr_b16, the
// transposed 16-bit read that feeds the P.V contraction its V^T operand.
template <int W>
__global__ __launch_bounds__(64 * W) void lds_tr_probe(int iters, uint64_t* cycles, uint32_t* sink) {
  __shared__ __attribute__((aligned(1024))) uint8_t buf[65536];
  for (int i = threadIdx.x; i < 65536 / 16; i += 64 * W)
    reinterpret_cast<u32x4*>(buf)[i] = u32x4{(uint32_t)i, 1u, 2u, 3u};
  __syncthreads();
  const int lane = threadIdx.x & 63;
  const uint32_t base = (uint32_t)(uintptr_t)(LDS_AS uint8_t*)buf + 8 * lane;
  const uint64_t c0 = __builtin_amdgcn_s_memtime();
  const uint64_t r0 = __builtin_amdgcn_s_memrealtime();
  uint32_t acc = 0;
  for (int it = 0; it < iters; ++it) {
#pragma unroll
    for (int b = 0; b < 64; b += 8) {
      typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
      u32x2 v[8];
#pragma unroll
      for (int k = 0; k < 8; ++k)
        asm volatile("ds_read_b64_tr_b16 %0, %1 offset:%2" : "=v"(v[k]) : "v"(base), "i"((b + k) * 512));
      // the wait is tied to every loaded value, so no use can move above it
#pragma unroll
      for (int k = 0; k < 8; ++k) asm volatile("s_waitcnt lgkmcnt(0)" : "+v"(v[k]));
#pragma unroll
      for (int k = 0; k < 8; ++k) acc ^= v[k][0] + v[k][1];
    }
  }
  __syncthreads();
  if (threadIdx.x == 0) stamp(cycles, c0, r0);
  if (acc == 0x9e3779b9u) sink[threadIdx.x] = acc;
}

// The tile loop of stage 1 without its bookkeeping: 4 waves, tiles as in
// stream_probe (ring of 3, the decode's 16-row x 64-byte copies), per tile and
// wave 36 MFMAs of S = K Q (K from the tile, Q in registers), a row max and
// exponentials of the 16 scores per lane, and 32 MFMAs of O += V P into 16
// accumulator blocks (V from the tile); copy k of the wave's 9 goes out after
// MFMA step floor(68 k / 9).  COPY = false: the same compute on a tile that
// stays in LDS (filled once).
template <bool COPY>
__global__ __launch_bounds__(256) void tileloop_probe(const uint8_t* __restrict__ pool,
                                                      const int32_t* __restrict__ pages,
                                                      int per_wg, uint64_t* cycles, float* sink) {
  constexpr int NBUF = 3;
  __shared__ __attribute__((aligned(1024))) uint8_t ring[NBUF * kTileBytes];
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int voff = (lane >> 2) * kRow + 16 * ((lane & 3) ^ (2 * ((lane >> 4) & 1) + ((lane >> 5) & 1)));
  const int t0 = blockIdx.x * per_wg;
  auto base_of = [&](int i) {
    const int t = t0 + i;
    const int64_t page = pages[t >> 1];
    return (uint64_t)(pool + (page * 64 + (t & 1) * 32) * (int64_t)kRow);
  };
  auto copy = [&](uint64_t base, int i, int k) {
    const int j = wave + 4 * k;
    const int src = (j / 18) * 16 * kRow + (j % 18) * 64;
    const __amdgpu_buffer_rsrc_t rs =
        __builtin_amdgcn_make_buffer_rsrc((void*)base, (short)0, kTileBytes, 0x00020000);
    __builtin_amdgcn_raw_ptr_buffer_load_lds(rs, (LDS_AS void*)(ring + (i % NBUF) * kTileBytes + j * 1024),
                                             16, voff + src, 0, 0, 0);
  };
  f32x16 o[16];
#pragma unroll
  for (int v = 0; v < 16; ++v) o[v] = f32x16{};
  bf16x8 q[24];
#pragma unroll
  for (int k = 0; k < 24; ++k)
#pragma unroll
    for (int e = 0; e < 8; ++e) q[k][e] = (__bf16)(0.01f * (k + e + lane));
  float lsum = 0.f;
  if constexpr (COPY) {
    for (int i = 0; i < NBUF - 1; ++i) {
      const uint64_t b = base_of(i);
#pragma unroll
      for (int k = 0; k < 9; ++k) copy(b, i, k);
    }
  } else {
    const uint64_t b = base_of(0);
#pragma unroll
    for (int k = 0; k < 9; ++k) copy(b, 0, k);
    wait_vmcnt<0>();
  }
  __builtin_amdgcn_s_barrier();
  const uint64_t c0 = __builtin_amdgcn_s_memtime();
  const uint64_t r0 = __builtin_amdgcn_s_memrealtime();
  for (int i = 0; i < per_wg; ++i) {
    if constexpr (COPY) {
      if (i + 1 < per_wg) wait_vmcnt<9>(); else wait_vmcnt<0>();
    }
    __builtin_amdgcn_s_barrier();
    const bool more = COPY && i + NBUF - 1 < per_wg;
    const uint64_t nb = more ? base_of(i + NBUF - 1) : 0;
    auto copy_at = [&](int step) {
#pragma unroll
      for (int k = 0; k < 9; ++k)
        if ((k * 68) / 9 == step && more) copy(nb, i + NBUF - 1, k);
    };
    const LDS_AS uint8_t* tile = (const LDS_AS uint8_t*)ring + (COPY ? (i % NBUF) : 0) * kTileBytes;
    f32x16 s = {};
    auto kq = [&](int ks) {
      return *reinterpret_cast<const LDS_AS bf16x8*>(tile + (ks >> 1) * 1024 + 16 * lane);
    };
    bf16x8 k0 = kq(0), k1 = kq(1);
#pragma unroll
    for (int ks = 0; ks < 36; ++ks) {
      bf16x8 k2 = k1;
      if (ks + 2 < 36) k2 = kq(ks + 2);
      s = __builtin_amdgcn_mfma_f32_32x32x16_bf16(k0, q[ks % 24], s, 0, 0, 0);
      copy_at(ks);
      __builtin_amdgcn_sched_barrier(0);
      k0 = k1;
      k1 = k2;
    }
    float m = s[0];
#pragma unroll
    for (int r = 1; r < 16; ++r) m = fmaxf(m, s[r]);
    m = fmaxf(m, __shfl_xor(m, 32));
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      s[r] = __builtin_amdgcn_exp2f(s[r] * 0.1f - m);
      lsum += s[r];
    }
    bf16x8 p0, p1;
#pragma unroll
    for (int r = 0; r < 8; ++r) {
      p0[r] = (__bf16)s[r];
      p1[r] = (__bf16)s[8 + r];
    }
    auto vq = [&](int st) {
      return *reinterpret_cast<const LDS_AS bf16x8*>(tile + ((st / 16) * 18 + st % 16) * 1024 + 16 * lane);
    };
    bf16x8 a0 = vq(0), a1 = vq(1);
#pragma unroll
    for (int st = 0; st < 32; ++st) {
      bf16x8 a2 = a1;
      if (st + 2 < 32) a2 = vq(st + 2);
      o[st % 16] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a0, (st / 16) ? p1 : p0, o[st % 16], 0, 0, 0);
      copy_at(36 + st);
      __builtin_amdgcn_sched_barrier(0);
      a0 = a1;
      a1 = a2;
    }
  }
  wait_vmcnt<0>();
  __builtin_amdgcn_s_barrier();
  if (threadIdx.x == 0) stamp(cycles, c0, r0);
  float t = lsum;
#pragma unroll
  for (int v = 0; v < 16; ++v) t += o[v][v];
  if (t == 1234.5f) sink[threadIdx.x] = t;
}

template <int W, int NBUF, bool ROWS, bool READ>
int launch_stream(const void* pool, const int32_t* pages, int grid, int per_wg, uint64_t* cyc,
                  uint32_t* sink, hipStream_t st) {
  hipLaunchKernelGGL((stream_probe<W, NBUF, ROWS, READ>), dim3(grid), dim3(64 * W), 0, st,
                     (const uint8_t*)pool, pages, per_wg, cyc, sink);
  return (int)hipGetLastError();
}

}  // namespace

extern "C" {

/* HBM -> LDS streaming probe.  pool: device buffer of 64-row pages of
 * 1152-byte rows; pages: device int32 list of grid * per_wg / 2 page numbers
 * (tile t is half t & 1 of page pages[t / 2]); per_wg even.  waves 4 or 8;
 * ring 2, 3 or 4 tiles; rows: 1 = the decode's 16-row x 64-byte load layout,
 * 0 = 1 KB contiguous per load; read: 1 = every wave reads each tile back
 * from LDS.  cycles: device uint64 [grid][2] {shader cycles, 100 MHz ticks};
 * sink: device uint32 [512] (never written in practice).  Returns 0 or a HIP
 * error code; -1 for an unsupported combination. */
int mla_peak_stream(const void* pool, const int32_t* pages, int grid, int per_wg, int waves,
                    int ring, int rows, int read, void* cycles, void* sink, void* stream) {
  hipStream_t st = (hipStream_t)stream;
  uint64_t* cyc = (uint64_t*)cycles;
  uint32_t* sk = (uint32_t*)sink;
  if (per_wg < 2 || per_wg % 2) return -1;
#define MLA_PEAK_CASE(W_, R_, ROWS_, RD_)                                                  \
  if (waves == W_ && ring == R_ && rows == ROWS_ && read == RD_)                            \
    return launch_stream<W_, R_, ROWS_ != 0, RD_ != 0>(pool, pages, grid, per_wg, cyc, sk, st);
  MLA_PEAK_CASE(4, 2, 1, 0) MLA_PEAK_CASE(4, 3, 1, 0) MLA_PEAK_CASE(4, 4, 1, 0)
  MLA_PEAK_CASE(4, 3, 0, 0) MLA_PEAK_CASE(4, 3, 1, 1) MLA_PEAK_CASE(8, 3, 1, 0)
  MLA_PEAK_CASE(8, 4, 1, 0) MLA_PEAK_CASE(8, 3, 1, 1)
#undef MLA_PEAK_CASE
  return -1;
}

/* MFMA probe: grid workgroups of 4 waves, each wave `iters` x 8 independent
 * v_mfma_f32_32x32x16_bf16 (32768 FLOP each).  cycles as above; sink: device
 * float [256]. */
int mla_peak_mfma(int grid, int iters, void* cycles, void* sink, void* stream) {
  hipLaunchKernelGGL(mfma_probe, dim3(grid), dim3(256), 0, (hipStream_t)stream, iters,
                     (uint64_t*)cycles, (float*)sink);
  return (int)hipGetLastError();
}

/* MFMA chain probe: as the MFMA probe, each wave's 8 MFMAs per round spread
 * over `chains` accumulators (1, 2, 4 or 8; anything else returns -1). */
int mla_peak_mfma_chain(int grid, int iters, int chains, void* cycles, void* sink, void* stream) {
  hipStream_t st = (hipStream_t)stream;
  uint64_t* c = (uint64_t*)cycles;
  float* k = (float*)sink;
  switch (chains) {
    case 1: hipLaunchKernelGGL(mfma_chain_probe<1>, dim3(grid), dim3(256), 0, st, iters, c, k); break;
    case 2: hipLaunchKernelGGL(mfma_chain_probe<2>, dim3(grid), dim3(256), 0, st, iters, c, k); break;
    case 4: hipLaunchKernelGGL(mfma_chain_probe<4>, dim3(grid), dim3(256), 0, st, iters, c, k); break;
    case 8: hipLaunchKernelGGL(mfma_chain_probe<8>, dim3(grid), dim3(256), 0, st, iters, c, k); break;
    default: return -1;
  }
  return (int)hipGetLastError();
}

/* LDS read probe: grid workgroups of `waves` (4 or 8) waves, each wave reading
 * iters x 64 KB with ds_read_b128 (tr = 0), or iters x 32 KB with
 * ds_read_b64_tr_b16 (tr = 1).  cycles and sink as above. */
int mla_peak_lds(int grid, int waves, int iters, int tr, void* cycles, void* sink, void* stream) {
  hipStream_t st = (hipStream_t)stream;
  if (tr) {
    if (waves == 4)
      hipLaunchKernelGGL(lds_tr_probe<4>, dim3(grid), dim3(256), 0, st, iters, (uint64_t*)cycles,
                         (uint32_t*)sink);
    else if (waves == 8)
      hipLaunchKernelGGL(lds_tr_probe<8>, dim3(grid), dim3(512), 0, st, iters, (uint64_t*)cycles,
                         (uint32_t*)sink);
    else
      return -1;
    return (int)hipGetLastError();
  }
  if (waves == 4)
    hipLaunchKernelGGL(lds_probe<4>, dim3(grid), dim3(256), 0, st, iters, (uint64_t*)cycles,
                       (uint32_t*)sink);
  else if (waves == 8)
    hipLaunchKernelGGL(lds_probe<8>, dim3(grid), dim3(512), 0, st, iters, (uint64_t*)cycles,
                       (uint32_t*)sink);
  else
    return -1;
  return (int)hipGetLastError();
}

/* Tile-loop probe: grid workgroups of 4 waves streaming per_wg tiles each
 * (pool and pages as for mla_peak_stream), with the stage-1 loop's MFMA, LDS
 * and VALU work per tile; copy = 0 runs the compute alone on the first tile.
 * cycles and sink (device float [256]) as above. */
int mla_peak_tileloop(const void* pool, const int32_t* pages, int grid, int per_wg, int copy,
                      void* cycles, void* sink, void* stream) {
  if (per_wg < 2 || per_wg % 2) return -1;
  if (copy)
    hipLaunchKernelGGL(tileloop_probe<true>, dim3(grid), dim3(256), 0, (hipStream_t)stream,
                       (const uint8_t*)pool, pages, per_wg, (uint64_t*)cycles, (float*)sink);
  else
    hipLaunchKernelGGL(tileloop_probe<false>, dim3(grid), dim3(256), 0, (hipStream_t)stream,
                       (const uint8_t*)pool, pages, per_wg, (uint64_t*)cycles, (float*)sink);
  return (int)hipGetLastError();
}

}  // extern "C"
