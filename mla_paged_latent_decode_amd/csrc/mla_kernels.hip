// HIP kernels of libmla for gfx950 (MI355X): MLA paged latent decode.
//
// Stage 1 (split-KV attention over one segment of one sequence).
//   One workgroup owns one work unit (a run of 32-position tiles of one or two
//   sequences) and one chunk of heads; each wave owns 16 or 32 heads.  Per
//   tile, the wave computes S^T[token, head] = K Q^T on bf16 MFMA (all heads
//   share the one latent row stream, multi-query attention; "Triton と MLA"
//   page, データフロー), updates the online softmax state (running max m,
//   running sum l, rescaled accumulator; "vLLM 中 Attention Kernel 如何并行处理
//   多个请求", section 七), and accumulates O^T[v, head] += V^T P^T on MFMA,
//   where V is the leading D_v columns of the same tile.  Pages are reached
//   through the block table (same article, section 十一).
//
//   Tiles stream HBM -> LDS with 16-byte buffer_load ... lds (no register
//   staging) into a ring of NBUF tiles, NBUF-1 tiles ahead of the compute.
//   The LDS tile is stored as 1 KB blocks of 16 positions x 64 bytes with an
//   XOR swizzle, so that both the QK^T read (ds_read_b128) and the
//   transposed V read (ds_read_b64_tr_b16) hit distinct banks.
//
//   Variants of the same kernel: narrow caches (e4m3fn with a per-tensor
//   scale, or e4m3fn / int8 / packed int4 codes with a per-token inline
//   scale, "Triton と MLA" page, 主要ファイル) are staged in LDS and widened
//   to bf16 there;
//   multi-token decode gives each query-token row its own causal limit
//   (article above, section 十); sparse decode takes its rows from a list of
//   logical positions (section 十三) through an index-driven gather.
//
// Stage 2 (merge).  Partials (o_s, lse_s) of a sequence are combined with the
//   log-sum-exp rule of the same article, section 十二:
//   lse = M + ln sum_s e^(lse_s - M),  o = sum_s e^(lse_s - lse) o_s.
#include <hip/hip_ext.h>

#include "mla_device.h"

namespace mla {
namespace {

// ---------------------------------------------------------------- stage 1

// PT: 0 = no per-token scales, 1 = per-token e4m3fn codes, 2 = per-token int8
// codes, 3 = per-token int4 codes (two per byte)
template <int HPW, int W, int D, int DV, int NBUF, bool F8, int PT = 0>
struct Cfg {
  static constexpr int NKQ = D / 32;                       // 32-wide d groups per row
  static constexpr int NBLK = 2 * NKQ;                     // 1 KB LDS blocks per tile
  static constexpr int NKS = HPW == 32 ? D / 16 : D / 32;  // QK k-steps
  // With 32 heads per wave and D = 576, the O accumulators (256 registers)
  // and all 36 Q fragments (144) leave too few registers for the rest of the
  // loop; the last QLDS k-steps of Q then live in LDS (1 KB per step/wave).
  static constexpr int QLDS = stage1_qlds_steps(HPW, W, D, F8, PT);
  static constexpr int NQR = NKS - QLDS;                   // Q k-steps held in VGPRs
  static constexpr int QLDS_BYTES = W * QLDS * 1024;
  static constexpr int LPW = NBLK / W;                     // bf16 blocks per wave per tile
  static constexpr int TILE_BYTES = NBLK * 1024;
  static constexpr int NVB = HPW == 32 ? DV / 32 : DV / 16;  // PV output blocks
  static constexpr int HEADS_PER_WG = HPW * W;
  static constexpr int CB = stage1_code_bytes(D, F8, PT);      // code bytes of a cache row
  static constexpr int SRC_ROW = PT ? CB + kPerTokenPad : CB;  // cache row bytes
  // 1-byte and 4-bit codes: a 16-row half tile (16*CB code bytes of one
  // page) is copied to a row-major staging tile with G-byte LDS DMA per lane
  // (consecutive lanes write consecutive G bytes), G = 16 when a half tile
  // is a whole number of 1 KB copies that never straddle a row, else 4;
  // bf16: one 16-byte copy per lane and block.  A wave stalls at each copy
  // it issues while the memory pipeline drains, so few wide copies beat many
  // narrow ones.  The 2*NIH copies of a tile are dealt round-robin: wave w
  // issues copies w, w+W, ..., at most NIW of them (narrow codes wait for all
  // of a wave's copies at once, so the counts may differ between waves).
  static constexpr int G = !F8 ? 16 : ((16 * CB) % 1024 == 0 && CB % 16 == 0) ? 16 : 4;
  static constexpr int NIH = F8 ? 16 * CB / (64 * G) : NKQ;  // DMA copies per half tile
  static constexpr int NIW = (2 * NIH + W - 1) / W;          // DMA copies per wave per tile
  static constexpr int STG_TILE = F8 ? kTile * CB : 0;       // staging tile bytes
  static constexpr int CVB = PT == 3 ? 4 : 8;                // code bytes of 8 elements
  static constexpr int STG_BYTES = 2 * STG_TILE;
  static constexpr int SCL_BYTES = stage1_scale_bytes(HPW, W, D, F8, PT);
  // Pipelined bf16 loop: the k-th of a wave's NIW tile loads goes out at step
  // dma_step(k) of the iteration's NKS QK^T + 2*NVB PV MFMA steps.  Spread
  // evenly, the loads leave the memory pipeline at about the rate HBM drains
  // it, so an issue rarely blocks the wave (and its MFMAs); bunched together
  // they would block while the pipeline runs dry for the rest of the tile.
  // With a ring of three the loads of tile j+2 must land before iteration
  // j+1 starts, so they go out over the first half of the QK^T steps.
  static constexpr int dma_step(int k) {
    return NBUF >= 4 ? k * (NKS + 2 * NVB) / NIW : k * (NKS / 2) / NIW;
  }
  // Software-pipelined loop (softmax of tile j interleaved with the QK^T of
  // tile j+1): kept for the bf16 4-tile ring (D = 320).  At D = 576 the
  // plain loop is as fast or faster (bf16: as fast with loads and faster
  // without; fp8: 8 % faster per decode step): within one wave gfx950 does
  // not overlap VALU work with an executing MFMA, so the interleaving buys
  // nothing, while the plain loop needs no second score buffer and can
  // spread a tile's loads over two iterations.
  static constexpr bool PIPE = HPW == 32 && !F8 && NBUF >= 4;
  static_assert(NBUF == stage1_ring_depth(HPW, W, D, F8, PT), "ring depth");
  static_assert(!PT || F8, "per-token rows hold narrow codes (e4m3fn, int8 or int4)");
  static_assert(!PT || CB % G == 0, "a copy never straddles a row's scale pad");
  static_assert(NBLK * 1024 == kTile * D * 2, "tile bytes");
  static_assert(NBLK % W == 0, "each wave loads or widens the same number of blocks");
  static_assert(!F8 || (16 * CB) % (64 * G) == 0, "narrow copy split");
  static_assert(F8 || (2 * NIH) % W == 0, "bf16 waits count the same copies in every wave");
  static_assert(F8 ? NIW <= 63 : (NBUF - 1) * LPW <= 63,
                "outstanding loads must fit the vmcnt counter");
  static_assert(NBUF * TILE_BYTES + STG_BYTES + QLDS_BYTES + SCL_BYTES <= kLdsBytes, "LDS budget");
  static_assert(D % 32 == 0 && DV % 32 == 0, "");
};


template <int HPW, int W, int D, int DV, int NBUF, bool F8, bool SP, int PT>
__global__ __launch_bounds__(64 * W) void mla_stage1(Stage1Params p) {
  using C = Cfg<HPW, W, D, DV, NBUF, F8, PT>;
  // [bf16 ring: NBUF tiles][fp8 staging: 2 tiles][Q k-steps of each wave]
  // [per-token scales: 2 staging slots of 2 x 256 B, NBUF ring slots of 256 B
  //  (32 scales, then their reciprocals)]
  __shared__ __attribute__((aligned(1024)))
  uint8_t ring[NBUF * C::TILE_BYTES + C::STG_BYTES + C::QLDS_BYTES + C::SCL_BYTES];
  uint8_t* const stg = ring + NBUF * C::TILE_BYTES;
  // LDS addresses (32-bit) of the per-token scale areas
  constexpr int kSclOff = NBUF * C::TILE_BYTES + C::STG_BYTES + C::QLDS_BYTES;
  const uint32_t scl_stage = (uint32_t)(uintptr_t)((LDS_AS uint8_t*)ring + kSclOff);
  const uint32_t scl_ring = scl_stage + 2 * 512;

  const int lane = threadIdx.x & 63;
  const int wave = uniform(threadIdx.x >> 6);

  // XCD-aware decode of the workgroup id.  Consecutive ids go to different
  // XCDs (id % 8), so XCD x is given the x-th contiguous run of units, and
  // the head chunks of one unit share it: neighbouring units mostly belong
  // to the same sequence, whose query rows then come from that XCD's L2
  // after the first read.
  const int id = blockIdx.x;
  const int num_units = p.split_mode == 0 ? p.batch * p.num_splits : p.num_splits;
  const int units_per_xcd = (num_units + 7) >> 3;
  const int hc = (id >> 3) % p.head_chunks;
  const int unit = (id & 7) * units_per_xcd + (id >> 3) / p.head_chunks;
  if (unit >= num_units) return;

  const int h0 = hc * C::HEADS_PER_WG + wave * HPW;  // first head of this wave
  const int H = p.heads;

  const int P = p.page_size;

  // ---------------- one segment [ts, te) of sequence b
  auto process = [&](int b, int ts, int te, bool final_out, int slot, int vis_n) __attribute__((always_inline)) {
    // The lane index once more, opaque to the compiler, so that the per-lane
    // offsets below (and the epilogue's addresses) are formed per segment:
    // derived from the kernel-wide lane they would be hoisted out of the
    // segment loop and held, spilled to scratch, across every epilogue.
    const int lane = vgpr_here(threadIdx.x & 63);
    // ---------------- per-lane constants of the LDS layout
    // DMA: lane l writes slot l of a block: position t16 = l / 4, chunk
    // c4 = (l % 4) ^ tile_swz(t16); its source offset within the 16-row page run.
    const int dma_t16 = lane >> 2;
    const int dma_c4 = (lane & 3) ^ tile_swz(dma_t16);
    const int dma_voff = dma_t16 * C::SRC_ROW + 16 * dma_c4;
    // fp8 widening: lane l converts chunk c4 = l % 4 of position t16 = l / 4
    // of a block, read from the row-major staging tile and written to the
    // chunk's slot of the bf16 tile layout
    const uint32_t cv_src = (uint32_t)((lane >> 2) * C::CB + C::CVB * (lane & 3));
    const uint32_t cv_dst = (uint32_t)(tile_slot(lane >> 2, lane & 3) * 16);
    int qk_off_e, qk_off_o, v_off0, v_off1;
    if constexpr (HPW == 32) {
      // QK A operand: position t = lane % 32, chunk 2*ks + lane / 32
      const int t = lane & 31, h2 = lane >> 5;
      const int thb = (t >> 4) * C::NKQ * 1024;
      qk_off_e = thb + tile_slot(t & 15, h2) * 16;      // ks even: c4 = h2
      qk_off_o = thb + tile_slot(t & 15, 2 + h2) * 16;  // ks odd:  c4 = 2 + h2
      // V^T A operand (transposed read): 4 positions x 16 v per 16-lane group
      const int g = lane >> 4, i = lane & 15, half = lane >> 5;
      const int c4 = 2 * (g & 1) + ((i >> 1) & 1);
      v_off0 = tile_slot(4 * half + (i >> 2), c4) * 16 + 8 * (i & 1);
      v_off1 = tile_slot(4 * half + (i >> 2) + 8, c4) * 16 + 8 * (i & 1);
    } else {
      qk_off_e = qk_off_o = tile_slot(lane & 15, lane >> 4) * 16;
      const int g = lane >> 4, i = lane & 15;
      const int t16 = 4 * g + (i >> 2);
      v_off0 = tile_slot(t16, (i >> 1) & 1) * 16 + 8 * (i & 1);      // even v-block
      v_off1 = tile_slot(t16, 2 + ((i >> 1) & 1)) * 16 + 8 * (i & 1);  // odd v-block
    }

    const int n_tiles = (te - ts + kTile - 1) / kTile;
    // this lane's row sees positions t < row_end (causal limit of its query
    // token; vis_n = n - q_len + 1 is the limit of token 0)
    const int row_end =
        vis_n + (h0 + (HPW == 32 ? (lane & 31) : (lane & 15))) / p.heads_per_token;
    // page cursor of the next 16-position half to load
    int cur_lb = ts / P;
    int cur_off = ts - cur_lb * P;
    int cur_tok = ts;
    // Block-table window: lane k holds the page of logical block win_lb + k.
    // One vector load per 64 pages; a page is then read with v_readlane.
    const int32_t* bt_row = p.block_table + (int64_t)b * p.bt_stride;
    const int lb_end = (te - 1) / P + 1;  // blocks this segment reads
    int win_lb = cur_lb;
    int win = 0;
    auto load_window = [&]() __attribute__((always_inline)) {
      const int k = win_lb + lane;
      win = k < lb_end ? bt_row[k] : 0;
    };
    if constexpr (!SP) load_window();

    // Sparse gather ("vLLM 中 Attention Kernel 如何并行处理多个请求", section
    // 十三: the request's top-k logical positions go through its block table
    // to physical slots).  Every lane loads the same row dma_t16 of each
    // 16-entry half of a tile, so per tile it needs two row offsets.  They
    // come from a per-lane pipeline: prepare(i) uses the pages of tile i
    // (loaded one tile earlier), loads the pages of tile i+1 from its
    // entries (loaded two tiles earlier) and loads the entries of tile i+2.
    // Entries past the segment get the offset pool_bytes, which the buffer
    // range check turns into zero rows.
    const int32_t* sp_list = SP ? p.topk_idx + (int64_t)b * p.topk_stride : nullptr;
    int spA0 = -1, spA1 = -1, spG0 = 0, spG1 = 0, spB0 = -1, spB1 = -1;
    // (positions outside [0, bt_stride * P) count as past the segment: zero rows)
    const uint32_t pos_cap = (uint32_t)min((int64_t)p.bt_stride * P, (int64_t)0x7fffffff);
    auto sp_entries = [&](int x, int& i0, int& i1) __attribute__((always_inline)) {
      const int e0 = ts + x * kTile + dma_t16;
      i0 = e0 < te ? sp_list[e0] : -1;
      i1 = e0 + 16 < te ? sp_list[e0 + 16] : -1;
      if ((uint32_t)i0 >= pos_cap) i0 = -1;
      if ((uint32_t)i1 >= pos_cap) i1 = -1;
    };
    auto sp_block = [&](int pos) __attribute__((always_inline)) {
      return p.page_shift >= 0 ? pos >> p.page_shift : pos / P;
    };
    auto sp_pages = [&](int i0, int i1, int& g0, int& g1) __attribute__((always_inline)) {
      g0 = i0 >= 0 ? bt_row[sp_block(i0)] : 0;
      g1 = i1 >= 0 ? bt_row[sp_block(i1)] : 0;
    };
    auto sp_offset = [&](int pos, int page) __attribute__((always_inline)) {
      return pos >= 0 && (uint32_t)page < p.num_blocks
                 ? ((uint32_t)page * (uint32_t)P + (uint32_t)(pos - sp_block(pos) * P)) *
                       (uint32_t)C::SRC_ROW
                 : p.pool_bytes;
    };
    if constexpr (SP) {
      sp_entries(0, spA0, spA1);
      sp_entries(1, spB0, spB1);
      sp_pages(spA0, spA1, spG0, spG1);
    }

    // Issue the loads of the next tile (ring slot i % NBUF).  Each 16-row
    // half lies in one page (P and 16-position boundaries are multiples of
    // 16); a buffer resource sized to the valid rows makes the loads of
    // positions past the segment return zeros, so those LDS rows hold zeros
    // and never the (possibly NaN) contents of unreferenced slots.
    struct TileLoad {  // plain fields: the buffer resources are built at each use
      uint64_t base[2];
      int bytes[2];
      uint32_t off[2];  // sparse: this lane's row offset in each half
      uint8_t* dst;
      int sslot;        // fp8: staging slot (per-token scales go to the same slot)
    };
    // Resources of the next tile to load (ring slot i % NBUF); advances the cursor.
    auto prepare = [&](int i) __attribute__((always_inline)) {
      TileLoad tl;
      tl.dst = F8 ? stg + (i & 1) * C::STG_TILE : ring + (i % NBUF) * C::TILE_BYTES;
      tl.sslot = i & 1;
      if constexpr (SP) {
        tl.off[0] = sp_offset(spA0, spG0);
        tl.off[1] = sp_offset(spA1, spG1);
        spA0 = spB0;
        spA1 = spB1;
        sp_pages(spA0, spA1, spG0, spG1);
        sp_entries(i + 2, spB0, spB1);
        return tl;
      }
#pragma unroll
      for (int th = 0; th < 2; ++th) {
        int nv = uniform(max(0, min(16, te - cur_tok)));
        uint64_t base = reinterpret_cast<uint64_t>(p.kv);
        if (nv > 0) {
          // The window load is read inside its own branch, so that the wait
          // for it stays there: a wait at the join would drain the ring.
          int64_t page;
          if (cur_lb - win_lb >= 64) {  // uniform: move the window (once per 64 pages)
            win_lb = cur_lb;
            load_window();
            page = __builtin_amdgcn_readlane(win, 0);
          } else {
            page = __builtin_amdgcn_readlane(win, cur_lb - win_lb);
          }
          // a page outside the pool reads as zero rows (an empty resource)
          if ((uint64_t)page < (uint64_t)p.num_blocks)
            base += (uint64_t)((page * P + cur_off) * (int64_t)C::SRC_ROW);
          else
            nv = 0;
        }
        // every field wave-uniform, so the resource lives in SGPRs
        base = ((uint64_t)(uint32_t)uniform((int)(base >> 32)) << 32) |
               (uint32_t)uniform((int)(uint32_t)base);
        tl.base[th] = base;
        tl.bytes[th] = nv * C::SRC_ROW;
        cur_tok += 16;
        cur_off += 16;
        if (cur_off == P) {
          cur_off = 0;
          ++cur_lb;
        }
      }
      return tl;
    };
    // The k-th of this wave's NIW copies of a prepared tile.  bf16: block j
    // of the tile layout, one 16-byte chunk per lane.  fp8: the r-th 64*G
    // bytes of a half tile into the row-major staging tile.
    auto dma = [&](const TileLoad& tl, int k) __attribute__((always_inline)) {
      const int j = wave + k * W;  // copy index
      if constexpr ((2 * C::NIH) % W != 0) {
        if (j >= 2 * C::NIH) return;  // (wave-uniform) this wave's share is done
      }
      const int th = j >= C::NIH ? 1 : 0;
      const int r = j - th * C::NIH;
      if constexpr (SP) {
        const __amdgpu_buffer_rsrc_t rs = __builtin_amdgcn_make_buffer_rsrc(
            (void*)p.kv, (short)0, (int)p.pool_bytes, 0x00020000);
        if constexpr (F8) {
          // 1-byte codes: the r-th 64*G bytes of half th go to the row-major
          // staging tile as in dense decode, but each row comes from its own
          // slot; lane 4t holds the offset of row t of the half
          // (dma_t16 = t there), read here with a lane shuffle
          const int c = C::G * lane + sgpr_here(r * 64 * C::G);  // code byte in the half
          const int row = c / C::CB;
          const uint32_t roff = (uint32_t)__shfl((int)(th ? tl.off[1] : tl.off[0]), 4 * row, 64);
          LDS_AS void* dst = (LDS_AS void*)(tl.dst + th * 16 * C::CB + r * 64 * C::G);
          const int voff = (int)(roff + (uint32_t)(c - row * C::CB));
          if constexpr (C::G == 16) __builtin_amdgcn_raw_ptr_buffer_load_lds(rs, dst, 16, voff, 0, 0, 0);
          else __builtin_amdgcn_raw_ptr_buffer_load_lds(rs, dst, 4, voff, 0, 0, 0);
          if constexpr (PT) {
            if (k == 0 && wave == 0) {
              // the 16 inline scales of each half: lane l < 16 reads row l's,
              // whose offset lane 4l holds (rows past the segment, and lanes
              // >= 16, read 0)
#pragma unroll
              for (int h2 = 0; h2 < 2; ++h2) {
                const uint32_t ro =
                    (uint32_t)__shfl((int)(h2 ? tl.off[1] : tl.off[0]), (4 * lane) & 63, 64);
                const int soff = lane < 16 ? (int)(ro + C::CB) : (int)p.pool_bytes;
                __builtin_amdgcn_raw_ptr_buffer_load_lds(
                    rs, (LDS_AS uint8_t*)ring + kSclOff + tl.sslot * 512 + h2 * 256, 4, soff,
                    0, 0, 0);
              }
            }
          }
        } else {
          __builtin_amdgcn_raw_ptr_buffer_load_lds(rs, (LDS_AS void*)(tl.dst + j * 1024), 16,
                                                   (int)((th ? tl.off[1] : tl.off[0]) +
                                                         16 * dma_c4) + sgpr_here(64 * r),
                                                   0, 0, 0);
        }
        return;
      }
      const __amdgpu_buffer_rsrc_t rs = __builtin_amdgcn_make_buffer_rsrc(
          (void*)(th ? tl.base[1] : tl.base[0]), (short)0, th ? tl.bytes[1] : tl.bytes[0],
          0x00020000);
      if constexpr (F8) {
        LDS_AS void* dst = (LDS_AS void*)(tl.dst + th * 16 * C::CB + r * 64 * C::G);
        int voff;
        if constexpr (PT) {
          // the codes of a half tile are contiguous in staging, but in the
          // cache each row is followed by its 16-byte scale pad
          // (formed here from an SGPR constant, not hoisted into a VGPR per copy)
          const uint32_t c = (uint32_t)(C::G * lane) + (uint32_t)sgpr_here(r * 64 * C::G);
          voff = (int)(c + (c / C::CB) * kPerTokenPad);  // c: code byte within the half tile
          if (k == 0 && wave == 0) {
            // the 16 inline scales of each half: lane l < 16 reads row l's
            // scale into slot l of a 256-byte area; rows past the segment
            // (and lanes >= 16) read as 0 through the range check
#pragma unroll
            for (int h2 = 0; h2 < 2; ++h2) {
              const __amdgpu_buffer_rsrc_t rsh = __builtin_amdgcn_make_buffer_rsrc(
                  (void*)tl.base[h2], (short)0, tl.bytes[h2], 0x00020000);
              const int soff = lane < 16 ? lane * C::SRC_ROW + C::CB : tl.bytes[h2];
              __builtin_amdgcn_raw_ptr_buffer_load_lds(
                  rsh, (LDS_AS uint8_t*)ring + kSclOff + tl.sslot * 512 + h2 * 256, 4, soff, 0, 0,
                  0);
            }
          }
        } else {
          voff = C::G * lane + sgpr_here(r * 64 * C::G);
        }
        // the size operand is spelled as a literal: given as a template
        // constant, the host pass drops the kernel's launch stub
        if constexpr (C::G == 16) __builtin_amdgcn_raw_ptr_buffer_load_lds(rs, dst, 16, voff, 0, 0, 0);
        else __builtin_amdgcn_raw_ptr_buffer_load_lds(rs, dst, 4, voff, 0, 0, 0);
      } else
        __builtin_amdgcn_raw_ptr_buffer_load_lds(rs, (LDS_AS void*)(tl.dst + j * 1024), 16,
                                                 dma_voff + sgpr_here(64 * r), 0, 0, 0);
    };
    auto issue = [&](int i) __attribute__((always_inline)) {
      const TileLoad tl = prepare(i);
#pragma unroll
      for (int k = 0; k < C::NIW; ++k) dma(tl, k);
    };
    // fp8: LDS addresses of the k-th of this wave's LPW widened blocks of
    // tile x (staging slot x % 2 -> ring slot x % NBUF)
    auto widen_src = [&](int x, int k) __attribute__((always_inline)) {
      const int j = wave + k * W;
      const int th = j >= C::NKQ ? 1 : 0;
      return cv_src + (uint32_t)sgpr_here((int)(uint32_t)(uintptr_t)stg + (x & 1) * C::STG_TILE +
                                          th * 16 * C::CB + 4 * C::CVB * (j - th * C::NKQ));
    };
    auto widen_dst = [&](int x, int k) __attribute__((always_inline)) {
      return cv_dst + (uint32_t)sgpr_here((int)(uint32_t)(uintptr_t)ring +
                                          (x % NBUF) * C::TILE_BYTES + (wave + k * W) * 1024);
    };
    // 8 code bytes per lane and block (4 for int4 codes): read, and the
    // widened 8 bf16 written to the block's slot of the bf16 tile
    using WRaw = std::conditional_t<PT == 3, uint32_t, u32x2>;
    auto widen_read = [&](int x, int k) __attribute__((always_inline)) {
      if constexpr (PT == 3) return ds_read_b32_asm(widen_src(x, k));
      else return ds_read_b64_asm(widen_src(x, k));
    };
    auto widen_write = [&](int x, int k, WRaw v) __attribute__((always_inline)) {
      if constexpr (PT == 3)
        ds_write_b128_asm(widen_dst(x, k), i4x8_to_bf16x8(v));
      else
        ds_write_b128_asm(widen_dst(x, k), PT == 2 ? i8x8_to_bf16x8(v) : e4m3x8_to_bf16x8(v));
    };
    // widen all of this wave's blocks of tile x, four reads in flight
    auto widen_blocks = [&](int x) __attribute__((always_inline)) {
      static_for<(C::LPW + 3) / 4>([&](auto bc) __attribute__((always_inline)) {
        constexpr int k0 = 4 * decltype(bc)::value;
        constexpr int nb = C::LPW - k0 < 4 ? C::LPW - k0 : 4;
        WRaw v[nb];
        static_for<nb>([&](auto ic) __attribute__((always_inline)) {
          v[decltype(ic)::value] = widen_read(x, k0 + decltype(ic)::value);
        });
        static_for<nb>([&](auto ic) __attribute__((always_inline)) {
          constexpr int i = decltype(ic)::value;
          // issued after read i: the other nb-1-i reads and i writes
          lds_wait<nb - 1>(v[i]);
          widen_write(x, k0 + i, v[i]);
        });
      });
    };
    // the tile's per-token scales (per-token caches)
    auto widen_scales = [&](int x) __attribute__((always_inline)) {
      if constexpr (PT) {
        // the tile's 32 token scales: staging slot x % 2 (two 256-byte
        // halves, row l of a half at float l) -> ring slot x % NBUF (float t),
        // and their reciprocals 128 bytes further (0 where the scale is 0,
        // subnormal or not finite)
        if (wave == 0 && lane < 32) {
          uint32_t sc = ds_read_b32_asm(scl_stage + (x & 1) * 512 + (lane >> 4) * 256 +
                                        (lane & 15) * 4);
          lds_wait<0>(sc);
          const float s = __uint_as_float(sc);
          const float as = __builtin_fabsf(s);
          const float inv = (as >= 0x1p-126f && as <= 0x1.fffffep127f) ? 1.f / s : 0.f;
          ds_write_b32_asm(scl_ring + (x % NBUF) * 256 + lane * 4, sc);
          ds_write_b32_asm(scl_ring + (x % NBUF) * 256 + 128 + lane * 4, __float_as_uint(inv));
        }
      }
    };
    auto widen_tile = [&](int x) __attribute__((always_inline)) {
      widen_blocks(x);
      widen_scales(x);
    };
    // per-token scales of the four consecutive positions t .. t+3 of ring
    // tile x, and their reciprocals
    auto token_scales4 = [&](int x, int t) __attribute__((always_inline)) {
      return ds_read_b128_asm(scl_ring + (x % NBUF) * 256 + t * 4);
    };
    auto token_inv4 = [&](int x, int t) __attribute__((always_inline)) {
      return ds_read_b128_asm(scl_ring + (x % NBUF) * 256 + 128 + t * 4);
    };

    // Q fragments of this wave's heads (B operand of S^T = K Q^T): the first
    // NQR k-steps in VGPRs, the rest in this wave's LDS region (lane-linear).
    // With 32-head waves the LDS part is held in registers until the first
    // tiles' loads are issued, so that the query, the block-table window and
    // the first tiles are all in flight together (one memory latency at the
    // start of a segment, not two).
    constexpr bool kEarlyRing = HPW == 32;
    if constexpr (!C::PIPE) {
      // Drain this wave's stores and loads of a previous segment once, so
      // that no wait for them lands between the loads below, then make sure
      // every wave is done with the ring of that segment.
      wait_vmcnt<0>();
      __builtin_amdgcn_s_barrier();
    }
    bf16x8 qf[C::NQR];
    bf16x8 qtmp[kEarlyRing ? (C::QLDS > 0 ? C::QLDS : 1) : 1];
    LDS_AS uint8_t* qlds =
        (LDS_AS uint8_t*)ring + NBUF * C::TILE_BYTES + C::STG_BYTES + wave * C::QLDS * 1024;
    {
      // this lane's row of q: columns d < D_v from q_nope, the rest from q_pe
      const int qrow = h0 + (HPW == 32 ? (lane & 31) : (lane & 15));
      const int dl = HPW == 32 ? 8 * (lane >> 5) : 8 * (lane >> 4);
      const __bf16* qn = p.q_nope + (int64_t)b * p.qn_seq + (int64_t)qrow * p.qn_row + dl;
      const __bf16* qp = p.q_pe + (int64_t)b * p.qp_seq + (int64_t)qrow * p.qp_row + dl;
      constexpr int KW = HPW == 32 ? 16 : 32;  // columns per k-step
      auto qchunk = [&](int ks) __attribute__((always_inline)) {
        return ks * KW < DV ? *reinterpret_cast<const bf16x8*>(qn + ks * KW)
                            : *reinterpret_cast<const bf16x8*>(qp + (ks * KW - DV));
      };
      static_assert(DV % 32 == 0, "a k-step never straddles q_nope and q_pe");
      if constexpr (HPW == 32) {
#pragma unroll
        for (int ks = 0; ks < C::NQR; ++ks) qf[ks] = qchunk(ks);
#pragma unroll
        for (int ks = C::NQR; ks < C::NKS; ++ks) {
          if constexpr (kEarlyRing)
            qtmp[ks - C::NQR] = qchunk(ks);
          else
            *reinterpret_cast<LDS_AS bf16x8*>(qlds + (ks - C::NQR) * 1024 + lane * 16) =
                qchunk(ks);
        }
      } else {
#pragma unroll
        for (int ks = 0; ks < C::NKS; ++ks) qf[ks] = qchunk(ks);
      }
    }

    float m_run = -INFINITY;  // running max (log2 units) used for the exponentials
    float l_part = 0.f;       // this lane's share of sum_t p_t (fp32 weights): for lse
    float lr_part = 0.f;      // the same over the bf16-rounded weights: normalises o
    typedef typename std::conditional<HPW == 32, f32x16, f32x4>::type acc_t;
    acc_t oacc[C::NVB];
    {
      // zeros from an opaque register: a constant zero vector would be kept
      // kernel-wide (and spilled) rather than rematerialised per segment
      const float zero = __uint_as_float((uint32_t)vgpr_here(0));
      acc_t z;
#pragma unroll
      for (int r = 0; r < (int)(sizeof(acc_t) / sizeof(float)); ++r) z[r] = zero;
#pragma unroll
      for (int vb = 0; vb < C::NVB; ++vb) oacc[vb] = z;
    }

    if constexpr (C::PIPE) {
      // ---- software-pipelined loop (bf16, 32-head waves, ring of 4: the
      // D = 320 shapes).  Iteration j runs the softmax of tile j interleaved
      // with the QK^T MFMAs of tile j+1, then the PV MFMAs of tile j.  The
      // ring holds tiles j (V) and j+1 (K); the loads of tile j+NBUF-1 go
      // straight into the ring, spread over the MFMA steps, with NBUF-2 tiles
      // in flight.  Past the segment, loads are issued with an empty resource
      // (they write zeros into a free slot), so every iteration issues the
      // same number of loads and the waits are constants.  (Measured on the
      // D = 576 shapes, bf16 and fp8, the plain loop below is faster.)
      static_assert(!F8, "1-byte caches take the plain loop");
      constexpr int AHEAD = NBUF - 1;  // tile whose loads iteration j issues: j + AHEAD
      // every wave is done with the ring of a previous segment; the first
      // tiles go out behind the query loads, then the query's LDS part is
      // stored (asm: no compiler wait for the ring loads it cannot alias)
      __builtin_amdgcn_s_barrier();
#pragma unroll
      for (int i = 0; i < NBUF - 1; ++i) issue(i);
#pragma unroll
      for (int k = 0; k < C::QLDS; ++k)
        ds_write_b128_asm((uint32_t)(uintptr_t)(qlds + k * 1024 + lane * 16),
                          __builtin_bit_cast(u32x4, qtmp[k]));
      wait_vmcnt<(NBUF - 2) * C::LPW>();
      __builtin_amdgcn_s_waitcnt(0xc07f);  // lgkmcnt(0): the query's LDS part is written
      __builtin_amdgcn_s_barrier();

      auto kread = [&](const LDS_AS uint8_t* t, int ks) __attribute__((always_inline)) {
        return *reinterpret_cast<const LDS_AS bf16x8*>(t + (ks >> 1) * 1024 +
                                                       ((ks & 1) ? qk_off_o : qk_off_e));
      };
      auto qread = [&](int ks) __attribute__((always_inline)) {
        return *reinterpret_cast<const LDS_AS bf16x8*>(qlds + (ks - C::NQR) * 1024 + lane * 16);
      };
      // S^T of one tile on two accumulator chains (even / odd k-steps, summed
      // by the softmax); hook(k-step) runs right after each MFMA is issued.
      struct S2 {
        f32x16 e, o;
      };
      auto qk = [&](const LDS_AS uint8_t* t, auto&& hook) __attribute__((always_inline)) {
        f32x16 se = {}, so = {};
        bf16x8 k0 = kread(t, 0), k1 = kread(t, 1);
        bf16x8 q0 = {}, q1 = {};
        if constexpr (C::NQR == 0) q0 = qread(0);
        if constexpr (C::NQR <= 1) q1 = qread(1);
        static_for<C::NKS>([&](auto ksc) __attribute__((always_inline)) {
          constexpr int ks = decltype(ksc)::value;
          bf16x8 k2 = k1, q2 = q1;
          if constexpr (ks + 2 < C::NKS) {
            k2 = kread(t, ks + 2);
            if constexpr (ks + 2 >= C::NQR) q2 = qread(ks + 2);
          }
          bf16x8 qv;
          if constexpr (ks < C::NQR) qv = qf[ks];
          else qv = q0;
          if constexpr (ks & 1) so = __builtin_amdgcn_mfma_f32_32x32x16_bf16(k0, qv, so, 0, 0, 0);
          else se = __builtin_amdgcn_mfma_f32_32x32x16_bf16(k0, qv, se, 0, 0, 0);
          hook(ksc);
          __builtin_amdgcn_sched_barrier(0);
          k0 = k1;
          k1 = k2;
          q0 = q1;
          q1 = q2;
        });
        return S2{se, so};
      };
      auto no_hook = [&](auto) __attribute__((always_inline)) {};

      f32x16 s_cur;  // scores of the tile whose softmax runs next
      {
        const S2 s0 = qk((const LDS_AS uint8_t*)ring, no_hook);  // S^T of tile 0
        s_cur = s0.e + s0.o;
      }
      for (int j = 0; j < n_tiles; ++j) {
        // tile j+1 is in the ring for every wave; tile j-1's slot is free
        wait_vmcnt<(NBUF - 3) * C::LPW>();
        __builtin_amdgcn_s_barrier();
        const LDS_AS uint8_t* tcur = (const LDS_AS uint8_t*)ring + (j % NBUF) * C::TILE_BYTES;
        const LDS_AS uint8_t* tnext =
            (const LDS_AS uint8_t*)ring + ((j + 1) % NBUF) * C::TILE_BYTES;
        const int nvalid = min(kTile, te - (ts + j * kTile));
        const TileLoad tl = prepare(j + AHEAD);

        float mt = -INFINITY, alpha = 1.f, m_exp = 0.f;
        bool rescale = false;
        bf16x8 p0, p1;
        f32x16& sv = s_cur;  // scores of tile j, turned into weights in place
        // Softmax of tile j, spread over the QK^T steps of tile j+1 at a few
        // VALU instructions per MFMA, so that the matrix core stays fed:
        //   0-3        running row max
        //   4          mask past the segment (last tile only)
        //   5          max across the two half-waves, new running max, rescale test
        //   6 .. 6+E   the 16 weights: exp2, sums, bf16 packing of each pair
        //   .. +L      sum of the bf16 weights (normalises o)
        constexpr int E = C::NKS - 8 < 16 ? C::NKS - 8 : 16;
        constexpr int L = C::NKS - 6 - E < 8 ? C::NKS - 6 - E : 8;
        static_assert(E >= 1 && L >= 1, "too few QK^T steps to hide the softmax");
        auto hook = [&](auto ksc) __attribute__((always_inline)) {
          constexpr int ks = decltype(ksc)::value;
          // the loads of tile j+NBUF-1, spread evenly over the QK^T and PV steps
          static_for<C::NIW>([&](auto kc) __attribute__((always_inline)) {
            if constexpr (C::dma_step(decltype(kc)::value) == ks) dma(tl, decltype(kc)::value);
          });
          if constexpr (ks < 4) {
            mt = fmaxf(mt, fmaxf(fmaxf(sv[4 * ks], sv[4 * ks + 1]), fmaxf(sv[4 * ks + 2], sv[4 * ks + 3])));
          } else if constexpr (ks == 4) {
            // position of sv[r] is 8*(r/4) + 4*(lane/32) + r%4; mask past the
            // segment and past the row's causal limit (multi-token decode)
            const int t0 = ts + j * kTile;
            if (nvalid < kTile || t0 + kTile > vis_n) {
              const int lim = min(nvalid, row_end - t0);
              mt = -INFINITY;
#pragma unroll
              for (int r = 0; r < 16; ++r) {
                const int t = 8 * (r >> 2) + 4 * (lane >> 5) + (r & 3);
                if (t >= lim) sv[r] = -INFINITY;
                mt = fmaxf(mt, sv[r]);
              }
            }
          } else if constexpr (ks == 5) {
            mt = max_halves(mt) * p.score_log2;
            const float m_new = fmaxf(m_run, mt);
            // the accumulator rescale itself waits until after the QK^T
            // stream (PV of this tile comes after it)
            if (j == 0) {
              m_run = m_new;  // nothing accumulated yet: no rescale
            } else if (__builtin_amdgcn_ballot_w64(m_new > m_run + kTau)) {
              // a row that has seen no position yet has nothing to rescale
              alpha = m_run == -INFINITY ? 0.f : __builtin_amdgcn_exp2f(m_run - m_new);
              rescale = true;
              m_run = m_new;
              l_part *= alpha;
              lr_part *= alpha;
            }
            // exponent base: a row with no visible position yet (m = -inf)
            // takes 0, so its masked scores give weight 0, not NaN
            m_exp = m_run == -INFINITY ? 0.f : m_run;
          } else {
            static_for<16>([&](auto rc) __attribute__((always_inline)) {
              constexpr int r = decltype(rc)::value;
              if constexpr (6 + r * E / 16 == ks) {
                sv[r] = __builtin_amdgcn_exp2f(__builtin_fmaf(sv[r], p.score_log2, -m_exp));
                l_part += sv[r];
                if constexpr (r & 1) {
                  const bf16x2 pk = __builtin_convertvector((f32x2){sv[r - 1], sv[r]}, bf16x2);
                  if constexpr (r < 8) {
                    p0[r - 1] = pk[0];
                    p0[r] = pk[1];
                  } else {
                    p1[r - 9] = pk[0];
                    p1[r - 8] = pk[1];
                  }
                }
              }
            });
            // the sum that normalises o adds the bf16 weights the MFMA uses,
            // so o is an exact convex combination of V rows with them
            static_for<8>([&](auto qc) __attribute__((always_inline)) {
              constexpr int q = decltype(qc)::value;
              if constexpr (6 + E + q * L / 8 == ks) {
                const bf16x8& pp = q < 4 ? p0 : p1;
                lr_part += (float)pp[(2 * q) & 7] + (float)pp[((2 * q) & 7) + 1];
              }
            });
          }
        };
        // QK^T of tile j+1 runs unconditionally: on the segment's last tile it
        // reads the zero-filled slot past the end and its scores are never
        // used.  A branch here would make the compiler zero the score
        // accumulators explicitly every tile instead of starting the chains
        // from an inline zero.
        const S2 s_next = qk(tnext, hook);
        if (rescale) {  // uniform, rare: the running max moved by more than kTau
#pragma unroll
          for (int vb = 0; vb < C::NVB; ++vb) scale_acc(oacc[vb], alpha);
        }

        // ---- O^T[v, head] += V^T P^T of tile j; k-half outer so that
        // consecutive MFMAs accumulate into different blocks
        {
          const uint32_t vbase0 = (uint32_t)(uintptr_t)tcur + v_off0;
          const uint32_t vbase1 = (uint32_t)(uintptr_t)tcur + v_off1;
          constexpr int NST = 2 * C::NVB;
          auto vread = [&](auto stc) __attribute__((always_inline)) {
            constexpr int st = decltype(stc)::value;
            constexpr int kk = st / C::NVB, vb = st % C::NVB;
            constexpr int off = (kk * C::NKQ + vb) * 1024;
            const u32x2 lo = ds_read_tr16_asm<off>(vbase0);
            const u32x2 hi = ds_read_tr16_asm<off>(vbase1);
            return u32x4{lo[0], lo[1], hi[0], hi[1]};
          };
          u32x4 a0 = vread(std::integral_constant<int, 0>{});
          u32x4 a1 = vread(std::integral_constant<int, 1>{});
          u32x4 a2 = vread(std::integral_constant<int, 2>{});
          static_for<NST>([&](auto stc) __attribute__((always_inline)) {
            constexpr int st = decltype(stc)::value;
            constexpr int kk = st / C::NVB, vb = st % C::NVB;
            u32x4 a3 = a2;
            if constexpr (st + 3 < NST) a3 = vread(std::integral_constant<int, st + 3>{});
            lds_wait<pv_reads_after<NST>(st)>(a0);
            oacc[vb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, a0),
                                                              kk ? p1 : p0, oacc[vb], 0, 0, 0);
            // scores of tile j+1: sum of its two QK^T chains
            if constexpr (st < 4) {
#pragma unroll
              for (int r = 4 * st; r < 4 * st + 4; ++r) s_cur[r] = s_next.e[r] + s_next.o[r];
            }
            // the rest of the loads of tile j+NBUF-1
            static_for<C::NIW>([&](auto kc) __attribute__((always_inline)) {
              if constexpr (C::dma_step(decltype(kc)::value) == C::NKS + st)
                dma(tl, decltype(kc)::value);
            });
            __builtin_amdgcn_sched_barrier(0);
            a0 = a1;
            a1 = a2;
            a2 = a3;
          });
        }
      }
    } else {
    // The first tiles go out behind the query loads; then the query's LDS
    // part is stored (asm: the compiler waits for the query registers it
    // reads, which are older than the ring loads, and for nothing else).
    // fp8 (ring of 2): iteration i loads tile i+2 into staging slot i % 2
    // over its QK^T MFMAs and widens tile i+1 into ring slot (i+1) % 2 at
    // its end; the barrier at the top of iteration i+1 publishes both.
    auto store_qlds = [&]() __attribute__((always_inline)) {
      if constexpr (kEarlyRing) {
#pragma unroll
        for (int k = 0; k < C::QLDS; ++k)
          ds_write_b128_asm((uint32_t)(uintptr_t)(qlds + k * 1024 + lane * 16),
                            __builtin_bit_cast(u32x4, qtmp[k]));
      }
    };
    if constexpr (F8) {
      issue(0);
      issue(1);
      store_qlds();
      wait_vmcnt<0>();
      __builtin_amdgcn_s_barrier();  // staging tiles 0 and 1 complete
      widen_tile(0);
    } else {
#pragma unroll
      for (int i = 0; i < NBUF - 1; ++i)
        if (i < n_tiles) issue(i);
      store_qlds();
    }

    for (int i = 0; i < n_tiles; ++i) {
      if constexpr (F8) {
        wait_vmcnt<0>();
      } else {
        const int ahead = min(NBUF - 2, n_tiles - 1 - i);
        if (ahead >= 2) wait_vmcnt<(NBUF >= 4 ? 2 : 0) * C::LPW>();
        else if (ahead == 1) wait_vmcnt<(NBUF >= 3 ? 1 : 0) * C::LPW>();
        else wait_vmcnt<0>();
      }
      __builtin_amdgcn_s_barrier();
      // The next tile's loads are spread over this tile's QK^T MFMAs: each
      // load instruction can hold the wave at issue while the vector-memory
      // queue drains, which the matrix core then overlaps.
      const bool more = F8 || i + NBUF - 1 < n_tiles;
      TileLoad tl;
      if (more) tl = prepare(F8 ? i + 2 : i + NBUF - 1);
      // Load k goes after step floor(k * TOT / NIW) of the tile's TOT MFMA
      // steps.  bf16, 32-head waves: the QK^T and the PV steps (the loaded
      // tile is not read before iteration i+NBUF-1, so the loads may be
      // spread over the whole iteration and leave the memory pipeline at
      // about the rate it drains instead of blocking the wave in a burst).
      // fp8 and 16-head waves: the QK^T steps only (an fp8 staging tile is
      // waited for at the top of the next iteration, so it lands during PV).
      constexpr int TOT_STEPS = (HPW == 32 && !F8) ? C::NKS + 2 * C::NVB : C::NKS;
      auto dma_at = [&](int step) __attribute__((always_inline)) {
#pragma unroll
        for (int k = 0; k < C::NIW; ++k)
          if ((k * TOT_STEPS) / C::NIW == step && more) dma(tl, k);
      };

      const LDS_AS uint8_t* tile = (const LDS_AS uint8_t*)ring + (i % NBUF) * C::TILE_BYTES;
      const int nvalid = min(kTile, te - (ts + i * kTile));

      if constexpr (HPW == 32) {
        // ---- S^T[32 positions, 32 heads] over D
        f32x16 s = {};
        {
          auto kread = [&](int ks) __attribute__((always_inline)) {
            return *reinterpret_cast<const LDS_AS bf16x8*>(
                tile + (ks >> 1) * 1024 + ((ks & 1) ? qk_off_o : qk_off_e));
          };
          auto qread = [&](int ks) __attribute__((always_inline)) {
            return *reinterpret_cast<const LDS_AS bf16x8*>(qlds + (ks - C::NQR) * 1024 +
                                                           lane * 16);
          };
          // software pipeline: the K chunk (and LDS Q fragment) of step ks+2
          // is in flight while step ks runs on the matrix core
          bf16x8 k0 = kread(0), k1 = kread(1);
          bf16x8 q0 = {}, q1 = {};
          if (C::NQR == 0) q0 = qread(0);
          if (C::NQR <= 1) q1 = qread(1);
          // (compile-time k-steps: Q fragments stay in registers)
          static_for<C::NKS>([&](auto ksc) __attribute__((always_inline)) {
            constexpr int ks = decltype(ksc)::value;
            bf16x8 k2 = k1, q2 = q1;
            if constexpr (ks + 2 < C::NKS) {
              k2 = kread(ks + 2);
              if constexpr (ks + 2 >= C::NQR) q2 = qread(ks + 2);
            }
            bf16x8 qv;
            if constexpr (ks < C::NQR) qv = qf[ks];
            else qv = q0;
            s = __builtin_amdgcn_mfma_f32_32x32x16_bf16(k0, qv, s, 0, 0, 0);
            dma_at(ks);
            __builtin_amdgcn_sched_barrier(0);
            k0 = k1;
            k1 = k2;
            q0 = q1;
            q1 = q2;
          });
        }
        // position of s[r] is 8*(r/4) + 4*(lane/32) + r%4.  Per-token caches:
        // scores and PV weights are multiplied by the scales of those
        // positions (read twice from LDS rather than held in 16 registers)
        auto scale_by_tokens = [&](f32x16& x) __attribute__((always_inline)) {
          u32x4 g[4];
#pragma unroll
          for (int q = 0; q < 4; ++q) g[q] = token_scales4(i, 8 * q + 4 * (lane >> 5));
          static_for<4>([&](auto qc) __attribute__((always_inline)) {
            constexpr int q = decltype(qc)::value;
            lds_wait<3 - q>(g[q]);
#pragma unroll
            for (int r = 0; r < 4; ++r) x[4 * q + r] *= __uint_as_float(g[q][r]);
          });
        };
        // Per-token caches: P V takes the weights w_t = bf16(p_t * scale_t)
        // (x holds p_t on entry and w_t on return).  o is normalised by the
        // sum of w_t / scale_t, formed as p_t + (w_t - p_t * scale_t) / scale_t,
        // which is p_t itself where the scale is 0: o is then an exact convex
        // combination of the cache rows with the weights the MFMA uses.
        auto pt_weights = [&](f32x16& x) __attribute__((always_inline)) {
          const int tl = 4 * (lane >> 5);
          u32x4 g[4], h[4];
          g[0] = token_scales4(i, tl);
          h[0] = token_inv4(i, tl);
          g[1] = token_scales4(i, 8 + tl);
          h[1] = token_inv4(i, 8 + tl);
          f32x4 racc = {};
          static_for<4>([&](auto qc) __attribute__((always_inline)) {
            constexpr int q = decltype(qc)::value;
            // LDS reads complete in order: after h[q] only the pair of q + 1 is
            // outstanding (none after the last pair)
            lds_wait<q < 3 ? 2 : 0>(g[q]);
            lds_wait<q < 3 ? 2 : 0>(h[q]);
            f32x4 pv, sv, iv;
#pragma unroll
            for (int r = 0; r < 4; ++r) {
              pv[r] = x[4 * q + r];
              sv[r] = __uint_as_float(g[q][r]);
              iv[r] = __uint_as_float(h[q][r]);
            }
            const f32x4 pw = pv * sv;
            const f32x4 wq = __builtin_convertvector(__builtin_convertvector(pw, bf16x4), f32x4);
#pragma unroll
            for (int r = 0; r < 4; ++r) {
              racc[r] += __builtin_fmaf(wq[r] - pw[r], iv[r], pv[r]);
              x[4 * q + r] = wq[r];
            }
            if constexpr (q + 2 < 4) {
              g[q + 2] = token_scales4(i, 8 * (q + 2) + tl);
              h[q + 2] = token_inv4(i, 8 * (q + 2) + tl);
            }
          });
          lr_part += (racc[0] + racc[1]) + (racc[2] + racc[3]);
        };
        if constexpr (PT) scale_by_tokens(s);  // before the mask: zero rows have scale 0
        // mask past the segment and past the row's causal limit (multi-token decode)
        const int t0 = ts + i * kTile;
        if (nvalid < kTile || t0 + kTile > vis_n) {
          const int lim = min(nvalid, row_end - t0);
#pragma unroll
          for (int r = 0; r < 16; ++r) {
            const int t = 8 * (r >> 2) + 4 * (lane >> 5) + (r & 3);
            if (t >= lim) s[r] = -INFINITY;
          }
        }
        float mt = s[0];
#pragma unroll
        for (int r = 1; r < 16; ++r) mt = fmaxf(mt, s[r]);
        mt = max_halves(mt) * p.score_log2;
        const float m_new = fmaxf(m_run, mt);
        if (i == 0) {
          m_run = m_new;  // nothing accumulated yet: no rescale
        } else if (__builtin_amdgcn_ballot_w64(m_new > m_run + kTau)) {
          const float alpha = m_run == -INFINITY ? 0.f : __builtin_amdgcn_exp2f(m_run - m_new);
          m_run = m_new;
          l_part *= alpha;
          lr_part *= alpha;
#pragma unroll
          for (int vb = 0; vb < C::NVB; ++vb) scale_acc(oacc[vb], alpha);
        }
        const float m_exp = m_run == -INFINITY ? 0.f : m_run;  // rows with no visible position
        f32x16 pr;
#pragma unroll
        for (int r = 0; r < 16; ++r)
          pr[r] = __builtin_amdgcn_exp2f(__builtin_fmaf(s[r], p.score_log2, -m_exp));
        {
          const f32x8 a = (f32x8){pr[0], pr[1], pr[2], pr[3], pr[4], pr[5], pr[6], pr[7]} +
                          (f32x8){pr[8], pr[9], pr[10], pr[11], pr[12], pr[13], pr[14], pr[15]};
          l_part += ((a[0] + a[1]) + (a[2] + a[3])) + ((a[4] + a[5]) + (a[6] + a[7]));
        }
        if constexpr (PT) pt_weights(pr);
        const bf16x8 p0 = __builtin_convertvector(
            (f32x8){pr[0], pr[1], pr[2], pr[3], pr[4], pr[5], pr[6], pr[7]}, bf16x8);
        const bf16x8 p1 = __builtin_convertvector(
            (f32x8){pr[8], pr[9], pr[10], pr[11], pr[12], pr[13], pr[14], pr[15]}, bf16x8);
        // the running sum that normalises o adds the bf16 weights the MFMA
        // uses, so o is an exact convex combination of V rows with them
        if constexpr (!PT) {
          const f32x8 r01 = __builtin_convertvector(p0, f32x8) + __builtin_convertvector(p1, f32x8);
          lr_part += ((r01[0] + r01[1]) + (r01[2] + r01[3])) + ((r01[4] + r01[5]) + (r01[6] + r01[7]));
        }
        // ---- O^T[v, head] += V^T P^T, V = leading DV columns of the tile
        {
          const uint32_t vbase0 = (uint32_t)(uintptr_t)tile + v_off0;
          const uint32_t vbase1 = (uint32_t)(uintptr_t)tile + v_off1;
          constexpr int NST = 2 * C::NVB;
          // fragment of step st: positions 16*(st/NVB) .. +15 of v-block st%NVB
          // (the half of the positions outer: 16 consecutive MFMAs share one
          // weight operand and write 16 different accumulators)
          auto vread = [&](auto stc) __attribute__((always_inline)) {
            constexpr int st = decltype(stc)::value;
            constexpr int off = ((st / C::NVB) * C::NKQ + st % C::NVB) * 1024;
            const u32x2 lo = ds_read_tr16_asm<off>(vbase0);
            const u32x2 hi = ds_read_tr16_asm<off>(vbase1);
            return u32x4{lo[0], lo[1], hi[0], hi[1]};
          };
          // 1-byte caches: the widening of tile i+1 rides along with these
          // MFMAs instead of following them (its staging tile is complete
          // and its ring slot free since the barrier at the top of this
          // iteration).  Block k of the wave is read after step 3k and
          // widened and written after step 3k+2: one LDS read, four
          // conversions and one LDS write per three MFMAs.
          constexpr bool kWidenHere = F8 && 3 * C::LPW <= NST;
          // LDS operations after the MFMA of step s: the write of block
          // (s-2)/3 and the read of block s/3
          constexpr auto wops = [](int s) constexpr {
            return kWidenHere ? ((s % 3 == 2 && s / 3 < C::LPW) ? 1 : 0) +
                                    ((s % 3 == 0 && s / 3 < C::LPW) ? 1 : 0)
                              : 0;
          };
          constexpr auto pairs = [](int s) constexpr { return s < NST ? 2 : 0; };
          WRaw wv[kWidenHere ? C::LPW : 1];
          u32x4 a0 = vread(std::integral_constant<int, 0>{});
          u32x4 a1 = vread(std::integral_constant<int, 1>{});
          static_for<NST>([&](auto stc) __attribute__((always_inline)) {
            constexpr int st = decltype(stc)::value;
            u32x4 a2 = a1;
            if constexpr (st + 2 < NST) a2 = vread(std::integral_constant<int, st + 2>{});
            // LDS operations issued after step st's pair: the pairs of steps
            // st+1 and st+2 and the widening's operations in between
            constexpr int later = st == 0   ? pairs(1) + pairs(2)
                                  : st == 1 ? pairs(2) + wops(0) + pairs(3)
                                            : wops(st - 2) + pairs(st + 1) + wops(st - 1) +
                                                  pairs(st + 2);
            lds_wait<later>(a0);
            oacc[st % C::NVB] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(
                __builtin_bit_cast(bf16x8, a0), st < C::NVB ? p0 : p1, oacc[st % C::NVB], 0, 0, 0);
            dma_at(C::NKS + st);
            if constexpr (kWidenHere) {
              if constexpr (st % 3 == 2 && st / 3 < C::LPW) {
                constexpr int k = st / 3;
                // issued after block k's read: the pairs of steps 3k+3, 3k+4
                lds_wait<pairs(3 * k + 3) + pairs(3 * k + 4)>(wv[k]);
                widen_write(i + 1, k, wv[k]);
              }
              if constexpr (st % 3 == 0 && st / 3 < C::LPW) wv[st / 3] = widen_read(i + 1, st / 3);
            }
            __builtin_amdgcn_sched_barrier(0);
            a0 = a1;
            a1 = a2;
          });
          if constexpr (kWidenHere) widen_scales(i + 1);
          else if constexpr (F8) widen_tile(i + 1);
        }
      } else {
        // ---- S^T over two 16-position halves x 16 heads
        f32x4 s0 = {}, s1 = {};
        static_for<C::NKS>([&](auto ksc) __attribute__((always_inline)) {
          constexpr int ks = decltype(ksc)::value;
          const bf16x8 k0 = *reinterpret_cast<const LDS_AS bf16x8*>(tile + ks * 1024 + qk_off_e);
          const bf16x8 k1 = *reinterpret_cast<const LDS_AS bf16x8*>(
              tile + (C::NKQ + ks) * 1024 + qk_off_e);
          s0 = __builtin_amdgcn_mfma_f32_16x16x32_bf16(k0, qf[ks], s0, 0, 0, 0);
          s1 = __builtin_amdgcn_mfma_f32_16x16x32_bf16(k1, qf[ks], s1, 0, 0, 0);
          dma_at(ks);
        });
        // position of s_th[r] is 16*th + 4*(lane/16) + r
        f32x8 tsc;  // per-token caches: the scale of each of those positions
        if constexpr (PT) {
          u32x4 g0 = token_scales4(i, 4 * (lane >> 4));
          u32x4 g1 = token_scales4(i, 16 + 4 * (lane >> 4));
          lds_wait<0>(g1);
          lds_wait<0>(g0);
#pragma unroll
          for (int r = 0; r < 4; ++r) {
            tsc[r] = __uint_as_float(g0[r]);
            tsc[4 + r] = __uint_as_float(g1[r]);
            s0[r] *= tsc[r];  // before the mask: zero rows have scale 0
            s1[r] *= tsc[4 + r];
          }
        }
        // mask past the segment and past the row's causal limit (multi-token decode)
        const int t0 = ts + i * kTile;
        if (nvalid < kTile || t0 + kTile > vis_n) {
          const int lim = min(nvalid, row_end - t0);
#pragma unroll
          for (int r = 0; r < 4; ++r) {
            const int t = 4 * (lane >> 4) + r;
            if (t >= lim) s0[r] = -INFINITY;
            if (t + 16 >= lim) s1[r] = -INFINITY;
          }
        }
        float mt = fmaxf(fmaxf(fmaxf(s0[0], s0[1]), fmaxf(s0[2], s0[3])),
                         fmaxf(fmaxf(s1[0], s1[1]), fmaxf(s1[2], s1[3])));
        mt = wave_max_xor(mt, 16);
        mt = max_halves(mt) * p.score_log2;
        const float m_new = fmaxf(m_run, mt);
        if (i == 0) {
          m_run = m_new;
        } else if (__builtin_amdgcn_ballot_w64(m_new > m_run + kTau)) {
          const float alpha = m_run == -INFINITY ? 0.f : __builtin_amdgcn_exp2f(m_run - m_new);
          m_run = m_new;
          l_part *= alpha;
          lr_part *= alpha;
#pragma unroll
          for (int vb = 0; vb < C::NVB; ++vb) scale_acc(oacc[vb], alpha);
        }
        const float m_exp = m_run == -INFINITY ? 0.f : m_run;  // rows with no visible position
        f32x8 pr;
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          pr[r] = __builtin_amdgcn_exp2f(__builtin_fmaf(s0[r], p.score_log2, -m_exp));
          pr[4 + r] = __builtin_amdgcn_exp2f(__builtin_fmaf(s1[r], p.score_log2, -m_exp));
        }
        l_part += ((pr[0] + pr[1]) + (pr[2] + pr[3])) + ((pr[4] + pr[5]) + (pr[6] + pr[7]));
        if constexpr (PT) {
          // per-token caches: weights w_t = bf16(p_t * scale_t); o is
          // normalised by the sum of p_t + (w_t - p_t * scale_t) / scale_t
          // (= w_t / scale_t, and p_t where the scale is 0), as in 32-head waves
          u32x4 h0 = token_inv4(i, 4 * (lane >> 4));
          u32x4 h1 = token_inv4(i, 16 + 4 * (lane >> 4));
          lds_wait<0>(h1);
          lds_wait<0>(h0);
          const f32x8 pw = pr * tsc;
          const f32x8 wq = __builtin_convertvector(__builtin_convertvector(pw, bf16x8), f32x8);
          f32x8 r;
#pragma unroll
          for (int k = 0; k < 4; ++k) {
            r[k] = __builtin_fmaf(wq[k] - pw[k], __uint_as_float(h0[k]), pr[k]);
            r[4 + k] = __builtin_fmaf(wq[4 + k] - pw[4 + k], __uint_as_float(h1[k]), pr[4 + k]);
          }
          lr_part += ((r[0] + r[1]) + (r[2] + r[3])) + ((r[4] + r[5]) + (r[6] + r[7]));
          pr = wq;
        } else {
          // the sum of the bf16 weights the MFMA uses normalises o
          const f32x8 r = __builtin_convertvector(__builtin_convertvector(pr, bf16x8), f32x8);
          lr_part += ((r[0] + r[1]) + (r[2] + r[3])) + ((r[4] + r[5]) + (r[6] + r[7]));
        }
        const bf16x8 pb = __builtin_convertvector(pr, bf16x8);
        {
          const uint32_t vbase0 = (uint32_t)(uintptr_t)tile + v_off0;
          const uint32_t vbase1 = (uint32_t)(uintptr_t)tile + v_off1;
          auto vread = [&](auto vbc) __attribute__((always_inline)) {
            constexpr int vb = decltype(vbc)::value;
            constexpr int off = (vb >> 1) * 1024;
            const uint32_t base = (vb & 1) ? vbase1 : vbase0;
            const u32x2 lo = ds_read_tr16_asm<off>(base);
            const u32x2 hi = ds_read_tr16_asm<off + C::NKQ * 1024>(base);
            return u32x4{lo[0], lo[1], hi[0], hi[1]};
          };
          u32x4 a0 = vread(std::integral_constant<int, 0>{});
          u32x4 a1 = vread(std::integral_constant<int, 1>{});
          static_for<C::NVB>([&](auto vbc) __attribute__((always_inline)) {
            constexpr int vb = decltype(vbc)::value;
            u32x4 a2 = a1;
            if constexpr (vb + 2 < C::NVB) a2 = vread(std::integral_constant<int, vb + 2>{});
            constexpr int later = 2 * ((vb + 2 < C::NVB ? vb + 2 : C::NVB - 1) - vb);
            lds_wait<later>(a0);
            oacc[vb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, a0), pb,
                                                               oacc[vb], 0, 0, 0);
            __builtin_amdgcn_sched_barrier(0);
            a0 = a1;
            a1 = a2;
          });
        }
      }
      if constexpr (F8 && HPW != 32) widen_tile(i + 1);
    }

    }

    // ---- epilogue: o = O / l, lse = ln(2) * (m + log2 l)
    float l_tot, lr_tot;
    if constexpr (HPW == 32) {
      l_tot = sum_halves(l_part);
      lr_tot = sum_halves(lr_part);
    } else {
      l_tot = sum_halves(l_part + __shfl_xor(l_part, 16, 64));
      lr_tot = sum_halves(lr_part + __shfl_xor(lr_part, 16, 64));
    }
    // a row that saw no position (multi-token decode) gets o = 0, lse = -inf
    const float inv = lr_tot > 0.f ? p.out_scale / lr_tot : 0.f;
    const float lse_v = (m_run + __builtin_amdgcn_logf(l_tot)) * kLn2;
    const int hl = HPW == 32 ? (lane & 31) : (lane & 15);
    const int h = h0 + hl;
    // lane holds O^T[v, h] for v = 32*vb + 8*g4 + 4*(lane/32) + i (32-head
    // waves) or v = 16*vb + 4*(lane/16) + i (16-head waves), i = 0..3
    auto vals = [&](int vb, int g4) __attribute__((always_inline)) {
      if constexpr (HPW == 32)
        return f32x4{oacc[vb][4 * g4], oacc[vb][4 * g4 + 1], oacc[vb][4 * g4 + 2],
                     oacc[vb][4 * g4 + 3]};
      else
        return (f32x4)oacc[vb];
    };
    auto col = [&](int vb, int g4) __attribute__((always_inline)) {
      return HPW == 32 ? 32 * vb + 8 * g4 + 4 * (lane >> 5) : 16 * vb + 4 * (lane >> 4);
    };
    constexpr int NG4 = HPW == 32 ? 4 : 1;
    if (final_out) {
      // the sequence's final o (bf16 or fp32) and lse
      const size_t row = (size_t)b * H + h;
#pragma unroll
      for (int vb = 0; vb < C::NVB; ++vb) {
#pragma unroll
        for (int g4 = 0; g4 < NG4; ++g4) {
          const f32x4 val = vals(vb, g4) * inv;
          const int v = col(vb, g4);
          if (!p.o_f32)
            *reinterpret_cast<bf16x4*>(reinterpret_cast<__bf16*>(p.o) + row * DV + v) =
                __builtin_convertvector(val, bf16x4);
          else
            *reinterpret_cast<f32x4*>(reinterpret_cast<float*>(p.o) + row * DV + v) = val;
        }
      }
      if (HPW == 32 ? (lane < 32) : (lane < 16)) p.lse[row] = lse_v;
    } else {
      // A partial (o_s, lse_s) for the merge.  o_s is stored in fp16 as
      // o_s * 2^-e, with e chosen per row so that the row's largest |value|
      // lands in [2^14, 2^15): no overflow whatever the cache's range, and a
      // relative rounding error of at most 2^-12 of that largest value.
      const size_t row = (size_t)slot * H + h;
      float mx = 0.f;
#pragma unroll
      for (int vb = 0; vb < C::NVB; ++vb)
#pragma unroll
        for (int r = 0; r < (HPW == 32 ? 16 : 4); ++r)
          mx = fmaxf(mx, fabsf(HPW == 32 ? acc_read(oacc[vb][r]) : oacc[vb][r]));
      if constexpr (HPW == 16) mx = fmaxf(mx, __shfl_xor(mx, 16, 64));
      mx = max_halves(mx) * inv;
      int e = 0;
      if (mx > 0.f && mx <= 3.0e38f) {
        int ex;
        (void)frexpf(mx, &ex);  // mx in [2^(ex-1), 2^ex)
        e = ex - 15;
      }
      const float sinv = ldexpf(inv, -e);
      _Float16* dst = p.ws_o + row * DV;
#pragma unroll
      for (int vb = 0; vb < C::NVB; ++vb) {
        if constexpr (HPW == 32) {
          // g4 pairs (0,1) and (2,3): the two half-waves swap halves so that
          // each lane stores 8 consecutive columns (16 bytes)
#pragma unroll
          for (int gp = 0; gp < 2; ++gp) {
            typedef _Float16 f16x4 __attribute__((ext_vector_type(4)));
            const u32x2 a = __builtin_bit_cast(
                u32x2, __builtin_convertvector(vals(vb, 2 * gp) * sinv, f16x4));
            const u32x2 c = __builtin_bit_cast(
                u32x2, __builtin_convertvector(vals(vb, 2 * gp + 1) * sinv, f16x4));
            // lanes 0-31 end with columns +0..7, lanes 32-63 with +8..15
            const auto s0 = __builtin_amdgcn_permlane32_swap(a[0], c[0], false, false);
            const auto s1 = __builtin_amdgcn_permlane32_swap(a[1], c[1], false, false);
            const u32x4 w = {s0[0], s1[0], s0[1], s1[1]};
            const int v = 32 * vb + 16 * gp + 8 * (lane >> 5);
            *reinterpret_cast<u32x4*>(dst + v) = w;
          }
        } else {
          typedef _Float16 f16x4 __attribute__((ext_vector_type(4)));
          *reinterpret_cast<f16x4*>(dst + col(vb, 0)) =
              __builtin_convertvector(vals(vb, 0) * sinv, f16x4);
        }
      }
      if (HPW == 32 ? (lane < 32) : (lane < 16)) p.ws_ls[row] = f32x2{lse_v, ldexpf(1.f, e)};
    }
  };

  // ---------------- enumerate this unit's segments; process has one call site
  int b = 0, ts = 0, te = 0, slot = 0, vis_n = 0;
  bool fin = false;
  int64_t st = 0, a0 = 0, a1 = 0;  // balanced mode: tile cursor and unit range
  int64_t TC = 0;                   // balanced mode: length of the cost stream
  if (p.split_mode == 0) {
    const int S = p.num_splits;
    b = unit / S;
    const int s = unit % S;
    const int n = seq_len_at(p.seq_lens, b, p.len_cap);
    if (n <= 0) {
      if (s == 0) {  // empty sequence: o = 0, lse = -inf
        const int h = h0 + (HPW == 32 ? (lane & 31) : (lane & 15));
        const size_t obase = ((size_t)b * H + h) * DV;
        constexpr int per_lane = DV * HPW / 64;
        const int part = HPW == 32 ? (lane >> 5) : (lane >> 4);
        for (int k = 0; k < per_lane; k += 4)
          store_out4(p.o, p.o_f32, obase + part * per_lane + k, f32x4{0.f, 0.f, 0.f, 0.f});
        if (HPW == 32 ? lane < 32 : lane < 16) p.lse[(size_t)b * H + h] = -INFINITY;
      }
      return;
    }
    const int Cb = per_seq_chunk(n, S);
    ts = s * Cb;
    if (ts >= n) return;
    te = min(ts + Cb, n);
    fin = (n + Cb - 1) / Cb == 1;
    slot = b * S + s;
    vis_n = n - (p.q_len - 1);
  } else {
    // the unit covers positions [a0, a1) of the batch's cost stream
    const int U = p.num_splits;
    TC = uniform64(total_cost(p.seq_lens, p.batch, p.seg_cost, p.len_cap, lane));
    if (TC == 0) return;
    a0 = (int64_t)unit * TC / U;
    a1 = (int64_t)(unit + 1) * TC / U;
    if (a0 >= a1) return;
    // first sequence whose cost range reaches past a0, and where it starts
    for (int c0 = 0; c0 < p.batch; c0 += 64) {
      const int bl = c0 + lane;
      const int ntl = bl < p.batch ? cost_of(seq_len_at(p.seq_lens, bl, p.len_cap), p.seg_cost) : 0;
      const int incl = wave_incl_scan(ntl, lane);
      const uint64_t past = __builtin_amdgcn_ballot_w64(bl < p.batch && st + incl > a0);
      if (past) {
        const int k = __builtin_ctzll(past);
        b = c0 + k;
        st += __shfl(incl - ntl, k, 64);
        break;
      }
      st += __shfl(incl, 63, 64);
    }
    b = uniform(b);
    st = uniform64(st);
  }
  for (;;) {
    if (p.split_mode != 0) {
      const int n = seq_len_at(p.seq_lens, b, p.len_cap);
      const int nt = tiles_of(n);
      const int64_t rs = st + (nt > 0 ? p.seg_cost : 0);  // position of tile 0
      const int64_t lo = (a0 > rs ? a0 : rs) - rs;
      const int64_t hi = (a1 < rs + nt ? a1 : rs + nt) - rs;
      ts = (int)lo * kTile;
      te = hi > lo ? min((int)hi * kTile, n) : ts;
      fin = lo == 0 && hi == nt;
      slot = unit + b;
      vis_n = n - (p.q_len - 1);
      if (lo == 0 && hi > 0 && hc == 0 && threadIdx.x == 0) {
        // this unit owns tile 0 of sequence b: record the slots of its partials for
        // stage 2 (count 1: the result is final; -1: some unit of the run
        // owns no tile, and stage 2 works the range out itself)
        const int ul = unit_of_tile(rs + nt - 1, TC, p.num_splits);
        p.ws_seg[2 * b] = slot;
        p.ws_seg[2 * b + 1] = p.num_splits <= TC ? ul - unit + 1 : -1;
      }
      st += cost_of(n, p.seg_cost);
    }
    if (te > ts) process(b, ts, te, fin, slot, vis_n);
    if (p.split_mode == 0) break;
    ++b;
    if (b >= p.batch || st >= a1) break;
  }
}

// ---------------------------------------------------------------- stage 2

struct Stage2Params {
  const int32_t* seq_lens;
  const _Float16* ws_o;
  const f32x2* ws_ls;
  const int32_t* ws_seg;
  void* o;
  float* lse;
  int32_t batch, heads, o_f32, split_mode, num_splits, head_groups, kgroups;
  int32_t seg_cost;  // balanced mode: the same cost stream as stage 1
  int32_t len_cap;   // the same length clamp as stage 1
};

// One workgroup per (sequence, 8/KG heads, 256 output columns), 256 threads:
// 32 threads per (head, partial group), each owning 8 consecutive columns
// (one 16-byte fp16 load per partial).  The KG groups of a head take every
// KG-th partial and are combined through LDS at the end, so a sequence with
// hundreds of partials is read by many threads at once; each thread keeps 8
// partial loads in flight.
constexpr int kS2Rows = 8, kS2Cols = 256, kS2Batch = 8;
typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));

__device__ __forceinline__ void store_out8(void* o, int o_f32, size_t idx, const f32x8& v) {
  if (o_f32) {
    *reinterpret_cast<f32x4*>(reinterpret_cast<float*>(o) + idx) = f32x4{v[0], v[1], v[2], v[3]};
    *reinterpret_cast<f32x4*>(reinterpret_cast<float*>(o) + idx + 4) = f32x4{v[4], v[5], v[6], v[7]};
  } else {
    *reinterpret_cast<bf16x8*>(reinterpret_cast<__bf16*>(o) + idx) = __builtin_convertvector(v, bf16x8);
  }
}

template <int DV>
__global__ __launch_bounds__(256) void mla_stage2(Stage2Params p) {
  static_assert(DV % kS2Cols == 0, "");
  constexpr int NVC = DV / kS2Cols;
  __shared__ f32x8 red_o[kS2Rows][32];
  __shared__ float red_m[kS2Rows], red_l[kS2Rows];
  const int KG = p.kgroups;               // partial groups per head (1, 2, 4 or 8)
  const int HPB = kS2Rows / KG;           // heads per workgroup
  int id = blockIdx.x;
  const int vc = id % NVC;
  id /= NVC;
  const int hg = id % p.head_groups;
  const int b = id / p.head_groups;
  const int t = threadIdx.x;
  const int lane = t & 63;
  const int row = t >> 5, j = t & 31;
  const int hl = row / KG, g = row % KG;
  const int H = p.heads;
  const int h = hg * HPB + hl;  // < H: H is a multiple of 16
  const int v = vc * kS2Cols + 8 * j;
  const int n = seq_len_at(p.seq_lens, b, p.len_cap);

  int first, count;
  bool all_live = true;
  int unit0 = 0, units = 1;
  int64_t tiles_total = 1;
  if (p.split_mode == 0) {
    const int S = p.num_splits;
    if (n <= 0) return;  // stage 1 wrote o = 0, lse = -inf
    const int Cb = per_seq_chunk(n, S);
    const int nseg = (n + Cb - 1) / Cb;
    if (nseg <= 1) return;  // stage 1 wrote the final result
    first = b * S;
    count = nseg;
  } else if (n > 0 && p.ws_seg[2 * b + 1] > 0) {
    // the partial range stage 1 recorded for this sequence
    count = p.ws_seg[2 * b + 1];
    if (count == 1) return;  // stage 1 wrote the final result
    first = p.ws_seg[2 * b];
  } else {
    const int U = p.num_splits;
    // cost before sequence b, and in total
    int64_t before = 0, TT = 0;
    for (int c0 = 0; c0 < p.batch; c0 += 64) {
      const int bl = c0 + lane;
      const int nt = bl < p.batch ? cost_of(seq_len_at(p.seq_lens, bl, p.len_cap), p.seg_cost) : 0;
      const int incl = wave_incl_scan(nt, lane);
      const int tot = __shfl(incl, 63, 64);
      if (b >= c0 + 64) before += tot;
      else if (b >= c0) before += __shfl(incl - nt, b - c0, 64);
      TT += tot;
    }
    const int nt = tiles_of(n);
    if (nt == 0) {
      if (g == 0) {
        store_out8(p.o, p.o_f32, ((size_t)b * H + h) * DV + v, f32x8{});
        if (vc == 0 && j == 0) p.lse[(size_t)b * H + h] = -INFINITY;
      }
      return;
    }
    const int64_t rs = before + p.seg_cost;  // position of the sequence's tile 0
    const int uf = unit_of_tile(rs, TT, U);
    const int ul = unit_of_tile(rs + nt - 1, TT, U);
    if (uf == ul) return;  // stage 1 wrote the final result
    first = uf + b;
    count = ul - uf + 1;
    // with more units than tiles, some units own no tile and wrote no
    // partial: they get weight 0 and their slots are never read
    all_live = U <= TT;
    tiles_total = TT;
    units = U;
    unit0 = uf;
  }
  auto live = [&](int k) {
    if (all_live) return true;
    const int64_t u = unit0 + k;
    return (u + 1) * tiles_total / units > u * tiles_total / units;
  };
  const f32x2* ls_h = p.ws_ls + (size_t)first * H + h;  // partial k at ls_h[k * H]
  const size_t stride = (size_t)H * DV;  // elements between consecutive partials
  const _Float16* src = p.ws_o + ((size_t)first * H + h) * DV + v;

  // One pass over this group's partials k = g, g + KG, ..., kS2Batch at a
  // time: all of a batch's rows and {lse, 2^e} pairs are loaded before any is
  // used, then folded into a running max m, weight sum tot and accumulator
  // (the stored row is o_k * 2^-e_k, so it enters with e^(lse_k - m) * 2^e_k)
  float m = -INFINITY, tot = 0.f;
  f32x8 acc = {};
  for (int k0 = g; k0 < count; k0 += kS2Batch * KG) {
    f16x8 x[kS2Batch];
    f32x2 ls[kS2Batch];
#pragma unroll
    for (int i = 0; i < kS2Batch; ++i) {
      const int k = k0 + i * KG;
      const bool use = k < count && live(k);  // a slot without a partial may hold anything
      x[i] = use ? *reinterpret_cast<const f16x8*>(src + (size_t)k * stride) : f16x8{};
      ls[i] = use ? ls_h[(size_t)k * H] : f32x2{-INFINITY, 0.f};
    }
    float mb = m;
#pragma unroll
    for (int i = 0; i < kS2Batch; ++i) mb = fmaxf(mb, ls[i][0]);
    if (mb == -INFINITY) continue;  // nothing live yet
    const float r = m == -INFINITY ? 0.f : __expf(m - mb);  // nothing accumulated yet
    tot *= r;
    acc *= r;
#pragma unroll
    for (int i = 0; i < kS2Batch; ++i) {
      const float w = __expf(ls[i][0] - mb);  // 0 for the unused entries
      tot += w;
      acc += (w * ls[i][1]) * __builtin_convertvector(x[i], f32x8);
    }
    m = mb;
  }

  // combine the KG groups of each head (every group saw at least one partial)
  if (KG > 1) {
    red_o[row][j] = acc;
    if (j == 0) {
      red_m[row] = m;
      red_l[row] = tot;
    }
    __syncthreads();
    if (g != 0) return;
    float M = m;
    for (int r2 = row + 1; r2 < row + KG; ++r2) M = fmaxf(M, red_m[r2]);
    // groups (or whole rows, in multi-token decode) with no visible
    // position carry m = -inf and weight 0
    const float r0 = m == -INFINITY ? 0.f : __expf(m - M);
    acc *= r0;
    tot *= r0;
    for (int r2 = row + 1; r2 < row + KG; ++r2) {
      const float rr = red_m[r2] == -INFINITY ? 0.f : __expf(red_m[r2] - M);
      acc += rr * red_o[r2][j];
      tot += rr * red_l[r2];
    }
    m = M;
  }
  const bool any = tot > 0.f;  // a row that saw no position: o = 0, lse = -inf
  store_out8(p.o, p.o_f32, ((size_t)b * H + h) * DV + v, any ? acc * (1.f / tot) : f32x8{});
  if (vc == 0 && j == 0) p.lse[(size_t)b * H + h] = any ? m + __logf(tot) : -INFINITY;
}

// ---------------------------------------------------------------- dispatch

// A kernel launch; with events pending for this stage (mla_time_next_launch)
// the launch records the kernel's own start and end into them.
template <typename K, typename P>
int launch_timed(int stage, K kernel, dim3 grid, dim3 block, hipStream_t st, const P& params) {
  LaunchTiming& t = g_launch_timing[stage];
  if (t.start || t.stop) {
    const LaunchTiming ev = t;
    t = LaunchTiming{};
    hipExtLaunchKernelGGL(kernel, grid, block, 0, st, reinterpret_cast<hipEvent_t>(ev.start),
                          reinterpret_cast<hipEvent_t>(ev.stop), 0, params);
  } else {
    hipLaunchKernelGGL(kernel, grid, block, 0, st, params);
  }
  return (int)hipGetLastError();
}

template <int HPW, int W, int D, int DV, bool F8, bool SP = false, int PT = 0>
int launch_stage1(const Stage1Params& sp, int grid, hipStream_t st) {
  constexpr int NBUF = stage1_ring_depth(HPW, W, D, F8, PT);
  return launch_timed(0, mla_stage1<HPW, W, D, DV, NBUF, F8, SP, PT>, dim3(grid), dim3(64 * W), st,
                      sp);
}

template <int D, int DV, bool F8, int PT = 0, bool SP = false>
int launch_stage1_for(const HeadTiling& ht, const Stage1Params& sp, int grid, hipStream_t st) {
  if (ht.heads_per_wave == 32) {
    switch (ht.waves) {
      case 4: return launch_stage1<32, 4, D, DV, F8, SP, PT>(sp, grid, st);
      case 2: return launch_stage1<32, 2, D, DV, F8, SP, PT>(sp, grid, st);
      default: return launch_stage1<32, 1, D, DV, F8, SP, PT>(sp, grid, st);
    }
  }
  // 16-head waves only arise for an odd number of 16-head groups (H % 32 != 0),
  // which always gives one wave per workgroup
  return launch_stage1<16, 1, D, DV, F8, SP, PT>(sp, grid, st);
}

}  // namespace

// The stage-1 launches of one group of variants.  This source is compiled
// once per group (MLA_STAGE1_GROUP = 0..9: sparse gather or not x bf16,
// per-tensor fp8, per-token fp8, per-token int8 or per-token int4 cache) and once with
// MLA_MAIN for the rest, so that the many template instances build in
// parallel.
#define MLA_CAT2(a, b) a##b
#define MLA_CAT(a, b) MLA_CAT2(a, b)
#define MLA_DECLARE_GROUP(g)                                                              \
  int MLA_CAT(launch_stage1_group, g)(int head_size, const HeadTiling& ht,               \
                                      const Stage1Params& sp, int grid, hipStream_t st);
MLA_DECLARE_GROUP(0)
MLA_DECLARE_GROUP(1)
MLA_DECLARE_GROUP(2)
MLA_DECLARE_GROUP(3)
MLA_DECLARE_GROUP(4)
MLA_DECLARE_GROUP(5)
MLA_DECLARE_GROUP(6)
MLA_DECLARE_GROUP(7)
MLA_DECLARE_GROUP(8)
MLA_DECLARE_GROUP(9)

#ifdef MLA_STAGE1_GROUP
int MLA_CAT(launch_stage1_group, MLA_STAGE1_GROUP)(int head_size, const HeadTiling& ht,
                                                   const Stage1Params& sp, int grid,
                                                   hipStream_t st) {
  constexpr bool SP = MLA_STAGE1_GROUP >= 5;
  // 0 bf16, 1 fp8 with k_scale, per token: 2 fp8, 3 int8, 4 int4
  constexpr int fmt = MLA_STAGE1_GROUP % 5;
  constexpr bool F8 = fmt != 0;
  constexpr int PT = fmt >= 2 ? fmt - 1 : 0;
  return head_size == 576 ? launch_stage1_for<576, 512, F8, PT, SP>(ht, sp, grid, st)
                          : launch_stage1_for<320, 256, F8, PT, SP>(ht, sp, grid, st);
}
#endif

#ifdef MLA_MAIN
// What starting a segment costs, in tiles of the balanced cost stream: the
// query rows of a workgroup's heads and one partial row per head, plus about
// one tile of latency.  Measured on the dsv3 shape (128 heads per
// workgroup) a segment start costs about as much as 8-9 tiles.
int segment_cost_tiles(int heads, const HeadTiling& ht) {
  const int per_wg = heads / ht.head_chunks;
  return 1 + (per_wg + 15) / 16;
}

int launch_decode(const DecodeArgs& a, void* stream, int stages) {
  hipStream_t st = reinterpret_cast<hipStream_t>(stream);
  const HeadTiling ht = head_tiling(a.heads);

  Stage1Params sp;
  sp.q_nope = reinterpret_cast<const __bf16*>(a.q_nope);
  sp.q_pe = reinterpret_cast<const __bf16*>(a.q_pe);
  sp.qn_seq = a.qn_seq;
  sp.qn_row = a.qn_row;
  sp.qp_seq = a.qp_seq;
  sp.qp_row = a.qp_row;
  sp.kv = reinterpret_cast<const uint8_t*>(a.kv);
  sp.block_table = a.block_table;
  sp.seq_lens = a.seq_lens;
  sp.o = a.o;
  sp.lse = a.lse;
  sp.ws_o = reinterpret_cast<_Float16*>(a.ws_o);
  sp.ws_ls = reinterpret_cast<f32x2*>(a.ws_ls);
  sp.ws_seg = reinterpret_cast<int32_t*>(a.ws_seg);
  sp.batch = a.batch;
  sp.heads = a.heads;
  sp.page_size = a.page_size;
  sp.bt_stride = a.bt_stride;
  sp.o_f32 = a.o_f32;
  sp.split_mode = a.split_mode;
  sp.num_splits = a.num_splits;
  sp.head_chunks = ht.head_chunks;
  sp.seg_cost = segment_cost_tiles(a.heads, ht);
  sp.q_len = a.q_len;
  sp.heads_per_token = a.heads / a.q_len;
  sp.topk_idx = a.topk_idx;
  sp.topk_stride = a.topk_stride;
  sp.pool_bytes = (uint32_t)a.pool_bytes;
  sp.num_blocks = (uint32_t)a.num_blocks;
  {
    // sparse decode: a list holds at most topk entries; dense decode: a table
    // row of bt_stride pages holds at most bt_stride * page_size positions
    const int64_t cap = a.topk_idx ? (int64_t)a.topk_stride : (int64_t)a.bt_stride * a.page_size;
    sp.len_cap = (int32_t)(cap < 0x7fffffff ? cap : 0x7fffffff);
  }
  sp.page_shift = -1;
  for (int sh = 0; sh < 31; ++sh)
    if ((1 << sh) == a.page_size) sp.page_shift = sh;
  // a per-tensor fp8 scale multiplies every score and o; per-token scales
  // are applied inside the kernel, position by position
  const bool tensor_scale = a.kv_fp8 && !a.kv_pt;
  sp.score_log2 = a.scale * kLog2e * (tensor_scale ? a.k_scale : 1.f);
  sp.out_scale = tensor_scale ? a.k_scale : 1.f;

  // stage 2's partial groups per head: about a quarter of the mean partial
  // count per sequence (units / batch + 1), a power of two up to 8; one
  // workgroup per (sequence, head group, 256 columns)
  const int per_seq = a.split_mode == 0 ? a.num_splits : a.num_splits / a.batch + 1;
  const int kgroups = per_seq >= 32 ? 8 : per_seq >= 16 ? 4 : per_seq >= 8 ? 2 : 1;
  const int head_groups = a.heads / (kS2Rows / kgroups);
  const int64_t units = a.split_mode == 0 ? (int64_t)a.batch * a.num_splits : a.num_splits;
  const int64_t grid1_64 = (units + 7) / 8 * 8 * ht.head_chunks;
  const int64_t grid2_64 = (int64_t)a.batch * head_groups * (a.d_v / kS2Cols);
  // nothing is enqueued for a shape whose grid HIP cannot launch
  if (grid1_64 > kMaxGrid || grid2_64 > kMaxGrid) return kGridTooLarge;
  const int grid1 = (int)grid1_64;
  if (stages & kStage1) {
    // the group of variants: gather (+5) and cache format
    const int fmt = a.kv_pt ? 1 + a.kv_pt : (a.kv_fp8 ? 1 : 0);
    const int group = (a.topk_idx ? 5 : 0) + fmt;
    int err;
    switch (group) {
      case 0: err = launch_stage1_group0(a.head_size, ht, sp, grid1, st); break;
      case 1: err = launch_stage1_group1(a.head_size, ht, sp, grid1, st); break;
      case 2: err = launch_stage1_group2(a.head_size, ht, sp, grid1, st); break;
      case 3: err = launch_stage1_group3(a.head_size, ht, sp, grid1, st); break;
      case 4: err = launch_stage1_group4(a.head_size, ht, sp, grid1, st); break;
      case 5: err = launch_stage1_group5(a.head_size, ht, sp, grid1, st); break;
      case 6: err = launch_stage1_group6(a.head_size, ht, sp, grid1, st); break;
      case 7: err = launch_stage1_group7(a.head_size, ht, sp, grid1, st); break;
      case 8: err = launch_stage1_group8(a.head_size, ht, sp, grid1, st); break;
      default: err = launch_stage1_group9(a.head_size, ht, sp, grid1, st); break;
    }
    if (err) return err;
  }
  const bool merge = a.split_mode == 1 || a.num_splits > 1;
  if (!merge || !(stages & kStage2)) return 0;
  Stage2Params s2;
  s2.seq_lens = a.seq_lens;
  s2.ws_o = reinterpret_cast<const _Float16*>(a.ws_o);
  s2.ws_ls = reinterpret_cast<const f32x2*>(a.ws_ls);
  s2.ws_seg = reinterpret_cast<const int32_t*>(a.ws_seg);
  s2.o = a.o;
  s2.lse = a.lse;
  s2.batch = a.batch;
  s2.heads = a.heads;
  s2.o_f32 = a.o_f32;
  s2.split_mode = a.split_mode;
  s2.num_splits = a.num_splits;
  s2.seg_cost = sp.seg_cost;
  s2.len_cap = sp.len_cap;
  s2.kgroups = kgroups;
  s2.head_groups = head_groups;
  const int grid2 = (int)grid2_64;
  return a.d_v == 512 ? launch_timed(1, mla_stage2<512>, dim3(grid2), dim3(256), st, s2)
                     : launch_timed(1, mla_stage2<256>, dim3(grid2), dim3(256), st, s2);
}
#endif  // MLA_MAIN

}  // namespace mla
