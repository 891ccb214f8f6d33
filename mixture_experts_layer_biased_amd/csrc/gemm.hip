// Grouped expert GEMMs over the FFN-routed rows only.
//
// Method: "LongCat-Flash" (llm-wiki entity page), section 2.1: only the
// FFN experts cost FLOPs; section 1 table: expert intermediate size 2048.
// Expert e (SiLU-gated, W13 = [gate rows; up rows] [2I][d], W2 [d][I]):
//   gate/up:  H = silu(X_e W_gate^T) * (X_e W_up^T)   [rows_e][I], bf16
//   down:     Y = H W2^T                               [rows_e][d], bf16
// with X_e the rows of x gathered through the expert's slots (perm).
//
// Every expert with routed rows, decode batches included: M-tiles of up to
// 320 token rows (kBigTileRows) x 256 weight rows per block, 8 waves (2 x 4),
// v_mfma_f32_32x32x16_bf16, both operands copied HBM -> LDS by
// global_load_lds_dwordx4 in a multi-stage ring; the tiles of one expert
// (column slices, M-tiles) are adjacent on one XCD (blockIdx % 8) so its
// gathered x rows are shared through that XCD's L2. With a handful of rows
// (decode) the tile's MFMA work is small and the kernel is a stream of whole
// 128-byte weight lines, which measured faster than streaming the weights
// into MFMA operand registers (half-line requests) at every batch size.
// fp8 (E4M3FN, one fp32 scale per 128x128 block) weights are converted in
// registers: bf16(fl32(q) * s), then the same bf16 MFMA.
#include <type_traits>

#include "common.h"
#include "kernels.h"

namespace lcmoe {

__device__ __forceinline__ float silu_f(float g) { return g / (1.0f + expf(-g)); }

// ===========================================================================
// large-M kernel: direct-to-LDS pipeline (bf16 or fp8 weights)
//
// Tile up to 320 token rows x 256 weight rows; the k loop runs in stages of
// 64. Both operands move HBM -> LDS with global_load_lds_dwordx4 (no
// register staging) into a ring of LDS slots, all but one in flight while
// one is multiplied. A stage moves a whole 128-byte line of every x row and
// bf16 weight row (eight lanes per row, eight rows per copy instruction):
// the L1/L2 request rate, not the byte rate, bounds these copies, so whole
// lines carry twice the bytes of 64-byte half-line requests. fp8 codes stay
// one byte in LDS (64 bytes per weight row per stage) and become
// bf16(fl32(q) * s) in registers after the LDS read. The token rows form ten
// 32-row fragments, fragment i belonging to wave row i & 1, so any row count
// splits evenly over the two waves that share a SIMD.
//
// LDS layouts (16-byte chunks; gfx950 LDS has 64 banks, so each group of 16
// lanes must touch 16 distinct 16-byte slots of a 256-byte window):
//   x tile and bf16 weight tile: 128-byte rows, chunk c of row r at
//     c ^ ((r >> 1) & 7);
//   fp8 weight tile: 64-byte rows, chunk c of row r at c ^ ((r >> 2) & 3).
// One copy instruction fills a contiguous 1 KB block: lane l writes the
// block's l-th chunk, so it loads the logical chunk the swizzle puts there.
//
// k order inside a 64-wide stage (the same for both operands, as the MFMA
// requires), for half kk (0, 1), k-step j (0, 1) and lane half h: bf16
// weights: k = 32 kk + 16 j + 8 h + [0, 8) (operand chunk 4 kk + 2 j + h);
// fp8 weights: k = 32 kk + 16 h + 8 j + [0, 8) (x chunk 4 kk + 2 h + j), so
// one 16-byte read of weight chunk 2 kk + h gives lane half h its 16 codes
// for both k-steps of the half.
//
// Each wave waits for its own copies of a stage (s_waitcnt vmcnt with the
// count of its younger copies still allowed in flight) and a raw s_barrier
// then publishes the stage; no fence, which would drain the pipeline.
// ===========================================================================
constexpr int DBK = 64;  // k per pipeline stage

template <int N>
__device__ __forceinline__ void wait_vmcnt() {
  // gfx9 s_waitcnt: vmcnt[3:0], expcnt[6:4], lgkmcnt[11:8], vmcnt[5:4] at [15:14]
  __builtin_amdgcn_s_waitcnt((N & 15) | (7 << 4) | (15 << 8) | ((N >> 4) << 14));
}
// Wait until at most n (0..31) of this wave's vector memory operations remain.
__device__ __forceinline__ void wait_vmcnt_upto(int n) {
  switch (n) {
    case 0: wait_vmcnt<0>(); break;
    case 1: wait_vmcnt<1>(); break;
    case 2: wait_vmcnt<2>(); break;
    case 3: wait_vmcnt<3>(); break;
    case 4: wait_vmcnt<4>(); break;
    case 5: wait_vmcnt<5>(); break;
    case 6: wait_vmcnt<6>(); break;
    case 7: wait_vmcnt<7>(); break;
    case 8: wait_vmcnt<8>(); break;
    case 9: wait_vmcnt<9>(); break;
    case 10: wait_vmcnt<10>(); break;
    case 11: wait_vmcnt<11>(); break;
    case 12: wait_vmcnt<12>(); break;
    case 13: wait_vmcnt<13>(); break;
    case 14: wait_vmcnt<14>(); break;
    case 15: wait_vmcnt<15>(); break;
    case 16: wait_vmcnt<16>(); break;
    case 17: wait_vmcnt<17>(); break;
    case 18: wait_vmcnt<18>(); break;
    case 19: wait_vmcnt<19>(); break;
    case 20: wait_vmcnt<20>(); break;
    case 21: wait_vmcnt<21>(); break;
    case 22: wait_vmcnt<22>(); break;
    case 23: wait_vmcnt<23>(); break;
    case 24: wait_vmcnt<24>(); break;
    case 25: wait_vmcnt<25>(); break;
    case 26: wait_vmcnt<26>(); break;
    case 27: wait_vmcnt<27>(); break;
    case 28: wait_vmcnt<28>(); break;
    case 29: wait_vmcnt<29>(); break;
    case 30: wait_vmcnt<30>(); break;
    default: wait_vmcnt<31>(); break;
  }
}
__device__ __forceinline__ void raw_barrier() {
  asm volatile("" ::: "memory");
  __builtin_amdgcn_s_barrier();
  asm volatile("" ::: "memory");
}
// One global_load_lds_dwordx4 in its scalar-base form: lane l copies 16
// bytes from sbase + voff (voff a 32-bit unsigned per-lane byte offset, sbase
// wave-uniform) into LDS at lds + 16*l. Issued as inline asm so the compiler
// does not track it: every wait on these copies is the explicit wait_vmcnt
// above. M0 (the LDS base of the copy) is written here and used by nothing
// else in these kernels.
__device__ __forceinline__ void dma16(const char* sbase, uint32_t voff, const uint4* lds) {
  const uint32_t l = (uint32_t)__builtin_amdgcn_readfirstlane((int)(uint32_t)(uintptr_t)lds);
  const uint64_t b = (uint64_t)(uintptr_t)sbase;
  const uint64_t bs = ((uint64_t)(uint32_t)__builtin_amdgcn_readfirstlane((int)(b >> 32)) << 32) |
                      (uint32_t)__builtin_amdgcn_readfirstlane((int)(uint32_t)b);
  asm volatile("s_mov_b32 m0, %2\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %0, %1"
               :: "v"(voff), "s"(bs), "s"(l) : "memory");
}
// 64-byte LDS rows (fp8 weight tile): chunk c of row r lives at c ^ ((r >> 2) & 3).
__device__ __forceinline__ int swz64(int row, int chunk) {
  return row * 4 + (chunk ^ ((row >> 2) & 3));
}

// The ring lives in one 160 KB LDS array (all of a CU's LDS). A slot holds
// the x rows of the tile (8-row groups, 128 B per row) followed by the
// weight tile; the slot count is what fits for the tile's actual row count,
// capped at 3: with bf16 weights 3 slots up to 168 rows, which covers an
// expert's rows at a prefill batch (about 128 +- 12); in 144 KB, tiles past
// 128 rows had 2.
template <bool FP8>
struct DmaTile {
  static constexpr int LDS_CHUNKS = 10240;                  // 160 KB
  static constexpr int MAX_SLOTS = 3;
  static constexpr int B_CHUNKS = FP8 ? 256 * 4 : 256 * 8;  // weight tile, 16 or 32 KB
  static constexpr int AGROUPS = kBigTileRows / 8;          // 8-row copy groups of the x tile
  static constexpr int AG_PER_WAVE = AGROUPS / 8;           // 5
  static constexpr int BG_PER_WAVE = FP8 ? 2 : 4;           // weight copies per wave
};

template <bool GATEUP, bool FP8, bool BWD = false>
__global__ __launch_bounds__(512) void gemm_big_dma_kernel(GemmArgs a) {
  static_assert(!BWD || (GATEUP && !FP8), "the backward epilogue is for bf16 gate/up");
  using TL = DmaTile<FP8>;
  __shared__ uint4 lds[TL::LDS_CHUNKS];
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int wm = wave >> 2, wn = wave & 3;
  const int h = lane >> 5;
  const int kdim = a.kdim;

  // Tile order (expert, column slice, M-tile); each XCD takes a contiguous
  // run of that order so neighbouring tiles share its L2.
  const int total = a.meta[1] * a.nslices;
  const int per_xcd = (total + 7) >> 3;
  const int xcd = blockIdx.x & 7, pos = blockIdx.x >> 3;
  if (pos >= per_xcd) return;
  const int L = xcd * per_xcd + pos;
  if (L >= total) return;
  int lo = 0, hi = a.n_ffn - 1;
  while (lo < hi) {
    const int mid = (lo + hi + 1) >> 1;
    if (a.mt_prefix[mid] * a.nslices <= L) lo = mid; else hi = mid - 1;
  }
  const int e = lo;
  const int mt = a.mt_prefix[e + 1] - a.mt_prefix[e];
  const int local = L - a.mt_prefix[e] * a.nslices;
  const int slice = local / mt, m = local - slice * mt;
  const int cnt = a.counts[e];
  const int r0 = (int)((long long)m * cnt / mt);
  const int rows = (int)((long long)(m + 1) * cnt / mt) - r0;
  const int rowbase = a.offsets[e] + r0;

  auto wrow_of = [&](int j) -> int {  // LDS weight-tile row -> weight row (or -1)
    if (GATEUP) {
      const int col = slice * kBigColsGateUp + (j & 127);
      if (col >= a.n_out) return -1;
      return j < 128 ? col : a.n_out + col;
    } else {
      const int col = slice * kBigColsDown + j;
      return col < a.n_out ? col : -1;
    }
  };

  // Copy assignment. x tile: wave w fills 8-row groups w + 8 g (1 KB each,
  // eight lanes per row). bf16 weights: 8-row groups w + 8 g; fp8 weights:
  // 16-row groups w + 8 g (64 B per row, four lanes per row). Groups wholly
  // outside the valid rows are skipped. When kdim is an odd multiple of 32
  // the last stage holds only the first 32 k of each row: lanes past the end
  // of a row then load that row's chunk c - 4, which no MFMA reads.
  //
  // Byte offsets of each lane's copies from the operand bases (all of x, the
  // tile's first H row, or this expert's weight matrix; below 4 GiB, which
  // the host checks); the k position goes into the scalar base.
  uint32_t aoff[TL::AG_PER_WAVE], boff[TL::BG_PER_WAVE];
  bool ause[TL::AG_PER_WAVE], buse[TL::BG_PER_WAVE];
  const int esz = FP8 ? 1 : 2;  // weight bytes per element
  const char* wexp = static_cast<const char*>(a.w) + (size_t)e * a.rows_total * kdim * esz;
  const char* abase = reinterpret_cast<const char*>(a.src) + (GATEUP ? 0 : (size_t)rowbase * kdim * 2);
  // Logical chunk loaded by this lane into an 8-row group g (row 8 g + (lane >> 3)):
  // (row >> 1) & 7 = (4 g + (lane >> 4)) & 7 depends on g only through g & 1,
  // which is wave & 1 for every group g = wave + 8 g2 of this wave.
  const int ac = (lane & 7) ^ ((4 * (wave & 1) + (lane >> 4)) & 7);
#pragma unroll
  for (int g2 = 0; g2 < TL::AG_PER_WAVE; ++g2) {
    const int g = wave + 8 * g2;
    const int row = 8 * g + (lane >> 3);
    ause[g2] = 8 * g < rows;
    const int rr = row < rows ? row : 0;
    const size_t srow = GATEUP ? (size_t)(a.perm[rowbase + rr] / a.topk) : (size_t)rr;
    aoff[g2] = (uint32_t)(srow * kdim * 2 + 16 * ac);
  }
  if (FP8) {
#pragma unroll
    for (int g2 = 0; g2 < TL::BG_PER_WAVE; ++g2) {
      const int g = wave + 8 * g2;
      const int row = 16 * g + (lane >> 2);
      const int c = (lane & 3) ^ ((row >> 2) & 3);
      const int wr = wrow_of(row);
      buse[g2] = wrow_of(16 * g) >= 0;
      boff[g2] = (uint32_t)((size_t)(wr >= 0 ? wr : 0) * kdim + 16 * c);
    }
  } else {
#pragma unroll
    for (int g2 = 0; g2 < TL::BG_PER_WAVE; ++g2) {
      const int g = wave + 8 * g2;
      const int row = 8 * g + (lane >> 3);
      const int wr = wrow_of(row);
      buse[g2] = wrow_of(8 * g) >= 0;
      boff[g2] = (uint32_t)(((size_t)(wr >= 0 ? wr : 0) * kdim + 8 * ac) * 2);
    }
  }
  int per_stage = 0;
#pragma unroll
  for (int g2 = 0; g2 < TL::AG_PER_WAVE; ++g2) per_stage += (int)ause[g2];
#pragma unroll
  for (int g2 = 0; g2 < TL::BG_PER_WAVE; ++g2) per_stage += (int)buse[g2];
  const int nst = (kdim + DBK - 1) / DBK;
  const bool half_tail = (kdim % DBK) != 0;  // last stage holds 32 k
  // Ring geometry for this tile (wave-uniform).
  const int a_chunks = ((rows + 7) >> 3) * 64;
  const int slot = a_chunks + TL::B_CHUNKS;
  const int nslots = min(TL::MAX_SLOTS, TL::LDS_CHUNKS / slot);

  auto issue = [&](int s) {
    const int k0 = s * DBK;
    const char* xs = abase + 2 * (size_t)k0;
    const char* ws = wexp + (size_t)k0 * esz;
    // Tail stage of an odd multiple of 32 (bf16 only): chunks 4..7 of a row
    // do not exist; those lanes load chunk c - 4 (64 bytes back) instead.
    const uint32_t back = (half_tail && s == nst - 1 && ac >= 4) ? 64u : 0u;
    const uint4* base = lds + (s % nslots) * slot;
#pragma unroll
    for (int g2 = 0; g2 < TL::AG_PER_WAVE; ++g2)
      if (ause[g2]) dma16(xs, aoff[g2] - back, base + (wave + 8 * g2) * 64);
#pragma unroll
    for (int g2 = 0; g2 < TL::BG_PER_WAVE; ++g2)
      if (buse[g2]) dma16(ws, boff[g2] - (FP8 ? 0u : back), base + a_chunks + (wave + 8 * g2) * 64);
  };

  constexpr int MF = kBigTileRows / 64;  // fragments per wave (5)
  f32x16_t acc[MF][2];
#pragma unroll
  for (int i = 0; i < MF; ++i)
#pragma unroll
    for (int f = 0; f < 2; ++f)
#pragma unroll
      for (int v = 0; v < 16; ++v) acc[i][f][v] = 0.f;
  // Token row of this wave's j-th fragment: fragment 2j + wm.
  auto frow = [&](int j) { return 32 * (2 * j + wm); };

  const int bbase0 = GATEUP ? 32 * wn : 64 * wn;
  const int bbase1 = GATEUP ? 128 + 32 * wn : 64 * wn + 32;
  const int brow0 = bbase0 + (lane & 31), brow1 = bbase1 + (lane & 31);
  // fp8: the two weight fragments' block scales for every 128-wide k block,
  // loaded once before the k loop (lane l holds blocks l and l+64) and read
  // per stage with v_readlane, so the loop issues no memory op besides the
  // copies it counts.
  const int kblocks = kdim >> 7;
  int scv[2][2] = {{0, 0}, {0, 0}};
  if (FP8) {
    const int wr0 = wrow_of(bbase0), wr1 = wrow_of(bbase1);
    const float* sr0 = a.wscale + ((size_t)e * (a.rows_total >> 7) + (wr0 >= 0 ? wr0 >> 7 : 0)) * kblocks;
    const float* sr1 = a.wscale + ((size_t)e * (a.rows_total >> 7) + (wr1 >= 0 ? wr1 >> 7 : 0)) * kblocks;
#pragma unroll
    for (int j = 0; j < 2; ++j) {
      const int kb = lane + 64 * j;
      scv[0][j] = (wr0 >= 0 && kb < kblocks) ? __float_as_int(sr0[kb]) : 0;
      scv[1][j] = (wr1 >= 0 && kb < kblocks) ? __float_as_int(sr1[kb]) : 0;
    }
  }
  wait_vmcnt<0>();  // every load before the copies has landed
  // 32-row fragments of this wave that hold routed rows (wave-uniform):
  // fragments 2j + wm with 32 (2j + wm) < rows.
  const int nact = __builtin_amdgcn_readfirstlane(
      max(0, min(MF, (rows - 32 * wm + 63) / 64)));

  // Multiply half kk of one stage: all LDS operand reads first, then the MFMAs.
  auto compute_half = [&](auto NA_c, int s, int kk) {
    constexpr int NA = decltype(NA_c)::value;
    const uint4* A = lds + (s % nslots) * slot;
    const uint4* B = A + a_chunks;
    bf16x8_t Bv[2][2], Av[2][NA > 0 ? NA : 1];
    if (FP8) {
      const uint4 q0 = B[swz64(brow0, 2 * kk + h)];
      const uint4 q1 = B[swz64(brow1, 2 * kk + h)];
      const int kb = (s * DBK) >> 7;
      const float s0 = __int_as_float(__builtin_amdgcn_readlane(scv[0][kb >> 6], kb & 63));
      const float s1 = __int_as_float(__builtin_amdgcn_readlane(scv[1][kb >> 6], kb & 63));
      Bv[0][0] = as_bf16x8(fp8x8_scaled_to_bf16x8(q0.x, q0.y, s0));
      Bv[1][0] = as_bf16x8(fp8x8_scaled_to_bf16x8(q0.z, q0.w, s0));
      Bv[0][1] = as_bf16x8(fp8x8_scaled_to_bf16x8(q1.x, q1.y, s1));
      Bv[1][1] = as_bf16x8(fp8x8_scaled_to_bf16x8(q1.z, q1.w, s1));
    } else {
#pragma unroll
      for (int j = 0; j < 2; ++j) {
        Bv[j][0] = as_bf16x8(B[swz128(brow0, 4 * kk + 2 * j + h)]);
        Bv[j][1] = as_bf16x8(B[swz128(brow1, 4 * kk + 2 * j + h)]);
      }
    }
#pragma unroll
    for (int j = 0; j < 2; ++j) {
      const int c = FP8 ? 4 * kk + 2 * h + j : 4 * kk + 2 * j + h;
#pragma unroll
      for (int i = 0; i < NA; ++i)
        Av[j][i] = as_bf16x8(A[swz128(frow(i) + (lane & 31), c)]);
    }
#pragma unroll
    for (int j = 0; j < 2; ++j)
#pragma unroll
      for (int i = 0; i < NA; ++i) {
        // bf16 weights: transposed tile (weights as the first operand, lane =
        // token row) for the LDS-staged epilogue; fp8 weights: direct tile
        // (lane = output column), which measured faster there.
        if (!FP8) {
          acc[i][0] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(Bv[j][0], Av[j][i], acc[i][0], 0, 0, 0);
          acc[i][1] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(Bv[j][1], Av[j][i], acc[i][1], 0, 0, 0);
        } else {
          acc[i][0] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(Av[j][i], Bv[j][0], acc[i][0], 0, 0, 0);
          acc[i][1] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(Av[j][i], Bv[j][1], acc[i][1], 0, 0, 0);
        }
      }
  };
  // Stage s: wait for its copies (younger stages stay in flight), publish,
  // queue stage s+nslots-1 into the slot freed by stage s-1, multiply. The
  // loop is instantiated per active-fragment count (straight-line code).
  auto kloop = [&](auto NA_c) {
    for (int s = 0; s < nslots - 1 && s < nst; ++s) issue(s);
    for (int s = 0; s < nst; ++s) {
      wait_vmcnt_upto(per_stage * min(nslots - 2, nst - 1 - s));
      raw_barrier();
      if (s + nslots - 1 < nst) issue(s + nslots - 1);
      compute_half(NA_c, s, 0);
      if (!(half_tail && s == nst - 1)) compute_half(NA_c, s, 1);
    }
  };
  switch (nact) {
    case 5: kloop(std::integral_constant<int, 5>{}); break;
    case 4: kloop(std::integral_constant<int, 4>{}); break;
    case 3: kloop(std::integral_constant<int, 3>{}); break;
    case 2: kloop(std::integral_constant<int, 2>{}); break;
    case 1: kloop(std::integral_constant<int, 1>{}); break;
    default: kloop(std::integral_constant<int, 0>{}); break;
  }

  if (FP8) {
    // fp8 weights, direct tile: lane = output column, 16 rows per fragment.
#pragma unroll
    for (int i = 0; i < MF; ++i) {
      if (frow(i) >= rows) continue;
#pragma unroll
      for (int v = 0; v < 16; ++v) {
        const int tr = frow(i) + 8 * (v >> 2) + 4 * h + (v & 3);
        if (tr >= rows) continue;
        uint16_t* orow = a.out + (size_t)(rowbase + tr) * a.n_out;
        if (GATEUP) {
          const int col = slice * kBigColsGateUp + 32 * wn + (lane & 31);
          if (col < a.n_out) orow[col] = f32_to_bf16(silu_f(acc[i][0][v]) * acc[i][1][v]);
        } else {
#pragma unroll
          for (int f = 0; f < 2; ++f) {
            const int col = slice * kBigColsDown + 64 * wn + 32 * f + (lane & 31);
            if (col < a.n_out) orow[col] = f32_to_bf16(acc[i][f][v]);
          }
        }
      }
    }
    return;
  }
  if (BWD) {
    // Backward of the SiLU gate for slot row s = rowbase + tr, columns j of
    // this lane (a = gate pre-activation, c = up): h = silu(a) c; dh = g Q;
    // dU = [dh c silu'(a); dh silu(a)]; g h; and <Q, h> over the lane's
    // columns, summed with the other lane of the row: one partial per row,
    // slice and wave (32 columns). Q comes in, and dU and g h go out, through
    // this wave's 10 KB of LDS (the ring is free after the barrier): Q as
    // whole 128-byte row segments (8 rows per load, chunk c of row r at
    // c ^ (r & 7)), the outputs as 64-byte row segments (16 rows per store,
    // chunk c of row r at c ^ ((r >> 2) & 3)).
    raw_barrier();
    const int pcount = 4 * a.nslices;
    uint4* sq = lds + wave * 640;  // Q: 32 rows x 8 chunks
    uint4* so = sq + 256;          // dU gate, dU up, g h: 3 x 32 rows x 4 chunks
    const int col0 = slice * kBigColsGateUp + 32 * wn;
    auto sw4 = [](int r) { return (r >> 2) & 3; };
#pragma unroll
    for (int i = 0; i < MF; ++i) {
      if (frow(i) >= rows) continue;
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const int rr = 8 * j + lane / 8, c = lane % 8;
        const int tr = frow(i) + rr, col = col0 + 4 * c;
        uint4 v = make_uint4(0u, 0u, 0u, 0u);
        if (tr < rows && col < a.n_out)
          v = *reinterpret_cast<const uint4*>(a.bq + (size_t)(rowbase + tr) * a.n_out + col);
        sq[rr * 8 + (c ^ (rr & 7))] = v;
      }
      const int lr = lane & 31;
      const int r = frow(i) + lr;
      const bool ok = r < rows;
      const size_t srow = (size_t)rowbase + (ok ? r : 0);
      const float g = ok ? a.bgate[a.perm[srow]] : 0.f;
      float part = 0.f;
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const int j = col0 + 8 * q + 4 * h;
        const uint4 qw = sq[lr * 8 + ((2 * q + h) ^ (lr & 7))];
        const float qa[4] = {__uint_as_float(qw.x), __uint_as_float(qw.y), __uint_as_float(qw.z),
                             __uint_as_float(qw.w)};
        float da[4], dc[4], hg[4];
#pragma unroll
        for (int u = 0; u < 4; ++u) {
          const float av = acc[i][0][4 * q + u], cv = acc[i][1][4 * q + u];
          const float sg = 1.0f / (1.0f + expf(-av));
          const float si = av * sg;
          const float hv = si * cv;
          if (ok && j < a.n_out) part += qa[u] * hv;
          const float dh = g * qa[u];
          da[u] = dh * cv * (sg * (1.0f + av * (1.0f - sg)));
          dc[u] = dh * si;
          hg[u] = g * hv;
        }
        const int off = lr * 4 + (q ^ sw4(lr));
        *reinterpret_cast<uint2*>(reinterpret_cast<char*>(so + off) + 8 * h) =
            make_uint2(pack_bf16x2(da[0], da[1]), pack_bf16x2(da[2], da[3]));
        *reinterpret_cast<uint2*>(reinterpret_cast<char*>(so + 128 + off) + 8 * h) =
            make_uint2(pack_bf16x2(dc[0], dc[1]), pack_bf16x2(dc[2], dc[3]));
        *reinterpret_cast<uint2*>(reinterpret_cast<char*>(so + 256 + off) + 8 * h) =
            make_uint2(pack_bf16x2(hg[0], hg[1]), pack_bf16x2(hg[2], hg[3]));
      }
      part += __shfl_xor(part, 32, kWave);
      if (ok && h == 0) a.bdgp[srow * pcount + 4 * slice + wn] = part;
#pragma unroll
      for (int j = 0; j < 2; ++j) {
        const int rr = 16 * j + lane / 4, c = lane % 4;
        const int tr = frow(i) + rr, col = col0 + 8 * c;
        if (tr < rows && col < a.n_out) {
          const size_t orow = (size_t)rowbase + tr;
          const int off = rr * 4 + (c ^ sw4(rr));
          *reinterpret_cast<uint4*>(a.bdu + orow * 2 * a.n_out + col) = so[off];
          *reinterpret_cast<uint4*>(a.bdu + orow * 2 * a.n_out + a.n_out + col) = so[128 + off];
          *reinterpret_cast<uint4*>(a.out + orow * a.n_out + col) = so[256 + off];
        }
      }
    }
    return;
  }
  // bf16 weights. The accumulators hold the transposed tile: lane l has token row
  // frow(i) + l % 32 and, per fragment, the 4 consecutive output columns
  // 8 q + 4 (l / 32) + [0, 4) for q = 0..3. Each 32-row fragment goes out
  // through this wave's 4 KB of LDS (the ring is free after the barrier), so
  // a global store instruction writes whole row segments of the wave's
  // columns: 128 bytes (down, 64 columns) or 64 bytes (gate/up, 32 columns).
  // Row r's 16-byte chunk c sits at c ^ ((r >> 1) & 7) (down, 8 chunks per
  // row) or c ^ ((r >> 2) & 3) (gate/up, 4 chunks): conflict-free both ways.
  if (GATEUP && a.usave != nullptr) {
    // u = [a; c] of every row for the backward: 16-byte stores, 4 columns each
#pragma unroll
    for (int i = 0; i < MF; ++i) {
      const int r = frow(i) + (lane & 31);
      if (frow(i) >= rows || r >= rows) continue;
      float* u = a.usave + (size_t)(rowbase + r) * 2 * a.n_out;
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const int j = slice * kBigColsGateUp + 32 * wn + 8 * q + 4 * h;
        if (j >= a.n_out) continue;
        const f32x16_t& g = acc[i][0];
        const f32x16_t& v = acc[i][1];
        *reinterpret_cast<float4*>(u + j) = make_float4(g[4 * q], g[4 * q + 1], g[4 * q + 2], g[4 * q + 3]);
        *reinterpret_cast<float4*>(u + a.n_out + j) =
            make_float4(v[4 * q], v[4 * q + 1], v[4 * q + 2], v[4 * q + 3]);
      }
    }
  }
  raw_barrier();
  constexpr int CPR = GATEUP ? 4 : 8;  // 16-byte chunks per staged row
  uint4* st = lds + wave * 256;
  auto sw_of = [&](int r) { return GATEUP ? ((r >> 2) & 3) : ((r >> 1) & 7); };
  const int col0 = GATEUP ? slice * kBigColsGateUp + 32 * wn : slice * kBigColsDown + 64 * wn;
#pragma unroll
  for (int i = 0; i < MF; ++i) {
    if (frow(i) >= rows) continue;
    const int r = lane & 31;
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      if (GATEUP) {
        const f32x16_t& g = acc[i][0];
        const f32x16_t& u = acc[i][1];
        *reinterpret_cast<uint2*>(reinterpret_cast<char*>(st + r * CPR + (q ^ sw_of(r))) + 8 * h) =
            make_uint2(pack_bf16x2(silu_f(g[4 * q]) * u[4 * q], silu_f(g[4 * q + 1]) * u[4 * q + 1]),
                       pack_bf16x2(silu_f(g[4 * q + 2]) * u[4 * q + 2],
                                   silu_f(g[4 * q + 3]) * u[4 * q + 3]));
      } else {
#pragma unroll
        for (int f = 0; f < 2; ++f) {
          const f32x16_t& y = acc[i][f];
          const int c = 4 * f + q;
          *reinterpret_cast<uint2*>(reinterpret_cast<char*>(st + r * CPR + (c ^ sw_of(r))) + 8 * h) =
              make_uint2(pack_bf16x2(y[4 * q], y[4 * q + 1]), pack_bf16x2(y[4 * q + 2], y[4 * q + 3]));
        }
      }
    }
    constexpr int RPI = 64 / CPR;  // rows per read instruction
#pragma unroll
    for (int j = 0; j < 32 / RPI; ++j) {
      const int rr = RPI * j + lane / CPR, c = lane % CPR;
      const uint4 v = st[rr * CPR + (c ^ sw_of(rr))];
      const int tr = frow(i) + rr, col = col0 + 8 * c;
      if (tr < rows && col < a.n_out)
        *reinterpret_cast<uint4*>(a.out + (size_t)(rowbase + tr) * a.n_out + col) = v;
    }
  }
}

// ===========================================================================
// large-M kernel with fp8 weights and fp8 activations
//
// Same tiles, tile order and direct-to-LDS ring as above, with both operands
// E4M3FN codes: a stage is 128 k = one whole 128-byte line of every x (or H)
// row and every weight row (eight lanes per row, eight rows per copy), and
// one 128-wide weight-scale block. Per stage and 32x32 fragment pair, two
// v_mfma_scale_f32_32x32x64_f8f6f4 (unit E8M0 scales) accumulate the raw
// code products of the block into a fresh fp32 tile T, then acc += T * s_w
// (the weight block scale, a wave-uniform value). The per-row activation
// scale multiplies the finished accumulator in the epilogue.
//
// MFMA operand (both sides identically): lane l supplies row (l & 31) and
// bytes 32 (l >> 5) + [0, 32) of the 64-wide k step, i.e. chunks
// 4 m + 2 h and 4 m + 2 h + 1 of the stage's 128-byte row for step m; the
// 128-byte-row swizzle c ^ ((r >> 1) & 7) keeps each 16-lane read
// conflict-free.
// ===========================================================================
typedef int i32x8_t __attribute__((ext_vector_type(8)));

__device__ __forceinline__ i32x8_t as_i32x8(uint4 lo, uint4 hi) {
  i32x8_t r;
  r[0] = lo.x; r[1] = lo.y; r[2] = lo.z; r[3] = lo.w;
  r[4] = hi.x; r[5] = hi.y; r[6] = hi.z; r[7] = hi.w;
  return r;
}

template <bool GATEUP>
__global__ __launch_bounds__(512) void gemm_big_a8_kernel(GemmArgs a) {
  constexpr int LDS_CHUNKS = 9216;       // 144 KB
  constexpr int MAX_SLOTS = 3;
  constexpr int B_CHUNKS = 256 * 8;      // 256 weight rows x 128 B
  constexpr int ROWS = kBigTileRows;     // 320 token rows
  constexpr int AG = ROWS / 8 / 8;       // x copy groups per wave (5)
  constexpr int BG = 4;                  // weight copy groups per wave
  constexpr int MF = ROWS / 64;          // token fragments per wave (5)
  constexpr int SK = 128;                // k per stage
  __shared__ uint4 lds[LDS_CHUNKS];
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int wm = wave >> 2, wn = wave & 3;
  const int h = lane >> 5, lrow = lane & 31;
  const int kdim = a.kdim;  // elements = bytes per row

  const int total = a.meta[1] * a.nslices;
  const int per_xcd = (total + 7) >> 3;
  const int xcd = blockIdx.x & 7, pos = blockIdx.x >> 3;
  if (pos >= per_xcd) return;
  const int L = xcd * per_xcd + pos;
  if (L >= total) return;
  int lo = 0, hi = a.n_ffn - 1;
  while (lo < hi) {
    const int mid = (lo + hi + 1) >> 1;
    if (a.mt_prefix[mid] * a.nslices <= L) lo = mid; else hi = mid - 1;
  }
  const int e = lo;
  const int mt = a.mt_prefix[e + 1] - a.mt_prefix[e];
  const int local = L - a.mt_prefix[e] * a.nslices;
  const int slice = local / mt, m = local - slice * mt;
  const int cnt = a.counts[e];
  const int r0 = (int)((long long)m * cnt / mt);
  const int rows = (int)((long long)(m + 1) * cnt / mt) - r0;
  const int rowbase = a.offsets[e] + r0;

  auto wrow_of = [&](int j) -> int {
    if (GATEUP) {
      const int col = slice * kBigColsGateUp + (j & 127);
      if (col >= a.n_out) return -1;
      return j < 128 ? col : a.n_out + col;
    } else {
      const int col = slice * kBigColsDown + j;
      return col < a.n_out ? col : -1;
    }
  };

  // Copies: 8-row groups w + 8 g2 of the x (or H) codes and of the weight
  // codes, eight lanes per 128-byte row; byte offsets from the operand bases.
  uint32_t aoff[AG], boff[BG];
  bool ause[AG], buse[BG];
  const char* wexp = static_cast<const char*>(a.w) + (size_t)e * a.rows_total * kdim;
  const char* abase = reinterpret_cast<const char*>(a.src8) + (GATEUP ? 0 : (size_t)rowbase * kdim);
  const int ac = (lane & 7) ^ ((4 * (wave & 1) + (lane >> 4)) & 7);
#pragma unroll
  for (int g2 = 0; g2 < AG; ++g2) {
    const int g = wave + 8 * g2;
    const int row = 8 * g + (lane >> 3);
    ause[g2] = 8 * g < rows;
    const int rr = row < rows ? row : 0;
    const size_t srow = GATEUP ? (size_t)(a.perm[rowbase + rr] / a.topk) : (size_t)rr;
    aoff[g2] = (uint32_t)(srow * kdim + 16 * ac);
  }
#pragma unroll
  for (int g2 = 0; g2 < BG; ++g2) {
    const int g = wave + 8 * g2;
    const int row = 8 * g + (lane >> 3);
    const int wr = wrow_of(row);
    buse[g2] = wrow_of(8 * g) >= 0;
    boff[g2] = (uint32_t)((size_t)(wr >= 0 ? wr : 0) * kdim + 16 * ac);
  }
  int per_stage = 0;
#pragma unroll
  for (int g2 = 0; g2 < AG; ++g2) per_stage += (int)ause[g2];
#pragma unroll
  for (int g2 = 0; g2 < BG; ++g2) per_stage += (int)buse[g2];
  const int nst = kdim / SK;
  const int a_chunks = ((rows + 7) >> 3) * 64;
  const int slot = a_chunks + B_CHUNKS;
  const int nslots = min(MAX_SLOTS, LDS_CHUNKS / slot);

  auto issue = [&](int s) {
    const char* xs = abase + (size_t)s * SK;
    const char* ws = wexp + (size_t)s * SK;
    const uint4* base = lds + (s % nslots) * slot;
#pragma unroll
    for (int g2 = 0; g2 < BG; ++g2)
      if (buse[g2]) dma16(ws, boff[g2], base + a_chunks + (wave + 8 * g2) * 64);
#pragma unroll
    for (int g2 = 0; g2 < AG; ++g2)
      if (ause[g2]) dma16(xs, aoff[g2], base + (wave + 8 * g2) * 64);
  };

  f32x16_t acc[MF][2];
#pragma unroll
  for (int i = 0; i < MF; ++i)
#pragma unroll
    for (int f = 0; f < 2; ++f)
#pragma unroll
      for (int v = 0; v < 16; ++v) acc[i][f][v] = 0.f;
  auto frow = [&](int j) { return 32 * (2 * j + wm); };
  const int bbase0 = GATEUP ? 32 * wn : 64 * wn;
  const int bbase1 = GATEUP ? 128 + 32 * wn : 64 * wn + 32;

  // Weight block scales for every 128-wide k block (one per stage) of the
  // tile's two 128-row weight blocks (gate/up: the gate and the up block of
  // the slice; down: blocks 2 slice and 2 slice + 1), staged in LDS once.
  // Wave-uniform reads per stage: fragment f uses row sq[f].
  __shared__ float sscale[2][128];
  const int kblocks = kdim >> 7;
  for (int j = tid; j < 2 * kblocks; j += 512) {
    const int q = j / kblocks, kb = j - q * kblocks;
    const int brow = GATEUP ? (q ? (a.n_out >> 7) + slice : slice) : 2 * slice + q;
    sscale[q][kb] = brow < (a.rows_total >> 7)
                        ? a.wscale[((size_t)e * (a.rows_total >> 7) + brow) * kblocks + kb]
                        : 0.f;
  }
  const int sq0 = GATEUP ? 0 : (wn >> 1), sq1 = GATEUP ? 1 : (wn >> 1);
  wait_vmcnt<0>();
  __syncthreads();
  const int nact = __builtin_amdgcn_readfirstlane(
      max(0, min(MF, (rows - 32 * wm + 63) / 64)));
  const int sw = (lrow >> 1) & 7;  // swizzle term of every row this lane reads

  auto compute = [&](auto NA_c, int s) {
    constexpr int NA = decltype(NA_c)::value;
    const uint4* A = lds + (s % nslots) * slot + frow(0) * 8 + lrow * 8;
    const uint4* B = lds + (s % nslots) * slot + a_chunks + lrow * 8;
    const float s0 = sscale[sq0][s], s1 = sscale[sq1][s];
    i32x8_t Bv[2][2];
#pragma unroll
    for (int mm = 0; mm < 2; ++mm) {
      const int c0 = (4 * mm + 2 * h) ^ sw, c1 = (4 * mm + 2 * h + 1) ^ sw;
      Bv[mm][0] = as_i32x8(B[bbase0 * 8 + c0], B[bbase0 * 8 + c1]);
      Bv[mm][1] = as_i32x8(B[bbase1 * 8 + c0], B[bbase1 * 8 + c1]);
    }
#pragma unroll
    for (int i = 0; i < NA; ++i) {
      i32x8_t Av[2];
#pragma unroll
      for (int mm = 0; mm < 2; ++mm) {
        const int c0 = (4 * mm + 2 * h) ^ sw, c1 = (4 * mm + 2 * h + 1) ^ sw;
        const int rb = (frow(i) - frow(0)) * 8;
        Av[mm] = as_i32x8(A[rb + c0], A[rb + c1]);
      }
#pragma unroll
      for (int f = 0; f < 2; ++f) {
        f32x16_t t;
#pragma unroll
        for (int v = 0; v < 16; ++v) t[v] = 0.f;
        // transposed tile (weights as the first operand): lane = token row
        t = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(Bv[0][f], Av[0], t, 0, 0, 0, 127, 0, 127);
        t = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(Bv[1][f], Av[1], t, 0, 0, 0, 127, 0, 127);
        const float sc = f ? s1 : s0;
#pragma unroll
        for (int v = 0; v < 16; ++v) acc[i][f][v] = __builtin_fmaf(t[v], sc, acc[i][f][v]);
      }
    }
  };
  auto kloop = [&](auto NA_c) {
    for (int s = 0; s < nslots - 1 && s < nst; ++s) issue(s);
    for (int s = 0; s < nst; ++s) {
      wait_vmcnt_upto(per_stage * min(nslots - 2, nst - 1 - s));
      raw_barrier();
      if (s + nslots - 1 < nst) issue(s + nslots - 1);
      compute(NA_c, s);
    }
  };
  switch (nact) {
    case 5: kloop(std::integral_constant<int, 5>{}); break;
    case 4: kloop(std::integral_constant<int, 4>{}); break;
    case 3: kloop(std::integral_constant<int, 3>{}); break;
    case 2: kloop(std::integral_constant<int, 2>{}); break;
    case 1: kloop(std::integral_constant<int, 1>{}); break;
    default: kloop(std::integral_constant<int, 0>{}); break;
  }

  // Epilogue: the per-row activation scale, then SiLU-gating (gate/up) or
  // the store of Y (down). Transposed tile as in the bf16 kernel: lane =
  // token row, 4 consecutive output columns per fragment and q.
#pragma unroll
  for (int i = 0; i < MF; ++i) {
    const int tr = frow(i) + lrow;
    if (frow(i) >= rows || tr >= rows) continue;
    const float sa = GATEUP ? a.ascale[a.perm[rowbase + tr] / a.topk] : a.ascale[rowbase + tr];
    uint16_t* orow = a.out + (size_t)(rowbase + tr) * a.n_out;
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      if (GATEUP) {
        const int col = slice * kBigColsGateUp + 32 * wn + 8 * q + 4 * h;
        if (col < a.n_out) {
          float o[4];
#pragma unroll
          for (int r = 0; r < 4; ++r)
            o[r] = silu_f(acc[i][0][4 * q + r] * sa) * (acc[i][1][4 * q + r] * sa);
          *reinterpret_cast<uint2*>(orow + col) =
              make_uint2(pack_bf16x2(o[0], o[1]), pack_bf16x2(o[2], o[3]));
        }
      } else {
#pragma unroll
        for (int f = 0; f < 2; ++f) {
          const int col = slice * kBigColsDown + 64 * wn + 32 * f + 8 * q + 4 * h;
          const f32x16_t& y = acc[i][f];
          if (col < a.n_out)
            *reinterpret_cast<uint2*>(orow + col) =
                make_uint2(pack_bf16x2(y[4 * q] * sa, y[4 * q + 1] * sa),
                           pack_bf16x2(y[4 * q + 2] * sa, y[4 * q + 3] * sa));
        }
      }
    }
  }
}

// ===========================================================================
// launchers
// ===========================================================================
void launch_gemm_big(const GemmArgs& a, bool gateup, bool fp8, int grid, hipStream_t s) {
  if (gateup) {
    if (fp8) gemm_big_dma_kernel<true, true><<<grid, 512, 0, s>>>(a);
    else gemm_big_dma_kernel<true, false><<<grid, 512, 0, s>>>(a);
  } else {
    if (fp8) gemm_big_dma_kernel<false, true><<<grid, 512, 0, s>>>(a);
    else gemm_big_dma_kernel<false, false><<<grid, 512, 0, s>>>(a);
  }
}

void launch_gemm_big_bwd_u(const GemmArgs& a, int grid, hipStream_t s) {
  gemm_big_dma_kernel<true, false, true><<<grid, 512, 0, s>>>(a);
}

void launch_gemm_big_a8(const GemmArgs& a, bool gateup, int grid, hipStream_t s) {
  if (gateup) gemm_big_a8_kernel<true><<<grid, 512, 0, s>>>(a);
  else gemm_big_a8_kernel<false><<<grid, 512, 0, s>>>(a);
}

}  // namespace lcmoe
