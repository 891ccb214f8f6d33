// Grouped expert GEMMs over the FFN-routed rows only.
//
// Method: "LongCat-Flash" (llm-wiki entity page), section 2.1: only the
// FFN experts cost FLOPs; section 1 table: expert intermediate size 2048.
// Expert e (SiLU-gated, W13 = [gate rows; up rows] [2I][d], W2 [d][I]):
//   gate/up:  H = silu(X_e W_gate^T) * (X_e W_up^T)   [rows_e][I], bf16
//   down:     Y = H W2^T                               [rows_e][d], bf16
// with X_e the rows of x gathered through the expert's slots (perm).
//
// Two kernels, picked per expert on the device from its routed row count:
//  * small-M (1..32 rows, decode batches): weights stream from HBM straight
//    into MFMA A-operand registers (v_mfma_f32_16x16x32_bf16, weights as the
//    16-row side, tokens as the 16-column side staged in LDS). Weight bytes
//    dominate; every weight of a touched expert is read once.
//  * large-M (33+ rows, prefill batches): LDS-tiled, 256 token rows x 256
//    weight rows x 64 k per stage, 8 waves (2 x 4), v_mfma_f32_32x32x16_bf16,
//    each weight tile read once per M-tile; the M-tiles of an expert and
//    its column slices are adjacent on one XCD (blockIdx % 8) so the x rows
//    and repeated weight tiles are shared through that XCD's L2.
// fp8 (E4M3FN, one fp32 scale per 128x128 block) weights are converted in
// registers: bf16(fl32(q) * s), then the same bf16 MFMA.
#include <type_traits>

#include "common.h"
#include "kernels.h"

namespace lcmoe {

__device__ __forceinline__ float silu_f(float g) { return g / (1.0f + expf(-g)); }

// ===========================================================================
// small-M kernel
// ===========================================================================
constexpr int kSmallLdsChunks = 4096;  // 64 KB of staged token rows
// Token rows are staged with a pitch of 128 or 256 chunks (a multiple of
// the 256-byte bank window), chunk c of row r at c ^ (r & 15): the 16 rows
// one MFMA operand read touches at the same chunk hit 16 distinct slots.

template <bool GATEUP, bool FP8>
__global__ __launch_bounds__(256) void gemm_small_kernel(GemmArgs a) {
  __shared__ uint4 sX[kSmallLdsChunks];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int lr = lane & 15, lq = lane >> 4;
  const int total = a.meta[0] * a.nslices;
  const int kdim = a.kdim;

  for (int L = blockIdx.x; L < total; L += gridDim.x) {
    const int e = a.small_list[L / a.nslices];
    const int slice = L % a.nslices;
    const int rows = a.counts[e];
    const int row0 = a.offsets[e];
    const int ncb = rows <= 16 ? 1 : 2;
    const int kc = (kSmallLdsChunks * 8) / (16 * ncb);  // k elements per LDS fill
    const int cpr = kc >> 3;                              // LDS row pitch (chunks)

    // Two 16-row weight fragments per wave.
    int fbase0, fbase1, ocol0;
    if (GATEUP) {
      ocol0 = slice * kSmallColsGateUp + wave * 16;
      fbase0 = ocol0;             // gate rows
      fbase1 = a.n_out + ocol0;   // matching up rows
    } else {
      ocol0 = slice * kSmallColsDown + wave * 32;
      fbase0 = ocol0;
      fbase1 = ocol0 + 16;
    }
    const bool active = ocol0 < a.n_out;  // n_out % 32 == 0: whole fragments valid

    f32x4_t acc[2][2];
#pragma unroll
    for (int f = 0; f < 2; ++f)
#pragma unroll
      for (int c = 0; c < 2; ++c) acc[f][c] = f32x4_t{0.f, 0.f, 0.f, 0.f};

    const size_t wrow0 = (size_t)e * a.rows_total + (active ? fbase0 : 0) + lr;
    const size_t wrow1 = (size_t)e * a.rows_total + (active ? fbase1 : 0) + lr;
    const int sblk0 = (active ? fbase0 : 0) >> 7, sblk1 = (active ? fbase1 : 0) >> 7;

    // Weight fragments for one 128-wide k step: four 16-byte loads per
    // fragment (bf16), or two (fp8, 16 codes each).
    auto load_w = [&](uint4 (&wv)[2][4], int kb) {
      if (FP8) {
        const uint8_t* w8 = static_cast<const uint8_t*>(a.w);
#pragma unroll
        for (int j = 0; j < 2; ++j) {
          wv[0][j] = *reinterpret_cast<const uint4*>(w8 + wrow0 * kdim + kb + 64 * j + 16 * lq);
          wv[1][j] = *reinterpret_cast<const uint4*>(w8 + wrow1 * kdim + kb + 64 * j + 16 * lq);
        }
      } else {
        const uint16_t* w16 = static_cast<const uint16_t*>(a.w);
#pragma unroll
        for (int s = 0; s < 4; ++s) {
          const int k = kb + 32 * s + 8 * lq;
          if (kb + 32 * s < kdim) {
            wv[0][s] = *reinterpret_cast<const uint4*>(w16 + wrow0 * kdim + k);
            wv[1][s] = *reinterpret_cast<const uint4*>(w16 + wrow1 * kdim + k);
          }
        }
      }
    };
    auto compute = [&](const uint4 (&wv)[2][4], int kb, int kc0) {
      float sc0 = 1.f, sc1 = 1.f;
      if (FP8) {
        const int kblocks = kdim >> 7;
        const size_t sbase = (size_t)e * (a.rows_total >> 7);
        sc0 = a.wscale[(sbase + sblk0) * kblocks + (kb >> 7)];
        sc1 = a.wscale[(sbase + sblk1) * kblocks + (kb >> 7)];
      }
      const int cb0 = (kb - kc0) >> 3;
#pragma unroll
      for (int s = 0; s < 4; ++s) {
        if (kb + 32 * s >= kdim) break;
        bf16x8_t A0, A1;
        int ch;
        if (FP8) {
          const int j = s >> 1, h = s & 1;
          A0 = as_bf16x8(fp8x8_scaled_to_bf16x8(h ? wv[0][j].z : wv[0][j].x,
                                                h ? wv[0][j].w : wv[0][j].y, sc0));
          A1 = as_bf16x8(fp8x8_scaled_to_bf16x8(h ? wv[1][j].z : wv[1][j].x,
                                                h ? wv[1][j].w : wv[1][j].y, sc1));
          ch = cb0 + 8 * j + 2 * lq + h;
        } else {
          A0 = as_bf16x8(wv[0][s]);
          A1 = as_bf16x8(wv[1][s]);
          ch = cb0 + 4 * s + lq;
        }
#pragma unroll
        for (int c = 0; c < 2; ++c) {
          if (c < ncb) {
            const int r = 16 * c + lr;
            const bf16x8_t B = as_bf16x8(sX[r * cpr + (ch ^ (r & 15))]);
            acc[0][c] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(A0, B, acc[0][c], 0, 0, 0);
            acc[1][c] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(A1, B, acc[1][c], 0, 0, 0);
          }
        }
      }
    };

    for (int kc0 = 0; kc0 < kdim; kc0 += kc) {
      const int kcl = min(kc, kdim - kc0);
      const int ccl = kcl >> 3;
      __syncthreads();  // previous LDS fill fully consumed
      for (int id = tid; id < rows * ccl; id += 256) {
        const int r = id / ccl, c = id - r * ccl;
        const uint16_t* srow;
        if (GATEUP)
          srow = a.src + (size_t)(a.perm[row0 + r] / a.topk) * kdim;
        else
          srow = a.src + (size_t)(row0 + r) * kdim;
        sX[r * cpr + (c ^ (r & 15))] = *reinterpret_cast<const uint4*>(srow + kc0 + 8 * c);
      }
      __syncthreads();
      if (active) {
        const int kend = kc0 + kcl;
        uint4 w0[2][4], w1[2][4];
        load_w(w0, kc0);
        for (int kb = kc0; kb < kend; kb += 256) {
          if (kb + 128 < kend) load_w(w1, kb + 128);
          compute(w0, kb, kc0);
          if (kb + 128 < kend) {
            if (kb + 256 < kend) load_w(w0, kb + 256);
            compute(w1, kb + 128, kc0);
          }
        }
      }
    }

    if (active) {
#pragma unroll
      for (int c = 0; c < 2; ++c) {
        const int r = 16 * c + lr;
        if (c < ncb && r < rows) {
          if (GATEUP) {
            const int col = ocol0 + 4 * lq;
            float h[4];
#pragma unroll
            for (int v = 0; v < 4; ++v) h[v] = silu_f(acc[0][c][v]) * acc[1][c][v];
            *reinterpret_cast<uint2*>(a.out + (size_t)(row0 + r) * a.n_out + col) =
                make_uint2(pack_bf16x2(h[0], h[1]), pack_bf16x2(h[2], h[3]));
          } else {
#pragma unroll
            for (int f = 0; f < 2; ++f) {
              const int col = ocol0 + 16 * f + 4 * lq;
              *reinterpret_cast<uint2*>(a.out + (size_t)(row0 + r) * a.n_out + col) =
                  make_uint2(pack_bf16x2(acc[f][c][0], acc[f][c][1]),
                             pack_bf16x2(acc[f][c][2], acc[f][c][3]));
            }
          }
        }
      }
    }
  }
}

// ===========================================================================
// large-M kernel
// ===========================================================================
constexpr int BK = 64;

template <bool GATEUP, bool FP8>
__global__ __launch_bounds__(512) void gemm_big_kernel(GemmArgs a) {
  __shared__ uint4 sA[2][256 * 8];
  __shared__ uint4 sB[2][256 * 8];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int wm = wave >> 2, wn = wave & 3;
  const int kdim = a.kdim;

  // Tile order (expert, column slice, M-tile); each XCD takes a contiguous
  // run of that order so neighbouring tiles share its L2.
  const int total = a.meta[1] * a.nslices;
  const int per = (total + 7) >> 3;
  const int xcd = blockIdx.x & 7, pos = blockIdx.x >> 3;
  if (pos >= per) return;
  const int L = xcd * per + pos;
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

  // Per-thread load assignment: A and bf16 B: rows (tid>>3)+64u, chunk tid&7.
  const int lc = tid & 7;
  const uint16_t* asrc[4];
  bool aval[4];
#pragma unroll
  for (int u = 0; u < 4; ++u) {
    const int r = (tid >> 3) + 64 * u;
    aval[u] = r < rows;
    const int rr = aval[u] ? r : 0;
    if (GATEUP)
      asrc[u] = a.src + (size_t)(a.perm[rowbase + rr] / a.topk) * kdim + 8 * lc;
    else
      asrc[u] = a.src + (size_t)(rowbase + rr) * kdim + 8 * lc;
  }
  auto wrow_of = [&](int j) -> int {  // LDS B row -> weight row (or -1)
    if (GATEUP) {
      const int col = slice * kBigColsGateUp + (j & 127);
      if (col >= a.n_out) return -1;
      return j < 128 ? col : a.n_out + col;
    } else {
      const int col = slice * kBigColsDown + j;
      return col < a.n_out ? col : -1;
    }
  };
  constexpr int NB = FP8 ? 2 : 4;
  const void* bsrc[NB];
  bool bval[NB];
  int bsblk[NB];
#pragma unroll
  for (int u = 0; u < NB; ++u) {
    const int j = FP8 ? (tid >> 2) + 128 * u : (tid >> 3) + 64 * u;
    const int wr = wrow_of(j);
    bval[u] = wr >= 0;
    const size_t wrow = (size_t)e * a.rows_total + (bval[u] ? wr : 0);
    bsblk[u] = (bval[u] ? wr : 0) >> 7;
    if (FP8)
      bsrc[u] = static_cast<const uint8_t*>(a.w) + wrow * kdim + 16 * (tid & 3);
    else
      bsrc[u] = static_cast<const uint16_t*>(a.w) + wrow * kdim + 8 * lc;
  }

  // Two register stages in flight (stage s lives in R[s & 1]) on top of the
  // two LDS buffers: while stage s is multiplied out of LDS, stages s+1 and
  // s+2 are on their way from memory.
  uint4 ra[2][4], rb[2][NB];
  auto load_stage = [&](int r, int k0) {
#pragma unroll
    for (int u = 0; u < 4; ++u)
      ra[r][u] = (aval[u] && k0 + 8 * lc < kdim)
                     ? *reinterpret_cast<const uint4*>(asrc[u] + k0)
                     : make_uint4(0, 0, 0, 0);
#pragma unroll
    for (int u = 0; u < NB; ++u) {
      if (FP8)
        rb[r][u] = bval[u]
                       ? *reinterpret_cast<const uint4*>(static_cast<const uint8_t*>(bsrc[u]) + k0)
                       : make_uint4(0, 0, 0, 0);
      else
        rb[r][u] = (bval[u] && k0 + 8 * lc < kdim)
                       ? *reinterpret_cast<const uint4*>(static_cast<const uint16_t*>(bsrc[u]) + k0)
                       : make_uint4(0, 0, 0, 0);
    }
  };
  auto store_stage = [&](int r, int buf, int k0) {
#pragma unroll
    for (int u = 0; u < 4; ++u) sA[buf][swz128((tid >> 3) + 64 * u, lc)] = ra[r][u];
    if (FP8) {
      const int kblocks = kdim >> 7;
      const size_t sbase = (size_t)e * (a.rows_total >> 7);
#pragma unroll
      for (int u = 0; u < NB; ++u) {
        const int j = (tid >> 2) + 128 * u, c4 = tid & 3;
        const float sc = bval[u] ? a.wscale[(sbase + bsblk[u]) * kblocks + (k0 >> 7)] : 0.f;
        sB[buf][swz128(j, 2 * c4)] = fp8x8_scaled_to_bf16x8(rb[r][u].x, rb[r][u].y, sc);
        sB[buf][swz128(j, 2 * c4 + 1)] = fp8x8_scaled_to_bf16x8(rb[r][u].z, rb[r][u].w, sc);
      }
    } else {
#pragma unroll
      for (int u = 0; u < NB; ++u) sB[buf][swz128((tid >> 3) + 64 * u, lc)] = rb[r][u];
    }
  };

  f32x16_t acc[4][2];
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int f = 0; f < 2; ++f)
#pragma unroll
      for (int v = 0; v < 16; ++v) acc[i][f][v] = 0.f;

  const int brow0 = GATEUP ? 32 * wn + (lane & 31) : 64 * wn + (lane & 31);
  const int brow1 = GATEUP ? 128 + 32 * wn + (lane & 31) : 64 * wn + 32 + (lane & 31);
  const int nst = (kdim + BK - 1) / BK;

  auto compute_stage = [&](int buf) {
#pragma unroll
    for (int s = 0; s < 4; ++s) {
      const int chunk = 2 * s + (lane >> 5);
      const bf16x8_t B0 = as_bf16x8(sB[buf][swz128(brow0, chunk)]);
      const bf16x8_t B1 = as_bf16x8(sB[buf][swz128(brow1, chunk)]);
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        if (wm * 128 + 32 * i < rows) {
          const bf16x8_t A = as_bf16x8(sA[buf][swz128(wm * 128 + 32 * i + (lane & 31), chunk)]);
          acc[i][0] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(A, B0, acc[i][0], 0, 0, 0);
          acc[i][1] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(A, B1, acc[i][1], 0, 0, 0);
        }
      }
    }
  };
  // One pipeline step: stage st computes from LDS[p], stage st+2 is requested
  // into R[p], stage st+1 (requested one step earlier) moves R[q] -> LDS[q].
  auto pipe_step = [&](int st, int p) {
    const int q = p ^ 1;
    if (st + 2 < nst) load_stage(p, (st + 2) * BK);
    compute_stage(p);
    if (st + 1 < nst) store_stage(q, q, (st + 1) * BK);
    __syncthreads();
  };

  load_stage(0, 0);
  if (nst > 1) load_stage(1, BK);
  store_stage(0, 0, 0);
  __syncthreads();
  for (int st = 0; st < nst; st += 2) {
    pipe_step(st, 0);
    if (st + 1 < nst) pipe_step(st + 1, 1);
  }

#pragma unroll
  for (int i = 0; i < 4; ++i) {
    if (wm * 128 + 32 * i >= rows) continue;
#pragma unroll
    for (int v = 0; v < 16; ++v) {
      const int tr = wm * 128 + 32 * i + 8 * (v >> 2) + 4 * (lane >> 5) + (v & 3);
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
}

// ===========================================================================
// large-M kernel, bf16 weights: direct-to-LDS pipeline
//
// Tile 256 token rows x 256 weight rows; the k loop runs in stages of 32.
// Both operands move HBM -> LDS with global_load_lds_dwordx4 (no register
// staging), four LDS stages, three in flight while the fourth is multiplied.
// LDS rows are 64 bytes (32 bf16); chunk c of row r is stored at
// c ^ ((r >> 2) & 3), so the sixteen rows a 32x32x16 operand read touches
// per LDS cycle land in distinct bank slots. A DMA instruction fills 16 rows
// (1 KB): lane l writes row l/4, physical chunk l%4, and therefore loads
// logical chunk (l%4) ^ ((row >> 2) & 3) of its row.
//
// Each wave waits for its own copies of a stage (s_waitcnt vmcnt with the
// count of its copies still allowed in flight) and a raw s_barrier then
// publishes the stage to all waves; no fence that would drain the pipeline.
// ===========================================================================
constexpr int DBK = 32;  // k per pipeline stage

template <int N>
__device__ __forceinline__ void wait_vmcnt() {
  // gfx9 s_waitcnt: vmcnt[3:0], expcnt[6:4], lgkmcnt[11:8], vmcnt[5:4] at [15:14]
  __builtin_amdgcn_s_waitcnt((N & 15) | (7 << 4) | (15 << 8) | ((N >> 4) << 14));
}
// Wait until at most n (0..8) of this wave's vector memory operations remain.
__device__ __forceinline__ void wait_vmcnt_upto8(int n) {
  switch (n) {
    case 0: wait_vmcnt<0>(); break;
    case 1: wait_vmcnt<1>(); break;
    case 2: wait_vmcnt<2>(); break;
    case 3: wait_vmcnt<3>(); break;
    case 4: wait_vmcnt<4>(); break;
    case 5: wait_vmcnt<5>(); break;
    case 6: wait_vmcnt<6>(); break;
    case 7: wait_vmcnt<7>(); break;
    default: wait_vmcnt<8>(); break;
  }
}
__device__ __forceinline__ void raw_barrier() {
  asm volatile("" ::: "memory");
  __builtin_amdgcn_s_barrier();
  asm volatile("" ::: "memory");
}
// One global_load_lds_dwordx4: lane l copies 16 bytes from g into LDS at
// lds + 16*l. Issued as inline asm so the compiler does not track it: every
// wait on these copies is the explicit wait_vmcnt above. M0 (the LDS base of
// the copy) is written here and used by nothing else in these kernels.
__device__ __forceinline__ void dma16(const void* g, const uint4* lds) {
  const uint32_t l = (uint32_t)__builtin_amdgcn_readfirstlane((int)(uint32_t)(uintptr_t)lds);
  asm volatile("s_mov_b32 m0, %1\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %0, off"
               :: "v"(g), "s"(l) : "memory");
}
// 64-byte LDS rows: chunk c of row r lives at c ^ ((r >> 2) & 3).
__device__ __forceinline__ int swz64(int row, int chunk) {
  return row * 4 + (chunk ^ ((row >> 2) & 3));
}

template <bool GATEUP>
__global__ __launch_bounds__(512) void gemm_big_dma_kernel(GemmArgs a) {
  __shared__ uint4 sA0[1024], sA1[1024], sA2[1024], sA3[1024];
  __shared__ uint4 sB0[1024], sB1[1024], sB2[1024], sB3[1024];
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int wm = wave >> 2, wn = wave & 3;
  const int kdim = a.kdim;

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

  auto wrow_of = [&](int j) -> int {  // LDS B row -> weight row (or -1)
    if (GATEUP) {
      const int col = slice * kBigColsGateUp + (j & 127);
      if (col >= a.n_out) return -1;
      return j < 128 ? col : a.n_out + col;
    } else {
      const int col = slice * kBigColsDown + j;
      return col < a.n_out ? col : -1;
    }
  };

  // Copy assignment: wave w fills row groups w and w+8 (16 rows each) of
  // both operands; groups wholly outside the valid rows are skipped.
  const uint16_t* w16 = static_cast<const uint16_t*>(a.w);
  const uint16_t* asrc[2];
  const uint16_t* bsrc[2];
  bool ause[2], buse[2];
#pragma unroll
  for (int h = 0; h < 2; ++h) {
    const int g = wave + 8 * h;
    const int row = 16 * g + (lane >> 2);
    const int c = (lane & 3) ^ ((row >> 2) & 3);
    ause[h] = 16 * g < rows;
    const int rr = row < rows ? row : 0;
    if (GATEUP)
      asrc[h] = a.src + (size_t)(a.perm[rowbase + rr] / a.topk) * kdim + 8 * c;
    else
      asrc[h] = a.src + (size_t)(rowbase + rr) * kdim + 8 * c;
    buse[h] = wrow_of(16 * g) >= 0;
    const int wr = wrow_of(row);
    bsrc[h] = w16 + ((size_t)e * a.rows_total + (wr >= 0 ? wr : 0)) * kdim + 8 * c;
  }
  const int per_stage = (int)ause[0] + (int)ause[1] + (int)buse[0] + (int)buse[1];
  const int nst = kdim / DBK;

  auto issue = [&](int s, uint4* A, uint4* B) {
    const int k0 = s * DBK;
    if (ause[0]) dma16(asrc[0] + k0, A + wave * 64);
    if (ause[1]) dma16(asrc[1] + k0, A + (wave + 8) * 64);
    if (buse[0]) dma16(bsrc[0] + k0, B + wave * 64);
    if (buse[1]) dma16(bsrc[1] + k0, B + (wave + 8) * 64);
  };

  f32x16_t acc[4][2];
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int f = 0; f < 2; ++f)
#pragma unroll
      for (int v = 0; v < 16; ++v) acc[i][f][v] = 0.f;

  const int brow0 = GATEUP ? 32 * wn + (lane & 31) : 64 * wn + (lane & 31);
  const int brow1 = GATEUP ? 128 + 32 * wn + (lane & 31) : 64 * wn + 32 + (lane & 31);
  // 32-row fragments of this wave that hold routed rows (wave-uniform).
  const int nact = __builtin_amdgcn_readfirstlane(max(0, min(4, (rows - wm * 128 + 31) / 32)));
  // Multiply one stage: all LDS operand reads of both k-steps first, then
  // the MFMAs, so the reads overlap instead of waiting one by one.
  auto compute_n = [&](auto NA_c, const uint4* A, const uint4* B) {
    constexpr int NA = decltype(NA_c)::value;
    bf16x8_t Bv[2][2], Av[2][NA > 0 ? NA : 1];
#pragma unroll
    for (int ks = 0; ks < 2; ++ks) {
      const int c = 2 * ks + (lane >> 5);
      Bv[ks][0] = as_bf16x8(B[swz64(brow0, c)]);
      Bv[ks][1] = as_bf16x8(B[swz64(brow1, c)]);
#pragma unroll
      for (int i = 0; i < NA; ++i)
        Av[ks][i] = as_bf16x8(A[swz64(wm * 128 + 32 * i + (lane & 31), c)]);
    }
#pragma unroll
    for (int ks = 0; ks < 2; ++ks)
#pragma unroll
      for (int i = 0; i < NA; ++i) {
        acc[i][0] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(Av[ks][i], Bv[ks][0], acc[i][0], 0, 0, 0);
        acc[i][1] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(Av[ks][i], Bv[ks][1], acc[i][1], 0, 0, 0);
      }
  };
  // Stage s: wait for its copies (stages s+1, s+2 may stay in flight),
  // publish, queue stage s+3 into the buffer freed by stage s-1, multiply.
  // The loop is instantiated per active-fragment count so each variant is
  // straight-line code.
  auto kloop = [&](auto NA_c) {
    auto step = [&](int s, const uint4* A, const uint4* B, uint4* An, uint4* Bn) {
      wait_vmcnt_upto8(per_stage * min(2, nst - 1 - s));
      raw_barrier();
      if (s + 3 < nst) issue(s + 3, An, Bn);
      compute_n(NA_c, A, B);
    };
    issue(0, sA0, sB0);
    if (nst > 1) issue(1, sA1, sB1);
    if (nst > 2) issue(2, sA2, sB2);
    for (int s = 0; s < nst; s += 4) {
      step(s, sA0, sB0, sA3, sB3);
      if (s + 1 < nst) step(s + 1, sA1, sB1, sA0, sB0);
      if (s + 2 < nst) step(s + 2, sA2, sB2, sA1, sB1);
      if (s + 3 < nst) step(s + 3, sA3, sB3, sA2, sB2);
    }
  };
  switch (nact) {
    case 4: kloop(std::integral_constant<int, 4>{}); break;
    case 3: kloop(std::integral_constant<int, 3>{}); break;
    case 2: kloop(std::integral_constant<int, 2>{}); break;
    case 1: kloop(std::integral_constant<int, 1>{}); break;
    default: kloop(std::integral_constant<int, 0>{}); break;
  }

#pragma unroll
  for (int i = 0; i < 4; ++i) {
    if (wm * 128 + 32 * i >= rows) continue;
#pragma unroll
    for (int v = 0; v < 16; ++v) {
      const int tr = wm * 128 + 32 * i + 8 * (v >> 2) + 4 * (lane >> 5) + (v & 3);
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
}

// ===========================================================================
// launchers
// ===========================================================================
void launch_gemm_small(const GemmArgs& a, bool gateup, bool fp8, int grid, hipStream_t s) {
  if (gateup) {
    if (fp8) gemm_small_kernel<true, true><<<grid, 256, 0, s>>>(a);
    else gemm_small_kernel<true, false><<<grid, 256, 0, s>>>(a);
  } else {
    if (fp8) gemm_small_kernel<false, true><<<grid, 256, 0, s>>>(a);
    else gemm_small_kernel<false, false><<<grid, 256, 0, s>>>(a);
  }
}

void launch_gemm_big(const GemmArgs& a, bool gateup, bool fp8, int grid, hipStream_t s) {
  if (gateup) {
    if (fp8) gemm_big_kernel<true, true><<<grid, 512, 0, s>>>(a);
    else gemm_big_dma_kernel<true><<<grid, 512, 0, s>>>(a);
  } else {
    if (fp8) gemm_big_kernel<false, true><<<grid, 512, 0, s>>>(a);
    else gemm_big_dma_kernel<false><<<grid, 512, 0, s>>>(a);
  }
}

}  // namespace lcmoe
