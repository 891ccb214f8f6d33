// Routing kernels: router logits, biased top-K with softmax gates, and the
// per-expert counting sort of the FFN slots.
//
// Method: "LongCat-Flash" (llm-wiki entity page), section 2.1: the router
// picks K of the N+Z experts per token; T_i counts the tokens routed to
// expert i. The bias is added to the fp32 logit for selection only; gates
// are softmax(z) over all experts (section 2.3.2 names softmax gating).
#include "common.h"
#include "kernels.h"

namespace lcmoe {

// ---------------------------------------------------------------------------
// Router GEMM: zpart[s][t][e] = sum_{k in split s} x[t][k] * W_r[e][k].
//
// Exact fp32 products on bf16 MFMA: each fp32 router weight is split into
// three bf16 planes w = hi + mid + lo (each residual of a round-to-nearest
// bf16 conversion is exact in fp32 and the last one fits in 8 bits), x is
// bf16, so every product x*hi, x*mid, x*lo is exact in the fp32 accumulator
// (Henry, Tang & Heinecke, "Leveraging the bfloat16 Artificial Intelligence
// Datatype for Higher-Precision Computations", ARITH 2019).
//
// Tile 256 tokens x 128 experts x 32 k per stage, 8 waves (2 x 4), each wave
// 128 tokens x 32 experts: 4 x-fragments against the expert fragment's three
// planes, 12 v_mfma_f32_32x32x16_bf16 per 16 k. The tall token side keeps the
// 4-byte router weights' re-reads low. Global -> registers (the weights are
// split there) -> swizzled LDS, two LDS buffers, one barrier per stage.
// LDS rows are 64 bytes; chunk c of row r lives at c ^ ((r >> 2) & 3).
// ---------------------------------------------------------------------------
constexpr int RBM = 256, RBN = 128, RBK = 32;

__device__ __forceinline__ int rswz(int row, int chunk) {
  return row * 4 + (chunk ^ ((row >> 2) & 3));
}

__global__ __launch_bounds__(512) void router_gemm_kernel(const uint16_t* __restrict__ x,
                                                          const float* __restrict__ wr,
                                                          float* __restrict__ zpart, int T,
                                                          int E, int d, int kchunk) {
  __shared__ uint4 sA[2][RBM * 4];
  __shared__ uint4 sB[2][3][RBN * 4];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int wm = wave >> 2, wn = wave & 3, h = lane >> 5;
  const int t0 = blockIdx.x * RBM, e0 = blockIdx.y * RBN, sp = blockIdx.z;
  const int kbeg = sp * kchunk;
  const int kend = min(d, kbeg + kchunk);
  const int nst = (kend - kbeg) / RBK;  // d and kchunk are multiples of 32

  uint4 ra[2];
  float4 rb[2];
  auto load_stage = [&](int k0) {
#pragma unroll
    for (int u = 0; u < 2; ++u) {
      const int id = tid + 512 * u;
      const int row = id >> 2, c = id & 3;
      const int t = t0 + row;
      ra[u] = t < T ? *reinterpret_cast<const uint4*>(x + (size_t)t * d + k0 + 8 * c)
                    : make_uint4(0, 0, 0, 0);
    }
#pragma unroll
    for (int u = 0; u < 2; ++u) {
      const int id = tid + 512 * u;
      const int row = id >> 3, q = id & 7;
      const int e = e0 + row;
      rb[u] = e < E ? *reinterpret_cast<const float4*>(wr + (size_t)e * d + k0 + 4 * q)
                    : make_float4(0.f, 0.f, 0.f, 0.f);
    }
  };
  auto store_stage = [&](int buf) {
#pragma unroll
    for (int u = 0; u < 2; ++u) {
      const int id = tid + 512 * u;
      sA[buf][rswz(id >> 2, id & 3)] = ra[u];
    }
#pragma unroll
    for (int u = 0; u < 2; ++u) {
      const int id = tid + 512 * u;
      const int row = id >> 3, q = id & 7;
      uint16_t hh[4], mm[4], ll[4];
      split3(rb[u].x, hh[0], mm[0], ll[0]);
      split3(rb[u].y, hh[1], mm[1], ll[1]);
      split3(rb[u].z, hh[2], mm[2], ll[2]);
      split3(rb[u].w, hh[3], mm[3], ll[3]);
      const int slot = rswz(row, q >> 1) * 2 + (q & 1);  // 8-byte half chunk
      reinterpret_cast<uint2*>(sB[buf][0])[slot] =
          make_uint2(hh[0] | ((uint32_t)hh[1] << 16), hh[2] | ((uint32_t)hh[3] << 16));
      reinterpret_cast<uint2*>(sB[buf][1])[slot] =
          make_uint2(mm[0] | ((uint32_t)mm[1] << 16), mm[2] | ((uint32_t)mm[3] << 16));
      reinterpret_cast<uint2*>(sB[buf][2])[slot] =
          make_uint2(ll[0] | ((uint32_t)ll[1] << 16), ll[2] | ((uint32_t)ll[3] << 16));
    }
  };

  f32x16_t acc[4];
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int v = 0; v < 16; ++v) acc[i][v] = 0.f;

  const int brow = 32 * wn + (lane & 31);
  load_stage(kbeg);
  store_stage(0);
  __syncthreads();
  for (int st = 0; st < nst; ++st) {
    const int buf = st & 1;
    if (st + 1 < nst) load_stage(kbeg + (st + 1) * RBK);
#pragma unroll
    for (int ks = 0; ks < 2; ++ks) {
      const int c = 2 * ks + h;
      const bf16x8_t b0 = as_bf16x8(sB[buf][0][rswz(brow, c)]);
      const bf16x8_t b1 = as_bf16x8(sB[buf][1][rswz(brow, c)]);
      const bf16x8_t b2 = as_bf16x8(sB[buf][2][rswz(brow, c)]);
      bf16x8_t av[4];
#pragma unroll
      for (int i = 0; i < 4; ++i)
        av[i] = as_bf16x8(sA[buf][rswz(128 * wm + 32 * i + (lane & 31), c)]);
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        acc[i] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(av[i], b2, acc[i], 0, 0, 0);
        acc[i] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(av[i], b1, acc[i], 0, 0, 0);
        acc[i] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(av[i], b0, acc[i], 0, 0, 0);
      }
    }
    if (st + 1 < nst) store_stage(buf ^ 1);
    __syncthreads();
  }

  const int e = e0 + brow;
  if (e < E) {
    float* zp = zpart + (size_t)sp * T * E;
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
      for (int v = 0; v < 16; ++v) {
        const int t = t0 + 128 * wm + 32 * i + 8 * (v >> 2) + 4 * (lane >> 5) + (v & 3);
        if (t < T) zp[(size_t)t * E + e] = acc[i][v];
      }
  }
}

// ---------------------------------------------------------------------------
// Biased top-K and gates. One wavefront per token; lane l holds experts
// l, l+64, ... (J of them). Selection key: order-preserving bits of
// s = fl32(z + b) (with -0 folded to +0) in the high word, ~expert in the low
// word, so one unsigned max picks (score desc, index asc). K rounds of
// lane-local max + 64-lane butterfly max. Gates: exp(z - max) / sum over
// all E, in fp32; the bias never enters them.
// ---------------------------------------------------------------------------
template <int J>
__global__ __launch_bounds__(256) void topk_kernel(const float* __restrict__ zpart, int ks,
                                                   const float* __restrict__ bias, int T, int E,
                                                   int K, int* __restrict__ idx_out,
                                                   float* __restrict__ gate_out,
                                                   float* __restrict__ logits_out) {
  const int lane = threadIdx.x & 63;
  const int t = blockIdx.x * 4 + (threadIdx.x >> 6);
  if (t >= T) return;
  float z[J];
  uint64_t key[J];
  float zmax = -INFINITY;
  // Split-K partial logits, summed in split order: all J loads of one split
  // are issued together, splits follow each other.
#pragma unroll
  for (int j = 0; j < J; ++j) {
    const int e = lane + 64 * j;
    z[j] = e < E ? zpart[(size_t)t * E + e] : 0.f;
  }
  for (int s = 1; s < ks; ++s) {
    const float* zs = zpart + ((size_t)s * T + t) * E;
    float v[J];
#pragma unroll
    for (int j = 0; j < J; ++j) v[j] = (lane + 64 * j < E) ? zs[lane + 64 * j] : 0.f;
#pragma unroll
    for (int j = 0; j < J; ++j) z[j] += v[j];
  }
#pragma unroll
  for (int j = 0; j < J; ++j) {
    const int e = lane + 64 * j;
    if (e < E) {
      const float v = z[j];
      if (logits_out) logits_out[(size_t)t * E + e] = v;
      float sc = v + bias[e];
      if (sc == 0.0f) sc = 0.0f;  // -0 -> +0
      const uint32_t u = __float_as_uint(sc);
      const uint32_t o = (u & 0x80000000u) ? ~u : (u | 0x80000000u);
      key[j] = ((uint64_t)o << 32) | (uint64_t)(0xFFFFFFFFu - (uint32_t)e);
      zmax = fmaxf(zmax, v);
    } else {
      z[j] = -INFINITY;
      key[j] = 0;
    }
  }
  zmax = wave_max(zmax);
  float p[J];
  float sum = 0.f;
#pragma unroll
  for (int j = 0; j < J; ++j) {
    p[j] = (lane + 64 * j < E) ? expf(z[j] - zmax) : 0.f;
    sum += p[j];
  }
  sum = wave_sum(sum);

  int my_e = 0;
  float my_p = 0.f;
  for (int k = 0; k < K; ++k) {
    uint64_t best = key[0];
#pragma unroll
    for (int j = 1; j < J; ++j) best = key[j] > best ? key[j] : best;
    best = wave_max_u64(best);
    const int e = (int)(0xFFFFFFFFu - (uint32_t)best);
    const int owner = e & 63, jj = e >> 6;
    float pv = 0.f;
    if (lane == owner) {
#pragma unroll
      for (int j = 0; j < J; ++j)
        if (j == jj) {
          pv = p[j];
          key[j] = 0;
        }
    }
    pv = __shfl(pv, owner, kWave);
    if (lane == k) {
      my_e = e;
      my_p = pv;
    }
  }
  if (lane < K) {
    idx_out[(size_t)t * K + lane] = my_e;
    gate_out[(size_t)t * K + lane] = my_p / sum;
  }
}

// ---------------------------------------------------------------------------
// Counting sort of the FFN slots, in three passes over 64-token tiles.
//  hist:    per tile, a 64-bit token mask per expert (LDS atomics OR), and
//           the tile's count per expert (popcount), stored expert-major.
//  colscan: per expert, exclusive prefix of the tile counts -> tile offsets,
//           and the total T_i.
//  schedule (one block): offsets over the FFN experts, the prefix of their
//           M-tile counts for the grouped GEMMs, and the number of touched
//           FFN experts.
//  scatter: slot (t,k) with expert e < N goes to
//           offsets[e] + tileoff[e][tile] + popcount(mask[tile][e] below t),
//           i.e. ascending slot order inside each expert (stable).
// A token selects an expert at most once, so within an expert slot order is
// token order.
// ---------------------------------------------------------------------------
__global__ __launch_bounds__(256) void hist_kernel(const int* __restrict__ idx, int T, int K,
                                                   int E, int ntile,
                                                   unsigned long long* __restrict__ masks,
                                                   int* __restrict__ tilecnt) {
  extern __shared__ unsigned long long smask[];
  const int b = blockIdx.x, tid = threadIdx.x;
  const int t0 = b * 64;
  const int nt = min(64, T - t0);
  for (int e = tid; e < E; e += 256) smask[e] = 0ull;
  __syncthreads();
  for (int j = tid; j < nt * K; j += 256) {
    const int tl = j / K;
    const int e = idx[(size_t)t0 * K + j];
    if ((unsigned)e < (unsigned)E) atomicOr(&smask[e], 1ull << tl);
  }
  __syncthreads();
  for (int e = tid; e < E; e += 256) {
    const unsigned long long m = smask[e];
    masks[(size_t)b * E + e] = m;
    tilecnt[(size_t)e * ntile + b] = __popcll(m);
  }
}

__global__ __launch_bounds__(64) void colscan_kernel(const int* __restrict__ tilecnt,
                                                     int* __restrict__ tileoff, int ntile,
                                                     int* __restrict__ counts) {
  const int e = blockIdx.x, lane = threadIdx.x;
  int carry = 0;
  for (int c0 = 0; c0 < ntile; c0 += 64) {
    const int b = c0 + lane;
    const int v = b < ntile ? tilecnt[(size_t)e * ntile + b] : 0;
    const int inc = wave_incl_scan(v, lane);
    if (b < ntile) tileoff[(size_t)e * ntile + b] = carry + inc - v;
    carry += __shfl(inc, 63, kWave);
  }
  if (lane == 0) counts[e] = carry;
}

// Exclusive scan over a 1024-thread block; returns the prefix, writes total.
__device__ int block_excl_scan_1024(int v, int* sh, int& total) {
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int inc = wave_incl_scan(v, lane);
  if (lane == 63) sh[wave] = inc;
  __syncthreads();
  if (wave == 0) {
    const int w = lane < 16 ? sh[lane] : 0;
    const int wi = wave_incl_scan(w, lane);
    if (lane < 16) sh[16 + lane] = wi - w;
    if (lane == 15) sh[32] = wi;
  }
  __syncthreads();
  const int out = sh[16 + wave] + inc - v;
  total = sh[32];
  __syncthreads();
  return out;
}

__global__ __launch_bounds__(1024) void schedule_kernel(const int* __restrict__ counts, int N,
                                                        int big_bm, int* __restrict__ offsets,
                                                        int* __restrict__ mt_prefix,
                                                        int* __restrict__ meta) {
  __shared__ int sh[40];
  const int tid = threadIdx.x;
  const int e0 = 2 * tid, e1 = 2 * tid + 1;
  const int c0 = e0 < N ? counts[e0] : 0;
  const int c1 = e1 < N ? counts[e1] : 0;
  const int m0 = (c0 + big_bm - 1) / big_bm, m1 = (c1 + big_bm - 1) / big_bm;  // 0 for no rows
  int tc, tt, tm;
  const int xc = block_excl_scan_1024(c0 + c1, sh, tc);
  block_excl_scan_1024((c0 > 0) + (c1 > 0), sh, tt);
  const int xm = block_excl_scan_1024(m0 + m1, sh, tm);
  if (e0 < N) {
    offsets[e0] = xc;
    mt_prefix[e0] = xm;
  }
  if (e1 < N) {
    offsets[e1] = xc + c0;
    mt_prefix[e1] = xm + m0;
  }
  if (tid == 0) {
    offsets[N] = tc;
    mt_prefix[N] = tm;
    meta[0] = tt;
    meta[1] = tm;
    meta[2] = tc;
  }
}

__global__ __launch_bounds__(256) void scatter_kernel(const int* __restrict__ idx, int T, int K,
                                                      int E, int N, int ntile,
                                                      const unsigned long long* __restrict__ masks,
                                                      const int* __restrict__ tileoff,
                                                      const int* __restrict__ offsets,
                                                      int* __restrict__ perm,
                                                      int* __restrict__ row_of_slot) {
  const int b = blockIdx.x, tid = threadIdx.x;
  const int t0 = b * 64;
  const int nt = min(64, T - t0);
  for (int j = tid; j < nt * K; j += 256) {
    const int slot = t0 * K + j;
    const int tl = j / K;
    const int e = idx[slot];
    if ((unsigned)e < (unsigned)N) {
      const unsigned long long m = masks[(size_t)b * E + e];
      const int rank = __popcll(m & ((1ull << tl) - 1ull));
      const int pos = offsets[e] + tileoff[(size_t)e * ntile + b] + rank;
      perm[pos] = slot;
      row_of_slot[slot] = pos;
    } else {
      row_of_slot[slot] = -1;
    }
  }
  const int S = offsets[N];
  const int TK = T * K;
  for (int p = S + b * 256 + tid; p < TK; p += gridDim.x * 256) perm[p] = -1;
}

// ---------------------------------------------------------------------------
// Launchers
// ---------------------------------------------------------------------------
void launch_router(const uint16_t* x, const float* wr, float* zpart, int T, int E, int d,
                   int ks, int kchunk, hipStream_t s) {
  dim3 grid((T + RBM - 1) / RBM, (E + RBN - 1) / RBN, ks);
  router_gemm_kernel<<<grid, 512, 0, s>>>(x, wr, zpart, T, E, d, kchunk);
}

void launch_topk(const float* zpart, int ks, const float* bias, int T, int E, int K, int* idx,
                 float* gate, float* logits_out, hipStream_t s) {
  const int J = (E + 63) / 64;
  dim3 grid((T + 3) / 4);
#define LCMOE_TOPK(JJ) topk_kernel<JJ><<<grid, 256, 0, s>>>(zpart, ks, bias, T, E, K, idx, gate, logits_out)
  if (J <= 1) LCMOE_TOPK(1);
  else if (J <= 2) LCMOE_TOPK(2);
  else if (J <= 4) LCMOE_TOPK(4);
  else if (J <= 8) LCMOE_TOPK(8);
  else if (J <= 12) LCMOE_TOPK(12);
  else if (J <= 16) LCMOE_TOPK(16);
  else if (J <= 24) LCMOE_TOPK(24);
  else LCMOE_TOPK(32);
#undef LCMOE_TOPK
}

void launch_permute(const int* idx, int T, int K, int E, int N, int ntile,
                    unsigned long long* masks, int* tilecnt, int* tileoff, int* counts,
                    int* offsets, int* mt_prefix, int* meta, int* perm,
                    int* row_of_slot, hipStream_t s) {
  hist_kernel<<<ntile, 256, (size_t)E * 8, s>>>(idx, T, K, E, ntile, masks, tilecnt);
  colscan_kernel<<<E, 64, 0, s>>>(tilecnt, tileoff, ntile, counts);
  schedule_kernel<<<1, 1024, 0, s>>>(counts, N, kBigTileRows, offsets, mt_prefix, meta);
  if (perm != nullptr)
    scatter_kernel<<<ntile, 256, 0, s>>>(idx, T, K, E, N, ntile, masks, tileoff, offsets, perm,
                                         row_of_slot);
}

}  // namespace lcmoe
