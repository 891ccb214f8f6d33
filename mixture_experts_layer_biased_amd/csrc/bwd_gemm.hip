// Grouped GEMMs of the backward pass (bf16 operands, fp32 accumulation on
// v_mfma_f32_32x32x16_bf16), one kernel for the four operand arrangements
// the backward needs:
//
//   C_e[m][n] = sum_k A_e(m, k) * B_e(n, k)   for every FFN expert e
//
// Each operand is a bf16 matrix view: element (i, k) lives at
//   row(i) * ld + k   ("k-contiguous", rows indexed by i), or
//   row(k) * ld + i   ("i-contiguous", rows indexed by k),
// where a row index is one of: a row of the expert's weight matrix (base +
// e * estride), a slot row of the expert's FFN slots (offsets[e] + r), or
// the token of such a slot (perm[offsets[e] + r] / K). The expert's extent
// is either M = its slot count (dgrad: one output row per slot) or K = its
// slot count (wgrad: the reduction runs over the expert's slots).
//
// Tiles of 128 x 128 x 32, 256 threads (2 x 2 waves of 64 x 64 = 2 x 2
// fragments), register-staged double buffering: the next k stage is loaded
// into registers while the current one is multiplied from LDS. LDS tiles
// are [128 rows][32 k] bf16 (64-byte rows, chunk c of row r at
// c ^ ((r >> 2) & 3)); i-contiguous operands are transposed on the way in.
#include "common.h"
#include "kernels.h"

namespace lcmoe {

namespace {

constexpr int BT = 128;  // tile rows (m and n)
constexpr int BKB = 32;  // k per stage

__device__ __forceinline__ int sw64(int row, int chunk) { return row * 4 + (chunk ^ ((row >> 2) & 3)); }

struct OpView {
  const uint16_t* base;
  long long ld;
  long long estride;  // weight rows: element offset per expert
  int ic;             // 1: i-contiguous
  int rows;           // BwdRow: 0 weight, 1 slot, 2 token of slot
};

}  // namespace

// Row index -> global row of the operand's matrix, for expert e.
__device__ __forceinline__ long long bwd_row(const BwdGemmArgs& g, int src, int e, int r) {
  if (src == kBwdRowWeight) return r;
  const int s = g.offsets[e] + r;
  return src == kBwdRowSlot ? (long long)s : (long long)(g.perm[s] / g.topk);
}

template <bool A_IC, bool B_IC, bool OUT_F32>
__global__ __launch_bounds__(256) void bwd_gemm_kernel(BwdGemmArgs g) {
  __shared__ uint4 sA[2][BT * 4];
  __shared__ uint4 sB[2][BT * 4];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int wm = wave >> 1, wn = wave & 1;

  // Work item -> (expert, m tile, n tile).
  int e, mt, nt;
  const int ntn = (g.N + BT - 1) / BT;
  if (g.m_is_slots) {
    const int total = g.tile_prefix[g.n_ffn] * ntn;
    if ((int)blockIdx.x >= total) return;
    int lo = 0, hi = g.n_ffn - 1;
    const int L = blockIdx.x;
    while (lo < hi) {
      const int mid = (lo + hi + 1) >> 1;
      if (g.tile_prefix[mid] * ntn <= L) lo = mid; else hi = mid - 1;
    }
    e = lo;
    const int local = L - g.tile_prefix[e] * ntn;
    mt = local / ntn;
    nt = local - mt * ntn;
  } else {
    const int ntm = (g.M + BT - 1) / BT;
    const int per = ntm * ntn;
    e = blockIdx.x / per;
    if (e >= g.n_ffn) return;
    const int local = blockIdx.x - e * per;
    mt = local / ntn;
    nt = local - mt * ntn;
  }
  const int cnt = g.counts[e];
  const int M = g.m_is_slots ? cnt : g.M;
  const int N = g.N;
  const int K = g.m_is_slots ? g.K : cnt;
  const int m0 = mt * BT, n0 = nt * BT;

  const uint16_t* abase = g.a + (g.a_rows == kBwdRowWeight ? (long long)e * g.a_estride : 0);
  const uint16_t* bbase = g.b + (g.b_rows == kBwdRowWeight ? (long long)e * g.b_estride : 0);

  // Staging registers: two 16-byte chunks per operand per thread.
  uint4 ra[2], rb[2];
  auto load = [&](int k0) {
#pragma unroll
    for (int j = 0; j < 2; ++j) {
      const int q = tid + 256 * j;
      // A
      if (!A_IC) {
        const int r = q >> 2, c = q & 3;
        const int i = m0 + r, k = k0 + 8 * c;
        ra[j] = make_uint4(0, 0, 0, 0);
        if (i < M && k < K)
          ra[j] = *reinterpret_cast<const uint4*>(abase + bwd_row(g, g.a_rows, e, i) * g.a_ld + k);
      } else {
        const int kr = q >> 4, ic = q & 15;
        const int k = k0 + kr, i = m0 + 8 * ic;
        ra[j] = make_uint4(0, 0, 0, 0);
        if (k < K && i < M)
          ra[j] = *reinterpret_cast<const uint4*>(abase + bwd_row(g, g.a_rows, e, k) * g.a_ld + i);
      }
      // B
      if (!B_IC) {
        const int r = q >> 2, c = q & 3;
        const int i = n0 + r, k = k0 + 8 * c;
        rb[j] = make_uint4(0, 0, 0, 0);
        if (i < N && k < K)
          rb[j] = *reinterpret_cast<const uint4*>(bbase + bwd_row(g, g.b_rows, e, i) * g.b_ld + k);
      } else {
        const int kr = q >> 4, ic = q & 15;
        const int k = k0 + kr, i = n0 + 8 * ic;
        rb[j] = make_uint4(0, 0, 0, 0);
        if (k < K && i < N)
          rb[j] = *reinterpret_cast<const uint4*>(bbase + bwd_row(g, g.b_rows, e, k) * g.b_ld + i);
      }
    }
  };
  auto store = [&](int buf) {
#pragma unroll
    for (int j = 0; j < 2; ++j) {
      const int q = tid + 256 * j;
      if (!A_IC) {
        sA[buf][sw64(q >> 2, q & 3)] = ra[j];
      } else {
        const int kr = q >> 4, i8 = 8 * (q & 15);
        uint16_t* s = reinterpret_cast<uint16_t*>(sA[buf]);
        const uint32_t w[4] = {ra[j].x, ra[j].y, ra[j].z, ra[j].w};
#pragma unroll
        for (int u = 0; u < 8; ++u) {
          const int row = i8 + u;
          s[sw64(row, kr >> 3) * 8 + (kr & 7)] = (uint16_t)(w[u >> 1] >> (16 * (u & 1)));
        }
      }
      if (!B_IC) {
        sB[buf][sw64(q >> 2, q & 3)] = rb[j];
      } else {
        const int kr = q >> 4, i8 = 8 * (q & 15);
        uint16_t* s = reinterpret_cast<uint16_t*>(sB[buf]);
        const uint32_t w[4] = {rb[j].x, rb[j].y, rb[j].z, rb[j].w};
#pragma unroll
        for (int u = 0; u < 8; ++u) {
          const int row = i8 + u;
          s[sw64(row, kr >> 3) * 8 + (kr & 7)] = (uint16_t)(w[u >> 1] >> (16 * (u & 1)));
        }
      }
    }
  };

  f32x16_t acc[2][2];
#pragma unroll
  for (int i = 0; i < 2; ++i)
#pragma unroll
    for (int f = 0; f < 2; ++f)
#pragma unroll
      for (int v = 0; v < 16; ++v) acc[i][f][v] = 0.f;

  const int h = lane >> 5, lr = lane & 31;
  const int nst = (K + BKB - 1) / BKB;
  if (nst > 0) {
    load(0);
    store(0);
    __syncthreads();
  }
  for (int s = 0; s < nst; ++s) {
    const int buf = s & 1;
    if (s + 1 < nst) load((s + 1) * BKB);
#pragma unroll
    for (int ks = 0; ks < 2; ++ks) {
      bf16x8_t av[2], bv[2];
#pragma unroll
      for (int i = 0; i < 2; ++i) av[i] = as_bf16x8(sA[buf][sw64(64 * wm + 32 * i + lr, 2 * ks + h)]);
#pragma unroll
      for (int f = 0; f < 2; ++f) bv[f] = as_bf16x8(sB[buf][sw64(64 * wn + 32 * f + lr, 2 * ks + h)]);
#pragma unroll
      for (int i = 0; i < 2; ++i)
#pragma unroll
        for (int f = 0; f < 2; ++f)
          acc[i][f] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(av[i], bv[f], acc[i][f], 0, 0, 0);
    }
    if (s + 1 < nst) {
      store(buf ^ 1);
      __syncthreads();
    }
  }

  // Epilogue: rows are slot rows (m_is_slots) or rows of the expert's
  // output matrix.
  char* cbase = static_cast<char*>(g.c);
#pragma unroll
  for (int i = 0; i < 2; ++i)
#pragma unroll
    for (int f = 0; f < 2; ++f)
#pragma unroll
      for (int v = 0; v < 16; ++v) {
        const int m = m0 + 64 * wm + 32 * i + 8 * (v >> 2) + 4 * h + (v & 3);
        const int n = n0 + 64 * wn + 32 * f + lr;
        if (m >= M || n >= N) continue;
        const long long row = g.m_is_slots ? (long long)g.offsets[e] + m
                                           : (long long)e * g.M + m;
        const long long idx = row * g.c_ld + n;
        if (OUT_F32) reinterpret_cast<float*>(cbase)[idx] = acc[i][f][v];
        else reinterpret_cast<uint16_t*>(cbase)[idx] = f32_to_bf16(acc[i][f][v]);
      }
}

void launch_bwd_gemm(const BwdGemmArgs& g, bool a_ic, bool b_ic, bool out_f32, int grid,
                     hipStream_t s) {
#define LCMOE_BWD(AI, BI, OF) bwd_gemm_kernel<AI, BI, OF><<<grid, 256, 0, s>>>(g)
  if (!a_ic && !b_ic) { if (out_f32) LCMOE_BWD(false, false, true); else LCMOE_BWD(false, false, false); }
  else if (!a_ic && b_ic) { if (out_f32) LCMOE_BWD(false, true, true); else LCMOE_BWD(false, true, false); }
  else if (a_ic && b_ic) { if (out_f32) LCMOE_BWD(true, true, true); else LCMOE_BWD(true, true, false); }
  else { if (out_f32) LCMOE_BWD(true, false, true); else LCMOE_BWD(true, false, false); }
#undef LCMOE_BWD
}

}  // namespace lcmoe
