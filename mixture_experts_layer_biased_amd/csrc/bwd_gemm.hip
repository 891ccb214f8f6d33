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
// into registers while the current one is multiplied from LDS. Both
// operand forms are stored in LDS as they sit in memory, 16 bytes at a time:
//   k-contiguous: [128 rows][32 k] (64-byte rows, chunk c of row r at
//     c ^ ((r >> 2) & 3)), read with 16-byte loads;
//   i-contiguous: [32 k][128 i] (256-byte rows, 64-byte window w of row k at
//     w ^ (k & 3)), read with the gfx950 transposing LDS load
//     (ds_read_b64_tr_b16), which hands each lane 4 consecutive k of one i.
// The MFMA computes the transposed tile (B as its first operand), so each
// lane holds 4 consecutive n of one output row: 16-byte (fp32) or 8-byte
// (bf16) stores.
#include "common.h"
#include "kernels.h"

namespace lcmoe {

namespace {

constexpr int BT = 128;  // tile rows (m and n)
constexpr int BKB = 32;  // k per stage

__device__ __forceinline__ int sw64(int row, int chunk) { return row * 4 + (chunk ^ ((row >> 2) & 3)); }

// i-contiguous tile [32 k][128 i]: element offset of (k, i), i a multiple of 4.
__device__ __forceinline__ int swkm(int k, int i) {
  return k * 128 + ((((i >> 5) ^ (k & 3)) << 5) | (i & 31));
}

typedef short s16x4_t __attribute__((ext_vector_type(4)));

// MFMA operand (rows base + lane % 32, k 16 ks + 8 (lane / 32) + [0, 8)) from
// an i-contiguous tile. ds_read_b64_tr_b16 works on groups of 16 lanes: lane
// s of a group names 4 consecutive i of one k row; the lane j of the group
// receives, for t = 0..3, element j % 4 of the group's lane j / 4 + 4 t. With
// lane s reading row k0 + s / 4 at i0 + 4 (s % 4), lane j gets (i0 + j,
// k0 + t): four consecutive k of one row of the operand.
__device__ __forceinline__ bf16x8_t km_frag(const uint16_t* tile, int base, int ks, int lane) {
  const int g = lane >> 4, s = lane & 15;
  const int i = base + 16 * (g & 1) + 4 * (s & 3);
  const int k = 16 * ks + 8 * (g >> 1) + (s >> 2);
  typedef __attribute__((address_space(3))) s16x4_t lds_s16x4;
  const s16x4_t lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
      (lds_s16x4*)(tile + swkm(k, i)));
  const s16x4_t hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
      (lds_s16x4*)(tile + swkm(k + 4, i)));
  return __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7);
}

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
      if (!A_IC) sA[buf][sw64(q >> 2, q & 3)] = ra[j];
      else *reinterpret_cast<uint4*>(reinterpret_cast<uint16_t*>(sA[buf]) +
                                     swkm(q >> 4, 8 * (q & 15))) = ra[j];
      if (!B_IC) sB[buf][sw64(q >> 2, q & 3)] = rb[j];
      else *reinterpret_cast<uint4*>(reinterpret_cast<uint16_t*>(sB[buf]) +
                                     swkm(q >> 4, 8 * (q & 15))) = rb[j];
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
      for (int i = 0; i < 2; ++i)
        av[i] = A_IC ? km_frag(reinterpret_cast<const uint16_t*>(sA[buf]), 64 * wm + 32 * i, ks,
                               lane)
                     : as_bf16x8(sA[buf][sw64(64 * wm + 32 * i + lr, 2 * ks + h)]);
#pragma unroll
      for (int f = 0; f < 2; ++f)
        bv[f] = B_IC ? km_frag(reinterpret_cast<const uint16_t*>(sB[buf]), 64 * wn + 32 * f, ks,
                               lane)
                     : as_bf16x8(sB[buf][sw64(64 * wn + 32 * f + lr, 2 * ks + h)]);
      // transposed tile: rows n (B), columns m (A)
#pragma unroll
      for (int i = 0; i < 2; ++i)
#pragma unroll
        for (int f = 0; f < 2; ++f)
          acc[i][f] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(bv[f], av[i], acc[i][f], 0, 0, 0);
    }
    if (s + 1 < nst) {
      store(buf ^ 1);
      __syncthreads();
    }
  }

  // Epilogue: lane holds output row m = lane % 32 of its fragment and, for
  // q = 0..3, columns 8 q + 4 (lane / 32) + [0, 4). Rows are slot rows
  // (m_is_slots) or rows of the expert's output matrix.
  char* cbase = static_cast<char*>(g.c);
#pragma unroll
  for (int i = 0; i < 2; ++i) {
    const int m = m0 + 64 * wm + 32 * i + lr;
    if (m >= M) continue;
    const long long row = g.m_is_slots ? (long long)g.offsets[e] + m : (long long)e * g.M + m;
#pragma unroll
    for (int f = 0; f < 2; ++f)
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const int n = n0 + 64 * wn + 32 * f + 8 * q + 4 * h;
        if (n >= N) continue;
        const long long idx = row * g.c_ld + n;
        const f32x16_t& a = acc[i][f];
        if (OUT_F32) {
          *reinterpret_cast<float4*>(reinterpret_cast<float*>(cbase) + idx) =
              make_float4(a[4 * q], a[4 * q + 1], a[4 * q + 2], a[4 * q + 3]);
        } else {
          *reinterpret_cast<uint2*>(reinterpret_cast<uint16_t*>(cbase) + idx) =
              make_uint2(pack_bf16x2(a[4 * q], a[4 * q + 1]), pack_bf16x2(a[4 * q + 2], a[4 * q + 3]));
        }
      }
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
