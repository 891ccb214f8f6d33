// Backward of the layer: the element-wise and per-token steps, and the fp32
// router-gradient GEMMs. Chain rule of the layer ("LongCat-Flash" section
// 2.1: y_t = sum_k g_tk v_tk with g from one softmax over all N+Z experts,
// v the SiLU-gated FFN expert or, for a zero expert, x_t itself):
//
//   dg_tk = <dy_t, v_tk>, with v_tk = W2 h for an FFN slot (so
//           dg = <W2^T dy_t, h> = <Q_s, h_s>) and x_t for a zero slot
//   FFN slot s: dh = g Q_s; da = dh c silu'(a); dc = dh silu(a)
//   dz_t = p_t * (dp_t - <dp_t, p_t>), dp_t[idx_tk] = dg_tk
//   dx_t = sum_FFN (dU W13)_s + (sum_zero g_tk) dy_t + (dz W_r)_t
//
// The expert GEMMs (U, Q, dU W13, the weight gradients) are in bwd_gemm.hip.
#include <algorithm>

#include "common.h"
#include "kernels.h"

namespace lcmoe {

// prefix[e] = sum_{e' < e} ceil(counts[e'] / rows), one wave (N <= 2048).
__global__ __launch_bounds__(64) void tile_prefix_kernel(const int* __restrict__ counts, int N,
                                                         int rows, int* __restrict__ prefix) {
  const int lane = threadIdx.x;
  const int per = (N + 63) / 64;
  const int lo = lane * per, hi = min(N, lo + per);
  int s = 0;
  for (int e = lo; e < hi; ++e) s += (counts[e] + rows - 1) / rows;
  const int incl = wave_incl_scan(s, lane);
  int run = incl - s;
  for (int e = lo; e < hi; ++e) {
    prefix[e] = run;
    run += (counts[e] + rows - 1) / rows;
  }
  if (lane == 63) prefix[N] = incl;
}

__device__ __forceinline__ float sigmoid_f(float a) { return 1.0f / (1.0f + expf(-a)); }

// One wave per FFN slot row s < S (S read on the device): h = silu(a) c from
// U = [a; c]; dg = <Q_s, h>; dU_s = [dh c silu'(a); dh silu(a)] with
// dh = g Q_s (bf16); Hg_s = g h (bf16, the dW2 operand).
__global__ __launch_bounds__(256) void bwd_rows_kernel(const float* __restrict__ U,
                                                       const float* __restrict__ Q,
                                                       const int* __restrict__ perm,
                                                       const float* __restrict__ gate,
                                                       const int* __restrict__ s_dev, int I,
                                                       uint16_t* __restrict__ dU,
                                                       uint16_t* __restrict__ Hg,
                                                       float* __restrict__ dg) {
  const int lane = threadIdx.x & 63;
  const int S = *s_dev;
  const int wpb = blockDim.x >> 6;
  for (int s = blockIdx.x * wpb + (threadIdx.x >> 6); s < S; s += gridDim.x * wpb) {
    const int slot = perm[s];
    const float g = gate[slot];
    const float* u = U + (size_t)s * 2 * I;
    const float* q = Q + (size_t)s * I;
    float part = 0.f;
    for (int j = lane; j < I; j += 64) {
      const float a = u[j], c = u[I + j];
      const float sg = sigmoid_f(a);
      const float si = a * sg;
      const float h = si * c;
      const float qq = q[j];
      part += qq * h;
      const float dh = g * qq;
      dU[(size_t)s * 2 * I + j] = f32_to_bf16(dh * c * (sg * (1.0f + a * (1.0f - sg))));
      dU[(size_t)s * 2 * I + I + j] = f32_to_bf16(dh * si);
      Hg[(size_t)s * I + j] = f32_to_bf16(g * h);
    }
    part = wave_sum(part);
    if (lane == 0) dg[slot] = part;
  }
}

// One wave per token: dg of its zero-computation slots, <dy_t, x_t>.
__global__ __launch_bounds__(256) void bwd_zero_dg_kernel(const uint16_t* __restrict__ x,
                                                          const uint16_t* __restrict__ dy,
                                                          const int* __restrict__ idx, int T,
                                                          int d, int K, int N,
                                                          float* __restrict__ dg) {
  const int lane = threadIdx.x & 63;
  const int wpb = blockDim.x >> 6;
  for (int t = blockIdx.x * wpb + (threadIdx.x >> 6); t < T; t += gridDim.x * wpb) {
    bool any = false;
    for (int k = 0; k < K; ++k) any |= idx[(size_t)t * K + k] >= N;
    if (!any) continue;
    const uint4* xr = reinterpret_cast<const uint4*>(x + (size_t)t * d);
    const uint4* gr = reinterpret_cast<const uint4*>(dy + (size_t)t * d);
    float part = 0.f;
    for (int c = lane; c < (d >> 3); c += 64) {
      const uint4 a = xr[c], b = gr[c];
      const uint32_t ua[4] = {a.x, a.y, a.z, a.w}, ub[4] = {b.x, b.y, b.z, b.w};
#pragma unroll
      for (int q = 0; q < 4; ++q)
        part += bf16_lo(ua[q]) * bf16_lo(ub[q]) + bf16_hi(ua[q]) * bf16_hi(ub[q]);
    }
    part = wave_sum(part);
    if (lane == 0)
      for (int k = 0; k < K; ++k)
        if (idx[(size_t)t * K + k] >= N) dg[(size_t)t * K + k] = part;
  }
}

// One wave per token: p = softmax(z_t) over all E, c = sum_k dg_tk g_tk,
// dz_i = p_i (dp_i - c) with dp_i = dg_tk at the selected experts.
__global__ __launch_bounds__(256) void bwd_router_dz_kernel(const float* __restrict__ logits,
                                                            const int* __restrict__ idx,
                                                            const float* __restrict__ gate,
                                                            const float* __restrict__ dg, int T,
                                                            int E, int K, float* __restrict__ dz) {
  const int lane = threadIdx.x & 63;
  const int wpb = blockDim.x >> 6;
  for (int t = blockIdx.x * wpb + (threadIdx.x >> 6); t < T; t += gridDim.x * wpb) {
    const float* z = logits + (size_t)t * E;
    float m = -INFINITY;
    for (int i = lane; i < E; i += 64) m = fmaxf(m, z[i]);
    m = wave_max(m);
    float s = 0.f;
    for (int i = lane; i < E; i += 64) s += expf(z[i] - m);
    s = wave_sum(s);
    float c = 0.f;
    for (int k = 0; k < K; ++k) c += dg[(size_t)t * K + k] * gate[(size_t)t * K + k];
    for (int i = lane; i < E; i += 64) {
      float dp = 0.f;
      for (int k = 0; k < K; ++k)
        if (idx[(size_t)t * K + k] == i) dp = dg[(size_t)t * K + k];
      const float p = expf(z[i] - m) / s;
      dz[(size_t)t * E + i] = p * (dp - c);
    }
  }
}

// fp32 GEMM for the router gradients, C[m][n] = sum_k A(m, k) B(n, k):
// A(m, k) at a[m * lda + k] (A_T: a[k * lda + m]); B(n, k) likewise, B in
// fp32 or bf16. 64 x 64 tiles, k stages of 16, 256 threads with 4 x 4
// outputs each, fp32 FMA in k order. Grid: x over m tiles, y over n tiles.
template <bool A_T, bool B_T, bool B_BF16>
__global__ __launch_bounds__(256) void f32_gemm_kernel(const float* __restrict__ a, long long lda,
                                                       const void* __restrict__ bv, long long ldb,
                                                       float* __restrict__ c, long long ldc,
                                                       int M, int N, int K) {
  __shared__ float sa[16][64 + 1];
  __shared__ float sb[16][64 + 1];
  const int tid = threadIdx.x;
  const int m0 = blockIdx.x * 64, n0 = blockIdx.y * 64;
  const int tm = (tid >> 4) * 4, tn = (tid & 15) * 4;
  float acc[4][4] = {};
  for (int k0 = 0; k0 < K; k0 += 16) {
    for (int q = tid; q < 16 * 64; q += 256) {
      const int kk = A_T ? q >> 6 : q & 15, mm = A_T ? q & 63 : q >> 4;
      const int gm = m0 + mm, gk = k0 + kk;
      sa[kk][mm] = (gm < M && gk < K)
                       ? (A_T ? a[(long long)gk * lda + gm] : a[(long long)gm * lda + gk])
                       : 0.f;
      const int kb = B_T ? q >> 6 : q & 15, nn = B_T ? q & 63 : q >> 4;
      const int gn = n0 + nn, gk2 = k0 + kb;
      float bvv = 0.f;
      if (gn < N && gk2 < K) {
        const long long off = B_T ? (long long)gk2 * ldb + gn : (long long)gn * ldb + gk2;
        bvv = B_BF16 ? bf16_to_f32(static_cast<const uint16_t*>(bv)[off])
                     : static_cast<const float*>(bv)[off];
      }
      sb[kb][nn] = bvv;
    }
    __syncthreads();
#pragma unroll
    for (int kk = 0; kk < 16; ++kk) {
      float av[4], bw[4];
#pragma unroll
      for (int i = 0; i < 4; ++i) av[i] = sa[kk][tm + i];
#pragma unroll
      for (int j = 0; j < 4; ++j) bw[j] = sb[kk][tn + j];
#pragma unroll
      for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j) acc[i][j] = __builtin_fmaf(av[i], bw[j], acc[i][j]);
    }
    __syncthreads();
  }
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int gm = m0 + tm + i, gn = n0 + tn + j;
      if (gm < M && gn < N) c[(long long)gm * ldc + gn] = acc[i][j];
    }
}

// One block per token: dx_t = sum over its FFN slots (k order) of the dXs
// rows + (sum over its zero slots of g) dy_t + dxr_t, fp32.
__global__ __launch_bounds__(256) void bwd_dx_kernel(const float* __restrict__ dXs,
                                                     const uint16_t* __restrict__ dy,
                                                     const float* __restrict__ dxr,
                                                     const int* __restrict__ row_of_slot,
                                                     const float* __restrict__ gate, int d, int K,
                                                     float* __restrict__ dx) {
  __shared__ int srow[64];
  __shared__ float sg[64];
  const int t = blockIdx.x, tid = threadIdx.x;
  if (tid < K) {
    srow[tid] = row_of_slot[(size_t)t * K + tid];
    sg[tid] = gate[(size_t)t * K + tid];
  }
  __syncthreads();
  float gz = 0.f;
  for (int k = 0; k < K; ++k)
    if (srow[k] < 0) gz += sg[k];
  for (int c = tid; c < d; c += 256) {
    float v = 0.f;
    for (int k = 0; k < K; ++k)
      if (srow[k] >= 0) v += dXs[(size_t)srow[k] * d + c];
    v += gz * bf16_to_f32(dy[(size_t)t * d + c]);
    v += dxr[(size_t)t * d + c];
    dx[(size_t)t * d + c] = v;
  }
}

void launch_tile_prefix(const int* counts, int N, int rows, int* prefix, hipStream_t s) {
  tile_prefix_kernel<<<1, 64, 0, s>>>(counts, N, rows, prefix);
}
void launch_bwd_rows(const float* U, const float* Q, const int* perm, const float* gate,
                     const int* s_dev, int I, uint16_t* dU, uint16_t* Hg, float* dg, int grid,
                     hipStream_t s) {
  bwd_rows_kernel<<<grid, 256, 0, s>>>(U, Q, perm, gate, s_dev, I, dU, Hg, dg);
}
void launch_bwd_zero_dg(const uint16_t* x, const uint16_t* dy, const int* idx, int T, int d, int K,
                        int N, float* dg, hipStream_t s) {
  const int grid = std::max(1, std::min(2048, (T + 3) / 4));
  bwd_zero_dg_kernel<<<grid, 256, 0, s>>>(x, dy, idx, T, d, K, N, dg);
}
void launch_bwd_router_dz(const float* logits, const int* idx, const float* gate, const float* dg,
                          int T, int E, int K, float* dz, hipStream_t s) {
  const int grid = std::max(1, std::min(2048, (T + 3) / 4));
  bwd_router_dz_kernel<<<grid, 256, 0, s>>>(logits, idx, gate, dg, T, E, K, dz);
}
void launch_router_grads(const float* dz, const uint16_t* x, const float* wr, int T, int E, int d,
                         float* dwr, float* dxr, hipStream_t s) {
  // dW_r[i][c] = sum_t dz[t][i] x[t][c]
  f32_gemm_kernel<true, true, true><<<dim3((E + 63) / 64, (d + 63) / 64), 256, 0, s>>>(
      dz, E, x, d, dwr, d, E, d, T);
  // dxr[t][c] = sum_i dz[t][i] W_r[i][c]
  f32_gemm_kernel<false, true, false><<<dim3((T + 63) / 64, (d + 63) / 64), 256, 0, s>>>(
      dz, E, wr, d, dxr, d, T, d, E);
}
void launch_bwd_dx(const float* dXs, const uint16_t* dy, const float* dxr, const int* row_of_slot,
                   const float* gate, int T, int d, int K, float* dx, hipStream_t s) {
  bwd_dx_kernel<<<T, 256, 0, s>>>(dXs, dy, dxr, row_of_slot, gate, d, K, dx);
}

}  // namespace lcmoe
