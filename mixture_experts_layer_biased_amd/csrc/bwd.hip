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
// The expert GEMMs are in bwd_gemm.hip (W2^T dy, dU W13, the weight
// gradients) and gemm.hip (u = W13 x with the SiLU backward in its epilogue).
#include <algorithm>

#include "common.h"
#include "kernels.h"

namespace lcmoe {

// prefix[e] = sum_{e' < e} ceil(counts[e'] / rows), one wave (N <= 2048).
__global__ __launch_bounds__(64) void tile_prefix_kernel(const int* __restrict__ counts, int N,
                                                         int rows, int* __restrict__ prefix,
                                                         int* __restrict__ total) {
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
  if (lane == 63) {
    prefix[N] = incl;
    if (total != nullptr) *total = incl;
  }
}

// One thread per FFN slot row s < S (S read on the device): dg of its slot
// is the sum of the row's P partials of <Q, h>, in order.
__global__ __launch_bounds__(256) void bwd_dg_reduce_kernel(const float* __restrict__ dgp, int P,
                                                            const int* __restrict__ perm,
                                                            const int* __restrict__ s_dev,
                                                            float* __restrict__ dg) {
  const int S = *s_dev;
  for (int s = blockIdx.x * 256 + threadIdx.x; s < S; s += gridDim.x * 256) {
    const float* p = dgp + (size_t)s * P;
    float v = 0.f;
    for (int j = 0; j < P; ++j) v += p[j];
    dg[perm[s]] = v;
  }
}

// One wave per FFN slot row s < S (S read on the device), from the forward's
// saved u = [a; c] (fp32) and Q_s = (W2^T dy)_s: h = silu(a) c; dg = <Q_s, h>;
// dh = g Q_s; dU = [dh c silu'(a); dh silu(a)] and g h (bf16). Four columns
// per lane and step.
__global__ __launch_bounds__(256) void bwd_silu_saved_kernel(const float* __restrict__ U,
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
    uint16_t* du = dU + (size_t)s * 2 * I;
    uint16_t* hg = Hg + (size_t)s * I;
    float part = 0.f;
    for (int j = 4 * lane; j < I; j += 256) {
      const float4 av = *reinterpret_cast<const float4*>(u + j);
      const float4 cv = *reinterpret_cast<const float4*>(u + I + j);
      const float4 qv = *reinterpret_cast<const float4*>(q + j);
      const float a[4] = {av.x, av.y, av.z, av.w};
      const float c[4] = {cv.x, cv.y, cv.z, cv.w};
      const float qa[4] = {qv.x, qv.y, qv.z, qv.w};
      float da[4], dc[4], h[4];
#pragma unroll
      for (int t = 0; t < 4; ++t) {
        const float sg = 1.0f / (1.0f + expf(-a[t]));
        const float si = a[t] * sg;
        const float hv = si * c[t];
        part += qa[t] * hv;
        const float dh = g * qa[t];
        da[t] = dh * c[t] * (sg * (1.0f + a[t] * (1.0f - sg)));
        dc[t] = dh * si;
        h[t] = g * hv;
      }
      *reinterpret_cast<uint2*>(du + j) = make_uint2(pack_bf16x2(da[0], da[1]), pack_bf16x2(da[2], da[3]));
      *reinterpret_cast<uint2*>(du + I + j) =
          make_uint2(pack_bf16x2(dc[0], dc[1]), pack_bf16x2(dc[2], dc[3]));
      *reinterpret_cast<uint2*>(hg + j) = make_uint2(pack_bf16x2(h[0], h[1]), pack_bf16x2(h[2], h[3]));
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
// dz_i = p_i (dp_i - c) with dp_i = dg_tk at the selected experts. dz is
// written as its three exact bf16 planes (hi, mid, lo), experts padded to Ep
// with zeros, in the two layouts the router-gradient GEMMs read:
//   dzp[t][6 Ep]: segments (hi, hi, mid, hi, lo, mid), the A operand of
//     dx_r = dz W_r against W_r's planes (hi, mid, hi, lo, hi, mid): the six
//     plane products above 2^-24 of the product;
//   dzt[j T + t][Ep]: plane j, the A operand of dW_r = dz^T x (x is bf16, so
//     the three plane products are exact).
__global__ __launch_bounds__(256) void bwd_router_dz_kernel(const float* __restrict__ logits,
                                                            const int* __restrict__ idx,
                                                            const float* __restrict__ gate,
                                                            const float* __restrict__ dg, int T,
                                                            int E, int Ep, int K,
                                                            uint16_t* __restrict__ dzp,
                                                            uint16_t* __restrict__ dzt) {
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
    uint16_t* prow = dzp + (size_t)t * 6 * Ep;
    for (int i = lane; i < Ep; i += 64) {
      float v = 0.f;
      if (i < E) {
        float dp = 0.f;
        for (int k = 0; k < K; ++k)
          if (idx[(size_t)t * K + k] == i) dp = dg[(size_t)t * K + k];
        const float p = expf(z[i] - m) / s;
        v = p * (dp - c);
      }
      uint16_t hi, mid, lo;
      split3(v, hi, mid, lo);
      prow[i] = hi;
      prow[Ep + i] = hi;
      prow[2 * Ep + i] = mid;
      prow[3 * Ep + i] = hi;
      prow[4 * Ep + i] = lo;
      prow[5 * Ep + i] = mid;
      dzt[(size_t)t * Ep + i] = hi;
      dzt[((size_t)T + t) * Ep + i] = mid;
      dzt[((size_t)2 * T + t) * Ep + i] = lo;
    }
  }
}

// W_r's planes stacked to match dzp: wsp[s Ep + i][c] for segments s = 0..5
// = planes (hi, mid, hi, lo, hi, mid) of W_r[i][c], rows i >= E zero. Thread
// 0 also writes the one-group metadata of the two router-gradient GEMMs:
// rg = {T, 0, 0, ceil(T / kBwdTileM), 3 T, 0} (counts, offsets and tile prefix of
// dx_r; counts and offsets of dW_r).
__global__ __launch_bounds__(256) void router_w_split_kernel(const float* __restrict__ wr, int E,
                                                             int Ep, int d, int T,
                                                             uint16_t* __restrict__ wsp,
                                                             int* __restrict__ rg) {
  if (blockIdx.x == 0 && threadIdx.x == 0) {
    rg[0] = T;
    rg[1] = 0;
    rg[2] = 0;
    rg[3] = (T + kBwdTileM - 1) / kBwdTileM;
    rg[4] = 3 * T;
    rg[5] = 0;
  }
  const long long n4 = (long long)Ep * d / 4;
  for (long long q = blockIdx.x * 256ll + threadIdx.x; q < n4; q += (long long)gridDim.x * 256) {
    const long long el = q * 4;
    const int i = (int)(el / d), c = (int)(el - (long long)i * d);
    float4 w = make_float4(0.f, 0.f, 0.f, 0.f);
    if (i < E) w = *reinterpret_cast<const float4*>(wr + (size_t)i * d + c);
    uint16_t h[4], m[4], l[4];
    split3(w.x, h[0], m[0], l[0]);
    split3(w.y, h[1], m[1], l[1]);
    split3(w.z, h[2], m[2], l[2]);
    split3(w.w, h[3], m[3], l[3]);
    const uint2 H = make_uint2(h[0] | (uint32_t)h[1] << 16, h[2] | (uint32_t)h[3] << 16);
    const uint2 M = make_uint2(m[0] | (uint32_t)m[1] << 16, m[2] | (uint32_t)m[3] << 16);
    const uint2 Lo = make_uint2(l[0] | (uint32_t)l[1] << 16, l[2] | (uint32_t)l[3] << 16);
    const uint2 seg[6] = {H, M, H, Lo, H, M};
#pragma unroll
    for (int sg = 0; sg < 6; ++sg)
      *reinterpret_cast<uint2*>(wsp + ((size_t)sg * Ep + i) * d + c) = seg[sg];
  }
}

// One block per token: dx_t = sum over its FFN slots (k order) of the dXs
// rows + (sum over its zero slots of g) dy_t + dxr_t, fp32. Four columns per
// thread (16-byte loads and stores; d is a multiple of 32).
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
  for (int c = 4 * tid; c < d; c += 4 * 256) {
    float4 v = make_float4(0.f, 0.f, 0.f, 0.f);
    for (int k = 0; k < K; ++k)
      if (srow[k] >= 0) {
        const float4 r = *reinterpret_cast<const float4*>(dXs + (size_t)srow[k] * d + c);
        v.x += r.x;
        v.y += r.y;
        v.z += r.z;
        v.w += r.w;
      }
    const uint2 yb = *reinterpret_cast<const uint2*>(dy + (size_t)t * d + c);
    const float4 xr = *reinterpret_cast<const float4*>(dxr + (size_t)t * d + c);
    v.x += gz * bf16_lo(yb.x);
    v.y += gz * bf16_hi(yb.x);
    v.z += gz * bf16_lo(yb.y);
    v.w += gz * bf16_hi(yb.y);
    v.x += xr.x;
    v.y += xr.y;
    v.z += xr.z;
    v.w += xr.w;
    *reinterpret_cast<float4*>(dx + (size_t)t * d + c) = v;
  }
}

void launch_tile_prefix(const int* counts, int N, int rows, int* prefix, int* total,
                        hipStream_t s) {
  tile_prefix_kernel<<<1, 64, 0, s>>>(counts, N, rows, prefix, total);
}
void launch_bwd_dg_reduce(const float* dgp, int P, const int* perm, const int* s_dev, float* dg,
                          int grid, hipStream_t s) {
  bwd_dg_reduce_kernel<<<grid, 256, 0, s>>>(dgp, P, perm, s_dev, dg);
}
void launch_bwd_silu_saved(const float* U, const float* Q, const int* perm, const float* gate,
                           const int* s_dev, int I, uint16_t* dU, uint16_t* Hg, float* dg, int grid,
                           hipStream_t s) {
  bwd_silu_saved_kernel<<<grid, 256, 0, s>>>(U, Q, perm, gate, s_dev, I, dU, Hg, dg);
}
void launch_bwd_zero_dg(const uint16_t* x, const uint16_t* dy, const int* idx, int T, int d, int K,
                        int N, float* dg, hipStream_t s) {
  const int grid = std::max(1, std::min(2048, (T + 3) / 4));
  bwd_zero_dg_kernel<<<grid, 256, 0, s>>>(x, dy, idx, T, d, K, N, dg);
}
void launch_bwd_router_dz(const float* logits, const int* idx, const float* gate, const float* dg,
                          int T, int E, int Ep, int K, uint16_t* dzp, uint16_t* dzt, hipStream_t s) {
  const int grid = std::max(1, std::min(2048, (T + 3) / 4));
  bwd_router_dz_kernel<<<grid, 256, 0, s>>>(logits, idx, gate, dg, T, E, Ep, K, dzp, dzt);
}
void launch_router_grads(const uint16_t* dzp, const uint16_t* dzt, const uint16_t* x,
                         const float* wr, int T, int E, int Ep, int d, uint16_t* wsp, int* rg,
                         float* dwr, float* dxr, hipStream_t s) {
  const long long n4 = (long long)Ep * d / 4;
  router_w_split_kernel<<<(int)std::min<long long>(4096, (n4 + 255) / 256), 256, 0, s>>>(
      wr, E, Ep, d, T, wsp, rg);
  BwdGemmArgs g{};
  g.n_ffn = 1;
  // dx_r[t][c] = sum over the six plane products of dz[t][i] W_r[i][c]
  g.a = dzp; g.a_ld = 6ll * Ep;
  g.b = wsp; g.b_ld = d; g.b_estride = 0;
  g.c = dxr; g.c_ld = d; g.N = d; g.K = 6 * Ep;
  g.counts = rg; g.offsets = rg + 1; g.tile_prefix = rg + 2;
  launch_bwd_dgrad(g, kBwdRouterDx, bwd_dgrad_grid(T, 1, d), s);
  // dW_r[i][c] = sum over the 3 T plane rows k of dz[k][i] x[k mod T][c]
  BwdGemmArgs w{};
  w.n_ffn = 1;
  w.a = dzt; w.a_ld = Ep;
  w.b = x; w.b_ld = d; w.b_wrap = T;
  w.c = dwr; w.c_ld = d; w.M = Ep; w.m_store = E; w.N = d;
  w.counts = rg + 4; w.offsets = rg + 5;
  launch_bwd_wgrad_f32(w, s);
}
void launch_bwd_dx(const float* dXs, const uint16_t* dy, const float* dxr, const int* row_of_slot,
                   const float* gate, int T, int d, int K, float* dx, hipStream_t s) {
  bwd_dx_kernel<<<T, 256, 0, s>>>(dXs, dy, dxr, row_of_slot, gate, d, K, dx);
}

}  // namespace lcmoe
