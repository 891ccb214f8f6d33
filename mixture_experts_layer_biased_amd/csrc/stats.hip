// Router-side statistics: the device-level load-balance statistic with the
// zero-computation experts as one extra group, and the hidden z-loss.
//
// Method: "LongCat-Flash" (llm-wiki entity page), section 2.1, load-balance
// control (L_LB = alpha * sum over the D+1 groups of f_j P_j, zero experts as
// group D+1), and the training-stability section, activation stability
// (L_Z = lambda/T * sum_t (log sum_i exp|h_t^i|)^2). Forward values only.
//
// Groups: FFN expert i is in group i / (N/D); all zero experts in group D.
// P_j = mean over tokens of the softmax mass (all E unbiased logits) in group
// j; f_j = (share of the T*K slots in group j) / (target share), target
// K_e/(K D) per FFN group and (K-K_e)/K for the zero group (0 -> f_j = 0).
// The hidden states are the layer input x.
//
// Two launches, both deterministic (fixed summation orders, no atomics):
//  * stats_partial_kernel: kStatsBlocks blocks over contiguous token ranges,
//    one wave per token; per token the softmax masses of the groups (fp32)
//    and lse(|x_t|)^2 (fp32), accumulated per wave in fp64, the four waves
//    then added in order into the block's row of partials.
//  * stats_final_kernel: one block sums each column of partials (one wave
//    per column, fixed order; fp64), counts slots per group from the expert
//    counts (int64) and forms f_j, P_j, L_LB and L_Z.
#include <math.h>

#include "common.h"
#include "kernels.h"

namespace lcmoe {

constexpr int kStatsWaves = 4;

// Dynamic LDS: per wave, D + 2 doubles of sums over tokens, then E floats
// holding exp(z - max) of the wave's current token.
size_t stats_lds_bytes(int E, int D) {
  return (size_t)kStatsWaves * ((size_t)(D + 2) * sizeof(double) + (size_t)E * sizeof(float));
}

__global__ __launch_bounds__(256) void stats_partial_kernel(
    const float* __restrict__ logits, const uint16_t* __restrict__ x, int T, int E, int d, int N,
    int D, double* __restrict__ part) {
  extern __shared__ double lds_stats[];
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
  const int ng = D + 2;  // D + 1 group masses, then sum of lse^2
  const int gs = N / D;
  double* accw = lds_stats + (size_t)w * ng;
  float* eww = reinterpret_cast<float*>(lds_stats + (size_t)kStatsWaves * ng) + (size_t)w * E;
  for (int j = lane; j < ng; j += 64) accw[j] = 0.0;
  const int t0 = (int)((long long)blockIdx.x * T / gridDim.x);
  const int t1 = (int)((long long)(blockIdx.x + 1) * T / gridDim.x);
  for (int t = t0 + w; t < t1; t += kStatsWaves) {
    // softmax over all E logits of token t
    const float* z = logits + (size_t)t * E;
    float m = -INFINITY;
    for (int i = lane; i < E; i += 64) m = fmaxf(m, z[i]);
    m = wave_max(m);
    float s = 0.f;
    for (int i = lane; i < E; i += 64) {
      const float e = expf(z[i] - m);
      eww[i] = e;
      s += e;
    }
    const float tot = wave_sum(s);
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
    // group masses
    if (gs % 64 == 0) {
      // groups are whole 64-expert chunks: one wave sum per chunk, chunks
      // of a group added in order (lane 0)
      float g = 0.f;
      for (int c = 0; c < N / 64; ++c) {
        const float cs = wave_sum(eww[64 * c + lane]);
        g += cs;
        if (((c + 1) * 64) % gs == 0) {
          if (lane == 0) accw[(c * 64) / gs] += (double)(g / tot);
          g = 0.f;
        }
      }
      float zs = 0.f;
      for (int i = N + lane; i < E; i += 64) zs += eww[i];
      zs = wave_sum(zs);
      if (lane == 0) accw[D] += (double)(zs / tot);
    } else {
      // one lane per group, experts in ascending order
      for (int j = lane; j <= D; j += 64) {
        const int lo = j < D ? j * gs : N, hi = j < D ? lo + gs : E;
        float g = 0.f;
        for (int i = lo; i < hi; ++i) g += eww[i];
        accw[j] += (double)(g / tot);
      }
    }
    // hidden z-loss term: log-sum-exp of |x_t| with its maximum factored out
    // (one pass: each lane keeps a running maximum and a sum rescaled to it,
    // then the lanes' pairs are merged onto the wave maximum)
    const uint4* xr = reinterpret_cast<const uint4*>(x + (size_t)t * d);
    const int nch = d >> 3;
    float lm = 0.f, ls = 0.f;
    for (int c = lane; c < nch; c += 64) {
      const uint4 v = xr[c];
      const uint32_t u[4] = {v.x, v.y, v.z, v.w};
      float a[8];
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        a[2 * q] = fabsf(bf16_lo(u[q]));
        a[2 * q + 1] = fabsf(bf16_hi(u[q]));
      }
      float cm = a[0];
#pragma unroll
      for (int q = 1; q < 8; ++q) cm = fmaxf(cm, a[q]);
      if (cm > lm) {
        ls *= expf(lm - cm);
        lm = cm;
      }
#pragma unroll
      for (int q = 0; q < 8; ++q) ls += expf(a[q] - lm);
    }
    const float mx = wave_max(lm);
    const float se = wave_sum(ls * expf(lm - mx));
    if (lane == 0) {
      const float lse = mx + logf(se);
      accw[D + 1] += (double)lse * (double)lse;
    }
    // eww is rewritten by the next token: every lane has read it
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
  }
  __syncthreads();
  for (int j = threadIdx.x; j < ng; j += blockDim.x) {
    double v = lds_stats[j];
#pragma unroll
    for (int q = 1; q < kStatsWaves; ++q) v += lds_stats[(size_t)q * ng + j];
    part[(size_t)blockIdx.x * ng + j] = v;
  }
}

// Final step: wave w sums columns w, w + 16, ... of the partial rows (lanes
// strided over the rows in order, then the fixed butterfly of wave_sum_f64);
// thread 0 then forms f_j, P_j and the two losses in group order.
__device__ __forceinline__ double wave_sum_f64(double v) {
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) v += __shfl_xor(v, off, kWave);
  return v;
}

constexpr int kFinalWaves = 16;

__global__ __launch_bounds__(kFinalWaves * 64) void stats_final_kernel(
    const double* __restrict__ part, int nblocks, int T, int K, const int* __restrict__ counts,
    int N, int E, int D, double k_e, double alpha, double lambda, double* __restrict__ stats) {
#pragma clang fp contract(off)
  extern __shared__ double colsum[];  // D + 2 column sums, then D + 1 slot counts
  long long* slots_of = reinterpret_cast<long long*>(colsum + D + 2);
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6;
  const int ng = D + 2, gs = N / D;
  for (int j = w; j < ng; j += kFinalWaves) {
    double v = 0.0;
    for (int b = lane; b < nblocks; b += 64) v += part[(size_t)b * ng + j];
    v = wave_sum_f64(v);
    if (lane == 0) colsum[j] = v;
    if (j <= D) {  // slots of group j: an integer sum, exact in any order
      const int lo = j < D ? j * gs : N, hi = j < D ? lo + gs : E;
      long long c = 0;
      for (int i = lo + lane; i < hi; i += 64) c += counts[i];
#pragma unroll
      for (int off = 32; off >= 1; off >>= 1) c += __shfl_xor(c, off, kWave);
      if (lane == 0) slots_of[j] = c;
    }
  }
  __syncthreads();
  if (threadIdx.x != 0) return;
  double l = 0.0;  // sum_j f_j P_j in group order
  for (int j = 0; j <= D; ++j) {
    const long long slots = slots_of[j];
    double f = 0.0, P = 0.0;
    if (T > 0) {
      P = colsum[j] / (double)T;
      const double share = (double)slots / (double)((long long)T * K);
      const double target = j < D ? k_e / (double)((long long)K * D) : ((double)K - k_e) / (double)K;
      f = target > 0.0 ? share / target : 0.0;
    }
    stats[2 + j] = f;
    stats[3 + D + j] = P;
    l += f * P;
  }
  stats[0] = alpha * l;
  stats[1] = T > 0 ? lambda / (double)T * colsum[D + 1] : 0.0;
}

void launch_router_stats(const float* logits, const uint16_t* x, int T, int E, int d, int N, int D,
                         int K, const int* counts, double k_e, double alpha, double lambda,
                         double* part, double* stats, hipStream_t s) {
  const size_t lds = stats_lds_bytes(E, D);
  if (lds > 64 * 1024)  // above the default dynamic-LDS limit (at most ~98 KB here)
    (void)hipFuncSetAttribute(reinterpret_cast<const void*>(stats_partial_kernel),
                              hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
  stats_partial_kernel<<<kStatsBlocks, 256, lds, s>>>(logits, x, T, E, d, N, D, part);
  stats_final_kernel<<<1, kFinalWaves * 64, (size_t)(2 * D + 3) * sizeof(double), s>>>(
      part, kStatsBlocks, T, K, counts, N, E, D, k_e, alpha, lambda, stats);
}

}  // namespace lcmoe
