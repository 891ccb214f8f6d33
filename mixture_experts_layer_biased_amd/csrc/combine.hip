// Weighted combine with the zero-computation-expert identity, and the
// expert-bias update.
#include "common.h"
#include "kernels.h"

namespace lcmoe {

// ---------------------------------------------------------------------------
// Combine ("LongCat-Flash" llm-wiki entity page, section 2.1: the MoE sum
// over all N+Z experts with gates g_i; a zero-computation expert returns its
// input unchanged and costs no FLOPs):
//   y_t = sum_k g_tk * v_tk,  v_tk = Y[row_of_slot(t,k)] for an FFN slot,
//                             v_tk = x_t for a zero-computation slot,
// accumulated in fp32 in k order, rounded once to bf16. One block per token,
// 16-byte coalesced loads of whole rows.
// ---------------------------------------------------------------------------
__global__ __launch_bounds__(256) void combine_kernel(const uint16_t* __restrict__ x,
                                                      const uint16_t* __restrict__ Y,
                                                      const float* __restrict__ gate,
                                                      const int* __restrict__ row_of_slot,
                                                      int d, int K, uint16_t* __restrict__ y) {
  __shared__ float sg[64];
  __shared__ int srow[64];
  const int t = blockIdx.x, tid = threadIdx.x;
  if (tid < K) {
    sg[tid] = gate[(size_t)t * K + tid];
    srow[tid] = row_of_slot[(size_t)t * K + tid];
  }
  __syncthreads();
  const int nch = d >> 3;
  for (int c = tid; c < nch; c += 256) {
    const uint4 xv = *reinterpret_cast<const uint4*>(x + (size_t)t * d + 8 * c);
    float acc[8];
#pragma unroll
    for (int i = 0; i < 8; ++i) acc[i] = 0.f;
    // Four slots' rows are requested together, then added in k order.
    for (int k0 = 0; k0 < K; k0 += 4) {
      uint4 v[4];
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const int r = k0 + j < K ? srow[k0 + j] : -1;
        v[j] = r >= 0 ? *reinterpret_cast<const uint4*>(Y + (size_t)r * d + 8 * c) : xv;
      }
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        if (k0 + j >= K) break;
        const float g = sg[k0 + j];
        acc[0] += g * bf16_lo(v[j].x);
        acc[1] += g * bf16_hi(v[j].x);
        acc[2] += g * bf16_lo(v[j].y);
        acc[3] += g * bf16_hi(v[j].y);
        acc[4] += g * bf16_lo(v[j].z);
        acc[5] += g * bf16_hi(v[j].z);
        acc[6] += g * bf16_lo(v[j].w);
        acc[7] += g * bf16_hi(v[j].w);
      }
    }
    uint4 o;
    o.x = pack_bf16x2(acc[0], acc[1]);
    o.y = pack_bf16x2(acc[2], acc[3]);
    o.z = pack_bf16x2(acc[4], acc[5]);
    o.w = pack_bf16x2(acc[6], acc[7]);
    *reinterpret_cast<uint4*>(y + (size_t)t * d + 8 * c) = o;
  }
}

// ---------------------------------------------------------------------------
// Expert-bias update ("LongCat-Flash" section 2.1, the bias-adaptation law
// db_i = mu (K_e/K * 1/N - T_i/(K T_all))), FFN experts only, evaluated as
// the single fraction mu*(K_e*T_all - N*T_i)/(K*N*T_all) in fp64, one IEEE
// operation at a time (no contraction), then rounded once into fp32.
// ---------------------------------------------------------------------------
__global__ __launch_bounds__(256) void bias_update_kernel(const int* __restrict__ counts, int N,
                                                          int K, int t_all, double mu,
                                                          double k_e, float* __restrict__ bias) {
#pragma clang fp contract(off)
  const int i = blockIdx.x * blockDim.x + threadIdx.x;
  if (i >= N) return;
  const double den = (double)K * (double)N * (double)t_all;
  const double num = k_e * (double)t_all - (double)N * (double)counts[i];
  const double delta = (mu * num) / den;
  bias[i] = (float)((double)bias[i] + delta);
}

void launch_combine(const uint16_t* x, const uint16_t* Y, const int* /*idx*/, const float* gate,
                    const int* row_of_slot, int T, int d, int K, uint16_t* y, hipStream_t s) {
  combine_kernel<<<T, 256, 0, s>>>(x, Y, gate, row_of_slot, d, K, y);
}

void launch_bias_update(const int* counts, int N, int K, int t_all, double mu, double k_e,
                        float* bias, hipStream_t s) {
  bias_update_kernel<<<(N + 255) / 256, 256, 0, s>>>(counts, N, K, t_all, mu, k_e, bias);
}

}  // namespace lcmoe
