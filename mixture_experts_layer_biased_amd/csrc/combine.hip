// Weighted combine with the zero-computation-expert identity, and the
// expert-bias update.
#include <algorithm>

#include "common.h"
#include "kernels.h"

namespace lcmoe {

// ---------------------------------------------------------------------------
// Combine ("LongCat-Flash" llm-wiki entity page, section 2.1: the MoE sum
// over all N+Z experts with gates g_i; a zero-computation expert returns its
// input unchanged and costs no FLOPs):
//   y_t = sum_k g_tk * v_tk,  v_tk = Y[row_of_slot(t,k)] for an FFN slot,
//                             v_tk = x_t for a zero-computation slot,
// accumulated in fp32 in k order, rounded once to bf16.
//
// A token's row is 16-byte chunks, one per thread; the threads of a token
// are the chunk count rounded up to a power of two, 64 to 256. A 256-thread
// block holds 1, 2 or 4 tokens (narrow rows fill the block). A row wider
// than 256 chunks is walked by its threads in turn, or, for a batch under
// 1,024 tokens, spread over gridDim.y blocks so that the batch covers the
// chip (at 8,192 LongCat-shape tokens the spread form was 6% slower: the
// three pieces of a 12 KB row are then read far apart in time). The rows of
// four slots are requested together, then added in k order (eight at a time
// measured 8% slower at that batch).
// ---------------------------------------------------------------------------
__global__ __launch_bounds__(256) void combine_kernel(const uint16_t* __restrict__ x,
                                                      const uint16_t* __restrict__ Y,
                                                      const float* __restrict__ gate,
                                                      const int* __restrict__ row_of_slot, int T,
                                                      int d, int K, int tpt_log2,
                                                      uint16_t* __restrict__ y) {
  __shared__ float sg[256];  // tokens per block (<= 4) x K (<= 64)
  __shared__ int srow[256];
  const int tid = threadIdx.x;
  const int tpt = 1 << tpt_log2, tpb = 256 >> tpt_log2;
  const int t0 = blockIdx.x * tpb;
  for (int i = tid; i < tpb * K; i += 256) {
    const bool ok = t0 + i / K < T;
    sg[i] = ok ? gate[(size_t)t0 * K + i] : 0.f;
    srow[i] = ok ? row_of_slot[(size_t)t0 * K + i] : -1;
  }
  __syncthreads();
  const int lt = tid >> tpt_log2;
  const int t = t0 + lt;
  if (t >= T) return;
  const float* g = sg + lt * K;
  const int* rows = srow + lt * K;
  for (int c = blockIdx.y * tpt + (tid & (tpt - 1)); c < (d >> 3); c += tpt * gridDim.y) {
    const uint4 xv = *reinterpret_cast<const uint4*>(x + (size_t)t * d + 8 * c);
    float acc[8];
#pragma unroll
    for (int i = 0; i < 8; ++i) acc[i] = 0.f;
    for (int k0 = 0; k0 < K; k0 += 4) {
      uint4 v[4];
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const int r = k0 + j < K ? rows[k0 + j] : -1;
        v[j] = r >= 0 ? *reinterpret_cast<const uint4*>(Y + (size_t)r * d + 8 * c) : xv;
      }
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        if (k0 + j >= K) break;
        const float gk = g[k0 + j];
        acc[0] += gk * bf16_lo(v[j].x);
        acc[1] += gk * bf16_hi(v[j].x);
        acc[2] += gk * bf16_lo(v[j].y);
        acc[3] += gk * bf16_hi(v[j].y);
        acc[4] += gk * bf16_lo(v[j].z);
        acc[5] += gk * bf16_hi(v[j].z);
        acc[6] += gk * bf16_lo(v[j].w);
        acc[7] += gk * bf16_hi(v[j].w);
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

// Zero fill of a caller buffer (outputs of calls with no tokens). A kernel
// rather than a memset node, so every entry point enqueues kernels only and
// can be captured into a HIP graph. Words before the first 16-byte boundary
// and after the last are written one at a time, the rest 16 bytes at a time.
__global__ __launch_bounds__(256) void zero_fill_kernel(uint32_t* __restrict__ p, size_t head,
                                                        size_t nvec, size_t tail) {
  const size_t i = (size_t)blockIdx.x * blockDim.x + threadIdx.x;
  const size_t stride = (size_t)gridDim.x * blockDim.x;
  if (i < head) p[i] = 0u;
  uint4* v = reinterpret_cast<uint4*>(p + head);
  for (size_t j = i; j < nvec; j += stride) v[j] = make_uint4(0u, 0u, 0u, 0u);
  if (i < tail) p[head + 4 * nvec + i] = 0u;
}

void launch_zero_fill(void* p, size_t bytes, hipStream_t s) {
  const size_t words = bytes / 4;
  if (words == 0) return;
  const size_t mis = ((uintptr_t)p & 15u) / 4;  // p is 4-byte aligned
  const size_t head = std::min(words, mis ? 4 - mis : 0);
  const size_t nvec = (words - head) / 4;
  const size_t tail = words - head - 4 * nvec;
  const size_t blocks = std::max<size_t>(1, std::min<size_t>(8192, (nvec + 255) / 256));
  zero_fill_kernel<<<(unsigned)blocks, 256, 0, s>>>(static_cast<uint32_t*>(p), head, nvec, tail);
}

void launch_combine(const uint16_t* x, const uint16_t* Y, const int* /*idx*/, const float* gate,
                    const int* row_of_slot, int T, int d, int K, uint16_t* y, hipStream_t s) {
  const int nch = d / 8;
  int lg = 6;  // threads per token: 64..256, at least the chunk count when it fits
  while (lg < 8 && (1 << lg) < nch) ++lg;
  const dim3 grid((unsigned)((T + (256 >> lg) - 1) / (256 >> lg)),
                  T < 1024 ? (unsigned)((nch + (1 << lg) - 1) >> lg) : 1u);
  combine_kernel<<<grid, 256, 0, s>>>(x, Y, gate, row_of_slot, T, d, K, lg, y);
}

void launch_bias_update(const int* counts, int N, int K, int t_all, double mu, double k_e,
                        float* bias, hipStream_t s) {
  bias_update_kernel<<<(N + 255) / 256, 256, 0, s>>>(counts, N, K, t_all, mu, k_e, bias);
}

}  // namespace lcmoe
