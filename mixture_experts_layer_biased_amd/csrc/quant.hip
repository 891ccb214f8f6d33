// Per-row fp8 activation quantization, for fp8 weights with fp8 activations.
//
// Method: the "LongCat-Flash" pages name FP8 quantization and an FP8
// deployment without the activation scheme; the reading used throughout:
// each row v (an expert input row x_t, or an intermediate row H after its
// bf16 rounding) gets one fp32 scale s = fl32(amax|v| / 448) (1 for an
// all-zero row), codes q = round-to-nearest-even E4M3FN of fl32(v / s)
// clamped to +-448 (one correctly rounded fp32 division per element, then
// the hardware conversion), value q * s.
#include "common.h"
#include "kernels.h"

namespace lcmoe {

// One wave per row (grid-stride): pass 1 takes the row's |max|, pass 2
// quantizes eight values per lane step.
__global__ __launch_bounds__(256) void quant_rows_kernel(const uint16_t* __restrict__ src, int rows,
                                                         const int* __restrict__ rows_dev,
                                                         int cols, uint8_t* __restrict__ q,
                                                         float* __restrict__ scale) {
  const int lane = threadIdx.x & 63;
  const int nrows = rows_dev != nullptr ? *rows_dev : rows;
  const int wpb = blockDim.x >> 6;
  const int nch = cols >> 3;
  for (int r = blockIdx.x * wpb + (threadIdx.x >> 6); r < nrows; r += gridDim.x * wpb) {
    const uint4* row = reinterpret_cast<const uint4*>(src + (size_t)r * cols);
    float m = 0.f;
    for (int c = lane; c < nch; c += 64) {
      const uint4 v = row[c];
      const uint32_t u[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
      for (int k = 0; k < 4; ++k) m = fmaxf(m, fmaxf(fabsf(bf16_lo(u[k])), fabsf(bf16_hi(u[k]))));
    }
    m = wave_max(m);
    const float s = m > 0.f ? m / 448.f : 1.f;
    for (int c = lane; c < nch; c += 64) {
      const uint4 v = row[c];
      const uint32_t u[4] = {v.x, v.y, v.z, v.w};
      float y[8];
#pragma unroll
      for (int k = 0; k < 4; ++k) {
        y[2 * k] = fminf(fmaxf(bf16_lo(u[k]) / s, -448.f), 448.f);
        y[2 * k + 1] = fminf(fmaxf(bf16_hi(u[k]) / s, -448.f), 448.f);
      }
      int w0 = __builtin_amdgcn_cvt_pk_fp8_f32(y[0], y[1], 0, false);
      w0 = __builtin_amdgcn_cvt_pk_fp8_f32(y[2], y[3], w0, true);
      int w1 = __builtin_amdgcn_cvt_pk_fp8_f32(y[4], y[5], 0, false);
      w1 = __builtin_amdgcn_cvt_pk_fp8_f32(y[6], y[7], w1, true);
      *reinterpret_cast<uint2*>(q + (size_t)r * cols + 8 * c) = make_uint2(w0, w1);
    }
    if (lane == 0) scale[r] = s;
  }
}

void launch_quant_rows(const uint16_t* src, int rows, const int* rows_dev, int cols, uint8_t* q,
                       float* scale, int grid, hipStream_t s) {
  quant_rows_kernel<<<grid, 256, 0, s>>>(src, rows, rows_dev, cols, q, scale);
}

}  // namespace lcmoe
