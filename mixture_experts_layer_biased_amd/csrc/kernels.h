// Internal launcher interface between the C-ABI host code and the kernels.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace lcmoe {

// Every FFN expert with routed rows runs on the LDS-tiled grouped GEMM in
// M-tiles of at most kBigTileRows rows (320 = mean 256 rows per expert at the
// fp8 batch plus its spread, so those experts stream their weights once).
constexpr int kBigTileRows = 320;

// Grouped GEMM tile widths (output columns per block).
constexpr int kBigColsGateUp = 128;    // H columns per large gate/up block
constexpr int kBigColsDown = 256;      // Y columns per large down block

struct GemmArgs {
  const void* w;           // expert weights [N][rows_total][kdim], bf16 or fp8 codes
  const float* wscale;     // fp8: [N][rows_total/128][kdim/128]
  const uint16_t* src;     // gate/up: x [T][d]; down: H [S][I]
  const uint8_t* src8;     // fp8 activations: E4M3FN codes of src, same layout
  const float* ascale;     // fp8 activations: per-row scale (gate/up: [T]; down: [S])
  const int* perm;         // FFN slot ids grouped by expert (gate/up gather)
  const int* offsets;      // [N+1]
  const int* counts;       // [E]
  const int* mt_prefix;    // [N+1] M-tile prefix over the FFN experts
  const int* meta;         // [0] #touched FFN experts, [1] #M-tiles, [2] S
  uint16_t* out;           // gate/up: H [S][I]; down: Y [S][d]
  int kdim;                // reduction length (d or I)
  int n_out;               // output columns (I or d)
  int rows_total;          // weight rows per expert (2I or d)
  int topk;
  int n_ffn;
  int nslices;             // column blocks per expert
  // Gate/up with bf16 weights: when not null, the pre-activations u = [a; c]
  // of every slot row are also stored, fp32 [S][2I] in slot order.
  float* usave;
  // Backward of gate/up (launch_gemm_big_bwd_u only): per slot row s,
  // Q = W2^T dy [S][I] fp32 and the slot gates (indexed by slot id) are read;
  // out receives g h (bf16 [S][I]), bdu dU = [dh c silu'(a); dh silu(a)]
  // (bf16 [S][2I]) and bdgp the partial sums of <Q, h> per 32 columns
  // (fp32 [S][4 nslices]).
  const float* bq;
  const float* bgate;
  uint16_t* bdu;
  float* bdgp;
};

void launch_router(const uint16_t* x, const float* wr, float* zpart, int T, int E, int d,
                   int ks, int kchunk, hipStream_t s);
void launch_topk(const float* zpart, int ks, const float* bias, int T, int E, int K, int* idx,
                 float* gate, float* logits_out, hipStream_t s);
void launch_permute(const int* idx, int T, int K, int E, int N, int ntile,
                    unsigned long long* masks, int* tilecnt, int* tileoff, int* counts,
                    int* offsets, int* mt_prefix, int* meta, int* perm,
                    int* row_of_slot, hipStream_t s);
void launch_gemm_big(const GemmArgs& a, bool gateup, bool fp8, int grid, hipStream_t s);
// The large-M gate/up GEMM with the backward epilogue (bf16 weights; every
// expert with slots, M-tiles from mt_prefix, meta[1] = tile count).
void launch_gemm_big_bwd_u(const GemmArgs& a, int grid, hipStream_t s);
// Large-M GEMM with fp8 weights and fp8 activations (src8, ascale).
void launch_gemm_big_a8(const GemmArgs& a, bool gateup, int grid, hipStream_t s);
// Per-row E4M3FN quantization of bf16 rows: q [rows][cols] codes, scale
// [rows] = amax/448 (1 for a zero row). The row count is read on the device
// (*rows_dev) when rows_dev is not null, else `rows`; grid-stride over rows.
void launch_quant_rows(const uint16_t* src, int rows, const int* rows_dev, int cols, uint8_t* q,
                       float* scale, int grid, hipStream_t s);
void launch_combine(const uint16_t* x, const uint16_t* Y, const int* idx, const float* gate,
                    const int* row_of_slot, int T, int d, int K, uint16_t* y, hipStream_t s);
// Zero bytes [p, p + bytes) of a 4-byte aligned buffer (bytes % 4 == 0).
void launch_zero_fill(void* p, size_t bytes, hipStream_t s);
void launch_bias_update(const int* counts, int N, int K, int t_all, double mu, double k_e,
                        float* bias, hipStream_t s);

// Backward grouped GEMMs: C_e[m][n] = sum_k A_e(m, k) B_e(n, k) per FFN
// expert (see bwd_gemm.hip). dgrad: A = slot rows (k-contiguous), B = the
// expert's weight matrix read i-contiguous, M = the expert's slot count,
// output rows = slot rows (fp32). wgrad: A and B = slot rows read
// i-contiguous, K = the slot count, output rows e * M + m.
constexpr int kBwdTileM = 256;       // rows per dgrad M tile (slot rows)
constexpr int kBwdTileNDgrad = 256;  // columns per dgrad tile
struct BwdGemmArgs {
  const uint16_t* a;       // A base (bf16): slot-row matrix, row 0 = slot row 0
  long long a_ld;          // row stride (elements)
  const uint16_t* b;       // B base: weights [N][rows][b_ld] (dgrad) or slot rows (wgrad)
  long long b_ld;
  long long b_estride;     // dgrad: elements per expert of B
  void* c;                 // output, fp32 or bf16
  long long c_ld;
  int M, N, K;             // fixed extents (M unused in dgrad, K in wgrad)
  int m_store;             // wgrad: output rows stored, m < min(M, m_store)
  const int* counts;
  const int* offsets;
  const int* tile_prefix;  // [N+1] prefix of ceil(count / kBwdTileM) (dgrad)
  int n_ffn;
  int b_wrap;              // f32 wgrad: B row k is row k mod b_wrap (0: no wrap)
};
int bwd_dgrad_grid(long long smax, int n_ffn, int n_cols);
// Persistent weight-gradient grid: one block per CU, at most max_blocks when
// max_blocks > 0 (a multiple of 8).
int bwd_wgrad_grid(int n_ffn, int M, int N, int max_blocks = 0);
// Compute units of the current device (256 if the query fails).
int bwd_device_cus();
// The backward's grouped GEMMs on the ring kernel (dgrad, weights read
// k-major: W2^T dy, dU W13, the router's dz W_r; wgrad: the weight
// gradients, dW_r).
enum BwdOp { kBwdQ = 2, kBwdDx, kBwdDw2, kBwdDw13, kBwdRouterDx, kBwdRouterDw };
void launch_bwd_dgrad(const BwdGemmArgs& g, BwdOp op, int grid, hipStream_t s);
void launch_bwd_wgrad(const BwdGemmArgs& g, BwdOp op, int grid, hipStream_t s);
// wgrad with fp32 output and 128 x 128 tiles (the router gradient: few tiles, long k)
void launch_bwd_wgrad_f32(const BwdGemmArgs& g, hipStream_t s);
void launch_gather_rows(const uint16_t* x, const uint16_t* dy, const int* perm, const int* s_dev,
                        int topk, int d, uint16_t* xs, uint16_t* dys, int grid, hipStream_t s);
// prefix[e] = sum_{e' < e} ceil(counts[e'] / rows), prefix[N] the total,
// also written to *total when total is not null.
void launch_tile_prefix(const int* counts, int N, int rows, int* prefix, int* total,
                        hipStream_t s);
// dg of the FFN slots: dg[perm[s]] = sum over the P partials of row s, in order.
void launch_bwd_dg_reduce(const float* dgp, int P, const int* perm, const int* s_dev, float* dg,
                          int grid, hipStream_t s);
// The SiLU backward per FFN slot row from the forward's saved u (fp32): dU,
// g h and dg of the slot.
void launch_bwd_silu_saved(const float* U, const float* Q, const int* perm, const float* gate,
                           const int* s_dev, int I, uint16_t* dU, uint16_t* Hg, float* dg, int grid,
                           hipStream_t s);
void launch_bwd_zero_dg(const uint16_t* x, const uint16_t* dy, const int* idx, int T, int d, int K,
                        int N, float* dg, hipStream_t s);
void launch_bwd_router_dz(const float* logits, const int* idx, const float* gate, const float* dg,
                          int T, int E, int Ep, int K, uint16_t* dzp, uint16_t* dzt, hipStream_t s);
// Router gradients on bf16 MFMA from exact planes: dx_r = dz W_r, dW_r = dz^T x
// (the three dz planes stacked along k, x read in place for each).
// wsp [6 Ep][d] and rg [6] are scratch.
void launch_router_grads(const uint16_t* dzp, const uint16_t* dzt, const uint16_t* x,
                         const float* wr, int T, int E, int Ep, int d, uint16_t* wsp, int* rg,
                         float* dwr, float* dxr, hipStream_t s);
void launch_bwd_dx(const float* dXs, const uint16_t* dy, const float* dxr, const int* row_of_slot,
                   const float* gate, int T, int d, int K, float* dx, hipStream_t s);

// Router-side statistics: kStatsBlocks partial rows of D+2 doubles in `part`.
constexpr int kStatsBlocks = 1024;
void launch_router_stats(const float* logits, const uint16_t* x, int T, int E, int d, int N, int D,
                         int K, const int* counts, double k_e, double alpha, double lambda,
                         double* part, double* stats, hipStream_t s);

}  // namespace lcmoe
