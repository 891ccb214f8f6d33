// Grouped GEMMs of the backward pass (bf16 operands, fp32 accumulation on
// v_mfma_f32_32x32x16_bf16):
//
//   C_e[m][n] = sum_k A_e(m, k) * B_e(n, k)   for every FFN expert e
//
// Two modes:
//   dgrad (bwd_dgrad_kernel): M = the expert's slot count. A is a matrix of
//     slot rows stored k-contiguous (the gathered dy rows, or dU); B is the
//     expert's weight matrix read i-contiguous (W2 for W2^T dy, W13 for
//     dU W13). Output rows are slot rows. The router's dz W_r runs in this
//     mode as one group of T rows.
//   wgrad (bwd_wgrad_stream_kernel, bf16 out; bwd_wgrad_f32_kernel, fp32
//     out): K = the expert's slot count. A and B are slot-row matrices read
//     i-contiguous (element (i, k) at row k, column i): dW2 = dY^T (g h),
//     dW13 = dU^T X. Output rows are rows of the expert's gradient matrix;
//     an expert without slots gets zeros. The router's dz^T x runs in this
//     mode (fp32) as one group of 3T plane rows.
//
// Tiles of BM x BN (per wave FM x FN fragments of 32 x 32), k stages of 64
// moved HBM/L2 -> LDS by global_load_lds_dwordx4 (one instruction fills
// 1 KB of LDS) in a ring of stages, as in the forward's large-M kernel: per
// stage, wait for this wave's copies of the stage, a raw barrier, queue the
// next stage into the slot just freed, multiply.
//
// LDS tile forms, both conflict-free for 16-lane groups:
//   k-contiguous [rows][64 k]: 128-byte rows, chunk c of row r at
//     c ^ ((r >> 1) & 7); MFMA operands read with 16-byte loads.
//   i-contiguous [64 k][128 i] sub-tiles: 256-byte rows, 64-byte window w of
//     row k at w ^ (k & 3); operands read with ds_read_b64_tr_b16, the gfx950
//     transposing LDS load, which gives each lane 4 consecutive k of one i.
// The MFMA computes the transposed tile (B as its first operand), so a lane
// holds 4 consecutive output columns of one row; each wave's 64 x 64
// sub-tiles go out through LDS as whole-row stores.
//
// Work items are laid out per XCD (blockIdx % 8): each XCD takes a
// contiguous run of (expert, n tile, m tile) (dgrad) or (expert, m tile,
// n tile) (wgrad), so the M tiles of one weight tile, and all tiles of one
// expert's operands, meet in one L2.
#include <algorithm>
#include <type_traits>

#include "common.h"
#include "kernels.h"

namespace lcmoe {

namespace {

constexpr int BK = 64;  // k per stage
// Weight-gradient tile: 2 x 4 waves of 4 x 2 fragments (256 x 256), two
// stages of 64 KB in the ring. (Measured at the prefill batch against 128 x
// 128, 128 x 256 and 256 x 128 tiles and a persistent producer/consumer
// variant: the largest tile halves the L2 -> LDS bytes per output and wins.)
constexpr int kWgWM = 2, kWgWN = 4, kWgFM = 4, kWgFN = 2;
constexpr int kWgradBM = 32 * kWgFM * kWgWM;
constexpr int kWgradBN = 32 * kWgFN * kWgWN;

template <int N>
__device__ __forceinline__ void bwait_vmcnt() {
  // gfx9 s_waitcnt: vmcnt[3:0], expcnt[6:4], lgkmcnt[11:8], vmcnt[5:4] at [15:14]
  __builtin_amdgcn_s_waitcnt((N & 15) | (7 << 4) | (15 << 8) | ((N >> 4) << 14));
}
// Wait until at most n (0..31) of this wave's vector memory operations remain.
__device__ __forceinline__ void bwait_vmcnt_upto(int n) {
  switch (n) {
    case 0: bwait_vmcnt<0>(); break;
    case 1: bwait_vmcnt<1>(); break;
    case 2: bwait_vmcnt<2>(); break;
    case 3: bwait_vmcnt<3>(); break;
    case 4: bwait_vmcnt<4>(); break;
    case 5: bwait_vmcnt<5>(); break;
    case 6: bwait_vmcnt<6>(); break;
    case 7: bwait_vmcnt<7>(); break;
    case 8: bwait_vmcnt<8>(); break;
    case 9: bwait_vmcnt<9>(); break;
    case 10: bwait_vmcnt<10>(); break;
    case 11: bwait_vmcnt<11>(); break;
    case 12: bwait_vmcnt<12>(); break;
    case 13: bwait_vmcnt<13>(); break;
    case 14: bwait_vmcnt<14>(); break;
    case 15: bwait_vmcnt<15>(); break;
    case 16: bwait_vmcnt<16>(); break;
    case 17: bwait_vmcnt<17>(); break;
    case 18: bwait_vmcnt<18>(); break;
    case 19: bwait_vmcnt<19>(); break;
    case 20: bwait_vmcnt<20>(); break;
    case 21: bwait_vmcnt<21>(); break;
    case 22: bwait_vmcnt<22>(); break;
    case 23: bwait_vmcnt<23>(); break;
    default: bwait_vmcnt<24>(); break;
  }
}
__device__ __forceinline__ void braw_barrier() {
  asm volatile("" ::: "memory");
  __builtin_amdgcn_s_barrier();
  asm volatile("" ::: "memory");
}
// global_load_lds_dwordx4, scalar-base form: lane l copies 16 bytes from
// sbase + voff into LDS at lds + 16 l. Inline asm, so the compiler does not
// track it; every wait on these copies is an explicit vmcnt wait.
__device__ __forceinline__ void bdma16(const char* sbase, uint32_t voff, const uint4* lds) {
  const uint32_t l = (uint32_t)__builtin_amdgcn_readfirstlane((int)(uint32_t)(uintptr_t)lds);
  const uint64_t b = (uint64_t)(uintptr_t)sbase;
  const uint64_t bs = ((uint64_t)(uint32_t)__builtin_amdgcn_readfirstlane((int)(b >> 32)) << 32) |
                      (uint32_t)__builtin_amdgcn_readfirstlane((int)(uint32_t)b);
  asm volatile("s_mov_b32 m0, %2\n\ts_nop 0\n\tglobal_load_lds_dwordx4 %0, %1"
               :: "v"(voff), "s"(bs), "s"(l) : "memory");
}

// k-contiguous tile: chunk offset of (row, chunk), 128-byte rows.
__device__ __forceinline__ int kc_off(int row, int chunk) { return row * 8 + (chunk ^ ((row >> 1) & 7)); }
// i-contiguous [64 k][128 i] sub-tile: element offset of (k, i), i % 4 == 0.
__device__ __forceinline__ int km_off(int k, int i) {
  return k * 128 + ((((i >> 5) ^ (k & 3)) << 5) | (i & 31));
}

typedef short s16x4_t __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) s16x4_t lds_s16x4_t;

// MFMA operand (rows base + lane % 32, k 16 kk + 8 (lane / 32) + [0, 8)) from
// an i-contiguous sub-tile. ds_read_b64_tr_b16 works on groups of 16 lanes:
// lane s of a group names 4 consecutive i of one k row, and lane j of the
// group receives, for t = 0..3, element j % 4 of the group's lane j / 4 + 4 t.
// With lane s reading row k0 + s / 4 at i0 + 4 (s % 4), lane j gets
// (i0 + j, k0 + t): four consecutive k of one operand row.
__device__ __forceinline__ bf16x8_t km_frag(const uint4* sub, int base, int kk, int lane) {
  const uint16_t* tile = reinterpret_cast<const uint16_t*>(sub);
  const int g = lane >> 4, s = lane & 15;
  const int i = base + 16 * (g & 1) + 4 * (s & 3);
  const int k = 16 * kk + 8 * (g >> 1) + (s >> 2);
  const s16x4_t lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4_t*)(tile + km_off(k, i)));
  const s16x4_t hi =
      __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_s16x4_t*)(tile + km_off(k + 4, i)));
  return __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7);
}

// Zero the operand elements whose k (16 kk + 8 h + t within the stage) is at
// or past krem, a dword (two elements) at a time.
__device__ __forceinline__ bf16x8_t mask_k(bf16x8_t v, int kk, int h, int krem) {
  const int nv = krem - (16 * kk + 8 * h);  // valid elements among the lane's 8
  uint4 u = *reinterpret_cast<uint4*>(&v);
  auto keep = [&](int j) {  // dword j holds elements 2 j (low half) and 2 j + 1
    return nv >= 2 * j + 2 ? 0xffffffffu : (nv == 2 * j + 1 ? 0x0000ffffu : 0u);
  };
  u.x &= keep(0);
  u.y &= keep(1);
  u.z &= keep(2);
  u.w &= keep(3);
  return *reinterpret_cast<bf16x8_t*>(&u);
}

// Store one wave's (32 NI) x 64 output sub-tile (the transposed-MFMA layout:
// lane holds row 32 i + lane % 32, columns 32 f + 8 q + 4 (lane / 32) +
// [0, 4)) through LDS, so each global store instruction writes whole rows:
// 128 bytes per row (bf16, 8 rows per instruction) or 256 bytes (fp32, 4
// rows). st: this wave's 4 NI KB (bf16) or 8 NI KB (fp32) of LDS; rows of 8 or 16
// chunks, chunk c of row r at c ^ ((r >> 1) & 7) (bf16) or c ^ (r & 15)
// (fp32), conflict-free for the writes and the row-major reads. obase:
// element (0, 0) of the sub-tile in the output, ld its row stride; rows at or
// past rvalid and columns at or past cvalid are not written.
template <bool F32, int NI = 2>
__device__ __forceinline__ void store_subtile(const f32x16_t (&acc)[NI][2], uint4* st, int lane,
                                              char* obase, long long ld, int rvalid, int cvalid) {
  constexpr int RC = F32 ? 16 : 8;  // 16-byte chunks per sub-tile row
  constexpr int ESZ = F32 ? 4 : 2;
  const int h = lane >> 5, lr = lane & 31;
#pragma unroll
  for (int i = 0; i < NI; ++i)
#pragma unroll
    for (int f = 0; f < 2; ++f)
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const int r = 32 * i + lr;
        const f32x16_t& a = acc[i][f];
        if (F32) {
          const int c = 8 * f + 2 * q + h;
          st[r * RC + (c ^ (r & 15))] = make_uint4(__float_as_uint(a[4 * q]), __float_as_uint(a[4 * q + 1]),
                                                   __float_as_uint(a[4 * q + 2]), __float_as_uint(a[4 * q + 3]));
        } else {
          const int c = 4 * f + q;
          *reinterpret_cast<uint2*>(reinterpret_cast<char*>(st + r * RC + (c ^ ((r >> 1) & 7))) + 8 * h) =
              make_uint2(pack_bf16x2(a[4 * q], a[4 * q + 1]), pack_bf16x2(a[4 * q + 2], a[4 * q + 3]));
        }
      }
  constexpr int RPI = 64 / RC;  // rows per read instruction
#pragma unroll
  for (int j = 0; j < 32 * NI / RPI; ++j) {
    const int r = RPI * j + lane / RC, c = lane % RC;
    const uint4 v = st[r * RC + (F32 ? (c ^ (r & 15)) : (c ^ ((r >> 1) & 7)))];
    const int col = c * (16 / ESZ);
    if (r < rvalid && col < cvalid)
      *reinterpret_cast<uint4*>(obase + ((long long)r * ld + col) * ESZ) = v;
  }
}

}  // namespace

// The router's weight gradient dW_r = dz^T x (fp32 output): the wgrad form
// with one group (counts[0] = K rows, M and N fixed), both operands read
// i-contiguous from slot-row matrices. Few tiles and a long k: a ring of
// NSLOT stages per tile, all slots filled at the start; per stage, wait for
// this wave's copies of the stage, a raw barrier, queue the next stage into
// the slot just freed, multiply. OP (a BwdOp) only names the launch, so
// profiles tell the GEMMs apart.
template <int WM, int WN, int FM, int FN, int NSLOT, int OP>
__global__ __launch_bounds__(64 * WM * WN) void bwd_wgrad_f32_kernel(BwdGemmArgs g) {
  constexpr int NW = WM * WN;
  constexpr int BM = 32 * FM * WM, BN = 32 * FN * WN;  // wave tile (32 FM) x (32 FN)
  static_assert(FM % 2 == 0 && FN % 2 == 0, "stores go by 64 x 64 sub-tiles");
  constexpr int A_CH = BM * 8, B_CH = BN * 8;  // 16-byte chunks per stage
  constexpr int SLOT = A_CH + B_CH;
  constexpr int NB = SLOT / 64;                // 1 KB copy blocks per stage
  constexpr int CPW = NB / NW;                 // copies per wave per stage
  constexpr int JA = (A_CH / 64) / NW;         // the first JA of them fill A
  static_assert(NB % NW == 0 && (A_CH / 64) % NW == 0, "copy blocks must split evenly");
  static_assert(NW * 1024 <= NSLOT * SLOT, "epilogue staging fits in the ring");
  static_assert((NSLOT - 1) * (NB / NW) <= 24, "vmcnt range of the waits");
  static_assert(BM % 128 == 0 && BN % 128 == 0, "i-contiguous tiles are 128 wide");
  __shared__ uint4 lds[NSLOT * SLOT];

  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int wm = wave / WN, wn = wave % WN;

  // ---- work item -> (expert, m tile, n tile), per-XCD contiguous runs ----
  const int ntn = (g.N + BN - 1) / BN, mtn = (g.M + BM - 1) / BM;
  const int total = g.n_ffn * mtn * ntn;
  const int per_xcd = (total + 7) >> 3;
  const int pos = blockIdx.x >> 3;
  if (pos >= per_xcd) return;
  const int L = (int)(blockIdx.x & 7) * per_xcd + pos;
  if (L >= total) return;
  const int e = L / (mtn * ntn);
  const int local = L - e * mtn * ntn;
  const int mt = local / ntn, nt = local - mt * ntn;
  const int off_e = g.offsets[e];
  const int M = g.M, N = g.N, K = g.counts[e];
  const int m0 = mt * BM, n0 = nt * BN;
  const char* abase = reinterpret_cast<const char*>(g.a) + (size_t)off_e * g.a_ld * 2;
  const char* bbase = reinterpret_cast<const char*>(g.b) + (size_t)off_e * g.b_ld * 2;
  const int nst = (K + BK - 1) / BK;

  // ---- per-lane copy descriptors (stage independent) ----
  // Copy j of this wave fills 1 KB block b = wave + NW j of the stage (A
  // blocks first, then B): sub-tile b / 16, k rows 4 (b % 16) + lane / 16,
  // swizzled 64-byte window of the lane.
  uint32_t voff[CPW];
  int krow[CPW];
#pragma unroll
  for (int j = 0; j < CPW; ++j) {
    const bool isA = j < JA;
    const int b = isA ? wave + NW * j : wave + NW * j - A_CH / 64;
    const int q = b >> 4, bb = b & 15;
    const int k = 4 * bb + (lane >> 4), pc = lane & 15;
    const int c = ((((pc >> 2) ^ (k & 3))) << 2) | (pc & 3);
    const int ext = isA ? M : N;
    int col = (isA ? m0 : n0) + 128 * q + 8 * c;
    if (col > ext - 8) col = ext - 8;
    krow[j] = k;
    voff[j] = (uint32_t)(col * 2);
  }

  // With b_wrap > 0, B row k is row k mod b_wrap (the router's dW_r: the
  // three dz planes stacked along k all multiply x, read in place).
  const int bwrap = g.b_wrap;
  auto issue = [&](int s) {
    const int k0 = s * BK;
    const int kmax = K - 1 - k0;  // rows past K re-load row K - 1
    uint4* slot = lds + (s % NSLOT) * SLOT;
#pragma unroll
    for (int j = 0; j < CPW; ++j) {
      const bool isA = j < JA;
      const long long ld = isA ? g.a_ld : g.b_ld;
      const int k = krow[j] < kmax ? krow[j] : kmax;
      if (!isA && bwrap > 0) {
        const int kr = (k0 + k) % bwrap;
        bdma16(bbase, voff[j] + (uint32_t)kr * (uint32_t)(ld * 2), slot + 64 * (wave + NW * j));
      } else {
        bdma16((isA ? abase : bbase) + (size_t)k0 * ld * 2, voff[j] + (uint32_t)(k * ld * 2),
               slot + 64 * (wave + NW * j));
      }
    }
  };

  f32x16_t acc[FM][FN];
#pragma unroll
  for (int i = 0; i < FM; ++i)
#pragma unroll
    for (int f = 0; f < FN; ++f)
#pragma unroll
      for (int v = 0; v < 16; ++v) acc[i][f][v] = 0.f;

  bwait_vmcnt<0>();  // every load before the copies has landed

  auto compute = [&](int s) {
    const uint4* A = lds + (s % NSLOT) * SLOT;
    const uint4* B = A + A_CH;
    const int krem = K - s * BK;  // valid k in this stage
    const int nkk = min(4, (krem + 15) >> 4);
    const int h = lane >> 5;
#pragma unroll
    for (int kk = 0; kk < 4; ++kk) {
      if (kk >= nkk) break;
      bf16x8_t av[FM], bv[FN];
#pragma unroll
      for (int i = 0; i < FM; ++i) {
        const int r = 32 * FM * wm + 32 * i;
        av[i] = km_frag(A + (r >> 7) * 1024, r & 127, kk, lane);
      }
#pragma unroll
      for (int f = 0; f < FN; ++f) {
        const int r = 32 * FN * wn + 32 * f;
        bv[f] = km_frag(B + (r >> 7) * 1024, r & 127, kk, lane);
      }
      // k rows past K hold copies of row K - 1: zeroing them in one operand
      // removes their products.
      if (16 * kk + 16 > krem) {
#pragma unroll
        for (int f = 0; f < FN; ++f) bv[f] = mask_k(bv[f], kk, h, krem);
      }
#pragma unroll
      for (int i = 0; i < FM; ++i)
#pragma unroll
        for (int f = 0; f < FN; ++f)
          acc[i][f] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(bv[f], av[i], acc[i][f], 0, 0, 0);
    }
  };

  // Every slot is free at the start, so NSLOT stages go out at once; from
  // stage 1 on, the next stage goes into the slot stage s - 1 has released.
  const int per_stage = CPW;
  int issued = min(NSLOT, nst);
  for (int s = 0; s < issued; ++s) issue(s);
  for (int s = 0; s < nst; ++s) {
    bwait_vmcnt_upto(per_stage * (issued - 1 - s));
    braw_barrier();
    if (s >= 1 && issued < nst) issue(issued++);
    compute(s);
  }

  // ---- epilogue through LDS (the ring is free once every wave is done) ----
  braw_barrier();
  const int rlim = min(M, g.m_store);
#pragma unroll
  for (int i2 = 0; i2 < FM / 2; ++i2)
#pragma unroll
    for (int f2 = 0; f2 < FN / 2; ++f2) {
      const int r0 = m0 + 32 * FM * wm + 64 * i2, c0 = n0 + 32 * FN * wn + 64 * f2;
      char* obase = static_cast<char*>(g.c) + (((long long)e * M + r0) * g.c_ld + c0) * 4;
      const f32x16_t sub[2][2] = {{acc[2 * i2][2 * f2], acc[2 * i2][2 * f2 + 1]},
                                  {acc[2 * i2 + 1][2 * f2], acc[2 * i2 + 1][2 * f2 + 1]}};
      store_subtile<true>(sub, lds + wave * 1024, lane, obase, g.c_ld, rlim - r0, N - c0);
    }
}

// Data gradients (W2^T dy, dU W13, the router's dz W_r): C[m][n] = sum_k
// A(m, k) B_e(n, k) with A slot rows read k-contiguous and the weights read
// i-contiguous. An M tile holds up to kBwdTileM (256) slot rows, so at a
// prefill batch (about 128 rows per expert, rarely past 170) every expert's
// rows share one tile and each weight tile is multiplied once. 2 x 4 waves
// over a 256 x 256 tile: wave (wm, wn) holds the 32-row fragments 2 j + wm
// (j < 4) and 64 columns; only the fragments that hold rows are multiplied
// (the k loop is instantiated per active count, straight-line code). A stage
// is the tile's rows in whole 32-row fragments (rows past the count re-load
// the last row) and two [64 k][128 i] weight sub-tiles; the ring holds as
// many stages as fit in 160 KB of LDS, up to 3 (3 for up to 160 rows).
template <bool OUT_F32, int OP>
__global__ __launch_bounds__(512) void bwd_dgrad_kernel(BwdGemmArgs g) {
  constexpr int NW = 8, WN = 4, FM = 4, FN = 2;
  constexpr int BM = kBwdTileM, BN = kBwdTileNDgrad;
  static_assert(BM == 32 * FM * 2 && BN == 32 * FN * WN, "256 x 256 tiles");
  constexpr int B_CH = BN * 8;     // weight sub-tiles per stage (16-byte chunks)
  constexpr int LDS_CH = 10240;    // 160 KB
  constexpr int MAX_SLOTS = 3;
  constexpr int ACPW = BM / 8 / NW;  // A copy groups per wave, at most (4)
  constexpr int BCPW = B_CH / 64 / NW;  // weight copies per wave (4)
  static_assert(NW * (OUT_F32 ? 512 : 256) <= LDS_CH, "epilogue staging fits");
  __shared__ uint4 lds[LDS_CH];

  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int wm = wave / WN, wn = wave % WN;
  const int h = lane >> 5, lr = lane & 31;

  // ---- work item -> (expert, n tile, m tile), per-XCD contiguous runs ----
  const int ntn = (g.N + BN - 1) / BN;
  const int total = g.tile_prefix[g.n_ffn] * ntn;
  const int per_xcd = (total + 7) >> 3;
  const int pos = blockIdx.x >> 3;
  if (pos >= per_xcd) return;
  const int L = (int)(blockIdx.x & 7) * per_xcd + pos;
  if (L >= total) return;
  int lo = 0, hi = g.n_ffn - 1;
  while (lo < hi) {
    const int mid = (lo + hi + 1) >> 1;
    if (g.tile_prefix[mid] * ntn <= L) lo = mid; else hi = mid - 1;
  }
  const int e = lo;
  const int mtiles = g.tile_prefix[e + 1] - g.tile_prefix[e];
  const int local = L - g.tile_prefix[e] * ntn;
  const int nt = local / mtiles, mt = local - nt * mtiles;
  const int off_e = g.offsets[e];
  const int m0 = mt * BM, n0 = nt * BN;
  const int rows = min(BM, g.counts[e] - m0);  // >= 1: tiles cover counts exactly
  const int N = g.N, K = g.K;
  const int nfr = (rows + 31) >> 5;            // 32-row fragments holding rows
  const int a_ch = nfr * 256;                  // A chunks per stage (8 rows per 64)
  const int slot = a_ch + B_CH;
  const int nslots = min(MAX_SLOTS, LDS_CH / slot);
  const int nst = (K + BK - 1) / BK;
  const bool half_tail = (K % BK) != 0;        // K is a multiple of 32

  const char* abase = reinterpret_cast<const char*>(g.a) + (size_t)off_e * g.a_ld * 2;
  const char* bbase = reinterpret_cast<const char*>(g.b) + (size_t)e * g.b_estride * 2;

  // ---- per-lane copy descriptors ----
  // A group j of this wave: 8 rows 8 (wave + NW j) + lane / 8 of the tile,
  // chunk lane % 8 of the swizzled row (holding logical chunk c). Weight copy
  // j: 1 KB block b = wave + NW j of the stage, sub-tile b / 16, k row
  // 4 (b % 16) + lane / 16, swizzled 64-byte window of the lane.
  uint32_t aoff[ACPW];
  const int a_groups = nfr * 4;
  int acnt = 0, kcc = 0;  // kcc: the logical chunk (the same for all groups: NW is even)
#pragma unroll
  for (int j = 0; j < ACPW; ++j) {
    const int row = 8 * (wave + NW * j) + (lane >> 3);
    const int c = (lane & 7) ^ ((row >> 1) & 7);
    const int rr = m0 + min(row, rows - 1);
    aoff[j] = (uint32_t)((size_t)rr * g.a_ld * 2 + 16 * c);
    acnt += (wave + NW * j < a_groups) ? 1 : 0;
    kcc = c;
  }
  uint32_t boff[BCPW];
  int krow[BCPW];
#pragma unroll
  for (int j = 0; j < BCPW; ++j) {
    const int b = wave + NW * j;
    const int q = b >> 4, bb = b & 15;
    const int k = 4 * bb + (lane >> 4), pc = lane & 15;
    const int c = ((((pc >> 2) ^ (k & 3))) << 2) | (pc & 3);
    int col = n0 + 128 * q + 8 * c;
    if (col > N - 8) col = N - 8;
    krow[j] = k;
    boff[j] = (uint32_t)(col * 2);
  }
  const int per_stage = acnt + BCPW;

  auto issue = [&](int s, int si) {
    const int k0 = s * BK;
    const int kmax = K - 1 - k0;  // weight rows past K re-load row K - 1
    // tail stage of an odd multiple of 32: chunks 4..7 of the A rows do not
    // exist; those lanes load chunk c - 4 (64 bytes back), which no MFMA reads.
    const uint32_t back = (half_tail && s == nst - 1 && kcc >= 4) ? 64u : 0u;
    uint4* dst = lds + si * slot;
#pragma unroll
    for (int j = 0; j < ACPW; ++j)
      if (wave + NW * j < a_groups) bdma16(abase + 2 * (size_t)k0, aoff[j] - back, dst + 64 * (wave + NW * j));
#pragma unroll
    for (int j = 0; j < BCPW; ++j) {
      const int k = krow[j] < kmax ? krow[j] : kmax;
      bdma16(bbase + (size_t)k0 * g.b_ld * 2, boff[j] + (uint32_t)(k * g.b_ld * 2),
             dst + a_ch + 64 * (wave + NW * j));
    }
  };

  const int nact = __builtin_amdgcn_readfirstlane(max(0, min(FM, (nfr - wm + 1) >> 1)));
  bwait_vmcnt<0>();  // the loads of the setup have landed

  auto run = [&](auto NA_c) {
    constexpr int NA = decltype(NA_c)::value;
    f32x16_t acc[NA > 0 ? NA : 1][FN];
#pragma unroll
    for (int i = 0; i < NA; ++i)
#pragma unroll
      for (int f = 0; f < FN; ++f)
#pragma unroll
        for (int v = 0; v < 16; ++v) acc[i][f][v] = 0.f;
    int issued = min(nslots, nst);
    for (int s = 0; s < issued; ++s) issue(s, s);
    int si = 0;  // slot of stage s
    for (int s = 0; s < nst; ++s) {
      bwait_vmcnt_upto(per_stage * (issued - 1 - s));
      braw_barrier();
      if (s >= 1 && issued < nst) {  // into the slot stage s - 1 released
        issue(issued, si == 0 ? nslots - 1 : si - 1);
        ++issued;
      }
      const uint4* A = lds + si * slot;
      const uint4* B = A + a_ch;
      const int nkk = (half_tail && s == nst - 1) ? 2 : 4;
#pragma unroll
      for (int kk = 0; kk < 4; ++kk) {
        if (kk >= nkk) break;
        bf16x8_t av[NA > 0 ? NA : 1], bv[FN];
#pragma unroll
        for (int f = 0; f < FN; ++f) {
          const int r = 32 * FN * wn + 32 * f;
          bv[f] = km_frag(B + (r >> 7) * 1024, r & 127, kk, lane);
        }
#pragma unroll
        for (int i = 0; i < NA; ++i) av[i] = as_bf16x8(A[kc_off(32 * (2 * i + wm) + lr, 2 * kk + h)]);
#pragma unroll
        for (int i = 0; i < NA; ++i)
#pragma unroll
          for (int f = 0; f < FN; ++f)
            acc[i][f] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(bv[f], av[i], acc[i][f], 0, 0, 0);
      }
      si = si + 1 == nslots ? 0 : si + 1;
    }
    // ---- epilogue through LDS (the ring is free once every wave is done) ----
    braw_barrier();
    uint4* st = lds + wave * (OUT_F32 ? 512 : 256);
#pragma unroll
    for (int i = 0; i < NA; ++i) {
      const int r0 = 32 * (2 * i + wm), c0 = n0 + 64 * wn;
      char* obase = static_cast<char*>(g.c) +
                    (((long long)off_e + m0 + r0) * g.c_ld + c0) * (OUT_F32 ? 4 : 2);
      const f32x16_t sub[1][2] = {{acc[i][0], acc[i][1]}};
      store_subtile<OUT_F32, 1>(sub, st, lane, obase, g.c_ld, rows - r0, N - c0);
    }
  };
  switch (nact) {
    case 4: run(std::integral_constant<int, 4>{}); break;
    case 3: run(std::integral_constant<int, 3>{}); break;
    case 2: run(std::integral_constant<int, 2>{}); break;
    case 1: run(std::integral_constant<int, 1>{}); break;
    default: run(std::integral_constant<int, 0>{}); break;
  }
}

// Weight-gradient GEMMs (bf16 outputs dW2, dW13), persistent: one block per
// CU walks a run of its XCD's tiles (positions pos, pos + P, ... of the XCD's
// contiguous run, so the tiles running at once on an XCD stay adjacent), and
// the k stages of its consecutive tiles form one stream through the
// two-slot ring. At a prefill batch K (an expert's slot count) is about 128,
// two stages: a tile of its own would wait for its first loads, multiply
// for two stages and store; in the stream, the next tile's first stage
// loads while the current tile finishes and stores. A tile's epilogue
// stages through the slot its last stage has just released. Every wait
// drains all of this wave's outstanding memory operations (copies and the
// previous epilogue's stores alike). Tiles of experts without slots (zero
// gradient) are written with plain stores, outside the stream.
template <int WM, int WN, int FM, int FN, int OP>
__global__ __launch_bounds__(64 * WM * WN) void bwd_wgrad_stream_kernel(BwdGemmArgs g) {
  constexpr int NW = WM * WN, NT = 64 * NW;
  constexpr int BM = 32 * FM * WM, BN = 32 * FN * WN;
  constexpr int A_CH = BM * 8, B_CH = BN * 8;  // 16-byte chunks per stage
  constexpr int SLOT = A_CH + B_CH;
  constexpr int NB = SLOT / 64;                // 1 KB copy blocks per stage
  constexpr int CPW = NB / NW;                 // copies per wave per stage
  constexpr int JA = (A_CH / 64) / NW;         // the first JA of them fill A
  static_assert(FM % 2 == 0 && FN % 2 == 0, "stores go by 64 x 64 sub-tiles");
  static_assert(NB % NW == 0 && (A_CH / 64) % NW == 0, "copy blocks must split evenly");
  static_assert(NW * 512 <= SLOT, "the epilogue stages through one slot");
  static_assert(BM % 128 == 0 && BN % 128 == 0, "i-contiguous tiles are 128 wide");
  constexpr int MAX_N = 2048;  // FFN experts (the shape check caps E at 2048)
  __shared__ uint4 lds[2 * SLOT];
  // Every expert's slot count and first slot, read once: a tile's setup
  // then costs LDS reads instead of two dependent global loads.
  __shared__ int s_cnt[MAX_N], s_off[MAX_N];

  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int wm = wave / WN, wn = wave % WN;
  const int h = lane >> 5, lr = lane & 31;

  const int ntn = (g.N + BN - 1) / BN, mtn = (g.M + BM - 1) / BM;
  const int total = g.n_ffn * mtn * ntn;
  const int per_xcd = (total + 7) >> 3;
  const int xcd = blockIdx.x & 7, pstep = gridDim.x >> 3;
  const int rlim = min(g.M, g.m_store);  // output rows stored

  struct Tile {
    bool valid;
    int e, m0, n0, K, nst;
    const char* abase;
    const char* bbase;
  };
  // Walk of the block's tiles (positions pos, pos + pstep, ... of its XCD's
  // run) as a cursor (e, m tile, n tile): a step adds the stride's fixed
  // decomposition with carries, so no division runs per tile.
  struct Cursor {
    int pos, e, mt, nt;
  };
  const int dn = pstep % ntn, dm = (pstep / ntn) % mtn, de = pstep / (ntn * mtn);
  auto cursor_at = [&](int pos) {
    const int L = xcd * per_xcd + pos;
    const int e = L / (mtn * ntn), local = L - e * mtn * ntn;
    return Cursor{pos, e, local / ntn, local % ntn};
  };
  auto step = [&](Cursor c) {
    c.pos += pstep;
    c.nt += dn;
    int carry = c.nt >= ntn;
    c.nt -= carry ? ntn : 0;
    c.mt += dm + carry;
    carry = c.mt >= mtn;
    c.mt -= carry ? mtn : 0;
    c.e += de + carry;
    return c;
  };
  auto tile_at = [&](const Cursor& c) {
    Tile t{};
    t.valid = c.pos < per_xcd && xcd * per_xcd + c.pos < total;
    if (!t.valid) return t;
    t.e = c.e;
    t.m0 = c.mt * BM;
    t.n0 = c.nt * BN;
    t.K = s_cnt[t.e];
    t.nst = (t.K + BK - 1) / BK;
    const int off_e = s_off[t.e];
    t.abase = reinterpret_cast<const char*>(g.a) + (size_t)off_e * g.a_ld * 2;
    t.bbase = reinterpret_cast<const char*>(g.b) + (size_t)off_e * g.b_ld * 2;
    return t;
  };
  // A tile of an expert without slots: zeros, written directly.
  auto store_zero_tile = [&](const Tile& t) {
    for (int id = tid; id < BM * (BN / 8); id += NT) {
      const int r = t.m0 + id / (BN / 8), c = t.n0 + 8 * (id % (BN / 8));
      if (r < rlim && c < g.N)
        *reinterpret_cast<uint4*>(static_cast<char*>(g.c) +
                                  (((long long)t.e * g.M + r) * g.c_ld + c) * 2) =
            make_uint4(0u, 0u, 0u, 0u);
    }
  };
  // The first tile at or after c with slots (zero-filling the tiles before
  // it when asked), or an invalid one.
  auto next_with_slots = [&](Cursor c, bool zero_fill) {
    for (;; c = step(c)) {
      const Tile t = tile_at(c);
      if (!t.valid || t.nst > 0) return c;
      if (zero_fill) store_zero_tile(t);
    }
  };

  // Per-lane copy descriptors (tile independent): copy j of this wave fills
  // 1 KB block wave + NW j of the stage (A blocks first, then B); both
  // operands are i-contiguous [64 k][128 i] sub-tiles: sub-tile b / 16, k
  // rows 4 (b % 16) + lane / 16, swizzled 64-byte window of the lane.
  int ccol[CPW], krow[CPW];
#pragma unroll
  for (int j = 0; j < CPW; ++j) {
    const int b = j < JA ? wave + NW * j : wave + NW * j - A_CH / 64;
    const int q = b >> 4, bb = b & 15;
    const int k = 4 * bb + (lane >> 4), pc = lane & 15;
    const int c = ((((pc >> 2) ^ (k & 3))) << 2) | (pc & 3);
    ccol[j] = 128 * q + 8 * c;
    krow[j] = k;
  }
  auto issue = [&](const Tile& t, int s, int slot) {
    const int k0 = s * BK;
    const int kmax = t.K - 1 - k0;  // rows past K re-load row K - 1
    uint4* dst = lds + slot * SLOT;
#pragma unroll
    for (int j = 0; j < CPW; ++j) {
      const bool isA = j < JA;
      const long long ld = isA ? g.a_ld : g.b_ld;
      const int ext = isA ? g.M : g.N;
      int col = (isA ? t.m0 : t.n0) + ccol[j];
      if (col > ext - 8) col = ext - 8;
      const int k = krow[j] < kmax ? krow[j] : kmax;
      bdma16((isA ? t.abase : t.bbase) + (size_t)k0 * ld * 2,
             (uint32_t)(col * 2) + (uint32_t)(k * ld * 2), dst + 64 * (wave + NW * j));
    }
  };

  f32x16_t acc[FM][FN];
  auto compute = [&](const Tile& t, int s, int slot) {
    const uint4* A = lds + slot * SLOT;
    const uint4* B = A + A_CH;
    const int krem = t.K - s * BK;  // valid k in this stage
    const int nkk = min(4, (krem + 15) >> 4);
#pragma unroll
    for (int kk = 0; kk < 4; ++kk) {
      if (kk >= nkk) break;
      bf16x8_t av[FM], bv[FN];
#pragma unroll
      for (int i = 0; i < FM; ++i) {
        const int r = 32 * FM * wm + 32 * i;
        av[i] = km_frag(A + (r >> 7) * 1024, r & 127, kk, lane);
      }
#pragma unroll
      for (int f = 0; f < FN; ++f) {
        const int r = 32 * FN * wn + 32 * f;
        bv[f] = km_frag(B + (r >> 7) * 1024, r & 127, kk, lane);
      }
      // k rows past K hold copies of row K - 1: zeroing them in one operand
      // removes their products.
      if (16 * kk + 16 > krem) {
#pragma unroll
        for (int f = 0; f < FN; ++f) bv[f] = mask_k(bv[f], kk, h, krem);
      }
#pragma unroll
      for (int i = 0; i < FM; ++i)
#pragma unroll
        for (int f = 0; f < FN; ++f)
          acc[i][f] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(bv[f], av[i], acc[i][f], 0, 0, 0);
    }
  };

  for (int j = tid; j < g.n_ffn; j += NT) {
    s_cnt[j] = g.counts[j];
    s_off[j] = g.offsets[j];
  }
  __syncthreads();
  Cursor cur_c = next_with_slots(cursor_at((int)(blockIdx.x >> 3)), true);
  Tile cur = tile_at(cur_c);
  if (!cur.valid) return;  // block-uniform
  // The stream: stage number n of the block goes into slot n & 1; `la` is
  // the next stage to issue (tile la_t at cursor la_c, stage la_s).
  Cursor la_c = cur_c;
  int la_s = 0;
  Tile la_t = cur;
  int issued = 0;
  auto issue_next = [&]() {
    if (!la_t.valid) return;
    issue(la_t, la_s, issued & 1);
    ++issued;
    if (++la_s >= la_t.nst) {
      la_c = next_with_slots(step(la_c), true);
      la_t = tile_at(la_c);
      la_s = 0;
    }
  };
  bwait_vmcnt<0>();  // the loads of the tile setup have landed
  issue_next();      // stage 0
  int n = 0;         // stream stage being multiplied
  for (;;) {
#pragma unroll
    for (int i = 0; i < FM; ++i)
#pragma unroll
      for (int f = 0; f < FN; ++f)
#pragma unroll
        for (int v = 0; v < 16; ++v) acc[i][f][v] = 0.f;
    for (int s = 0; s < cur.nst; ++s, ++n) {
      // Stage n has landed (and anything older, a previous epilogue's stores
      // included); the barrier publishes it and frees slot (n + 1) & 1, which
      // held stage n - 1 or the previous tile's epilogue staging.
      bwait_vmcnt<0>();
      braw_barrier();
      issue_next();  // stage n + 1
      compute(cur, s, n & 1);
    }
    // Epilogue through the slot of the stage just multiplied (stage n - 1)
    // once every wave is done with it; stage n may be loading into the other.
    braw_barrier();
    uint4* st = lds + ((n - 1) & 1) * SLOT + wave * 512;
#pragma unroll
    for (int i2 = 0; i2 < FM / 2; ++i2)
#pragma unroll
      for (int f2 = 0; f2 < FN / 2; ++f2) {
        const int r0 = cur.m0 + 32 * FM * wm + 64 * i2, c0 = cur.n0 + 32 * FN * wn + 64 * f2;
        char* obase = static_cast<char*>(g.c) + (((long long)cur.e * g.M + r0) * g.c_ld + c0) * 2;
        const f32x16_t sub[2][2] = {{acc[2 * i2][2 * f2], acc[2 * i2][2 * f2 + 1]},
                                    {acc[2 * i2 + 1][2 * f2], acc[2 * i2 + 1][2 * f2 + 1]}};
        store_subtile<false>(sub, st, lane, obase, g.c_ld, rlim - r0, g.N - c0);
      }
    cur_c = next_with_slots(step(cur_c), false);
    cur = tile_at(cur_c);
    if (!cur.valid) break;  // block-uniform; nothing is left in flight but stores
  }
}

// One wave per FFN slot row s < S (S read on the device): the token's x and
// dy rows copied into slot order.
__global__ __launch_bounds__(256) void gather_rows_kernel(const uint16_t* __restrict__ x,
                                                          const uint16_t* __restrict__ dy,
                                                          const int* __restrict__ perm,
                                                          const int* __restrict__ s_dev, int topk,
                                                          int d, uint16_t* __restrict__ xs,
                                                          uint16_t* __restrict__ dys) {
  const int lane = threadIdx.x & 63;
  const int S = *s_dev;
  const int wpb = blockDim.x >> 6;
  for (int s = blockIdx.x * wpb + (threadIdx.x >> 6); s < S; s += gridDim.x * wpb) {
    const size_t t = (size_t)(perm[s] / topk);
    const uint4* xr = reinterpret_cast<const uint4*>(x + t * d);
    const uint4* gr = reinterpret_cast<const uint4*>(dy + t * d);
    uint4* xo = reinterpret_cast<uint4*>(xs + (size_t)s * d);
    uint4* go = reinterpret_cast<uint4*>(dys + (size_t)s * d);
    for (int c = lane; c < (d >> 3); c += 64) {
      xo[c] = xr[c];
      go[c] = gr[c];
    }
  }
}

// Grid of the dgrad launch: an upper bound of the work items (every expert's
// M tiles of kBwdTileM rows, over all slots) rounded for the per-XCD layout.
int bwd_dgrad_grid(long long smax, int n_ffn, int n_cols) {
  const long long items = (smax / kBwdTileM + n_ffn) * ((n_cols + kBwdTileNDgrad - 1) / kBwdTileNDgrad);
  return (int)std::min<long long>(items + 8, 1ll << 30);
}
int bwd_device_cus() {
  static int cus = 0;
  if (cus == 0) {
    int dev = 0, n = 0;
    if (hipGetDevice(&dev) != hipSuccess ||
        hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || n <= 0)
      n = 256;
    cus = n;
  }
  return cus;
}
// Grid of the persistent weight-gradient launch: one block per CU (its LDS
// ring takes most of a CU's 160 KB), or max_blocks when given, a multiple of
// 8 for the per-XCD layout, and no more blocks than tiles allow.
int bwd_wgrad_grid(int n_ffn, int M, int N, int max_blocks) {
  const int cus = bwd_device_cus();
  const long long items = (long long)n_ffn * ((M + kWgradBM - 1) / kWgradBM) *
                          ((N + kWgradBN - 1) / kWgradBN);
  long long blocks = std::min<long long>((cus + 7) / 8 * 8, (items + 7) / 8 * 8);
  if (max_blocks > 0) blocks = std::min<long long>(blocks, max_blocks / 8 * 8);
  return (int)std::max<long long>(8, blocks);
}

void launch_bwd_dgrad(const BwdGemmArgs& g, BwdOp op, int grid, hipStream_t s) {
  switch (op) {
    case kBwdQ: bwd_dgrad_kernel<true, kBwdQ><<<grid, 512, 0, s>>>(g); break;
    case kBwdDx: bwd_dgrad_kernel<true, kBwdDx><<<grid, 512, 0, s>>>(g); break;
    default: bwd_dgrad_kernel<true, kBwdRouterDx><<<grid, 512, 0, s>>>(g); break;
  }
}
void launch_bwd_wgrad(const BwdGemmArgs& g, BwdOp op, int grid, hipStream_t s) {
  if (op == kBwdDw2)
    bwd_wgrad_stream_kernel<kWgWM, kWgWN, kWgFM, kWgFN, kBwdDw2><<<grid, 64 * kWgWM * kWgWN, 0, s>>>(g);
  else
    bwd_wgrad_stream_kernel<kWgWM, kWgWN, kWgFM, kWgFN, kBwdDw13><<<grid, 64 * kWgWM * kWgWN, 0, s>>>(g);
}
void launch_bwd_wgrad_f32(const BwdGemmArgs& g, hipStream_t s) {
  const long long items = (long long)g.n_ffn * ((g.M + 127) / 128) * ((g.N + 127) / 128);
  // Two slots (64 KB of LDS) so two blocks share a CU: the router's 288
  // tiles at E = 768, d = 6144 then run in one round on 256 CUs.
  bwd_wgrad_f32_kernel<2, 2, 2, 2, 2, kBwdRouterDw>
      <<<(int)std::min<long long>(items + 8, 1ll << 30), 256, 0, s>>>(g);
}
void launch_gather_rows(const uint16_t* x, const uint16_t* dy, const int* perm, const int* s_dev,
                        int topk, int d, uint16_t* xs, uint16_t* dys, int grid, hipStream_t s) {
  gather_rows_kernel<<<grid, 256, 0, s>>>(x, dy, perm, s_dev, topk, d, xs, dys);
}

}  // namespace lcmoe
