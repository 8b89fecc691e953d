// fp16 MFMA GEMM kernel template for gfx950 with fused epilogues.
//
//   C[m, n] = sum_k A[m, k] * B[n, k]
//
// A is the activation matrix [M, K] (row-major, K contiguous); B is a packed weight in
// the nn.Linear layout [Npad, K] (K contiguous, rows zero-padded to a multiple of 256).
// Both operands are therefore K-contiguous, which is what the MFMA operand layout wants:
// each lane feeds 8 consecutive k of one row.
//
// Structure:
//   - block tile BM x BN, k-tile 64; waves tile the block as (BM/WM) x (BN/WN); each wave
//     owns a WM x WN sub-tile made of 32x32 accumulators (v_mfma_f32_32x32x16_f16, fp32
//     accumulation);
//   - two LDS stages, one barrier per k-tile: the loads of tile k+1 are in flight while
//     tile k is multiplied. Loads go either global -> VGPR -> LDS, or straight from
//     global memory into LDS (global_load_lds_dwordx4: each lane of a load instruction
//     deposits its 16 bytes at LDS slot base + lane, so the permutation that builds the
//     swizzled layout is applied to the global addresses instead);
//   - LDS rows are 128 bytes (64 halfs); 16-byte chunks are XOR-swizzled by (row % 8) so
//     the 16-byte fragment reads of 8 consecutive rows hit distinct banks;
//   - block ids are remapped so that the tiles of one XCD (block id % 8 on MI355X's
//     round-robin dispatch) form a contiguous, grouped region of the output: blocks
//     sharing A rows / B rows then share that XCD's L2.
//
// Rows of A beyond M are read from row M-1 (never out of bounds) and not stored.
#pragma once
#include "tf_internal.h"

namespace tfp {
namespace gemm {

constexpr int BK = 64;
constexpr int GROUP_M = 4;

typedef __attribute__((address_space(3))) void* lds_ptr;

__device__ __forceinline__ f32x16 mfma32(f16x8 a, f16x8 b, f32x16 c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_f16(a, b, c, 0, 0, 0);
}

// halfs offset of 16-byte chunk `chunk` of tile row `row` in the swizzled LDS layout
__device__ __forceinline__ int swz(int row, int chunk) {
  return row * BK + ((chunk ^ (row & 7)) << 3);
}

__device__ __forceinline__ void wait_vmcnt0() { __builtin_amdgcn_s_waitcnt(0x0F70); }

__device__ __forceinline__ float silu_f(float g) { return g / (1.0f + __expf(-g)); }

__device__ __forceinline__ float gelu_tanh_f(float v) {
  // 0.5 v (1 + tanh(sqrt(2/pi) (v + 0.044715 v^3))), tanh(y) = 1 - 2 / (e^{2y} + 1)
  const float y = 0.7978845608028654f * (v + 0.044715f * v * v * v);
  const float t = 1.0f - 2.0f / (__expf(2.0f * y) + 1.0f);
  return 0.5f * v * (1.0f + t);
}

template <int BM_, int BN_, int WM_, int WN_, bool DMA_>
struct Cfg {
  static constexpr int BM = BM_, BN = BN_, WM = WM_, WN = WN_;
  static constexpr bool DMA = DMA_;
  static constexpr int NWM = BM / WM, NWN = BN / WN, NW = NWM * NWN;
  static constexpr int NT = NW * 64;
  static constexpr int TM = WM / 32, TN = WN / 32;
  static constexpr int CA = BM * 8 / NT;  // 16-byte chunks of A per thread per k-tile
  static constexpr int CB = BN * 8 / NT;
  static constexpr int STAGE = (BM + BN) * BK;  // halfs per LDS stage
  // LDS: two k-tile stages, reused after the main loop to stage the output tile
  // (BM x (BN + 8) fp16, or BM/2 x (BN + 4) fp32)
  static constexpr int STAGE_OUT = BM * (BN + 8) > BM / 2 * (BN + 4) * 2 ? BM * (BN + 8) : BM / 2 * (BN + 4) * 2;
  static constexpr int SMEM_HALFS = 2 * STAGE > STAGE_OUT ? 2 * STAGE : STAGE_OUT;
  static_assert(BM * 8 % NT == 0 && BN * 8 % NT == 0, "load split");
  static_assert(WN % 64 == 0, "epilogues need 64-column aligned wave tiles");
};

template <class C, int EPI>
__global__ void __launch_bounds__(C::NT)
gemm_kernel(const GemmArgs g) {
  constexpr int BM = C::BM, BN = C::BN, WM = C::WM, WN = C::WN;
  __shared__ __attribute__((aligned(16))) f16 smem[C::SMEM_HALFS];

  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);  // wave-uniform (SGPR)
  const int nbm = (g.M + BM - 1) / BM, nbn = g.Npad / BN;
  const int ntiles = nbm * nbn;

  // XCD-aware remap: block id b runs on XCD b % 8; give each XCD a contiguous range.
  int tile;
  {
    const int q = ntiles >> 3, r = ntiles & 7, x = blockIdx.x & 7, loc = blockIdx.x >> 3;
    tile = (x < r) ? x * (q + 1) + loc : r * (q + 1) + (x - r) * q + loc;
  }
  // Grouped order inside the range: GROUP_M tile-rows sweep the tile-columns together.
  const int per_group = GROUP_M * nbn;
  const int first_m = (tile / per_group) * GROUP_M;
  const int gm = min(nbm - first_m, GROUP_M);
  const int tm = first_m + (tile % per_group) % gm;
  const int tn = (tile % per_group) / gm;
  const int m0 = tm * BM, n0 = tn * BN;

  const int wm = wave / C::NWN, wn = wave % C::NWN;

  // Load assignment. VGPR path: chunk q = tid + i*NT is row q/8, chunk q%8 (LDS offset
  // swizzled). DMA path: instruction i of wave w fills LDS slots (w*CA + i)*64 + lane;
  // slot s holds row s/8, chunk (s%8) ^ (row%8).
  int goa[C::CA], loa[C::CA], gob[C::CB], lob[C::CB];
#pragma unroll
  for (int i = 0; i < C::CA; ++i) {
    int row, ch;
    if constexpr (C::DMA) {
      const int s = (wave * C::CA + i) * 64 + lane;
      row = s >> 3;
      ch = (s & 7) ^ (row & 7);
      loa[i] = (wave * C::CA + i) * 512;
    } else {
      const int q = tid + i * C::NT;
      row = q >> 3;
      ch = q & 7;
      loa[i] = swz(row, ch);
    }
    goa[i] = min(m0 + row, g.M - 1) * g.lda + ch * 8;
  }
#pragma unroll
  for (int i = 0; i < C::CB; ++i) {
    int row, ch;
    if constexpr (C::DMA) {
      const int s = (wave * C::CB + i) * 64 + lane;
      row = s >> 3;
      ch = (s & 7) ^ (row & 7);
      lob[i] = BM * BK + (wave * C::CB + i) * 512;
    } else {
      const int q = tid + i * C::NT;
      row = q >> 3;
      ch = q & 7;
      lob[i] = BM * BK + swz(row, ch);
    }
    gob[i] = (n0 + row) * g.ldb + ch * 8;
  }

  f32x16 acc[C::TM][C::TN];
#pragma unroll
  for (int i = 0; i < C::TM; ++i)
#pragma unroll
    for (int j = 0; j < C::TN; ++j)
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[i][j][r] = 0.0f;

  const int KT = g.K / BK;
  const int frow = lane & 31, fch = lane >> 5;

  auto compute = [&](const f16* s) {
#pragma unroll
    for (int kk = 0; kk < BK / 16; ++kk) {
      f16x8 af[C::TM], bf[C::TN];
#pragma unroll
      for (int i = 0; i < C::TM; ++i)
        af[i] = *reinterpret_cast<const f16x8*>(s + swz(wm * WM + i * 32 + frow, kk * 2 + fch));
#pragma unroll
      for (int j = 0; j < C::TN; ++j)
        bf[j] = *reinterpret_cast<const f16x8*>(
            s + BM * BK + swz(wn * WN + j * 32 + frow, kk * 2 + fch));
#pragma unroll
      for (int i = 0; i < C::TM; ++i)
#pragma unroll
        for (int j = 0; j < C::TN; ++j) acc[i][j] = mfma32(af[i], bf[j], acc[i][j]);
    }
  };

  if constexpr (C::DMA) {
    auto issue = [&](int kt, int stage) {
      const int ko = kt * BK;
      f16* d = smem + stage * C::STAGE;
#pragma unroll
      for (int i = 0; i < C::CA; ++i)
        __builtin_amdgcn_global_load_lds((const void*)(g.A + goa[i] + ko), (lds_ptr)(d + loa[i]), 16, 0, 0);
#pragma unroll
      for (int i = 0; i < C::CB; ++i)
        __builtin_amdgcn_global_load_lds((const void*)(g.B + gob[i] + ko), (lds_ptr)(d + lob[i]), 16, 0, 0);
    };
    issue(0, 0);
    wait_vmcnt0();
    __syncthreads();
    for (int kt = 0; kt < KT; ++kt) {
      if (kt + 1 < KT) issue(kt + 1, (kt + 1) & 1);
      compute(smem + (kt & 1) * C::STAGE);
      wait_vmcnt0();
      __syncthreads();
    }
  } else {
    f16x8 ra[C::CA], rb[C::CB];
#pragma unroll
    for (int i = 0; i < C::CA; ++i) ra[i] = *reinterpret_cast<const f16x8*>(g.A + goa[i]);
#pragma unroll
    for (int i = 0; i < C::CB; ++i) rb[i] = *reinterpret_cast<const f16x8*>(g.B + gob[i]);
#pragma unroll
    for (int i = 0; i < C::CA; ++i) *reinterpret_cast<f16x8*>(smem + loa[i]) = ra[i];
#pragma unroll
    for (int i = 0; i < C::CB; ++i) *reinterpret_cast<f16x8*>(smem + lob[i]) = rb[i];
    __syncthreads();
    for (int kt = 0; kt < KT; ++kt) {
      if (kt + 1 < KT) {
        const int ko = (kt + 1) * BK;
#pragma unroll
        for (int i = 0; i < C::CA; ++i) ra[i] = *reinterpret_cast<const f16x8*>(g.A + goa[i] + ko);
#pragma unroll
        for (int i = 0; i < C::CB; ++i) rb[i] = *reinterpret_cast<const f16x8*>(g.B + gob[i] + ko);
      }
      compute(smem + (kt & 1) * C::STAGE);
      if (kt + 1 < KT) {
        f16* d = smem + ((kt + 1) & 1) * C::STAGE;
#pragma unroll
        for (int i = 0; i < C::CA; ++i) *reinterpret_cast<f16x8*>(d + loa[i]) = ra[i];
#pragma unroll
        for (int i = 0; i < C::CB; ++i) *reinterpret_cast<f16x8*>(d + lob[i]) = rb[i];
      }
      __syncthreads();
    }
  }

  // ------------------------------------------------------------------ epilogue
  // Accumulator (i, j) register r of this lane holds tile element
  //   row wm*WM + 32i + 8(r/4) + 4(lane/32) + r%4,  column wn*WN + 32j + lane%32.
  // Values are finished in registers (bias, activation, rotary), staged in LDS in the
  // output type, then written out as 16-byte row segments (fp32 outputs: two passes of
  // half the tile rows each, so the staging fits in LDS).
  constexpr bool F32OUT = (EPI == EPI_STORE_F32 || EPI == EPI_RESID_ADD);
  constexpr int OCOLS = EPI == EPI_SWIGLU ? BN / 2 : BN;         // output columns per tile
  constexpr int PASSES = F32OUT ? 2 : 1;
  constexpr int PR = BM / PASSES;                                 // tile rows per pass
  constexpr int ESZ = F32OUT ? 4 : 2;
  constexpr int PITCH = OCOLS + 16 / ESZ;                          // staging row pitch (elements)
  static_assert(PR * PITCH * ESZ <= (int)sizeof(smem), "staging must fit in LDS");
  static_assert(PASSES == 1 || (WM == PR && C::NWM == 2), "fp32 passes split the tile by wave rows");
  const int ocol0 = EPI == EPI_SWIGLU ? n0 / 2 : n0;               // first output column
  const int ncols = min(OCOLS, g.N - ocol0);                       // valid output columns
  const int hi4 = 4 * (lane >> 5), l32 = lane & 31;

  // Per-lane column facts (bias, rotary partner) for EPI_QKV_ROPE.
  [[maybe_unused]] float bj[C::TN];
  [[maybe_unused]] int ej[C::TN];
  [[maybe_unused]] bool rj[C::TN];
  if constexpr (EPI != EPI_SWIGLU) {
#pragma unroll
    for (int j = 0; j < C::TN; ++j) {
      const int n = n0 + wn * WN + 32 * j + l32;
      bj[j] = (g.bias && n < g.N) ? g.bias[n] : 0.0f;
      if constexpr (EPI == EPI_QKV_ROPE) {
        ej[j] = n % g.head_dim;
        rj[j] = n < 2 * g.hd && ej[j] < 2 * g.rot_half;
      }
    }
  }

#pragma unroll
  for (int pass = 0; pass < PASSES; ++pass) {
    if (pass > 0) __syncthreads();  // previous pass fully copied out
    if (PASSES == 1 || wm == pass) {
      f16* st16 = smem;
      float* st32 = reinterpret_cast<float*>(smem);
#pragma unroll
      for (int i = 0; i < C::TM; ++i) {
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const int trow = (PASSES == 1 ? wm * WM : 0) + 32 * i + 8 * (r >> 2) + hi4 + (r & 3);
          if constexpr (EPI == EPI_SWIGLU) {
#pragma unroll
            for (int j = 0; j < C::TN; j += 2) {
              const int oc = (wn * WN + 32 * j) / 2 + l32;
              st16[trow * PITCH + oc] = (f16)(silu_f(acc[i][j][r]) * acc[i][j + 1][r]);
            }
          } else if constexpr (EPI == EPI_QKV_ROPE) {
            const int m = m0 + wm * WM + 32 * i + 8 * (r >> 2) + hi4 + (r & 3);
            const int p = m % g.seq;
            const int half = g.rot_half;
#pragma unroll
            for (int j = 0; j < C::TN; ++j) {
              float v = acc[i][j][r] + bj[j];
              if (half > 0) {
                // partner column e +/- half: a neighbouring lane (half <= 16) or the
                // neighbouring 32-column block (half == 32)
                const float pv = half <= 16 ? __shfl_xor(v, half) : acc[i][j ^ 1][r] + bj[j ^ 1];
                if (rj[j] && m < g.M) {
                  const int e = ej[j];
                  const int fi = e < half ? e : e - half;
                  const float cs = g.rope_cos[p * half + fi];
                  const float sn = g.rope_sin[p * half + fi];
                  v = e < half ? v * cs - pv * sn : v * cs + pv * sn;
                }
              }
              st16[trow * PITCH + wn * WN + 32 * j + l32] = (f16)v;
            }
          } else {
#pragma unroll
            for (int j = 0; j < C::TN; ++j) {
              const float v = acc[i][j][r] + bj[j];
              const int oc = wn * WN + 32 * j + l32;
              if constexpr (F32OUT) st32[trow * PITCH + oc] = v;
              else if constexpr (EPI == EPI_GELU) st16[trow * PITCH + oc] = (f16)gelu_tanh_f(v);
              else st16[trow * PITCH + oc] = (f16)v;
            }
          }
        }
      }
    }
    __syncthreads();
    // Copy-out: 16-byte vectors along rows; scalar tail where a vector would cross N or
    // the output rows are not 16-byte aligned.
    constexpr int VE = 16 / ESZ;            // elements per vector
    constexpr int VPR = OCOLS / VE;         // vectors per tile row
    const int rbase = m0 + pass * PR;
    const bool vec_ok = ((g.ldo * ESZ) & 15) == 0 &&
        ((reinterpret_cast<uintptr_t>(F32OUT ? (void*)g.out32 : (void*)g.out16)) & 15) == 0;
    for (int v = tid; v < PR * VPR; v += C::NT) {
      const int tr = v / VPR, vc = (v % VPR) * VE;
      const int m = rbase + tr;
      if (m >= g.M || vc >= ncols) continue;
      const size_t o = (size_t)m * g.ldo + ocol0 + vc;
      if (vec_ok && vc + VE <= ncols) {
        if constexpr (F32OUT) {
          f32x4 x = *reinterpret_cast<const f32x4*>(reinterpret_cast<float*>(smem) + tr * PITCH + vc);
          if constexpr (EPI == EPI_RESID_ADD) x += *reinterpret_cast<const f32x4*>(g.out32 + o);
          *reinterpret_cast<f32x4*>(g.out32 + o) = x;
        } else {
          *reinterpret_cast<f16x8*>(g.out16 + o) = *reinterpret_cast<const f16x8*>(smem + tr * PITCH + vc);
        }
      } else {
        const int ne = min(VE, ncols - vc);
        for (int e = 0; e < ne; ++e) {
          if constexpr (F32OUT) {
            const float x = reinterpret_cast<float*>(smem)[tr * PITCH + vc + e];
            if constexpr (EPI == EPI_RESID_ADD) g.out32[o + e] += x;
            else g.out32[o + e] = x;
          } else {
            g.out16[o + e] = smem[tr * PITCH + vc + e];
          }
        }
      }
    }
  }
}

template <class C>
hipError_t launch(const GemmArgs& a, hipStream_t st) {
  const int nbm = (a.M + C::BM - 1) / C::BM, nbn = a.Npad / C::BN;
  const dim3 grid(nbm * nbn), block(C::NT);
  switch (a.epi) {
    case EPI_STORE_F32: hipLaunchKernelGGL((gemm_kernel<C, EPI_STORE_F32>), grid, block, 0, st, a); break;
    case EPI_STORE_F16: hipLaunchKernelGGL((gemm_kernel<C, EPI_STORE_F16>), grid, block, 0, st, a); break;
    case EPI_RESID_ADD: hipLaunchKernelGGL((gemm_kernel<C, EPI_RESID_ADD>), grid, block, 0, st, a); break;
    case EPI_SWIGLU: hipLaunchKernelGGL((gemm_kernel<C, EPI_SWIGLU>), grid, block, 0, st, a); break;
    case EPI_GELU: hipLaunchKernelGGL((gemm_kernel<C, EPI_GELU>), grid, block, 0, st, a); break;
    case EPI_QKV_ROPE: hipLaunchKernelGGL((gemm_kernel<C, EPI_QKV_ROPE>), grid, block, 0, st, a); break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

}  // namespace gemm
}  // namespace tfp
