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

constexpr int GROUP_M = 4;

typedef __attribute__((address_space(3))) void* lds_ptr;

__device__ __forceinline__ f32x16 mfma32(f16x8 a, f16x8 b, f32x16 c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_f16(a, b, c, 0, 0, 0);
}

// s_waitcnt vmcnt(N) (gfx9 encoding: vmcnt bits [3:0] and [15:14]; expcnt, lgkmcnt left
// at their maxima so they are not waited for).
template <int N>
__device__ __forceinline__ void wait_vmcnt() {
  static_assert(N >= 0 && N < 64, "vmcnt range");
  __builtin_amdgcn_s_waitcnt((N & 15) | ((N >> 4) << 14) | (7 << 4) | (15 << 8));
}

__device__ __forceinline__ float silu_f(float g) { return g / (1.0f + __expf(-g)); }

__device__ __forceinline__ float gelu_tanh_f(float v) {
  // 0.5 v (1 + tanh(sqrt(2/pi) (v + 0.044715 v^3))), tanh(y) = 1 - 2 / (e^{2y} + 1)
  const float y = 0.7978845608028654f * (v + 0.044715f * v * v * v);
  const float t = 1.0f - 2.0f / (__expf(2.0f * y) + 1.0f);
  return 0.5f * v * (1.0f + t);
}

// BM x BN block tile, WM x WN wave tile, BK k-tile, NS LDS stages.
template <int BM_, int BN_, int WM_, int WN_, int BK_, int NS_>
struct Cfg {
  static constexpr int BM = BM_, BN = BN_, WM = WM_, WN = WN_, BK = BK_, NS = NS_;
  static constexpr int NWM = BM / WM, NWN = BN / WN, NW = NWM * NWN;
  static constexpr int NT = NW * 64;
  static constexpr int TM = WM / 32, TN = WN / 32;
  static constexpr int CPR = BK / 8;    // 16-byte chunks per tile row
  static constexpr int RPL = 128 / BK;  // tile rows per 256-byte line (64 banks x 4 bytes)
  // global_load_lds instructions per wave per k-tile (each fills 64 16-byte slots)
  static constexpr int LA = BM * CPR / 64 / NW, LB = BN * CPR / 64 / NW, LPT = LA + LB;
  static constexpr int STAGE = (BM + BN) * BK;  // halfs per LDS stage
  // LDS: NS k-tile stages, reused after the main loop to stage the output tile
  // (BM x (BN + 8) fp16, or BM/2 x (BN + 4) fp32)
  static constexpr int STAGE_OUT = BM * (BN + 8) > BM / 2 * (BN + 4) * 2 ? BM * (BN + 8) : BM / 2 * (BN + 4) * 2;
  static constexpr int SMEM_HALFS = NS * STAGE > STAGE_OUT ? NS * STAGE : STAGE_OUT;
  static_assert(LA * 64 * NW == BM * CPR && LB * 64 * NW == BN * CPR, "load split");
  static_assert(BK == 32 || BK == 64, "k-tile");
  static_assert(NS >= 2 && (NS - 2) * LPT < 64, "stages");
  static_assert(WN % 64 == 0, "epilogues need 64-column aligned wave tiles");
  // halfs offset of 16-byte chunk `chunk` of tile row `row`: chunks are XOR-swizzled by
  // the index of the row's 256-byte line, so the 16-byte reads of 16 consecutive rows at
  // one logical chunk (one 16-lane group of a ds_read_b128) cover all 64 banks once
  static __device__ __forceinline__ int swz(int row, int chunk) {
    return row * BK + ((chunk ^ ((row / RPL) % CPR)) << 3);
  }
};

template <class C, int EPI>
__global__ void __launch_bounds__(C::NT)
gemm_kernel(const GemmArgs g) {
  constexpr int BM = C::BM, BN = C::BN, WM = C::WM, WN = C::WN, BK = C::BK, NS = C::NS;
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

  // Load assignment: global_load_lds instruction i of wave w deposits lane l's 16 bytes
  // at LDS slot (w*L + i)*64 + l; slot s of the A (B) region holds tile row s / CPR,
  // logical chunk (s % CPR) ^ ((row / RPL) % CPR) -- i.e. exactly C::swz's layout.
  int goa[C::LA], loa[C::LA], gob[C::LB], lob[C::LB];
#pragma unroll
  for (int i = 0; i < C::LA; ++i) {
    const int s = (wave * C::LA + i) * 64 + lane;
    const int row = s / C::CPR, ch = (s % C::CPR) ^ ((row / C::RPL) % C::CPR);
    goa[i] = min(m0 + row, g.M - 1) * g.lda + ch * 8;
    loa[i] = (wave * C::LA + i) * 512;
  }
#pragma unroll
  for (int i = 0; i < C::LB; ++i) {
    const int s = (wave * C::LB + i) * 64 + lane;
    const int row = s / C::CPR, ch = (s % C::CPR) ^ ((row / C::RPL) % C::CPR);
    gob[i] = (n0 + row) * g.ldb + ch * 8;
    lob[i] = BM * BK + (wave * C::LB + i) * 512;
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

  // Fragments of k-step kk (16 k) from LDS stage s.
  auto frags = [&](const f16* s, int kk, f16x8 (&af)[C::TM], f16x8 (&bf)[C::TN]) {
#pragma unroll
    for (int i = 0; i < C::TM; ++i)
      af[i] = *reinterpret_cast<const f16x8*>(s + C::swz(wm * WM + i * 32 + frow, kk * 2 + fch));
#pragma unroll
    for (int j = 0; j < C::TN; ++j)
      bf[j] = *reinterpret_cast<const f16x8*>(
          s + BM * BK + C::swz(wn * WN + j * 32 + frow, kk * 2 + fch));
  };
  auto issue = [&](int kt, int stage) {
    const int ko = kt * BK;
    f16* d = smem + stage * C::STAGE;
#pragma unroll
    for (int i = 0; i < C::LA; ++i)
      __builtin_amdgcn_global_load_lds((const void*)(g.A + goa[i] + ko), (lds_ptr)(d + loa[i]), 16, 0, 0);
#pragma unroll
    for (int i = 0; i < C::LB; ++i)
      __builtin_amdgcn_global_load_lds((const void*)(g.B + gob[i] + ko), (lds_ptr)(d + lob[i]), 16, 0, 0);
  };

  // Pipeline. All NS stages start filled (tiles 0..NS-1 in flight). In k-tile kt, the
  // fragments of k-step kk+1 are read while the MFMAs of k-step kk run (registers double
  // buffered); before the last k-step's MFMAs the wave waits for tile kt+1, joins the
  // barrier (which also frees tile kt's stage: every wave has read its fragments), reads
  // tile kt+1's first fragments and refills the freed stage with tile kt+NS -- so the
  // barrier and the LDS latency of the next tile hide behind the last k-step's MFMAs.
  // The refill is unconditional (past the end it reloads the last tile into a stage that
  // is never read again), which keeps the loop body free of branches: a branch join would
  // make the compiler wait for the next tile's fragment reads before the last MFMAs.
  constexpr int KS = BK / 16;  // k-steps per k-tile
  constexpr int NR = C::TM + C::TN, NM = C::TM * C::TN;
  auto mfmas = [&](const f16x8 (&a)[C::TM], const f16x8 (&b)[C::TN]) {
#pragma unroll
    for (int i = 0; i < C::TM; ++i)
#pragma unroll
      for (int j = 0; j < C::TN; ++j) acc[i][j] = mfma32(a[i], b[j], acc[i][j]);
  };
  auto hint = [&]() {
#pragma unroll
    for (int x = 0; x < NR; ++x) {
      __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);  // one MFMA
      __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);  // one LDS read
    }
    __builtin_amdgcn_sched_group_barrier(0x008, NM - NR, 0);
  };
#pragma unroll
  for (int st = 0; st < NS; ++st) issue(min(st, KT - 1), st);
  wait_vmcnt<(NS - 1) * C::LPT>();
  __syncthreads();
  f16x8 af[2][C::TM], bf[2][C::TN];
  frags(smem, 0, af[0], bf[0]);
  for (int kt = 0; kt < KT - 1; ++kt) {
    const f16* s = smem + (kt % NS) * C::STAGE;
#pragma unroll
    for (int kk = 0; kk < KS; ++kk) {
      const int cur = kk & 1;
      if (kk + 1 < KS) {
        frags(s, kk + 1, af[cur ^ 1], bf[cur ^ 1]);
      } else {
        wait_vmcnt<(NS - 2) * C::LPT>();  // tile kt+1 landed (kt+2 .. kt+NS-1 may fly)
        __syncthreads();
        frags(smem + ((kt + 1) % NS) * C::STAGE, 0, af[cur ^ 1], bf[cur ^ 1]);
        issue(min(kt + NS, KT - 1), kt % NS);
      }
      mfmas(af[cur], bf[cur]);
      hint();
    }
  }
  {  // last k-tile
    const f16* s = smem + ((KT - 1) % NS) * C::STAGE;
#pragma unroll
    for (int kk = 0; kk < KS; ++kk) {
      const int cur = kk & 1;
      if (kk + 1 < KS) frags(s, kk + 1, af[cur ^ 1], bf[cur ^ 1]);
      mfmas(af[cur], bf[cur]);
      if (kk + 1 < KS) hint();
    }
  }
  wait_vmcnt<0>();  // the refills past the end must land before the stages are reused
  __syncthreads();  // every wave is done with the stages before they are reused below

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

  // RoPE factors for this lane's rows: the 16 accumulator rows of block i come in 4
  // groups of 4 consecutive rows; the transposed table gives a group's 4 positions in one
  // 16-byte load when they do not straddle a batch row. Loaded per block i, just before use.
  [[maybe_unused]] bool rope_on = false;
  [[maybe_unused]] const int half = g.rot_half;
  [[maybe_unused]] const float* rct = nullptr;
  [[maybe_unused]] const float* rst = nullptr;
  if constexpr (EPI == EPI_QKV_ROPE) {
    // every tile column lies in one section: Q and K tiles rotate, V tiles do not
    rope_on = half > 0 && n0 < 2 * g.hd;
    int fi = 0;
#pragma unroll
    for (int j = 0; j < C::TN; ++j)
      if (rj[j]) fi = ej[j] < half ? ej[j] : ej[j] - half;
    rct = g.rope_cos + (size_t)fi * g.rope_ld;
    rst = g.rope_sin + (size_t)fi * g.rope_ld;
  }
  auto rope_rows = [&](int i, f32x4 (&rcs)[4], f32x4 (&rsn)[4]) {
    const bool vec4 = (g.seq & 3) == 0;
#pragma unroll
    for (int g4 = 0; g4 < 4; ++g4) {
      // rows past M are never stored; clamp them onto in-bounds rows (with seq % 4 == 0
      // onto the last aligned group, so the 16-byte load stays inside one table row)
      const int mraw = m0 + wm * WM + 32 * i + 8 * g4 + hi4;
      const int mb = vec4 ? min(mraw, g.M - 4) : min(mraw, g.M - 1);
      const int p = mb % g.seq;
      if (vec4) {
        rcs[g4] = *reinterpret_cast<const f32x4*>(rct + p);
        rsn[g4] = *reinterpret_cast<const f32x4*>(rst + p);
      } else {
#pragma unroll
        for (int t = 0; t < 4; ++t) {
          const int pt = min(mb + t, g.M - 1) % g.seq;
          rcs[g4][t] = rct[pt];
          rsn[g4][t] = rst[pt];
        }
      }
    }
  };

#pragma unroll
  for (int pass = 0; pass < PASSES; ++pass) {
    if (pass > 0) __syncthreads();  // previous pass fully copied out
    if (PASSES == 1 || wm == pass) {
      f16* st16 = smem;
      float* st32 = reinterpret_cast<float*>(smem);
#pragma unroll
      for (int i = 0; i < C::TM; ++i) {
        [[maybe_unused]] f32x4 rcs[4], rsn[4];
        if constexpr (EPI == EPI_QKV_ROPE) {
          if (rope_on) rope_rows(i, rcs, rsn);
        }
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
#pragma unroll
            for (int j = 0; j < C::TN; ++j) {
              float v = acc[i][j][r] + bj[j];
              if (rope_on) {
                // partner column e +/- half: a neighbouring lane (half <= 16; half == 8 is
                // a DPP rotate by 8 within each 16-lane row) or the neighbouring 32-column
                // block (half == 32)
                float pv;
                if (half == 8)
                  pv = __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(v), 0x128, 0xF, 0xF, false));
                else if (half <= 16)
                  pv = __shfl_xor(v, half);
                else
                  pv = acc[i][j ^ 1][r] + bj[j ^ 1];
                if (rj[j]) {
                  const float cs = rcs[r >> 2][r & 3], sn = rsn[r >> 2][r & 3];
                  v = ej[j] < half ? v * cs - pv * sn : v * cs + pv * sn;
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
