// fp16 MFMA GEMM for gfx950 with fused epilogues.
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
//   - global -> VGPR -> LDS staging, two LDS stages, one barrier per k-tile: the global
//     loads of tile k+1 are in flight while tile k is multiplied;
//   - LDS rows are 128 bytes (64 halfs); 16-byte chunks are XOR-swizzled by (row % 8) so
//     the 16-byte fragment reads of 8 consecutive rows hit distinct banks;
//   - block ids are remapped so that the tiles of one XCD (block id % 8 on MI355X's
//     round-robin dispatch) form a contiguous, grouped region of the output: blocks
//     sharing A rows / B rows then share that XCD's L2.
//
// Rows of A beyond M are read from row M-1 (never out of bounds) and not stored.
#include "tf_internal.h"

namespace tfp {

namespace {

constexpr int BK = 64;
constexpr int GROUP_M = 4;

__device__ __forceinline__ f32x16 mfma32(f16x8 a, f16x8 b, f32x16 c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_f16(a, b, c, 0, 0, 0);
}

__device__ __forceinline__ int swz(int row, int chunk) {
  return row * BK + ((chunk ^ (row & 7)) << 3);
}

__device__ __forceinline__ float silu_f(float g) { return g / (1.0f + __expf(-g)); }

__device__ __forceinline__ float gelu_tanh_f(float v) {
  // 0.5 v (1 + tanh(sqrt(2/pi) (v + 0.044715 v^3))), tanh(y) = 1 - 2 / (e^{2y} + 1)
  const float y = 0.7978845608028654f * (v + 0.044715f * v * v * v);
  const float t = 1.0f - 2.0f / (__expf(2.0f * y) + 1.0f);
  return 0.5f * v * (1.0f + t);
}

template <int BM, int BN, int WM, int WN>
struct Cfg {
  static constexpr int NWM = BM / WM, NWN = BN / WN;
  static constexpr int NT = NWM * NWN * 64;
  static constexpr int TM = WM / 32, TN = WN / 32;
  static constexpr int CA = BM * 8 / NT;
  static constexpr int CB = BN * 8 / NT;
  static constexpr int STAGE = (BM + BN) * BK;  // halfs per LDS stage
  static_assert(BM * 8 % NT == 0 && BN * 8 % NT == 0, "load split");
  static_assert(WN % 64 == 0, "epilogues need 64-column aligned wave tiles");
};

template <int BM, int BN, int WM, int WN, int EPI>
__global__ void __launch_bounds__((BM / WM) * (BN / WN) * 64)
gemm_kernel(const GemmArgs g) {
  using C = Cfg<BM, BN, WM, WN>;
  __shared__ __attribute__((aligned(16))) f16 smem[2 * C::STAGE];

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
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

  // Global load assignment: chunk q = tid + i*NT covers row q/8, 16-byte chunk q%8.
  int goa[C::CA], loa[C::CA], gob[C::CB], lob[C::CB];
#pragma unroll
  for (int i = 0; i < C::CA; ++i) {
    const int q = tid + i * C::NT, row = q >> 3, ch = q & 7;
    const int gr = min(m0 + row, g.M - 1);
    goa[i] = gr * g.lda + ch * 8;
    loa[i] = swz(row, ch);
  }
#pragma unroll
  for (int i = 0; i < C::CB; ++i) {
    const int q = tid + i * C::NT, row = q >> 3, ch = q & 7;
    gob[i] = (n0 + row) * g.ldb + ch * 8;
    lob[i] = BM * BK + swz(row, ch);
  }

  f32x16 acc[C::TM][C::TN];
#pragma unroll
  for (int i = 0; i < C::TM; ++i)
#pragma unroll
    for (int j = 0; j < C::TN; ++j)
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[i][j][r] = 0.0f;

  f16x8 ra[C::CA], rb[C::CB];
  const int KT = g.K / BK;

#pragma unroll
  for (int i = 0; i < C::CA; ++i) ra[i] = *reinterpret_cast<const f16x8*>(g.A + goa[i]);
#pragma unroll
  for (int i = 0; i < C::CB; ++i) rb[i] = *reinterpret_cast<const f16x8*>(g.B + gob[i]);
#pragma unroll
  for (int i = 0; i < C::CA; ++i) *reinterpret_cast<f16x8*>(smem + loa[i]) = ra[i];
#pragma unroll
  for (int i = 0; i < C::CB; ++i) *reinterpret_cast<f16x8*>(smem + lob[i]) = rb[i];
  __syncthreads();

  const int frow = lane & 31, fch = lane >> 5;
  for (int kt = 0; kt < KT; ++kt) {
    const f16* s = smem + (kt & 1) * C::STAGE;
    if (kt + 1 < KT) {
      const int ko = (kt + 1) * BK;
#pragma unroll
      for (int i = 0; i < C::CA; ++i)
        ra[i] = *reinterpret_cast<const f16x8*>(g.A + goa[i] + ko);
#pragma unroll
      for (int i = 0; i < C::CB; ++i)
        rb[i] = *reinterpret_cast<const f16x8*>(g.B + gob[i] + ko);
    }
#pragma unroll
    for (int kk = 0; kk < BK / 16; ++kk) {
      f16x8 af[C::TM], bf[C::TN];
#pragma unroll
      for (int i = 0; i < C::TM; ++i)
        af[i] = *reinterpret_cast<const f16x8*>(
            s + swz(wm * WM + i * 32 + frow, kk * 2 + fch));
#pragma unroll
      for (int j = 0; j < C::TN; ++j)
        bf[j] = *reinterpret_cast<const f16x8*>(
            s + BM * BK + swz(wn * WN + j * 32 + frow, kk * 2 + fch));
#pragma unroll
      for (int i = 0; i < C::TM; ++i)
#pragma unroll
        for (int j = 0; j < C::TN; ++j) acc[i][j] = mfma32(af[i], bf[j], acc[i][j]);
    }
    if (kt + 1 < KT) {
      f16* d = smem + ((kt + 1) & 1) * C::STAGE;
#pragma unroll
      for (int i = 0; i < C::CA; ++i) *reinterpret_cast<f16x8*>(d + loa[i]) = ra[i];
#pragma unroll
      for (int i = 0; i < C::CB; ++i) *reinterpret_cast<f16x8*>(d + lob[i]) = rb[i];
    }
    __syncthreads();
  }

  // ------------------------------------------------------------------ epilogue
  // Accumulator (i, j) register r of this lane holds
  //   row m = m0 + wm*WM + 32i + 8(r/4) + 4(lane/32) + r%4,  col n = n0 + wn*WN + 32j + lane%32.
  const int mrow0 = m0 + wm * WM + 4 * (lane >> 5);
  const int ncol0 = n0 + wn * WN + (lane & 31);

  if constexpr (EPI == EPI_STORE_F32 || EPI == EPI_STORE_F16 || EPI == EPI_RESID_ADD ||
                EPI == EPI_GELU) {
#pragma unroll
    for (int j = 0; j < C::TN; ++j) {
      const int n = ncol0 + 32 * j;
      if (n >= g.N) continue;
      const float bv = g.bias ? g.bias[n] : 0.0f;
#pragma unroll
      for (int i = 0; i < C::TM; ++i) {
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const int m = mrow0 + 32 * i + 8 * (r >> 2) + (r & 3);
          if (m >= g.M) continue;
          const float v = acc[i][j][r] + bv;
          const size_t o = (size_t)m * g.ldo + n;
          if constexpr (EPI == EPI_STORE_F32) g.out32[o] = v;
          else if constexpr (EPI == EPI_STORE_F16) g.out16[o] = (f16)v;
          else if constexpr (EPI == EPI_RESID_ADD) g.out32[o] += v;
          else g.out16[o] = (f16)gelu_tanh_f(v);
        }
      }
    }
  } else if constexpr (EPI == EPI_SWIGLU) {
    // Packed 32-column block p: even p = gate columns, odd p = the matching up columns.
#pragma unroll
    for (int j = 0; j < C::TN; j += 2) {
      const int pb = (n0 + wn * WN) / 32 + j;
      const int n = (pb >> 1) * 32 + (lane & 31);
      if (n >= g.N) continue;
#pragma unroll
      for (int i = 0; i < C::TM; ++i) {
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const int m = mrow0 + 32 * i + 8 * (r >> 2) + (r & 3);
          if (m >= g.M) continue;
          g.out16[(size_t)m * g.ldo + n] = (f16)(silu_f(acc[i][j][r]) * acc[i][j + 1][r]);
        }
      }
    }
  } else {  // EPI_QKV_ROPE: bias, RoPE on the Q and K columns, fp16 row-major [M, 3hd]
    const int d = g.head_dim, hd = g.hd, seq = g.seq;
    const int half = g.rot_half;
    // Per 32-column block: bias and the head dim of this lane's column; the rotary only
    // touches the Q and K sections (columns < 2hd).
    float bj[C::TN];
    int ej[C::TN];
    bool rj[C::TN];
#pragma unroll
    for (int j = 0; j < C::TN; ++j) {
      const int n = ncol0 + 32 * j;
      bj[j] = (g.bias && n < g.N) ? g.bias[n] : 0.0f;
      ej[j] = n % d;
      rj[j] = n < 2 * hd && ej[j] < 2 * half;
    }
    const bool vec4 = (seq & 3) == 0;
#pragma unroll
    for (int i = 0; i < C::TM; ++i) {
#pragma unroll
      for (int r4 = 0; r4 < 16; r4 += 4) {
        const int mb = mrow0 + 32 * i + 8 * (r4 >> 2);
        int pt[4];
        pt[0] = mb % seq;
#pragma unroll
        for (int t = 1; t < 4; ++t) pt[t] = vec4 ? pt[0] + t : (mb + t) % seq;
#pragma unroll
        for (int j = 0; j < C::TN; ++j) {
          const int n = ncol0 + 32 * j;
#pragma unroll
          for (int t = 0; t < 4; ++t) {
            const int r = r4 + t, m = mb + t;
            float v = acc[i][j][r] + bj[j];
            if (half > 0) {
              // partner column e +/- half: a neighbouring lane (half <= 16) or the
              // neighbouring 32-column block (half == 32)
              const float pv = half <= 16 ? __shfl_xor(v, half) : acc[i][j ^ 1][r] + bj[j ^ 1];
              if (rj[j] && m < g.M) {
                const int e = ej[j];
                const int fi = e < half ? e : e - half;
                const float cs = g.rope_cos[pt[t] * half + fi];
                const float sn = g.rope_sin[pt[t] * half + fi];
                v = e < half ? v * cs - pv * sn : v * cs + pv * sn;
              }
            }
            if (m < g.M && n < g.N) g.out16[(size_t)m * g.ldo + n] = (f16)v;
          }
        }
      }
    }
  }
}

template <int BM, int BN, int WM, int WN>
hipError_t launch_cfg(const GemmArgs& a, hipStream_t st) {
  using C = Cfg<BM, BN, WM, WN>;
  const int nbm = (a.M + BM - 1) / BM, nbn = a.Npad / BN;
  const dim3 grid(nbm * nbn), block(C::NT);
  switch (a.epi) {
    case EPI_STORE_F32: hipLaunchKernelGGL((gemm_kernel<BM, BN, WM, WN, EPI_STORE_F32>), grid, block, 0, st, a); break;
    case EPI_STORE_F16: hipLaunchKernelGGL((gemm_kernel<BM, BN, WM, WN, EPI_STORE_F16>), grid, block, 0, st, a); break;
    case EPI_RESID_ADD: hipLaunchKernelGGL((gemm_kernel<BM, BN, WM, WN, EPI_RESID_ADD>), grid, block, 0, st, a); break;
    case EPI_SWIGLU: hipLaunchKernelGGL((gemm_kernel<BM, BN, WM, WN, EPI_SWIGLU>), grid, block, 0, st, a); break;
    case EPI_GELU: hipLaunchKernelGGL((gemm_kernel<BM, BN, WM, WN, EPI_GELU>), grid, block, 0, st, a); break;
    case EPI_QKV_ROPE: hipLaunchKernelGGL((gemm_kernel<BM, BN, WM, WN, EPI_QKV_ROPE>), grid, block, 0, st, a); break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

}  // namespace

int gemm_pick_tile(int M, int N) {
  // Large problems: 256x256 block tiles fill 256 CUs with whole waves of tiles.
  if (M >= 2048 && N >= 2048) return TILE_256x256;
  if (M >= 256) return TILE_128x128;
  return TILE_64x128;
}

hipError_t launch_gemm(const GemmArgs& a, int tile, hipStream_t st) {
  if (a.M <= 0) return hipSuccess;
  if (a.K % BK != 0 || a.Npad % 256 != 0) return hipErrorInvalidValue;
  switch (tile) {
    case TILE_256x256: return launch_cfg<256, 256, 128, 64>(a, st);
    case TILE_128x128: return launch_cfg<128, 128, 64, 64>(a, st);
    case TILE_64x128: return launch_cfg<64, 128, 32, 64>(a, st);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace tfp
