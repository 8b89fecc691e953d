// Instantiations of the fp16 MFMA GEMM (gemm_kernel.h) used by the forward pass, and the
// per-problem choice of block tile.
#include "gemm_kernel.h"

namespace tfp {

namespace {
using Big = gemm::Cfg<256, 256, 128, 64, 64, 2>;
using Mid = gemm::Cfg<128, 128, 64, 64, 64, 2>;
using Small = gemm::Cfg<64, 128, 32, 64, 64, 2>;
}  // namespace

int gemm_pick_tile(int M, int N) {
  // Large problems: 256x256 block tiles fill 256 CUs with whole waves of tiles. Running
  // them on three quarters of the CUs still beats 128x128 tiles (whose LDS traffic per
  // FLOP is a third higher), but not on a quarter or less: below 128 big tiles (one
  // batch row of 2048 tokens at hidden 2048 makes 64) the 128x128 tiles take over.
  const int big = ((M + 255) / 256) * ((N + 255) / 256);
  if (M >= 2048 && N >= 2048 && big >= 128) return TILE_256x256;
  if (M >= 256) return TILE_128x128;
  return TILE_64x128;
}

namespace {
// Tiles of a configuration for an M x N output.
int tiles_of(int tile, int M, int N) {
  const int bm = tile == TILE_256x256 ? 256 : tile == TILE_128x128 ? 128 : 64;
  const int bn = tile == TILE_256x256 ? 256 : 128;
  const int npad = (N + 255) / 256 * 256;
  return (M + bm - 1) / bm * (npad / bn);
}

// x[m, n] (+)= sum_s part[s][m, n] (+ bias[n]); one thread per 4 consecutive columns
// when N and ldo are multiples of 4 (16-byte aligned rows), else per column.
template <int VEC>
__global__ void __launch_bounds__(256)
splitk_reduce_kernel(const float* __restrict__ part, int S, size_t stride, int M, int N,
                     int ldo, const float* __restrict__ bias, float* __restrict__ out,
                     int accumulate) {
  const int cpr = N / VEC;  // vector columns per row
  const int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (i >= (int64_t)M * cpr) return;
  const int m = (int)(i / cpr), n = (int)(i % cpr) * VEC;
  const size_t o = (size_t)m * ldo + n;
  float v[VEC], t[VEC];
  auto ld = [&](const float* p, float* d) {
    if constexpr (VEC == 4) {
      const float4 q = *reinterpret_cast<const float4*>(p);
      d[0] = q.x; d[1] = q.y; d[2] = q.z; d[3] = q.w;
    } else {
      d[0] = *p;
    }
  };
  ld(part + o, v);
  for (int s = 1; s < S; ++s) {
    ld(part + (size_t)s * stride + o, t);
#pragma unroll
    for (int e = 0; e < VEC; ++e) v[e] += t[e];
  }
  if (bias) {
#pragma unroll
    for (int e = 0; e < VEC; ++e) v[e] += bias[n + e];
  }
  if (accumulate) {
    ld(out + o, t);
#pragma unroll
    for (int e = 0; e < VEC; ++e) v[e] = t[e] + v[e];
  }
  if constexpr (VEC == 4) {
    *reinterpret_cast<float4*>(out + o) = make_float4(v[0], v[1], v[2], v[3]);
  } else {
    out[o] = v[0];
  }
}
}  // namespace

int gemm_splitk(int M, int N, int K, int epi) {
  // Only the fp32-output epilogues reduce linearly; only one-tile-per-block tiles split.
  if (epi != EPI_RESID_ADD && epi != EPI_STORE_F32) return 1;
  const int tile = gemm_pick_tile(M, N);
  if (tile == TILE_256x256 || M <= 0 || K % 64 != 0) return 1;
  // Double the splits while the doubled block count still fits one block per CU of a
  // 256-CU MI355X (a fixed target, so workspace sizing does not depend on the device)
  // and every split keeps at least 4 k-tiles. (Splitting 192 tiles in two was measured
  // slower: the reduction's traffic outweighs the quarter of the chip it fills.)
  const int ntiles = tiles_of(tile, M, N), kt = K / 64;
  int S = 1;
  while (S < 8 && ntiles * 2 * S <= 256 && kt % (2 * S) == 0 && kt / (2 * S) >= 4) S *= 2;
  // a long K (>= 4096) also splits in two when that gives every CU two blocks
  if (S == 1 && ntiles <= 256 && kt >= 64 && kt % 2 == 0) S = 2;
  return S;
}

hipError_t launch_splitk_reduce(const float* part, int S, size_t stride, int M, int N, int ldo,
                                const float* bias, float* out, int accumulate, hipStream_t st) {
  if (M <= 0 || N <= 0) return hipSuccess;
  const bool vec = N % 4 == 0 && ldo % 4 == 0 && (reinterpret_cast<uintptr_t>(part) & 15) == 0 &&
                   (reinterpret_cast<uintptr_t>(out) & 15) == 0 && stride % 4 == 0 &&
                   (!bias || (reinterpret_cast<uintptr_t>(bias) & 15) == 0);
  const int64_t n = (int64_t)M * (vec ? N / 4 : N);
  const dim3 grid((unsigned)((n + 255) / 256));
  if (vec)
    hipLaunchKernelGGL(splitk_reduce_kernel<4>, grid, dim3(256), 0, st, part, S, stride, M, N,
                       ldo, bias, out, accumulate);
  else
    hipLaunchKernelGGL(splitk_reduce_kernel<1>, grid, dim3(256), 0, st, part, S, stride, M, N,
                       ldo, bias, out, accumulate);
  return hipGetLastError();
}

hipError_t launch_gemm(const GemmArgs& a, int tile, hipStream_t st) {
  if (a.M <= 0) return hipSuccess;
  if (a.K % 64 != 0 || a.Npad % 256 != 0) return hipErrorInvalidValue;
  // operand loads address each operand with a 32-bit byte offset from its base
  if ((int64_t)a.M * a.lda * 2 >= ((int64_t)1 << 32) ||
      (int64_t)a.Npad * a.ldb * 2 >= ((int64_t)1 << 32))
    return hipErrorInvalidValue;
  // rotary spans of at most 8 frequencies stage the table rows in LDS with the row length
  // fixed at compile time (frequencies rounded up to 4)
  if ((a.epi == EPI_QKV_ROPE || a.epi == EPI_QKV_HLN_ROPE) && a.rot_half > 0 &&
      a.rot_half <= 8 && a.rope_ld != (a.rot_half > 4 ? 8 : 4))
    return hipErrorInvalidValue;
  // the fused per-head LayerNorm takes 64-column heads (one per wave tile)
  if (a.epi == EPI_QKV_HLN_ROPE &&
      (a.head_dim != 64 || !a.hln_q || !a.hln_k || a.hln_hd % 64 || a.rot_cols % 64))
    return hipErrorInvalidValue;
  // Split-K when the tiles cannot fill the chip and scratch for the partials was given:
  // the partials are plain fp32 stores (no bias), reduced in split order into out32.
  const int S = tile == gemm_pick_tile(a.M, a.N) ? gemm_splitk(a.M, a.N, a.K, a.epi) : 1;
  if (S > 1 && a.part && a.part_elems >= (size_t)S * a.M * a.ldo) {
    GemmArgs p = a;
    p.epi = EPI_STORE_F32;
    p.bias = nullptr;
    p.out32 = a.part;
    p.split_stride = (size_t)a.M * a.ldo;
    hipError_t e = tile == TILE_128x128 ? gemm::launch<Mid>(p, st, S)
                                        : gemm::launch<Small>(p, st, S);
    if (e != hipSuccess) return e;
    return launch_splitk_reduce(a.part, S, p.split_stride, a.M, a.N, a.ldo, a.bias, a.out32,
                                a.epi == EPI_RESID_ADD, st);
  }
  GemmArgs u = a;
  u.split_stride = 0;
  switch (tile) {
    case TILE_256x256: return gemm::launch<Big>(u, st);
    case TILE_128x128: return gemm::launch<Mid>(u, st);
    case TILE_64x128: return gemm::launch<Small>(u, st);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace tfp
