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
  // Large problems: 256x256 block tiles fill 256 CUs with whole waves of tiles.
  if (M >= 2048 && N >= 2048) return TILE_256x256;
  if (M >= 256) return TILE_128x128;
  return TILE_64x128;
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
  if (a.epi == EPI_QKV_ROPE && a.rot_half > 0 && a.rot_half <= 8 &&
      a.rope_ld != (a.rot_half > 4 ? 8 : 4))
    return hipErrorInvalidValue;
  switch (tile) {
    case TILE_256x256: return gemm::launch<Big>(a, st);
    case TILE_128x128: return gemm::launch<Mid>(a, st);
    case TILE_64x128: return gemm::launch<Small>(a, st);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace tfp
