// Q8_0 weight encoding (GGUF's 8-bit format): a row is split into blocks of 32
// consecutive values; a block keeps d = max|x| / 127 as float16 and int8 codes
// q = round(x * (1 / d)), rounded half away from zero, with d and 1/d in float32; a value
// decodes as q * d.
//
// quantize: one thread per block (pack time). The scale and the codes are decided with
// correctly rounded float32 division, reciprocal and multiply, so the codes are a
// function of the float16 input alone.
// dequantize: one thread per 8 codes (every forward, in front of each GEMM): an 8-byte
// load of codes, the block's float16 scale, a 16-byte store of float16 values into the
// GEMM's MFMA fragment order (below); lanes cover consecutive 8-value groups.
//
// Fragment order of a weight [rows, K] (rows a multiple of 32, K of 16): the 32-row x
// 16-k block (rb, ks) is 512 values at offset (rb * K/16 + ks) * 512; its 16-byte piece l
// (l = 0..63) holds row 32 rb + l % 32, k 16 ks + 8 (l / 32) .. +7 -- one MFMA lane's
// operand. pack_fragments rewrites a row-major matrix into that order.
#include "tf_internal.h"

namespace tfp {

namespace {

constexpr int QBLK = 32;

__global__ void __launch_bounds__(256)
quantize_q8_0_kernel(const f16* __restrict__ w, int64_t nblocks, int8_t* __restrict__ q,
                     f16* __restrict__ d) {
  const int64_t b = blockIdx.x * (int64_t)blockDim.x + threadIdx.x;
  if (b >= nblocks) return;
  const f16x8* src = reinterpret_cast<const f16x8*>(w + b * QBLK);
  float x[QBLK];
#pragma unroll
  for (int c = 0; c < QBLK / 8; ++c) {
    const f16x8 v = src[c];
#pragma unroll
    for (int e = 0; e < 8; ++e) x[8 * c + e] = (float)v[e];
  }
  float amax = 0.f;
#pragma unroll
  for (int e = 0; e < QBLK; ++e) amax = fmaxf(amax, fabsf(x[e]));
  const float dd = __fdiv_rn(amax, 127.0f);
  const float inv = dd != 0.f ? __frcp_rn(dd) : 0.f;
  int8_t codes[QBLK];
#pragma unroll
  for (int e = 0; e < QBLK; ++e) codes[e] = (int8_t)roundf(__fmul_rn(x[e], inv));
  int4* dst = reinterpret_cast<int4*>(q + b * QBLK);
  dst[0] = *reinterpret_cast<const int4*>(codes);
  dst[1] = *reinterpret_cast<const int4*>(codes + 16);
  d[b] = (f16)dd;
}


__global__ void __launch_bounds__(256)
dequantize_q8_0_kernel(const int8_t* __restrict__ q, const f16* __restrict__ d, int64_t npieces,
                       int64_t cols, f16* __restrict__ out) {
  // one thread per 16-byte piece of the fragment-order output, so the stores are
  // contiguous; piece l of block (rb, ks) is row 32 rb + l % 32, k 16 ks + 8 (l / 32)
  const int64_t pi = blockIdx.x * (int64_t)blockDim.x + threadIdx.x;
  if (pi >= npieces) return;
  const int64_t ksr = cols / 16, l = pi & 63, blk = pi >> 6;
  const int64_t r = (blk / ksr) * 32 + (l & 31), k0 = (blk % ksr) * 16 + 8 * (l >> 5);
  const int64_t e0 = r * cols + k0;
  const int2 c = *reinterpret_cast<const int2*>(q + e0);
  const float s = (float)d[e0 / QBLK];
  const int8_t* cb = reinterpret_cast<const int8_t*>(&c);
  f16x8 o;
#pragma unroll
  for (int e = 0; e < 8; ++e) o[e] = (f16)((float)cb[e] * s);
  *reinterpret_cast<f16x8*>(out + pi * 8) = o;
}

// one thread per 16-byte piece of the output (so the stores are contiguous)
__global__ void __launch_bounds__(256)
pack_fragments_kernel(const f16* __restrict__ src, int64_t npieces, int64_t cols,
                      f16* __restrict__ dst) {
  const int64_t pi = blockIdx.x * (int64_t)blockDim.x + threadIdx.x;
  if (pi >= npieces) return;
  const int64_t ksr = cols / 16, l = pi & 63, blk = pi >> 6;
  const int64_t r = (blk / ksr) * 32 + (l & 31), k0 = (blk % ksr) * 16 + 8 * (l >> 5);
  *reinterpret_cast<f16x8*>(dst + pi * 8) = *reinterpret_cast<const f16x8*>(src + r * cols + k0);
}

}  // namespace

hipError_t launch_quantize_q8_0(const f16* w, int64_t rows, int64_t cols, int8_t* q, f16* d,
                                hipStream_t st) {
  if (rows <= 0 || cols <= 0) return hipSuccess;
  if (cols % QBLK) return hipErrorInvalidValue;
  const int64_t nb = rows * (cols / QBLK);
  hipLaunchKernelGGL(quantize_q8_0_kernel, dim3((unsigned)((nb + 255) / 256)), dim3(256), 0, st,
                     w, nb, q, d);
  return hipGetLastError();
}

hipError_t launch_dequantize_q8_0(const int8_t* q, const f16* d, int64_t rows, int64_t cols,
                                  f16* out, hipStream_t st) {
  if (rows <= 0 || cols <= 0) return hipSuccess;
  if (cols % QBLK) return hipErrorInvalidValue;
  if (rows % 32 || cols % 16) return hipErrorInvalidValue;
  const int64_t ng = rows * cols / 8;
  hipLaunchKernelGGL(dequantize_q8_0_kernel, dim3((unsigned)((ng + 255) / 256)), dim3(256), 0,
                     st, q, d, ng, cols, out);
  return hipGetLastError();
}

hipError_t launch_pack_fragments(const f16* src, int64_t rows, int64_t cols, f16* dst,
                                 hipStream_t st) {
  if (rows <= 0 || cols <= 0) return hipSuccess;
  if (rows % 32 || cols % 16 || src == dst) return hipErrorInvalidValue;
  const int64_t np = rows * cols / 8;
  hipLaunchKernelGGL(pack_fragments_kernel, dim3((unsigned)((np + 255) / 256)), dim3(256), 0, st,
                     src, np, cols, dst);
  return hipGetLastError();
}

}  // namespace tfp
