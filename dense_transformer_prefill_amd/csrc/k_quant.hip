// Q8_0 weight encoding (GGUF's 8-bit format): a row is split into blocks of 32
// consecutive values; a block keeps d = max|x| / 127 as float16 and int8 codes
// q = round(x * (1 / d)), rounded half away from zero, with d and 1/d in float32; a value
// decodes as q * d.
//
// quantize: one thread per block (pack time). The scale and the codes are decided with
// correctly rounded float32 division, reciprocal and multiply, so the codes are a
// function of the float16 input alone.
// dequantize: one thread per 8 codes (every forward, in front of each GEMM): an 8-byte
// load of codes, the block's float16 scale, a 16-byte store of float16 values; lanes
// cover consecutive 8-value groups, so loads and stores are contiguous across a wave.
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
dequantize_q8_0_kernel(const int8_t* __restrict__ q, const f16* __restrict__ d, int64_t ngroups,
                       f16* __restrict__ out) {
  const int64_t gi = blockIdx.x * (int64_t)blockDim.x + threadIdx.x;  // group of 8 codes
  if (gi >= ngroups) return;
  const int2 c = *reinterpret_cast<const int2*>(q + gi * 8);
  const float s = (float)d[gi / (QBLK / 8)];
  const int8_t* cb = reinterpret_cast<const int8_t*>(&c);
  f16x8 o;
#pragma unroll
  for (int e = 0; e < 8; ++e) o[e] = (f16)((float)cb[e] * s);
  *reinterpret_cast<f16x8*>(out + gi * 8) = o;
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
  const int64_t ng = rows * cols / 8;
  hipLaunchKernelGGL(dequantize_q8_0_kernel, dim3((unsigned)((ng + 255) / 256)), dim3(256), 0,
                     st, q, d, ng, out);
  return hipGetLastError();
}

}  // namespace tfp
