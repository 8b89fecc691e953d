// Row kernels: embedding gather, LayerNorm / RMSNorm, post-norm RMS + residual add,
// the full-width QK RMSNorm with RoPE, and a dtype conversion used by the packer.
//
// All of them are HBM-bound streaming kernels: one 64-lane wavefront owns one row of
// `hidden` elements, keeps it in registers (float4 per lane per 256 elements) and reduces
// with cross-lane shuffles, so every element is read once and written once. Statistics
// are fp32; means and variances are two-pass (mean first, then centred squares).
#include "tf_internal.h"

namespace tfp {

namespace {

constexpr int ROWS_PER_BLOCK = 4;  // 4 wavefronts, one row each

__device__ __forceinline__ float wave_sum(float v) {
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) v += __shfl_xor(v, o);
  return v;
}

// ---------------------------------------------------------------------------- embedding
// x32[t] = E[ids[t]] (fp32), plus the learned position row P[t % seq] when P is given;
// with ln_w: LayerNorm(that; ln_w, ln_b) instead. Also the fp16 copy x16 when requested.
// Ids outside [0, vocab) give a NaN row (never read OOB).
template <int NCH>
__global__ void __launch_bounds__(64 * ROWS_PER_BLOCK)
embed_kernel(const int32_t* __restrict__ ids, const f16* __restrict__ E, int vocab, int T,
             int h, const f16* __restrict__ P, int seq, const float* __restrict__ ln_w,
             const float* __restrict__ ln_b, float eps, float* __restrict__ x32,
             f16* __restrict__ x16) {
  const int lane = threadIdx.x & 63;
  const int t = blockIdx.x * ROWS_PER_BLOCK + (threadIdx.x >> 6);
  if (t >= T) return;
  const int id = ids[t];
  const bool ok = id >= 0 && id < vocab;
  const f16* src = E + (size_t)(ok ? id : 0) * h;
  float4 v[NCH];
#pragma unroll
  for (int c = 0; c < NCH; ++c) {
    const int col = (c * 64 + lane) * 4;
    const f16x4 e = *reinterpret_cast<const f16x4*>(src + col);
    v[c] = ok ? make_float4((float)e[0], (float)e[1], (float)e[2], (float)e[3])
              : make_float4(__builtin_nanf(""), __builtin_nanf(""), __builtin_nanf(""),
                            __builtin_nanf(""));
  }
  if (P) {
    const f16* prow = P + (size_t)(t % seq) * h;
#pragma unroll
    for (int c = 0; c < NCH; ++c) {
      const int col = (c * 64 + lane) * 4;
      const f16x4 p = *reinterpret_cast<const f16x4*>(prow + col);
      v[c].x += (float)p[0]; v[c].y += (float)p[1]; v[c].z += (float)p[2]; v[c].w += (float)p[3];
    }
  }
  if (ln_w) {
    float s = 0.f;
#pragma unroll
    for (int c = 0; c < NCH; ++c) s += (v[c].x + v[c].y) + (v[c].z + v[c].w);
    const float mu = wave_sum(s) / h;
    float q = 0.f;
#pragma unroll
    for (int c = 0; c < NCH; ++c) {
      v[c].x -= mu; v[c].y -= mu; v[c].z -= mu; v[c].w -= mu;
      q += (v[c].x * v[c].x + v[c].y * v[c].y) + (v[c].z * v[c].z + v[c].w * v[c].w);
    }
    const float rs = rsqrtf(wave_sum(q) / h + eps);
#pragma unroll
    for (int c = 0; c < NCH; ++c) {
      const int col = (c * 64 + lane) * 4;
      const float4 w = *reinterpret_cast<const float4*>(ln_w + col);
      const float4 b = *reinterpret_cast<const float4*>(ln_b + col);
      v[c].x = v[c].x * rs * w.x + b.x; v[c].y = v[c].y * rs * w.y + b.y;
      v[c].z = v[c].z * rs * w.z + b.z; v[c].w = v[c].w * rs * w.w + b.w;
    }
  }
#pragma unroll
  for (int c = 0; c < NCH; ++c) {
    const int col = (c * 64 + lane) * 4;
    *reinterpret_cast<float4*>(x32 + (size_t)t * h + col) = v[c];
    if (x16) {
      f16x4 o = {(f16)v[c].x, (f16)v[c].y, (f16)v[c].z, (f16)v[c].w};
      *reinterpret_cast<f16x4*>(x16 + (size_t)t * h + col) = o;
    }
  }
}

// ------------------------------------------------------------------------ LayerNorm / RMS
// The block's rows share the gains (and biases): they are deposited in dynamic LDS by DMA
// (`global_load_lds`, 256 floats per instruction) before the rows are read, so they arrive
// with the rows, once per block, and hold no registers. Waves past the last row still take
// part in the DMA and the barrier.
typedef __attribute__((address_space(3))) void* lds_ptr;

template <int NCH>
__device__ __forceinline__ void vec_to_lds(const float* __restrict__ src, float* dst, int wave,
                                           int waves, int lane) {
  for (int k = wave; k < NCH; k += waves)
    __builtin_amdgcn_global_load_lds((const void*)(src + k * 256 + lane * 4),
                                     (lds_ptr)(dst + k * 256), 16, 0, 0);
}

// out16[t] = LN(x32[t]) * w + b   (rms == 0)   or   x32[t] / rms(x32[t]) * w   (rms == 1)
template <int NCH>
__global__ void __launch_bounds__(64 * ROWS_PER_BLOCK)
norm_kernel(const float* __restrict__ x32, int T, int h, int rms, const float* __restrict__ w,
            const float* __restrict__ b, float eps, f16* __restrict__ out16) {
  extern __shared__ __attribute__((aligned(16))) float nrm_lds[];  // gains [h], biases [h]
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int t = blockIdx.x * ROWS_PER_BLOCK + wave;
  vec_to_lds<NCH>(w, nrm_lds, wave, ROWS_PER_BLOCK, lane);
  if (b) vec_to_lds<NCH>(b, nrm_lds + h, wave, ROWS_PER_BLOCK, lane);
  const bool valid = t < T;
  const float* row = x32 + (size_t)(valid ? t : T - 1) * h;
  float4 v[NCH];
#pragma unroll
  for (int c = 0; c < NCH; ++c) v[c] = *reinterpret_cast<const float4*>(row + (c * 64 + lane) * 4);
  float rs;
  if (!rms) {
    float s = 0.f;
#pragma unroll
    for (int c = 0; c < NCH; ++c) s += (v[c].x + v[c].y) + (v[c].z + v[c].w);
    const float mu = wave_sum(s) / h;
    float q = 0.f;
#pragma unroll
    for (int c = 0; c < NCH; ++c) {
      v[c].x -= mu; v[c].y -= mu; v[c].z -= mu; v[c].w -= mu;
      q += (v[c].x * v[c].x + v[c].y * v[c].y) + (v[c].z * v[c].z + v[c].w * v[c].w);
    }
    rs = rsqrtf(wave_sum(q) / h + eps);
  } else {
    float q = 0.f;
#pragma unroll
    for (int c = 0; c < NCH; ++c)
      q += (v[c].x * v[c].x + v[c].y * v[c].y) + (v[c].z * v[c].z + v[c].w * v[c].w);
    rs = rsqrtf(wave_sum(q) / h + eps);
  }
  __builtin_amdgcn_s_waitcnt((7 << 4) | (15 << 8));  // vmcnt(0): this wave's DMA landed
  __syncthreads();                                    // everyone's
  if (!valid) return;
#pragma unroll
  for (int c = 0; c < NCH; ++c) {
    const int col = (c * 64 + lane) * 4;
    const float4 g = *reinterpret_cast<const float4*>(nrm_lds + col);
    float4 y = make_float4(v[c].x * rs * g.x, v[c].y * rs * g.y, v[c].z * rs * g.z, v[c].w * rs * g.w);
    if (b) {
      const float4 bb = *reinterpret_cast<const float4*>(nrm_lds + h + col);
      y.x += bb.x; y.y += bb.y; y.z += bb.z; y.w += bb.w;
    }
    f16x4 o = {(f16)y.x, (f16)y.y, (f16)y.z, (f16)y.w};
    *reinterpret_cast<f16x4*>(out16 + (size_t)t * h + col) = o;
  }
}

// --------------------------------------------------------------- post-norm residual add
// x32[t] += a32[t] / rms(a32[t]) * w ;  x16[t] = fp16(x32[t])  (gains by DMA as above; the
// residual row is requested with a32's row, before the reduction)
template <int NCH>
__global__ void __launch_bounds__(64 * ROWS_PER_BLOCK)
rms_add_kernel(const float* __restrict__ a32, const float* __restrict__ w, float eps,
               float* __restrict__ x32, f16* __restrict__ x16, int T, int h) {
  extern __shared__ __attribute__((aligned(16))) float nrm_lds[];  // gains [h]
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int t = blockIdx.x * ROWS_PER_BLOCK + wave;
  vec_to_lds<NCH>(w, nrm_lds, wave, ROWS_PER_BLOCK, lane);
  const bool valid = t < T;
  const size_t r0 = (size_t)(valid ? t : T - 1) * h;
  float4 v[NCH], x[NCH];
  float q = 0.f;
#pragma unroll
  for (int c = 0; c < NCH; ++c) {
    v[c] = *reinterpret_cast<const float4*>(a32 + r0 + (c * 64 + lane) * 4);
    x[c] = *reinterpret_cast<const float4*>(x32 + r0 + (c * 64 + lane) * 4);
  }
#pragma unroll
  for (int c = 0; c < NCH; ++c)
    q += (v[c].x * v[c].x + v[c].y * v[c].y) + (v[c].z * v[c].z + v[c].w * v[c].w);
  const float rs = rsqrtf(wave_sum(q) / h + eps);
  __builtin_amdgcn_s_waitcnt((7 << 4) | (15 << 8));  // vmcnt(0): this wave's DMA landed
  __syncthreads();
  if (!valid) return;
#pragma unroll
  for (int c = 0; c < NCH; ++c) {
    const int col = (c * 64 + lane) * 4;
    const float4 g = *reinterpret_cast<const float4*>(nrm_lds + col);
    float4 y = x[c];
    y.x += v[c].x * rs * g.x; y.y += v[c].y * rs * g.y;
    y.z += v[c].z * rs * g.z; y.w += v[c].w * rs * g.w;
    *reinterpret_cast<float4*>(x32 + (size_t)t * h + col) = y;
    f16x4 o = {(f16)y.x, (f16)y.y, (f16)y.z, (f16)y.w};
    *reinterpret_cast<f16x4*>(x16 + (size_t)t * h + col) = o;
  }
}

// ------------------------------------------------------------------- QK norm + RoPE
// One 256-thread block per token row of qk32 [T, hd + kvd] (Q | K, fp32; the V columns of
// qkv16 are written by the GEMM itself).
// Mode 1 (whole-row RMSNorm): the RMS of the whole Q row and of the whole K row.
// Mode 2 (per-head LayerNorm, no bias): mean and variance of each head's d values, one wave
// per head, two passes over values held in registers.
// Then gains, RoPE (pairs (e, e + rot/2) inside each head), the query scale on the Q part
// (q_scale, applied in fp32 so q is rounded to fp16 once) and fp16 into the Q | K columns
// of qkv16 [T, hd + 2 kvd].
constexpr int QKN_THREADS = 256;
constexpr int QKN_MAX_HEADS = 256;  // query + key heads of one row (hidden <= 8192, d >= 64)
constexpr int QKN_HOLD = 8;         // 4-value groups a thread holds in the whole-row path

// The whole-row RMSNorm path (mode 1 with the conditions below) takes the gains and the
// position's cos / sin rows through LDS: floats of dynamic LDS it needs.
__host__ __device__ inline bool qkn_whole_row(int mode, int qk, int rot) {
  const int half = rot >> 1, pl = half >> 2, n = qk / (4 * QKN_THREADS);
  return mode == 1 && half % 4 == 0 && pl <= 32 && (pl & (pl - 1)) == 0 &&
         n * 4 * QKN_THREADS == qk && n <= QKN_HOLD;
}
__host__ __device__ inline int qkn_rope_lds(int rot, int rope_ld) {
  return rot > 0 ? (rope_ld + 63) / 64 * 64 : 0;  // per table
}

__global__ void __launch_bounds__(QKN_THREADS)
qknorm_rope_kernel(const float* __restrict__ qk32, int mode, const float* __restrict__ qw,
                   const float* __restrict__ kw, float eps, const float* __restrict__ cos_t,
                   const float* __restrict__ sin_t, int rope_ld, int rot, int seq, int H,
                   int Hkv, int d, float q_scale, f16* __restrict__ qkv16) {
  __shared__ float red[2][QKN_THREADS / 64];
  __shared__ float mu[QKN_MAX_HEADS], rsd[QKN_MAX_HEADS];
  extern __shared__ __attribute__((aligned(16))) float qkn_dyn[];
  const int t = blockIdx.x;
  const int hd = H * d, kvd = Hkv * d, ld = hd + 2 * kvd, qk = hd + kvd;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const float* row = qk32 + (size_t)t * qk;
  f16* orow = qkv16 + (size_t)t * ld;
  // Rows hold whole heads of d (a multiple of 64) values, so every row segment below is
  // a whole number of 4-value groups at 16-byte (fp32) / 8-byte (fp16) aligned offsets.
  auto ld4 = [](const float* p) { return *reinterpret_cast<const float4*>(p); };
  auto st4 = [](f16* p, float a, float b, float c, float e) {
    *reinterpret_cast<f16x4*>(p) = f16x4{(f16)a, (f16)b, (f16)c, (f16)e};
  };
  auto sumsq4 = [](float4 x) { return (x.x * x.x + x.y * x.y) + (x.z * x.z + x.w * x.w); };
  // Whole-row RMS with the row's Q and K values held in registers (up to QKN_HOLD 4-value
  // groups per thread): the row is read once. Thread i holds columns 4i + 1024 k, so a
  // column's rotary partner, half columns away, is held by thread i ^ (half / 4) of the
  // same wave when half / 4 is a power of two up to 32 (heads are d / 4 threads, a
  // multiple of half / 2), and is taken by a lane exchange instead of a second read.
  {
    const int half = rot >> 1, pl = half >> 2;
    const int n = qk / (4 * QKN_THREADS);
    if (qkn_whole_row(mode, qk, rot)) {
      // The gains ([qk]) and the cos / sin rows of this position go into LDS by DMA first,
      // so they arrive with the row instead of in a second memory round trip after the
      // block reduction (and hold no registers meanwhile).
      const int p = t % seq;
      const int rl = qkn_rope_lds(rot, rope_ld);
      float* const gl = qkn_dyn;
      float* const cl = qkn_dyn + qk;
      float* const sl = cl + rl;
      for (int k = wave; k < qk / 256; k += QKN_THREADS / 64) {  // 256 floats per instruction
        const int c = k * 256 + lane * 4;
        const float* src = c < hd ? qw + c : kw + (c - hd);
        __builtin_amdgcn_global_load_lds((const void*)src, (lds_ptr)(gl + k * 256), 16, 0, 0);
      }
      for (int k = wave; k < 2 * (rl / 64); k += QKN_THREADS / 64) {  // 64 floats each
        const int tb = k / (rl / 64), c = (k % (rl / 64)) * 64;
        const float* src = (tb ? sin_t : cos_t) + (size_t)p * rope_ld + min(c + lane, rope_ld - 1);
        __builtin_amdgcn_global_load_lds((const void*)src, (lds_ptr)((tb ? sl : cl) + c), 4, 0, 0);
      }
      float4 xs[QKN_HOLD];
      float sq = 0.f, sk = 0.f;
#pragma unroll
      for (int i = 0; i < QKN_HOLD; ++i) {
        if (i < n) {
          const int c = 4 * threadIdx.x + i * 4 * QKN_THREADS;
          xs[i] = ld4(row + c);
          if (c < hd) sq += sumsq4(xs[i]);
          else sk += sumsq4(xs[i]);
        }
      }
      sq = wave_sum(sq);
      sk = wave_sum(sk);
      if (lane == 0) {
        red[0][wave] = sq;
        red[1][wave] = sk;
      }
      // this wave's DMA has landed (s_waitcnt vmcnt(0)); the barrier makes all of it visible
      __builtin_amdgcn_s_waitcnt((7 << 4) | (15 << 8));
      __syncthreads();
      sq = 0.f;
      sk = 0.f;
#pragma unroll
      for (int i = 0; i < QKN_THREADS / 64; ++i) {
        sq += red[0][i];
        sk += red[1][i];
      }
      const float hq = rsqrtf(sq / hd + eps), hk = rsqrtf(sk / kvd + eps);
#pragma unroll
      for (int i = 0; i < QKN_HOLD; ++i) {
        if (i < n) {
          const int c = 4 * threadIdx.x + i * 4 * QKN_THREADS;
          const bool isq = c < hd;
          const int e = c % d;
          const float r = isq ? hq : hk, os = isq ? q_scale : 1.f;
          const float4 g = *reinterpret_cast<const float4*>(gl + c);
          float4 v = make_float4(xs[i].x * r * g.x, xs[i].y * r * g.y, xs[i].z * r * g.z,
                                 xs[i].w * r * g.w);
          if (pl > 0) {  // every lane takes part in the exchange
            const float4 pv = make_float4(__shfl_xor(v.x, pl), __shfl_xor(v.y, pl),
                                          __shfl_xor(v.z, pl), __shfl_xor(v.w, pl));
            if (e < rot) {
              const int fi = e < half ? e : e - half;
              const float4 cs = *reinterpret_cast<const float4*>(cl + fi);
              const float4 sn = *reinterpret_cast<const float4*>(sl + fi);
              const float sg = e < half ? -1.f : 1.f;
              v = make_float4(v.x * cs.x + sg * pv.x * sn.x, v.y * cs.y + sg * pv.y * sn.y,
                              v.z * cs.z + sg * pv.z * sn.z, v.w * cs.w + sg * pv.w * sn.w);
            }
          }
          st4(orow + c, v.x * os, v.y * os, v.z * os, v.w * os);
        }
      }
      return;
    }
  }
  float rq = 0.f, rk = 0.f;
  if (mode == 1) {
    float sq = 0.f, sk = 0.f;
    for (int c = 4 * threadIdx.x; c < hd; c += 4 * QKN_THREADS) sq += sumsq4(ld4(row + c));
    for (int c = 4 * threadIdx.x; c < kvd; c += 4 * QKN_THREADS) sk += sumsq4(ld4(row + hd + c));
    sq = wave_sum(sq);
    sk = wave_sum(sk);
    if (lane == 0) {
      red[0][wave] = sq;
      red[1][wave] = sk;
    }
    __syncthreads();
    sq = 0.f;
    sk = 0.f;
#pragma unroll
    for (int i = 0; i < QKN_THREADS / 64; ++i) {
      sq += red[0][i];
      sk += red[1][i];
    }
    rq = rsqrtf(sq / hd + eps);
    rk = rsqrtf(sk / kvd + eps);
  } else {
    // head j covers columns [j d, j d + d): query heads first, then key heads. A wave
    // takes heads wave, wave + 4, ...; the values of up to 8 of its heads are requested
    // together (one memory round trip per 8 heads, not per head).
    const int per = d >> 6;  // values per lane (d is 64 or 128)
    constexpr int HB = 8, WS = QKN_THREADS / 64;
    for (int j0 = wave; j0 < H + Hkv; j0 += WS * HB) {
      float v[HB][2];
#pragma unroll
      for (int b = 0; b < HB; ++b) {
        const int j = j0 + WS * b;
#pragma unroll
        for (int u = 0; u < 2; ++u)
          v[b][u] = (j < H + Hkv && u < per) ? row[j * d + u * 64 + lane] : 0.f;
      }
#pragma unroll
      for (int b = 0; b < HB; ++b) {
        const int j = j0 + WS * b;
        if (j >= H + Hkv) break;  // wave-uniform
        float s = 0.f;
#pragma unroll
        for (int u = 0; u < 2; ++u)
          if (u < per) s += v[b][u];
        const float m = wave_sum(s) / d;
        float q = 0.f;
#pragma unroll
        for (int u = 0; u < 2; ++u)
          if (u < per) q += (v[b][u] - m) * (v[b][u] - m);
        const float r = rsqrtf(wave_sum(q) / d + eps);
        if (lane == 0) {
          mu[j] = m;
          rsd[j] = r;
        }
      }
    }
    __syncthreads();
  }
  const int p = t % seq;
  const int half = rot >> 1;
  if (half % 4 == 0) {
    // four consecutive columns per thread: one head, one side of the rotary split (or
    // all past it), partners four consecutive columns half away, four frequencies per
    // cos / sin load (rope_ld is a multiple of 4); unrolled so the loads of several
    // iterations are in flight together
#pragma unroll 4
    for (int c = 4 * threadIdx.x; c < qk; c += 4 * QKN_THREADS) {
      const bool isq = c < hd;
      const int e = c % d;
      float m = 0.f, r = isq ? rq : rk;
      if (mode != 1) {
        m = mu[c / d];
        r = rsd[c / d];
      }
      const float* gw = isq ? qw + c : kw + (c - hd);
      const float4 x = ld4(row + c), g = ld4(gw);
      float4 v = make_float4((x.x - m) * r * g.x, (x.y - m) * r * g.y, (x.z - m) * r * g.z,
                             (x.w - m) * r * g.w);
      if (e < rot) {
        const int off = e < half ? half : -half;
        const float4 px = ld4(row + c + off), pg = ld4(gw + off);
        const float4 pv = make_float4((px.x - m) * r * pg.x, (px.y - m) * r * pg.y,
                                      (px.z - m) * r * pg.z, (px.w - m) * r * pg.w);
        const int fi = e < half ? e : e - half;
        const float4 cs = ld4(cos_t + (size_t)p * rope_ld + fi);
        const float4 sn = ld4(sin_t + (size_t)p * rope_ld + fi);
        const float sg = e < half ? -1.f : 1.f;  // low side x c - y s, high side y c + x s
        v = make_float4(v.x * cs.x + sg * pv.x * sn.x, v.y * cs.y + sg * pv.y * sn.y,
                        v.z * cs.z + sg * pv.z * sn.z, v.w * cs.w + sg * pv.w * sn.w);
      }
      const float os = isq ? q_scale : 1.f;
      st4(orow + c, v.x * os, v.y * os, v.z * os, v.w * os);
    }
    return;
  }
  for (int c = threadIdx.x; c < qk; c += QKN_THREADS) {
    const bool isq = c < hd;
    const int e = c % d;
    float m = 0.f, r = isq ? rq : rk;
    if (mode != 1) {
      m = mu[c / d];
      r = rsd[c / d];
    }
    float v = (row[c] - m) * r * (isq ? qw[c] : kw[c - hd]);
    if (e < rot) {
      const int pc = e < half ? c + half : c - half;
      const float pv = (row[pc] - m) * r * (isq ? qw[pc] : kw[pc - hd]);
      const int fi = e < half ? e : e - half;
      const float cs = cos_t[p * rope_ld + fi], sn = sin_t[p * rope_ld + fi];
      v = e < half ? v * cs - pv * sn : v * cs + pv * sn;
    }
    orow[c] = (f16)(isq ? v * q_scale : v);
  }
}

// ------------------------------------------------------------------------ padding mask
// One wave per 64-key word: bit l of word w of row r is mask[r, 64w + l] != 0 (0 past s).
__global__ void __launch_bounds__(256)
mask_bits_kernel(const int32_t* __restrict__ mask, int b, int s, int words,
                 uint64_t* __restrict__ bits) {
  const int wid = blockIdx.x * 4 + (threadIdx.x >> 6), lane = threadIdx.x & 63;
  if (wid >= b * words) return;  // wave-uniform
  const int r = wid / words, j = (wid % words) * 64 + lane;
  const bool tok = j < s && mask[(size_t)r * s + j] != 0;
  const uint64_t w = __ballot(tok);
  if (lane == 0) bits[wid] = w;
}

// ------------------------------------------------------------- last-position softmax
// One 1024-thread block per batch row: max, then sum of exp(x - max), then the
// probabilities, over the logits of the row's last position.
constexpr int LSM_THREADS = 1024;

template <class T>
__global__ void __launch_bounds__(LSM_THREADS)
last_softmax_kernel(const T* __restrict__ logits, int s, int V, float* __restrict__ probs) {
  __shared__ float red[LSM_THREADS / 64];
  const int r = blockIdx.x, tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const T* x = logits + ((size_t)r * s + s - 1) * V;
  float m = -INFINITY;
  for (int i = tid; i < V; i += LSM_THREADS) m = fmaxf(m, (float)x[i]);
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) m = fmaxf(m, __shfl_xor(m, o));
  if (lane == 0) red[wave] = m;
  __syncthreads();
  m = red[0];
#pragma unroll
  for (int i = 1; i < LSM_THREADS / 64; ++i) m = fmaxf(m, red[i]);
  __syncthreads();
  float z = 0.f;
  for (int i = tid; i < V; i += LSM_THREADS) z += __expf((float)x[i] - m);
  z = wave_sum(z);
  if (lane == 0) red[wave] = z;
  __syncthreads();
  z = 0.f;
#pragma unroll
  for (int i = 0; i < LSM_THREADS / 64; ++i) z += red[i];
  const float inv = 1.0f / z;
  for (int i = tid; i < V; i += LSM_THREADS) probs[(size_t)r * V + i] = __expf((float)x[i] - m) * inv;
}

__global__ void f16_to_f32_kernel(const f16* __restrict__ s, float* __restrict__ d, int64_t n) {
  for (int64_t i = blockIdx.x * (int64_t)blockDim.x + threadIdx.x; i < n;
       i += (int64_t)gridDim.x * blockDim.x)
    d[i] = (float)s[i];
}

}  // namespace

#define TFP_DISPATCH_NCH(nch, CALL) \
  switch (nch) {                    \
    case 1: CALL(1); break;         \
    case 2: CALL(2); break;         \
    case 3: CALL(3); break;         \
    case 4: CALL(4); break;         \
    case 6: CALL(6); break;         \
    case 8: CALL(8); break;         \
    case 12: CALL(12); break;       \
    case 16: CALL(16); break;       \
    case 24: CALL(24); break;       \
    case 32: CALL(32); break;       \
    default: return hipErrorInvalidValue; \
  }

static inline int row_blocks(int T) { return (T + ROWS_PER_BLOCK - 1) / ROWS_PER_BLOCK; }

hipError_t launch_embed(const int32_t* ids, const f16* E, int vocab, int T, int h,
                        const f16* P, int seq, const float* ln_w, const float* ln_b,
                        float eps, float* x32, f16* x16, hipStream_t st) {
  if (T <= 0) return hipSuccess;
  if (h % 256 || seq <= 0) return hipErrorInvalidValue;
#define CALL(N) hipLaunchKernelGGL(embed_kernel<N>, dim3(row_blocks(T)), dim3(64 * ROWS_PER_BLOCK), 0, st, ids, E, vocab, T, h, P, seq, ln_w, ln_b, eps, x32, x16)
  TFP_DISPATCH_NCH(h / 256, CALL)
#undef CALL
  return hipGetLastError();
}

hipError_t launch_norm(const float* x32, int T, int h, int rms, const float* w,
                       const float* b, float eps, f16* out16, hipStream_t st) {
  if (T <= 0) return hipSuccess;
  if (h % 256) return hipErrorInvalidValue;
  const size_t lds = (size_t)(b ? 2 : 1) * h * sizeof(float);
#define CALL(N) hipLaunchKernelGGL(norm_kernel<N>, dim3(row_blocks(T)), dim3(64 * ROWS_PER_BLOCK), lds, st, x32, T, h, rms, w, b, eps, out16)
  TFP_DISPATCH_NCH(h / 256, CALL)
#undef CALL
  return hipGetLastError();
}

hipError_t launch_rms_add(const float* a32, const float* w, float eps, float* x32, f16* x16,
                          int T, int h, hipStream_t st) {
  if (T <= 0) return hipSuccess;
  if (h % 256) return hipErrorInvalidValue;
  const size_t lds = (size_t)h * sizeof(float);
#define CALL(N) hipLaunchKernelGGL(rms_add_kernel<N>, dim3(row_blocks(T)), dim3(64 * ROWS_PER_BLOCK), lds, st, a32, w, eps, x32, x16, T, h)
  TFP_DISPATCH_NCH(h / 256, CALL)
#undef CALL
  return hipGetLastError();
}

hipError_t launch_qknorm_rope(const float* qk32, int mode, const float* qw, const float* kw,
                              float eps, const float* cos_t, const float* sin_t, int rope_ld,
                              int rot_dim, int batch, int seq, int n_heads, int n_kv_heads,
                              int head_dim, float q_scale, f16* qkv16, hipStream_t st) {
  const int T = batch * seq;
  if (T <= 0) return hipSuccess;
  if ((mode != 1 && mode != 2) || (head_dim != 64 && head_dim != 128) ||
      n_heads + n_kv_heads > QKN_MAX_HEADS)
    return hipErrorInvalidValue;
  const int qk = (n_heads + n_kv_heads) * head_dim;
  const size_t lds = qkn_whole_row(mode, qk, rot_dim)
                         ? (size_t)(qk + 2 * qkn_rope_lds(rot_dim, rope_ld)) * sizeof(float) : 0;
  hipLaunchKernelGGL(qknorm_rope_kernel, dim3(T), dim3(QKN_THREADS), lds, st, qk32, mode, qw, kw,
                     eps, cos_t, sin_t, rope_ld, rot_dim, seq, n_heads, n_kv_heads, head_dim,
                     q_scale, qkv16);
  return hipGetLastError();
}

hipError_t launch_mask_bits(const int32_t* mask, int b, int s, uint64_t* bits, hipStream_t st) {
  if (b <= 0 || s <= 0) return hipSuccess;
  const int words = (s + 63) / 64, waves = b * words;
  hipLaunchKernelGGL(mask_bits_kernel, dim3((waves + 3) / 4), dim3(256), 0, st, mask, b, s,
                     words, bits);
  return hipGetLastError();
}

hipError_t launch_last_softmax(const void* logits, int f16, int b, int s, int V, float* probs,
                               hipStream_t st) {
  if (b <= 0 || s <= 0 || V <= 0) return hipSuccess;
  if (f16)
    hipLaunchKernelGGL(last_softmax_kernel<tfp::f16>, dim3(b), dim3(LSM_THREADS), 0, st,
                       reinterpret_cast<const tfp::f16*>(logits), s, V, probs);
  else
    hipLaunchKernelGGL(last_softmax_kernel<float>, dim3(b), dim3(LSM_THREADS), 0, st,
                       reinterpret_cast<const float*>(logits), s, V, probs);
  return hipGetLastError();
}

hipError_t launch_f16_to_f32(const f16* src, float* dst, int64_t n, hipStream_t st) {
  if (n <= 0) return hipSuccess;
  const int64_t blocks = (n + 255) / 256;
  hipLaunchKernelGGL(f16_to_f32_kernel, dim3((unsigned)(blocks < 4096 ? blocks : 4096)),
                     dim3(256), 0, st, src, dst, n);
  return hipGetLastError();
}

}  // namespace tfp
