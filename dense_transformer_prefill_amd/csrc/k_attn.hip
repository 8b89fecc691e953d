// Causal flash attention for gfx950 (fp16 MFMA, fp32 online softmax).
//
// For one (batch row, head) and a block of queries, the kernel streams 64-key tiles of
// K and V^T through LDS (two stages) and keeps a running row max, row sum and output
// accumulator, so the [s, s] score matrix never exists in memory.
//
// The scores are computed transposed, S^T = K Q^T, with v_mfma_f32_32x32x16_f16:
//   - A operand = K tile rows (keys), B operand = Q rows (queries, kept in registers);
//   - a lane of the 32x32 accumulator holds ONE query column and 16 of its keys, so the
//     row max / row sum of the softmax are in-lane reductions plus one swap with lane^32;
//   - the accumulator is then already the B operand of O^T = V^T P^T: the 8 probabilities
//     a lane feeds to one MFMA k-step are keys {4g..4g+3, 8+4g..8+4g+3} of a 16-key group
//     (g = lane/32). V tiles are transposed on their way into LDS (V^T rows = head dims),
//     with their 4-key units permuted to that order, so the matching A operand is one
//     16-byte read per lane.
// Q, K and V are read from the token-major projection output [b*s, 3*H*d].
// Softmax runs in the exp2 domain with the scale log2(e)/sqrt(d) folded into the scores;
// ALiBi adds slope*log2(e)*(j - i). P is rounded to fp16 (round to nearest even) for the
// PV product; the row sum uses the fp32 values.
//
// Work order: query blocks are issued latest (longest key range) first.
#include "tf_internal.h"

namespace tfp {

namespace {

constexpr int KT = 64;  // keys per tile

__device__ __forceinline__ f32x16 mfma32(f16x8 a, f16x8 b, f32x16 c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_f16(a, b, c, 0, 0, 0);
}

// Position of key k (0..63) inside a 64-key row of the V^T tile: within each 16-key group
// the 4-key units (0, 1, 2, 3) are stored in the order (0, 2, 1, 3).
__device__ __forceinline__ int vt_key_pos(int k) {
  const int w = k & 15, u = w >> 2;
  return (k & ~15) + (((u & 1) << 1) | (u >> 1)) * 4 + (w & 3);
}

template <int D, int QW, int NW, bool ALIBI>
__global__ void __launch_bounds__(NW * 64)
attn_kernel(const AttnArgs g) {
  constexpr int NT = NW * 64;
  constexpr int QB = NW * QW;     // queries per block
  constexpr int NQB = QW / 32;    // 32-query column blocks per wave
  constexpr int DS = D / 16;      // k-steps of the S^T product
  constexpr int DB = D / 32;      // 32-row d blocks of O^T
  constexpr int DCH = D / 8;      // 16-byte chunks per K / V row
  constexpr int KSTAGE = KT * D, VSTAGE = D * KT;
  constexpr int CK = KT * DCH / NT;        // K chunks per thread per tile
  constexpr int CV = (KT / 2) * DCH / NT;  // V (key pair, d chunk) items per thread per tile
  static_assert(CK * NT == KT * DCH && CV * NT == (KT / 2) * DCH, "tile split");
  __shared__ __attribute__((aligned(16))) f16 smem[2 * (KSTAGE + VSTAGE)];

  const int seq = g.seq, H = g.n_heads, BH = g.batch * g.n_heads;
  const int hd = H * D, ld = 3 * hd;
  const int nqblk = (seq + QB - 1) / QB;
  const int qblk = nqblk - 1 - (int)(blockIdx.x / BH);
  const int bh = blockIdx.x % BH;
  const int bi = bh / H, a = bh - bi * H;
  const int q0 = qblk * QB;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int qw0 = q0 + wave * QW;
  const int l32 = lane & 31, hi = lane >> 5;

  const f16* base = g.qkv + (size_t)bi * seq * ld + a * D;
  const f16* Qh = base;
  const f16* Kh = base + hd;
  const f16* Vh = base + 2 * hd;

  // Q fragments: lane holds Q[qw0 + 32qb + l32][16ks + 8hi .. +7]
  f16x8 qf[NQB][DS];
#pragma unroll
  for (int qb = 0; qb < NQB; ++qb) {
    const int qr = min(qw0 + 32 * qb + l32, seq - 1);
#pragma unroll
    for (int ks = 0; ks < DS; ++ks)
      qf[qb][ks] = *reinterpret_cast<const f16x8*>(Qh + (size_t)qr * ld + 16 * ks + 8 * hi);
  }

  f32x16 o[DB][NQB];
#pragma unroll
  for (int db = 0; db < DB; ++db)
#pragma unroll
    for (int qb = 0; qb < NQB; ++qb)
#pragma unroll
      for (int r = 0; r < 16; ++r) o[db][qb][r] = 0.f;
  float mrow[NQB], lrow[NQB];
#pragma unroll
  for (int qb = 0; qb < NQB; ++qb) {
    mrow[qb] = -INFINITY;
    lrow[qb] = 0.f;
  }
  const float slope = ALIBI ? g.alibi_log2[a] : 0.f;

  const int kv_end = min(seq, q0 + QB);
  const int ntiles = (kv_end + KT - 1) / KT;

  const f16x8 zero8 = {0, 0, 0, 0, 0, 0, 0, 0};
  f16x8 rk[CK], rv[CV][2];
  auto gload = [&](int t) {
    const int k0 = t * KT;
#pragma unroll
    for (int i = 0; i < CK; ++i) {
      const int c = tid + i * NT, row = c / DCH, ch = c % DCH;
      const int key = k0 + row;
      rk[i] = key < seq ? *reinterpret_cast<const f16x8*>(Kh + (size_t)key * ld + ch * 8) : zero8;
    }
#pragma unroll
    for (int i = 0; i < CV; ++i) {
      const int c = tid + i * NT, kp = c / DCH, ch = c % DCH;
      const int key = k0 + 2 * kp;
      rv[i][0] = key < seq ? *reinterpret_cast<const f16x8*>(Vh + (size_t)key * ld + ch * 8) : zero8;
      rv[i][1] = key + 1 < seq ? *reinterpret_cast<const f16x8*>(Vh + (size_t)(key + 1) * ld + ch * 8) : zero8;
    }
  };
  auto sstore = [&](int stage) {
    f16* sk = smem + stage * (KSTAGE + VSTAGE);
    f16* sv = sk + KSTAGE;
#pragma unroll
    for (int i = 0; i < CK; ++i) {
      const int c = tid + i * NT, row = c / DCH, ch = c % DCH;
      *reinterpret_cast<f16x8*>(sk + row * D + ((ch ^ (row & 7)) << 3)) = rk[i];
    }
    // V^T: for each of the 8 head dims of the chunk, the two keys of the pair side by side
#pragma unroll
    for (int i = 0; i < CV; ++i) {
      const int c = tid + i * NT, kp = c / DCH, ch = c % DCH;
      const int pos = vt_key_pos(2 * kp);
      const int kc = pos >> 3, ko = pos & 7;
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        const int row = ch * 8 + e;
        f16x2 w = {rv[i][0][e], rv[i][1][e]};
        *reinterpret_cast<f16x2*>(sv + row * KT + ((kc ^ (row & 7)) << 3) + ko) = w;
      }
    }
  };

  gload(0);
  sstore(0);
  __syncthreads();

  for (int t = 0; t < ntiles; ++t) {
    const int k0 = t * KT;
    if (t + 1 < ntiles) gload(t + 1);
    const f16* sk = smem + (t & 1) * (KSTAGE + VSTAGE);
    const f16* sv = sk + KSTAGE;

    if (k0 <= qw0 + QW - 1) {  // this wave sees at least one key of the tile
      const bool need_mask = (k0 + KT - 1 > qw0) || (k0 + KT > seq);
      f32x16 s[2][NQB];
#pragma unroll
      for (int kb = 0; kb < 2; ++kb) {
#pragma unroll
        for (int qb = 0; qb < NQB; ++qb)
#pragma unroll
          for (int r = 0; r < 16; ++r) s[kb][qb][r] = 0.f;
        const int krow = kb * 32 + l32;
#pragma unroll
        for (int ks = 0; ks < DS; ++ks) {
          const f16x8 kf = *reinterpret_cast<const f16x8*>(
              sk + krow * D + (((2 * ks + hi) ^ (krow & 7)) << 3));
#pragma unroll
          for (int qb = 0; qb < NQB; ++qb) s[kb][qb] = mfma32(kf, qf[qb][ks], s[kb][qb]);
        }
      }

      f16x8 pf[2][2][NQB];  // [kb][half][qb]
#pragma unroll
      for (int qb = 0; qb < NQB; ++qb) {
        const int qi = qw0 + 32 * qb + l32;
        float mx = -INFINITY;
#pragma unroll
        for (int kb = 0; kb < 2; ++kb)
#pragma unroll
          for (int r = 0; r < 16; ++r) {
            const int key = k0 + 32 * kb + 8 * (r >> 2) + 4 * hi + (r & 3);
            float x = s[kb][qb][r] * g.scale_log2;
            if (ALIBI) x += slope * (float)(key - qi);
            if (need_mask && (key > qi || key >= seq)) x = -INFINITY;
            s[kb][qb][r] = x;
            mx = fmaxf(mx, x);
          }
        mx = fmaxf(mx, __shfl_xor(mx, 32));
        const float mnew = fmaxf(mrow[qb], mx);
        const float muse = mnew == -INFINITY ? 0.f : mnew;
        const float alpha = __builtin_amdgcn_exp2f(mrow[qb] - muse);
        mrow[qb] = mnew;
        float sum = 0.f;
#pragma unroll
        for (int kb = 0; kb < 2; ++kb)
#pragma unroll
          for (int r = 0; r < 16; ++r) {
            const float p = __builtin_amdgcn_exp2f(s[kb][qb][r] - muse);
            s[kb][qb][r] = p;
            sum += p;
          }
        sum += __shfl_xor(sum, 32);
        lrow[qb] = lrow[qb] * alpha + sum;
#pragma unroll
        for (int db = 0; db < DB; ++db)
#pragma unroll
          for (int r = 0; r < 16; ++r) o[db][qb][r] *= alpha;
#pragma unroll
        for (int kb = 0; kb < 2; ++kb)
#pragma unroll
          for (int hs = 0; hs < 2; ++hs)
#pragma unroll
            for (int e = 0; e < 8; ++e) pf[kb][hs][qb][e] = (f16)s[kb][qb][8 * hs + e];
      }

#pragma unroll
      for (int kb = 0; kb < 2; ++kb)
#pragma unroll
        for (int hs = 0; hs < 2; ++hs) {
          const int ch = 2 * (2 * kb + hs) + hi;
#pragma unroll
          for (int db = 0; db < DB; ++db) {
            const int vrow = db * 32 + l32;
            const f16x8 vf = *reinterpret_cast<const f16x8*>(
                sv + vrow * KT + ((ch ^ (vrow & 7)) << 3));
#pragma unroll
            for (int qb = 0; qb < NQB; ++qb) o[db][qb] = mfma32(vf, pf[kb][hs][qb], o[db][qb]);
          }
        }
    }

    if (t + 1 < ntiles) sstore((t + 1) & 1);
    __syncthreads();
  }

  // O^T accumulator (db, qb) register r: d = 32db + 8(r/4) + 4hi + r%4, query 32qb + l32.
#pragma unroll
  for (int qb = 0; qb < NQB; ++qb) {
    const int qi = qw0 + 32 * qb + l32;
    if (qi >= seq) continue;
    const float inv = 1.0f / lrow[qb];
    f16* dst = g.out + ((size_t)bi * seq + qi) * hd + a * D;
#pragma unroll
    for (int db = 0; db < DB; ++db)
#pragma unroll
      for (int r4 = 0; r4 < 16; r4 += 4) {
        const int d0 = 32 * db + 8 * (r4 >> 2) + 4 * hi;
        f16x4 pk = {(f16)(o[db][qb][r4] * inv), (f16)(o[db][qb][r4 + 1] * inv),
                    (f16)(o[db][qb][r4 + 2] * inv), (f16)(o[db][qb][r4 + 3] * inv)};
        *reinterpret_cast<f16x4*>(dst + d0) = pk;
      }
  }
}

template <int D, int QW, int NW>
hipError_t launch_t(const AttnArgs& a, hipStream_t st) {
  constexpr int QB = NW * QW;
  const int nqblk = (a.seq + QB - 1) / QB;
  const dim3 grid(nqblk * a.batch * a.n_heads), block(NW * 64);
  if (a.alibi_log2) hipLaunchKernelGGL((attn_kernel<D, QW, NW, true>), grid, block, 0, st, a);
  else hipLaunchKernelGGL((attn_kernel<D, QW, NW, false>), grid, block, 0, st, a);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_attention(const AttnArgs& a, hipStream_t st) {
  if (a.batch <= 0 || a.seq <= 0) return hipSuccess;
  if (a.head_dim == 64) return launch_t<64, 64, 4>(a, st);
  if (a.head_dim == 128) return launch_t<128, 32, 4>(a, st);
  return hipErrorInvalidValue;
}

}  // namespace tfp
