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
#ifndef ATTN_NW
#define ATTN_NW 8
#endif

__device__ __forceinline__ f32x16 mfma32(f16x8 a, f16x8 b, f32x16 c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_f16(a, b, c, 0, 0, 0);
}

// Position of key k (0..63) inside a 64-key row of the V^T tile: within each 16-key group
// the 4-key units (0, 1, 2, 3) are stored in the order (0, 2, 1, 3).
__device__ __forceinline__ int vt_key_pos(int k) {
  const int w = k & 15, u = w >> 2;
  return (k & ~15) + (((u & 1) << 1) | (u >> 1)) * 4 + (w & 3);
}

template <int D, int NW, bool ALIBI, bool PIPE>
__global__ void __launch_bounds__(NW * 64)
attn_kernel(const AttnArgs g) {
  constexpr int NT = NW * 64;
  constexpr int QW = 32;          // queries per wave: one 32-query column block
  constexpr int QB = NW * QW;     // queries per block
  constexpr int DS = D / 16;      // k-steps of the S^T product
  constexpr int DB = D / 32;      // 32-row d blocks of O^T
  constexpr int DCH = D / 8;      // 16-byte chunks per K / V row
  constexpr int KSTAGE = KT * D, VSTAGE = D * KT;
  constexpr int NKI = KT * DCH, NVI = (KT / 2) * DCH;  // K chunks, V (key pair, chunk) items
  constexpr int CK = (NKI + NT - 1) / NT;  // per thread per tile (the last may be partial)
  constexpr int CV = (NVI + NT - 1) / NT;
  constexpr int OPITCH = D + 8;            // output staging row pitch (halfs)
  constexpr int NSTG = 3;                  // K / V^T tile stages in LDS
  constexpr int SMEM = NSTG * (KSTAGE + VSTAGE) > QB * OPITCH ? NSTG * (KSTAGE + VSTAGE) : QB * OPITCH;
  __shared__ __attribute__((aligned(16))) f16 smem[SMEM];

  const int seq = g.seq, H = g.n_heads, BH = g.batch * g.n_heads;
  const int hd = H * D, ld = 3 * hd;
  const int nqblk = (seq + QB - 1) / QB;
  const int qblk = nqblk - 1 - (int)(blockIdx.x / BH);
  const int bh = blockIdx.x % BH;
  const int bi = bh / H, a = bh - bi * H;
  const int q0 = qblk * QB;
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int qw0 = q0 + wave * QW;
  const int l32 = lane & 31, hi = lane >> 5;
  const int qi = qw0 + l32;  // this lane's query

  const f16* base = g.qkv + (size_t)bi * seq * ld + a * D;
  const f16* Qh = base;
  const f16* Kh = base + hd;
  const f16* Vh = base + 2 * hd;

  // Q fragments (B operand of S^T = K Q^T): lane holds Q[qi][16ks + 8hi .. +7]
  f16x8 qf[DS];
  {
    const int qr = min(qi, seq - 1);
#pragma unroll
    for (int ks = 0; ks < DS; ++ks)
      qf[ks] = *reinterpret_cast<const f16x8*>(Qh + (size_t)qr * ld + 16 * ks + 8 * hi);
  }

  f32x16 o[DB];
#pragma unroll
  for (int db = 0; db < DB; ++db)
#pragma unroll
    for (int r = 0; r < 16; ++r) o[db][r] = 0.f;
  // Running max of this query's scores (log2 domain, scale applied) and this lane's
  // partial row sum (the lane holds half of the query's keys; halves meet at the end).
  float mrow = -INFINITY, lpart = 0.f;
  const float c = g.scale_log2;
  const float slope = ALIBI ? g.alibi_log2[a] : 0.f;

  const int kv_end = min(seq, q0 + QB);
  const int ntiles = (kv_end + KT - 1) / KT;

  const f16x8 zero8 = {0, 0, 0, 0, 0, 0, 0, 0};
  f16x8 rk[CK], rv[CV][2];
  auto gload = [&](int t) {
    const int k0 = t * KT;
#pragma unroll
    for (int i = 0; i < CK; ++i) {
      const int cc = tid + i * NT, row = cc / DCH, ch = cc % DCH;
      const int key = k0 + row;
      rk[i] = (cc < NKI && key < seq)
                  ? *reinterpret_cast<const f16x8*>(Kh + (size_t)key * ld + ch * 8) : zero8;
    }
#pragma unroll
    for (int i = 0; i < CV; ++i) {
      const int cc = tid + i * NT, kp = cc / DCH, ch = cc % DCH;
      const int key = k0 + 2 * kp;
      const bool ok = cc < NVI;
      rv[i][0] = (ok && key < seq)
                     ? *reinterpret_cast<const f16x8*>(Vh + (size_t)key * ld + ch * 8) : zero8;
      rv[i][1] = (ok && key + 1 < seq)
                     ? *reinterpret_cast<const f16x8*>(Vh + (size_t)(key + 1) * ld + ch * 8) : zero8;
    }
  };
  // K tile rows are D halfs; chunks XOR-swizzled so 16 consecutive rows' 16-byte reads
  // at one logical chunk cover all 64 banks. V^T rows are 64 keys (128 bytes).
  auto kswz = [](int row, int ch) {
    return row * D + ((ch ^ (D == 64 ? ((row >> 1) & 7) : (row & 15))) << 3);
  };
  auto vswz = [](int row, int ch) { return row * KT + ((ch ^ ((row >> 1) & 7)) << 3); };
  auto sstore = [&](int stage) {
    f16* sk = smem + stage * (KSTAGE + VSTAGE);
    f16* sv = sk + KSTAGE;
#pragma unroll
    for (int i = 0; i < CK; ++i) {
      const int cc = tid + i * NT, row = cc / DCH, ch = cc % DCH;
      if (cc < NKI) *reinterpret_cast<f16x8*>(sk + kswz(row, ch)) = rk[i];
    }
    // V^T: for each of the 8 head dims of the chunk, the two keys of the pair side by side
#pragma unroll
    for (int i = 0; i < CV; ++i) {
      const int cc = tid + i * NT, kp = cc / DCH, ch = cc % DCH;
      if (cc >= NVI) continue;
      const int pos = vt_key_pos(2 * kp);
      const int kc = pos >> 3, ko = pos & 7;
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        const int row = ch * 8 + e;
        f16x2 w = {rv[i][0][e], rv[i][1][e]};
        *reinterpret_cast<f16x2*>(sv + vswz(row, kc) + ko) = w;
      }
    }
  };

  // S^T = K Q^T for the tile in LDS stage sk (8 MFMAs at d = 64, 16 at d = 128).
  auto scores = [&](const f16* sk, f32x16 (&sc)[2]) {
#pragma unroll
    for (int kb = 0; kb < 2; ++kb) {
#pragma unroll
      for (int r = 0; r < 16; ++r) sc[kb][r] = 0.f;
      const int krow = kb * 32 + l32;
#pragma unroll
      for (int ks = 0; ks < DS; ++ks) {
        const f16x8 kf = *reinterpret_cast<const f16x8*>(sk + kswz(krow, 2 * ks + hi));
        sc[kb] = mfma32(kf, qf[ks], sc[kb]);
      }
    }
  };
  // Online softmax of tile t's scores, then O^T += V^T P^T from LDS stage sv.
  auto softmax_pv = [&](f32x16 (&sc)[2], int k0, const f16* sv) {
    // Scores in the log2 domain are t = s*c (+ slope*(key - q)); masked keys -> -inf.
    const bool need_mask = (k0 + KT - 1 > qw0) || (k0 + KT > seq);
    float mx = -INFINITY;
    if constexpr (ALIBI) {
#pragma unroll
      for (int kb = 0; kb < 2; ++kb)
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const int key = k0 + 32 * kb + 8 * (r >> 2) + 4 * hi + (r & 3);
          float x = sc[kb][r] * c + slope * (float)(key - qi);
          if (need_mask && (key > qi || key >= seq)) x = -INFINITY;
          sc[kb][r] = x;
          mx = fmaxf(mx, x);
        }
    } else {
      if (need_mask) {
#pragma unroll
        for (int kb = 0; kb < 2; ++kb)
#pragma unroll
          for (int r = 0; r < 16; ++r) {
            const int key = k0 + 32 * kb + 8 * (r >> 2) + 4 * hi + (r & 3);
            if (key > qi || key >= seq) sc[kb][r] = -INFINITY;
          }
      }
#pragma unroll
      for (int kb = 0; kb < 2; ++kb)
#pragma unroll
        for (int r = 0; r < 16; ++r) mx = fmaxf(mx, sc[kb][r]);
      mx *= c;  // max of the scaled scores (c > 0)
    }
    mx = fmaxf(mx, __shfl_xor(mx, 32));
    const float mnew = fmaxf(mrow, mx);
    const float muse = mnew == -INFINITY ? 0.f : mnew;
    // Rescale the running output only when some query's max moved in this tile.
    if (__any(mnew > mrow)) {
      const float alpha = __builtin_amdgcn_exp2f(mrow - muse);
      lpart *= alpha;
#pragma unroll
      for (int db = 0; db < DB; ++db)
#pragma unroll
        for (int r = 0; r < 16; ++r) o[db][r] *= alpha;
    }
    mrow = mnew;
    f16x8 pf[2][2];
#pragma unroll
    for (int kb = 0; kb < 2; ++kb)
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const float p = ALIBI ? __builtin_amdgcn_exp2f(sc[kb][r] - muse)
                              : __builtin_amdgcn_exp2f(__builtin_fmaf(sc[kb][r], c, -muse));
        lpart += p;
        pf[kb][r >> 3][r & 7] = (f16)p;
      }
#pragma unroll
    for (int kb = 0; kb < 2; ++kb)
#pragma unroll
      for (int hs = 0; hs < 2; ++hs) {
        const int ch = 2 * (2 * kb + hs) + hi;
#pragma unroll
        for (int db = 0; db < DB; ++db) {
          const f16x8 vf = *reinterpret_cast<const f16x8*>(sv + vswz(db * 32 + l32, ch));
          o[db] = mfma32(vf, pf[kb][hs], o[db]);
        }
      }
  };
  auto stage_k = [&](int t) { return smem + (t % NSTG) * (KSTAGE + VSTAGE); };
  auto needs = [&](int t) { return t * KT <= qw0 + QW - 1; };  // wave sees a key of tile t

  // Pipeline over key tiles. Tiles t+1 and t+2 are in LDS / in flight while tile t is
  // processed. With PIPE each wave issues the score MFMAs of tile t+1 before the softmax
  // of tile t, so its VALU work can overlap its own MFMAs (the block barrier otherwise
  // keeps every wave of a SIMD in the same phase); measured faster at d = 64 only.
  gload(0);
  sstore(0);
  if (ntiles > 1) {
    gload(1);
    sstore(1);
  }
  __syncthreads();
  f32x16 sA[2], sB[2];
  if (PIPE && needs(0)) scores(stage_k(0), sA);
  auto step = [&](int t, f32x16 (&cur)[2], f32x16 (&nxt)[2]) {
    if (t + 2 < ntiles) gload(t + 2);
    if constexpr (PIPE) {
      if (t + 1 < ntiles && needs(t + 1)) scores(stage_k(t + 1), nxt);
    } else {
      if (needs(t)) scores(stage_k(t), cur);
    }
    if (needs(t)) softmax_pv(cur, t * KT, stage_k(t) + KSTAGE);
    if (t + 2 < ntiles) sstore((t + 2) % NSTG);
    __syncthreads();
  };
  for (int t = 0; t < ntiles; t += 2) {
    step(t, sA, sB);
    if (t + 1 < ntiles) step(t + 1, sB, sA);
  }

  // Normalise and stage O[q][d] in LDS, then write 16-byte row segments.
  // O^T accumulator db register r: d = 32db + 8(r/4) + 4hi + r%4, query l32 of the wave.
  const float lsum = lpart + __shfl_xor(lpart, 32);
  const float inv = 1.0f / lsum;
  f16* so = smem + (wave * QW + l32) * OPITCH;
#pragma unroll
  for (int db = 0; db < DB; ++db)
#pragma unroll
    for (int r4 = 0; r4 < 16; r4 += 4) {
      const int d0 = 32 * db + 8 * (r4 >> 2) + 4 * hi;
      f16x4 pk = {(f16)(o[db][r4] * inv), (f16)(o[db][r4 + 1] * inv),
                  (f16)(o[db][r4 + 2] * inv), (f16)(o[db][r4 + 3] * inv)};
      *reinterpret_cast<f16x4*>(so + d0) = pk;
    }
  __syncthreads();
  for (int v = tid; v < QB * DCH; v += NT) {
    const int qr = v / DCH, ch = v % DCH;
    const int q = q0 + qr;
    if (q < seq)
      *reinterpret_cast<f16x8*>(g.out + ((size_t)bi * seq + q) * hd + a * D + ch * 8) =
          *reinterpret_cast<const f16x8*>(smem + qr * OPITCH + ch * 8);
  }
}

template <int D, int NW>
hipError_t launch_t(const AttnArgs& a, hipStream_t st) {
  constexpr int QB = NW * 32;
  const int nqblk = (a.seq + QB - 1) / QB;
  const dim3 grid(nqblk * a.batch * a.n_heads), block(NW * 64);
  constexpr bool PIPE = D == 64;
  if (a.alibi_log2) hipLaunchKernelGGL((attn_kernel<D, NW, true, PIPE>), grid, block, 0, st, a);
  else hipLaunchKernelGGL((attn_kernel<D, NW, false, PIPE>), grid, block, 0, st, a);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_attention(const AttnArgs& a, hipStream_t st) {
  if (a.batch <= 0 || a.seq <= 0) return hipSuccess;
  if (a.head_dim == 64) return launch_t<64, ATTN_NW>(a, st);
  if (a.head_dim == 128) return launch_t<128, ATTN_NW>(a, st);
  return hipErrorInvalidValue;
}

}  // namespace tfp
