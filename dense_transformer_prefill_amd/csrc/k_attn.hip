// Causal flash attention for gfx950 (fp16 MFMA, fp32 online softmax).
//
// For one (batch row, head) and a block of queries, the kernel streams 64-key tiles of
// K and V through LDS (four stages, filled by global_load_lds: no VGPR round trip) and
// keeps a running row max, row sum and output accumulator, so the [s, s] score matrix
// never exists in memory.
//
// The scores are computed transposed, S^T = K Q^T, with v_mfma_f32_32x32x16_f16:
//   - A operand = K tile rows (keys), B operand = Q rows (queries, kept in registers);
//   - a lane of the 32x32 accumulator holds ONE query column and 16 of its keys, so the
//     row max / row sum of the softmax are in-lane reductions plus one swap with lane^32;
//   - the accumulator is then already the B operand of O^T = V^T P^T: the 8 probabilities
//     a lane feeds to one MFMA k-step are keys {4g..4g+3, 8+4g..8+4g+3} of a 16-key group
//     (g = lane/32). V stays row-major in LDS; the matching A operand (8 keys of one head
//     dim per lane) is two ds_read_b64_tr_b16 transposed reads: within each 16-lane group
//     that instruction hands lane i element k of the 8-byte piece source lane 4k + i/4
//     read, element i%4 of it -- so source lanes pointed at 4 rows x 16 columns give lane
//     i the 4 keys of column i.
// Q, K and V are read from the token-major projection output [b*s, (H + 2 H_kv) d].
// Softmax runs in the exp2 domain. The producer of Q (the QKV GEMM's epilogue or the
// QK-norm kernel) has already multiplied it by log2(e)/sqrt(d) in fp32 before its one
// fp16 rounding, so q . k is the score in the log2 domain; ALiBi adds
// slope*log2(e)*(j - i). Without ALiBi each score accumulator starts at minus the running
// max (a register tile kept at that value is the first MFMA's C operand), so the score
// MFMAs hand exp2 its argument directly; only a step that moves the running max
// subtracts the difference from its scores. P is rounded to fp16 (round to nearest even)
// for the PV product; the row sum adds those fp16 values in fp32 in each lane (its 32 keys
// of a tile, two per v_dot2_f32_f16) and the two lanes of a query once at the end, so
// numerator and denominator take the same probabilities.
// The running max moves (and the output is rescaled) only when some query's tile max
// exceeds it by more than RESCALE_MARGIN in the log2 domain: against a stale max the
// probabilities are at most 2^RESCALE_MARGIN, well inside fp16, and softmax does not
// depend on the shift as long as numerator and denominator use the same one.
//
// Work order: query blocks are issued latest (longest key range) first. Launches with at
// most one 8-wave block of 256 queries per CU (one 2048-token row, short sequences) run
// blocks of 128 queries whose waves split each query's key range in two (KSPLIT below),
// so the longest wave walks half the key tiles.
#include "tf_internal.h"

namespace tfp {

namespace {

constexpr int KT = 64;  // keys per tile
constexpr float RESCALE_MARGIN = 8.0f;
typedef __attribute__((address_space(3))) void* lds_ptr;
typedef short s16x4 __attribute__((ext_vector_type(4)));

// s_waitcnt vmcnt(N) (gfx9 encoding; expcnt, lgkmcnt left at their maxima).
template <int N>
__device__ __forceinline__ void wait_vmcnt() {
  static_assert(N >= 0 && N < 64, "vmcnt range");
  __builtin_amdgcn_s_waitcnt((N & 15) | ((N >> 4) << 14) | (7 << 4) | (15 << 8));
}
// s_waitcnt lgkmcnt(0).
__device__ __forceinline__ void wait_lgkmcnt0() {
  __builtin_amdgcn_s_waitcnt(15 | (3 << 14) | (7 << 4));
}
#ifndef ATTN_NW
#define ATTN_NW 8
#endif
#ifndef ATTN_NSTG
#define ATTN_NSTG 4
#endif

__device__ __forceinline__ f32x16 mfma32(f16x8 a, f16x8 b, f32x16 c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_f16(a, b, c, 0, 0, 0);
}

// A d = 64 block is held to 128 VGPRs, so two blocks (four waves per SIMD) share a CU
// and hide each other's latency (measured 20 % faster than two waves per SIMD with the
// next tile's score MFMAs issued ahead of the softmax). d = 128 runs one block per CU
// (its four K/V stages take 128 KB of LDS).
// KSPLIT (launches with at most one block per CU): the waves split each query's key range
// in two. Waves 0..NW/2-1 take the first half of the block's key tiles and the others the
// second half, over the same NW/2 column blocks of 32 queries; every step loads one tile
// of each half, and at the end each second-half wave hands its running max, row sum and
// output accumulator to its first-half partner through LDS, which merges them (the usual
// rescale by 2^(m_half - m)). The longest wave then walks half the key tiles.
template <int D, int NW, bool ALIBI, bool KMASK, bool KSPLIT>
__global__ void __launch_bounds__(NW * 64)
__attribute__((amdgpu_waves_per_eu(D == 64 && !KSPLIT ? 4 : 1)))
attn_kernel(const AttnArgs g) {
  constexpr int NT = NW * 64;
  constexpr int QW = 32;          // queries per wave: one 32-query column block
  constexpr int NQC = KSPLIT ? NW / 2 : NW;  // 32-query column blocks per block
  constexpr int QB = NQC * QW;    // queries per block
  constexpr int DS = D / 16;      // k-steps of the S^T product
  constexpr int DB = D / 32;      // 32-row d blocks of O^T
  constexpr int DCH = D / 8;      // 16-byte chunks per K / V row
  constexpr int KSTAGE = KT * D, VSTAGE = KT * D;
  constexpr int LT = 2 * KT * DCH / NT;    // global_load_lds per thread per tile (K and V)
  static_assert(KT * DCH % NT == 0, "K and V tiles split evenly over the block");
  static_assert(KT * DCH % 64 == 0, "a wave's 64 load slots lie in one of K or V");
  constexpr int OPITCH = D + 8;            // output staging row pitch (halfs)
  constexpr int NSTG = ATTN_NSTG;          // K / V tile stages in LDS
  static_assert(NSTG >= 3, "tiles t and t+1 are read while later ones load");
  constexpr int NHALF = KSPLIT ? 2 : 1;    // K/V tiles per stage (one per key half)
  constexpr int TSTAGE = KSTAGE + VSTAGE;  // one K/V tile (halfs)
  constexpr int LTS = NHALF * LT;          // global_load_lds per thread per step
  static_assert(!KSPLIT || NW % 2 == 0, "key halves take half the waves each");
  // merge (KSPLIT): after the output staging, per second-half wave 64 lanes x (max, sum,
  // 16 DB accumulator values) floats
  constexpr int MFLT = 2 + 16 * DB;
  constexpr int EPIH = QB * OPITCH + (KSPLIT ? NQC * 64 * MFLT * 2 : 0);
  constexpr int SMEM = NSTG * NHALF * TSTAGE > EPIH ? NSTG * NHALF * TSTAGE : EPIH;
  __shared__ __attribute__((aligned(16))) f16 smem[SMEM];

  const int seq = g.seq, H = g.n_heads, BH = g.batch * g.n_heads;
  const int hd = H * D, kvd = g.n_kv_heads * D, ld = hd + 2 * kvd;
  const int nqblk = (seq + QB - 1) / QB;
  const int qblk = nqblk - 1 - (int)(blockIdx.x / BH);
  const int bh = blockIdx.x % BH;
  const int bi = bh / H, a = bh - bi * H;
  const int q0 = qblk * QB;
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int wc = KSPLIT ? wave % NQC : wave;  // this wave's query column block
  const int kh = KSPLIT ? wave / NQC : 0;     // and key half
  const int qw0 = q0 + wc * QW;
  const int l32 = lane & 31, hi = lane >> 5;
  const int qi = qw0 + l32;  // this lane's query

  // grouped heads: H / Hkv consecutive query heads read one key/value head
  const int kvh = a / (H / g.n_kv_heads);
  const f16* base = g.qkv + (size_t)bi * seq * ld;
  const f16* Qh = base + a * D;
  const f16* Kh = base + hd + kvh * D;  // V of the head follows K by kvd columns

  // Q fragments (B operand of S^T = K Q^T): lane holds Q[qi][16ks + 8hi .. +7], already
  // scaled to the log2 domain
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
  // Running max of this query's scores (log2 domain, scale applied; may lag the true max
  // by up to RESCALE_MARGIN), this lane's share of the row sum (lane ^ 32 holds the other
  // keys of the query), and minus offset() (below) in every register.
  float mrow = -INFINITY;
  float lsum = 0.f;
  constexpr bool KEEP_NEGOFF = !ALIBI && !KMASK;
  f32x16 negoff;
#pragma unroll
  for (int r = 0; r < 16; ++r) negoff[r] = 0.f;
  const float slope = ALIBI ? g.alibi_log2[a] : 0.f;

  const int kv_end = min(seq, q0 + QB);
  const int ntiles = (kv_end + KT - 1) / KT;
  // steps of the tile pipeline: with KSPLIT the first half's tiles 0..nA-1, step t also
  // loading (and the second half computing) tile nA + t
  const int nA = KSPLIT ? (ntiles + 1) / 2 : ntiles;

  // K tile rows are D halfs; 16-byte chunks XOR-swizzled so 16 consecutive rows' 16-byte
  // reads at one logical chunk cover all 64 banks. V tile rows are D halfs with chunks
  // XOR-swizzled by 4 (d = 64: by row pair; d = 128: by row % 4) so the 8 rows x 64 bytes
  // of one transposed read take the minimum two LDS passes.
  auto kx = [](int row) { return D == 64 ? ((row >> 1) & 7) : (row & 15); };
  auto vx = [](int row) { return D == 64 ? 4 * ((row >> 1) & 1) : 4 * (row & 3); };
  auto kswz = [&](int row, int ch) { return row * D + ((ch ^ kx(row)) << 3); };
  // Tile t into stage st: global_load_lds instruction i of wave w deposits lane l's 16
  // bytes at slot w*64 + i*NT + l of the stage (slots [0, KT*DCH) are K, the rest V; the
  // LDS base of an instruction is wave-uniform and the hardware adds 16 bytes per lane),
  // so the swizzle is applied to the global addresses. Keys past the sequence read its
  // last row (finite: their scores are masked, and 0 * V must stay 0).
  // The address is the tile's first K row (wave-uniform) plus a 32-bit per-lane byte
  // offset: row part (clamped to the last key only in a tail tile) and chunk part.
  auto issue_tile = [&](int t, f16* d) {
    const char* tile = reinterpret_cast<const char*>(Kh + (size_t)t * KT * ld);
    const bool tail = t * KT + KT > seq;
    const uint32_t last = (uint32_t)(seq - 1 - t * KT) * (uint32_t)ld * 2u;  // t*KT < seq
#pragma unroll
    for (int i = 0; i < LT; ++i) {
      const int slot0 = wave * 64 + i * NT;            // wave-uniform
      const bool isv = slot0 >= KT * DCH;              // a wave's 64 slots never straddle
      const int sl0 = isv ? slot0 - KT * DCH : slot0;
      const int sl = sl0 + lane;
      const int row = sl / DCH, pch = sl % DCH;
      const int lch = pch ^ (isv ? vx(row) : kx(row));
      const uint32_t orow = (uint32_t)row * (uint32_t)ld * 2u;
      const uint32_t och = (isv ? (uint32_t)kvd * 2u : 0u) + (uint32_t)lch * 16u;
      const uint32_t off = (tail ? min(orow, last) : orow) + och;
      __builtin_amdgcn_global_load_lds((const void*)(tile + off),
                                       (lds_ptr)(d + (isv ? KSTAGE : 0) + sl0 * 8), 16, 0, 0);
    }
  };
  // Step s into stage st: tile s, and with KSPLIT tile nA + s of the second half (past the
  // last tile the last tile again, so every step issues the same number of loads and the
  // vmcnt waits below count whole steps; the second half does not compute on it).
  auto issue = [&](int s, int st) {
    f16* d = smem + st * NHALF * TSTAGE;
    issue_tile(s, d);
    if constexpr (KSPLIT) issue_tile(min(nA + s, ntiles - 1), d + TSTAGE);
  };
  // A operand of O^T = V^T P^T for d-block db and the 16-key group at key kg of the tile:
  // lane (d = 32db + lane%32, g = lane/32) gets keys kg + {4g..4g+3, 8+4g..8+4g+3}.
  auto vfrag = [&](const f16* sv, int db, int kg) {
    const int j = lane & 15, hh = lane >> 5;
    const int dcol = 32 * db + 16 * ((lane >> 4) & 1) + 4 * (j & 3);
    f16x8 out;
#pragma unroll
    for (int c = 0; c < 2; ++c) {
      const int row = kg + 8 * c + 4 * hh + (j >> 2);
      const f16* ptr = sv + row * D + (((dcol >> 3) ^ vx(row)) << 3) + (dcol & 7);
      const s16x4 w = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
          (__attribute__((address_space(3))) s16x4*)(ptr));
      const f16x4 h = __builtin_bit_cast(f16x4, w);
#pragma unroll
      for (int e = 0; e < 4; ++e) out[4 * c + e] = h[e];
    }
    return out;
  };

  // The offset a score accumulator starts at: the running max (0 before the first key and
  // with ALiBi, whose scores are scaled after the MFMAs).
  auto offset = [&]() { return (ALIBI || mrow == -INFINITY) ? 0.f : mrow; };
  // S^T = K Q^T for the tile in LDS stage sk (8 MFMAs at d = 64, 16 at d = 128), each
  // accumulator started at -offset(): from the negoff tile, or (with the padding mask,
  // whose bit tests leave no room for that tile at d = 64) from registers set per tile.
  auto scores = [&](const f16* sk, f32x16 (&sc)[2]) {
    f32x16 start;
    if constexpr (KEEP_NEGOFF) {
      start = negoff;
    } else {
      const float no = ALIBI ? 0.f : -offset();
#pragma unroll
      for (int r = 0; r < 16; ++r) start[r] = no;
    }
#pragma unroll
    for (int kb = 0; kb < 2; ++kb) {
      const int krow = kb * 32 + l32;
#pragma unroll
      for (int ks = 0; ks < DS; ++ks) {
        const f16x8 kf = *reinterpret_cast<const f16x8*>(sk + kswz(krow, 2 * ks + hi));
        sc[kb] = mfma32(kf, qf[ks], ks == 0 ? start : sc[kb]);
      }
    }
  };
  // Online softmax of tile t's scores (started at -off), then O^T += V^T P^T from LDS
  // stage sv.
  auto softmax_pv = [&](f32x16 (&sc)[2], int k0, const f16* sv, float off) {
    // Scores in the log2 domain are t = q.k (+ slope*(key - q)); masked keys -> -inf.
    // Key k0 + 32kb + 8(r/4) + 4hi + r%4 is masked when it exceeds min(q, seq - 1).
    const bool need_mask = (k0 + KT - 1 > qw0) || (k0 + KT > seq);
    const int lim = min(qi, seq - 1) - k0 - 4 * hi;
    // padding keys of this tile (one 64-bit word per 64-key tile, uniform over the block);
    // this lane's keys are bits 32kb + 8(r/4) + 4hi + r%4 of the word, so after one shift
    // by 4hi per key half, bit 8(r/4) + r%4 of kw32[kb] (a compile-time position) is key r
    [[maybe_unused]] uint64_t kw = ~0ull;
    if constexpr (KMASK) kw = g.key_bits[(size_t)bi * g.key_words + k0 / KT];
    [[maybe_unused]] const uint32_t kw32[2] = {(uint32_t)(kw >> (4 * hi)),
                                               (uint32_t)(kw >> (32 + 4 * hi))};
    auto padded = [&](int kb, int r) {
      return ((kw32[kb] >> (8 * (r >> 2) + (r & 3))) & 1u) == 0;
    };
    float mx = -INFINITY;
    if constexpr (ALIBI) {
#pragma unroll
      for (int kb = 0; kb < 2; ++kb)
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const int kr = 32 * kb + 8 * (r >> 2) + (r & 3);
          const int key = k0 + kr + 4 * hi;
          float x = sc[kb][r] + slope * (float)(key - qi);
          if (need_mask && kr > lim) x = -INFINITY;
          if (KMASK && padded(kb, r)) x = -INFINITY;
          sc[kb][r] = x;
          mx = fmaxf(mx, x);
        }
    } else {
      if (need_mask) {
#pragma unroll
        for (int kb = 0; kb < 2; ++kb)
#pragma unroll
          for (int r = 0; r < 16; ++r)
            if (32 * kb + 8 * (r >> 2) + (r & 3) > lim) sc[kb][r] = -INFINITY;
      }
      if constexpr (KMASK) {
        if (kw != ~0ull) {  // uniform: a tile without padding keys skips the tests
#pragma unroll
          for (int kb = 0; kb < 2; ++kb)
#pragma unroll
            for (int r = 0; r < 16; ++r)
              if (padded(kb, r)) sc[kb][r] = -INFINITY;
        }
      }
#pragma unroll
      for (int kb = 0; kb < 2; ++kb)
#pragma unroll
        for (int r = 0; r < 16; ++r) mx = fmaxf(mx, sc[kb][r]);
      mx += off;  // max of the scaled scores
    }
    {  // combine the two key halves of each query (lanes l and l ^ 32) in registers
      const auto sw = __builtin_amdgcn_permlane32_swap(__float_as_uint(mx), __float_as_uint(mx),
                                                       false, false);
      mx = fmaxf(__uint_as_float(sw[0]), __uint_as_float(sw[1]));
    }
    // Move the running max (and rescale) only when some query's max grew by more than
    // the margin; the first tile always moves it from -inf.
    if (__any(mx > mrow + RESCALE_MARGIN)) {
      const float mnew = fmaxf(mrow, mx);
      // 0 on a query's first tile with a key; a query with no key yet (padding) stays at
      // -inf with nothing accumulated
      const float alpha = (KMASK && mnew == -INFINITY) ? 1.f
                                                       : __builtin_amdgcn_exp2f(mrow - mnew);
      lsum *= alpha;
#pragma unroll
      for (int db = 0; db < DB; ++db)
#pragma unroll
        for (int r = 0; r < 16; ++r) o[db][r] *= alpha;
      mrow = mnew;
      if constexpr (KEEP_NEGOFF) {
        const float no = -offset();
#pragma unroll
        for (int r = 0; r < 16; ++r) negoff[r] = no;
      }
    }
    // finite once a query has had a key (without padding, key 0 is in its first tile); a
    // query that has none so far sees only -inf scores, and exp2(-inf - 0) = 0
    const float muse = (KMASK && mrow == -INFINITY) ? 0.f : mrow;
    // exp2 argument t - muse = (score - off) - (muse - off); the difference is 0 unless
    // this step moved the running max (or, with ALiBi, off = 0)
    const float dlt = muse - off;
    if (ALIBI || __any(dlt != 0.f)) {
#pragma unroll
      for (int kb = 0; kb < 2; ++kb)
#pragma unroll
        for (int r = 0; r < 16; ++r) sc[kb][r] -= dlt;
    }
    f16x8 pf[2][2];
#pragma unroll
    for (int kb = 0; kb < 2; ++kb)
#pragma unroll
      for (int r = 0; r < 16; ++r) pf[kb][r >> 3][r & 7] = (f16)__builtin_amdgcn_exp2f(sc[kb][r]);
    // row sum of the fp16 probabilities the PV product takes, accumulated in fp32, two per
    // v_dot2_f32_f16 against (1, 1)
    const f16x2 one2 = {1, 1};
    float ps[2] = {0.f, 0.f};
#pragma unroll
    for (int kb = 0; kb < 2; ++kb)
#pragma unroll
      for (int hs = 0; hs < 2; ++hs)
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const f16x2 pr = {pf[kb][hs][2 * e], pf[kb][hs][2 * e + 1]};
          ps[e & 1] = __builtin_amdgcn_fdot2(pr, one2, ps[e & 1], false);
        }
    lsum += ps[0] + ps[1];
#pragma unroll
    for (int kb = 0; kb < 2; ++kb)
#pragma unroll
      for (int hs = 0; hs < 2; ++hs)
#pragma unroll
        for (int db = 0; db < DB; ++db)
          o[db] = mfma32(vfrag(sv, db, 32 * kb + 16 * hs), pf[kb][hs], o[db]);
  };
  auto stage_k = [&](int t) { return smem + (t % NSTG) * NHALF * TSTAGE + kh * TSTAGE; };
  auto needs = [&](int t) { return t * KT <= qw0 + QW - 1; };  // wave sees a key of tile t
  // this wave's tile at pipeline step t (KSPLIT: the second half's waves run tile nA + t),
  // and whether the wave computes on it
  auto tile_at = [&](int t) { return KSPLIT && kh ? nA + t : t; };
  auto works = [&](int t) { return t < nA && tile_at(t) < ntiles && needs(tile_at(t)); };

  // Pipeline over key tiles: step t issues tile t+NSTG-1 into the stage tile t-1 used,
  // and ends with tile t+2 landed (tiles t+3.. may still fly), so every load has
  // NSTG-2 steps to arrive.
  constexpr int AHEAD = NSTG - 1;  // tiles in LDS or in flight ahead of the current one
#pragma unroll
  for (int t = 0; t < AHEAD; ++t)
    if (t < nA) issue(t, t);
  if (nA >= AHEAD) wait_vmcnt<(NSTG - 3) * LTS>(); else wait_vmcnt<0>();
  __syncthreads();
  // d = 128 (two waves per SIMD, one block per CU): each wave issues the score MFMAs of
  // step t+1 (landed at the end of step t-1) before the softmax of step t, so its own
  // matrix-core work overlaps its VALU work. d = 64 relies on the other block's waves (and
  // with KSPLIT, at two waves per SIMD, the look-ahead measured no faster).
  constexpr bool LOOK = D == 128;
  f32x16 sA[2], sB[2];
  float oA = 0.f, oB = 0.f;  // offsets sA and sB were started at
  if (LOOK && works(0)) scores(stage_k(0), sA);
  auto step = [&](int t, f32x16 (&cur)[2], f32x16 (&nxt)[2], float& ocur, float& onxt) {
    const bool more = t + AHEAD < nA;
    if (more) issue(t + AHEAD, (t + AHEAD) % NSTG);
    if constexpr (LOOK) {
      if (works(t + 1)) {
        onxt = offset();
        scores(stage_k(t + 1), nxt);
      }
      if (works(t)) softmax_pv(cur, tile_at(t) * KT, stage_k(t) + KSTAGE, ocur);
    } else {
      if (works(t)) {
        ocur = offset();
        scores(stage_k(t), cur);
        softmax_pv(cur, tile_at(t) * KT, stage_k(t) + KSTAGE, ocur);
      }
    }
    // tile t+2 landed (later ones may still fly; with nothing issued this step the count
    // is unknown, so wait for all); this wave's LDS reads of tile t's stage are complete
    // before the barrier (the stage is refilled through the memory path)
    if (more) wait_vmcnt<(NSTG - 3) * LTS>(); else wait_vmcnt<0>();
    wait_lgkmcnt0();
    __syncthreads();
  };
  for (int t = 0; t < nA; t += 2) {
    step(t, sA, sB, oA, oB);
    if (t + 1 < nA) step(t + 1, sB, sA, oB, oA);
  }

  if constexpr (KSPLIT) {
    // every load has landed and every K/V read is done (the last step waited for all and
    // joined the barrier): the second-half wave of each column block parks its state
    // after the output staging area, lane-major, and the first-half wave merges it
    float* mg = reinterpret_cast<float*>(smem + QB * OPITCH) + wc * 64 * MFLT;
    if (kh == 1) {
      mg[lane] = mrow;
      mg[64 + lane] = lsum;
#pragma unroll
      for (int db = 0; db < DB; ++db)
#pragma unroll
        for (int r = 0; r < 16; ++r) mg[(2 + 16 * db + r) * 64 + lane] = o[db][r];
    }
    __syncthreads();
    if (kh == 0) {
      const float mb = mg[lane], lb = mg[64 + lane];
      const float m = fmaxf(mrow, mb);
      // a half that saw no key of this query (max -inf) contributes nothing
      const float sa = mrow == -INFINITY ? 0.f : __builtin_amdgcn_exp2f(mrow - m);
      const float sb = mb == -INFINITY ? 0.f : __builtin_amdgcn_exp2f(mb - m);
      lsum = lsum * sa + lb * sb;
#pragma unroll
      for (int db = 0; db < DB; ++db)
#pragma unroll
        for (int r = 0; r < 16; ++r)
          o[db][r] = o[db][r] * sa + mg[(2 + 16 * db + r) * 64 + lane] * sb;
    }
  }

  // Normalise and stage O[q][d] in LDS, then write 16-byte row segments.
  // O^T accumulator db register r: d = 32db + 8(r/4) + 4hi + r%4, query l32 of the wave.
  // a query that never had a key (padding before the row's first token) outputs zero
  const float tot = lsum + __shfl_xor(lsum, 32);
  const float inv = (KMASK && !(tot > 0.f)) ? 0.f : 1.0f / tot;
  if (!KSPLIT || kh == 0) {  // (KSPLIT: the merged first-half waves)
    f16* so = smem + (wc * QW + l32) * OPITCH;
#pragma unroll
    for (int db = 0; db < DB; ++db)
#pragma unroll
      for (int r4 = 0; r4 < 16; r4 += 4) {
        const int d0 = 32 * db + 8 * (r4 >> 2) + 4 * hi;
        f16x4 pk = {(f16)(o[db][r4] * inv), (f16)(o[db][r4 + 1] * inv),
                    (f16)(o[db][r4 + 2] * inv), (f16)(o[db][r4 + 3] * inv)};
        *reinterpret_cast<f16x4*>(so + d0) = pk;
      }
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

template <int D, int NW, bool KSPLIT>
hipError_t launch_t(const AttnArgs& a, hipStream_t st) {
  constexpr int QB = (KSPLIT ? NW / 2 : NW) * 32;
  const int nqblk = (a.seq + QB - 1) / QB;
  const dim3 grid(nqblk * a.batch * a.n_heads), block(NW * 64);
  if (a.key_bits) {
    if (a.alibi_log2) hipLaunchKernelGGL((attn_kernel<D, NW, true, true, KSPLIT>), grid, block, 0, st, a);
    else hipLaunchKernelGGL((attn_kernel<D, NW, false, true, KSPLIT>), grid, block, 0, st, a);
  } else {
    if (a.alibi_log2) hipLaunchKernelGGL((attn_kernel<D, NW, true, false, KSPLIT>), grid, block, 0, st, a);
    else hipLaunchKernelGGL((attn_kernel<D, NW, false, false, KSPLIT>), grid, block, 0, st, a);
  }
  return hipGetLastError();
}

}  // namespace

hipError_t launch_attention(const AttnArgs& a, hipStream_t st) {
  if (a.batch <= 0 || a.seq <= 0) return hipSuccess;
  if (a.n_kv_heads <= 0 || a.n_heads % a.n_kv_heads) return hipErrorInvalidValue;
  if (a.key_bits && a.key_words != (a.seq + 63) / 64) return hipErrorInvalidValue;
  if (a.head_dim == 64) {
    // at most one 8-wave block of 256 queries per CU of a 256-CU MI355X (one 2048-token
    // row, or a short sequence): the split key range halves the longest wave's walk
    const int blocks = (a.seq + 8 * 32 - 1) / (8 * 32) * a.batch * a.n_heads;
    if (blocks <= 256) return launch_t<64, 8, true>(a, st);
    return launch_t<64, ATTN_NW, false>(a, st);
  }
  if (a.head_dim == 128) return launch_t<128, ATTN_NW, false>(a, st);
  return hipErrorInvalidValue;
}

}  // namespace tfp
