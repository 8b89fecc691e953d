// fp16 MFMA GEMM kernel template for gfx950 with fused epilogues.
//
//   C[m, n] = sum_k A[m, k] * B[n, k]
//
// A is the activation matrix [M, K] (row-major, K contiguous). B is a weight [Npad, K]
// (nn.Linear's [out, in], rows zero-padded to a multiple of 256) stored by the packer in
// MFMA fragment order: the 32-row x 16-k block (rb, ks) is 1 KB at byte offset
// (rb * K/16 + ks) * 1024, lane l's 16 bytes holding row 32 rb + l % 32, k 16 ks + 8 (l / 32)
// .. +7 -- exactly what lane l feeds one v_mfma_f32_32x32x16_f16. A fragment is thus one
// fully contiguous 1 KB global_load_lds, and its LDS copy is read back conflict-free at
// lane * 16 bytes.
//
// Structure:
//   - block tile BM x BN, k-tile 64; waves tile the block as (BM/WM) x (BN/WN); each wave
//     owns a WM x WN sub-tile made of 32x32 accumulators (v_mfma_f32_32x32x16_f16, fp32
//     accumulation);
//   - two LDS stages, one barrier per k-tile: the loads of tile k+1 are in flight while
//     tile k is multiplied. Loads go straight from global memory into LDS
//     (global_load_lds_dwordx4: each lane of a load instruction deposits its 16 bytes at
//     LDS slot base + lane, so the permutation that builds the swizzled A layout is applied
//     to the global addresses instead; a B fragment arrives whole, in fragment order);
//   - A's LDS rows are 128 bytes (64 halfs) with XOR-swizzled 16-byte chunks, so the
//     fragment reads of 16 consecutive rows cover all 64 banks;
//   - block ids are remapped so that the tiles of one XCD (block id % 8 on MI355X's
//     round-robin dispatch) form a contiguous, grouped region of the output: blocks
//     sharing A rows / B rows then share that XCD's L2.
//
// Rows of A beyond M are read from row M-1 (never out of bounds) and not stored.
#pragma once
#include <atomic>

#include "tf_internal.h"

namespace tfp {
namespace gemm {

constexpr int GROUP_M = 4;
#ifndef GEMM_EARLY  // 0: the next tile's first k-tile is always loaded from the epilogue
#define GEMM_EARLY 1
#endif

typedef __attribute__((address_space(3))) void* lds_ptr;

__device__ __forceinline__ f32x16 mfma32(f16x8 a, f16x8 b, f32x16 c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_f16(a, b, c, 0, 0, 0);
}

// One accumulator element read out of its AGPR at the point of use. With 256
// accumulators per lane (one wave per SIMD) they live in AGPRs; read through plain code,
// the compiler copies all of them into VGPRs at once when the main loop ends, which needs
// more VGPRs than exist.
__device__ __forceinline__ float rd_acc(float a) {
  float v;
  asm volatile("v_accvgpr_read_b32 %0, %1" : "=v"(v) : "a"(a));
  return v;
}

// s_waitcnt vmcnt(N) (gfx9 encoding: vmcnt bits [3:0] and [15:14]; expcnt, lgkmcnt left
// at their maxima so they are not waited for).
template <int N>
__device__ __forceinline__ void wait_vmcnt() {
  static_assert(N >= 0 && N < 64, "vmcnt range");
  __builtin_amdgcn_s_waitcnt((N & 15) | ((N >> 4) << 14) | (7 << 4) | (15 << 8));
}

// s_waitcnt lgkmcnt(0) (vmcnt and expcnt left at their maxima).
__device__ __forceinline__ void wait_lgkmcnt0() {
  __builtin_amdgcn_s_waitcnt((15) | (3 << 14) | (7 << 4) | (0 << 8));
}

// SiLU g * sigmoid(g); the reciprocal is the hardware one (about 1 ulp), far below the
// fp16 rounding of the result.
__device__ __forceinline__ float silu_f(float g) {
  return g * __builtin_amdgcn_rcpf(1.0f + __expf(-g));
}

__device__ __forceinline__ float gelu_tanh_f(float v) {
  // 0.5 v (1 + tanh(sqrt(2/pi) (v + 0.044715 v^3))), tanh(y) = 1 - 2 / (e^{2y} + 1)
  const float y = 0.7978845608028654f * (v + 0.044715f * v * v * v);
  const float t = 1.0f - 2.0f * __builtin_amdgcn_rcpf(__expf(2.0f * y) + 1.0f);
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
  static constexpr int FPT = BK / 16;   // B fragments per 32-row block and k-tile
  // global_load_lds instructions per wave per k-tile (each fills 64 16-byte slots): A rows,
  // and one whole B fragment each
  static constexpr int LA = BM * CPR / 64 / NW, LB = (BN / 32) * FPT / NW;
  static constexpr int LPT = LA + LB;
  static constexpr int STAGE = (BM + BN) * BK;  // halfs per LDS stage
  // Output staging (after the main loop, above stage 0, which by then loads the next
  // tile), in passes of whole 32-row blocks: fp16 in two passes of BM/2 rows (pitch BN+8),
  // the SwiGLU output (BN/2 columns) in one pass, fp32 in passes of BM/4 rows (pitch BN+4).
  static constexpr int R16 = BM / 2 >= 32 ? BM / 2 : 32;
  static constexpr int RSW = BM;
  static constexpr int R32 = BM / 4 >= 32 ? BM / 4 : 32;
  static constexpr int S16 = R16 * (BN + 8), SSW = RSW * (BN / 2 + 8), S32 = R32 * (BN + 4) * 2;
  static constexpr int SOUT = S16 > SSW ? (S16 > S32 ? S16 : S32) : (SSW > S32 ? SSW : S32);
  static constexpr int SMEM_HALFS = NS * STAGE > STAGE + SOUT ? NS * STAGE : STAGE + SOUT;
  // Persistent (one block per CU looping over tiles, the next tile's loads overlapping
  // this tile's epilogue) when the LDS admits only one block per CU anyway; smaller tiles
  // run one tile per block and overlap across co-resident blocks instead.
  static constexpr bool PERSIST = SMEM_HALFS * 2 > 80 * 1024;
  static_assert(LA * 64 * NW == BM * CPR && LB * NW == (BN / 32) * FPT, "load split");
  static_assert(BK == 32 || BK == 64, "k-tile");
  static_assert(NS >= 2 && (NS - 2) * LPT < 64, "stages");
  static_assert(WN % 64 == 0, "epilogues need 64-column aligned wave tiles");
  // A tile: halfs offset of 16-byte chunk `chunk` of tile row `row`: chunks are XOR-swizzled by
  // the index of the row's 256-byte line, so the 16-byte reads of 16 consecutive rows at
  // one logical chunk (one 16-lane group of a ds_read_b128) cover all 64 banks once
  static __device__ __forceinline__ int swz(int row, int chunk) {
    return row * BK + ((chunk ^ ((row / RPL) % CPR)) << 3);
  }
};

template <class C, int EPI, int RH>
__global__ void __launch_bounds__(C::NT)
gemm_kernel(const GemmArgs g) {
  constexpr int BM = C::BM, BN = C::BN, WM = C::WM, WN = C::WN, BK = C::BK, NS = C::NS;
  // Epilogue operands of the tile in flight, deposited by global_load_lds when the tile's
  // first loads are issued (so they hold no registers and have landed by the epilogue):
  // the bias of the tile's BN columns, and for the rotary epilogue with at most 8
  // frequencies the cos and sin rows of the tile's BM positions ([BM][RLD] each). They
  // sit at the end of the one LDS array (a second __shared__ object that DMA writes into
  // makes the compiler wait for every DMA before each LDS read in the main loop).
  // (with the per-head LayerNorm, also the gains of the tile's BN columns)
  constexpr bool HAS_BIAS = EPI != EPI_SWIGLU;
  constexpr bool HLN = EPI == EPI_QKV_HLN_ROPE;
  constexpr bool QKV = EPI == EPI_QKV_ROPE || HLN;
  constexpr bool ROPE = QKV && RH > 0;
  constexpr bool ROPE_LDS = ROPE && RH <= 8;
  constexpr int RLD = RH > 4 ? 8 : 4;  // the table's row length (frequencies rounded up to 4)
  constexpr int XOP = (HAS_BIAS ? BN : 0) + (ROPE_LDS ? 2 * BM * RLD : 0) + (HLN ? BN : 0);  // floats
  static_assert(!HLN || WN == 64, "the per-head LayerNorm needs one 64-column head per wave tile");
  __shared__ __attribute__((aligned(16))) f16 smem[C::SMEM_HALFS + 2 * XOP];
  float* const xop = reinterpret_cast<float*>(smem + C::SMEM_HALFS);
  [[maybe_unused]] float* const bias_lds = xop;
  [[maybe_unused]] float* const cos_lds = xop + (HAS_BIAS ? BN : 0);
  [[maybe_unused]] float* const sin_lds = cos_lds + BM * RLD;
  [[maybe_unused]] float* const gain_lds = cos_lds + (ROPE_LDS ? 2 * BM * RLD : 0);

  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);  // wave-uniform (SGPR)
  const int wm = wave / C::NWN, wn = wave % C::NWN;
  const int nbm = (g.M + BM - 1) / BM, nbn = g.Npad / BN;
  const int ntiles = nbm * nbn;
  // Split-K (one-tile-per-block launches only): blockIdx.y takes k-tiles
  // [y KT, (y+1) KT) and writes its fp32 partial at out32 + y * split_stride.
  const int KT = g.K / BK / (int)gridDim.y;
  const int kbase = (int)blockIdx.y * KT * BK;
  float* const out32 = g.out32 ? g.out32 + (size_t)blockIdx.y * g.split_stride : nullptr;

  // Persistent blocks: block b takes virtual tiles v = b, b + G, b + 2G, ... (G = grid
  // size, a multiple of 8 whenever G < ntiles). Virtual tile v is mapped as a block id of
  // a one-tile-per-block launch would be: v runs on XCD v % 8 (MI355X dispatches block ids
  // round-robin over its 8 XCDs), each XCD gets a contiguous range of tiles, and inside
  // the range GROUP_M tile-rows sweep the tile-columns together, so the tiles an XCD runs
  // at one time share A rows and B rows in its L2.
  auto tile_of = [&](int v, int& m0, int& n0) {
    const int q = ntiles >> 3, r = ntiles & 7, x = v & 7, loc = v >> 3;
    const int tile = (x < r) ? x * (q + 1) + loc : r * (q + 1) + (x - r) * q + loc;
    const int per_group = GROUP_M * nbn;
    const int first_m = (tile / per_group) * GROUP_M;
    const int gm = min(nbm - first_m, GROUP_M);
    m0 = (first_m + (tile % per_group) % gm) * BM;
    n0 = ((tile % per_group) / gm) * BN;
  };

  // Load assignment: global_load_lds instruction i of wave w deposits lane l's 16 bytes
  // at LDS slot (w*L + i)*64 + l; slot s of the A (B) region holds tile row s / CPR,
  // logical chunk (s % CPR) ^ ((row / RPL) % CPR) -- i.e. exactly C::swz's layout.
  // Global offsets are 32-bit byte offsets from the (uniform) operand base, so the loads
  // use the scalar-base + 32-bit-offset address form (half the per-lane address data of
  // a 64-bit address).
  // B fragments: DMA instruction i of wave w moves fragment f = w * LB + i of the tile
  // (32-row block f / FPT, k-step f % FPT), 1 KB contiguous in global memory and in LDS.
  const int KSt = g.K / 16;  // k-steps of the whole matrix (fragment pitch of a row block)
  uint32_t goa[C::LA], gob[C::LB];
  int loa[C::LA], lob[C::LB];
#pragma unroll
  for (int i = 0; i < C::LA; ++i) loa[i] = (wave * C::LA + i) * 512;
#pragma unroll
  for (int i = 0; i < C::LB; ++i) lob[i] = BM * BK + (wave * C::LB + i) * 512;
  auto set_offsets = [&](int m0, int n0) {
#pragma unroll
    for (int i = 0; i < C::LA; ++i) {
      const int s = (wave * C::LA + i) * 64 + lane;
      const int row = s / C::CPR, ch = (s % C::CPR) ^ ((row / C::RPL) % C::CPR);
      goa[i] = (uint32_t)(min(m0 + row, g.M - 1) * g.lda + ch * 8) * 2u;
    }
#pragma unroll
    for (int i = 0; i < C::LB; ++i) {
      const int f = wave * C::LB + i;
      gob[i] = (uint32_t)((n0 / 32 + f / C::FPT) * KSt + f % C::FPT) * 1024u + lane * 16u;
    }
  };

  const int frow = lane & 31, fch = lane >> 5;
  // Fragments of k-step kk (16 k) from LDS stage s.
  auto frag_a = [&](const f16* s, int kk, int i) {
    return *reinterpret_cast<const f16x8*>(s + C::swz(wm * WM + i * 32 + frow, kk * 2 + fch));
  };
  auto frag_b = [&](const f16* s, int kk, int j) {
    return *reinterpret_cast<const f16x8*>(
        s + BM * BK + (((wn * WN) / 32 + j) * C::FPT + kk) * 512 + lane * 8);
  };

  auto load_one = [&](f16* d, int ko, int li) {
    if (li < C::LA)
      __builtin_amdgcn_global_load_lds((const void*)(reinterpret_cast<const char*>(g.A + kbase + ko) + goa[li]),
                                       (lds_ptr)(d + loa[li]), 16, 0, 0);
    else
      __builtin_amdgcn_global_load_lds((const void*)(reinterpret_cast<const char*>(g.B) +
                                                     (size_t)(kbase + ko) * 64 + gob[li - C::LA]),
                                       (lds_ptr)(d + lob[li - C::LA]), 16, 0, 0);
  };
  // A stage's refill goes out in two parts: LP1 loads in the last k-step of the tile that
  // frees it, the rest in the first k-step of the next tile (see the main loop). Measured
  // per epilogue: halving it makes the fp32-logits GEMM (lm_head) 2.6-3.4 % faster and
  // the residual-add GEMMs 3-5 % slower, the others unchanged.
  constexpr int LP1 = EPI == EPI_STORE_F32 ? C::LPT / 2 : C::LPT;
  constexpr bool SPLIT = LP1 < C::LPT;
  auto issue = [&](int kt, int stage) {
#pragma unroll
    for (int li = 0; li < C::LPT; ++li) load_one(smem + stage * C::STAGE, kt * BK, li);
  };
  auto issue_part = [&](int kt, int stage, int lb, int le) {
#pragma unroll
    for (int li = 0; li < C::LPT; ++li)
      if (li >= lb && li < le) load_one(smem + stage * C::STAGE, kt * BK, li);
  };
  // Epilogue operands of tile (m0, n0) into xop. Bias: 4-byte deposits, one instruction
  // per 64 columns (columns past N read column N-1: they are never stored). Rotary rows:
  // 16-byte deposits, RLD / 4 per position; rows past M read row M-1. Instruction k goes
  // to wave k % NW; the LDS base of an instruction is wave-uniform and the hardware adds
  // the lane's deposit size.
  auto op_copy = [&](const float* src, float* dst, int bytes) {
    if (bytes == 4) __builtin_amdgcn_global_load_lds((const void*)src, (lds_ptr)dst, 4, 0, 0);
    else __builtin_amdgcn_global_load_lds((const void*)src, (lds_ptr)dst, 16, 0, 0);
  };
  auto issue_ops = [&](int m0, int n0) {
    if constexpr (HAS_BIAS) {
      if (g.bias) {
        for (int k = wave; k < BN / 64; k += C::NW) {
          const int n = min(n0 + k * 64 + lane, g.N - 1);
          op_copy(g.bias + n, bias_lds + k * 64, 4);
        }
      }
    }
    if constexpr (HLN) {
      if (n0 < g.rot_cols) {  // gains of Q / K columns (past them: the last K gain, unused)
        for (int k = wave; k < BN / 64; k += C::NW) {
          const int n = min(n0 + k * 64 + lane, g.rot_cols - 1);
          const float* src = n < g.hln_hd ? g.hln_q + n : g.hln_k + (n - g.hln_hd);
          op_copy(src, gain_lds + k * 64, 4);
        }
      }
    }
    if constexpr (ROPE_LDS) {
      if (n0 < g.rot_cols) {
        constexpr int CPRW = RLD / 4;              // 16-byte chunks per position
        constexpr int NI = BM * CPRW / 64;         // instructions per table
        static_assert(NI * 64 == BM * CPRW, "rotary rows split into whole instructions");
        for (int k = wave; k < 2 * NI; k += C::NW) {
          const int kk = k % NI, c = kk * 64 + lane, r = c / CPRW, sub = c % CPRW;
          const int p = min(m0 + r, g.M - 1) % g.seq;
          const float* src = (k < NI ? g.rope_cos : g.rope_sin) + (size_t)p * RLD + sub * 4;
          float* dst = (k < NI ? cos_lds : sin_lds) + kk * 256;
          op_copy(src, dst, 16);
        }
      }
    }
  };

  f32x16 acc[C::TM][C::TN];
  f16x8 af[2][C::TM], bf[2][C::TN];
  constexpr int KS = BK / 16;  // k-steps per k-tile
  constexpr int NR = C::TM + C::TN, NM = C::TM * C::TN;
  static_assert(KS % 2 == 0, "fragment buffers alternate by k-step parity across k-tiles");
  static_assert(NS == 2 || !C::PERSIST, "the main loop's vmcnt(0) also covers the previous tile's stores");
  auto frags0 = [&](const f16* s) {
#pragma unroll
    for (int j = 0; j < C::TN; ++j) bf[0][j] = frag_b(s, 0, j);
#pragma unroll
    for (int i = 0; i < C::TM; ++i) af[0][i] = frag_a(s, 0, i);
  };
  // One k-step, as NM MFMA slots in a fixed order (i-major). The fragment reads of the
  // next k-step (from stage `rs`, k-step `rkk`, into the other register buffer) take one
  // slot each from slot 0, so every read has at least NM - NR MFMAs to land. On the last
  // k-step of a k-tile the refill loads of the freed stage `ld` take one slot each too:
  // one k-tile's loads keep the CU's address unit busy for a good part of a k-tile, and
  // issued as a burst they stall the issuing waves while their matrix cores idle.
  // sched_barrier pins the order: the compiler would otherwise bunch the loads.
  // (Loads lb .. le-1 of the refill of stage `ld` with k-tile offset `ko`, when `lo`, take
  // one slot each from slot 0.)
  auto kstep = [&](int cur, const f16* rs, int rkk, bool rd, f16* ld, int ko, bool lo,
                   int lb = 0, int le = C::LPT) {
    auto read_ahead = [&](int x) {
      if (x < C::TN) bf[cur ^ 1][x] = frag_b(rs, rkk, x);
      else af[cur ^ 1][x - C::TN] = frag_a(rs, rkk, x - C::TN);
    };
#pragma unroll
    for (int x = 0; x < NM; ++x) {
      const int i = x / C::TN, j = x % C::TN;
      acc[i][j] = mfma32(bf[cur][j], af[cur][i], acc[i][j]);  // block transposed
      if (rd && x < NR) read_ahead(x);
      if (lo && x < le - lb) load_one(ld, ko, lb + x);
      __builtin_amdgcn_sched_barrier(0);
    }
#pragma unroll
    for (int x = NM; x < NR; ++x)
      if (rd) read_ahead(x);
#pragma unroll
    for (int x = NM; x < C::LPT; ++x)
      if (lo && x < le - lb) load_one(ld, ko, lb + x);
  };

  // ------------------------------------------------------------------ epilogue layout
  // The MFMAs produce every 32x32 block transposed (the B fragment is the MFMA's first
  // operand), so accumulator (i, j) register r = 4 g + t of this lane holds tile element
  //   row wm*WM + 32i + lane%32,  column wn*WN + 32j + 8g + 4(lane/32) + t:
  // each register group g is four consecutive columns of one row -- one 8-byte (fp16) or
  // 16-byte (fp32) LDS write when the tile is staged. Values are finished in registers
  // (bias, activation, rotary), staged in LDS in the output type above stage 0 (which by
  // then is already loading the next tile), in passes of PR tile rows, then written out as
  // 16-byte row segments.
  constexpr bool F32OUT = (EPI == EPI_STORE_F32 || EPI == EPI_RESID_ADD);
  // more accumulators than half the VGPRs: one wave per SIMD, accumulators in AGPRs
  constexpr bool AGPR_ACC = C::TM * C::TN * 16 > 128;
  constexpr int OCOLS = EPI == EPI_SWIGLU ? BN / 2 : BN;         // output columns per tile
  constexpr int PR = F32OUT ? C::R32 : EPI == EPI_SWIGLU ? C::RSW : C::R16;  // rows per pass
  constexpr int PASSES = BM / PR;
  constexpr int ESZ = F32OUT ? 4 : 2;
  // staging row pitch (elements): row r starts 4r banks further on (mod 64), so the 32
  // rows x 2 column groups of one LDS write spread evenly over the 64 banks
  constexpr int PITCH = OCOLS + 16 / ESZ;
  static_assert(PR % 32 == 0 && BM % PR == 0, "a pass holds whole 32-row accumulator blocks");
  static_assert(C::STAGE * 2 + PR * PITCH * ESZ <= C::SMEM_HALFS * 2, "staging must fit in LDS");
  const int hi4 = 4 * (lane >> 5), l32 = lane & 31;
  f16* st16 = smem + C::STAGE;
  float* st32 = reinterpret_cast<float*>(smem + C::STAGE);

  const int G = gridDim.x;
  int v = blockIdx.x;
  int m0, n0;
  tile_of(v, m0, n0);
  set_offsets(m0, n0);
  // first tile: its epilogue operands, then all NS stages, start in flight (the operands
  // come first, so every wait for a stage also covers them)
  issue_ops(m0, n0);
  if constexpr (SPLIT) {
    issue(0, 0);
    issue_part(min(1, KT - 1), 1, 0, LP1);  // the rest goes out in the first k-step
    wait_vmcnt<LP1>();
  } else {
#pragma unroll
    for (int st = 0; st < NS; ++st) issue(min(st, KT - 1), st);
    wait_vmcnt<(NS - 1) * C::LPT>();
  }
  __syncthreads();
  frags0(smem);

  for (;;) {
#pragma unroll
    for (int i = 0; i < C::TM; ++i)
#pragma unroll
      for (int j = 0; j < C::TN; ++j)
#pragma unroll
        for (int r = 0; r < 16; ++r) acc[i][j][r] = 0.0f;

    // The next tile (persistent blocks). With an even number of k-tiles its first k-tile
    // is loaded by the refill slots of k-tile KT-2 (which would otherwise reload the last
    // k-tile), into stage 0, which the epilogue leaves alone: it is in flight a k-tile
    // before the epilogue begins instead of from the epilogue's start.
    const int vn = v + G;
    const bool has_next = C::PERSIST && vn < ntiles;
    int m0n = 0, n0n = 0;
    if (has_next) tile_of(vn, m0n, n0n);
    const bool early = GEMM_EARLY && !SPLIT && has_next && KT % 2 == 0;

    // Main loop. Before the last k-step of k-tile kt the wave waits for tile kt+1 and
    // joins the barrier, which frees tile kt's stage (the explicit lgkmcnt wait completes
    // this wave's reads of it first: the refill writes it through the memory path, which
    // is not ordered with LDS reads); the last k-step reads tile kt+1's first fragments
    // and refills the freed stage with tile kt+NS (SPLIT: only its first LP1 loads; the
    // others go out in the first k-step of tile kt+1, as the stage stays free until tile
    // kt+1's barrier). The refill is unconditional (past the end it reloads the last tile
    // into a stage that is never read again), which keeps the loop body free of branches.
    static_assert(!SPLIT || NS == 2, "a split refill spans the next tile's first k-step");
    for (int kt = 0; kt < KT - 1; ++kt) {
      const f16* s = smem + (kt % NS) * C::STAGE;
      if constexpr (SPLIT) {
        kstep(0, s, 1, true, smem + ((kt + 1) % NS) * C::STAGE, min(kt + 1, KT - 1) * BK,
              true, LP1, C::LPT);
#pragma unroll
        for (int kk = 1; kk < KS - 1; ++kk) kstep(kk & 1, s, kk + 1, true, nullptr, 0, false);
      } else {
#pragma unroll
        for (int kk = 0; kk < KS - 1; ++kk) kstep(kk & 1, s, kk + 1, true, nullptr, 0, false);
      }
      wait_vmcnt<(NS - 2) * C::LPT>();  // tile kt+1 landed (kt+2 .. kt+NS-1 may fly)
      wait_lgkmcnt0();
      __syncthreads();
      const bool nx = early && kt == KT - 2;  // (stage kt % NS is then stage 0)
      if (nx) set_offsets(m0n, n0n);
      kstep((KS - 1) & 1, smem + ((kt + 1) % NS) * C::STAGE, 0, true,
            smem + (kt % NS) * C::STAGE, nx ? 0 : min(kt + NS, KT - 1) * BK, true, 0, LP1);
    }
    {  // last k-tile
      const f16* s = smem + ((KT - 1) % NS) * C::STAGE;
      if constexpr (SPLIT) {
        kstep(0, s, 1, KS > 1, smem + (KT % NS) * C::STAGE, (KT - 1) * BK, true, LP1, C::LPT);
#pragma unroll
        for (int kk = 1; kk < KS; ++kk) kstep(kk & 1, s, kk + 1, kk + 1 < KS, nullptr, 0, false);
      } else {
#pragma unroll
        for (int kk = 0; kk < KS; ++kk) kstep(kk & 1, s, kk + 1, kk + 1 < KS, nullptr, 0, false);
      }
    }
    // the refills past the end land before the stages are reused (early: the only one
    // went to stage 0, which the epilogue does not use; the first pass waits for it)
    if (!early) wait_vmcnt<0>();
    wait_lgkmcnt0();
    __syncthreads();  // every wave is done with the stages

    // ---------------------------------------------------------------- epilogue
    // The copy-out index math starts from an opaque copy of the thread id, so none of it
    // is hoisted above the main loop (where its registers would be live all along).
    int etid = tid;
    asm volatile("" : "+v"(etid));
    // The bias and (up to 8 frequencies) the rotary factors are in LDS already. The first
    // slice of the residual is requested before the next tile's first loads, so its
    // latency overlaps those loads and the staging writes.
    const int ocol0 = EPI == EPI_SWIGLU ? n0 / 2 : n0;               // first output column
    const int ncols = min(OCOLS, g.N - ocol0);                       // valid output columns
    // Rotary factors of a row: NG 16-byte groups of four consecutive frequencies. Spans
    // of at most 8 frequencies read the tile's rows staged in LDS; wider spans load from
    // the position-major table [max_seq][rope_ld] per row block.
    constexpr int NG = RH >= 32 ? 4 : RH >= 16 ? 2 : 1;
    [[maybe_unused]] const bool rq = ROPE && n0 < g.rot_cols;  // tile holds Q or K columns
    auto rope_load = [&](int i, f32x4 (&rc)[NG], f32x4 (&rs)[NG]) {
      const int r = wm * WM + 32 * i + l32;  // tile row
      if constexpr (ROPE_LDS) {
        const int off = RH >= 8 ? hi4 : 0;
        rc[0] = *reinterpret_cast<const f32x4*>(cos_lds + r * RLD + off);
        rs[0] = *reinterpret_cast<const f32x4*>(sin_lds + r * RLD + off);
      } else {
        const int p = min(m0 + r, g.M - 1) % g.seq;
        const float* ct = g.rope_cos + (size_t)p * g.rope_ld;
        const float* sn = g.rope_sin + (size_t)p * g.rope_ld;
#pragma unroll
        for (int q = 0; q < NG; ++q) {
          rc[q] = *reinterpret_cast<const f32x4*>(ct + 8 * q + hi4);
          rs[q] = *reinterpret_cast<const f32x4*>(sn + 8 * q + hi4);
        }
      }
    };
    // Copy-out geometry: 16-byte vectors along rows. A pass is "full" when all its rows
    // and columns are in range and the output rows are 16-byte aligned; a full pass is
    // copied with a fixed number of vectors per thread (NIT), unrolled.
    constexpr int VE = 16 / ESZ;            // elements per vector
    constexpr int VPR = OCOLS / VE;         // vectors per tile row
    constexpr int NIT = PR * VPR / C::NT;
    constexpr bool NIT_OK = NIT * C::NT == PR * VPR;
    const bool vec_ok = ((g.ldo * ESZ) & 15) == 0 &&
        ((reinterpret_cast<uintptr_t>(F32OUT ? (void*)out32 : (void*)g.out16)) & 15) == 0;
    auto full_pass = [&](int pass) {
      return NIT_OK && vec_ok && ncols == OCOLS && m0 + (pass + 1) * PR <= g.M;
    };
    // Full-pass addresses: thread etid's vector u sits in tile row etr + u * TRS, column
    // evc, of the pass. Each address is a wave-uniform base (the row of the pass, its first
    // column) plus this thread's 32-bit byte offset, the same for every u -- so no
    // per-thread 64-bit address stays live across the passes. In the residual epilogue
    // such addresses were spilled, and each reload waited for every store in flight (this
    // form: o / down projections 9 % / 5 % faster). The fp32-logits epilogue keeps one
    // full address per vector, which measured 0.5-1 % faster there.
    constexpr int TRS = C::NT / VPR;
    static_assert(!NIT_OK || TRS * VPR == C::NT, "a thread's vectors share one column");
    const int etr = etid / VPR, evc = (etid % VPR) * VE;
    const uint32_t eoff = (uint32_t)(etr * g.ldo + evc) * (uint32_t)ESZ;
    auto vec_addr = [&](auto* base, int pass, int u) {
      if constexpr (EPI == EPI_STORE_F32) {
        const int e = etid + u * C::NT, tr = e / VPR, vc = (e % VPR) * VE;
        return base + (size_t)(m0 + pass * PR + tr) * g.ldo + ocol0 + vc;
      } else
        return reinterpret_cast<decltype(base)>(
            reinterpret_cast<char*>(base + (size_t)(m0 + pass * PR + u * TRS) * g.ldo + ocol0) + eoff);
    };
    // Residual vectors of a full pass (RESID_ADD): thread tid's vectors u = 0..NIT-1 are
    // element tid + u*NT of the pass, row-major over PR rows x VPR vectors.
    [[maybe_unused]] f32x4 res[EPI == EPI_RESID_ADD && NIT_OK ? NIT : 1];
    auto res_load = [&](int pass) {
      if constexpr (EPI == EPI_RESID_ADD && NIT_OK) {
#pragma unroll
        for (int u = 0; u < NIT; ++u) res[u] = *reinterpret_cast<const f32x4*>(vec_addr(out32, pass, u));
      }
    };
    if (full_pass(0)) res_load(0);

    // Otherwise the next tile's first k-tile goes into stage 0 now, so its load latency
    // hides behind this tile's epilogue.
    if (has_next && !early) {
      set_offsets(m0n, n0n);
      issue(0, 0);
    }

#pragma unroll
    for (int pass = 0; pass < PASSES; ++pass) {
      if (pass > 0) __syncthreads();  // previous pass fully copied out
#pragma unroll
      for (int i = 0; i < C::TM; ++i) {
        if ((wm * WM + 32 * i) / PR != pass) continue;  // wave-uniform
        const int trow = wm * WM + 32 * i - pass * PR + l32;
        // this 32-row block's accumulators, in VGPRs for the epilogue arithmetic
        f32x16 ev[C::TN];
#pragma unroll
        for (int j = 0; j < C::TN; ++j)
#pragma unroll
          for (int r = 0; r < 16; ++r) ev[j][r] = AGPR_ACC ? rd_acc(acc[i][j][r]) : acc[i][j][r];
        if constexpr (EPI == EPI_SWIGLU) {
#pragma unroll
          for (int j = 0; j < C::TN; j += 2)
#pragma unroll
            for (int g4 = 0; g4 < 4; ++g4) {
              f16x4 o;
#pragma unroll
              for (int t = 0; t < 4; ++t)
                o[t] = (f16)(silu_f(ev[j][4 * g4 + t]) * ev[j + 1][4 * g4 + t]);
              const int oc = (wn * WN + 32 * j) / 2 + 8 * g4 + hi4;
              *reinterpret_cast<f16x4*>(st16 + trow * PITCH + oc) = o;
            }
        } else {
          if (g.bias) {
#pragma unroll
            for (int j = 0; j < C::TN; ++j)
#pragma unroll
              for (int g4 = 0; g4 < 4; ++g4) {
                const f32x4 b = *reinterpret_cast<const f32x4*>(bias_lds + wn * WN + 32 * j + 8 * g4 + hi4);
#pragma unroll
                for (int t = 0; t < 4; ++t) ev[j][4 * g4 + t] += b[t];
              }
          }
          // Rotary (QKV epilogue): NeoX halves within each head; dim e < half pairs with
          // e + half at frequency index e, over dims [0, 2 half) of Q and K heads. Every
          // stored group is computed from read-only accumulator values; the partner of an
          // element is, by span: half 1 / 2 -> register t ^ 1 / t ^ 2, half 4 -> the same
          // register of lane ^ 32, half 8 / 16 -> register group g ^ 1 / g ^ 2, half 32 ->
          // block j ^ 1.
          // Per-head LayerNorm (no bias): the wave's 64 columns are one head; a row's 64
          // values are this lane's 32 (blocks j, register groups g) and lane ^ 32's 32.
          // Mean first, then the centred squares; then the gains.
          if constexpr (HLN) {
            if (n0 + wn * WN < g.rot_cols) {  // wave-uniform: a Q or K head
              float sm = 0.f;
#pragma unroll
              for (int j = 0; j < C::TN; ++j)
#pragma unroll
                for (int r = 0; r < 16; ++r) sm += ev[j][r];
              const float mean = (sm + __shfl_xor(sm, 32)) * (1.0f / 64.0f);
              float sq = 0.f;
#pragma unroll
              for (int j = 0; j < C::TN; ++j)
#pragma unroll
                for (int r = 0; r < 16; ++r) {
                  const float dv = ev[j][r] - mean;
                  sq += dv * dv;
                }
              const float rsd = rsqrtf((sq + __shfl_xor(sq, 32)) * (1.0f / 64.0f) + g.hln_eps);
#pragma unroll
              for (int j = 0; j < C::TN; ++j)
#pragma unroll
                for (int g4 = 0; g4 < 4; ++g4) {
                  const f32x4 gw = *reinterpret_cast<const f32x4*>(gain_lds + wn * WN + 32 * j + 8 * g4 + hi4);
#pragma unroll
                  for (int t = 0; t < 4; ++t)
                    ev[j][4 * g4 + t] = (ev[j][4 * g4 + t] - mean) * rsd * gw[t];
                }
            }
          }
          [[maybe_unused]] f32x4 rc[NG], rs[NG];
          if constexpr (ROPE) {
            if (rq) rope_load(i, rc, rs);
          }
#pragma unroll
          for (int j = 0; j < C::TN; ++j) {
            [[maybe_unused]] const int cb = n0 + wn * WN + 32 * j;
            [[maybe_unused]] const int eb = cb % g.head_dim;
            // Q and K end on a head boundary, so a 32-column block lies wholly on one side
            [[maybe_unused]] const bool rj = rq && cb < g.rot_cols;
#pragma unroll
            for (int g4 = 0; g4 < 4; ++g4) {
              f32x4 o;
#pragma unroll
              for (int t = 0; t < 4; ++t) o[t] = ev[j][4 * g4 + t];
              if constexpr (ROPE) {
                // (x, y) pairs: low side x c - y s, high side y c + x s
#pragma unroll
                for (int t = 0; t < 4; ++t) {
                  const float x = ev[j][4 * g4 + t];
                  if constexpr (RH == 32) {
                    if (rj && (j & 1) == 0 && j + 1 < C::TN && eb == 0)
                      o[t] = x * rc[g4][t] - ev[(j + 1) % C::TN][4 * g4 + t] * rs[g4][t];
                    if (rj && (j & 1) == 1 && eb == 32)
                      o[t] = x * rc[g4][t] + ev[j - 1 + ((j & 1) == 0)][4 * g4 + t] * rs[g4][t];
                  } else if constexpr (RH == 16) {
                    if (rj && eb == 0)
                      o[t] = g4 < 2 ? x * rc[g4 & 1][t] - ev[j][4 * (g4 + 2 * (g4 < 2) - 2 * (g4 >= 2) ) + t] * rs[g4 & 1][t]
                                    : x * rc[g4 & 1][t] + ev[j][4 * (g4 - 2 + 4 * (g4 < 2)) + t] * rs[g4 & 1][t];
                  } else if constexpr (RH == 8) {
                    if (rj && eb == 0 && g4 < 2)
                      o[t] = g4 == 0 ? x * rc[0][t] - ev[j][4 + t] * rs[0][t]
                                     : x * rc[0][t] + ev[j][t] * rs[0][t];
                  } else if constexpr (RH == 4) {
                    if (g4 == 0) {
                      const float pv = __shfl_xor(x, 32);  // every lane takes part
                      if (rj && eb == 0)
                        o[t] = hi4 == 0 ? x * rc[0][t] - pv * rs[0][t] : x * rc[0][t] + pv * rs[0][t];
                    }
                  } else if constexpr (RH == 2) {
                    if (rj && eb == 0 && g4 == 0 && hi4 == 0)
                      o[t] = t < 2 ? x * rc[0][t] - ev[j][t + 2] * rs[0][t]
                                   : x * rc[0][t & 1] + ev[j][(t + 2) & 3] * rs[0][t & 1];
                  } else {  // RH == 1
                    if (rj && eb == 0 && g4 == 0 && hi4 == 0 && t < 2)
                      o[t] = t == 0 ? x * rc[0][0] - ev[j][1] * rs[0][0]
                                    : x * rc[0][0] + ev[j][0] * rs[0][0];
                  }
                }
              }
              if constexpr (QKV) {
                // the query scale, on the finished fp32 values, before the one rounding
                if (cb < g.q_cols) {
#pragma unroll
                  for (int t = 0; t < 4; ++t) o[t] *= g.q_scale;
                }
              }
              const int oc = wn * WN + 32 * j + 8 * g4 + hi4;
              if constexpr (F32OUT) {
                *reinterpret_cast<f32x4*>(st32 + trow * PITCH + oc) = o;
              } else {
                f16x4 h;
#pragma unroll
                for (int t = 0; t < 4; ++t) h[t] = (f16)(EPI == EPI_GELU ? gelu_tanh_f(o[t]) : o[t]);
                *reinterpret_cast<f16x4*>(st16 + trow * PITCH + oc) = h;
              }
            }
          }
        }
      }
      // The next tile's stage 0 has landed once this wave's loads are done; wait before
      // any store of this epilogue is issued, so the count holds only those loads (loads
      // and stores are not retired in order relative to each other). The barrier below
      // then makes every wave's part visible.
      if (pass == 0 && has_next) wait_vmcnt<0>();
      __syncthreads();
      // Copy-out. A full pass: NIT vectors per thread, LDS reads first, then the stores
      // (with the residual requested one pass ahead). Otherwise 16-byte vectors with a
      // scalar tail where a vector would cross N or the output rows are not 16-byte
      // aligned.
      const int rbase = m0 + pass * PR;
      if (full_pass(pass)) {
        constexpr int NB = NIT < 4 ? NIT : 4;  // LDS reads in flight per group (registers)
#pragma unroll
        for (int i0 = 0; i0 < NIT; i0 += NB) {
          if constexpr (F32OUT) {
            f32x4 x[NB];
#pragma unroll
            for (int u = 0; u < NB; ++u) {
              const int e = etid + (i0 + u) * C::NT, tr = e / VPR, vc = (e % VPR) * VE;
              x[u] = *reinterpret_cast<const f32x4*>(st32 + tr * PITCH + vc);
            }
#pragma unroll
            for (int u = 0; u < NB; ++u) {
              if constexpr (EPI == EPI_RESID_ADD) x[u] += res[i0 + u];
              *reinterpret_cast<f32x4*>(vec_addr(out32, pass, i0 + u)) = x[u];
            }
          } else {
            f16x8 x[NB];
#pragma unroll
            for (int u = 0; u < NB; ++u) {
              const int e = etid + (i0 + u) * C::NT, tr = e / VPR, vc = (e % VPR) * VE;
              x[u] = *reinterpret_cast<const f16x8*>(st16 + tr * PITCH + vc);
            }
#pragma unroll
            for (int u = 0; u < NB; ++u)
              *reinterpret_cast<f16x8*>(vec_addr(g.out16, pass, i0 + u)) = x[u];
          }
        }
        if constexpr (EPI == EPI_RESID_ADD) {
          if (pass + 1 < PASSES && full_pass(pass + 1)) res_load(pass + 1);
        }
        continue;
      }
      for (int e = etid; e < PR * VPR; e += C::NT) {
        const int tr = e / VPR, vc = (e % VPR) * VE;
        const int m = rbase + tr;
        if (m >= g.M || vc >= ncols) continue;
        const size_t o = (size_t)m * g.ldo + ocol0 + vc;
        if (vec_ok && vc + VE <= ncols) {
          if constexpr (F32OUT) {
            f32x4 x = *reinterpret_cast<const f32x4*>(st32 + tr * PITCH + vc);
            if constexpr (EPI == EPI_RESID_ADD) x += *reinterpret_cast<const f32x4*>(out32 + o);
            *reinterpret_cast<f32x4*>(out32 + o) = x;
          } else {
            *reinterpret_cast<f16x8*>(g.out16 + o) = *reinterpret_cast<const f16x8*>(st16 + tr * PITCH + vc);
          }
        } else {
          const int ne = min(VE, ncols - vc);
          for (int q = 0; q < ne; ++q) {
            if constexpr (F32OUT) {
              const float x = st32[tr * PITCH + vc + q];
              if constexpr (EPI == EPI_RESID_ADD) out32[o + q] += x;
              else out32[o + q] = x;
            } else {
              g.out16[o + q] = st16[tr * PITCH + vc + q];
            }
          }
        }
      }
    }
    if (!has_next) break;

    // Next tile: its other k-tiles go into stages 1.. once every wave's staging reads are
    // done (stage 0 is complete and visible since the first pass's barrier); the main
    // loop's first wait covers them and this epilogue's stores.
    wait_lgkmcnt0();
    __syncthreads();
    v = vn;
    m0 = m0n;
    n0 = n0n;
    issue_ops(m0, n0);  // ahead of stages 1..: the main loop's first wait covers them
    if constexpr (SPLIT) {
      issue_part(min(1, KT - 1), 1, 0, LP1);  // the rest goes out in the first k-step
    } else {
#pragma unroll
      for (int st = 1; st < NS; ++st) issue(min(st, KT - 1), st);
    }
    frags0(smem);
  }
}

// Compute units of the current device (cached per device).
inline int device_cus() {
  static std::atomic<int> cache[64];
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return 256;
  int n = cache[dev].load(std::memory_order_relaxed);
  if (n <= 0) {
    if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || n <= 0)
      n = 256;
    cache[dev].store(n, std::memory_order_relaxed);
  }
  return n;
}

// splits > 1 (one-tile-per-block configurations only): a second grid dimension of K
// splits, each writing its partial at out32 + y * split_stride.
template <class C>
hipError_t launch(const GemmArgs& a, hipStream_t st, int splits = 1) {
  const int nbm = (a.M + C::BM - 1) / C::BM, nbn = a.Npad / C::BN;
  const int ntiles = nbm * nbn;
  // one block per compute unit (the LDS allows one), a multiple of 8 so a virtual tile's
  // XCD is its block's; a smaller problem gets one block per tile
  const int cus = device_cus() / 8 * 8;
  const int grid = (!C::PERSIST || ntiles <= cus) ? ntiles : (cus > 0 ? cus : 8);
  if (splits > 1 && (grid != ntiles || (a.K / C::BK) % splits != 0)) return hipErrorInvalidValue;
  const dim3 block(C::NT);
#define TFP_GEMM_LAUNCH(E, R) hipLaunchKernelGGL((gemm_kernel<C, E, R>), dim3(grid, splits), block, 0, st, a)
  switch (a.epi) {
    case EPI_STORE_F32: TFP_GEMM_LAUNCH(EPI_STORE_F32, 0); break;
    case EPI_STORE_F16: TFP_GEMM_LAUNCH(EPI_STORE_F16, 0); break;
    case EPI_RESID_ADD: TFP_GEMM_LAUNCH(EPI_RESID_ADD, 0); break;
    case EPI_SWIGLU: TFP_GEMM_LAUNCH(EPI_SWIGLU, 0); break;
    case EPI_GELU: TFP_GEMM_LAUNCH(EPI_GELU, 0); break;
    case EPI_QKV_ROPE:  // the rotary span is a compile-time constant of the epilogue
      switch (a.rot_half) {
        case 0: TFP_GEMM_LAUNCH(EPI_QKV_ROPE, 0); break;
        case 1: TFP_GEMM_LAUNCH(EPI_QKV_ROPE, 1); break;
        case 2: TFP_GEMM_LAUNCH(EPI_QKV_ROPE, 2); break;
        case 4: TFP_GEMM_LAUNCH(EPI_QKV_ROPE, 4); break;
        case 8: TFP_GEMM_LAUNCH(EPI_QKV_ROPE, 8); break;
        case 16: TFP_GEMM_LAUNCH(EPI_QKV_ROPE, 16); break;
        case 32: TFP_GEMM_LAUNCH(EPI_QKV_ROPE, 32); break;
        default: return hipErrorInvalidValue;
      }
      break;
    case EPI_QKV_HLN_ROPE:
      switch (a.rot_half) {
        case 0: TFP_GEMM_LAUNCH(EPI_QKV_HLN_ROPE, 0); break;
        case 8: TFP_GEMM_LAUNCH(EPI_QKV_HLN_ROPE, 8); break;
        case 16: TFP_GEMM_LAUNCH(EPI_QKV_HLN_ROPE, 16); break;
        case 32: TFP_GEMM_LAUNCH(EPI_QKV_HLN_ROPE, 32); break;
        default: return hipErrorInvalidValue;
      }
      break;
    default: return hipErrorInvalidValue;
  }
#undef TFP_GEMM_LAUNCH
  return hipGetLastError();
}

}  // namespace gemm
}  // namespace tfp
