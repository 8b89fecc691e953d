// Internal declarations shared by the library's translation units: vector types,
// kernel argument structs and host launchers. Not part of the public ABI.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace tfp {

typedef _Float16 f16;
typedef f16 f16x2 __attribute__((ext_vector_type(2)));
typedef f16 f16x4 __attribute__((ext_vector_type(4)));
typedef f16 f16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));

// ----------------------------------------------------------------------------- GEMM
// C[m, n] = sum_k A[m, k] * B[n, k]   (A: activations [M, K]; B: packed weight [Npad, K])
// followed by one of the epilogues below.
enum GemmEpi {
  EPI_STORE_F32 = 0,  // out32[m*ldo + n] = acc (+ bias[n])
  EPI_STORE_F16 = 1,  // out16[m*ldo + n] = fp16(acc (+ bias[n]))
  EPI_RESID_ADD = 2,  // out32[m*ldo + n] += acc (+ bias[n])      (fp32 residual stream)
  EPI_SWIGLU = 3,     // gate/up interleaved in 32-column groups -> out16 = SiLU(g) * u
  EPI_GELU = 4,       // out16 = GELU_tanh(acc + bias[n])
  EPI_QKV_ROPE = 5,   // out16 = acc + bias, RoPE on the Q and K columns (token-major
                      // [M, hd + 2 kvd]: Q | K | V, columns below rot_cols are Q or K),
                      // Q columns (below q_cols) times q_scale in fp32 before the rounding
  EPI_QKV_HLN_ROPE = 6,  // as EPI_QKV_ROPE, with a LayerNorm without bias over each 64-column
                         // Q and K head (gains hln_q / hln_k, eps hln_eps) after the bias and
                         // before the rotary; head_dim 64 only
};

struct GemmArgs {
  const f16* A;
  int lda;
  const f16* B;  // the weight in MFMA fragment order (launch_pack_fragments)
  int ldb;
  int M, N, K;   // N: real output columns (B has Npad >= N rows, zero-padded)
  int Npad;
  int epi;
  // epilogue operands
  const float* bias;  // [N] fp32 or nullptr
  float* out32;       // EPI_STORE_F32 / EPI_RESID_ADD
  f16* out16;         // EPI_STORE_F16 / EPI_SWIGLU / EPI_GELU / EPI_QKV_ROPE
  int ldo;            // leading dimension of the output (elements)
  // EPI_QKV_ROPE
  const float* rope_cos;  // [max_seq][rope_ld] (position-major; rope_ld >= rot_half, multiple of 4)
  const float* rope_sin;
  int rot_half, rope_ld;
  int seq, head_dim;
  int rot_cols;  // output columns [0, rot_cols) hold Q and K heads (rotated); V follows
  int q_cols;       // output columns [0, q_cols) hold Q heads, multiplied by q_scale
  float q_scale;
  // EPI_QKV_HLN_ROPE: gains of the Q heads [hln_hd] and of the K heads [rot_cols - hln_hd]
  const float* hln_q;
  const float* hln_k;
  float hln_eps;
  int hln_hd;
  // split-K scratch for EPI_RESID_ADD / EPI_STORE_F32 (fp32, capacity in floats), or
  // nullptr; when the launcher splits K it writes one [M, ldo] partial per split here and
  // reduces them in a fixed order into out32 (bias added once)
  float* part;
  size_t part_elems;
  size_t split_stride;  // set by the launcher: floats between consecutive partials
};

// Tile configurations the GEMM is instantiated with.
enum GemmTile { TILE_256x256 = 0, TILE_128x128 = 1, TILE_64x128 = 2, TILE_COUNT = 3 };
int gemm_pick_tile(int M, int N);
// K splits the launcher uses for an EPI_RESID_ADD / EPI_STORE_F32 GEMM of this shape when
// given enough split-K scratch (1 = no split); scratch floats needed = splits * M * ldo.
int gemm_splitk(int M, int N, int K, int epi);
hipError_t launch_gemm(const GemmArgs& a, int tile, hipStream_t st);

// ------------------------------------------------------------------------ row kernels
// x32 = E[ids] (+ P[t % seq] with learned positions P [max_seq, h]) in fp32; optional
// LayerNorm of the embedding; optional fp16 copy.
hipError_t launch_embed(const int32_t* ids, const f16* E, int vocab, int T, int h,
                        const f16* P, int seq, const float* ln_w, const float* ln_b,
                        float eps, float* x32, f16* x16, hipStream_t st);
// out16 = norm(x32) with LayerNorm (w, b) or RMSNorm (w, b == nullptr when rms).
hipError_t launch_norm(const float* x32, int T, int h, int rms, const float* w,
                       const float* b, float eps, f16* out16, hipStream_t st);
// x32 += RMS(a32) * w ; x16 = fp16(x32)
hipError_t launch_rms_add(const float* a32, const float* w, float eps, float* x32, f16* x16,
                          int T, int h, hipStream_t st);
// bits [b][ceil(s/64)] uint64 from mask int32 [b, s]: bit j%64 of word j/64 = mask != 0
hipError_t launch_mask_bits(const int32_t* mask, int b, int s, uint64_t* bits, hipStream_t st);
// probs[r, :] = softmax(logits[r*s + s - 1, :]) for r < b (fp32 out; logits fp32 or fp16)
hipError_t launch_last_softmax(const void* logits, int f16, int b, int s, int V, float* probs,
                               hipStream_t st);
// Q8_0: w fp16 [rows, cols] -> codes int8 [rows, cols] + scales fp16 [rows, cols / 32]
hipError_t launch_quantize_q8_0(const f16* w, int64_t rows, int64_t cols, int8_t* q, f16* d,
                                hipStream_t st);
// Q8_0 codes + scales of a row-major [rows, cols] matrix -> fp16 in the GEMM's MFMA
// fragment order (rows % 32 == 0, cols % 16 == 0; see pack_fragments)
hipError_t launch_dequantize_q8_0(const int8_t* q, const f16* d, int64_t rows, int64_t cols,
                                  f16* out, hipStream_t st);
// Row-major fp16 [rows, cols] -> the GEMM's B-operand order: 32-row x 16-k blocks of 1 KB
// at (rb * cols/16 + ks) * 512 values, piece l (16 bytes) of a block = row 32 rb + l % 32,
// k 16 ks + 8 (l / 32) .. +7. rows % 32 == 0, cols % 16 == 0, src != dst.
hipError_t launch_pack_fragments(const f16* src, int64_t rows, int64_t cols, f16* dst,
                                 hipStream_t st);
// out[m, n] (+)= sum_{s < S} part[s][m, n] (+ bias[n]), s in increasing order; row pitch
// ldo for part and out, partial s at part + s * stride
hipError_t launch_splitk_reduce(const float* part, int S, size_t stride, int M, int N, int ldo,
                                const float* bias, float* out, int accumulate, hipStream_t st);
// The device workspace of tf_prefill_noalloc (one static array per GPU): its size, and the
// current device's address of it (looked up once per device, on the first call there).
constexpr size_t NOALLOC_SCRATCH_BYTES = (size_t)96 << 20;
hipError_t noalloc_scratch(void** out);

// fp16 -> fp32 conversion (packing of gains / biases)
hipError_t launch_f16_to_f32(const f16* src, float* dst, int64_t n, hipStream_t st);

// ------------------------------------------------------------------------- QK norm
// qk32 [T, hd + kvd] fp32 (Q | K projections; hd = n_heads * head_dim, kvd =
// n_kv_heads * head_dim) -> normalisation of Q and K (mode 1: RMSNorm over each whole Q row
// and whole K row; mode 2: LayerNorm without bias over each head's head_dim values), gains
// qw [hd], kw [kvd], RoPE, Q times q_scale (the attention's score scale, in fp32), fp16 into
// columns [0, hd + kvd) of qkv16 [T, hd + 2 kvd] (its V columns are not touched).
hipError_t launch_qknorm_rope(const float* qk32, int mode, const float* qw, const float* kw,
                              float eps, const float* cos_t, const float* sin_t, int rope_ld,
                              int rot_dim, int batch, int seq, int n_heads, int n_kv_heads,
                              int head_dim, float q_scale, f16* qkv16, hipStream_t st);

// ------------------------------------------------------------------------ attention
struct AttnArgs {
  const f16* qkv;  // [b*s, (H + 2 Hkv) d] token-major: Q (H heads) | K (Hkv) | V (Hkv),
                   // head a of a part at columns a*d..a*d+d-1 of that part; Q is stored
                   // already multiplied by log2(e) / sqrt(d) (the score scale in the exp2
                   // domain), so q . k is the log2-domain score
  f16* out;        // [b*s, H*d] token-major (heads side by side)
  int batch, n_heads, n_kv_heads, seq, head_dim;  // query head a reads kv head a / (H / Hkv)
  const float* alibi_log2;   // [H] slope * log2(e), or nullptr
  // padding keys, or nullptr: bit j%64 of word [bi * key_words + j/64] is 1 for a token
  const uint64_t* key_bits;
  int key_words;             // ceil(seq / 64)
};
hipError_t launch_attention(const AttnArgs& a, hipStream_t st);

}  // namespace tfp
