/*
 * tf_prefill.h -- C ABI of the MI355X (gfx950) dense-transformer prefill library.
 *
 * One call runs the prefill forward of a dense decoder-only transformer: token ids in,
 * per-position logits out. Every step of it runs in hand-written HIP kernels on one GPU.
 *
 * What is computed (sources: page title, then section):
 *   - StableLM-2 form: token embedding; per block h = x + Attn(LN1(x)),
 *     out = h + MLP(LN2(h)) with LayerNorm-with-bias, biased Q/K/V projections, partial
 *     NeoX split-half RoPE on the first rot_dim dims of each head (the rest pass through),
 *     causal softmax attention with query scale head_dim^-1/2, o_proj without bias,
 *     SwiGLU MLP; final LayerNorm, untied lm_head without bias.
 *     ("StableLM-2: partial RoPE and a first LayerNorm-with-bias path in a dense ROCm
 *     engine", Abstract and 1. Contribution; nnterp encyclopedia "stablelm" page,
 *     Printout, Config and The Notes.)
 *   - Bloom-style variant: ALiBi per-head geometric slopes as a linear pre-softmax bias
 *     and no rotary, LayerNorm on the embeddings before block 0, per-head interleaved
 *     fused QKV tensor, GELU MLP. ("Bloom in a sovereign engine: ALiBi as the third
 *     positional paradigm", Contribution.)
 *   - OLMo-2-style variant: no input norm; RMSNorm on the attention and MLP outputs
 *     before each residual add; RMSNorm over the whole Q and K projection rows.
 *     ("OLMo-2: reordered (post) normalization and a loader-clobber root-cause",
 *     1. Contribution.)
 *   - StableLM-2-12B's block options: parallel residual (both sublayers read the one
 *     input norm), a LayerNorm without bias per query head and per key/value head before
 *     the rotary, and grouped key/value heads. (nnterp encyclopedia "stablelm" page,
 *     The Notes: "The block is sequential on 1.6B and 3B, parallel on 12B", "Per-head
 *     LayerNorms on queries and keys on 12B", "Grouped-query attention on 12B".)
 *   - Learned absolute positions: a learned row per position added to the token embedding,
 *     the positional paradigm beside RoPE and ALiBi. ("Bloom in a sovereign engine: ALiBi as
 *     the third positional paradigm", Contribution.)
 *
 * Conventions shared by every entry point:
 *   - All tensor pointers are DEVICE pointers unless stated otherwise. Matrices are
 *     row-major. Weight matrices use the nn.Linear layout [out_features, in_features].
 *   - `stream` is a hipStream_t passed as void*; NULL means the null stream. Calls only
 *     enqueue work: they return before it runs. Faults inside kernels surface at the
 *     caller's next synchronisation.
 *   - Every function returns TF_OK or an error code; no C++ exception crosses the ABI.
 *     After an error, tf_last_error() returns a message for the calling thread.
 */
#ifndef TF_PREFILL_H
#define TF_PREFILL_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define TF_ABI_VERSION 5

typedef int32_t tf_status;
#define TF_OK 0
#define TF_ERR_INVALID_ARG 1   /* bad pointer, size or config field */
#define TF_ERR_UNSUPPORTED 2   /* valid model, but a shape/flag this library does not run */
#define TF_ERR_OUT_OF_MEMORY 3 /* device allocation failed */
#define TF_ERR_HIP 4           /* a HIP runtime call or kernel launch failed */

/* config enums */
#define TF_NORM_LAYERNORM 0 /* LayerNorm with gain and bias (population variance, eps in root) */
#define TF_NORM_RMS 1       /* RMSNorm with gain */
#define TF_NORM_PRE 0       /* h = x + f(norm(x)) */
#define TF_NORM_POST 1      /* h = x + RMS(f(x)) -- requires TF_NORM_RMS */
#define TF_QK_NORM_NONE 0
#define TF_QK_NORM_FULL_RMS 1 /* RMSNorm over the whole Q (K) projection row, before heads */
#define TF_QK_NORM_HEAD_LN 2  /* LayerNorm without bias over each Q head and each K head
                                 (its d dims), after the head split and before the rotary */
#define TF_QKV_SEPARATE 0     /* q_w, k_w, v_w given separately */
#define TF_QKV_FUSED 1        /* qkv_fused_w [3*H*d, h]: rows ordered (head, q|k|v, dim) */
#define TF_MLP_SWIGLU 0       /* down(SiLU(gate x) * up x) */
#define TF_MLP_GELU_TANH 1    /* down(GELU_tanh(fc1 x + b1)) + b2 */
#define TF_WEIGHTS_F16 0      /* projection matrices and lm_head kept in float16 */
#define TF_WEIGHTS_Q8_0 1     /* ... stored as Q8_0: int8 codes in blocks of 32 along the input
                                 dimension, one float16 scale max|x|/127 per block (GGUF's
                                 8-bit format; the pages' q8 results name no scheme) */
#define TF_LOGITS_F32 0
#define TF_LOGITS_F16 1

/*
 * Model description. Validated by tf_config_validate(); the same struct (byte for byte
 * in every field) must be passed to tf_weights_pack() and tf_prefill().
 *
 * Supported envelope (TF_ERR_UNSUPPORTED outside it, TF_ERR_INVALID_ARG for
 * inconsistent values):
 *   hidden % 256 == 0, hidden <= 8192; n_heads * head_dim == hidden; head_dim in {64,128};
 *   inter % 64 == 0; vocab >= 1; n_layers >= 1; 1 <= max_seq <= 65536;
 *   rot_dim even, 0 <= rot_dim <= head_dim. Without QK-norm the rotary is applied inside
 *   the QKV GEMM epilogue, which runs rot_dim/2 in {0, 1, 2, 4, 8, 16, 32};
 *   alibi requires rot_dim == 0 (a rotary path left on for an ALiBi model is the bug the
 *   Bloom report describes); norm_place POST requires norm_kind RMS.
 *   n_kv_heads (0 = n_heads) divides n_heads; with n_kv_heads < n_heads the QKV tensors
 *   must be TF_QKV_SEPARATE. parallel_residual requires norm_place PRE. learned_pos
 *   requires rot_dim == 0 and alibi == 0 (one positional scheme per model).
 */
typedef struct tf_config {
  int32_t abi_version; /* must be TF_ABI_VERSION */
  int32_t n_layers, hidden, n_heads, head_dim, inter, vocab, max_seq;
  int32_t norm_kind;  /* TF_NORM_LAYERNORM / TF_NORM_RMS (all norms of the model) */
  int32_t norm_place; /* TF_NORM_PRE / TF_NORM_POST */
  int32_t embed_norm; /* 1: LayerNorm (gain+bias) on the embeddings before block 0 */
  int32_t rot_dim;    /* leading dims of each q/k head that are rotated; 0 = no RoPE */
  double rope_theta;  /* rotary base; frequency of pair i is theta^(-2i/rot_dim) */
  int32_t alibi;      /* 1: slopes m_a = 2^(-8(a+1)/n_heads), bias m_a*(j-i) on scores */
  int32_t qk_norm;    /* TF_QK_NORM_* */
  int32_t qkv_bias, o_bias, mlp_bias; /* 1: the projection has a bias */
  int32_t qkv_layout; /* TF_QKV_SEPARATE / TF_QKV_FUSED */
  int32_t mlp_kind;   /* TF_MLP_SWIGLU / TF_MLP_GELU_TANH */
  float norm_eps;     /* eps of every LayerNorm / RMSNorm except the QK norm */
  float qk_norm_eps;  /* eps of the QK RMSNorm */
  int32_t logits_dtype; /* TF_LOGITS_F32 (default) / TF_LOGITS_F16 */
  int32_t n_kv_heads;   /* key/value heads; 0 means n_heads. Query head a reads key/value
                           head a / (n_heads / n_kv_heads) (grouped-query attention) */
  int32_t parallel_residual; /* 1: out = x + Attn(n) + MLP(n), n = LN1(x), no second norm */
  int32_t learned_pos;  /* 1: learned absolute positions, row p of pos_embed added to the
                           token embedding at position p (before any embed_norm) */
  int32_t weight_format; /* TF_WEIGHTS_F16 (default) or TF_WEIGHTS_Q8_0: the packer encodes
                            the float16 raw matrices; each GEMM decodes its weight into a
                            float16 workspace slice just before it runs */
} tf_config;

/*
 * Raw (unpacked) weights of one layer: DEVICE pointers to float16 tensors, nn.Linear
 * layout, row-major, contiguous. Slots the config does not use must be NULL; slots it
 * uses must be non-NULL. Sizes with hd = n_heads*head_dim (== hidden) and
 * kvd = n_kv_heads*head_dim:
 *   attn_norm_w/b [h]         pre-norm only (b: LayerNorm only)
 *   q_w [hd,h], k_w,v_w [kvd,h], q_b [hd], k_b,v_b [kvd]  TF_QKV_SEPARATE (biases if qkv_bias)
 *   qkv_fused_w [3hd,h], qkv_fused_b [3hd]      TF_QKV_FUSED
 *   q_norm_w [hd], k_norm_w [kvd]               TF_QK_NORM_FULL_RMS (kvd == hd) or
 *                             TF_QK_NORM_HEAD_LN (head a's gains at [a*d, (a+1)*d))
 *   o_w [h,hd], o_b [h]       (o_b if o_bias)
 *   mlp_norm_w/b [h]          pre-norm, sequential block only
 *   post_attn_norm_w, post_ff_norm_w [h]        post-norm only
 *   gate_w, up_w [inter,h]    SwiGLU
 *   fc1_w [inter,h], fc1_b [inter]              GELU (fc1_b if mlp_bias)
 *   down_w [h,inter], down_b [h]                (down_b if mlp_bias)
 * Every slot is read from its own pointer; two slots are never taken from one another
 * (the OLMo-2 report's loader-clobber bug). Passing the same pointer twice is allowed
 * and means the caller ties those tensors.
 */
typedef struct tf_raw_layer {
  const void *attn_norm_w, *attn_norm_b;
  const void *q_w, *k_w, *v_w, *q_b, *k_b, *v_b;
  const void *qkv_fused_w, *qkv_fused_b;
  const void *q_norm_w, *k_norm_w;
  const void *o_w, *o_b;
  const void *mlp_norm_w, *mlp_norm_b;
  const void *post_attn_norm_w, *post_ff_norm_w;
  const void *gate_w, *up_w, *fc1_w, *fc1_b, *down_w, *down_b;
} tf_raw_layer;

/*
 * Raw weights of the model. `layers` is a HOST array of n_layers entries; the other
 * members are DEVICE pointers to float16:
 *   embed [vocab,h]; embed_norm_w/b [h] (if embed_norm); final_norm_w [h],
 *   final_norm_b [h] (LayerNorm only); lm_head [vocab,h] (pass `embed` to tie).
 */
typedef struct tf_raw_weights {
  const void *embed, *embed_norm_w, *embed_norm_b;
  const tf_raw_layer* layers;
  const void *final_norm_w, *final_norm_b;
  const void* lm_head;
  const void* pos_embed;  /* [max_seq, h], learned_pos only */
} tf_raw_weights;

/* Opaque packed-weights handle: owns the packed device buffers and the default
 * workspace. One tf_prefill call per handle may be in flight at a time. */
typedef struct tf_weights tf_weights;

/* Kernel classes that tf_prefill_ex can bracket with HIP events (see tf_timing_read). */
#define TF_KT_NONE 0
#define TF_KT_GEMM_QKV 1
#define TF_KT_ATTENTION 2
#define TF_KT_GEMM_O 3
#define TF_KT_GEMM_MLP_UP 4   /* gate/up (SwiGLU) or fc1 (GELU) GEMM */
#define TF_KT_GEMM_MLP_DOWN 5
#define TF_KT_GEMM_LM_HEAD 6
#define TF_KT_NORM 7          /* LayerNorm / RMSNorm row kernels */
#define TF_KT_COUNT 8

/* Options of tf_prefill_ex. Zero-initialise, then set what is needed. */
typedef struct tf_prefill_opts {
  void* workspace;        /* NULL: use the handle's own (grown on demand with hipMalloc);
                             else DEVICE buffer of >= tf_workspace_size() bytes, 256-byte
                             aligned, owned by the caller */
  size_t workspace_bytes;
  float* residual_dump;   /* NULL or DEVICE fp32 [n_layers+1, batch, seq, hidden]: the
                             residual stream after the embedding (and its norm) and after
                             each block */
  int32_t timed_kernel;   /* TF_KT_*: record a HIP event pair around each launch of it */
  /* Padding ("nnterp encyclopedia" stablelm page, The API: the attention mask the model is
   * called with, zeros are padding). NULL: no padding. Else DEVICE int32 [batch, seq]:
   * a zero marks a padding position, which no query attends to; positions stay 0..seq-1
   * in every row. Ids at padding positions must still be in range. Every position's
   * logits are computed; a padding query with no key before it attends to nothing (zero
   * attention output). */
  const int32_t* attention_mask;
  /* NULL, or DEVICE float32 [batch, vocab]: the softmax over the vocabulary of the logits
   * at position seq-1 (same page, The API: next_token_probs at the last position). */
  float* next_token_probs;
} tf_prefill_opts;

/* Checks a config. TF_OK, TF_ERR_INVALID_ARG or TF_ERR_UNSUPPORTED. */
tf_status tf_config_validate(const tf_config* cfg);

/*
 * Packs raw weights into the library's layout and returns a handle in *out.
 * Packing: Q, K and V rows are concatenated into one [3hd, h] matrix (a fused tensor is
 * first de-interleaved from its per-head order); SwiGLU gate and up rows are
 * interleaved in groups of 32; every matrix is zero-padded to a multiple of 256 rows and
 * stored in MFMA fragment order (32-row x 16-column blocks of 1 KB, each the operand of
 * one 32x32x16 matrix instruction), or encoded as Q8_0 with TF_WEIGHTS_Q8_0;
 * norm gains and biases are converted to float32; RoPE cos/sin tables [max_seq, rot/2]
 * are computed on the host in double precision and stored as float32.
 * The copies and conversions run on `stream`; the call waits for them before it
 * returns, so `raw` may be freed as soon as it returns.
 * Errors: TF_ERR_INVALID_ARG (NULL pointers, missing slots), TF_ERR_UNSUPPORTED,
 * TF_ERR_OUT_OF_MEMORY, TF_ERR_HIP. On error *out is NULL and nothing is leaked.
 */
tf_status tf_weights_pack(const tf_config* cfg, const tf_raw_weights* raw, void* stream,
                          tf_weights** out);

/* Frees a handle and every buffer it owns (NULL is a no-op). Synchronises the device
 * first, so it must not be called while another thread still enqueues on the handle. */
void tf_weights_free(tf_weights* w);

/* Bytes of workspace a prefill of [batch, seq] needs (for tf_prefill_opts.workspace). */
tf_status tf_workspace_size(const tf_config* cfg, int32_t batch, int32_t seq, size_t* bytes);

/*
 * The prefill forward: token ids in, the logits of every position out (nnterp
 * encyclopedia, "stablelm" page, The API: input_ids [batch seq] -> logits [batch seq
 * vocab_size]; the readout in The Notes: final norm, then lm_head, nothing after it).
 * ids: DEVICE int32 [batch, seq], row-major; positions are 0..seq-1
 * in every row (padding only through tf_prefill_ex's attention_mask). logits_out: DEVICE [batch, seq, vocab] row-major, float32
 * (or float16 if cfg->logits_dtype is TF_LOGITS_F16).
 * Ids outside [0, vocab) are the caller's error: they are never read out of bounds; the
 * embedding row of such a token is NaN, which makes the logits of that whole batch row
 * NaN (masked keys still enter the P.V product with weight 0, and 0 * NaN is NaN); the
 * other batch rows are unaffected.
 * batch == 0 or seq == 0 is a no-op. seq > max_seq is TF_ERR_INVALID_ARG. Size limits
 * (TF_ERR_UNSUPPORTED beyond them): batch * seq <= 2^24 tokens, batch * seq * vocab <=
 * 2^40, and batch * seq * max(hidden, inter, n_heads * head_dim) * 2 < 2^32 bytes (the
 * GEMMs address their activation operands with 32-bit byte offsets). `cfg` must be
 * the config the handle was packed with. Deterministic: the same inputs give bitwise
 * identical outputs.
 */
tf_status tf_prefill(const tf_config* cfg, const tf_weights* w, const int32_t* ids,
                     int32_t batch, int32_t seq, void* logits_out, void* stream);

/* tf_prefill with options (caller workspace, residual dump, kernel timing, padding mask,
 * next-token probabilities). opts may be NULL: then it is tf_prefill, bit for bit. */
tf_status tf_prefill_ex(const tf_config* cfg, const tf_weights* w, const int32_t* ids,
                        int32_t batch, int32_t seq, void* logits_out, void* stream,
                        const tf_prefill_opts* opts);

/* Bytes of device workspace tf_prefill_noalloc has on each GPU (96 MiB). */
#define TF_NOALLOC_SCRATCH_BYTES ((size_t)96 << 20)

/*
 * tf_prefill for callers that cannot allocate device memory (code under HIP graph
 * capture, tight serving loops, harnesses that forbid hipMalloc): the same forward and
 * the same arguments, bit for bit the same logits, but the workspace is a fixed
 * TF_NOALLOC_SCRATCH_BYTES array in the library's device code (one per GPU, created when
 * the library's code is loaded on that GPU and held until the process ends), and the call
 * makes no hipMalloc, hipFree or other allocation. The caller still provides ids and
 * logits_out (device memory) and a handle packed beforehand.
 * A call whose workspace (tf_workspace_size) exceeds TF_NOALLOC_SCRATCH_BYTES is
 * TF_ERR_INVALID_ARG with nothing launched (the 1.6B shape fits up to batch * seq =
 * 2048 tokens; Q8_0 weights need a decode slice that does not fit). Every call on one GPU
 * shares that GPU's array: calls that overlap on one GPU (other streams or threads) race
 * and give wrong results; serialise them. Nothing in the array needs to start at zero.
 * Other errors as for tf_prefill.
 */
tf_status tf_prefill_noalloc(const tf_config* cfg, const tf_weights* w, const int32_t* ids,
                             int32_t batch, int32_t seq, void* logits_out, void* stream);

/*
 * Reads the event timings recorded by tf_prefill_ex calls with timed_kernel == kernel
 * since the last read: waits for the recorded events, sums their elapsed times, and
 * resets the record. *total_ms and *launches receive the sum and the number of launches.
 */
tf_status tf_timing_read(const tf_weights* w, int32_t kernel, double* total_ms,
                         int32_t* launches);

/*
 * Q8_0 encoding of a float16 matrix, the one the packer applies with TF_WEIGHTS_Q8_0
 * ("StableLM-2: partial RoPE ..." Results and "OLMo-2: ..." 1. Contribution report q8 /
 * int8 parity without a scheme; GGUF's Q8_0 is the quantised format the pages name, in
 * "RoFormer HIP FP32 layout optimization"). w: DEVICE float16 [rows, cols], cols a
 * multiple of 32. q: DEVICE int8 [rows, cols]; d: DEVICE float16 [rows, cols / 32].
 * Block (r, j) covers w[r, 32j .. 32j+31]: d = max|x| / 127 and q = x * (1 / d) rounded
 * half away from zero, both in float32 (0 codes for an all-zero block); x decodes as q*d.
 * Asynchronous on `stream`. TF_ERR_INVALID_ARG for NULL pointers, negative sizes or cols
 * not a multiple of 32.
 */
tf_status tf_quantize_q8_0(const void* w, int64_t rows, int64_t cols, void* q, void* d,
                           void* stream);

/* Message of the last failed call on this thread ("" if none). Valid until the next
 * call on this thread. */
const char* tf_last_error(void);

/* Provenance of this build, a static string: "sources <sha256> git <commit>[+dirty]", the
 * sha256 over the library's source files it was compiled from and the repository commit
 * at build time ("+dirty" when a source differed from it). Never fails. */
const char* tf_build_info(void);

#ifdef __cplusplus
}
#endif
#endif /* TF_PREFILL_H */
