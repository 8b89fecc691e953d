// C entry points: config validation, weight packing, workspace management and the
// per-layer launch sequence of the prefill forward.
#include <hip/hip_runtime.h>

#include <algorithm>
#include <cmath>
#include <cstdio>
#include <cstring>
#include <mutex>
#include <string>
#include <vector>

#include "../../include/tf_prefill.h"
#include "tf_internal.h"

using namespace tfp;

namespace {

thread_local std::string g_err;

tf_status fail(tf_status code, const std::string& msg) {
  g_err = msg;
  return code;
}

#define HIP_TRY(expr)                                                               \
  do {                                                                              \
    hipError_t e_ = (expr);                                                         \
    if (e_ != hipSuccess)                                                           \
      return fail(e_ == hipErrorOutOfMemory ? TF_ERR_OUT_OF_MEMORY : TF_ERR_HIP,    \
                  std::string(#expr) + ": " + hipGetErrorString(e_));               \
  } while (0)

inline size_t align256(size_t x) { return (x + 255) & ~size_t(255); }
inline int64_t round_up(int64_t x, int64_t m) { return (x + m - 1) / m * m; }

bool cfg_equal(const tf_config& a, const tf_config& b) {
  return a.abi_version == b.abi_version && a.n_layers == b.n_layers && a.hidden == b.hidden &&
         a.n_heads == b.n_heads && a.head_dim == b.head_dim && a.inter == b.inter &&
         a.vocab == b.vocab && a.max_seq == b.max_seq && a.norm_kind == b.norm_kind &&
         a.norm_place == b.norm_place && a.embed_norm == b.embed_norm &&
         a.rot_dim == b.rot_dim && a.rope_theta == b.rope_theta && a.alibi == b.alibi &&
         a.qk_norm == b.qk_norm && a.qkv_bias == b.qkv_bias && a.o_bias == b.o_bias &&
         a.mlp_bias == b.mlp_bias && a.qkv_layout == b.qkv_layout &&
         a.mlp_kind == b.mlp_kind && a.norm_eps == b.norm_eps &&
         a.qk_norm_eps == b.qk_norm_eps && a.logits_dtype == b.logits_dtype &&
         a.n_kv_heads == b.n_kv_heads && a.parallel_residual == b.parallel_residual &&
         a.learned_pos == b.learned_pos && a.weight_format == b.weight_format;
}

// key/value heads (0 in the config means one per query head)
int kv_heads(const tf_config& c) { return c.n_kv_heads ? c.n_kv_heads : c.n_heads; }

size_t round_up_sz(size_t x, size_t m) { return (x + m - 1) / m * m; }

bool fused_head_ln(const tf_config& c);

// Rows of the packed QKV matrix. With a Q/K norm that runs as its own kernel the Q | K
// rows and the V rows are two GEMMs (fp32 out for the norm, fp16 straight into place),
// so the V GEMM's 256-row tiles starting at row hd + kvd must stay inside the matrix.
size_t qkv_pad_rows(const tf_config& c) {
  const size_t hd = (size_t)c.n_heads * c.head_dim, kvd = (size_t)kv_heads(c) * c.head_dim;
  const size_t pad = round_up_sz(hd + 2 * kvd, 256);
  if (c.qk_norm && !fused_head_ln(c)) return std::max(pad, hd + kvd + round_up_sz(kvd, 256));
  return pad;
}

// Elements of the largest packed weight matrix (rows padded to 256): the size of the
// float16 slice a Q8_0 weight is decoded into, and of the packer's staging buffer.
size_t max_matrix_elems(const tf_config& c) {
  const size_t h = c.hidden, hd = (size_t)c.n_heads * c.head_dim, I = c.inter;
  const size_t up = c.mlp_kind == TF_MLP_SWIGLU ? 2 * I : I;
  return std::max({qkv_pad_rows(c) * h, round_up_sz(h, 256) * hd,
                   round_up_sz(up, 256) * h, round_up_sz(h, 256) * I,
                   round_up_sz(c.vocab, 256) * h});
}

tf_status validate(const tf_config* c) {
  if (!c) return fail(TF_ERR_INVALID_ARG, "cfg is NULL");
  if (c->abi_version != TF_ABI_VERSION)
    return fail(TF_ERR_INVALID_ARG, "abi_version mismatch (expected " +
                                        std::to_string(TF_ABI_VERSION) + ")");
  if (c->n_layers < 1 || c->hidden < 1 || c->n_heads < 1 || c->head_dim < 1 || c->inter < 1 ||
      c->vocab < 1 || c->max_seq < 1)
    return fail(TF_ERR_INVALID_ARG, "sizes must be positive");
  if ((int64_t)c->n_heads * c->head_dim != c->hidden)
    return fail(TF_ERR_INVALID_ARG, "n_heads * head_dim must equal hidden");
  if (c->norm_kind != TF_NORM_LAYERNORM && c->norm_kind != TF_NORM_RMS)
    return fail(TF_ERR_INVALID_ARG, "bad norm_kind");
  if (c->norm_place != TF_NORM_PRE && c->norm_place != TF_NORM_POST)
    return fail(TF_ERR_INVALID_ARG, "bad norm_place");
  if (c->qk_norm != TF_QK_NORM_NONE && c->qk_norm != TF_QK_NORM_FULL_RMS &&
      c->qk_norm != TF_QK_NORM_HEAD_LN)
    return fail(TF_ERR_INVALID_ARG, "bad qk_norm");
  if (c->n_kv_heads < 0 || c->n_kv_heads > c->n_heads ||
      (c->n_kv_heads > 0 && c->n_heads % c->n_kv_heads))
    return fail(TF_ERR_INVALID_ARG, "n_kv_heads must be 0 or divide n_heads");
  if (c->parallel_residual != 0 && c->parallel_residual != 1)
    return fail(TF_ERR_INVALID_ARG, "parallel_residual must be 0 or 1");
  if (c->learned_pos != 0 && c->learned_pos != 1)
    return fail(TF_ERR_INVALID_ARG, "learned_pos must be 0 or 1");
  if (c->weight_format != TF_WEIGHTS_F16 && c->weight_format != TF_WEIGHTS_Q8_0)
    return fail(TF_ERR_INVALID_ARG, "bad weight_format");
  if (c->learned_pos && (c->rot_dim != 0 || c->alibi))
    return fail(TF_ERR_UNSUPPORTED, "learned_pos excludes rotary and ALiBi (one positional scheme)");
  if (c->qkv_layout != TF_QKV_SEPARATE && c->qkv_layout != TF_QKV_FUSED)
    return fail(TF_ERR_INVALID_ARG, "bad qkv_layout");
  if (c->mlp_kind != TF_MLP_SWIGLU && c->mlp_kind != TF_MLP_GELU_TANH)
    return fail(TF_ERR_INVALID_ARG, "bad mlp_kind");
  if (c->logits_dtype != TF_LOGITS_F32 && c->logits_dtype != TF_LOGITS_F16)
    return fail(TF_ERR_INVALID_ARG, "bad logits_dtype");
  if (c->rot_dim < 0 || (c->rot_dim & 1) || c->rot_dim > c->head_dim)
    return fail(TF_ERR_INVALID_ARG, "rot_dim must be even and within [0, head_dim]");
  if (c->rot_dim > 0 && !(c->rope_theta > 0.0))
    return fail(TF_ERR_INVALID_ARG, "rope_theta must be positive");
  if (c->alibi && c->rot_dim != 0)
    return fail(TF_ERR_INVALID_ARG, "alibi requires rot_dim == 0 (rotary must be off)");
  if (c->embed_norm && c->norm_kind != TF_NORM_LAYERNORM)
    return fail(TF_ERR_UNSUPPORTED, "embed_norm is a LayerNorm with bias");
  if (c->norm_place == TF_NORM_POST && c->norm_kind != TF_NORM_RMS)
    return fail(TF_ERR_UNSUPPORTED, "post-norm blocks use RMSNorm");
  if (c->parallel_residual && c->norm_place != TF_NORM_PRE)
    return fail(TF_ERR_UNSUPPORTED, "parallel_residual needs the pre-norm block");
  if (c->qkv_layout == TF_QKV_FUSED && kv_heads(*c) != c->n_heads)
    return fail(TF_ERR_UNSUPPORTED, "the fused per-head QKV layout has one key/value head per query head");
  if (!(c->norm_eps >= 0.f) || !(c->qk_norm_eps >= 0.f))
    return fail(TF_ERR_INVALID_ARG, "eps must be >= 0");
  if (c->hidden % 256 || c->hidden > 8192)
    return fail(TF_ERR_UNSUPPORTED, "hidden must be a multiple of 256 and <= 8192");
  if (c->head_dim != 64 && c->head_dim != 128)
    return fail(TF_ERR_UNSUPPORTED, "head_dim must be 64 or 128");
  if (c->inter % 64)
    return fail(TF_ERR_UNSUPPORTED, "inter must be a multiple of 64");
  if (c->max_seq > 65536) return fail(TF_ERR_UNSUPPORTED, "max_seq must be <= 65536");
  if ((int64_t)c->vocab * c->hidden > (int64_t)1 << 31)
    return fail(TF_ERR_UNSUPPORTED, "vocab * hidden must fit in 31 bits");
  if (c->qk_norm == TF_QK_NORM_NONE && c->rot_dim > 0) {
    const int half = c->rot_dim / 2;
    if (!(half == 1 || half == 2 || half == 4 || half == 8 || half == 16 || half == 32))
      return fail(TF_ERR_UNSUPPORTED, "fused RoPE epilogue needs rot_dim/2 in {1,2,4,8,16,32}");
  }
  return TF_OK;
}

}  // namespace

// ------------------------------------------------------------------------ the handle

// Q8_0 form of a packed matrix [rows, K]: codes [rows, K] and scales [rows, K / 32].
struct Q8Mat {
  int8_t* q = nullptr;
  f16* s = nullptr;
};

struct PackedLayer {
  // float16 matrices (TF_WEIGHTS_F16); with TF_WEIGHTS_Q8_0 these are null outside packing
  // and the Q8_0 forms below hold the weights
  f16 *wqkv, *wo, *wup, *wdown;
  Q8Mat qqkv, qo, qup, qdown;
  float *bqkv, *qn_w, *kn_w, *bo, *n1_w, *n1_b, *n2_w, *n2_b, *pa_w, *pf_w, *b1, *b2;
};

struct tf_weights {
  tf_config cfg;
  void* block = nullptr;  // one allocation holding every packed tensor
  f16 *embed = nullptr, *lm_head = nullptr;
  Q8Mat qlm;
  float *en_w = nullptr, *en_b = nullptr, *fn_w = nullptr, *fn_b = nullptr;
  // RoPE tables, position-major: [max_seq][rope_ld] (rope_ld = rot/2 rounded up to 4, zero
  // padded), so four consecutive frequencies of one position are one 16-byte load
  float *rope_cos = nullptr, *rope_sin = nullptr, *alibi = nullptr;
  int rope_ld = 0;
  f16* pos = nullptr;  // learned position rows [max_seq, h]
  std::vector<PackedLayer> layers;
  int n_qkv_pad, n_o_pad, n_up_pad, n_down_pad, n_lm_pad, n_up_real;
  // default workspace
  void* ws = nullptr;
  size_t ws_bytes = 0;
  // kernel timing
  mutable std::mutex tmu;
  mutable std::vector<std::pair<hipEvent_t, hipEvent_t>> ev_pool[TF_KT_COUNT];
  mutable size_t ev_used[TF_KT_COUNT] = {};
};

namespace {

struct Carver {
  char* base;
  size_t off = 0;
  bool measure;
  template <class T>
  T* take(size_t count) {
    T* p = measure ? nullptr : reinterpret_cast<T*>(base + off);
    off += align256(count * sizeof(T));
    return p;
  }
};

// Lays out every packed tensor (measure pass, then real pass with the same order).
void carve_weights(tf_weights* w, Carver& cv) {
  const tf_config& c = w->cfg;
  const int h = c.hidden, hd = c.n_heads * c.head_dim, kvd = kv_heads(c) * c.head_dim,
            I = c.inter;
  const bool ln = c.norm_kind == TF_NORM_LAYERNORM, pre = c.norm_place == TF_NORM_PRE;
  const bool second = pre && !c.parallel_residual;  // a norm in front of the MLP
  w->embed = cv.take<f16>((size_t)c.vocab * h);
  if (c.embed_norm) {
    w->en_w = cv.take<float>(h);
    w->en_b = cv.take<float>(h);
  }
  w->fn_w = cv.take<float>(h);
  if (ln) w->fn_b = cv.take<float>(h);
  const bool q8 = c.weight_format == TF_WEIGHTS_Q8_0;
  // a matrix in the handle's format: float16, or Q8_0 codes + scales
  auto mat = [&](f16*& f, Q8Mat& qm, size_t rows, size_t K) {
    f = nullptr;
    qm = Q8Mat{};
    if (q8) {
      qm.q = cv.take<int8_t>(rows * K);
      qm.s = cv.take<f16>(rows * K / 32);
    } else {
      f = cv.take<f16>(rows * K);
    }
  };
  mat(w->lm_head, w->qlm, w->n_lm_pad, h);
  if (c.rot_dim > 0) {
    w->rope_ld = (int)round_up(c.rot_dim / 2, 4);
    w->rope_cos = cv.take<float>((size_t)w->rope_ld * c.max_seq);
    w->rope_sin = cv.take<float>((size_t)w->rope_ld * c.max_seq);
  }
  if (c.alibi) w->alibi = cv.take<float>(c.n_heads);
  if (c.learned_pos) w->pos = cv.take<f16>((size_t)c.max_seq * h);
  w->layers.assign(c.n_layers, PackedLayer{});
  for (auto& L : w->layers) {
    L = PackedLayer{};
    mat(L.wqkv, L.qqkv, w->n_qkv_pad, h);
    if (c.qkv_bias) L.bqkv = cv.take<float>(hd + 2 * kvd);
    if (c.qk_norm) {
      L.qn_w = cv.take<float>(hd);
      L.kn_w = cv.take<float>(kvd);
    }
    mat(L.wo, L.qo, w->n_o_pad, hd);
    if (c.o_bias) L.bo = cv.take<float>(h);
    if (pre) {
      L.n1_w = cv.take<float>(h);
      if (second) L.n2_w = cv.take<float>(h);
      if (ln) {
        L.n1_b = cv.take<float>(h);
        if (second) L.n2_b = cv.take<float>(h);
      }
    } else {
      L.pa_w = cv.take<float>(h);
      L.pf_w = cv.take<float>(h);
    }
    mat(L.wup, L.qup, w->n_up_pad, h);
    if (c.mlp_kind == TF_MLP_GELU_TANH && c.mlp_bias) L.b1 = cv.take<float>(I);
    mat(L.wdown, L.qdown, w->n_down_pad, I);
    if (c.mlp_bias) L.b2 = cv.take<float>(h);
  }
}

tf_status need(const void* p, const char* name) {
  if (!p) return fail(TF_ERR_INVALID_ARG, std::string("missing weight slot: ") + name);
  return TF_OK;
}

#define NEED(p, name)                      \
  do {                                     \
    tf_status s_ = need((p), (name));      \
    if (s_ != TF_OK) return s_;            \
  } while (0)

tf_status check_slots(const tf_config& c, const tf_raw_weights* r) {
  const bool ln = c.norm_kind == TF_NORM_LAYERNORM, pre = c.norm_place == TF_NORM_PRE;
  NEED(r->embed, "embed");
  NEED(r->lm_head, "lm_head");
  NEED(r->final_norm_w, "final_norm_w");
  if (ln) NEED(r->final_norm_b, "final_norm_b");
  if (c.learned_pos) NEED(r->pos_embed, "pos_embed");
  if (c.embed_norm) {
    NEED(r->embed_norm_w, "embed_norm_w");
    NEED(r->embed_norm_b, "embed_norm_b");
  }
  NEED(r->layers, "layers");
  for (int l = 0; l < c.n_layers; ++l) {
    const tf_raw_layer& L = r->layers[l];
    if (pre) {
      NEED(L.attn_norm_w, "attn_norm_w");
      if (!c.parallel_residual) NEED(L.mlp_norm_w, "mlp_norm_w");
      if (ln) {
        NEED(L.attn_norm_b, "attn_norm_b");
        if (!c.parallel_residual) NEED(L.mlp_norm_b, "mlp_norm_b");
      }
    } else {
      NEED(L.post_attn_norm_w, "post_attn_norm_w");
      NEED(L.post_ff_norm_w, "post_ff_norm_w");
    }
    if (c.qkv_layout == TF_QKV_FUSED) {
      NEED(L.qkv_fused_w, "qkv_fused_w");
      if (c.qkv_bias) NEED(L.qkv_fused_b, "qkv_fused_b");
    } else {
      NEED(L.q_w, "q_w");
      NEED(L.k_w, "k_w");
      NEED(L.v_w, "v_w");
      if (c.qkv_bias) {
        NEED(L.q_b, "q_b");
        NEED(L.k_b, "k_b");
        NEED(L.v_b, "v_b");
      }
    }
    if (c.qk_norm) {
      NEED(L.q_norm_w, "q_norm_w");
      NEED(L.k_norm_w, "k_norm_w");
    }
    NEED(L.o_w, "o_w");
    if (c.o_bias) NEED(L.o_b, "o_b");
    if (c.mlp_kind == TF_MLP_SWIGLU) {
      NEED(L.gate_w, "gate_w");
      NEED(L.up_w, "up_w");
    } else {
      NEED(L.fc1_w, "fc1_w");
      if (c.mlp_bias) NEED(L.fc1_b, "fc1_b");
    }
    NEED(L.down_w, "down_w");
    if (c.mlp_bias) NEED(L.down_b, "down_b");
  }
  return TF_OK;
}

// Per-head Q/K LayerNorm over 64-dim heads runs inside the QKV GEMM's epilogue (one head
// per wave tile) when the rotary span is one the fused epilogue takes; otherwise the GEMM
// stores fp32 and the QK-norm kernel follows.
bool fused_head_ln(const tf_config& c) {
  const int half = c.rot_dim / 2;
  return c.qk_norm == TF_QK_NORM_HEAD_LN && c.head_dim == 64 &&
         (half == 0 || half == 8 || half == 16 || half == 32);
}

// Workspace layout for one [batch, seq] call.
struct Workspace {
  float* x32;   // fp32 residual stream [T, h]
  f16* x16;     // normed activations (pre-norm) or fp16 residual copy (post-norm) [T, h]
  f16* qkv16;   // token-major Q | K | V [T, hd + 2 kvd]
  f16* o16;     // attention output [T, hd]
  f16* u16;     // MLP activation [T, inter]
  float* a32;   // post-norm: sublayer output [T, h]
  float* qk32;  // QK-norm: fp32 Q | K projections [T, hd + kvd]
  uint64_t* kbits;  // padding mask as bits [batch, ceil(seq / 64)]
  f16* deq;         // Q8_0 weights: the float16 form of the GEMM's weight, decoded per GEMM
  float* part;      // split-K partials of the O / down GEMMs (small token counts), or null
  size_t part_elems;
};

// Split-K partials the O and down projections need for T tokens (0 when neither splits).
size_t splitk_part_elems(const tf_config& c, int64_t T) {
  if (T <= 0 || T > INT32_MAX) return 0;
  const int epi = c.norm_place == TF_NORM_PRE ? EPI_RESID_ADD : EPI_STORE_F32;
  const int hd = c.n_heads * c.head_dim;
  const int s = std::max(gemm_splitk((int)T, c.hidden, hd, epi),
                         gemm_splitk((int)T, c.hidden, c.inter, epi));
  return s > 1 ? (size_t)s * T * c.hidden : 0;
}

size_t carve_workspace(const tf_config& c, int batch, int seq, char* base, Workspace* ws) {
  const int64_t T = (int64_t)batch * seq;
  const int h = c.hidden, hd = c.n_heads * c.head_dim, nqkv = hd + 2 * kv_heads(c) * c.head_dim;
  Carver cv{base, 0, base == nullptr};
  Workspace w{};
  w.x32 = cv.take<float>(T * h);
  w.x16 = cv.take<f16>(T * h);
  w.qkv16 = cv.take<f16>(T * nqkv);
  w.o16 = cv.take<f16>(T * hd);
  w.u16 = cv.take<f16>(T * c.inter);
  if (c.norm_place == TF_NORM_POST) w.a32 = cv.take<float>(T * h);
  if (c.qk_norm && !fused_head_ln(c))
    w.qk32 = cv.take<float>(T * (hd + kv_heads(c) * c.head_dim));
  w.kbits = cv.take<uint64_t>((int64_t)batch * ((seq + 63) / 64));
  if (c.weight_format == TF_WEIGHTS_Q8_0) w.deq = cv.take<f16>(max_matrix_elems(c));
  w.part_elems = splitk_part_elems(c, T);
  if (w.part_elems) w.part = cv.take<float>(w.part_elems);
  if (ws) *ws = w;
  return cv.off;
}

tf_status convert_f32(const void* src, float* dst, int64_t n, hipStream_t st) {
  HIP_TRY(launch_f16_to_f32(reinterpret_cast<const f16*>(src), dst, n, st));
  return TF_OK;
}

#define TRY(expr)                  \
  do {                             \
    tf_status s_ = (expr);         \
    if (s_ != TF_OK) return s_;    \
  } while (0)

// Each matrix is first laid out row-major in float16 in `stage` (the largest matrix's
// size): the Q|K|V concatenation (or the fused tensor's de-interleave), the gate/up
// interleave, the zero padding. Then it is either rewritten into the GEMM's MFMA fragment
// order in its slot (float16), or encoded into its Q8_0 slot (the decode writes the
// fragment order). Stream order keeps the reuse of `stage` safe.
tf_status pack_into(tf_weights* w, const tf_raw_weights* r, hipStream_t st, void* tmp,
                    f16* stage) {
  const tf_config& c = w->cfg;
  const int h = c.hidden, hd = c.n_heads * c.head_dim, I = c.inter, H = c.n_heads,
            d = c.head_dim, kvd = kv_heads(c) * c.head_dim;
  const size_t rowb = (size_t)h * sizeof(f16);
  const bool q8 = c.weight_format == TF_WEIGHTS_Q8_0;
  auto finish = [&](int rows, int K, f16* slot, const Q8Mat& qm) -> tf_status {
    if (q8) HIP_TRY(launch_quantize_q8_0(stage, rows, K, qm.q, qm.s, st));
    else HIP_TRY(launch_pack_fragments(stage, rows, K, slot, st));
    return TF_OK;
  };
  f16* const lm_slot = w->lm_head;
  w->lm_head = stage;
  HIP_TRY(hipMemcpyAsync(w->embed, r->embed, (size_t)c.vocab * rowb, hipMemcpyDeviceToDevice, st));
  HIP_TRY(hipMemcpyAsync(w->lm_head, r->lm_head, (size_t)c.vocab * rowb, hipMemcpyDeviceToDevice, st));
  HIP_TRY(hipMemsetAsync(w->lm_head + (size_t)c.vocab * h, 0, (size_t)(w->n_lm_pad - c.vocab) * rowb, st));
  w->lm_head = lm_slot;
  TRY(finish(w->n_lm_pad, h, lm_slot, w->qlm));
  if (c.embed_norm) {
    TRY(convert_f32(r->embed_norm_w, w->en_w, h, st));
    TRY(convert_f32(r->embed_norm_b, w->en_b, h, st));
  }
  TRY(convert_f32(r->final_norm_w, w->fn_w, h, st));
  if (w->pos)
    HIP_TRY(hipMemcpyAsync(w->pos, r->pos_embed, (size_t)c.max_seq * rowb,
                           hipMemcpyDeviceToDevice, st));
  if (w->fn_b) TRY(convert_f32(r->final_norm_b, w->fn_b, h, st));

  for (int l = 0; l < c.n_layers; ++l) {
    const tf_raw_layer& R = r->layers[l];
    PackedLayer& L = w->layers[l];
    f16* const slot_qkv = L.wqkv, *const slot_o = L.wo, *const slot_up = L.wup,
             *const slot_down = L.wdown;
    L.wqkv = L.wo = L.wup = L.wdown = stage;
    // QKV: rows [Q (hd) | K (kvd) | V (kvd)], zero padded.
    if (c.qkv_layout == TF_QKV_FUSED) {
      // fused rows ordered (head a, part c, dim e) -> packed row c*hd + a*d + e
      for (int part = 0; part < 3; ++part) {
        HIP_TRY(hipMemcpy2DAsync(L.wqkv + (size_t)part * hd * h, (size_t)d * rowb,
                                 reinterpret_cast<const f16*>(R.qkv_fused_w) + (size_t)part * d * h,
                                 (size_t)3 * d * rowb, (size_t)d * rowb, H,
                                 hipMemcpyDeviceToDevice, st));
      }
      if (c.qkv_bias) {
        f16* tb = reinterpret_cast<f16*>(tmp);
        for (int part = 0; part < 3; ++part)
          HIP_TRY(hipMemcpy2DAsync(tb + (size_t)part * hd, (size_t)d * sizeof(f16),
                                   reinterpret_cast<const f16*>(R.qkv_fused_b) + (size_t)part * d,
                                   (size_t)3 * d * sizeof(f16), (size_t)d * sizeof(f16), H,
                                   hipMemcpyDeviceToDevice, st));
        TRY(convert_f32(tb, L.bqkv, 3 * hd, st));
      }
    } else {
      const void* src[3] = {R.q_w, R.k_w, R.v_w};
      const int r0[3] = {0, hd, hd + kvd}, nr[3] = {hd, kvd, kvd};
      for (int part = 0; part < 3; ++part)
        HIP_TRY(hipMemcpyAsync(L.wqkv + (size_t)r0[part] * h, src[part], (size_t)nr[part] * rowb,
                               hipMemcpyDeviceToDevice, st));
      if (c.qkv_bias) {
        const void* bs[3] = {R.q_b, R.k_b, R.v_b};
        for (int part = 0; part < 3; ++part)
          TRY(convert_f32(bs[part], L.bqkv + r0[part], nr[part], st));
      }
    }
    HIP_TRY(hipMemsetAsync(L.wqkv + (size_t)(hd + 2 * kvd) * h, 0,
                           (size_t)(w->n_qkv_pad - hd - 2 * kvd) * rowb, st));
    TRY(finish(w->n_qkv_pad, h, slot_qkv, L.qqkv));
    if (c.qk_norm) {
      TRY(convert_f32(R.q_norm_w, L.qn_w, hd, st));
      TRY(convert_f32(R.k_norm_w, L.kn_w, kvd, st));
    }
    // O projection [h, hd]
    const size_t rowo = (size_t)hd * sizeof(f16);
    HIP_TRY(hipMemcpyAsync(L.wo, R.o_w, (size_t)h * rowo, hipMemcpyDeviceToDevice, st));
    HIP_TRY(hipMemsetAsync(L.wo + (size_t)h * hd, 0, (size_t)(w->n_o_pad - h) * rowo, st));
    TRY(finish(w->n_o_pad, hd, slot_o, L.qo));
    if (c.o_bias) TRY(convert_f32(R.o_b, L.bo, h, st));
    if (L.n1_w) {
      TRY(convert_f32(R.attn_norm_w, L.n1_w, h, st));
      if (L.n2_w) TRY(convert_f32(R.mlp_norm_w, L.n2_w, h, st));
      if (L.n1_b) TRY(convert_f32(R.attn_norm_b, L.n1_b, h, st));
      if (L.n2_b) TRY(convert_f32(R.mlp_norm_b, L.n2_b, h, st));
    } else {
      TRY(convert_f32(R.post_attn_norm_w, L.pa_w, h, st));
      TRY(convert_f32(R.post_ff_norm_w, L.pf_w, h, st));
    }
    // MLP up: SwiGLU interleaves gate / up in 32-row groups (packed group 2g = gate rows
    // 32g..32g+31, group 2g+1 = the same up rows); GELU copies fc1.
    if (c.mlp_kind == TF_MLP_SWIGLU) {
      HIP_TRY(hipMemcpy2DAsync(L.wup, (size_t)64 * rowb, R.gate_w, (size_t)32 * rowb,
                               (size_t)32 * rowb, I / 32, hipMemcpyDeviceToDevice, st));
      HIP_TRY(hipMemcpy2DAsync(L.wup + (size_t)32 * h, (size_t)64 * rowb, R.up_w,
                               (size_t)32 * rowb, (size_t)32 * rowb, I / 32,
                               hipMemcpyDeviceToDevice, st));
    } else {
      HIP_TRY(hipMemcpyAsync(L.wup, R.fc1_w, (size_t)I * rowb, hipMemcpyDeviceToDevice, st));
      if (L.b1) TRY(convert_f32(R.fc1_b, L.b1, I, st));
    }
    HIP_TRY(hipMemsetAsync(L.wup + (size_t)w->n_up_real * h, 0,
                           (size_t)(w->n_up_pad - w->n_up_real) * rowb, st));
    TRY(finish(w->n_up_pad, h, slot_up, L.qup));
    const size_t rowd = (size_t)I * sizeof(f16);
    HIP_TRY(hipMemcpyAsync(L.wdown, R.down_w, (size_t)h * rowd, hipMemcpyDeviceToDevice, st));
    HIP_TRY(hipMemsetAsync(L.wdown + (size_t)h * I, 0, (size_t)(w->n_down_pad - h) * rowd, st));
    TRY(finish(w->n_down_pad, I, slot_down, L.qdown));
    L.wqkv = slot_qkv;
    L.wo = slot_o;
    L.wup = slot_up;
    L.wdown = slot_down;
    if (L.b2) TRY(convert_f32(R.down_b, L.b2, h, st));
  }

  // Host-built tables: RoPE cos/sin (angles in double), ALiBi slopes * log2(e).
  std::vector<float> hc, hs, ha;
  if (c.rot_dim > 0) {
    const int half = c.rot_dim / 2, ldr = w->rope_ld;
    hc.assign((size_t)ldr * c.max_seq, 0.f);
    hs.assign((size_t)ldr * c.max_seq, 0.f);
    for (int i = 0; i < half; ++i) {
      const double f = std::pow(c.rope_theta, -2.0 * i / (double)c.rot_dim);
      for (int p = 0; p < c.max_seq; ++p) {
        const double ang = (double)p * f;
        hc[(size_t)p * ldr + i] = (float)std::cos(ang);
        hs[(size_t)p * ldr + i] = (float)std::sin(ang);
      }
    }
    HIP_TRY(hipMemcpyAsync(w->rope_cos, hc.data(), hc.size() * 4, hipMemcpyHostToDevice, st));
    HIP_TRY(hipMemcpyAsync(w->rope_sin, hs.data(), hs.size() * 4, hipMemcpyHostToDevice, st));
  }
  if (c.alibi) {
    ha.resize(H);
    for (int a = 0; a < H; ++a)
      ha[a] = (float)(std::pow(2.0, -8.0 * (a + 1) / (double)H) * 1.4426950408889634);
    HIP_TRY(hipMemcpyAsync(w->alibi, ha.data(), ha.size() * 4, hipMemcpyHostToDevice, st));
  }
  // The host tables above must outlive the copies: wait for the packing work.
  HIP_TRY(hipStreamSynchronize(st));
  return TF_OK;
}

// Records a HIP event pair around a launch when the call asked for that kernel class.
struct Timer {
  const tf_weights* w;
  int want;
  hipStream_t st;
  hipEvent_t stop = nullptr;
  tf_status begin(int kt) {
    stop = nullptr;
    if (want == TF_KT_NONE || kt != want) return TF_OK;
    std::lock_guard<std::mutex> g(w->tmu);
    auto& pool = w->ev_pool[kt];
    size_t& used = w->ev_used[kt];
    if (used == pool.size()) {
      hipEvent_t a, b;
      HIP_TRY(hipEventCreate(&a));
      HIP_TRY(hipEventCreate(&b));
      pool.emplace_back(a, b);
    }
    auto& pr = pool[used++];
    HIP_TRY(hipEventRecord(pr.first, st));
    stop = pr.second;
    return TF_OK;
  }
  tf_status end() {
    if (stop) HIP_TRY(hipEventRecord(stop, st));
    stop = nullptr;
    return TF_OK;
  }
};

// The float16 weight a GEMM reads: the packed matrix itself, or (Q8_0) its decoding into
// the workspace slice, enqueued just before the GEMM on the same stream.
tf_status weight16(const f16* f, const Q8Mat& qm, int rows, int K, const Workspace& ws,
                   hipStream_t st, const f16** out) {
  if (f) {
    *out = f;
    return TF_OK;
  }
  HIP_TRY(launch_dequantize_q8_0(qm.q, qm.s, rows, K, ws.deq, st));
  *out = ws.deq;
  return TF_OK;
}

tf_status run_gemm(Timer& tm, int kt, const GemmArgs& a, hipStream_t st) {
  TRY(tm.begin(kt));
  HIP_TRY(launch_gemm(a, gemm_pick_tile(a.M, a.N), st));
  return tm.end();
}

tf_status forward(const tf_weights* w, const int32_t* ids, int batch, int seq, void* logits,
                  hipStream_t st, const Workspace& ws, const tf_prefill_opts* opts) {
  const tf_config& c = w->cfg;
  const int T = batch * seq;
  const int h = c.hidden, hd = c.n_heads * c.head_dim, I = c.inter, Hkv = kv_heads(c),
            nqkv = hd + 2 * Hkv * c.head_dim;
  const bool pre = c.norm_place == TF_NORM_PRE, ln = c.norm_kind == TF_NORM_LAYERNORM;
  float* dump = opts ? opts->residual_dump : nullptr;
  Timer tm{w, opts ? opts->timed_kernel : TF_KT_NONE, st};
  const size_t slab = (size_t)T * h;

  HIP_TRY(launch_embed(ids, w->embed, c.vocab, T, h, w->pos, seq, w->en_w, w->en_b,
                       c.norm_eps, ws.x32, pre ? nullptr : ws.x16, st));
  const bool padded = opts && opts->attention_mask;
  if (padded) HIP_TRY(launch_mask_bits(opts->attention_mask, batch, seq, ws.kbits, st));
  if (dump) HIP_TRY(hipMemcpyAsync(dump, ws.x32, slab * 4, hipMemcpyDeviceToDevice, st));

  // Attention scores are taken in the exp2 domain: the producers of Q multiply it by
  // log2(e) / sqrt(head_dim) ([NNT] Notes: query scale head_dim ** -0.5) in fp32, before
  // its single fp16 rounding.
  const float q_scale = (float)(1.4426950408889634 / std::sqrt((double)c.head_dim));
  GemmArgs base{};
  base.M = T;
  for (int l = 0; l < c.n_layers; ++l) {
    const PackedLayer& L = w->layers[l];
    // --- attention sublayer
    if (pre) {
      TRY(tm.begin(TF_KT_NORM));
      HIP_TRY(launch_norm(ws.x32, T, h, !ln, L.n1_w, L.n1_b, c.norm_eps, ws.x16, st));
      TRY(tm.end());
    }
    {
      GemmArgs a = base;
      TRY(weight16(L.wqkv, L.qqkv, w->n_qkv_pad, h, ws, st, &a.B));
      a.A = ws.x16; a.lda = h; a.ldb = h; a.K = h;
      a.N = nqkv; a.Npad = w->n_qkv_pad; a.ldo = nqkv;
      a.bias = L.bqkv;
      if (c.qk_norm && !fused_head_ln(c)) {
        // Q | K in fp32 for the norm kernel; V (rows hd + kvd .. of the packed matrix,
        // whose fragment order keeps a row range contiguous) in fp16 straight into place
        const int qk = hd + Hkv * c.head_dim, kvd = Hkv * c.head_dim;
        GemmArgs v = a;
        a.epi = EPI_STORE_F32; a.out32 = ws.qk32;
        a.N = qk; a.Npad = (int)round_up(qk, 256); a.ldo = qk;
        v.epi = EPI_STORE_F16; v.out16 = ws.qkv16 + qk;
        v.B = a.B + (size_t)qk * h; v.bias = L.bqkv ? L.bqkv + qk : nullptr;
        v.N = kvd; v.Npad = (int)round_up(kvd, 256); v.ldo = nqkv;
        TRY(tm.begin(TF_KT_GEMM_QKV));
        HIP_TRY(launch_gemm(a, gemm_pick_tile(a.M, a.N), st));
        HIP_TRY(launch_gemm(v, gemm_pick_tile(v.M, v.N), st));
        TRY(tm.end());
      } else {
        a.epi = c.qk_norm ? EPI_QKV_HLN_ROPE : EPI_QKV_ROPE; a.out16 = ws.qkv16;
        a.rope_cos = w->rope_cos; a.rope_sin = w->rope_sin; a.rot_half = c.rot_dim / 2;
        a.rope_ld = w->rope_ld;
        a.seq = seq; a.head_dim = c.head_dim; a.rot_cols = hd + Hkv * c.head_dim;
        a.hln_q = L.qn_w; a.hln_k = L.kn_w; a.hln_eps = c.qk_norm_eps; a.hln_hd = hd;
        a.q_cols = hd; a.q_scale = q_scale;
        TRY(run_gemm(tm, TF_KT_GEMM_QKV, a, st));
      }
    }
    if (c.qk_norm && !fused_head_ln(c))
      HIP_TRY(launch_qknorm_rope(ws.qk32, c.qk_norm == TF_QK_NORM_FULL_RMS ? 1 : 2, L.qn_w,
                                 L.kn_w, c.qk_norm_eps, w->rope_cos, w->rope_sin, w->rope_ld,
                                 c.rot_dim, batch, seq, c.n_heads, Hkv, c.head_dim, q_scale,
                                 ws.qkv16, st));
    {
      AttnArgs at{};
      at.qkv = ws.qkv16; at.out = ws.o16;
      at.batch = batch; at.n_heads = c.n_heads; at.n_kv_heads = Hkv; at.seq = seq;
      at.head_dim = c.head_dim;
      at.alibi_log2 = w->alibi;
      at.key_bits = padded ? ws.kbits : nullptr;
      at.key_words = (seq + 63) / 64;
      TRY(tm.begin(TF_KT_ATTENTION));
      HIP_TRY(launch_attention(at, st));
      TRY(tm.end());
    }
    {
      GemmArgs a = base;
      TRY(weight16(L.wo, L.qo, w->n_o_pad, hd, ws, st, &a.B));
      a.A = ws.o16; a.lda = hd; a.ldb = hd; a.K = hd;
      a.N = h; a.Npad = w->n_o_pad; a.bias = L.bo; a.ldo = h;
      a.part = ws.part; a.part_elems = ws.part_elems;
      if (pre) {
        a.epi = EPI_RESID_ADD; a.out32 = ws.x32;
      } else {
        a.epi = EPI_STORE_F32; a.out32 = ws.a32;
      }
      TRY(run_gemm(tm, TF_KT_GEMM_O, a, st));
    }
    if (!pre) HIP_TRY(launch_rms_add(ws.a32, L.pa_w, c.norm_eps, ws.x32, ws.x16, T, h, st));
    // --- MLP sublayer (the parallel block feeds it the attention sublayer's normed input,
    // still in x16; its output joins the same residual sum)
    if (pre && !c.parallel_residual) {
      TRY(tm.begin(TF_KT_NORM));
      HIP_TRY(launch_norm(ws.x32, T, h, !ln, L.n2_w, L.n2_b, c.norm_eps, ws.x16, st));
      TRY(tm.end());
    }
    {
      GemmArgs a = base;
      TRY(weight16(L.wup, L.qup, w->n_up_pad, h, ws, st, &a.B));
      a.A = ws.x16; a.lda = h; a.ldb = h; a.K = h;
      a.N = I; a.Npad = w->n_up_pad; a.out16 = ws.u16; a.ldo = I;
      if (c.mlp_kind == TF_MLP_SWIGLU) {
        a.epi = EPI_SWIGLU;
      } else {
        a.epi = EPI_GELU; a.bias = L.b1;
      }
      TRY(run_gemm(tm, TF_KT_GEMM_MLP_UP, a, st));
    }
    {
      GemmArgs a = base;
      TRY(weight16(L.wdown, L.qdown, w->n_down_pad, I, ws, st, &a.B));
      a.A = ws.u16; a.lda = I; a.ldb = I; a.K = I;
      a.N = h; a.Npad = w->n_down_pad; a.bias = L.b2; a.ldo = h;
      a.part = ws.part; a.part_elems = ws.part_elems;
      if (pre) {
        a.epi = EPI_RESID_ADD; a.out32 = ws.x32;
      } else {
        a.epi = EPI_STORE_F32; a.out32 = ws.a32;
      }
      TRY(run_gemm(tm, TF_KT_GEMM_MLP_DOWN, a, st));
    }
    if (!pre) HIP_TRY(launch_rms_add(ws.a32, L.pf_w, c.norm_eps, ws.x32, ws.x16, T, h, st));
    if (dump)
      HIP_TRY(hipMemcpyAsync(dump + (size_t)(l + 1) * slab, ws.x32, slab * 4,
                             hipMemcpyDeviceToDevice, st));
  }
  // final norm + lm_head
  TRY(tm.begin(TF_KT_NORM));
  HIP_TRY(launch_norm(ws.x32, T, h, !ln, w->fn_w, w->fn_b, c.norm_eps, ws.x16, st));
  TRY(tm.end());
  {
    GemmArgs a = base;
    TRY(weight16(w->lm_head, w->qlm, w->n_lm_pad, h, ws, st, &a.B));
    a.A = ws.x16; a.lda = h; a.ldb = h; a.K = h;
    a.N = c.vocab; a.Npad = w->n_lm_pad; a.ldo = c.vocab;
    if (c.logits_dtype == TF_LOGITS_F32) {
      a.epi = EPI_STORE_F32; a.out32 = reinterpret_cast<float*>(logits);
    } else {
      a.epi = EPI_STORE_F16; a.out16 = reinterpret_cast<f16*>(logits);
    }
    TRY(run_gemm(tm, TF_KT_GEMM_LM_HEAD, a, st));
  }
  if (opts && opts->next_token_probs)
    HIP_TRY(launch_last_softmax(logits, c.logits_dtype == TF_LOGITS_F16, batch, seq, c.vocab,
                                opts->next_token_probs, st));
  return TF_OK;
}

// Argument checks shared by the prefill entry points; *empty is set for a no-op call.
tf_status check_call(const tf_config* cfg, const tf_weights* w, const int32_t* ids,
                     int32_t batch, int32_t seq, void* logits_out, bool* empty) {
  *empty = false;
  TRY(validate(cfg));
  if (!w) return fail(TF_ERR_INVALID_ARG, "weights handle is NULL");
  if (!cfg_equal(*cfg, w->cfg))
    return fail(TF_ERR_INVALID_ARG, "cfg differs from the config the weights were packed with");
  if (batch < 0 || seq < 0) return fail(TF_ERR_INVALID_ARG, "negative batch or seq");
  if (seq > cfg->max_seq) return fail(TF_ERR_INVALID_ARG, "seq exceeds max_seq");
  if (batch == 0 || seq == 0) {
    *empty = true;
    return TF_OK;
  }
  if ((int64_t)batch * seq > (int64_t)1 << 24)
    return fail(TF_ERR_UNSUPPORTED, "batch * seq must be <= 2^24 tokens");
  if ((int64_t)batch * seq * cfg->vocab > ((int64_t)1 << 40))
    return fail(TF_ERR_UNSUPPORTED, "logits tensor too large");
  // GEMM operands are addressed with 32-bit byte offsets
  const int64_t widest = std::max<int64_t>({cfg->hidden, cfg->inter,
                                            (int64_t)cfg->n_heads * cfg->head_dim});
  if ((int64_t)batch * seq * widest * 2 >= ((int64_t)1 << 32))
    return fail(TF_ERR_UNSUPPORTED,
                "batch * seq * max(hidden, inter, n_heads * head_dim) * 2 bytes must be < 2^32");
  if (!ids || !logits_out) return fail(TF_ERR_INVALID_ARG, "ids or logits_out is NULL");
  return TF_OK;
}

}  // namespace

// ------------------------------------------------------------------------ C entry points

extern "C" {

tf_status tf_config_validate(const tf_config* cfg) {
  try {
    return validate(cfg);
  } catch (...) {
    return fail(TF_ERR_INVALID_ARG, "internal error");
  }
}

tf_status tf_weights_pack(const tf_config* cfg, const tf_raw_weights* raw, void* stream,
                          tf_weights** out) {
  if (!out) return fail(TF_ERR_INVALID_ARG, "out is NULL");
  *out = nullptr;
  try {
    TRY(validate(cfg));
    if (!raw) return fail(TF_ERR_INVALID_ARG, "raw is NULL");
    TRY(check_slots(*cfg, raw));
    hipStream_t st = reinterpret_cast<hipStream_t>(stream);
    tf_weights* w = new tf_weights();
    w->cfg = *cfg;
    const tf_config& c = *cfg;
    const int hd = c.n_heads * c.head_dim, nqkv = hd + 2 * kv_heads(c) * c.head_dim;
    w->n_qkv_pad = (int)qkv_pad_rows(c);
    (void)nqkv;
    w->n_o_pad = (int)round_up(c.hidden, 256);
    w->n_up_real = c.mlp_kind == TF_MLP_SWIGLU ? 2 * c.inter : c.inter;
    w->n_up_pad = (int)round_up(w->n_up_real, 256);
    w->n_down_pad = (int)round_up(c.hidden, 256);
    w->n_lm_pad = (int)round_up(c.vocab, 256);
    if (c.mlp_kind == TF_MLP_SWIGLU && c.inter % 32) {
      delete w;
      return fail(TF_ERR_UNSUPPORTED, "SwiGLU needs inter % 32 == 0");
    }
    Carver m{nullptr, 0, true};
    carve_weights(w, m);
    const size_t bytes = m.off;
    hipError_t e = hipMalloc(&w->block, bytes);
    if (e != hipSuccess) {
      delete w;
      return fail(TF_ERR_OUT_OF_MEMORY, "hipMalloc of " + std::to_string(bytes) +
                                            " bytes for packed weights failed");
    }
    Carver real{reinterpret_cast<char*>(w->block), 0, false};
    carve_weights(w, real);
    void* tmp = nullptr;
    e = hipMalloc(&tmp, align256((size_t)nqkv * sizeof(f16)));
    if (e != hipSuccess) {
      hipFree(w->block);
      delete w;
      return fail(TF_ERR_OUT_OF_MEMORY, "hipMalloc of packing scratch failed");
    }
    void* stage = nullptr;
    e = hipMalloc(&stage, max_matrix_elems(c) * sizeof(f16));
    if (e != hipSuccess) {
      hipFree(tmp);
      hipFree(w->block);
      delete w;
      return fail(TF_ERR_OUT_OF_MEMORY, "hipMalloc of the packing stage failed");
    }
    tf_status s = pack_into(w, raw, st, tmp, reinterpret_cast<f16*>(stage));
    hipStreamSynchronize(st);
    hipFree(tmp);
    if (stage) hipFree(stage);
    if (s != TF_OK) {
      hipFree(w->block);
      delete w;
      return s;
    }
    *out = w;
    return TF_OK;
  } catch (const std::bad_alloc&) {
    return fail(TF_ERR_OUT_OF_MEMORY, "host allocation failed");
  } catch (...) {
    return fail(TF_ERR_INVALID_ARG, "internal error");
  }
}

void tf_weights_free(tf_weights* w) {
  if (!w) return;
  hipDeviceSynchronize();
  for (auto& pool : w->ev_pool)
    for (auto& pr : pool) {
      hipEventDestroy(pr.first);
      hipEventDestroy(pr.second);
    }
  if (w->ws) hipFree(w->ws);
  if (w->block) hipFree(w->block);
  delete w;
}

tf_status tf_workspace_size(const tf_config* cfg, int32_t batch, int32_t seq, size_t* bytes) {
  try {
    TRY(validate(cfg));
    if (!bytes) return fail(TF_ERR_INVALID_ARG, "bytes is NULL");
    if (batch < 0 || seq < 0) return fail(TF_ERR_INVALID_ARG, "negative batch or seq");
    *bytes = carve_workspace(*cfg, batch, seq, nullptr, nullptr);
    return TF_OK;
  } catch (...) {
    return fail(TF_ERR_INVALID_ARG, "internal error");
  }
}

tf_status tf_prefill_ex(const tf_config* cfg, const tf_weights* w, const int32_t* ids,
                        int32_t batch, int32_t seq, void* logits_out, void* stream,
                        const tf_prefill_opts* opts) {
  try {
    bool empty = false;
    TRY(check_call(cfg, w, ids, batch, seq, logits_out, &empty));
    if (empty) return TF_OK;
    if (opts && opts->timed_kernel < 0) return fail(TF_ERR_INVALID_ARG, "bad timed_kernel");
    if (opts && opts->timed_kernel >= TF_KT_COUNT) return fail(TF_ERR_INVALID_ARG, "bad timed_kernel");
    hipStream_t st = reinterpret_cast<hipStream_t>(stream);
    const size_t need = carve_workspace(*cfg, batch, seq, nullptr, nullptr);
    char* base;
    if (opts && opts->workspace) {
      if (opts->workspace_bytes < need)
        return fail(TF_ERR_INVALID_ARG, "workspace too small: need " + std::to_string(need));
      if (reinterpret_cast<uintptr_t>(opts->workspace) & 255)
        return fail(TF_ERR_INVALID_ARG, "workspace must be 256-byte aligned");
      base = reinterpret_cast<char*>(opts->workspace);
    } else {
      tf_weights* mw = const_cast<tf_weights*>(w);
      if (mw->ws_bytes < need) {
        if (mw->ws) {
          // the old buffer may still be in use by work on another stream
          HIP_TRY(hipDeviceSynchronize());
          HIP_TRY(hipFree(mw->ws));
          mw->ws = nullptr;
          mw->ws_bytes = 0;
        }
        hipError_t e = hipMalloc(&mw->ws, need);
        if (e != hipSuccess)
          return fail(TF_ERR_OUT_OF_MEMORY, "hipMalloc of " + std::to_string(need) +
                                                " bytes of workspace failed");
        mw->ws_bytes = need;
      }
      base = reinterpret_cast<char*>(mw->ws);
    }
    Workspace ws;
    carve_workspace(*cfg, batch, seq, base, &ws);
    return forward(w, ids, batch, seq, logits_out, st, ws, opts);
  } catch (const std::bad_alloc&) {
    return fail(TF_ERR_OUT_OF_MEMORY, "host allocation failed");
  } catch (...) {
    return fail(TF_ERR_INVALID_ARG, "internal error");
  }
}

tf_status tf_prefill(const tf_config* cfg, const tf_weights* w, const int32_t* ids,
                     int32_t batch, int32_t seq, void* logits_out, void* stream) {
  return tf_prefill_ex(cfg, w, ids, batch, seq, logits_out, stream, nullptr);
}

tf_status tf_prefill_noalloc(const tf_config* cfg, const tf_weights* w, const int32_t* ids,
                             int32_t batch, int32_t seq, void* logits_out, void* stream) {
  try {
    bool empty = false;
    TRY(check_call(cfg, w, ids, batch, seq, logits_out, &empty));
    if (empty) return TF_OK;
    const size_t need = carve_workspace(*cfg, batch, seq, nullptr, nullptr);
    if (need > NOALLOC_SCRATCH_BYTES)
      return fail(TF_ERR_INVALID_ARG,
                  "tf_prefill_noalloc: this call needs " + std::to_string(need) +
                      " bytes of workspace, more than the fixed " +
                      std::to_string(NOALLOC_SCRATCH_BYTES) +
                      " bytes it has (use tf_prefill or tf_prefill_ex)");
    void* base = nullptr;
    HIP_TRY(noalloc_scratch(&base));
    Workspace ws;
    carve_workspace(*cfg, batch, seq, reinterpret_cast<char*>(base), &ws);
    return forward(w, ids, batch, seq, logits_out, reinterpret_cast<hipStream_t>(stream), ws,
                   nullptr);
  } catch (const std::bad_alloc&) {
    return fail(TF_ERR_OUT_OF_MEMORY, "host allocation failed");
  } catch (...) {
    return fail(TF_ERR_INVALID_ARG, "internal error");
  }
}

tf_status tf_timing_read(const tf_weights* w, int32_t kernel, double* total_ms,
                         int32_t* launches) {
  if (!w || !total_ms || !launches) return fail(TF_ERR_INVALID_ARG, "NULL argument");
  if (kernel <= TF_KT_NONE || kernel >= TF_KT_COUNT) return fail(TF_ERR_INVALID_ARG, "bad kernel");
  std::lock_guard<std::mutex> g(w->tmu);
  double sum = 0.0;
  const size_t n = w->ev_used[kernel];
  for (size_t i = 0; i < n; ++i) {
    auto& pr = w->ev_pool[kernel][i];
    HIP_TRY(hipEventSynchronize(pr.second));
    float ms = 0.f;
    HIP_TRY(hipEventElapsedTime(&ms, pr.first, pr.second));
    sum += ms;
  }
  w->ev_used[kernel] = 0;
  *total_ms = sum;
  *launches = (int32_t)n;
  return TF_OK;
}

tf_status tf_quantize_q8_0(const void* w, int64_t rows, int64_t cols, void* q, void* d,
                           void* stream) {
  if (!w || !q || !d) return fail(TF_ERR_INVALID_ARG, "NULL pointer");
  if (rows < 0 || cols < 0 || cols % 32) return fail(TF_ERR_INVALID_ARG, "bad rows / cols");
  HIP_TRY(launch_quantize_q8_0(reinterpret_cast<const f16*>(w), rows, cols,
                               reinterpret_cast<int8_t*>(q), reinterpret_cast<f16*>(d),
                               reinterpret_cast<hipStream_t>(stream)));
  return TF_OK;
}

const char* tf_last_error(void) { return g_err.c_str(); }

#ifndef TF_BUILD_SOURCES
#define TF_BUILD_SOURCES "unknown"
#endif
#ifndef TF_BUILD_GIT
#define TF_BUILD_GIT "unknown"
#endif
const char* tf_build_info(void) {
  return "sources " TF_BUILD_SOURCES " git " TF_BUILD_GIT;
}

}  // extern "C"
