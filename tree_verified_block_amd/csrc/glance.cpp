// C ABI of libglance: argument validation, workspace layout and the launch
// sequence of each step.  Every check runs on the host before anything is
// enqueued; on error nothing is launched.
#include <hip/hip_runtime.h>

#include <algorithm>
#include <cmath>
#include <cstdarg>
#include <cstdio>
#include <string>

#include "common.h"
#include "kernels.h"
#include "walk_impl.h"

namespace glance {

namespace {

thread_local std::string g_last_error;

glance_status fail(glance_status st, const char* fmt, ...) {
  char buf[512];
  va_list ap;
  va_start(ap, fmt);
  std::vsnprintf(buf, sizeof(buf), fmt, ap);
  va_end(ap);
  g_last_error = buf;
  return st;
}

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

size_t round256(size_t b) { return (b + 255) & ~static_cast<size_t>(255); }

// The output-projection part of a glance_attn_pack copy (after the q/k/v part).
const void* packed_wo(const void* packed, int d_model, int Hq, int Hkv, int D) {
  return static_cast<const char*>(packed) + round256(proj_pack_bytes((Hq + 2 * Hkv) * D, d_model));
}

#define REQUIRE(cond, ...)                                               \
  do {                                                                   \
    if (!(cond)) return fail(GLANCE_ERR_INVALID_ARG, __VA_ARGS__);       \
  } while (0)
#define REQUIRE_PTR(p)                                                   \
  do {                                                                   \
    if ((p) == nullptr) return fail(GLANCE_ERR_INVALID_ARG, "%s is NULL", #p); \
    if (!aligned16(p)) return fail(GLANCE_ERR_ALIGNMENT, "%s is not 16-byte aligned", #p); \
  } while (0)
#define REQUIRE_ALIGNED_OR_NULL(p)                                       \
  do {                                                                   \
    if ((p) != nullptr && !aligned16(p))                                 \
      return fail(GLANCE_ERR_ALIGNMENT, "%s is not 16-byte aligned", #p); \
  } while (0)

glance_status check_ws(const void* ws, size_t ws_bytes, size_t need) {
  if (need == 0) return GLANCE_OK;
  if (ws == nullptr) return fail(GLANCE_ERR_WORKSPACE, "workspace is NULL (%zu bytes needed)", need);
  if ((reinterpret_cast<uintptr_t>(ws) & 255u) != 0)
    return fail(GLANCE_ERR_WORKSPACE, "workspace is not 256-byte aligned");
  if (ws_bytes < need)
    return fail(GLANCE_ERR_WORKSPACE, "workspace has %zu bytes, %zu needed", ws_bytes, need);
  return GLANCE_OK;
}

// Shape bounds that keep every size and grid computation inside 32-bit ints
// (entry points return GLANCE_ERR_UNSUPPORTED beyond them, sizers 0).
constexpr int32_t kMaxSeqs = 1 << 16;
constexpr int32_t kMaxDModel = 1 << 16;
constexpr int32_t kMaxHeads = 1024;
constexpr int32_t kMaxInter = 1 << 20;
constexpr int32_t kMaxHeadVocab = 1 << 24;
constexpr int32_t kMaxHeadRows = 1 << 20;
constexpr int64_t kMaxPrefix = (int64_t(1) << 31) - 1 - GLANCE_MAX_ROWS;

bool attn_in_bounds(int nseq, int64_t max_prefix, int d_model, int Hq, int inter) {
  return nseq <= kMaxSeqs && max_prefix <= kMaxPrefix && d_model <= kMaxDModel && Hq <= kMaxHeads &&
         inter <= kMaxInter;
}

bool head_in_bounds(int R, int V, int d_model) {
  return R <= kMaxHeadRows && V <= kMaxHeadVocab && d_model <= kMaxDModel;
}

// ---------------------------------------------------------------- tree_attn ws
struct AttnWs {
  int n_split = 0;
  size_t off_qkv = 0, off_q = 0, off_qlo = 0, off_k = 0, off_v = 0, off_part = 0, off_x = 0,
         bytes = 0;
  size_t off_kpart = 0, off_kcnt = 0, off_acnt = 0;
  // full layer (inter > 0): normalised rows, fp32 q/k/v, h1 and the MLP activation
  size_t off_xn = 0, off_qkv32 = 0, off_h1 = 0, off_act = 0;
};

AttnWs attn_ws_layout(int dtype, int nseq, int n_rows, int64_t max_prefix, int d_model, int Hq,
                      int Hkv, int D, int inter = 0) {
  AttnWs w;
  const size_t R = static_cast<size_t>(nseq) * n_rows;
  size_t off = 0;
  auto take = [&](size_t bytes) {
    const size_t o = off;
    off += round256(bytes);
    return o;
  };
  if (dtype == GLANCE_BF16) {
    w.off_q = take(R * Hq * D * 2);
    w.off_qlo = take(R * Hq * D * 2);
    w.off_k = take(R * Hkv * D * 2);
    w.off_v = take(R * Hkv * D * 2);
    w.n_split = attn_splits(nseq, max_prefix, n_rows, Hq, Hkv);
    w.off_part = take(attn_part_floats(nseq, n_rows, Hq, Hkv, w.n_split) * sizeof(float));
    // arrival counters of the attention's in-kernel split merge (returned to zero)
    w.off_acnt = take(attn_arrival_words(nseq, n_rows, Hq, Hkv) * sizeof(unsigned));
    w.off_x = take(R * Hq * D * sizeof(float));
    // split-K scratch shared by the projections (q/k/v, output and, in a full
    // layer, gate/up and down)
    const int M = static_cast<int>(R);
    const int nb_qkv = (Hq + 2 * Hkv) * 8, nb_o = (d_model + 15) / 16;
    size_t pf = std::max(proj_part_floats(M, nb_qkv, d_model), proj_part_floats(M, nb_o, Hq * D));
    size_t nc = std::max(proj_counters(M, nb_qkv, d_model), proj_counters(M, nb_o, Hq * D));
    if (inter > 0) {
      const int nb_gu = 2 * inter / 16;
      pf = std::max({pf, proj_part_floats(M, nb_gu, d_model), proj_part_floats(M, nb_o, inter)});
      nc = std::max({nc, proj_counters(M, nb_gu, d_model), proj_counters(M, nb_o, inter)});
    }
    w.off_kpart = take(pf * sizeof(float));
    // arrival counters of the split-K groups (each projection returns them to zero)
    w.off_kcnt = take(nc * sizeof(unsigned));
    if (inter > 0) {
      w.off_xn = take(R * d_model * 2);
      w.off_qkv32 = take(R * static_cast<size_t>(Hq + 2 * Hkv) * D * sizeof(float));
      w.off_h1 = take(R * d_model * 2);
      w.off_act = take(R * static_cast<size_t>(inter) * 2);
    }
  } else {
    w.off_qkv = take(R * static_cast<size_t>(Hq + 2 * Hkv) * D * sizeof(float));
    w.off_x = take(R * Hq * D * sizeof(float));
  }
  w.bytes = off;
  return w;
}

}  // namespace

glance_status hip_fail(hipError_t e) {
  g_last_error = std::string("HIP error: ") + hipGetErrorString(e);
  return GLANCE_ERR_HIP;
}

}  // namespace glance

using namespace glance;

extern "C" {

const char* glance_status_string(int32_t status) {
  switch (status) {
    case GLANCE_OK: return "ok";
    case GLANCE_ERR_INVALID_ARG: return "invalid argument";
    case GLANCE_ERR_ALIGNMENT: return "misaligned device pointer";
    case GLANCE_ERR_WORKSPACE: return "workspace missing, misaligned or too small";
    case GLANCE_ERR_UNSUPPORTED: return "unsupported shape";
    case GLANCE_ERR_HIP: return "HIP launch failure";
    default: return "unknown status";
  }
}

const char* glance_last_error(void) { return g_last_error.c_str(); }

int32_t glance_abi_version(void) { return 1; }

// ------------------------------------------------------------------ step 1+2
size_t glance_build_tree_ws(int32_t nseq, int32_t L, int32_t V, int32_t N) {
  (void)N;
  if (nseq < 1 || L < 1 || L > GLANCE_MAX_L || V < 2 || V > (1 << 18)) return 0;
  return tree_ws_layout(nseq, L, V).bytes;
}

size_t glance_build_tree_flag_offset(int32_t nseq, int32_t L, int32_t V, int32_t N) {
  if (glance_build_tree_ws(nseq, L, V, N) == 0) return 0;
  return tree_ws_layout(nseq, L, V).off_flag;
}

glance_status glance_build_tree(const void* draft_logits, int32_t dtype,
                                const int32_t* root_token, int32_t nseq, int32_t L,
                                int32_t V, int32_t N, int32_t* parent, int32_t* depth,
                                int32_t* token, uint64_t* anc, float* score,
                                int32_t* n_valid, void* ws, size_t ws_bytes, void* stream) {
  g_last_error.clear();
  REQUIRE(dtype == GLANCE_F32 || dtype == GLANCE_BF16, "dtype %d is not GLANCE_F32/BF16", dtype);
  REQUIRE(nseq >= 1, "nseq = %d < 1", nseq);
  REQUIRE(L >= 1 && L <= GLANCE_MAX_L, "L = %d outside [1, %d]", L, GLANCE_MAX_L);
  REQUIRE(V >= 2, "V = %d < 2", V);
  REQUIRE(N >= 0 && N <= GLANCE_MAX_ROWS - 1, "N = %d outside [0, %d]", N, GLANCE_MAX_ROWS - 1);
  if (V > (dtype == GLANCE_BF16 ? (1 << 18) : (1 << 17)))
    return fail(GLANCE_ERR_UNSUPPORTED, "V = %d above 2^18 (bf16) / 2^17 (fp32)", V);
  REQUIRE_PTR(draft_logits);
  REQUIRE_PTR(root_token);
  REQUIRE_PTR(parent);
  REQUIRE_PTR(depth);
  REQUIRE_PTR(token);
  REQUIRE_PTR(anc);
  REQUIRE_PTR(score);
  REQUIRE_PTR(n_valid);
  const TreeWs w = tree_ws_layout(nseq, L, V);
  glance_status st = check_ws(ws, ws_bytes, w.bytes);
  if (st != GLANCE_OK) return st;
  return launch_build_tree(draft_logits, dtype, root_token, nseq, L, V, N, parent, depth, token,
                           anc, score, n_valid, ws, static_cast<hipStream_t>(stream));
}

glance_status glance_build_tree_shared(const void* draft_logits, int32_t dtype,
                                       const int32_t* root_token, const float* log_weight,
                                       int32_t nseq, int32_t L, int32_t V, int32_t n_max,
                                       int32_t budget, float min_log_value, int32_t* parent,
                                       int32_t* depth, int32_t* token, uint64_t* anc, float* score,
                                       int32_t* n_valid, void* ws, size_t ws_bytes, void* stream) {
  g_last_error.clear();
  REQUIRE(dtype == GLANCE_F32 || dtype == GLANCE_BF16, "dtype %d is not GLANCE_F32/BF16", dtype);
  REQUIRE(nseq >= 1 && nseq <= GLANCE_MAX_SHARED, "nseq = %d outside [1, %d]", nseq, GLANCE_MAX_SHARED);
  REQUIRE(L >= 1 && L <= GLANCE_MAX_L, "L = %d outside [1, %d]", L, GLANCE_MAX_L);
  REQUIRE(V >= 2, "V = %d < 2", V);
  REQUIRE(n_max >= 0 && n_max <= GLANCE_MAX_ROWS - 1, "n_max = %d outside [0, %d]", n_max,
          GLANCE_MAX_ROWS - 1);
  REQUIRE(budget >= 0, "budget = %d < 0", budget);
  REQUIRE(!std::isnan(min_log_value), "min_log_value is NaN");
  if (V > (dtype == GLANCE_BF16 ? (1 << 18) : (1 << 17)))
    return fail(GLANCE_ERR_UNSUPPORTED, "V = %d above 2^18 (bf16) / 2^17 (fp32)", V);
  REQUIRE_PTR(draft_logits);
  REQUIRE_PTR(root_token);
  REQUIRE_PTR(log_weight);
  REQUIRE_PTR(parent);
  REQUIRE_PTR(depth);
  REQUIRE_PTR(token);
  REQUIRE_PTR(anc);
  REQUIRE_PTR(score);
  REQUIRE_PTR(n_valid);
  const TreeWs w = tree_ws_layout(nseq, L, V);
  glance_status st = check_ws(ws, ws_bytes, w.bytes);
  if (st != GLANCE_OK) return st;
  return launch_build_tree(draft_logits, dtype, root_token, nseq, L, V, n_max, parent, depth, token,
                           anc, score, n_valid, ws, static_cast<hipStream_t>(stream), log_weight,
                           budget, min_log_value);
}

glance_status glance_entropy_log_value(const float* entropy, int32_t nseq, int32_t stride, float b0,
                                       float b1, int32_t L, float* log_weight, void* stream) {
  g_last_error.clear();
  REQUIRE(nseq >= 1, "nseq = %d < 1", nseq);
  REQUIRE(stride >= 1, "stride = %d < 1", stride);
  REQUIRE(L >= 1, "L = %d < 1", L);
  REQUIRE(std::isfinite(b0) && std::isfinite(b1), "b0 = %g, b1 = %g are not both finite",
          static_cast<double>(b0), static_cast<double>(b1));
  REQUIRE(entropy != nullptr, "entropy is NULL");
  REQUIRE(log_weight != nullptr, "log_weight is NULL");
  if ((reinterpret_cast<uintptr_t>(entropy) & 3u) || (reinterpret_cast<uintptr_t>(log_weight) & 3u))
    return fail(GLANCE_ERR_ALIGNMENT, "entropy and log_weight must be 4-byte aligned");
  return launch_entropy_log_value(entropy, nseq, stride, b0, b1, L, log_weight,
                                  static_cast<hipStream_t>(stream));
}

// ------------------------------------------------------------------- step 3
size_t glance_tree_attn_ws(int32_t nseq, int32_t n_rows, int64_t max_prefix, int32_t d_model,
                           int32_t Hq, int32_t Hkv, int32_t D) {
  if (nseq < 1 || n_rows < 1 || n_rows > GLANCE_MAX_ROWS || max_prefix < 0 || Hkv < 1 ||
      Hq < Hkv || D < 2 || D > 128 || d_model < 1 || !attn_in_bounds(nseq, max_prefix, d_model, Hq, 0))
    return 0;
  // the larger of the two dtypes' layouts, so one size fits either
  const AttnWs a = attn_ws_layout(GLANCE_BF16, nseq, n_rows, max_prefix, d_model, Hq, Hkv, D);
  const AttnWs b = attn_ws_layout(GLANCE_F32, nseq, n_rows, max_prefix, d_model, Hq, Hkv, D);
  return a.bytes > b.bytes ? a.bytes : b.bytes;
}

glance_status glance_tree_attn(const glance_attn_layer* layer, int32_t dtype, const void* embed,
                               const int32_t* token, const void* h_in, void* h_out,
                               const int64_t* kv_offsets, int64_t max_prefix,
                               const int32_t* depth, const uint64_t* anc,
                               const float* rope_cos, const float* rope_sin, int32_t n_pos,
                               int32_t nseq, int32_t n_rows, int32_t d_model, int32_t Hq,
                               int32_t Hkv, int32_t D, float* attn_out, void* tree_k,
                               void* tree_v, void* ws, size_t ws_bytes, void* stream) {
  g_last_error.clear();
  REQUIRE(layer != nullptr, "layer is NULL");
  REQUIRE(dtype == GLANCE_F32 || dtype == GLANCE_BF16, "dtype %d is not GLANCE_F32/BF16", dtype);
  REQUIRE(nseq >= 1, "nseq = %d < 1", nseq);
  REQUIRE(n_rows >= 1 && n_rows <= GLANCE_MAX_ROWS, "n_rows = %d outside [1, %d]", n_rows,
          GLANCE_MAX_ROWS);
  REQUIRE(Hkv >= 1 && Hq >= Hkv && Hq % Hkv == 0, "Hq = %d is not a multiple of Hkv = %d", Hq, Hkv);
  REQUIRE(d_model >= 1, "d_model = %d < 1", d_model);
  REQUIRE(max_prefix >= 0, "max_prefix < 0");
  REQUIRE(embed != nullptr || h_in != nullptr, "both embed and h_in are NULL");
  REQUIRE(max_prefix <= static_cast<int64_t>(n_pos) - n_rows,
          "n_pos = %d is below max_prefix %lld + n_rows %d (every row's position P + depth "
          "needs a table row)", n_pos, static_cast<long long>(max_prefix), n_rows);
  if (dtype == GLANCE_BF16) {
    if (D != 128) return fail(GLANCE_ERR_UNSUPPORTED, "bf16 tree attention needs D = 128 (got %d)", D);
    if (d_model % 256 != 0 || (Hq * D) % 256 != 0)
      return fail(GLANCE_ERR_UNSUPPORTED, "bf16 needs d_model and Hq*D multiples of 256");
  } else {
    if (D < 2 || D > 128 || D % 2 != 0)
      return fail(GLANCE_ERR_UNSUPPORTED, "fp32 tree attention needs even D <= 128 (got %d)", D);
    if (max_prefix > 8192)
      return fail(GLANCE_ERR_UNSUPPORTED, "fp32 tree attention needs max_prefix <= 8192");
    if (layer->packed)
      return fail(GLANCE_ERR_UNSUPPORTED, "packed attention weights are bf16 only");
  }
  if (layer->packed) {
    REQUIRE_PTR(layer->packed);
  } else {
    REQUIRE_PTR(layer->wq);
    REQUIRE_PTR(layer->wk);
    REQUIRE_PTR(layer->wv);
    REQUIRE_PTR(layer->wo);
  }
  REQUIRE_PTR(layer->k_cache);
  REQUIRE_PTR(layer->v_cache);
  REQUIRE_ALIGNED_OR_NULL(embed);
  REQUIRE_ALIGNED_OR_NULL(h_in);
  REQUIRE_PTR(token);
  REQUIRE_PTR(h_out);
  REQUIRE_PTR(kv_offsets);
  REQUIRE_PTR(depth);
  REQUIRE_PTR(anc);
  REQUIRE_PTR(rope_cos);
  REQUIRE_PTR(rope_sin);
  REQUIRE_ALIGNED_OR_NULL(attn_out);
  REQUIRE_ALIGNED_OR_NULL(tree_k);
  REQUIRE_ALIGNED_OR_NULL(tree_v);
  if (!attn_in_bounds(nseq, max_prefix, d_model, Hq, 0))
    return fail(GLANCE_ERR_UNSUPPORTED, "shape beyond the library's bounds (nseq <= %d, max_prefix "
                "<= %lld, d_model <= %d, Hq <= %d)", kMaxSeqs, static_cast<long long>(kMaxPrefix),
                kMaxDModel, kMaxHeads);
  const AttnWs w = attn_ws_layout(dtype, nseq, n_rows, max_prefix, d_model, Hq, Hkv, D);
  glance_status st = check_ws(ws, ws_bytes, w.bytes);
  if (st != GLANCE_OK) return st;

  hipStream_t hs = static_cast<hipStream_t>(stream);
  char* base = static_cast<char*>(ws);
  float* attn_x = reinterpret_cast<float*>(base + w.off_x);
  const int R = nseq * n_rows;
  const int qd = Hq * D, kd = Hkv * D;
  float* kpart = reinterpret_cast<float*>(base + w.off_kpart);
  unsigned* kcnt = reinterpret_cast<unsigned*>(base + w.off_kcnt);
  if (dtype == GLANCE_BF16) {
    if (tree_k == nullptr) tree_k = base + w.off_k;
    if (tree_v == nullptr) tree_v = base + w.off_v;
  }

  // 1. q, k, v of every row (layer input: embedding rows or h_in)
  GemmArgs g{};
  g.x = embed ? embed : h_in;
  g.gather = embed ? token : nullptr;
  g.w.w[0] = layer->wq;
  g.w.w[1] = layer->wk;
  g.w.w[2] = layer->wv;
  g.w.n_end[0] = qd;
  g.w.n_end[1] = qd + kd;
  g.w.n_end[2] = qd + 2 * kd;
  g.w.nseg = 3;
  g.M = R;
  g.N = qd + 2 * kd;
  g.K = d_model;
  if (dtype == GLANCE_BF16) {
    g.epi = EPI_QKV;
    g.w_packed = layer->packed;
    g.Hq = Hq;
    g.Hkv = Hkv;
    g.q_out = base + w.off_q;
    g.q_lo_out = base + w.off_qlo;
    g.k_out = tree_k;
    g.v_out = tree_v;
    g.kv_offsets = kv_offsets;
    g.depth = depth;
    g.n_rows = n_rows;
    g.rope_cos = rope_cos;
    g.rope_sin = rope_sin;
    g.n_pos = n_pos;
    g.kpart = kpart;
    g.kcnt = kcnt;
    st = launch_gemm_bf16(g, hs);
  } else {
    g.epi = EPI_STORE_F32;
    g.out_f32 = reinterpret_cast<float*>(base + w.off_qkv);
    st = launch_gemm_f32(g, hs);
  }
  if (st != GLANCE_OK) return st;

  // 2. attention over prefix + ancestors
  AttnArgs a{};
  a.dtype = dtype;
  a.qkv = reinterpret_cast<const float*>(base + w.off_qkv);
  a.q = base + w.off_q;
  a.q_lo = base + w.off_qlo;
  a.k_cache = layer->k_cache;
  a.v_cache = layer->v_cache;
  a.kv_offsets = kv_offsets;
  a.depth = depth;
  a.anc = anc;
  a.token = token;
  a.rope_cos = rope_cos;
  a.rope_sin = rope_sin;
  a.n_pos = n_pos;
  a.nseq = nseq;
  a.n_rows = n_rows;
  a.Hq = Hq;
  a.Hkv = Hkv;
  a.D = D;
  a.max_prefix = max_prefix;
  a.n_split = w.n_split;
  a.part = reinterpret_cast<float*>(base + w.off_part);
  a.arrivals = reinterpret_cast<unsigned*>(base + w.off_acnt);
  a.attn_out = attn_out;
  a.attn_x = attn_x;
  a.tree_k = tree_k;
  a.tree_v = tree_v;
  st = launch_tree_attention(a, hs);
  if (st != GLANCE_OK) return st;

  // 3. h_out = h_in + attn Wo^T (padding rows -> 0); the fp32 attention output
  // enters the bf16 products as its rounding plus the rounded remainder
  GemmArgs o{};
  o.x = attn_x;
  o.x_f32 = dtype == GLANCE_BF16;
  o.gather = nullptr;
  o.w.w[0] = layer->wo;
  o.w.n_end[0] = d_model;
  o.w.nseg = 1;
  o.M = R;
  o.N = d_model;
  o.K = qd;
  o.epi = EPI_RESID;
  o.resid = embed ? embed : h_in;
  o.resid_tok = token;
  o.resid_by_token = embed != nullptr;
  o.out_res = h_out;
  o.kpart = kpart;
  o.kcnt = kcnt;
  if (layer->packed) o.w_packed = packed_wo(layer->packed, d_model, Hq, Hkv, D);
  return dtype == GLANCE_BF16 ? launch_gemm_bf16(o, hs) : launch_gemm_f32(o, hs);
}

// --------------------------------------------------------- step 3, full layer
size_t glance_tree_layer_ws(int32_t nseq, int32_t n_rows, int64_t max_prefix, int32_t d_model,
                            int32_t Hq, int32_t Hkv, int32_t D, int32_t inter) {
  if (nseq < 1 || n_rows < 1 || n_rows > GLANCE_MAX_ROWS || max_prefix < 0 || Hkv < 1 ||
      Hq < Hkv || D != 128 || inter < 256 || d_model < 256 ||
      !attn_in_bounds(nseq, max_prefix, d_model, Hq, inter))
    return 0;
  return attn_ws_layout(GLANCE_BF16, nseq, n_rows, max_prefix, d_model, Hq, Hkv, D, inter).bytes;
}

glance_status glance_tree_layer(const glance_full_layer* layer, const void* embed,
                                const int32_t* token, const void* h_in, void* h_out,
                                const int64_t* kv_offsets, int64_t max_prefix, const int32_t* depth,
                                const uint64_t* anc, const float* rope_cos, const float* rope_sin,
                                int32_t n_pos, int32_t nseq, int32_t n_rows, int32_t d_model,
                                int32_t Hq, int32_t Hkv, int32_t D, float* attn_out, void* tree_k,
                                void* tree_v, void* ws, size_t ws_bytes, void* stream) {
  g_last_error.clear();
  REQUIRE(layer != nullptr, "layer is NULL");
  REQUIRE(nseq >= 1, "nseq = %d < 1", nseq);
  REQUIRE(n_rows >= 1 && n_rows <= GLANCE_MAX_ROWS, "n_rows = %d outside [1, %d]", n_rows,
          GLANCE_MAX_ROWS);
  REQUIRE(Hkv >= 1 && Hq >= Hkv && Hq % Hkv == 0, "Hq = %d is not a multiple of Hkv = %d", Hq, Hkv);
  REQUIRE(d_model >= 1, "d_model = %d < 1", d_model);
  REQUIRE(max_prefix >= 0, "max_prefix < 0");
  REQUIRE(embed != nullptr || h_in != nullptr, "both embed and h_in are NULL");
  REQUIRE(max_prefix <= static_cast<int64_t>(n_pos) - n_rows,
          "n_pos = %d is below max_prefix %lld + n_rows %d (every row's position P + depth "
          "needs a table row)", n_pos, static_cast<long long>(max_prefix), n_rows);
  REQUIRE(std::isfinite(layer->eps) && layer->eps >= 0.f, "eps = %g is not finite and >= 0",
          static_cast<double>(layer->eps));
  const int inter = layer->inter;
  if (D != 128 || d_model % 256 != 0 || (Hq * D) % 256 != 0 || inter < 256 || inter % 256 != 0)
    return fail(GLANCE_ERR_UNSUPPORTED,
                "full layer needs D = 128 and d_model, Hq*D, inter multiples of 256 (got D %d, "
                "d_model %d, Hq*D %d, inter %d)", D, d_model, Hq * D, inter);
  const glance_attn_layer* at = &layer->attn;
  if (at->packed) {
    REQUIRE_PTR(at->packed);
  } else {
    REQUIRE_PTR(at->wq);
    REQUIRE_PTR(at->wk);
    REQUIRE_PTR(at->wv);
    REQUIRE_PTR(at->wo);
  }
  REQUIRE_PTR(at->k_cache);
  REQUIRE_PTR(at->v_cache);
  REQUIRE_PTR(layer->g_attn);
  REQUIRE_PTR(layer->g_q);
  REQUIRE_PTR(layer->g_k);
  REQUIRE_PTR(layer->g_mlp);
  if (layer->mlp_packed) {
    REQUIRE_PTR(layer->mlp_packed);
  } else {
    REQUIRE_PTR(layer->w_gate);
    REQUIRE_PTR(layer->w_up);
    REQUIRE_PTR(layer->w_down);
  }
  REQUIRE_ALIGNED_OR_NULL(embed);
  REQUIRE_ALIGNED_OR_NULL(h_in);
  REQUIRE_PTR(token);
  REQUIRE_PTR(h_out);
  REQUIRE_PTR(kv_offsets);
  REQUIRE_PTR(depth);
  REQUIRE_PTR(anc);
  REQUIRE_PTR(rope_cos);
  REQUIRE_PTR(rope_sin);
  REQUIRE_ALIGNED_OR_NULL(attn_out);
  REQUIRE_ALIGNED_OR_NULL(tree_k);
  REQUIRE_ALIGNED_OR_NULL(tree_v);
  if (!attn_in_bounds(nseq, max_prefix, d_model, Hq, inter))
    return fail(GLANCE_ERR_UNSUPPORTED, "shape beyond the library's bounds (nseq <= %d, max_prefix "
                "<= %lld, d_model <= %d, Hq <= %d, inter <= %d)", kMaxSeqs,
                static_cast<long long>(kMaxPrefix), kMaxDModel, kMaxHeads, kMaxInter);
  const AttnWs w = attn_ws_layout(GLANCE_BF16, nseq, n_rows, max_prefix, d_model, Hq, Hkv, D, inter);
  glance_status st = check_ws(ws, ws_bytes, w.bytes);
  if (st != GLANCE_OK) return st;

  hipStream_t hs = static_cast<hipStream_t>(stream);
  char* base = static_cast<char*>(ws);
  const int R = nseq * n_rows;
  const int qd = Hq * D, kd = Hkv * D;
  float* kpart = reinterpret_cast<float*>(base + w.off_kpart);
  unsigned* kcnt = reinterpret_cast<unsigned*>(base + w.off_kcnt);
  void* xn = base + w.off_xn;
  void* h1 = base + w.off_h1;
  void* act = base + w.off_act;
  float* qkv32 = reinterpret_cast<float*>(base + w.off_qkv32);
  if (tree_k == nullptr) tree_k = base + w.off_k;
  if (tree_v == nullptr) tree_v = base + w.off_v;
  const void* h0 = embed ? embed : h_in;

  // 1. x = RMSNorm(h) g_attn; 2. q, k, v in fp32; 3. q/k head norms, RoPE, bf16
  st = launch_rmsnorm(h0, embed ? token : nullptr, token, R, d_model, layer->g_attn, layer->eps, xn, hs);
  if (st != GLANCE_OK) return st;
  GemmArgs g{};
  g.x = xn;
  g.w.w[0] = at->wq;
  g.w.w[1] = at->wk;
  g.w.w[2] = at->wv;
  g.w.n_end[0] = qd;
  g.w.n_end[1] = qd + kd;
  g.w.n_end[2] = qd + 2 * kd;
  g.w.nseg = 3;
  g.M = R;
  g.N = qd + 2 * kd;
  g.K = d_model;
  g.epi = EPI_STORE_F32;
  g.w_packed = at->packed;
  g.Hq = Hq;
  g.Hkv = Hkv;
  g.out_f32 = qkv32;
  g.kpart = kpart;
  g.kcnt = kcnt;
  st = launch_gemm_bf16(g, hs);
  if (st != GLANCE_OK) return st;
  st = launch_qkv_finish(qkv32, R, Hq, Hkv, layer->g_q, layer->g_k, layer->eps, kv_offsets, depth,
                         n_rows, rope_cos, rope_sin, n_pos, base + w.off_q, base + w.off_qlo,
                         tree_k, tree_v, hs);
  if (st != GLANCE_OK) return st;

  // 4. attention over prefix + ancestors
  AttnArgs a{};
  a.dtype = GLANCE_BF16;
  a.q = base + w.off_q;
  a.q_lo = base + w.off_qlo;
  a.k_cache = at->k_cache;
  a.v_cache = at->v_cache;
  a.kv_offsets = kv_offsets;
  a.depth = depth;
  a.anc = anc;
  a.token = token;
  a.rope_cos = rope_cos;
  a.rope_sin = rope_sin;
  a.n_pos = n_pos;
  a.nseq = nseq;
  a.n_rows = n_rows;
  a.Hq = Hq;
  a.Hkv = Hkv;
  a.D = D;
  a.max_prefix = max_prefix;
  a.n_split = w.n_split;
  a.part = reinterpret_cast<float*>(base + w.off_part);
  a.arrivals = reinterpret_cast<unsigned*>(base + w.off_acnt);
  a.attn_out = attn_out;
  a.attn_x = reinterpret_cast<float*>(base + w.off_x);
  a.tree_k = tree_k;
  a.tree_v = tree_v;
  st = launch_tree_attention(a, hs);
  if (st != GLANCE_OK) return st;

  // 5. h1 = h + attn Wo^T
  GemmArgs o{};
  o.x = base + w.off_x;
  o.x_f32 = true;
  o.w.w[0] = at->wo;
  o.w.n_end[0] = d_model;
  o.w.nseg = 1;
  o.M = R;
  o.N = d_model;
  o.K = qd;
  o.epi = EPI_RESID;
  o.resid = h0;
  o.resid_tok = token;
  o.resid_by_token = embed != nullptr;
  o.out_res = h1;
  o.kpart = kpart;
  o.kcnt = kcnt;
  if (at->packed) o.w_packed = packed_wo(at->packed, d_model, Hq, Hkv, D);
  st = launch_gemm_bf16(o, hs);
  if (st != GLANCE_OK) return st;

  // 6. x2 = RMSNorm(h1) g_mlp; 7. act = silu(x2 Wg^T) * (x2 Wu^T); 8. h' = h1 + act Wd^T
  st = launch_rmsnorm(h1, nullptr, token, R, d_model, layer->g_mlp, layer->eps, xn, hs);
  if (st != GLANCE_OK) return st;
  GemmArgs gu{};
  gu.x = xn;
  gu.w.w[0] = layer->w_gate;
  gu.w.w[1] = layer->w_up;
  gu.w.n_end[0] = inter;
  gu.w.n_end[1] = 2 * inter;
  gu.w.nseg = 2;
  gu.M = R;
  gu.N = 2 * inter;
  gu.K = d_model;
  gu.epi = EPI_SWIGLU;
  gu.w_packed = layer->mlp_packed;
  gu.out_res = act;
  gu.kpart = kpart;
  gu.kcnt = kcnt;
  st = launch_gemm_bf16(gu, hs);
  if (st != GLANCE_OK) return st;
  GemmArgs dn{};
  dn.x = act;
  dn.w.w[0] = layer->w_down;
  dn.w.n_end[0] = d_model;
  dn.w.nseg = 1;
  dn.M = R;
  dn.N = d_model;
  dn.K = inter;
  dn.epi = EPI_RESID;
  dn.resid = h1;
  dn.resid_tok = token;
  dn.resid_by_token = false;
  dn.out_res = h_out;
  dn.kpart = kpart;
  dn.kcnt = kcnt;
  if (layer->mlp_packed)
    dn.w_packed = static_cast<const char*>(layer->mlp_packed) + round256(proj_pack_bytes(2 * inter, d_model));
  return launch_gemm_bf16(dn, hs);
}

size_t glance_attn_pack_bytes(int32_t d_model, int32_t Hq, int32_t Hkv, int32_t D) {
  if (d_model < 256 || d_model % 256 != 0 || Hkv < 1 || Hq < Hkv || Hq % Hkv != 0 || D != 128 ||
      d_model > kMaxDModel || Hq > kMaxHeads)
    return 0;
  const int qd = Hq * D, kd = Hkv * D;
  if (qd % 256 != 0) return 0;
  return round256(proj_pack_bytes(qd + 2 * kd, d_model)) + proj_pack_bytes(d_model, qd);
}

glance_status glance_attn_pack(const void* wq, const void* wk, const void* wv, const void* wo,
                               int32_t d_model, int32_t Hq, int32_t Hkv, int32_t D, void* packed,
                               void* stream) {
  g_last_error.clear();
  if (glance_attn_pack_bytes(d_model, Hq, Hkv, D) == 0)
    return fail(GLANCE_ERR_UNSUPPORTED, "packed attention weights need D = 128, Hq a multiple of "
                "Hkv and d_model, Hq*D multiples of 256 (got d_model %d, Hq %d, Hkv %d, D %d)",
                d_model, Hq, Hkv, D);
  REQUIRE_PTR(wq);
  REQUIRE_PTR(wk);
  REQUIRE_PTR(wv);
  REQUIRE_PTR(wo);
  REQUIRE_PTR(packed);
  hipStream_t hs = static_cast<hipStream_t>(stream);
  const int qd = Hq * D, kd = Hkv * D;
  GemmArgs g{};
  g.w.w[0] = wq;
  g.w.w[1] = wk;
  g.w.w[2] = wv;
  g.w.n_end[0] = qd;
  g.w.n_end[1] = qd + kd;
  g.w.n_end[2] = qd + 2 * kd;
  g.w.nseg = 3;
  g.N = qd + 2 * kd;
  g.K = d_model;
  g.epi = EPI_QKV;
  g.Hq = Hq;
  g.Hkv = Hkv;
  glance_status st = launch_proj_pack(g, packed, hs);
  if (st != GLANCE_OK) return st;
  GemmArgs o{};
  o.w.w[0] = wo;
  o.w.n_end[0] = d_model;
  o.w.nseg = 1;
  o.N = d_model;
  o.K = qd;
  o.epi = EPI_RESID;
  return launch_proj_pack(o, const_cast<void*>(packed_wo(packed, d_model, Hq, Hkv, D)), hs);
}

size_t glance_mlp_pack_bytes(int32_t d_model, int32_t inter) {
  if (d_model < 256 || d_model % 256 != 0 || inter < 256 || inter % 256 != 0 ||
      d_model > kMaxDModel || inter > kMaxInter)
    return 0;
  return round256(proj_pack_bytes(2 * inter, d_model)) + proj_pack_bytes(d_model, inter);
}

glance_status glance_mlp_pack(const void* w_gate, const void* w_up, const void* w_down,
                              int32_t d_model, int32_t inter, void* packed, void* stream) {
  g_last_error.clear();
  if (glance_mlp_pack_bytes(d_model, inter) == 0)
    return fail(GLANCE_ERR_UNSUPPORTED, "packed MLP needs d_model and inter multiples of 256 (got %d, %d)",
                d_model, inter);
  REQUIRE_PTR(w_gate);
  REQUIRE_PTR(w_up);
  REQUIRE_PTR(w_down);
  REQUIRE_PTR(packed);
  hipStream_t hs = static_cast<hipStream_t>(stream);
  GemmArgs gu{};
  gu.w.w[0] = w_gate;
  gu.w.w[1] = w_up;
  gu.w.n_end[0] = inter;
  gu.w.n_end[1] = 2 * inter;
  gu.w.nseg = 2;
  gu.N = 2 * inter;
  gu.K = d_model;
  gu.epi = EPI_SWIGLU;
  glance_status st = launch_proj_pack(gu, packed, hs);
  if (st != GLANCE_OK) return st;
  GemmArgs dn{};
  dn.w.w[0] = w_down;
  dn.w.n_end[0] = d_model;
  dn.w.nseg = 1;
  dn.N = d_model;
  dn.K = inter;
  dn.epi = EPI_RESID;
  return launch_proj_pack(dn, static_cast<char*>(packed) + round256(proj_pack_bytes(gu.N, d_model)), hs);
}

// ------------------------------------------------------------------- step 4
size_t glance_verify_head_ws(int32_t R, int32_t V, int32_t d_model, int32_t dtype) {
  if (R < 1 || V < 2 || !head_in_bounds(R, V, d_model)) return 0;
  // bf16: 5 floats of statistics and 3 of the sampled draw per row and partial,
  // then the arrival counter of glance_verify_head_walk
  if (dtype == GLANCE_BF16)
    return round256(static_cast<size_t>(R) * gemm_bf16_head_parts(V) * 8 * sizeof(float)) + 256;
  return round256(static_cast<size_t>(R) * V * sizeof(float));
}

// Events of glance_head_timing (process-wide; null: not recorded).
static hipEvent_t g_head_ev_start = nullptr;
static hipEvent_t g_head_ev_stop = nullptr;

// One of the timing events on the head GEMM's stream, when the hook is set.
static glance_status head_event(hipEvent_t ev, hipStream_t hs) {
  if (!ev) return GLANCE_OK;
  const hipError_t e = hipEventRecord(ev, hs);
  return e == hipSuccess ? GLANCE_OK : hip_fail(e);
}

static glance_status verify_head(const void* h, const void* w_head, const void* w_packed,
                                 int32_t dtype, int32_t R, int32_t d_model, int32_t V,
                                 int32_t* argmax, float* top1, float* gap, float* entropy,
                                 float* logits, void* ws, size_t ws_bytes, HeadDraw dr,
                                 hipStream_t hs, const WalkArgs* wk = nullptr) {
  REQUIRE(dtype == GLANCE_F32 || dtype == GLANCE_BF16, "dtype %d is not GLANCE_F32/BF16", dtype);
  REQUIRE(R >= 1, "R = %d < 1", R);
  REQUIRE(V >= 2, "V = %d < 2", V);
  REQUIRE(d_model >= 1, "d_model = %d < 1", d_model);
  if (dtype == GLANCE_BF16 && d_model % 256 != 0)
    return fail(GLANCE_ERR_UNSUPPORTED, "bf16 head needs d_model %% 256 == 0 (got %d)", d_model);
  if (!head_in_bounds(R, V, d_model))
    return fail(GLANCE_ERR_UNSUPPORTED, "head beyond the library's bounds (R <= %d, V <= %d, "
                "d_model <= %d)", kMaxHeadRows, kMaxHeadVocab, kMaxDModel);
  REQUIRE_PTR(h);
  if (w_packed)
    REQUIRE_PTR(w_packed);
  else
    REQUIRE_PTR(w_head);
  REQUIRE_PTR(argmax);
  REQUIRE_PTR(top1);
  REQUIRE_PTR(gap);
  REQUIRE_PTR(entropy);
  REQUIRE_ALIGNED_OR_NULL(logits);
  const size_t need = glance_verify_head_ws(R, V, d_model, dtype);
  glance_status st = check_ws(ws, ws_bytes, need);
  if (st != GLANCE_OK) return st;
  GemmArgs g{};
  g.x = h;
  g.w.w[0] = w_head;
  g.w.n_end[0] = V;
  g.w.nseg = 1;
  g.M = R;
  g.N = V;
  g.K = d_model;
  g.epi = EPI_HEAD;
  if (dtype == GLANCE_BF16) {
    const int parts = gemm_bf16_head_parts(V);
    g.w_packed = w_packed;
    g.part = static_cast<float*>(ws);
    g.logits = logits;
    if (dr.tok) {
      g.spart = g.part + static_cast<size_t>(R) * parts * 5;
      g.inv_temp = dr.inv_temp;
      g.seed_lo = dr.seed_lo;
      g.seed_hi = dr.seed_hi;
      g.rnd_lo = dr.rnd_lo;
      g.rnd_hi = dr.rnd_hi;
      dr.spart = g.spart;
    }
    const hipEvent_t e0 = g_head_ev_start, e1 = g_head_ev_stop;
    st = head_event(e0, hs);
    if (st == GLANCE_OK) st = launch_gemm_bf16(g, hs);
    if (st == GLANCE_OK) st = head_event(e1, hs);
    if (st != GLANCE_OK) return st;
    if (wk) {
      unsigned* arrivals = reinterpret_cast<unsigned*>(static_cast<char*>(ws) + need - 256);
      return launch_head_merge_walk(g.part, parts, R, argmax, top1, gap, entropy, dr, *wk, arrivals,
                                    hs);
    }
    return launch_head_merge(g.part, parts, R, argmax, top1, gap, entropy, dr, hs);
  }
  g.logits = logits ? logits : static_cast<float*>(ws);
  const hipEvent_t e0 = g_head_ev_start, e1 = g_head_ev_stop;
  st = head_event(e0, hs);
  if (st == GLANCE_OK) st = launch_gemm_f32(g, hs);
  if (st == GLANCE_OK) st = head_event(e1, hs);
  if (st != GLANCE_OK) return st;
  return launch_head_rowstats_f32(g.logits, R, V, argmax, top1, gap, entropy, dr, hs);
}

glance_status glance_verify_head(const void* h, const void* w_head, int32_t dtype, int32_t R,
                                 int32_t d_model, int32_t V, int32_t* argmax, float* top1,
                                 float* gap, float* entropy, float* logits, void* ws,
                                 size_t ws_bytes, void* stream) {
  g_last_error.clear();
  return verify_head(h, w_head, nullptr, dtype, R, d_model, V, argmax, top1, gap, entropy, logits,
                     ws, ws_bytes, HeadDraw{}, static_cast<hipStream_t>(stream));
}

glance_status glance_verify_head_sampled(const void* h, const void* w_head, int32_t dtype,
                                         int32_t R, int32_t d_model, int32_t V,
                                         float temperature, uint64_t seed, uint64_t round_id,
                                         int32_t* argmax, float* top1, float* gap,
                                         float* entropy, int32_t* sample_tok, float* sample_gap,
                                         float* logits, void* ws, size_t ws_bytes, void* stream) {
  g_last_error.clear();
  REQUIRE(std::isfinite(temperature) && temperature > 0.f,
          "temperature = %g is not a finite positive number", static_cast<double>(temperature));
  REQUIRE_PTR(sample_tok);
  REQUIRE_PTR(sample_gap);
  HeadDraw dr;
  dr.tok = sample_tok;
  dr.gap = sample_gap;
  dr.inv_temp = 1.f / temperature;
  dr.seed_lo = static_cast<uint32_t>(seed);
  dr.seed_hi = static_cast<uint32_t>(seed >> 32);
  dr.rnd_lo = static_cast<uint32_t>(round_id);
  dr.rnd_hi = static_cast<uint32_t>(round_id >> 32);
  return verify_head(h, w_head, nullptr, dtype, R, d_model, V, argmax, top1, gap, entropy, logits,
                     ws, ws_bytes, dr, static_cast<hipStream_t>(stream));
}

size_t glance_head_pack_bytes(int32_t V, int32_t d_model) {
  if (V < 2 || d_model < 256 || d_model % 256 != 0 || !head_in_bounds(1, V, d_model)) return 0;
  return head_pack_bytes(V, d_model);
}

glance_status glance_head_pack(const void* w_head, int32_t V, int32_t d_model, void* w_packed,
                               void* stream) {
  g_last_error.clear();
  REQUIRE(V >= 2, "V = %d < 2", V);
  if (d_model < 256 || d_model % 256 != 0 || !head_in_bounds(1, V, d_model))
    return fail(GLANCE_ERR_UNSUPPORTED, "packed head needs d_model %% 256 == 0, d_model <= %d and "
                "V <= %d (got %d, %d)", kMaxDModel, kMaxHeadVocab, d_model, V);
  REQUIRE_PTR(w_head);
  REQUIRE_PTR(w_packed);
  return launch_head_pack(w_head, V, d_model, w_packed, static_cast<hipStream_t>(stream));
}

glance_status glance_verify_head_packed(const void* h, const void* w_packed, int32_t R,
                                        int32_t d_model, int32_t V, float temperature,
                                        uint64_t seed, uint64_t round_id, int32_t* argmax,
                                        float* top1, float* gap, float* entropy,
                                        int32_t* sample_tok, float* sample_gap, float* logits,
                                        void* ws, size_t ws_bytes, void* stream) {
  g_last_error.clear();
  HeadDraw dr;
  if (sample_tok || sample_gap) {
    REQUIRE(std::isfinite(temperature) && temperature > 0.f,
            "temperature = %g is not a finite positive number", static_cast<double>(temperature));
    REQUIRE_PTR(sample_tok);
    REQUIRE_PTR(sample_gap);
    dr.tok = sample_tok;
    dr.gap = sample_gap;
    dr.inv_temp = 1.f / temperature;
    dr.seed_lo = static_cast<uint32_t>(seed);
    dr.seed_hi = static_cast<uint32_t>(seed >> 32);
    dr.rnd_lo = static_cast<uint32_t>(round_id);
    dr.rnd_hi = static_cast<uint32_t>(round_id >> 32);
  }
  REQUIRE(w_packed != nullptr, "w_packed is NULL");
  return verify_head(h, nullptr, w_packed, GLANCE_BF16, R, d_model, V, argmax, top1, gap, entropy,
                     logits, ws, ws_bytes, dr, static_cast<hipStream_t>(stream));
}

glance_status glance_verify_head_walk(const void* h, const void* w_packed, int32_t R,
                                      int32_t d_model, int32_t V, float temperature, uint64_t seed,
                                      uint64_t round_id, int32_t* argmax, float* top1, float* gap,
                                      float* entropy, int32_t* sample_tok, float* sample_gap,
                                      float* logits, const glance_walk* walk, void* ws,
                                      size_t ws_bytes, void* stream) {
  g_last_error.clear();
  REQUIRE(walk != nullptr, "walk is NULL");
  REQUIRE(walk->nseq >= 1, "nseq = %d < 1", walk->nseq);
  REQUIRE(walk->n_rows >= 1 && walk->n_rows <= GLANCE_MAX_ROWS, "n_rows = %d outside [1, %d]",
          walk->n_rows, GLANCE_MAX_ROWS);
  REQUIRE(static_cast<int64_t>(walk->nseq) * walk->n_rows == R,
          "R = %d is not nseq %d x n_rows %d", R, walk->nseq, walk->n_rows);
  REQUIRE(walk->L >= 1 && walk->L <= GLANCE_MAX_L, "L = %d outside [1, %d]", walk->L, GLANCE_MAX_L);
  REQUIRE(!std::isnan(walk->gap_flag), "gap_flag is NaN");
  REQUIRE_PTR(walk->parent);
  REQUIRE_PTR(walk->token);
  REQUIRE_PTR(walk->n_valid);
  REQUIRE_PTR(walk->n_accept);
  REQUIRE_PTR(walk->out_tokens);
  REQUIRE_PTR(walk->path_rows);
  REQUIRE_PTR(walk->flagged);
  HeadDraw dr;
  if (sample_tok || sample_gap) {
    REQUIRE(std::isfinite(temperature) && temperature > 0.f,
            "temperature = %g is not a finite positive number", static_cast<double>(temperature));
    REQUIRE_PTR(sample_tok);
    REQUIRE_PTR(sample_gap);
    dr.tok = sample_tok;
    dr.gap = sample_gap;
    dr.inv_temp = 1.f / temperature;
    dr.seed_lo = static_cast<uint32_t>(seed);
    dr.seed_hi = static_cast<uint32_t>(seed >> 32);
    dr.rnd_lo = static_cast<uint32_t>(round_id);
    dr.rnd_hi = static_cast<uint32_t>(round_id >> 32);
  }
  REQUIRE(w_packed != nullptr, "w_packed is NULL");
  WalkArgs wk;
  wk.parent = walk->parent;
  wk.token = walk->token;
  wk.n_valid = walk->n_valid;
  wk.nseq = walk->nseq;
  wk.n_rows = walk->n_rows;
  wk.L = walk->L;
  wk.gap_flag = walk->gap_flag;
  wk.n_accept = walk->n_accept;
  wk.out_tokens = walk->out_tokens;
  wk.path_rows = walk->path_rows;
  wk.flagged = walk->flagged;
  return verify_head(h, nullptr, w_packed, GLANCE_BF16, R, d_model, V, argmax, top1, gap, entropy,
                     logits, ws, ws_bytes, dr, static_cast<hipStream_t>(stream), &wk);
}

glance_status glance_verify_head_packed_noalloc(const void* h, const void* w_packed, int32_t R,
                                                int32_t d_model, int32_t V, float temperature,
                                                uint64_t seed, uint64_t round_id, int32_t* argmax,
                                                float* top1, float* gap, float* entropy,
                                                int32_t* sample_tok, float* sample_gap,
                                                float* logits, void* stream) {
  g_last_error.clear();
  REQUIRE(R >= 1, "R = %d < 1", R);
  REQUIRE(V >= 2, "V = %d < 2", V);
  const size_t need = glance_verify_head_ws(R, V, d_model, GLANCE_BF16);
  if (need == 0)
    return fail(GLANCE_ERR_UNSUPPORTED, "head beyond the library's bounds (R <= %d, V <= %d, "
                "d_model <= %d)", kMaxHeadRows, kMaxHeadVocab, kMaxDModel);
  if (need > kHeadScratchFloats * sizeof(float))
    return fail(GLANCE_ERR_UNSUPPORTED,
                "R = %d rows of V = %d need %zu bytes of head scratch; the fixed array holds %zu",
                R, V, need, kHeadScratchFloats * sizeof(float));
  float* scratch = nullptr;
  const glance_status st = head_scratch_ptr(&scratch);
  if (st != GLANCE_OK) return st;
  return glance_verify_head_packed(h, w_packed, R, d_model, V, temperature, seed, round_id, argmax,
                                   top1, gap, entropy, sample_tok, sample_gap, logits, scratch,
                                   kHeadScratchFloats * sizeof(float), stream);
}

glance_status glance_read_probe(const void* buf, size_t bytes, int32_t n_wg, uint32_t* out,
                                void* stream) {
  g_last_error.clear();
  REQUIRE(bytes >= 16 && bytes % 16 == 0, "bytes = %zu is not a positive multiple of 16", bytes);
  REQUIRE(n_wg >= 1 && n_wg <= 65536, "n_wg = %d outside [1, 65536]", n_wg);
  REQUIRE_PTR(buf);
  REQUIRE_PTR(out);
  return launch_read_probe(buf, bytes, n_wg, out, static_cast<hipStream_t>(stream));
}

glance_status glance_head_timing(void* start, void* stop) {
  g_last_error.clear();
  REQUIRE((start == nullptr) == (stop == nullptr), "start and stop must both be set or both be NULL");
  g_head_ev_start = static_cast<hipEvent_t>(start);
  g_head_ev_stop = static_cast<hipEvent_t>(stop);
  return GLANCE_OK;
}

// ------------------------------------------------------------------- step 5
glance_status glance_accept_walk(const int32_t* parent, const int32_t* token,
                                 const int32_t* n_valid, const int32_t* argmax, const float* gap,
                                 int32_t nseq, int32_t n_rows, int32_t L, float gap_flag,
                                 int32_t* n_accept, int32_t* out_tokens, int32_t* path_rows,
                                 int32_t* flagged, void* stream) {
  g_last_error.clear();
  REQUIRE(nseq >= 1, "nseq = %d < 1", nseq);
  REQUIRE(n_rows >= 1 && n_rows <= GLANCE_MAX_ROWS, "n_rows = %d outside [1, %d]", n_rows,
          GLANCE_MAX_ROWS);
  REQUIRE(L >= 1 && L <= GLANCE_MAX_L, "L = %d outside [1, %d]", L, GLANCE_MAX_L);
  REQUIRE(!std::isnan(gap_flag), "gap_flag is NaN");
  REQUIRE_PTR(parent);
  REQUIRE_PTR(token);
  REQUIRE_PTR(n_valid);
  REQUIRE_PTR(argmax);
  REQUIRE_PTR(gap);
  REQUIRE_PTR(n_accept);
  REQUIRE_PTR(out_tokens);
  REQUIRE_PTR(path_rows);
  REQUIRE_PTR(flagged);
  return launch_accept_walk(parent, token, n_valid, argmax, gap, nseq, n_rows, L, gap_flag,
                            n_accept, out_tokens, path_rows, flagged,
                            static_cast<hipStream_t>(stream));
}


// -------------------------------------------------------------- after step 5
glance_status glance_commit_kv(const void* tree_k, const void* tree_v, int32_t dtype,
                               const int32_t* path_rows, const int32_t* n_accept, int32_t nseq,
                               int32_t L, int32_t Hkv, int32_t D, const int64_t* kv_offsets,
                               void* k_cache, void* v_cache, int64_t cap, void* stream) {
  g_last_error.clear();
  REQUIRE(dtype == GLANCE_F32 || dtype == GLANCE_BF16, "dtype = %d is not GLANCE_F32 or GLANCE_BF16", dtype);
  if (nseq != 1) return fail(GLANCE_ERR_UNSUPPORTED, "nseq = %d: packed sequences cannot grow in place", nseq);
  REQUIRE(L >= 1 && L <= GLANCE_MAX_L, "L = %d outside [1, %d]", L, GLANCE_MAX_L);
  REQUIRE(Hkv >= 1 && D >= 1, "Hkv = %d, D = %d", Hkv, D);
  REQUIRE(cap >= 0, "cap = %lld < 0", static_cast<long long>(cap));
  const size_t row_bytes = static_cast<size_t>(Hkv) * D * (dtype == GLANCE_BF16 ? 2 : 4);
  REQUIRE(row_bytes % 16 == 0, "Hkv * D * element size = %zu is not a multiple of 16", row_bytes);
  REQUIRE_PTR(tree_k);
  REQUIRE_PTR(tree_v);
  REQUIRE_PTR(path_rows);
  REQUIRE_PTR(n_accept);
  REQUIRE_PTR(kv_offsets);
  REQUIRE_PTR(k_cache);
  REQUIRE_PTR(v_cache);
  return launch_commit_kv(tree_k, tree_v, path_rows, n_accept, kv_offsets, cap, L, row_bytes,
                          k_cache, v_cache, static_cast<hipStream_t>(stream));
}

glance_status glance_advance_round(const int32_t* n_accept, const int32_t* out_tokens, int32_t nseq,
                                   int64_t* kv_offsets, int32_t* root_token, void* stream) {
  g_last_error.clear();
  if (nseq != 1) return fail(GLANCE_ERR_UNSUPPORTED, "nseq = %d: only one sequence advances in place", nseq);
  REQUIRE_PTR(n_accept);
  REQUIRE_PTR(out_tokens);
  REQUIRE_PTR(kv_offsets);
  REQUIRE_PTR(root_token);
  return launch_advance_round(n_accept, out_tokens, kv_offsets, root_token,
                              static_cast<hipStream_t>(stream));
}

}  // extern "C"
