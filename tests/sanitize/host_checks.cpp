// Host-side argument validation of every C-ABI entry point, built with
// AddressSanitizer and UndefinedBehaviorSanitizer on the host code that
// validates (glance.cpp).  Every call below must be rejected before anything
// is launched (no GPU is used), and every workspace sizer is driven to extreme
// sizes, where an overflowing intermediate would be reported by the sanitizer.
// Exit status: the number of failed expectations.
#include <cmath>
#include <cstdint>
#include <cstdio>
#include <cstring>
#include <limits>

#include "glance.h"

static int g_fail = 0;
#define EXPECT(cond)                                                              \
  do {                                                                            \
    if (!(cond)) {                                                                \
      std::fprintf(stderr, "FAILED %s:%d: %s (last error: %s)\n", __FILE__,        \
                   __LINE__, #cond, glance_last_error());                         \
      ++g_fail;                                                                   \
    }                                                                             \
  } while (0)

// 16-byte aligned stand-ins: every call below fails validation before using them
static char* const P = reinterpret_cast<char*>(0x100000);
static void* const WS = reinterpret_cast<void*>(0x1000000);
static const size_t BIG = size_t(1) << 40;
static const float NaN = std::numeric_limits<float>::quiet_NaN();
static const float Inf = std::numeric_limits<float>::infinity();

template <typename T>
static T* ptr(char* p) { return reinterpret_cast<T*>(p); }

static void helpers() {
  EXPECT(glance_abi_version() == 1);
  for (int s = -10; s <= 3; ++s) EXPECT(glance_status_string(s) != nullptr);
  EXPECT(std::strcmp(glance_status_string(0), "ok") == 0);
  EXPECT(glance_last_error() != nullptr);
}

static void sizers() {
  const int32_t I = std::numeric_limits<int32_t>::max();
  const int64_t J = std::numeric_limits<int64_t>::max();
  // valid sizes give nonzero bytes, invalid ones zero; extremes must not overflow
  EXPECT(glance_build_tree_ws(1, 15, 151936, 63) > 0);
  EXPECT(glance_build_tree_ws(0, 15, 151936, 63) == 0);
  (void)glance_build_tree_ws(I, 16, 1 << 18, 63);
  (void)glance_build_tree_ws(1, 16, I, 63);
  (void)glance_build_tree_ws(-1, -1, -1, -1);
  EXPECT(glance_build_tree_flag_offset(1, 0, 151936, 63) == 0);
  (void)glance_build_tree_flag_offset(I, 16, I, 63);
  EXPECT(glance_tree_attn_ws(1, 64, 1024, 4096, 32, 8, 128) > 0);
  EXPECT(glance_tree_attn_ws(0, 64, 1024, 4096, 32, 8, 128) == 0);
  (void)glance_tree_attn_ws(I, 64, J, I, I, 8, 128);
  (void)glance_tree_attn_ws(1, 64, J, 4096, 32, 8, 128);
  (void)glance_tree_attn_ws(I, 64, 1 << 20, 4096, 32, 8, 128);
  EXPECT(glance_tree_layer_ws(1, 64, 1024, 4096, 32, 8, 128, 12288) > 0);
  (void)glance_tree_layer_ws(I, 64, J, I, I, 8, 128, I);
  EXPECT(glance_verify_head_ws(64, 151936, 4096, 1) > 0);
  EXPECT(glance_verify_head_ws(0, 151936, 4096, 1) == 0);
  (void)glance_verify_head_ws(I, I, I, 1);
  (void)glance_verify_head_ws(I, I, I, 0);
  EXPECT(glance_head_pack_bytes(151936, 4096) > 0);
  EXPECT(glance_head_pack_bytes(151936, 4000) == 0);
  (void)glance_head_pack_bytes(I, 1 << 30);
  EXPECT(glance_attn_pack_bytes(4096, 32, 8, 128) > 0);
  EXPECT(glance_attn_pack_bytes(4096, 32, 8, 64) == 0);
  (void)glance_attn_pack_bytes(1 << 30, I / 128, 1, 128);
  EXPECT(glance_mlp_pack_bytes(4096, 12288) > 0);
  EXPECT(glance_mlp_pack_bytes(4000, 12288) == 0);
  (void)glance_mlp_pack_bytes(1 << 30, 1 << 30);
}

static int32_t tree(int nseq = 1, int L = 15, int V = 151936, int N = 63, int dtype = 1,
                    char* logits = P, char* out = P, void* ws = WS, size_t ws_bytes = BIG) {
  return glance_build_tree(logits, dtype, ptr<int32_t>(P), nseq, L, V, N, ptr<int32_t>(out),
                           ptr<int32_t>(out), ptr<int32_t>(out), ptr<uint64_t>(out),
                           ptr<float>(out), ptr<int32_t>(out), ws, ws_bytes, nullptr);
}

static void build_tree() {
  EXPECT(tree(0) == -1);
  EXPECT(tree(1, 0) == -1);
  EXPECT(tree(1, 17) == -1);
  EXPECT(tree(1, 15, 1) == -1);
  EXPECT(tree(1, 15, 151936, 64) == -1);
  EXPECT(tree(1, 15, 151936, -1) == -1);
  EXPECT(tree(1, 15, 151936, 63, 7) == -1);
  EXPECT(tree(1, 15, 1 << 19) == -4);
  EXPECT(tree(1, 15, 151936, 63, 1, nullptr) == -1);
  EXPECT(tree(1, 15, 151936, 63, 1, P + 2) == -2);
  EXPECT(tree(1, 15, 151936, 63, 1, P, P + 4) == -2);
  EXPECT(tree(1, 15, 151936, 63, 1, P, P, nullptr) == -3);
  EXPECT(tree(1, 15, 151936, 63, 1, P, P, static_cast<char*>(WS) + 16) == -3);
  EXPECT(tree(1, 15, 151936, 63, 1, P, P, WS, 16) == -3);
  EXPECT(tree(std::numeric_limits<int32_t>::max(), 16, 1 << 18, 63, 1, P, P, WS, 16) != 0);

  auto shared = [](int nseq, int n_max, int budget, float tau, char* w, size_t ws_bytes,
                   int dtype = 1, int V = 151936) {
    return glance_build_tree_shared(P, dtype, ptr<int32_t>(P), ptr<float>(w), nseq, 15, V, n_max,
                                    budget, tau, ptr<int32_t>(P), ptr<int32_t>(P), ptr<int32_t>(P),
                                    ptr<uint64_t>(P), ptr<float>(P), ptr<int32_t>(P), WS, ws_bytes,
                                    nullptr);
  };
  EXPECT(shared(0, 63, 10, -Inf, P, BIG) == -1);
  EXPECT(shared(17, 63, 10, -Inf, P, BIG) == -1);
  EXPECT(shared(4, 64, 10, -Inf, P, BIG) == -1);
  EXPECT(shared(4, 63, -1, -Inf, P, BIG) == -1);
  EXPECT(shared(4, 63, 10, NaN, P, BIG) == -1);
  EXPECT(shared(4, 63, 10, -Inf, nullptr, BIG) == -1);
  EXPECT(shared(4, 63, 10, -Inf, P + 4, BIG) == -2);
  EXPECT(shared(4, 63, 10, -Inf, P, 64) == -3);
  EXPECT(shared(4, 63, 10, -Inf, P, BIG, 0, 200000) == -4);

  auto lv = [](int nseq, int stride, float b0, float b1, int L, char* h, char* o) {
    return glance_entropy_log_value(ptr<float>(h), nseq, stride, b0, b1, L, ptr<float>(o), nullptr);
  };
  EXPECT(lv(0, 1, 0.96f, 0.63f, 15, P, P) == -1);
  EXPECT(lv(4, 0, 0.96f, 0.63f, 15, P, P) == -1);
  EXPECT(lv(4, 1, 0.96f, 0.63f, 0, P, P) == -1);
  EXPECT(lv(4, 1, NaN, 0.63f, 15, P, P) == -1);
  EXPECT(lv(4, 1, 0.96f, Inf, 15, P, P) == -1);
  EXPECT(lv(4, 1, 0.96f, 0.63f, 15, nullptr, P) == -1);
  EXPECT(lv(4, 1, 0.96f, 0.63f, 15, P, nullptr) == -1);
  EXPECT(lv(4, 1, 0.96f, 0.63f, 15, P + 2, P) == -2);
}

static glance_attn_layer layer(char* w = P, const void* packed = nullptr) {
  glance_attn_layer a;
  a.wq = a.wk = a.wv = a.wo = w;
  a.k_cache = a.v_cache = P;
  a.packed = packed;
  return a;
}

static int32_t attn(const glance_attn_layer* lay, int dtype = 1, int n_rows = 64, int d = 4096,
                    int Hq = 32, int Hkv = 8, int D = 128, int64_t max_prefix = 1024,
                    int n_pos = 2048, size_t ws_bytes = BIG, char* embed = P) {
  return glance_tree_attn(lay, dtype, embed, ptr<int32_t>(P), nullptr, P, ptr<int64_t>(P),
                          max_prefix, ptr<int32_t>(P), ptr<uint64_t>(P), ptr<float>(P),
                          ptr<float>(P), n_pos, 1, n_rows, d, Hq, Hkv, D, nullptr, nullptr,
                          nullptr, WS, ws_bytes, nullptr);
}

static void tree_attn() {
  glance_attn_layer ok = layer();
  EXPECT(attn(nullptr) == -1);
  EXPECT(attn(&ok, 7) == -1);
  EXPECT(attn(&ok, 1, 0) == -1);
  EXPECT(attn(&ok, 1, 65) == -1);
  EXPECT(attn(&ok, 1, 64, 4096, 30, 8) == -1);
  EXPECT(attn(&ok, 1, 64, 4000) == -4);
  EXPECT(attn(&ok, 1, 64, 4096, 32, 8, 64) == -4);
  EXPECT(attn(&ok, 1, 64, 4096, 32, 8, 128, -1) == -1);
  EXPECT(attn(&ok, 1, 64, 4096, 32, 8, 128, 1024, 1024 + 63) == -1);
  EXPECT(attn(&ok, 1, 64, 4096, 32, 8, 128, 1024, 1088, 1000) == -3);
  EXPECT(attn(&ok, 1, 64, 4096, 32, 8, 128, std::numeric_limits<int64_t>::max(),
              std::numeric_limits<int32_t>::max()) != 0);
  EXPECT(attn(&ok, 1, 64, 4096, 32, 8, 128, 1024, 2048, BIG, nullptr) == -1);
  glance_attn_layer bad = layer(P + 8);
  EXPECT(attn(&bad) == -2);
  glance_attn_layer f32_packed = layer(P, P);
  EXPECT(attn(&f32_packed, 0, 64, 64, 2, 1, 32) == -4);
  glance_attn_layer packed = layer(nullptr, P);
  EXPECT(attn(&packed, 1, 64, 4096, 32, 8, 128, 1024, 2048, 100) == -3);

  auto full = [](int inter, float eps, int D, int d, size_t ws_bytes) {
    glance_full_layer f;
    f.attn = layer();
    f.g_attn = f.g_q = f.g_k = f.g_mlp = P;
    f.w_gate = f.w_up = f.w_down = P;
    f.inter = inter;
    f.eps = eps;
    f.mlp_packed = nullptr;
    return glance_tree_layer(&f, P, ptr<int32_t>(P), nullptr, P, ptr<int64_t>(P), 1024,
                             ptr<int32_t>(P), ptr<uint64_t>(P), ptr<float>(P), ptr<float>(P), 2048,
                             1, 64, d, 32, 8, D, nullptr, nullptr, nullptr, WS, ws_bytes, nullptr);
  };
  EXPECT(glance_tree_layer(nullptr, P, ptr<int32_t>(P), nullptr, P, ptr<int64_t>(P), 1024,
                           ptr<int32_t>(P), ptr<uint64_t>(P), ptr<float>(P), ptr<float>(P), 2048,
                           1, 64, 4096, 32, 8, 128, nullptr, nullptr, nullptr, WS, BIG,
                           nullptr) == -1);
  EXPECT(full(1000, 1e-6f, 128, 4096, BIG) == -4);
  EXPECT(full(12288, NaN, 128, 4096, BIG) == -1);
  EXPECT(full(12288, -1.f, 128, 4096, BIG) == -1);
  EXPECT(full(12288, 1e-6f, 64, 4096, BIG) == -4);
  EXPECT(full(12288, 1e-6f, 128, 4000, BIG) == -4);
  EXPECT(full(12288, 1e-6f, 128, 4096, 100) == -3);

  EXPECT(glance_attn_pack(P, P, P, P, 4096, 32, 8, 64, P, nullptr) == -4);
  EXPECT(glance_attn_pack(nullptr, P, P, P, 4096, 32, 8, 128, P, nullptr) == -1);
  EXPECT(glance_attn_pack(P, P, P, P + 8, 4096, 32, 8, 128, P, nullptr) == -2);
  EXPECT(glance_mlp_pack(P, P, P, 4000, 12288, P, nullptr) == -4);
  EXPECT(glance_mlp_pack(P, nullptr, P, 4096, 12288, P, nullptr) == -1);
}

static void head() {
  auto vh = [](int dtype, int R, int d, int V, char* w, size_t ws_bytes) {
    return glance_verify_head(P, w, dtype, R, d, V, ptr<int32_t>(P), ptr<float>(P), ptr<float>(P),
                              ptr<float>(P), nullptr, WS, ws_bytes, nullptr);
  };
  EXPECT(vh(1, 0, 4096, 151936, P, BIG) == -1);
  EXPECT(vh(1, 64, 4096, 1, P, BIG) == -1);
  EXPECT(vh(1, 64, 4000, 151936, P, BIG) == -4);
  EXPECT(vh(1, 64, 4096, 151936, P + 8, BIG) == -2);
  EXPECT(vh(1, 64, 4096, 151936, P, 100) == -3);
  EXPECT(vh(5, 64, 4096, 151936, P, BIG) == -1);
  EXPECT(vh(1, std::numeric_limits<int32_t>::max(), 4096, std::numeric_limits<int32_t>::max(), P,
            100) != 0);

  auto vs = [](float T, char* tok, char* sgap) {
    return glance_verify_head_sampled(P, P, 1, 64, 4096, 151936, T, (uint64_t(1) << 63) + 5,
                                      (uint64_t(1) << 40) + 3, ptr<int32_t>(P), ptr<float>(P),
                                      ptr<float>(P), ptr<float>(P), ptr<int32_t>(tok),
                                      ptr<float>(sgap), nullptr, WS, BIG, nullptr);
  };
  EXPECT(vs(0.f, P, P) == -1);
  EXPECT(vs(-1.f, P, P) == -1);
  EXPECT(vs(NaN, P, P) == -1);
  EXPECT(vs(Inf, P, P) == -1);
  EXPECT(vs(1.f, nullptr, P) == -1);
  EXPECT(vs(1.f, P, nullptr) == -1);
  EXPECT(vs(1.f, P + 2, P) == -2);

  EXPECT(glance_head_pack(P, 1, 4096, P, nullptr) == -1);
  EXPECT(glance_head_pack(P, 1000, 4000, P, nullptr) == -4);
  EXPECT(glance_head_pack(nullptr, 1000, 256, P, nullptr) == -1);
  EXPECT(glance_head_pack(P, 1000, 256, P + 8, nullptr) == -2);

  auto vp = [](char* w, int R, int d, float T, char* tok, size_t ws_bytes) {
    return glance_verify_head_packed(P, w, R, d, 151936, T, 1, 2, ptr<int32_t>(P), ptr<float>(P),
                                     ptr<float>(P), ptr<float>(P), ptr<int32_t>(tok),
                                     ptr<float>(tok), nullptr, WS, ws_bytes, nullptr);
  };
  EXPECT(vp(nullptr, 64, 4096, 1.f, nullptr, BIG) == -1);
  EXPECT(vp(P + 4, 64, 4096, 1.f, nullptr, BIG) == -2);
  EXPECT(vp(P, 0, 4096, 1.f, nullptr, BIG) == -1);
  EXPECT(vp(P, 64, 4000, 1.f, nullptr, BIG) == -4);
  EXPECT(vp(P, 64, 4096, 1.f, nullptr, 100) == -3);
  EXPECT(vp(P, 64, 4096, 0.f, P, BIG) == -1);

  // the allocation-free head: rows checked and sizes beyond its fixed scratch
  // rejected before any device call
  auto na = [](int R) {
    return glance_verify_head_packed_noalloc(P, P, R, 4096, 151936, 1.f, 1, 2, ptr<int32_t>(P),
                                             ptr<float>(P), ptr<float>(P), ptr<float>(P), nullptr,
                                             nullptr, nullptr, nullptr);
  };
  EXPECT(na(0) == -1);
  EXPECT(na(552) == -4);
  EXPECT(na(std::numeric_limits<int32_t>::max()) == -4);
}

static void walk() {
  auto aw = [](int nseq, int n_rows, int L, float flag, char* parent) {
    return glance_accept_walk(ptr<int32_t>(parent), ptr<int32_t>(P), ptr<int32_t>(P),
                              ptr<int32_t>(P), ptr<float>(P), nseq, n_rows, L, flag,
                              ptr<int32_t>(P), ptr<int32_t>(P), ptr<int32_t>(P), ptr<int32_t>(P),
                              nullptr);
  };
  EXPECT(aw(0, 64, 15, 1e-3f, P) == -1);
  EXPECT(aw(1, 0, 15, 1e-3f, P) == -1);
  EXPECT(aw(1, 65, 15, 1e-3f, P) == -1);
  EXPECT(aw(1, 64, 0, 1e-3f, P) == -1);
  EXPECT(aw(1, 64, 15, NaN, P) == -1);
  EXPECT(aw(1, 64, 15, 1e-3f, nullptr) == -1);
  EXPECT(aw(1, 64, 15, 1e-3f, P + 2) == -2);

  auto ck = [](int dtype, int nseq, int L, int Hkv, int D, int64_t cap, char* tk) {
    return glance_commit_kv(tk, P, dtype, ptr<int32_t>(P), ptr<int32_t>(P), nseq, L, Hkv, D,
                            ptr<int64_t>(P), P, P, cap, nullptr);
  };
  EXPECT(ck(1, 1, 15, 8, 128, 4096, nullptr) == -1);
  EXPECT(ck(7, 1, 15, 8, 128, 4096, P) == -1);
  EXPECT(ck(1, 0, 15, 8, 128, 4096, P) == -4);
  EXPECT(ck(1, 1, 15, 8, 128, -1, P) == -1);
  EXPECT(ck(1, 1, 15, 8, 128, 4096, P + 2) == -2);

  EXPECT(glance_advance_round(ptr<int32_t>(P), nullptr, 1, ptr<int64_t>(P), ptr<int32_t>(P),
                              nullptr) == -1);
  EXPECT(glance_advance_round(ptr<int32_t>(P), ptr<int32_t>(P), 1, ptr<int64_t>(P + 4),
                              ptr<int32_t>(P), nullptr) == -2);
}

int main() {
  helpers();
  sizers();
  build_tree();
  tree_attn();
  head();
  walk();
  std::printf("host checks: %d failed\n", g_fail);
  return g_fail;
}
