// Steps 1-2 of the verify round: log-softmax and per-offset top-K of the draft
// marginals, then the top-N prefix-closed candidate tree.
//
// Paper "Vision Is Not Overhead: One-Pass Block Drafting for Lossless
// Speculative Decoding in Vision-Language Models", §3.2 Assumption 1 (one
// marginal q_j per offset, prefixes ranked by the plug-in score prod_j q_j(y_j))
// and Def. 1 (S is prefix-closed, depth <= L, N = |S|); project page "Verify
// pass" (the builder keeps the N prefixes of highest plug-in score).
//
// Only the K_j = min(N - j + 1, V) best tokens of offset j can appear at depth j:
// a depth-j node of rank r is preceded by its r - 1 better siblings and its j - 1
// ancestors, all of which must also be in S.  So each offset keeps <= 63 tokens.
//
// Kernels
//   lsm_chunk   grid (chunks, L, nseq) x 256: per chunk of one offset's logits,
//               the chunk maximum, sum exp(z - max), and the chunk's K_j best
//               tokens by an LDS radix select on the key (logit, -token id).
//   lsm_merge   grid (L, nseq) x 256: merges the chunks of one offset into
//               log q_j(v) = (z_v - max) - ln(sum exp(z - max)) for its K_j best
//               tokens, ordered by (logit desc, token id asc).
//   build_tree  grid nseq x 64: one wavefront runs best-first selection over the
//               ranked lists (each lane holds one frontier prefix; a pop is a
//               wave-wide max), then lays the nodes out breadth-first and builds
//               the ancestor masks.
#include "common.h"
#include "kernels.h"

namespace glance {

namespace {

constexpr int kTopThreads = 256;
constexpr int kSlots = 64;  // candidate slots per (offset, chunk); K_j <= 63

__device__ __forceinline__ int k_of(int N, int V, int j) {
  int k = N - j;
  if (k > V) k = V;
  return k > 0 ? k : 0;
}

__device__ __forceinline__ unsigned long long make_comp(float v, uint32_t idx) {
  return (static_cast<unsigned long long>(float_key(v)) << 32) |
         static_cast<unsigned long long>(0xFFFFFFFFu - idx);
}

// Block-wide radix select over 64-bit keys held in registers (IPT per thread).
// Returns T such that exactly K of the valid keys are >= T, or 0 when at most K
// keys are valid (then every valid key is selected).  Keys are distinct.
template <int IPT>
__device__ unsigned long long block_threshold(const unsigned long long (&comp)[IPT],
                                              const bool (&ok)[IPT], int K, int n_ok,
                                              unsigned* hist, unsigned long long* s_prefix,
                                              int* s_krem, int* s_done) {
  if (n_ok <= K) return 0ull;
  unsigned long long prefix = 0ull, mask = 0ull;
  int krem = K;
  for (int shift = 56; shift >= 0; shift -= 8) {
    for (int i = threadIdx.x; i < 256; i += blockDim.x) hist[i] = 0u;
    __syncthreads();
#pragma unroll
    for (int i = 0; i < IPT; ++i)
      if (ok[i] && (comp[i] & mask) == prefix)
        atomicAdd(&hist[(comp[i] >> shift) & 255ull], 1u);
    __syncthreads();
    if (threadIdx.x < kWave) {
      const int lane = threadIdx.x;
      unsigned c[4];
#pragma unroll
      for (int b = 0; b < 4; ++b) c[b] = hist[4 * lane + b];
      const unsigned s = c[0] + c[1] + c[2] + c[3];
      unsigned inc = s;
#pragma unroll
      for (int d = 1; d < kWave; d <<= 1) {
        unsigned o = __shfl_down(inc, d, kWave);
        if (lane + d < kWave) inc += o;
      }
      unsigned above = inc - s;  // keys in the bins of higher lanes
#pragma unroll
      for (int b = 3; b >= 0; --b) {
        if (above < static_cast<unsigned>(krem) && static_cast<unsigned>(krem) <= above + c[b]) {
          *s_prefix = prefix | (static_cast<unsigned long long>(4 * lane + b) << shift);
          *s_krem = krem - static_cast<int>(above);
          *s_done = (c[b] == static_cast<unsigned>(krem) - above) ? 1 : 0;
        }
        above += c[b];
      }
    }
    __syncthreads();
    prefix = *s_prefix;
    krem = *s_krem;
    const int done = *s_done;
    mask |= 0xFFull << shift;
    __syncthreads();
    if (done) break;
  }
  return prefix;
}

// Descending sort of one wavefront's 64 keys (one per lane), bitonic network.
__device__ __forceinline__ unsigned long long wave_sort_desc(unsigned long long key) {
  const int lane = lane_id();
#pragma unroll
  for (int k = 2; k <= kWave; k <<= 1) {
#pragma unroll
    for (int j = k >> 1; j > 0; j >>= 1) {
      unsigned long long other = __shfl_xor(key, j, kWave);
      const bool desc_seg = (lane & k) == 0;
      const bool lower = (lane & j) == 0;
      const unsigned long long hi = key > other ? key : other;
      const unsigned long long lo = key > other ? other : key;
      key = (lower == desc_seg) ? hi : lo;
    }
  }
  return key;
}

template <typename T>
__device__ __forceinline__ float load_logit(const T* p);
template <>
__device__ __forceinline__ float load_logit<float>(const float* p) { return *p; }
template <>
__device__ __forceinline__ float load_logit<uint16_t>(const uint16_t* p) { return bf16_to_f32(*p); }

template <typename T, int IPT>
__global__ __launch_bounds__(kTopThreads) void lsm_chunk_kernel(
    const T* __restrict__ logits, int L, int V, int N, int chunk, int nch,
    float* __restrict__ cstat, unsigned long long* __restrict__ ccand) {
  __shared__ unsigned hist[256];
  __shared__ unsigned long long s_prefix;
  __shared__ int s_krem, s_done, s_count;
  __shared__ float red[kTopThreads / kWave];
  __shared__ int redi[kTopThreads / kWave];

  const int j = blockIdx.y, s = blockIdx.z, c = blockIdx.x;
  const int row = s * L + j;
  const int K = k_of(N, V, j);
  const T* base = logits + static_cast<size_t>(row) * V;
  const int c0 = c * chunk;
  const int c1 = min(c0 + chunk, V);
  const int tid = threadIdx.x, w = tid / kWave, lane = lane_id();

  float v[IPT];
  bool ok[IPT];
  unsigned long long comp[IPT];
  float mx = -INFINITY;
  int cnt = 0;
#pragma unroll
  for (int i = 0; i < IPT; ++i) {
    const int idx = c0 + i * kTopThreads + tid;
    ok[i] = idx < c1;
    v[i] = ok[i] ? load_logit<T>(base + idx) : -INFINITY;
    comp[i] = make_comp(v[i], static_cast<uint32_t>(idx));
    mx = fmaxf(mx, v[i]);
    cnt += ok[i] ? 1 : 0;
  }
  // chunk maximum
  mx = wave_max(mx);
  if (lane == 0) red[w] = mx;
  cnt = wave_sum_i(cnt);
  if (lane == 0) redi[w] = cnt;
  __syncthreads();
  float cmax = red[0];
  int n_ok = redi[0];
#pragma unroll
  for (int i = 1; i < kTopThreads / kWave; ++i) {
    cmax = fmaxf(cmax, red[i]);
    n_ok += redi[i];
  }
  __syncthreads();
  // sum exp(z - chunk max), fixed reduction order
  float sum = 0.f;
  if (cmax != -INFINITY) {
#pragma unroll
    for (int i = 0; i < IPT; ++i) sum += ok[i] ? expf(v[i] - cmax) : 0.f;
  }
  sum = wave_sum(sum);
  if (lane == 0) red[w] = sum;
  __syncthreads();
  if (tid == 0) {
    float t = 0.f;
    for (int i = 0; i < kTopThreads / kWave; ++i) t += red[i];
    float* st = cstat + (static_cast<size_t>(row) * nch + c) * 2;
    st[0] = cmax;
    st[1] = t;
  }
  // the chunk's K best (logit desc, token id asc)
  unsigned long long* out = ccand + (static_cast<size_t>(row) * nch + c) * kSlots;
  if (tid < kSlots) out[tid] = 0ull;  // slot 0 = empty
  if (tid == 0) s_count = 0;
  __syncthreads();
  if (K > 0) {
    const unsigned long long T0 =
        block_threshold<IPT>(comp, ok, K, n_ok, hist, &s_prefix, &s_krem, &s_done);
#pragma unroll
    for (int i = 0; i < IPT; ++i) {
      if (ok[i] && comp[i] >= T0) {
        const int slot = atomicAdd(&s_count, 1);
        out[slot] = comp[i];
      }
    }
  }
}

template <int IPT>
__global__ __launch_bounds__(kTopThreads) void lsm_merge_kernel(
    int L, int V, int N, int nch, const float* __restrict__ cstat,
    const unsigned long long* __restrict__ ccand, float* __restrict__ top_logq,
    int32_t* __restrict__ top_id) {
  __shared__ unsigned hist[256];
  __shared__ unsigned long long s_prefix;
  __shared__ int s_krem, s_done, s_count;
  __shared__ int redi[kTopThreads / kWave];
  __shared__ float s_M, s_lnS;
  __shared__ unsigned long long sel[kSlots];

  const int j = blockIdx.x, s = blockIdx.y;
  const int row = s * L + j;
  const int K = k_of(N, V, j);
  const int tid = threadIdx.x, w = tid / kWave, lane = lane_id();
  const float* st = cstat + static_cast<size_t>(row) * nch * 2;
  if (tid == 0) {
    float M = -INFINITY;
    for (int c = 0; c < nch; ++c) M = fmaxf(M, st[2 * c]);
    float S = 0.f;
    if (M != -INFINITY)
      for (int c = 0; c < nch; ++c)
        if (st[2 * c + 1] > 0.f) S += st[2 * c + 1] * expf(st[2 * c] - M);
    s_M = M;
    s_lnS = logf(S);
    s_count = 0;
  }
  const unsigned long long* cand = ccand + static_cast<size_t>(row) * nch * kSlots;
  const int total = nch * kSlots;
  unsigned long long comp[IPT];
  bool ok[IPT];
  int cnt = 0;
#pragma unroll
  for (int i = 0; i < IPT; ++i) {
    const int e = i * kTopThreads + tid;
    comp[i] = e < total ? cand[e] : 0ull;
    ok[i] = comp[i] != 0ull;
    cnt += ok[i] ? 1 : 0;
  }
  cnt = wave_sum_i(cnt);
  if (lane == 0) redi[w] = cnt;
  if (tid < kSlots) sel[tid] = 0ull;
  __syncthreads();
  int n_ok = 0;
#pragma unroll
  for (int i = 0; i < kTopThreads / kWave; ++i) n_ok += redi[i];
  if (K > 0) {
    const unsigned long long T0 =
        block_threshold<IPT>(comp, ok, K, n_ok, hist, &s_prefix, &s_krem, &s_done);
#pragma unroll
    for (int i = 0; i < IPT; ++i) {
      if (ok[i] && comp[i] >= T0) {
        const int slot = atomicAdd(&s_count, 1);
        sel[slot] = comp[i];
      }
    }
  }
  __syncthreads();
  if (tid < kWave) {
    const unsigned long long key = wave_sort_desc(sel[tid]);
    const float M = s_M, lnS = s_lnS;
    float lq = -INFINITY;
    int id = -1;
    if (key != 0ull && tid < K) {
      const float z = key_float(static_cast<uint32_t>(key >> 32));
      id = static_cast<int>(0xFFFFFFFFu - static_cast<uint32_t>(key));
      lq = (M == -INFINITY) ? -INFINITY : (z - M) - lnS;
    }
    top_logq[static_cast<size_t>(row) * kSlots + tid] = lq;
    top_id[static_cast<size_t>(row) * kSlots + tid] = id;
  }
}

// Frontier key of the best-first search: higher score first, then smaller
// depth, then the earlier-selected parent, then the better-ranked token.
__device__ __forceinline__ unsigned long long frontier_key(float score, int depth, int ppop,
                                                           int rank) {
  const uint32_t tie = (static_cast<uint32_t>(depth) << 16) |
                       (static_cast<uint32_t>(ppop + 1) << 8) | static_cast<uint32_t>(rank);
  return (static_cast<unsigned long long>(float_key(score)) << 32) |
         static_cast<unsigned long long>(0xFFFFFFFFu - tie);
}

__global__ __launch_bounds__(kWave) void build_tree_kernel(
    const float* __restrict__ top_logq, const int32_t* __restrict__ top_id,
    const int32_t* __restrict__ root_token, int L, int V, int N, int32_t* __restrict__ parent,
    int32_t* __restrict__ depth_out, int32_t* __restrict__ token_out,
    uint64_t* __restrict__ anc_out, float* __restrict__ score_out,
    int32_t* __restrict__ n_valid_out) {
  __shared__ float lq[GLANCE_MAX_L][kSlots];
  __shared__ int tk[GLANCE_MAX_L][kSlots];
  __shared__ float pop_score[kSlots];
  __shared__ int row_of_pop[kSlots];
  __shared__ unsigned long long anc_row[kSlots];

  const int s = blockIdx.x, lane = lane_id();
  const int R = N + 1;
  for (int j = 0; j < L; ++j) {
    lq[j][lane] = top_logq[(static_cast<size_t>(s) * L + j) * kSlots + lane];
    tk[j][lane] = top_id[(static_cast<size_t>(s) * L + j) * kSlots + lane];
  }
  __syncthreads();

  // ---- best-first selection: lane holds one frontier prefix (key 0 = empty)
  bool has = false;
  float f_score = 0.f;
  int f_depth = 0, f_ppop = -1, f_rank = 0;
  if (lane == 0 && N > 0 && k_of(N, V, 0) > 0 && lq[0][0] != -INFINITY) {
    has = true;
    f_score = 0.f + lq[0][0];
    f_depth = 1;
  }
  // popped node fields (lane i keeps node i)
  float n_score = 0.f;
  int n_depth = 0, n_ppop = -1, n_token = -1;
  int n_pop = 0;
  for (int i = 0; i < N; ++i) {
    const unsigned long long key = has ? frontier_key(f_score, f_depth, f_ppop, f_rank) : 0ull;
    const unsigned long long best = wave_max_u64(key);
    if (best == 0ull) break;
    const unsigned long long win_mask = __ballot(key == best);
    const int win = __ffsll(static_cast<long long>(win_mask)) - 1;
    const float w_score = __shfl(f_score, win, kWave);
    const int w_depth = __shfl(f_depth, win, kWave);
    const int w_ppop = __shfl(f_ppop, win, kWave);
    const int w_rank = __shfl(f_rank, win, kWave);
    const int w_token = tk[w_depth - 1][w_rank];
    if (lane == i) {
      n_score = w_score;
      n_depth = w_depth;
      n_ppop = w_ppop;
      n_token = w_token;
      pop_score[i] = w_score;
    }
    // the winner's slot takes its next sibling
    if (lane == win) {
      const int r2 = w_rank + 1;
      const int jd = w_depth - 1;
      if (r2 < k_of(N, V, jd) && lq[jd][r2] != -INFINITY) {
        const float ps = (w_ppop < 0) ? 0.f : pop_score[w_ppop];
        f_score = ps + lq[jd][r2];
        f_rank = r2;
      } else {
        has = false;
      }
    }
    // the popped node's first child takes the lowest empty slot
    if (w_depth < L && k_of(N, V, w_depth) > 0 && lq[w_depth][0] != -INFINITY) {
      const unsigned long long empty = __ballot(!has);
      const int tgt = __ffsll(static_cast<long long>(empty)) - 1;
      if (lane == tgt) {
        has = true;
        f_score = w_score + lq[w_depth][0];
        f_depth = w_depth + 1;
        f_ppop = i;
        f_rank = 0;
      }
    }
    __syncthreads();
    n_pop = i + 1;
  }

  // ---- breadth-first layout: rows by (depth, parent row, token id)
  const size_t ob = static_cast<size_t>(s) * R;
  if (lane == 0) {
    anc_row[0] = 1ull;
    parent[ob] = -1;
    depth_out[ob] = 0;
    token_out[ob] = root_token[s];
    anc_out[ob] = 1ull;
    score_out[ob] = 0.f;
    n_valid_out[s] = n_pop + 1;
  }
  __syncthreads();
  int base = 1;
  for (int d = 1; d <= L; ++d) {
    const bool in_level = lane < n_pop && n_depth == d;
    const unsigned long long lvl = __ballot(in_level);
    if (lvl == 0ull) break;
    const int prow = in_level ? (n_ppop < 0 ? 0 : row_of_pop[n_ppop]) : 0;
    const unsigned long long mykey =
        (static_cast<unsigned long long>(prow) << 32) | static_cast<uint32_t>(n_token);
    int rank = 0;
    unsigned long long m = lvl;
    while (m) {
      const int jl = __ffsll(static_cast<long long>(m)) - 1;
      m &= m - 1;
      const unsigned long long other = __shfl(mykey, jl, kWave);
      rank += (other < mykey) ? 1 : 0;
    }
    if (in_level) {
      const int r = base + rank;
      row_of_pop[lane] = r;
      const unsigned long long a = anc_row[prow] | (1ull << r);
      anc_row[r] = a;
      parent[ob + r] = prow;
      depth_out[ob + r] = d;
      token_out[ob + r] = n_token;
      anc_out[ob + r] = a;
      score_out[ob + r] = n_score;
    }
    base += __popcll(lvl);
    __syncthreads();
  }
  // padding rows
  for (int r = n_pop + 1 + lane; r < R; r += kWave) {
    parent[ob + r] = -1;
    depth_out[ob + r] = 0;
    token_out[ob + r] = -1;
    anc_out[ob + r] = 0ull;
    score_out[ob + r] = -INFINITY;
  }
}

}  // namespace

// Host side -------------------------------------------------------------------
TreeWs tree_ws_layout(int nseq, int L, int V) {
  TreeWs w;
  // chunk size: 4096 logits (16 per thread) while V <= 64 chunks of it, else
  // 16384 (64 per thread); V <= 2^20 keeps the chunk count <= 64.
  if (V <= 64 * 4096) {
    w.chunk = 4096;
    w.ipt = 16;
  } else {
    w.chunk = 16384;
    w.ipt = 64;
  }
  w.nch = (V + w.chunk - 1) / w.chunk;
  const size_t rows = static_cast<size_t>(nseq) * L;
  size_t off = 0;
  auto take = [&](size_t bytes) {
    size_t o = off;
    off += (bytes + 255) & ~static_cast<size_t>(255);
    return o;
  };
  w.off_cstat = take(rows * w.nch * 2 * sizeof(float));
  w.off_ccand = take(rows * w.nch * kSlots * sizeof(unsigned long long));
  w.off_logq = take(rows * kSlots * sizeof(float));
  w.off_id = take(rows * kSlots * sizeof(int32_t));
  w.bytes = off;
  return w;
}

glance_status launch_build_tree(const void* logits, int dtype, const int32_t* root, int nseq,
                                int L, int V, int N, int32_t* parent, int32_t* depth,
                                int32_t* token, uint64_t* anc, float* score,
                                int32_t* n_valid, void* ws, hipStream_t st) {
  const TreeWs w = tree_ws_layout(nseq, L, V);
  char* base = static_cast<char*>(ws);
  float* cstat = reinterpret_cast<float*>(base + w.off_cstat);
  unsigned long long* ccand = reinterpret_cast<unsigned long long*>(base + w.off_ccand);
  float* logq = reinterpret_cast<float*>(base + w.off_logq);
  int32_t* id = reinterpret_cast<int32_t*>(base + w.off_id);
  dim3 ga(w.nch, L, nseq);
  if (dtype == GLANCE_BF16) {
    const uint16_t* z = static_cast<const uint16_t*>(logits);
    if (w.ipt == 16)
      lsm_chunk_kernel<uint16_t, 16><<<ga, kTopThreads, 0, st>>>(z, L, V, N, w.chunk, w.nch, cstat, ccand);
    else
      lsm_chunk_kernel<uint16_t, 64><<<ga, kTopThreads, 0, st>>>(z, L, V, N, w.chunk, w.nch, cstat, ccand);
  } else {
    const float* z = static_cast<const float*>(logits);
    if (w.ipt == 16)
      lsm_chunk_kernel<float, 16><<<ga, kTopThreads, 0, st>>>(z, L, V, N, w.chunk, w.nch, cstat, ccand);
    else
      lsm_chunk_kernel<float, 64><<<ga, kTopThreads, 0, st>>>(z, L, V, N, w.chunk, w.nch, cstat, ccand);
  }
  GLANCE_LAUNCH_CHECK();
  lsm_merge_kernel<16><<<dim3(L, nseq), kTopThreads, 0, st>>>(L, V, N, w.nch, cstat, ccand, logq, id);
  GLANCE_LAUNCH_CHECK();
  build_tree_kernel<<<nseq, kWave, 0, st>>>(logq, id, root, L, V, N, parent, depth, token, anc,
                                            score, n_valid);
  GLANCE_LAUNCH_CHECK();
  return GLANCE_OK;
}

}  // namespace glance
