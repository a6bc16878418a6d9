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
// Tokens are ranked by the key (logit desc, token id asc); keys are distinct.
//
// Kernels
//   lsm_chunk   grid (chunks, L, nseq) x 256.  One chunk (4096 bf16 or 2048 fp32
//               logits) of one offset row, held in registers after one wave of
//               16-byte streaming loads: the chunk maximum, the sum of
//               exp(z - max) and the chunk's K best keys, sorted (block_topk).
//   lsm_merge   grid (L, nseq) x 256.  Combines the chunk statistics into the
//               row's max and ln(sum exp), selects the K best of the <= 64 chunk
//               lists (block_topk again) and writes them as
//               log q_j(v) = (z_v - max) - ln(sum exp(z - max)) with their ids.
//   build_tree  grid nseq x 256.  The ranked lists go to LDS; wave 0 runs
//               best-first selection: lane 0 is the root and lane i the i-th
//               selected node; every lane holds the best not-yet-selected child
//               of its node, so a selection is one wave max and touches two
//               lanes.  Finally the nodes are laid out breadth-first with their
//               ancestor masks.
//
// block_topk finds the K largest of the keys a block holds in registers: the
// K-th largest of the per-thread best keys, T, bounds the K-th largest key from
// below (K threads each hold a key >= T), so only keys >= T (about K of them)
// are gathered to LDS and ranked exactly by counting; when more than kCap keys
// reach T (massive ties) an exact 8-bit radix select runs instead.
#include "common.h"
#include "kernels.h"

namespace glance {

namespace {

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

constexpr int kChunkThreads = 256;
constexpr int kCap = 1024;      // candidates gathered above the threshold
constexpr int kChunkVecs = 2;   // 16-byte vectors per thread per chunk
constexpr int kMergeItems = 16; // list entries per thread in the merge (nch <= 64)

// Shared memory of block_topk.
template <int NT>
struct TopkSmem {
  unsigned long long bests[NT];
  unsigned long long cand[kCap];
  unsigned hist[256];
  unsigned long long prefix, T;
  int krem, done, count;
};

// Rank of key k among n keys of an LDS array (the number of larger keys),
// reading 2 keys per 16-byte load, 8 in flight.
__device__ __forceinline__ int count_greater(const unsigned long long* a, int n,
                                             unsigned long long k) {
  int rank = 0;
  int o = 0;
  for (; o + 8 <= n; o += 8) {
    ulonglong2 v[4];
#pragma unroll
    for (int u = 0; u < 4; ++u) v[u] = *reinterpret_cast<const ulonglong2*>(a + o + 2 * u);
#pragma unroll
    for (int u = 0; u < 4; ++u) rank += (v[u].x > k ? 1 : 0) + (v[u].y > k ? 1 : 0);
  }
  for (; o < n; ++o) rank += a[o] > k ? 1 : 0;
  return rank;
}

// The K (<= 63) largest of the distinct nonzero keys held by the block's
// threads (IPT per thread, 0 = no key), written to sel[0..63] sorted
// descending (0 where fewer exist).  The K-th largest per-thread best key T
// bounds the K-th largest key from below (K threads each hold a key >= T), so
// only keys >= T are gathered (about K of them) and ranked exactly by counting.
// If more than kCap keys are >= T (many ties), an exact radix select runs.
template <int NT, int IPT>
__device__ void block_topk(const unsigned long long (&items)[IPT], int K, unsigned long long* sel,
                           TopkSmem<NT>& sm) {
  const int tid = threadIdx.x, lane = lane_id();
  unsigned long long best = 0ull;
#pragma unroll
  for (int i = 0; i < IPT; ++i) best = items[i] > best ? items[i] : best;
  for (int i = tid; i < kSlots; i += NT) sel[i] = 0ull;
  sm.bests[tid] = best;
  if (tid == 0) {
    sm.count = 0;
    sm.T = 0ull;
  }
  const int n_ok = __syncthreads_count(best != 0ull);
  if (K <= 0) return;
  if (n_ok > K && best != 0ull && count_greater(sm.bests, NT, best) == K - 1) sm.T = best;
  __syncthreads();
  const unsigned long long T = sm.T;
#pragma unroll
  for (int i = 0; i < IPT; ++i) {
    if (items[i] != 0ull && items[i] >= T) {
      const int slot = atomicAdd(&sm.count, 1);
      if (slot < kCap) sm.cand[slot] = items[i];
    }
  }
  __syncthreads();
  const int C = sm.count;
  if (C <= kCap) {
    for (int e = tid; e < C; e += NT) {
      const unsigned long long k = sm.cand[e];
      const int rank = count_greater(sm.cand, C, k);
      if (rank < K) sel[rank] = k;
    }
    __syncthreads();
    return;
  }
  // exact radix select over every key
  __syncthreads();
  if (tid == 0) sm.count = 0;
  unsigned long long prefix = 0ull, mask = 0ull;
  int krem = K;
  for (int shift = 56; shift >= 0; shift -= 8) {
    for (int i = tid; i < 256; i += NT) sm.hist[i] = 0u;
    __syncthreads();
#pragma unroll
    for (int i = 0; i < IPT; ++i)
      if (items[i] != 0ull && (items[i] & mask) == prefix)
        atomicAdd(&sm.hist[(items[i] >> shift) & 255ull], 1u);
    __syncthreads();
    if (tid < kWave) {
      unsigned cc[4];
#pragma unroll
      for (int b = 0; b < 4; ++b) cc[b] = sm.hist[4 * lane + b];
      const unsigned sc = cc[0] + cc[1] + cc[2] + cc[3];
      unsigned inc = sc;
#pragma unroll
      for (int d = 1; d < kWave; d <<= 1) {
        unsigned o = __shfl_down(inc, d, kWave);
        if (lane + d < kWave) inc += o;
      }
      unsigned above = inc - sc;
#pragma unroll
      for (int b = 3; b >= 0; --b) {
        if (above < static_cast<unsigned>(krem) && static_cast<unsigned>(krem) <= above + cc[b]) {
          sm.prefix = prefix | (static_cast<unsigned long long>(4 * lane + b) << shift);
          sm.krem = krem - static_cast<int>(above);
          sm.done = (cc[b] == static_cast<unsigned>(krem) - above) ? 1 : 0;
        }
        above += cc[b];
      }
    }
    __syncthreads();
    prefix = sm.prefix;
    krem = sm.krem;
    const int done = sm.done;
    mask |= 0xFFull << shift;
    __syncthreads();
    if (done) break;
  }
#pragma unroll
  for (int i = 0; i < IPT; ++i) {
    if (items[i] != 0ull && items[i] >= prefix) {
      const int slot = atomicAdd(&sm.count, 1);
      if (slot < kSlots) sm.cand[slot] = items[i];
    }
  }
  __syncthreads();
  if (tid < K) sel[count_greater(sm.cand, K, sm.cand[tid])] = sm.cand[tid];
  __syncthreads();
}

template <typename T>
__device__ __forceinline__ float load_logit(const T* p);
template <>
__device__ __forceinline__ float load_logit<float>(const float* p) { return *p; }
template <>
__device__ __forceinline__ float load_logit<uint16_t>(const uint16_t* p) { return bf16_to_f32(*p); }

// One chunk of kChunkThreads * kChunkVecs * E logits (E per 16 bytes) of one
// offset row; every load is issued before any is used.
template <typename T>
__global__ __launch_bounds__(kChunkThreads) void lsm_chunk_kernel(
    const T* __restrict__ logits, int L, int V, int N, int nch,
    float* __restrict__ cstat, unsigned long long* __restrict__ clist) {
  constexpr int E = 16 / sizeof(T);
  constexpr int IPT = kChunkVecs * E;
  __shared__ float redf[kChunkThreads / kWave];
  __shared__ float s_M;
  __shared__ __attribute__((aligned(16))) TopkSmem<kChunkThreads> sm;
  __shared__ unsigned long long sel[kSlots];

  const int c = blockIdx.x, j = blockIdx.y, sq = blockIdx.z;
  const int row = sq * L + j;
  const int K = k_of(N, V, j);
  const int tid = threadIdx.x, w = tid / kWave, lane = lane_id();
  const T* base = logits + static_cast<size_t>(row) * V;
  const int c0 = c * kChunkThreads * IPT;
  const bool vec = (V % E) == 0;

  float z[IPT];
  int idx[IPT];
  if (vec) {
    uint4 u[kChunkVecs];
#pragma unroll
    for (int v = 0; v < kChunkVecs; ++v) {
      const int e0 = c0 + (v * kChunkThreads + tid) * E;
      u[v] = e0 < V ? load_stream(base + e0) : make_uint4(0, 0, 0, 0);
    }
#pragma unroll
    for (int v = 0; v < kChunkVecs; ++v) {
      const int e0 = c0 + (v * kChunkThreads + tid) * E;
      const uint32_t wd[4] = {u[v].x, u[v].y, u[v].z, u[v].w};
#pragma unroll
      for (int e = 0; e < E; ++e) {
        idx[v * E + e] = e0 + e;
        float x;
        if constexpr (sizeof(T) == 2)
          x = bf16_to_f32(static_cast<uint16_t>(e & 1 ? wd[e >> 1] >> 16 : wd[e >> 1] & 0xFFFF));
        else
          x = __uint_as_float(wd[e]);
        z[v * E + e] = e0 < V ? x : -INFINITY;
      }
    }
  } else {
#pragma unroll
    for (int e = 0; e < IPT; ++e) {
      idx[e] = c0 + e * kChunkThreads + tid;
      z[e] = idx[e] < V ? load_logit<T>(base + idx[e]) : -INFINITY;
    }
  }

  // running max, rescaled sum of exp, keys (logit desc, token id asc)
  float m = -INFINITY;
#pragma unroll
  for (int e = 0; e < IPT; ++e) m = fmaxf(m, z[e]);
  float sum = 0.f;
  unsigned long long keys[IPT];
#pragma unroll
  for (int e = 0; e < IPT; ++e) {
    const bool ok = idx[e] < V;
    if (ok && z[e] != -INFINITY) sum += expf(z[e] - m);
    keys[e] = ok ? make_comp(z[e], static_cast<uint32_t>(idx[e])) : 0ull;
  }
  const float wm = wave_max(m);
  if (lane == 0) redf[w] = wm;
  __syncthreads();
  if (tid == 0) {
    float M = redf[0];
    for (int i = 1; i < kChunkThreads / kWave; ++i) M = fmaxf(M, redf[i]);
    s_M = M;
  }
  __syncthreads();
  const float M = s_M;
  float part = (M == -INFINITY || m == -INFINITY) ? 0.f : sum * expf(m - M);
  part = wave_sum(part);
  __syncthreads();
  if (lane == 0) redf[w] = part;
  __syncthreads();
  if (tid == 0) {
    float S = 0.f;
    for (int i = 0; i < kChunkThreads / kWave; ++i) S += redf[i];
    float* st = cstat + (static_cast<size_t>(row) * nch + c) * 2;
    st[0] = M;
    st[1] = S;
  }
  block_topk<kChunkThreads, IPT>(keys, K, sel, sm);
  if (tid < kSlots) clist[(static_cast<size_t>(row) * nch + c) * kSlots + tid] = sel[tid];
}

// Merge of one offset's sorted chunk lists into its K best, as log q.
__global__ __launch_bounds__(kChunkThreads) void lsm_merge_kernel(
    int L, int V, int N, int nch, const float* __restrict__ cstat,
    const unsigned long long* __restrict__ clist, float* __restrict__ top_logq,
    int32_t* __restrict__ top_id) {
  __shared__ __attribute__((aligned(16))) TopkSmem<kChunkThreads> sm;
  __shared__ unsigned long long sel[kSlots];
  __shared__ float s_M, s_lnS;
  const int j = blockIdx.x, sq = blockIdx.y;
  const int row = sq * L + j;
  const int K = k_of(N, V, j);
  const int tid = threadIdx.x;
  const size_t rowc = static_cast<size_t>(row) * nch;
  const unsigned long long* lists = clist + rowc * kSlots;
  const int n = nch * kSlots;
  unsigned long long items[kMergeItems];
#pragma unroll
  for (int i = 0; i < kMergeItems; ++i) {
    const int e = i * kChunkThreads + tid;
    items[i] = e < n ? lists[e] : 0ull;
  }
  if (tid < kWave) {
    // row maximum and ln(sum exp(z - max)) from the chunk statistics (<= 64)
    const int c = tid;
    const float cm = c < nch ? cstat[(rowc + c) * 2] : -INFINITY;
    const float cs = c < nch ? cstat[(rowc + c) * 2 + 1] : 0.f;
    const float M = wave_max(cm);
    float t = (M == -INFINITY || cs <= 0.f) ? 0.f : cs * expf(cm - M);
    t = wave_sum(t);
    if (tid == 0) {
      s_M = M;
      s_lnS = logf(t);
    }
  }
  block_topk<kChunkThreads, kMergeItems>(items, K, sel, sm);
  if (tid < kSlots) {
    const unsigned long long k = sel[tid];
    float lq = -INFINITY;
    int id = -1;
    if (k != 0ull) {
      const float zz = key_float(static_cast<uint32_t>(k >> 32));
      const float M = s_M;
      id = static_cast<int>(0xFFFFFFFFu - static_cast<uint32_t>(k));
      lq = (M == -INFINITY || zz == -INFINITY) ? -INFINITY : (zz - M) - s_lnS;
    }
    top_logq[static_cast<size_t>(row) * kSlots + tid] = lq;
    top_id[static_cast<size_t>(row) * kSlots + tid] = id;
  }
}

__global__ __launch_bounds__(4 * kWave) void build_tree_kernel(
    const float* __restrict__ top_logq, const int32_t* __restrict__ top_id,
    const int32_t* __restrict__ root_token, int L, int V, int N, int32_t* __restrict__ parent,
    int32_t* __restrict__ depth_out, int32_t* __restrict__ token_out,
    uint64_t* __restrict__ anc_out, float* __restrict__ score_out,
    int32_t* __restrict__ n_valid_out) {
  __shared__ float lq[GLANCE_MAX_L][kSlots];
  __shared__ int tk[GLANCE_MAX_L][kSlots];
  __shared__ int row_of_lane[kSlots];
  __shared__ unsigned long long anc_row[kSlots];

  const int s = blockIdx.x, lane = lane_id(), wv = threadIdx.x / kWave;

  // the ranked lists of every offset
  {
    float vq[GLANCE_MAX_L * kSlots / (4 * kWave)];
    int vt[GLANCE_MAX_L * kSlots / (4 * kWave)];
#pragma unroll
    for (int u = 0; u < GLANCE_MAX_L * kSlots / (4 * kWave); ++u) {
      const int e = u * 4 * kWave + threadIdx.x;
      vq[u] = e < L * kSlots ? top_logq[static_cast<size_t>(s) * L * kSlots + e] : -INFINITY;
      vt[u] = e < L * kSlots ? top_id[static_cast<size_t>(s) * L * kSlots + e] : -1;
    }
#pragma unroll
    for (int u = 0; u < GLANCE_MAX_L * kSlots / (4 * kWave); ++u) {
      const int e = u * 4 * kWave + threadIdx.x;
      lq[e / kSlots][e % kSlots] = vq[u];
      tk[e / kSlots][e % kSlots] = vt[u];
    }
  }
  __syncthreads();
  if (wv != 0) return;  // the rest is one wavefront; no block barrier follows

  // ---- best-first selection.  Lane 0 is the root, lane i the i-th selected
  // node; each lane offers the best not-yet-selected child of its node (the
  // next entry of the next offset's ranked list).  Equal scores: smaller depth,
  // then the earlier-selected parent (smaller lane); one offer per lane.
  const int R = N + 1;
  const float fq = lane < L ? lq[lane][0] : -INFINITY;  // first entry of each offset
  float n_score = 0.f;
  int n_depth = 0, n_par = -1, n_rank = 0, n_next = 0;
  float c_score = 0.f, nx_q = -INFINITY;
  uint32_t c_hi = 0u;
  // the candidate is child n_next of this node with log q `q`; prefetch the next one
  auto offer = [&](float q) {
    c_hi = 0u;
    if (n_depth < L && n_next < k_of(N, V, n_depth) && q != -INFINITY) {
      c_score = n_score + q;
      c_hi = float_key(c_score);
    }
    const int nn = n_next + 1;
    nx_q = (n_depth < L && nn < kSlots) ? lq[n_depth][nn] : -INFINITY;
  };
  if (lane == 0) offer(fq);
  int n_pop = 0;
  for (int i = 1; i <= N; ++i) {
    const uint32_t mh = wave_umax(c_hi);
    if (mh == 0u) break;
    unsigned long long cm = __ballot(c_hi == mh);
    if (__popcll(cm) > 1) {  // equal scores: the smallest child depth, then the lowest lane
      const uint32_t lo = (c_hi == mh) ? ~static_cast<uint32_t>(n_depth) : 0u;
      const uint32_t ml = wave_umax(lo);
      cm = __ballot(c_hi == mh && ~static_cast<uint32_t>(n_depth) == ml);
    }
    const int p = __ffsll(static_cast<long long>(cm)) - 1;
    const float w_score = readlane_f(c_score, p);
    const int w_depth = readlane_i(n_depth, p) + 1;
    const int w_rank = readlane_i(n_next, p);
    const float q0 = readlane_f(fq, w_depth < L ? w_depth : 0);
    if (lane == i) {
      n_score = w_score;
      n_depth = w_depth;
      n_par = p;
      n_rank = w_rank;
      n_next = 0;
      offer(w_depth < L ? q0 : -INFINITY);
    }
    if (lane == p) {
      ++n_next;
      offer(nx_q);
    }
    n_pop = i;
  }

  // ---- breadth-first layout: rows by (depth, parent row, token id)
  const int n_token = (lane >= 1 && lane <= n_pop) ? tk[n_depth - 1][n_rank] : -1;
  const size_t ob = static_cast<size_t>(s) * R;
  if (lane == 0) {
    row_of_lane[0] = 0;
    anc_row[0] = 1ull;
    parent[ob] = -1;
    depth_out[ob] = 0;
    token_out[ob] = root_token[s];
    anc_out[ob] = 1ull;
    score_out[ob] = 0.f;
    n_valid_out[s] = n_pop + 1;
  }
  __builtin_amdgcn_wave_barrier();  // one wave: LDS is in order
  int base = 1;
  for (int d = 1; d <= L; ++d) {
    const bool in_level = lane >= 1 && lane <= n_pop && n_depth == d;
    const unsigned long long lvl = __ballot(in_level);
    if (lvl == 0ull) break;
    const int prow = in_level ? row_of_lane[n_par] : 0;
    int rank = 0;
    unsigned long long mm = lvl;
    while (mm) {
      const int jl = __ffsll(static_cast<long long>(mm)) - 1;
      mm &= mm - 1;
      const int op = readlane_i(prow, jl), ot = readlane_i(n_token, jl);
      rank += (op < prow || (op == prow && ot < n_token)) ? 1 : 0;
    }
    if (in_level) {
      const int r = base + rank;
      row_of_lane[lane] = r;
      const unsigned long long a = anc_row[prow] | (1ull << r);
      anc_row[r] = a;
      parent[ob + r] = prow;
      depth_out[ob + r] = d;
      token_out[ob + r] = n_token;
      anc_out[ob + r] = a;
      score_out[ob + r] = n_score;
    }
    base += __popcll(lvl);
    __builtin_amdgcn_wave_barrier();  // one wave: LDS is in order
  }
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
  // chunks of 256 threads x 2 vectors of 16 bytes: 4096 bf16 or 2048 fp32
  // logits; the merge takes up to 64 chunks per row (V <= 2^18 bf16, 2^17 fp32)
  w.chunk = kChunkThreads * kChunkVecs * 4;
  w.nch = (V + w.chunk - 1) / w.chunk;
  const size_t r = static_cast<size_t>(nseq) * L;
  auto up = [](size_t b) { return (b + 255) & ~static_cast<size_t>(255); };
  const int nch_max = w.nch;
  w.off_cstat = 0;
  w.off_clist = up(r * nch_max * 2 * sizeof(float));
  w.off_logq = w.off_clist + up(r * nch_max * kSlots * sizeof(unsigned long long));
  w.off_id = w.off_logq + up(r * kSlots * sizeof(float));
  w.bytes = w.off_id + up(r * kSlots * sizeof(int32_t));
  return w;
}

glance_status launch_build_tree(const void* logits, int dtype, const int32_t* root, int nseq,
                                int L, int V, int N, int32_t* parent, int32_t* depth,
                                int32_t* token, uint64_t* anc, float* score,
                                int32_t* n_valid, void* ws, hipStream_t st) {
  const TreeWs w = tree_ws_layout(nseq, L, V);
  char* base = static_cast<char*>(ws);
  float* cstat = reinterpret_cast<float*>(base + w.off_cstat);
  unsigned long long* clist = reinterpret_cast<unsigned long long*>(base + w.off_clist);
  // chunk size in logits: 256 threads x 2 x 16 bytes
  const int E = dtype == GLANCE_BF16 ? 8 : 4;
  const int nch = (V + kChunkThreads * kChunkVecs * E - 1) / (kChunkThreads * kChunkVecs * E);
  dim3 ga(nch, L, nseq);
  if (dtype == GLANCE_BF16)
    lsm_chunk_kernel<uint16_t><<<ga, kChunkThreads, 0, st>>>(static_cast<const uint16_t*>(logits), L, V, N,
                                                             nch, cstat, clist);
  else
    lsm_chunk_kernel<float><<<ga, kChunkThreads, 0, st>>>(static_cast<const float*>(logits), L, V, N, nch,
                                                          cstat, clist);
  GLANCE_LAUNCH_CHECK();
  float* logq = reinterpret_cast<float*>(base + w.off_logq);
  int32_t* id = reinterpret_cast<int32_t*>(base + w.off_id);
  lsm_merge_kernel<<<dim3(L, nseq), kChunkThreads, 0, st>>>(L, V, N, nch, cstat, clist, logq, id);
  GLANCE_LAUNCH_CHECK();
  build_tree_kernel<<<nseq, 4 * kWave, 0, st>>>(logq, id, root, L, V, N, parent, depth, token, anc,
                                                score, n_valid);
  GLANCE_LAUNCH_CHECK();
  return GLANCE_OK;
}

}  // namespace glance
