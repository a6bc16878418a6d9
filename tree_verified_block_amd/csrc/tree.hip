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
// One launch, grid (chunk, offset row, sequence) x 256 threads, three phases:
//   1. every work-group streams its chunk of an offset row once (every load
//      issued up front): max, sum of exp, and the chunk's K best keys through a
//      per-wave threshold and exact rank counting;
//   2. the last chunk of a row to finish merges the row's chunk lists into the
//      offset's K best tokens with log q_j(v) = (z_v - max) - ln(sum exp(z - max));
//   3. the last row of a sequence to be merged runs best-first selection in one
//      wavefront (lane 0 is the root, lane i the i-th selected node; every lane
//      offers the best not-yet-selected child of its node, so a selection is one
//      wave max and touches two lanes) and lays the nodes out breadth-first with
//      their ancestor masks.
// Work-groups meet through arrival counters (device-scope atomics); everything
// they publish to each other is stored and loaded with device-coherent accesses.
#include "common.h"
#include "kernels.h"

namespace glance {

namespace {

constexpr int kSlots = 64;  // candidate slots per (offset, chunk); K_j <= 63
constexpr int kLqRow = 72;  // LDS row of a ranked list: 64 entries and -inf padding

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
constexpr int kChunkWaves = kChunkThreads / kWave;
constexpr int kMaxVec = 8;       // 16-byte vectors per thread
constexpr int kMaxChunks = 16;   // chunk lists per offset row
constexpr int kCap = 2048;       // candidates gathered above the threshold

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

__device__ __forceinline__ unsigned long long umax64(unsigned long long a, unsigned long long b) {
  return a > b ? a : b;
}
__device__ __forceinline__ unsigned long long umin64(unsigned long long a, unsigned long long b) {
  return a > b ? b : a;
}

// Wave-wide float max and sum through DPP row shifts and row broadcasts: lane
// 63 ends with the result over all 64 lanes (lanes that receive no source
// combine with the identity), read back as a wave-uniform value.
#define GLANCE_DPP_STEP(v, op, id, ctrl, rm) \
  v = op(v, __int_as_float(__builtin_amdgcn_update_dpp(id, __float_as_int(v), ctrl, rm, 0xF, false)))
__device__ __forceinline__ float fadd2(float a, float b) { return a + b; }
__device__ __forceinline__ float wave_fmax_u(float v) {
  constexpr int kNegInf = static_cast<int>(0xFF800000u);
  GLANCE_DPP_STEP(v, fmaxf, kNegInf, 0x111, 0xF);
  GLANCE_DPP_STEP(v, fmaxf, kNegInf, 0x112, 0xF);
  GLANCE_DPP_STEP(v, fmaxf, kNegInf, 0x114, 0xF);
  GLANCE_DPP_STEP(v, fmaxf, kNegInf, 0x118, 0xF);
  GLANCE_DPP_STEP(v, fmaxf, kNegInf, 0x142, 0xA);
  GLANCE_DPP_STEP(v, fmaxf, kNegInf, 0x143, 0xC);
  return readlane_f(v, 63);
}
__device__ __forceinline__ float wave_fsum_u(float v) {
  GLANCE_DPP_STEP(v, fadd2, 0, 0x111, 0xF);
  GLANCE_DPP_STEP(v, fadd2, 0, 0x112, 0xF);
  GLANCE_DPP_STEP(v, fadd2, 0, 0x114, 0xF);
  GLANCE_DPP_STEP(v, fadd2, 0, 0x118, 0xF);
  GLANCE_DPP_STEP(v, fadd2, 0, 0x142, 0xA);
  GLANCE_DPP_STEP(v, fadd2, 0, 0x143, 0xC);
  return readlane_f(v, 63);
}
#undef GLANCE_DPP_STEP

// The value of lane (lane ^ J), on the vector ALU only: DPP quad permutations
// for 1 and 2, row shifts by 4 (left for lanes with bit 2 clear, right
// otherwise) for 4, a row rotation by 8 for 8, and the row-pair and half swaps
// of the 16- and 32-lane permutes for 16 and 32.
template <int J>
__device__ __forceinline__ uint32_t xor_lane(uint32_t v) {
  const int x = static_cast<int>(v);
  if constexpr (J == 1)
    return static_cast<uint32_t>(__builtin_amdgcn_update_dpp(0, x, 0xB1, 0xF, 0xF, false));
  else if constexpr (J == 2)
    return static_cast<uint32_t>(__builtin_amdgcn_update_dpp(0, x, 0x4E, 0xF, 0xF, false));
  else if constexpr (J == 4) {
    const int up = __builtin_amdgcn_update_dpp(0, x, 0x104, 0xF, 0xF, false);    // row_shl:4
    const int down = __builtin_amdgcn_update_dpp(0, x, 0x114, 0xF, 0xF, false);  // row_shr:4
    return static_cast<uint32_t>((lane_id() & 4) ? down : up);
  } else if constexpr (J == 8)
    return static_cast<uint32_t>(__builtin_amdgcn_update_dpp(0, x, 0x128, 0xF, 0xF, false));
  else if constexpr (J == 16) {
    const auto r = __builtin_amdgcn_permlane16_swap(v, v, false, false);
    return (lane_id() & 16) ? r[0] : r[1];
  } else {
    static_assert(J == 32, "lane exchange distance");
    const auto r = __builtin_amdgcn_permlane32_swap(v, v, false, false);
    return lane_id() < 32 ? r[1] : r[0];
  }
}
template <int J>
__device__ __forceinline__ unsigned long long xor_lane64(unsigned long long v) {
  const uint32_t lo = xor_lane<J>(static_cast<uint32_t>(v)), hi = xor_lane<J>(static_cast<uint32_t>(v >> 32));
  return (static_cast<unsigned long long>(hi) << 32) | lo;
}
template <int J>
__device__ __forceinline__ unsigned long long cleave(unsigned long long v) {
  const unsigned long long o = xor_lane64<J>(v);
  return (lane_id() & J) ? umin64(v, o) : umax64(v, o);
}

// One step of the bitonic sorting network over the 64 lanes: blocks of size
// K2 alternate direction (descending first), J is the exchange distance.
template <int K2, int J>
__device__ __forceinline__ unsigned long long bitonic_step(unsigned long long v) {
  const unsigned long long o = xor_lane64<J>(v);
  const int lane = lane_id();
  const bool keep_max = ((lane & J) == 0) == ((lane & K2) == 0);
  return keep_max ? umax64(v, o) : umin64(v, o);
}

// Descending sort of one key per lane (21 compare-exchange steps).
__device__ __forceinline__ unsigned long long wave_sort64_desc(unsigned long long v) {
  v = bitonic_step<2, 1>(v);
  v = bitonic_step<4, 2>(v);
  v = bitonic_step<4, 1>(v);
  v = bitonic_step<8, 4>(v);
  v = bitonic_step<8, 2>(v);
  v = bitonic_step<8, 1>(v);
  v = bitonic_step<16, 8>(v);
  v = bitonic_step<16, 4>(v);
  v = bitonic_step<16, 2>(v);
  v = bitonic_step<16, 1>(v);
  v = bitonic_step<32, 16>(v);
  v = bitonic_step<32, 8>(v);
  v = bitonic_step<32, 4>(v);
  v = bitonic_step<32, 2>(v);
  v = bitonic_step<32, 1>(v);
  v = bitonic_step<64, 32>(v);
  v = bitonic_step<64, 16>(v);
  v = bitonic_step<64, 8>(v);
  v = bitonic_step<64, 4>(v);
  v = bitonic_step<64, 2>(v);
  v = bitonic_step<64, 1>(v);
  return v;
}

// z[e] for a lane-dependent e < N, by a binary tree of selects on the bits of e
// (register arrays are never indexed dynamically).
template <int N>
__device__ __forceinline__ float select_elem(const float (&z)[N], int e) {
  float t[N];
#pragma unroll
  for (int k = 0; k < N; ++k) t[k] = z[k];
#pragma unroll
  for (int bit = 0; bit < 7; ++bit) {
    constexpr int one = 1;
    const int step = one << bit;
    if (step >= N) break;
    const bool hi = ((e >> bit) & 1) != 0;
#pragma unroll
    for (int k = 0; k + step < N; k += 2 * step) t[k] = hi ? t[k + step] : t[k];
  }
  return t[0];
}

// Top 64 of two descending 64-key lists, descending: lane l holds a = A[l] and
// b = B[63 - l].  max(a, b) over the lanes is a bitonic sequence holding the 64
// largest keys of A and B; six half-cleaner stages sort it.
__device__ __forceinline__ unsigned long long merge_top64(unsigned long long a, unsigned long long b) {
  unsigned long long v = umax64(a, b);
  v = cleave<32>(v);
  v = cleave<16>(v);
  v = cleave<8>(v);
  v = cleave<4>(v);
  v = cleave<2>(v);
  v = cleave<1>(v);
  return v;
}

template <typename T>
__device__ __forceinline__ float load_logit(const T* p);
template <>
__device__ __forceinline__ float load_logit<float>(const float* p) { return *p; }
template <>
__device__ __forceinline__ float load_logit<uint16_t>(const uint16_t* p) { return bf16_to_f32(*p); }

// Phase 1, one chunk of an offset row: 256 threads x NV vectors of 16 bytes,
// every load issued before any is used.  Publishes the chunk's maximum and sum
// of exp(z - max) and its K best keys, sorted descending (0 where fewer exist),
// with device-coherent stores.
// Threshold: each wave finds, on ballots, the largest 16-bit prefix that k =
// ceil(K/4) of its per-thread best keys reach; the smallest over the four waves
// is a lower bound of the chunk's K-th largest key (each wave holds k keys above
// it).  Only the keys above it (about K of them) are gathered to LDS.  When no
// wave holds more than 64 of them, each wave sorts its keys (bitonic network)
// and the four sorted lists are merged; otherwise they are ranked exactly by
// counting, and more than a wave's share of kCap of them (massive ties)
// switches to an exact 8-bit radix select.
template <typename T, int NV>
__device__ __forceinline__ void chunk_topk(const T* __restrict__ logits, int L, int V, int N, int nch,
                                           unsigned long long* __restrict__ cstat,
                                           unsigned long long* __restrict__ clist,
                                           unsigned long long* cand, unsigned* __restrict__ flag) {
  constexpr int E = 16 / sizeof(T);
  constexpr int IPT = NV * E;
  __shared__ unsigned long long sel[kSlots];
  __shared__ uint32_t wt[kChunkWaves];
  __shared__ int wcnt[kChunkWaves];
  __shared__ float red_m[kChunkWaves], red_s[kChunkWaves];
  __shared__ unsigned hist[256];
  __shared__ int s_count, s_krem, s_done;
  __shared__ unsigned long long s_prefix;

  const int c = blockIdx.x, j = blockIdx.y, sq = blockIdx.z;
  const int row = sq * L + j;
  const int K = k_of(N, V, j);
  const int tid = threadIdx.x, w = tid / kWave, lane = lane_id();
  const T* base = logits + static_cast<size_t>(row) * V;
  const int c0 = c * kChunkThreads * IPT;  // first logit of the chunk

  // element e: vector path token idx0 + (e/E)*256*E + e%E (V % E == 0), else
  // token idx0 + e*256; token ids increase with e
  const bool vec = V % E == 0;
  const int idx0 = vec ? c0 + tid * E : c0 + tid;
  auto tok = [&](int e) { return vec ? idx0 + (e / E) * kChunkThreads * E + (e % E) : idx0 + e * kChunkThreads; };
  float z[IPT];
  bool ok[IPT];
  if (vec) {
    uint4 u[NV];
#pragma unroll
    for (int b = 0; b < NV; ++b) {
      const int i = idx0 + b * kChunkThreads * E;
      u[b] = i < V ? *reinterpret_cast<const uint4*>(base + i) : make_uint4(0, 0, 0, 0);
    }
#pragma unroll
    for (int b = 0; b < NV; ++b) {
      const bool vb = idx0 + b * kChunkThreads * E < V;
      const uint32_t wd[4] = {u[b].x, u[b].y, u[b].z, u[b].w};
#pragma unroll
      for (int e = 0; e < E; ++e) {
        if constexpr (sizeof(T) == 2)
          z[b * E + e] = bf16_to_f32(static_cast<uint16_t>(e & 1 ? wd[e >> 1] >> 16 : wd[e >> 1] & 0xFFFF));
        else
          z[b * E + e] = __uint_as_float(wd[e]);
        ok[b * E + e] = vb;
      }
    }
  } else {
#pragma unroll
    for (int e = 0; e < IPT; ++e) {
      const int i = idx0 + e * kChunkThreads;
      ok[e] = i < V;
      z[e] = ok[e] ? load_logit<T>(base + i) : 0.f;
    }
  }

  // running max and best (strict comparison: the smallest id wins a tie); NaN
  // and +inf logits are reported in the flag word (bit 0 and bit 1)
  float m = -INFINITY, bz = -INFINITY;
  int bi = -1;
  bool nan_seen = false, pinf_seen = false;
#pragma unroll
  for (int e = 0; e < IPT; ++e) {
    if (ok[e]) {
      m = fmaxf(m, z[e]);
      nan_seen |= z[e] != z[e];
      pinf_seen |= z[e] == INFINITY;
      if (bi < 0 || z[e] > bz) {
        bz = z[e];
        bi = tok(e);
      }
    }
  }
  {
    const bool bn = __ballot(nan_seen) != 0ull, bp = __ballot(pinf_seen) != 0ull;
    if (lane == 0 && (bn || bp))
      __hip_atomic_fetch_or(flag, (bn ? 1u : 0u) | (bp ? 2u : 0u), __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  }
  // sum of exp(z - m) through the hardware exp2 (z - m <= 0)
  float s = 0.f;
  if (m != -INFINITY) {
#pragma unroll
    for (int e = 0; e < IPT; ++e)
      if (ok[e]) s += __builtin_amdgcn_exp2f((z[e] - m) * 1.4426950408889634f);
  }
  const float wm = wave_fmax_u(m);
  float part = (wm == -INFINITY || m == -INFINITY) ? 0.f : s * __builtin_amdgcn_exp2f((m - wm) * 1.4426950408889634f);
  part = wave_fsum_u(part);
  // this wave's threshold t: the largest value with zero low 16 bits that at
  // least k = ceil(K/4) of the per-thread best keys (high 32 bits) reach, found
  // bit by bit on ballots; the minimum T over the four waves is then reached by
  // at least K keys of the chunk
  // A -inf logit (a token of probability 0) never enters a tree: it takes no
  // part in the threshold or the gather.  (Its key, float_key(-inf), sits just
  // below every finite key; a threshold at its 16-bit prefix would map back to
  // a NaN and gather nothing.)  Finite keys are >= 0x00800000, so the threshold
  // is 0 or a finite value's prefix.
  const int kw = (K + kChunkWaves - 1) / kChunkWaves;
  const uint32_t kb = (bi >= 0 && bz > -INFINITY) ? float_key(bz) : 0u;
  uint32_t t = 0u;
  if (kw > 0) {
#pragma unroll
    for (int bit = 31; bit >= 16; --bit) {
      const uint32_t tc = t | (1u << bit);
      if (static_cast<int>(__popcll(__ballot(kb >= tc))) >= kw) t = tc;
    }
  }
  if (lane == 0) {
    red_m[w] = wm;
    red_s[w] = part;
    wt[w] = t;
  }
  if (tid < kSlots) sel[tid] = 0ull;
  __syncthreads();
  if (tid == 0) {
    float M = -INFINITY;
    for (int i = 0; i < kChunkWaves; ++i) M = fmaxf(M, red_m[i]);
    float S = 0.f;
    for (int i = 0; i < kChunkWaves; ++i)
      if (red_m[i] != -INFINITY) S += red_s[i] * __builtin_amdgcn_exp2f((red_m[i] - M) * 1.4426950408889634f);
    const unsigned long long ms = (static_cast<unsigned long long>(__float_as_uint(S)) << 32) | __float_as_uint(M);
    __hip_atomic_store(cstat + static_cast<size_t>(row) * nch + c, ms, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  }
  unsigned long long* out = clist + (static_cast<size_t>(row) * nch + c) * kSlots;
  if (K <= 0) {  // (uniform) nothing of this offset can enter the tree
    if (tid < kSlots) __hip_atomic_store(out + tid, 0ull, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    return;
  }
  uint32_t thr = wt[0];
#pragma unroll
  for (int i = 1; i < kChunkWaves; ++i) thr = min(thr, wt[i]);
  // Gather every key whose value reaches key_float(thr) (a superset of the keys
  // with high part >= thr; thr = 0: every valid key) into this wave's region of
  // the candidate array, at ballot offsets; a region that overflows sends the
  // chunk to the radix select.
  const float zT = thr == 0u ? -INFINITY : key_float(thr);
  constexpr int RW = kCap / kChunkWaves;
  unsigned long long* cw = cand + w * RW;
  // this thread's elements that reach zT as a bit mask, its slots from a wave
  // prefix sum; only the set bits are visited
  unsigned long long pm = 0ull;
#pragma unroll
  for (int e = 0; e < IPT; ++e)
    if (ok[e] && z[e] >= zT && z[e] > -INFINITY) pm |= 1ull << e;
  const int pc = __popcll(pm);
  const int incl = wave_incl_sum(pc);
  const int run = readlane_i(incl, kWave - 1);
  int slot = incl - pc;
  while (pm != 0ull) {
    const int e = __builtin_ctzll(pm);
    pm &= pm - 1ull;
    if (slot < RW) cw[slot] = make_comp(select_elem(z, e), static_cast<uint32_t>(tok(e)));
    ++slot;
  }
  if (lane == 0) wcnt[w] = run;
  __syncthreads();
  int cn[kChunkWaves], C = 0;
  bool over = false, small = true;
#pragma unroll
  for (int i = 0; i < kChunkWaves; ++i) {
    cn[i] = wcnt[i];
    over |= cn[i] > RW;
    small &= cn[i] <= kWave;
    C += cn[i];
  }
  if (small) {
    // every wave sorts its candidates (one per lane); the four sorted lists are
    // then merged pairwise
    unsigned long long x = lane < cn[w] ? cw[lane] : 0ull;
    x = wave_sort64_desc(x);
    cw[lane] = x;
    __syncthreads();
    if (w < 2) {
      x = merge_top64(x, cand[(w + 2) * RW + (kWave - 1 - lane)]);
      cw[lane] = x;
    }
    __syncthreads();
    if (w == 0) {
      x = merge_top64(x, cand[RW + (kWave - 1 - lane)]);
      sel[lane] = lane < K ? x : 0ull;
    }
  } else if (!over) {
    // exact ranks by counting over the four regions
    for (int x = tid; x < C; x += kChunkThreads) {
      int r = 0, o = x;
#pragma unroll
      for (int i = 0; i < kChunkWaves - 1; ++i)
        if (r == i && o >= cn[i]) {
          o -= cn[i];
          r = i + 1;
        }
      const unsigned long long k = cand[r * RW + o];
      int rank = 0;
#pragma unroll
      for (int i = 0; i < kChunkWaves; ++i) rank += count_greater(cand + i * RW, cn[i], k);
      if (rank < K) sel[rank] = k;
    }
  } else {
    // exact radix select of the K-th largest key, 8 bits at a time
    unsigned long long prefix = 0ull, mask = 0ull;
    int krem = K;
    for (int shift = 56; shift >= 0; shift -= 8) {
      for (int i = tid; i < 256; i += kChunkThreads) hist[i] = 0u;
      __syncthreads();
#pragma unroll
      for (int e = 0; e < IPT; ++e) {
        if (ok[e]) {
          const unsigned long long key = make_comp(z[e], static_cast<uint32_t>(tok(e)));
          if ((key & mask) == prefix) atomicAdd(&hist[(key >> shift) & 255ull], 1u);
        }
      }
      __syncthreads();
      if (tid < kWave) {
        unsigned cc[4];
#pragma unroll
        for (int b = 0; b < 4; ++b) cc[b] = hist[4 * lane + b];
        const unsigned sc = cc[0] + cc[1] + cc[2] + cc[3];
        unsigned above = sc;  // keys in this lane's bins and all higher bins
#pragma unroll
        for (int d = 1; d < kWave; d <<= 1) {
          const unsigned o = __shfl_down(above, d, kWave);
          if (lane + d < kWave) above += o;
        }
        above -= sc;
#pragma unroll
        for (int b = 3; b >= 0; --b) {
          if (above < static_cast<unsigned>(krem) && static_cast<unsigned>(krem) <= above + cc[b]) {
            s_prefix = prefix | (static_cast<unsigned long long>(4 * lane + b) << shift);
            s_krem = krem - static_cast<int>(above);
            s_done = cc[b] == static_cast<unsigned>(krem) - above ? 1 : 0;
          }
          above += cc[b];
        }
      }
      __syncthreads();
      prefix = s_prefix;
      krem = s_krem;
      const int done = s_done;
      mask |= 0xFFull << shift;
      __syncthreads();
      if (done) break;
    }
    // exactly K keys are >= prefix (keys are distinct)
    if (tid == 0) s_count = 0;
    __syncthreads();
#pragma unroll
    for (int e = 0; e < IPT; ++e) {
      if (ok[e]) {
        const unsigned long long key = make_comp(z[e], static_cast<uint32_t>(tok(e)));
        if (key >= prefix) {
          const int at = atomicAdd(&s_count, 1);
          if (at < kSlots) cand[at] = key;
        }
      }
    }
    __syncthreads();
    if (tid < K) sel[count_greater(cand, K, cand[tid])] = cand[tid];
  }
  __syncthreads();
  if (tid < kSlots) __hip_atomic_store(out + tid, sel[tid], __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// Phase 2, the last chunk of offset row `row` to finish: merge the row's chunk
// lists (each sorted descending, 0 past its end) into the row's K best tokens,
// ranked, with log q_j(v) = (z_v - M) - ln S.  Wave w folds lists w, w + 4, ...
// into a running top 64 held one key per lane (bitonic merges), then the four
// waves' lists are merged pairwise.  Writes lq[row][64] (log q in rank order,
// -inf past K) and tk[row][64] (token ids, -1 past K).
__device__ __noinline__ void merge_row(const unsigned long long* __restrict__ cstat,
                                       const unsigned long long* __restrict__ clist, int nch,
                                       int row, int K, float* __restrict__ lq_out,
                                       int* __restrict__ tk_out, unsigned long long* buf) {
  __shared__ float s_lnS, s_M;
  const int tid = threadIdx.x, w = tid / kWave, lane = lane_id();
  unsigned long long* lists = buf;                          // [nch][64]
  unsigned long long* part = buf + kMaxChunks * kSlots;     // [4][64] per-wave results
  constexpr int PER = kMaxChunks * kSlots / kChunkThreads;
  unsigned long long key[PER];
#pragma unroll
  for (int i = 0; i < PER; ++i) {
    const int idx = tid + i * kChunkThreads;
    key[i] = (idx >> 6) < nch
                 ? __hip_atomic_load(clist + static_cast<size_t>(row) * nch * kSlots + idx, __ATOMIC_RELAXED,
                                     __HIP_MEMORY_SCOPE_AGENT)
                 : 0ull;
  }
  if (w == 0) {
    const unsigned long long ms = lane < nch ? __hip_atomic_load(cstat + static_cast<size_t>(row) * nch + lane,
                                                                 __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT)
                                             : 0ull;
    const float m = lane < nch ? __uint_as_float(static_cast<uint32_t>(ms)) : -INFINITY;
    const float sm = lane < nch ? __uint_as_float(static_cast<uint32_t>(ms >> 32)) : 0.f;
    const float M = wave_max(m);
    float t = (M == -INFINITY || sm <= 0.f) ? 0.f : sm * __builtin_amdgcn_exp2f((m - M) * 1.4426950408889634f);
    t = wave_sum(t);
    if (lane == 0) {
      s_M = M;
      s_lnS = logf(t);
    }
  }
#pragma unroll
  for (int i = 0; i < PER; ++i) {
    const int idx = tid + i * kChunkThreads;
    if ((idx >> 6) < nch) lists[idx] = key[i];
  }
  __syncthreads();
  unsigned long long v = w < nch ? lists[w * kSlots + lane] : 0ull;
  for (int c = w + kChunkWaves; c < nch; c += kChunkWaves)
    v = merge_top64(v, lists[c * kSlots + (kSlots - 1 - lane)]);
  part[w * kSlots + lane] = v;
  __syncthreads();
  if (w < 2) {
    v = merge_top64(v, part[(w + 2) * kSlots + (kSlots - 1 - lane)]);
    part[w * kSlots + lane] = v;
  }
  __syncthreads();
  if (w == 0) {
    v = merge_top64(v, part[kSlots + (kSlots - 1 - lane)]);
    const float M = s_M, lnS = s_lnS;
    float lq = -INFINITY;
    int tk = -1;
    if (lane < K && v != 0ull) {
      const float zz = key_float(static_cast<uint32_t>(v >> 32));
      lq = (M == -INFINITY || zz == -INFINITY) ? -INFINITY : (zz - M) - lnS;
      tk = static_cast<int>(0xFFFFFFFFu - static_cast<uint32_t>(v));
    }
    __hip_atomic_store(lq_out + static_cast<size_t>(row) * kSlots + lane, lq, __ATOMIC_RELAXED,
                       __HIP_MEMORY_SCOPE_AGENT);
    __hip_atomic_store(tk_out + static_cast<size_t>(row) * kSlots + lane, tk, __ATOMIC_RELAXED,
                       __HIP_MEMORY_SCOPE_AGENT);
  }
}

// A selected node as its lane holds it after the selection (lane i = the i-th
// selected node): depth, token id, parent lane and plug-in log score.
struct PopState {
  int depth;
  int token;
  int par;
  float score;
};

// Phase 3a, one wavefront: best-first selection of up to N nodes over the ranked
// lists in LDS.  Returns the number of selected nodes (wave-uniform); lane i
// (1 <= i <= that number) holds the i-th selected node.
__device__ __forceinline__ int select_pops(const float (*lq)[kLqRow], const int (*tk)[kSlots], int L,
                                           int N, PopState& ps) {
  const int lane = lane_id();
  // Lane 0 is the root, lane i the i-th selected node; each lane offers the
  // best not-yet-selected child of its node (the next entry of the list of its
  // depth).  Equal scores: smaller depth, then the earlier-selected parent
  // (smaller lane); a lane offers one child at a time.  Scores are sums of
  // log q <= 0, so the order key of a score v is 0x7F800000 - bits(|v|): larger
  // scores give larger keys, -inf (no offer) gives 0, and the key maps back to
  // -|v| on the scalar unit.  Per iteration only the winner p and the new node
  // i change, from scalar values; every lane re-reads the log q after its
  // offered child and the first log q of the list below its offered child, so
  // both reads are issued one iteration ahead of their use and the winner's
  // two values come from two independent lane reads.
  // Lane state: st = depth << 16 | own rank << 8 | rank of the offered child.
  auto okey = [](float v) { return 0x7F800000u - (__float_as_uint(v) & 0x7FFFFFFFu); };
  const float fq = lane <= L ? lq[lane][0] : -INFINITY;  // first entry of each list
  int st = 0;
  float n_score = 0.f;
  int n_par = -1;
  uint32_t c_hi = lane == 0 ? okey(fq) : 0u;
  float nx_q = lq[0][1];  // log q after the offered child (lane 0: the root's second child)
  float fqn = lq[1][0];   // first log q below the offered child (lane 0: list 1)
  int n_pop = 0;
  uint32_t mh = N >= 1 ? wave_umax(c_hi) : 0u;
  for (int i = 1; mh != 0u;) {
    unsigned long long cm = __ballot(c_hi == mh);
    if (__builtin_expect((cm & (cm - 1ull)) != 0ull, 0)) {  // equal scores: the smallest depth, then the lowest lane
      const uint32_t lo = (c_hi == mh) ? ~static_cast<uint32_t>(st >> 16) : 0u;
      const uint32_t ml = wave_umax(lo);
      cm = __ballot(c_hi == mh && ~static_cast<uint32_t>(st >> 16) == ml);
    }
    const int p = __builtin_ctzll(cm);  // cm holds the lane of mh, never empty
    const int w_st = readlane_i(st, p);
    const int dn = (w_st >> 16) + 1;                        // the new node's depth
    const int new_st = (dn << 16) | ((w_st & 255) << 8);    // its own rank, first child offered
    const float w_score = __uint_as_float((0x7F800000u - mh) | 0x80000000u);
    const float q0 = readlane_f(fqn, p);
    const bool isp = lane == p, isi = lane == i;
    st += isp ? 1 : 0;
    st = isi ? new_st : st;
    n_score = isi ? w_score : n_score;
    n_par = isi ? p : n_par;
    n_pop = i;
    if (++i > N) break;  // (the offers and reads below serve only a next pop)
    const uint32_t k = okey(n_score + (isi ? q0 : nx_q));
    c_hi = (isp | isi) ? k : c_hi;
    // the old log q is dead here: the next reads may load straight into its
    // register (issued above this point, they would land in a temporary whose
    // copy at the end of the iteration waits for them)
    __builtin_amdgcn_sched_barrier(0);
    nx_q = lq[st >> 16][(st & 255) + 1];
    fqn = lq[min((st >> 16) + 1, L)][0];
    mh = wave_umax(c_hi);
  }
  const int n_depth = st >> 16;
  const bool member = lane >= 1 && lane <= n_pop;
  ps.depth = n_depth;
  ps.token = member ? tk[n_depth - 1][(st >> 8) & 255] : -1;
  ps.par = n_par;
  ps.score = n_score;
  return n_pop;
}

// Phase 3b, one wavefront: the breadth-first layout of the first n_use selected
// nodes (any prefix of the selection order is prefix-closed) into rows
// [s][0, R): rows by (depth, parent row, token id), level by level; a node's row
// and ancestor mask come from its parent's lane.  Rows past n_use + 1 are padding.
__device__ __forceinline__ void layout_tree(const PopState& ps, int n_use, int s, int root, int L,
                                          int R, int32_t* __restrict__ parent,
                                          int32_t* __restrict__ depth_out,
                                          int32_t* __restrict__ token_out,
                                          uint64_t* __restrict__ anc_out,
                                          float* __restrict__ score_out,
                                          int32_t* __restrict__ n_valid_out) {
  const int lane = lane_id();
  const int n_depth = ps.depth;
  const bool member = lane >= 1 && lane <= n_use;
  const int n_token = member ? ps.token : -1;
  const int par_addr = (ps.par < 0 ? 0 : ps.par) * 4;
  int row = 0, prow = -1;
  unsigned long long anc = 1ull;
  int base = 1;
  for (int d = 1; d <= L; ++d) {
    const bool in_level = member && n_depth == d;
    const unsigned long long lvl = __ballot(in_level);
    if (lvl == 0ull) break;
    const int pr = __builtin_amdgcn_ds_bpermute(par_addr, row);
    const uint32_t alo = __builtin_amdgcn_ds_bpermute(par_addr, static_cast<int>(anc));
    const uint32_t ahi = __builtin_amdgcn_ds_bpermute(par_addr, static_cast<int>(anc >> 32));
    const int key = (pr << 18) | (n_token & 0x3FFFF);  // token ids < 2^18
    int rank = 0;
    unsigned long long mm = lvl;
    while (mm) {
      const int jl = __ffsll(static_cast<long long>(mm)) - 1;
      mm &= mm - 1;
      rank += readlane_i(key, jl) < key ? 1 : 0;
    }
    if (in_level) {
      row = base + rank;
      prow = pr;
      anc = ((static_cast<unsigned long long>(ahi) << 32) | alo) | (1ull << row);
    }
    base += __popcll(lvl);
  }
  const size_t ob = static_cast<size_t>(s) * R;
  if (lane == 0) {
    parent[ob] = -1;
    depth_out[ob] = 0;
    token_out[ob] = root;
    anc_out[ob] = 1ull;
    score_out[ob] = 0.f;
    n_valid_out[s] = n_use + 1;
  }
  if (member) {
    parent[ob + row] = prow;
    depth_out[ob + row] = n_depth;
    token_out[ob + row] = n_token;
    anc_out[ob + row] = anc;
    score_out[ob + row] = ps.score;
  }
  for (int r = n_use + 1 + lane; r < R; r += kWave) {
    parent[ob + r] = -1;
    depth_out[ob + r] = 0;
    token_out[ob + r] = -1;
    anc_out[ob + r] = 0ull;
    score_out[ob + r] = -INFINITY;
  }
}

// Arrival of this work-group at a counter shared by `total` work-groups: true
// for the last one, which returns the counter to zero.  Every store the
// work-group made before is complete (waited for) when it is counted.
__device__ __forceinline__ bool arrive_last(unsigned* ctr, int total) {
  __shared__ int s_last;
  __builtin_amdgcn_s_waitcnt(0);
  __syncthreads();
  if (threadIdx.x == 0) {
    const unsigned old = __hip_atomic_fetch_add(ctr, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    const bool last = old == static_cast<unsigned>(total - 1);
    if (last) __hip_atomic_store(ctr, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    s_last = last;
  }
  __syncthreads();
  return s_last != 0;
}

// The whole tree phase in one launch, grid (chunk, offset, sequence): every
// work-group ranks its chunk (phase 1); the last chunk of each offset row to
// finish merges the row (phase 2); the last row of each sequence to be merged
// builds the tree (phase 3).  Work-groups meet only through device-scope
// atomics: published values are stored and loaded with device-coherent
// accesses and are complete before the arrival that announces them.
// Shared budget over the batch (null log_weight: every sequence takes N nodes).
struct SharedArgs {
  const float* log_weight;  // [nseq] ln V(H_s), the value of sequence s's node masses
  int budget;               // nodes over the batch
  float tau;                // keys below it are not taken
  int nseq;
  int4* pops;               // [nseq][64] published selections (depth, token, parent, score)
  unsigned* batch_cnt;      // arrivals of the sequences (zero between calls)
};

// The batch's cut and the trees, by the work-group of the last sequence to finish
// its selection (all threads).  Sequence s's i-th selected node has the key
// log_weight[s] + its score; keys are non-increasing in selection order, so a
// candidate's rank among the admissible keys (>= tau, > -inf) of the batch,
// ordered by (key desc, sequence, selection order), is its own index plus, for
// every other sequence, a binary search in that sequence's keys.  The nodes of
// rank < budget are taken: a prefix of each sequence's selection order.
__device__ void shared_cut_and_layout(const SharedArgs& sh, int L, int N,
                                      const int32_t* __restrict__ root_token,
                                      int32_t* __restrict__ parent, int32_t* __restrict__ depth_out,
                                      int32_t* __restrict__ token_out, uint64_t* __restrict__ anc_out,
                                      float* __restrict__ score_out, int32_t* __restrict__ n_valid_out) {
  __shared__ float keys[kMaxShared][kWave];
  __shared__ int adm[kMaxShared], nsel[kMaxShared];
  const int tid = threadIdx.x, nseq = sh.nseq;
  for (int idx = tid; idx < nseq * kWave; idx += kChunkThreads) {
    const int s = idx / kWave, l = idx - s * kWave;
    const uint64_t* src = reinterpret_cast<const uint64_t*>(sh.pops + idx);
    const uint64_t lo = __hip_atomic_load(src, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    const uint64_t hi = __hip_atomic_load(src + 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    if (l == 0) {
      adm[s] = static_cast<int>(static_cast<uint32_t>(lo));  // lane 0 carries the count
    } else {
      keys[s][l - 1] = sh.log_weight[s] + __uint_as_float(static_cast<uint32_t>(hi >> 32));
    }
  }
  __syncthreads();
  if (tid < nseq) {
    int a = 0;
    const int n = adm[tid];
    while (a < n && keys[tid][a] >= sh.tau && keys[tid][a] > -INFINITY) ++a;
    adm[tid] = a;
    nsel[tid] = 0;
  }
  __syncthreads();
  for (int idx = tid; idx < nseq * kWave; idx += kChunkThreads) {
    const int s = idx / kWave, i = idx - s * kWave;
    if (i >= adm[s]) continue;
    const float key = keys[s][i];
    int rank = i;
    for (int s2 = 0; s2 < nseq; ++s2) {
      if (s2 == s) continue;
      int lo = 0, hi = adm[s2];
      while (lo < hi) {  // entries of s2 ordered before (s, i): a prefix of its keys
        const int mid = (lo + hi) >> 1;
        const bool before = s2 < s ? keys[s2][mid] >= key : keys[s2][mid] > key;
        if (before) lo = mid + 1; else hi = mid;
      }
      rank += lo;
    }
    if (rank < sh.budget) atomicMax(&nsel[s], i + 1);
  }
  __syncthreads();
  const int w = tid / kWave, lane = tid - w * kWave;
  for (int s = w; s < nseq; s += kChunkThreads / kWave) {
    const uint64_t* src = reinterpret_cast<const uint64_t*>(sh.pops + s * kWave + lane);
    const uint64_t lo = __hip_atomic_load(src, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    const uint64_t hi = __hip_atomic_load(src + 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    PopState ps;
    ps.depth = lane == 0 ? 0 : static_cast<int>(static_cast<uint32_t>(lo));
    ps.token = static_cast<int>(static_cast<uint32_t>(lo >> 32));
    ps.par = static_cast<int>(static_cast<uint32_t>(hi));
    ps.score = __uint_as_float(static_cast<uint32_t>(hi >> 32));
    layout_tree(ps, nsel[s], s, root_token[s], L, N + 1, parent, depth_out, token_out, anc_out,
                score_out, n_valid_out);
  }
}

template <typename T, int NV>
__global__ __launch_bounds__(kChunkThreads) void tree_kernel(
    const T* __restrict__ logits, int L, int V, int N, int nch, unsigned long long* __restrict__ cstat,
    unsigned long long* __restrict__ clist, float* __restrict__ lq_g, int* __restrict__ tk_g,
    unsigned* __restrict__ row_cnt, unsigned* __restrict__ seq_cnt, const int32_t* __restrict__ root_token,
    int32_t* __restrict__ parent, int32_t* __restrict__ depth_out, int32_t* __restrict__ token_out,
    uint64_t* __restrict__ anc_out, float* __restrict__ score_out, int32_t* __restrict__ n_valid_out,
    SharedArgs sh, unsigned* __restrict__ flag) {
  __shared__ __attribute__((aligned(16))) unsigned long long buf[kCap];
  const int j = blockIdx.y, sq = blockIdx.z;
  const int row = sq * L + j;
  chunk_topk<T, NV>(logits, L, V, N, nch, cstat, clist, buf, flag);
  if (!arrive_last(row_cnt + row, nch)) return;
  const int K = k_of(N, V, j);
  if (K > 0) {
    __syncthreads();  // buf is reused
    merge_row(cstat, clist, nch, row, K, lq_g, tk_g, buf);
  } else if (threadIdx.x < kSlots) {
    __hip_atomic_store(lq_g + static_cast<size_t>(row) * kSlots + threadIdx.x, -INFINITY, __ATOMIC_RELAXED,
                       __HIP_MEMORY_SCOPE_AGENT);
    __hip_atomic_store(tk_g + static_cast<size_t>(row) * kSlots + threadIdx.x, -1, __ATOMIC_RELAXED,
                       __HIP_MEMORY_SCOPE_AGENT);
  }
  if (!arrive_last(seq_cnt + sq, L)) return;
  // ranked lists of every offset, -inf past each list (reads reach entry 65);
  // row L is all -inf (depth-L nodes have no children)
  __shared__ float lq[GLANCE_MAX_L + 1][kLqRow];
  __shared__ int tk[GLANCE_MAX_L][kSlots];
  for (int idx = threadIdx.x; idx < (L + 1) * kLqRow; idx += kChunkThreads) {
    const int jj = idx / kLqRow, r = idx - jj * kLqRow;
    float v = -INFINITY;
    if (jj < L && r < kSlots) {
      const size_t o = (static_cast<size_t>(sq) * L + jj) * kSlots + r;
      v = __hip_atomic_load(lq_g + o, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      tk[jj][r] = __hip_atomic_load(tk_g + o, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    }
    lq[jj][r] = v;
  }
  __syncthreads();
  if (sh.log_weight) {
    // shared budget: publish this sequence's selection (up to N nodes); the last
    // sequence to arrive cuts the batch and lays out every tree
    if (threadIdx.x < kWave) {
      PopState ps;
      const int n_pop = select_pops(lq, tk, L, N, ps);
      const int lane = threadIdx.x;
      const uint32_t d = lane == 0 ? static_cast<uint32_t>(n_pop) : static_cast<uint32_t>(ps.depth);
      uint64_t* dst = reinterpret_cast<uint64_t*>(sh.pops + sq * kWave + lane);
      __hip_atomic_store(dst, (static_cast<uint64_t>(static_cast<uint32_t>(ps.token)) << 32) | d,
                         __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      __hip_atomic_store(dst + 1,
                         (static_cast<uint64_t>(__float_as_uint(ps.score)) << 32) |
                             static_cast<uint32_t>(ps.par),
                         __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    }
    if (!arrive_last(sh.batch_cnt, sh.nseq)) return;
    shared_cut_and_layout(sh, L, N, root_token, parent, depth_out, token_out, anc_out, score_out,
                          n_valid_out);
    return;
  }
  if (threadIdx.x >= kWave) return;  // the rest is one wavefront
  PopState ps;
  const int n_pop = select_pops(lq, tk, L, N, ps);
  layout_tree(ps, n_pop, sq, root_token[sq], L, N + 1, parent, depth_out, token_out, anc_out, score_out,
              n_valid_out);
}

}  // namespace

// ln V(H) of each sequence's root entropy under the entropy law: the match
// probability p = sigma(b0 - b1 H) (paper §6, Eq. 2), the expected accepted
// length truncated at the horizon, sum_{l<=L} p^l = p (1 - p^L) / (1 - p) (App.
// B), and the value V = E[a|H] (1 - p) = p (1 - p^L) (App. B.5, Eq. 5), taken
// in the log domain as ln p + ln(1 - p^L) with ln p = -softplus(-x) and
// 1 - p^L = -expm1(L ln p), both without cancellation.  NaN entropy: -inf.
__global__ __launch_bounds__(256) void entropy_log_value_kernel(const float* __restrict__ H, int nseq,
                                                                int stride, float b0, float b1, int L,
                                                                float* __restrict__ out) {
  const int s = blockIdx.x * 256 + threadIdx.x;
  if (s >= nseq) return;
  const float h = H[static_cast<size_t>(s) * stride];
  if (h != h) {
    out[s] = -INFINITY;
    return;
  }
  const float x = b0 - b1 * h;
  const float lnp = -(fmaxf(-x, 0.f) + log1pf(expf(-fabsf(x))));
  out[s] = lnp + logf(-expm1f(static_cast<float>(L) * lnp));
}

// Host side -------------------------------------------------------------------
namespace {
struct TreeBufs {
  unsigned long long* cstat;
  unsigned long long* clist;
  float* lq;
  int* tk;
  unsigned* row_cnt;
  unsigned* seq_cnt;
  unsigned* flag;
};

template <typename T>
void launch_tree(int nv, dim3 ga, const T* logits, int L, int V, int N, int nch, const TreeBufs& b,
                 const int32_t* root, int32_t* parent, int32_t* depth, int32_t* token, uint64_t* anc,
                 float* score, int32_t* n_valid, const SharedArgs& sh, hipStream_t st) {
  switch (nv) {
#define GLANCE_TREE_CASE(n)                                                                         \
  case n:                                                                                          \
    tree_kernel<T, n><<<ga, kChunkThreads, 0, st>>>(logits, L, V, N, nch, b.cstat, b.clist, b.lq, b.tk, \
                                                   b.row_cnt, b.seq_cnt, root, parent, depth, token, \
                                                   anc, score, n_valid, sh, b.flag);                \
    break;
    GLANCE_TREE_CASE(1)
    GLANCE_TREE_CASE(2)
    GLANCE_TREE_CASE(3)
    GLANCE_TREE_CASE(4)
    GLANCE_TREE_CASE(5)
    GLANCE_TREE_CASE(6)
    GLANCE_TREE_CASE(7)
    GLANCE_TREE_CASE(8)
#undef GLANCE_TREE_CASE
    default: break;
  }
}
}  // namespace

TreeWs tree_ws_layout(int nseq, int L, int V) {
  (void)V;
  TreeWs w;
  const size_t r = static_cast<size_t>(nseq) * L;
  auto up = [](size_t b) { return (b + 255) & ~static_cast<size_t>(255); };
  size_t off = 0;
  auto take = [&](size_t bytes) {
    const size_t o = off;
    off += up(bytes);
    return o;
  };
  w.off_cstat = take(r * kMaxChunks * sizeof(unsigned long long));
  w.off_clist = take(r * kMaxChunks * kSlots * sizeof(unsigned long long));
  w.off_lq = take(r * kSlots * sizeof(float));
  w.off_tk = take(r * kSlots * sizeof(int));
  w.off_row_cnt = take(r * sizeof(unsigned));
  w.off_seq_cnt = take(static_cast<size_t>(nseq) * sizeof(unsigned));
  w.off_pops = take(static_cast<size_t>(nseq) * kWave * sizeof(int4));
  w.off_batch_cnt = take(sizeof(unsigned));
  w.off_flag = take(sizeof(unsigned));
  w.bytes = off;
  return w;
}

glance_status launch_build_tree(const void* logits, int dtype, const int32_t* root, int nseq,
                                int L, int V, int N, int32_t* parent, int32_t* depth,
                                int32_t* token, uint64_t* anc, float* score,
                                int32_t* n_valid, void* ws, hipStream_t st,
                                const float* log_weight, int budget, float tau) {
  const TreeWs w = tree_ws_layout(nseq, L, V);
  SharedArgs sh{};
  sh.log_weight = log_weight;
  sh.budget = budget;
  sh.tau = tau;
  sh.nseq = nseq;
  sh.pops = reinterpret_cast<int4*>(static_cast<char*>(ws) + w.off_pops);
  sh.batch_cnt = reinterpret_cast<unsigned*>(static_cast<char*>(ws) + w.off_batch_cnt);
  char* base = static_cast<char*>(ws);
  TreeBufs b;
  b.cstat = reinterpret_cast<unsigned long long*>(base + w.off_cstat);
  b.clist = reinterpret_cast<unsigned long long*>(base + w.off_clist);
  b.lq = reinterpret_cast<float*>(base + w.off_lq);
  b.tk = reinterpret_cast<int*>(base + w.off_tk);
  b.row_cnt = reinterpret_cast<unsigned*>(base + w.off_row_cnt);
  b.seq_cnt = reinterpret_cast<unsigned*>(base + w.off_seq_cnt);
  b.flag = reinterpret_cast<unsigned*>(base + w.off_flag);
  // at most kMaxChunks chunks of 256 threads x nv vectors per offset row
  const int E = dtype == GLANCE_BF16 ? 8 : 4;
  const int per_vec = kChunkThreads * E;
  int nv = (V + per_vec * kMaxChunks - 1) / (per_vec * kMaxChunks);
  if (nv < 1) nv = 1;
  if (nv > kMaxVec) return GLANCE_ERR_UNSUPPORTED;
  const int nch = (V + per_vec * nv - 1) / (per_vec * nv);
  const dim3 ga(nch, L, nseq);
  if (dtype == GLANCE_BF16)
    launch_tree<uint16_t>(nv, ga, static_cast<const uint16_t*>(logits), L, V, N, nch, b, root, parent,
                          depth, token, anc, score, n_valid, sh, st);
  else
    launch_tree<float>(nv, ga, static_cast<const float*>(logits), L, V, N, nch, b, root, parent, depth,
                       token, anc, score, n_valid, sh, st);
  GLANCE_LAUNCH_CHECK();
  return GLANCE_OK;
}

glance_status launch_entropy_log_value(const float* H, int nseq, int stride, float b0, float b1,
                                       int L, float* out, hipStream_t st) {
  entropy_log_value_kernel<<<(nseq + 255) / 256, 256, 0, st>>>(H, nseq, stride, b0, b1, L, out);
  GLANCE_LAUNCH_CHECK();
  return GLANCE_OK;
}

}  // namespace glance
