// Packed, ancestor-masked GQA attention of the verify rows (step 3).
//
// Paper §3.2 Def. 1 and App. B.1 (proof of Theorem 1): packing the tree into
// one pass with ancestor-only masking changes the attention layout, not a row's
// conditioning, so the row of node i attends to the cached prefix of its round
// plus exactly the tree rows j that are i itself or its ancestors (bit j of
// anc[i]), which is the causal sequence x o b o y_{1:d(i)}.
//
// bf16 path (head_dim 128, gfx950 MFMA v_mfma_f32_32x32x16_bf16).  A wave owns
// one KV head h of one round and a block of 32 of its queries (query q = row * G
// + j, the G = Hq/Hkv query heads of h times the round's rows).  The round's
// keys are its prefix [0, P) followed by its tree rows: key P + i is tree row i,
// visible to a query iff bit i of the query row's ancestor word is set.  Keys
// are streamed in blocks of 32 with an online softmax:
//   S^T = K Q^T     K from an LDS tile (lane (j, g) holds key j, dims 64 g ..
//                   64 g + 63 over the eight 16-deep steps); q enters as its
//                   bf16 rounding plus the bf16 remainder (two products), so
//                   the scores see q to ~16 bits.
//   P = 2^(S - m)   in fp32, then split the same way into a bf16 part and the
//                   bf16 remainder of what it left out.
//   O^T += V^T P^T  V through an LDS tile stored transposed; P^T stays in
//                   registers: each lane already holds, for its query, the keys
//                   that the MFMA B operand wants from it, provided the V^T tile
//                   stores the keys in that order (the slot permutation below).
// Kernel (tree_attn_tile_kernel): the four (or two) waves of a work-group own
// consecutive query blocks of one head and one key split, and share each
// 32-key K / V^T tile, loaded once per work-group, two blocks ahead, into a
// double-buffered LDS pair.  The number of splits fills the CUs once but keeps
// every split at least GLANCE_ATTN_MINBLK blocks long, since each split costs
// a 528-byte record (max, sum, O) per query; the split records are merged in
// split order, by the last work-group of a query group to finish when the
// records are few, else by attn_combine4_kernel (attn_combine_kernel when Hq
// is not a multiple of 4).  Work-group ids put the query groups and splits of
// one KV head on the same XCD (id mod 8 = h when Hkv = 8), so the head's K/V
// cross HBM once and are shared through that XCD's L2.  The output o = O / sum
// is written in fp32; the output projection takes it as a bf16 pair too, so
// q, P and o all enter the products with ~16 significant bits.
//
// fp32 path (tiny shapes): one work-group per (row, query head), scores in LDS,
// plain fp32 loops.
#include <type_traits>

#include "common.h"
#include "kernels.h"

namespace glance {

namespace {

constexpr int kQW = 32;               // queries per work-group
constexpr int kKB = 32;               // keys per block
constexpr int kHD = 128;              // head_dim of the bf16 path
constexpr int kVtRow = 40;            // bf16 slots per V^T row: 32 keys + 8 padding (80 bytes)
constexpr int kRec = kHD + 4;         // split record per query: m, l, -, -, o[128]
constexpr int kMaxSplit = 16;

// position P + depth of a row, clamped into the cos/sin tables
__device__ __forceinline__ int row_pos(const AttnArgs& a, int P, int row) {
  const int p = P + a.depth[row];
  return p < 0 ? 0 : (p < a.n_pos - 1 ? p : a.n_pos - 1);
}

// Prefix length of round s, read as at most max_prefix keys.
__device__ __forceinline__ int prefix_len(const AttnArgs& a, int s) {
  int64_t P = a.kv_offsets[s + 1] - a.kv_offsets[s];
  if (P > a.max_prefix) P = a.max_prefix;
  return P < 0 ? 0 : static_cast<int>(P);
}

__device__ __forceinline__ float rope_pair(const float* x, int i, int half, float c, float s) {
  // rotate-half: (x_i, x_{i+half}) -> (x_i c - x_{i+half} s, x_{i+half} c + x_i s)
  return i < half ? x[i] * c - x[i + half] * s : x[i] * c + x[i - half] * s;
}

// Visibility of keys t0 .. t0 + 31 to a query whose row has ancestor word anc:
// bit k set iff key t0 + k is before t_end and is a prefix key (< P) or tree
// row t0 + k - P with its bit set in anc.  Branch-free.
__device__ __forceinline__ uint32_t block_mask(int t0, int t_end, int P, uint64_t anc) {
  const int nv = min(max(t_end - t0, 0), 32);  // keys of the block in the range
  const int np = min(max(P - t0, 0), nv);      // prefix keys among them
  const uint32_t valid = nv == 32 ? 0xFFFFFFFFu : ((1u << nv) - 1u);
  const uint32_t pref = np == 32 ? 0xFFFFFFFFu : ((1u << np) - 1u);
  const int sh = t0 - P;  // tree index of key t0 (< 64 while t0 < T; keys past T are not valid)
  const uint32_t right = static_cast<uint32_t>(anc >> (sh & 63));
  const uint32_t left = static_cast<uint32_t>(anc << ((-sh) & 63));
  const uint32_t tree = sh >= 0 ? right : (sh > -32 ? left : 0u);
  return pref | (tree & valid & ~pref);
}

// The other half of a wave (lane l ^ 32) without an LDS round trip: with both
// operands the same register, v_permlane32_swap leaves a lane's own value in one
// result and its partner's in the other, so their max (or sum) is the pair's.
__device__ __forceinline__ float max_halves(float v) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
__device__ __forceinline__ float sum_halves(float v) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}

// Slot quad of key quad kq (keys 4 kq .. 4 kq + 3 of a 32-key block) in the V^T
// tile.  The S^T accumulator gives lane (j, g) the keys 8 i + 4 g + u (i, u < 4)
// of query j; the MFMA B operand of 16-key step t takes from it the keys of
// quads 4 t + g and 4 t + 2 + g, in that order.  So quad 4 t + 2 a + g goes to
// slot quad 4 t + 2 g + a: the A operand (V^T, lane (dim, g)) of step t is then
// slot quads 4 t + 2 g and 4 t + 2 g + 1.  Slot quads are further XOR-swizzled
// by (dim / 8) mod 8 against LDS bank conflicts.
__device__ __forceinline__ int slot_quad(int kq) {
  return (kq & 4) | ((kq & 1) << 1) | ((kq >> 1) & 1);
}

// One of the two bf16 halves of a pair of 32-bit words: the low (sel = 0x05040100)
// or high (0x07060302) 16 bits of a, then of b, packed into one word.
__device__ __forceinline__ uint32_t pick16(uint32_t a, uint32_t b, uint32_t sel) {
  return __builtin_amdgcn_perm(b, a, sel);
}

// The W waves of a work-group own W consecutive blocks of 32 queries of one KV
// head and all keys of one key split.  Every 32-key block is loaded once per
// work-group, cooperatively (threads below 128 take the V pieces, the rest, or
// the same threads when W = 2, the K pieces), two blocks ahead of its use, into
// a double-buffered pair of LDS tiles (K rows with the XOR swizzle, V^T in the
// slot order of the P operand), and read by every wave.  One barrier per block.
// Each wave then does the per-block work for its own queries (S^T = K Q^T with
// q as a bf16 pair, the lazy online softmax, P as a bf16 pair, O^T += V^T P^T)
// and, at the end, writes its queries' split records (or, with one split, their
// outputs).
template <int W>
__global__ __launch_bounds__(W * kWave, 1) void tree_attn_tile_kernel(AttnArgs a, int nqb, int fuse) {
  constexpr int KT = kKB * kHD;        // K tile (elements)
  constexpr int VT = kHD * kVtRow;     // V^T tile (elements)
  __shared__ __attribute__((aligned(16))) uint16_t tiles[2][KT + VT];

  const int Hkv = a.Hkv;
  int id = blockIdx.x;
  const int h = id % Hkv;
  id /= Hkv;
  const int nqg = (nqb + W - 1) / W;
  const int qg = id % nqg;
  id /= nqg;
  const int c = id % a.n_split;
  const int s = id / a.n_split;
  const int tid = threadIdx.x, l = tid & 63, j = l & 31, g = l >> 5;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int G = a.Hq / Hkv;
  const int Qn = a.n_rows * G;
  const int qb = qg * W + w;  // this wave's query block (past nqb: no queries, still loads)

  // ---- this lane's query as bf16 + remainder (queries past Qn read row 0 and
  // are never stored)
  const int q = qb * kQW + j;
  const bool qvalid = qb < nqb && q < Qn;
  const int grow = s * a.n_rows + (qvalid ? q / G : 0);
  const uint64_t qanc = qvalid ? a.anc[grow] : 0ull;
  bf16x8 qhi[8], qlo[8];  // loaded below, behind the first K/V blocks
  const size_t qoff = (static_cast<size_t>(grow) * a.Hq + h * G + (qvalid ? q % G : 0)) * kHD + 64 * g;
  const int64_t kv0 = a.kv_offsets[s];
  const int P = prefix_len(a, s);
  const int T = P + a.n_rows;
  // this work-group's keys: split c of n_split, in whole blocks
  const int per = ((T + a.n_split - 1) / a.n_split + kKB - 1) / kKB * kKB;
  const int t_beg = c * per;
  const int t_end = min(t_beg + per, T);
  const int nblk = t_end > t_beg ? (t_end - t_beg + kKB - 1) / kKB : 0;

  const int kstr = Hkv * kHD;
  const uint16_t* kc0 = static_cast<const uint16_t*>(a.k_cache) + (kv0 * Hkv + h) * kHD;
  const uint16_t* vc0 = static_cast<const uint16_t*>(a.v_cache) + (kv0 * Hkv + h) * kHD;
  const size_t trow0 = (static_cast<size_t>(s) * a.n_rows * Hkv + h) * kHD;
  const uint16_t* tk0 = static_cast<const uint16_t*>(a.tree_k) + trow0;
  const uint16_t* tv0 = static_cast<const uint16_t*>(a.tree_v) + trow0;
  auto row_of = [&](const uint16_t* c0, const uint16_t* t0p, int t) {
    const bool pre = t < P;
    const int i = (t < T && !pre) ? t - P : 0;
    return (pre ? c0 : t0p) + (pre ? t : i) * kstr;
  };
  // loading roles, per 32-key block: 512 K pieces (key pi / 16, 16-byte unit
  // pi % 16; thread lt takes pi = lt + 128 i) and 128 V pieces (dims 8 vx .. + 7
  // of the four keys of quad kq).  With four waves, waves 0-1 load V and waves
  // 2-3 load K (one register set each); with two, every thread loads both.
  const bool vrole = W == 4 ? w < 2 : true;
  const bool krole = W == 4 ? w >= 2 : true;
  constexpr int NP = W == 4 ? 4 : 8;   // 16-byte pieces per thread and block
  constexpr int VO = W == 4 ? 0 : 4;   // index of the first V piece
  const int lt = tid & 127;
  const int vx = lt & 15, kq = lt >> 4;
  // Byte offsets of this thread's pieces from the start of a block, the same
  // for every block (K piece i: key lt / 16 + 8 i, unit lt % 16; V piece i: key
  // 4 kq + i, dims 8 vx ..); with four waves a thread's offsets are its role's.
  uint32_t koff[4], voff[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    koff[i] = 2u * static_cast<uint32_t>(((lt >> 4) + 8 * i) * kstr + 8 * (lt & 15));
    voff[i] = 2u * static_cast<uint32_t>((4 * kq + i) * kstr + 8 * vx);
    if (W == 4 && !krole) koff[i] = voff[i];
  }
  // A block of prefix keys is one base address plus those offsets; a block that
  // reaches the tree rows or the end picks each key's row.  Either way every
  // load is issued (the role picks the address): a load under a branch that the
  // other side lacks would make the compiler wait for every load in flight.
  auto load = [&](int t0, u32x4 (&d)[NP]) {
    if (t0 + kKB <= P) {  // (uniform)
      const char* kb = reinterpret_cast<const char*>(kc0 + static_cast<int64_t>(t0) * kstr);
      const char* vb = reinterpret_cast<const char*>(vc0 + static_cast<int64_t>(t0) * kstr);
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        if (W == 4) {
          d[i] = *reinterpret_cast<const u32x4*>((krole ? kb : vb) + koff[i]);
        } else {
          d[i] = *reinterpret_cast<const u32x4*>(kb + koff[i]);
          d[VO + i] = *reinterpret_cast<const u32x4*>(vb + voff[i]);
        }
      }
    } else {
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const uint16_t* kp = row_of(kc0, tk0, t0 + (lt >> 4) + 8 * i) + 8 * (lt & 15);
        const uint16_t* vp = row_of(vc0, tv0, t0 + 4 * kq + i) + 8 * vx;
        if (W == 4) {
          d[i] = *reinterpret_cast<const u32x4*>(krole ? kp : vp);
        } else {
          d[i] = *reinterpret_cast<const u32x4*>(kp);
          d[VO + i] = *reinterpret_cast<const u32x4*>(vp);
        }
      }
    }
  };
  // K tile: key k's row at k * 128, its 16-byte unit p at unit p ^ (k mod 8);
  // V^T tile: dim 8 vx + e, the slot quad of key quad kq, four keys per write
  auto store = [&](int buf, const u32x4 (&d)[NP]) {
    uint16_t* kt = tiles[buf];
    uint16_t* vt = tiles[buf] + KT;
    if (krole) {
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int k = (lt >> 4) + 8 * i;
        *reinterpret_cast<u32x4*>(kt + k * kHD + 8 * ((lt & 15) ^ (k & 7))) = d[i];
      }
    }
    if (vrole) {
      const int sq = slot_quad(kq) ^ (vx & 7);
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        const uint32_t sel = (e & 1) ? 0x07060302u : 0x05040100u;
        const uint32_t x0 = d[VO][e >> 1], x1 = d[VO + 1][e >> 1];
        const uint32_t x2 = d[VO + 2][e >> 1], x3 = d[VO + 3][e >> 1];
        *reinterpret_cast<uint2*>(vt + (8 * vx + e) * kVtRow + 4 * sq) =
            make_uint2(pick16(x0, x1, sel), pick16(x2, x3, sel));
      }
    }
  };

  const float scale_log2 = 1.4426950408889634f / sqrtf(static_cast<float>(kHD));
  f32x16 acc_o[4] = {};
  float m_ref = -INFINITY, l_run = 0.f;
  // blocks 0 and 1 in flight; block 0 into tile 0.  Loads past the last block
  // re-read it (no conditional load).
  const int tlast = t_beg + (nblk > 0 ? nblk - 1 : 0) * kKB;
  u32x4 pf[2][NP];
  load(t_beg, pf[0]);
  load(min(t_beg + kKB, tlast), pf[1]);
  // the query (bf16 pair, the B operand of S^T: dims 64 g + 8 ks .. + 7) in
  // flight behind the first two blocks
  {
    const uint16_t* qp = static_cast<const uint16_t*>(a.q) + qoff;
    const uint16_t* qlp = static_cast<const uint16_t*>(a.q_lo) + qoff;
#pragma unroll
    for (int ks = 0; ks < 8; ++ks) {
      qhi[ks] = __builtin_bit_cast(bf16x8, *reinterpret_cast<const uint4*>(qp + 8 * ks));
      qlo[ks] = __builtin_bit_cast(bf16x8, *reinterpret_cast<const uint4*>(qlp + 8 * ks));
    }
  }
  store(0, pf[0]);
  load(min(t_beg + 2 * kKB, tlast), pf[0]);
  __syncthreads();
  // block b of the range; cur = b mod 2 is a compile-time constant so that the
  // register set of the block after next is named statically
  auto block = [&](int b, auto par, auto first) {
    constexpr int cur = decltype(par)::value;
    if constexpr (decltype(first)::value) {
      // in flight here: block 0, block 1, the 16 query loads, block 2 (NP loads
      // each, completing in order); the query is complete once at most NP remain
      __builtin_amdgcn_s_waitcnt(0x0F70 | NP);  // vmcnt(NP), expcnt and lgkmcnt not waited
    }
    const int t0 = t_beg + b * kKB;
    const uint16_t* kt = tiles[cur];
    const uint16_t* vt = tiles[cur] + KT;
    // ---- S^T = K Q^T with q = hi + lo (all eight operand reads first)
    bf16x8 kop[8];
#pragma unroll
    for (int ks = 0; ks < 8; ++ks)
      kop[ks] = *reinterpret_cast<const bf16x8*>(kt + j * kHD + 8 * ((8 * g + ks) ^ (j & 7)));
    // one accumulator: each 16-deep step adds its q-part and remainder products
    f32x16 sa = {};
#pragma unroll
    for (int ks = 0; ks < 8; ++ks) {
      sa = __builtin_amdgcn_mfma_f32_32x32x16_bf16(kop[ks], qhi[ks], sa, 0, 0, 0);
      sa = __builtin_amdgcn_mfma_f32_32x32x16_bf16(kop[ks], qlo[ks], sa, 0, 0, 0);
    }
    if (b + 1 < nblk) store(cur ^ 1, pf[cur ^ 1]);
    load(min(t0 + 3 * kKB, tlast), pf[cur ^ 1]);
    // ---- mask (element v: key t0 + 8 (v / 4) + 4 g + v % 4, query j), block
    // maximum of the raw scores, scaled once (the scale is positive, so the
    // maximum commutes with it)
    float sc[16], mraw = -INFINITY;
    if (t0 + kKB <= min(P, t_end)) {  // (uniform) every key of the block is a visible prefix key
#pragma unroll
      for (int v = 0; v < 16; ++v) {
        sc[v] = sa[v];
        mraw = fmaxf(mraw, sc[v]);
      }
    } else {
      const uint32_t vm = block_mask(t0, t_end, P, qanc) >> (4 * g);
#pragma unroll
      for (int v = 0; v < 16; ++v) {
        const bool vis = (vm >> (8 * (v >> 2) + (v & 3))) & 1u;
        sc[v] = vis ? sa[v] : -INFINITY;
        mraw = fmaxf(mraw, sc[v]);
      }
    }
    mraw = max_halves(mraw);
    const float mb = mraw * scale_log2;
    const bool raise = mb > m_ref + 8.f;  // also when m_ref is still -inf
    if (__ballot(raise) != 0ull) {  // (uniform per wave) rare after the first block
      const float m_new = raise ? mb : m_ref;
      const float alpha = m_ref == -INFINITY ? 0.f : __builtin_amdgcn_exp2f(m_ref - m_new);
      m_ref = m_new;
      l_run *= alpha;
#pragma unroll
      for (int db = 0; db < 4; ++db)
#pragma unroll
        for (int v = 0; v < 16; ++v) acc_o[db][v] *= alpha;
    }
    const float mz = m_ref == -INFINITY ? 0.f : m_ref;
    uint32_t ph[8], pl[8];
#pragma unroll
    for (int pr = 0; pr < 8; ++pr) {
      const float p0 = __builtin_amdgcn_exp2f(fmaf(sc[2 * pr], scale_log2, -mz));
      const float p1 = __builtin_amdgcn_exp2f(fmaf(sc[2 * pr + 1], scale_log2, -mz));
      ph[pr] = pack_bf16x2(p0, p1);
      pl[pr] = pack_bf16x2(p0 - __uint_as_float(ph[pr] << 16), p1 - __uint_as_float(ph[pr] & 0xFFFF0000u));
      l_run += p0 + p1;
    }
    // ---- O^T += V^T P^T, two 16-key steps (operand reads first)
    bf16x8 vop[2][4];
#pragma unroll
    for (int t = 0; t < 2; ++t)
#pragma unroll
      for (int db = 0; db < 4; ++db) {
        const int dim = 32 * db + j;
        const int sw = (dim >> 3) & 7;
        const uint16_t* row = vt + dim * kVtRow;
        const uint2 lo = *reinterpret_cast<const uint2*>(row + 4 * ((4 * t + 2 * g) ^ sw));
        const uint2 hi = *reinterpret_cast<const uint2*>(row + 4 * ((4 * t + 2 * g + 1) ^ sw));
        vop[t][db] = __builtin_bit_cast(bf16x8, make_uint4(lo.x, lo.y, hi.x, hi.y));
      }
#pragma unroll
    for (int t = 0; t < 2; ++t) {
      const bf16x8 bh = __builtin_bit_cast(bf16x8, make_uint4(ph[4 * t], ph[4 * t + 1], ph[4 * t + 2], ph[4 * t + 3]));
      const bf16x8 bl = __builtin_bit_cast(bf16x8, make_uint4(pl[4 * t], pl[4 * t + 1], pl[4 * t + 2], pl[4 * t + 3]));
#pragma unroll
      for (int db = 0; db < 4; ++db) {
        acc_o[db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(vop[t][db], bh, acc_o[db], 0, 0, 0);
        acc_o[db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(vop[t][db], bl, acc_o[db], 0, 0, 0);
      }
    }
    // every wave's reads of this block end before the next iteration stores
    // into this buffer; the stores of the next block are visible after it
    __syncthreads();
  };
  // Block 0 alone (its products are the first use of q, so only it waits for
  // the query loads), then whole pairs, then the last block alone: every back
  // edge follows an even block, and no loop iteration waits for q or for the
  // loads just issued (an optional second block, or q still pending at the loop
  // entry, would make the compiler's waits drain the prefetch).
  using C0 = std::integral_constant<int, 0>;
  using C1 = std::integral_constant<int, 1>;
  using First = std::true_type;
  using Later = std::false_type;
  if (nblk > 0) {  // (the loop is reachable only through block 0)
    block(0, C0{}, First{});
    int b = 1;
    for (; b + 1 < nblk; b += 2) {
      block(b, C1{}, Later{});
      block(b + 1, C0{}, Later{});
    }
    if (b < nblk) block(b, C1{}, Later{});
  }
  const float l_tot = sum_halves(l_run);
  // lane (j, g) holds dims 32 db + 8 i + 4 g + u (u < 4 consecutive) of query j
  if (a.n_split > 1) {
    const size_t blk = (static_cast<size_t>(s) * Hkv + h) * nqb + qb;
    const size_t cs = static_cast<size_t>(kQW) * kRec;  // one split's records of a query block
    float* rec0 = a.part + (blk * a.n_split * kQW + j) * kRec;  // split 0 of this lane's query
    if (qvalid) {
      float* rec = rec0 + c * cs;
      if (g == 0) *reinterpret_cast<float2*>(rec) = make_float2(m_ref, l_tot);
#pragma unroll
      for (int db = 0; db < 4; ++db)
#pragma unroll
        for (int i = 0; i < 4; ++i)
          *reinterpret_cast<float4*>(rec + 4 + 32 * db + 8 * i + 4 * g) =
              make_float4(acc_o[db][4 * i], acc_o[db][4 * i + 1], acc_o[db][4 * i + 2], acc_o[db][4 * i + 3]);
    }
    if (!fuse) return;  // attn_combine_kernel merges
    // In-kernel merge: the records reach L2 (every wave waits for its stores),
    // the group's counter is raised with release ordering (the L2 write-back
    // makes the whole work-group's records visible device-wide), and the last
    // of the group's n_split work-groups to arrive acquires them and merges,
    // with attn_combine_kernel's arithmetic in the same order.
    __builtin_amdgcn_s_waitcnt(0);
    __shared__ int s_last;
    __syncthreads();
    if (tid == 0) {
      unsigned* cnt = a.arrivals + (static_cast<size_t>(s) * Hkv + h) * nqg + qg;
      const unsigned old = __hip_atomic_fetch_add(cnt, 1u, __ATOMIC_ACQ_REL, __HIP_MEMORY_SCOPE_AGENT);
      const bool last = old == static_cast<unsigned>(a.n_split - 1);
      if (last) __hip_atomic_store(cnt, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      s_last = last;
    }
    __syncthreads();
    if (!s_last || !qvalid) return;
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "agent");
    // lane (j, g): query qb * 32 + j, dims 64 g .. 64 g + 63
    float M = -INFINITY;
    for (int cc = 0; cc < a.n_split; ++cc) M = fmaxf(M, rec0[cc * cs]);
    float L = 0.f;
    float acc[64];
#pragma unroll
    for (int d = 0; d < 64; ++d) acc[d] = 0.f;
    for (int cc = 0; cc < a.n_split; ++cc) {
      const float* rc = rec0 + cc * cs;
      const float mc = rc[0];
      const float f = mc == -INFINITY ? 0.f : __builtin_amdgcn_exp2f(mc - M);
      L += rc[1] * f;
      float4 v[16];
#pragma unroll
      for (int d4 = 0; d4 < 16; ++d4) v[d4] = *reinterpret_cast<const float4*>(rc + 4 + 64 * g + 4 * d4);
#pragma unroll
      for (int d4 = 0; d4 < 16; ++d4) {
        acc[4 * d4] += v[d4].x * f;
        acc[4 * d4 + 1] += v[d4].y * f;
        acc[4 * d4 + 2] += v[d4].z * f;
        acc[4 * d4 + 3] += v[d4].w * f;
      }
    }
    const int rr = q / G;
    const int growq = s * a.n_rows + rr;
    const bool live = a.token[growq] >= 0;
    const size_t off = static_cast<size_t>(growq) * a.Hq * kHD + (h * G + q % G) * kHD + 64 * g;
#pragma unroll
    for (int d4 = 0; d4 < 16; ++d4) {
      float4 o;
      o.x = (live && L > 0.f) ? acc[4 * d4] / L : 0.f;
      o.y = (live && L > 0.f) ? acc[4 * d4 + 1] / L : 0.f;
      o.z = (live && L > 0.f) ? acc[4 * d4 + 2] / L : 0.f;
      o.w = (live && L > 0.f) ? acc[4 * d4 + 3] / L : 0.f;
      *reinterpret_cast<float4*>(a.attn_x + off + 4 * d4) = o;
      if (a.attn_out) *reinterpret_cast<float4*>(a.attn_out + off + 4 * d4) = o;
    }
    return;
  }
  if (!qvalid) return;
  const int rr = q / G;
  const int growq = s * a.n_rows + rr;
  const bool live = a.token[growq] >= 0;
  const float inv = (live && l_tot > 0.f) ? 1.f / l_tot : 0.f;
  const size_t off = static_cast<size_t>(growq) * a.Hq * kHD + (h * G + q % G) * kHD;
#pragma unroll
  for (int db = 0; db < 4; ++db)
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int d = 32 * db + 8 * i + 4 * g;
      const float4 v = make_float4(acc_o[db][4 * i] * inv, acc_o[db][4 * i + 1] * inv,
                                   acc_o[db][4 * i + 2] * inv, acc_o[db][4 * i + 3] * inv);
      *reinterpret_cast<float4*>(a.attn_x + off + d) = v;
      if (a.attn_out) *reinterpret_cast<float4*>(a.attn_out + off + d) = v;
    }
}

// Merge of the split records of every (row, query head): one work-group per row
// and query head, one thread per head dimension, splits in order.  NS >=
// n_split is the unrolled load count.
template <int NS>
__global__ __launch_bounds__(kHD) void attn_combine_kernel(AttnArgs a, int nqb) {
  const int grow = blockIdx.x, qh = blockIdx.y, dim = threadIdx.x;
  const int s = grow / a.n_rows, r = grow % a.n_rows;
  const int G = a.Hq / a.Hkv;
  const int h = qh / G, q = r * G + qh % G;
  const size_t blk = (static_cast<size_t>(s) * a.Hkv + h) * nqb + q / kQW;
  const float* rec = a.part + (blk * a.n_split * kQW + q % kQW) * kRec;
  const size_t cs = static_cast<size_t>(kQW) * kRec;
  // every load first (splits past n_split re-read the last record, weight 0)
  float mm[NS], ll[NS], vv[NS];
#pragma unroll
  for (int c = 0; c < NS; ++c) {
    const float* rc = rec + min(c, a.n_split - 1) * cs;
    mm[c] = rc[0];
    ll[c] = rc[1];
    vv[c] = rc[4 + dim];
  }
  const bool live = a.token[grow] >= 0;
  float M = -INFINITY;
#pragma unroll
  for (int c = 0; c < NS; ++c) M = fmaxf(M, c < a.n_split ? mm[c] : -INFINITY);
  float L = 0.f, acc = 0.f;
#pragma unroll
  for (int c = 0; c < NS; ++c) {
    const float f = (c >= a.n_split || mm[c] == -INFINITY) ? 0.f : __builtin_amdgcn_exp2f(mm[c] - M);
    L += ll[c] * f;
    acc += vv[c] * f;
  }
  const float o = (live && L > 0.f) ? acc / L : 0.f;
  const size_t off = static_cast<size_t>(grow) * a.Hq * kHD + qh * kHD + dim;
  a.attn_x[off] = o;
  if (a.attn_out) a.attn_out[off] = o;
}

// The same merge with 16-byte loads: a work-group of 128 threads takes four
// query heads of one row, a thread four consecutive dimensions (Hq % 4 == 0);
// per element the arithmetic and its order are those of attn_combine_kernel.
template <int NS>
__global__ __launch_bounds__(128) void attn_combine4_kernel(AttnArgs a, int nqb) {
  const int grow = blockIdx.x, tid = threadIdx.x;
  const int qh = blockIdx.y * 4 + (tid >> 5), d0 = (tid & 31) * 4;
  const int s = grow / a.n_rows, r = grow % a.n_rows;
  const int G = a.Hq / a.Hkv;
  const int h = qh / G, q = r * G + qh % G;
  const size_t blk = (static_cast<size_t>(s) * a.Hkv + h) * nqb + q / kQW;
  const float* rec = a.part + (blk * a.n_split * kQW + q % kQW) * kRec;
  const size_t cs = static_cast<size_t>(kQW) * kRec;
  float mm[NS], ll[NS];
  float4 vv[NS];
#pragma unroll
  for (int c = 0; c < NS; ++c) {
    const float* rc = rec + min(c, a.n_split - 1) * cs;
    const float2 ml = *reinterpret_cast<const float2*>(rc);
    mm[c] = ml.x;
    ll[c] = ml.y;
    vv[c] = *reinterpret_cast<const float4*>(rc + 4 + d0);
  }
  const bool live = a.token[grow] >= 0;
  float M = -INFINITY;
#pragma unroll
  for (int c = 0; c < NS; ++c) M = fmaxf(M, c < a.n_split ? mm[c] : -INFINITY);
  float L = 0.f;
  float4 acc = make_float4(0.f, 0.f, 0.f, 0.f);
#pragma unroll
  for (int c = 0; c < NS; ++c) {
    const float f = (c >= a.n_split || mm[c] == -INFINITY) ? 0.f : __builtin_amdgcn_exp2f(mm[c] - M);
    L += ll[c] * f;
    acc.x += vv[c].x * f;
    acc.y += vv[c].y * f;
    acc.z += vv[c].z * f;
    acc.w += vv[c].w * f;
  }
  const bool ok = live && L > 0.f;
  const float4 o = make_float4(ok ? acc.x / L : 0.f, ok ? acc.y / L : 0.f, ok ? acc.z / L : 0.f,
                               ok ? acc.w / L : 0.f);
  const size_t off = static_cast<size_t>(grow) * a.Hq * kHD + qh * kHD + d0;
  *reinterpret_cast<float4*>(a.attn_x + off) = o;
  if (a.attn_out) *reinterpret_cast<float4*>(a.attn_out + off) = o;
}

// ------------------------------------------------------------------ fp32 path
constexpr int kF32MaxKeys = 8192 + GLANCE_MAX_ROWS;

__global__ __launch_bounds__(128) void tree_attn_f32_kernel(AttnArgs a) {
  __shared__ float sc[kF32MaxKeys];
  __shared__ float qs[kHD];
  __shared__ float red[2];
  const int grow = blockIdx.x, qh = blockIdx.y;
  const int s = grow / a.n_rows;
  const int G = a.Hq / a.Hkv, h = qh / G, D = a.D, half = D / 2;
  const int nq_total = (a.Hq + 2 * a.Hkv) * D;
  const int tid = threadIdx.x;
  float* ox = a.attn_x + static_cast<size_t>(grow) * a.Hq * D + qh * D;
  if (a.token[grow] < 0) {
    for (int d = tid; d < D; d += 128) {
      ox[d] = 0.f;
      if (a.attn_out) a.attn_out[static_cast<size_t>(grow) * a.Hq * D + qh * D + d] = 0.f;
    }
    return;
  }
  const int64_t kv0 = a.kv_offsets[s];
  const int P = prefix_len(a, s);
  const uint64_t anc = a.anc[grow];
  {
    const int pos = row_pos(a, P, grow);
    const float* xq = a.qkv + static_cast<size_t>(grow) * nq_total + qh * D;
    for (int i = tid; i < D; i += 128) {
      const int ii = i % half;
      qs[i] = rope_pair(xq, i, half, a.rope_cos[static_cast<size_t>(pos) * half + ii],
                        a.rope_sin[static_cast<size_t>(pos) * half + ii]);
    }
  }
  __syncthreads();
  const int T = P + a.n_rows;
  const float scale = 1.f / sqrtf(static_cast<float>(D));
  float mx = -INFINITY;
  for (int t = tid; t < T; t += 128) {
    float dot = -INFINITY;
    if (t < P) {
      const float* k = static_cast<const float*>(a.k_cache) + (static_cast<size_t>(kv0 + t) * a.Hkv + h) * D;
      float acc = 0.f;
      for (int i = 0; i < D; ++i) acc = fmaf(qs[i], k[i], acc);
      dot = acc * scale;
    } else {
      const int tr = t - P;
      if ((anc >> tr) & 1ull) {
        const int trow = s * a.n_rows + tr;
        const int pos = row_pos(a, P, trow);
        const float* xk = a.qkv + static_cast<size_t>(trow) * nq_total + a.Hq * D + h * D;
        float acc = 0.f;
        for (int i = 0; i < D; ++i) {
          const int ii = i % half;
          const float kr = rope_pair(xk, i, half, a.rope_cos[static_cast<size_t>(pos) * half + ii],
                                     a.rope_sin[static_cast<size_t>(pos) * half + ii]);
          acc = fmaf(qs[i], kr, acc);
        }
        dot = acc * scale;
      }
    }
    sc[t] = dot;
    mx = fmaxf(mx, dot);
  }
  mx = wave_max(mx);
  if ((tid & 63) == 0) red[tid >> 6] = mx;
  __syncthreads();
  mx = fmaxf(red[0], red[1]);
  __syncthreads();
  float sum = 0.f;
  for (int t = tid; t < T; t += 128) {
    const float p = sc[t] == -INFINITY ? 0.f : expf(sc[t] - mx);
    sc[t] = p;
    sum += p;
  }
  sum = wave_sum(sum);
  if ((tid & 63) == 0) red[tid >> 6] = sum;
  __syncthreads();
  sum = red[0] + red[1];
  for (int d = tid; d < D; d += 128) {
    float acc = 0.f;
    for (int t = 0; t < T; ++t) {
      const float p = sc[t];
      if (p == 0.f) continue;
      float v;
      if (t < P)
        v = static_cast<const float*>(a.v_cache)[(static_cast<size_t>(kv0 + t) * a.Hkv + h) * D + d];
      else
        v = a.qkv[static_cast<size_t>(s * a.n_rows + (t - P)) * nq_total + (a.Hq + a.Hkv) * D + h * D + d];
      acc = fmaf(p, v, acc);
    }
    const float o = acc / sum;
    ox[d] = o;
    if (a.attn_out) a.attn_out[static_cast<size_t>(grow) * a.Hq * D + qh * D + d] = o;
  }
  // this row's own cache entries, written once per KV head
  if (qh % G == 0) {
    const int pos = row_pos(a, P, grow);
    const float* xk = a.qkv + static_cast<size_t>(grow) * nq_total + a.Hq * D + h * D;
    for (int i = tid; i < D; i += 128) {
      const size_t o = (static_cast<size_t>(grow) * a.Hkv + h) * D + i;
      const int ii = i % half;
      if (a.tree_k)
        static_cast<float*>(a.tree_k)[o] = rope_pair(xk, i, half, a.rope_cos[static_cast<size_t>(pos) * half + ii],
                                                     a.rope_sin[static_cast<size_t>(pos) * half + ii]);
      if (a.tree_v) static_cast<float*>(a.tree_v)[o] = xk[a.Hkv * D + i];
    }
  }
}

}  // namespace

static int attn_qblocks(int n_rows, int Hq, int Hkv) { return (n_rows * (Hq / Hkv) + kQW - 1) / kQW; }

// Split policy: enough work-groups to fill the CUs once, but no split shorter
// than GLANCE_ATTN_MINBLK blocks of 32 keys (each split adds a 528-byte record
// per query and KV head).
#ifndef GLANCE_ATTN_FILL
#define GLANCE_ATTN_FILL 256
#endif
#ifndef GLANCE_ATTN_MINBLK
#define GLANCE_ATTN_MINBLK 4
#endif
#ifndef GLANCE_ATTN_FUSE
#define GLANCE_ATTN_FUSE 8
#endif

namespace {
struct AttnPlan {
  int waves;  // waves per work-group of the shared-tile kernel (4 or 2)
  int n_split;
  bool fuse;  // the last split of a query group merges the records (no attn_combine)
};

int tile_splits(int nseq, int64_t max_prefix, int nqb, int Hkv, int W) {
  const int64_t base = static_cast<int64_t>(nseq) * Hkv * ((nqb + W - 1) / W);
  const int64_t fill = (GLANCE_ATTN_FILL + base - 1) / base;
  const int64_t len = max_prefix / (kKB * GLANCE_ATTN_MINBLK);
  int64_t n = fill < len ? fill : len;
  if (n < 1) n = 1;
  if (n > kMaxSplit) n = kMaxSplit;
  return static_cast<int>(n);
}

// Four waves per work-group share each tile four ways; when the rounds are too
// short for four-wave groups to fill the CUs (splits kept >= the minimum
// length), two-wave groups give twice the work-groups for the same splits.
AttnPlan attn_plan(int nseq, int64_t max_prefix, int n_rows, int Hq, int Hkv) {
  const int nqb = attn_qblocks(n_rows, Hq, Hkv);
  const int64_t T = max_prefix + n_rows;
  const int n4 = tile_splits(nseq, T, nqb, Hkv, 4);
  const int64_t wg4 = static_cast<int64_t>(nseq) * Hkv * ((nqb + 3) / 4) * n4;
  AttnPlan p{4, n4, false};
  if (wg4 < GLANCE_ATTN_FILL && nqb > 2) p = AttnPlan{2, tile_splits(nseq, T, nqb, Hkv, 2), false};
  // in-kernel merge when a query group's records are few: the last work-group
  // to arrive reads n_split x waves x 32 records of 528 bytes
  p.fuse = p.n_split > 1 && p.n_split * p.waves <= GLANCE_ATTN_FUSE;
  return p;
}
}  // namespace

int attn_splits(int nseq, int64_t max_prefix, int n_rows, int Hq, int Hkv) {
  return attn_plan(nseq, max_prefix, n_rows, Hq, Hkv).n_split;
}

size_t attn_arrival_words(int nseq, int n_rows, int Hq, int Hkv) {
  return static_cast<size_t>(nseq) * Hkv * attn_qblocks(n_rows, Hq, Hkv);
}

size_t attn_part_floats(int nseq, int n_rows, int Hq, int Hkv, int n_split) {
  if (n_split <= 1) return 0;
  return static_cast<size_t>(nseq) * Hkv * attn_qblocks(n_rows, Hq, Hkv) * n_split * kQW * kRec;
}

glance_status launch_tree_attention(const AttnArgs& a, hipStream_t st) {
  if (a.dtype == GLANCE_BF16) {
    const int nqb = attn_qblocks(a.n_rows, a.Hq, a.Hkv);
    // the plan that sized the workspace's split records
    const AttnPlan pl = attn_plan(a.nseq, a.max_prefix, a.n_rows, a.Hq, a.Hkv);
    if (pl.n_split != a.n_split) return GLANCE_ERR_INVALID_ARG;
    const int grid = a.nseq * a.n_split * ((nqb + pl.waves - 1) / pl.waves) * a.Hkv;
    const int fuse = pl.fuse && a.arrivals != nullptr;
    if (pl.waves == 4)
      tree_attn_tile_kernel<4><<<grid, 4 * kWave, 0, st>>>(a, nqb, fuse);
    else
      tree_attn_tile_kernel<2><<<grid, 2 * kWave, 0, st>>>(a, nqb, fuse);
    GLANCE_LAUNCH_CHECK();
    if (fuse) return GLANCE_OK;
    if (a.n_split > 1) {
      if (a.Hq % 4 == 0) {
        const dim3 cg(a.nseq * a.n_rows, a.Hq / 4);
        if (a.n_split <= 4)
          attn_combine4_kernel<4><<<cg, 128, 0, st>>>(a, nqb);
        else if (a.n_split <= 8)
          attn_combine4_kernel<8><<<cg, 128, 0, st>>>(a, nqb);
        else
          attn_combine4_kernel<kMaxSplit><<<cg, 128, 0, st>>>(a, nqb);
      } else {
        const dim3 cg(a.nseq * a.n_rows, a.Hq);
        if (a.n_split <= 4)
          attn_combine_kernel<4><<<cg, kHD, 0, st>>>(a, nqb);
        else if (a.n_split <= 8)
          attn_combine_kernel<8><<<cg, kHD, 0, st>>>(a, nqb);
        else
          attn_combine_kernel<kMaxSplit><<<cg, kHD, 0, st>>>(a, nqb);
      }
      GLANCE_LAUNCH_CHECK();
    }
  } else {
    dim3 grid(a.nseq * a.n_rows, a.Hq);
    tree_attn_f32_kernel<<<grid, 128, 0, st>>>(a);
    GLANCE_LAUNCH_CHECK();
  }
  return GLANCE_OK;
}

}  // namespace glance
