// Packed, ancestor-masked GQA attention of the verify rows (step 3).
//
// Paper §3.2 Def. 1 and App. B.1 (proof of Theorem 1): packing the tree into
// one pass with ancestor-only masking changes the attention layout, not a row's
// conditioning, so the row of node i attends to the cached prefix of its round
// plus exactly the tree rows j that are i itself or its ancestors (bit j of
// anc[i]), which is the causal sequence x o b o y_{1:d(i)}.
//
// bf16 path (head_dim 128, gfx950 MFMA v_mfma_f32_32x32x16_bf16).  Grid
// (prefix splits + 1, Hkv x query blocks, rounds), 256 threads: the queries of
// one KV head are its Hq/Hkv query heads times the round's rows (<= 128 per
// work-group, 32 per wave; smaller blocks spread a round over more CUs).  Split c takes prefix keys [c*128, (c+1)*128) as
// one tile: the query, K and V loads are all issued before any is used; K is
// staged in LDS as [key][dim], V transposed as [dim][key]; each wave forms
// S^T = K Q^T (one query per lane, so the row max and sum stay inside a lane
// and its partner lane l^32), rounds P to bf16 into its own LDS tile and forms
// O^T = V^T P^T.  The extra split n_split takes the round's tree rows as keys:
// the rotated bf16 K and bf16 V rows the q/k/v projection wrote (a storage
// point), masked by anc.  Each (split, query) leaves (max, sum, unnormalised
// O); attn_combine merges them.
//
// fp32 path (tiny shapes): one work-group per (row, query head), scores in LDS,
// plain fp32 loops.
#include "common.h"
#include "kernels.h"

namespace glance {

namespace {

constexpr int kAThreads = 256;
constexpr int kQWave = 32;
constexpr int kQBlock = 128;
constexpr int kKT = 128;         // keys per work-group tile (one prefix split)
constexpr int kHD = 128;         // head_dim of the bf16 path
constexpr int kTPad = 136;       // row stride of the K, V^T and P tiles (bf16)
constexpr int kRec = kHD + 4;    // partial record: m, l, -, -, o[128]

// position P + depth of a row, clamped into the cos/sin tables
__device__ __forceinline__ int row_pos(const AttnArgs& a, int P, int row) {
  const int p = P + a.depth[row];
  return p < a.n_pos - 1 ? p : a.n_pos - 1;
}

__device__ __forceinline__ float rope_pair(const float* x, int i, int half, float c, float s) {
  // rotate-half: (x_i, x_{i+half}) -> (x_i c - x_{i+half} s, x_{i+half} c + x_i s)
  return i < half ? x[i] * c - x[i + half] * s : x[i] * c + x[i - half] * s;
}

__global__ __launch_bounds__(kAThreads) void tree_attn_bf16_kernel(AttnArgs a) {
  __shared__ __attribute__((aligned(16))) uint16_t Ks[kKT][kTPad];
  __shared__ __attribute__((aligned(16))) uint16_t Vt[kHD][kTPad];
  __shared__ __attribute__((aligned(16))) uint16_t Ps[kAThreads / kWave][kQWave][kTPad];

  const int c = blockIdx.x, s = blockIdx.z;
  const int h = blockIdx.y % a.Hkv, qb = blockIdx.y / a.Hkv;
  const int G = a.Hq / a.Hkv;
  const int Qn = a.n_rows * G;
  const int tid = threadIdx.x, w = tid >> 6, l = tid & 63, j = l & 31, g = l >> 5;
  const bool tree_split = (c == a.n_split);
  const int64_t kv0 = a.kv_offsets[s];
  const int P = static_cast<int>(a.kv_offsets[s + 1] - kv0);

  // ---- this lane's query: q index, row, head (rotated and rounded by the projection)
  const int q = qb * kQBlock + w * kQWave + j;
  const bool qvalid = q < Qn;
  const int r = qvalid ? q / G : 0;
  const int qh = h * G + (qvalid ? q % G : 0);
  const int grow = s * a.n_rows + r;
  const uint64_t qanc = qvalid ? a.anc[grow] : 0ull;

  int kbeg, kend;
  if (tree_split) {
    kbeg = 0;
    kend = a.n_rows;
  } else {
    kbeg = c * a.split;
    kend = min(kbeg + a.split, P);
  }
  const int nk = kend - kbeg;  // <= kKT keys in this tile

  // ---- every load of the tile issued up front: the query, then K and V.  The
  // query is loaded for padding rows too (their records are never combined:
  // each query's scores and output stay in its own lanes), so that its loads
  // do not wait for the row's token
  bf16x8 qf[8];
  {
    const uint16_t* xq = static_cast<const uint16_t*>(a.q) + static_cast<size_t>(grow) * a.Hq * kHD + qh * kHD;
#pragma unroll
    for (int ks = 0; ks < 8; ++ks)
      qf[ks] = __builtin_bit_cast(bf16x8, *reinterpret_cast<const uint4*>(xq + ks * 16 + 8 * g));
  }
  constexpr int kPass = kKT * (kHD / 8) / kAThreads;  // 16-byte pieces per thread
  uint4 kb_[kPass], vb_[kPass];
  {
    const uint16_t* kbase = tree_split ? static_cast<const uint16_t*>(a.tree_k)
                                       : static_cast<const uint16_t*>(a.k_cache);
    const uint16_t* vbase = tree_split ? static_cast<const uint16_t*>(a.tree_v)
                                       : static_cast<const uint16_t*>(a.v_cache);
#pragma unroll
    for (int pass = 0; pass < kPass; ++pass) {
      const int idx = pass * kAThreads + tid;
      const int kr = idx >> 4, col = (idx & 15) * 8;
      kb_[pass] = make_uint4(0, 0, 0, 0);
      vb_[pass] = make_uint4(0, 0, 0, 0);
      if (kr < nk) {
        const int64_t krow = tree_split ? static_cast<int64_t>(s) * a.n_rows + kr : kv0 + kbeg + kr;
        const size_t off = (static_cast<size_t>(krow) * a.Hkv + h) * kHD + col;
        kb_[pass] = load_stream(kbase + off);
        vb_[pass] = load_stream(vbase + off);
      }
    }
  }
  // K as [key][dim]; V transposed to [dim][key], its 8-key blocks XOR-swizzled by
  // the dim's 8-row block so that the transposing stores spread over the banks
#pragma unroll
  for (int pass = 0; pass < kPass; ++pass) {
    const int idx = pass * kAThreads + tid;
    const int kr = idx >> 4, col = (idx & 15) * 8;
    *reinterpret_cast<uint4*>(&Ks[kr][col]) = kb_[pass];
    const uint32_t vw[4] = {vb_[pass].x, vb_[pass].y, vb_[pass].z, vb_[pass].w};
    const int kcol = 8 * ((kr >> 3) ^ ((col >> 3) & 15)) + (kr & 7);
#pragma unroll
    for (int t = 0; t < 4; ++t) {
      Vt[col + 2 * t][kcol] = static_cast<uint16_t>(vw[t] & 0xFFFF);
      Vt[col + 2 * t + 1][kcol] = static_cast<uint16_t>(vw[t] >> 16);
    }
  }
  __syncthreads();

  // ---- S^T = K Q^T: kKT keys x this wave's 32 queries (32-key blocks past the
  // tile's keys are skipped: they are masked)
  f32x16 acc_s[kKT / 32] = {};
#pragma unroll
  for (int kb = 0; kb < kKT / 32; ++kb) {
    if (kb * 32 >= nk) break;  // (uniform)
#pragma unroll
    for (int ks = 0; ks < 8; ++ks) {
      const bf16x8 av = *reinterpret_cast<const bf16x8*>(&Ks[kb * 32 + j][ks * 16 + 8 * g]);
      acc_s[kb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(av, qf[ks], acc_s[kb], 0, 0, 0);
    }
  }
  // element v of acc_s[kb]: key kb*32 + 8 (v/4) + 4 g + v%4 of the tile, query j
  const float scale_log2 = 1.4426950408889634f / sqrtf(static_cast<float>(kHD));
  float m = -INFINITY;
  if (!tree_split && nk == kKT) {  // (uniform) a full prefix tile: every key visible
#pragma unroll
    for (int kb = 0; kb < kKT / 32; ++kb)
#pragma unroll
      for (int v = 0; v < 16; ++v) {
        acc_s[kb][v] *= scale_log2;
        m = fmaxf(m, acc_s[kb][v]);
      }
  } else {
#pragma unroll
    for (int kb = 0; kb < kKT / 32; ++kb) {
#pragma unroll
      for (int v = 0; v < 16; ++v) {
        const int key = kb * 32 + 8 * (v >> 2) + 4 * g + (v & 3);
        bool vis = key < nk;
        if (tree_split) vis = vis && ((qanc >> key) & 1ull);
        const float sv = vis ? acc_s[kb][v] * scale_log2 : -INFINITY;
        acc_s[kb][v] = sv;
        m = fmaxf(m, sv);
      }
    }
  }
  m = fmaxf(m, __shfl_xor(m, 32, kWave));
  // P rounded to bf16 in pairs (hardware round-to-nearest-even); l sums the
  // rounded values, so that it normalises exactly the P that enters O
  const float mz = m == -INFINITY ? 0.f : m;  // (no visible key: every p is exp2(-inf) = 0)
  float lsum = 0.f;
#pragma unroll
  for (int kb = 0; kb < kKT / 32; ++kb) {
#pragma unroll
    for (int vg = 0; vg < 4; ++vg) {
      uint32_t pw[2];
#pragma unroll
      for (int t = 0; t < 2; ++t) {
        const float p0 = __builtin_amdgcn_exp2f(acc_s[kb][4 * vg + 2 * t] - mz);
        const float p1 = __builtin_amdgcn_exp2f(acc_s[kb][4 * vg + 2 * t + 1] - mz);
        pw[t] = pack_bf16x2(p0, p1);
        lsum += __uint_as_float(pw[t] << 16) + __uint_as_float(pw[t] & 0xFFFF0000u);
      }
      *reinterpret_cast<uint2*>(&Ps[w][j][kb * 32 + 8 * vg + 4 * g]) = make_uint2(pw[0], pw[1]);
    }
  }
  lsum += __shfl_xor(lsum, 32, kWave);
  __builtin_amdgcn_wave_barrier();  // the wave's own P tile: same-wave LDS accesses are in order

  // ---- O^T = V^T P^T
  f32x16 acc_o[4] = {};
#pragma unroll
  for (int db = 0; db < 4; ++db) {
    const int dim = db * 32 + j;
#pragma unroll
    for (int ks = 0; ks < kKT / 16; ++ks) {
      if (ks * 16 >= nk) break;  // (uniform) keys past the tile have p = 0
      const int kblk = (ks * 16 + 8 * g) >> 3;
      const bf16x8 av = *reinterpret_cast<const bf16x8*>(&Vt[dim][8 * (kblk ^ ((dim >> 3) & 15))]);
      const bf16x8 bv = *reinterpret_cast<const bf16x8*>(&Ps[w][j][ks * 16 + 8 * g]);
      acc_o[db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(av, bv, acc_o[db], 0, 0, 0);
    }
  }

  // ---- partial record of (split, query): m (log2 units), l, unnormalised O
  if (qvalid) {
    float* rec = a.part +
                 ((static_cast<size_t>(s) * a.Hkv + h) * (a.n_split + 1) + c) * static_cast<size_t>(Qn) * kRec +
                 static_cast<size_t>(q) * kRec;
    if (g == 0) {
      rec[0] = m;
      rec[1] = lsum;
    }
#pragma unroll
    for (int db = 0; db < 4; ++db)
#pragma unroll
      for (int vg = 0; vg < 4; ++vg) {
        const int dim = db * 32 + 8 * vg + 4 * g;
        *reinterpret_cast<float4*>(rec + 4 + dim) =
            make_float4(acc_o[db][4 * vg], acc_o[db][4 * vg + 1], acc_o[db][4 * vg + 2], acc_o[db][4 * vg + 3]);
      }
  }
}

// Merge the split partials of every (row, query head) into the attention output:
// one work-group per row and query head, one thread per head dimension, splits
// folded in order in batches of 16 with a running maximum.
__global__ __launch_bounds__(kHD) void attn_combine_kernel(AttnArgs a) {
  const int grow = blockIdx.x, qh = blockIdx.y, dim = threadIdx.x;
  const int s = grow / a.n_rows, r = grow % a.n_rows;
  const int G = a.Hq / a.Hkv;
  const int Qn = a.n_rows * G;
  const int h = qh / G, q = r * G + qh % G;
  // the records are read whatever the row's token (in bounds for every row), so
  // that their loads do not wait for the token's; padding rows give 0
  const bool live = a.token[grow] >= 0;
  float o;
  {
    const float* rec = a.part + ((static_cast<size_t>(s) * a.Hkv + h) * (a.n_split + 1) *
                                     static_cast<size_t>(Qn) + q) * kRec;
    const size_t stride = static_cast<size_t>(Qn) * kRec;
    const int ns = a.n_split + 1;
    // 16 splits at a time: every load of the batch issued first, then the
    // batch maximum, then the rescaled sums
    float M = -INFINITY, Ls = 0.f, acc = 0.f;
    for (int c0 = 0; c0 < ns; c0 += 16) {
      float mm[16], ll[16], vv[16];
#pragma unroll
      for (int u = 0; u < 16; ++u) {
        const size_t cc = static_cast<size_t>(min(c0 + u, ns - 1)) * stride;
        mm[u] = rec[cc];
        ll[u] = rec[cc + 1];
        vv[u] = rec[cc + 4 + dim];
      }
      float Mb = M;
#pragma unroll
      for (int u = 0; u < 16; ++u)
        if (c0 + u < ns && ll[u] > 0.f) Mb = fmaxf(Mb, mm[u]);
      const float fo = (M == -INFINITY) ? 0.f : __builtin_amdgcn_exp2f(M - Mb);
      Ls *= fo;
      acc *= fo;
#pragma unroll
      for (int u = 0; u < 16; ++u) {
        // splits without visible keys have l = 0 and contribute nothing
        const float f = (c0 + u < ns && ll[u] > 0.f) ? __builtin_amdgcn_exp2f(mm[u] - Mb) : 0.f;
        Ls += ll[u] * f;
        acc += vv[u] * f;
      }
      M = Mb;
    }
    o = live ? acc / Ls : 0.f;
  }
  const size_t off = static_cast<size_t>(grow) * a.Hq * kHD + qh * kHD + dim;
  if (a.attn_out) a.attn_out[off] = o;
  static_cast<uint16_t*>(a.attn_x)[off] = f32_to_bf16(o);
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
  float* ox = static_cast<float*>(a.attn_x) + static_cast<size_t>(grow) * a.Hq * D + qh * D;
  if (a.token[grow] < 0) {
    for (int d = tid; d < D; d += 128) {
      ox[d] = 0.f;
      if (a.attn_out) a.attn_out[static_cast<size_t>(grow) * a.Hq * D + qh * D + d] = 0.f;
    }
    return;
  }
  const int64_t kv0 = a.kv_offsets[s];
  const int P = static_cast<int>(a.kv_offsets[s + 1] - kv0);
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

int attn_split_len(int64_t max_prefix, int nseq, int Hkv) {
  (void)max_prefix;
  (void)nseq;
  (void)Hkv;
  return kKT;  // one tile per split work-group
}

size_t attn_part_floats(int nseq, int n_rows, int Hq, int Hkv, int D, int n_split) {
  (void)D;
  const size_t Qn = static_cast<size_t>(n_rows) * (Hq / Hkv);
  return static_cast<size_t>(nseq) * Hkv * (n_split + 1) * Qn * kRec;
}

glance_status launch_tree_attention(const AttnArgs& a, hipStream_t st) {
  if (a.dtype == GLANCE_BF16) {
    const int Qn = a.n_rows * (a.Hq / a.Hkv);
    const int nqb = (Qn + kQBlock - 1) / kQBlock;
    dim3 grid(a.n_split + 1, a.Hkv * nqb, a.nseq);
    tree_attn_bf16_kernel<<<grid, kAThreads, 0, st>>>(a);
    GLANCE_LAUNCH_CHECK();
    attn_combine_kernel<<<dim3(a.nseq * a.n_rows, a.Hq), kHD, 0, st>>>(a);
    GLANCE_LAUNCH_CHECK();
  } else {
    dim3 grid(a.nseq * a.n_rows, a.Hq);
    tree_attn_f32_kernel<<<grid, 128, 0, st>>>(a);
    GLANCE_LAUNCH_CHECK();
  }
  return GLANCE_OK;
}

}  // namespace glance
