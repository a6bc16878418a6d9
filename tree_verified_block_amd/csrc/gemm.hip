// Skinny GEMMs of the verify pass: C = X W^T for the few verify rows X [M][K]
// against a streamed weight matrix W [N][K] (out x in), with the epilogue fused:
//   EPI_QKV    the q/k/v projection: q and k rotated (rotate-half RoPE at the
//              row's position), q, k, v rounded to bf16 (k and v are the rows'
//              new cache entries, a storage point);
//   EPI_RESID  the output projection plus residual, rounded to bf16 (the
//              layer's output, a storage point);
//   EPI_HEAD   the LM head: per row, partial (max, argmax, second max,
//              sum e^(z-max), sum e^(z-max)(z-max)) of the work-group's columns,
//              merged by head_merge into argmax, top-1, top-2 gap and entropy
//              (paper §3.1 greedy token; App. B.1 top-2 gap; §6 root entropy).
//
// bf16 path, gfx950 MFMA v_mfma_f32_16x16x32_bf16.  W is cut into 16-row blocks
// (the MFMA A operand: lane l holds row l%16, k = 8(l/16)..+7 of a 32-deep step).
// A 256-thread work-group is 4 waves; each wave owns B blocks of one K-slice
// (S slices per work-group: S = 1 for the LM head, S = 4 for the small
// projections so that hundreds of work-groups share their few thousand rows).
// The loop runs over K outermost: every 64-deep chunk of the 64 activation rows
// is staged once in LDS and shared by the work-group, while each wave streams
// its blocks' weights from HBM straight into a ring of registers (the loads of
// chunk c + DEPTH are issued before chunk c waits on its LDS barrier) and keeps
// all its accumulators in registers.  At M <= 64 the weight
// stream is the whole cost (64 flop per weight byte, far below the MFMA ridge),
// so the kernel is judged against HBM bandwidth.  Blocks are dealt round-robin
// over all waves of the grid (9496 blocks over 2048 waves for V = 151936), and
// the M-tiles of one weight range are placed on the same XCD back to back so
// that the weights are fetched from HBM once per XCD L2.
#include "common.h"
#include "kernels.h"

namespace glance {

namespace {

constexpr int kGThreads = 256;
constexpr int kTileM = 64;
constexpr int kKc = 64;            // K chunk staged per step
constexpr int kXP = kKc + 8;       // LDS row stride (bf16), padded against bank conflicts
constexpr int kXS = kTileM * kXP;  // one staged sub-chunk (elements)

struct HeadPart {
  float m;   // max logit
  int am;    // its token id (smallest on ties)
  float m2;  // best logit of any other token
  float s;   // sum exp(z - m)
  float t;   // sum exp(z - m) (z - m)
};

__device__ __forceinline__ HeadPart head_empty() {
  HeadPart p;
  p.m = -INFINITY;
  p.am = 0x7FFFFFFF;
  p.m2 = -INFINITY;
  p.s = 0.f;
  p.t = 0.f;
  return p;
}

// Merge two partials.  Max/argmax/second are exact; the sums are rescaled to
// the merged maximum: s = sa + sb e^(mb-m), t = ta + e^(mb-m) (tb + (mb-m) sb).
__device__ __forceinline__ HeadPart head_combine(HeadPart a, HeadPart b) {
  if (b.m > a.m || (b.m == a.m && b.am < a.am)) {
    HeadPart tmp = a;
    a = b;
    b = tmp;
  }
  HeadPart r;
  r.m = a.m;
  r.am = a.am;
  r.m2 = fmaxf(a.m2, b.m);
  r.s = a.s;
  r.t = a.t;
  if (b.s > 0.f) {
    const float d = b.m - a.m;
    const float e = expf(d);
    r.s = a.s + b.s * e;
    r.t = a.t + e * (b.t + d * b.s);
  }
  return r;
}

__device__ __forceinline__ HeadPart head_elem(float z, int n) {
  HeadPart p;
  p.m = z;
  p.am = n;
  p.m2 = -INFINITY;
  p.s = 1.f;
  p.t = 0.f;
  return p;
}

__device__ __forceinline__ HeadPart shfl_part(const HeadPart& p, int src) {
  HeadPart r;
  r.m = __shfl(p.m, src, kWave);
  r.am = __shfl(p.am, src, kWave);
  r.m2 = __shfl(p.m2, src, kWave);
  r.s = __shfl(p.s, src, kWave);
  r.t = __shfl(p.t, src, kWave);
  return r;
}


__device__ __forceinline__ const uint16_t* x_row_ptr(const GemmArgs& a, int m) {
  if (m >= a.M) return nullptr;
  if (a.gather) {
    const int tok = a.gather[m];
    if (tok < 0) return nullptr;
    return static_cast<const uint16_t*>(a.x) + static_cast<size_t>(tok) * a.K;
  }
  return static_cast<const uint16_t*>(a.x) + static_cast<size_t>(m) * a.K;
}

// W row of row i (0..15) of block b.  For EPI_QKV the q and k blocks pair head
// dims so that rows i and i+8 are RoPE partners: block j of a head holds dims
// 8j..8j+7 and 64+8j..64+8j+7.
template <int EPI>
__device__ __forceinline__ int block_row(const GemmArgs& a, int b, int i) {
  if constexpr (EPI == EPI_QKV) {
    const int nq = a.Hq * 8, nk = a.Hkv * 8;
    if (b < nq + nk) {
      const int base = b < nq ? 0 : a.Hq * 128;
      const int bb = b < nq ? b : b - nq;
      const int dim = (i < 8) ? 8 * (bb & 7) + i : 64 + 8 * (bb & 7) + (i - 8);
      return base + (bb >> 3) * 128 + dim;
    }
    return (a.Hq + a.Hkv) * 128 + (b - nq - nk) * 16 + i;
  } else {
    return b * 16 + i;
  }
}

__device__ __forceinline__ const uint16_t* w_row_ptr(const GemmArgs& a, int row) {
  int start = 0, sidx = 0;
  while (sidx < a.w.nseg - 1 && row >= a.w.n_end[sidx]) start = a.w.n_end[sidx++];
  return static_cast<const uint16_t*>(a.w.w[sidx]) + static_cast<size_t>(row - start) * a.K;
}

__device__ __forceinline__ uint2 pack4_bf16(float x0, float x1, float x2, float x3) {
  uint2 u;
  u.x = static_cast<uint32_t>(f32_to_bf16(x0)) | (static_cast<uint32_t>(f32_to_bf16(x1)) << 16);
  u.y = static_cast<uint32_t>(f32_to_bf16(x2)) | (static_cast<uint32_t>(f32_to_bf16(x3)) << 16);
  return u;
}

template <int EPI, int B, int S, int DEPTH>
__global__ __launch_bounds__(kGThreads, 2) void gemm_bf16_kernel(GemmArgs a, int NB, int NG,
                                                                 int nWG, int nMT) {
  constexpr int GPW = 4 / S;  // block groups per work-group
  // The LM head streams its weights with full-line non-temporal loads and
  // transposes them to the MFMA layout through a per-wave LDS tile; the
  // projections load the MFMA layout directly.
  constexpr bool CW = EPI == EPI_HEAD;
  __shared__ __attribute__((aligned(16))) uint16_t xs[2 * S * kXS];
  __shared__ __attribute__((aligned(16))) uint16_t wtile[CW ? 4 * B * 16 * kXP : 8];
  __shared__ HeadPart hred[4][kTileM];

  const int bid = blockIdx.x;
  const int xcd = bid & 7, kk = bid >> 3;
  const int mt = kk % nMT;
  const int wg = (kk / nMT) * 8 + xcd;
  if (wg >= nWG) return;
  const int m0 = mt * kTileM;
  const int tid = threadIdx.x, w = tid >> 6, l = tid & 63, lr = l & 15, lg = l >> 4;
  const int q = w % S, gi = w / S;
  const int G = wg * GPW + gi;
  const int Ks = a.K / S;
  const int kbase = q * Ks;
  const int nck = Ks / kKc;
  uint16_t* wt = wtile + (CW ? w * B * 16 * kXP : 0);

  // this wave's blocks.  Weight load i of a block (i = 0, 1) per chunk: in the
  // MFMA operand layout, rows lr at k = 32 i + 8 lg; coalesced (CW), rows
  // 8 i + l/8 at k = 8 (l%8), i.e. eight full 128-byte row segments per load.
  int blk[B];
  bool bval[B];
  const uint16_t* wp[B][2];
#pragma unroll
  for (int t = 0; t < B; ++t) {
    blk[t] = G + t * NG;
    bval[t] = G < NG && blk[t] < NB;
#pragma unroll
    for (int i = 0; i < 2; ++i) {
      const int ri = CW ? 8 * i + (l >> 3) : lr;
      int row = bval[t] ? block_row<EPI>(a, blk[t], ri) : 0;
      if (row > a.N - 1) row = a.N - 1;
      wp[t][i] = w_row_ptr(a, row) + kbase + (CW ? 8 * (l & 7) : 32 * i + 8 * lg);
    }
  }

  // activation rows this thread stages: S sub-chunks x 64 rows x 8 pieces of 16 B
  const uint16_t* xr[2 * S];
  int xoff[2 * S], xlds[2 * S];
#pragma unroll
  for (int e = 0; e < 2 * S; ++e) {
    const int idx = e * kGThreads + tid;
    const int sub = idx >> 9, r = (idx >> 3) & 63, cc = (idx & 7) * 8;
    xr[e] = x_row_ptr(a, m0 + r);
    xoff[e] = sub * Ks + cc;
    xlds[e] = sub * kXS + r * kXP + cc;
  }

  f32x4 acc[B][4];
#pragma unroll
  for (int t = 0; t < B; ++t)
#pragma unroll
    for (int mb = 0; mb < 4; ++mb) acc[t][mb] = f32x4{0.f, 0.f, 0.f, 0.f};
  // Rings of DEPTH + 1 chunk slots in registers for the weights and for the
  // activation chunks on their way to LDS.  Iteration c issues the activation
  // loads of chunk c + DEPTH, then the weight loads of chunk c + DEPTH, and at
  // its end stores chunk c + 1 to the other LDS stage.  Loads complete in issue
  // order, so every wait is for data that is due anyway: DEPTH chunks stay in
  // flight through the barriers.
  constexpr int RS = DEPTH + 1;
  static_assert(RS % 2 == 0, "ring slots and LDS stages must unroll together");
  uint4 wbuf[RS][B][2];
  uint4 xbuf[RS][2 * S];
  auto wload = [&](int c, uint4 (&dst)[B][2]) {
#pragma unroll
    for (int t = 0; t < B; ++t)
#pragma unroll
      for (int i = 0; i < 2; ++i) {
        if constexpr (CW)
          dst[t][i] = load_stream(wp[t][i] + c * kKc);
        else
          dst[t][i] = *reinterpret_cast<const uint4*>(wp[t][i] + c * kKc);
      }
  };
  auto xload = [&](int c, uint4 (&dst)[2 * S]) {
#pragma unroll
    for (int e = 0; e < 2 * S; ++e) {
      dst[e] = make_uint4(0, 0, 0, 0);
      if (xr[e]) dst[e] = *reinterpret_cast<const uint4*>(xr[e] + xoff[e] + c * kKc);
    }
  };

  // prologue: X chunk 0 -> LDS stage 0; X chunks 1 .. DEPTH-1 and W chunks
  // 0 .. DEPTH-1 -> registers, each W chunk after the X chunk due before it
  xload(0, xbuf[0]);
#pragma unroll
  for (int e = 0; e < 2 * S; ++e) *reinterpret_cast<uint4*>(&xs[xlds[e]]) = xbuf[0][e];
#pragma unroll
  for (int d = 0; d < DEPTH; ++d) {
    if (d + 1 < DEPTH && d + 1 < nck) xload(d + 1, xbuf[d + 1]);
    if (d < nck) wload(d, wbuf[d]);
  }

  for (int c0 = 0; c0 < nck; c0 += RS) {
#pragma unroll
    for (int u = 0; u < RS; ++u) {
      const int c = c0 + u;
      if (c < nck) {
        if (c + DEPTH < nck) {
          xload(c + DEPTH, xbuf[(u + DEPTH) % RS]);
          wload(c + DEPTH, wbuf[(u + DEPTH) % RS]);
        }
        if constexpr (CW) {
          // this wave's weight chunk into its LDS tile, row-major (same-wave
          // LDS accesses complete in order, so no barrier is needed)
#pragma unroll
          for (int t = 0; t < B; ++t)
#pragma unroll
            for (int i = 0; i < 2; ++i)
              *reinterpret_cast<uint4*>(wt + (t * 16 + 8 * i + (l >> 3)) * kXP + 8 * (l & 7)) = wbuf[u][t][i];
        }
        __syncthreads();
        const uint16_t* xq = xs + ((u & 1) * S + q) * kXS;
#pragma unroll
        for (int s = 0; s < 2; ++s) {
          bf16x8 bx[4];
#pragma unroll
          for (int mb = 0; mb < 4; ++mb)
            bx[mb] = *reinterpret_cast<const bf16x8*>(xq + (mb * 16 + lr) * kXP + s * 32 + 8 * lg);
#pragma unroll
          for (int t = 0; t < B; ++t) {
            bf16x8 av;
            if constexpr (CW)
              av = *reinterpret_cast<const bf16x8*>(wt + (t * 16 + lr) * kXP + s * 32 + 8 * lg);
            else
              av = __builtin_bit_cast(bf16x8, wbuf[u][t][s]);
#pragma unroll
            for (int mb = 0; mb < 4; ++mb)
              acc[t][mb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(av, bx[mb], acc[t][mb], 0, 0, 0);
          }
        }
        if (c + 1 < nck) {
#pragma unroll
          for (int e = 0; e < 2 * S; ++e)
            *reinterpret_cast<uint4*>(&xs[((u + 1) & 1) * S * kXS + xlds[e]]) = xbuf[(u + 1) % RS][e];
        }
      }
    }
  }

  // ------------------------------------------------------------------ epilogues
  // acc[t][mb][v]: row i = 4 lg + v of block blk[t], activation row m0 + 16 mb + lr.
  if constexpr (EPI == EPI_HEAD) {
    HeadPart hp[4];
#pragma unroll
    for (int mb = 0; mb < 4; ++mb) hp[mb] = head_empty();
#pragma unroll
    for (int t = 0; t < B; ++t) {
      if (!bval[t]) continue;
#pragma unroll
      for (int v = 0; v < 4; ++v) {
        const int n = blk[t] * 16 + 4 * lg + v;
        if (n < a.N) {
#pragma unroll
          for (int mb = 0; mb < 4; ++mb) {
            hp[mb] = head_combine(hp[mb], head_elem(acc[t][mb][v], n));
            const int m = m0 + mb * 16 + lr;
            if (a.logits && m < a.M) a.logits[static_cast<size_t>(m) * a.N + n] = acc[t][mb][v];
          }
        }
      }
    }
#pragma unroll
    for (int mb = 0; mb < 4; ++mb) {
      hp[mb] = head_combine(hp[mb], shfl_part(hp[mb], l ^ 16));
      hp[mb] = head_combine(hp[mb], shfl_part(hp[mb], l ^ 32));
      if (lg == 0) hred[w][mb * 16 + lr] = hp[mb];
    }
    __syncthreads();
    if (tid < kTileM) {
      HeadPart p = hred[0][tid];
#pragma unroll
      for (int ww = 1; ww < 4; ++ww) p = head_combine(p, hred[ww][tid]);
      const int m = m0 + tid;
      if (m < a.M) {
        float* o = a.part + (static_cast<size_t>(m) * nWG + wg) * 5;
        o[0] = p.m;
        o[1] = __int_as_float(p.am);
        o[2] = p.m2;
        o[3] = p.s;
        o[4] = p.t;
      }
    }
  } else {
    // sum the S K-slice partials of each block in LDS (fixed order), then write
    static_assert(B == 1, "projection epilogues take one block per wave");
    float* red = reinterpret_cast<float*>(xs);  // [GPW][S][16][64]
    __syncthreads();
#pragma unroll
    for (int mb = 0; mb < 4; ++mb)
#pragma unroll
      for (int v = 0; v < 4; ++v)
        red[((gi * S + q) * 16 + 4 * lg + v) * 64 + mb * 16 + lr] = acc[0][mb][v];
    __syncthreads();
    if (!bval[0]) return;
    const int lt = q * 64 + l;  // thread index within the block group (S*64 threads)
    const float* rg = red + gi * S * 1024;
    auto sumq = [&](int i, int m) {
      float x = 0.f;
#pragma unroll
      for (int qq = 0; qq < S; ++qq) x += rg[(qq * 16 + i) * 64 + m];
      return x;
    };
    if constexpr (EPI == EPI_RESID) {
      // 16 rows x 64 activations = 256 items of 4 consecutive columns
      for (int it = lt; it < 256; it += S * 64) {
        const int m = it & 63, i0 = (it >> 6) * 4;
        const int gm = m0 + m;
        if (gm >= a.M) continue;
        const int n = blk[0] * 16 + i0;
        if (n >= a.N) continue;
        float x[4];
#pragma unroll
        for (int v = 0; v < 4; ++v) x[v] = sumq(i0 + v, m);
        uint2 o = make_uint2(0, 0);
        const int tok = a.resid_tok[gm];
        if (tok >= 0) {
          const uint16_t* rp = static_cast<const uint16_t*>(a.resid) +
                               static_cast<size_t>(a.resid_by_token ? tok : gm) * a.N + n;
          const uint2 r = *reinterpret_cast<const uint2*>(rp);
          o = pack4_bf16(bf16_to_f32(r.x & 0xFFFF) + x[0], bf16_to_f32(r.x >> 16) + x[1],
                         bf16_to_f32(r.y & 0xFFFF) + x[2], bf16_to_f32(r.y >> 16) + x[3]);
        }
        *reinterpret_cast<uint2*>(static_cast<uint16_t*>(a.out_res) + static_cast<size_t>(gm) * a.N + n) = o;
      }
    } else {  // EPI_QKV
      const int b = blk[0];
      const int nq = a.Hq * 8, nk = a.Hkv * 8;
      if (b < nq + nk) {
        // q or k block: rows i < 8 are dims 8j+i, rows 8+i their RoPE partners 64+8j+i
        const int bb = b < nq ? b : b - nq;
        const int head = bb >> 3, j8 = (bb & 7) * 8;
        for (int it = lt; it < 128; it += S * 64) {
          const int m = it & 63, i0 = (it >> 6) * 4;
          const int gm = m0 + m;
          if (gm >= a.M) continue;
          const int sq = gm / a.n_rows;
          int pos = static_cast<int>(a.kv_offsets[sq + 1] - a.kv_offsets[sq]) + a.depth[gm];
          if (pos > a.n_pos - 1) pos = a.n_pos - 1;
          float lo[4], hi[4];
#pragma unroll
          for (int v = 0; v < 4; ++v) {
            const int d = j8 + i0 + v;
            const float c = a.rope_cos[static_cast<size_t>(pos) * 64 + d];
            const float sn = a.rope_sin[static_cast<size_t>(pos) * 64 + d];
            const float x1 = sumq(i0 + v, m), x2 = sumq(8 + i0 + v, m);
            lo[v] = x1 * c - x2 * sn;
            hi[v] = x2 * c + x1 * sn;
          }
          uint16_t* op = b < nq ? static_cast<uint16_t*>(a.q_out) + static_cast<size_t>(gm) * a.Hq * 128
                                : static_cast<uint16_t*>(a.k_out) + static_cast<size_t>(gm) * a.Hkv * 128;
          op += head * 128 + j8 + i0;
          *reinterpret_cast<uint2*>(op) = pack4_bf16(lo[0], lo[1], lo[2], lo[3]);
          *reinterpret_cast<uint2*>(op + 64) = pack4_bf16(hi[0], hi[1], hi[2], hi[3]);
        }
      } else {
        const int vr = (b - nq - nk) * 16;  // first v row of the block
        for (int it = lt; it < 256; it += S * 64) {
          const int m = it & 63, i0 = (it >> 6) * 4;
          const int gm = m0 + m;
          if (gm >= a.M) continue;
          uint16_t* op = static_cast<uint16_t*>(a.v_out) + static_cast<size_t>(gm) * a.Hkv * 128 + vr + i0;
          *reinterpret_cast<uint2*>(op) = pack4_bf16(sumq(i0, m), sumq(i0 + 1, m), sumq(i0 + 2, m), sumq(i0 + 3, m));
        }
      }
    }
  }
}

__global__ __launch_bounds__(256) void head_merge_kernel(const float* __restrict__ part, int nNT,
                                                         int32_t* __restrict__ argmax,
                                                         float* __restrict__ top1,
                                                         float* __restrict__ gap,
                                                         float* __restrict__ entropy) {
  __shared__ HeadPart red[256];
  const int r = blockIdx.x, tid = threadIdx.x;
  HeadPart p = head_empty();
  for (int t = tid; t < nNT; t += 256) {
    const float* q = part + (static_cast<size_t>(r) * nNT + t) * 5;
    HeadPart e;
    e.m = q[0];
    e.am = __float_as_int(q[1]);
    e.m2 = q[2];
    e.s = q[3];
    e.t = q[4];
    p = head_combine(p, e);
  }
  red[tid] = p;
  __syncthreads();
  for (int st = 128; st > 0; st >>= 1) {
    if (tid < st) red[tid] = head_combine(red[tid], red[tid + st]);
    __syncthreads();
  }
  if (tid == 0) {
    const HeadPart f = red[0];
    argmax[r] = f.am;
    top1[r] = f.m;
    gap[r] = f.m - f.m2;
    entropy[r] = logf(f.s) - f.t / f.s;
  }
}

// ------------------------------------------------------------ fp32 path
// Plain fp32 kernels for the fp32 workloads (tiny shapes): one thread per output,
// sequential k loop.
__global__ __launch_bounds__(64) void gemm_f32_kernel(GemmArgs a) {
  const int n = blockIdx.x * 64 + threadIdx.x, m = blockIdx.y;
  if (n >= a.N) return;
  const float* xrow = nullptr;
  if (a.gather) {
    const int tok = a.gather[m];
    if (tok >= 0) xrow = static_cast<const float*>(a.x) + static_cast<size_t>(tok) * a.K;
  } else {
    xrow = static_cast<const float*>(a.x) + static_cast<size_t>(m) * a.K;
  }
  int start = 0, sidx = 0;
  while (sidx < a.w.nseg - 1 && n >= a.w.n_end[sidx]) start = a.w.n_end[sidx++];
  const float* wrow = static_cast<const float*>(a.w.w[sidx]) + static_cast<size_t>(n - start) * a.K;
  float acc = 0.f;
  if (xrow)
    for (int k = 0; k < a.K; ++k) acc = fmaf(xrow[k], wrow[k], acc);
  const size_t o = static_cast<size_t>(m) * a.N + n;
  if (a.epi == EPI_STORE_F32) {
    a.out_f32[o] = acc;
  } else if (a.epi == EPI_RESID) {
    const float* rp = nullptr;
    const int tok = a.resid_tok[m];
    if (tok >= 0)
      rp = static_cast<const float*>(a.resid) + static_cast<size_t>(a.resid_by_token ? tok : m) * a.N;
    static_cast<float*>(a.out_res)[o] = rp ? rp[n] + acc : 0.f;
  } else {
    a.logits[o] = acc;
  }
}

__global__ __launch_bounds__(256) void head_rowstats_f32_kernel(const float* __restrict__ logits,
                                                                int V, int32_t* __restrict__ argmax,
                                                                float* __restrict__ top1,
                                                                float* __restrict__ gap,
                                                                float* __restrict__ entropy) {
  __shared__ HeadPart red[256];
  const int r = blockIdx.x, tid = threadIdx.x;
  const float* z = logits + static_cast<size_t>(r) * V;
  HeadPart p = head_empty();
  for (int n = tid; n < V; n += 256) p = head_combine(p, head_elem(z[n], n));
  red[tid] = p;
  __syncthreads();
  for (int st = 128; st > 0; st >>= 1) {
    if (tid < st) red[tid] = head_combine(red[tid], red[tid + st]);
    __syncthreads();
  }
  if (tid == 0) {
    const HeadPart f = red[0];
    argmax[r] = f.am;
    top1[r] = f.m;
    gap[r] = f.m - f.m2;
    entropy[r] = logf(f.s) - f.t / f.s;
  }
}

}  // namespace

namespace {
constexpr int kHeadB = 5;      // weight blocks per wave in the LM head
constexpr int kHeadWaves = 2048;  // waves the LM head grid aims for (256 CUs x 8)

struct HeadGrid {
  int NB, NG, nWG;
};
HeadGrid head_grid(int N) {
  HeadGrid g;
  g.NB = (N + 15) / 16;
  int ng = g.NB < kHeadWaves ? g.NB : kHeadWaves;
  const int need = (g.NB + kHeadB - 1) / kHeadB;
  if (ng < need) ng = need;
  g.NG = ng;
  g.nWG = (ng + 3) / 4;
  return g;
}
}  // namespace

int gemm_bf16_head_parts(int N) { return head_grid(N).nWG; }

glance_status launch_gemm_bf16(const GemmArgs& a, hipStream_t st) {
  const int nMT = (a.M + kTileM - 1) / kTileM;
  if (a.epi == EPI_HEAD) {
    const HeadGrid g = head_grid(a.N);
    const int grid = ((g.nWG + 7) / 8) * 8 * nMT;
    gemm_bf16_kernel<EPI_HEAD, kHeadB, 1, 1><<<grid, kGThreads, 0, st>>>(a, g.NB, g.NG, g.nWG, nMT);
  } else {
    // one 16-row block per work-group, its K split over the 4 waves
    int NB;
    if (a.epi == EPI_QKV)
      NB = (a.Hq + 2 * a.Hkv) * 8;
    else
      NB = (a.N + 15) / 16;
    const int nWG = NB;
    const int grid = ((nWG + 7) / 8) * 8 * nMT;
    if (a.epi == EPI_QKV)
      gemm_bf16_kernel<EPI_QKV, 1, 4, 3><<<grid, kGThreads, 0, st>>>(a, NB, NB, nWG, nMT);
    else
      gemm_bf16_kernel<EPI_RESID, 1, 4, 3><<<grid, kGThreads, 0, st>>>(a, NB, NB, nWG, nMT);
  }
  GLANCE_LAUNCH_CHECK();
  return GLANCE_OK;
}

glance_status launch_gemm_f32(const GemmArgs& a, hipStream_t st) {
  dim3 grid((a.N + 63) / 64, a.M);
  gemm_f32_kernel<<<grid, 64, 0, st>>>(a);
  GLANCE_LAUNCH_CHECK();
  return GLANCE_OK;
}

glance_status launch_head_merge(const float* part, int n_tiles, int R, int32_t* argmax,
                                float* top1, float* gap, float* entropy, hipStream_t st) {
  head_merge_kernel<<<R, 256, 0, st>>>(part, n_tiles, argmax, top1, gap, entropy);
  GLANCE_LAUNCH_CHECK();
  return GLANCE_OK;
}

glance_status launch_head_rowstats_f32(const float* logits, int R, int V, int32_t* argmax,
                                       float* top1, float* gap, float* entropy,
                                       hipStream_t st) {
  head_rowstats_f32_kernel<<<R, 256, 0, st>>>(logits, V, argmax, top1, gap, entropy);
  GLANCE_LAUNCH_CHECK();
  return GLANCE_OK;
}

}  // namespace glance
