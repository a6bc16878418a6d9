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
#include <mutex>
#include <type_traits>

#include "common.h"
#include "kernels.h"
#include "walk_impl.h"

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

// Philox4x32-10 (Salmon et al., SC 2011): round (c0, c1, c2, c3) ->
// (hi(M1 c2) ^ c1 ^ k0, lo(M1 c2), hi(M0 c0) ^ c3 ^ k1, lo(M0 c0)); the key
// grows by the Weyl increments before every round but the first.
__device__ __forceinline__ uint4 philox4x32_10(uint4 c, uint32_t k0, uint32_t k1) {
#pragma unroll
  for (int r = 0; r < 10; ++r) {
    if (r > 0) {
      k0 += 0x9E3779B9u;
      k1 += 0xBB67AE85u;
    }
    const uint32_t hi0 = __umulhi(0xD2511F53u, c.x), lo0 = 0xD2511F53u * c.x;
    const uint32_t hi1 = __umulhi(0xCD9E8D57u, c.z), lo1 = 0xCD9E8D57u * c.z;
    c = make_uint4(hi1 ^ c.y ^ k0, lo1, hi0 ^ c.w ^ k1, lo0);
  }
  return c;
}

// Gumbel noise -ln(-ln U) from a Philox word: U = (top 23 bits + 1/2) / 2^23.
// Its numerator has at most 24 bits, so U is exact in float32 and never 0 or 1;
// a finer grid would round near 1, where the winning draws' 1 - U lives.
__device__ __forceinline__ float gumbel(uint32_t x) {
  const float u = (static_cast<float>(x >> 9) + 0.5f) * (1.0f / 8388608.0f);
  return -logf(-logf(u));
}

// A partial draw: the best perturbed score, its token (smallest on ties) and the
// best score of any other token.
struct Draw {
  float m;
  int tok;
  float m2;
};
__device__ __forceinline__ Draw draw_empty() { return Draw{-INFINITY, 0x7FFFFFFF, -INFINITY}; }
__device__ __forceinline__ Draw draw_combine(Draw a, Draw b) {
  if (b.m > a.m || (b.m == a.m && b.tok < a.tok)) {
    const Draw t = a;
    a = b;
    b = t;
  }
  return Draw{a.m, a.tok, fmaxf(a.m2, b.m)};
}
__device__ __forceinline__ Draw shfl_draw(const Draw& d, int src) {
  return Draw{__shfl(d.m, src, kWave), __shfl(d.tok, src, kWave), __shfl(d.m2, src, kWave)};
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


// Activation row m of X (a gathered embedding row when a.gather is set).  Rows
// past M and gathered rows with token < 0 are zero: they get row 0's address
// (always valid) and a zero mask, so their loads need no branch.
__device__ __forceinline__ void x_row_masked(const GemmArgs& a, int m, const uint16_t*& p,
                                             uint32_t& mask) {
  int row = m;
  bool ok = m < a.M;
  if (ok && a.gather) {
    row = a.gather[m];
    ok = row >= 0;
  }
  if (!ok) row = 0;
  p = static_cast<const uint16_t*>(a.x) + static_cast<size_t>(row) * a.K;
  mask = ok ? 0xFFFFFFFFu : 0u;
}

__device__ __forceinline__ uint4 mask4(uint4 v, uint32_t mask) {
  return make_uint4(v.x & mask, v.y & mask, v.z & mask, v.w & mask);
}

// W row of row i (0..15) of block b.  For EPI_QKV the q and k blocks pair head
// dims so that rows i and i+8 are RoPE partners: block j of a head holds dims
// 8j..8j+7 and 64+8j..64+8j+7.
template <int EPI>
__device__ __forceinline__ int block_row(const GemmArgs& a, int b, int i) {
  if constexpr (EPI == EPI_SWIGLU) {
    // rows i < 8: gate rows 8b + i; rows 8 + i: the matching up rows
    return i < 8 ? 8 * b + i : a.N / 2 + 8 * b + (i - 8);
  } else if constexpr (EPI == EPI_QKV || EPI == EPI_STORE_F32) {
    // q and k blocks pair head dims 8j + i with their RoPE partners 64 + 8j + i
    // (the fp32 store of full layers keeps the same order, so that one packed
    // copy of the weights serves both)
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

// Row statistics of one lane's logits acc[t][mb][v] (vocabulary row
// blk[t]*16 + 4 lg + v, activation row 16 mb + l%16): per activation row the max,
// its smallest token id and the best other logit in one select-only pass (rows
// are visited in increasing token order, so a strict comparison keeps the
// smallest id), then the two sums relative to that max through the hardware
// exp2.  EDGE: some rows are past the vocabulary; they enter as -inf and d is
// kept finite so that e * d is 0 for them (e = 0).
template <int B, bool EDGE>
__device__ __forceinline__ void head_row_stats(const f32x4 (&acc)[B][4], const int (&blk)[B],
                                               const bool (&bval)[B], int lg, int N, HeadPart (&hp)[4]) {
  bool nval[B][4];
#pragma unroll
  for (int t = 0; t < B; ++t)
#pragma unroll
    for (int v = 0; v < 4; ++v) nval[t][v] = !EDGE || (bval[t] & (blk[t] * 16 + 4 * lg + v < N));
#pragma unroll
  for (int mb = 0; mb < 4; ++mb) {
    float mx = -INFINITY, m2 = -INFINITY;
    int am = 0x7FFFFFFF;
#pragma unroll
    for (int t = 0; t < B; ++t)
#pragma unroll
      for (int v = 0; v < 4; ++v) {
        const float z = nval[t][v] ? acc[t][mb][v] : -INFINITY;
        const bool gt = z > mx;
        m2 = gt ? mx : fmaxf(m2, z);
        am = gt ? blk[t] * 16 + 4 * lg + v : am;
        mx = fmaxf(mx, z);
      }
    const float ms = EDGE && mx == -INFINITY ? 0.f : mx;
    float sum = 0.f, tsum = 0.f;
#pragma unroll
    for (int t = 0; t < B; ++t)
#pragma unroll
      for (int v = 0; v < 4; ++v) {
        const float z = nval[t][v] ? acc[t][mb][v] : -INFINITY;
        const float d = EDGE ? fmaxf(z - ms, -1e30f) : z - ms;
        const float e = __builtin_amdgcn_exp2f(d * 1.4426950408889634f);
        sum += e;
        tsum = fmaf(e, d, tsum);
      }
    hp[mb].m = mx;
    hp[mb].am = am;
    hp[mb].m2 = m2;
    hp[mb].s = sum;
    hp[mb].t = tsum;
  }
}

// ------------------------------------------------------------------ LM head
// Work-group = 4 waves over one 64-row activation tile; wave G owns blocks
// G, G + NG, ... (B of them).  Each weight chunk (64 deep) of a block is loaded
// with two full-line non-temporal loads (rows 8 i + l/8, k = 8 (l%8)), written
// to the wave's own LDS tile and read back in the MFMA operand layout (row
// l%16, k = 32 s + 8 (l/16)).  Same-wave LDS accesses complete in order, so the
// tile needs no barrier.  The activation chunks are staged in LDS for all
// waves in a ring of 2 SB one-chunk stages: SB chunks are computed between two
// barriers while the next SB chunks are loaded and written to the other half,
// so the waves meet once per SB chunks (a barrier per chunk costs several
// percent of the weight stream: the waves wait for the slowest one's loads).
// LDS rows are 128 bytes, unpadded, with the 16-byte unit XOR-swizzled by the
// row's low 3 bits against bank conflicts.  The weights of chunk c + 1 are
// loaded into a second register slot while chunk c is computed.
//
// PACKED: W was reordered once into the head's own tile order (head_pack_kernel):
// for chunk c, wave G, its t-th block (t < per) and half s, 1 KB holding lane l's
// 16 bytes of the MFMA operand (row l%16, k = 64 c + 32 s + 8 (l/16)) at l * 16.
// The weights then go from HBM straight into MFMA operands: no LDS tile, every
// load a contiguous kilobyte, and all waves of chunk c read one contiguous band.
// The freed LDS deepens the activation ring (the waves meet less often).
__device__ __forceinline__ int swz(int row, int unit) { return row * kKc + 8 * (unit ^ (row & 7)); }

// MT > 1 (packed weights only): each work-group applies every weight chunk to
// MT tiles of 64 activation rows (nMT counts groups of MT tiles), so that rows
// past the first 64 re-use the weights from registers instead of re-reading
// them through the caches.
template <int B, int SB, bool SAMPLE, bool PACKED, int MT = 1>
__global__ __launch_bounds__(kGThreads, MT == 1 ? 2 : 1) void head_bf16_kernel(GemmArgs a, int NB, int NG,
                                                                              int nWG, int nMT, int per) {
  static_assert(MT == 1 || (PACKED && MT == 2), "two activation tiles per work-group, packed weights only");
  constexpr int XST = kTileM * kKc;  // one activation stage (elements)
  __shared__ __attribute__((aligned(16))) uint16_t xs[2 * SB * XST * MT];
  __shared__ __attribute__((aligned(16))) uint16_t wtile[PACKED ? 8 : 4 * B * 16 * kKc];
  __shared__ HeadPart hred[4][kTileM];

  const int bid = blockIdx.x;
  const int xcd = bid & 7, kk = bid >> 3;
  const int mt = kk % nMT;
  const int wg = (kk / nMT) * 8 + xcd;
  if (wg >= nWG) return;
  const int m0 = mt * MT * kTileM;
  const int tid = threadIdx.x, w = tid >> 6, l = tid & 63, lr = l & 15, lg = l >> 4;
  const int G = wg * 4 + w;
  const int nck = a.K / kKc;
  uint16_t* wt = PACKED ? wtile : wtile + w * B * 16 * kKc;

  int blk[B];
  bool bval[B];
  const uint16_t* wp[B][2];
  // packed: one base per lane (the wave's first tile), wave-uniform tile offsets;
  // consecutive chunks of a tile are a band (NG per tiles) apart.  Waves and
  // blocks past the grid re-read a valid tile (their results are never stored).
  const uint4* wq0 = nullptr;
  int toff[B];
  const size_t cstride = static_cast<size_t>(NG) * per * 128;
  if constexpr (PACKED) {
    const int gc = G < NG ? G : NG - 1;
    wq0 = static_cast<const uint4*>(a.w_packed) + static_cast<size_t>(gc) * per * 128 + l;
  }
#pragma unroll
  for (int t = 0; t < B; ++t) {
    blk[t] = G + t * NG;
    bval[t] = G < NG && blk[t] < NB;
    toff[t] = (t < per ? t : per - 1) * 128;
#pragma unroll
    for (int i = 0; i < 2; ++i) {
      if constexpr (PACKED) {
        wp[t][i] = nullptr;
      } else {
        int row = bval[t] ? blk[t] * 16 + 8 * i + (l >> 3) : 0;
        if (row > a.N - 1) row = a.N - 1;
        wp[t][i] = w_row_ptr(a, row) + 8 * (l & 7);
      }
    }
  }
  // activation pieces this thread stages: 64 rows x 8 units of 16 B per chunk.
  // Rows past M read row 0 unmasked: their results are never stored.
  // (tile mm of MT: rows m0 + 64 mm ..; stage st of tile mm at (st * MT + mm) * XST)
  const uint16_t* xr[MT][2];
  int xlds[2];
#pragma unroll
  for (int e = 0; e < 2; ++e) {
    const int idx = e * kGThreads + tid;
    const int r = idx >> 3, cc = idx & 7;
#pragma unroll
    for (int mm = 0; mm < MT; ++mm) {
      const int rr = m0 + mm * kTileM + r;
      const int row = rr < a.M ? rr : 0;
      xr[mm][e] = static_cast<const uint16_t*>(a.x) + static_cast<size_t>(row) * a.K + 8 * cc;
    }
    xlds[e] = swz(r, cc);
  }

  f32x4 acc[MT][B][4];
#pragma unroll
  for (int mm = 0; mm < MT; ++mm)
#pragma unroll
    for (int t = 0; t < B; ++t)
#pragma unroll
      for (int mb = 0; mb < 4; ++mb) acc[mm][t][mb] = f32x4{0.f, 0.f, 0.f, 0.f};
  uint4 wbuf[2][B][2];
  uint4 xb[SB][MT][2];
  auto wload = [&](int c, uint4 (&dst)[B][2]) {
#pragma unroll
    for (int t = 0; t < B; ++t)
#pragma unroll
      for (int i = 0; i < 2; ++i) {
        if constexpr (PACKED)
          dst[t][i] = load_stream(wq0 + (c * cstride + toff[t] + i * 64));
        else
          dst[t][i] = load_stream(wp[t][i] + c * kKc);
      }
  };
  auto xload = [&](int c, uint4 (&dst)[MT][2]) {
#pragma unroll
    for (int mm = 0; mm < MT; ++mm)
#pragma unroll
      for (int e = 0; e < 2; ++e) dst[mm][e] = *reinterpret_cast<const uint4*>(xr[mm][e] + c * kKc);
  };
  auto xstore = [&](int stage, const uint4 (&src)[MT][2]) {
#pragma unroll
    for (int mm = 0; mm < MT; ++mm)
#pragma unroll
      for (int e = 0; e < 2; ++e) *reinterpret_cast<uint4*>(&xs[(stage * MT + mm) * XST + xlds[e]]) = src[mm][e];
  };

  // nck is a multiple of SB; loads past the last chunk are clamped to it, so no
  // load is conditional (a conditional load would make the compiler's wait
  // counts conservative and drain the loads in flight)
#pragma unroll
  for (int j = 0; j < SB; ++j) xload(j, xb[j]);
#pragma unroll
  for (int j = 0; j < SB; ++j) xstore(j, xb[j]);
  wload(0, wbuf[0]);
  __syncthreads();
  if constexpr (PACKED) {
    static_assert(SB == 2, "the packed head computes two chunks per stage half");
  // packed: the same schedule written out with named registers (no lambdas or
  // arrays for the activation stage, which the compiler would otherwise keep in
  // scratch memory).  An empty asm statement with a memory clobber after each
  // chunk's weight loads keeps the scheduler from sinking them to their use
  // (the loaded registers feed the matrix cores directly).  The next stage
  // half was last read before the previous barrier, so it is written between
  // the two chunks and its registers live across one chunk only.
#define GLANCE_PACKED_CHUNK(U)                                                              \
  {                                                                                         \
    const int cn = min(c0 + (U) + 1, nck - 1);                                              \
    _Pragma("unroll") for (int t = 0; t < B; ++t)                                           \
      _Pragma("unroll") for (int i = 0; i < 2; ++i)                                         \
        wbuf[((U) + 1) & 1][t][i] = load_stream(wq0 + (cn * cstride + toff[t] + i * 64));   \
    asm volatile("" ::: "memory");                                                          \
    _Pragma("unroll") for (int mm = 0; mm < MT; ++mm) {                                     \
      const uint16_t* xq = xs + ((half * 2 + (U)) * MT + mm) * XST;                         \
      _Pragma("unroll") for (int s = 0; s < 2; ++s) {                                       \
        bf16x8 bx[4];                                                                       \
        _Pragma("unroll") for (int mb = 0; mb < 4; ++mb) bx[mb] =                           \
            *reinterpret_cast<const bf16x8*>(xq + swz(mb * 16 + lr, 4 * s + lg));           \
        _Pragma("unroll") for (int t = 0; t < B; ++t) {                                     \
          const bf16x8 av = __builtin_bit_cast(bf16x8, wbuf[(U) & 1][t][s]);                \
          _Pragma("unroll") for (int mb = 0; mb < 4; ++mb) acc[mm][t][mb] =                 \
              __builtin_amdgcn_mfma_f32_16x16x32_bf16(av, bx[mb], acc[mm][t][mb], 0, 0, 0); \
        }                                                                                   \
      }                                                                                     \
    }                                                                                       \
  }
  for (int c0 = 0; c0 < nck; c0 += 2) {
    const int half = (c0 / 2) & 1;
    const int ca = min(c0 + 2, nck - 1), cb = min(c0 + 3, nck - 1);
    // named registers (tile 0: x*, tile 1: y*), no arrays: see above
    const uint4 xa0 = *reinterpret_cast<const uint4*>(xr[0][0] + ca * kKc);
    const uint4 xa1 = *reinterpret_cast<const uint4*>(xr[0][1] + ca * kKc);
    const uint4 xb0 = *reinterpret_cast<const uint4*>(xr[0][0] + cb * kKc);
    const uint4 xb1 = *reinterpret_cast<const uint4*>(xr[0][1] + cb * kKc);
    uint4 ya0, ya1, yb0, yb1;
    if constexpr (MT == 2) {
      ya0 = *reinterpret_cast<const uint4*>(xr[MT - 1][0] + ca * kKc);
      ya1 = *reinterpret_cast<const uint4*>(xr[MT - 1][1] + ca * kKc);
      yb0 = *reinterpret_cast<const uint4*>(xr[MT - 1][0] + cb * kKc);
      yb1 = *reinterpret_cast<const uint4*>(xr[MT - 1][1] + cb * kKc);
    }
    GLANCE_PACKED_CHUNK(0)
    *reinterpret_cast<uint4*>(&xs[(((half ^ 1) * 2) * MT) * XST + xlds[0]]) = xa0;
    *reinterpret_cast<uint4*>(&xs[(((half ^ 1) * 2) * MT) * XST + xlds[1]]) = xa1;
    *reinterpret_cast<uint4*>(&xs[(((half ^ 1) * 2 + 1) * MT) * XST + xlds[0]]) = xb0;
    *reinterpret_cast<uint4*>(&xs[(((half ^ 1) * 2 + 1) * MT) * XST + xlds[1]]) = xb1;
    if constexpr (MT == 2) {
      *reinterpret_cast<uint4*>(&xs[(((half ^ 1) * 2) * MT + 1) * XST + xlds[0]]) = ya0;
      *reinterpret_cast<uint4*>(&xs[(((half ^ 1) * 2) * MT + 1) * XST + xlds[1]]) = ya1;
      *reinterpret_cast<uint4*>(&xs[(((half ^ 1) * 2 + 1) * MT + 1) * XST + xlds[0]]) = yb0;
      *reinterpret_cast<uint4*>(&xs[(((half ^ 1) * 2 + 1) * MT + 1) * XST + xlds[1]]) = yb1;
    }
    GLANCE_PACKED_CHUNK(1)
    __syncthreads();
  }
#undef GLANCE_PACKED_CHUNK
  } else {
  for (int c0 = 0; c0 < nck; c0 += SB) {
    const int half = (c0 / SB) & 1;  // stage half holding chunks c0 .. c0 + SB - 1
#pragma unroll
    for (int j = 0; j < SB; ++j) xload(min(c0 + SB + j, nck - 1), xb[j]);
#pragma unroll
    for (int u = 0; u < SB; ++u) {
      const int c = c0 + u;
      wload(min(c + 1, nck - 1), wbuf[(u + 1) & 1]);
#pragma unroll
      for (int t = 0; t < B; ++t)
#pragma unroll
        for (int i = 0; i < 2; ++i)
          *reinterpret_cast<uint4*>(wt + swz(t * 16 + 8 * i + (l >> 3), l & 7)) = wbuf[u & 1][t][i];
      const uint16_t* xq = xs + (half * SB + u) * XST;
#pragma unroll
      for (int s = 0; s < 2; ++s) {
        bf16x8 bx[4];
#pragma unroll
        for (int mb = 0; mb < 4; ++mb) bx[mb] = *reinterpret_cast<const bf16x8*>(xq + swz(mb * 16 + lr, 4 * s + lg));
#pragma unroll
        for (int t = 0; t < B; ++t) {
          const bf16x8 av = *reinterpret_cast<const bf16x8*>(wt + swz(t * 16 + lr, 4 * s + lg));
#pragma unroll
          for (int mb = 0; mb < 4; ++mb)
            acc[0][t][mb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(av, bx[mb], acc[0][t][mb], 0, 0, 0);
        }
      }
    }
    // the next SB chunks go to the other half, whose last reads came before the
    // previous barrier (after the last chunk these are clamped copies nobody reads)
#pragma unroll
    for (int j = 0; j < SB; ++j) xstore((half ^ 1) * SB + j, xb[j]);
    __syncthreads();
  }
  }

  // per activation tile: the statistics of its 64 rows (the LDS reduction
  // buffers are reused tile after tile); the tile index is a compile-time
  // constant so that the accumulators stay in registers
  auto epilogue = [&](auto mmc) {
    constexpr int mm = decltype(mmc)::value;
    const int mt0 = m0 + mm * kTileM;
    // acc[mm][t][mb][v]: vocabulary row blk[t]*16 + 4 lg + v, activation row mt0 + 16 mb + lr.
    HeadPart hp[4];
    if (bval[B - 1] && blk[B - 1] * 16 + 16 <= a.N)  // (wave-uniform) every row of the wave exists
      head_row_stats<B, false>(acc[mm], blk, bval, lg, a.N, hp);
    else
      head_row_stats<B, true>(acc[mm], blk, bval, lg, a.N, hp);
    if (a.logits) {
  #pragma unroll
      for (int t = 0; t < B; ++t)
  #pragma unroll
        for (int v = 0; v < 4; ++v) {
          const int n = blk[t] * 16 + 4 * lg + v;
          if (bval[t] && n < a.N) {
  #pragma unroll
            for (int mb = 0; mb < 4; ++mb) {
              const int m = mt0 + mb * 16 + lr;
              if (m < a.M) a.logits[static_cast<size_t>(m) * a.N + n] = acc[mm][t][mb][v];
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
    if constexpr (SAMPLE) {
      // the draw of every activation row from softmax(z / T): Gumbel-max over this
      // lane's tokens (one Philox call gives the noise of 4 consecutive tokens),
      // then over lanes and waves as for the statistics
      __shared__ Draw dred[4][kTileM];
      Draw dp[4];
  #pragma unroll
      for (int mb = 0; mb < 4; ++mb) {
        dp[mb] = draw_empty();
        const uint32_t row = static_cast<uint32_t>(mt0 + mb * 16 + lr);
  #pragma unroll
        for (int t = 0; t < B; ++t) {
          const uint4 x = philox4x32_10(
              make_uint4(static_cast<uint32_t>(blk[t] * 4 + lg), row, a.rnd_lo, a.rnd_hi), a.seed_lo,
              a.seed_hi);
          const uint32_t xs4[4] = {x.x, x.y, x.z, x.w};
  #pragma unroll
          for (int v = 0; v < 4; ++v) {
            const int n = blk[t] * 16 + 4 * lg + v;
            const float sc = (bval[t] & (n < a.N)) ? fmaf(acc[mm][t][mb][v], a.inv_temp, gumbel(xs4[v])) : -INFINITY;
            const bool gt = sc > dp[mb].m;
            dp[mb].m2 = gt ? dp[mb].m : fmaxf(dp[mb].m2, sc);
            dp[mb].tok = gt ? n : dp[mb].tok;
            dp[mb].m = fmaxf(dp[mb].m, sc);
          }
        }
        dp[mb] = draw_combine(dp[mb], shfl_draw(dp[mb], l ^ 16));
        dp[mb] = draw_combine(dp[mb], shfl_draw(dp[mb], l ^ 32));
        if (lg == 0) dred[w][mb * 16 + lr] = dp[mb];
      }
      __syncthreads();
      if (tid < kTileM && mt0 + tid < a.M) {
        Draw d = dred[0][tid];
  #pragma unroll
        for (int ww = 1; ww < 4; ++ww) d = draw_combine(d, dred[ww][tid]);
        float* o = a.spart + (static_cast<size_t>(mt0 + tid) * nWG + wg) * 3;
        o[0] = d.m;
        o[1] = __int_as_float(d.tok);
        o[2] = d.m2;
      }
    }
    __syncthreads();
    if (tid < kTileM) {
      HeadPart p = hred[0][tid];
  #pragma unroll
      for (int ww = 1; ww < 4; ++ww) p = head_combine(p, hred[ww][tid]);
      const int m = mt0 + tid;
      if (m < a.M) {
        float* o = a.part + (static_cast<size_t>(m) * nWG + wg) * 5;
        o[0] = p.m;
        o[1] = __int_as_float(p.am);
        o[2] = p.m2;
        o[3] = p.s;
        o[4] = p.t;
      }
    }
  };
  epilogue(std::integral_constant<int, 0>{});
  if constexpr (MT == 2) {
    __syncthreads();
    epilogue(std::integral_constant<int, MT - 1>{});
  }
}

// -------------------------------------------------------------- projections
// What the epilogue of block b reads for activation row gm besides the sums,
// loaded ahead of the split-K hand-over: the q/k rows' RoPE position (or the
// output projection's residual token) at the start of the kernel, the RoPE
// values at that position (or the residual row) right after the K loop, so
// that they arrive while the partial sums are stored and counted.
struct EpiIn {
  int key;           // q/k: RoPE position, residual: token (-1: none / zero row)
  float c[8], sn[8];  // q/k: cos and sin of head dims j8 .. j8 + 7 at the position
  uint4 r[2];        // residual: the 16 residual values of the block
};

template <int EPI>
__device__ __forceinline__ int epi_key(const GemmArgs& a, int b, int gm) {
  if constexpr (EPI == EPI_QKV) {
    if (b >= (a.Hq + a.Hkv) * 8) return -1;
    const int sq = gm / a.n_rows;
    const int pos = static_cast<int>(a.kv_offsets[sq + 1] - a.kv_offsets[sq]) + a.depth[gm];
    return pos < 0 ? 0 : (pos > a.n_pos - 1 ? a.n_pos - 1 : pos);
  } else if constexpr (EPI == EPI_RESID) {
    return a.resid_tok[gm];
  } else {
    return -1;
  }
}

template <int EPI>
__device__ __forceinline__ void epi_load(const GemmArgs& a, int b, int gm, EpiIn& in) {
  if constexpr (EPI == EPI_QKV) {
    if (in.key >= 0) {
      const int nq = a.Hq * 8;
      const int j8 = ((b < nq ? b : b - nq) & 7) * 8;
      const float* cp = a.rope_cos + static_cast<size_t>(in.key) * 64 + j8;
      const float* sp = a.rope_sin + static_cast<size_t>(in.key) * 64 + j8;
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        in.c[i] = cp[i];
        in.sn[i] = sp[i];
      }
    }
  } else if constexpr (EPI == EPI_RESID) {
    if (in.key >= 0) {
      const uint16_t* rp = static_cast<const uint16_t*>(a.resid) +
                           static_cast<size_t>(a.resid_by_token ? in.key : gm) * a.N + b * 16;
      in.r[0] = *reinterpret_cast<const uint4*>(rp);
      in.r[1] = *reinterpret_cast<const uint4*>(rp + 8);
    }
  }
}

// Epilogue of one 16-row weight block for activation row gm: x[i] is the
// block's row i (of the summed K slices).  q/k blocks are rotated (rows i and
// 8+i are RoPE partners), v rows copied, output-projection rows added to the
// residual; everything is rounded to bf16.
template <int EPI>
__device__ __forceinline__ void proj_store(const GemmArgs& a, int b, int gm, const float (&x)[16],
                                           const EpiIn& in) {
  if constexpr (EPI == EPI_RESID) {
    const int n = b * 16;
    uint4 o[2] = {make_uint4(0, 0, 0, 0), make_uint4(0, 0, 0, 0)};
    if (in.key >= 0) {
#pragma unroll
      for (int h = 0; h < 2; ++h) {
        const uint4 r = in.r[h];
        const uint32_t rw[4] = {r.x, r.y, r.z, r.w};
        uint32_t ow[4];
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          const float lo = bf16_to_f32(rw[j] & 0xFFFF) + x[8 * h + 2 * j];
          const float hi = bf16_to_f32(rw[j] >> 16) + x[8 * h + 2 * j + 1];
          ow[j] = static_cast<uint32_t>(f32_to_bf16(lo)) | (static_cast<uint32_t>(f32_to_bf16(hi)) << 16);
        }
        o[h] = make_uint4(ow[0], ow[1], ow[2], ow[3]);
      }
    }
    uint4* op = reinterpret_cast<uint4*>(static_cast<uint16_t*>(a.out_res) + static_cast<size_t>(gm) * a.N + n);
    op[0] = o[0];
    op[1] = o[1];
  } else if constexpr (EPI == EPI_STORE_F32) {
    // rows i < 8 and 8 + i are two runs of 8 columns (block_row)
    float* orow = a.out_f32 + static_cast<size_t>(gm) * a.N;
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      float4* op = reinterpret_cast<float4*>(orow + block_row<EPI>(a, b, 8 * h));
      op[0] = make_float4(x[8 * h], x[8 * h + 1], x[8 * h + 2], x[8 * h + 3]);
      op[1] = make_float4(x[8 * h + 4], x[8 * h + 5], x[8 * h + 6], x[8 * h + 7]);
    }
  } else if constexpr (EPI == EPI_SWIGLU) {
    // x[i] the gate and x[8 + i] the up projection of intermediate unit 8b + i
    uint32_t ow[4];
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const float g0 = x[2 * j], g1 = x[2 * j + 1];
      const float v0 = g0 / (1.f + expf(-g0)) * x[8 + 2 * j];
      const float v1 = g1 / (1.f + expf(-g1)) * x[8 + 2 * j + 1];
      ow[j] = pack_bf16x2(v0, v1);
    }
    *reinterpret_cast<uint4*>(static_cast<uint16_t*>(a.out_res) + static_cast<size_t>(gm) * (a.N / 2) + 8 * b) =
        make_uint4(ow[0], ow[1], ow[2], ow[3]);
  } else {  // EPI_QKV
    const int nq = a.Hq * 8, nk = a.Hkv * 8;
    if (b < nq + nk) {
      // rows i < 8 are head dims 8j + i, rows 8 + i their RoPE partners 64 + 8j + i
      const int bb = b < nq ? b : b - nq;
      const int head = bb >> 3, j8 = (bb & 7) * 8;
      // lw/hw: the rotated pair rounded to bf16; lr/hr (q only): what the
      // rounding left out, rounded to bf16 (q enters the scores as the sum)
      uint32_t lw[4], hw[4], lr[4], hr[4];
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        float lo[2], hi[2];
#pragma unroll
        for (int h = 0; h < 2; ++h) {
          const int i = 2 * j + h;
          const float c = in.c[i];
          const float sn = in.sn[i];
          lo[h] = x[i] * c - x[i + 8] * sn;
          hi[h] = x[i + 8] * c + x[i] * sn;
        }
        lw[j] = static_cast<uint32_t>(f32_to_bf16(lo[0])) | (static_cast<uint32_t>(f32_to_bf16(lo[1])) << 16);
        hw[j] = static_cast<uint32_t>(f32_to_bf16(hi[0])) | (static_cast<uint32_t>(f32_to_bf16(hi[1])) << 16);
        lr[j] = pack_bf16x2(lo[0] - __uint_as_float(lw[j] << 16), lo[1] - __uint_as_float(lw[j] & 0xFFFF0000u));
        hr[j] = pack_bf16x2(hi[0] - __uint_as_float(hw[j] << 16), hi[1] - __uint_as_float(hw[j] & 0xFFFF0000u));
      }
      const size_t ro = b < nq ? static_cast<size_t>(gm) * a.Hq * 128 + head * 128 + j8
                               : static_cast<size_t>(gm) * a.Hkv * 128 + head * 128 + j8;
      uint16_t* op = (b < nq ? static_cast<uint16_t*>(a.q_out) : static_cast<uint16_t*>(a.k_out)) + ro;
      *reinterpret_cast<uint4*>(op) = make_uint4(lw[0], lw[1], lw[2], lw[3]);
      *reinterpret_cast<uint4*>(op + 64) = make_uint4(hw[0], hw[1], hw[2], hw[3]);
      if (b < nq) {
        uint16_t* rp = static_cast<uint16_t*>(a.q_lo_out) + ro;
        *reinterpret_cast<uint4*>(rp) = make_uint4(lr[0], lr[1], lr[2], lr[3]);
        *reinterpret_cast<uint4*>(rp + 64) = make_uint4(hr[0], hr[1], hr[2], hr[3]);
      }
    } else {
      const int vr = (b - nq - nk) * 16;  // first v dim of the block
      uint32_t ow[8];
#pragma unroll
      for (int j = 0; j < 8; ++j)
        ow[j] = static_cast<uint32_t>(f32_to_bf16(x[2 * j])) | (static_cast<uint32_t>(f32_to_bf16(x[2 * j + 1])) << 16);
      uint4* op = reinterpret_cast<uint4*>(static_cast<uint16_t*>(a.v_out) + static_cast<size_t>(gm) * a.Hkv * 128 + vr);
      op[0] = make_uint4(ow[0], ow[1], ow[2], ow[3]);
      op[1] = make_uint4(ow[4], ow[5], ow[6], ow[7]);
    }
  }
}

// Split-K in one kernel: work-group (group g, slice q, tile mt) computes blocks
// 4g .. 4g+3 (one per wave, MFMA-layout weight loads) over the K-slice q of S
// and stores the fp32 partial; the activation chunk in LDS is shared by the four
// blocks, so the activations are read once per 64 weight rows.  The last of the
// group's S work-groups to finish sums the partials, one thread per (block,
// activation row), and applies the epilogue.  The S x nMT work-groups of a
// group are dealt to the same XCD.
//
// XF: the activations are fp32 (the attention output) and enter as two bf16
// matrices, their rounding and the rounded remainder, each chunk staged as both
// and multiplied by the same weight operand (two products per step): the
// output projection then sees its input to ~16 significant bits.
//
// KW = 2: eight waves, the four blocks times two halves of the slice, each half
// staging its own activation chunks; the halves' sums meet in LDS before the
// epilogue (two waves per SIMD at one work-group per CU, no more partials).
//
// MT > 1 (more than 64 activation rows, K split over work-groups, four waves):
// each work-group applies its weight stream to MT tiles of 64 rows (nMT then
// counts groups of MT tiles), so the weights are loaded once for MT tiles.
template <int EPI, int DEPTH, bool XF, int KW, int MT = 1>
__global__ __launch_bounds__(kGThreads * KW, (XF || DEPTH > 7 || KW > 1 || MT > 2) ? 1 : 2) void proj_bf16_kernel(
    GemmArgs a, int NB, int NGr, int S, int nMT, int bpg) {
  static_assert(MT == 1 || KW == 1, "activation tiles per work-group with one wave group per slice");
  constexpr int NX = XF ? 4 : 2;  // 16-byte activation loads per thread and chunk
  constexpr int XH = (XF ? 4 : 2) * kXS;  // one half's stage ring (elements), per tile
  __shared__ __attribute__((aligned(16))) uint16_t xs_all[KW * XH * MT];

  const int bid = blockIdx.x;
  const int xcd = bid & 7, kk = bid >> 3;
  const int mt = kk % nMT;
  const int q = (kk / nMT) % S;
  const int g = (kk / (nMT * S)) * 8 + xcd;
  if (g >= NGr) return;
  const int m0 = mt * MT * kTileM;
  const int tid_all = threadIdx.x, l = tid_all & 63, lr = l & 15, lg = l >> 4;
  const int w = (tid_all >> 6) & 3;  // block of the group
  const int wk = tid_all >> 8;       // half of the slice (KW = 2)
  const int tid = tid_all & (kGThreads - 1);
  uint16_t* xs = xs_all + wk * XH;  // tile mm's stages at xs + mm * XH
  // block of this wave: the group's w-th of bpg (3 or 4) blocks; with bpg = 3
  // the fourth wave re-reads the group's first block (its sums are dropped) so
  // that its loads need no branch
  const int b = g * bpg + (w < bpg ? w : 0);
  const bool bv = w < bpg && b < NB;
  const int Ks = a.K / S;
  const int kbase = q * Ks + wk * (Ks / KW);
  const int nck = Ks / KW / kKc;
  // the epilogue's own inputs for activation row m0 + l (rows past M: the last)
  const int gme = min(m0 + l, a.M - 1);
  EpiIn ein;
  ein.key = bv ? epi_key<EPI>(a, b, gme) : -1;

  // weight operand of chunk c, half i: wb + c * wcs + i * whs (bytes).  Row-major
  // W: row block_row(b, l%16), columns 64 c + 32 i + 8 (l/16); packed W (see
  // proj_pack_kernel): the same 16 bytes, each half a contiguous kilobyte.
  const char* wb;
  size_t wcs, whs;
  if (a.w_packed) {
    // the packed layout keeps four consecutive blocks as one contiguous stream
    // over the chunks; block b is entry b % 4 of quad b / 4
    const int bb = b < NB ? b : NB - 1;
    wb = static_cast<const char*>(a.w_packed) +
         (((static_cast<size_t>(bb >> 2) * (a.K / kKc) + kbase / kKc) * 4 + (bb & 3)) * 128 + l) * 16;
    wcs = 4 * 2048;
    whs = 1024;
  } else {
    int row = b < NB ? block_row<EPI>(a, b, lr) : 0;
    if (row > a.N - 1) row = a.N - 1;
    wb = reinterpret_cast<const char*>(w_row_ptr(a, row) + kbase + 8 * lg);
    wcs = kKc * 2;
    whs = 64;
  }
  // piece e of this thread: 8 activations of row m0 + 64 mm + r, columns cc .. cc + 7 of the chunk
  const char* xr[MT][2];
  uint32_t xm[MT][2];
  int xlds[2];
#pragma unroll
  for (int e = 0; e < 2; ++e) {
    const int idx = e * kGThreads + tid;
    const int r = idx >> 3, cc = (idx & 7) * 8;
#pragma unroll
    for (int mm = 0; mm < MT; ++mm) {
      const uint16_t* p16;
      x_row_masked(a, m0 + mm * kTileM + r, p16, xm[mm][e]);
      if constexpr (XF) {
        const size_t row = static_cast<size_t>(p16 - static_cast<const uint16_t*>(a.x)) / a.K;
        xr[mm][e] = reinterpret_cast<const char*>(static_cast<const float*>(a.x) + row * a.K + kbase + cc);
      } else {
        xr[mm][e] = reinterpret_cast<const char*>(p16 + kbase + cc);
      }
    }
    xlds[e] = r * kXP + cc;
  }
  constexpr int xcs = XF ? kKc * 4 : kKc * 2;  // bytes per chunk along a row

  f32x4 acc[MT][4];
#pragma unroll
  for (int mm = 0; mm < MT; ++mm)
#pragma unroll
    for (int mb = 0; mb < 4; ++mb) acc[mm][mb] = f32x4{0.f, 0.f, 0.f, 0.f};
  constexpr int RS = DEPTH + 1;
  static_assert(RS % 2 == 0, "ring slots and LDS stages must unroll together");
  uint4 wbuf[RS][2];
  uint4 xbuf[RS][MT][NX];
  auto wload = [&](int c, uint4 (&dst)[2]) {
#pragma unroll
    for (int i = 0; i < 2; ++i) dst[i] = *reinterpret_cast<const uint4*>(wb + c * wcs + i * whs);
  };
  // raw loads; the row mask is applied when the chunk is written to LDS
  auto xload = [&](int c, uint4 (&dst)[MT][NX]) {
#pragma unroll
    for (int mm = 0; mm < MT; ++mm)
#pragma unroll
      for (int e = 0; e < NX; ++e)
        dst[mm][e] = *reinterpret_cast<const uint4*>(xr[mm][e * 2 / NX] + c * xcs + (XF ? (e & 1) * 16 : 0));
  };
  // chunk pieces -> LDS stage st (bf16 rounding; with XF also the remainder in
  // the second half of the stage ring)
  auto xstage = [&](int st, const uint4 (&srcs)[MT][NX]) {
#pragma unroll
    for (int mm = 0; mm < MT; ++mm)
#pragma unroll
    for (int e = 0; e < 2; ++e) {
      const uint4 (&src)[NX] = srcs[mm];
      uint16_t* xt = xs + mm * XH;
      if constexpr (XF) {
        const uint4 f0 = mask4(src[2 * e], xm[mm][e]), f1 = mask4(src[2 * e + 1], xm[mm][e]);
        const float v[8] = {__uint_as_float(f0.x), __uint_as_float(f0.y), __uint_as_float(f0.z),
                            __uint_as_float(f0.w), __uint_as_float(f1.x), __uint_as_float(f1.y),
                            __uint_as_float(f1.z), __uint_as_float(f1.w)};
        uint32_t hw[4], lw[4];
#pragma unroll
        for (int k = 0; k < 4; ++k) {
          hw[k] = pack_bf16x2(v[2 * k], v[2 * k + 1]);
          lw[k] = pack_bf16x2(v[2 * k] - __uint_as_float(hw[k] << 16),
                              v[2 * k + 1] - __uint_as_float(hw[k] & 0xFFFF0000u));
        }
        *reinterpret_cast<uint4*>(&xt[st * kXS + xlds[e]]) = make_uint4(hw[0], hw[1], hw[2], hw[3]);
        *reinterpret_cast<uint4*>(&xt[(2 + st) * kXS + xlds[e]]) = make_uint4(lw[0], lw[1], lw[2], lw[3]);
      } else {
        *reinterpret_cast<uint4*>(&xt[st * kXS + xlds[e]]) = mask4(src[e], xm[mm][e]);
      }
    }
  };

  // nck is a multiple of RS; loads past the last chunk are clamped to it, so no
  // load is conditional (a conditional load would make the compiler's wait
  // counts conservative and drain the ring every chunk).  The whole ring is in
  // flight before the first activation chunk is waited for.
  xload(0, xbuf[0]);
#pragma unroll
  for (int d = 0; d < DEPTH; ++d) {
    if (d + 1 < DEPTH) xload(min(d + 1, nck - 1), xbuf[d + 1]);
    wload(min(d, nck - 1), wbuf[d]);
  }
  xstage(0, xbuf[0]);
  for (int c0 = 0; c0 < nck; c0 += RS) {
#pragma unroll
    for (int u = 0; u < RS; ++u) {
      const int c = c0 + u;
      {
        const int cn = min(c + DEPTH, nck - 1);
        xload(cn, xbuf[(u + DEPTH) % RS]);
        wload(cn, wbuf[(u + DEPTH) % RS]);
        __syncthreads();
        // every activation operand of a tile's chunk is read from LDS before
        // the tile's first product, so the reads overlap instead of each
        // product waiting on its own read
#pragma unroll
        for (int mm = 0; mm < MT; ++mm) {
          const uint16_t* xq = xs + mm * XH + (u & 1) * kXS;
          constexpr int NV = XF ? 2 : 1;
          bf16x8 bx[2][4][NV];
#pragma unroll
          for (int s = 0; s < 2; ++s)
#pragma unroll
            for (int mb = 0; mb < 4; ++mb)
#pragma unroll
              for (int v = 0; v < NV; ++v)
                bx[s][mb][v] = *reinterpret_cast<const bf16x8*>(
                    xq + 2 * v * kXS + (mb * 16 + lr) * kXP + s * 32 + 8 * lg);
          __builtin_amdgcn_sched_barrier(0);
#pragma unroll
          for (int s = 0; s < 2; ++s) {
            const bf16x8 av = __builtin_bit_cast(bf16x8, wbuf[u][s]);
#pragma unroll
            for (int v = 0; v < NV; ++v)
#pragma unroll
              for (int mb = 0; mb < 4; ++mb)
                acc[mm][mb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(av, bx[s][mb][v], acc[mm][mb], 0, 0, 0);
          }
        }
        // (after the last chunk this stores a clamped copy nobody reads)
        xstage((u + 1) & 1, xbuf[(u + 1) % RS]);
      }
    }
  }

  if constexpr (MT > 1) {
    // K is split (S > 1): every tile's partial is stored, one arrival counts the
    // work-group's tiles, and the last work-group of the group sums each tile's
    // slices in slice order and applies the epilogue (same hand-over as below)
#pragma unroll
    for (int mm = 0; mm < MT; ++mm) {
      if (m0 + mm * kTileM >= a.M) break;  // (uniform) a tile past the rows: no partial
      const size_t grp = static_cast<size_t>(mt * MT + mm) * NGr + g;
      float* pp = a.kpart + ((grp * S + q) * 4 + w) * 1024;
#pragma unroll
      for (int mb = 0; mb < 4; ++mb)
#pragma unroll
        for (int v = 0; v < 4; ++v)
          __hip_atomic_store(pp + (4 * lg + v) * 64 + mb * 16 + lr, acc[mm][mb][v], __ATOMIC_RELAXED,
                             __HIP_MEMORY_SCOPE_AGENT);
    }
    __builtin_amdgcn_s_waitcnt(0);
    __shared__ int s_last_t;
    __syncthreads();
    if (tid_all == 0) {
      unsigned* cnt = a.kcnt + static_cast<size_t>(mt) * NGr + g;
      const unsigned old = __hip_atomic_fetch_add(cnt, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      const bool last = old == static_cast<unsigned>(S - 1);
      if (last) __hip_atomic_store(cnt, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      s_last_t = last;
    }
    __syncthreads();
    if (!s_last_t || !bv) return;
#pragma unroll
    for (int mm = 0; mm < MT; ++mm) {
      if (m0 + mm * kTileM >= a.M) break;  // (uniform) no rows in this tile
      // thread (w, l): activation row m0 + 64 mm + l of block b
      const int gm = m0 + mm * kTileM + l;
      EpiIn et;
      et.key = epi_key<EPI>(a, b, min(gm, a.M - 1));
      epi_load<EPI>(a, b, min(gm, a.M - 1), et);
      const size_t grp = static_cast<size_t>(mt * MT + mm) * NGr + g;
      float x[16];
#pragma unroll
      for (int i = 0; i < 16; ++i) x[i] = 0.f;
      constexpr int kSB = 8;
      for (int q0 = 0; q0 < S; q0 += kSB) {
        float y[kSB][16];
#pragma unroll
        for (int j = 0; j < kSB; ++j) {
          if (q0 + j < S) {
            const float* src = a.kpart + ((grp * S + q0 + j) * 4 + w) * 1024 + l;
#pragma unroll
            for (int i = 0; i < 16; ++i) y[j][i] = __hip_atomic_load(src + i * 64, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
          }
        }
#pragma unroll
        for (int j = 0; j < kSB; ++j)
          if (q0 + j < S) {
#pragma unroll
            for (int i = 0; i < 16; ++i) x[i] += y[j][i];
          }
      }
      if (gm < a.M) proj_store<EPI>(a, b, gm, x, et);
    }
  } else {
    // partial of this wave's block: [16 block rows][64 activation rows], stored
    // with device-coherent stores; the group's last work-group to arrive sums the
    // S slices in slice order (deterministic) and applies the epilogue.  Only the
    // counter and the partials are shared, both through device-scope atomic
    // accesses (write-through stores and coherent loads), and every store has
    // completed before the arrival is counted, so no cache write-back is needed.
    if constexpr (KW > 1) {
      // the second half's sums join the first's (same lane layout) through LDS
      float* hp = reinterpret_cast<float*>(xs_all) + w * 1024 + l;
      __syncthreads();
      if (wk == 1) {
  #pragma unroll
        for (int mb = 0; mb < 4; ++mb)
  #pragma unroll
          for (int v = 0; v < 4; ++v) hp[(mb * 4 + v) * 64] = acc[0][mb][v];
      }
      __syncthreads();
      if (wk == 0) {
  #pragma unroll
        for (int mb = 0; mb < 4; ++mb)
  #pragma unroll
          for (int v = 0; v < 4; ++v) acc[0][mb][v] += hp[(mb * 4 + v) * 64];
      }
    }
    if (bv) epi_load<EPI>(a, b, gme, ein);
    if (S == 1) {
      // no other slice: the block's 16 x 64 result goes through LDS (the stage
      // ring is free after the barrier) to one thread per activation row
      float* tr = reinterpret_cast<float*>(xs_all) + w * 1024;
      __syncthreads();
      if (wk == 0) {
  #pragma unroll
        for (int mb = 0; mb < 4; ++mb)
  #pragma unroll
          for (int v = 0; v < 4; ++v) tr[(4 * lg + v) * 64 + mb * 16 + lr] = acc[0][mb][v];
      }
      __syncthreads();
      if (wk != 0 || !bv || m0 + l >= a.M) return;
      float x[16];
  #pragma unroll
      for (int i = 0; i < 16; ++i) x[i] = tr[i * 64 + l];
      proj_store<EPI>(a, b, m0 + l, x, ein);
      return;
    }
    // Hand-over to the group's last work-group.  Invariant: the partials are
    // written and read only with device-scope atomic accesses (performed at
    // the device-coherent level, never in a per-XCD cache), every store is
    // complete (s_waitcnt 0) before this work-group's arrival increment, and
    // the last work-group loads them only after it has seen the final count.
    const size_t grp = static_cast<size_t>(mt) * NGr + g;
    float* pp = a.kpart + ((grp * S + q) * 4 + w) * 1024;
    if (wk == 0) {
  #pragma unroll
      for (int mb = 0; mb < 4; ++mb)
  #pragma unroll
        for (int v = 0; v < 4; ++v)
          __hip_atomic_store(pp + (4 * lg + v) * 64 + mb * 16 + lr, acc[0][mb][v], __ATOMIC_RELAXED,
                             __HIP_MEMORY_SCOPE_AGENT);
    }
    __builtin_amdgcn_s_waitcnt(0);
    __shared__ int s_last;
    __syncthreads();
    if (tid_all == 0) {
      const unsigned old = __hip_atomic_fetch_add(a.kcnt + grp, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      const bool last = old == static_cast<unsigned>(S - 1);
      if (last) __hip_atomic_store(a.kcnt + grp, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      s_last = last;
    }
    __syncthreads();
    if (!s_last || !bv || wk != 0) return;
    // thread (w, l): activation row m0 + l of block b
    float x[16];
  #pragma unroll
    for (int i = 0; i < 16; ++i) x[i] = 0.f;
    // up to 8 slices' loads in flight at once (one round trip per 8 slices),
    // summed in slice order
    constexpr int kSB = 8;
    for (int q0 = 0; q0 < S; q0 += kSB) {
      float y[kSB][16];
  #pragma unroll
      for (int j = 0; j < kSB; ++j) {
        if (q0 + j < S) {
          const float* src = a.kpart + ((grp * S + q0 + j) * 4 + w) * 1024 + l;
  #pragma unroll
          for (int i = 0; i < 16; ++i) y[j][i] = __hip_atomic_load(src + i * 64, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        }
      }
  #pragma unroll
      for (int j = 0; j < kSB; ++j)
        if (q0 + j < S) {
  #pragma unroll
          for (int i = 0; i < 16; ++i) x[i] += y[j][i];
        }
    }
    const int gm = m0 + l;
    if (gm >= a.M) return;
    proj_store<EPI>(a, b, gm, x, ein);
  }
}

// WALK: the row outputs are published with a release increment of an arrival
// counter; the last row to arrive acquires all of them and runs the accept walk
// of every round (the step that follows the head) in its first wave, then
// returns the counter to zero.
template <bool WALK>
__global__ __launch_bounds__(256) void head_merge_kernel(const float* __restrict__ part, int nNT,
                                                         int32_t* __restrict__ argmax,
                                                         float* __restrict__ top1,
                                                         float* __restrict__ gap,
                                                         float* __restrict__ entropy,
                                                         HeadDraw dr, WalkArgs wk,
                                                         unsigned* __restrict__ arrivals) {
  __shared__ HeadPart red[4];
  __shared__ Draw dred[4];
  const int r = blockIdx.x, tid = threadIdx.x;
  HeadPart p = head_empty();
  Draw d = draw_empty();
  for (int t = tid; t < nNT; t += 256) {
    const float* q = part + (static_cast<size_t>(r) * nNT + t) * 5;
    HeadPart e;
    e.m = q[0];
    e.am = __float_as_int(q[1]);
    e.m2 = q[2];
    e.s = q[3];
    e.t = q[4];
    p = head_combine(p, e);
    if (dr.tok) {
      const float* u = dr.spart + (static_cast<size_t>(r) * nNT + t) * 3;
      d = draw_combine(d, Draw{u[0], __float_as_int(u[1]), u[2]});
    }
  }
  // within each wave by lane exchanges, then the four waves in order
  const int lane = tid & 63, wv = tid >> 6;
#pragma unroll
  for (int off = 32; off > 0; off >>= 1) {
    p = head_combine(p, shfl_part(p, lane ^ off));
    if (dr.tok) d = draw_combine(d, shfl_draw(d, lane ^ off));
  }
  if (lane == 0) {
    red[wv] = p;
    dred[wv] = d;
  }
  __syncthreads();
  if (tid == 0) {
    HeadPart f = red[0];
    Draw g = dred[0];
#pragma unroll
    for (int k = 1; k < 4; ++k) {
      f = head_combine(f, red[k]);
      g = draw_combine(g, dred[k]);
    }
    argmax[r] = f.am;
    top1[r] = f.m;
    gap[r] = f.m - f.m2;
    entropy[r] = logf(f.s) - f.t / f.s;
    if (dr.tok) {
      dr.tok[r] = g.tok;
      dr.gap[r] = g.m - g.m2;
    }
  }
  if constexpr (WALK) {
    __shared__ int s_last;
    if (tid == 0) {
      // release: this thread's row outputs above; acquire: every earlier row's
      const unsigned old = __hip_atomic_fetch_add(arrivals, 1u, __ATOMIC_ACQ_REL,
                                                  __HIP_MEMORY_SCOPE_AGENT);
      const bool last = old == gridDim.x - 1u;
      if (last) __hip_atomic_store(arrivals, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      s_last = last;
    }
    __syncthreads();
    if (!s_last || tid >= kWave) return;
    // the walking wave's own loads of the other rows' outputs come after an
    // acquire of its own (the increment above acquired for thread 0 only)
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "agent");
    const int32_t* pick = dr.tok ? dr.tok : argmax;
    const float* pgap = dr.tok ? dr.gap : gap;
    for (int s = 0; s < wk.nseq; ++s) walk_round(wk, pick, pgap, s);
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
                                                                float* __restrict__ entropy,
                                                                HeadDraw dr) {
  __shared__ HeadPart red[256];
  __shared__ Draw dred[256];
  const int r = blockIdx.x, tid = threadIdx.x;
  const float* z = logits + static_cast<size_t>(r) * V;
  HeadPart p = head_empty();
  Draw d = draw_empty();
  for (int n = tid; n < V; n += 256) {
    p = head_combine(p, head_elem(z[n], n));
    if (dr.tok) {
      const uint4 x = philox4x32_10(make_uint4(static_cast<uint32_t>(n >> 2), static_cast<uint32_t>(r),
                                               dr.rnd_lo, dr.rnd_hi), dr.seed_lo, dr.seed_hi);
      const uint32_t w = (n & 3) == 0 ? x.x : (n & 3) == 1 ? x.y : (n & 3) == 2 ? x.z : x.w;
      d = draw_combine(d, Draw{fmaf(z[n], dr.inv_temp, gumbel(w)), n, -INFINITY});
    }
  }
  red[tid] = p;
  dred[tid] = d;
  __syncthreads();
  for (int st = 128; st > 0; st >>= 1) {
    if (tid < st) {
      red[tid] = head_combine(red[tid], red[tid + st]);
      dred[tid] = draw_combine(dred[tid], dred[tid + st]);
    }
    __syncthreads();
  }
  if (tid == 0) {
    const HeadPart f = red[0];
    argmax[r] = f.am;
    top1[r] = f.m;
    gap[r] = f.m - f.m2;
    entropy[r] = logf(f.s) - f.t / f.s;
    if (dr.tok) {
      dr.tok[r] = dred[0].tok;
      dr.gap[r] = dred[0].m - dred[0].m2;
    }
  }
}

}  // namespace

namespace {
constexpr int kHeadB = 5;      // weight blocks per wave in the LM head
constexpr int kHeadWaves = 2048;  // waves the LM head grid aims for (256 CUs x 8)

struct HeadGrid {
  int NB, NG, nWG, per;
};
HeadGrid head_grid(int N) {
  // the fewest waves (at most kHeadWaves while blocks per wave <= kHeadB) that
  // give every wave the same number of blocks, up to one
  HeadGrid g;
  g.NB = (N + 15) / 16;
  int per = (g.NB + kHeadWaves - 1) / kHeadWaves;
  if (per > kHeadB) per = kHeadB;
  g.per = per;
  g.NG = (g.NB + per - 1) / per;
  g.nWG = (g.NG + 3) / 4;
  return g;
}

// Packed LM-head weights: [K/64 chunks][NG waves][per blocks][2 halves][64 lanes]
// x 16 bytes; block t of wave G is vocabulary block G + t NG; lane l of half s
// holds row 16 (G + t NG) + l%16, columns 64 c + 32 s + 8 (l/16) .. + 8; rows
// past N are zero.
__global__ __launch_bounds__(256) void head_pack_kernel(const uint16_t* __restrict__ w, int N,
                                                        int K, int NG, int per, size_t n16,
                                                        uint4* __restrict__ out) {
  for (size_t o = static_cast<size_t>(blockIdx.x) * 256 + threadIdx.x; o < n16;
       o += static_cast<size_t>(gridDim.x) * 256) {
    const int l = static_cast<int>(o & 63), s = static_cast<int>((o >> 6) & 1);
    size_t rest = o >> 7;
    const int t = static_cast<int>(rest % per);
    rest /= per;
    const int G = static_cast<int>(rest % NG);
    const int c = static_cast<int>(rest / NG);
    const int row = (G + t * NG) * 16 + (l & 15);
    const int col = c * kKc + 32 * s + 8 * (l >> 4);
    out[o] = row < N ? *reinterpret_cast<const uint4*>(w + static_cast<size_t>(row) * K + col)
                     : make_uint4(0u, 0u, 0u, 0u);
  }
}
}  // namespace

// Packed projection weights: [NB/4 groups][K/64 chunks][4 blocks][2 halves]
// [64 lanes] x 16 bytes, so that the four blocks one work-group multiplies are
// a single contiguous stream; lane l of half s of block b = 4 g + j holds row
// block_row(b, l%16), columns 64 c + 32 s + 8 (l/16) .. + 8 (the MFMA operand
// of that block and chunk).  Blocks past NB are zero.
template <int EPI>
__global__ __launch_bounds__(256) void proj_pack_kernel(GemmArgs a, int NB, size_t n16,
                                                        uint4* __restrict__ out) {
  const int nch = a.K / kKc;
  for (size_t o = static_cast<size_t>(blockIdx.x) * 256 + threadIdx.x; o < n16;
       o += static_cast<size_t>(gridDim.x) * 256) {
    const int l = static_cast<int>(o & 63), s = static_cast<int>((o >> 6) & 1);
    const size_t rest = o >> 7;
    const int j = static_cast<int>(rest & 3);
    const int c = static_cast<int>((rest >> 2) % nch);
    const int b = static_cast<int>((rest >> 2) / nch) * 4 + j;
    if (b >= NB) {
      out[o] = make_uint4(0u, 0u, 0u, 0u);
      continue;
    }
    const int row = block_row<EPI>(a, b, l & 15);
    const int col = c * kKc + 32 * s + 8 * (l >> 4);
    out[o] = *reinterpret_cast<const uint4*>(w_row_ptr(a, row) + col);
  }
}

int gemm_bf16_head_parts(int N) { return head_grid(N).nWG; }

// ------------------------------------------------- head without a workspace
// Scratch of glance_verify_head_packed_noalloc: the head's per-row partial
// statistics (and draws) live in this array instead of a caller workspace.
// Each GPU the library runs on holds its own copy until the process ends; host
// code must not pass the array's name to a kernel (on the host it is only a
// stand-in symbol), but the device address looked up for the current device.
static __device__ __align__(256) float scratch[kHeadScratchFloats];

glance_status head_scratch_ptr(float** out) {
  static std::mutex mu;
  static float* per_device[64] = {};
  int dev = -1;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return hip_fail(e);
  if (dev < 0 || dev >= 64) return GLANCE_ERR_UNSUPPORTED;
  std::lock_guard<std::mutex> lock(mu);
  if (per_device[dev] == nullptr) {
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return hip_fail(e);
    per_device[dev] = static_cast<float*>(p);
  }
  *out = per_device[dev];
  return GLANCE_OK;
}

size_t proj_pack_bytes(int N, int K) {
  return static_cast<size_t>(K / kKc) * (((N + 15) / 16 + 3) / 4) * 4 * 2048;
}

glance_status launch_proj_pack(const GemmArgs& a, void* w_packed, hipStream_t st) {
  const int NB = proj_blocks(a);
  const size_t n16 = proj_pack_bytes(a.N, a.K) / 16;
  size_t blocks = (n16 + 255) / 256;
  if (blocks > 8192) blocks = 8192;
  if (a.epi == EPI_SWIGLU)
    proj_pack_kernel<EPI_SWIGLU><<<static_cast<unsigned>(blocks), 256, 0, st>>>(a, NB, n16, static_cast<uint4*>(w_packed));
  else if (a.epi == EPI_QKV)
    proj_pack_kernel<EPI_QKV><<<static_cast<unsigned>(blocks), 256, 0, st>>>(a, NB, n16, static_cast<uint4*>(w_packed));
  else
    proj_pack_kernel<EPI_RESID><<<static_cast<unsigned>(blocks), 256, 0, st>>>(a, NB, n16, static_cast<uint4*>(w_packed));
  GLANCE_LAUNCH_CHECK();
  return GLANCE_OK;
}

size_t head_pack_bytes(int N, int K) {
  const HeadGrid g = head_grid(N);
  return static_cast<size_t>(K / kKc) * g.NG * g.per * 2 * 64 * 16;
}

glance_status launch_head_pack(const void* w, int N, int K, void* w_packed, hipStream_t st) {
  const HeadGrid g = head_grid(N);
  const size_t n16 = head_pack_bytes(N, K) / 16;
  size_t blocks = (n16 + 255) / 256;
  if (blocks > 8192) blocks = 8192;
  head_pack_kernel<<<static_cast<unsigned>(blocks), 256, 0, st>>>(
      static_cast<const uint16_t*>(w), N, K, g.NG, g.per, n16, static_cast<uint4*>(w_packed));
  return GLANCE_OK;
}

#ifndef GLANCE_PROJ_WGS
#define GLANCE_PROJ_WGS 256
#endif
#ifndef GLANCE_PROJ_MINBPG
#define GLANCE_PROJ_MINBPG 3
#endif
// 64-row tiles per work-group of the q/k/v projection above 64 rows (1, 2 or 4)
#ifndef GLANCE_PROJ_QKV_TILES
#define GLANCE_PROJ_QKV_TILES 2
#endif
// Work-groups of a projection: NGr groups of bpg 16-row blocks times S K-slices
// (S a divisor of half the chunk count, so each slice is an even number of
// chunks).  The most work-groups up to about one per CU, from groups of four
// blocks or of three (three-block groups let 384 blocks fill 256 CUs exactly);
// wide projections (more groups than CUs, the MLP) take groups of four and no
// split: every work-group is resident at two per CU and no partial sums cross
// work-groups.
ProjGrid proj_grid(int K, int NB) {
  const int nch = K / kKc;
  ProjGrid best{4, (NB + 3) / 4, 1};
  int best_wgs = 0;
  for (int bpg = 4; bpg >= GLANCE_PROJ_MINBPG; --bpg) {
    const int NGr = (NB + bpg - 1) / bpg;
    int S = 1;
    for (int c = 1; c <= nch / 2; ++c)
      if ((nch / 2) % c == 0 && NGr * c <= GLANCE_PROJ_WGS) S = c;
    if (NGr * S <= GLANCE_PROJ_WGS && NGr * S > best_wgs) {
      best = ProjGrid{bpg, NGr, S};
      best_wgs = NGr * S;
    }
  }
  return best;
}

int proj_blocks(const GemmArgs& a) {
  return a.epi == EPI_QKV ? (a.Hq + 2 * a.Hkv) * 8 : (a.N + 15) / 16;
}

size_t proj_part_floats(int M, int NB, int K) {
  // tiles of 64 rows, rounded up to a multiple of the most tiles a work-group takes
  const int nMT = ((M + kTileM - 1) / kTileM + 3) / 4 * 4;
  const ProjGrid pg = proj_grid(K, NB);
  return static_cast<size_t>(nMT) * pg.NGr * pg.S * 4 * 1024;
}

size_t proj_counters(int M, int NB, int K) {
  const int nMT = (M + kTileM - 1) / kTileM;
  return static_cast<size_t>(nMT) * proj_grid(K, NB).NGr;
}

glance_status launch_gemm_bf16(const GemmArgs& a, hipStream_t st) {
  const int nMT = (a.M + kTileM - 1) / kTileM;
  if (a.epi == EPI_HEAD) {
    const HeadGrid g = head_grid(a.N);
    const int grid = ((g.nWG + 7) / 8) * 8 * nMT;
    if (a.w_packed && nMT >= 2) {
      // two activation tiles per work-group (weights applied from registers twice)
      const int nMT2 = (nMT + 1) / 2;
      const int grid2 = ((g.nWG + 7) / 8) * 8 * nMT2;
      if (a.spart)
        head_bf16_kernel<kHeadB, 2, true, true, 2><<<grid2, kGThreads, 0, st>>>(a, g.NB, g.NG, g.nWG, nMT2, g.per);
      else
        head_bf16_kernel<kHeadB, 2, false, true, 2><<<grid2, kGThreads, 0, st>>>(a, g.NB, g.NG, g.nWG, nMT2, g.per);
    } else if (a.w_packed) {
      if (a.spart)
        head_bf16_kernel<kHeadB, 2, true, true><<<grid, kGThreads, 0, st>>>(a, g.NB, g.NG, g.nWG, nMT, g.per);
      else
        head_bf16_kernel<kHeadB, 2, false, true><<<grid, kGThreads, 0, st>>>(a, g.NB, g.NG, g.nWG, nMT, g.per);
    } else if (a.spart) {
      head_bf16_kernel<kHeadB, 2, true, false><<<grid, kGThreads, 0, st>>>(a, g.NB, g.NG, g.nWG, nMT, g.per);
    } else {
      head_bf16_kernel<kHeadB, 2, false, false><<<grid, kGThreads, 0, st>>>(a, g.NB, g.NG, g.nWG, nMT, g.per);
    }
  } else {
    const int NB = proj_blocks(a);
    const ProjGrid pg = proj_grid(a.K, NB);
    const int NGr = pg.NGr, S = pg.S, bpg = pg.bpg;
    // more than 64 rows with K split: several 64-row tiles per work-group (four
    // for the q/k/v projection, two for the fp32-input output projection), a
    // ring of 4 chunks (2 when a slice has fewer)
    const bool tiled = nMT >= 2 && S > 1 &&
                       ((a.epi == EPI_QKV && GLANCE_PROJ_QKV_TILES > 1) || (a.epi == EPI_RESID && a.x_f32));
    if (tiled) {
      const int nckt = a.K / S / kKc;
      const bool r4 = nckt % 4 == 0;
      const int mtt = (a.epi == EPI_QKV && nMT >= 4 && GLANCE_PROJ_QKV_TILES == 4) ? 4 : 2;
      const int nMTg = (nMT + mtt - 1) / mtt;
      const int gridt = ((NGr + 7) / 8) * 8 * S * nMTg;
      if (a.epi == EPI_QKV) {
        if (mtt == 4) {
          if (r4) proj_bf16_kernel<EPI_QKV, 3, false, 1, 4><<<gridt, kGThreads, 0, st>>>(a, NB, NGr, S, nMTg, bpg);
          else proj_bf16_kernel<EPI_QKV, 1, false, 1, 4><<<gridt, kGThreads, 0, st>>>(a, NB, NGr, S, nMTg, bpg);
        } else {
          if (r4) proj_bf16_kernel<EPI_QKV, 3, false, 1, 2><<<gridt, kGThreads, 0, st>>>(a, NB, NGr, S, nMTg, bpg);
          else proj_bf16_kernel<EPI_QKV, 1, false, 1, 2><<<gridt, kGThreads, 0, st>>>(a, NB, NGr, S, nMTg, bpg);
        }
      } else {
        if (r4) proj_bf16_kernel<EPI_RESID, 3, true, 1, 2><<<gridt, kGThreads, 0, st>>>(a, NB, NGr, S, nMTg, bpg);
        else proj_bf16_kernel<EPI_RESID, 1, true, 1, 2><<<gridt, kGThreads, 0, st>>>(a, NB, NGr, S, nMTg, bpg);
      }
      GLANCE_LAUNCH_CHECK();
      return GLANCE_OK;
    }
    const int grid = ((NGr + 7) / 8) * 8 * S * nMT;
    // at most one work-group per CU: eight waves splitting the slice in two
    // halves (two waves per SIMD); wider grids: four waves.  Ring depth: the
    // largest of 8, 4, 2 slots dividing the chunk count of a wave's range (4 at
    // most for fp32 activations in eight-wave groups, for registers).
    const int kw = grid <= 256 && (a.K / S / kKc) % 4 == 0 ? 2 : 1;
    const int nck = a.K / S / kw / kKc;
    int rs = nck % 8 == 0 ? 8 : nck % 4 == 0 ? 4 : 2;
    if (kw == 2 && a.x_f32 && rs > 4) rs = 4;
    const unsigned nthr = kGThreads * kw;
#define GLANCE_PROJ_KW(E, X, KW)                                                      \
  if (rs == 8)                                                                       \
    proj_bf16_kernel<E, 7, X, KW><<<grid, nthr, 0, st>>>(a, NB, NGr, S, nMT, bpg);         \
  else if (rs == 4)                                                                  \
    proj_bf16_kernel<E, 3, X, KW><<<grid, nthr, 0, st>>>(a, NB, NGr, S, nMT, bpg);         \
  else                                                                               \
    proj_bf16_kernel<E, 1, X, KW><<<grid, nthr, 0, st>>>(a, NB, NGr, S, nMT, bpg);
#define GLANCE_PROJ(E, X)    \
  if (kw == 2) {             \
    GLANCE_PROJ_KW(E, X, 2)  \
  } else {                   \
    GLANCE_PROJ_KW(E, X, 1)  \
  }
    if (a.epi == EPI_QKV) {
      GLANCE_PROJ(EPI_QKV, false)
    } else if (a.epi == EPI_SWIGLU) {
      GLANCE_PROJ(EPI_SWIGLU, false)
    } else if (a.epi == EPI_STORE_F32) {
      GLANCE_PROJ(EPI_STORE_F32, false)
    } else if (a.x_f32) {
      if (kw == 2) {
        if (rs == 4)
          proj_bf16_kernel<EPI_RESID, 3, true, 2><<<grid, nthr, 0, st>>>(a, NB, NGr, S, nMT, bpg);
        else
          proj_bf16_kernel<EPI_RESID, 1, true, 2><<<grid, nthr, 0, st>>>(a, NB, NGr, S, nMT, bpg);
      } else {
        GLANCE_PROJ_KW(EPI_RESID, true, 1)
      }
    } else {
      GLANCE_PROJ(EPI_RESID, false)
    }
#undef GLANCE_PROJ_KW
#undef GLANCE_PROJ
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
                                float* top1, float* gap, float* entropy, const HeadDraw& dr,
                                hipStream_t st) {
  head_merge_kernel<false><<<R, 256, 0, st>>>(part, n_tiles, argmax, top1, gap, entropy, dr,
                                              WalkArgs{}, nullptr);
  GLANCE_LAUNCH_CHECK();
  return GLANCE_OK;
}

glance_status launch_head_merge_walk(const float* part, int n_tiles, int R, int32_t* argmax,
                                     float* top1, float* gap, float* entropy, const HeadDraw& dr,
                                     const WalkArgs& wk, unsigned* arrivals, hipStream_t st) {
  head_merge_kernel<true><<<R, 256, 0, st>>>(part, n_tiles, argmax, top1, gap, entropy, dr, wk,
                                             arrivals);
  GLANCE_LAUNCH_CHECK();
  return GLANCE_OK;
}

glance_status launch_head_rowstats_f32(const float* logits, int R, int V, int32_t* argmax,
                                       float* top1, float* gap, float* entropy,
                                       const HeadDraw& dr, hipStream_t st) {
  head_rowstats_f32_kernel<<<R, 256, 0, st>>>(logits, V, argmax, top1, gap, entropy, dr);
  GLANCE_LAUNCH_CHECK();
  return GLANCE_OK;
}

}  // namespace glance
