// Skinny GEMMs of the verify pass: C = X W^T for the few verify rows X
// [M][K] against a streamed weight matrix W [N][K] (out x in), with the
// epilogue fused:
//   EPI_STORE_F32  the QKV projection (fp32 out, RoPE is applied by the
//                  attention kernel that reads it);
//   EPI_RESID      the output projection plus residual, rounded to the storage
//                  dtype (a storage point of the layer);
//   EPI_HEAD       the LM head: per row and per 128-column tile, the partial
//                  (max, argmax, second max, sum e^(z-max), sum e^(z-max)(z-max)),
//                  merged by head_merge into argmax, top-1, top-2 gap and entropy
//                  (paper §3.1 greedy token; App. B.1 top-2 gap; §6 root entropy).
//
// bf16 path (gfx950 MFMA v_mfma_f32_32x32x16_bf16): a 256-thread work-group
// owns a 128 (N) x 64 (M) output tile.  Each wave streams its 32 weight rows
// straight from HBM into registers (one 16-byte load per lane per 16-deep
// k-step, a whole 256-deep chunk prefetched ahead), while the 64 activation rows
// of the chunk are staged once per work-group in LDS (double-buffered, rows
// padded by 16 bytes against bank conflicts).  At M <= 64 the weight stream is
// the whole cost (64 flop per weight byte, below the MFMA ridge), so the kernel
// is judged against HBM bandwidth.  Work-group ids are mapped so that the
// M-tiles of one N-tile land on the same XCD back to back and share its L2.
#include "common.h"
#include "kernels.h"

namespace glance {

namespace {

constexpr int kGThreads = 256;
constexpr int kTileN = 128;
constexpr int kTileM = 64;
constexpr int kKc = 256;          // K chunk staged per step
constexpr int kXPad = kKc + 8;    // LDS row stride (bf16 elements)
constexpr int kKSteps = kKc / 16;

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

template <int EPI>
__global__ __launch_bounds__(kGThreads, 2) void gemm_bf16_kernel(GemmArgs a, int nNT, int nMT) {
  __shared__ __attribute__((aligned(16))) uint16_t xs[2][kTileM][kXPad];
  __shared__ HeadPart red[4][kTileM];

  const int b = blockIdx.x;
  const int xcd = b & 7, kk = b >> 3;
  const int mt = kk % nMT;
  const int nt = (kk / nMT) * 8 + xcd;
  if (nt >= nNT) return;
  const int n0 = nt * kTileN, m0 = mt * kTileM;
  const int tid = threadIdx.x, w = tid >> 6, l = tid & 63, li = l & 31, g = l >> 5;

  // this lane's weight row (clamped into range; outputs past N are masked)
  int wrow = n0 + w * 32 + li;
  if (wrow > a.N - 1) wrow = a.N - 1;
  const uint16_t* wp;
  {
    int start = 0, sidx = 0;
    while (sidx < a.w.nseg - 1 && wrow >= a.w.n_end[sidx]) start = a.w.n_end[sidx++];
    wp = static_cast<const uint16_t*>(a.w.w[sidx]) + static_cast<size_t>(wrow - start) * a.K + 8 * g;
  }

  // activation rows this thread copies into LDS: rows tid/32 + 8 p, 16 bytes at col (tid%32)*8
  const uint16_t* xr[8];
#pragma unroll
  for (int p = 0; p < 8; ++p) xr[p] = x_row_ptr(a, m0 + p * 8 + (tid >> 5));
  const int xc = (tid & 31) * 8;

  const int nch = a.K / kKc;
  f32x16 acc0 = {}, acc1 = {};
  uint4 wcur[kKSteps], wnext[kKSteps];
  uint4 xnext[8];

  // prologue: chunk 0
#pragma unroll
  for (int p = 0; p < 8; ++p) {
    uint4 v = make_uint4(0, 0, 0, 0);
    if (xr[p]) v = *reinterpret_cast<const uint4*>(xr[p] + xc);
    *reinterpret_cast<uint4*>(&xs[0][p * 8 + (tid >> 5)][xc]) = v;
  }
#pragma unroll
  for (int s = 0; s < kKSteps; ++s) wcur[s] = *reinterpret_cast<const uint4*>(wp + s * 16);

  for (int c = 0; c < nch; ++c) {
    const int buf = c & 1;
    const bool more = c + 1 < nch;
    if (more) {
      const int k1 = (c + 1) * kKc;
#pragma unroll
      for (int p = 0; p < 8; ++p) {
        xnext[p] = make_uint4(0, 0, 0, 0);
        if (xr[p]) xnext[p] = *reinterpret_cast<const uint4*>(xr[p] + k1 + xc);
      }
#pragma unroll
      for (int s = 0; s < kKSteps; ++s)
        wnext[s] = *reinterpret_cast<const uint4*>(wp + k1 + s * 16);
    }
    __syncthreads();
#pragma unroll
    for (int s = 0; s < kKSteps; ++s) {
      const bf16x8 av = __builtin_bit_cast(bf16x8, wcur[s]);
      const bf16x8 b0 = *reinterpret_cast<const bf16x8*>(&xs[buf][li][s * 16 + 8 * g]);
      const bf16x8 b1 = *reinterpret_cast<const bf16x8*>(&xs[buf][32 + li][s * 16 + 8 * g]);
      acc0 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(av, b0, acc0, 0, 0, 0);
      acc1 = __builtin_amdgcn_mfma_f32_32x32x16_bf16(av, b1, acc1, 0, 0, 0);
    }
    if (more) {
#pragma unroll
      for (int p = 0; p < 8; ++p)
        *reinterpret_cast<uint4*>(&xs[buf ^ 1][p * 8 + (tid >> 5)][xc]) = xnext[p];
#pragma unroll
      for (int s = 0; s < kKSteps; ++s) wcur[s] = wnext[s];
    }
  }

  // ------------------------------------------------------------- epilogues
  // acc element v of this lane: output row n = n0 + 32 w + 8 (v/4) + 4 g + v%4,
  // activation row m = m0 + li (acc0) or m0 + 32 + li (acc1).
  const int nb = n0 + w * 32 + 4 * g;
#pragma unroll
  for (int h = 0; h < 2; ++h) {
    const f32x16 acc = h ? acc1 : acc0;
    const int m = m0 + h * 32 + li;
    if constexpr (EPI == EPI_STORE_F32) {
      if (m < a.M) {
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          const int n = nb + 8 * q;
          if (n < a.N) {
            float4 o = make_float4(acc[4 * q], acc[4 * q + 1], acc[4 * q + 2], acc[4 * q + 3]);
            *reinterpret_cast<float4*>(a.out_f32 + static_cast<size_t>(m) * a.N + n) = o;
          }
        }
      }
    } else if constexpr (EPI == EPI_RESID) {
      if (m < a.M) {
        const uint16_t* rp = nullptr;
        const int tok = a.resid_tok[m];
        if (tok >= 0)
          rp = static_cast<const uint16_t*>(a.resid) +
               static_cast<size_t>(a.resid_by_token ? tok : m) * a.N;
        uint16_t* op = static_cast<uint16_t*>(a.out_res) + static_cast<size_t>(m) * a.N;
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          const int n = nb + 8 * q;
          if (n < a.N) {
            uint2 o = make_uint2(0, 0);
            if (rp) {
              const uint2 r = *reinterpret_cast<const uint2*>(rp + n);
              const float r0 = bf16_to_f32(static_cast<uint16_t>(r.x & 0xFFFF));
              const float r1 = bf16_to_f32(static_cast<uint16_t>(r.x >> 16));
              const float r2 = bf16_to_f32(static_cast<uint16_t>(r.y & 0xFFFF));
              const float r3 = bf16_to_f32(static_cast<uint16_t>(r.y >> 16));
              o.x = static_cast<uint32_t>(f32_to_bf16(r0 + acc[4 * q])) |
                    (static_cast<uint32_t>(f32_to_bf16(r1 + acc[4 * q + 1])) << 16);
              o.y = static_cast<uint32_t>(f32_to_bf16(r2 + acc[4 * q + 2])) |
                    (static_cast<uint32_t>(f32_to_bf16(r3 + acc[4 * q + 3])) << 16);
            }
            *reinterpret_cast<uint2*>(op + n) = o;
          }
        }
      }
    } else {  // EPI_HEAD
      HeadPart p = head_empty();
#pragma unroll
      for (int v = 0; v < 16; ++v) {
        const int n = nb + 8 * (v >> 2) + (v & 3);
        if (n < a.N) {
          p = head_combine(p, head_elem(acc[v], n));
          if (a.logits && m < a.M) a.logits[static_cast<size_t>(m) * a.N + n] = acc[v];
        }
      }
      p = head_combine(p, shfl_part(p, l ^ 32));
      if (g == 0) red[w][h * 32 + li] = p;
    }
  }
  if constexpr (EPI == EPI_HEAD) {
    __syncthreads();
    if (tid < kTileM) {
      HeadPart p = red[0][tid];
#pragma unroll
      for (int q = 1; q < 4; ++q) p = head_combine(p, red[q][tid]);
      const int m = m0 + tid;
      if (m < a.M) {
        float* o = a.part + (static_cast<size_t>(m) * nNT + nt) * 5;
        o[0] = p.m;
        o[1] = __int_as_float(p.am);
        o[2] = p.m2;
        o[3] = p.s;
        o[4] = p.t;
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

int gemm_bf16_n_tiles(int N) { return (N + kTileN - 1) / kTileN; }

glance_status launch_gemm_bf16(const GemmArgs& a, hipStream_t st) {
  const int nNT = gemm_bf16_n_tiles(a.N);
  const int nMT = (a.M + kTileM - 1) / kTileM;
  const int grid = ((nNT + 7) / 8) * 8 * nMT;
  switch (a.epi) {
    case EPI_STORE_F32:
      gemm_bf16_kernel<EPI_STORE_F32><<<grid, kGThreads, 0, st>>>(a, nNT, nMT);
      break;
    case EPI_RESID:
      gemm_bf16_kernel<EPI_RESID><<<grid, kGThreads, 0, st>>>(a, nNT, nMT);
      break;
    default:
      gemm_bf16_kernel<EPI_HEAD><<<grid, kGThreads, 0, st>>>(a, nNT, nMT);
      break;
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
