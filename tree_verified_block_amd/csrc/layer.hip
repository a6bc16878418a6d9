// The parts of a full decoder layer around the projections and the attention:
// RMSNorm of the verify rows and the q/k head normalisation with RoPE.
//
// The pages name the target family but not its layer internals; the full
// layer follows that family's public decoder-layer shape: RMSNorm(h) g_attn
// before the q/k/v projection, every q and k head RMS-normalised with its own
// gain before the rotation, and RMSNorm(h1) g_mlp before a SwiGLU MLP, with
// RMSNorm(x) = x / sqrt(mean(x^2) + eps).  The normalised rows, the rotated k,
// v and every layer output are bf16 storage points.
#include <hip/hip_runtime.h>

#include "common.h"
#include "kernels.h"

namespace glance {

namespace {

constexpr int kNormThreads = 256;

// One work-group per row: out[m] = bf16(x[m] / sqrt(mean(x[m]^2) + eps) * g),
// x[m] the row itself or, with gather, x[gather[m]]; rows whose token is
// negative (padding) are written as 0.  d is a multiple of 8.
__global__ __launch_bounds__(kNormThreads) void rmsnorm_kernel(const uint16_t* __restrict__ x,
                                                               const int32_t* __restrict__ gather,
                                                               const int32_t* __restrict__ token,
                                                               int d, const uint16_t* __restrict__ g,
                                                               float eps, uint16_t* __restrict__ out) {
  __shared__ float red[kNormThreads / kWave];
  const int m = blockIdx.x, tid = threadIdx.x;
  const int src = gather ? gather[m] : m;
  const bool live = token[m] >= 0 && src >= 0;
  const uint16_t* xr = x + static_cast<size_t>(live ? src : 0) * d;
  const int nv = d / 8;
  float ss = 0.f;
  for (int v = tid; v < nv; v += kNormThreads) {
    const uint4 u = *reinterpret_cast<const uint4*>(xr + 8 * v);
    const uint32_t w[4] = {u.x, u.y, u.z, u.w};
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const float a = bf16_to_f32(w[j] & 0xFFFF), b = bf16_to_f32(w[j] >> 16);
      ss = fmaf(a, a, fmaf(b, b, ss));
    }
  }
  ss = wave_sum(ss);
  if ((tid & (kWave - 1)) == 0) red[tid / kWave] = ss;
  __syncthreads();
  float tot = 0.f;
#pragma unroll
  for (int i = 0; i < kNormThreads / kWave; ++i) tot += red[i];
  const float r = live ? 1.f / sqrtf(tot / static_cast<float>(d) + eps) : 0.f;
  uint16_t* orow = out + static_cast<size_t>(m) * d;
  for (int v = tid; v < nv; v += kNormThreads) {
    const uint4 u = *reinterpret_cast<const uint4*>(xr + 8 * v);
    const uint4 gv = *reinterpret_cast<const uint4*>(g + 8 * v);
    const uint32_t w[4] = {u.x, u.y, u.z, u.w}, gw[4] = {gv.x, gv.y, gv.z, gv.w};
    uint32_t o[4];
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const float a = bf16_to_f32(w[j] & 0xFFFF) * r * bf16_to_f32(gw[j] & 0xFFFF);
      const float b = bf16_to_f32(w[j] >> 16) * r * bf16_to_f32(gw[j] >> 16);
      o[j] = pack_bf16x2(a, b);
    }
    *reinterpret_cast<uint4*>(orow + 8 * v) = make_uint4(o[0], o[1], o[2], o[3]);
  }
}

// One wave per (row, head) of the fp32 projections qkv [R][(Hq + 2 Hkv) 128]:
// q and k heads are RMS-normalised with their gain, then rotated at the row's
// position P_s + depth (clamped into the tables) and rounded to bf16; v heads
// are rounded.  Lane l holds dims l and l + 64, the rotate-half partners.
__global__ __launch_bounds__(kNormThreads) void qkv_finish_kernel(
    const float* __restrict__ qkv, int R, int Hq, int Hkv, const uint16_t* __restrict__ g_q,
    const uint16_t* __restrict__ g_k, float eps, const int64_t* __restrict__ kv_offsets,
    const int32_t* __restrict__ depth, int n_rows, const float* __restrict__ rope_cos,
    const float* __restrict__ rope_sin, int n_pos, uint16_t* __restrict__ q_out,
    uint16_t* __restrict__ q_lo_out, uint16_t* __restrict__ k_out, uint16_t* __restrict__ v_out) {
  const int nh = Hq + 2 * Hkv;
  const int item = blockIdx.x * (kNormThreads / kWave) + threadIdx.x / kWave;
  if (item >= R * nh) return;  // (wave-uniform)
  const int row = item / nh, head = item - row * nh, l = threadIdx.x & (kWave - 1);
  const float* src = qkv + static_cast<size_t>(row) * nh * 128 + head * 128;
  float a = src[l], b = src[l + 64];
  if (head < Hq + Hkv) {
    const uint16_t* g = head < Hq ? g_q : g_k;
    const float r = 1.f / sqrtf(wave_sum(fmaf(a, a, b * b)) / 128.f + eps);
    a *= r * bf16_to_f32(g[l]);
    b *= r * bf16_to_f32(g[l + 64]);
    const int s = row / n_rows;
    int p = static_cast<int>(kv_offsets[s + 1] - kv_offsets[s]) + depth[row];
    p = p < 0 ? 0 : (p > n_pos - 1 ? n_pos - 1 : p);
    const float c = rope_cos[static_cast<size_t>(p) * 64 + l], sn = rope_sin[static_cast<size_t>(p) * 64 + l];
    const float ra = a * c - b * sn, rb = b * c + a * sn;
    const size_t o = head < Hq ? (static_cast<size_t>(row) * Hq + head) * 128
                               : (static_cast<size_t>(row) * Hkv + (head - Hq)) * 128;
    uint16_t* dst = (head < Hq ? q_out : k_out) + o;
    const uint16_t qa = f32_to_bf16(ra), qb = f32_to_bf16(rb);
    dst[l] = qa;
    dst[l + 64] = qb;
    if (head < Hq) {  // q also leaves its rounding remainder (q = hi + lo in the scores)
      q_lo_out[o + l] = f32_to_bf16(ra - bf16_to_f32(qa));
      q_lo_out[o + l + 64] = f32_to_bf16(rb - bf16_to_f32(qb));
    }
  } else {
    uint16_t* dst = v_out + (static_cast<size_t>(row) * Hkv + (head - Hq - Hkv)) * 128;
    dst[l] = f32_to_bf16(a);
    dst[l + 64] = f32_to_bf16(b);
  }
}

}  // namespace

glance_status launch_rmsnorm(const void* x, const int32_t* gather, const int32_t* token, int M,
                             int d, const void* g, float eps, void* out, hipStream_t st) {
  rmsnorm_kernel<<<M, kNormThreads, 0, st>>>(static_cast<const uint16_t*>(x), gather, token, d,
                                             static_cast<const uint16_t*>(g), eps,
                                             static_cast<uint16_t*>(out));
  GLANCE_LAUNCH_CHECK();
  return GLANCE_OK;
}

glance_status launch_qkv_finish(const float* qkv, int R, int Hq, int Hkv, const void* g_q,
                                const void* g_k, float eps, const int64_t* kv_offsets,
                                const int32_t* depth, int n_rows, const float* rope_cos,
                                const float* rope_sin, int n_pos, void* q_out, void* q_lo_out,
                                void* k_out, void* v_out, hipStream_t st) {
  const int items = R * (Hq + 2 * Hkv);
  const int per = kNormThreads / kWave;
  qkv_finish_kernel<<<(items + per - 1) / per, kNormThreads, 0, st>>>(
      qkv, R, Hq, Hkv, static_cast<const uint16_t*>(g_q), static_cast<const uint16_t*>(g_k), eps,
      kv_offsets, depth, n_rows, rope_cos, rope_sin, n_pos, static_cast<uint16_t*>(q_out),
      static_cast<uint16_t*>(q_lo_out), static_cast<uint16_t*>(k_out), static_cast<uint16_t*>(v_out));
  GLANCE_LAUNCH_CHECK();
  return GLANCE_OK;
}

}  // namespace glance
