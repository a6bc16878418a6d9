// Step 5: the greedy accept walk (paper §3.2 Def. 1; App. B.1, proof of
// Theorem 1).  From the root row, with y the row's greedy token: if the row has
// a child carrying y, commit y and descend; otherwise emit y as the next root
// and stop.  The walk visits at most L + 1 rows, so one wavefront per round
// does it: lane c holds row c's parent and token, and a child lookup is one
// ballot.
//
// After the walk (paper §3.1 and App. B.1: the next round conditions on
// x o b o Y_{1:A}): the K/V entries of the path's rows (the root and the A
// accepted nodes, rotated at positions P..P+A by the verify pass) are appended
// to the cache, then the prefix end moves by A + 1 and the emitted token becomes
// the next root, all on the device.
#include "common.h"
#include "kernels.h"
#include "walk_impl.h"

namespace glance {

namespace {

__global__ __launch_bounds__(kWave) void accept_walk_kernel(WalkArgs w, const int32_t* __restrict__ argmax,
                                                            const float* __restrict__ gap) {
  walk_round(w, argmax, gap, blockIdx.x);
}

// Block k copies the K and V entries of path row k (k <= A) to cache row
// kv_offsets[1] + k; rows at or past the cache's capacity are not written.
__global__ __launch_bounds__(kWave) void commit_kv_kernel(
    const uint4* __restrict__ tree_k, const uint4* __restrict__ tree_v,
    const int32_t* __restrict__ path_rows, const int32_t* __restrict__ n_accept,
    const int64_t* __restrict__ kv_offsets, int64_t cap, int row_vec, uint4* __restrict__ k_cache,
    uint4* __restrict__ v_cache) {
  // the three index loads are independent (path_rows has L + 1 >= gridDim.x
  // entries), so they are issued together
  const int k = blockIdx.x;
  const int a = n_accept[0];
  const int64_t dst = kv_offsets[1] + k;
  const int prow = path_rows[k];
  if (k > a) return;
  if (dst < 0 || dst >= cap) return;
  const size_t src = static_cast<size_t>(prow) * row_vec;
  for (int i = threadIdx.x; i < row_vec; i += kWave) {
    k_cache[static_cast<size_t>(dst) * row_vec + i] = tree_k[src + i];
    v_cache[static_cast<size_t>(dst) * row_vec + i] = tree_v[src + i];
  }
}

__global__ void advance_round_kernel(const int32_t* __restrict__ n_accept,
                                     const int32_t* __restrict__ out_tokens,
                                     int64_t* __restrict__ kv_offsets, int32_t* __restrict__ root) {
  const int a = n_accept[0];
  kv_offsets[1] += a + 1;
  root[0] = out_tokens[a];
}

}  // namespace

glance_status launch_commit_kv(const void* tree_k, const void* tree_v, const int32_t* path_rows,
                               const int32_t* n_accept, const int64_t* kv_offsets, int64_t cap,
                               int L, size_t row_bytes, void* k_cache, void* v_cache,
                               hipStream_t st) {
  commit_kv_kernel<<<L + 1, kWave, 0, st>>>(
      static_cast<const uint4*>(tree_k), static_cast<const uint4*>(tree_v), path_rows, n_accept,
      kv_offsets, cap, static_cast<int>(row_bytes / sizeof(uint4)), static_cast<uint4*>(k_cache),
      static_cast<uint4*>(v_cache));
  GLANCE_LAUNCH_CHECK();
  return GLANCE_OK;
}

glance_status launch_advance_round(const int32_t* n_accept, const int32_t* out_tokens,
                                   int64_t* kv_offsets, int32_t* root, hipStream_t st) {
  advance_round_kernel<<<1, 1, 0, st>>>(n_accept, out_tokens, kv_offsets, root);
  GLANCE_LAUNCH_CHECK();
  return GLANCE_OK;
}

// Read-bandwidth calibration: a grid-stride pass over n16 16-byte words with
// the LM head's non-temporal loads, four words per thread in flight per step
// (an index past the end re-reads the last word and adds nothing), the XOR of
// each work-group's words into out[work-group].
__global__ __launch_bounds__(256) void read_probe_kernel(const uint4* __restrict__ p, size_t n16,
                                                         uint32_t* __restrict__ out) {
  constexpr int U = 4;
  const size_t stride = static_cast<size_t>(gridDim.x) * 256 * U;
  uint32_t acc = 0;
  for (size_t i = static_cast<size_t>(blockIdx.x) * 256 * U + threadIdx.x; i < n16; i += stride) {
    uint4 v[U];
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const size_t k = i + static_cast<size_t>(u) * 256;
      v[u] = load_stream(p + (k < n16 ? k : n16 - 1));
    }
#pragma unroll
    for (int u = 0; u < U; ++u)
      if (i + static_cast<size_t>(u) * 256 < n16) acc ^= v[u].x ^ v[u].y ^ v[u].z ^ v[u].w;
  }
  __shared__ uint32_t red[256 / kWave];
#pragma unroll
  for (int off = 32; off > 0; off >>= 1) acc ^= static_cast<uint32_t>(__shfl_xor(static_cast<int>(acc), off, kWave));
  if ((threadIdx.x & (kWave - 1)) == 0) red[threadIdx.x / kWave] = acc;
  __syncthreads();
  if (threadIdx.x == 0) out[blockIdx.x] = red[0] ^ red[1] ^ red[2] ^ red[3];
}

glance_status launch_read_probe(const void* buf, size_t bytes, int n_wg, uint32_t* out, hipStream_t st) {
  read_probe_kernel<<<n_wg, 256, 0, st>>>(static_cast<const uint4*>(buf), bytes / 16, out);
  GLANCE_LAUNCH_CHECK();
  return GLANCE_OK;
}

glance_status launch_accept_walk(const int32_t* parent, const int32_t* token,
                                 const int32_t* n_valid, const int32_t* argmax,
                                 const float* gap, int nseq, int n_rows, int L, float gap_flag,
                                 int32_t* n_accept, int32_t* out_tokens, int32_t* path_rows,
                                 int32_t* flagged, hipStream_t st) {
  WalkArgs w;
  w.parent = parent;
  w.token = token;
  w.n_valid = n_valid;
  w.nseq = nseq;
  w.n_rows = n_rows;
  w.L = L;
  w.gap_flag = gap_flag;
  w.n_accept = n_accept;
  w.out_tokens = out_tokens;
  w.path_rows = path_rows;
  w.flagged = flagged;
  accept_walk_kernel<<<nseq, kWave, 0, st>>>(w, argmax, gap);
  GLANCE_LAUNCH_CHECK();
  return GLANCE_OK;
}

}  // namespace glance
