// Internal launchers of libglance; the C ABI in glance.cpp validates every
// argument before calling these.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

#include "glance.h"

namespace glance {

// ------------------------------------------------------------------ tree.hip
struct TreeWs {
  // per-chunk (max, sum exp) [nseq*L][16], sorted key lists [nseq*L][16][64],
  // merged rows (log q [nseq*L][64], token ids [nseq*L][64]), the arrival
  // counters of the rows [nseq*L] and sequences [nseq] (zero between calls),
  // for a shared budget the published selections [nseq][64] and the batch
  // counter, and the sticky non-finite flag word (bit 0 NaN, bit 1 +inf logits)
  size_t off_cstat = 0, off_clist = 0, off_lq = 0, off_tk = 0, off_row_cnt = 0, off_seq_cnt = 0,
         off_pops = 0, off_batch_cnt = 0, off_flag = 0, bytes = 0;
};
// Sequences of one shared-budget batch (the cut keeps their keys in LDS).
constexpr int kMaxShared = GLANCE_MAX_SHARED;
TreeWs tree_ws_layout(int nseq, int L, int V);
glance_status launch_build_tree(const void* logits, int dtype, const int32_t* root, int nseq,
                                int L, int V, int N, int32_t* parent, int32_t* depth,
                                int32_t* token, uint64_t* anc, float* score,
                                int32_t* n_valid, void* ws, hipStream_t st,
                                const float* log_weight = nullptr, int budget = 0,
                                float tau = 0.f);

// ------------------------------------------------------------------ gemm.hip
// C = X W^T with X [M][K] (rows optionally gathered by token id) and W the
// concatenation along N of up to three [n_i][K] row-major segments.
struct GemmSeg {
  const void* w[3];
  int n_end[3];  // cumulative row counts
  int nseg;
};
// EPI_SWIGLU (bf16): W = [W_gate; W_up] (two segments of N/2 rows); the output
// out_res [M][N/2] is silu(x W_gate^T) * (x W_up^T) rounded to bf16.
enum GemmEpi { EPI_STORE_F32 = 0, EPI_RESID = 1, EPI_HEAD = 2, EPI_QKV = 3, EPI_SWIGLU = 4 };
struct GemmArgs {
  const void* x;          // [M][K] in the storage dtype, or fp32 when x_f32
  bool x_f32;             // bf16 projections: X is fp32, used as the sum of two bf16
                          // matrices (its bf16 rounding and the remainder)
  const int32_t* gather;  // NULL or [M] token ids (row m of X = x[gather[m]], -1 = zero row)
  GemmSeg w;
  int M, N, K;
  int epi;
  float* out_f32;          // EPI_STORE_F32: [M][N]
  const void* resid;       // EPI_RESID: residual rows, [M][N] or a table indexed by token
  const int32_t* resid_tok;  // EPI_RESID: [M] token ids; rows with token < 0 are written as 0
  bool resid_by_token;     // residual row m is resid[resid_tok[m]] (else resid[m])
  void* out_res;           // EPI_RESID: [M][N] in the storage dtype
  // bf16: W in the kernel's packed tile order (glance_head_pack for the head,
  // glance_mlp_pack for the MLP projections), or null for row-major W
  const void* w_packed;
  float* part;             // EPI_HEAD: [M][n_part] partial statistics (5 floats)
  float* logits;           // EPI_HEAD: optional [M][N]
  // EPI_HEAD, sampling at temperature T: [M][n_part] partial draws (3 floats:
  // best perturbed score, its token, second best), 1/T, Philox key and round
  float* spart;
  float inv_temp;
  uint32_t seed_lo, seed_hi, rnd_lo, rnd_hi;
  // EPI_QKV (bf16, head_dim 128): W = [Wq; Wk; Wv]; q and k rotated at the row's
  // position, everything rounded to bf16; q also leaves its rounding remainder.
  int Hq, Hkv;
  void* q_out;             // [M][Hq*128]
  void* q_lo_out;          // [M][Hq*128]: q - bf16(q), rounded to bf16
  void* k_out;             // [M][Hkv][128]
  void* v_out;             // [M][Hkv][128]
  const int64_t* kv_offsets;
  const int32_t* depth;
  int n_rows;
  const float* rope_cos;
  const float* rope_sin;
  int n_pos;
  // EPI_QKV / EPI_RESID (bf16): split-K partials and one arrival counter per
  // group of work-groups (zero before the call; the call leaves them zero)
  float* kpart;
  unsigned* kcnt;
};
// ln V(H) of the entropy law for nseq entropies H[s * stride].
glance_status launch_entropy_log_value(const float* H, int nseq, int stride, float b0, float b1,
                                       int L, float* out, hipStream_t st);
// Number of per-row partial records the bf16 LM-head GEMM leaves (the merge input).
int gemm_bf16_head_parts(int N);
// The head's scratch for callers that cannot allocate: a fixed device array of
// kHeadScratchFloats floats (8 MiB), its address on the current device.
constexpr size_t kHeadScratchFloats = size_t(1) << 21;
glance_status head_scratch_ptr(float** out);
// Bytes of the packed LM-head weights for N vocabulary rows of K (bf16), and the
// packing kernel (row-major [N][K] -> packed tile order).
size_t head_pack_bytes(int N, int K);
glance_status launch_head_pack(const void* w, int N, int K, void* w_packed, hipStream_t st);
// Bytes of a packed projection weight (N output rows of K, bf16) and its packing
// kernel (in the block order of a.epi: EPI_SWIGLU pairs gate and up rows).
size_t proj_pack_bytes(int N, int K);
glance_status launch_proj_pack(const GemmArgs& a, void* w_packed, hipStream_t st);
glance_status launch_gemm_bf16(const GemmArgs& a, hipStream_t st);
// Scratch of the bf16 projections: number of 16-row weight blocks, K-split,
// partial floats and arrival counters for M activation rows.
int proj_blocks(const GemmArgs& a);
struct ProjGrid {
  int bpg;  // 16-row blocks per group (4 or 3)
  int NGr;  // groups
  int S;    // K-slices
};
ProjGrid proj_grid(int K, int NB);
size_t proj_part_floats(int M, int NB, int K);
size_t proj_counters(int M, int NB, int K);
glance_status launch_gemm_f32(const GemmArgs& a, hipStream_t st);
// Sampling outputs of the head: token drawn per row and the gap between its
// perturbed score and the next one (null when not sampling).
struct HeadDraw {
  int32_t* tok = nullptr;
  float* gap = nullptr;
  const float* spart = nullptr;  // bf16 path: partial draws
  float inv_temp = 1.f;
  uint32_t seed_lo = 0, seed_hi = 0, rnd_lo = 0, rnd_hi = 0;
};
// Row statistics of the head from bf16 partials, or from full fp32 logits.
glance_status launch_head_merge(const float* part, int n_tiles, int R, int32_t* argmax,
                                float* top1, float* gap, float* entropy, const HeadDraw& dr,
                                hipStream_t st);
struct WalkArgs;
// The merge with the accept walk of every round fused behind it (the last row
// to arrive walks); `arrivals` is a zero word the kernel returns to zero.
glance_status launch_head_merge_walk(const float* part, int n_tiles, int R, int32_t* argmax,
                                     float* top1, float* gap, float* entropy, const HeadDraw& dr,
                                     const WalkArgs& wk, unsigned* arrivals, hipStream_t st);
glance_status launch_head_rowstats_f32(const float* logits, int R, int V, int32_t* argmax,
                                       float* top1, float* gap, float* entropy,
                                       const HeadDraw& dr, hipStream_t st);

// ------------------------------------------------------------------ attn.hip
struct AttnArgs {
  int dtype;
  const float* qkv;        // fp32 path: [R][(Hq + 2 Hkv) D] projections (before RoPE)
  const void* q;           // bf16 path: [R][Hq D] rotated queries rounded to bf16 (tree K/V in tree_k/v)
  const void* q_lo;        // bf16 path: [R][Hq D] the rounding remainder q - bf16(q), in bf16
  const void* k_cache;     // [sum P][Hkv][D]
  const void* v_cache;
  const int64_t* kv_offsets;
  const int32_t* depth;
  const uint64_t* anc;
  const int32_t* token;    // -1 marks padding rows
  const float* rope_cos;
  const float* rope_sin;
  int n_pos;               // table rows (the host checks max_prefix + n_rows <= n_pos)
  int nseq, n_rows, Hq, Hkv, D;
  int64_t max_prefix;      // prefixes longer than this are read as this long
  int n_split;             // bf16: key splits per (sequence, KV head, query block)
  float* part;             // bf16, n_split > 1: partial (m, l, o[D]) per split and query
  float* attn_out;         // NULL or [R][Hq D] fp32
  float* attn_x;           // [R][Hq D] fp32: input of the output projection
  void* tree_k;            // [R][Hkv][D]: written by the fp32 path (if not NULL), read by bf16
  void* tree_v;
  unsigned* arrivals;      // bf16: arrival counters of the in-kernel split merge (zero-filled,
                           // returned to zero), attn_arrival_words of them
};
// Key splits of the bf16 attention (from the grid and the longest prefix), and
// the floats of its split records.
int attn_splits(int nseq, int64_t max_prefix, int n_rows, int Hq, int Hkv);
size_t attn_part_floats(int nseq, int n_rows, int Hq, int Hkv, int n_split);
size_t attn_arrival_words(int nseq, int n_rows, int Hq, int Hkv);
glance_status launch_tree_attention(const AttnArgs& a, hipStream_t st);

// ----------------------------------------------------------------- layer.hip
// out[m] = bf16(RMSNorm(x[gather ? gather[m] : m]) * g); rows with token[m] < 0 -> 0
glance_status launch_rmsnorm(const void* x, const int32_t* gather, const int32_t* token, int M,
                             int d, const void* g, float eps, void* out, hipStream_t st);
// fp32 q/k/v [R][(Hq + 2 Hkv) 128] -> head-normalised, rotated bf16 q (and its
// rounding remainder), k and bf16 v
glance_status launch_qkv_finish(const float* qkv, int R, int Hq, int Hkv, const void* g_q,
                                const void* g_k, float eps, const int64_t* kv_offsets,
                                const int32_t* depth, int n_rows, const float* rope_cos,
                                const float* rope_sin, int n_pos, void* q_out, void* q_lo_out,
                                void* k_out, void* v_out, hipStream_t st);

// ------------------------------------------------------------------ walk.hip
glance_status launch_accept_walk(const int32_t* parent, const int32_t* token,
                                 const int32_t* n_valid, const int32_t* argmax,
                                 const float* gap, int nseq, int n_rows, int L, float gap_flag,
                                 int32_t* n_accept, int32_t* out_tokens, int32_t* path_rows,
                                 int32_t* flagged, hipStream_t st);
glance_status launch_commit_kv(const void* tree_k, const void* tree_v, const int32_t* path_rows,
                               const int32_t* n_accept, const int64_t* kv_offsets, int64_t cap,
                               int L, size_t row_bytes, void* k_cache, void* v_cache,
                               hipStream_t st);
glance_status launch_advance_round(const int32_t* n_accept, const int32_t* out_tokens,
                                   int64_t* kv_offsets, int32_t* root, hipStream_t st);
glance_status launch_read_probe(const void* buf, size_t bytes, int n_wg, uint32_t* out,
                                hipStream_t st);

}  // namespace glance
