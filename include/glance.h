/*
 * glance.h -- C ABI of the per-round verify path of one-pass block drafting with
 * tree-verified acceptance, for AMD Instinct MI355X (gfx950).
 *
 * Sources.  "The paper" is "Vision Is Not Overhead: One-Pass Block Drafting for
 * Lossless Speculative Decoding in Vision-Language Models" (arXiv 2609.00355);
 * "the project page" is the GLANCE project page.  A round starts from a cached
 * prefix x and a pending root token b (paper §3.1).  The draft head gives one
 * marginal q_j over the vocabulary at every offset j = 1..L (paper §3.2,
 * Assumption 1); the N prefixes of highest plug-in score prod_j q_j(y_j) form a
 * prefix-closed tree S (paper §3.2 Def. 1, §4.2; project page "Verify pass");
 * one ancestor-masked target pass gives every node's row p(. | x o b o y_{1:d});
 * the walk commits the target's greedy tokens Y_{1:A(S)} and emits the next
 * greedy token as the new root (paper Def. 1; App. B.1 proof of Theorem 1).
 *
 * Conventions shared by every call.
 *   - Every pointer argument is a DEVICE pointer unless marked (host).
 *   - Every call is asynchronous in stream order on `stream` (a hipStream_t;
 *     NULL means the default stream).  No call synchronises the host.
 *   - The caller owns every buffer.  The library allocates nothing and keeps no
 *     state between calls; scratch memory is the caller's workspace `ws` of at
 *     least the size the matching *_ws() function returns, aligned to 256 bytes.
 *     A workspace must be zero-filled before its first use: it holds arrival
 *     counters of work-groups that split one reduction, and every call returns
 *     them to zero before it completes, so a workspace stays ready for the next
 *     call.  Calls that share a workspace must not overlap in time.
 *   - Arguments are checked on the host before anything is enqueued.  On error
 *     nothing is launched and a negative glance_status is returned;
 *     glance_last_error() then describes it (per thread).
 *   - Device buffers must be 16-byte aligned.
 *   - dtype GLANCE_F32: every floating tensor is float32.  GLANCE_BF16: stored
 *     tensors (draft logits, embeddings, weights, caches, hidden rows) are
 *     bfloat16; products accumulate in float32; softmax, logits and statistics
 *     are float32.
 *   - Verify rows of a round: row 0 is the root b, rows 1..|S| the tree nodes in
 *     breadth-first order (depth, then parent row, then token id), rows past
 *     n_valid are padding.  A batch of nseq rounds stores its rows back to back,
 *     n_rows = N + 1 per round (row r of round s is global row s*n_rows + r).
 */
#ifndef GLANCE_H
#define GLANCE_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum { GLANCE_F32 = 0, GLANCE_BF16 = 1 } glance_dtype;

typedef enum {
  GLANCE_OK = 0,
  GLANCE_ERR_INVALID_ARG = -1, /* a size, count or pointer is out of range     */
  GLANCE_ERR_ALIGNMENT = -2,   /* a device pointer is not 16-byte aligned       */
  GLANCE_ERR_WORKSPACE = -3,   /* ws is NULL, too small or not 256-byte aligned */
  GLANCE_ERR_UNSUPPORTED = -4, /* a shape this build does not implement         */
  GLANCE_ERR_HIP = -5          /* a HIP launch failed                           */
} glance_status;

#define GLANCE_MAX_L 16     /* offsets per block (the paper uses B = 16, L = 15) */
#define GLANCE_MAX_ROWS 64  /* N + 1 verify rows per round, one 64-bit mask word */

/* ---------------------------------------------------------------- step 1 + 2 --
 * glance_build_tree: log-softmax of every draft marginal, the best tokens of each
 * offset, and the top-N prefix-closed tree with its verify-row layout.
 *
 * Defines (paper §3.2 Assumption 1 and Def. 1; §4.2; project page "Verify
 * pass"): S = the N prefixes y_{1:d}, 1 <= d <= L, of highest plug-in score,
 * ranked in the log domain by score(y_{1:d}) = sum_{j<=d} log q_j(y_j), with
 * log q_j(v) = (z_jv - max_w z_jw) - ln sum_w exp(z_jw - max_w z_jw), all in
 * float32, the score accumulated in depth order.  Equal scores: smaller depth
 * first, then the parent selected earlier, then the token ranked earlier within
 * its offset (larger logit, then smaller token id).  Prefixes whose score is
 * -inf are never selected, so |S| < N is possible.
 *
 *   draft_logits [nseq][L][V]   dtype; the draft head's logits z_j
 *   root_token   [nseq]         int32 in [0, V): b of each round (row 0)
 *   N            tree budget, 0 <= N <= GLANCE_MAX_ROWS - 1 (the root is extra)
 * Outputs ([nseq][N+1] each, row layout above; padding rows: parent -1, depth 0,
 * token -1, anc 0, score -inf):
 *   parent   int32   parent row (-1 for the root)
 *   depth    int32   d of the node (0 for the root)
 *   token    int32   last token y_d (b for the root)
 *   anc      uint64  bit j set iff row j is the row itself or one of its
 *                    ancestors (the root row is an ancestor of every row)
 *   score    float   the node's log plug-in score (0 for the root)
 *   n_valid  [nseq] int32: 1 + |S|
 * Limits: 1 <= L <= GLANCE_MAX_L, nseq >= 1, 2 <= V <= 2^18 (bf16) or 2^17
 * (fp32); larger V returns GLANCE_ERR_UNSUPPORTED.
 */
glance_status glance_build_tree(const void* draft_logits, int32_t dtype,
                                const int32_t* root_token, int32_t nseq, int32_t L,
                                int32_t V, int32_t N, int32_t* parent, int32_t* depth,
                                int32_t* token, uint64_t* anc, float* score,
                                int32_t* n_valid, void* ws, size_t ws_bytes,
                                void* stream);

size_t glance_build_tree_ws(int32_t nseq, int32_t L, int32_t V, int32_t N);

/* glance_build_tree_flag_offset: byte offset, inside a glance_build_tree (or
 * glance_build_tree_shared) workspace of these sizes, of a uint32 word that
 * reports non-finite draft logits: every call ORs in bit 0 when a logit it read
 * is NaN and bit 1 when one is +inf (a -inf logit is a token of probability 0,
 * legal, and not reported).  The word is sticky: the library never clears it;
 * it starts at 0 in a zero-filled workspace, and the caller resets it by
 * writing 0.  The trees of a call that set it are unspecified (NaN has no
 * place in the score order).  Host function, pure; 0 on invalid sizes (the
 * word never sits at offset 0). */
size_t glance_build_tree_flag_offset(int32_t nseq, int32_t L, int32_t V, int32_t N);

/* glance_build_tree_shared: steps 1-2 for a batch of rounds that share one
 * budget of tree nodes (paper App. B.5, Proposition 4 and Eq. 5: under a
 * shared verifier budget the best allocation takes the globally highest node
 * masses, each round's masses indexed by its value V(H)).
 *
 * Defines: sequence s's prefixes carry the key log_weight[s] + sum_j log q_j(y_j)
 * (log_weight[s] = ln V(H_s), e.g. from glance_entropy_log_value; any finite or
 * -inf weights are accepted).  The batch takes the `budget`
 * highest keys, equal keys going to the lower sequence and, within a
 * sequence, following the order of glance_build_tree (score, depth, parent,
 * token); every sequence keeps at most n_max nodes, and keys below
 * min_log_value (the stopping rule, log units; -INFINITY disables it) or equal
 * to -inf are never taken.  Within a sequence the keys fall along that order,
 * so each sequence keeps its own top-n_s tree (prefix-closed), laid out as
 * glance_build_tree lays out a tree of n_max + 1 rows.
 *
 *   log_weight  [nseq] float32, device; not NaN
 *   n_max       0 <= n_max <= GLANCE_MAX_ROWS - 1 (rows per sequence n_max + 1)
 *   budget      >= 0 nodes over the batch (sum_s n_s <= budget)
 *   outputs     as glance_build_tree with N = n_max; n_valid[s] = n_s + 1
 * Limits: 1 <= nseq <= GLANCE_MAX_SHARED; the rest as glance_build_tree, whose
 * workspace size (glance_build_tree_ws) also serves this call.
 */
/* glance_entropy_log_value: the per-round log weights of glance_build_tree_shared
 * from each round's root entropy, through the entropy law of draftability
 * (paper §6, Eq. 2; App. B; App. B.5, Eq. 5 and Proposition 4; project page
 * "An Entropy Law of Draftability"):
 *   p_m(H)   = 1 / (1 + exp(-(b0 - b1 H)))         match probability at the root
 *   E[a | H] = sum_{l=1}^{L} p_m^l                  accepted length, horizon L
 *   V(H)     = E[a | H] (1 - p_m(H)) = p_m (1 - p_m^L)
 *   log_weight[s] = ln V(H_s)                       float32
 * (V is defined up to a factor common to all rounds, which leaves the
 * allocation unchanged.)  V is largest at intermediate entropy: rounds whose
 * acceptance is hopeless or already deep gain least from more width.
 *
 *   entropy     device float32, H_s = entropy[s * stride] in nats (e.g. the
 *               entropy output of glance_verify_head with stride n_rows, row 0
 *               of each sequence); a NaN entropy gives -inf (no width)
 *   nseq >= 1, stride >= 1
 *   b0, b1      the law's intercept and slope (finite; the pages fit b1 > 0)
 *   L >= 1      block horizon (the tree depth)
 *   log_weight  [nseq] device float32 output
 * Pointers 4-byte aligned.  Asynchronous on `stream`.
 */
glance_status glance_entropy_log_value(const float* entropy, int32_t nseq, int32_t stride, float b0,
                                       float b1, int32_t L, float* log_weight, void* stream);

#define GLANCE_MAX_SHARED 16
glance_status glance_build_tree_shared(const void* draft_logits, int32_t dtype,
                                       const int32_t* root_token, const float* log_weight,
                                       int32_t nseq, int32_t L, int32_t V, int32_t n_max,
                                       int32_t budget, float min_log_value, int32_t* parent,
                                       int32_t* depth, int32_t* token, uint64_t* anc, float* score,
                                       int32_t* n_valid, void* ws, size_t ws_bytes, void* stream);

/* -------------------------------------------------------------------- step 3 --
 * glance_tree_attn: one target layer over every verify row of nseq rounds, as a
 * single packed pass with ancestor-only masking.
 *
 * Defines (paper §3.2 Def. 1; App. B.1 proof: ancestor-only masking and token
 * packing change the attention layout, not a row's conditioning): the output of
 * row i equals that of the last position of the explicit causal sequence
 * x o b o y_{1:d(i)}.  The layer, whose internals the pages do not give, is an
 * attention-only residual block:
 *   q = h Wq^T, k = h Wk^T, v = h Wv^T split in heads of D; q and k rotated by
 *   rotate-half RoPE at position P_s + depth(i); query head g reads KV head
 *   g / (Hq / Hkv); a = softmax(q k^T / sqrt(D)) v over the round's prefix keys
 *   and the keys of the rows j with bit j of anc[i] set;
 *   h_out = h_in + concat_g(a_g) Wo^T.
 * bf16 runs round to bf16 at the storage points: each row's new K and V entries
 * and h_out.
 *
 *   layer        weights and prefix cache of this layer (struct below)
 *   embed        [V][d_model] dtype or NULL.  If not NULL the layer input of row
 *                i is embed[token[i]] (first layer) and h_in is ignored.
 *   token        [nseq*n_rows] int32 (tree output; -1 marks a padding row).
 *                Every other value must lie in [0, V): with embed, row i reads
 *                embed[token[i]] unchecked (V is not an argument), so the tree
 *                outputs must hold a built tree, or at least every row marked
 *                as padding, before this call
 *   h_in         [nseq*n_rows][d_model] dtype, or NULL when embed is given
 *   h_out        [nseq*n_rows][d_model] dtype; padding rows are written as 0
 *   kv_offsets   [nseq+1] int64: round s's prefix is cache rows
 *                [kv_offsets[s], kv_offsets[s+1]); P_s = the difference >= 0
 *   max_prefix   (host) an upper bound of every P_s, used to size the launch
 *   depth, anc   [nseq*n_rows] tree outputs
 *   rope_cos/sin [n_pos][D/2] float32 cos/sin of the rotary angles; they must
 *                cover every position P_s + depth (n_pos > max_prefix is checked;
 *                positions outside the table are clamped into it)
 *   attn_out     [nseq*n_rows][Hq*D] float32 or NULL: concat_g(a_g) per row
 *   tree_k/v     [nseq*n_rows][Hkv][D] dtype or NULL: the rows' new cache
 *                entries (k after RoPE)
 * Limits: Hq % Hkv == 0; 1 <= n_rows <= GLANCE_MAX_ROWS.  bf16: D == 128,
 * d_model % 256 == 0, Hq*D % 256 == 0.  f32: D <= 128 even, max_prefix <= 8192.
 */
typedef struct {
  const void* wq;      /* [Hq*D][d_model]  (out x in, row-major) */
  const void* wk;      /* [Hkv*D][d_model]                        */
  const void* wv;      /* [Hkv*D][d_model]                        */
  const void* wo;      /* [d_model][Hq*D]                         */
  const void* k_cache; /* [sum P][Hkv][D], keys already rotated   */
  const void* v_cache; /* [sum P][Hkv][D]                         */
  const void* packed;  /* NULL, or wq/wk/wv/wo as glance_attn_pack wrote them
                          (bf16; then those four are not read)     */
} glance_attn_layer;

glance_status glance_tree_attn(const glance_attn_layer* layer, int32_t dtype,
                               const void* embed, const int32_t* token, const void* h_in,
                               void* h_out, const int64_t* kv_offsets, int64_t max_prefix,
                               const int32_t* depth, const uint64_t* anc,
                               const float* rope_cos, const float* rope_sin, int32_t n_pos,
                               int32_t nseq, int32_t n_rows, int32_t d_model, int32_t Hq,
                               int32_t Hkv, int32_t D, float* attn_out, void* tree_k,
                               void* tree_v, void* ws, size_t ws_bytes, void* stream);

size_t glance_tree_attn_ws(int32_t nseq, int32_t n_rows, int64_t max_prefix,
                           int32_t d_model, int32_t Hq, int32_t Hkv, int32_t D);

/* glance_tree_layer: step 3 with a full decoder layer instead of the
 * attention-only block (bf16).  The pages name the target family (Qwen3-VL-8B)
 * but not its layer internals; this is that family's public decoder-layer
 * shape:
 *   x   = RMSNorm(h) * g_attn                                (bf16)
 *   q, k, v = x Wq^T, x Wk^T, x Wv^T; each q and k head RMSNorm(.) * g_q / g_k,
 *         then rotated as in glance_tree_attn (k and v: bf16 cache entries)
 *   h1  = h + attention Wo^T                                 (bf16)
 *   x2  = RMSNorm(h1) * g_mlp                                (bf16)
 *   act = silu(x2 W_gate^T) * (x2 W_up^T)                    (bf16)
 *   h'  = h1 + act W_down^T                                  (bf16, h_out)
 * with RMSNorm(x) = x / sqrt(mean(x^2) + eps), silu(z) = z / (1 + e^-z) and the
 * attention of glance_tree_attn (same masks, positions, caches).  Arguments as
 * glance_tree_attn; layer->attn holds the attention weights and caches.
 *   g_attn, g_mlp [d_model], g_q, g_k [D]          bf16 gains
 *   w_gate, w_up  [inter][d_model], w_down [d_model][inter]   bf16
 * Limits: D == 128; d_model, Hq*D and inter multiples of 256; eps >= 0.
 * Workspace: glance_tree_layer_ws (zero-filled, as every workspace).
 */
typedef struct {
  glance_attn_layer attn;
  const void* g_attn;
  const void* g_q;
  const void* g_k;
  const void* g_mlp;
  const void* w_gate;
  const void* w_up;
  const void* w_down;
  int32_t inter;
  float eps;
  const void* mlp_packed; /* NULL, or w_gate/w_up/w_down as glance_mlp_pack wrote
                             them (then those three are not read)         */
} glance_full_layer;

glance_status glance_tree_layer(const glance_full_layer* layer, const void* embed,
                                const int32_t* token, const void* h_in, void* h_out,
                                const int64_t* kv_offsets, int64_t max_prefix, const int32_t* depth,
                                const uint64_t* anc, const float* rope_cos, const float* rope_sin,
                                int32_t n_pos, int32_t nseq, int32_t n_rows, int32_t d_model,
                                int32_t Hq, int32_t Hkv, int32_t D, float* attn_out, void* tree_k,
                                void* tree_v, void* ws, size_t ws_bytes, void* stream);

size_t glance_tree_layer_ws(int32_t nseq, int32_t n_rows, int64_t max_prefix, int32_t d_model,
                            int32_t Hq, int32_t Hkv, int32_t D, int32_t inter);

/* glance_attn_pack: the attention weights of a layer (wq, wk, wv, wo, bf16)
 * copied once, at load time, into the projection kernel's tile order, for
 * glance_tree_attn and glance_tree_layer alike: for every block of 16 output
 * rows and 64-deep chunk of the input, the 16 x 64 tile laid out as the
 * matrix-core operand (each weight load a contiguous kilobyte), the tiles of
 * four consecutive blocks side by side and those of one group of four blocks
 * contiguous over all chunks (a work-group's weights are one stream).  The
 * q/k/v blocks pair each head's dims 8j..8j+7 with their rotary partners
 * 64+8j..64+8j+7 (v blocks: 16 consecutive rows).  q/k/v first, then wo at the
 * next 256-byte boundary; size from glance_attn_pack_bytes (0 if unsupported).
 * Results with the packed copy are identical to those with the row-major
 * weights.  Limits: D == 128, Hq % Hkv == 0, d_model and Hq*D multiples of 256.
 */
size_t glance_attn_pack_bytes(int32_t d_model, int32_t Hq, int32_t Hkv, int32_t D);
glance_status glance_attn_pack(const void* wq, const void* wk, const void* wv, const void* wo,
                               int32_t d_model, int32_t Hq, int32_t Hkv, int32_t D, void* packed,
                               void* stream);

/* glance_mlp_pack: the MLP weights of a full layer copied once, at load time,
 * into the projection kernel's tile order (as glance_attn_pack: 16 x 64
 * matrix-core tiles, groups of four 16-row blocks contiguous over the input
 * chunks), the gate/up blocks pairing gate rows 8b..8b+7 with the matching up
 * rows.
 * Gate/up first, then w_down at the next 256-byte boundary; size from
 * glance_mlp_pack_bytes (0 if unsupported).  Results with the packed copy are
 * identical to those with the row-major weights.  Limits: d_model and inter
 * multiples of 256.
 */
size_t glance_mlp_pack_bytes(int32_t d_model, int32_t inter);
glance_status glance_mlp_pack(const void* w_gate, const void* w_up, const void* w_down,
                              int32_t d_model, int32_t inter, void* packed, void* stream);

/* -------------------------------------------------------------------- step 4 --
 * glance_verify_head: LM head of the verify rows with a fused row epilogue.
 *
 * Defines: z = h W_head^T (float32 accumulation).  Per row: the greedy token
 * argmax_v z_v (paper §3.1; the smallest token id on exact ties), its logit top1,
 * the top-2 gap top1 - max_{v != argmax} z_v (paper App. B.1, gamma_k; 0 on an
 * exact tie), and the next-token entropy H = -sum_v p_v ln p_v of p =
 * softmax(z), in nats (paper §6 and the project page's entropy law: H at the
 * round root is row 0 of each round).
 *
 *   h        [R][d_model] dtype (final hidden rows)
 *   w_head   [V][d_model] dtype (out x in)
 *   argmax   [R] int32; top1, gap, entropy [R] float
 *   logits   [R][V] float32 or NULL
 * Limits: R >= 1, V >= 2.  bf16: d_model % 256 == 0.
 */
glance_status glance_verify_head(const void* h, const void* w_head, int32_t dtype,
                                 int32_t R, int32_t d_model, int32_t V, int32_t* argmax,
                                 float* top1, float* gap, float* entropy, float* logits,
                                 void* ws, size_t ws_bytes, void* stream);

size_t glance_verify_head_ws(int32_t R, int32_t V, int32_t d_model, int32_t dtype);

/* glance_verify_head_sampled: the same head, and one token drawn per row from the
 * target's own distribution at temperature T (paper §5.4, Table 3, and App. D:
 * under sampling the committed tokens are the target's draws, so the output
 * distribution is the target's).  Reading taken: row i draws
 *   y_i = argmax_v (z_iv / T + G_iv),  G = -ln(-ln U)   (Gumbel-max rule),
 * with U_iv from Philox4x32-10 (Salmon et al., SC 2011) under key (seed low,
 * seed high 32 bits), counter (v / 4, i, round_id low, round_id high), output
 * word v % 4, and U = ((word >> 9) + 1/2) / 2^23 (exact in float32, so the
 * noise is never infinite).  Every row has its own stream,
 * so a row's draw does not depend on the path that reaches it; pass the draws
 * to glance_accept_walk in place of argmax (and sample_gap in place of gap).
 *
 *   temperature  finite, > 0 (the scores use 1/T in float32)
 *   seed, round_id  Philox key and the round's counter words
 *   sample_tok   [R] int32: y_i (the smallest token id on exact ties)
 *   sample_gap   [R] float: best minus second-best perturbed score of row i
 * All other arguments, the limits and the workspace are those of
 * glance_verify_head (whose outputs this call also writes).
 */
glance_status glance_verify_head_sampled(const void* h, const void* w_head, int32_t dtype,
                                         int32_t R, int32_t d_model, int32_t V,
                                         float temperature, uint64_t seed, uint64_t round_id,
                                         int32_t* argmax, float* top1, float* gap,
                                         float* entropy, int32_t* sample_tok, float* sample_gap,
                                         float* logits, void* ws, size_t ws_bytes, void* stream);

/* glance_head_pack / glance_verify_head_packed: the same LM head (bf16) over
 * weights reordered once, at load time, into the head kernel's own tile order:
 * for every 64-deep chunk of d_model, every wave of the head grid and each of
 * its vocabulary blocks, the 16 x 64 bf16 tile laid out as the matrix-core
 * operand (16 bytes per lane, lanes consecutive).  The kernel then streams the
 * weights from HBM straight into the matrix cores in contiguous kilobytes, with
 * no transposition through LDS.  The layout depends only on (V, d_model); its
 * size is glance_head_pack_bytes(V, d_model) (0 if unsupported), a little above
 * V * d_model * 2 (vocabulary rows padded with zeros to whole wave blocks).
 *
 * glance_head_pack: w_head [V][d_model] bf16 row-major -> w_packed (device,
 * 16-byte aligned, caller-owned, that many bytes).  Limits: V >= 2,
 * d_model % 256 == 0.
 * glance_verify_head_packed: glance_verify_head's outputs, workspace and limits
 * for dtype bf16 (identical results: same products, same accumulation order),
 * from w_packed; with sample_tok and sample_gap not NULL also the draws of
 * glance_verify_head_sampled (temperature, seed and round_id as there; all three
 * ignored when both are NULL).
 */
size_t glance_head_pack_bytes(int32_t V, int32_t d_model);
glance_status glance_head_pack(const void* w_head, int32_t V, int32_t d_model, void* w_packed,
                               void* stream);
glance_status glance_verify_head_packed(const void* h, const void* w_packed, int32_t R,
                                        int32_t d_model, int32_t V, float temperature,
                                        uint64_t seed, uint64_t round_id, int32_t* argmax,
                                        float* top1, float* gap, float* entropy,
                                        int32_t* sample_tok, float* sample_gap, float* logits,
                                        void* ws, size_t ws_bytes, void* stream);

/* glance_verify_head_walk: glance_verify_head_packed followed by
 * glance_accept_walk in the same launches: the head's last row to finish runs
 * the walk of every round (greedy: over argmax and gap; sampling: over
 * sample_tok and sample_gap), so the round needs no separate walk launch.
 * Results equal the two calls made in turn.  `walk` gives the walk's inputs and
 * outputs as glance_accept_walk takes them; R must be walk->nseq *
 * walk->n_rows.  The workspace (glance_verify_head_ws, zero-filled once) holds
 * the arrival word, which every call returns to zero; calls that overlap on
 * one workspace race. */
typedef struct {
  const int32_t* parent;   /* [nseq*n_rows] tree outputs */
  const int32_t* token;
  const int32_t* n_valid;  /* [nseq] */
  int32_t nseq;
  int32_t n_rows;
  int32_t L;
  float gap_flag;          /* as glance_accept_walk (not NaN) */
  int32_t* n_accept;       /* [nseq] */
  int32_t* out_tokens;     /* [nseq][L+1] */
  int32_t* path_rows;      /* [nseq][L+1] */
  int32_t* flagged;        /* [nseq] */
} glance_walk;

glance_status glance_verify_head_walk(const void* h, const void* w_packed, int32_t R,
                                      int32_t d_model, int32_t V, float temperature, uint64_t seed,
                                      uint64_t round_id, int32_t* argmax, float* top1, float* gap,
                                      float* entropy, int32_t* sample_tok, float* sample_gap,
                                      float* logits, const glance_walk* walk, void* ws,
                                      size_t ws_bytes, void* stream);

/* glance_verify_head_packed_noalloc: glance_verify_head_packed without a
 * workspace argument, for callers that cannot allocate device memory (code
 * under HIP graph capture, tight serving loops, harnesses that forbid
 * allocation).  The head's partial statistics go to a fixed device array of
 * 8 MiB inside the library (one per GPU, held until the process ends, found on
 * the first call on each device); the call allocates nothing.  Limit:
 * glance_verify_head_ws(R, V, d_model, GLANCE_BF16) <= 8 MiB (R <= 551 rows at
 * V = 151936); larger sizes return GLANCE_ERR_UNSUPPORTED.  Every call on a GPU
 * shares that GPU's array: calls that overlap on one GPU (concurrent streams,
 * threads) race and must be serialised by the caller.  Arguments, outputs and
 * results are those of glance_verify_head_packed. */
glance_status glance_verify_head_packed_noalloc(const void* h, const void* w_packed, int32_t R,
                                                int32_t d_model, int32_t V, float temperature,
                                                uint64_t seed, uint64_t round_id, int32_t* argmax,
                                                float* top1, float* gap, float* entropy,
                                                int32_t* sample_tok, float* sample_gap,
                                                float* logits, void* stream);

/* -------------------------------------------------------------------- step 5 --
 * glance_accept_walk: the greedy accept walk of every round.
 *
 * Defines (paper §3.2 Def. 1; App. B.1 proof): from the root row r = 0, with
 * y = argmax[r]: if a row c < n_valid has parent r and token y, commit y and
 * descend to c; otherwise emit y as the new root and stop.  This yields
 * A(S) = max{k : Y_{1:j} in S for all j <= k}, the committed Y_{1:A(S)} and the
 * new root Y_{A(S)+1}; a round commits A(S) + 1 tokens (paper §3.1, Eq. (1)).
 * Sibling tokens are distinct, so at most one child matches.
 *
 *   parent, token [nseq*n_rows], n_valid [nseq]: tree outputs
 *   argmax, gap   [nseq*n_rows]: verify-head outputs
 *   gap_flag      a round is flagged when a visited row has gap <= gap_flag (not NaN)
 *                 (near-ties, where packed and unpacked evaluation may pick
 *                 different tokens; paper Theorem 1); <= 0 disables flagging
 * Outputs: n_accept [nseq] = A(S); out_tokens [nseq][L+1] (entries 0..A-1 the
 * committed tokens, entry A the new root, the rest -1); path_rows [nseq][L+1]
 * (entry k = the row whose argmax gave out_tokens[k], the rest -1);
 * flagged [nseq] (0/1).
 * Limits: 1 <= L <= GLANCE_MAX_L, 1 <= n_rows <= GLANCE_MAX_ROWS.
 */
glance_status glance_accept_walk(const int32_t* parent, const int32_t* token,
                                 const int32_t* n_valid, const int32_t* argmax,
                                 const float* gap, int32_t nseq, int32_t n_rows, int32_t L,
                                 float gap_flag, int32_t* n_accept, int32_t* out_tokens,
                                 int32_t* path_rows, int32_t* flagged, void* stream);

/* ------------------------------------------------------- after step 5 --
 * glance_commit_kv: append one round's accepted path to one layer's cache.
 *
 * Defines (paper §3.1; App. B.1, proof of Theorem 1: the next round conditions
 * on x o b o Y_{1:A(S)}): the K and V entries of path rows 0..A (the root b and
 * the A accepted nodes, at positions P..P+A, K already rotated by the verify
 * pass) become cache rows P..P+A of the round's sequence, P = kv_offsets[1].
 * Call it once per layer after glance_accept_walk, then glance_advance_round.
 *
 *   tree_k, tree_v    [n_rows][Hkv][D] dtype: this layer's tree-row K/V (the
 *                     tree_k / tree_v outputs of its glance_tree_attn call)
 *   path_rows, n_accept  glance_accept_walk outputs
 *   kv_offsets        [2] int64: the sequence's prefix is cache rows
 *                     [kv_offsets[0], kv_offsets[1]); read only here
 *   k_cache, v_cache  [cap][Hkv][D] dtype: this layer's caches
 *   cap               (host) rows the caches hold.  The caller keeps
 *                     kv_offsets[1] + L + 1 <= cap; rows at or past cap are
 *                     not written (never out of bounds).
 * Limits: nseq == 1 (several packed sequences have no room to grow in place;
 * other values return GLANCE_ERR_UNSUPPORTED); 1 <= L <= GLANCE_MAX_L;
 * Hkv * D * element size a multiple of 16 bytes.
 */
glance_status glance_commit_kv(const void* tree_k, const void* tree_v, int32_t dtype,
                               const int32_t* path_rows, const int32_t* n_accept, int32_t nseq,
                               int32_t L, int32_t Hkv, int32_t D, const int64_t* kv_offsets,
                               void* k_cache, void* v_cache, int64_t cap, void* stream);

/* glance_advance_round: after every layer's glance_commit_kv, move the prefix
 * end past the committed entries and install the emitted token as the next
 * root: kv_offsets[1] += A + 1; root_token[0] = out_tokens[A] (paper §3.1: a
 * round commits A(S) + 1 tokens, the last being the next round's root).
 *   n_accept [1], out_tokens [L+1]: glance_accept_walk outputs
 *   kv_offsets [2] int64, root_token [1] int32: updated in place
 * Limits: nseq == 1.
 */
glance_status glance_advance_round(const int32_t* n_accept, const int32_t* out_tokens, int32_t nseq,
                                   int64_t* kv_offsets, int32_t* root_token, void* stream);

/* glance_head_timing: a measurement hook for the LM-head GEMM, the kernel that
 * streams the head weights in the verify-head calls above.  start and stop are
 * hipEvent_t handles that the caller created (and keeps alive), or both NULL to
 * stop.  While they are set, every verify-head call records start on its stream
 * just before the head GEMM kernel and stop just after it (before the row merge
 * and the walk), so that hipEventElapsedTime(start, stop) after the call is
 * that kernel's duration.  The setting is process-wide and not synchronised:
 * set it from the thread that makes the calls.  Errors: GLANCE_ERR_INVALID_ARG
 * when exactly one of the two is NULL; a failed record makes the verify-head
 * call return GLANCE_ERR_HIP. */
glance_status glance_head_timing(void* start, void* stop);

/* glance_read_probe: a calibration pass that measures the read bandwidth the
 * device actually delivers to the load kind the LM head streams its weights
 * with (16-byte non-temporal loads), the figure the head's achieved bandwidth
 * is set against beside the nominal peak.  Every 16-byte word of
 * buf[0, bytes) is read once by n_wg work-groups of 256 threads in a
 * grid-stride loop; work-group w writes the XOR of every 32-bit word it read to
 * out[w], so the XOR over out[0, n_wg) is the XOR of the whole buffer.
 *   buf    device pointer; bytes a positive multiple of 16
 *   n_wg   1 .. 65536;  out: n_wg uint32 (device)
 * buf and out 16-byte aligned.
 * Errors: GLANCE_ERR_INVALID_ARG (sizes, NULL), GLANCE_ERR_ALIGNMENT. */
glance_status glance_read_probe(const void* buf, size_t bytes, int32_t n_wg, uint32_t* out,
                                void* stream);

/* ------------------------------------------------------------------ helpers -- */
const char* glance_status_string(int32_t status); /* static text (host)       */
const char* glance_last_error(void);              /* this thread's last error */
int32_t glance_abi_version(void);                 /* 1                        */

#ifdef __cplusplus
}
#endif
#endif /* GLANCE_H */
