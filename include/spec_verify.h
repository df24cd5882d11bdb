/*
 * spec_verify.h — C ABI of the batched speculative-decoding verify step on one
 * AMD Instinct MI355X (gfx950).
 *
 * The operations are the verify half of one speculative step as defined in
 *   [SB] "7.6 Speculative Decoding: Draft Models, Medusa, EAGLE & Lookahead"
 *        (LLM stack book): sections "The rule", "The proof that this is exact",
 *        "Extending to a chain of γ draft tokens", "A From-Scratch
 *        Implementation" (apply_temperature, speculative_step), "Tree Attention"
 *        and Exercise 5 (verify_tree_greedy);
 *   [DM] "Speculative Decoding: Draft Models, EAGLE, and How to Actually Use
 *        It": section "The Algorithm" (steps 1–4 and the k=4 worked example);
 *   [SS] "Medusa, EAGLE and self-speculation": "Copying, verified against plain
 *        greedy" (greedy argmax-match verification).
 *
 * Conventions shared by every entry point
 * ---------------------------------------
 * Memory.   Every array argument is a DEVICE pointer owned by the caller. The
 *           library never allocates, frees or synchronizes; all work is enqueued
 *           on `stream` (a hipStream_t, passed as void*; NULL = the null stream)
 *           and the outputs are valid once the caller has synchronized with it.
 * Logits.   Row-major. `dtype` (sv_dtype_t) covers every logits tensor of a
 *           call. Consecutive rows are `row_stride` ELEMENTS apart (>= V); a
 *           row of sequence b at position i starts at element
 *           (b * rows_per_seq + i) * row_stride. Rows whose byte address is a
 *           multiple of 16 take the vectorized path; others are read element by
 *           element (correct, slower).
 * Values.   A logit is any finite value, -inf or +inf, never NaN. -inf marks
 *           a token of probability 0 (a masked entry). Sampled rows are
 *           computed in fp32 from l / T: log-probabilities carry an absolute
 *           rounding error of about |l| / T * 2^-24, so very large positive
 *           logits (|l| / T in the thousands and up) cost accuracy, and l / T
 *           must stay below 2^126 / log2(e). Greedy verification
 *           (temperature 0, spec_verify_greedy, spec_verify_tree) takes the
 *           argmax of any such row, +inf being the largest value. For a
 *           sampled sequence of spec_verify_sample, every row the accept tests
 *           read (target and draft rows 0 .. gamma-1) must define softmax(l / T):
 *           some entry above -inf and none +inf; a NaN anywhere in them is also
 *           caught. A sequence breaking this gets SV_SEQ_BAD_LOGITS, as does
 *           one whose bonus row (read only when every draft is accepted) has no
 *           entry above -inf; a +inf in the bonus row is drawn (the lowest index
 *           among several). spec_verify_tree_sample requires finite or -inf
 *           entries with at least one finite entry per row it reads.
 * Errors.   The return value reports host-side argument validation (done before
 *           any HIP call, so nothing is enqueued on failure) and launch
 *           failures (SV_ERR_HIP). Problems that only the device can see are
 *           reported per sequence in the outputs (see each entry point).
 * Workspace.Each call needs `workspace_bytes >= sv_workspace_bytes(...)` of
 *           device memory, 256-byte aligned, that is ALL ZERO before the first
 *           call (allocate it zeroed, or call sv_workspace_init once). Every
 *           call returns it to all-zero before its last kernel ends, so it can
 *           be reused by later calls of any size that fits. Two calls that use
 *           one workspace must be ordered (same stream); overlapping calls on
 *           one workspace race.
 * Random.   Randomness is counter-based Philox4x32-10 (Salmon et al., SC'11)
 *           with key = (seed low 32 bits, seed high 32 bits) and counter words
 *           (c0, c1, c2, c3) = (c0, position, seq_base + b, 2*offset + stream):
 *             stream 0, c0 = 0       : accept uniform of position i = word 0;
 *             stream 1, c0 = v / 4   : Gumbel noise of vocab entry v = word v%4.
 *           A word w maps to u = (w >> 8) * 2^-24 (accept test, u in [0,1)) or
 *           to U = ((w >> 8) + 0.5) * 2^-24 in (0,1) and Gumbel noise
 *           G = -ln(-ln U). Identical inputs, seed and offset give bitwise
 *           identical outputs, whatever the grid size or run.
 * Determinism of ties. Every argmax takes the LOWEST index among equal values.
 */
#ifndef SPEC_VERIFY_H
#define SPEC_VERIFY_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum { SV_DTYPE_F32 = 0, SV_DTYPE_BF16 = 1 } sv_dtype_t;

typedef enum {
  SV_OK = 0,
  SV_ERR_NULL_ARG = 1,   /* a required pointer is NULL                         */
  SV_ERR_BAD_SHAPE = 2,  /* B, gamma/N, V or max_depth out of range            */
  SV_ERR_BAD_DTYPE = 3,  /* dtype is not an sv_dtype_t value                   */
  SV_ERR_BAD_ARG = 4,    /* row stride < V, offset >= 2^31, seq_base + B > 2^32,
                          * misaligned workspace                             */
  SV_ERR_WORKSPACE = 5,  /* workspace NULL or smaller than sv_workspace_bytes  */
  SV_ERR_HIP = 6,        /* a HIP runtime call or kernel launch failed         */
  SV_ERR_SCRATCH_LIMIT = 7 /* spec_verify_sample_noalloc: the call needs more
                          * than SV_NOALLOC_SCRATCH_BYTES of scratch          */
} sv_status_t;

/* Limits checked on the host. */
#define SV_NOALLOC_SCRATCH_BYTES (32u << 20) /* static scratch of spec_verify_sample_noalloc, per GPU */
#define SV_MAX_GAMMA 16
#define SV_MAX_TREE_NODES 1024
#define SV_MAX_BATCH (1 << 20)

/* Per-sequence device-detected error codes written to out_num_accepted[b]
 * (chains) or out_path_len[b] (trees); the other outputs of b are then -1. */
#define SV_SEQ_BAD_TOKEN (-1)       /* a drafted / node token outside [0, V)      */
#define SV_SEQ_BAD_TEMPERATURE (-2) /* temperature < 0, NaN or infinite           */
#define SV_SEQ_BAD_TREE (-3)        /* parents/depth do not describe a tree       */
#define SV_SEQ_INTERNAL (-4)        /* a bounded device-side wait gave up; the
                                     * workspace is then left dirty and must be
                                     * re-initialized (sv_workspace_init) before
                                     * its next use                               */
#define SV_SEQ_BAD_LOGITS (-5)      /* a sampled sequence's row defines no
                                     * distribution (see "Values" above)         */

/* Optional diagnostics of spec_verify_sample; the struct and each field may
 * be NULL. All are device arrays of fp32. */
typedef struct {
  float* accept_prob;   /* [B, gamma]  a_{b,i} = min(1, p_i(x_i) / q_i(x_i)) for
                         *             every i (not only up to the first
                         *             rejection); greedy sequences: 1 if x_i
                         *             equals the target argmax, else 0.        */
  float* logz_target;   /* [B, gamma]  ln sum_v exp(l_{b,i,v} / T_b) of target
                         *             rows 0..gamma-1; NaN for greedy sequences */
  float* logz_draft;    /* [B, gamma]  the same for draft rows; NaN for greedy
                         *             sequences and for the one-hot draft       */
  float* residual_mass; /* [B]         beta = sum_v (p_v - q_v)_+ at the first
                         *             rejected position (one-hot draft:
                         *             1 - p(x)); NaN when the bonus token was
                         *             drawn or the sequence is greedy           */
} sv_diag_t;

/* Bytes of workspace any entry point needs for B sequences of `rows` logit
 * rows each (gamma + 1 for the chain entry points, N for the tree) over a
 * vocabulary of V. Returns 0 for out-of-range arguments. */
size_t sv_workspace_bytes(int32_t B, int32_t rows, int32_t V);

/* Zero `workspace_bytes` bytes of `workspace` on `stream` (a fill kernel, not
 * hipMemsetAsync). Needed once, before the first call, unless the memory was
 * allocated zeroed. */
sv_status_t sv_workspace_init(void* workspace, size_t workspace_bytes, void* stream);

/* Static description of a status code. Never NULL. */
const char* sv_status_string(sv_status_t status);

/*
 * spec_verify_sample — modified rejection sampling over a batch of chains.
 * [SB] "The rule", "Extending to a chain of γ draft tokens", speculative_step;
 * [DM] "The Algorithm" steps 2–4.
 *
 * For each sequence b with temperature T = temperature[b] > 0:
 *   p_i = softmax(target row i / T), q_i = softmax(draft row i / T), i < gamma;
 *   a_i = min(1, p_i(x_i) / q_i(x_i)), x_i = draft_ids[b, i];
 *   accept x_i iff u_i < a_i (u_i from Philox stream 0 at position i);
 *   n = index of the first rejected position (gamma if none);
 *   if n < gamma: the correction token is drawn from (p_n - q_n)_+ normalized,
 *                 by Gumbel-max over ln((p_n - q_n)_+) with stream-1 noise at
 *                 position n;
 *   else:         the bonus token is drawn from p_gamma = softmax(target row
 *                 gamma / T) by Gumbel-max over l/T with stream-1 noise at
 *                 position gamma.
 *   If rounding leaves (p_n - q_n)_+ empty, the correction is drawn from p_n
 *   instead (same noise). With draft_logits == NULL the draft is one-hot at x_i
 *   ([SB] Exercise 4): a_i = p_i(x_i) and the residual is p_n without x_n.
 * For T == 0 the sequence is verified greedily ([SB] "Extending to a chain of
 * γ draft tokens", its temperature-0 paragraph): x_i is accepted iff it
 * equals argmax_v of target row i (lowest index on ties); the correction is
 * that argmax, the bonus the argmax of row gamma; draft logits and randomness
 * are not used.
 *
 * target_logits  [B, gamma+1, V] rows, stride target_row_stride elements.
 * draft_logits   [B, gamma, V] rows, stride draft_row_stride, or NULL.
 * draft_ids      [B, gamma] int32.
 * temperature    [B] fp32 (device).
 * seed, offset   Philox key and per-step counter word (offset < 2^31).
 * seq_base       counter word 2 of sequence b is seq_base + b (seq_base + B
 *                <= 2^32): a batch split over several calls (or GPUs) gives
 *                each call its first sequence's global index, and the split
 *                calls reproduce the single call bit for bit.
 * out_tokens     [B, gamma+1] int32: x_0 .. x_{n-1}, then the correction or
 *                bonus token, then -1 padding.
 * out_num_accepted [B] int32: n in [0, gamma], or an SV_SEQ_* code (< 0):
 *                SV_SEQ_BAD_TEMPERATURE, SV_SEQ_BAD_TOKEN or SV_SEQ_BAD_LOGITS
 *                (the first that applies), or SV_SEQ_INTERNAL.
 * diag           optional diagnostics (see sv_diag_t), may be NULL.
 */
sv_status_t spec_verify_sample(const void* target_logits, int64_t target_row_stride,
                               const void* draft_logits, int64_t draft_row_stride,
                               sv_dtype_t dtype, const int32_t* draft_ids,
                               const float* temperature, int32_t B, int32_t gamma,
                               int32_t V, uint64_t seed, uint64_t offset, uint32_t seq_base,
                               int32_t* out_tokens, int32_t* out_num_accepted,
                               const sv_diag_t* diag, void* workspace,
                               size_t workspace_bytes, void* stream);

/* spec_verify_sample_noalloc — spec_verify_sample for callers that cannot
 * allocate device memory (code under HIP graph capture, tight serving loops,
 * harnesses that forbid hipMalloc). It takes no workspace: its scratch is a
 * static device array of SV_NOALLOC_SCRATCH_BYTES (32 MiB) that the library
 * holds on every GPU it runs on until the process ends, and it calls no
 * hipMalloc, hipFree or allocating routine. Each call first zeroes the part
 * it uses (sv_workspace_bytes(B, gamma + 1, V) bytes, with a fill kernel on
 * `stream`), so a call that follows an aborted one starts clean. All calls on
 * one GPU share that array: calls that overlap on one GPU (different streams,
 * or host threads) race and must be ordered by the caller. The caller still
 * owns every input and output. Arguments, outputs and errors are those of
 * spec_verify_sample, plus SV_ERR_SCRATCH_LIMIT when the call needs more than
 * SV_NOALLOC_SCRATCH_BYTES (for example B = 512, gamma = 6, V = 152064 needs
 * about 13 MiB). */
sv_status_t spec_verify_sample_noalloc(const void* target_logits, int64_t target_row_stride,
                                       const void* draft_logits, int64_t draft_row_stride,
                                       sv_dtype_t dtype, const int32_t* draft_ids,
                                       const float* temperature, int32_t B, int32_t gamma, int32_t V,
                                       uint64_t seed, uint64_t offset, uint32_t seq_base,
                                       int32_t* out_tokens, int32_t* out_num_accepted,
                                       const sv_diag_t* diag, void* stream);

/* sv_debug_sample_tiled — spec_verify_sample with its tiling fixed by the
 * caller instead of chosen by the library (for tests that check that results
 * do not depend on the tiling; no operation of the pages). p1_vectors: 16-byte
 * vectors per thread in a pass-1 chunk (1, 2, 4 or 8; 0 = chosen); p2_chunks:
 * pass-2 chunks per drawn row (0 = chosen; capped at one per streaming
 * round, i.e. at least one vector per thread in a chunk). Everything else is as for spec_verify_sample; SV_ERR_BAD_ARG for
 * other tiling values. */
sv_status_t sv_debug_sample_tiled(const void* target_logits, int64_t target_row_stride,
                                  const void* draft_logits, int64_t draft_row_stride,
                                  sv_dtype_t dtype, const int32_t* draft_ids,
                                  const float* temperature, int32_t B, int32_t gamma, int32_t V,
                                  uint64_t seed, uint64_t offset, uint32_t seq_base,
                                  int32_t* out_tokens, int32_t* out_num_accepted,
                                  const sv_diag_t* diag, void* workspace, size_t workspace_bytes,
                                  void* stream, int32_t p1_vectors, int32_t p2_chunks);

/*
 * spec_verify_greedy — argmax-match verification of a batch of chains.
 * [SB] "Extending to a chain of γ draft tokens" (temperature 0); [SS]
 * "Copying, verified against plain greedy" (speculative_greedy ; row j of the
 * verify pass predicts the token after position j).
 *
 * g_i = argmax_v target[b, i, v] (lowest index on ties); x_i accepted iff
 * x_i == g_i; n = first mismatch (gamma if none); emitted: x_0..x_{n-1}, then
 * g_n (correction) or g_gamma (bonus). Same output layout as
 * spec_verify_sample; out_num_accepted[b] = SV_SEQ_BAD_TOKEN for a drafted id
 * outside [0, V).
 */
sv_status_t spec_verify_greedy(const void* target_logits, int64_t target_row_stride,
                               sv_dtype_t dtype, const int32_t* draft_ids, int32_t B,
                               int32_t gamma, int32_t V, int32_t* out_tokens,
                               int32_t* out_num_accepted, void* workspace,
                               size_t workspace_bytes, void* stream);

/*
 * spec_verify_tree — greedy verification of a token tree.
 * [SB] "Tree Attention" (accept the longest surviving root-to-leaf path, bonus
 * from the deepest accepted node) and Exercise 5 (verify_tree_greedy: a child
 * is accepted iff its token equals the argmax of the target row of its parent).
 *
 * parents [N] int32 (device): parents[0] = -1, 0 <= parents[i] < i.
 * depth   [N] int32 (device): depth[0] = 0, depth[i] = depth[parents[i]] + 1,
 *         depth[i] <= max_depth.
 * node_tokens [B, N] int32: node_tokens[b, 0] is the committed root (unused).
 * target_logits [B, N, V]: row i predicts the token that follows node i.
 * Rule: g_i = argmax of row i; node 0 is valid; node c > 0 is valid iff its
 * parent is valid and node_tokens[b, c] == g_{parents[c]}. The accepted node is
 * the deepest valid node (smallest index among equally deep ones); the path is
 * its ancestors from the root, and the bonus token is its argmax.
 * out_path     [B, max_depth+1] int32: node indices root first, -1 padded.
 * out_path_len [B] int32: depth(accepted node) + 1, or an SV_SEQ_* code.
 * out_bonus    [B] int32: bonus token, -1 on error.
 */
sv_status_t spec_verify_tree(const void* target_logits, int64_t target_row_stride,
                             sv_dtype_t dtype, const int32_t* parents, const int32_t* depth,
                             const int32_t* node_tokens, int32_t B, int32_t N, int32_t V,
                             int32_t max_depth, int32_t* out_path, int32_t* out_path_len,
                             int32_t* out_bonus, void* workspace, size_t workspace_bytes,
                             void* stream);

/* spec_verify_tree_sample — sampled verification of a draft tree by
 * multi-round rejection sampling ([SB] "Tree Attention": the children of a
 * node are tested one by one; after each rejection the target distribution
 * becomes the normalized residual (p - q)_+ / ||(p - q)_+||_1 and the next
 * sibling is tested against it; if every child is rejected the replacement
 * token is drawn from the final residual; a leaf ends the path with a bonus
 * token drawn from p there). A residual with no mass (p and q equal wherever
 * p is not below q, in the arithmetic of the call) leaves the target
 * distribution as it was.
 *   target_logits: device [B, N, V] (row stride target_row_stride elements):
 *     row v of sequence b scores the token after node v.
 *   draft_logits: device [B, N, V] (row stride draft_row_stride): row v is
 *     the draft distribution q at node v, from which v's children were drawn
 *     (i.i.d.); rows of leaves are not read.
 *   parents, depth: device [N], a tree in parent-before-child order rooted at
 *     node 0 (as for spec_verify_tree); node_tokens: device [B, N], token of
 *     each node (node 0's is not read); temperature: device [B], each > 0.
 *   seed, offset, seq_base: Philox key, per-step counter word and the
 *     global index of the first sequence, as for spec_verify_sample. The accept uniform of the j-th sibling tested under
 *     node v is word 0 of counter (j, v, b, 2 offset); the noise of a draw at
 *     node v is that of position v. A tree shaped like a chain therefore
 *     verifies exactly as spec_verify_sample verifies the chain.
 *   siblings_without_replacement: 0 when a node's children were drawn i.i.d.
 *     from q; 1 when they were drawn without replacement ([SB] "Tree
 *     Attention": q renormalized over the remaining candidates). Then the
 *     j-th sibling's round uses q over the tokens not drawn before it,
 *     renormalized, both in its accept test and in the residual after a
 *     rejection, and siblings must carry distinct tokens (else code -1).
 *   Outputs (device): out_path [B, max_depth + 1] (accepted nodes from the
 *     root, -1 padded), out_path_len [B] (nodes on the path; -1 a node token
 *     out of range, -2 a temperature not > 0, -3 an invalid tree, -4 a bounded
 *     wait gave up), out_token [B] (the bonus or replacement token).
 *   workspace: sv_workspace_bytes(B, N, V) bytes, as for spec_verify_tree.
 * Returns SV_ERR_NULL_ARG, SV_ERR_BAD_SHAPE (B, N, V or max_depth out of
 * range, or a vocabulary too long for one launch), SV_ERR_BAD_DTYPE,
 * SV_ERR_BAD_ARG (a stride < V, offset >= 2^31, seq_base + B > 2^32,
 * siblings_without_replacement not 0 or 1), SV_ERR_WORKSPACE or SV_ERR_HIP; nothing is launched on an error. */
sv_status_t spec_verify_tree_sample(const void* target_logits, int64_t target_row_stride, const void* draft_logits,
                                    int64_t draft_row_stride, sv_dtype_t dtype, const int32_t* parents,
                                    const int32_t* depth, const int32_t* node_tokens, const float* temperature,
                                    int32_t B, int32_t N, int32_t V, int32_t max_depth, uint64_t seed,
                                    uint64_t offset, uint32_t seq_base, int32_t siblings_without_replacement,
                                    int32_t* out_path,
                                    int32_t* out_path_len, int32_t* out_token, void* workspace,
                                    size_t workspace_bytes, void* stream);

/* sv_tree_mask — the attention mask and position ids of a token tree packed
 * into one forward pass ("7.6 Speculative Decoding", "Tree Attention:
 * Verifying Many Candidates at Once", build_tree_attn; "Medusa, EAGLE and
 * self-speculation", "Verifying a tree instead of a line"): node i may attend to node
 * j iff j is i or one of its ancestors, and node i's position id is its depth
 * plus the sequence's offset.
 *   parents: device int32, N entries per sequence, rows parents_stride apart
 *     (0: one tree for every sequence). parents[0] = -1 (the root), and every
 *     other parent is an earlier node.
 *   position_offset [B]: device int32 or NULL (0), e.g. the root's position
 *     in the sequence so that ids continue the committed prefix.
 *   out_mask [B, N, N]: device bytes, 1 = may attend (torch.bool's layout), or
 *     NULL. out_mask_bits [B, N, ceil(N / 32)]: device 32-bit words, column j
 *     at bit j % 32 of word j / 32, or NULL. out_position_ids [B, N]: device
 *     int32 or NULL. At least one output.
 *   A sequence whose tree breaks the order gets an all-zero mask and position
 *   ids -1.
 * Returns SV_ERR_NULL_ARG (parents, or every output, NULL), SV_ERR_BAD_SHAPE
 * (B < 0, N outside 1 .. 1024, a stride below N other than 0) or SV_ERR_HIP;
 * nothing is launched on an error, and nothing is written when B is 0. */
sv_status_t sv_tree_mask(const int32_t* parents, int64_t parents_stride, int32_t B, int32_t N,
                         const int32_t* position_offset, uint8_t* out_mask, uint32_t* out_mask_bits,
                         int32_t* out_position_ids, void* stream);

/* sv_kv_rollback_layers — sv_kv_rollback for caches kept as one tensor per
 * layer (the page's key_cache[l] / value_cache[l]).
 *   k_layers, v_layers: DEVICE arrays of L device pointers, each to a
 *     contiguous, 16-byte aligned [B, H, S, D] cache of elem_bytes elements
 *     (the caller's to keep valid for the call); v_layers may be NULL.
 *   Everything else, the in-place move and the status codes are as for
 *   sv_kv_rollback (the layer pointers themselves cannot be checked on the
 *   host: a misaligned one is the caller's error). */
sv_status_t sv_kv_rollback_layers(void* const* k_layers, void* const* v_layers, int32_t elem_bytes, int32_t L,
                                  int32_t B, int32_t H, int32_t S, int32_t D, const int32_t* root_pos,
                                  const int32_t* path, int32_t P, const int32_t* path_len, int32_t* cache_len,
                                  void* stream);

/* sv_ngram_draft — prompt-lookup / n-gram drafting: one-hot draft proposals
 * copied from earlier in each sequence ("7.6 Speculative Decoding", Exercise
 * 4; "Medusa, EAGLE and self-speculation", "Copying, verified against plain greedy").
 * The last `ngram` tokens of sequence b are looked up at the earlier start
 * positions T - ngram - 1 down to 0; the most recent match i gives the
 * proposal tokens[b][i + ngram ...].
 *   tokens [B, stride] int32, lengths [B] int32: device. Row b holds
 *     lengths[b] tokens; entries from there to the stride are never read.
 *   ngram: 1 .. 16 (1 is the exercise's last-token key; the lookup page uses
 *     3). gamma >= 1: tokens proposed.
 *   pad_with_last = 1 (the exercise): always gamma tokens; positions past the
 *     end of the sequence, and all of them when there is no match (or the
 *     sequence is shorter than ngram + 1), propose the last token again. The
 *     output is a fixed-length one-hot draft (spec_verify_sample with
 *     draft_logits NULL).
 *   pad_with_last = 0 (the lookup page): the continuation, cut at the end of
 *     the sequence; no proposal without a match.
 *   out_draft [B, gamma] (device, out): the proposal, -1 past out_count[b].
 *   out_count [B] (device, out): tokens proposed, or -1 for an invalid length
 *     (below 0, above the stride, or 0 with pad_with_last = 1).
 *   out_match [B] (device, out, may be NULL): the match's start i, or -1.
 * Returns SV_ERR_NULL_ARG, SV_ERR_BAD_SHAPE (B < 0, stride < 1 or above
 * 2^31 - 1, ngram outside 1 .. 16, gamma < 1), SV_ERR_BAD_ARG (pad_with_last
 * not 0 or 1) or SV_ERR_HIP; nothing is launched on an error, and nothing is
 * written when B is 0. */
sv_status_t sv_ngram_draft(const int32_t* tokens, int64_t stride, const int32_t* lengths, int32_t B, int32_t ngram,
                           int32_t gamma, int32_t pad_with_last, int32_t* out_draft, int32_t* out_count,
                           int32_t* out_match, void* stream);

/* sv_kv_rollback — rolls a KV cache back to the accepted tokens after a
 * verify step ([SB] "KV-Cache Reuse and Rollback": a chain step crops every
 * layer's cache to keep = T + n positions; a tree step keeps the accepted
 * root-to-leaf path, gathered along the sequence dimension with the node
 * positions as index).
 *   k_cache, v_cache: device, each [L, B, H, S, D] contiguous elements of
 *     elem_bytes (1, 2 or 4) bytes, 16-byte aligned; v_cache may be NULL.
 *     Node i of sequence b's tree sits at position root_pos[b] + i; node 0,
 *     the root, is the last committed token, whose entry the verify pass
 *     wrote. A chain of gamma drafts is the tree 0 - 1 - ... - gamma.
 *   path [B, P], path_len [B]: device, the verify step's accepted path (root
 *     first), e.g. spec_verify_tree_sample's outputs; for a chain, path =
 *     0 .. n and path_len = n + 1.
 *   In place: for every layer, sequence and head, the entry at position
 *   root_pos[b] + path[b][k] moves to root_pos[b] + k (k < path_len[b]);
 *   positions before the root are untouched, those from the new length on
 *   are left as they were. cache_len[b] (device, out) = root_pos[b] +
 *   path_len[b], the number of valid positions (for a chain, T + n), or -1
 *   when the path is not root-first, strictly increasing and inside the cache
 *   (that sequence is left untouched).
 * Returns SV_ERR_NULL_ARG, SV_ERR_BAD_SHAPE (a dimension < 0, S, D or P < 1,
 * P > 1024, a row of D * elem_bytes bytes not a multiple of 16 or above 16 KiB), SV_ERR_BAD_DTYPE
 * (elem_bytes), SV_ERR_BAD_ARG (a cache not 16-byte aligned) or SV_ERR_HIP;
 * nothing is launched on an error, and nothing is written when L, B or H is 0. */
sv_status_t sv_kv_rollback(void* k_cache, void* v_cache, int32_t elem_bytes, int32_t L, int32_t B, int32_t H,
                           int32_t S, int32_t D, const int32_t* root_pos, const int32_t* path, int32_t P,
                           const int32_t* path_len, int32_t* cache_len, void* stream);

/*
 * Diagnostic entry points: the random primitives of the kernels, element by
 * element, so that they can be checked against their definitions. All arrays
 * are device arrays owned by the caller; work is enqueued on `stream`.
 *
 * sv_debug_philox — out[4i..4i+3] = Philox4x32-10(counter ctr[4i..4i+3],
 *   key key[2i..2i+1]) for i < n (Salmon et al., SC'11).
 * sv_debug_noise — for each 32-bit word w = words[i], i < n:
 *   uniform_out[i] = (w >> 8) * 2^-24 (the accept uniform) and
 *   gumbel_out[i] = -ln(-ln(((w >> 8) + 0.5) * 2^-24)) (the Gumbel noise),
 *   each output optional (NULL).
 * They return SV_ERR_NULL_ARG / SV_ERR_BAD_SHAPE (n < 0) / SV_ERR_HIP.
 */
sv_status_t sv_debug_philox(const uint32_t* ctr, const uint32_t* key, uint32_t* out, int32_t n, void* stream);
sv_status_t sv_debug_noise(const uint32_t* words, float* gumbel_out, float* uniform_out, int32_t n,
                           void* stream);
/* sv_debug_wave_max — for each group w < nwaves of 64 consecutive inputs, one
 * wavefront reduces in[64w .. 64w+63] with the kernels' wave-wide maximum and
 * every lane writes its result: out[64w + j] = max of the group, for all j.
 * in, out: device fp32 arrays of 64 * nwaves elements. */
sv_status_t sv_debug_wave_max(const float* in, float* out, int32_t nwaves, void* stream);
/* sv_debug_read_stream — the read-bandwidth yardstick for the verify kernels
 * (no operation of the pages): reads the `bytes` bytes at src (device,
 * 16-byte aligned, bytes a multiple of 16) once with 16-byte nontemporal
 * loads over a grid of nblocks workgroups of 256 threads (each a contiguous
 * share of the buffer), and writes the XOR
 * of the 32-bit words each wavefront read to out[4 * block + wave] (out:
 * device, 4 * nblocks words). Returns SV_ERR_NULL_ARG, SV_ERR_BAD_SHAPE
 * (nblocks < 1 or bytes not a multiple of 16), SV_ERR_BAD_ARG (src not 16-byte
 * aligned) or SV_ERR_HIP. */
sv_status_t sv_debug_read_stream(const void* src, size_t bytes, uint32_t* out, int32_t nblocks, void* stream);

#ifdef __cplusplus
}
#endif

#endif /* SPEC_VERIFY_H */
