/*
 * specverify.h -- C ABI of libspecverify: the batched verify-and-sample step of
 * speculative decoding and the MTP token shift/insert, on AMD Instinct MI355X
 * (gfx950).
 *
 * The operations are those of "Accelerating Sonar through speculation"
 * (Perplexity Research, 2025): a target model scores n drafted tokens plus one
 * bonus position in one pass; the longest acceptable prefix is kept and the
 * target supplies one more token (Speculative decoding section, second paragraph
 * and the four inference stages).  The acceptance test and the residual
 * distribution are those of "Fast Inference from Transformers via Speculative
 * Decoding", the first reference that page lists.
 *
 * Conventions shared by every entry point
 *   - Every array argument is DEVICE memory owned by the caller, row-major and
 *     contiguous.  The library never allocates, frees or synchronises: each call
 *     validates its host-side arguments, enqueues kernels on `stream` (a
 *     hipStream_t; NULL means the null stream) and returns.  Outputs are ready
 *     when the stream reaches them.
 *   - Logits are IEEE binary32 (SV_F32) or bfloat16 (SV_BF16).  bfloat16 is
 *     widened to binary32 exactly; all arithmetic is binary32 except the
 *     per-sequence decision, which is binary64.
 *   - Status codes report host-checkable errors synchronously: SV_EINVAL for a
 *     NULL required pointer, B < 0, n outside [0, SV_MAX_DRAFT], V < 1, H < 0,
 *     an unknown dtype or sizes whose element count overflows; SV_EALIGN for a
 *     pointer not aligned to its element type; SV_EWORKSPACE when the workspace
 *     is NULL or smaller than sv_workspace_bytes(); SV_EHIP when a launch fails
 *     (the HIP error string is then available from sv_last_hip_error()).  On
 *     any non-OK status nothing has been enqueued by the failing call.  Kernel
 *     faults surface at the caller's next synchronisation.
 *   - Values that live on the device cannot be checked synchronously.  They
 *     follow fixed fallback rules and set bits in *err_flags (OR-ed in; the
 *     caller clears the word):
 *       draft_lens[b] outside [0, n]   -> clamped                SV_FLAG_LEN_CLAMPED
 *       draft token outside [0, V)     -> rejected at its slot   SV_FLAG_TOKEN_OOR
 *       temperature < 0 or NaN         -> treated as 0 (greedy)  SV_FLAG_BAD_TEMP
 *       uniform NaN or < 0 / >= 1      -> 0 / largest float < 1  SV_FLAG_BAD_UNIFORM
 *       residual mass not positive     -> draw from p_k          SV_FLAG_ZERO_RESIDUAL
 *       row_index[b] outside [0, R)    -> clamped                SV_FLAG_ROW_CLAMPED
 *   - Rows the step does not need never enter a result: target rows r > L_b,
 *     draft rows r >= L_b, and draft rows of sequences with T_b = 0.  The
 *     sampling calls never load them; the greedy calls may fetch the first few
 *     KB of an unneeded target row (its loads start before the draft length has
 *     arrived) and discard them, so those rows must be allocated (they are: the
 *     target buffer is [B][n+1][V]) but may hold anything, NaN included.
 *   - Calls that share one workspace must not overlap in time (same stream, or
 *     ordered by events).
 */
#ifndef SPECVERIFY_H
#define SPECVERIFY_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define SV_MAX_DRAFT 64

typedef enum { SV_F32 = 0, SV_BF16 = 1 } sv_dtype_t;

typedef enum {
    SV_OK = 0,
    SV_EINVAL = 1,
    SV_EALIGN = 2,
    SV_EWORKSPACE = 3,
    SV_EHIP = 4
} sv_status_t;

enum {
    SV_FLAG_LEN_CLAMPED = 1,
    SV_FLAG_TOKEN_OOR = 2,
    SV_FLAG_BAD_TEMP = 4,
    SV_FLAG_BAD_UNIFORM = 8,
    SV_FLAG_ZERO_RESIDUAL = 16,
    SV_FLAG_ROW_CLAMPED = 32,
    SV_FLAG_BAD_PARENT = 64,
    SV_FLAG_TREE_TRUNCATED = 128
};

/* Bytes of device workspace spec_verify_sample() and spec_verify_greedy() need
 * for these sizes (0 on invalid sizes).  The workspace holds per-chunk partial
 * results and per-sequence arrival counters.  It must be filled with zero bytes
 * before its first use (hipMemset, or sv_workspace_clear()); every call that
 * completes leaves it zero-filled again, so one clear at allocation suffices. */
size_t sv_workspace_bytes(int B, int n, int V, sv_dtype_t dt);

/* Enqueue a fill of `workspace` with zero bytes on `stream` (a kernel, not a
 * memset node, so it may be captured in a HIP graph). */
sv_status_t sv_workspace_clear(void *workspace, size_t workspace_bytes, void *stream);

/* Static description of a status code. */
const char *sv_status_string(sv_status_t s);

/* Text of the last HIP error seen by this library in the calling thread
 * ("" if none). */
const char *sv_last_hip_error(void);

/* Verify-and-sample for a batch of B sequences with n draft slots each.
 *
 * Follows the Speculative decoding section (acceptance and target-generation
 * stages) and the Target-draft section's decode paragraph of "Accelerating Sonar
 * through speculation"; draft length 0 is the standard sampling of one token
 * that the Target-draft section prescribes for batches without speculation.
 *
 * For sequence b with L = draft_lens[b], T = temperature[b], drafts x_j =
 * draft_tokens[b][j] and p_r = softmax(target[b][r] / T), q_r = softmax(draft[b][r] / T):
 *   - T > 0: draft j (j < L) is accepted iff u[b][j] < p_j(x_j) / q_j(x_j); the
 *     first rejection k ends the scan.  The token after the accepted prefix is
 *     drawn by inverse CDF with u[b][n] from max(0, p_k - q_k) (normalised) after
 *     a rejection, or from p_L when all L drafts are accepted (k = L).
 *   - T = 0: draft j is accepted iff it equals the argmax of target row j (raw
 *     logits, lowest index on ties); the emitted token is the argmax of row k.
 * Outputs: accepted_len[b] = k (0 <= k <= L <= n); emitted[b][0..k-1] = x_0..x_{k-1},
 * emitted[b][k] = the drawn token, emitted[b][k+1..n] = -1.
 *
 *   target_logits [B][n+1][V] dt    draft_logits [B][n][V] dt (may be NULL when every
 *                                   T_b = 0; never read for T_b = 0 sequences)
 *   draft_tokens  [B][n] int32      draft_lens [B] int32     temperature [B] float
 *   uniforms      [B][n+1] float in [0,1): [b][j] drives test j, [b][n] the draw
 *   accepted_len  [B] int32 out     emitted [B][n+1] int32 out
 *   row_lse       [B][2n+1] float out, nullable: ln sum exp(z/T) of target rows
 *                 0..n then draft rows 0..n-1; NaN for rows not read (and for
 *                 every row of a T_b = 0 sequence)
 *   err_flags     [1] uint32, nullable: SV_FLAG_* bits OR-ed in
 *   workspace     device scratch of at least sv_workspace_bytes(B, n, V, dt) bytes,
 *                 zero-filled before first use
 */
sv_status_t spec_verify_sample(const void *target_logits, const void *draft_logits,
                               sv_dtype_t dt, const int32_t *draft_tokens,
                               const int32_t *draft_lens, const float *temperature,
                               const float *uniforms, int B, int n, int V,
                               int32_t *accepted_len, int32_t *emitted, float *row_lse,
                               uint32_t *err_flags, void *workspace, size_t workspace_bytes,
                               void *stream);

/* Greedy verify: the T = 0 rule of spec_verify_sample() for every sequence,
 * without draft logits, temperatures or uniforms.  Accepts the longest prefix of
 * drafts equal to the argmax of their target rows (lowest index on ties) and
 * emits the argmax of the first mismatching row, or of row L when all match.
 * Target-draft section, decode paragraph, of "Accelerating Sonar through
 * speculation": the draft takes its highest-scoring token at each stage; the
 * argmax is sampling at T -> 0.
 * Arguments as in spec_verify_sample(). */
sv_status_t spec_verify_greedy(const void *target_logits, sv_dtype_t dt,
                               const int32_t *draft_tokens, const int32_t *draft_lens, int B,
                               int n, int V, int32_t *accepted_len, int32_t *emitted,
                               uint32_t *err_flags, void *workspace, size_t workspace_bytes,
                               void *stream);

/* Greedy tree verification.  "Accelerating Sonar through speculation", EAGLE
 * section: the draft explores a tree of candidate tokens, the target scores the
 * candidate sequences, the longest suitable one is kept and one more token from
 * the target is appended.  The greedy reading of "suitable":
 *   - node 0 is the root (the last committed token); node j + 1 (j < L_b) holds
 *     draft_tokens[b][j] and hangs below node draft_parents[b][j], which must lie
 *     in [0, j] (nodes in topological order; any other parent leaves the node
 *     out and sets SV_FLAG_BAD_PARENT);
 *   - target row r (of [B][n+1][V]) holds the target's logits after node r, as
 *     the target's tree-masked forward produces them; g_r = its argmax (lowest
 *     index on ties);
 *   - node i is accepted iff its parent p is accepted (the root is) and its
 *     token equals g_p;
 *   - the kept path runs from the root to the deepest accepted node (the
 *     lowest-numbered among equally deep ones).
 * Outputs: accepted_len[b] = the kept path's length; emitted[b] = its draft
 * tokens in order, then g of its last node, then -1; path[b] (nullable) = its
 * node indices (root excluded), then -1.  With draft_parents[b][j] = j (a chain)
 * the result is spec_verify_greedy's.  Tokens outside [0, V) are never accepted
 * (SV_FLAG_TOKEN_OOR).  Rows r > L_b are not used.  Sizes, workspace and
 * errors as in spec_verify_greedy().
 *   draft_tokens, draft_parents [B][n] int32     draft_lens [B] int32
 *   accepted_len [B] int32 out   emitted [B][n+1] int32 out   path [B][n] int32 out, nullable */
sv_status_t spec_verify_tree_greedy(const void *target_logits, sv_dtype_t dt, const int32_t *draft_tokens,
                                    const int32_t *draft_parents, const int32_t *draft_lens, int B, int n,
                                    int V, int32_t *accepted_len, int32_t *emitted, int32_t *path,
                                    uint32_t *err_flags, void *workspace, size_t workspace_bytes,
                                    void *stream);

/* Sampling tree verification.  "Accelerating Sonar through speculation", EAGLE
 * section: the draft explores a tree of candidate tokens, the target scores
 * every candidate sequence, the longest suitable one is kept and one more token
 * from the target is appended.  The page gives no acceptance rule for sampling;
 * the rule is SpecInfer's multi-step speculative sampling (Miao et al.,
 * "SpecInfer: Accelerating Large Language Model Serving with Tree-based
 * Speculative Inference and Verification"), under which the emitted tokens
 * follow the target's distribution when the children of every node are
 * independent draws from the draft's distribution at that node:
 *   - tree as in spec_verify_tree_greedy(): node 0 the root, node j + 1 holds
 *     draft_tokens[b][j] below draft_parents[b][j] in [0, j];
 *   - target row r = the target's logits after node r; draft row r (r < n) = the
 *     draft's logits at node r, from which node r's children were drawn;
 *     p_r = softmax(target row / T_b), q_r = softmax(draft row / T_b);
 *   - at node u the children are tested in index order against the current
 *     target residual p' (p_u at first): child j + 1 is accepted iff
 *     uniforms[b][j] < p'(x_j) / q_u(x_j); an accepted child moves the walk down;
 *     a rejected one replaces p' by max(0, p' - q_u) normalised; with no child
 *     left the token is drawn by inverse CDF with uniforms[b][n] from p' (from
 *     p_u itself at a node with no children);
 *   - T_b = 0: the greedy rule of spec_verify_tree_greedy().
 * Each test after a rejection at a node needs the residual's mass, a full
 * reduction of that node's row pair; one reduction per pending walk is made by
 * each of `max_rounds` round kernels (sv_tree_rounds() gives the bound for one
 * tree).  A walk that would need more leaves the remaining children of that
 * node untested and draws from the current residual -- the same rule on a
 * smaller tree, so the law is kept -- and sets SV_FLAG_TREE_TRUNCATED.
 * Outputs as in spec_verify_tree_greedy(): accepted_len = the kept path's
 * length, emitted = its tokens, the drawn token, then -1; path (nullable) = its
 * nodes.  Other arguments, limits and errors as in spec_verify_sample();
 * draft_logits [B][n][V] is required when n > 0.  max_rounds outside
 * [0, 4096] returns SV_EINVAL.  Launches 2 + max_rounds kernels. */
sv_status_t spec_verify_tree_sample(const void *target_logits, const void *draft_logits, sv_dtype_t dt,
                                    const int32_t *draft_tokens, const int32_t *draft_parents,
                                    const int32_t *draft_lens, const float *temperature,
                                    const float *uniforms, int B, int n, int V, int max_rounds,
                                    int32_t *accepted_len, int32_t *emitted, int32_t *path,
                                    uint32_t *err_flags, void *workspace, size_t workspace_bytes,
                                    void *stream);

/* Host helper: the number of rounds spec_verify_tree_sample() needs for one tree
 * so that no walk is truncated: the largest, over the tree's root-to-node paths,
 * of the sum over the path's nodes of (number of children - 1).  parents: HOST
 * array of L entries (node j + 1 below parents[j]; entries outside [0, j] leave
 * the node out).  Returns 0 for L <= 0 or NULL. */
int sv_tree_rounds(const int32_t *parents, int L);

/* MTP bookkeeping on the device, with no host synchronisation.
 *
 * MTP section, first paragraph, and Single-token MTP scheduling section, third
 * paragraph, of "Accelerating Sonar through speculation": the draft predicts
 * from a hidden state and the token that follows it (token t_{i+1} comes from
 * logits L_i, which come from hidden state H_i), so its input token buffer is
 * the target's shifted left one step relative to the target's hidden states, and
 * a kernel writes the target's next token into its slot.
 *
 * For each sequence b with a = clamp(accepted_len[b], 0, n):
 *   tokens[b][i] <- tokens[b][i+1]  for i < n;  tokens[b][n] keeps its value;
 *   tokens[b][a] <- emitted[b][a]   (the token the verify step produced).
 * Before the call, slot 0 holds the last committed token and slots 1..n the
 * drafts; afterwards slot i <= a holds the committed token that follows
 * position i, and slots past a hold unaccepted drafts (redundant work the draft
 * re-run may do).
 * Hidden states are carried unshifted: hidden_dst[b][i][:] = hidden_src[b][i][:]
 * (a bit copy of B*(n+1)*H bfloat16 values).  hidden_dst == hidden_src, or both
 * NULL, copies nothing.  Partially overlapping hidden buffers are SV_EINVAL.
 *
 *   tokens       [B][n+1] int32, in/out     accepted_len [B] int32
 *   emitted      [B][n+1] int32             hidden_src / hidden_dst [B][n+1][H] bf16
 */
sv_status_t mtp_shift_insert(int32_t *tokens, const void *hidden_src, void *hidden_dst, int H,
                             const int32_t *accepted_len, const int32_t *emitted, int B, int n,
                             void *stream);

/* One decode step's verification and MTP bookkeeping in one call.
 *
 * spec_verify_greedy_mtp() has the effect of spec_verify_greedy() followed by
 * mtp_shift_insert(tokens, hidden_src, hidden_dst, H, accepted_len, emitted, B, n)
 * on the same stream; spec_verify_sample_mtp() likewise with spec_verify_sample().
 * The step the pages describe (Speculative decoding section, four inference
 * stages; Single-token MTP scheduling section, third paragraph: the insert kernel
 * runs right after verification) has no host work between the two, so the
 * library fuses them: the hidden-state carry runs inside the verify kernels
 * (every workgroup of the statistics pass copies an equal share after its rows),
 * the token shift is done by the per-sequence decision and the drawn token is
 * written to both outputs.  No
 * extra launch is made when hidden_src and hidden_dst are 16-byte aligned and
 * B*(n+1)*H is a multiple of 8 (or nothing is copied); otherwise the MTP kernel
 * runs after the verify kernels.
 *
 * Because the copy overlaps the verification, tokens and hidden_dst must not
 * overlap any other argument (SV_EINVAL otherwise), and hidden_src must not be
 * written by the call (it is only read).  Other arguments and status codes are
 * those of the two calls it replaces.
 */
sv_status_t spec_verify_greedy_mtp(const void *target_logits, sv_dtype_t dt,
                                   const int32_t *draft_tokens, const int32_t *draft_lens, int B,
                                   int n, int V, int32_t *accepted_len, int32_t *emitted,
                                   uint32_t *err_flags, int32_t *tokens, const void *hidden_src,
                                   void *hidden_dst, int H, void *workspace,
                                   size_t workspace_bytes, void *stream);

sv_status_t spec_verify_sample_mtp(const void *target_logits, const void *draft_logits,
                                   sv_dtype_t dt, const int32_t *draft_tokens,
                                   const int32_t *draft_lens, const float *temperature,
                                   const float *uniforms, int B, int n, int V,
                                   int32_t *accepted_len, int32_t *emitted, float *row_lse,
                                   uint32_t *err_flags, int32_t *tokens, const void *hidden_src,
                                   void *hidden_dst, int H, void *workspace,
                                   size_t workspace_bytes, void *stream);

/* spec_verify_sample() with two optional parts, each NULL to leave it out:
 *
 *   draft_stats [B][n][2] float: the {m, S} statistics of every draft row at the
 *     sequence's temperature, as sv_sample_rows() writes them when the draft
 *     samples its tokens (the draft-target loop of the Target-draft section,
 *     decode paragraph: the draft samples from q_j, which already needs q_j's
 *     normaliser).  The verify step then reads no draft row in full: q_j(x_j)
 *     takes one gathered logit and the residual draw re-reads only draft row k.
 *     Entries for rows j >= L_b and for T_b = 0 sequences are not read.
 *     draft_logits must still be given.  Statistics that do not belong to the
 *     rows (another temperature, other logits) give undefined tokens, never an
 *     out-of-bounds access.  row_lse entries of draft rows come from draft_stats.
 *   tokens, hidden_src, hidden_dst, H: the fused MTP step of
 *     spec_verify_sample_mtp() (tokens NULL: no MTP step; hidden pointers must
 *     then be NULL too).
 */
sv_status_t spec_verify_sample_ex(const void *target_logits, const void *draft_logits,
                                  sv_dtype_t dt, const int32_t *draft_tokens,
                                  const int32_t *draft_lens, const float *temperature,
                                  const float *uniforms, const float *draft_stats, int B, int n,
                                  int V, int32_t *accepted_len, int32_t *emitted, float *row_lse,
                                  uint32_t *err_flags, int32_t *tokens, const void *hidden_src,
                                  void *hidden_dst, int H, void *workspace,
                                  size_t workspace_bytes, void *stream);

/* spec_verify_sample_ex() without a workspace argument and without any device
 * allocation, for callers that cannot allocate: code under HIP graph capture,
 * tight serving loops, harnesses that forbid allocation.
 *
 * The workspace is a device array of SV_NOALLOC_SCRATCH_BYTES bytes inside the
 * library, one per GPU, held until the process ends.  Sizes whose
 * sv_workspace_bytes(B, n, V, dt) exceed it return SV_EWORKSPACE before anything
 * is touched (B up to 5262 at n = 8, V = 152064 bf16; 6422 at n = 4, V = 128256).  The first
 * call on a GPU enqueues a clear of the array (a kernel) on `stream`; every
 * call leaves it zero-filled again.  All calls on one GPU share the array, so
 * calls that overlap in time on one GPU (different streams, or threads) race
 * and give undefined results; order them (one stream, or events).  Arguments,
 * results and other status codes are those of spec_verify_sample_ex(). */
#define SV_NOALLOC_SCRATCH_BYTES (16u << 20)
sv_status_t spec_verify_sample_ex_noalloc(const void *target_logits, const void *draft_logits,
                                          sv_dtype_t dt, const int32_t *draft_tokens,
                                          const int32_t *draft_lens, const float *temperature,
                                          const float *uniforms, const float *draft_stats, int B, int n,
                                          int V, int32_t *accepted_len, int32_t *emitted, float *row_lse,
                                          uint32_t *err_flags, int32_t *tokens, const void *hidden_src,
                                          void *hidden_dst, int H, void *stream);

/* Standard sampling of one token per sequence from a row chosen on the device.
 *
 * Sequence b draws from logits[b][r_b][:] with r_b = row_index[b] (clamped to
 * [0, R); row 0 when row_index is NULL): inverse CDF of softmax(z / T_b) with
 * uniforms[b], or the argmax (lowest index) when T_b = 0 -- the rule of
 * spec_verify_sample() with no drafts.  Two uses from "Accelerating Sonar
 * through speculation": the first draft token of the next step comes from the
 * carried draft logits at the accepted slot a_b (Target-draft section, decode
 * paragraph; Single-token MTP scheduling section, second paragraph: pass the
 * [B][n+1][V] draft/MTP logits, R = n + 1 and row_index = accepted_len), and the
 * draft's own per-step sampling (R = 1, row_index = NULL).  No host sync.
 * One kernel launch: the statistics pass's per-sequence decision also makes
 * the draw (as do the spec_verify_sample calls with n = 0).
 *
 *   logits     [B][R][V] dt      row_index [B] int32, nullable
 *   temperature [B] float        uniforms [B] float in [0,1)
 *   tokens     [B] int32 out     err_flags [1] uint32, nullable
 *   row_stats  [B][2] float out, nullable: {m, S} of the row drawn from, with
 *              m = max_i z_i and S = sum_i 2^((z_i - m) log2(e) / T_b) (NaN for
 *              T_b = 0).  These are the draft-row statistics that
 *              spec_verify_sample_ex() accepts, so the verify step need not
 *              stream the draft rows again.
 *   workspace  >= sv_workspace_bytes(B, 0, V, dt) bytes, zero-filled before first use
 */
sv_status_t sv_sample_rows(const void *logits, sv_dtype_t dt, int R, const int32_t *row_index,
                           const float *temperature, const float *uniforms, int B, int V,
                           int32_t *tokens, uint32_t *err_flags, float *row_stats, void *workspace,
                           size_t workspace_bytes, void *stream);

/* Greedy verify fused with the target's logit projection: the [B][n+1][V]
 * logits are never written to memory.
 *
 * "Accelerating Sonar through speculation": the model produces logits from
 * which the next token is sampled (Inference with speculative decoding section,
 * first paragraph) through its logit projection, which the MTP head reuses and
 * which is about 2 GB for a 70B Llama (MTP section, the paragraph on the head's
 * normalisation layers).  The greedy rule (spec_verify_greedy()) needs only
 * the argmax of each row, so each workgroup of the projection reduces its tile
 * of logits to a per-row (max, lowest index) in registers.
 *
 * The logits are z[b][r][v] = sum_k hidden[b][r][k] * weight[v][k], products
 * of bfloat16 values accumulated in binary32 on the matrix cores (summation
 * order unspecified); the greedy rule of spec_verify_greedy() is applied to
 * them: lowest index on ties, rows r > L_b take no part.  Where two logits of
 * a row are closer than the binary32 summation error, which one is the larger
 * can differ from exact arithmetic; when every partial sum is exactly
 * representable the result does not depend on the order.
 *
 *   hidden        [B][n+1][H] bf16, 16-byte aligned: the target's final hidden states
 *                 (after its last normalisation), one per verified position
 *   weight        [V][H] bf16, 16-byte aligned: the logit projection, one row per
 *                 vocabulary entry
 *   H             a multiple of 64 (SV_EINVAL otherwise); V * H and B*(n+1) * H
 *                 below 2^34
 *   draft_tokens, draft_lens, accepted_len, emitted, err_flags: as in spec_verify_greedy()
 *   tokens        [B][n+1] int32 in/out, nullable: the MTP token shift/insert of
 *                 mtp_shift_insert() done by the decision
 *   hidden_dst    [B][n+1][H] bf16, nullable (needs tokens), 16-byte aligned: the
 *                 MTP hidden-state carry (a bit copy of hidden), done by the
 *                 projection's workgroups, each copying an equal share after its
 *                 tile; hidden_dst == hidden copies nothing
 *   workspace     >= sv_workspace_bytes(B, n, V, SV_BF16) bytes, zero-filled before
 *                 first use and left zero-filled
 * tokens and hidden_dst must not overlap any other argument (SV_EINVAL).
 */
sv_status_t spec_verify_greedy_lmhead(const void *hidden, const void *weight, int H,
                                      const int32_t *draft_tokens, const int32_t *draft_lens, int B,
                                      int n, int V, int32_t *accepted_len, int32_t *emitted,
                                      uint32_t *err_flags, int32_t *tokens, void *hidden_dst,
                                      void *workspace, size_t workspace_bytes, void *stream);

/* Parity/debug only (not on the hot path): the binary32 logits of the logit
 * projection that spec_verify_greedy_lmhead() reduces, computed by the same
 * kernel.  hidden [M][H], weight [V][H] bf16 (16-byte aligned, H a multiple of
 * 64), logits_out [M][V] float. */
sv_status_t sv_lmhead_logits_debug(const void *hidden, const void *weight, int M, int H, int V,
                                   float *logits_out, void *stream);

/* Parity/debug only (not on the hot path): full binary32 probabilities
 * softmax(logits[r] / temperature[r]) of `rows` rows of length V, computed with
 * the same row statistics the verify kernels use.  temperature[r] must be > 0
 * (rows with T <= 0 or NaN are written as NaN).  probs_out [rows][V] float. */
sv_status_t sv_softmax_rows_debug(const void *logits, sv_dtype_t dt, const float *temperature,
                                  int rows, int V, float *probs_out, void *stream);

/* Parity/debug only (not on the hot path): the residual weights a draw after a
 * rejection scans, for `rows` row pairs (target_rows[r], draft_rows[r], each
 * [V] dt, temperature[r] > 0), formed by the draw pass's own device code.
 * After a rejection the token is drawn from max(0, p - q) normalised (the first
 * reference of "Accelerating Sonar through speculation"; that page's
 * Target-draft section, decode paragraph, compares the full distributions).
 *   weights_out      [rows][V] float: each token's weight, up to a factor common
 *                    to the row (NaN for rows with T <= 0 or NaN)
 *   tile_weights_out [rows][NT] double, nullable: the per-tile weights the tile
 *                    pick uses (NT = ceil(V / 2048) for bf16, ceil(V / 1024) for f32)
 *   info_out         [rows][4] float, nullable: {the form: 0 far, 1 near from
 *                    the chunks' sums, 2 near formed by one workgroup (each
 *                    row relative to its own maximum, differences scaled to the
 *                    largest of them), 3 that form with its weights formed from
 *                    their log2; the near form is taken when the residual mass
 *                    is below 0.01), lambda of the far form (else 0), kappa of
 *                    the near form (else 0), the residual mass sum max(0, p - q)}
 * The row statistics come from this call's own reduction of each row, so the
 * tile weights may differ from a verify call's in the last digits; the element
 * weights do not depend on them. */
sv_status_t sv_residual_weights_debug(const void *target_rows, const void *draft_rows, sv_dtype_t dt,
                                      const float *temperature, int rows, int V, float *weights_out,
                                      double *tile_weights_out, float *info_out, void *stream);

#ifdef __cplusplus
}
#endif

#endif /* SPECVERIFY_H */
