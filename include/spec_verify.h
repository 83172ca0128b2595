/*
 * spec_verify.h -- C ABI of the speculative verification library (gfx950 / MI355X).
 *
 * The library implements the verification / speculative-sampling step of speculative
 * decoding.  A cheap draft proposes k tokens; the target model scores all of them in one
 * pass; the sampler keeps the longest acceptable prefix and adds one token taken from the
 * target's own distribution ("Accelerating Sonar through speculation", section
 * "Speculative decoding": the acceptance and target-generation stages).  A draft token is
 * kept outright when the target is at least as confident in it as the draft, otherwise
 * with a probability that shrinks as the gap grows; a rejected token is replaced by a draw
 * from an adjusted distribution, so the output follows the target's law exactly
 * ("Speculative decoding explained: how any LLM can get 3x faster inference", section
 * "Draft and verification loop").
 *
 * Readings where the pages are silent (all entry points):
 *   p_j = softmax(l_j / T) over the vocabulary (T applies to target logits only);
 *   draft token x at position j is kept iff  u_acc(b, j) * q_j(x) < p_j(x);
 *   n = first rejected position (k when none);
 *   correction (n < k): y ~ max(0, p_n - q_n) / S  (S = 0 falls back to p_n);
 *   bonus (n = k):      y ~ p_k;
 *   a draw y ~ w with uniform u is the smallest token id i with C_i > u * S,
 *   C the running sum of w in ascending token id.
 *   (u_acc, u_smp) for sequence b and position/node j are the top 24 bits (times 2^-24) of
 *   words 0 and 1 of Philox4x64-10 with counter (j, b, offset, 0) and key (seed, 0)
 *   (Salmon et al., SC'11).
 *   Draft tokens outside [0, V) are rejected (p(x) = 0; q(x) is not read).
 *   Logits may be -inf (probability 0) but each row needs one finite value; NaN is not
 *   supported.
 *
 * Conventions shared by every entry point:
 *   - Tensor arguments are DEVICE pointers owned by the caller, dense row-major, with the
 *     vocabulary as the contiguous axis.  Logits / probabilities must be aligned to their
 *     element size; 16-byte aligned rows are fastest.
 *   - Every call only enqueues work on `stream` (a hipStream_t; NULL = the null stream)
 *     and returns; it never synchronises and never allocates.  Outputs are valid once that
 *     stream's work has completed.
 *   - `workspace` is caller-owned device memory of at least
 *     spec_verify_workspace_bytes(kind, ...) bytes, zero-filled before its first use
 *     (hipMemset, torch.zeros).  Every call leaves it valid for any later call on the same
 *     stream (of any kind and sizes that fit it); its contents are the library's.  Calls
 *     that may run concurrently must not share a workspace.  Its first 4 bytes are a
 *     status word: non-zero after a call means a wait between the kernel's workgroups ran
 *     out (only possible when other work holds the chip for a second or more) and that
 *     call's outputs are not valid; it stays set until the caller clears it.
 *   - Return value: SV_OK (0) or a negative SV_E_* code, decided on the host before any
 *     launch (except SV_E_LAUNCH, reported when the runtime refuses a launch).
 *   - B = 0 is a valid empty call (nothing is launched).
 */
#ifndef SPEC_VERIFY_H
#define SPEC_VERIFY_H

#include <stddef.h>
#include <stdint.h>

#if defined(__GNUC__) || defined(__clang__)
#define SV_API __attribute__((visibility("default")))
#else
#define SV_API
#endif

#ifdef __cplusplus
extern "C" {
#endif

typedef enum { SV_F32 = 0, SV_BF16 = 1 } sv_dtype;

enum {
  SV_OK = 0,
  SV_E_NULL = -1,       /* a required pointer is NULL                                   */
  SV_E_SHAPE = -2,      /* B < 0, k < 0, k + 1 > 64, N > 64, V < 1, H < 1, size overflow */
  SV_E_DTYPE = -3,      /* dtype is not SV_F32 / SV_BF16                                */
  SV_E_TEMP = -4,       /* temperature not finite or <= 0                               */
  SV_E_TREE = -5,       /* parent array is not a BFS-ordered tree                       */
  SV_E_WORKSPACE = -6,  /* workspace NULL or smaller than required                      */
  SV_E_DEVICE = -7,     /* current HIP device is not gfx950                             */
  SV_E_LAUNCH = -8,     /* the HIP runtime refused a kernel launch                      */
  SV_E_ALIGN = -9,      /* a tensor pointer is not aligned to its element size          */
  SV_E_SCRATCH = -10    /* sizes need more than the static scratch of the _noalloc call */
};

enum { SV_KIND_LINEAR = 0, SV_KIND_GREEDY = 1, SV_KIND_TREE = 2, SV_KIND_LMHEAD = 3 };

/*
 * Linear speculative sampling ("Accelerating Sonar through speculation", section
 * "Speculative decoding", acceptance and target-generation stages; "Speculative decoding
 * explained", section "Draft and verification loop").
 *
 *   target_logits  [B, k+1, V] (lt)  row j = target logits after draft tokens 0..j-1
 *   draft_probs    [B, k, V]   (qt)  draft probabilities (not logits), used as given
 *   draft_tokens   [B, k] int32      drafted tokens
 *   temperature    T > 0, finite; scales the target logits only
 *   seed, offset   Philox key word and counter word 2 (vary offset per decoding step)
 *   out_tokens     [B, k+1] int32    emitted tokens: x_0..x_{n-1}, y, then -1 padding
 *   out_accept_len [B] int32         n in [0, k] accepted drafts (emitted = n + 1)
 *   out_target_prob [B, k] f32 or NULL   p_j(x_j) for every position (0 if x_j invalid)
 *   out_accept_prob [B, k] f32 or NULL   min(1, p_j(x_j) / q_j(x_j)) (q = 0: 1 if p > 0)
 * k = 0 is plain sampling from p_0; draft_probs / draft_tokens may then be NULL.
 */
SV_API int spec_verify_linear(const void* target_logits, int lt, const void* draft_probs, int qt,
                       const int32_t* draft_tokens, int32_t B, int32_t k, int32_t V,
                       float temperature, uint64_t seed, uint64_t offset,
                       int32_t* out_tokens, int32_t* out_accept_len,
                       float* out_target_prob, float* out_accept_prob,
                       void* workspace, size_t workspace_bytes, void* stream);

/*
 * spec_verify_linear without a workspace, for callers that cannot allocate device memory
 * (code under HIP graph capture, tight serving loops, harnesses that forbid hipMalloc).
 * Same arguments, kernels and results as spec_verify_linear, minus the workspace: the
 * per-sequence and per-row words live in a static device array of 4 MiB that the library
 * holds on every device it runs on until the process ends.  Each call clears the part it
 * uses (one small fill kernel on `stream`) and allocates nothing.  Every call on one
 * device shares that array, so calls that may overlap on one device (concurrent streams,
 * several host threads) race and must be serialised by the caller.
 * Returns SV_E_SCRATCH when spec_verify_workspace_bytes(SV_KIND_LINEAR, B, k, V, 0) exceeds
 * 4 MiB, decided before any device call.
 */
SV_API int spec_verify_linear_noalloc(const void* target_logits, int lt, const void* draft_probs, int qt,
                       const int32_t* draft_tokens, int32_t B, int32_t k, int32_t V,
                       float temperature, uint64_t seed, uint64_t offset,
                       int32_t* out_tokens, int32_t* out_accept_len,
                       float* out_target_prob, float* out_accept_prob, void* stream);

/*
 * Greedy verification: draft token j is kept while it equals the argmax of target row j
 * (lowest token id among equal maxima, raw logits, no temperature); the token after the
 * kept prefix is the argmax of target row n.  Same shapes and outputs as above.
 */
SV_API int spec_verify_greedy(const void* target_logits, int lt, const int32_t* draft_tokens,
                       int32_t B, int32_t k, int32_t V,
                       int32_t* out_tokens, int32_t* out_accept_len,
                       void* workspace, size_t workspace_bytes, void* stream);

/*
 * Static-tree (EAGLE-style) verification ("Accelerating Sonar through speculation",
 * section "EAGLE": a static tree of drafts is explored and the longest acceptable
 * sequence is kept, plus one target token).
 *
 *   target_logits [B, N, V] (lt)  row u = target logits after the path root..u
 *   draft_probs   [B, N, V] (qt)  row u = draft distribution u's children were taken from
 *   node_tokens   [B, N] int32    token of node c (entry 0, the root, is ignored)
 *   parent_host   [N] int32, HOST memory: parent[0] = -1, 0 <= parent[c] < c,
 *                 non-decreasing (BFS order, siblings left to right); N <= 64.
 *   Node c >= 1 with parent u is accepted iff u_acc(b, c) * q_u(tok_c) < p_u(tok_c); a node
 *   is alive when it and all its ancestors are accepted; the chosen node c* is the deepest
 *   alive node (lowest index on ties: the leftmost path); the bonus token is drawn from
 *   p_{c*} with u_smp(b, c*).  (This rule does not preserve the target law exactly.)
 *   out_tokens    [B, D+1] int32  tokens of the path root..c* (root excluded), then the
 *                                 bonus, then -1; D = depth of the tree
 *   out_accept_len [B] int32      depth of c*
 *   out_path      [B, D+1] int32 or NULL   node ids root..c*, then -1
 */
SV_API int spec_verify_tree(const void* target_logits, int lt, const void* draft_probs, int qt,
                     const int32_t* node_tokens, const int32_t* parent_host,
                     int32_t B, int32_t N, int32_t V, float temperature,
                     uint64_t seed, uint64_t offset,
                     int32_t* out_tokens, int32_t* out_accept_len, int32_t* out_path,
                     void* workspace, size_t workspace_bytes, void* stream);

/*
 * Lossless static-tree verification: the same tree as spec_verify_tree, with candidates
 * that are fixed top-K draft tokens ("Accelerating Sonar through speculation", section
 * "EAGLE": Top-K candidates at every node), verified so that the emitted tokens follow
 * the target law exactly ("Speculative decoding explained", section "Draft and
 * verification loop"; the pages give no multi-candidate procedure, this is a reading).
 * No draft probabilities are read: each candidate's draft law is a point mass.
 *
 * From the root, at node u with children c_1..c_m (sibling order) and p = p_u: child c_i
 * (token x) is kept iff x is in [0, V), no earlier sibling has token x, and
 * u_acc(b, c_i) * W_i < p(x), where W_i = 1 - sum of p over the distinct valid tokens of
 * c_1..c_{i-1} (summed in sibling order).  The first kept child is the next node; if none
 * is kept the extra token is drawn by inverse CDF with u_smp(b, u) from p with the
 * children's valid tokens removed (from p itself when u has no children, or when the
 * remaining mass is 0 through rounding).
 *
 *   target_logits [B, N, V] (lt), node_tokens [B, N], parent_host [N] (HOST): as for
 *   spec_verify_tree.  Outputs and workspace (SV_KIND_TREE): as for spec_verify_tree;
 *   out_accept_len is the depth of the node where the walk stopped.
 */
SV_API int spec_verify_tree_lossless(const void* target_logits, int lt, const int32_t* node_tokens,
                       const int32_t* parent_host, int32_t B, int32_t N, int32_t V,
                       float temperature, uint64_t seed, uint64_t offset,
                       int32_t* out_tokens, int32_t* out_accept_len, int32_t* out_path,
                       void* workspace, size_t workspace_bytes, void* stream);

/*
 * LM-head projection feeding linear verification ("Accelerating Sonar through
 * speculation", sections "EAGLE" and "Training MTP heads": the heads share the target's
 * LM head, ~2 GB in bf16 for a 70B model).
 *
 *   hidden     [B, k+1, H] bf16   final hidden states of the k+1 verified positions
 *   lm_head    [H, V] bf16        row-major (vocabulary contiguous)
 *   logits_out [B, k+1, V] f32    REQUIRED: receives hidden @ lm_head (fp32 accumulation);
 *                                 linear verification then runs on it.
 *   Other arguments as in spec_verify_linear.  H must be a multiple of 64 and `hidden`
 *   16-byte aligned; V is arbitrary.  With 16-byte aligned lm_head rows and logits_out
 *   (V % 8 == 0 and aligned bases) and 16-byte aligned draft_probs, the GEMM also leaves
 *   each row's softmax partials per block of 512 columns in the workspace and
 *   verification starts from them (no second pass over the logits); other shapes verify
 *   the written logits as spec_verify_linear does.  Results are the same either way.
 *   logits_out is overwritten on every call.  Workspace: spec_verify_workspace_bytes
 *   (SV_KIND_LMHEAD, B, k, V, H); its partials section is rewritten by every call, the
 *   rest is returned to zero.
 */
SV_API int spec_lmhead_verify(const void* hidden, const void* lm_head,
                       const void* draft_probs, int qt, const int32_t* draft_tokens,
                       int32_t B, int32_t k, int32_t H, int32_t V, float temperature,
                       uint64_t seed, uint64_t offset, float* logits_out,
                       int32_t* out_tokens, int32_t* out_accept_len,
                       float* out_target_prob, float* out_accept_prob,
                       void* workspace, size_t workspace_bytes, void* stream);

/*
 * The LM-head projection alone, the first stage of spec_lmhead_verify ("Accelerating
 * Sonar through speculation", sections "EAGLE" and "Training MTP heads"): logits_out =
 * hidden @ lm_head with fp32 accumulation, the same kernels and the same bits as the
 * logits spec_lmhead_verify writes.  For callers that verify the logits themselves (for
 * example greedily, with spec_verify_greedy).
 *
 *   hidden     [M, H] bf16   16-byte aligned; H a multiple of 64
 *   lm_head    [H, V] bf16   row-major (vocabulary contiguous)
 *   logits_out [M, V] f32    overwritten
 * M = 0 does nothing.  Errors: SV_E_NULL, SV_E_SHAPE, SV_E_ALIGN, SV_E_DEVICE, SV_E_LAUNCH.
 * No workspace.
 */
SV_API int spec_lmhead_logits(const void* hidden, const void* lm_head, int32_t M, int32_t H, int32_t V,
                       float* logits_out, void* stream);

/*
 * On-device token plug ("Accelerating Sonar through speculation", section "MTP schedule for
 * one token": after the target's input tokens are shifted, a kernel plugs the next tokens
 * into their positions, so the accepted lengths need no GPU-to-CPU read before the next
 * step is set up).  Reads the outputs of a verify call and, for every sequence b with
 * n = out_accept_len[b]:
 *   history[b, seq_len[b] + i] = out_tokens[b, i]   for i = 0..n (positions >= cap dropped)
 *   next_token[b] = out_tokens[b, n]                (the input of the next draft step)
 *   seq_len[b]    = min(seq_len[b] + n + 1, cap)
 *   status[b]     = 0, or 1 when tokens were dropped at cap, or 2 when n is not in
 *                   [0, W-1] or seq_len[b] is not in [0, cap] (nothing is written then).
 *
 *   out_tokens     [B, W] int32   as written by a verify call (W = k+1; tree: D+1)
 *   out_accept_len [B] int32
 *   seq_len        [B] int32      in/out
 *   history        [B, cap] int32 in/out (row-major, one row of capacity cap per sequence)
 *   next_token     [B] int32 or NULL
 *   status         [B] int32 or NULL
 * Needs no workspace.  W must be in [1, 64], cap >= 1.
 */
SV_API int spec_plug_tokens(const int32_t* out_tokens, const int32_t* out_accept_len, int32_t B, int32_t W,
                     int32_t* seq_len, int32_t* history, int32_t cap, int32_t* next_token, int32_t* status,
                     void* stream);

/*
 * Prompt-lookup drafting ("Speculative decoding explained", section "Variants without a
 * separate draft model": with no draft model, drafts are phrases found again in the prompt
 * and history).  For each sequence b with history h = history[b, 0..len), len = seq_len[b]:
 * for n = max_ngram down to min_ngram, the phrase h[len-n .. len) is looked up at the
 * earliest start i with i + n < len and h[i .. i+n) equal to it; the first n that matches
 * gives out_drafts[b] = h[i+n .. min(i+n+k, len)) padded with -1 and out_count[b] = their
 * number.  No match (or len outside [0, cap]) gives out_count[b] = 0 and all -1.  The drafts
 * can be verified as one-hot draft distributions or greedily.
 *
 *   history    [B, cap] int32      seq_len [B] int32
 *   out_drafts [B, k] int32        out_count [B] int32
 * 1 <= min_ngram <= max_ngram <= 16, 1 <= k <= 64, cap >= 1.  Needs no workspace.
 */
SV_API int spec_lookup_drafts(const int32_t* history, const int32_t* seq_len, int32_t B, int32_t cap,
                       int32_t min_ngram, int32_t max_ngram, int32_t k, int32_t* out_drafts,
                       int32_t* out_count, void* stream);

/* Workspace bytes for a call of `kind` (SV_KIND_*) with the given sizes (k_or_N = k for
 * linear / greedy / lmhead, N for tree; H is used by lmhead only).  Returns 0 for invalid
 * arguments. */
SV_API size_t spec_verify_workspace_bytes(int kind, int32_t B, int32_t k_or_N, int32_t V, int32_t H);

/* Static, human-readable text for a return code. */
SV_API const char* spec_verify_strerror(int code);

#ifdef __cplusplus
}
#endif

#endif /* SPEC_VERIFY_H */
