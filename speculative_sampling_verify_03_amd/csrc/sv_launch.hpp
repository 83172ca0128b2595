// Kernel parameter blocks and launchers shared by the kernels and the C-ABI layer.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

#include "validate.hpp"

namespace sv {

// Linear / tree row kernel.  R = k+1 rows per sequence (linear) or N nodes (tree).
struct RowParams {
  const void* logits;      // [B, R, V], float32 or bfloat16
  const void* probs;       // linear [B, k, V], tree [B, N, V]
  const int32_t* tokens;   // linear [B, k], tree [B, N]
  int32_t B, R, V, k;
  int32_t ntiles;          // tiles per row; 1 = the row stays in registers
  int32_t q_bf16;          // probs dtype
  float c;                 // log2(e) / T
  double T;
  uint64_t seed, offset;
  int32_t* out_tokens;
  int32_t* out_accept_len;
  float* out_tprob;        // linear only, may be null
  float* out_aprob;        // linear only, may be null
  int32_t* out_path;       // tree only, may be null
  uint32_t* counters;      // [B] arrival tickets
  uint64_t* seqword;       // [B][2] linear: inverted (row, token) key of the earliest
                           //     candidate, and 64 - row of the earliest rejection seen;
                           //     tree: mask of accepted nodes (word 0)
  uint64_t* rowword;       // [B * R] tree: candidate token + 1 of each node (low half);
                           //     with tree_skip, bit 63 once the node has decided its
                           //     children and the kept ones above bit 32 (relative to its
                           //     first child)
  int32_t tree_skip;       // tree: nodes off every accepted path skip their draw (every
                           //     node has at most 31 children)
  int32_t leaf_wait;       // lossless tree (with tree_skip): a leaf streams its row only
                           //     after its parent kept it and no decided node above
                           //     dropped its path
  // Linear multi-tile rows (help_on): the rows after a sequence's earliest rejection
  // compute residual tiles of that rejected row (verify_rows.hip).
  uint64_t* help_words;    // per row help_stride words: (m, Z), tile claims, unit totals
  int32_t help_stride;
  int32_t help_on;
  int32_t bonus_wait;      // set by the launcher: the last row of a sequence waits for the
                           //     earlier rows' decisions before it streams (help_on grids
                           //     that run in one round)
  uint32_t* errword;       // sticky: set when a wait for another workgroup ran out
  // every word above except errword is zero on entry and is returned to zero before the
  // kernel ends
};

// Static tree, BFS order, at most 64 nodes; passed by value in the kernel arguments.
struct TreeDesc {
  int8_t parent[64];
  int8_t first_child[64];
  int8_t nchild[64];
  int8_t depth[64];
  int32_t N;
  int32_t D;  // maximum depth
};

constexpr int kRowConfigs = 5;
struct RowConfig {
  int cfg;      // index into the (threads, vectors per thread) table
  int threads;
  int ntiles;
};
RowConfig choose_row_config(bool bf16, int V, int head_max, int64_t rows);
// qmode: 0 element-wise q reads, 1 16-byte q vectors in phase with the logits vectors,
// 2 float32 logits with 8-byte bfloat16 q chunks in phase with them.
hipError_t launch_rows(const RowParams& P, const TreeDesc& td, bool bf16, bool tree, int qmode, int cfg,
                       int grid, hipStream_t st);

// Linear kernel with each row split over S co-resident workgroups:
// at most kSplitSlices slices per row, at most kSplitRows rows (the workspace holds slots
// for those; validate.hpp).
constexpr int kSplitShapeCount = 4;   // (threads, vectors per thread) instances
struct SplitParams {
  const void* logits;      // [B, R, V], float32 or bfloat16
  const void* probs;       // [B, k, V]
  const int32_t* tokens;   // [B, k]
  int32_t B, R, V, k;
  int32_t S, chunk;        // slices per row, vectors per slice
  int32_t q_bf16;
  float c;                 // log2(e) / T
  double invT;             // 1 / T
  uint64_t seed, offset;
  int32_t* out_tokens;
  int32_t* out_accept_len;
  float* out_tprob;
  float* out_aprob;
  // The workspace's fixed prefix (validate.hpp): zero when the workspace is first used;
  // afterwards each call leaves these words for the next (see verify_split.hip).
  uint64_t* gen;           // [B] generation counters: generation = ticket >> 16
  uint64_t* first_rej;     // [B] (generation << 8) | (64 - row) of the earliest rejection seen
  uint64_t* words;         // [B * R][kSplitWordsPerRow] tagged words of each row
  uint32_t* errword;       // sticky: set when a wait for another workgroup ran out
};
struct SplitConfig {
  int shape, S, chunk, threads;
};
// qmode as for launch_rows (0 element loads, 1 vectors in phase); false = use the row kernel
bool choose_split(bool bf16, int qmode, int V, int head_max, int64_t rows, SplitConfig* out);
hipError_t launch_split(const SplitParams& P, bool bf16, int qmode, const SplitConfig& sc, hipStream_t st);

// Greedy kernel: grid = B * R * S workgroups (S splits per row).
struct GreedyParams {
  const void* logits;
  const int32_t* tokens;
  int32_t B, R, V, k, S;
  // flat path (16-byte aligned base and rows): nvec vectors per row, G workgroups over
  // the B * R * nvec vectors of the whole tensor; flat = 0 selects the per-row split path
  int32_t flat, nvec, G;
  int32_t* out_tokens;
  int32_t* out_accept_len;
  uint32_t* counters;  // [B] arrival tickets (zero on entry and exit)
  uint64_t* rowword;   // [B * R] orderable (value, lowest index) key of each row's maximum
  // flat path in two launches (phase 1, then 2; phase 0 = one launch over every row):
  // phase 1 covers positions 0 .. P0-1 of every sequence, phase 2 positions P0 .. k of the
  // sequences that kept all of their first P0 drafts, listed by phase 1
  int32_t phase, P0;
  uint32_t* alive;     // [B] sequences left for phase 2, then their count, then phase 2's
                       //     workgroup tickets (zero on entry and exit)
};
constexpr int kGreedyThreads = 256;
constexpr int kGreedyUnroll = 8;
constexpr int kGreedyFlatUnroll = 8;          // 16-byte loads in flight per thread
constexpr int kGreedyFlatMaxGroups = 2048;   // eight 256-thread workgroups on each of 256 CUs
constexpr int kGreedyFlatMinVectors = 2048;  // at least one full batch per thread and a half
hipError_t launch_greedy(const GreedyParams& P, bool bf16, hipStream_t st);

// LM-head GEMM: logits[M, V] (fp32) = hidden[M, H] (bf16) @ W[H, V] (bf16).  The direct
// kernel (lmhead_gemm_direct: V % 8 == 0, W and logits 16-byte aligned) can also write, for
// every row and block of kLmhBlockCols columns, the (max, sum of 2^((l - max) c)) pair of
// those logits into part[M][ceil(V / kLmhBlockCols)] (high half max, low half sum, float32).
constexpr int kLmhBlockCols = 512;
bool lmhead_gemm_direct(const void* w, const float* logits, int V);
hipError_t launch_lmhead_gemm(const void* hidden, const void* w, float* logits, int M, int H, int V,
                              hipStream_t st, uint64_t* part = nullptr, float c = 0.f);

// Verification of the LM head's logits from those partials (lmhead_verify.hip): a decide
// kernel (one workgroup per sequence) and a draw kernel (one wave per block of columns of
// each sequence's emitted row).
struct LmhParams {
  const float* logits;     // [B * R, V] float32, as the GEMM wrote them
  const void* probs;       // [B, k, V], float32 or bfloat16, 16-byte aligned (k > 0)
  const int32_t* tokens;   // [B, k]
  int32_t B, R, k, V;
  int32_t nb;              // column blocks per row = ceil(V / kLmhBlockCols)
  int32_t nchunks;         // residual chunks per row = ceil(V / 8192)
  int32_t cstride;         // chunk words per sequence in cmass (>= nchunks, <= 64)
  int32_t q_bf16;
  float c;                 // log2(e) / T
  double T;
  uint64_t seed, offset;
  int32_t* out_tokens;
  int32_t* out_accept_len;
  float* out_tprob;
  float* out_aprob;
  const uint64_t* part;    // [B * R][nb] the GEMM's partials (rewritten by every call)
  // zero on entry, returned to zero by the draw kernel:
  uint64_t* seqw;          // [B][2] emitted position n + 1, and row n's (max, sum)
  uint32_t* cmass;         // [B][cstride] residual mass of each chunk of row n
  uint32_t* ccnt;          // [B] column blocks counted
};
constexpr int kLmhMaxBlocks = 1024;  // nb limit of the draw kernel's block pick
hipError_t launch_lmhead_verify(const LmhParams& P, hipStream_t st);

// Token plug: one wave per sequence.
struct PlugParams {
  const int32_t* tokens;      // [B, W]
  const int32_t* accept_len;  // [B]
  int32_t* seq_len;           // [B] in/out
  int32_t* history;           // [B, cap] in/out
  int32_t* next_token;        // [B] or null
  int32_t* status;            // [B] or null
  int64_t B;
  int32_t W, cap;
};
hipError_t launch_plug(const PlugParams& P, hipStream_t st);

// Prompt lookup: one workgroup per sequence.
constexpr int kMaxNgram = 16;
struct LookupParams {
  const int32_t* history;  // [B, cap]
  const int32_t* seq_len;  // [B]
  int64_t B;
  int32_t cap, min_ngram, max_ngram, k;
  int32_t* drafts;         // [B, k]
  int32_t* count;          // [B]
};
hipError_t launch_lookup(const LookupParams& P, hipStream_t st);

}  // namespace sv
