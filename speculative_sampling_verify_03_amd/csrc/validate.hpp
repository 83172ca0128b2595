// Host-side argument checks and workspace layout of the C ABI.  Pure C++ (no HIP), so
// it also builds with g++ and the host sanitizers.
#pragma once

#include <stddef.h>
#include <stdint.h>

namespace sv {

constexpr int kMaxRows = 64;   // k + 1 and N: one wave covers a sequence's rows
constexpr size_t kWsAlign = 256;

// Every workspace, whatever the kind and sizes, starts with the same fixed prefix:
//   status word u32 (first 256 bytes);
//   generation counters u64[kSplitRows] and earliest-rejection words u64[kSplitRows], one
//   per sequence of the split kernel;
//   the split kernel's tagged words, kSplitWordsPerRow u64 per row for up to kSplitRows rows.
// Its place never depends on the sizes, so words a split call leaves behind are never
// read as anything else by a later call of any kind (they carry tags no later call will
// look for).  After it come the sections of the row, greedy and tree kernels, which they
// return to zero before they end: arrival counters u32[B], per-sequence words u64[B][2],
// per-row words u64[B * rows] (rows = k + 1, or N for a tree), and for linear kinds the
// help section described below.  Sections are 256-byte aligned.
constexpr int64_t kSplitRows = 2048;
constexpr int kSplitSlices = 8;
// per row: (max, sum) pair of each slice (4 words), the row's two uniforms (4 words),
// residual mass of each slice (2 words), the row's decision (1 word)
constexpr int kSplitWordsPerRow = 6 * kSplitSlices + 5;

// Linear rows drawn by the row kernel in tiles can be helped by the later rows of their
// sequence (residual tiles computed there) when the launch has at most kHelpRows rows.
// The help section holds per row help_stride(V) u64 words: its (max, sum), a tile claim
// counter and one total per (tile, wave) unit.
constexpr int64_t kHelpRows = 2048;
inline int32_t help_stride(int32_t V) { return 2 + (V + 3) / 4096 + 9; }

// The LM-head call adds, after the linear sections, the GEMM's softmax partials (one u64
// per row and block of 512 columns, rewritten by every call), two hand-over words and a
// chunk counter per sequence, and one residual mass per sequence and chunk of 8192 columns
// (returned to zero by every call).
inline int64_t lmh_blocks(int32_t V) { return (static_cast<int64_t>(V) + 511) / 512; }
inline int64_t lmh_chunks(int32_t V) {
  const int64_t c = (static_cast<int64_t>(V) + 8191) / 8192;
  return c < 64 ? c : 64;
}

struct WsLayout {
  size_t status_off, gen_off, rej_off, words_off;  // fixed prefix
  size_t counters_off, seq_off, row_off;           // row kernel, greedy and tree kernels
  size_t help_off;                                 // row kernel, linear (0 size otherwise)
  size_t lmh_part_off, lmh_seq_off, lmh_mass_off, lmh_cnt_off;  // LM-head (0 size otherwise)
  size_t total;
};
bool workspace_layout(int kind, int32_t B, int32_t k_or_N, int32_t V, int32_t H, WsLayout* out);
// Number of workgroups each row is split over by the greedy kernel.
int greedy_splits(int32_t B, int32_t R, int32_t V);

int check_dtype(int dt);
int check_temperature(float T);
int check_aligned(const void* p, int dt);

// Shape / pointer validation of each entry point (no device access).
int validate_linear(const void* logits, int lt, const void* probs, int qt, const int32_t* tokens,
                    int32_t B, int32_t k, int32_t V, float T, const int32_t* out_tokens,
                    const int32_t* out_len, const void* ws, size_t ws_bytes);
int validate_greedy(const void* logits, int lt, const int32_t* tokens, int32_t B, int32_t k, int32_t V,
                    const int32_t* out_tokens, const int32_t* out_len, const void* ws, size_t ws_bytes);

struct TreeInfo {
  int8_t parent[64];
  int8_t first_child[64];
  int8_t nchild[64];
  int8_t depth[64];
  int32_t N;
  int32_t D;
};
// Checks the parent array (parent[0] = -1, 0 <= parent[c] < c, non-decreasing) and fills
// children ranges and depths.
int build_tree(const int32_t* parent, int32_t N, TreeInfo* out);
int validate_tree(const void* logits, int lt, const void* probs, int qt, const int32_t* node_tokens,
                  const int32_t* parent_host, int32_t B, int32_t N, int32_t V, float T,
                  const int32_t* out_tokens, const int32_t* out_len, const void* ws, size_t ws_bytes,
                  TreeInfo* tree);
int validate_tree_lossless(const void* logits, int lt, const int32_t* node_tokens, const int32_t* parent_host,
                           int32_t B, int32_t N, int32_t V, float T, const int32_t* out_tokens,
                           const int32_t* out_len, const void* ws, size_t ws_bytes, TreeInfo* tree);
int validate_lmhead(const void* hidden, const void* w, const void* probs, int qt, const int32_t* tokens,
                    int32_t B, int32_t k, int32_t H, int32_t V, float T, const float* logits_out,
                    const int32_t* out_tokens, const int32_t* out_len, const void* ws, size_t ws_bytes);

int validate_lmhead_logits(const void* hidden, const void* w, int32_t M, int32_t H, int32_t V,
                           const float* logits_out);

int validate_plug(const int32_t* tokens, const int32_t* accept_len, int32_t B, int32_t W, const int32_t* seq_len,
                  const int32_t* history, int32_t cap, const int32_t* next_token, const int32_t* status);

int validate_lookup(const int32_t* history, const int32_t* seq_len, int32_t B, int32_t cap, int32_t min_ngram,
                    int32_t max_ngram, int32_t k, const int32_t* drafts, const int32_t* count);

}  // namespace sv
