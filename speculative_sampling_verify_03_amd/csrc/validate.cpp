// Host-side validation of the C-ABI arguments and the workspace layout (no HIP calls).
#include "validate.hpp"

#include <cmath>
#include <cstring>

#include "spec_verify.h"

namespace sv {

namespace {
constexpr int64_t kMaxTotalRows = int64_t(1) << 22;  // B * rows: keeps grid sizes in range
constexpr int32_t kMaxV = int32_t(1) << 26;

size_t round_up(size_t x) { return (x + kWsAlign - 1) / kWsAlign * kWsAlign; }

bool mul_ok(int64_t a, int64_t b, int64_t limit) { return a >= 0 && b >= 0 && (b == 0 || a <= limit / b); }
}  // namespace

int greedy_splits(int32_t B, int32_t R, int32_t V) {
  // About 8192 workgroups (four rounds of the 2048 that fit the chip at once), so the last
  // round is a small share of the time; at most one split per 16K vocabulary entries, since
  // every split adds two device-scope atomics on the row's words (B=256, k=8, V=128256:
  // 4 splits measured 128 us against 134 us for 1, 149 us for 8 and 255 us for 16).
  const int64_t rows = static_cast<int64_t>(B) * R;
  if (rows <= 0) return 1;
  int64_t want = (8192 + rows - 1) / rows;
  int64_t cap = V / 16384;
  if (cap < 1) cap = 1;
  if (want > cap) want = cap;
  if (want > 64) want = 64;
  return static_cast<int>(want < 1 ? 1 : want);
}

bool workspace_layout(int kind, int32_t B, int32_t k_or_N, int32_t V, int32_t H, WsLayout* out) {
  (void)H;
  if (B < 0 || k_or_N < 0 || V < 1) return false;
  int64_t rows_per_seq;
  switch (kind) {
    case SV_KIND_LINEAR:
    case SV_KIND_LMHEAD:
    case SV_KIND_GREEDY:
      rows_per_seq = static_cast<int64_t>(k_or_N) + 1;
      break;
    case SV_KIND_TREE:
      rows_per_seq = k_or_N;
      if (rows_per_seq < 1) return false;
      break;
    default:
      return false;
  }
  if (rows_per_seq > kMaxRows) return false;
  const size_t b = static_cast<size_t>(B);
  const size_t rows = b * static_cast<size_t>(rows_per_seq);
  const size_t w = sizeof(uint64_t);
  const size_t splits = static_cast<size_t>(kSplitRows);
  out->status_off = 0;
  out->gen_off = kWsAlign;
  out->rej_off = out->gen_off + round_up(splits * w);
  out->words_off = out->rej_off + round_up(splits * w);
  out->counters_off = out->words_off + round_up(splits * kSplitWordsPerRow * w);
  out->seq_off = out->counters_off + round_up(b * sizeof(uint32_t));
  out->row_off = out->seq_off + round_up(2 * b * w);
  out->help_off = out->row_off + round_up(rows * w);
  const bool linear = kind == SV_KIND_LINEAR || kind == SV_KIND_LMHEAD;
  const size_t hrows = linear ? (rows < static_cast<size_t>(kHelpRows) ? rows : static_cast<size_t>(kHelpRows)) : 0;
  out->lmh_part_off = out->help_off + round_up(hrows * static_cast<size_t>(help_stride(V)) * w);
  const bool lmh = kind == SV_KIND_LMHEAD;
  const size_t nb = lmh ? static_cast<size_t>(lmh_blocks(V)) : 0;
  out->lmh_seq_off = out->lmh_part_off + round_up(rows * nb * w);
  out->lmh_mass_off = out->lmh_seq_off + round_up((lmh ? 2 * b : 0) * w);
  const size_t nch = lmh ? static_cast<size_t>(lmh_chunks(V)) : 0;
  out->lmh_cnt_off = out->lmh_mass_off + round_up(b * nch * sizeof(uint32_t));
  out->total = out->lmh_cnt_off + round_up((lmh ? b : 0) * sizeof(uint32_t));
  return true;
}

int check_dtype(int dt) { return (dt == SV_F32 || dt == SV_BF16) ? SV_OK : SV_E_DTYPE; }

int check_temperature(float T) { return (std::isfinite(T) && T > 0.0f) ? SV_OK : SV_E_TEMP; }

int check_aligned(const void* p, int dt) {
  const uintptr_t a = reinterpret_cast<uintptr_t>(p);
  return (a % (dt == SV_BF16 ? 2 : 4)) == 0 ? SV_OK : SV_E_ALIGN;
}

static int check_rows(int32_t B, int64_t R, int32_t V) {
  if (B < 0 || R < 1 || R > kMaxRows || V < 1 || V > kMaxV) return SV_E_SHAPE;
  if (!mul_ok(B, R, kMaxTotalRows)) return SV_E_SHAPE;
  return SV_OK;
}

static int check_ws(const void* ws, size_t ws_bytes, int kind, int32_t B, int32_t kn, int32_t V, int32_t H) {
  WsLayout L;
  if (!workspace_layout(kind, B, kn, V, H, &L)) return SV_E_SHAPE;
  if (ws == nullptr || ws_bytes < L.total) return SV_E_WORKSPACE;
  return SV_OK;
}

int validate_linear(const void* logits, int lt, const void* probs, int qt, const int32_t* tokens,
                    int32_t B, int32_t k, int32_t V, float T, const int32_t* out_tokens,
                    const int32_t* out_len, const void* ws, size_t ws_bytes) {
  int rc;
  if ((rc = check_dtype(lt)) || (rc = check_dtype(qt))) return rc;
  if (k < 0) return SV_E_SHAPE;
  if ((rc = check_rows(B, static_cast<int64_t>(k) + 1, V))) return rc;
  if ((rc = check_temperature(T))) return rc;
  if (B == 0) return SV_OK;
  if (!logits || !out_tokens || !out_len) return SV_E_NULL;
  if (k > 0 && (!probs || !tokens)) return SV_E_NULL;
  if ((rc = check_aligned(logits, lt))) return rc;
  if (k > 0 && (rc = check_aligned(probs, qt))) return rc;
  return check_ws(ws, ws_bytes, SV_KIND_LINEAR, B, k, V, 0);
}

int validate_greedy(const void* logits, int lt, const int32_t* tokens, int32_t B, int32_t k, int32_t V,
                    const int32_t* out_tokens, const int32_t* out_len, const void* ws, size_t ws_bytes) {
  int rc;
  if ((rc = check_dtype(lt))) return rc;
  if (k < 0) return SV_E_SHAPE;
  if ((rc = check_rows(B, static_cast<int64_t>(k) + 1, V))) return rc;
  if (B == 0) return SV_OK;
  if (!logits || !out_tokens || !out_len) return SV_E_NULL;
  if (k > 0 && !tokens) return SV_E_NULL;
  if ((rc = check_aligned(logits, lt))) return rc;
  return check_ws(ws, ws_bytes, SV_KIND_GREEDY, B, k, V, 0);
}

int build_tree(const int32_t* parent, int32_t N, TreeInfo* t) {
  if (N < 1 || N > kMaxRows) return SV_E_SHAPE;
  if (!parent) return SV_E_NULL;
  std::memset(t, 0, sizeof(*t));
  if (parent[0] != -1) return SV_E_TREE;
  t->N = N;
  for (int c = 0; c < N; ++c) t->first_child[c] = 0;
  int D = 0;
  for (int c = 1; c < N; ++c) {
    const int32_t p = parent[c];
    if (p < 0 || p >= c) return SV_E_TREE;
    if (c > 1 && p < parent[c - 1]) return SV_E_TREE;  // BFS order, siblings contiguous
    if (t->nchild[p] == 0) t->first_child[p] = static_cast<int8_t>(c);
    t->nchild[p] = static_cast<int8_t>(t->nchild[p] + 1);
    t->parent[c] = static_cast<int8_t>(p);
    t->depth[c] = static_cast<int8_t>(t->depth[p] + 1);
    if (t->depth[c] > D) D = t->depth[c];
  }
  t->parent[0] = -1;
  // BFS order also means depths never decrease along the array
  for (int c = 2; c < N; ++c)
    if (t->depth[c] < t->depth[c - 1]) return SV_E_TREE;
  t->D = D;
  return SV_OK;
}

int validate_tree(const void* logits, int lt, const void* probs, int qt, const int32_t* node_tokens,
                  const int32_t* parent_host, int32_t B, int32_t N, int32_t V, float T,
                  const int32_t* out_tokens, const int32_t* out_len, const void* ws, size_t ws_bytes,
                  TreeInfo* tree) {
  int rc;
  if ((rc = check_dtype(lt)) || (rc = check_dtype(qt))) return rc;
  if ((rc = check_rows(B, N, V))) return rc;
  if ((rc = check_temperature(T))) return rc;
  if ((rc = build_tree(parent_host, N, tree))) return rc;
  if (B == 0) return SV_OK;
  if (!logits || !out_tokens || !out_len) return SV_E_NULL;
  if (N > 1 && (!probs || !node_tokens)) return SV_E_NULL;
  if ((rc = check_aligned(logits, lt))) return rc;
  if (N > 1 && (rc = check_aligned(probs, qt))) return rc;
  return check_ws(ws, ws_bytes, SV_KIND_TREE, B, N, V, 0);
}

int validate_tree_lossless(const void* logits, int lt, const int32_t* node_tokens, const int32_t* parent_host,
                           int32_t B, int32_t N, int32_t V, float T, const int32_t* out_tokens,
                           const int32_t* out_len, const void* ws, size_t ws_bytes, TreeInfo* tree) {
  int rc;
  if ((rc = check_dtype(lt))) return rc;
  if ((rc = check_rows(B, N, V))) return rc;
  if ((rc = check_temperature(T))) return rc;
  if ((rc = build_tree(parent_host, N, tree))) return rc;
  if (B == 0) return SV_OK;
  if (!logits || !out_tokens || !out_len) return SV_E_NULL;
  if (N > 1 && !node_tokens) return SV_E_NULL;
  if ((rc = check_aligned(logits, lt))) return rc;
  return check_ws(ws, ws_bytes, SV_KIND_TREE, B, N, V, 0);
}

int validate_lmhead(const void* hidden, const void* w, const void* probs, int qt, const int32_t* tokens,
                    int32_t B, int32_t k, int32_t H, int32_t V, float T, const float* logits_out,
                    const int32_t* out_tokens, const int32_t* out_len, const void* ws, size_t ws_bytes) {
  int rc;
  if ((rc = check_dtype(qt))) return rc;
  if (k < 0 || H < 1 || H % 64 != 0 || H > (1 << 20)) return SV_E_SHAPE;
  if ((rc = check_rows(B, static_cast<int64_t>(k) + 1, V))) return rc;
  if ((rc = check_temperature(T))) return rc;
  if (B == 0) return SV_OK;
  if (!hidden || !w || !logits_out || !out_tokens || !out_len) return SV_E_NULL;
  if (k > 0 && (!probs || !tokens)) return SV_E_NULL;
  if ((reinterpret_cast<uintptr_t>(hidden) & 15) || (reinterpret_cast<uintptr_t>(w) & 1)) return SV_E_ALIGN;
  if ((reinterpret_cast<uintptr_t>(logits_out) & 3)) return SV_E_ALIGN;
  if (k > 0 && (rc = check_aligned(probs, qt))) return rc;
  return check_ws(ws, ws_bytes, SV_KIND_LMHEAD, B, k, V, H);
}

int validate_lmhead_logits(const void* hidden, const void* w, int32_t M, int32_t H, int32_t V,
                           const float* logits_out) {
  if (M < 0 || H < 1 || H % 64 != 0 || H > (1 << 20) || V < 1 || V > kMaxV) return SV_E_SHAPE;
  if (!mul_ok(M, 1, kMaxTotalRows * kMaxRows)) return SV_E_SHAPE;
  if (M == 0) return SV_OK;
  if (!hidden || !w || !logits_out) return SV_E_NULL;
  if ((reinterpret_cast<uintptr_t>(hidden) & 15) || (reinterpret_cast<uintptr_t>(w) & 1)) return SV_E_ALIGN;
  if ((reinterpret_cast<uintptr_t>(logits_out) & 3)) return SV_E_ALIGN;
  return SV_OK;
}

int validate_plug(const int32_t* tokens, const int32_t* accept_len, int32_t B, int32_t W, const int32_t* seq_len,
                  const int32_t* history, int32_t cap, const int32_t* next_token, const int32_t* status) {
  if (B < 0 || W < 1 || W > kMaxRows || cap < 1) return SV_E_SHAPE;
  if (!mul_ok(B, W, int64_t(1) << 40) || !mul_ok(B, cap, int64_t(1) << 50)) return SV_E_SHAPE;
  if (B == 0) return SV_OK;
  if (!tokens || !accept_len || !seq_len || !history) return SV_E_NULL;
  const void* ptrs[6] = {tokens, accept_len, seq_len, history, next_token, status};
  for (const void* p : ptrs)
    if (reinterpret_cast<uintptr_t>(p) & 3) return SV_E_ALIGN;
  return SV_OK;
}

int validate_lookup(const int32_t* history, const int32_t* seq_len, int32_t B, int32_t cap, int32_t min_ngram,
                    int32_t max_ngram, int32_t k, const int32_t* drafts, const int32_t* count) {
  constexpr int kMaxNgramArg = 16;  // the kernel holds the phrase in registers
  if (B < 0 || cap < 1 || k < 1 || k > kMaxRows) return SV_E_SHAPE;
  if (min_ngram < 1 || max_ngram < min_ngram || max_ngram > kMaxNgramArg) return SV_E_SHAPE;
  if (!mul_ok(B, cap, int64_t(1) << 50) || B > (int64_t(1) << 31) - 1) return SV_E_SHAPE;
  if (B == 0) return SV_OK;
  if (!history || !seq_len || !drafts || !count) return SV_E_NULL;
  const void* ptrs[4] = {history, seq_len, drafts, count};
  for (const void* p : ptrs)
    if (reinterpret_cast<uintptr_t>(p) & 3) return SV_E_ALIGN;
  return SV_OK;
}

}  // namespace sv
