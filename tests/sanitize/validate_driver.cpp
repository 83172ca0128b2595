// Drives the host-side argument validation of the C ABI through every error path.  Built
// by tests/test_validate_sanitized.py with g++ and the address and undefined-behaviour
// sanitizers; exits non-zero when a call returns a code other than the expected one (or
// a sanitizer aborts the run).  No device is touched: the pointers are never dereferenced.
#include <cmath>
#include <cstdint>
#include <cstdio>
#include <limits>
#include <vector>

#include "spec_verify.h"
#include "validate.hpp"

namespace {

int failures = 0;
int checks = 0;

void expect(int got, int want, const char* what, int line) {
  ++checks;
  if (got != want) {
    std::printf("FAIL line %d: %s returned %d, expected %d\n", line, what, got, want);
    ++failures;
  }
}
#define EXPECT(call, want) expect((call), (want), #call, __LINE__)

const void* P = reinterpret_cast<const void*>(0x1000);
const int32_t* I = reinterpret_cast<const int32_t*>(0x2000);
const float* F = reinterpret_cast<const float*>(0x3000);
const void* WS = reinterpret_cast<const void*>(0x4000);
const size_t BIG = size_t(1) << 30;
const float NaN = std::numeric_limits<float>::quiet_NaN();
const float Inf = std::numeric_limits<float>::infinity();

void linear() {
  using sv::validate_linear;
  EXPECT(validate_linear(P, SV_BF16, P, SV_BF16, I, 4, 3, 100, 1.f, I, I, WS, BIG), SV_OK);
  EXPECT(validate_linear(P, SV_BF16, P, SV_BF16, I, 0, 3, 100, 1.f, nullptr, nullptr, nullptr, 0), SV_OK);
  EXPECT(validate_linear(nullptr, SV_BF16, P, SV_BF16, I, 4, 3, 100, 1.f, I, I, WS, BIG), SV_E_NULL);
  EXPECT(validate_linear(P, SV_BF16, nullptr, SV_BF16, I, 4, 3, 100, 1.f, I, I, WS, BIG), SV_E_NULL);
  EXPECT(validate_linear(P, SV_BF16, P, SV_BF16, nullptr, 4, 3, 100, 1.f, I, I, WS, BIG), SV_E_NULL);
  EXPECT(validate_linear(P, SV_BF16, nullptr, SV_BF16, nullptr, 4, 0, 100, 1.f, I, I, WS, BIG), SV_OK);
  EXPECT(validate_linear(P, SV_BF16, P, SV_BF16, I, 4, 3, 100, 1.f, nullptr, I, WS, BIG), SV_E_NULL);
  EXPECT(validate_linear(P, SV_BF16, P, SV_BF16, I, 4, 3, 100, 1.f, I, nullptr, WS, BIG), SV_E_NULL);
  EXPECT(validate_linear(P, SV_BF16, P, SV_BF16, I, -1, 3, 100, 1.f, I, I, WS, BIG), SV_E_SHAPE);
  EXPECT(validate_linear(P, SV_BF16, P, SV_BF16, I, 4, -1, 100, 1.f, I, I, WS, BIG), SV_E_SHAPE);
  EXPECT(validate_linear(P, SV_BF16, P, SV_BF16, I, 4, 63, 100, 1.f, I, I, WS, BIG), SV_OK);
  EXPECT(validate_linear(P, SV_BF16, P, SV_BF16, I, 4, 64, 100, 1.f, I, I, WS, BIG), SV_E_SHAPE);
  EXPECT(validate_linear(P, SV_BF16, P, SV_BF16, I, 4, INT32_MAX, 100, 1.f, I, I, WS, BIG), SV_E_SHAPE);
  EXPECT(validate_linear(P, SV_BF16, P, SV_BF16, I, 4, 3, 0, 1.f, I, I, WS, BIG), SV_E_SHAPE);
  EXPECT(validate_linear(P, SV_BF16, P, SV_BF16, I, 4, 3, INT32_MAX, 1.f, I, I, WS, BIG), SV_E_SHAPE);
  EXPECT(validate_linear(P, SV_BF16, P, SV_BF16, I, INT32_MAX, 63, 100, 1.f, I, I, WS, BIG), SV_E_SHAPE);
  EXPECT(validate_linear(P, 2, P, SV_BF16, I, 4, 3, 100, 1.f, I, I, WS, BIG), SV_E_DTYPE);
  EXPECT(validate_linear(P, SV_BF16, P, -1, I, 4, 3, 100, 1.f, I, I, WS, BIG), SV_E_DTYPE);
  EXPECT(validate_linear(P, SV_BF16, P, SV_BF16, I, 4, 3, 100, 0.f, I, I, WS, BIG), SV_E_TEMP);
  EXPECT(validate_linear(P, SV_BF16, P, SV_BF16, I, 4, 3, 100, -2.f, I, I, WS, BIG), SV_E_TEMP);
  EXPECT(validate_linear(P, SV_BF16, P, SV_BF16, I, 4, 3, 100, NaN, I, I, WS, BIG), SV_E_TEMP);
  EXPECT(validate_linear(P, SV_BF16, P, SV_BF16, I, 4, 3, 100, Inf, I, I, WS, BIG), SV_E_TEMP);
  EXPECT(validate_linear(P, SV_BF16, P, SV_BF16, I, 4, 3, 100, 1.f, I, I, nullptr, BIG), SV_E_WORKSPACE);
  EXPECT(validate_linear(P, SV_BF16, P, SV_BF16, I, 4, 3, 100, 1.f, I, I, WS, 8), SV_E_WORKSPACE);
  EXPECT(validate_linear(reinterpret_cast<const void*>(0x1001), SV_BF16, P, SV_BF16, I, 4, 3, 100, 1.f, I, I, WS,
                         BIG), SV_E_ALIGN);
  EXPECT(validate_linear(reinterpret_cast<const void*>(0x1002), SV_F32, P, SV_BF16, I, 4, 3, 100, 1.f, I, I, WS,
                         BIG), SV_E_ALIGN);
  EXPECT(validate_linear(P, SV_BF16, reinterpret_cast<const void*>(0x1006), SV_F32, I, 4, 3, 100, 1.f, I, I, WS,
                         BIG), SV_E_ALIGN);
}

void greedy() {
  using sv::validate_greedy;
  EXPECT(validate_greedy(P, SV_F32, I, 4, 3, 100, I, I, WS, BIG), SV_OK);
  EXPECT(validate_greedy(nullptr, SV_F32, I, 4, 3, 100, I, I, WS, BIG), SV_E_NULL);
  EXPECT(validate_greedy(P, SV_F32, nullptr, 4, 3, 100, I, I, WS, BIG), SV_E_NULL);
  EXPECT(validate_greedy(P, SV_F32, nullptr, 4, 0, 100, I, I, WS, BIG), SV_OK);
  EXPECT(validate_greedy(P, SV_F32, I, 4, 64, 100, I, I, WS, BIG), SV_E_SHAPE);
  EXPECT(validate_greedy(P, 9, I, 4, 3, 100, I, I, WS, BIG), SV_E_DTYPE);
  EXPECT(validate_greedy(P, SV_F32, I, 4, 3, 100, I, I, WS, 4), SV_E_WORKSPACE);
  EXPECT(validate_greedy(reinterpret_cast<const void*>(0x1003), SV_BF16, I, 4, 3, 100, I, I, WS, BIG),
         SV_E_ALIGN);
  for (int B : {1, 7, 64, 256, 100000})
    for (int R : {1, 2, 9, 64})
      for (int V : {1, 1000, 16384, 128256, 1 << 26}) {
        const int s = sv::greedy_splits(B, R, V);
        ++checks;
        if (s < 1 || s > 64) {
          std::printf("FAIL greedy_splits(%d, %d, %d) = %d\n", B, R, V, s);
          ++failures;
        }
      }
}

void trees() {
  sv::TreeInfo t;
  const int32_t good[] = {-1, 0, 0, 0, 0, 1, 1, 2, 2, 3, 3, 4, 4};
  EXPECT(sv::build_tree(good, 13, &t), SV_OK);
  expect(t.D, 2, "depth of the 4-2 tree", __LINE__);
  expect(t.first_child[0], 1, "first child of the root", __LINE__);
  expect(t.nchild[0], 4, "children of the root", __LINE__);
  expect(t.first_child[2], 7, "first child of node 2", __LINE__);
  const int32_t root_only[] = {-1};
  EXPECT(sv::build_tree(root_only, 1, &t), SV_OK);
  EXPECT(sv::build_tree(nullptr, 3, &t), SV_E_NULL);
  EXPECT(sv::build_tree(good, 0, &t), SV_E_SHAPE);
  EXPECT(sv::build_tree(good, 65, &t), SV_E_SHAPE);
  const int32_t bad_root[] = {0, 0, 0};
  EXPECT(sv::build_tree(bad_root, 3, &t), SV_E_TREE);
  const int32_t forward[] = {-1, 1, 0};
  EXPECT(sv::build_tree(forward, 3, &t), SV_E_TREE);
  const int32_t not_bfs[] = {-1, 0, 1, 0};
  EXPECT(sv::build_tree(not_bfs, 4, &t), SV_E_TREE);
  const int32_t neg[] = {-1, -1};
  EXPECT(sv::build_tree(neg, 2, &t), SV_E_TREE);
  const int32_t self[] = {-1, 0, 2};
  EXPECT(sv::build_tree(self, 3, &t), SV_E_TREE);
  std::vector<int32_t> chain(64);
  chain[0] = -1;
  for (int c = 1; c < 64; ++c) chain[c] = c - 1;
  EXPECT(sv::build_tree(chain.data(), 64, &t), SV_OK);
  expect(t.D, 63, "depth of a 64-node chain", __LINE__);
  std::vector<int32_t> star(64, 0);
  star[0] = -1;
  EXPECT(sv::build_tree(star.data(), 64, &t), SV_OK);

  using sv::validate_tree;
  EXPECT(validate_tree(P, SV_BF16, P, SV_BF16, I, good, 4, 13, 100, 1.f, I, I, WS, BIG, &t), SV_OK);
  EXPECT(validate_tree(P, SV_BF16, P, SV_BF16, I, good, 0, 13, 100, 1.f, nullptr, nullptr, nullptr, 0, &t),
         SV_OK);
  EXPECT(validate_tree(P, SV_BF16, nullptr, SV_BF16, I, good, 4, 13, 100, 1.f, I, I, WS, BIG, &t), SV_E_NULL);
  EXPECT(validate_tree(P, SV_BF16, nullptr, SV_BF16, nullptr, root_only, 4, 1, 100, 1.f, I, I, WS, BIG, &t),
         SV_OK);
  EXPECT(validate_tree(P, SV_BF16, P, SV_BF16, I, good, 4, 13, 100, 0.f, I, I, WS, BIG, &t), SV_E_TEMP);
  EXPECT(validate_tree(P, SV_BF16, P, SV_BF16, I, not_bfs, 4, 4, 100, 1.f, I, I, WS, BIG, &t), SV_E_TREE);
  EXPECT(validate_tree(P, SV_BF16, P, 3, I, good, 4, 13, 100, 1.f, I, I, WS, BIG, &t), SV_E_DTYPE);
  EXPECT(validate_tree(P, SV_BF16, P, SV_BF16, I, good, 4, 13, 100, 1.f, I, I, WS, 16, &t), SV_E_WORKSPACE);
  EXPECT(validate_tree(P, SV_BF16, reinterpret_cast<const void*>(0x1001), SV_BF16, I, good, 4, 13, 100, 1.f, I, I,
                       WS, BIG, &t), SV_E_ALIGN);
  EXPECT(validate_tree(P, SV_BF16, P, SV_BF16, I, star.data(), 4, 65, 100, 1.f, I, I, WS, BIG, &t), SV_E_SHAPE);

  using sv::validate_tree_lossless;
  EXPECT(validate_tree_lossless(P, SV_F32, I, good, 4, 13, 100, 1.f, I, I, WS, BIG, &t), SV_OK);
  EXPECT(validate_tree_lossless(P, SV_F32, nullptr, good, 4, 13, 100, 1.f, I, I, WS, BIG, &t), SV_E_NULL);
  EXPECT(validate_tree_lossless(P, SV_F32, nullptr, root_only, 4, 1, 100, 1.f, I, I, WS, BIG, &t), SV_OK);
  EXPECT(validate_tree_lossless(P, SV_F32, I, forward, 4, 3, 100, 1.f, I, I, WS, BIG, &t), SV_E_TREE);
  EXPECT(validate_tree_lossless(P, SV_F32, I, good, 4, 13, 100, NaN, I, I, WS, BIG, &t), SV_E_TEMP);
  EXPECT(validate_tree_lossless(reinterpret_cast<const void*>(0x1002), SV_F32, I, good, 4, 13, 100, 1.f, I, I, WS,
                                BIG, &t), SV_E_ALIGN);
}

void lmhead() {
  using sv::validate_lmhead;
  EXPECT(validate_lmhead(P, P, P, SV_BF16, I, 4, 3, 128, 100, 1.f, F, I, I, WS, BIG), SV_OK);
  EXPECT(validate_lmhead(nullptr, P, P, SV_BF16, I, 4, 3, 128, 100, 1.f, F, I, I, WS, BIG), SV_E_NULL);
  EXPECT(validate_lmhead(P, P, P, SV_BF16, I, 4, 3, 128, 100, 1.f, nullptr, I, I, WS, BIG), SV_E_NULL);
  EXPECT(validate_lmhead(P, P, P, SV_BF16, I, 4, 3, 100, 100, 1.f, F, I, I, WS, BIG), SV_E_SHAPE);
  EXPECT(validate_lmhead(P, P, P, SV_BF16, I, 4, 3, 0, 100, 1.f, F, I, I, WS, BIG), SV_E_SHAPE);
  EXPECT(validate_lmhead(P, P, P, SV_BF16, I, 4, 3, 1 << 21, 100, 1.f, F, I, I, WS, BIG), SV_E_SHAPE);
  EXPECT(validate_lmhead(P, P, P, SV_BF16, I, 4, 3, INT32_MIN, 100, 1.f, F, I, I, WS, BIG), SV_E_SHAPE);
  EXPECT(validate_lmhead(P, P, P, SV_BF16, I, 4, 64, 128, 100, 1.f, F, I, I, WS, BIG), SV_E_SHAPE);
  EXPECT(validate_lmhead(P, P, P, 4, I, 4, 3, 128, 100, 1.f, F, I, I, WS, BIG), SV_E_DTYPE);
  EXPECT(validate_lmhead(P, P, P, SV_BF16, I, 4, 3, 128, 100, -1.f, F, I, I, WS, BIG), SV_E_TEMP);
  EXPECT(validate_lmhead(reinterpret_cast<const void*>(0x1008), P, P, SV_BF16, I, 4, 3, 128, 100, 1.f, F, I, I,
                         WS, BIG), SV_E_ALIGN);
  EXPECT(validate_lmhead(P, reinterpret_cast<const void*>(0x1001), P, SV_BF16, I, 4, 3, 128, 100, 1.f, F, I, I,
                         WS, BIG), SV_E_ALIGN);
  EXPECT(validate_lmhead(P, P, P, SV_BF16, I, 4, 3, 128, 100, 1.f, reinterpret_cast<const float*>(0x3002), I, I,
                         WS, BIG), SV_E_ALIGN);
  EXPECT(validate_lmhead(P, P, P, SV_BF16, I, 4, 3, 128, 100, 1.f, F, I, I, WS, 1), SV_E_WORKSPACE);

  using sv::validate_lmhead_logits;
  EXPECT(validate_lmhead_logits(P, P, 24, 128, 100, F), SV_OK);
  EXPECT(validate_lmhead_logits(nullptr, nullptr, 0, 128, 100, nullptr), SV_OK);
  EXPECT(validate_lmhead_logits(nullptr, P, 24, 128, 100, F), SV_E_NULL);
  EXPECT(validate_lmhead_logits(P, nullptr, 24, 128, 100, F), SV_E_NULL);
  EXPECT(validate_lmhead_logits(P, P, 24, 128, 100, nullptr), SV_E_NULL);
  EXPECT(validate_lmhead_logits(P, P, -1, 128, 100, F), SV_E_SHAPE);
  EXPECT(validate_lmhead_logits(P, P, INT32_MAX, 128, 100, F), SV_E_SHAPE);
  EXPECT(validate_lmhead_logits(P, P, 24, 96, 100, F), SV_E_SHAPE);
  EXPECT(validate_lmhead_logits(P, P, 24, INT32_MIN, 100, F), SV_E_SHAPE);
  EXPECT(validate_lmhead_logits(P, P, 24, 128, 0, F), SV_E_SHAPE);
  EXPECT(validate_lmhead_logits(P, P, 24, 128, INT32_MAX, F), SV_E_SHAPE);
  EXPECT(validate_lmhead_logits(reinterpret_cast<const void*>(0x1008), P, 24, 128, 100, F), SV_E_ALIGN);
  EXPECT(validate_lmhead_logits(P, reinterpret_cast<const void*>(0x1001), 24, 128, 100, F), SV_E_ALIGN);
  EXPECT(validate_lmhead_logits(P, P, 24, 128, 100, reinterpret_cast<const float*>(0x3002)), SV_E_ALIGN);
}

void plug_lookup() {
  using sv::validate_plug;
  int32_t* O = const_cast<int32_t*>(I);
  EXPECT(validate_plug(I, I, 4, 6, O, O, 100, nullptr, nullptr), SV_OK);
  EXPECT(validate_plug(I, I, 0, 6, nullptr, nullptr, 100, nullptr, nullptr), SV_OK);
  EXPECT(validate_plug(nullptr, I, 4, 6, O, O, 100, nullptr, nullptr), SV_E_NULL);
  EXPECT(validate_plug(I, I, 4, 6, nullptr, O, 100, nullptr, nullptr), SV_E_NULL);
  EXPECT(validate_plug(I, I, 4, 0, O, O, 100, nullptr, nullptr), SV_E_SHAPE);
  EXPECT(validate_plug(I, I, 4, 65, O, O, 100, nullptr, nullptr), SV_E_SHAPE);
  EXPECT(validate_plug(I, I, 4, 6, O, O, 0, nullptr, nullptr), SV_E_SHAPE);
  EXPECT(validate_plug(I, I, -3, 6, O, O, 100, nullptr, nullptr), SV_E_SHAPE);
  EXPECT(validate_plug(I, I, INT32_MAX, 64, O, O, 1 << 19, nullptr, nullptr), SV_OK);
  EXPECT(validate_plug(I, I, INT32_MAX, 64, O, O, INT32_MAX, nullptr, nullptr), SV_E_SHAPE);  // B * cap > 2^50
  EXPECT(validate_plug(I, I, 4, 6, O, O, 100, reinterpret_cast<int32_t*>(0x2002), nullptr), SV_E_ALIGN);

  using sv::validate_lookup;
  EXPECT(validate_lookup(I, I, 4, 100, 1, 3, 5, O, O), SV_OK);
  EXPECT(validate_lookup(nullptr, I, 4, 100, 1, 3, 5, O, O), SV_E_NULL);
  EXPECT(validate_lookup(I, I, 4, 100, 0, 3, 5, O, O), SV_E_SHAPE);
  EXPECT(validate_lookup(I, I, 4, 100, 4, 3, 5, O, O), SV_E_SHAPE);
  EXPECT(validate_lookup(I, I, 4, 100, 1, 17, 5, O, O), SV_E_SHAPE);
  EXPECT(validate_lookup(I, I, 4, 100, 1, 3, 0, O, O), SV_E_SHAPE);
  EXPECT(validate_lookup(I, I, 4, 100, 1, 3, 65, O, O), SV_E_SHAPE);
  EXPECT(validate_lookup(I, I, 4, 0, 1, 3, 5, O, O), SV_E_SHAPE);
  EXPECT(validate_lookup(I, I, INT32_MAX, 1 << 19, 1, 3, 5, O, O), SV_OK);
  EXPECT(validate_lookup(I, I, INT32_MAX, INT32_MAX, 1, 3, 5, O, O), SV_E_SHAPE);  // B * cap > 2^50
  EXPECT(validate_lookup(I, I, 4, 100, 1, 3, 5, reinterpret_cast<int32_t*>(0x2001), O), SV_E_ALIGN);
}

void workspace() {
  sv::WsLayout L;
  const int kinds[] = {SV_KIND_LINEAR, SV_KIND_GREEDY, SV_KIND_TREE, SV_KIND_LMHEAD};
  for (int kind : kinds)
    for (int32_t B : {0, 1, 64, 100000, INT32_MAX})
      for (int32_t kn : {0, 1, 5, 63, 64}) {
        const bool ok = sv::workspace_layout(kind, B, kn, 100, 128, &L);
        const int64_t rows = kind == SV_KIND_TREE ? kn : int64_t(kn) + 1;
        const bool want = rows >= 1 && rows <= 64;
        ++checks;
        if (ok != want) {
          std::printf("FAIL workspace_layout(%d, %d, %d) -> %d\n", kind, B, kn, ok);
          ++failures;
          continue;
        }
        if (!ok) continue;
        ++checks;
        const size_t need = size_t(B) * 4 + size_t(B) * 16 + size_t(B) * size_t(rows) * 8;
        if (L.total < need || L.seq_off % 256 || L.row_off % 256 || L.seq_off < size_t(B) * 4 ||
            L.row_off < L.seq_off + size_t(B) * 16) {
          std::printf("FAIL layout kind %d B %d kn %d: total %zu\n", kind, B, kn, L.total);
          ++failures;
        }
      }
  // the prefix never moves with the sizes or the kind
  sv::WsLayout A, Bl;
  EXPECT(sv::workspace_layout(SV_KIND_LINEAR, 64, 5, 32000, 0, &A), true);
  EXPECT(sv::workspace_layout(SV_KIND_TREE, 3, 61, 7, 0, &Bl), true);
  ++checks;
  if (A.status_off != Bl.status_off || A.gen_off != Bl.gen_off || A.rej_off != Bl.rej_off ||
      A.words_off != Bl.words_off || A.counters_off != Bl.counters_off || A.counters_off <= A.words_off) {
    std::printf("FAIL the workspace prefix moved between layouts\n");
    ++failures;
  }
  // the LM-head kind adds its sections after the linear ones: partials per row and 512-column
  // block, two words per sequence, one mass per sequence and 8192-column chunk, a counter
  sv::WsLayout Li, Lm;
  EXPECT(sv::workspace_layout(SV_KIND_LINEAR, 32, 5, 128256, 8192, &Li), true);
  EXPECT(sv::workspace_layout(SV_KIND_LMHEAD, 32, 5, 128256, 8192, &Lm), true);
  ++checks;
  if (Lm.lmh_part_off != Li.total || Lm.lmh_seq_off < Lm.lmh_part_off + size_t(192) * 251 * 8 ||
      Lm.lmh_mass_off < Lm.lmh_seq_off + size_t(32) * 16 || Lm.lmh_cnt_off < Lm.lmh_mass_off + size_t(32) * 16 * 4 ||
      Lm.total < Lm.lmh_cnt_off + size_t(32) * 4 || Lm.lmh_part_off % 256 || Lm.lmh_cnt_off % 256) {
    std::printf("FAIL LM-head sections: part %zu seq %zu mass %zu cnt %zu total %zu (linear total %zu)\n",
                Lm.lmh_part_off, Lm.lmh_seq_off, Lm.lmh_mass_off, Lm.lmh_cnt_off, Lm.total, Li.total);
    ++failures;
  }
  EXPECT(sv::workspace_layout(7, 1, 1, 1, 1, &L), false);
  EXPECT(sv::workspace_layout(SV_KIND_LINEAR, -1, 1, 1, 1, &L), false);
  EXPECT(sv::workspace_layout(SV_KIND_LINEAR, 1, 1, 0, 1, &L), false);
}

}  // namespace

int main() {
  linear();
  greedy();
  trees();
  lmhead();
  plug_lookup();
  workspace();
  std::printf("%d checks, %d failures\n", checks, failures);
  return failures == 0 ? 0 : 1;
}
