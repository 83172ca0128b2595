// C-ABI entry points: validate on the host, carve the caller's workspace, enqueue the
// kernels on the caller's stream.  Nothing here allocates or synchronises.
#include <algorithm>
#include <cmath>
#include <cstring>
#include <mutex>

#include "spec_verify.h"
#include "sv_launch.hpp"
#include "validate.hpp"

namespace {

// gfx950 check, cached per device ordinal.
int check_device() {
  static std::mutex mu;
  static int state[64] = {0};  // 0 unknown, 1 ok, -1 not gfx950
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return SV_E_DEVICE;
  {
    std::lock_guard<std::mutex> g(mu);
    if (state[dev] == 0) {
      hipDeviceProp_t prop;
      if (hipGetDeviceProperties(&prop, dev) != hipSuccess) return SV_E_DEVICE;
      state[dev] = (std::strncmp(prop.gcnArchName, "gfx950", 6) == 0) ? 1 : -1;
    }
    return state[dev] == 1 ? SV_OK : SV_E_DEVICE;
  }
}

// ---------------------------------------------------------------- static scratch
// Backing store of spec_verify_linear_noalloc: the per-sequence and per-row words that
// the other entry points keep in the caller's workspace.  One copy per device, held until
// the process ends.  In host code `scratch` names a host-side stand-in, never the device
// array: its device address comes from hipGetSymbolAddress, resolved once per device
// (with that device current) and cached below.
constexpr size_t kScratchBytes = size_t(4) << 20;
static __device__ __align__(256) unsigned char scratch[kScratchBytes];

// Device address of this device's `scratch`, or nullptr if the runtime cannot give it.
void* scratch_device_ptr() {
  static std::mutex mu;
  static void* ptrs[64] = {};
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return nullptr;
  std::lock_guard<std::mutex> g(mu);
  if (ptrs[dev] == nullptr) {
    void* p = nullptr;
    if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || p == nullptr) return nullptr;
    ptrs[dev] = p;
  }
  return ptrs[dev];
}

// Zero n 32-bit words (a fill kernel rather than a memset node, so that the call stays
// safe to record in a graph).
__global__ void zero_words_kernel(uint32_t* p, uint32_t n) {
  for (uint32_t i = blockIdx.x * blockDim.x + threadIdx.x; i < n; i += gridDim.x * blockDim.x) p[i] = 0u;
}

int head_max(const void* p, int32_t V, int dt) {
  const int eb = dt == SV_BF16 ? 2 : 4;
  const int ve = 16 / eb;
  if ((static_cast<int64_t>(V) * eb) % 16 == 0) return static_cast<int>((reinterpret_cast<uintptr_t>(p) & 15) / eb);
  return ve - 1;
}

int run_rows(bool tree, bool lossless, const void* logits, int lt, const void* probs, int qt, const int32_t* tokens,
             int32_t B, int32_t R, int32_t k, int32_t V, float T, uint64_t seed, uint64_t offset,
             int32_t* out_tokens, int32_t* out_len, float* tprob, float* aprob, int32_t* out_path,
             const sv::TreeInfo* ti, void* ws, hipStream_t st) {
  sv::WsLayout L;
  sv::workspace_layout(tree ? SV_KIND_TREE : SV_KIND_LINEAR, B, tree ? R : k, V, 0, &L);
  sv::RowParams P{};
  P.logits = logits;
  P.probs = probs;
  P.tokens = tokens;
  P.B = B;
  P.R = R;
  P.V = V;
  P.k = k;
  P.q_bf16 = (qt == SV_BF16);
  P.T = static_cast<double>(T);
  P.c = static_cast<float>(1.4426950408889634 / static_cast<double>(T));
  P.seed = seed;
  P.offset = offset;
  P.out_tokens = out_tokens;
  P.out_accept_len = out_len;
  P.out_tprob = tprob;
  P.out_aprob = aprob;
  P.out_path = out_path;
  P.counters = reinterpret_cast<uint32_t*>(static_cast<char*>(ws) + L.counters_off);
  P.seqword = reinterpret_cast<uint64_t*>(static_cast<char*>(ws) + L.seq_off);
  P.rowword = reinterpret_cast<uint64_t*>(static_cast<char*>(ws) + L.row_off);
  const bool bf16 = (lt == SV_BF16);
  const sv::RowConfig rc = sv::choose_row_config(bf16, V, head_max(logits, V, lt), static_cast<int64_t>(B) * R);
  P.ntiles = rc.ntiles;
  P.errword = reinterpret_cast<uint32_t*>(static_cast<char*>(ws) + L.status_off);
  P.help_words = reinterpret_cast<uint64_t*>(static_cast<char*>(ws) + L.help_off);
  P.help_stride = sv::help_stride(V);
  sv::TreeDesc td{};
  if (tree) {
    std::memcpy(td.parent, ti->parent, 64);
    std::memcpy(td.first_child, ti->first_child, 64);
    std::memcpy(td.nchild, ti->nchild, 64);
    std::memcpy(td.depth, ti->depth, 64);
    td.N = ti->N;
    td.D = ti->D;
    P.tree_skip = 1;
    for (int u = 0; u < ti->N; ++u)
      if (ti->nchild[u] > 31) P.tree_skip = 0;
    P.leaf_wait = P.tree_skip && lossless;
  }
  // How the residual reads q rows (see launch_rows): every logits row must have the same
  // 16-byte phase (whole-vector pitch), and the matching q chunks must line up with it.
  int qmode = lossless ? 3 : 0;  // 3: the lossless tree, which reads no q rows
  const uintptr_t la = reinterpret_cast<uintptr_t>(logits), qa = reinterpret_cast<uintptr_t>(probs);
  if (!tree && k > 0) {
    if (lt == qt && (static_cast<int64_t>(V) * (bf16 ? 2 : 4)) % 16 == 0 && (la & 15) == (qa & 15)) {
      qmode = 1;
    } else if (lt == SV_F32 && qt == SV_BF16 && (static_cast<int64_t>(V) * 4) % 16 == 0 &&
               (static_cast<int64_t>(V) * 2) % 8 == 0 && ((qa - 2 * ((la & 15) / 4)) & 7) == 0) {
      qmode = 2;
    }
  }
  (void)hipGetLastError();
  // Linear batches whose rows, cut into slices of one tile each, all fit the chip at once
  // take the split kernel: every row is reduced and drawn by several CUs together.
  sv::SplitConfig sc;
  if (!tree && sv::choose_split(bf16, qmode == 1 ? 1 : 0, V, head_max(logits, V, lt), static_cast<int64_t>(B) * R,
                                &sc)) {
    sv::SplitParams S{};
    S.logits = logits;
    S.probs = probs;
    S.tokens = tokens;
    S.B = B;
    S.R = R;
    S.V = V;
    S.k = k;
    S.S = sc.S;
    S.chunk = sc.chunk;
    S.q_bf16 = P.q_bf16;
    S.c = P.c;
    S.invT = 1.0 / P.T;
    S.seed = seed;
    S.offset = offset;
    S.out_tokens = out_tokens;
    S.out_accept_len = out_len;
    S.out_tprob = tprob;
    S.out_aprob = aprob;
    char* w = static_cast<char*>(ws);
    S.gen = reinterpret_cast<uint64_t*>(w + L.gen_off);
    S.first_rej = reinterpret_cast<uint64_t*>(w + L.rej_off);
    S.words = reinterpret_cast<uint64_t*>(w + L.words_off);
    S.errword = reinterpret_cast<uint32_t*>(w + L.status_off);
    const hipError_t e = sv::launch_split(S, bf16, qmode == 1 ? 1 : 0, sc, st);
    return e == hipSuccess ? SV_OK : SV_E_LAUNCH;
  }
  // A rejected row walked in tiles gets help from the later rows of its sequence when a
  // row's units fit one wave's lanes (the row waits for the tiles its helpers claimed;
  // a helper claims only while it runs, so no wait depends on a workgroup not yet started).
  const int64_t rows = static_cast<int64_t>(B) * R;
  P.help_on = !tree && k > 0 && rc.ntiles > 1 && rows <= sv::kHelpRows && rc.ntiles * (rc.threads / 64) <= 64 &&
              rc.ntiles * (rc.threads / 64) + 3 <= P.help_stride;
  const hipError_t e = sv::launch_rows(P, td, bf16, tree, qmode, rc.cfg, B * R, st);
  return e == hipSuccess ? SV_OK : SV_E_LAUNCH;
}

}  // namespace

extern "C" {

int spec_verify_linear(const void* target_logits, int lt, const void* draft_probs, int qt,
                       const int32_t* draft_tokens, int32_t B, int32_t k, int32_t V, float temperature,
                       uint64_t seed, uint64_t offset, int32_t* out_tokens, int32_t* out_accept_len,
                       float* out_target_prob, float* out_accept_prob, void* workspace,
                       size_t workspace_bytes, void* stream) {
  int rc = sv::validate_linear(target_logits, lt, draft_probs, qt, draft_tokens, B, k, V, temperature,
                               out_tokens, out_accept_len, workspace, workspace_bytes);
  if (rc != SV_OK || B == 0) return rc;
  if ((rc = check_device())) return rc;
  return run_rows(false, false, target_logits, lt, draft_probs, qt, draft_tokens, B, k + 1, k, V, temperature,
                  seed, offset, out_tokens, out_accept_len, out_target_prob, out_accept_prob, nullptr,
                  nullptr, workspace, static_cast<hipStream_t>(stream));
}

int spec_verify_greedy(const void* target_logits, int lt, const int32_t* draft_tokens, int32_t B, int32_t k,
                       int32_t V, int32_t* out_tokens, int32_t* out_accept_len, void* workspace,
                       size_t workspace_bytes, void* stream) {
  int rc = sv::validate_greedy(target_logits, lt, draft_tokens, B, k, V, out_tokens, out_accept_len,
                               workspace, workspace_bytes);
  if (rc != SV_OK || B == 0) return rc;
  if ((rc = check_device())) return rc;
  sv::WsLayout L;
  sv::workspace_layout(SV_KIND_GREEDY, B, k, V, 0, &L);
  sv::GreedyParams P{};
  P.logits = target_logits;
  P.tokens = draft_tokens;
  P.B = B;
  P.R = k + 1;
  P.V = V;
  P.k = k;
  P.S = sv::greedy_splits(B, k + 1, V);
  // flat path: the tensor starts on a 16-byte boundary and every row is whole vectors
  const int64_t row_bytes = static_cast<int64_t>(V) * (lt == SV_BF16 ? 2 : 4);
  const int64_t nvec = row_bytes / 16;
  P.flat = 0;
  if (row_bytes % 16 == 0 && (reinterpret_cast<uintptr_t>(target_logits) & 15) == 0 &&
      static_cast<int64_t>(k + 1) * nvec < (int64_t(1) << 31)) {
    const int64_t total = static_cast<int64_t>(B) * (k + 1) * nvec;
    int64_t G = (total + sv::kGreedyFlatMinVectors - 1) / sv::kGreedyFlatMinVectors;
    if (G > sv::kGreedyFlatMaxGroups) G = sv::kGreedyFlatMaxGroups;
    P.flat = 1;
    P.nvec = static_cast<int32_t>(nvec);
    P.G = static_cast<int32_t>(G < 1 ? 1 : G);
    // Two launches (the first two positions of every sequence, then the rest of the
    // sequences that kept both) when the tensor is larger than one round of pieces of the
    // minimum size would cover twice over.
    constexpr int kFirstPositions = 2;
    if (k + 1 > kFirstPositions && total >= int64_t(2) * sv::kGreedyFlatMaxGroups * sv::kGreedyFlatMinVectors) {
      P.phase = 1;
      P.P0 = kFirstPositions;
    }
  }
  P.alive = reinterpret_cast<uint32_t*>(static_cast<char*>(workspace) + L.seq_off);
  P.out_tokens = out_tokens;
  P.out_accept_len = out_accept_len;
  P.counters = reinterpret_cast<uint32_t*>(static_cast<char*>(workspace) + L.counters_off);
  P.rowword = reinterpret_cast<uint64_t*>(static_cast<char*>(workspace) + L.row_off);
  (void)hipGetLastError();
  const hipError_t e = sv::launch_greedy(P, lt == SV_BF16, static_cast<hipStream_t>(stream));
  return e == hipSuccess ? SV_OK : SV_E_LAUNCH;
}

int spec_verify_tree(const void* target_logits, int lt, const void* draft_probs, int qt,
                     const int32_t* node_tokens, const int32_t* parent_host, int32_t B, int32_t N, int32_t V,
                     float temperature, uint64_t seed, uint64_t offset, int32_t* out_tokens,
                     int32_t* out_accept_len, int32_t* out_path, void* workspace, size_t workspace_bytes,
                     void* stream) {
  sv::TreeInfo ti;
  int rc = sv::validate_tree(target_logits, lt, draft_probs, qt, node_tokens, parent_host, B, N, V, temperature,
                             out_tokens, out_accept_len, workspace, workspace_bytes, &ti);
  if (rc != SV_OK || B == 0) return rc;
  if ((rc = check_device())) return rc;
  return run_rows(true, false, target_logits, lt, draft_probs, qt, node_tokens, B, N, 0, V, temperature, seed, offset,
                  out_tokens, out_accept_len, nullptr, nullptr, out_path, &ti, workspace,
                  static_cast<hipStream_t>(stream));
}

int spec_verify_tree_lossless(const void* target_logits, int lt, const int32_t* node_tokens,
                              const int32_t* parent_host, int32_t B, int32_t N, int32_t V, float temperature,
                              uint64_t seed, uint64_t offset, int32_t* out_tokens, int32_t* out_accept_len,
                              int32_t* out_path, void* workspace, size_t workspace_bytes, void* stream) {
  sv::TreeInfo ti;
  int rc = sv::validate_tree_lossless(target_logits, lt, node_tokens, parent_host, B, N, V, temperature, out_tokens,
                                      out_accept_len, workspace, workspace_bytes, &ti);
  if (rc != SV_OK || B == 0) return rc;
  if ((rc = check_device())) return rc;
  return run_rows(true, true, target_logits, lt, nullptr, lt, node_tokens, B, N, 0, V, temperature, seed, offset,
                  out_tokens, out_accept_len, nullptr, nullptr, out_path, &ti, workspace,
                  static_cast<hipStream_t>(stream));
}

int spec_lmhead_verify(const void* hidden, const void* lm_head, const void* draft_probs, int qt,
                       const int32_t* draft_tokens, int32_t B, int32_t k, int32_t H, int32_t V,
                       float temperature, uint64_t seed, uint64_t offset, float* logits_out,
                       int32_t* out_tokens, int32_t* out_accept_len, float* out_target_prob,
                       float* out_accept_prob, void* workspace, size_t workspace_bytes, void* stream) {
  int rc = sv::validate_lmhead(hidden, lm_head, draft_probs, qt, draft_tokens, B, k, H, V, temperature,
                               logits_out, out_tokens, out_accept_len, workspace, workspace_bytes);
  if (rc != SV_OK || B == 0) return rc;
  if ((rc = check_device())) return rc;
  const hipStream_t st = static_cast<hipStream_t>(stream);
  (void)hipGetLastError();
  // The direct GEMM kernel also writes each row's softmax partials per block of 512 columns;
  // verification then starts from them instead of re-reading the float32 logits.  Other
  // shapes and alignments verify the written logits with the row kernels.
  const bool fused = sv::lmhead_gemm_direct(lm_head, logits_out, V) && sv::lmh_blocks(V) <= sv::kLmhMaxBlocks &&
                     (k == 0 || (reinterpret_cast<uintptr_t>(draft_probs) & 15) == 0);
  sv::WsLayout L;
  sv::workspace_layout(SV_KIND_LMHEAD, B, k, V, H, &L);
  char* w = static_cast<char*>(workspace);
  const float c = static_cast<float>(1.4426950408889634 / static_cast<double>(temperature));
  uint64_t* part = fused ? reinterpret_cast<uint64_t*>(w + L.lmh_part_off) : nullptr;
  if (sv::launch_lmhead_gemm(hidden, lm_head, logits_out, B * (k + 1), H, V, st, part, c) != hipSuccess)
    return SV_E_LAUNCH;
  if (!fused)
    return run_rows(false, false, logits_out, SV_F32, draft_probs, qt, draft_tokens, B, k + 1, k, V, temperature,
                    seed, offset, out_tokens, out_accept_len, out_target_prob, out_accept_prob, nullptr, nullptr,
                    workspace, st);
  sv::LmhParams P{};
  P.logits = logits_out;
  P.probs = draft_probs;
  P.tokens = draft_tokens;
  P.B = B;
  P.R = k + 1;
  P.k = k;
  P.V = V;
  P.nb = static_cast<int32_t>(sv::lmh_blocks(V));
  P.nchunks = static_cast<int32_t>((static_cast<int64_t>(V) + 8191) / 8192);
  P.cstride = static_cast<int32_t>(sv::lmh_chunks(V));
  P.q_bf16 = (qt == SV_BF16);
  P.c = c;
  P.T = static_cast<double>(temperature);
  P.seed = seed;
  P.offset = offset;
  P.out_tokens = out_tokens;
  P.out_accept_len = out_accept_len;
  P.out_tprob = out_target_prob;
  P.out_aprob = out_accept_prob;
  P.part = part;
  P.seqw = reinterpret_cast<uint64_t*>(w + L.lmh_seq_off);
  P.cmass = reinterpret_cast<uint32_t*>(w + L.lmh_mass_off);
  P.ccnt = reinterpret_cast<uint32_t*>(w + L.lmh_cnt_off);
  return sv::launch_lmhead_verify(P, st) == hipSuccess ? SV_OK : SV_E_LAUNCH;
}

int spec_lmhead_logits(const void* hidden, const void* lm_head, int32_t M, int32_t H, int32_t V, float* logits_out,
                       void* stream) {
  int rc = sv::validate_lmhead_logits(hidden, lm_head, M, H, V, logits_out);
  if (rc != SV_OK || M == 0) return rc;
  if ((rc = check_device())) return rc;
  (void)hipGetLastError();
  return sv::launch_lmhead_gemm(hidden, lm_head, logits_out, M, H, V, static_cast<hipStream_t>(stream)) == hipSuccess
             ? SV_OK
             : SV_E_LAUNCH;
}

int spec_verify_linear_noalloc(const void* target_logits, int lt, const void* draft_probs, int qt,
                               const int32_t* draft_tokens, int32_t B, int32_t k, int32_t V, float temperature,
                               uint64_t seed, uint64_t offset, int32_t* out_tokens, int32_t* out_accept_len,
                               float* out_target_prob, float* out_accept_prob, void* stream) {
  sv::WsLayout L;
  if (k >= 0 && sv::workspace_layout(SV_KIND_LINEAR, B, k, V, 0, &L) && L.total > kScratchBytes)
    return SV_E_SCRATCH;
  // the scratch stands in for the workspace in validation (any non-null pointer will do)
  int rc = sv::validate_linear(target_logits, lt, draft_probs, qt, draft_tokens, B, k, V, temperature, out_tokens,
                               out_accept_len, &kScratchBytes, kScratchBytes);
  if (rc != SV_OK || B == 0) return rc;
  if ((rc = check_device())) return rc;
  void* ws = scratch_device_ptr();
  if (ws == nullptr) return SV_E_DEVICE;
  const hipStream_t st = static_cast<hipStream_t>(stream);
  (void)hipGetLastError();
  // the words must be zero on entry: clear the ones this call uses
  const uint32_t words = static_cast<uint32_t>(L.total / 4);
  const int blocks = static_cast<int>(std::min<uint32_t>(64u, (words + 255u) / 256u));
  hipLaunchKernelGGL(zero_words_kernel, dim3(blocks), dim3(256), 0, st, static_cast<uint32_t*>(ws), words);
  if (hipGetLastError() != hipSuccess) return SV_E_LAUNCH;
  return run_rows(false, false, target_logits, lt, draft_probs, qt, draft_tokens, B, k + 1, k, V, temperature,
                  seed, offset, out_tokens, out_accept_len, out_target_prob, out_accept_prob, nullptr,
                  nullptr, ws, st);
}

size_t spec_verify_workspace_bytes(int kind, int32_t B, int32_t k_or_N, int32_t V, int32_t H) {
  sv::WsLayout L;
  if (!sv::workspace_layout(kind, B, k_or_N, V, H, &L)) return 0;
  return L.total;
}

const char* spec_verify_strerror(int code) {
  switch (code) {
    case SV_OK: return "ok";
    case SV_E_NULL: return "a required pointer is NULL";
    case SV_E_SHAPE: return "invalid shape (B, k+1 <= 64, N <= 64, V, H)";
    case SV_E_DTYPE: return "dtype must be SV_F32 or SV_BF16";
    case SV_E_TEMP: return "temperature must be finite and > 0";
    case SV_E_TREE: return "parent array is not a BFS-ordered tree with parent[0] = -1";
    case SV_E_WORKSPACE: return "workspace is NULL or too small";
    case SV_E_DEVICE: return "current HIP device is not gfx950";
    case SV_E_LAUNCH: return "kernel launch failed";
    case SV_E_ALIGN: return "tensor pointer is misaligned for its element type";
    case SV_E_SCRATCH: return "sizes need more than the library's static scratch (4 MiB per device)";
    default: return "unknown error";
  }
}

int spec_plug_tokens(const int32_t* out_tokens, const int32_t* out_accept_len, int32_t B, int32_t W,
                     int32_t* seq_len, int32_t* history, int32_t cap, int32_t* next_token, int32_t* status,
                     void* stream) {
  int rc = sv::validate_plug(out_tokens, out_accept_len, B, W, seq_len, history, cap, next_token, status);
  if (rc != SV_OK || B == 0) return rc;
  if ((rc = check_device())) return rc;
  sv::PlugParams P{};
  P.tokens = out_tokens;
  P.accept_len = out_accept_len;
  P.seq_len = seq_len;
  P.history = history;
  P.next_token = next_token;
  P.status = status;
  P.B = B;
  P.W = W;
  P.cap = cap;
  (void)hipGetLastError();
  return sv::launch_plug(P, static_cast<hipStream_t>(stream)) == hipSuccess ? SV_OK : SV_E_LAUNCH;
}

int spec_lookup_drafts(const int32_t* history, const int32_t* seq_len, int32_t B, int32_t cap, int32_t min_ngram,
                       int32_t max_ngram, int32_t k, int32_t* out_drafts, int32_t* out_count, void* stream) {
  int rc = sv::validate_lookup(history, seq_len, B, cap, min_ngram, max_ngram, k, out_drafts, out_count);
  if (rc != SV_OK || B == 0) return rc;
  if ((rc = check_device())) return rc;
  sv::LookupParams P{};
  P.history = history;
  P.seq_len = seq_len;
  P.B = B;
  P.cap = cap;
  P.min_ngram = min_ngram;
  P.max_ngram = max_ngram;
  P.k = k;
  P.drafts = out_drafts;
  P.count = out_count;
  (void)hipGetLastError();
  return sv::launch_lookup(P, static_cast<hipStream_t>(stream)) == hipSuccess ? SV_OK : SV_E_LAUNCH;
}

}  // extern "C"
