// Prompt-lookup drafting ("Speculative decoding explained", section "Variants without a
// separate draft model"): drafts are the tokens that followed an earlier occurrence of the
// history's last phrase, found by scanning the history itself; no draft model.

#include "sv_device.hpp"
#include "sv_launch.hpp"

namespace sv {

constexpr int kLookupThreads = 1024;
constexpr int kLookupPer = 8;                              // end positions per thread and tile
constexpr int kLookupTile = kLookupThreads * kLookupPer;   // end positions per tile
constexpr int kLookupHalo = kMaxNgram;                     // tokens left of a tile's first end
constexpr int kLookupLoads = (kLookupTile + kLookupHalo + kLookupThreads - 1) / kLookupThreads;

// One workgroup per sequence, one pass over the history for every phrase length at once.
// An occurrence of the n-token phrase that starts at i ends at j = i + n - 1, and it is a
// match exactly when the history up to j and the whole phrase share a common suffix of at
// least n tokens.  So each end position j < len - 1 (at least one token must follow) gets
// that suffix length L(j), capped at max_ngram, and every n <= L(j) records start j - n + 1.
// Ends are visited in ascending tiles, so the first start recorded for a length is its
// earliest occurrence; once the longest length has one the scan stops, since the longest
// matching length decides.  The history is staged tile by tile through LDS, the next
// tile's tokens loaded into registers while the current one is compared.
template <int MAXN>  // phrase lengths up to MAXN (>= max_ngram) held in registers
__global__ __launch_bounds__(kLookupThreads) void lookup_kernel(LookupParams P) {
  __shared__ int s_tok[kLookupLoads * kLookupThreads];
  __shared__ int s_best[kMaxNgram];  // earliest start per phrase length n (index n - 1)
  const int tid = threadIdx.x;
  const int64_t b = blockIdx.x;
  const SV_GLOBAL int32_t* h = gptr<int32_t>(P.history) + b * P.cap;
  int len = P.seq_len[b];
  if (len < 0 || len > P.cap) len = 0;  // an invalid length drafts nothing
  const int maxn = P.max_ngram, minn = P.min_ngram;

  // the phrase, last token first: rev[r] = h[len - 1 - r]
  int rev[MAXN];
#pragma unroll
  for (int r = 0; r < MAXN; ++r) {
    const int pos = len - 1 - r;
    rev[r] = (r < maxn && pos >= 0) ? h[pos] : 0;
  }
  if (tid < kMaxNgram) s_best[tid] = INT_MAX;

  const int nend = len - 1;  // ends j in [0, len - 1)
  auto load_tile = [&](int c0, int (&v)[kLookupLoads]) {
#pragma unroll
    for (int u = 0; u < kLookupLoads; ++u) {
      const int p = c0 - kLookupHalo + u * kLookupThreads + tid;
      const bool ok = p >= 0 && p < len;
      v[u] = h[ok ? p : 0];
      if (!ok) v[u] = 0;
    }
  };
  int nxt[kLookupLoads];
  if (nend > 0) load_tile(0, nxt);
  // bit r set for the compared suffix positions r < max_ngram
  const uint32_t live = maxn >= 32 ? ~0u : (1u << maxn) - 1u;

  for (int c0 = 0; c0 < nend; c0 += kLookupTile) {
#pragma unroll
    for (int u = 0; u < kLookupLoads; ++u) s_tok[u * kLookupThreads + tid] = nxt[u];
    __syncthreads();
    if (c0 + kLookupTile < nend) load_tile(c0 + kLookupTile, nxt);

    int best[MAXN];
#pragma unroll
    for (int n = 0; n < MAXN; ++n) best[n] = INT_MAX;
#pragma unroll
    for (int s = kLookupPer - 1; s >= 0; --s) {  // descending, so the lowest end wins
      const int e = s * kLookupThreads + tid;
      const int j = c0 + e;
      int v[MAXN];
#pragma unroll
      for (int r = 0; r < MAXN; ++r) v[r] = s_tok[e + kLookupHalo - r];  // always inside s_tok
      uint32_t eq = 0;
#pragma unroll
      for (int r = 0; r < MAXN; ++r) eq |= (v[r] == rev[r] && r <= j) ? 1u << r : 0u;
      eq &= live;
      const int L = j < nend ? __builtin_ctz(~eq) : 0;  // leading run of equal tokens
#pragma unroll
      for (int n = 0; n < MAXN; ++n)
        if (n < L) best[n] = j - n;  // start of the (n + 1)-token occurrence ending at j
    }
#pragma unroll
    for (int n = 0; n < MAXN; ++n)
      if (n + 1 >= minn && n < maxn && best[n] != INT_MAX) atomicMin(&s_best[n], best[n]);
    __syncthreads();
    if (s_best[maxn - 1] != INT_MAX) break;  // the longest length matched: it decides
  }
  __syncthreads();

  int match = -1, nmatch = 0;
  for (int n = maxn; n >= minn; --n) {
    if (s_best[n - 1] != INT_MAX) {
      match = s_best[n - 1];
      nmatch = n;
      break;
    }
  }
  if (tid < P.k) {
    int t = -1;
    if (match >= 0) {
      const int pos = match + nmatch + tid;
      if (pos < len) t = h[pos];
    }
    P.drafts[b * P.k + tid] = t;
  }
  if (tid == 0) P.count[b] = match >= 0 ? min(P.k, len - match - nmatch) : 0;
}

hipError_t launch_lookup(const LookupParams& P, hipStream_t st) {
  const dim3 grid(static_cast<unsigned>(P.B)), block(kLookupThreads);
  if (P.max_ngram <= 4)
    hipLaunchKernelGGL(lookup_kernel<4>, grid, block, 0, st, P);
  else if (P.max_ngram <= 8)
    hipLaunchKernelGGL(lookup_kernel<8>, grid, block, 0, st, P);
  else
    hipLaunchKernelGGL(lookup_kernel<kMaxNgram>, grid, block, 0, st, P);
  return hipGetLastError();
}

}  // namespace sv
