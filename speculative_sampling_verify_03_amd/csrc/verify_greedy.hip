// Greedy verification: a draft token is kept while it equals the target's argmax, and the
// target's argmax at the first mismatch (or after the last draft) is appended.  This is
// the "sample the top token" drafting mode of "Accelerating Sonar through speculation"
// (section "Target-Draft") checked with an exact argmax instead of a probability test.
//
// Each row is split over S workgroups that stream their slice once with 16-byte loads
// and reduce (value, lowest index); the slices of a row merge through an atomic max of an
// orderable key, and the last workgroup of a sequence to arrive finds the first mismatch
// with a ballot and writes the outputs.

#include <climits>

#include "sv_device.hpp"
#include "sv_launch.hpp"

namespace sv {

template <bool BF16>
__global__ __launch_bounds__(kGreedyThreads) void greedy_kernel(GreedyParams P) {
  using E = Elem<BF16>;
  constexpr int VE = E::kPerVec;
  constexpr int EB = E::kBytes;
  constexpr int NT = kGreedyThreads;
  constexpr int U = kGreedyUnroll;
  constexpr int NW = NT / kWave;
  __shared__ float s_v[NW];
  __shared__ int s_i[NW];
  __shared__ int s_last;

  const int tid = threadIdx.x;
  const int lane = tid & (kWave - 1);
  const int wid = tid / kWave;
  const int S = P.S;
  const int r = blockIdx.x / S;
  const int s = blockIdx.x - r * S;
  const int b = r / P.R;
  const int V = P.V;

  const char* rowp = static_cast<const char*>(P.logits) + static_cast<size_t>(r) * V * EB;
  const uintptr_t ra = reinterpret_cast<uintptr_t>(rowp);
  const int h = static_cast<int>(ra & 15) / EB;
  const SV_GLOBAL Vec16* vrow = gptr<Vec16>(reinterpret_cast<const void*>(ra - (ra & 15)));
  const int nvec = (V + h + VE - 1) / VE;
  const int chunk = (nvec + S - 1) / S;
  const int vbeg = s * chunk;
  const int vend = min(nvec, vbeg + chunk);

  float bv = -INFINITY;
  int bi = INT_MAX;
  for (int base = vbeg + tid; base < vend; base += NT * U) {
    Vec16 t[U];
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int vi = base + u * NT;
      t[u] = ld16(vrow, vi, vend);
    }
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int vi = base + u * NT;
      const int e0 = vi * VE - h;
      const bool full = vi < vend && e0 >= 0 && e0 + VE <= V;
#pragma unroll
      for (int e = 0; e < VE; ++e) {
        const bool ok = full || (vi < vend && e0 + e >= 0 && e0 + e < V);
        if (ok) argmax_merge(bv, bi, E::at(t[u], e), e0 + e);
      }
    }
  }
  wave_argmax(bv, bi);
  if (lane == 0) {
    s_v[wid] = bv;
    s_i[wid] = bi;
  }
  __syncthreads();
  if (tid == 0) {
    float v = s_v[0];
    int i = s_i[0];
    for (int w = 1; w < NW; ++w) argmax_merge(v, i, s_v[w], s_i[w]);
    // the row's slices merge through one atomic max of an orderable (value, index) key
    const uint64_t old = atomic_max_u64(&P.rowword[r], argmax_key(v, i));
    after_value(old);
    const uint32_t prev = take_ticket(&P.counters[b]);
    s_last = prev == static_cast<uint32_t>(P.R * S - 1);
  }
  __syncthreads();
  if (!s_last || wid != 0) return;

  // last arrival: each row's argmax, then the first mismatch
  const int k = P.k;
  int g = -1;
  if (lane < P.R) g = argmax_key_index(atomic_xchg_u64(&P.rowword[static_cast<size_t>(b) * P.R + lane], 0ull));
  int x = -1;
  if (lane < k) x = gptr<int32_t>(P.tokens)[static_cast<size_t>(b) * k + lane];
  const uint64_t miss = __ballot(lane < k && g != x);
  const int n = miss ? __ffsll(static_cast<long long>(miss)) - 1 : k;
  const int y = lane_value(g, n);
  if (lane < P.R) {
    int t = -1;
    if (lane < n) t = x;
    else if (lane == n) t = y;
    P.out_tokens[static_cast<size_t>(b) * P.R + lane] = t;
  }
  if (lane == 0) {
    P.out_accept_len[b] = n;
    reset_ticket(&P.counters[b]);
  }
}

hipError_t launch_greedy(const GreedyParams& P, bool bf16, hipStream_t st) {
  const int grid = P.B * P.R * P.S;
  if (bf16) hipLaunchKernelGGL(greedy_kernel<true>, dim3(grid), dim3(kGreedyThreads), 0, st, P);
  else hipLaunchKernelGGL(greedy_kernel<false>, dim3(grid), dim3(kGreedyThreads), 0, st, P);
  return hipGetLastError();
}

}  // namespace sv
