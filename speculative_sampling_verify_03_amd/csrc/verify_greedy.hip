// Greedy verification: a draft token is kept while it equals the target's argmax, and the
// target's argmax at the first mismatch (or after the last draft) is appended.  This is
// the "sample the top token" drafting mode of "Accelerating Sonar through speculation"
// (section "Target-Draft") checked with an exact argmax instead of a probability test.
//
// Each row is split over S workgroups that stream their slice once with 16-byte loads
// and reduce (value, lowest index); the slices of a row merge through an atomic max of an
// orderable key, and the last workgroup of a sequence to arrive finds the first mismatch
// with a ballot and writes the outputs.  Tensors whose rows are whole 16-byte vectors take
// the flat path below instead (equal contiguous ranges of the whole tensor).

#include <climits>
#include <mutex>

#include "sv_device.hpp"
#include "sv_launch.hpp"

namespace sv {

__device__ void greedy_finish(const GreedyParams& P, int b, int lane);
__device__ void greedy_first_positions(const GreedyParams& P, int b, int lane);

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

  // Whole vectors: a max per element, and the first vector reaching the running maximum
  // kept with its data (its element index looked up once at the end).  The row's first and
  // last vectors may be partial: those take the exact per-element (value, index) merge.
  float best = -INFINITY;
  int best_vi = -1;
  Vec16 best_v{};
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
      float vm = E::at(t[u], 0);
#pragma unroll
      for (int e = 1; e < VE; ++e) vm = fmaxf(vm, E::at(t[u], e));
      const bool take = full && (vm > best || best_vi < 0);
      best = take ? vm : best;
      best_vi = take ? vi : best_vi;
#pragma unroll
      for (int w = 0; w < 4; ++w) best_v.w[w] = take ? t[u].w[w] : best_v.w[w];
    }
  }
  // The partial edge vectors (the row's first when it starts inside a vector, its last
  // when it ends inside one) are merged element by element by the thread whose stride
  // passed them, after the loop: a branch inside the loop kept every loaded vector live.
  for (int ev = 0; ev < 2; ++ev) {
    const int vi = ev == 0 ? 0 : nvec - 1;
    const int e0 = vi * VE - h;
    const bool partial = e0 < 0 || e0 + VE > V;
    if (partial && vi >= vbeg && vi < vend && (vi - vbeg) % NT == tid && (ev == 0 || vi != 0)) {
      const Vec16 t = ld16(vrow, vi, nvec);
      for (int e = 0; e < VE; ++e)
        if (e0 + e >= 0 && e0 + e < V) argmax_merge(bv, bi, E::at(t, e), e0 + e);
    }
  }
  if (best_vi >= 0) {
    int idx = INT_MAX;
#pragma unroll
    for (int e = VE - 1; e >= 0; --e)
      if (E::at(best_v, e) == best) idx = best_vi * VE - h + e;
    argmax_merge(bv, bi, best, idx);
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

  greedy_finish(P, b, lane);  // last arrival
}

// Last arrival of sequence b: each row's argmax from its key word (which is cleared for
// the next call), then the first mismatch by ballot, then the outputs.  One wave.
__device__ void greedy_finish(const GreedyParams& P, int b, int lane) {
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

// Flat path, for a 16-byte aligned tensor whose rows are whole vectors: the B * R * nvec
// vectors of the tensor are cut into G equal contiguous ranges, one per workgroup, so every
// workgroup streams the same number of bytes and the grid fits the chip in one round.  A
// range is walked in pieces that end at row boundaries; each piece's (value, lowest index)
// goes into its row's key word with one atomic max, and its vector count into the
// sequence's counter, so the piece that brings the count to R * nvec is the sequence's
// last and writes its outputs.  Large tensors take two launches of this kernel (phase 1:
// positions 0 and 1 of every sequence; phase 2: the later positions of the sequences that
// kept both, listed by phase 1), since the rows after a sequence's first mismatch are never
// examined by the sequential rule.
template <bool BF16>
__global__ __launch_bounds__(kGreedyThreads) void greedy_flat_kernel(GreedyParams P) {
  using E = Elem<BF16>;
  constexpr int VE = E::kPerVec;
  constexpr int NT = kGreedyThreads;
  constexpr int U = kGreedyFlatUnroll;
  constexpr int NW = NT / kWave;
  __shared__ float s_v[NW];
  __shared__ int s_i[NW];
  __shared__ int s_last;

  const int tid = threadIdx.x;
  const int lane = tid & (kWave - 1);
  const int wid = tid / kWave;
  const int64_t nvec = P.nvec;
  // The rows of this launch, numbered t = a * RP + jj: phase 0 every row, phase 1 the first
  // P0 positions of every sequence, phase 2 the later positions of the listed sequences.
  const int phase = P.phase;
  const int RP = phase == 0 ? P.R : phase == 1 ? P.P0 : P.R - P.P0;
  const int j0 = phase == 2 ? P.P0 : 0;
  uint32_t* const nalive = P.alive + P.B;
  int64_t nseq = P.B;
  if (phase == 2) nseq = __hip_atomic_load(nalive, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  const int64_t total = nseq * RP * nvec;
  const int64_t beg = total * blockIdx.x / P.G;
  const int64_t end = total * (blockIdx.x + 1) / P.G;
  const SV_GLOBAL Vec16* base = gptr<Vec16>(P.logits);
  // a sequence's vectors counted when this launch's share of it is done
  const uint32_t seq_vectors = static_cast<uint32_t>((phase == 1 ? P.P0 : P.R) * nvec);

  int64_t pos = beg;
  int64_t t = beg / nvec;
  while (pos < end) {
    const int64_t row0 = t * nvec;
    const int64_t piece_end = min(end, row0 + nvec);
    const int n = static_cast<int>(piece_end - pos);    // vectors in this piece
    const int first = static_cast<int>(pos - row0);     // its first vector inside the row
    const int64_t a = t / RP;
    const int b = phase == 2 ? static_cast<int>(P.alive[a]) : static_cast<int>(a);
    const int64_t r = static_cast<int64_t>(b) * P.R + j0 + (t - a * RP);
    const SV_GLOBAL Vec16* pp = base + r * nvec + first;
    // Per thread: the largest vector maximum, the first of this thread's vectors (they
    // ascend) that reaches it, and that vector's data; the element index is looked up once
    // at the end.  A max per element instead of a (value, index) compare and select.
    float best = -INFINITY;
    int best_i = -1;
    Vec16 best_v{};
    for (int i0 = tid; i0 < n; i0 += NT * U) {
      Vec16 t[U];
#pragma unroll
      for (int u = 0; u < U; ++u) t[u] = ld16_stream(pp, i0 + u * NT, n);  // i >= n: unused below
#pragma unroll
      for (int u = 0; u < U; ++u) {
        const int i = i0 + u * NT;
        float vm = E::at(t[u], 0);
#pragma unroll
        for (int e = 1; e < VE; ++e) vm = fmaxf(vm, E::at(t[u], e));
        const bool take = i < n && (vm > best || best_i < 0);
        best = take ? vm : best;
        best_i = take ? i : best_i;
#pragma unroll
        for (int w = 0; w < 4; ++w) best_v.w[w] = take ? t[u].w[w] : best_v.w[w];
      }
    }
    float bv = -INFINITY;
    int bi = INT_MAX;
    if (best_i >= 0) {
      bv = best;
#pragma unroll
      for (int e = VE - 1; e >= 0; --e)
        if (E::at(best_v, e) == best) bi = (first + best_i) * VE + e;
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
      const uint64_t old = atomic_max_u64(&P.rowword[r], argmax_key(v, i));
      after_value(old);  // the key is in place before the count says so
      const uint32_t prev = atomicAdd(&P.counters[b], static_cast<uint32_t>(n));
      s_last = prev + static_cast<uint32_t>(n) == seq_vectors;
    }
    __syncthreads();  // also: s_v is rewritten by the next piece only after this
    if (s_last && wid == 0) {
      if (phase == 1) greedy_first_positions(P, b, lane);
      else greedy_finish(P, b, lane);
    }
    pos = piece_end;
    ++t;
  }
  if (phase == 2) {
    // the last workgroup of phase 2 clears the list, its count and these tickets (every
    // workgroup has read the list before taking its ticket)
    if (tid == 0) s_last = take_ticket(nalive + 1) == static_cast<uint32_t>(P.G - 1);
    __syncthreads();
    if (s_last && wid == 0) {
      for (int64_t q = lane; q < nseq; q += kWave)
        __hip_atomic_store(&P.alive[q], 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      if (lane == 0) {
        reset_ticket(nalive);
        reset_ticket(nalive + 1);
      }
    }
  }
}

// Phase 1's last arrival for sequence b (positions 0 .. P0-1 done, P0 <= k): a mismatch
// among them ends the sequence here (outputs, its words cleared); otherwise it is listed
// for phase 2, whose last arrival reads every row's key.  One wave.
__device__ void greedy_first_positions(const GreedyParams& P, int b, int lane) {
  const int P0 = P.P0;
  uint64_t* keys = P.rowword + static_cast<size_t>(b) * P.R;
  int g = -1, x = -1;
  if (lane < P0) {
    g = argmax_key_index(__hip_atomic_load(keys + lane, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT));
    x = gptr<int32_t>(P.tokens)[static_cast<size_t>(b) * P.k + lane];
  }
  const uint64_t miss = __ballot(lane < P0 && g != x);
  if (miss) {
    const int n = __ffsll(static_cast<long long>(miss)) - 1;
    const int y = lane_value(g, n);
    if (lane < P.R) {
      int tk = -1;
      if (lane < n) tk = x;
      else if (lane == n) tk = y;
      P.out_tokens[static_cast<size_t>(b) * P.R + lane] = tk;
    }
    if (lane < P0) (void)atomic_xchg_u64(keys + lane, 0ull);
    if (lane == 0) {
      P.out_accept_len[b] = n;
      reset_ticket(&P.counters[b]);
    }
  } else if (lane == 0) {
    const uint32_t at = __hip_atomic_fetch_add(P.alive + P.B, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    __hip_atomic_store(&P.alive[at], static_cast<uint32_t>(b), __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  }
}

// Workgroups of the flat kernel that the current device holds at once (occupancy x CUs),
// cached per device and dtype; 0 if the runtime cannot say.
static int flat_resident_groups(bool bf16) {
  static std::mutex mu;
  static int cache[64][2] = {};
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return 0;
  std::lock_guard<std::mutex> g(mu);
  int& c = cache[dev][bf16 ? 1 : 0];
  if (c == 0) {
    int per_cu = 0, cus = 0;
    const hipError_t e1 = bf16 ? hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, greedy_flat_kernel<true>,
                                                                             kGreedyThreads, 0)
                               : hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, greedy_flat_kernel<false>,
                                                                             kGreedyThreads, 0);
    const hipError_t e2 = hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev);
    if (e1 != hipSuccess || e2 != hipSuccess || per_cu < 1 || cus < 1) return 0;
    c = per_cu * cus;
  }
  return c;
}

hipError_t launch_greedy(const GreedyParams& P0, bool bf16, hipStream_t st) {
  if (P0.flat) {
    // one round: no more workgroups than the chip holds at once
    GreedyParams P = P0;
    const int resident = flat_resident_groups(bf16);
    auto run = [&](GreedyParams& Q) {
      if (bf16) hipLaunchKernelGGL(greedy_flat_kernel<true>, dim3(Q.G), dim3(kGreedyThreads), 0, st, Q);
      else hipLaunchKernelGGL(greedy_flat_kernel<false>, dim3(Q.G), dim3(kGreedyThreads), 0, st, Q);
      return hipGetLastError();
    };
    if (P.phase == 0) {
      if (resident > 0 && P.G > resident) P.G = resident;
      return run(P);
    }
    // Two launches: the first P0 positions of every sequence, then the rest of the
    // sequences that kept all of them (the sequential rule stops at the first mismatch,
    // so the later rows of the others are never read).  Phase 2 does not know its size
    // on the host: it takes the whole resident grid and each workgroup reads the count.
    const int64_t total1 = static_cast<int64_t>(P.B) * P.P0 * P.nvec;
    int64_t G1 = (total1 + kGreedyFlatMinVectors - 1) / kGreedyFlatMinVectors;
    const int cap = resident > 0 ? resident : kGreedyFlatMaxGroups;
    if (G1 > cap) G1 = cap;
    P.phase = 1;
    P.G = static_cast<int32_t>(G1 < 1 ? 1 : G1);
    hipError_t e = run(P);
    if (e != hipSuccess) return e;
    P.phase = 2;
    P.G = cap;
    return run(P);
  }
  const GreedyParams& P = P0;
  const int grid = P.B * P.R * P.S;
  if (bf16) hipLaunchKernelGGL(greedy_kernel<true>, dim3(grid), dim3(kGreedyThreads), 0, st, P);
  else hipLaunchKernelGGL(greedy_kernel<false>, dim3(grid), dim3(kGreedyThreads), 0, st, P);
  return hipGetLastError();
}

}  // namespace sv
