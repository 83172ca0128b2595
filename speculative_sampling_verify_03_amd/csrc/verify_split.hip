// Linear speculative sampling with every vocabulary row split over S workgroups that run
// at the same time ("Accelerating Sonar through speculation", section "Speculative
// decoding": acceptance stage and target-generation stage; "Speculative decoding
// explained", section "Draft and verification loop": keep x with a probability that falls
// with the gap between the draft's and the target's confidence, else draw from the
// adjusted distribution).
//
// For batches whose rows all fit the chip at once when cut into S slices, each slice of a
// row is one workgroup that keeps its share of the row in registers.  The row's work is
//   1. every slice streams its share once (16-byte non-temporal loads) and reduces it to a
//      (max, sum of exp) pair, which it publishes in the row's slot for that slice;
//   2. every slice waits for the row's S pairs and merges them in slice order, so all of
//      them hold bit-identical (m, Z) and take the same acceptance decision for the draft
//      token (p(x) in float64, as the row kernel does); slice 0 publishes the decision;
//   3. a row whose token is rejected computes the residual max(0, p - q) over every slice
//      at once (the draft row is read by all S slices in parallel), publishes each slice's
//      residual mass, waits for the S masses and locates u * S: only the slice holding it
//      walks down to the token (wave totals, slot totals, lane scan, element walk, all on
//      values still in registers);
//   4. the last row (all drafts kept) draws from p itself: the pass-1 pairs already give
//      every slice's mass, so only the winning slice acts, with no second exchange;
//   5. the slice that drew reads the decisions of the sequence's earlier rows: when they
//      were all kept, its row is where the sequence ends and it writes the outputs.
//
// Every message between workgroups is made of 64-bit words, each written whole by an
// agent-scope atomic store and read whole by agent-scope atomic loads; a word holds a
// 48-bit tag and 16 bits of the message, and a reader acts on a word only once it carries
// the tag it expects, so no ordering between different words is needed: relaxed atomics
// suffice and no cache write-back or invalidation is issued (agent-scope release or
// acquire fences each write back or invalidate a whole L2 on this chip, measured at
// 17-24 us per launch).  Words are never cleared.  A tag names the sequence and the call:
// (generation + 1) << 11 | b.  Every workgroup takes a ticket on its sequence's 64-bit
// counter when it starts; the counter sits at a multiple of 2^16 when a call begins, so
// all R * S workgroups of the sequence read the same generation (ticket >> 16), and the
// one that draws the last ticket of the call moves the counter on to the next multiple.
// A sequence's generation grows with every call that includes it, and the words live in a
// prefix of the workspace whose place never depends on the sizes of a call, so a word
// left by an earlier call never carries a tag a later call expects.
//
// Waits: a slice waits only for the other slices of its row and, before writing the
// outputs, for the decisions of earlier rows of its sequence.  Both have lower or nearby
// workgroup indices (rows are laid out position by position, a row's slices next to each
// other), and the host launches the split kernel only when the whole grid fits the chip
// at once, so every awaited workgroup is running; workgroups are also dispatched in index
// order, so even on a chip shared with other work the lowest waiting row always has all
// the workgroups it waits for started.  Every wait is bounded all the same: one that runs
// out sets a sticky error word and the workgroup carries on, so the kernel always ends.

#include <mutex>

#include "sv_device.hpp"
#include "sv_launch.hpp"

namespace sv {

namespace {

constexpr int kQElemS = 0, kQVecS = 1;  // draft rows: element loads, or 16-byte vectors in phase with the logits
constexpr int kSpinLimit = 1 << 20;     // polls before a wait gives up (about a second)

__device__ __forceinline__ void word_put(uint64_t* p, uint64_t v) {
  __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ uint64_t word_get(uint64_t* p) {
  return __hip_atomic_load(p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
// A tagged word: the 48-bit tag above 16 bits of payload.
__device__ __forceinline__ uint64_t tagged(uint64_t tag, uint32_t payload16) {
  return (tag << 16) | (payload16 & 0xffffu);
}
// Two words carrying the halves of a 32-bit value.
__device__ __forceinline__ void put32(uint64_t* p, uint64_t tag, uint32_t v) {
  word_put(p, tagged(tag, v & 0xffffu));
  word_put(p + 1, tagged(tag, v >> 16));
}

// Called by every lane of a wave: lane l < n waits until word base[l * stride] carries
// `tag` and returns that word's 16-bit payload (lanes >= n return 0).  `first` is a value
// of the word read earlier (0 if none).  One read in flight at a time: a read still in
// flight when the wait ends would hold up the wave's next wait for memory (and two reads
// in flight saw the word no sooner: its write, not the polling, sets the pace).  The waves
// that poll are not the ones that publish, for the same reason: a wave's wait for a read
// also waits for its own earlier stores.
__device__ uint32_t wait_tagged(uint64_t* base, int stride, int n, uint64_t tag, int lane, uint32_t* err,
                                uint64_t first = 0) {
  const bool mine = lane < n;
  uint64_t* p = base + static_cast<ptrdiff_t>(mine ? lane : 0) * stride;
  uint64_t v = first;
  bool have = !mine || (v >> 16) == tag;
  for (int it = 0;; ++it) {
    if (__ballot(!have) == 0) break;
    if (it == kSpinLimit) {
      if (lane == 0) __hip_atomic_fetch_or(err, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      break;
    }
    if (!have) {
      v = word_get(p);
      have = (v >> 16) == tag;
    }
  }
  return mine ? static_cast<uint32_t>(v & 0xffffu) : 0u;
}
// The 32-bit value whose halves lanes 2i (low) and 2i + 1 (high) hold, in lane 2i.
__device__ __forceinline__ uint32_t join32(uint32_t half) {
  return half | (static_cast<uint32_t>(__shfl_down(static_cast<int>(half), 1)) << 16);
}

// One inverse-CDF step over weights held one per lane (w >= 0; lanes past the count hold
// 0), with its target t: the first lane of positive weight whose inclusive prefix exceeds t,
// with that lane's exclusive prefix in `before`.  When none does (t at or past the total,
// through rounding) or `clamp` is already set, the last lane of positive weight, and
// `clamp` is set (every level below then takes its last positive weight too).  -1 when
// every weight is 0.  The prefixes come from a tree-ordered scan, so they need not grow
// from lane to lane by exactly each lane's weight: a lane of zero weight is never taken.
__device__ __forceinline__ int pick_lane(float w, float incl, float t, bool& clamp, float& before) {
  const uint64_t pos = __ballot(w > 0.f);
  const uint64_t hit = clamp ? 0ull : __ballot(w > 0.f && incl > t);
  before = 0.f;
  if (hit) {
    const int l = __ffsll(static_cast<long long>(hit)) - 1;
    if (l > 0) before = lane_value(incl, l - 1);
    return l;
  }
  clamp = true;
  return pos ? 63 - __clzll(static_cast<long long>(pos)) : -1;
}

// Copies vector i (vector 0 when i is out of range) of every lane straight into LDS, at
// lds + 16 * lane (lds the same for the whole wave): no register holds the bytes in flight.
// The wave must wait for its vector-memory count before reading them.
__device__ __forceinline__ void ld16_to_lds(const SV_GLOBAL Vec16* p, int i, int n, Vec16* lds) {
  __builtin_amdgcn_global_load_lds(p + (static_cast<unsigned>(i) < static_cast<unsigned>(n) ? i : 0),
                                   (__attribute__((address_space(3))) void*)(lds), 16, 0, 0);
}
// s_waitcnt vmcnt(0), expcnt and lgkmcnt left at their maximum (gfx9 encoding)
__device__ __forceinline__ void wait_vmem_all() { __builtin_amdgcn_s_waitcnt(0x70 | 0xf00); }

// Inclusive prefix sums over lanes 0..n-1, n <= 8 (valid in those lanes; the slices of a
// row and the waves of a workgroup are at most 8); n is the same for the whole wave.
__device__ __forceinline__ float scan8(float x, int n = 8) {
  if (n > 1) x += dpp_f<kDppShr1>(0.f, x);
  if (n > 2) x += dpp_f<kDppShr2>(0.f, x);
  if (n > 4) x += dpp_f<kDppShr4>(0.f, x);
  return x;
}
// The (max, sum) pairs of lanes 0..n-1 (n <= 8, the same for the whole wave) merged, in
// every lane: the order depends on n alone, so every slice of a row gets the same bits.
__device__ __forceinline__ void merge_pairs8(float& m, float& s, float c, int n = 8) {
  if (n > 1) merge_step<kDppShr1>(m, s, c);
  if (n > 2) merge_step<kDppShr2>(m, s, c);
  if (n > 4) merge_step<kDppShr4>(m, s, c);
  m = lane_value(m, n - 1);
  s = lane_value(s, n - 1);
}

template <bool BF16>
__device__ __forceinline__ Vec16 ninf_vec() {
  Vec16 v;
  const uint32_t w = BF16 ? 0xff80ff80u : 0xff800000u;
  v.w[0] = v.w[1] = v.w[2] = v.w[3] = w;
  return v;
}

constexpr uint32_t kKept = 1u, kRejected = 2u;  // decision word payloads
// Draws from p leave out vectors whose weight sum (against a largest weight of 1) is below
// 2^-122: such a vector's largest element, one of at most 8, is then at least 2^-125.
constexpr float kTinyMass = 0x1p-122f;
constexpr uint32_t kMassSkip = 0x80000000u;     // in a residual mass (a sign bit): the row stands down
// a row's words: 4 per slice for its (max, sum) pair and 4 right after the S pairs for the
// row's uniforms (written by slice 0), 2 per slice for its residual mass, 1 for the row's
// decision
constexpr int kPairWord = 0, kMassWord = 4 * kSplitSlices + 4, kDecisionWord = 6 * kSplitSlices + 4;
static_assert(kDecisionWord + 1 == kSplitWordsPerRow, "row word layout");

}  // namespace

template <bool BF16, int NT, int NV, int QMODE>
__global__ __launch_bounds__(NT) void row_split_kernel(SplitParams P) {
  using E = Elem<BF16>;
  constexpr int VE = E::kPerVec;
  constexpr int EB = E::kBytes;
  constexpr int NW = NT / kWave;
  __shared__ float s_wm[NW], s_ws[NW], s_wt[NW];  // per wave: pass-1 pair, draw total
  __shared__ float s_m, s_Z;                      // the row's (max, sum)
  // the slice that draws: its index, the target t = u * S and the mass of the slices
  // before it; clamp: t lay past the total
  __shared__ float s_t, s_before;
  __shared__ int s_cand, s_skip, s_skipmine, s_win, s_clamp, s_fromp;
  // a rejected row's draft vectors, when read in vectors: wave w's vector i of lane l at
  // [(w * NV + i) * 64 + l] (kept out of registers, which hold the row's weights)
  __shared__ Vec16 s_q[QMODE == kQVecS ? NT * NV : 1];
  __shared__ uint64_t s_gen;

  const int tid = threadIdx.x;
  const int lane = tid & (kWave - 1);
  const int wid = tid / kWave;
  const int S = P.S;
  // Position-major: the S slices of a row are consecutive workgroups, rows ordered by
  // position j first, so every sequence's early rows (where first rejections fall) start
  // together and before the rows that wait for their decisions.
  const int rowpos = static_cast<int>(blockIdx.x) / S;
  const int slice = static_cast<int>(blockIdx.x) - rowpos * S;
  const int j = rowpos / P.B;
  const int b = rowpos - j * P.B;
  const int r = b * P.R + j;
  const int V = P.V;
  const int k = P.k;
  const float c = P.c;
  const int RS = P.R * S;

  // the call's generation for this sequence (thread 0; consumed after pass 1)
  uint64_t ticket = 0;
  if (tid == 0) ticket = __hip_atomic_fetch_add(&P.gen[b], 1ull, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);

  const char* rowp = static_cast<const char*>(P.logits) + static_cast<size_t>(r) * V * EB;
  const uintptr_t ra = reinterpret_cast<uintptr_t>(rowp);
  const int h = static_cast<int>(ra & 15) / EB;
  const SV_GLOBAL Vec16* vrow = gptr<Vec16>(reinterpret_cast<const void*>(ra - (ra & 15)));
  const int nvec = (V + h + VE - 1) / VE;
  const int vbeg = slice * P.chunk;
  const int vend = min(nvec, vbeg + P.chunk);
  const int qeb = P.q_bf16 ? 2 : 4;
  uint64_t* row_words = P.words + static_cast<size_t>(r) * kSplitWordsPerRow;
  uint64_t* seq_words = P.words + static_cast<size_t>(b) * P.R * kSplitWordsPerRow;  // row 0 of the sequence

  // The draft token (thread 0) is loaded before the row so that its gathers can follow
  // the row loads without holding them up.
  int g_x = -1;
  if (tid == 0 && j < k) g_x = gptr<int32_t>(P.tokens)[static_cast<size_t>(b) * k + j];
  // The position's pair of uniforms: drawn by one wave of slice 0 (the publishing wave, in
  // scalar code while its row loads are in flight) and sent to the other slices with its
  // (max, sum) pair.  Drawn by every wave of every slice, the Philox rounds kept each CU's
  // one scalar unit busy for microseconds.
  const bool publisher = tid == NT - kWave;  // lane 0 of the last wave
  float u_acc = 0.f, u_smp = 0.f;
  if (slice == 0 && wid == NW - 1) {
    draw_uniforms(P.seed, P.offset, static_cast<uint32_t>(b), static_cast<uint32_t>(j), u_acc, u_smp);
    // computed here (left alone, the compiler moves the rounds to their first use)
    asm volatile("" ::"s"(__float_as_uint(u_acc)), "s"(__float_as_uint(u_smp)));
  }

  // ---- pass 1: this slice's vectors, all loads in flight before any arithmetic
  const int v0 = vbeg + wid * (NV * kWave) + lane;
  Vec16 buf[NV];
#pragma unroll
  for (int i = 0; i < NV; ++i) buf[i] = ld16_stream(vrow, v0 + i * kWave, vend);
  bool g_valid = false;
  float g_l = 0.f, g_q = 0.f;
  const char* qrowp = static_cast<const char*>(P.probs) + (static_cast<size_t>(b) * k + (j < k ? j : 0)) * V * qeb;
  if (tid == 0 && g_x >= 0 && g_x < V) {
    g_valid = true;
    g_l = load_elem(rowp, g_x, BF16);
    g_q = load_elem(qrowp, g_x, P.q_bf16 != 0);
  }
#pragma unroll
  for (int i = 0; i < NV; ++i) {
    const int vi = v0 + i * kWave;
    buf[i] = vi < vend ? mask_edges<BF16>(buf[i], vi * VE - h, V) : ninf_vec<BF16>();
  }
  float tm = -INFINITY;
#pragma unroll
  for (int i = 0; i < NV; ++i)
#pragma unroll
    for (int e = 0; e < VE; ++e) tm = fmaxf(tm, E::at(buf[i], e));
  pin_packed(buf);  // unpack again below instead of holding the row twice
  const bool own_any = tm != -INFINITY;  // any element of this thread's share is above -inf
  const float ref = own_any ? tm : 0.f;
  float ts = 0.f;
  // per element 2^((l - ref) c), against this thread's own maximum: every later weight is
  // this times one factor, so the residual and the walks need no exponential of their own
  float ev[NV][VE];
#pragma unroll
  for (int i = 0; i < NV; ++i) {
    float vs = 0.f;
#pragma unroll
    for (int e = 0; e < VE; ++e) {
      ev[i][e] = fast_exp2((E::at(buf[i], e) - ref) * c);
      vs += ev[i][e];
    }
    ts += vs;
  }
  wave_merge_max_sum(tm, ts, c);
  if (lane == 0) {
    s_wm[wid] = tm;
    s_ws[wid] = ts;
  }
  if (tid == 0) s_gen = ticket >> 16;
  // From here on the workgroup runs short dependent chains (exchanges, decision, draw)
  // while other workgroups on the same CU are still in pass 1's arithmetic: its waves
  // take issue priority over theirs.
  __builtin_amdgcn_s_setprio(2);
  __syncthreads();

  // ---- exchange 1: the slices' (max, sum) pairs.  The last wave publishes, wave 0 polls.
  const uint64_t gen = s_gen;
  // never 0, so a zeroed word is never current; (gen + 1) < 2^37 for any realistic run
  const uint64_t tag = (((gen + 1) & ((1ull << 37) - 1)) << 11) | static_cast<uint64_t>(b & 2047);
  if (wid == NW - 1) {
    // the slice's pair: the waves' pairs (lane w: wave w) merged across lanes
    float m_s = lane < NW ? s_wm[lane < NW ? lane : 0] : -INFINITY;
    float z_s = lane < NW ? s_ws[lane < NW ? lane : 0] : 0.f;
    merge_pairs8(m_s, z_s, c, NW);
    if (publisher) {
      put32(row_words + kPairWord + 4 * slice, tag, __float_as_uint(m_s));
      put32(row_words + kPairWord + 4 * slice + 2, tag, __float_as_uint(z_s));
      if (slice == 0) {
        put32(row_words + kPairWord + 4 * S, tag, __float_as_uint(u_acc));
        put32(row_words + kPairWord + 4 * S + 2, tag, __float_as_uint(u_smp));
      }
    }
  }
  if (tid == 0) {
    // the call's last ticket for this sequence moves the counter to the next multiple of 2^16
    // (thread 0's wave polls next, but this atomic was issued after the loads it waits for)
    if (static_cast<int>(ticket & 0xffff) == RS - 1)
      (void)__hip_atomic_fetch_add(&P.gen[b], (1ull << 16) - static_cast<uint64_t>(RS), __ATOMIC_RELAXED,
                                   __HIP_MEMORY_SCOPE_AGENT);
  }
  // Wave 0 polls, merges the pairs (a lane-parallel merge: the same order in every slice,
  // so all of them hold bit-identical (m, Z)) and takes the acceptance decision (lane 0 =
  // thread 0, which holds the draft token's gathered values).  For the last row it also
  // picks the slice of the draw from p; a rejected row picks it only if its residual
  // turns out empty.
  double g_e = 0.0;
  float u_smp_w = 0.f, pm = -INFINITY, ps = 0.f, mr = -INFINITY;
  // a draw from p: slice masses against the row maximum, in lane s.  A slice whose mass is
  // below twice kTinyMass per vector it holds is left out, so that a slice taken holds a
  // vector that is not left out below.  Lane 0 posts the pick.
  auto pick_from_p = [&]() {
    float ms = lane < S ? ps * fast_exp2((pm - mr) * c) : 0.f;
    if (ms < 2.f * kTinyMass * static_cast<float>(NT * NV)) ms = 0.f;
    const float incl = scan8(ms, S);
    const float tt = u_smp_w * lane_value(incl, S - 1);
    bool cl = false;
    float bef = 0.f;
    const int win = pick_lane(ms, incl, tt, cl, bef);
    if (lane == 0) {
      s_fromp = 1;
      s_win = win;
      s_t = tt;
      s_before = bef;
      s_clamp = cl;
    }
  };
  if (wid == 0) {
    // lane 4s + 0..3: halves of slice s's max, then of its sum; lanes 4S + 0..3: halves of
    // the two uniforms
    const uint32_t v = join32(wait_tagged(row_words + kPairWord, 1, 4 * S + 4, tag, lane, P.errword));
    const uint32_t vz = static_cast<uint32_t>(__shfl_down(static_cast<int>(v), 2));
    const float u_acc_w = __uint_as_float(static_cast<uint32_t>(lane_value(static_cast<int>(v), 4 * S)));
    u_smp_w = __uint_as_float(static_cast<uint32_t>(lane_value(static_cast<int>(vz), 4 * S)));
    // slice s's pair to lane s (every lane takes part in the shuffles)
    const uint32_t gm = static_cast<uint32_t>(__shfl(static_cast<int>(v), (4 * lane) & (kWave - 1)));
    const uint32_t gz = static_cast<uint32_t>(__shfl(static_cast<int>(vz), (4 * lane) & (kWave - 1)));
    pm = lane < S ? __uint_as_float(gm) : -INFINITY;
    ps = lane < S ? __uint_as_float(gz) : 0.f;
    mr = pm;
    float zr = ps;
    merge_pairs8(mr, zr, c, S);
    // acceptance test: u * q(x) < p(x) = e / Z with e = exp((l_x - m) / T) in float64,
    // compared as u * q(x) * Z < e so that no division sits on the path to the decision
    bool acc = false;
    if (lane == 0 && j < k) {
      if (g_valid) g_e = exp((static_cast<double>(g_l) - static_cast<double>(mr)) * P.invT);
      acc = g_valid && (static_cast<double>(u_acc_w) * static_cast<double>(g_q) * static_cast<double>(zr) < g_e);
    }
    if (j == k) pick_from_p();
    if (lane == 0) {
      s_m = mr;
      s_Z = zr;
      s_cand = (j == k) || !acc;
      s_skip = 0;
    }
  }
  __syncthreads();
  const float m = s_m, Z = s_Z;
  const bool cand = s_cand != 0;
  const bool resid_row = cand && j < k;

  // Memory reads first, then the stores: a wave's wait for a read also waits for whatever
  // it issued before it.  The draft vectors go straight to LDS and are used as loaded:
  // where a vector lies past this slice's share, or an element outside the row, the logit
  // is -inf and the residual weight max(0, 0 - q) is 0 whatever q holds (a probability of
  // this row or the next).
  const int wid_u = __builtin_amdgcn_readfirstlane(wid);
  if (resid_row && QMODE == kQVecS) {
    const uintptr_t qa = reinterpret_cast<uintptr_t>(qrowp);
    const SV_GLOBAL Vec16* vq = gptr<Vec16>(reinterpret_cast<const void*>(qa - (qa & 15)));
#pragma unroll
    for (int i = 0; i < NV; ++i) ld16_to_lds(vq, v0 + i * kWave, vend, &s_q[(wid_u * NV + i) * kWave]);
  }
  // the decisions of the sequence's earlier rows (lane l: row l), read by every wave now so
  // that whichever wave draws the token finds them in its registers
  uint64_t dec_early = 0;
  int tok_early = -1;  // and the sequence's draft tokens, which the outputs repeat
  if (cand && lane < j) {
    dec_early = word_get(seq_words + kDecisionWord + static_cast<size_t>(lane) * kSplitWordsPerRow);
    tok_early = gptr<int32_t>(P.tokens)[static_cast<size_t>(b) * k + lane];
  }
  // The publisher of slice 0 reports the decision and, for a rejection, raises the
  // sequence's earliest-rejection word (generation in the high bits: a word from an earlier
  // call never outranks this one); thread 0 of each slice of a rejected row reads that word,
  // so that a row that is not the sequence's first rejection can stand down.
  uint64_t rej_seen = 0;
  if (tid == 0 && resid_row) rej_seen = __hip_atomic_load(&P.first_rej[b], __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  if (publisher && slice == 0 && j < k) {
    word_put(row_words + kDecisionWord, tagged(tag, cand ? kRejected : kKept));
    if (cand) (void)atomic_max_u64(&P.first_rej[b], (gen << 8) | static_cast<uint64_t>(64 - j));
  }
  // p(x) and min(1, p/q) for the caller (slice 0 of a draft row), once the reads are issued
  if (tid == 0 && slice == 0 && j < k) {
    const double px = g_e / static_cast<double>(Z);
    const size_t o = static_cast<size_t>(b) * k + j;
    if (P.out_tprob) P.out_tprob[o] = static_cast<float>(px);
    if (P.out_aprob) {
      double ap;
      if (g_q > 0.f) ap = px / static_cast<double>(g_q) < 1.0 ? px / static_cast<double>(g_q) : 1.0;
      else ap = px > 0.0 ? 1.0 : 0.0;
      P.out_aprob[o] = static_cast<float>(ap);
    }
  }
  if (!cand) return;  // a kept draft: nothing more for this row (uniform over the workgroup)

  float seg[NV];
  float slot_tot[NV];
  // 2^((l - m) c) = 2^((l - ref) c) * scale; a thread whose share is all -inf has no weight
  const float scale = own_any ? fast_exp2((ref - m) * c) : 0.f;
  const float scale_z = scale / Z;
  // residual weights of one vector: max(0, p - q) with p = 2^((l - m) c) / Z; qvec is its
  // draft vector when the draft row is read in vectors
  auto resid_weights = [&](const float* evi, const Vec16& qvec, int vi, float* w) {
    const int e0 = vi * VE - h;
#pragma unroll
    for (int e = 0; e < VE; ++e) {
      float q;
      if (QMODE == kQVecS) q = E::at(qvec, e);
      else q = (vi < vend && e0 + e >= 0 && e0 + e < V) ? load_elem(qrowp, e0 + e, P.q_bf16 != 0) : 0.f;
      w[e] = fmaxf(0.f, fmaf(evi[e], scale_z, -q));
    }
  };
  auto p_weights = [&](const float* evi, float* w) {
#pragma unroll
    for (int e = 0; e < VE; ++e) w[e] = evi[e] * scale;
  };
  // the wave's total of seg[] in one reduction, so that the mass goes out first; the slot
  // totals follow while it travels and may differ from their sum in the last bits, which
  // the walk's clamping covers
  auto wave_total = [&]() -> float {
    float ts = 0.f;
#pragma unroll
    for (int i = 0; i < NV; ++i) ts += seg[i];
    return wave_sum(ts);
  };

  if (resid_row) {
    // ---- residual at a rejected position.  A row that is not the sequence's first
    // rejection stands down once any of its slices has seen an earlier one: that slice
    // flags its mass word and ends, the others end on reading the flag.  The slices
    // compute their masses meanwhile rather than wait for the word they read.
    if (QMODE == kQVecS) wait_vmem_all();  // this wave's draft vectors are in LDS
#pragma unroll
    for (int i = 0; i < NV; ++i) {
      float w[VE];
      resid_weights(ev[i], QMODE == kQVecS ? s_q[(wid * NV + i) * kWave + lane] : Vec16{}, v0 + i * kWave, w);
      float sg = 0.f;
#pragma unroll
      for (int e = 0; e < VE; ++e) sg += w[e];
      seg[i] = sg;
    }
    const float wt = wave_total();
    if (lane == 0) s_wt[wid] = wt;
    if (tid == 0) s_skipmine = (rej_seen >> 8) == gen && static_cast<int>(rej_seen & 0xff) > 64 - j;
    __syncthreads();
    const bool skip_mine = s_skipmine != 0;
    if (wid == NW - 1) {
      const float mass = lane_value(scan8(lane < NW ? s_wt[lane < NW ? lane : 0] : 0.f, NW), NW - 1);
      if (publisher) put32(row_words + kMassWord + 2 * slice, tag, __float_as_uint(mass) | (skip_mine ? kMassSkip : 0u));
    }
    if (skip_mine) return;  // uniform: the other slices learn it from the flag
    // each wave's slot totals, for the walk, while the masses travel
#pragma unroll
    for (int i = 0; i < NV; ++i) slot_tot[i] = wave_sum(seg[i]);
    if (wid == 0) {
      // lane 2s + 0..1: halves of slice s's residual mass; slice s's mass to lane s
      const uint32_t v = join32(wait_tagged(row_words + kMassWord, 1, 2 * S, tag, lane, P.errword));
      const bool any_skip = __ballot(lane < 2 * S && (lane & 1) == 0 && (v & kMassSkip)) != 0;
      const uint32_t g = static_cast<uint32_t>(__shfl(static_cast<int>(v), (2 * lane) & (kWave - 1)));
      const float mass = lane < S ? __uint_as_float(g & ~kMassSkip) : 0.f;
      const float incl = scan8(mass, S);
      const float tot = lane_value(incl, S - 1);
      if (tot > 0.f) {
        bool cl = false;
        float bef = 0.f;
        const float tt = u_smp_w * tot;
        const int win = pick_lane(mass, incl, tt, cl, bef);
        if (lane == 0) {
          s_fromp = 0;
          s_win = win;
          s_t = tt;
          s_before = bef;
          s_clamp = cl;
        }
      } else {
        pick_from_p();  // the residual is empty through rounding: draw from p itself
      }
      if (lane == 0) s_skip = any_skip;
    }
    __syncthreads();
    if (s_skip) return;  // uniform: an earlier row rejected, this row's token is not needed
  }
  const bool from_p = s_fromp != 0;
  const int winner = s_win;
  const float t = s_t, before = s_before;
  bool clamp = s_clamp != 0;
  if (winner != slice) return;  // uniform
  if (from_p) {
    // this slice's vector sums of p against the row maximum; a vector whose sum is below
    // kTinyMass is left out, so that a vector taken holds an element whose own weight is a
    // normal number
#pragma unroll
    for (int i = 0; i < NV; ++i) {
      float v = 0.f;
#pragma unroll
      for (int e = 0; e < VE; ++e) v += ev[i][e];
      v *= scale;
      seg[i] = v >= kTinyMass ? v : 0.f;
    }
    float wt = 0.f;
#pragma unroll
    for (int i = 0; i < NV; ++i) {
      slot_tot[i] = wave_sum(seg[i]);
      wt += slot_tot[i];
    }
    if (lane == 0) s_wt[wid] = wt;
    __syncthreads();
  }

  // ---- walk: wave, then slot, then lane, then element (each level sums the values the
  // level above summed, up to the rescaling of a draw from p; a target past a level's
  // total takes the last positive weight, which only happens within rounding of a
  // boundary).  Single precision throughout: the target u * S is rounded once, which moves
  // the draw only when u lies within about 1e-7 of a boundary, far inside the near-tie
  // band of 1e-6 that parity with the float64 oracle leaves out.
  const float t1 = t - before;
  float wbefore = 0.f;
  int wstar;
  {
    const float wv = lane < NW ? s_wt[lane < NW ? lane : 0] : 0.f;
    wstar = pick_lane(wv, scan8(wv, NW), t1, clamp, wbefore);
  }
  if (wstar < 0) wstar = 0;  // no positive weight (not reachable for finite inputs)
  if (wid != wstar) return;
  const float t2 = t1 - wbefore;
  int istar = -1, ilast = -1;
  float icum = 0.f, ibefore = 0.f;
#pragma unroll
  for (int i = 0; i < NV; ++i) {
    const float nc = icum + slot_tot[i];
    if (slot_tot[i] > 0.f) ilast = i;
    if (!clamp && istar < 0 && nc > t2) {
      istar = i;
      ibefore = icum;
    }
    icum = nc;
  }
  if (istar < 0) {
    istar = ilast < 0 ? 0 : ilast;
    clamp = true;
  }
  // the chosen slot's values, selected with compile-time indices (a run-time index into a
  // register array would move it to scratch memory)
  float sg = 0.f;
  float es[VE];

#pragma unroll
  for (int e = 0; e < VE; ++e) es[e] = ev[0][e];
#pragma unroll
  for (int i = 1; i < NV; ++i)
    if (i == istar) {
#pragma unroll
      for (int e = 0; e < VE; ++e) es[e] = ev[i][e];
    }
#pragma unroll
  for (int i = 0; i < NV; ++i)
    if (i == istar) {
      sg = seg[i];
    }
  const float scan = wave_inclusive_scan(sg);
  const float t3 = t2 - ibefore;
  const uint64_t hit = __ballot(sg > 0.f && scan > t3);  // a tree-ordered scan: see pick_lane
  const uint64_t pos = __ballot(sg > 0.f);
  int lstar;
  if (!clamp && hit) {
    lstar = __ffsll(static_cast<long long>(hit)) - 1;
  } else {
    lstar = pos ? 63 - __clzll(static_cast<long long>(pos)) : 0;
    clamp = true;
  }
  const float excl = lane_value(scan, lstar > 0 ? lstar - 1 : 0);
  int y = -1;
  if (lane == lstar) {
    const int vi = v0 + istar * kWave;
    float w[VE];
    if (from_p) p_weights(es, w);
    else resid_weights(es, QMODE == kQVecS ? s_q[(wid * NV + istar) * kWave + lane] : Vec16{}, vi, w);
    const float t4 = t3 - (lstar > 0 ? excl : 0.f);
    int ye = -1, ylast = -1;
    float ec = 0.f;
#pragma unroll
    for (int e = 0; e < VE; ++e) {
      ec += w[e];
      if (w[e] > 0.f) {
        ylast = e;
        if (!clamp && ye < 0 && ec > t4) ye = e;
      }
    }
    if (ye < 0) ye = ylast < 0 ? 0 : ylast;  // (no positive weight: not reachable for finite inputs)
    y = vi * VE - h + ye;
  }
  y = lane_value(y, lstar);

  // ---- the sequence ends here if every earlier row kept its draft: this wave writes the
  // outputs
  const uint32_t d = wait_tagged(seq_words + kDecisionWord, kSplitWordsPerRow, j, tag, lane, P.errword, dec_early);
  if (__ballot(lane < j && d != kKept) != 0) return;
  if (lane < P.R) P.out_tokens[static_cast<size_t>(b) * P.R + lane] = lane < j ? tok_early : (lane == j ? y : -1);
  if (lane == 0) P.out_accept_len[b] = j;
}

// ------------------------------------------------------------------ launch
// Shapes (threads x 16-byte vectors per thread); a slice is at most one tile of its shape.
struct SplitShape {
  int nt, nv;
};
// Tried in this order; for one vocabulary size fewer, wider slices run faster (B=64 k=5
// V=32000 bf16: 2 slices of 512 x 4 14.4 us, 3 of 384 x 4 15.8, 4 of 256 x 4 15.9,
// 2 of 1024 x 2 15.9, 2 of 256 x 8 15.0).
static const SplitShape kSplitShapes[kSplitShapeCount] = {{512, 4}, {256, 4}, {256, 8}, {128, 8}};

template <bool BF16, int NT, int NV, int QMODE>
static const void* split_fn() {
  return reinterpret_cast<const void*>(&row_split_kernel<BF16, NT, NV, QMODE>);
}

template <bool BF16, int QMODE>
static const void* split_fn_shape(int shape) {
  switch (shape) {
    case 0: return split_fn<BF16, 512, 4, QMODE>();
    case 1: return split_fn<BF16, 256, 4, QMODE>();
    case 2: return split_fn<BF16, 256, 8, QMODE>();
    default: return split_fn<BF16, 128, 8, QMODE>();
  }
}

static const void* split_kernel(bool bf16, int qmode, int shape) {
  if (bf16) return qmode == kQVecS ? split_fn_shape<true, kQVecS>(shape) : split_fn_shape<true, kQElemS>(shape);
  return qmode == kQVecS ? split_fn_shape<false, kQVecS>(shape) : split_fn_shape<false, kQElemS>(shape);
}

// Workgroups of one instance the current device holds at once (occupancy x CUs), cached
// per device and instance; 0 if the runtime cannot say.
static int split_capacity(bool bf16, int qmode, int shape) {
  static std::mutex mu;
  static int cache[64][2][2][kSplitShapeCount] = {};
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return 0;
  std::lock_guard<std::mutex> g(mu);
  int& cap = cache[dev][bf16 ? 1 : 0][qmode][shape];
  if (cap == 0) {
    int per_cu = 0, cus = 0;
    if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, split_kernel(bf16, qmode, shape),
                                                     kSplitShapes[shape].nt, 0) != hipSuccess ||
        hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || per_cu < 1 ||
        cus < 1)
      return 0;
    cap = per_cu * cus;
  }
  return cap;
}

bool choose_split(bool bf16, int qmode, int V, int head_max, int64_t rows, SplitConfig* out) {
  if ((qmode != kQElemS && qmode != kQVecS) || rows <= 0 || rows > kSplitRows) return false;
  const int ve = bf16 ? 8 : 4;
  const int64_t nvec = (static_cast<int64_t>(V) + head_max + ve - 1) / ve;
  for (int shape = 0; shape < kSplitShapeCount; ++shape) {
    const int64_t tile = static_cast<int64_t>(kSplitShapes[shape].nt) * kSplitShapes[shape].nv;
    const int64_t S = (nvec + tile - 1) / tile;
    if (S < 2 || S > kSplitSlices) continue;
    const int cap = split_capacity(bf16, qmode, shape);
    if (cap <= 0 || rows * S > cap) continue;  // the whole grid must fit the chip at once
    out->shape = shape;
    out->S = static_cast<int>(S);
    out->chunk = static_cast<int>((nvec + S - 1) / S);
    out->threads = kSplitShapes[shape].nt;
    return true;
  }
  return false;
}

hipError_t launch_split(const SplitParams& P, bool bf16, int qmode, const SplitConfig& sc, hipStream_t st) {
  const int grid = P.B * P.R * sc.S;
  SplitParams arg = P;
  void* args[] = {&arg};
  return hipLaunchKernel(split_kernel(bf16, qmode, sc.shape), dim3(grid), dim3(sc.threads), args, 0, st);
}

}  // namespace sv
