// Row-parallel verification kernels: linear speculative sampling and static-tree
// verification ("Accelerating Sonar through speculation", sections "Speculative
// decoding" and "EAGLE"; "Speculative decoding explained", section "Draft and
// verification loop").
//
// One workgroup owns one vocabulary row of the target logits (row j of sequence b; for a
// tree, the row of node u).  It
//   1. streams the row from HBM once with 16-byte loads (each wave reads contiguous 1 KB
//      spans) and keeps it in registers when it fits one tile (NT threads x NV vectors),
//      computing the row max and sum of exp in one online pass;
//   2. runs the acceptance test(s) that read this row: position j's draft token
//      (linear) or the tokens of u's children (tree);
//   3. if the extra token may come from this row (a rejected position or the last row for
//      linear, a node with no accepted child for the tree), draws the candidate token by
//      inverse CDF: per-(tile, wave) totals, then inside the winning wave the slot
//      totals, the slot's lane scan and the element walk (DPP scans throughout);
//   4. publishes its result with one device-scope atomic and takes a ticket on its
//      sequence's counter; the last workgroup to arrive writes the sequence's outputs.
//      Linear: the first rejected position is the smallest candidate row, so candidates
//      post an atomic max of the inverted key (row, token).  Tree: accepted children go
//      into a node mask, candidates into per-node slots.
// A single launch covers the whole step.
//
// The lossless tree variant (QMODE kQLossless) tests a node's children in sibling order,
// each against the target mass left after the earlier siblings were rejected, keeps only
// the first that passes, and draws the extra token from p without the children's tokens.
// Each node's outcome depends on its own row only, so the rows still run independently;
// the one kept child per node makes the alive set a single path.

#include "sv_device.hpp"
#include "sv_launch.hpp"

namespace sv {

// QMODE selects how the residual reads the draft-probability row q:
//   kQVec  q has the logits' dtype and 16-byte phase: the same 16-byte vector loads;
//   kQHalf float32 logits with bfloat16 q whose 8-byte chunks line up with the logits
//          vectors (the fused LM-head case): one 8-byte load per vector;
//   kQElem anything else: element loads.
// kQLossless is the lossless tree: no q rows at all (each candidate is a fixed top-K
// token, so its draft law is a point mass).
constexpr int kQElem = 0, kQVec = 1, kQHalf = 2, kQLossless = 3;
constexpr int kHelpSpin = 1 << 20;  // polls before a wait on the help words gives up


// s_waitcnt vmcnt(0), expcnt and lgkmcnt left at their maximum (gfx9 encoding): this
// wave's loads, stores and atomics have all been acknowledged
__device__ __forceinline__ void wait_vmem_all() { __builtin_amdgcn_s_waitcnt(0x70 | 0xf00); }

// Occupancy target: at least two waves per SIMD (up to 256 VGPRs).  Holding the
// multi-tile 512 x 16 configurations to 128 VGPRs (two workgroups per CU) spilled the
// linear instantiations to scratch; with a whole tile's loads in flight per thread one
// workgroup per CU already keeps enough bytes moving there.
template <int NT, int NV>
struct RowOccupancy {
  static constexpr int kWavesPerEU = 2;
};
// 512 x 8 rows are single-tile: two workgroups per CU (128 VGPRs) fit without spilling.
// The lossless tree is held to 128 VGPRs too (a few bytes of spill): four 256-thread
// workgroups per CU keep a 976-row step (16 trees of 61 nodes) resident in one round,
// which measured 78 us against 87 us at 137 VGPRs.
template <>
struct RowOccupancy<512, 8> {
  static constexpr int kWavesPerEU = 4;
};

// STOP: linear rows walked in 256 x 16 tiles stop streaming once an earlier position of
// their sequence has rejected (an instance of its own, launched for grids of several rounds).
template <bool BF16, int NT, int NV, bool TREE, int QMODE, bool STOP = false>
__global__ __launch_bounds__(NT) __attribute__((amdgpu_waves_per_eu(QMODE == kQLossless ? 4 : RowOccupancy<NT, NV>::kWavesPerEU)))
void row_verify_kernel(RowParams P, TreeDesc td) {
  using E = Elem<BF16>;
  constexpr int VE = E::kPerVec;
  constexpr int EB = E::kBytes;
  constexpr int NW = NT / kWave;
  constexpr int TILE = NT * NV;  // vectors per tile

  // dynamic LDS, 3 x [ntiles * NW]: per-(tile, wave) softmax partials (max, scaled sum)
  // from pass 1, and per-(tile, wave) candidate-weight totals from pass 2
  extern __shared__ float s_dyn[];
  const int nunits = P.ntiles * NW;
  float* s_pm = s_dyn;
  float* s_ps = s_dyn + nunits;
  float* s_tot = s_dyn + 2 * nunits;
  __shared__ int s_flag, s_y, s_last, s_skip;
  __shared__ float s_slot[NV];    // a cooperatively recomputed unit's slot totals
  __shared__ int s_claim[2], s_hr, s_help;  // residual tiles claimed; the row this one helps
  __shared__ int s_quit[NT / kWave];        // per wave: stopped streaming (below)
  __shared__ int s_pre;                     // the last row: an earlier row rejected (below)
  __shared__ float s_hm, s_hz;                      // the helped row's (max, sum)
  __shared__ float s_usmp;
  __shared__ int8_t s_par[64], s_fc[64], s_nc[64], s_dep[64];
  constexpr bool LOSSLESS = TREE && QMODE == kQLossless;
  // linear rows walked in tiles (16 vectors per thread: the single-tile shapes hold fewer)
  // can be helped by workgroups that are done (below)
  constexpr bool HELP = !TREE && NV == 16;
  // linear rows walked in tiles stop streaming once an earlier position has rejected
  // (below)
  constexpr bool QUIT = STOP && !TREE && NV == 16 && NT < 512;
  // single-tile linear rows with q vectors in phase: the rejection check is deferred (below)
  constexpr bool DEFER = !TREE && QMODE == kQVec && NV <= 8;
  // single-tile rows: a draw from p is walked from the registers (below)
  constexpr bool REG_DRAW = NV <= 8;
  // linear rows of several waves draw their position's pair in uniform control flow (below)
  constexpr bool UNIFORM_RNG = !TREE && NT >= 256;
  __shared__ int s_xtok[LOSSLESS ? 64 : 1];     // lossless: the children's valid tokens
  __shared__ float s_xsub[LOSSLESS ? 64 : 1];   // and their weights 2^((l - m) c)
  __shared__ int s_nx;

  const int tid = threadIdx.x;
  const int lane = tid & (kWave - 1);
  const int wid = tid / kWave;
  // Position-major dispatch: workgroup x takes row j = x / B of sequence b = x % B, so
  // every sequence's early rows (where its first rejection, and so its costly residual
  // draw, usually falls) start before the later rows, and a later row more often sees an
  // earlier rejection published before it decides whether to draw.
  const int j = static_cast<int>(blockIdx.x) / P.B;
  const int b = static_cast<int>(blockIdx.x) - j * P.B;
  const int r = b * P.R + j;
  const int V = P.V;
  const float c = P.c;

  const char* rowp = static_cast<const char*>(P.logits) + static_cast<size_t>(r) * V * EB;
  const uintptr_t ra = reinterpret_cast<uintptr_t>(rowp);
  const int h = static_cast<int>(ra & 15) / EB;  // elements before the row inside its first vector
  const SV_GLOBAL Vec16* vrow = gptr<Vec16>(reinterpret_cast<const void*>(ra - (ra & 15)));
  const int nvec = (V + h + VE - 1) / VE;
  const int qeb = P.q_bf16 ? 2 : 4;

  if (TREE) {  // per-lane indexing of the tree goes through LDS, not the kernel arguments
    if (tid < 64) {
      s_par[tid] = td.parent[tid];
      s_fc[tid] = td.first_child[tid];
      s_nc[tid] = td.nchild[tid];
      s_dep[tid] = td.depth[tid];
    }
    __syncthreads();
  }

  // ---- acceptance-test gathers.  The draft token is loaded before the row stream and the
  // values it indexes right after it: vector loads complete in issue order, so waiting for
  // the token then costs nothing extra, and the row stream is not held behind the chain.
  int g_node = -1;
  int g_x = -1;
  size_t g_qrow = 0;
  if (TREE) {
    if (tid < s_nc[j]) {
      g_node = s_fc[j] + tid;
      g_x = gptr<int32_t>(P.tokens)[static_cast<size_t>(b) * P.R + g_node];
    }
    g_qrow = static_cast<size_t>(b) * P.R + j;
  } else {
    if (tid == 0 && j < P.k) {
      g_node = j;
      g_x = gptr<int32_t>(P.tokens)[static_cast<size_t>(b) * P.k + j];
    }
    g_qrow = static_cast<size_t>(b) * P.k + j;
  }

  // ---- pass 1: online max / sum of 2^((l - m) c) over the row
  bool g_valid = false;
  float g_l = 0.f, g_q = 0.f, g_uacc = 0.f, g_usmp = 0.f;
  // Linear multi-tile rows of 512 x 16 (few rows in the batch) load tile t+1 while tile t
  // is reduced, so a row's tiles stream back to back.  Single-tile configurations have
  // nothing to prefetch; the tree kernels gain more from the occupancy the second buffer
  // would cost them (66 us with it off, 72 us on, for 61-node trees over V = 128256); and
  // 256 x 16 rows (many rows, two workgroups per CU either way) measured faster without it
  // (B=256 k=8 V=128256: 143 us against 148 us).
  constexpr bool PIPE = (NV == 16) && !TREE && NT >= 512;
  Vec16 buf[NV];
  Vec16 nxt[PIPE ? NV : 1];
  auto load_tile = [&](Vec16* dst, int tile) {
    const int v0 = tile * TILE + wid * (NV * kWave) + lane;
#pragma unroll
    for (int i = 0; i < NV; ++i) dst[i] = ld16_stream(vrow, v0 + i * kWave, nvec);  // edges: mask_edges
  };
  // A row after its sequence's earliest rejection supplies nothing to the outputs (the
  // sequential rule stops there), except p_j(x_j) when that is asked for (rows j < k).
  // Such a row reads the rejection word as each tile is issued and stops streaming once
  // it shows a rejection before j; the word only grows while the sequence is running.
  // Each wave decides for itself (the word may change between two waves' reads) and the
  // row stops when any of them did.  (Rows that prefetch the next tile are few per batch
  // and keep streaming.)
  const bool may_quit = QUIT && j > 0 && (j == P.k || (P.out_tprob == nullptr && P.out_aprob == nullptr));
  bool quit = false;
  // In a grid that runs in one round (bonus_wait, set by the launcher) the last row of a
  // sequence waits for the earlier rows' decisions before it streams: it is needed only
  // when all of them kept their drafts, and otherwise helps the earliest rejected row at
  // once, while the earlier rows have the bandwidth to themselves meanwhile.
  bool pre_quit = false;
  if (HELP && !PIPE && P.bonus_wait && j == P.k) {
    if (tid == 0) {
      uint64_t* dm = P.help_words + static_cast<size_t>(b * P.R) * P.help_stride + (P.help_stride - 1);
      const uint64_t low = (1ull << j) - 1ull;
      uint64_t v = 0;
      for (int spin = 0; spin < kHelpSpin && (v & low) != low; ++spin)
        v = __hip_atomic_load(dm, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      if ((v & low) != low) __hip_atomic_fetch_or(P.errword, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      // a row marks its decision after its rejection has been published
      const uint64_t seen = __hip_atomic_load(&P.seqword[2 * b + 1], __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      s_pre = seen > static_cast<uint64_t>(64 - j) ? 1 : 0;
    }
    __syncthreads();
    pre_quit = s_pre != 0;
  }
  // Lossless trees (leaf_wait, with tree_skip): every node keeps at most one child, so one
  // path is kept and a leaf's row serves only the extra token, drawn at the path's end.  A
  // leaf waits (one lane, bounded) for its parent's decisions and streams only when the
  // parent kept it and no decided node above dropped its path; the inner nodes, dispatched
  // before the leaves, have the bandwidth meanwhile.  (With independent tests per child,
  // many leaves stay kept and then stream late: that tree measured slower this way.)
  if (TREE && P.leaf_wait && j > 0 && s_nc[j] == 0) {
    if (wid == 0) {
      const int N = P.R;
      uint64_t* rw = P.rowword + static_cast<size_t>(b) * N;
      const int pa = s_par[j];
      int off = 0;
      if (lane == 0) {
        uint64_t w = 0;
        for (int spin = 0; spin < kHelpSpin && (w >> 63) == 0; ++spin)
          w = __hip_atomic_load(rw + pa, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        if ((w >> 63) == 0) __hip_atomic_fetch_or(P.errword, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        else off = (((w >> 32) >> (j - s_fc[pa])) & 1ull) == 0 ? 1 : 0;
      }
      off = __shfl(off, 0);
      if (!off) {  // the path above the parent: every node's word, one per lane
        uint64_t w = 0;
        if (lane < N) w = __hip_atomic_load(rw + lane, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        const bool decided = lane < N && (w >> 63) != 0;
        uint64_t kept = 0;
        if (decided) kept = ((w >> 32) & ((1ull << s_nc[lane]) - 1ull)) << s_fc[lane];
        const uint64_t dmask = __ballot(decided);
        uint32_t klo = static_cast<uint32_t>(kept), khi = static_cast<uint32_t>(kept >> 32);
        for (int o = 32; o >= 1; o >>= 1) {
          klo |= static_cast<uint32_t>(__shfl_xor(static_cast<int>(klo), o));
          khi |= static_cast<uint32_t>(__shfl_xor(static_cast<int>(khi), o));
        }
        const uint64_t amask = (static_cast<uint64_t>(khi) << 32) | klo;
        for (int x = pa; x != 0; x = s_par[x]) {
          const int px = s_par[x];
          if (((dmask >> px) & 1ull) != 0 && ((amask >> x) & 1ull) == 0) off = 1;
        }
      }
      if (lane == 0) s_pre = off;
    }
    __syncthreads();
    pre_quit = s_pre != 0;
  }
  const int stream_tiles = pre_quit ? 0 : P.ntiles;
  if (PIPE) load_tile(buf, 0);
  for (int tile = 0; tile < stream_tiles; ++tile) {
    const int v0 = tile * TILE + wid * (NV * kWave) + lane;
    // every load of the tile is in flight before the first edge mask
    if (!PIPE) load_tile(buf, tile);
    else if (tile + 1 < P.ntiles) load_tile(nxt, tile + 1);
    uint64_t chk = 0;
    if (QUIT) {  // every row reads it (a branch around the load made the compiler wait for
                 // it before the next tile's loads)
      asm volatile("" ::: "memory");  // issued behind the tile's loads
      chk = __hip_atomic_load(&P.seqword[2 * b + 1], __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    }
    // Linear rows of several waves: the pair of position j is the same for every thread,
    // so every thread draws it in uniform control flow (scalar instructions) while the
    // tile's loads are in flight, instead of one lane of wave 0 spending some 300 vector
    // issue slots on it inside pass 1 while the merge barrier waits for that wave
    // (B=64 k=5 V=32000: 18.3 -> 17.7 us).  A one-wave workgroup has no barrier to shorten
    // and measured slower this way (B=1000 k=4 V=1024: 13.3 -> 13.9 us), so it keeps the
    // one-lane draw.
    if (UNIFORM_RNG && tile == 0)
      draw_uniforms(P.seed, P.offset, static_cast<uint32_t>(b), static_cast<uint32_t>(j), g_uacc, g_usmp);
    // The gathers of a single-tile row are issued right behind its loads, before the edge
    // masks whose waits would hold them (and the one-lane uniform draw) until the whole
    // tile has arrived (B=1000 k=4 V=1024: 12.7 -> 12.2 us); multi-tile rows measured
    // nothing either way and keep them behind the masks.
    if constexpr (NV <= 8) {
      if (tile == 0 && g_node >= 0) {
        g_valid = (g_x >= 0 && g_x < V);
        if (g_valid) {
          g_l = load_elem(rowp, g_x, BF16);
          if (!LOSSLESS) g_q = load_elem(static_cast<const char*>(P.probs) + g_qrow * V * qeb, g_x, P.q_bf16);
        }
        if (!UNIFORM_RNG)
          draw_uniforms(P.seed, P.offset, static_cast<uint32_t>(b), static_cast<uint32_t>(g_node), g_uacc, g_usmp);
      }
    }
#pragma unroll
    for (int i = 0; i < NV; ++i) buf[i] = mask_edges<BF16>(buf[i], (v0 + i * kWave) * VE - h, V);
    if constexpr (NV > 8) {
      if (tile == 0 && g_node >= 0) {
        g_valid = (g_x >= 0 && g_x < V);
        if (g_valid) {
          g_l = load_elem(rowp, g_x, BF16);
          if (!LOSSLESS) g_q = load_elem(static_cast<const char*>(P.probs) + g_qrow * V * qeb, g_x, P.q_bf16);
        }
        if (!UNIFORM_RNG)
          draw_uniforms(P.seed, P.offset, static_cast<uint32_t>(b), static_cast<uint32_t>(g_node), g_uacc, g_usmp);
      }
    }
    if (QUIT) {
      asm volatile("" : "+v"(chk)::"memory");  // read here, once the tile has arrived
      if (may_quit && chk > static_cast<uint64_t>(64 - j)) {
        quit = true;
        break;
      }
    }
    float tm = -INFINITY;
#pragma unroll
    for (int i = 0; i < NV; ++i)
#pragma unroll
      for (int e = 0; e < VE; ++e) tm = fmaxf(tm, E::at(buf[i], e));
    pin_packed(buf);  // re-unpack below instead of holding 2x the row in float registers
    const float ref = tm == -INFINITY ? 0.f : tm;  // a share of only -inf contributes 0
    float ts = 0.f;
#pragma unroll
    for (int i = 0; i < NV; ++i) {
      float vs = 0.f;
#pragma unroll
      for (int e = 0; e < VE; ++e) vs += fast_exp2((E::at(buf[i], e) - ref) * c);
      ts += vs;
    }
    wave_merge_max_sum(tm, ts, c);  // this wave's share of this tile
    if (lane == 0) {
      s_pm[tile * NW + wid] = tm;
      s_ps[tile * NW + wid] = ts;
    }
    if (PIPE && tile + 1 < P.ntiles) {
#pragma unroll
      for (int i = 0; i < NV; ++i) buf[i] = nxt[i];
    }
  }
  pin_packed(buf);  // pass 2 starts again from the packed row
  if (may_quit && lane == 0) s_quit[wid] = quit ? 1 : 0;
  __syncthreads();
  bool row_quit = pre_quit;
  if (may_quit) {
#pragma unroll
    for (int w = 0; w < NT / kWave; ++w) row_quit = row_quit || s_quit[w] != 0;
  }
  // every thread merges the partials in the same order: the row's (m, Z) (meaningless for
  // a row that stopped, which uses neither)
  float m = -INFINITY, Z = 0.f;
  for (int q = 0; q < nunits; ++q) merge_max_sum(m, Z, s_pm[q], s_ps[q], c);

  // ---- acceptance tests: keep x iff u_acc * q(x) < p(x), with p(x) in double
  bool acc = false;
  double g_px = 0.0;
  if (g_node >= 0) {
    double px = 0.0;
    if (g_valid) px = exp((static_cast<double>(g_l) - static_cast<double>(m)) / P.T) / static_cast<double>(Z);
    g_px = px;
    acc = g_valid && (static_cast<double>(g_uacc) * static_cast<double>(g_q) < px);
    if (!TREE) {
      const size_t o = static_cast<size_t>(b) * P.k + j;
      if (P.out_tprob) P.out_tprob[o] = static_cast<float>(px);
      if (P.out_aprob) {
        double ap;
        if (g_q > 0.f) ap = px / static_cast<double>(g_q) < 1.0 ? px / static_cast<double>(g_q) : 1.0;
        else ap = px > 0.0 ? 1.0 : 0.0;
        P.out_aprob[o] = static_cast<float>(ap);
      }
    }
  }
  uint64_t child_acc = 0;  // tree: this node's accepted children, as node bits (wave 0)
  uint64_t rej_dep = 0;    // linear: value returned by the rejection publish (waited on later)
  uint64_t dec_dep = 0;    // tree: value returned by the early publish of the decisions
  if (LOSSLESS) {
    if (wid == 0) {
      // Sibling i (lane i) is tested against W_i = 1 - (mass of the distinct valid tokens
      // of siblings 0..i-1, summed in sibling order): keep with probability p(x) / W_i.
      // A repeated token has lost its mass with the earlier sibling and is never kept.
      const int nch = s_nc[j];
      bool dup = false;
      for (int l = 0; l < nch; ++l) {
        const int xl = __shfl(g_x, l);  // every lane takes part: the source lane must be active
        dup = dup || (l < lane && xl == g_x);
      }
      const double contrib = (g_valid && !dup) ? g_px : 0.0;
      const int64_t cbits = __double_as_longlong(contrib);
      const int clo = static_cast<int>(cbits), chi = static_cast<int>(cbits >> 32);
      double before = 0.0;
      for (int l = 0; l < nch; ++l) {
        const int64_t bl = (static_cast<int64_t>(__shfl(chi, l)) << 32) | static_cast<uint32_t>(__shfl(clo, l));
        if (l < lane) before += __longlong_as_double(bl);
      }
      const double W = 1.0 - before;
      acc = g_node >= 0 && g_valid && !dup && W > 0.0 && static_cast<double>(g_uacc) * W < g_px;
      const uint64_t am = __ballot(acc);
      child_acc = am ? 1ull << (s_fc[j] + __ffsll(static_cast<long long>(am)) - 1) : 0ull;
      // the children's valid tokens leave this node's draw
      const bool vx = g_node >= 0 && g_valid;
      const uint64_t vm = __ballot(vx);
      if (vx) {
        const int at = __popcll(vm & ((1ull << lane) - 1ull));
        s_xtok[at] = g_x;
        // its weight in the draw from p, taken out of its unit's pass-1 total below (a
        // repeated token once)
        s_xsub[at] = dup ? 0.f : fast_exp2((g_l - m) * c);
      }
      if (lane == 0) {
        s_nx = __popcll(vm);
        s_flag = (child_acc == 0ull);
      }
    }
  } else if (TREE) {
    if (wid == 0) {
      child_acc = __ballot(acc) << s_fc[j];
      if (lane == 0) s_flag = (child_acc == 0ull);
    }
  } else if (tid == 0) {
    const bool rejected = !acc && j < P.k && !row_quit;
    bool cand = !row_quit && ((j == P.k) || rejected);
    // A rejected row publishes its rejection at once (the word holds 64 - row of the
    // earliest rejection seen) and consults it before its costly candidate pass: only the
    // earliest rejected row can supply the emitted token, and the earliest one never sees
    // an earlier rejection, so skipping changes no result.  At B=64, k=5, V=32000 this
    // cut the draws per step from ~149 to ~82 and the step from 20.8 to 18.7 us: a later
    // rejected row's draw no longer ends the step when an earlier row has rejected.
    // A single-tile row reads the answer only at the barrier before its unit walk, so the
    // atomic's round trip overlaps its draft-row loads and residual weights; a multi-tile
    // row, whose draw re-reads its tiles, reads it before starting.
    if (HELP && P.help_on && rejected)  // the row's (m, Z), for the rows that may help it
      __hip_atomic_store(P.help_words + static_cast<size_t>(r) * P.help_stride,
                         (static_cast<uint64_t>(__float_as_uint(m)) << 32) | __float_as_uint(Z), __ATOMIC_RELAXED,
                         __HIP_MEMORY_SCOPE_AGENT);
    {
      if (rejected) {
        if (DEFER) {
          // a per-lane (opaque) address keeps the compiler from turning this into a
          // one-lane atomic plus a broadcast, which would wait for the result at once
          int zero;
          asm volatile("v_mov_b32 %0, 0" : "=v"(zero));
          rej_dep = atomic_max_u64(&P.seqword[2 * b + 1 + zero], static_cast<uint64_t>(64 - j));
        } else {
          const uint64_t seen = atomic_max_u64(&P.seqword[2 * b + 1], static_cast<uint64_t>(64 - j));
          rej_dep = seen;  // waited on before the ticket, so the reset cannot race it
          if (seen > static_cast<uint64_t>(64 - j)) cand = false;
        }
      } else if (cand) {  // the last row: any rejection makes it irrelevant
        if (DEFER) {
          // a single-tile row walks its draw from registers for less than the load's round
          // trip: it draws anyway and reads the answer only when it would post the draw
          int zero;
          asm volatile("v_mov_b32 %0, 0" : "=v"(zero));
          rej_dep = __hip_atomic_load(&P.seqword[2 * b + 1 + zero], __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        } else {
          const uint64_t seen =
              __hip_atomic_load(&P.seqword[2 * b + 1], __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
          if (seen > static_cast<uint64_t>(64 - j)) cand = false;
        }
      }
    }
    s_help = -1;
    if (HELP && P.help_on) {
      // Rows walked in tiles mark their decision in the sequence's mask, after publishing
      // any rejection; a later row waits for the earlier rows' marks (they decide without
      // waiting on anything, and start before it), then stands down if one of them
      // rejected and helps the earliest one with its residual tiles.
      uint64_t* dm = P.help_words + static_cast<size_t>(b * P.R) * P.help_stride + (P.help_stride - 1);
      (void)__hip_atomic_fetch_or(dm, 1ull << j, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      if (j > 0) {
        const uint64_t low = (1ull << j) - 1ull;
        uint64_t v = 0;
        for (int spin = 0; spin < kHelpSpin && (v & low) != low; ++spin)
          v = __hip_atomic_load(dm, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        const uint64_t seen = __hip_atomic_load(&P.seqword[2 * b + 1], __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        const int jf = seen > 0 ? 64 - static_cast<int>(seen) : P.R;
        if (jf < j) {
          cand = false;
          s_help = jf;
        }
      }
    }
    s_flag = cand;
  }
  if (TREE && pre_quit && tid == 0) s_flag = 0;  // a leaf off every kept path: no draw
  if (TREE && P.tree_skip && !pre_quit && wid == 0) {
    // A node publishes its children's decisions at once (bit 63 of its row word, the kept
    // children above bit 32, relative to its first child; its drawn token joins the low
    // half later).  A node that would draw first reads every node's word: the token is
    // emitted only from the deepest node on an accepted path (the leftmost of the
    // deepest), so the draw is skipped when a decided parent on its own path dropped it,
    // or when some node whose whole path is decided and kept lies deeper, or as deep and
    // further left.  Only decided parents count, so skipping changes no result.
    if (lane == 0 && s_nc[j] > 0)
      dec_dep = atomic_or_u64(&P.rowword[r], (1ull << 63) | ((child_acc >> s_fc[j]) << 32));
    if (child_acc == 0ull && j > 0) {
      const int N = P.R;
      uint64_t w = 0;
      if (lane < N)
        w = __hip_atomic_load(P.rowword + static_cast<size_t>(b) * N + lane, __ATOMIC_RELAXED,
                              __HIP_MEMORY_SCOPE_AGENT);
      const bool decided = lane < N && (w >> 63) != 0;
      uint64_t kept = 0;  // this lane's node's kept children, as node bits
      if (decided) kept = ((w >> 32) & ((1ull << s_nc[lane]) - 1ull)) << s_fc[lane];
      const uint64_t dmask = __ballot(decided);
      uint32_t klo = static_cast<uint32_t>(kept), khi = static_cast<uint32_t>(kept >> 32);
      for (int o = 32; o >= 1; o >>= 1) {
        klo |= static_cast<uint32_t>(__shfl_xor(static_cast<int>(klo), o));
        khi |= static_cast<uint32_t>(__shfl_xor(static_cast<int>(khi), o));
      }
      const uint64_t amask = (static_cast<uint64_t>(khi) << 32) | klo;
      // lane l's node: `sure` when every parent on its path decided and kept it, `off`
      // when one of them decided and dropped it
      bool sure = lane < N, off = false;
      for (int x = lane; lane < N && x != 0; x = s_par[x]) {
        const int px = s_par[x];
        if (((dmask >> px) & 1ull) == 0) sure = false;
        else if (((amask >> x) & 1ull) == 0) {
          off = true;
          sure = false;
        }
      }
      const int dj = s_dep[j];
      const bool ahead = sure && (s_dep[lane] > dj || (s_dep[lane] == dj && lane < j));
      const bool self_off = __shfl(static_cast<int>(off), j) != 0;
      if ((self_off || __ballot(ahead) != 0ull) && lane == 0) s_flag = 0;
    }
  }
  if (tid == 0) {
    float us = g_usmp;  // linear: the pair of position j (drawn above for rows j < k)
    if (TREE || (!UNIFORM_RNG && g_node < 0)) {
      float ua;
      draw_uniforms(P.seed, P.offset, static_cast<uint32_t>(b), static_cast<uint32_t>(j), ua, us);
    }
    s_usmp = us;
    s_y = -1;
    s_skip = 0;
  }
  __syncthreads();

  // ---- pass 2: candidate draw from this row.  The weights and tile sums below read the
  // row through cur_* (this row's; a helper points them at the row it helps, see below).
  const float invZ = 1.0f / Z;
  // linear: the residual at a rejected position
  bool resid = !TREE && (j < P.k);
  // lossless tree: p without the children's tokens
  bool masked = LOSSLESS && s_nx > 0;
  const int nx = LOSSLESS ? s_nx : 0;
  const SV_GLOBAL Vec16* cur_vrow = vrow;
  int cur_nvec = nvec, cur_h = h;
  float cur_m = m;
  const char* qrowp = static_cast<const char*>(P.probs) +
                      (static_cast<size_t>(b) * (TREE ? P.R : P.k) + (TREE || j < P.k ? j : 0)) * V * qeb;
  const SV_GLOBAL Vec16* vq = gptr<Vec16>(
      reinterpret_cast<const void*>(reinterpret_cast<uintptr_t>(qrowp) - (reinterpret_cast<uintptr_t>(qrowp) & 15)));
  auto load_q = [&](int vi) -> Vec16 {
    Vec16 v{};
    if (QMODE == kQVec && resid) v = ld16(vq, vi, cur_nvec);
    if (QMODE == kQHalf && resid) {  // branch free like ld16: lanes past the row load vector 0
      const bool in = vi < cur_nvec;
      const int e0 = (in ? vi : 0) * VE - cur_h;  // 8-byte aligned in q by the host's choice of mode
      const uint64_t d = *gptr<uint64_t>(qrowp + static_cast<ptrdiff_t>(e0) * 2);
      v.w[0] = in ? static_cast<uint32_t>(d) : 0u;
      v.w[1] = in ? static_cast<uint32_t>(d >> 32) : 0u;
    }
    return v;
  };
  // Lossless tree: bit i * VE + e of em[] is set when element e of this thread's vector
  // v0 + i * kWave is one of the children's tokens (rare: a vector with no bit set is
  // never touched by the mask).
  constexpr int kMaskWords = (NV * VE + 31) / 32;
  auto excl_bits = [&](int v0, uint32_t (&em)[kMaskWords]) {
#pragma unroll
    for (int k = 0; k < kMaskWords; ++k) em[k] = 0u;
    for (int ci = 0; ci < nx; ++ci) {
      const int pos = s_xtok[ci] + h;  // element position in the vector-aligned stream
      const int d = pos / VE - v0;
      if (d >= 0 && d < NV * kWave && (d & (kWave - 1)) == 0) {
        const int bit = (d / kWave) * VE + (pos - (pos / VE) * VE);
#pragma unroll
        for (int k = 0; k < kMaskWords; ++k)
          if (k == bit / 32) em[k] |= 1u << (bit & 31);
      }
    }
  };
  // the VE mask bits of vector vi alone
  auto vec_excl = [&](int vi) -> uint32_t {
    uint32_t xb = 0u;
    for (int ci = 0; ci < nx; ++ci) {
      const int pos = s_xtok[ci] + h;
      if (pos / VE == vi) xb |= 1u << (pos - (pos / VE) * VE);
    }
    return xb;
  };
  // the VE mask bits of slot i (i known at compile time in the tile loops)
  auto slot_bits = [&](const uint32_t (&em)[kMaskWords], int i) -> uint32_t {
    return (em[(i * VE) / 32] >> ((i * VE) & 31)) & ((1u << VE) - 1u);
  };
  // candidate weights of one vector: 2^((l - m) c) for a bonus / tree draw, or the
  // residual max(0, p - q) at a rejected linear position (edge padding is -inf: 0), or
  // for the lossless tree 2^((l - m) c) with the children's tokens at 0 (`xb`: the mask
  // bits of this vector).  Linear rows use one form for both: max(0, x * s - q) with
  // s = 1 / Z and q from the draft row for a residual, s = 1 and q = 0 otherwise (q
  // vectors are zero when not loaded), which is exactly x for x >= 0, so the residual
  // loop carries no per-element select.  Tree rows never take a residual: x itself.
  float wsc = resid ? invZ : 1.0f;
  auto weights = [&](const Vec16& lv, const Vec16& qv, int vi, float* w, uint32_t xb = 0u) {
    const int e0 = vi * VE - cur_h;
#pragma unroll
    for (int e = 0; e < VE; ++e) {
      const float x = fast_exp2((E::at(lv, e) - cur_m) * c);
      if (TREE) {
        w[e] = x;
        continue;
      }
      float q = 0.f;
      if (QMODE == kQVec) q = E::at(qv, e);
      else if (QMODE == kQHalf) q = Elem<true>::at(qv, e);
      else if (resid) q = (e0 + e >= 0 && e0 + e < V) ? load_elem(qrowp, e0 + e, P.q_bf16 != 0) : 0.f;
      w[e] = fmaxf(0.f, fmaf(x, wsc, -q));
    }
    if (LOSSLESS) {  // branch free: a branch here kept every vector's weights live at once
#pragma unroll
      for (int e = 0; e < VE; ++e) w[e] = ((xb >> e) & 1u) ? 0.f : w[e];
    }
  };
  // Per-vector sums of this thread's share of a tile (seg[]) and the wave's total (the
  // sequential sum of seg[], then a wave reduction: the same bits whichever workgroup
  // computes it).  The walk sums each slot over the wave (slot_total) from the same seg[].
  // A tile that is not in registers (`reload_row`) is re-read together with its first batch
  // of q vectors, so the two reads share one round trip.
  float seg[NV];
  auto slot_total = [&](int i) -> float { return lane_value(wave_inclusive_scan(seg[i]), 63); };
  auto tile_totals = [&](int v0, bool reload_row) -> float {
    constexpr int GQ = QMODE == kQElem ? 2 : (NT >= 512 && QMODE == kQVec) ? 8 : NV;
    constexpr int G = NV < GQ ? NV : GQ;
    if (reload_row) {
#pragma unroll
      for (int i = 0; i < NV; ++i) buf[i] = ld16_any(cur_vrow, v0 + i * kWave, cur_nvec);
    }
    uint32_t em[kMaskWords];
    if (masked) excl_bits(v0, em);
    else {
#pragma unroll
      for (int k = 0; k < kMaskWords; ++k) em[k] = 0u;
    }
#pragma unroll
    for (int g0 = 0; g0 < NV; g0 += G) {
      Vec16 qv[G] = {};
      if (resid) {  // one uniform branch around the whole batch of q loads
#pragma unroll
        for (int g = 0; g < G; ++g) qv[g] = load_q(v0 + (g0 + g) * kWave);
      }
      if (g0 == 0 && reload_row) {
#pragma unroll
        for (int i = 0; i < NV; ++i) buf[i] = mask_edges<BF16>(buf[i], (v0 + i * kWave) * VE - cur_h, V);
      }
#pragma unroll
      for (int g = 0; g < G; ++g) {
        float w[VE];
        weights(buf[g0 + g], qv[g], v0 + (g0 + g) * kWave, w, LOSSLESS ? slot_bits(em, g0 + g) : 0u);
        float sgm = 0.f;
#pragma unroll
        for (int e = 0; e < VE; ++e) sgm += w[e];
        seg[g0 + g] = sgm;
      }
    }
    float own = 0.f;
#pragma unroll
    for (int i = 0; i < NV; ++i) own += seg[i];
    return wave_sum(own);
  };

  if (s_flag) {
    const float u_smp = s_usmp;
    int loaded_tile = P.ntiles - 1;  // buf holds the last tile of pass 1
    for (int attempt = 0; attempt < 2; ++attempt) {
      // One loop, one copy of tile_totals: steps 0 .. ntiles-1 compute the residual totals
      // of every tile (residual draws only; the register-resident tile first, the others
      // re-read, mostly from cache); the last step locates the winning (tile, wave) and lets
      // that wave recompute its sums when they are not in registers already.
      bool empty = false, skip = false, coop = false;
      double t = 0.0, before = 0.0;
      bool clamp = false;
      int tile_s = 0, wave_s = 0;
      const int first = loaded_tile;
      // A masked draw (lossless tree) takes the pass-1 partials for every unit; a unit that
      // holds children's tokens has their weights taken out of its total (one thread, the
      // children in order, so the bits do not depend on timing; a total that rounding
      // leaves below 0 is 0).  s_tot < 0 marks a unit left as it was.  The walk recomputes
      // the winning unit with the tokens masked, which agrees with this to rounding.
      if (masked) {
        for (int q = tid; q < nunits; q += NT) s_tot[q] = -1.f;
        __syncthreads();
        if (tid == 0) {
          for (int ci = 0; ci < nx; ++ci) {
            const int vc = (s_xtok[ci] + h) / VE;
            const int q = (vc / TILE) * NW + (vc % TILE) / (NV * kWave);
            const float base = s_tot[q] >= 0.f ? s_tot[q] : s_ps[q] * fast_exp2((s_pm[q] - m) * c);
            s_tot[q] = fmaxf(0.f, base - s_xsub[ci]);
          }
        }
      }
      int step0 = resid ? 0 : P.ntiles;
      if (HELP && resid && P.help_on) {
        // The residual's tiles are claimed one at a time from the row's counter, which the
        // rows that help claim from too: the tile in registers first (never claimed), then
        // the claimed ones (the next claim in flight while a tile is summed), then the
        // totals of the tiles others claimed, which those workgroups publish as they finish.
        uint64_t* hw = P.help_words + static_cast<size_t>(r) * P.help_stride;
        uint64_t cl = 0;
        if (tid == 0) cl = __hip_atomic_fetch_add(&hw[1], 1ull, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        {
          const float wt = tile_totals(loaded_tile * TILE + wid * (NV * kWave) + lane, false);
          if (lane == 0) s_tot[loaded_tile * NW + wid] = wt;
        }
        if (tid == 0) s_claim[0] = static_cast<int>(cl);
        __syncthreads();
        uint64_t mine = 0;
        for (int it = 0;; ++it) {
          const int cc = s_claim[it & 1];
          if (cc >= P.ntiles - 1) break;
          if (tid == 0) cl = __hip_atomic_fetch_add(&hw[1], 1ull, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
          const float wt = tile_totals(cc * TILE + wid * (NV * kWave) + lane, true);
          loaded_tile = cc;
          if (lane == 0) s_tot[cc * NW + wid] = wt;
          mine |= 1ull << cc;
          if (tid == 0) s_claim[(it + 1) & 1] = static_cast<int>(cl);
          __syncthreads();
        }
        if (wid == 0) {
          // unit (t, w) of a tile summed elsewhere arrives in word 2 + t * NW + w (bit 32 set)
          const bool need = lane < (P.ntiles - 1) * NW && !((mine >> (lane / NW)) & 1ull);
          uint64_t v = 0;
          bool have = !need;
          for (int spin = 0;; ++spin) {
            if (__ballot(!have) == 0) break;
            if (spin == kHelpSpin) {
              if (lane == 0) __hip_atomic_fetch_or(P.errword, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
              break;
            }
            if (!have) {
              v = __hip_atomic_load(&hw[2 + lane], __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
              have = v != 0;
            }
          }
          if (need) s_tot[lane] = __uint_as_float(static_cast<uint32_t>(v));
        }
        step0 = P.ntiles;  // only the unit pick is left (its barrier follows)
      }
      for (int step = step0; step <= P.ntiles; ++step) {
        int tile;
        bool active;
        if (step < P.ntiles) {
          tile = first + step;  // (first + step) mod ntiles, both below ntiles
          if (tile >= P.ntiles) tile -= P.ntiles;
          active = resid;
        } else {
          // a single-tile rejected row's deferred check: an earlier rejection posted
          // meanwhile makes this draw irrelevant
          if (DEFER && resid && tid == 0) {
            uint64_t seen = rej_dep;
            asm volatile("" : "+v"(seen));  // the value is first needed here, not earlier
            s_skip = seen > static_cast<uint64_t>(64 - j) ? 1 : 0;
          }
          if (resid || masked) __syncthreads();
          if (DEFER && s_skip) {
            if (tid == 0) s_flag = 0;  // read again only by thread 0, when publishing
            skip = true;
            break;
          }
          // weight of each (tile, wave) unit: the residual totals, or for a draw from p
          // itself the pass-1 partials rescaled to the row max (nothing recomputed)
          auto unit = [&](int q) -> float {
            if (resid || (masked && s_tot[q] >= 0.f)) return s_tot[q];
            return s_ps[q] * fast_exp2((s_pm[q] - m) * c);
          };
          // every thread walks the units in the same order: S, then the winning unit
          float S = 0.f;
          for (int q = 0; q < nunits; ++q) S += unit(q);
          if (S <= 0.f) {  // residual or remainder empty through rounding: draw from p itself
            empty = true;
            break;
          }
          t = static_cast<double>(u_smp) * static_cast<double>(S);
          float cum = 0.f;
          int star = -1, last_pos = -1;
          for (int q = 0; q < nunits; ++q) {
            const float uq = unit(q);
            const float nc = cum + uq;
            if (uq > 0.f) last_pos = q;
            if (star < 0 && static_cast<double>(nc) > t) {
              star = q;
              before = cum;
            }
            cum = nc;
          }
          // Sums at different levels are rounded in different orders; when t falls past a
          // level's total (only within rounding of a CDF boundary) take the last positive
          // weight.
          if (star < 0) {
            star = last_pos;
            clamp = true;
          }
          tile_s = star / NW;
          wave_s = star - tile_s * NW;
          tile = tile_s;
          // The winning unit's weights are recomputed by every wave together (a quarter or an
          // eighth of its slots each, the unit reloaded) unless a residual draw already holds
          // them in the winner's registers.  Single-tile rows hold the whole row: a draw from
          // p there is walked by the winner wave from its registers after this step sums its
          // slots (B=1000 k=4 V=1024: 13.3 -> 12.8 us); a unit of a 16-vector tile is cheaper
          // to split over the waves (every wave summing its own measured 0.5 us slower).
          coop = REG_DRAW ? tile_s != loaded_tile : (!resid || tile_s != loaded_tile);
          active = REG_DRAW && !coop && !resid && wid == wave_s;
        }
        if (active) {
          const int v0 = tile * TILE + wid * (NV * kWave) + lane;
          const bool reload_row = tile != loaded_tile;  // only this wave's share when locating the winner
          loaded_tile = tile;
          // slot totals for the tile that stays in registers (the last step) and for the winner
          const float wt = tile_totals(v0, reload_row);
          if (step < P.ntiles && lane == 0) s_tot[tile * NW + wid] = wt;
        }
      }
      if (DEFER && skip) break;
      if (empty) {
        if (!resid && !masked) break;
        resid = false;
        masked = false;
        wsc = 1.0f;
        continue;
      }
      if (coop) {
        // wave w reloads slots [w * NS, (w + 1) * NS) of the unit, computes their weights and
        // slot totals; the wave that owns the winning slot walks it
        constexpr int NS = NV >= NW ? NV / NW : 1;
        const int ubase = tile_s * TILE + wave_s * (NV * kWave) + lane;  // slot i: ubase + 64 i
        const bool owns = wid * NS < NV;
        Vec16 cl[NS], cq[NS];
        float cs[NS];
#pragma unroll
        for (int ii = 0; ii < NS; ++ii) cl[ii] = ld16_any(vrow, ubase + (wid * NS + ii) * kWave, owns ? nvec : 0);
#pragma unroll
        for (int ii = 0; ii < NS; ++ii) cq[ii] = load_q(owns ? ubase + (wid * NS + ii) * kWave : nvec);
#pragma unroll
        for (int ii = 0; ii < NS; ++ii) {
          const int vi = ubase + (wid * NS + ii) * kWave;
          cl[ii] = mask_edges<BF16>(cl[ii], vi * VE - h, V);
          float w[VE];
          weights(cl[ii], cq[ii], vi, w, masked ? vec_excl(vi) : 0u);
          float sg = 0.f;
#pragma unroll
          for (int e = 0; e < VE; ++e) sg += w[e];
          cs[ii] = owns ? sg : 0.f;
          const float st = wave_sum(cs[ii]);
          if (owns && lane == 0) s_slot[wid * NS + ii] = st;
        }
        __syncthreads();
        // slot inside the unit (uniform walk over the slot totals)
        const double t1 = t - before;
        int istar = -1, ilast = -1;
        float icum = 0.f, ibefore = 0.f;
        for (int i = 0; i < NV; ++i) {
          const float st = s_slot[i];
          const float nc = icum + st;
          if (st > 0.f) ilast = i;
          if (!clamp && istar < 0 && static_cast<double>(nc) > t1) {
            istar = i;
            ibefore = icum;
          }
          icum = nc;
        }
        if (istar < 0) {
          istar = ilast < 0 ? 0 : ilast;
          clamp = true;
        }
        if (wid == istar / NS) {
          const int ii0 = istar - wid * NS;
          float sg = 0.f;
          Vec16 ls = cl[0], qs = cq[0];
#pragma unroll
          for (int ii = 0; ii < NS; ++ii)
            if (ii == ii0) {
              sg = cs[ii];
              ls = cl[ii];
              qs = cq[ii];
            }
          const int vi = ubase + istar * kWave;
          const float scan = wave_inclusive_scan(sg);
          const double t2 = t1 - static_cast<double>(ibefore);
          const uint64_t hit = __ballot(sg > 0.f && static_cast<double>(scan) > t2);
          const uint64_t pos = __ballot(sg > 0.f);
          int lstar;
          if (!clamp && hit) {
            lstar = __ffsll(static_cast<long long>(hit)) - 1;
          } else {
            lstar = pos ? 63 - __clzll(static_cast<long long>(pos)) : 0;
            clamp = true;
          }
          const float excl = lane_value(scan, lstar > 0 ? lstar - 1 : 0);
          if (lane == lstar) {
            float w[VE];
            weights(ls, qs, vi, w, masked ? vec_excl(vi) : 0u);
            const double t3 = t2 - (lstar > 0 ? static_cast<double>(excl) : 0.0);
            int y = -1, ylast = -1;
            float ec = 0.f;
#pragma unroll
            for (int e = 0; e < VE; ++e) {
              ec += w[e];
              if (w[e] > 0.f) {
                ylast = e;
                if (!clamp && y < 0 && static_cast<double>(ec) > t3) y = e;
              }
            }
            if (y < 0) y = ylast < 0 ? 0 : ylast;
            s_y = vi * VE - h + y;
          }
        }
      } else if (wid == wave_s) {
        const int v0 = tile_s * TILE + wid * (NV * kWave) + lane;
        // slot inside the wave (uniform walk over the slot totals)
        const double t1 = t - before;
        int istar = -1, ilast = -1;
        float icum = 0.f, ibefore = 0.f;
#pragma unroll
        for (int i = 0; i < NV; ++i) {
          const float st = slot_total(i);
          const float nc = icum + st;
          if (st > 0.f) ilast = i;
          if (!clamp && istar < 0 && static_cast<double>(nc) > t1) {
            istar = i;
            ibefore = icum;
          }
          icum = nc;
        }
        if (istar < 0) {
          istar = ilast < 0 ? 0 : ilast;
          clamp = true;
        }
        // The winning slot's logits are in buf (this wave's share of tile_s is what buf
        // holds now); no reload.  A 16-byte q vector is loaded before the lane scan, so
        // that its latency overlaps the scan.
        const int vis = v0 + istar * kWave;
        const Vec16 qs = QMODE == kQVec ? load_q(vis) : Vec16{};
        Vec16 ls = buf[0];
#pragma unroll
        for (int i = 1; i < NV; ++i)
          if (i == istar) ls = buf[i];
        // lane inside the slot: the slot's scan again (same inputs, same values)
        float sg = 0.f;
#pragma unroll
        for (int i = 0; i < NV; ++i)
          if (i == istar) sg = seg[i];
        const float scan = wave_inclusive_scan(sg);
        const double t2 = t1 - static_cast<double>(ibefore);
        // (the scan is tree-ordered: its prefixes need not grow by exactly each lane's
        // weight, so a lane of zero weight is never taken)
        const uint64_t hit = __ballot(sg > 0.f && static_cast<double>(scan) > t2);
        const uint64_t pos = __ballot(sg > 0.f);
        int lstar;
        if (!clamp && hit) {
          lstar = __ffsll(static_cast<long long>(hit)) - 1;
        } else {
          lstar = pos ? 63 - __clzll(static_cast<long long>(pos)) : 0;
          clamp = true;
        }
        const float excl = lane_value(scan, lstar > 0 ? lstar - 1 : 0);
        if (lane == lstar) {
          const int vi = vis;
          float w[VE];
          uint32_t xb = 0u;
          if (masked) {
            uint32_t em[kMaskWords];
            excl_bits(v0, em);
#pragma unroll
            for (int i = 0; i < NV; ++i)
              if (i == istar) xb = slot_bits(em, i);
          }
          weights(ls, QMODE == kQVec ? qs : load_q(vi), vi, w, xb);
          const double t3 = t2 - (lstar > 0 ? static_cast<double>(excl) : 0.0);
          int y = -1, ylast = -1;
          float ec = 0.f;
#pragma unroll
          for (int e = 0; e < VE; ++e) {
            ec += w[e];
            if (w[e] > 0.f) {
              ylast = e;
              if (!clamp && y < 0 && static_cast<double>(ec) > t3) y = e;
            }
          }
          if (y < 0) y = ylast;
          s_y = vi * VE - h + y;
        }
      }
      break;
    }
  }
  __syncthreads();

  // ---- help: a row after its sequence's earliest rejection supplies nothing to the
  // outputs; it claims residual tiles of that rejected row (from the row's own counter,
  // which the row claims from too) and publishes their per-wave totals (the same sums the
  // row's own workgroup would compute: tile_totals on that row)
  if (HELP && P.help_on) {
    if (tid == 0) {
      s_hr = -1;
      if (s_help >= 0) {
        const int hr = b * P.R + s_help;
        uint64_t mz = 0;
        for (int spin = 0; spin < kHelpSpin && mz == 0; ++spin)
          mz = __hip_atomic_load(P.help_words + static_cast<size_t>(hr) * P.help_stride, __ATOMIC_RELAXED,
                                 __HIP_MEMORY_SCOPE_AGENT);
        if (mz != 0) {
          s_hr = hr;
          s_hm = __uint_as_float(static_cast<uint32_t>(mz >> 32));
          s_hz = __uint_as_float(static_cast<uint32_t>(mz));
        }
      }
    }
    __syncthreads();
    const int hr = __builtin_amdgcn_readfirstlane(s_hr);
    if (hr >= 0) {
      uint64_t* hw = P.help_words + static_cast<size_t>(hr) * P.help_stride;
      // point the weights at row hr: its residual against its own (m, Z)
      const int hj = hr - b * P.R;
      const char* hrowp = static_cast<const char*>(P.logits) + static_cast<size_t>(hr) * V * EB;
      const uintptr_t hra = reinterpret_cast<uintptr_t>(hrowp);
      cur_h = static_cast<int>(hra & 15) / EB;
      cur_vrow = gptr<Vec16>(reinterpret_cast<const void*>(hra - (hra & 15)));
      cur_nvec = (V + cur_h + VE - 1) / VE;
      qrowp = static_cast<const char*>(P.probs) + (static_cast<size_t>(b) * P.k + hj) * V * qeb;
      vq = gptr<Vec16>(reinterpret_cast<const void*>(reinterpret_cast<uintptr_t>(qrowp) -
                                                      (reinterpret_cast<uintptr_t>(qrowp) & 15)));
      cur_m = __uint_as_float(__builtin_amdgcn_readfirstlane(__float_as_uint(s_hm)));
      wsc = 1.0f / __uint_as_float(__builtin_amdgcn_readfirstlane(__float_as_uint(s_hz)));
      resid = true;
      masked = false;
      if (tid == 0) s_claim[0] = static_cast<int>(__hip_atomic_fetch_add(&hw[1], 1ull, __ATOMIC_RELAXED,
                                                                        __HIP_MEMORY_SCOPE_AGENT));
      __syncthreads();
      for (int it = 0;; ++it) {
        const int cc = s_claim[it & 1];
        if (cc >= P.ntiles - 1) break;
        uint64_t cl = 0;
        if (tid == 0) cl = __hip_atomic_fetch_add(&hw[1], 1ull, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        const float wt = tile_totals(cc * TILE + wid * (NV * kWave) + lane, true);
        if (lane == 0)
          __hip_atomic_store(&hw[2 + cc * NW + wid], (1ull << 32) | __float_as_uint(wt), __ATOMIC_RELAXED,
                             __HIP_MEMORY_SCOPE_AGENT);
        if (tid == 0) s_claim[(it + 1) & 1] = static_cast<int>(cl);
        __syncthreads();
      }
    }
    // this workgroup's stores and atomics on the help words are acknowledged before its
    // ticket: the sequence's last workgroup clears them afterwards
    wait_vmem_all();
    __syncthreads();
  }

  // ---- publish this row's result, then take the sequence ticket
  if (tid == 0) {
    uint64_t dep = 0;
    if (TREE) {
      dep ^= dec_dep;
      if (child_acc) dep ^= atomic_or_u64(&P.seqword[2 * b], child_acc);
      if (s_flag) dep ^= atomic_or_u64(&P.rowword[r], static_cast<uint64_t>(static_cast<uint32_t>(s_y + 1)));
    } else {
      dep ^= rej_dep;
      // the last row's deferred check (single-tile rows): an earlier rejection makes its draw
      // irrelevant, so it is not posted
      const bool post = s_flag && !(DEFER && j == P.k && rej_dep > static_cast<uint64_t>(64 - j));
      if (post) {
        const uint64_t key = (static_cast<uint64_t>(j) << 32) | static_cast<uint32_t>(s_y);
        dep ^= atomic_max_u64(&P.seqword[2 * b], ~key);
      }
    }
    after_value(dep);
    const uint32_t prev = take_ticket(&P.counters[b]);
    s_last = (prev == static_cast<uint32_t>(P.R - 1));
  }
  __syncthreads();
  if (!s_last || wid != 0) return;

  // ---- last arrival: the sequence's outputs
  if (HELP && P.help_on) {  // the help words of the sequence's rows and its decision mask
    const int per = 2 + P.ntiles * NW;
    for (int q = lane; q < P.R * per; q += kWave)
      __hip_atomic_store(&P.help_words[static_cast<size_t>(b * P.R + q / per) * P.help_stride + q % per], 0ull,
                         __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    if (lane == 0)
      __hip_atomic_store(&P.help_words[static_cast<size_t>(b * P.R) * P.help_stride + (P.help_stride - 1)], 0ull,
                         __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  }
  if (!TREE) {
    const int k = P.k;
    // the draft tokens are read while the exchange below is in flight (k = 0 reads a
    // valid word of this kernel's own output instead)
    const int32_t* tp = k > 0 ? P.tokens + (static_cast<size_t>(b) * k + (lane < k ? lane : k - 1))
                              : P.out_accept_len + b;
    const int dtok = load_early_i32(tp);
    uint64_t best = 0;
    if (lane == 0) {
      best = atomic_xchg_u64(&P.seqword[2 * b], 0ull);
      (void)atomic_xchg_u64(&P.seqword[2 * b + 1], 0ull);
    }
    const uint32_t blo = static_cast<uint32_t>(lane_value(static_cast<int>(best), 0));
    const uint32_t bhi = static_cast<uint32_t>(lane_value(static_cast<int>(best >> 32), 0));
    const uint64_t key = ~((static_cast<uint64_t>(bhi) << 32) | blo);
    int n = static_cast<int>(key >> 32);
    int y = static_cast<int>(static_cast<uint32_t>(key));
    if (n < 0 || n > k) {  // no candidate posted (cannot happen: row k always posts)
      n = k;
      y = -1;
    }
    if (lane < P.R) {
      int t = -1;
      if (lane < n) t = dtok;
      else if (lane == n) t = y;
      P.out_tokens[static_cast<size_t>(b) * P.R + lane] = t;
    }
    if (lane == 0) {
      P.out_accept_len[b] = n;
      reset_ticket(&P.counters[b]);
    }
  } else {
    const int N = P.R;
    // lane l reads node l's token while the exchanges below are in flight
    const int ntok = load_early_i32(P.tokens + (static_cast<size_t>(b) * N + (lane < N ? lane : N - 1)));
    uint64_t mask = 0;
    if (lane == 0) mask = atomic_xchg_u64(&P.seqword[2 * b], 0ull);
    const uint32_t mlo = static_cast<uint32_t>(lane_value(static_cast<int>(mask), 0));
    const uint32_t mhi = static_cast<uint32_t>(lane_value(static_cast<int>(mask >> 32), 0));
    const uint64_t accm = (static_cast<uint64_t>(mhi) << 32) | mlo;
    int cand_c = -1, dep = 0, par = 0;
    if (lane < N) {
      cand_c = static_cast<int>(static_cast<uint32_t>(
                   atomic_xchg_u64(&P.rowword[static_cast<size_t>(b) * N + lane], 0ull))) - 1;
      dep = s_dep[lane];
      par = lane == 0 ? 0 : s_par[lane];
    }
    uint64_t alive = 1ull;
    for (int d = 1; d <= td.D; ++d) {
      const bool a = lane < N && dep == d && ((accm >> lane) & 1ull) && ((alive >> par) & 1ull);
      alive |= __ballot(a);
    }
    const int key = wave_max_int(((alive >> lane) & 1ull) ? dep * 64 + (63 - lane) : -1);
    const int cstar = 63 - (key & 63);
    const int dstar = key >> 6;
    const int ybonus = lane_value(cand_c, cstar);
    // ancestors of c*: lane d holds the node at depth d on the path (d <= dstar)
    int node = -1;
    {
      int cur = cstar;
      for (int d = dstar; d >= 0; --d) {
        if (lane == d) node = cur;
        cur = d > 0 ? s_par[cur] : 0;
      }
    }
    const int W = td.D + 1;
    const int nxt = __shfl(node, lane + 1 < kWave ? lane + 1 : kWave - 1);  // all lanes active
    const int tok_nxt = __shfl(ntok, nxt >= 0 ? nxt : 0);
    if (lane < W) {
      int t = -1;
      if (lane < dstar) t = tok_nxt;
      else if (lane == dstar) t = ybonus;
      P.out_tokens[static_cast<size_t>(b) * W + lane] = t;
      if (P.out_path) P.out_path[static_cast<size_t>(b) * W + lane] = lane <= dstar ? node : -1;
    }
    if (lane == 0) {
      P.out_accept_len[b] = dstar;
      reset_ticket(&P.counters[b]);
    }
  }
}

// ------------------------------------------------------------------ launch table
template <bool BF16, int NT, int NV, bool TREE, int QMODE, bool STOP = false>
static hipError_t launch_one(const RowParams& P, const TreeDesc& td, int grid, hipStream_t st) {
  const size_t lds = 3 * static_cast<size_t>(P.ntiles) * (NT / kWave) * sizeof(float);
  hipLaunchKernelGGL((row_verify_kernel<BF16, NT, NV, TREE, QMODE, STOP>), dim3(grid), dim3(NT), lds, st, P, td);
  return hipGetLastError();
}

// Linear rows of 256 x 16 tiles stop streaming after an earlier rejection only when the
// grid takes several rounds of workgroups: the rows of a later round then start after the
// earlier positions have decided (B=256 k=8 V=128256: 134 -> 113 us).  In a single round
// the per-tile reads of the rejection word cost more than they saved (B=256 k=1: 46.0 ->
// 46.8 us), so that grid runs the instance without them.
template <bool BF16, bool TREE, int QMODE>
static hipError_t launch_tiles_256(const RowParams& P, const TreeDesc& td, int grid, hipStream_t st) {
  if constexpr (TREE) return launch_one<BF16, 256, 16, TREE, QMODE>(P, td, grid, st);
  else {
    static int cap[64] = {};  // workgroups of the instance the device holds at once, per device
    int dev = 0, c = 0;
    if (hipGetDevice(&dev) == hipSuccess && dev >= 0 && dev < 64) {
      c = __atomic_load_n(&cap[dev], __ATOMIC_RELAXED);
      if (c == 0) {
        const size_t lds = 3 * static_cast<size_t>(P.ntiles) * (256 / kWave) * sizeof(float);
        int per_cu = 0, cus = 0;
        if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, row_verify_kernel<BF16, 256, 16, TREE, QMODE, true>,
                                                         256, lds) == hipSuccess &&
            hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) == hipSuccess && per_cu > 0 &&
            cus > 0) {
          c = per_cu * cus;
          __atomic_store_n(&cap[dev], c, __ATOMIC_RELAXED);
        }
      }
    }
    if (c > 0 && grid > c) return launch_one<BF16, 256, 16, TREE, QMODE, true>(P, td, grid, st);
    // one round: the last rows wait for the earlier rows' decisions when those fill the
    // chip's CUs on their own (B k >= 256, so their stream keeps HBM busy meanwhile)
    RowParams P1 = P;
    P1.bonus_wait = c > 0 && P.help_on && P.k > 0 && static_cast<int64_t>(P.B) * P.k >= 256;
    return launch_one<BF16, 256, 16, TREE, QMODE>(P1, td, grid, st);
  }
}

template <bool BF16, bool TREE, int QMODE>
static hipError_t launch_rows_t(const RowParams& P, const TreeDesc& td, int cfg, int grid, hipStream_t st) {
  switch (cfg) {
    case 0: return launch_one<BF16, 64, 4, TREE, QMODE>(P, td, grid, st);
    case 1: return launch_one<BF16, 256, 4, TREE, QMODE>(P, td, grid, st);
    case 2: return launch_one<BF16, 512, 8, TREE, QMODE>(P, td, grid, st);
    case 3: return launch_tiles_256<BF16, TREE, QMODE>(P, td, grid, st);
    default: return launch_one<BF16, 512, 16, TREE, QMODE>(P, td, grid, st);
  }
}

// A row that fits 64 x 4, 256 x 4 or 512 x 8 (the first that holds it) is one tile with
// few vectors per thread: the per-element work of both passes is then spread over more
// waves (512 x 8 measured faster than 256 x 16 and than 1024 x 4 at V = 32000 bf16).
// Longer rows are walked in tiles: of 256 x 16 when the batch has enough rows to give
// every CU two workgroups (occupancy hides latency best there), of 512 x 16 when it has
// few rows (each workgroup then keeps twice the bytes in flight).
RowConfig choose_row_config(bool bf16, int V, int head_max, int64_t rows) {
  static const int nt[kRowConfigs] = {64, 256, 512, 256, 512};
  static const int nv[kRowConfigs] = {4, 4, 8, 16, 16};
  constexpr int kSingleTileConfigs = 3;
  constexpr int64_t kManyRows = 512;
  const int ve = bf16 ? 8 : 4;
  const long long need = static_cast<long long>(V) + head_max;
  int cfg = rows >= kManyRows ? kRowConfigs - 2 : kRowConfigs - 1;
  for (int i = 0; i < kSingleTileConfigs; ++i) {
    if (static_cast<long long>(nt[i]) * nv[i] * ve >= need) {
      cfg = i;
      break;
    }
  }
  const long long cap = static_cast<long long>(nt[cfg]) * nv[cfg] * ve;
  RowConfig rc{};
  rc.cfg = cfg;
  rc.threads = nt[cfg];
  rc.ntiles = static_cast<int>((need + cap - 1) / cap);
  return rc;
}

hipError_t launch_rows(const RowParams& P, const TreeDesc& td, bool bf16, bool tree, int qmode, int cfg,
                       int grid, hipStream_t st) {
  if (tree && qmode == kQLossless)
    return bf16 ? launch_rows_t<true, true, kQLossless>(P, td, cfg, grid, st)
                : launch_rows_t<false, true, kQLossless>(P, td, cfg, grid, st);
  if (tree)  // the tree draws its extra token from p alone; q is read at the children only
    return bf16 ? launch_rows_t<true, true, kQElem>(P, td, cfg, grid, st)
                : launch_rows_t<false, true, kQElem>(P, td, cfg, grid, st);
  if (bf16)
    return qmode == kQVec ? launch_rows_t<true, false, kQVec>(P, td, cfg, grid, st)
                          : launch_rows_t<true, false, kQElem>(P, td, cfg, grid, st);
  if (qmode == kQVec) return launch_rows_t<false, false, kQVec>(P, td, cfg, grid, st);
  if (qmode == kQHalf) return launch_rows_t<false, false, kQHalf>(P, td, cfg, grid, st);
  return launch_rows_t<false, false, kQElem>(P, td, cfg, grid, st);
}

}  // namespace sv
