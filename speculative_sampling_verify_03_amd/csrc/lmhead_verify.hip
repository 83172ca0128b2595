// Verification of the LM head's logits from the softmax partials its GEMM writes
// ("Accelerating Sonar through speculation", sections "EAGLE" and "Training MTP heads": the
// heads share the target's LM head; section "Speculative decoding": acceptance stage and
// target-generation stage; "Speculative decoding explained", section "Draft and
// verification loop").
//
// The direct GEMM kernel leaves, for every row and every block of kLmhBlockCols columns,
// the (max, sum of 2^((l - max) c)) pair of those logits, so the rows' normalisers need no
// second pass over the float32 logits.
//   lmh_decide_kernel, one workgroup per sequence: each wave merges the pairs of a row
//     (lane l the blocks of its stretch in order, then one DPP tree), gathers l(x) and
//     q(x) and takes the acceptance decision u * q(x) < p(x) in float64; the first
//     rejection n (or k) gives the accepted tokens and the length, and n with row n's
//     (max, sum) is handed to the draw kernel.
//   lmh_draw_kernel, one wave per (column block, sequence): for a rejected position every
//     block's wave computes its residual mass max(0, p - q) and takes a ticket; the wave
//     that completes the count locates u * S over the blocks' masses (S = 0, a residual
//     emptied by rounding, draws from p), re-reads the winning block and walks it (lane
//     scan, then the lane's eight elements).  When every draft was kept, the extra token is
//     drawn from p of the last row by block 0's wave alone: the GEMM's pairs, rescaled to
//     the row maximum, already weigh the blocks.
// The draw kernel's hand-over words are results written before an arrival count (agent-
// scope atomic stores, acknowledged before the count's atomic) and read only by the
// arrival that completes it, which returns them to zero.
#include "sv_device.hpp"
#include "sv_launch.hpp"

namespace sv {

namespace {

constexpr int kDecideThreads = 512;
constexpr int kDecideWaves = kDecideThreads / kWave;
constexpr int kBlockPerLane = kLmhBlockCols / kWave;  // 8 consecutive columns per lane
constexpr int kMaxPer = kLmhMaxBlocks / kWave;       // column blocks per lane, at most
constexpr int kDrawThreads = 256;
constexpr int kDrawWaves = kDrawThreads / kWave;
constexpr int kChunkCols = 8192;                                 // residual chunk
constexpr int kChunkGroups = kChunkCols / (8 * kDrawThreads);    // 8-column groups per thread
static_assert(kChunkGroups * 8 * kDrawThreads == kChunkCols, "chunk = whole groups of every thread");

__device__ __forceinline__ void wait_vmem_all() { __builtin_amdgcn_s_waitcnt(0x70 | 0xf00); }

__device__ __forceinline__ uint64_t get64(uint64_t* p) {
  return __hip_atomic_load(p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ void put64(uint64_t* p, uint64_t v) {
  __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ void put32(uint32_t* p, uint32_t v) {
  __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ float hi_f(uint64_t w) { return __uint_as_float(static_cast<uint32_t>(w >> 32)); }
__device__ __forceinline__ float lo_f(uint64_t w) { return __uint_as_float(static_cast<uint32_t>(w)); }

// ---------------------------------------------------------------- decide
__global__ __launch_bounds__(kDecideThreads) void lmh_decide_kernel(LmhParams P) {
  __shared__ int s_acc[64];
  __shared__ float s_m[64], s_z[64];
  const int tid = threadIdx.x;
  const int lane = tid & (kWave - 1);
  const int wid = __builtin_amdgcn_readfirstlane(tid / kWave);
  const int b = blockIdx.x;
  const int k = P.k;
  for (int j = wid; j < P.R; j += kDecideWaves) {
    const int64_t r = static_cast<int64_t>(b) * P.R + j;
    // the draft token and the values it indexes are read while the pairs are merged
    int x = -1;
    if (j < k) x = P.tokens[static_cast<size_t>(b) * k + j];
    const bool valid = x >= 0 && x < P.V;
    float lx = 0.f, qx = 0.f;
    if (valid) {
      lx = P.logits[static_cast<size_t>(r) * P.V + x];
      qx = load_elem(P.probs, (static_cast<int64_t>(b) * k + j) * P.V + x, P.q_bf16 != 0);
    }
    // (m, Z): lane l merges blocks l, l + 64, ... in order (all loads issued first), then
    // the wave's DPP tree
    uint64_t pw[kMaxPer];
#pragma unroll
    for (int i = 0; i < kMaxPer; ++i) {
      const int t = lane + kWave * i;
      pw[i] = t < P.nb ? P.part[r * P.nb + t] : 0ull;
    }
    float m = -INFINITY, Z = 0.f;
#pragma unroll
    for (int i = 0; i < kMaxPer; ++i)
      if (lane + kWave * i < P.nb) merge_max_sum(m, Z, hi_f(pw[i]), lo_f(pw[i]), P.c);
    wave_merge_max_sum(m, Z, P.c);
    bool acc = false;
    if (j < k) {
      float ua, us;
      draw_uniforms(P.seed, P.offset, static_cast<uint32_t>(b), static_cast<uint32_t>(j), ua, us);
      double px = 0.0;
      if (valid) px = exp((static_cast<double>(lx) - static_cast<double>(m)) / P.T) / static_cast<double>(Z);
      acc = valid && (static_cast<double>(ua) * static_cast<double>(qx) < px);
      if (lane == 0) {
        const size_t o = static_cast<size_t>(b) * k + j;
        if (P.out_tprob) P.out_tprob[o] = static_cast<float>(px);
        if (P.out_aprob) {
          double ap;
          if (qx > 0.f) ap = px / static_cast<double>(qx) < 1.0 ? px / static_cast<double>(qx) : 1.0;
          else ap = px > 0.0 ? 1.0 : 0.0;
          P.out_aprob[o] = static_cast<float>(ap);
        }
      }
    }
    if (lane == 0) {
      s_acc[j] = acc ? 1 : 0;
      s_m[j] = m;
      s_z[j] = Z;
    }
  }
  __syncthreads();
  if (wid != 0) return;
  const int dtok = k > 0 ? P.tokens[static_cast<size_t>(b) * k + (lane < k ? lane : k - 1)] : -1;
  const uint64_t rej = __ballot(lane < k && s_acc[lane < k ? lane : 0] == 0);
  const int n = rej ? __ffsll(static_cast<long long>(rej)) - 1 : k;
  if (lane < P.R && lane != n) P.out_tokens[static_cast<size_t>(b) * P.R + lane] = lane < n ? dtok : -1;
  if (lane == 0) {
    P.out_accept_len[b] = n;
    put64(&P.seqw[2 * b + 1], (static_cast<uint64_t>(__float_as_uint(s_m[n])) << 32) | __float_as_uint(s_z[n]));
    put64(&P.seqw[2 * b], static_cast<uint64_t>(n + 1));
  }
}

// ---------------------------------------------------------------- draw
// The eight elements of columns col .. col + 7 of a row (whole vectors: V % 8 == 0).
struct Eight {
  float v[8];
};
__device__ __forceinline__ Eight load_f32x8(const float* p) {
  const SV_GLOBAL Vec16* g = gptr<Vec16>(p);
  const Vec16 a = ld16_any(g, 0, 2), c = ld16_any(g, 1, 2);
  Eight e;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    e.v[i] = __uint_as_float(a.w[i]);
    e.v[4 + i] = __uint_as_float(c.w[i]);
  }
  return e;
}
__device__ __forceinline__ Eight load_q8(const void* base, int64_t elem, bool bf16) {
  Eight e;
  if (bf16) {
    const Vec16 a = ld16_any(gptr<Vec16>(static_cast<const uint16_t*>(base) + elem), 0, 1);
#pragma unroll
    for (int i = 0; i < 8; ++i) e.v[i] = Elem<true>::at(a, i);
  } else {
    e = load_f32x8(static_cast<const float*>(base) + elem);
  }
  return e;
}

// Weight of logit l: the residual max(0, p - q) (p = 2^((l - m) c) / Z), or p unnormalised
// (from_p), the same expression wherever a block is summed or walked.
__device__ __forceinline__ float weight(float l, float q, float m, float c, float invZ, bool from_p) {
  const float x = fast_exp2((l - m) * c);
  return from_p ? x : fmaxf(0.f, fmaf(x, invZ, -q));
}

// Inverse-CDF step across the lanes of a wave (incl: the inclusive scan of the nonnegative
// weights w): the first lane of positive weight whose running sum passes t; when none does
// (t past the total, only within rounding of a CDF boundary) or clamp is already set, the
// last lane of positive weight, and clamp is set.  -1 when no weight is positive.
__device__ __forceinline__ int pick_lane(float w, float incl, double t, bool& clamp) {
  const uint64_t pos = __ballot(w > 0.f);
  if (!clamp) {
    const uint64_t above = __ballot(w > 0.f && static_cast<double>(incl) > t);
    if (above) return __ffsll(static_cast<long long>(above)) - 1;
  }
  clamp = true;
  return pos ? 63 - __clzll(static_cast<long long>(pos)) : -1;
}

// Token at offset t into block blk of row r (weights as `weight`), for one wave: lane l's
// eight columns blk * 512 + 8 l .. + 7 are summed in order, the lanes scanned, and the
// winning lane walks its eight.
__device__ int walk_block(const LmhParams& P, int64_t r, int64_t qr, int blk, float m, float invZ, bool from_p,
                          double t, bool clamp, int lane) {
  const int col = blk * kLmhBlockCols + kBlockPerLane * lane;
  const bool in = col < P.V;
  const int cs = in ? col : 0;
  const Eight l = load_f32x8(P.logits + r * P.V + cs);
  Eight q{};
  if (!from_p) q = load_q8(P.probs, qr * P.V + cs, P.q_bf16 != 0);
  float w[8];
  float s = 0.f;
#pragma unroll
  for (int e = 0; e < 8; ++e) {
    w[e] = in ? weight(l.v[e], q.v[e], m, P.c, invZ, from_p) : 0.f;
    s += w[e];
  }
  const float incl = wave_inclusive_scan(s);
  int ls = pick_lane(s, incl, t, clamp);
  const double t1 = t - (ls > 0 ? static_cast<double>(lane_value(incl, ls - 1)) : 0.0);
  if (ls < 0) ls = 0;
  int y = 0;
  if (lane == ls) {
    float ce = 0.f;
    int ek = -1, elast = -1;
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      const float nc = ce + w[e];
      if (w[e] > 0.f) elast = e;
      if (!clamp && ek < 0 && static_cast<double>(nc) > t1) ek = e;
      ce = nc;
    }
    if (ek < 0) ek = elast < 0 ? 0 : elast;
    y = col + ek;
  }
  return lane_value(y, ls);
}

// One draw from p of row r (row maximum m) with uniform u, for one wave: the GEMM's block
// pairs rescaled to m weigh the blocks (lane l the stretch [l * per, (l + 1) * per), loads
// issued together), the lanes are scanned, the winning lane walks its stretch, and
// walk_block finds the token inside the block.
__device__ int draw_from_p(const LmhParams& P, int64_t r, float m, float u, int lane) {
  const int per = (P.nb + kWave - 1) / kWave;
  const uint64_t* pr = P.part + r * P.nb;
  uint64_t pw[kMaxPer];
#pragma unroll
  for (int i = 0; i < kMaxPer; ++i) {
    const int bi = lane * per + i;
    pw[i] = (i < per && bi < P.nb) ? pr[bi] : 0ull;
  }
  float wv[kMaxPer];
  float own = 0.f;
#pragma unroll
  for (int i = 0; i < kMaxPer; ++i) {
    const float s = lo_f(pw[i]);
    wv[i] = s > 0.f ? s * fast_exp2((hi_f(pw[i]) - m) * P.c) : 0.f;
    own += wv[i];
  }
  const float incl = wave_inclusive_scan(own);
  const double t = static_cast<double>(u) * static_cast<double>(lane_value(incl, 63));
  bool clamp = false;
  int ls = pick_lane(own, incl, t, clamp);
  const double t1 = t - (ls > 0 ? static_cast<double>(lane_value(incl, ls - 1)) : 0.0);
  if (ls < 0) ls = 0;
  int blk = 0, cl = clamp ? 1 : 0;
  double tin = 0.0;
  if (lane == ls) {
    float ce = 0.f, before = 0.f;
    int found = -1, last = -1;
#pragma unroll
    for (int i = 0; i < kMaxPer; ++i) {
      const float nc = ce + wv[i];
      if (wv[i] > 0.f) last = i;
      if (!clamp && found < 0 && static_cast<double>(nc) > t1) {
        found = i;
        before = ce;
      }
      ce = nc;
    }
    if (found < 0) {
      found = last < 0 ? 0 : last;
      cl = 1;
    }
    blk = lane * per + found;
    tin = t1 - static_cast<double>(before);
  }
  blk = lane_value(blk, ls);
  clamp = lane_value(cl, ls) != 0;
  const int64_t tb = __double_as_longlong(tin);
  tin = __longlong_as_double((static_cast<int64_t>(lane_value(static_cast<int>(tb >> 32), ls)) << 32) |
                             static_cast<uint32_t>(lane_value(static_cast<int>(tb), ls)));
  return walk_block(P, r, 0, blk, m, 1.f, true, tin, clamp, lane);
}

// Thread tid's share of chunk cc of row r: groups g = tid + 256 i (i < kChunkGroups) of 8
// columns, col = cc * kChunkCols + 8 g; a group at or past V (V % 8 == 0) weighs 0.
template <bool QBF16>
struct ChunkShare {
  Eight l[kChunkGroups], q[kChunkGroups];
  bool in[kChunkGroups];
  __device__ __forceinline__ void load(const LmhParams& P, int64_t r, int64_t qr, int cc, int tid) {
#pragma unroll
    for (int i = 0; i < kChunkGroups; ++i) {
      const int col = cc * kChunkCols + 8 * (tid + kDrawThreads * i);
      in[i] = col < P.V;
      const int cs = in[i] ? col : 0;
      l[i] = load_f32x8(P.logits + r * P.V + cs);
      q[i] = load_q8(P.probs, qr * P.V + cs, QBF16);
    }
  }
  __device__ __forceinline__ float group_sum(int i, float m, float c, float invZ) const {
    float s = 0.f;
#pragma unroll
    for (int e = 0; e < 8; ++e) s += weight(l[i].v[e], q[i].v[e], m, c, invZ, false);
    return in[i] ? s : 0.f;
  }
};

template <bool QBF16>
__global__ __launch_bounds__(kDrawThreads) void lmh_draw_kernel(LmhParams P) {
  __shared__ uint64_t s_hdr[2];
  __shared__ float s_part[kChunkGroups][kDrawWaves];
  __shared__ int s_last, s_chunk, s_mode;
  __shared__ double s_t;
  const int tid = threadIdx.x;
  const int lane = tid & (kWave - 1);
  const int wid = __builtin_amdgcn_readfirstlane(tid / kWave);
  const int cc = blockIdx.x;
  const int b = blockIdx.y;
  if (tid == 0) {
    s_hdr[0] = get64(&P.seqw[2 * b]);
    s_hdr[1] = get64(&P.seqw[2 * b + 1]);
  }
  __syncthreads();
  const uint64_t h0 = s_hdr[0];
  if (h0 == 0) return;
  const int n = static_cast<int>(h0) - 1;
  const float m = hi_f(s_hdr[1]);
  const float invZ = 1.0f / lo_f(s_hdr[1]);
  const float c = P.c;
  const int64_t r = static_cast<int64_t>(b) * P.R + n;
  if (n == P.k) {  // every draft kept: the extra token from p of the last row, by one wave
    if (cc != 0 || wid != 0) return;
    float ua, us;
    draw_uniforms(P.seed, P.offset, static_cast<uint32_t>(b), static_cast<uint32_t>(n), ua, us);
    const int y = draw_from_p(P, r, m, us, lane);
    if (lane == 0) {
      P.out_tokens[static_cast<size_t>(b) * P.R + n] = y;
      put64(&P.seqw[2 * b], 0ull);
      put64(&P.seqw[2 * b + 1], 0ull);
    }
    return;
  }
  // residual at the first rejection: this chunk's mass, slot totals (waves in order) then
  // slots in order, as the walk below sums them
  const int64_t qr = static_cast<int64_t>(b) * P.k + n;
  ChunkShare<QBF16> sh;
  sh.load(P, r, qr, cc, tid);
#pragma unroll
  for (int i = 0; i < kChunkGroups; ++i) {
    const float a = wave_sum(sh.group_sum(i, m, c, invZ));
    if (lane == 0) s_part[i][wid] = a;
  }
  __syncthreads();
  if (tid == 0) {
    float mass = 0.f;
    for (int i = 0; i < kChunkGroups; ++i) {
      float ti = 0.f;
      for (int w = 0; w < kDrawWaves; ++w) ti += s_part[i][w];
      mass += ti;
    }
    put32(&P.cmass[static_cast<size_t>(b) * P.cstride + cc], __float_as_uint(mass));
    wait_vmem_all();
    s_last = take_ticket(&P.ccnt[b]) == static_cast<uint32_t>(P.nchunks - 1);
  }
  __syncthreads();
  if (!s_last) return;

  // ---- the chunk that completed the count: u * S over the chunk masses
  if (wid == 0) {
    float w = 0.f;
    if (lane < P.nchunks) {
      uint32_t* cw = &P.cmass[static_cast<size_t>(b) * P.cstride + lane];
      w = __uint_as_float(__hip_atomic_load(cw, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT));
      put32(cw, 0u);
    }
    float ua, us;
    draw_uniforms(P.seed, P.offset, static_cast<uint32_t>(b), static_cast<uint32_t>(n), ua, us);
    const float incl = wave_inclusive_scan(w);
    const float S = lane_value(incl, 63);
    int mode = 0, ch = 0;
    bool clamp = false;
    double t1 = 0.0;
    if (S > 0.f) {
      const double t = static_cast<double>(us) * static_cast<double>(S);
      const int cs = pick_lane(w, incl, t, clamp);
      t1 = t - (cs > 0 ? static_cast<double>(lane_value(incl, cs - 1)) : 0.0);
      ch = cs < 0 ? 0 : cs;
    } else {  // residual empty through rounding: draw from p itself
      mode = 1;
      const int y = draw_from_p(P, r, m, us, lane);
      if (lane == 0) P.out_tokens[static_cast<size_t>(b) * P.R + n] = y;
    }
    if (lane == 0) {
      s_chunk = ch;
      s_mode = mode | (clamp ? 2 : 0);
      s_t = t1;
      reset_ticket(&P.ccnt[b]);
      put64(&P.seqw[2 * b], 0ull);
      put64(&P.seqw[2 * b + 1], 0ull);
    }
  }
  __syncthreads();
  if (s_mode & 1) return;
  const int cs = s_chunk;
  bool clamp = (s_mode & 2) != 0;
  const double t1 = s_t;
  sh.load(P, r, qr, cs, tid);
  float gs[kChunkGroups];
#pragma unroll
  for (int i = 0; i < kChunkGroups; ++i) {
    gs[i] = sh.group_sum(i, m, c, invZ);
    const float a = wave_sum(gs[i]);
    if (lane == 0) s_part[i][wid] = a;
  }
  __syncthreads();
  // group slot, then wave, in the order the chunk's mass was summed (every thread alike)
  int is = -1, ilast = -1;
  float cum = 0.f, before = 0.f;
  for (int i = 0; i < kChunkGroups; ++i) {
    float ti = 0.f;
    for (int w = 0; w < kDrawWaves; ++w) ti += s_part[i][w];
    const float nc = cum + ti;
    if (ti > 0.f) ilast = i;
    if (!clamp && is < 0 && static_cast<double>(nc) > t1) {
      is = i;
      before = cum;
    }
    cum = nc;
  }
  if (is < 0) {
    clamp = true;
    is = ilast < 0 ? 0 : ilast;
  }
  const double t2 = t1 - static_cast<double>(before);
  int ws = -1, wlast = -1;
  cum = 0.f;
  before = 0.f;
  for (int w = 0; w < kDrawWaves; ++w) {
    const float tw = s_part[is][w];
    const float nc = cum + tw;
    if (tw > 0.f) wlast = w;
    if (!clamp && ws < 0 && static_cast<double>(nc) > t2) {
      ws = w;
      before = cum;
    }
    cum = nc;
  }
  if (ws < 0) {
    clamp = true;
    ws = wlast < 0 ? 0 : wlast;
  }
  if (wid != ws) return;
  const double t3 = t2 - static_cast<double>(before);
  float g = 0.f;
#pragma unroll
  for (int i = 0; i < kChunkGroups; ++i)
    if (i == is) g = gs[i];
  const float incl = wave_inclusive_scan(g);
  int ls = pick_lane(g, incl, t3, clamp);
  const double t4 = t3 - (ls > 0 ? static_cast<double>(lane_value(incl, ls - 1)) : 0.0);
  if (ls < 0) ls = 0;
  if (lane != ls) return;
  int ek = -1, elast = -1;
  float ce = 0.f;
#pragma unroll
  for (int i = 0; i < kChunkGroups; ++i) {
    if (i != is) continue;
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      const float x = sh.in[i] ? weight(sh.l[i].v[e], sh.q[i].v[e], m, c, invZ, false) : 0.f;
      const float nc = ce + x;
      if (x > 0.f) elast = e;
      if (!clamp && ek < 0 && static_cast<double>(nc) > t4) ek = e;
      ce = nc;
    }
  }
  if (ek < 0) ek = elast < 0 ? 0 : elast;
  P.out_tokens[static_cast<size_t>(b) * P.R + n] = cs * kChunkCols + 8 * (tid + kDrawThreads * is) + ek;
}

}  // namespace

hipError_t launch_lmhead_verify(const LmhParams& P, hipStream_t st) {
  if (P.nb < 1 || P.nb > kLmhMaxBlocks || P.R > 64 || P.nchunks < 1 || P.nchunks > P.cstride ||
      P.cstride > kWave || static_cast<int64_t>(P.nchunks) * kChunkCols < P.V)
    return hipErrorInvalidValue;
  hipLaunchKernelGGL(lmh_decide_kernel, dim3(static_cast<unsigned>(P.B)), dim3(kDecideThreads), 0, st, P);
  const hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  const dim3 grid(static_cast<unsigned>(P.nchunks), static_cast<unsigned>(P.B));
  if (P.q_bf16) hipLaunchKernelGGL(lmh_draw_kernel<true>, grid, dim3(kDrawThreads), 0, st, P);
  else hipLaunchKernelGGL(lmh_draw_kernel<false>, grid, dim3(kDrawThreads), 0, st, P);
  return hipGetLastError();
}

}  // namespace sv
