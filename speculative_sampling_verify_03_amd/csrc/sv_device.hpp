// Device-side building blocks shared by the verification kernels (gfx950, wave64).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include <climits>

namespace sv {

constexpr int kWave = 64;

// One 16-byte global load: 4 float32 or 8 bfloat16 values.
struct alignas(16) Vec16 {
  uint32_t w[4];
};

// Element views of a Vec16.  bfloat16 widens to float32 exactly (it is the top half).
template <bool BF16>
struct Elem;

template <>
struct Elem<false> {
  static constexpr int kPerVec = 4;
  static constexpr int kBytes = 4;
  __device__ static __forceinline__ float at(const Vec16& v, int e) { return __uint_as_float(v.w[e]); }
};

template <>
struct Elem<true> {
  static constexpr int kPerVec = 8;
  static constexpr int kBytes = 2;
  __device__ static __forceinline__ float at(const Vec16& v, int e) {
    const uint32_t w = v.w[e >> 1];
    return __uint_as_float((e & 1) ? (w & 0xffff0000u) : (w << 16));
  }
};

// Global-address-space views.  Pointers that come out of parameter structs are generic
// to the compiler, which then emits flat loads with a 64-bit address per lane; going
// through address space 1 gives global loads with a scalar base and a 32-bit offset.
#define SV_GLOBAL __attribute__((address_space(1)))
template <typename T>
__device__ __forceinline__ const SV_GLOBAL T* gptr(const void* p) {
  return (const SV_GLOBAL T*)(p);
}

// 16-byte load of vector i when 0 <= i < n, zeros otherwise (n >= 1).  Branch free: lanes
// out of range load vector 0 and discard it, so a run of ld16 calls stays in one basic
// block and issues back to back instead of one exec-masked block (and one wait) per load.
__device__ __forceinline__ Vec16 ld16(const SV_GLOBAL Vec16* p, int i, int n) {
  const bool in = static_cast<unsigned>(i) < static_cast<unsigned>(n);
  const SV_GLOBAL Vec16& g = p[in ? i : 0];
  const uint32_t w0 = g.w[0], w1 = g.w[1], w2 = g.w[2], w3 = g.w[3];
  Vec16 v;
  v.w[0] = in ? w0 : 0u;
  v.w[1] = in ? w1 : 0u;
  v.w[2] = in ? w2 : 0u;
  v.w[3] = in ? w3 : 0u;
  return v;
}

// 16-byte load of vector i when 0 <= i < n, else of vector 0 (n >= 1), with no select on the
// result: for logits rows, mask_edges below turns every element of a vector past the row
// into -inf anyway.  Loads with no consumer inside a conditional block (a tile's prefetch)
// then carry no wait with them.  Used where a draw re-reads a tile of its row.
__device__ __forceinline__ Vec16 ld16_any(const SV_GLOBAL Vec16* p, int i, int n) {
  const SV_GLOBAL Vec16& g = p[static_cast<unsigned>(i) < static_cast<unsigned>(n) ? i : 0];
  Vec16 v;
  v.w[0] = g.w[0];
  v.w[1] = g.w[1];
  v.w[2] = g.w[2];
  v.w[3] = g.w[3];
  return v;
}

// ld16_any as a non-temporal (streaming) load, for bytes that are read once: the logits of
// a row's first pass (its tiles and their prefetch) and of the greedy scan.  Measured on MI355X: greedy B=256 k=8
// V=128256 115 -> 104 us, linear B=64 k=5 V=32000 17.9 -> 17.1 us, B=256 k=8 141 -> 136 us.
__device__ __forceinline__ Vec16 ld16_stream(const SV_GLOBAL Vec16* p, int i, int n) {
  typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));
  const u32x4 x = __builtin_nontemporal_load(
      reinterpret_cast<const SV_GLOBAL u32x4*>(p + (static_cast<unsigned>(i) < static_cast<unsigned>(n) ? i : 0)));
  Vec16 v;
  v.w[0] = x.x;
  v.w[1] = x.y;
  v.w[2] = x.z;
  v.w[3] = x.w;
  return v;
}

// Elements of a vector that fall outside [0, V) (e0 = token id of element 0) are set to
// -inf: they then drop out of every max, exp-sum, residual and argmax without per-element
// bounds tests in the hot loops.  Only the first and last vector of a row can be partial.
template <bool BF16>
__device__ __forceinline__ Vec16 mask_edges(Vec16 v, int e0, int V) {
  constexpr int VE = BF16 ? 8 : 4;
  if (e0 >= 0 && e0 + VE <= V) return v;
#pragma unroll
  for (int e = 0; e < VE; ++e) {
    const bool out = (e0 + e < 0) || (e0 + e >= V);
    if (BF16) {
      uint32_t& w = v.w[e >> 1];
      if (out) w = (e & 1) ? ((w & 0x0000ffffu) | 0xff800000u) : ((w & 0xffff0000u) | 0x0000ff80u);
    } else {
      if (out) v.w[e] = 0xff800000u;
    }
  }
  return v;
}

// Opaque use of the packed row registers: the compiler must assume they changed, so
// values unpacked from them earlier cannot be kept alive and reused later.  Holding the
// unpacked floats would double the register footprint of a resident row.
template <int NV>
__device__ __forceinline__ void pin_packed(Vec16 (&buf)[NV]) {
#pragma unroll
  for (int i = 0; i < NV; ++i)
    asm volatile("" : "+v"(buf[i].w[0]), "+v"(buf[i].w[1]), "+v"(buf[i].w[2]), "+v"(buf[i].w[3]));
}

// Scalar load of element i of a float32 (bf16 = false) or bfloat16 array.
__device__ __forceinline__ float load_elem(const void* base, int64_t i, bool bf16) {
  if (bf16) return __uint_as_float(static_cast<uint32_t>(gptr<uint16_t>(base)[i]) << 16);
  return gptr<float>(base)[i];
}

// A 32-bit load issued where it stands: as a relaxed atomic it is an ordered access that
// the compiler does not sink to the value's first use (plain loads were moved past the
// atomics their value does not depend on, which added a round trip).
__device__ __forceinline__ int load_early_i32(const int32_t* p) {
  return __hip_atomic_load((SV_GLOBAL int32_t*)(p), __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP);
}

// 2^x with the hardware transcendental (v_exp_f32, ~1 ulp).  Results below 2^-126 flush
// to zero, which only drops terms smaller than 2^-126 of the row maximum.
__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }

// ---------------------------------------------------------------- wave collectives
// Built on DPP (data-parallel primitives): cross-lane moves inside the vector ALU that
// cost a few cycles, unlike LDS-routed shuffles (ds_bpermute / ds_swizzle, ~100+ cycles
// each) whose latency chains dominated every reduction.  An inclusive scan is the
// classic GCN sequence: row_shr 1, 2, 4, 8 inside each 16-lane row, then row_bcast15 into
// rows 1 and 3 and row_bcast31 into rows 2 and 3.  Lanes without a source read the
// operation's identity.  Reductions read lane 63 of the scan.
template <int CTRL, int ROW_MASK = 0xF>
__device__ __forceinline__ float dpp_f(float identity, float x) {
  return __int_as_float(__builtin_amdgcn_update_dpp(__float_as_int(identity), __float_as_int(x), CTRL, ROW_MASK,
                                                    0xF, false));
}
template <int CTRL, int ROW_MASK = 0xF>
__device__ __forceinline__ int dpp_i(int identity, int x) {
  return __builtin_amdgcn_update_dpp(identity, x, CTRL, ROW_MASK, 0xF, false);
}
constexpr int kDppShr1 = 0x111, kDppShr2 = 0x112, kDppShr4 = 0x114, kDppShr8 = 0x118;
constexpr int kDppBcast15 = 0x142, kDppBcast31 = 0x143;
constexpr int kDppRowBcast15 = 0x15F;  // row_newbcast:15, lane 15 of each row of 16 to the row

__device__ __forceinline__ float lane_value(float x, int lane) {
  return __int_as_float(__builtin_amdgcn_readlane(__float_as_int(x), lane));
}
__device__ __forceinline__ int lane_value(int x, int lane) { return __builtin_amdgcn_readlane(x, lane); }

// Inclusive prefix sum over the 64 lanes.
__device__ __forceinline__ float wave_inclusive_scan(float x) {
  x += dpp_f<kDppShr1>(0.f, x);
  x += dpp_f<kDppShr2>(0.f, x);
  x += dpp_f<kDppShr4>(0.f, x);
  x += dpp_f<kDppShr8>(0.f, x);
  x += dpp_f<kDppBcast15, 0xA>(0.f, x);
  x += dpp_f<kDppBcast31, 0xC>(0.f, x);
  return x;
}
__device__ __forceinline__ float wave_sum(float x) { return lane_value(wave_inclusive_scan(x), 63); }

__device__ __forceinline__ float wave_max(float x) {
  x = fmaxf(x, dpp_f<kDppShr1>(-INFINITY, x));
  x = fmaxf(x, dpp_f<kDppShr2>(-INFINITY, x));
  x = fmaxf(x, dpp_f<kDppShr4>(-INFINITY, x));
  x = fmaxf(x, dpp_f<kDppShr8>(-INFINITY, x));
  x = fmaxf(x, dpp_f<kDppBcast15, 0xA>(-INFINITY, x));
  x = fmaxf(x, dpp_f<kDppBcast31, 0xC>(-INFINITY, x));
  return lane_value(x, 63);
}

__device__ __forceinline__ int wave_max_int(int x) {
  x = max(x, dpp_i<kDppShr1>(INT_MIN, x));
  x = max(x, dpp_i<kDppShr2>(INT_MIN, x));
  x = max(x, dpp_i<kDppShr4>(INT_MIN, x));
  x = max(x, dpp_i<kDppShr8>(INT_MIN, x));
  x = max(x, dpp_i<kDppBcast15, 0xA>(INT_MIN, x));
  x = max(x, dpp_i<kDppBcast31, 0xC>(INT_MIN, x));
  return lane_value(x, 63);
}

// Running (max, scaled sum) pair of an online softmax in base-2 units: the pair (m, s)
// stands for s * 2^(m * c) where c = log2(e) / T.  Merging keeps the larger max.
__device__ __forceinline__ void merge_max_sum(float& m, float& s, float m2, float s2, float c) {
  const float mm = fmaxf(m, m2);
  if (mm == -INFINITY) {  // both empty
    s = 0.f;
    m = mm;
    return;
  }
  s = s * fast_exp2((m - mm) * c) + s2 * fast_exp2((m2 - mm) * c);
  m = mm;
}

template <int CTRL, int ROW_MASK = 0xF>
__device__ __forceinline__ void merge_step(float& m, float& s, float c) {
  const float m2 = dpp_f<CTRL, ROW_MASK>(-INFINITY, m);
  const float s2 = dpp_f<CTRL, ROW_MASK>(0.f, s);
  merge_max_sum(m, s, m2, s2, c);
}

// All lanes end with the wave's merged (max, sum) pair.
__device__ __forceinline__ void wave_merge_max_sum(float& m, float& s, float c) {
  merge_step<kDppShr1>(m, s, c);
  merge_step<kDppShr2>(m, s, c);
  merge_step<kDppShr4>(m, s, c);
  merge_step<kDppShr8>(m, s, c);
  merge_step<kDppBcast15, 0xA>(m, s, c);
  merge_step<kDppBcast31, 0xC>(m, s, c);
  m = lane_value(m, 63);
  s = lane_value(s, 63);
}

// (value, index) argmax with the lowest index winning ties.
__device__ __forceinline__ void argmax_merge(float& v, int& i, float v2, int i2) {
  if (v2 > v || (v2 == v && i2 < i)) {
    v = v2;
    i = i2;
  }
}

template <int CTRL, int ROW_MASK = 0xF>
__device__ __forceinline__ void argmax_step(float& v, int& i) {
  const float v2 = dpp_f<CTRL, ROW_MASK>(-INFINITY, v);
  const int i2 = dpp_i<CTRL, ROW_MASK>(INT_MAX, i);
  argmax_merge(v, i, v2, i2);
}

__device__ __forceinline__ void wave_argmax(float& v, int& i) {
  argmax_step<kDppShr1>(v, i);
  argmax_step<kDppShr2>(v, i);
  argmax_step<kDppShr4>(v, i);
  argmax_step<kDppShr8>(v, i);
  argmax_step<kDppBcast15, 0xA>(v, i);
  argmax_step<kDppBcast31, 0xC>(v, i);
  v = lane_value(v, 63);
  i = lane_value(i, 63);
}

// ---------------------------------------------------------------- Philox4x64-10
// Salmon, Moraes, Dror, Shaw, "Parallel random numbers: as easy as 1, 2, 3" (SC'11):
// ten rounds of the 4x64 Philox S-box (two 64x64->128 multiplies per round by fixed odd
// multipliers, high halves xor-ed with the other counter words and the key), with the
// key advanced by two Weyl increments between rounds.
struct Philox4x64 {
  static constexpr uint64_t kMulA = 0xD2E7470EE14C6C93ull;
  static constexpr uint64_t kMulB = 0xCA5A826395121157ull;
  static constexpr uint64_t kWeylA = 0x9E3779B97F4A7C15ull;
  static constexpr uint64_t kWeylB = 0xBB67AE8584CAA73Bull;

  __device__ static __forceinline__ void block(uint64_t x[4], uint64_t key0, uint64_t key1) {
#pragma unroll
    for (int round = 0; round < 10; ++round) {
      const uint64_t a_lo = kMulA * x[0], a_hi = __umul64hi(kMulA, x[0]);
      const uint64_t b_lo = kMulB * x[2], b_hi = __umul64hi(kMulB, x[2]);
      const uint64_t y0 = b_hi ^ x[1] ^ key0;
      const uint64_t y2 = a_hi ^ x[3] ^ key1;
      x[0] = y0;
      x[1] = b_lo;
      x[2] = y2;
      x[3] = a_lo;
      key0 += kWeylA;
      key1 += kWeylB;
    }
  }
};

// The two uniforms of sequence `seq`, position / node `pos`: acceptance (word 0) and
// sampling (word 1), each the top 24 bits scaled by 2^-24 (exact in float32).
__device__ __forceinline__ void draw_uniforms(uint64_t seed, uint64_t offset, uint32_t seq,
                                              uint32_t pos, float& u_acc, float& u_smp) {
  uint64_t x[4] = {pos, seq, offset, 0ull};
  Philox4x64::block(x, seed, 0ull);
  u_acc = static_cast<float>(static_cast<uint32_t>(x[0] >> 40)) * 0x1.0p-24f;
  u_smp = static_cast<float>(static_cast<uint32_t>(x[1] >> 40)) * 0x1.0p-24f;
}

// ---------------------------------------------------------------- cross-workgroup results
// Workgroups of one sequence publish their results with device-scope read-modify-write
// atomics, which are performed at the device's coherence point and so are seen across
// XCDs (whose L2 caches are not coherent with one another).  A workgroup waits for the
// value its RMW returns before taking its arrival ticket (after_value), so every
// published result is complete before the ticket that counts it; the last arrival reads
// the results back with RMW exchanges that also return the words to zero.
__device__ __forceinline__ uint64_t atomic_max_u64(uint64_t* p, uint64_t v) {
  return __hip_atomic_fetch_max(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ uint64_t atomic_or_u64(uint64_t* p, uint64_t v) {
  return __hip_atomic_fetch_or(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ uint64_t atomic_xchg_u64(uint64_t* p, uint64_t v) {
  return __hip_atomic_exchange(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
// Number of workgroups of this sequence that arrived before the caller.
__device__ __forceinline__ uint32_t take_ticket(uint32_t* counter) {
  return __hip_atomic_fetch_add(counter, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ void reset_ticket(uint32_t* counter) {
  (void)__hip_atomic_exchange(counter, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
// Consumes v: the compiler must wait for the load / atomic that produced it before any
// later memory operation.
__device__ __forceinline__ void after_value(uint64_t v) { asm volatile("" ::"v"(v) : "memory"); }

// Orderable 64-bit key of an argmax candidate: larger value first, then lower index.
// -0.0 is keyed as +0.0: the two compare equal, so between them the lower index must win,
// as it does in the float comparisons of the in-thread and in-wave merges.
__device__ __forceinline__ uint64_t argmax_key(float v, int idx) {
  uint32_t u = __float_as_uint(v);
  if ((u << 1) == 0u) u = 0u;
  const uint32_t o = (u & 0x80000000u) ? ~u : (u | 0x80000000u);
  return (static_cast<uint64_t>(o) << 32) | (0xffffffffu - static_cast<uint32_t>(idx));
}
__device__ __forceinline__ int argmax_key_index(uint64_t key) {
  return static_cast<int>(0xffffffffu - static_cast<uint32_t>(key));
}

}  // namespace sv
