// LM-head projection on the matrix cores: logits[M, V] (fp32) = hidden[M, H] (bf16) @
// W[H, V] (bf16, row-major, vocabulary contiguous).  The EAGLE / MTP heads of
// "Accelerating Sonar through speculation" (sections "EAGLE" and "Training MTP heads")
// share the target's LM head, about 2 GB in bf16 for a 70B model; at the verification
// shapes (M = B(k+1), a few hundred rows) the product is bound by streaming W from HBM
// once, so the kernel is built around keeping that stream busy.
//
// v_mfma_f32_16x16x32_bf16 takes, per lane, 8 consecutive k of one row of A (lane % 16)
// and 8 consecutive k of one column of B, k group lane / 16.  W is row-major in k, so no
// lane can load its B operand with one vector load.  Instead each lane loads an 8 (k) x 4
// (n) block of W with eight 8-byte loads (16 lanes cover 128 contiguous bytes of a row)
// and turns it into four B operands with byte permutes: operand j holds column
// 4*(lane % 16) + j.  So MFMA j of a wave computes the columns {4c + j}, and lane l ends
// up holding four adjacent output columns per row: the results leave as 16-byte stores.
//
// Two kernels share that operand scheme.  lmhead_gemm_dma_kernel (below) is the one used
// when W rows are 16-byte aligned (V % 8 == 0, the usual vocabulary sizes): it streams W
// and the hidden states through LDS with direct global-to-LDS copies.  lmhead_gemm_kernel
// is the general fallback: a workgroup of four waves owns 256 columns and up to
// BM = 16*MB rows, each wave 64 columns x BM rows (MB*4 accumulator tiles); the
// hidden-state slice of a 32-k step (BM x 64 bytes) is shared through LDS (two buffers,
// one barrier per step, 16-byte chunks XOR-swizzled by row) and both streams are
// prefetched kStages steps ahead into registers.  It loads W with 8-byte loads when
// V % 4 == 0 and element by element otherwise.

#include "sv_device.hpp"
#include "sv_launch.hpp"

namespace sv {

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef float f32x4_t __attribute__((ext_vector_type(4)));

constexpr int kGemmThreads = 256;
constexpr int kWaveCols = 64;                // output columns per wave
constexpr int kBN = 4 * kWaveCols;           // per workgroup
constexpr int kBK = 32;                      // k per step (one MFMA deep)

typedef uint32_t W8 __attribute__((ext_vector_type(2)));  // four bf16 columns of one k row

// Word 3 of a gfx9 buffer descriptor for untyped loads (32-bit data format).
constexpr int kBufferFlags = 0x00020000;

__device__ __forceinline__ int clamp_records(size_t bytes) {
  return static_cast<int>(bytes > 0xffffffffull ? 0xffffffffu : static_cast<uint32_t>(bytes));
}

template <int MB>
struct ARegs {
  static constexpr int kChunks = MB / 4;  // 16-byte chunks per thread per step
  Vec16 v[kChunks];
};

template <int MB, bool VEC>
__global__ __launch_bounds__(kGemmThreads) __attribute__((amdgpu_waves_per_eu(1, 1))) void
lmhead_gemm_kernel(const uint16_t* __restrict__ A_, const uint16_t* __restrict__ W_, float* __restrict__ C,
                   int M, int H, int V) {
  static_assert(MB % 4 == 0, "A chunks must split evenly over the workgroup");
  constexpr int BM = 16 * MB;
  constexpr int AQ = MB / 4;
  constexpr int kStageDw = BM * 16;  // dwords of one A buffer: BM rows x 64 bytes
  constexpr int kStages = VEC ? 4 : 2;  // steps of W and A in flight per lane
  __shared__ __attribute__((aligned(16))) uint32_t sA[2 * kStageDw];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wid = tid >> 6;
  const int kg = lane >> 4;  // k group of this lane's operands
  const int n_lane = blockIdx.x * kBN + wid * kWaveCols + 4 * (lane & 15);
  const bool n_ok = n_lane < V;
  const int m0 = blockIdx.y * BM;
  const int nsteps = H / kBK;
  const size_t ldw = static_cast<size_t>(V);

  // Loads go through buffer descriptors: a scalar base per step (or per row block) plus one
  // constant 32-bit lane offset, so no per-load 64-bit address arithmetic.
  // W: rows kg*8 + i of the step, columns n_lane..n_lane+3.  Lanes past V read column 0;
  // every output column depends on its own W column only and those are never stored.
  const uint32_t w_voff = static_cast<uint32_t>((kg * 8 * ldw + ((VEC && !n_ok) ? 0 : n_lane)) * 2);
  const uint32_t w_row_bytes = static_cast<uint32_t>(ldw * 2);
  const size_t w_total = static_cast<size_t>(H) * ldw * 2;
  // A: chunk ch = tid + 256 q is (row ch / 4, 16-byte chunk ch % 4) of the step's slice;
  // rows past M read row M - 1 and are never stored.
  const uint16_t* a_blk = A_ + static_cast<size_t>(m0) * H;
  const size_t a_total = static_cast<size_t>(M - m0) * H * 2;
  const __amdgpu_buffer_rsrc_t a_rsrc =
      __builtin_amdgcn_make_buffer_rsrc(const_cast<uint16_t*>(a_blk), 0, clamp_records(a_total), kBufferFlags);
  uint32_t a_voff[AQ];
  int a_dst[AQ];
#pragma unroll
  for (int q = 0; q < AQ; ++q) {
    const int ch = tid + kGemmThreads * q;
    const int r = ch >> 2, c = ch & 3;
    const int rr = (m0 + r < M) ? r : M - 1 - m0;
    a_voff[q] = static_cast<uint32_t>(rr) * static_cast<uint32_t>(H) * 2u + 16u * c;
    a_dst[q] = r * 16 + 4 * (c ^ ((r >> 2) & 3));
  }
  // operand read: row mb*16 + lane%16, chunk kg (the swizzle depends on lane%16 only)
  const int a_src = (lane & 15) * 16 + 4 * (kg ^ ((lane >> 2) & 3));

  auto load_w = [&](int s, W8 (&w)[8]) {
    const size_t base = static_cast<size_t>(s) * kBK * ldw;
    if (VEC) {
      const __amdgpu_buffer_rsrc_t r = __builtin_amdgcn_make_buffer_rsrc(
          const_cast<uint16_t*>(W_ + base), 0, clamp_records(w_total - base * 2), kBufferFlags);
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        w[i] = __builtin_amdgcn_raw_buffer_load_b64(r, w_voff, i * w_row_bytes, 0);
      }
    } else {
      const SV_GLOBAL uint16_t* p = gptr<uint16_t>(W_) + base + kg * 8 * ldw + n_lane;
#pragma unroll
      for (int i = 0; i < 8; ++i) {
        uint32_t e[4];
#pragma unroll
        for (int j = 0; j < 4; ++j) e[j] = (n_lane + j < V) ? p[i * ldw + j] : 0u;
        w[i] = W8{e[0] | (e[1] << 16), e[2] | (e[3] << 16)};
      }
    }
  };
  auto load_a = [&](int s, ARegs<MB>& a) {
#pragma unroll
    for (int q = 0; q < AQ; ++q) {
      const auto x = __builtin_amdgcn_raw_buffer_load_b128(a_rsrc, a_voff[q], s * kBK * 2, 0);
      a.v[q].w[0] = x[0];
      a.v[q].w[1] = x[1];
      a.v[q].w[2] = x[2];
      a.v[q].w[3] = x[3];
    }
  };

  f32x4_t acc[MB][4];
#pragma unroll
  for (int mb = 0; mb < MB; ++mb)
#pragma unroll
    for (int j = 0; j < 4; ++j) acc[mb][j] = f32x4_t{0.f, 0.f, 0.f, 0.f};

  // Every step issues the same loads (a step past the end reloads the last one), so the
  // compiler's count of loads in flight is the same on every path and its waits stay at
  // "the loads of kStages steps ago" instead of collapsing to "all loads".
  const int last = nsteps - 1;
  W8 wbuf[kStages][8];
  ARegs<MB> abuf[kStages];
#pragma unroll
  for (int p = 0; p < kStages; ++p) {
    load_w(p < last ? p : last, wbuf[p]);
    load_a(p < last ? p : last, abuf[p]);
  }

  auto step = [&](int s, W8 (&w)[8], ARegs<MB>& a, bool refill) {
    // B operands: operand j, dword d = (k 2d, k 2d+1) of column 4*(lane%16) + j
    bf16x8_t b[4];
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const uint32_t sel = (j & 1) ? 0x07060302u : 0x05040100u;
      Vec16 o;
#pragma unroll
      for (int d = 0; d < 4; ++d) {
        const uint32_t lo = w[2 * d][j >> 1];
        const uint32_t hi = w[2 * d + 1][j >> 1];
        o.w[d] = __builtin_amdgcn_perm(hi, lo, sel);
      }
      b[j] = __builtin_bit_cast(bf16x8_t, o);
    }
    __builtin_amdgcn_sched_barrier(0);  // the old W registers are dead before the refill
    uint32_t* st = sA + (s & 1) * kStageDw;
#pragma unroll
    for (int q = 0; q < AQ; ++q) *reinterpret_cast<Vec16*>(st + a_dst[q]) = a.v[q];
    __syncthreads();
    if (refill) {
      const int sn = s + kStages < last ? s + kStages : last;
      load_w(sn, w);
      load_a(sn, a);
    }
    // keep the program order: loads of step s + kStages before this step's MFMAs, and the
    // next step's waits after them
    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
    for (int mb = 0; mb < MB; ++mb) {
      const Vec16 av = *reinterpret_cast<const Vec16*>(st + mb * 256 + a_src);
      const bf16x8_t af = __builtin_bit_cast(bf16x8_t, av);
#pragma unroll
      for (int j = 0; j < 4; ++j) acc[mb][j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(af, b[j], acc[mb][j], 0, 0, 0);
    }
    __builtin_amdgcn_sched_barrier(0);
  };

  const int nfull = nsteps - nsteps % kStages;
  for (int s0 = 0; s0 < nfull; s0 += kStages) {
#pragma unroll
    for (int p = 0; p < kStages; ++p) step(s0 + p, wbuf[p], abuf[p], true);
  }
#pragma unroll
  for (int p = 0; p < kStages - 1; ++p)
    if (nfull + p < nsteps) step(nfull + p, wbuf[p], abuf[p], false);

  // D layout of a 16x16 tile: lane l holds rows 4*(l/16)+i of column slot l%16, and
  // slot c of MFMA j is column 4c + j, so each row's four values are adjacent.
  if (!n_ok) return;
#pragma unroll
  for (int mb = 0; mb < MB; ++mb)
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int row = m0 + mb * 16 + kg * 4 + i;
      if (row >= M) continue;
      float* out = C + static_cast<size_t>(row) * ldw + n_lane;
      if (VEC) {
        *reinterpret_cast<float4*>(out) = make_float4(acc[mb][0][i], acc[mb][1][i], acc[mb][2][i], acc[mb][3][i]);
      } else {
#pragma unroll
        for (int j = 0; j < 4; ++j)
          if (n_lane + j < V) out[j] = acc[mb][j][i];
      }
    }
}

// ---------------------------------------------------------------------------------------
// Streaming variant for 16-byte aligned rows (V % 8 == 0).  W and A travel global -> LDS
// with global_load_lds_dwordx4, which holds no registers for the bytes in flight, through
// a ring of kDmaStages stages; each step waits for its own stage with an explicit vmcnt
// (every step issues the same copies, so the count is a constant) and one barrier.
// Operands are then read from LDS: W as the same 8 (k) x 4 (n) lane blocks, permuted into
// B operands as above.
//
// A workgroup is eight waves (two per SIMD, at most 256 registers each) over 512 columns:
// at V = 128256 the grid is a single round of about one workgroup per CU, and each A slice
// is shared by eight waves.
//
// Stage layout, in operand order so that every operand read is one lane-linear LDS access
// (these are conflict free, where row-strided 16-byte reads measured 2-way bank conflicts):
// for each wave 4 KB of W, slice i (k row 8*kg + i of its lane blocks) at i*512, lane l's
// 8 bytes at l*8; then per 16-row block of A 1 KB, lane l's 16 bytes (row l%16, chunk
// l/16) at l*16.  Copy lanes pick their global source to match: a W copy lane fetches the
// 16 bytes of two neighbouring operand lanes, an A copy lane the chunk of one.
constexpr int kDmaThreads = 512;
constexpr int kDmaWaves = kDmaThreads / 64;
constexpr int kDmaBN = kDmaWaves * kWaveCols;  // 512
constexpr int kDmaStages = 3;
constexpr int kWWaveBytes = kBK * kWaveCols * 2;  // 4 KB
constexpr int kWStageBytes = kDmaWaves * kWWaveBytes;

template <int MB>
struct DmaShape {
  static constexpr int kAStageBytes = MB * 1024;  // MB copies of 16 rows x 64 bytes
  static constexpr int kStageBytes = kWStageBytes + kAStageBytes;
  static constexpr int kLdsBytes = kDmaStages * kStageBytes;
  static constexpr int kWCopies = kWWaveBytes / 1024;  // W copies each wave issues per step
  // A copy t goes to wave t % 8, so waves below MB % 8 (or all, when 8 divides MB) take
  // one more than the others
  static constexpr int kAHi = (MB + kDmaWaves - 1) / kDmaWaves;
  static constexpr int kALo = MB / kDmaWaves;
};

// s_waitcnt with only the vector-memory count limited (gfx9 encoding: vmcnt bits 3:0 and
// 15:14, expcnt and lgkmcnt left at their maximum).
template <int N>
__device__ __forceinline__ void wait_vmcnt() {
  static_assert(N >= 0 && N < 64, "vmcnt is six bits");
  __builtin_amdgcn_s_waitcnt((N & 0xf) | ((N >> 4) << 14) | 0x70 | 0xf00);
}

// Workgroup barrier that also orders LDS accesses around it: this wave's LDS reads have
// returned (so another wave's copy may overwrite them) and no memory access moves across.
__device__ __forceinline__ void lds_barrier() {
  asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
}

// aux 2 = non-temporal: W is streamed once per call (2.1 GB at V = 128256), while the
// hidden states are re-read by every column block and keep the default policy.
// Non-temporal W copies measured 424 -> 416 us per GEMM at B=32 k=5 H=8192 V=128256.
template <bool NT = false>
__device__ __forceinline__ void copy16_to_lds(const SV_GLOBAL void* src, uint8_t* lds_base) {
  __builtin_amdgcn_global_load_lds(src, (__attribute__((address_space(3))) void*)(lds_base), 16, 0, NT ? 2 : 0);
}

template <int MB>
__global__ __launch_bounds__(kDmaThreads) __attribute__((amdgpu_waves_per_eu(2, 2))) void
lmhead_gemm_dma_kernel(const uint16_t* __restrict__ A_, const uint16_t* __restrict__ W_, float* __restrict__ C,
                       int M, int H, int V, uint64_t* __restrict__ part, float c) {
  using S = DmaShape<MB>;
  extern __shared__ __attribute__((aligned(16))) uint8_t smem[];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wid = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int kg = lane >> 4;
  const int n0 = blockIdx.x * kDmaBN;
  const int n_lane = n0 + wid * kWaveCols + 4 * (lane & 15);
  const int m0 = blockIdx.y * (16 * MB);
  const int nsteps = H / kBK;
  const size_t ldw = static_cast<size_t>(V);

  // W copy u of this wave fills slices 2u, 2u+1: copy lane j writes slice 2u + j/32 for
  // operand lanes 2p, 2p+1 (p = j%32), i.e. k row 8*(p/8) + 2u + j/32 of the step, columns
  // 8*(p%8) .. +7 of the wave's 64.  Chunks past V (whole chunks, V % 8 == 0) read column
  // 0: their columns are never stored.
  const SV_GLOBAL uint16_t* W = gptr<uint16_t>(W_);
  const int wcol = n0 + wid * kWaveCols + 8 * (lane & 7);
  const uint32_t w_src = static_cast<uint32_t>((8 * ((lane & 31) >> 3) + (lane >> 5)) * ldw + (wcol < V ? wcol : 0));
  // A copy t (wave t % 8) fills block t: copy lane j fetches row 16t + j%16, chunk j/16.
  // Rows past M read row M - 1.
  const SV_GLOBAL uint16_t* Ablk = gptr<uint16_t>(A_) + static_cast<size_t>(m0) * H;
  uint32_t a_src[S::kAHi];
#pragma unroll
  for (int q = 0; q < S::kAHi; ++q) {
    const int t = wid + kDmaWaves * q;
    const int r = 16 * t + (lane & 15);
    const int rr = (m0 + r < M) ? r : M - 1 - m0;
    a_src[q] = static_cast<uint32_t>(rr) * static_cast<uint32_t>(H) + 8u * (lane >> 4);
  }
  const bool a_hi = wid < MB - kDmaWaves * S::kALo;  // takes kAHi copies (else kALo)

  auto issue = [&](int step, int buf) {
    uint8_t* stg = smem + buf * S::kStageBytes;
    const SV_GLOBAL uint16_t* wstep = W + static_cast<size_t>(step) * kBK * ldw + w_src;
#pragma unroll
    for (int u = 0; u < S::kWCopies; ++u)
      copy16_to_lds<true>(wstep + 2 * u * ldw, stg + wid * kWWaveBytes + u * 1024);
    const SV_GLOBAL uint16_t* astep = Ablk + step * kBK;
#pragma unroll
    for (int q = 0; q < S::kAHi; ++q)
      if (q < S::kALo || a_hi) copy16_to_lds(astep + a_src[q], stg + kWStageBytes + (wid + kDmaWaves * q) * 1024);
  };

  // Operand reads: W slice i at w_rd + i*512, A block mb at a_rd + mb*1024.
  const int w_rd = wid * kWWaveBytes + 8 * lane;
  const int a_rd = kWStageBytes + 16 * lane;

  f32x4_t acc[MB][4];
#pragma unroll
  for (int mb = 0; mb < MB; ++mb)
#pragma unroll
    for (int j = 0; j < 4; ++j) acc[mb][j] = f32x4_t{0.f, 0.f, 0.f, 0.f};

  const int last = nsteps - 1;
#pragma unroll
  for (int p = 0; p < kDmaStages - 1; ++p) issue(p < last ? p : last, p);

  int buf = 0;
  int nbuf = kDmaStages - 1;
  for (int s = 0; s < nsteps; ++s) {
    // this wave's copies for step s are done once at most the later stages' are pending
    if (a_hi)
      wait_vmcnt<(kDmaStages - 2) * (S::kWCopies + S::kAHi)>();
    else
      wait_vmcnt<(kDmaStages - 2) * (S::kWCopies + S::kALo)>();
    lds_barrier();
    // operand reads first, so that their latency overlaps the copy issue
    const uint8_t* stg = smem + buf * S::kStageBytes;
    uint64_t wr[8];
#pragma unroll
    for (int i = 0; i < 8; ++i) wr[i] = *reinterpret_cast<const uint64_t*>(stg + w_rd + i * 512);
    constexpr int kAF = 3;  // A operands in flight
    Vec16 af[kAF];
#pragma unroll
    for (int q = 0; q < kAF; ++q) af[q] = *reinterpret_cast<const Vec16*>(stg + a_rd + q * 1024);
    // every step issues its copies (past the end: the last step again, into a free buffer)
    issue(s + kDmaStages - 1 < last ? s + kDmaStages - 1 : last, nbuf);

    bf16x8_t b[4];
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const uint32_t sel = (j & 1) ? 0x07060302u : 0x05040100u;
      Vec16 o;
#pragma unroll
      for (int d = 0; d < 4; ++d) {
        const uint32_t lo = static_cast<uint32_t>(wr[2 * d] >> (32 * (j >> 1)));
        const uint32_t hi = static_cast<uint32_t>(wr[2 * d + 1] >> (32 * (j >> 1)));
        o.w[d] = __builtin_amdgcn_perm(hi, lo, sel);
      }
      b[j] = __builtin_bit_cast(bf16x8_t, o);
    }
    // m-block mb's four MFMAs, then the read of the A operand kAF blocks ahead
#pragma unroll
    for (int mb = 0; mb < MB; ++mb) {
      const bf16x8_t a = __builtin_bit_cast(bf16x8_t, af[mb % kAF]);
#pragma unroll
      for (int j = 0; j < 4; ++j) acc[mb][j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b[j], acc[mb][j], 0, 0, 0);
      if (mb + kAF < MB) af[mb % kAF] = *reinterpret_cast<const Vec16*>(stg + a_rd + (mb + kAF) * 1024);
    }
#pragma unroll
    for (int mb = 0; mb < MB; ++mb) {
      __builtin_amdgcn_sched_group_barrier(0x008, 4, 0);  // four MFMAs
      if (mb + kAF < MB) __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);  // one LDS read
    }
    buf = (buf + 1 == kDmaStages) ? 0 : buf + 1;
    nbuf = (nbuf + 1 == kDmaStages) ? 0 : nbuf + 1;
  }
  // no copy may still be writing this workgroup's LDS when it exits
  wait_vmcnt<0>();

  if (part != nullptr) {
    // Softmax partials of the verification that follows: per row, the (max, sum of
    // 2^((l - max) c)) pair of this workgroup's 512 columns, from the accumulators as they
    // are stored.  The 16 lanes of a k group (one DPP row) hold a row's 64 columns of this
    // wave: its maximum by DPP max steps (lane 15 of the row), broadcast along the row by
    // one more DPP move, then four exponentials per lane and DPP sums; the eight waves'
    // pairs are merged in wave order through LDS.
    lds_barrier();  // every wave has read its last stage: the ring's LDS is free
    float2* sp = reinterpret_cast<float2*>(smem);  // [wave][16 * MB rows]
    const bool col_ok = n_lane < V;                // four whole columns (V % 8 == 0)
#pragma unroll
    for (int mb = 0; mb < MB; ++mb)
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        float x = -INFINITY;
        if (col_ok) x = fmaxf(fmaxf(acc[mb][0][i], acc[mb][1][i]), fmaxf(acc[mb][2][i], acc[mb][3][i]));
        x = fmaxf(x, dpp_f<kDppShr1>(-INFINITY, x));
        x = fmaxf(x, dpp_f<kDppShr2>(-INFINITY, x));
        x = fmaxf(x, dpp_f<kDppShr4>(-INFINITY, x));
        x = fmaxf(x, dpp_f<kDppShr8>(-INFINITY, x));
        const float pm = dpp_f<kDppRowBcast15>(0.f, x);  // lane 15 of the row, to the whole row
        const float pmc = pm * c;
        float ps = 0.f;
        if (col_ok) {
#pragma unroll
          for (int j = 0; j < 4; ++j) ps += fast_exp2(fmaf(acc[mb][j][i], c, -pmc));
        }
        ps += dpp_f<kDppShr1>(0.f, ps);
        ps += dpp_f<kDppShr2>(0.f, ps);
        ps += dpp_f<kDppShr4>(0.f, ps);
        ps += dpp_f<kDppShr8>(0.f, ps);
        if ((lane & 15) == 15) sp[wid * (16 * MB) + mb * 16 + kg * 4 + i] = make_float2(pm, ps);
      }
    lds_barrier();
    for (int t = tid; t < 16 * MB; t += kDmaThreads) {
      if (m0 + t >= M) break;
      float pm = -INFINITY, ps = 0.f;
      for (int w = 0; w < kDmaWaves; ++w) {
        const float2 q = sp[w * (16 * MB) + t];
        merge_max_sum(pm, ps, q.x, q.y, c);
      }
      part[static_cast<size_t>(m0 + t) * gridDim.x + blockIdx.x] =
          (static_cast<uint64_t>(__float_as_uint(pm)) << 32) | __float_as_uint(ps);
    }
  }

  if (n_lane >= V) return;
#pragma unroll
  for (int mb = 0; mb < MB; ++mb)
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int row = m0 + mb * 16 + kg * 4 + i;
      if (row < M)
        *reinterpret_cast<float4*>(C + static_cast<size_t>(row) * ldw + n_lane) =
            make_float4(acc[mb][0][i], acc[mb][1][i], acc[mb][2][i], acc[mb][3][i]);
    }
}

template <int MB>
static hipError_t launch_dma(const uint16_t* A, const uint16_t* W, float* C, int M, int H, int V, int gy,
                             uint64_t* part, float c, hipStream_t st) {
  static bool attr_set[64] = {};
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess) return hipErrorInvalidDevice;
  if (dev < 64 && !attr_set[dev]) {
    const hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void*>(&lmhead_gemm_dma_kernel<MB>),
                                             hipFuncAttributeMaxDynamicSharedMemorySize, DmaShape<MB>::kLdsBytes);
    if (e != hipSuccess) return e;
    attr_set[dev] = true;
  }
  hipLaunchKernelGGL(lmhead_gemm_dma_kernel<MB>, dim3((V + kDmaBN - 1) / kDmaBN, gy), dim3(kDmaThreads),
                     DmaShape<MB>::kLdsBytes, st, A, W, C, M, H, V, part, c);
  return hipGetLastError();
}

template <bool VEC>
static void launch_mb(const uint16_t* A, const uint16_t* W, float* C, int M, int H, int V, hipStream_t st) {
  const int mblocks = (M + 15) / 16;
  const int gx = (V + kBN - 1) / kBN;
  if (mblocks <= 4) {
    hipLaunchKernelGGL((lmhead_gemm_kernel<4, VEC>), dim3(gx, 1), dim3(kGemmThreads), 0, st, A, W, C, M, H, V);
  } else if (mblocks <= 8) {
    hipLaunchKernelGGL((lmhead_gemm_kernel<8, VEC>), dim3(gx, 1), dim3(kGemmThreads), 0, st, A, W, C, M, H, V);
  } else {
    const int gy = (mblocks + 11) / 12;
    hipLaunchKernelGGL((lmhead_gemm_kernel<12, VEC>), dim3(gx, gy), dim3(kGemmThreads), 0, st, A, W, C, M, H, V);
  }
}

bool lmhead_gemm_direct(const void* w, const float* logits, int V) {
  // 16-byte copies of W need 16-byte aligned rows; 16-byte logits stores need 16-byte rows
  return V % 8 == 0 && (reinterpret_cast<uintptr_t>(w) & 15) == 0 && (reinterpret_cast<uintptr_t>(logits) & 15) == 0;
}

hipError_t launch_lmhead_gemm(const void* hidden, const void* w, float* logits, int M, int H, int V,
                              hipStream_t st, uint64_t* part, float c) {
  const auto* A = static_cast<const uint16_t*>(hidden);
  const auto* Wp = static_cast<const uint16_t*>(w);
  const uintptr_t wa = reinterpret_cast<uintptr_t>(w), ca = reinterpret_cast<uintptr_t>(logits);
  if (lmhead_gemm_direct(w, logits, V)) {
    const int mblocks = (M + 15) / 16;
    if (mblocks <= 4) return launch_dma<4>(A, Wp, logits, M, H, V, 1, part, c, st);
    if (mblocks <= 8) return launch_dma<8>(A, Wp, logits, M, H, V, 1, part, c, st);
    return launch_dma<12>(A, Wp, logits, M, H, V, (mblocks + 11) / 12, part, c, st);
  }
  if (part != nullptr) return hipErrorInvalidValue;  // partials come from the direct kernel only
  // 8-byte W loads need 8-byte aligned rows
  if (V % 4 == 0 && (wa & 7) == 0 && (ca & 15) == 0)
    launch_mb<true>(A, Wp, logits, M, H, V, st);
  else
    launch_mb<false>(A, Wp, logits, M, H, V, st);
  return hipGetLastError();
}

}  // namespace sv
