// LM-head projection on the matrix cores: logits[M, V] (fp32) = hidden[M, H] (bf16) @
// W[H, V] (bf16, row-major, vocabulary contiguous).  The EAGLE / MTP heads of
// "Accelerating Sonar through speculation" (sections "EAGLE" and "Training MTP heads")
// share the target's LM head, about 2 GB in bf16 for a 70B model; at the verification
// shapes (M = B(k+1) a few hundred rows) the product streams W from HBM once and is
// bandwidth-bound, so the kernel is built around one pass over W.
//
// Workgroup tile: BM = 16*MB rows x 256 columns, k-step 64, 4 waves of 64 columns each.
// v_mfma_f32_16x16x32_bf16 wants each lane to hold 8 consecutive k of one column of W,
// but W is row-major in k.  Each thread therefore loads an 8 (k) x 8 (n) block of W with
// 16-byte loads, transposes it in registers with byte permutes, and writes eight
// k-contiguous 16-byte vectors into LDS (row stride 144 B so the MFMA operand reads are
// bank-conflict free).  The hidden-state tile goes to LDS as is.  The next k-step's
// global loads are issued before the current step's MFMAs.

#include "sv_device.hpp"
#include "sv_launch.hpp"

namespace sv {

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef float f32x4_t __attribute__((ext_vector_type(4)));

constexpr int kGemmThreads = 256;
constexpr int kBN = 256;         // columns per workgroup
constexpr int kBK = 64;          // k per step
constexpr int kLdsStride = 72;   // bf16 per LDS row: 64 + 8 padding

__device__ __forceinline__ bf16x8_t as_bf16x8(const Vec16& v) {
  return __builtin_bit_cast(bf16x8_t, v);
}

template <int MB>
__global__ __launch_bounds__(kGemmThreads) void lmhead_gemm_kernel(const uint16_t* __restrict__ A,
                                                                   const uint16_t* __restrict__ W,
                                                                   float* __restrict__ C, int M, int H,
                                                                   int V, int vec_ok) {
  constexpr int BM = MB * 16;
  constexpr int ACH = (BM * 8 + kGemmThreads - 1) / kGemmThreads;  // 16-B chunks of A per thread
  __shared__ __attribute__((aligned(16))) uint16_t sW[kBN * kLdsStride];
  __shared__ __attribute__((aligned(16))) uint16_t sA[BM * kLdsStride];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wid = tid >> 6;
  const int n0 = blockIdx.x * kBN;
  const int m0 = blockIdx.y * BM;
  const int kg = tid & 7;   // k group of this thread's 8x8 block of W
  const int ng = tid >> 3;  // n group (0..31)
  const int wn = n0 + ng * 8;

  Vec16 wreg[8];
  Vec16 areg[ACH];
  f32x4_t acc[MB][4];
#pragma unroll
  for (int mb = 0; mb < MB; ++mb)
#pragma unroll
    for (int nb = 0; nb < 4; ++nb) acc[mb][nb] = f32x4_t{0.f, 0.f, 0.f, 0.f};

  auto load_tiles = [&](int k0) {
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const uint16_t* p = W + static_cast<size_t>(k0 + kg * 8 + i) * V + wn;
      if (vec_ok && wn + 8 <= V) {
        wreg[i] = *reinterpret_cast<const Vec16*>(p);
      } else {
        Vec16 v{};
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          const uint32_t x = (wn + e < V) ? p[e] : 0u;
          v.w[e >> 1] |= (e & 1) ? (x << 16) : x;
        }
        wreg[i] = v;
      }
    }
#pragma unroll
    for (int q = 0; q < ACH; ++q) {
      const int ch = tid + kGemmThreads * q;
      const int row = ch >> 3;
      const int m = m0 + row;
      if (ch < BM * 8 && m < M)
        areg[q] = *reinterpret_cast<const Vec16*>(A + static_cast<size_t>(m) * H + k0 + (ch & 7) * 8);
      else
        areg[q] = Vec16{};
    }
  };

  auto store_tiles = [&]() {
#pragma unroll
    for (int cc = 0; cc < 8; ++cc) {
      const uint32_t sel = (cc & 1) ? 0x07060302u : 0x05040100u;
      Vec16 o;
#pragma unroll
      for (int d = 0; d < 4; ++d)
        o.w[d] = __builtin_amdgcn_perm(wreg[2 * d + 1].w[cc >> 1], wreg[2 * d].w[cc >> 1], sel);
      *reinterpret_cast<Vec16*>(&sW[(ng * 8 + cc) * kLdsStride + kg * 8]) = o;
    }
#pragma unroll
    for (int q = 0; q < ACH; ++q) {
      const int ch = tid + kGemmThreads * q;
      if (ch < BM * 8) *reinterpret_cast<Vec16*>(&sA[(ch >> 3) * kLdsStride + (ch & 7) * 8]) = areg[q];
    }
  };

  load_tiles(0);
  for (int k0 = 0; k0 < H; k0 += kBK) {
    __syncthreads();
    store_tiles();
    __syncthreads();
    if (k0 + kBK < H) load_tiles(k0 + kBK);
#pragma unroll
    for (int kk = 0; kk < 2; ++kk) {
      const int kofs = kk * 32 + (lane >> 4) * 8;
      bf16x8_t bfrag[4];
#pragma unroll
      for (int nb = 0; nb < 4; ++nb) {
        const int nl = wid * 64 + nb * 16 + (lane & 15);
        bfrag[nb] = as_bf16x8(*reinterpret_cast<const Vec16*>(&sW[nl * kLdsStride + kofs]));
      }
#pragma unroll
      for (int mb = 0; mb < MB; ++mb) {
        const bf16x8_t afrag =
            as_bf16x8(*reinterpret_cast<const Vec16*>(&sA[(mb * 16 + (lane & 15)) * kLdsStride + kofs]));
#pragma unroll
        for (int nb = 0; nb < 4; ++nb)
          acc[mb][nb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(afrag, bfrag[nb], acc[mb][nb], 0, 0, 0);
      }
    }
  }

  // D layout of the 16x16 tile: lane l holds rows 4*(l/16)+i, column l%16
#pragma unroll
  for (int mb = 0; mb < MB; ++mb)
#pragma unroll
    for (int nb = 0; nb < 4; ++nb) {
      const int col = n0 + wid * 64 + nb * 16 + (lane & 15);
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int row = m0 + mb * 16 + (lane >> 4) * 4 + i;
        if (row < M && col < V) C[static_cast<size_t>(row) * V + col] = acc[mb][nb][i];
      }
    }
}

hipError_t launch_lmhead_gemm(const void* hidden, const void* w, float* logits, int M, int H, int V,
                              hipStream_t st) {
  const int vec_ok = (V % 8 == 0) && ((reinterpret_cast<uintptr_t>(w) & 15) == 0);
  const int mblocks = (M + 15) / 16;
  const int gx = (V + kBN - 1) / kBN;
  const auto* A = static_cast<const uint16_t*>(hidden);
  const auto* Wp = static_cast<const uint16_t*>(w);
  if (mblocks <= 4) {
    hipLaunchKernelGGL(lmhead_gemm_kernel<4>, dim3(gx, 1), dim3(kGemmThreads), 0, st, A, Wp, logits, M, H, V, vec_ok);
  } else if (mblocks <= 8) {
    hipLaunchKernelGGL(lmhead_gemm_kernel<8>, dim3(gx, 1), dim3(kGemmThreads), 0, st, A, Wp, logits, M, H, V, vec_ok);
  } else {
    const int gy = (mblocks + 11) / 12;
    hipLaunchKernelGGL(lmhead_gemm_kernel<12>, dim3(gx, gy), dim3(kGemmThreads), 0, st, A, Wp, logits, M, H, V, vec_ok);
  }
  return hipGetLastError();
}

}  // namespace sv
