// On-device token plug ("Accelerating Sonar through speculation", section "MTP schedule for
// one token"): after verification, each sequence's emitted tokens are appended to its token
// history and its length advanced on the GPU, so the next step can be set up without
// reading the accepted lengths back to the host.

#include "sv_device.hpp"
#include "sv_launch.hpp"

namespace sv {

constexpr int kPlugThreads = 256;

// One wave per sequence: lane i moves emitted token i (W <= 64).  Every lane reads the
// sequence's length before lane 0 rewrites it; the rewrite depends on the value read, so
// it cannot overtake the read.
__global__ __launch_bounds__(kPlugThreads) void plug_kernel(PlugParams P) {
  const int lane = threadIdx.x & (kWave - 1);
  const int64_t b = static_cast<int64_t>(blockIdx.x) * (kPlugThreads / kWave) + (threadIdx.x / kWave);
  if (b >= P.B) return;  // b is the same for the whole wave
  const int n = P.accept_len[b];
  const int len = P.seq_len[b];
  const bool ok = n >= 0 && n < P.W && len >= 0 && len <= P.cap;
  if (ok && lane <= n) {
    const int32_t t = P.tokens[b * P.W + lane];
    const int64_t pos = static_cast<int64_t>(len) + lane;
    if (pos < P.cap) P.history[b * P.cap + pos] = t;
    if (lane == n && P.next_token) P.next_token[b] = t;
  }
  if (lane == 0) {
    int st = 2;
    if (ok) {
      const int64_t end = static_cast<int64_t>(len) + n + 1;
      st = end > P.cap ? 1 : 0;
      P.seq_len[b] = static_cast<int32_t>(end > P.cap ? P.cap : end);
    }
    if (P.status) P.status[b] = st;
  }
}

hipError_t launch_plug(const PlugParams& P, hipStream_t st) {
  constexpr int kSeqPerBlock = kPlugThreads / kWave;
  const int64_t grid = (P.B + kSeqPerBlock - 1) / kSeqPerBlock;
  hipLaunchKernelGGL(plug_kernel, dim3(static_cast<unsigned>(grid)), dim3(kPlugThreads), 0, st, P);
  return hipGetLastError();
}

}  // namespace sv
