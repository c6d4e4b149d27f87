// Matrix-core peak probe: a measurement aid beside the roofline, not part of the method. Every
// wave runs `iters` rounds of kChains independent MFMA accumulation chains on register operands
// (no memory traffic in the loop) and writes its sums, so the measured rate is what the matrix
// cores sustain on this part and clock, to set against the datasheet peak.
#include "wbmm_device.hpp"
#include "wbmm_launch.hpp"

namespace wbmm {

namespace {

constexpr int kChains = 8;  // independent accumulators per wave (>= 4 keeps the pipe full)
constexpr int kRound = 128;  // bf16: chained steps per round

template <bool BF16>
__global__ void __launch_bounds__(kThreads) k_probe_mfma(float* out, int iters) {
  const int lane = threadIdx.x & 63;
  v4f acc[kChains];
#pragma unroll
  for (int c = 0; c < kChains; ++c) {
    const float s = (float)(c + 1) * 1e-3f;  // distinct chains: nothing to merge
    acc[c] = v4f{s, s, s, s};
  }
  // operands depend on the lane and on `iters`, so none of it is a compile-time constant
  const float av = 1.0f + (float)(lane & 7) * 1e-3f + (float)(iters & 1) * 1e-6f;
  const float bv = 1e-4f * (float)((lane >> 3) + 1);
  if constexpr (BF16) {
    const uint32_t ha = f2bf(av), hb = f2bf(bv);
    const uint32_t pa = ha | (ha << 16), pb = hb | (hb << 16);
    const u32x4 a4 = {pa, pa, pa, pa}, b4 = {pb, pb, pb, pb};
    const v8bf a = __builtin_bit_cast(v8bf, a4), b = __builtin_bit_cast(v8bf, b4);
    // rounds of kRound chained steps from a fixed accumulator, added into the running sums: the
    // loop-carried value is then a plain VGPR sum (a loop-carried MFMA accumulator is placed in
    // rotating AGPR tuples with register moves every step); 4 adds per kRound MFMAs per chain
    for (int it = 0; it < iters; it += kRound) {
      v4f t[kChains];
#pragma unroll
      for (int c = 0; c < kChains; ++c) {  // distinct starting values keep the chains apart
        const float s0 = (float)c * 1e-3f;
        t[c] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, v4f{s0, s0, s0, s0}, 0, 0, 0);
      }
#pragma unroll
      for (int k = 1; k < kRound; ++k)
#pragma unroll
        for (int c = 0; c < kChains; ++c)
          t[c] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, t[c], 0, 0, 0);
#pragma unroll
      for (int c = 0; c < kChains; ++c) acc[c] += t[c];
    }
  } else {
    for (int it = 0; it < iters; ++it)
#pragma unroll
      for (int c = 0; c < kChains; ++c) acc[c] = mfma_f32(av, bv, acc[c]);
  }
  float s = 0.f;
#pragma unroll
  for (int c = 0; c < kChains; ++c) s += acc[c][0] + acc[c][1] + acc[c][2] + acc[c][3];
  out[(size_t)blockIdx.x * kThreads + threadIdx.x] = s;
}

}  // namespace

double probe_mfma_flops(int bf16, int blocks, int iters) {
  const double per_mfma = bf16 ? 2.0 * 16 * 16 * 32 : 2.0 * 16 * 16 * 4;
  const int rounds = bf16 ? (iters + kRound - 1) / kRound * kRound : iters;  // whole bf16 rounds
  return (double)blocks * (kThreads / 64) * (double)rounds * kChains * per_mfma;
}

hipError_t launch_probe_mfma(int bf16, int blocks, int iters, float* out, hipStream_t st) {
  if (bf16) return launch_main(k_probe_mfma<true>, dim3(blocks), dim3(kThreads), 0, st, out, iters);
  return launch_main(k_probe_mfma<false>, dim3(blocks), dim3(kThreads), 0, st, out, iters);
}

}  // namespace wbmm
