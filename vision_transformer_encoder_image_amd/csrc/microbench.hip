// Measured dense-MFMA peak (a measurement aid beside the encoder's kernels): every
// wave of one 8-wave workgroup per CU issues back-to-back v_mfma_f32_32x32x16_bf16
// into four independent accumulators, with register operands that alternate
// between two random-looking bit patterns (so the matrix cores toggle as on real
// data) and no memory traffic inside the loop.  FLOPs per call: 256 workgroups x
// 8 waves x iters x 8 MFMAs x 32768.  The rate it reaches is the chip's attainable
// bf16 MFMA throughput at the clock it sustains under that load, which the
// encoder's kernels can be compared with besides the published peak.
#include "common.h"

namespace {

constexpr int kPeakWaves = 8;
constexpr int kPeakBlocks = 256;

VIT_DEV uint32_t mix(uint32_t x) {  // integer hash for operand bit patterns
  x ^= x >> 16;
  x *= 0x7feb352du;
  x ^= x >> 15;
  x *= 0x846ca68bu;
  x ^= x >> 16;
  return x;
}

__global__ __launch_bounds__(64 * kPeakWaves, 1) void mfma_peak_kernel(int iters, float* out) {
  const uint32_t t = blockIdx.x * 64 * kPeakWaves + threadIdx.x;
  u32x4 ra, rb, rc, rd;
#pragma unroll
  for (int e = 0; e < 4; ++e) {
    // keep the bf16 exponents moderate: bits 14..7 of every half in [0x3c, 0x43]
    ra[e] = (mix(t * 16 + e) & 0x807f807fu) | 0x3e003e00u;
    rb[e] = (mix(t * 16 + 4 + e) & 0x807f807fu) | 0x3e803e80u;
    rc[e] = (mix(t * 16 + 8 + e) & 0x807f807fu) | 0x3e003e00u;
    rd[e] = (mix(t * 16 + 12 + e) & 0x807f807fu) | 0x3e803e80u;
  }
  const bf16x8 a0 = __builtin_bit_cast(bf16x8, ra), b0 = __builtin_bit_cast(bf16x8, rb);
  const bf16x8 a1 = __builtin_bit_cast(bf16x8, rc), b1 = __builtin_bit_cast(bf16x8, rd);
  f32x16 acc[4] = {f32x16{}, f32x16{}, f32x16{}, f32x16{}};
  for (int i = 0; i < iters; ++i) {
#pragma unroll
    for (int j = 0; j < 4; ++j) acc[j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a0, b0, acc[j], 0, 0, 0);
#pragma unroll
    for (int j = 0; j < 4; ++j) acc[j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a1, b1, acc[j], 0, 0, 0);
  }
  float s = 0.f;
#pragma unroll
  for (int j = 0; j < 4; ++j)
#pragma unroll
    for (int e = 0; e < 16; ++e) s += acc[j][e];
  out[t] = s;
}

}  // namespace

int64_t mfma_peak_out_floats() { return (int64_t)kPeakBlocks * 64 * kPeakWaves; }

double mfma_peak_flops(int iters) {
  return (double)kPeakBlocks * kPeakWaves * iters * 8.0 * 32768.0;
}

hipError_t launch_mfma_peak(int iters, float* out, hipStream_t s) {
  if (iters <= 0) return hipErrorInvalidValue;
  mfma_peak_kernel<<<kPeakBlocks, 64 * kPeakWaves, 0, s>>>(iters, out);
  return hipGetLastError();
}
