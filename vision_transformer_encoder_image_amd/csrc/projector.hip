// PatchMerger projector pieces (DeepSeek-V4-Flash-Vision-NVFP4 model page: the
// projector merges every 2x2 group of encoder patches and maps the 4*d features
// to the LLM width; its parameter count gives a norm with weight and bias on the
// d patch features and two biased linear maps).
//
// ln_gather_kernel: LayerNorm of every patch row (fp32 math, population
// variance, eps inside the root, fp32 weight and bias) written straight into
// its slot of the merged-token matrix G [sum P/4, 4d]: patch (r, c) of an image
// goes to token (r/2)*(gw/2) + c/2 of that image, feature block 2*(r%2) + c%2
// (top-left, top-right, bottom-left, bottom-right, as the aligner's gather).
// One wave per row: the row stays in registers (16-byte chunks, at most
// kLnMaxChunks per lane), so the mean and the centred variance are two wave
// reductions.  HBM-bound: the row is read once and written once.
// The two linear maps run on the bf16 MFMA GEMM with its bias / bias+GELU
// epilogues.
#include "common.h"

namespace {

constexpr int kLnWaves = 4;
constexpr int kLnMaxChunks = 8;  // d <= 64 lanes * 8 chunks * 8 = 4096

__global__ __launch_bounds__(64 * kLnWaves) void ln_gather_kernel(
    const bf16* __restrict__ x, VarlenDesc desc, int d, const float* __restrict__ w,
    const float* __restrict__ b, float eps, bf16* __restrict__ G) {
  const int p = blockIdx.x * kLnWaves + (threadIdx.x >> 6);
  if (p >= desc.total) return;
  const int lane = threadIdx.x & 63;
  const int nch = d / 8;
  const bf16* row = x + (int64_t)p * d;
  float v[kLnMaxChunks][8];
  float s = 0.f;
#pragma unroll
  for (int c = 0; c < kLnMaxChunks; ++c) {
    const int ch = lane + 64 * c;
    if (ch < nch) {
      const bf16x8 q = __builtin_bit_cast(bf16x8, ld16(row + ch * 8));
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        v[c][e] = bf2f(q[e]);
        s += v[c][e];
      }
    } else {
#pragma unroll
      for (int e = 0; e < 8; ++e) v[c][e] = 0.f;
    }
  }
  const float mean = wave_sum(s) / (float)d;
  float ss = 0.f;
#pragma unroll
  for (int c = 0; c < kLnMaxChunks; ++c) {
    if (lane + 64 * c < nch) {
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        const float t = v[c][e] - mean;
        ss += t * t;
      }
    }
  }
  const float rstd = 1.0f / sqrtf(wave_sum(ss) / (float)d + eps);

  const int img = find_image(desc, p);
  const int q = p - desc.cu_seqlens[img];
  const int gw = desc.grid_w[img];
  const int r = q / gw, col = q % gw;
  const int64_t tok = desc.cu_seqlens[img] / 4 + (r / 2) * (gw / 2) + col / 2;
  bf16* dst = G + tok * 4 * d + (2 * (r % 2) + col % 2) * d;
#pragma unroll
  for (int c = 0; c < kLnMaxChunks; ++c) {
    const int ch = lane + 64 * c;
    if (ch < nch) {
      const f32x4 w0 = *reinterpret_cast<const f32x4*>(w + ch * 8);
      const f32x4 w1 = *reinterpret_cast<const f32x4*>(w + ch * 8 + 4);
      const f32x4 b0 = *reinterpret_cast<const f32x4*>(b + ch * 8);
      const f32x4 b1 = *reinterpret_cast<const f32x4*>(b + ch * 8 + 4);
      bf16x8 o;
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        o[e] = f2bf((v[c][e] - mean) * rstd * w0[e] + b0[e]);
        o[e + 4] = f2bf((v[c][e + 4] - mean) * rstd * w1[e] + b1[e]);
      }
      st16(dst + ch * 8, __builtin_bit_cast(u32x4, o));
    }
  }
}

}  // namespace

hipError_t launch_ln_gather(const void* x, const VarlenDesc& d, int dim, const float* w,
                            const float* b, float eps, void* G, hipStream_t s) {
  if (dim % 8 || dim > 64 * kLnMaxChunks * 8) return hipErrorInvalidValue;
  if (d.total == 0) return hipSuccess;
  const unsigned blocks = (unsigned)((d.total + kLnWaves - 1) / kLnWaves);
  ln_gather_kernel<<<blocks, 64 * kLnWaves, 0, s>>>((const bf16*)x, d, dim, w, b, eps, (bf16*)G);
  return hipGetLastError();
}
