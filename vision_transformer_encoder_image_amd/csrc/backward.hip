// Backward of the MLP half of an encoder block (NeMo Automodel vision page,
// DeepseekV4VisionBlock: y = x + mlp(norm2(x)), the MLP a bias-free SwiGLU;
// PR #3772 lists backward over ragged grids among the tested paths).  The
// GEMMs of the gradient run on the bf16 MFMA GEMM, whose operands are
// K-contiguous: the passes below produce the transposed operands, the SwiGLU
// gradient and the RMSNorm gradient.  All deterministic (fixed-order sums).
#include "common.h"

namespace {

constexpr int kThreads = 256;

// fp32 -> bf16, 4 elements per thread
__global__ __launch_bounds__(kThreads) void cast_bf16_kernel(const float* __restrict__ src,
                                                             int64_t n4, bf16* __restrict__ dst) {
  const int64_t i = (int64_t)blockIdx.x * kThreads + threadIdx.x;
  if (i >= n4) return;
  const f32x4 v = *reinterpret_cast<const f32x4*>(src + 4 * i);
  bf16x4 o;
#pragma unroll
  for (int e = 0; e < 4; ++e) o[e] = f2bf(v[e]);
  *reinterpret_cast<bf16x4*>(dst + 4 * i) = o;
}

// dst[c][j] = src[j][c] for j < R, 0 for R <= j < cols_out; c < C.  src rows
// have ld_src elements, dst rows ld_dst.  One 64x64 tile per block through LDS
// (rows padded by 8 elements against bank conflicts of the scattered writes).
// An fp32 source is rounded to bf16 on the way, and then also written row-major
// to copy [R, C] (the cast and the transpose of one operand in one pass).
constexpr int kTT = 64;
template <typename TS>
__global__ __launch_bounds__(kThreads) void transpose_bf16_kernel(
    const TS* __restrict__ src, int64_t R, int64_t C, int64_t ld_src, bf16* __restrict__ dst,
    int64_t cols_out, int64_t ld_dst, bf16* __restrict__ copy) {
  __shared__ bf16 tile[kTT][kTT + 8];
  const int64_t j0 = (int64_t)blockIdx.x * kTT;  // source row block = dst column block
  const int64_t c0 = (int64_t)blockIdx.y * kTT;  // source column block = dst row block
  // load: 64 rows x 8 chunks of 8 elements; two chunks per thread
#pragma unroll
  for (int k = 0; k < 2; ++k) {
    const int q = threadIdx.x + k * kThreads;
    const int r = q >> 3, ch = q & 7;
    const int64_t j = j0 + r, c = c0 + ch * 8;
    bf16x8 v;
    if (j < R && c + 8 <= C) {
      if constexpr (sizeof(TS) == 2) {
        v = __builtin_bit_cast(bf16x8, ld16(src + j * ld_src + c));
      } else {
        const f32x4 lo = *reinterpret_cast<const f32x4*>(src + j * ld_src + c);
        const f32x4 hi = *reinterpret_cast<const f32x4*>(src + j * ld_src + c + 4);
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          v[e] = f2bf(lo[e]);
          v[e + 4] = f2bf(hi[e]);
        }
        st16(copy + j * C + c, __builtin_bit_cast(u32x4, v));
      }
    } else {
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        if constexpr (sizeof(TS) == 2) {
          v[e] = (j < R && c + e < C) ? src[j * ld_src + c + e] : f2bf(0.f);
        } else {
          v[e] = (j < R && c + e < C) ? f2bf(src[j * ld_src + c + e]) : f2bf(0.f);
          if (j < R && c + e < C) copy[j * C + c + e] = v[e];
        }
      }
    }
#pragma unroll
    for (int e = 0; e < 8; ++e) tile[ch * 8 + e][r] = v[e];
  }
  __syncthreads();
  // store: dst row c0 + rr, columns j0 .. j0+63
#pragma unroll
  for (int k = 0; k < 2; ++k) {
    const int q = threadIdx.x + k * kThreads;
    const int rr = q >> 3, ch = q & 7;
    const int64_t c = c0 + rr, j = j0 + ch * 8;
    if (c >= C || j >= cols_out) continue;
    bf16x8 v;
#pragma unroll
    for (int e = 0; e < 8; ++e) v[e] = tile[rr][ch * 8 + e];
    if (j + 8 <= cols_out) {
      st16(dst + c * ld_dst + j, __builtin_bit_cast(u32x4, v));
    } else {
#pragma unroll
      for (int e = 0; e < 8; ++e)
        if (j + e < cols_out) dst[c * ld_dst + j + e] = v[e];
    }
  }
}

// SwiGLU gradient: g, u = gu[:, :h], gu[:, hp:hp+h] (fp32, rows of 2 hp, hp >= h
// the padded half width), da (fp32, [rows, h]) -> a = silu(g) u (bf16, [rows, h]),
// dg = da u (s + g s (1 - s)), du = da g s (bf16, side by side in dgdu [rows, 2 hp],
// columns h .. hp-1 of each half written zero); s = sigmoid(g)
__global__ __launch_bounds__(kThreads) void swiglu_bwd_kernel(const float* __restrict__ gu,
                                                              const float* __restrict__ da,
                                                              int64_t rows, int h, int hp,
                                                              bf16* __restrict__ a,
                                                              bf16* __restrict__ dgdu) {
  const int64_t i = (int64_t)blockIdx.x * kThreads + threadIdx.x;  // group of 4 columns
  const int h4 = hp / 4;
  if (i >= rows * h4) return;
  const int64_t r = i / h4;
  const int c = (int)(i % h4) * 4;
  if (c >= h) {  // padding of the K dimension of the dn GEMM
    const bf16x4 z = {f2bf(0.f), f2bf(0.f), f2bf(0.f), f2bf(0.f)};
    *reinterpret_cast<bf16x4*>(dgdu + r * 2 * hp + c) = z;
    *reinterpret_cast<bf16x4*>(dgdu + r * 2 * hp + hp + c) = z;
    return;
  }
  const f32x4 g = *reinterpret_cast<const f32x4*>(gu + r * 2 * hp + c);
  const f32x4 u = *reinterpret_cast<const f32x4*>(gu + r * 2 * hp + hp + c);
  const f32x4 d = *reinterpret_cast<const f32x4*>(da + r * h + c);
  bf16x4 av, dgv, duv;
#pragma unroll
  for (int e = 0; e < 4; ++e) {
    const float s = 1.0f / (1.0f + __expf(-g[e]));
    av[e] = f2bf(g[e] * s * u[e]);
    dgv[e] = f2bf(d[e] * u[e] * (s + g[e] * s * (1.0f - s)));
    duv[e] = f2bf(d[e] * g[e] * s);
  }
  *reinterpret_cast<bf16x4*>(a + r * h + c) = av;
  *reinterpret_cast<bf16x4*>(dgdu + r * 2 * hp + c) = dgv;
  *reinterpret_cast<bf16x4*>(dgdu + r * 2 * hp + hp + c) = duv;
}

// RMSNorm gradient plus the residual: per row, r = (mean(x^2) + eps)^-1/2,
// dx = dy + r (w dn) - x r^3 mean(w dn x); the rows of block b also add
// dn x r into partial[b][:] (fixed order: waves in turn, rows in turn).
constexpr int kNbRows = 16;       // rows per block (enough blocks to fill the CUs)
constexpr int kNbWaves = 8;
constexpr int kNbMaxChunks = 8;   // 4-column chunks per lane: d <= 64 * 4 * 8 = 2048
template <int NCH>  // 4-column chunks per lane (d <= 256 * NCH)
__global__ __launch_bounds__(64 * kNbWaves) void rmsnorm_bwd_kernel(
    const float* __restrict__ x, const float* __restrict__ w, const float* __restrict__ dn,
    const float* __restrict__ dy, int64_t rows, int d, float eps, float* __restrict__ dx,
    float* __restrict__ partial) {
  __shared__ float s_part[kNbWaves / 2][2048];
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int nch = d / 4;
  f32x4 acc[NCH];
#pragma unroll
  for (int k = 0; k < NCH; ++k) acc[k] = f32x4{};
  const int64_t r0 = (int64_t)blockIdx.x * kNbRows;
  for (int rr = wave; rr < kNbRows; rr += kNbWaves) {
    const int64_t r = r0 + rr;
    if (r >= rows) break;
    // every load of the row first (x, dn, the residual dy, w), then the two
    // row sums, then the stores
    f32x4 xv[NCH], nv[NCH], yv[NCH], gv[NCH];
#pragma unroll
    for (int k = 0; k < NCH; ++k) {
      const int ch = lane + 64 * k;
      xv[k] = nv[k] = yv[k] = f32x4{};
      if (ch < nch) {
        xv[k] = *reinterpret_cast<const f32x4*>(x + r * d + 4 * ch);
        nv[k] = *reinterpret_cast<const f32x4*>(dn + r * d + 4 * ch);
        if (dy) yv[k] = *reinterpret_cast<const f32x4*>(dy + r * d + 4 * ch);
      }
    }
    float ss = 0.f, sd = 0.f;
#pragma unroll
    for (int k = 0; k < NCH; ++k) {
      const int ch = lane + 64 * k;
      if (ch < nch) {
        const f32x4 wv = *reinterpret_cast<const f32x4*>(w + 4 * ch);
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          gv[k][e] = wv[e] * nv[k][e];
          ss += xv[k][e] * xv[k][e];
          sd += gv[k][e] * xv[k][e];
        }
      }
    }
    const float rs = 1.0f / sqrtf(wave_sum(ss) / (float)d + eps);
    const float coef = rs * rs * rs * wave_sum(sd) / (float)d;
#pragma unroll
    for (int k = 0; k < NCH; ++k) {
      const int ch = lane + 64 * k;
      if (ch < nch) {
        f32x4 o;
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          o[e] = yv[k][e] + rs * gv[k][e] - xv[k][e] * coef;
          acc[k][e] += nv[k][e] * xv[k][e] * rs;
        }
        *reinterpret_cast<f32x4*>(dx + r * d + 4 * ch) = o;
      }
    }
  }
  // the waves' column sums, combined in a fixed order: waves w and w + 4 first
  // (through LDS), then the four pairs
  if (wave >= kNbWaves / 2) {
#pragma unroll
    for (int k = 0; k < NCH; ++k) {
      const int ch = lane + 64 * k;
      if (ch < nch) *reinterpret_cast<f32x4*>(&s_part[wave - kNbWaves / 2][4 * ch]) = acc[k];
    }
  }
  __syncthreads();
  if (wave < kNbWaves / 2) {
#pragma unroll
    for (int k = 0; k < NCH; ++k) {
      const int ch = lane + 64 * k;
      if (ch < nch) {
        f32x4 t = *reinterpret_cast<const f32x4*>(&s_part[wave][4 * ch]);
        t += acc[k];
        *reinterpret_cast<f32x4*>(&s_part[wave][4 * ch]) = t;
      }
    }
  }
  __syncthreads();
  for (int c = threadIdx.x; c < d; c += 64 * kNbWaves) {
    float t = 0.f;
#pragma unroll
    for (int v = 0; v < kNbWaves / 2; ++v) t += s_part[v][c];
    partial[(int64_t)blockIdx.x * d + c] = t;
  }
}

// out[c] = sum over b < nb of partial[b][c]: block = 64 columns x 16 row
// groups; group q sums rows q, q+16, ... in order, then the groups are added
// in order through LDS (a fixed summation order)
constexpr int kCsGroups = 16;
__global__ __launch_bounds__(64 * kCsGroups) void colsum_kernel(const float* __restrict__ partial,
                                                                int nb, int d,
                                                                float* __restrict__ out) {
  __shared__ float s[kCsGroups][64];
  const int lane = threadIdx.x & 63, q = threadIdx.x >> 6;
  const int c = blockIdx.x * 64 + lane;
  float t = 0.f;
  if (c < d)
    for (int b = q; b < nb; b += kCsGroups) t += partial[(int64_t)b * d + c];
  s[q][lane] = t;
  __syncthreads();
  if (q == 0 && c < d) {
    float u = 0.f;
#pragma unroll
    for (int g = 0; g < kCsGroups; ++g) u += s[g][lane];
    out[c] = u;
  }
}

unsigned blocks_of(int64_t n) { return (unsigned)((n + kThreads - 1) / kThreads); }

}  // namespace

hipError_t launch_cast_bf16(const float* src, int64_t n, void* dst, hipStream_t s) {
  if (n % 4) return hipErrorInvalidValue;
  if (n == 0) return hipSuccess;
  cast_bf16_kernel<<<blocks_of(n / 4), kThreads, 0, s>>>(src, n / 4, (bf16*)dst);
  return hipGetLastError();
}

hipError_t launch_transpose_bf16(const void* src, int64_t R, int64_t C, int64_t ld_src, void* dst,
                                 int64_t cols_out, int64_t ld_dst, hipStream_t s) {
  if (R <= 0 || C <= 0 || cols_out <= 0) return hipSuccess;
  if (cols_out > ld_dst || ld_src < C || ld_src % 8 || ld_dst % 8) return hipErrorInvalidValue;
  const dim3 grid((unsigned)((cols_out + kTT - 1) / kTT), (unsigned)((C + kTT - 1) / kTT));
  transpose_bf16_kernel<bf16><<<grid, kThreads, 0, s>>>((const bf16*)src, R, C, ld_src,
                                                        (bf16*)dst, cols_out, ld_dst, nullptr);
  return hipGetLastError();
}

hipError_t launch_cast_transpose(const float* src, int64_t R, int64_t C, void* copy, void* dst,
                                 int64_t cols_out, int64_t ld_dst, hipStream_t s) {
  if (R <= 0 || C <= 0 || cols_out <= 0) return hipSuccess;
  if (cols_out > ld_dst || C % 8 || ld_dst % 8) return hipErrorInvalidValue;
  const dim3 grid((unsigned)((cols_out + kTT - 1) / kTT), (unsigned)((C + kTT - 1) / kTT));
  transpose_bf16_kernel<float><<<grid, kThreads, 0, s>>>(src, R, C, C, (bf16*)dst, cols_out,
                                                         ld_dst, (bf16*)copy);
  return hipGetLastError();
}

hipError_t launch_swiglu_bwd(const float* gu, const float* da, int64_t rows, int h, int hp,
                             void* a, void* dgdu, hipStream_t s) {
  if (h % 4 || hp % 4 || hp < h) return hipErrorInvalidValue;
  if (rows == 0) return hipSuccess;
  swiglu_bwd_kernel<<<blocks_of(rows * (hp / 4)), kThreads, 0, s>>>(gu, da, rows, h, hp, (bf16*)a,
                                                                    (bf16*)dgdu);
  return hipGetLastError();
}

int rmsnorm_bwd_blocks(int64_t rows) { return (int)((rows + kNbRows - 1) / kNbRows); }

hipError_t launch_rmsnorm_bwd(const float* x, const float* w, const float* dn, const float* dy,
                              int64_t rows, int d, float eps, float* dx, float* partial,
                              float* dw, hipStream_t s) {
  if (d % 4 || d > 64 * 4 * kNbMaxChunks) return hipErrorInvalidValue;
  if (rows == 0) return hipSuccess;
  const int nb = rmsnorm_bwd_blocks(rows);
  if (d <= 256 * 4)
    rmsnorm_bwd_kernel<4><<<nb, 64 * kNbWaves, 0, s>>>(x, w, dn, dy, rows, d, eps, dx, partial);
  else
    rmsnorm_bwd_kernel<kNbMaxChunks><<<nb, 64 * kNbWaves, 0, s>>>(x, w, dn, dy, rows, d, eps, dx,
                                                                  partial);
  colsum_kernel<<<(unsigned)((d + 63) / 64), 64 * kCsGroups, 0, s>>>(partial, nb, d, dw);
  return hipGetLastError();
}
