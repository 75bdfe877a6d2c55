// fp32 GEMM on the vector ALUs (single-precision mode of the encoder):
// C[M,N] = epilogue(A[M,K] . B[N,K]^T).  64x64 tiles, K step 16, 256 threads
// each computing a 4x4 micro-tile from LDS panels stored k-major so that the
// inner loop reads float4 rows.  Any M, N, K (K-tail loads are zero-filled).
#include "common.h"

namespace {

constexpr int TM = 64, TN = 64, TK = 16;
constexpr int kThreads = 256;

VIT_DEV float silu(float g) { return g / (1.0f + expf(-g)); }

template <int EPI, bool DUAL>
__global__ __launch_bounds__(kThreads) void gemm_f32_kernel(GemmArgs g) {
  __shared__ __attribute__((aligned(16))) float sA[TK][TM];
  __shared__ __attribute__((aligned(16))) float sB[TK][TN];
  __shared__ __attribute__((aligned(16))) float sB2[DUAL ? TK : 1][DUAL ? TN : 4];

  const float* __restrict__ A = (const float*)g.A;
  const float* __restrict__ B = (const float*)g.B;
  const float* __restrict__ B2 = (const float*)g.B2;
  const int64_t M = g.M, N = g.N, K = g.K;
  const int64_t m0 = (int64_t)blockIdx.y * TM, n0 = (int64_t)blockIdx.x * TN;
  const int tid = threadIdx.x;
  const int tx = tid & 15, ty = tid >> 4;

  float acc[4][4] = {}, acc2[4][4] = {};
  for (int64_t k0 = 0; k0 < K; k0 += TK) {
    // each thread stages 4 elements of A and of B (and B2)
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const int idx = tid + e * kThreads;  // 0..1023 over a 64 x 16 panel
      const int r = idx / TK, k = idx % TK;
      const int64_t gk = k0 + k;
      const int64_t am = m0 + r, bn = n0 + r;
      sA[k][r] = (am < M && gk < K) ? A[am * g.lda + gk] : 0.f;
      sB[k][r] = (bn < N && gk < K) ? B[bn * g.ldb + gk] : 0.f;
      if (DUAL) sB2[k][r] = (bn < N && gk < K) ? B2[bn * g.ldb + gk] : 0.f;
    }
    __syncthreads();
#pragma unroll
    for (int k = 0; k < TK; ++k) {
      const float4 a = *reinterpret_cast<const float4*>(&sA[k][ty * 4]);
      const float4 b = *reinterpret_cast<const float4*>(&sB[k][tx * 4]);
      const float av[4] = {a.x, a.y, a.z, a.w};
      const float bv[4] = {b.x, b.y, b.z, b.w};
#pragma unroll
      for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j) acc[i][j] = fmaf(av[i], bv[j], acc[i][j]);
      if (DUAL) {
        const float4 c = *reinterpret_cast<const float4*>(&sB2[k][tx * 4]);
        const float cv[4] = {c.x, c.y, c.z, c.w};
#pragma unroll
        for (int i = 0; i < 4; ++i)
#pragma unroll
          for (int j = 0; j < 4; ++j) acc2[i][j] = fmaf(av[i], cv[j], acc2[i][j]);
      }
    }
    __syncthreads();
  }
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int64_t m = m0 + ty * 4 + i;
    if (m >= M) continue;
    const int64_t orow = g.rowmap ? (int64_t)g.rowmap[m] : m;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int64_t n = n0 + tx * 4 + j;
      if (n >= N) continue;
      float* c = (float*)g.C + orow * g.ldc + n;
      if (EPI == VIT_EPI_ADD_F32)
        *c = *c + acc[i][j];
      else if (DUAL)
        *c = silu(acc[i][j]) * acc2[i][j];
      else
        *c = acc[i][j];
    }
  }
}

}  // namespace

hipError_t launch_gemm_f32(int epilogue, const GemmArgs& g, hipStream_t s) {
  if (g.M == 0 || g.N == 0) return hipSuccess;
  const dim3 grid((unsigned)((g.N + TN - 1) / TN), (unsigned)((g.M + TM - 1) / TM));
  switch (epilogue) {
    case VIT_EPI_STORE:
    case VIT_EPI_STORE_F32:
      gemm_f32_kernel<VIT_EPI_STORE_F32, false><<<grid, kThreads, 0, s>>>(g);
      break;
    case VIT_EPI_ADD_F32:
      gemm_f32_kernel<VIT_EPI_ADD_F32, false><<<grid, kThreads, 0, s>>>(g);
      break;
    case VIT_EPI_SWIGLU:
      gemm_f32_kernel<VIT_EPI_SWIGLU, true><<<grid, kThreads, 0, s>>>(g);
      break;
    default:
      return hipErrorInvalidValue;
  }
  return hipGetLastError();
}
