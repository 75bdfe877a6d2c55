// One-tile-per-workgroup variant of the multi-stage bf16 MFMA GEMM (gfx950):
// C[M,N] = epilogue(A[M,K] . B[N,K]^T).  The hardware dispatcher balances the
// tiles; measured faster than the persistent kernel (gemm_pipe.hip) for the
// 128x128 tile on short-K / N=1024 shapes.
//
// Both operands are K-contiguous.  Each 64-wide K-tile of A and B is copied
// straight from global memory into LDS with global_load_lds_dwordx4 (no VGPR
// staging).  STAGES LDS buffers rotate: while the waves multiply stage kt, the
// copy of stage kt+STAGES-1 is in flight.  Waits are exact (s_waitcnt vmcnt on
// the number of younger copies) and the workgroup barrier is taken before the
// last 16-wide k-step of a stage, so the fragments of the next stage are read
// from LDS while the current stage's last MFMAs run.  Fragments are always
// fetched one k-step ahead of their MFMAs.
//
// MFMA: v_mfma_f32_32x32x16_bf16 (32 cycles for 32K flops, full rate at one
// wave per SIMD on gfx950), issued as C^T = B . A^T with the weight fragment in
// the A slot, so a lane owns 4 groups of 4 consecutive output columns of one
// row: stores are 8/16-byte vectors and the fp32 residual add reads and writes
// 16 bytes at a time.  SwiGLU tiles carry gate and up rows side by side in the
// B tile so silu(gate) * up meets in one lane; the rotary epilogue finds both
// rotate_half partners (columns n and n+16) in the same lane.
//
// LDS rows are 128 bytes (64 bf16); 16-byte chunks are XOR-swizzled by
// (row >> 1) & 7 on the global side of the copy so that fragment reads of
// consecutive rows spread over the banks.
//
// Requirements (checked by the dispatcher): K a multiple of 64 for A (A may be
// zero-padded past the true K; B's reads are then clamped to its own valid K),
// N a multiple of 4, 16-byte aligned rows.
#include "common.h"
#include "gemm_pipe.h"

namespace {

constexpr int BK = 64;
constexpr int KSTEPS = BK / 16;
constexpr int kXcds = 8;
constexpr int kGroupM = 8;

VIT_DEV int chunk_swz(int row) { return (row >> 1) & 7; }

VIT_DEV float silu_f(float g) { return g / (1.0f + __expf(-g)); }

VIT_DEV int xcd_remap(int bid, int ntiles) {
  const int per = ntiles / kXcds, rem = ntiles % kXcds;
  const int xcd = bid % kXcds, idx = bid / kXcds;
  return xcd * per + min(xcd, rem) + idx;
}

template <int BM, int BN, int WM, int WN, int STAGES, int EPI, bool DUAL>
__global__ __launch_bounds__(WM * WN * 64, 1) void gemm_tile_kernel(GemmArgs g) {
  constexpr int NW = WM * WN;
  constexpr int TM = BM / WM, TN = BN / WN;  // wave tile
  constexpr int BI = TM / 32, BJ = TN / 32;  // 32x32 blocks per wave
  constexpr int ROWS = BM + BN;              // LDS rows per stage (A then B)
  constexpr int NI = ROWS / 8 / NW;          // 1 KB copies per wave per stage
  constexpr int BNO = DUAL ? BN / 2 : BN;    // output columns per tile
  static_assert(STAGES >= 3, "stages");
  static_assert(ROWS % (8 * NW) == 0, "copy split");
  static_assert(TM % 32 == 0 && TN % 32 == 0 && (!DUAL || BJ % 2 == 0), "wave tile");
  extern __shared__ __attribute__((aligned(16))) bf16 smem[];

  const bf16* __restrict__ A = (const bf16*)g.A;
  const bf16* __restrict__ B = (const bf16*)g.B;
  const bf16* __restrict__ B2 = (const bf16*)g.B2;
  const int M = (int)g.M, N = (int)g.N, K = (int)g.K, KB = (int)g.kb;
  const int tiles_m = (M + BM - 1) / BM;
  const int tiles_n = (N + BNO - 1) / BNO;
  const int L = xcd_remap(blockIdx.x, tiles_m * tiles_n);
  const int band = kGroupM * tiles_n;
  const int first_m = (L / band) * kGroupM;
  const int gm = min(tiles_m - first_m, kGroupM);
  const int tm = first_m + (L % band) % gm;
  const int tn = (L % band) / gm;
  const int m0 = tm * BM, n0 = tn * BNO;

  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int wm = wave / WN, wn = wave % WN;

  // Per-lane sources of this wave's copies: copy q fills LDS rows 8q..8q+7.
  const bf16* src[NI];
  int kcol[NI];
#pragma unroll
  for (int i = 0; i < NI; ++i) {
    const int q = wave + NW * i;
    const int row = 8 * q + (lane >> 3);
    const int kc = (lane & 7) ^ chunk_swz(row);
    kcol[i] = kc * 8;
    if (row < BM) {
      src[i] = A + (int64_t)min(m0 + row, M - 1) * g.lda;
    } else {
      const int r = row - BM;
      int brow = n0 + r;
      const bf16* base = B;
      if (DUAL) {  // per wave column: TN/2 gate rows, then the matching TN/2 up rows
        const int wc = r / TN, within = r % TN;
        brow = n0 + wc * (TN / 2) + within % (TN / 2);
        base = (within >= TN / 2) ? B2 : B;
      }
      src[i] = base + (int64_t)min(brow, N - 1) * g.ldb;
    }
  }
  // copy K-tile kt of A and B into LDS buffer kt % STAGES
#define VIT_ISSUE(kt)                                                                   \
  do {                                                                                  \
    const int k0_ = (kt) * BK;                                                          \
    bf16* dst_ = smem + ((kt) % STAGES) * ROWS * BK;                                    \
    _Pragma("unroll") for (int i = 0; i < NI; ++i) {                                    \
      const int q_ = wave + NW * i;                                                     \
      const int kk_ = (8 * q_ < BM) ? k0_ + kcol[i] : min(k0_ + kcol[i], KB - 8);       \
      copy16_to_lds(src[i] + kk_, dst_ + q_ * 512);                                     \
    }                                                                                   \
  } while (0)

  // fragment addressing: lane reads row (lane & 31) of a 32-row block, 16-byte
  // chunk 2*ks + (lane >> 5) of the 64-wide stage
  const int fr = lane & 31, fh = lane >> 5;
  int a_off[BI], b_off[BJ], a_sw[BI], b_sw[BJ];
#pragma unroll
  for (int i = 0; i < BI; ++i) {
    const int r = wm * TM + i * 32 + fr;
    a_off[i] = r * BK;
    a_sw[i] = chunk_swz(r);
  }
#pragma unroll
  for (int j = 0; j < BJ; ++j) {
    const int r = BM + wn * TN + j * 32 + fr;
    b_off[j] = r * BK;
    b_sw[j] = chunk_swz(r);
  }

  f32x16 acc[BI][BJ];
#pragma unroll
  for (int i = 0; i < BI; ++i)
#pragma unroll
    for (int j = 0; j < BJ; ++j) acc[i][j] = f32x16{};

  bf16x8 af[2][BI], bfr[2][BJ];
  // fragments of k-step ks of LDS stage `stage` into register set `buf`
#define VIT_LOAD_FRAGS(buf, stage, ks)                                                  \
  do {                                                                                  \
    const bf16* base_ = smem + (stage) * ROWS * BK;                                     \
    const int c_ = 2 * (ks) + fh;                                                       \
    _Pragma("unroll") for (int i = 0; i < BI; ++i) af[buf][i] =                         \
        *reinterpret_cast<const bf16x8*>(base_ + a_off[i] + ((c_ ^ a_sw[i]) << 3));     \
    _Pragma("unroll") for (int j = 0; j < BJ; ++j) bfr[buf][j] =                        \
        *reinterpret_cast<const bf16x8*>(base_ + b_off[j] + ((c_ ^ b_sw[j]) << 3));     \
  } while (0)
#define VIT_MFMAS(buf)                                                                  \
  do {                                                                                  \
    _Pragma("unroll") for (int i = 0; i < BI; ++i)                                      \
    _Pragma("unroll") for (int j = 0; j < BJ; ++j) acc[i][j] =                          \
        __builtin_amdgcn_mfma_f32_32x32x16_bf16(bfr[buf][j], af[buf][i], acc[i][j], 0, 0, 0); \
  } while (0)

  const int nk = K / BK;
  // prologue: stages 0..STAGES-2 in flight, wait for stage 0, first fragments
#pragma unroll
  for (int s = 0; s < STAGES - 1; ++s)
    if (s < nk) VIT_ISSUE(s);
  if (nk > STAGES - 2)
    wait_vmcnt<(STAGES - 2) * NI>();
  else
    wait_vmcnt<0>();
  lds_barrier();
  VIT_LOAD_FRAGS(0, 0, 0);

  for (int kt = 0; kt < nk; ++kt) {
    const int st = kt % STAGES;
#pragma unroll
    for (int ks = 0; ks < KSTEPS - 1; ++ks) {
      VIT_LOAD_FRAGS((ks + 1) & 1, st, ks + 1);
      VIT_MFMAS(ks & 1);
    }
    // stage kt+1 must have landed (younger stages may stay in flight); the
    // barrier also retires every wave's reads of stage kt-1, whose buffer the
    // next copy overwrites
    if (kt + 1 < nk) {
      if (kt + STAGES - 1 < nk)
        wait_vmcnt<(STAGES - 3) * NI>();
      else
        wait_vmcnt<0>();
    }
    lds_barrier();
    if (kt + STAGES - 1 < nk) VIT_ISSUE(kt + STAGES - 1);
    if (kt + 1 < nk) VIT_LOAD_FRAGS(KSTEPS & 1, (kt + 1) % STAGES, 0);
    VIT_MFMAS((KSTEPS - 1) & 1);
  }
#undef VIT_LOAD_FRAGS
#undef VIT_MFMAS
#undef VIT_ISSUE

  // epilogue: acc[i][j] lane holds row m = (lane & 31) of block i and, for
  // g = 0..3, columns 8g + 4*(lane >> 5) .. +3 of block j
  const int c4 = 4 * fh;
#pragma unroll
  for (int i = 0; i < BI; ++i) {
    const int m = m0 + wm * TM + i * 32 + fr;
    if (m >= M) continue;
    const int64_t orow = g.rowmap ? (int64_t)g.rowmap[m] : (int64_t)m;
    if (DUAL) {
#pragma unroll
      for (int j = 0; j < BJ / 2; ++j)
#pragma unroll
        for (int gq = 0; gq < 4; ++gq) {
          const int n = n0 + wn * (TN / 2) + j * 32 + 8 * gq + c4;
          if (n >= N) continue;
          bf16x4 v;
#pragma unroll
          for (int r = 0; r < 4; ++r)
            v[r] = f2bf(silu_f(acc[i][j][4 * gq + r]) * acc[i][j + BJ / 2][4 * gq + r]);
          *reinterpret_cast<bf16x4*>((bf16*)g.C + orow * g.ldc + n) = v;
        }
    } else {
      if constexpr (EPI == VIT_EPI_STORE_ROPE || EPI == VIT_EPI_QKV_VT) {
        // wave columns n0 + wn*64 .. +63 are one head (64 wide): block 0 holds the
        // row-angle half (quarters: columns 0-15 in g = 0,1 and 16-31 in g = 2,3),
        // block 1 the column-angle half
        static_assert(TN == 64, "rotary epilogue needs 64-wide waves");
        if (n0 + wn * TN < g.rope_cols) {
          const float2* tab = (const float2*)g.rope_table + (int64_t)m * 32;
#pragma unroll
          for (int half = 0; half < 2; ++half)
#pragma unroll
            for (int gq = 0; gq < 2; ++gq)
#pragma unroll
              for (int r = 0; r < 4; ++r) {
                const float2 cs = tab[half * 16 + 8 * gq + c4 + r];
                const float a1 = acc[i][half][4 * gq + r], a2 = acc[i][half][4 * (gq + 2) + r];
                acc[i][half][4 * gq + r] = a1 * cs.x - a2 * cs.y;
                acc[i][half][4 * (gq + 2) + r] = a2 * cs.x + a1 * cs.y;
              }
        }
      }
#pragma unroll
      for (int j = 0; j < BJ; ++j)
#pragma unroll
        for (int gq = 0; gq < 4; ++gq) {
          const int n = n0 + wn * TN + j * 32 + 8 * gq + c4;
          if (n >= N) continue;
          f32x4 v;
#pragma unroll
          for (int r = 0; r < 4; ++r) v[r] = acc[i][j][4 * gq + r];
          if (EPI == VIT_EPI_QKV_VT && n >= g.rope_cols) {
            bf16* vt = (bf16*)g.vt + (int64_t)(n - g.rope_cols) * g.vt_ld + g.vpos[m];
#pragma unroll
            for (int r = 0; r < 4; ++r) vt[r * g.vt_ld] = f2bf(v[r]);
          } else if (EPI == VIT_EPI_STORE || EPI == VIT_EPI_STORE_ROPE || EPI == VIT_EPI_QKV_VT) {
            bf16x4 b;
#pragma unroll
            for (int r = 0; r < 4; ++r) b[r] = f2bf(v[r]);
            *reinterpret_cast<bf16x4*>((bf16*)g.C + orow * g.ldc + n) = b;
          } else if (EPI == VIT_EPI_STORE_F32) {
            *reinterpret_cast<f32x4*>((float*)g.C + orow * g.ldc + n) = v;
          } else {  // VIT_EPI_ADD_F32
            f32x4* c = reinterpret_cast<f32x4*>((float*)g.C + orow * g.ldc + n);
            *c = *c + v;
          }
        }
    }
  }
}

template <int BM, int BN, int WM, int WN, int STAGES, int EPI, bool DUAL>
hipError_t launch_cfg(const GemmArgs& g, hipStream_t s) {
  constexpr int BNO = DUAL ? BN / 2 : BN;
  constexpr size_t lds = (size_t)STAGES * (BM + BN) * BK * sizeof(bf16);
  auto kern = gemm_tile_kernel<BM, BN, WM, WN, STAGES, EPI, DUAL>;
  static bool attr = false;
  if (!attr) {
    hipError_t e = hipFuncSetAttribute((const void*)kern,
                                       hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
    if (e != hipSuccess) return e;
    attr = true;
  }
  const int64_t tiles = ((g.M + BM - 1) / BM) * ((g.N + BNO - 1) / BNO);
  kern<<<dim3((unsigned)tiles), dim3(WM * WN * 64), lds, s>>>(g);
  return hipGetLastError();
}

template <int BM, int BN, int WM, int WN, int STAGES>
hipError_t launch_epi(int epi, const GemmArgs& g, hipStream_t s) {
  switch (epi) {
    case VIT_EPI_STORE: return launch_cfg<BM, BN, WM, WN, STAGES, VIT_EPI_STORE, false>(g, s);
    case VIT_EPI_STORE_F32: return launch_cfg<BM, BN, WM, WN, STAGES, VIT_EPI_STORE_F32, false>(g, s);
    case VIT_EPI_ADD_F32: return launch_cfg<BM, BN, WM, WN, STAGES, VIT_EPI_ADD_F32, false>(g, s);
    case VIT_EPI_SWIGLU: return launch_cfg<BM, BN, WM, WN, STAGES, VIT_EPI_SWIGLU, true>(g, s);
    case VIT_EPI_STORE_ROPE: return launch_cfg<BM, BN, WM, WN, STAGES, VIT_EPI_STORE_ROPE, false>(g, s);
    case VIT_EPI_QKV_VT: return launch_cfg<BM, BN, WM, WN, STAGES, VIT_EPI_QKV_VT, false>(g, s);
  }
  return hipErrorInvalidValue;
}

}  // namespace

hipError_t launch_gemm_tile128(int epi, const GemmArgs& g, hipStream_t s) {
  return launch_epi<128, 128, 2, 2, 3>(epi, g, s);
}
