// Multi-stage bf16 MFMA GEMM for gfx950: C[M,N] = epilogue(A[M,K] . B[N,K]^T).
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

constexpr int kXcds = 8;
constexpr int kGroupM = 8;

// 16-byte chunk swizzle of an LDS row of BK bf16: consecutive rows that share
// 64 banks get distinct chunk positions (BK 64: rows are 128 B, pairs of rows
// share a bank line; BK 32: 64 B rows, four rows per bank line).
template <int BK>
VIT_DEV int chunk_swz(int row) {
  return BK == 64 ? (row >> 1) & 7 : (row >> 2) & 3;
}

VIT_DEV float silu_f(float g) { return g / (1.0f + __expf(-g)); }

// Compute units of the current device (queried once per process).
int num_cus() {
  static int n = 0;
  if (n == 0) {
    int dev = 0, v = 0;
    if (hipGetDevice(&dev) == hipSuccess &&
        hipDeviceGetAttribute(&v, hipDeviceAttributeMultiprocessorCount, dev) == hipSuccess && v > 0)
      n = v;
    else
      n = 256;
  }
  return n;
}

VIT_DEV int xcd_remap(int bid, int ntiles) {
  const int per = ntiles / kXcds, rem = ntiles % kXcds;
  const int xcd = bid % kXcds, idx = bid / kXcds;
  return xcd * per + min(xcd, rem) + idx;
}

template <int BM, int BN, int BK, int WM, int WN, int STAGES, int OCC, int EPI, bool DUAL>
__global__ __launch_bounds__(WM * WN * 64, OCC) void gemm_pipe_kernel(GemmArgs g) {
  constexpr int KSTEPS = BK / 16;
  constexpr int CPR = BK / 8;    // 16-byte chunks per LDS row
  constexpr int RPC = 64 / CPR;  // LDS rows filled by one 1 KB wave copy
  constexpr int NW = WM * WN;
  constexpr int TM = BM / WM, TN = BN / WN;  // wave tile
  constexpr int BI = TM / 32, BJ = TN / 32;  // 32x32 blocks per wave
  constexpr int ROWS = BM + BN;              // LDS rows per stage (A then B)
  constexpr int NI = ROWS / RPC / NW;        // 1 KB copies per wave per stage
  constexpr int BNO = DUAL ? BN / 2 : BN;    // output columns per tile
  static_assert(STAGES >= 3, "stages");
  static_assert(ROWS % (RPC * NW) == 0 && (TN / 2) % RPC == 0, "copy split");
  static_assert(TM % 32 == 0 && TN % 32 == 0 && (!DUAL || BJ % 2 == 0), "wave tile");
  extern __shared__ __attribute__((aligned(16))) bf16 smem[];

  const bf16* __restrict__ A = (const bf16*)g.A;
  const bf16* __restrict__ B = (const bf16*)g.B;
  const bf16* __restrict__ B2 = (const bf16*)g.B2;
  const int M = (int)g.M, N = (int)g.N, K = (int)g.K, KB = (int)g.kb;
  const int tiles_m = (M + BM - 1) / BM;
  const int tiles_n = (N + BNO - 1) / BNO;
  const int ntiles = tiles_m * tiles_n;
  const int nk = K / BK;

  // Persistent schedule: the logical (grouped) tile order is cut into one
  // contiguous chunk per XCD; the workgroups of an XCD (ids = xcd mod 8) take
  // the tiles of their chunk round-robin.
  const int G = gridDim.x;
  int my_first, my_step, my_count;
  if (G % kXcds == 0) {
    const int xcd = blockIdx.x % kXcds, r = blockIdx.x / kXcds, per = G / kXcds;
    const int c0 = (int)((int64_t)xcd * ntiles / kXcds);
    const int c1 = (int)((int64_t)(xcd + 1) * ntiles / kXcds);
    my_first = c0 + r;
    my_step = per;
    my_count = my_first < c1 ? (c1 - my_first + per - 1) / per : 0;
  } else {
    my_first = blockIdx.x;
    my_step = G;
    my_count = my_first < ntiles ? (ntiles - my_first + G - 1) / G : 0;
  }
  const int band = kGroupM * tiles_n;
  auto tile_origin = [&](int j, int& m0, int& n0) __attribute__((always_inline)) {
    const int L = my_first + j * my_step;
    const int first_m = (L / band) * kGroupM;
    const int gm = min(tiles_m - first_m, kGroupM);
    m0 = (first_m + (L % band) % gm) * BM;
    n0 = ((L % band) / gm) * BNO;
  };

  const int lane = threadIdx.x & 63;
  // wave index, made provably uniform so copy bases and wave offsets live in SGPRs
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int wm = wave / WN, wn = wave % WN;

  // Copies: copy q (of this wave: q = wave + NW*i) fills LDS rows RPC*q.. of a
  // stage.  Each lane's source is a wave-uniform matrix base + K offset plus a
  // per-lane 32-bit byte offset that changes only between tiles, so the copy
  // needs no vector address arithmetic inside the K loop.
  int crow[NI], kcol[NI];
  uint32_t voff[NI];
#pragma unroll
  for (int i = 0; i < NI; ++i) {
    const int q = wave + NW * i;
    const int row = RPC * q + lane / CPR;
    crow[i] = row;
    kcol[i] = ((lane % CPR) ^ chunk_swz<BK>(row)) * 8;
  }
  auto tile_offsets = [&](int m0_, int n0_) __attribute__((always_inline)) {
#pragma unroll
    for (int i = 0; i < NI; ++i) {
      const int q = wave + NW * i;
      if (RPC * q < BM) {
        voff[i] = (uint32_t)(((int64_t)min(m0_ + crow[i], M - 1) * g.lda + kcol[i]) * 2);
      } else {
        const int r = crow[i] - BM;
        int brow = n0_ + r;
        if (DUAL) brow = n0_ + (r / TN) * (TN / 2) + (r % TN) % (TN / 2);
        voff[i] = (uint32_t)(((int64_t)min(brow, N - 1) * g.ldb + kcol[i]) * 2);
      }
    }
  };
  // copy K-tile ikt of the current copy tile into LDS buffer `stage` (constant)
#define VIT_ISSUE(stage)                                                                \
  do {                                                                                  \
    const int k0_ = ikt * BK;                                                           \
    bf16* dst_ = smem + (stage) * ROWS * BK;                                            \
    if (k0_ + BK <= KB) {                                                               \
      _Pragma("unroll") for (int i = 0; i < NI; ++i) {                                  \
        const int q_ = wave + NW * i;                                                   \
        const char* base_ = (const char*)((RPC * q_ < BM) ? A : B);                     \
        if (DUAL && RPC * q_ >= BM && ((RPC * q_ - BM) % TN) >= TN / 2)                 \
          base_ = (const char*)B2;                                                      \
        copy16_to_lds(base_ + 2 * (int64_t)k0_ + voff[i], dst_ + q_ * 512);             \
      }                                                                                 \
    } else { /* last K-tile of a zero-padded A: keep B's reads inside its rows */       \
      _Pragma("unroll") for (int i = 0; i < NI; ++i) {                                  \
        const int q_ = wave + NW * i;                                                   \
        const char* base_ = (const char*)((RPC * q_ < BM) ? A : B);                     \
        if (DUAL && RPC * q_ >= BM && ((RPC * q_ - BM) % TN) >= TN / 2)                 \
          base_ = (const char*)B2;                                                      \
        const int kk_ = (RPC * q_ < BM) ? k0_ : min(k0_ + kcol[i], KB - 8) - kcol[i];   \
        copy16_to_lds(base_ + 2 * (int64_t)kk_ + voff[i], dst_ + q_ * 512);             \
      }                                                                                 \
    }                                                                                   \
    if (++ikt == nk) { /* the copy stream moves on to the next tile */                  \
      ikt = 0;                                                                          \
      if (++ij < my_count) {                                                            \
        int m0n_, n0n_;                                                                 \
        tile_origin(ij, m0n_, n0n_);                                                    \
        tile_offsets(m0n_, n0n_);                                                       \
      }                                                                                 \
    }                                                                                   \
  } while (0)

  // fragment addressing: lane reads row (lane & 31) of a 32-row block, 16-byte
  // chunk 2*ks + (lane >> 5) of the 64-wide stage; offsets per k-step are
  // precomputed, the stage enters as an immediate (the K loop is unrolled by STAGES)
  const int fr = lane & 31, fh = lane >> 5;
  int a_off[KSTEPS][BI], b_off[KSTEPS][BJ];
#pragma unroll
  for (int ks = 0; ks < KSTEPS; ++ks) {
#pragma unroll
    for (int i = 0; i < BI; ++i) {
      const int r = wm * TM + i * 32 + fr;
      a_off[ks][i] = r * BK + (((2 * ks + fh) ^ chunk_swz<BK>(r)) << 3);
    }
#pragma unroll
    for (int j = 0; j < BJ; ++j) {
      const int r = BM + wn * TN + j * 32 + fr;
      b_off[ks][j] = r * BK + (((2 * ks + fh) ^ chunk_swz<BK>(r)) << 3);
    }
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
    _Pragma("unroll") for (int i = 0; i < BI; ++i) af[buf][i] =                         \
        *reinterpret_cast<const bf16x8*>(base_ + a_off[ks][i]);                         \
    _Pragma("unroll") for (int j = 0; j < BJ; ++j) bfr[buf][j] =                        \
        *reinterpret_cast<const bf16x8*>(base_ + b_off[ks][j]);                         \
  } while (0)
#define VIT_MFMAS(buf)                                                                  \
  do {                                                                                  \
    _Pragma("unroll") for (int i = 0; i < BI; ++i)                                      \
    _Pragma("unroll") for (int j = 0; j < BJ; ++j) acc[i][j] =                          \
        __builtin_amdgcn_mfma_f32_32x32x16_bf16(bfr[buf][j], af[buf][i], acc[i][j], 0, 0, 0); \
  } while (0)

  const int total = my_count * nk;  // K-iterations of all my tiles, one stream
  // copy-stream position: K-tile ikt of my tile ij
  int ij = 0, ikt = 0;
  if (my_count > 0) {
    int m0f, n0f;
    tile_origin(0, m0f, n0f);
    tile_offsets(m0f, n0f);
  }
  // prologue: iterations 0..STAGES-2 in flight, wait for the first, first fragments
#pragma unroll
  for (int s = 0; s < STAGES - 1; ++s)
    if (s < total) VIT_ISSUE(s);
  if (total > STAGES - 2)
    wait_vmcnt<(STAGES - 2) * NI>();
  else
    wait_vmcnt<0>();
  lds_barrier();
  if (total > 0) VIT_LOAD_FRAGS(0, 0, 0);

  int cj = 0, ckt = 0, cm0 = 0, cn0 = 0;  // tile, K-tile and tile origin of the current iteration
  if (my_count > 0) tile_origin(0, cm0, cn0);
  for (int gb = 0; gb < total; gb += STAGES) {
#pragma unroll
  for (int u = 0; u < STAGES; ++u) {
    const int gi = gb + u;
    if (gi >= total) break;
#pragma unroll
    for (int ks = 0; ks < KSTEPS - 1; ++ks) {
      VIT_LOAD_FRAGS((ks + 1) & 1, u, ks + 1);
      VIT_MFMAS(ks & 1);
    }
    // iteration gi+1 must have landed (younger ones may stay in flight); the
    // barrier also retires every wave's reads of iteration gi-1, whose buffer
    // the next copy overwrites
    if (gi + 1 < total) {
      if (gi + STAGES - 1 < total)
        wait_vmcnt<(STAGES - 3) * NI>();
      else
        wait_vmcnt<0>();
    }
    lds_barrier();
    if (gi + STAGES - 1 < total) VIT_ISSUE((u + STAGES - 1) % STAGES);
    if (gi + 1 < total) VIT_LOAD_FRAGS(KSTEPS & 1, (u + 1) % STAGES, 0);
    VIT_MFMAS((KSTEPS - 1) & 1);
    if (++ckt < nk) continue;

    // ---- epilogue of tile cj (the copies of the next tile are in flight) ----
    const int m0 = cm0, n0 = cn0;
    ckt = 0;
    if (++cj < my_count) tile_origin(cj, cm0, cn0);
    // acc[i][j] lane holds row m = (lane & 31) of block i and, for g = 0..3,
    // columns 8g + 4*(lane >> 5) .. +3 of block j
    const int c4 = 4 * fh;
#pragma unroll
    for (int i = 0; i < BI; ++i) {
      const int m = m0 + wm * TM + i * 32 + fr;
      if (m < M) {
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
            // wave columns n0 + wn*64 .. +63 are one head (64 wide): block 0 holds
            // the row-angle half (quarters: columns 0-15 in g = 0,1 and 16-31 in
            // g = 2,3), block 1 the column-angle half
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
                // v column: row (head, dim) = n - rope_cols of the transposed layout
                bf16* vt = (bf16*)g.vt + (int64_t)(n - g.rope_cols) * g.vt_ld + g.vpos[m];
#pragma unroll
                for (int r = 0; r < 4; ++r) vt[r * g.vt_ld] = f2bf(v[r]);
              } else if (EPI == VIT_EPI_STORE || EPI == VIT_EPI_STORE_ROPE ||
                         EPI == VIT_EPI_QKV_VT) {
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
#pragma unroll
    for (int i = 0; i < BI; ++i)
#pragma unroll
      for (int j = 0; j < BJ; ++j) acc[i][j] = f32x16{};
  }
  }
#undef VIT_LOAD_FRAGS
#undef VIT_MFMAS
#undef VIT_ISSUE
}

template <int BM, int BN, int BK, int WM, int WN, int STAGES, int OCC, int EPI, bool DUAL>
hipError_t launch_cfg(const GemmArgs& g, hipStream_t s) {
  constexpr int BNO = DUAL ? BN / 2 : BN;
  constexpr size_t lds = (size_t)STAGES * (BM + BN) * BK * sizeof(bf16);
  auto kern = gemm_pipe_kernel<BM, BN, BK, WM, WN, STAGES, OCC, EPI, DUAL>;
  static bool attr = false;
  if (!attr) {
    hipError_t e = hipFuncSetAttribute((const void*)kern,
                                       hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
    if (e != hipSuccess) return e;
    attr = true;
  }
  const int64_t tiles = ((g.M + BM - 1) / BM) * ((g.N + BNO - 1) / BNO);
  // persistent grid: OCC workgroups per CU (the LDS ring takes most of a CU)
  const int64_t slots = (int64_t)num_cus() * OCC;
  const int64_t grid = tiles < slots ? tiles : slots;
  kern<<<dim3((unsigned)grid), dim3(WM * WN * 64), lds, s>>>(g);
  return hipGetLastError();
}

template <int BM, int BN, int BK, int WM, int WN, int STAGES, int OCC>
hipError_t launch_epi(int epi, const GemmArgs& g, hipStream_t s) {
  switch (epi) {
    case VIT_EPI_STORE:
      return launch_cfg<BM, BN, BK, WM, WN, STAGES, OCC, VIT_EPI_STORE, false>(g, s);
    case VIT_EPI_STORE_F32:
      return launch_cfg<BM, BN, BK, WM, WN, STAGES, OCC, VIT_EPI_STORE_F32, false>(g, s);
    case VIT_EPI_ADD_F32:
      return launch_cfg<BM, BN, BK, WM, WN, STAGES, OCC, VIT_EPI_ADD_F32, false>(g, s);
    case VIT_EPI_SWIGLU:
      return launch_cfg<BM, BN, BK, WM, WN, STAGES, OCC, VIT_EPI_SWIGLU, true>(g, s);
    case VIT_EPI_STORE_ROPE:
      if constexpr (BN / WN == 64)
        return launch_cfg<BM, BN, BK, WM, WN, STAGES, OCC, VIT_EPI_STORE_ROPE, false>(g, s);
      return hipErrorInvalidValue;
    case VIT_EPI_QKV_VT:
      if constexpr (BN / WN == 64)
        return launch_cfg<BM, BN, BK, WM, WN, STAGES, OCC, VIT_EPI_QKV_VT, false>(g, s);
      return hipErrorInvalidValue;
  }
  return hipErrorInvalidValue;
}

}  // namespace

hipError_t launch_gemm_pipe(int cfg, int epi, const GemmArgs& g, hipStream_t s) {
  switch (cfg) {
    case GEMM_PIPE_128x128_S4: return launch_epi<128, 128, 64, 2, 2, 4, 1>(epi, g, s);
    case GEMM_PIPE_128x128_S3: return launch_epi<128, 128, 64, 2, 2, 3, 1>(epi, g, s);
    case GEMM_PIPE_256x128_S3: return launch_epi<256, 128, 64, 2, 2, 3, 1>(epi, g, s);
    case GEMM_PIPE_128x256_S3: return launch_epi<128, 256, 64, 2, 2, 3, 1>(epi, g, s);
    case GEMM_PIPE_256x128_W8_S3: return launch_epi<256, 128, 64, 4, 2, 3, 1>(epi, g, s);
    case GEMM_PIPE_256x256_K32_S4: return launch_epi<256, 256, 32, 2, 2, 4, 1>(epi, g, s);
    case GEMM_PIPE_256x256_W8_K32_S4: return launch_epi<256, 256, 32, 2, 4, 4, 1>(epi, g, s);
    case GEMM_PIPE_128x128_W2_K32_S4: return launch_epi<128, 128, 32, 1, 2, 4, 2>(epi, g, s);
  }
  return hipErrorInvalidValue;
}
