// bf16 MFMA GEMM for gfx950: C[M,N] = epilogue(A[M,K] . B[N,K]^T), one
// BM x BN output tile per workgroup of WM x WN waves (the hardware dispatcher
// balances the tiles).
//
// Operands: both matrices K-contiguous.  Each BK-wide K-tile of A and B is
// copied from global memory straight into LDS with global_load_lds_dwordx4 (no
// register staging) into a ring of STAGES buffers: while the waves multiply
// K-tile kt, the copies of kt+1 .. kt+STAGES-2 are in flight.  Waits are exact
// (s_waitcnt vmcnt on the number of younger copies), and the one workgroup
// barrier per K-tile is taken before its last 16-wide k-step, so the next
// K-tile's first fragments are read while the last MFMAs of this one run.
//
// MFMA: v_mfma_f32_32x32x16_bf16 (32 cycles for 32K flops), issued as
// C^T = B . A^T with the weight fragment in the A slot, so a lane owns 4 groups
// of 4 consecutive output columns of one row.  Fragment reads are issued one
// k-step ahead of the MFMAs that use them and retired (lgkmcnt 0) right after
// those MFMAs have been issued, when they are long complete; no read is then
// pending at a branch merge or the loop back-edge, where the compiler's own
// wait counting falls back to a full wait in front of the MFMAs.
//
// LDS rows hold BK bf16; 16-byte chunks are XOR-swizzled on the global side of
// the copy ((row >> 1) & 7 for BK 64, (row >> 2) & 3 for BK 32) so fragment
// reads of 32 consecutive rows spread over all banks.
//
// Tile shapes: a wave that multiplies a TM x TN sub-tile reads (TM + TN) rows
// of fragments per TM*TN/1024 MFMAs, so larger sub-tiles need less LDS
// bandwidth per flop but give fewer tiles; the dispatcher weighs that against
// wave quantisation over the 256 CUs.
//
// Epilogues: bf16 store, fp32 store, fp32 residual add, SwiGLU (gate and up rows
// side by side in the B tile so silu(gate) * up meets in one lane), bf16 store
// with an fp32 column bias (and GELU, erf form, for the projector), and the
// half-split 2D rotary on the q and k columns (both rotate_half partners,
// columns c and c+16 of a 32-wide block, sit in one lane), optionally with the
// v columns written transposed for the attention kernel.  bf16 and fp32-store
// outputs are staged through the idle LDS ring and written as row-contiguous
// 16-byte stores.
//
// Requirements (checked by the dispatcher): K a multiple of BK for A (A may be
// zero-padded past B's valid K), N a multiple of 4, 16-byte aligned rows, and
// matrices addressable with 32-bit byte offsets.
#include <type_traits>

#include "common.h"
#include "gemm_mfma.h"

namespace {

constexpr int kXcds = 8;
constexpr int kGroupM = 8;

template <int BK>
VIT_DEV int chunk_swz(int row) {
  return BK == 64 ? (row >> 1) & 7 : (row >> 2) & 3;
}

VIT_DEV float silu_f(float g) { return g / (1.0f + __expf(-g)); }
// GELU in its erf form, x * Phi(x)
VIT_DEV float gelu_f(float x) { return 0.5f * x * (1.0f + erff(x * 0.70710678118654752f)); }

// One output tile of GEMM g: tile L of its grid (before the XCD remap below).
template <int BM, int BN, int BK, int WM, int WN, int STAGES, int EPI, bool DUAL>
__device__ __forceinline__ void gemm_tile(const GemmArgs& g, int L) {
  constexpr int NW = WM * WN;
  constexpr int TM = BM / WM, TN = BN / WN;  // wave sub-tile
  constexpr int BI = TM / 32, BJ = TN / 32;  // 32x32 blocks per wave
  static_assert(TM % 32 == 0 && TN % 32 == 0, "wave tile");
  static_assert(BI >= 1 && BJ >= 1, "wave tile");
  constexpr int KSTEPS = BK / 16;
  constexpr int CPR = BK / 8;    // 16-byte chunks per LDS row
  constexpr int RPC = 64 / CPR;  // LDS rows filled by one 1 KB wave copy
  constexpr int ROWS = BM + BN;  // LDS rows per stage (A then B)
  constexpr int NI = ROWS / RPC / NW;
  constexpr int BNO = DUAL ? BN / 2 : BN;  // output columns per tile
  static_assert(STAGES >= 3, "stages");
  static_assert(ROWS % (RPC * NW) == 0 && (TN / 2) % RPC == 0, "copy split");
  static_assert(!DUAL || BJ % 2 == 0, "dual tile");
  extern __shared__ __attribute__((aligned(16))) bf16 smem[];

  const bf16* __restrict__ A = (const bf16*)g.A;
  const bf16* __restrict__ B = (const bf16*)g.B;
  const bf16* __restrict__ B2 = (const bf16*)g.B2;
  const int M = (int)g.M, N = (int)g.N, K = (int)g.K, KB = (int)g.kb;
  const int tiles_m = (M + BM - 1) / BM;
  const int tiles_n = (N + BNO - 1) / BNO;
  const int ntiles = tiles_m * tiles_n;
  const int nk = K / BK;

  // Workgroup ids go round-robin over the 8 XCDs; give each XCD a contiguous
  // run of the grouped tile order (kGroupM tile rows share a column band), so
  // the A rows and B columns one XCD touches stay in its own L2.
  {
    const int per = ntiles / kXcds, rem = ntiles % kXcds;
    const int xcd = L % kXcds, idx = L / kXcds;
    L = xcd * per + min(xcd, rem) + idx;
  }
  const int band = kGroupM * tiles_n;
  const int first_m = (L / band) * kGroupM;
  const int gm = min(tiles_m - first_m, kGroupM);
  const int m0 = (first_m + (L % band) % gm) * BM;
  const int n0 = ((L % band) / gm) * BNO;

  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int wm = wave / WN, wn = wave % WN;

  // copy i of this wave fills LDS rows RPC*(wave + NW*i) .. +RPC-1 of a stage
  // (copies i < NIA are A rows, the rest B rows).  voff is the lane's byte
  // offset from the wave-uniform matrix base: for A it includes the lane's
  // K chunk (the K-tile offset is added to the scalar base), for B only the
  // row, because B's K index is clamped to its valid width per K-tile.
  constexpr int NIA = BM / (RPC * NW);
  static_assert(BM % (RPC * NW) == 0, "A/B copy split");
  // gathered A (the aligner's 2x2 merge): A row m is source rows a_rows[4m + s],
  // s = 0..3, side by side; every K-tile lies in one a_seg-wide segment s, so a
  // copy slot keeps the byte offsets of its four source rows and picks one per
  // K-tile
  constexpr bool kGather = EPI == VIT_EPI_STORE_GATHER;
  uint32_t voff[NI];
  uint32_t vga[kGather ? NIA : 1][4];
  int kcol[NI];
#pragma unroll
  for (int i = 0; i < NI; ++i) {
    const int q = wave + NW * i;
    const int row = RPC * q + lane / CPR;
    kcol[i] = ((lane % CPR) ^ chunk_swz<BK>(row)) * 8;
    if (i < NIA) {
      if constexpr (kGather) {
        const int4 r4 = *reinterpret_cast<const int4*>(g.a_rows + 4 * (int64_t)min(m0 + row, M - 1));
        const int src[4] = {r4.x, r4.y, r4.z, r4.w};
#pragma unroll
        for (int sg = 0; sg < 4; ++sg)
          vga[i < NIA ? i : 0][sg] = (uint32_t)(((int64_t)src[sg] * g.lda + kcol[i]) * 2);
        voff[i] = 0;
      } else {
        voff[i] = (uint32_t)(((int64_t)min(m0 + row, M - 1) * g.lda + kcol[i]) * 2);
      }
    } else {
      const int r = row - BM;
      int brow = n0 + r;
      if (DUAL) brow = n0 + (r / TN) * (TN / 2) + (r % TN) % (TN / 2);
      voff[i] = (uint32_t)((int64_t)min(brow, N - 1) * g.ldb * 2);
    }
  }
  // copy K-tile kt_ into LDS buffer `stage` (a constant).  A may be zero-padded
  // past B's valid K (KB); B's K index is clamped into [0, KB) so its reads
  // stay inside its rows (the products with A's zero columns vanish).
  // segment seg_ of the gathered A operand holding K offset k0_, and the offset
  // kin_ inside it (unused without the gather)
  // (k0_ / a_seg as a multiply-high by ceil(2^32 / a_seg), exact for k0_ * a_seg
  // < 2^32; the segment's four offset masks select a copy slot's source row
  // without branches)
  const int segk = kGather ? (int)g.a_seg : 1;
  const uint32_t seg_magic = kGather ? (uint32_t)(((1ull << 32) + segk - 1) / segk) : 0u;
#define W_SEG(k0_)                                                                      \
  const int seg_ = kGather ? (int)(((uint64_t)(uint32_t)(k0_) * seg_magic) >> 32) : 0;  \
  const int kin_ = (k0_) - seg_ * segk;                                                 \
  const uint32_t sm0_ = seg_ == 0 ? ~0u : 0u, sm1_ = seg_ == 1 ? ~0u : 0u;              \
  const uint32_t sm2_ = seg_ == 2 ? ~0u : 0u, sm3_ = seg_ == 3 ? ~0u : 0u;              \
  (void)kin_;                                                                           \
  (void)sm0_;                                                                           \
  (void)sm1_;                                                                           \
  (void)sm2_;                                                                           \
  (void)sm3_
  // copy i of K-tile k0_/BK (k0_ a scalar) into the LDS buffer at dst_
#define W_COPY1(k0_, dst_, i)                                                           \
  do {                                                                                  \
    const int q_ = wave + NW * (i);                                                     \
    if ((i) < NIA) {                                                                    \
      if constexpr (kGather) {                                                          \
        const int ia_ = (i) < NIA ? (i) : 0;                                            \
        const uint32_t o_ = (vga[ia_][0] & sm0_) | (vga[ia_][1] & sm1_) |               \
                            (vga[ia_][2] & sm2_) | (vga[ia_][3] & sm3_);                \
        copy16_to_lds((const char*)A + 2 * (int64_t)kin_ + o_, (dst_) + q_ * 512);       \
      } else {                                                                          \
        copy16_to_lds((const char*)A + 2 * (int64_t)(k0_) + voff[i], (dst_) + q_ * 512); \
      }                                                                                 \
    } else {                                                                            \
      const char* b_ = (const char*)((DUAL && ((RPC * q_ - BM) % TN) >= TN / 2) ? B2 : B); \
      copy16_to_lds(b_ + (voff[i] + 2u * (uint32_t)min((k0_) + kcol[i], KB - 8)),        \
                    (dst_) + q_ * 512);                                                 \
    }                                                                                   \
  } while (0)
  // all copies of K-tile kt_ into LDS buffer `stage` (a constant)
#define W_ISSUE(stage, kt_)                                                             \
  do {                                                                                  \
    /* readfirstlane keeps the K offset a scalar: strength reduction would */           \
    /* otherwise turn every copy address into a 64-bit vector induction variable */     \
    const int k0_ = __builtin_amdgcn_readfirstlane((kt_) * BK);                         \
    W_SEG(k0_);                                                                         \
    bf16* dst_ = smem + (stage) * ROWS * BK;                                            \
    _Pragma("unroll") for (int i = 0; i < NI; ++i) W_COPY1(k0_, dst_, i);               \
  } while (0)

  // fragment reads: lane row (lane & 31) of a 32-row block, 16-byte chunk
  // 2*ks + (lane >> 5); the swizzle depends only on (lane & 31), so blocks of
  // one wave differ by a constant offset
  const int fr = lane & 31, fh = lane >> 5;
  int a_off[KSTEPS], b_off[KSTEPS];
#pragma unroll
  for (int ks = 0; ks < KSTEPS; ++ks) {
    const int ra = wm * TM + fr, rb = BM + wn * TN + fr;
    a_off[ks] = ra * BK + (((2 * ks + fh) ^ chunk_swz<BK>(ra)) << 3);
    b_off[ks] = rb * BK + (((2 * ks + fh) ^ chunk_swz<BK>(rb)) << 3);
  }

  f32x16 acc[BI][BJ];
#pragma unroll
  for (int i = 0; i < BI; ++i)
#pragma unroll
    for (int j = 0; j < BJ; ++j) acc[i][j] = f32x16{};

  // fp32 residual add: the rows to add to, and the folded-norm producer's norm
  // weights, are loaded into registers right after the copies of the last
  // K-tile are issued, so their reads overlap the MFMAs of the last STAGES-1
  // K-tiles instead of following them.  Those loads are younger than every
  // copy; the waits of the last K-tiles count them (kPreLoads).  Needs the last
  // copies issued inside the loop (nk >= STAGES), no row map, and at most
  // 32 + 8 registers per lane (more would spill with two waves per SIMD).
  // Every wave issues the same loads (without norm weights the first row of C
  // stands in), so the counts hold for all.
  constexpr bool kPre = EPI == VIT_EPI_ADD_F32 && BI * BJ <= 2 && STAGES <= 4;
  constexpr int kPreLoads = kPre ? BI * BJ * 4 + BJ * 4 : 0;
  const bool pre_on = kPre && nk >= STAGES && g.rowmap == nullptr;
  f32x4 pre[kPre ? BI : 1][kPre ? BJ : 1][4];
  f32x4 wpre[kPre ? BJ : 1][4];
  const int c4 = 4 * (lane >> 5);
#define W_PRELOAD()                                                                     \
  do {                                                                                  \
    _Pragma("unroll") for (int i = 0; i < (kPre ? BI : 0); ++i) {                       \
      const int m_ = min(m0 + wm * TM + i * 32 + (lane & 31), M - 1);                  \
      _Pragma("unroll") for (int j = 0; j < BJ; ++j)                                    \
      _Pragma("unroll") for (int gq = 0; gq < 4; ++gq) pre[i][j][gq] =                  \
          *reinterpret_cast<const f32x4*>((const float*)g.C + (int64_t)m_ * g.ldc +     \
                                          min(n0 + wn * TN + j * 32 + 8 * gq + c4, N - 4)); \
    }                                                                                   \
    if constexpr (kPre) {                                                               \
      const float* w_ = g.norm_w ? g.norm_w : (const float*)g.C;                        \
      _Pragma("unroll") for (int j = 0; j < BJ; ++j)                                    \
      _Pragma("unroll") for (int gq = 0; gq < 4; ++gq) wpre[j][gq] =                    \
          *reinterpret_cast<const f32x4*>(w_ + min(n0 + wn * TN + j * 32 + 8 * gq + c4, N - 4)); \
    }                                                                                   \
  } while (0)

  bf16x8 af[2][BI], bfr[2][BJ];
#define W_LOAD_FRAGS(buf, stage, ks)                                                    \
  do {                                                                                  \
    const bf16* base_ = smem + (stage) * ROWS * BK;                                     \
    _Pragma("unroll") for (int i = 0; i < BI; ++i) af[buf][i] =                         \
        *reinterpret_cast<const bf16x8*>(base_ + a_off[ks] + i * 32 * BK);              \
    _Pragma("unroll") for (int j = 0; j < BJ; ++j) bfr[buf][j] =                        \
        *reinterpret_cast<const bf16x8*>(base_ + b_off[ks] + j * 32 * BK);              \
  } while (0)
#define W_MFMAS(buf)                                                                    \
  do {                                                                                  \
    _Pragma("unroll") for (int i = 0; i < BI; ++i)                                      \
    _Pragma("unroll") for (int j = 0; j < BJ; ++j) acc[i][j] =                          \
        __builtin_amdgcn_mfma_f32_32x32x16_bf16(bfr[buf][j], af[buf][i], acc[i][j], 0, 0, 0); \
  } while (0)
  // the MFMAs of register set buf with the copies of K-tile kt_ (if it exists)
  // into buffer `stage` spread evenly between them: issued as one burst right
  // after the barrier, the copies of all waves queue at the texture unit and
  // hold up the MFMAs behind them
#define W_MFMAS_COPY(buf, stage, kt_)                                                   \
  do {                                                                                  \
    constexpr int NM_ = BI * BJ;                                                        \
    const bool iss_ = (kt_) < nk;                                                       \
    const int k0_ = __builtin_amdgcn_readfirstlane((kt_) * BK);                         \
    W_SEG(k0_);                                                                         \
    bf16* dst_ = smem + (stage) * ROWS * BK;                                            \
    _Pragma("unroll") for (int x = 0; x < NM_; ++x) {                                   \
      acc[x / BJ][x % BJ] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(                    \
          bfr[buf][x % BJ], af[buf][x / BJ], acc[x / BJ][x % BJ], 0, 0, 0);             \
      _Pragma("unroll") for (int c = 0; c < NI; ++c) {                                  \
        if (c * NM_ / NI == x && iss_) W_COPY1(k0_, dst_, c);                           \
      }                                                                                 \
      sched_fence();                                                                    \
    }                                                                                   \
    if (kPre && pre_on && (kt_) == nk - 1) W_PRELOAD();                                 \
    sched_fence();                                                                      \
  } while (0)

  // RMSNorm consumer: thread t < BM reads the partial sums of tile row t before
  // the first copies are issued (the prologue's vmcnt wait then covers them)
  // and leaves the row's rstd in LDS, past the ring, for the epilogue
  float* s_rstd = (float*)((char*)smem + STAGES * ROWS * BK * 2);
  const bool norm_in = g.ss_in != nullptr && threadIdx.x < BM;
  f32x4 part[kMaxNormGroups / 4];
  if (norm_in) {
    const int ldss = (g.ss_groups + 3) & ~3;
    const int m = min(m0 + (int)threadIdx.x, M - 1);
    const f32x4* row = reinterpret_cast<const f32x4*>(g.ss_in + (int64_t)m * ldss);
#pragma unroll
    for (int q = 0; q < kMaxNormGroups / 4; ++q) part[q] = row[min(q, ldss / 4 - 1)];
  }

  // prologue: K-tiles 0..STAGES-2 in flight, wait for the first, first fragments
#pragma unroll
  for (int s = 0; s < STAGES - 1; ++s)
    if (s < nk) W_ISSUE(s, s);
  if (nk > STAGES - 2)
    wait_vmcnt<(STAGES - 2) * NI>();
  else
    wait_vmcnt<0>();
  if (norm_in) {
    float t = 0.f;
#pragma unroll
    for (int k = 0; k < kMaxNormGroups; ++k) t += k < g.ss_groups ? part[k / 4][k % 4] : 0.f;
    s_rstd[threadIdx.x] = 1.0f / sqrtf(t * g.rms_inv_dim + g.rms_eps);
  }
  lds_barrier();
  W_LOAD_FRAGS(0, 0, 0);
  wait_lgkmcnt<0>();  // nothing pending on entry to the loop (see W_KTILE)
  sched_fence();

  // one K-tile (ring slot u, a constant): the fragments of each next k-step are
  // read while the MFMAs of the current one run
#define W_KTILE(u, kt)                                                                  \
  do {                                                                                  \
    _Pragma("unroll") for (int ks = 0; ks < KSTEPS - 1; ++ks) {                         \
      W_LOAD_FRAGS((ks + 1) & 1, u, ks + 1);                                            \
      sched_fence();                                                                    \
      W_MFMAS(ks & 1);                                                                  \
      sched_fence();                                                                    \
      wait_lgkmcnt<0>(); /* free: see below */                                          \
      sched_fence();                                                                    \
    }                                                                                   \
    /* K-tile kt+1 must have landed (younger copies may stay in flight); the */         \
    /* barrier also retires every wave's reads of K-tile kt-1, whose buffer */          \
    /* the next copy overwrites */                                                      \
    if ((kt) + 1 < nk) {                                                                \
      if ((kt) + STAGES - 1 < nk) {                                                     \
        wait_vmcnt<(STAGES - 3) * NI>();                                                \
      } else if (pre_on) { /* every copy issued, then the residual loads */             \
        if (STAGES >= 4 && (kt) + 3 == nk)                                              \
          wait_vmcnt<(STAGES >= 4 ? NI : 0) + kPreLoads>();                             \
        else                                                                            \
          wait_vmcnt<kPreLoads>();                                                      \
      } else {                                                                          \
        wait_vmcnt<0>();                                                                \
      }                                                                                 \
    }                                                                                   \
    lds_barrier();                                                                      \
    /* unconditional (after the last K-tile it reads a stale, in-bounds */              \
    /* buffer), so the LDS wait counts stay exact */                                    \
    W_LOAD_FRAGS(KSTEPS & 1, ((u) + 1) % STAGES, 0);                                    \
    sched_fence();                                                                      \
    W_MFMAS_COPY((KSTEPS - 1) & 1, ((u) + STAGES - 1) % STAGES, (kt) + STAGES - 1);      \
    sched_fence();                                                                      \
    /* those reads are long done once the MFMA pipe has taken these MFMAs; */           \
    /* waiting here leaves no read pending across branch merges and the loop */         \
    /* back-edge, where the compiler's wait counting would otherwise fall back */       \
    /* to lgkmcnt(0) right before the next MFMAs */                                     \
    wait_lgkmcnt<0>();                                                                  \
    sched_fence();                                                                      \
  } while (0)

  // whole turns of the ring without guards (exact wait counts in the hot
  // loop), then the remaining K-tiles each under a guard (a guarded body, not
  // a break: early exits from the unrolled ring make the register allocator
  // duplicate the accumulators)
  int kb0 = 0;
  for (; kb0 + STAGES <= nk; kb0 += STAGES) {
#pragma unroll
    for (int u = 0; u < STAGES; ++u) W_KTILE(u, kb0 + u);
  }
#pragma unroll
  for (int u = 0; u < STAGES - 1; ++u)
    if (kb0 + u < nk) W_KTILE(u, kb0 + u);
#undef W_KTILE
#undef W_LOAD_FRAGS
#undef W_MFMAS
#undef W_MFMAS_COPY
#undef W_PRELOAD
#undef W_ISSUE
#undef W_COPY1
#undef W_SEG

  // ---- epilogue: acc[i][j] lane holds row (lane & 31) of block i and, for
  // gq = 0..3, columns 8gq + 4*(lane >> 5) .. +3 of block j ----
  constexpr bool kF32Out = (EPI == VIT_EPI_STORE_F32 || EPI == VIT_EPI_ADD_F32);
  if (!kF32Out && g.ss_in) {
    // RMSNorm consumer: output rows times the rstd computed at kernel start
#pragma unroll
    for (int i = 0; i < BI; ++i) {
      const float rstd = s_rstd[wm * TM + i * 32 + fr];
#pragma unroll
      for (int j = 0; j < BJ; ++j) acc[i][j] *= rstd;
    }
  }
  // vmcnt also counts stores: a global load issued after stores is waited for
  // together with them.  Every load of the epilogue (row map, fp32 rows to
  // add to, norm weights, v positions) is therefore issued before the first
  // store, and the paths are specialised on whether a row map is present (a
  // load under a branch makes the compiler wait for all stores at its use).
  const bool has_rowmap = g.rowmap != nullptr;

  if constexpr (kF32Out && TN % 64 == 0) if (g.norm_w) {
    // RMSNorm producer (wave sub-tiles of whole 64-column groups; the
    // dispatcher picks such a tile).  Blocks 2q and 2q+1 of the wave are
    // group q; lanes l and l^32 hold the two halves of a row's group.  x_new goes straight back to the
    // fp32 stream; u = bf16(x_new * w) is staged through the idle LDS ring (as
    // the bf16 outputs below) and written as row-contiguous 16-byte stores.
    constexpr int UROWB = TN * 2;            // bytes per staged u row
    constexpr int UCPR = UROWB / 16, URPL = 256 / UROWB;
    static_assert(TM * UROWB * NW <= STAGES * ROWS * BK * 2, "u staging fits the ring");
    // x_new is staged too (after every wave's u rows) where the ring has room, so
    // its fp32 rows also leave as row-contiguous 16-byte stores; otherwise (and
    // with a row map) it is stored straight from the MFMA layout
    constexpr int XROWB = TN * 4, XCPR = XROWB / 16;
    constexpr bool kStageX = TM * (UROWB + XROWB) * NW <= STAGES * ROWS * BK * 2;
    const int n = n0 + wn * TN;
    const bool cols_ok = n < N;
    const int64_t ld_nout = g.ld_norm_out ? g.ld_norm_out : N;
    const int64_t ld_ss = g.ld_ss_out ? g.ld_ss_out : ((N / 64 + 3) & ~3);
    char* st = (char*)smem + wave * (TM * UROWB);
    char* xs = (char*)smem + NW * TM * UROWB + wave * (TM * XROWB);
    auto produce = [&](auto with_rowmap, auto with_pre) __attribute__((always_inline)) {
      int64_t orow[BI];
#pragma unroll
      for (int i = 0; i < BI; ++i) {
        const int m = min(m0 + wm * TM + i * 32 + fr, M - 1);
        if constexpr (with_rowmap) orow[i] = g.rowmap[m]; else orow[i] = m;
      }
      f32x4 w[BJ][4];
#pragma unroll
      for (int j = 0; j < BJ; ++j)
#pragma unroll
        for (int gq = 0; gq < 4; ++gq) {
          if constexpr (with_pre)
            w[j][gq] = wpre[kPre ? j : 0][gq];
          else
            w[j][gq] = *reinterpret_cast<const f32x4*>(g.norm_w + min(n + j * 32 + 8 * gq + c4, N - 4));
        }
      lds_barrier();  // every wave is done reading the ring
      constexpr int GI = BI % 2 == 0 ? 2 : 1;  // row blocks per load/store group (divides BI)
#pragma unroll
      for (int i0 = 0; i0 < BI; i0 += GI) {
        // loads of the group (unconditional, clamped in bounds) before its stores
        f32x4 v[GI][BJ][4];
#pragma unroll
        for (int ii = 0; ii < GI; ++ii)
#pragma unroll
          for (int j = 0; j < BJ; ++j)
#pragma unroll
            for (int gq = 0; gq < 4; ++gq) {
              const int i = i0 + ii;
#pragma unroll
              for (int e = 0; e < 4; ++e) v[ii][j][gq][e] = acc[i][j][4 * gq + e];
              if constexpr (EPI == VIT_EPI_ADD_F32 && with_pre)
                v[ii][j][gq] += pre[kPre ? i : 0][kPre ? j : 0][gq];
              else if constexpr (EPI == VIT_EPI_ADD_F32)
                v[ii][j][gq] += *reinterpret_cast<const f32x4*>(
                    (const float*)g.C + orow[i] * g.ldc + min(n + j * 32 + 8 * gq + c4, N - 4));
            }
#pragma unroll
        for (int ii = 0; ii < GI; ++ii) {
          const int i = i0 + ii;
          const int r = i * 32 + fr;
          const int m = m0 + wm * TM + r;
          const bool ok = cols_ok && m < M;
          const int sw = (r / URPL) % UCPR;
          float ssum[TN / 64] = {};
#pragma unroll
          for (int j = 0; j < BJ; ++j)
#pragma unroll
            for (int gq = 0; gq < 4; ++gq) {
              if constexpr (kStageX && !with_rowmap) {
                // chunk j*8 + 2*gq + fh of the row's 16, XOR-swizzled by the row
                const int c16x = j * 8 + 2 * gq + fh;
                *reinterpret_cast<f32x4*>(xs + r * XROWB + ((c16x ^ (r & 15)) << 4)) = v[ii][j][gq];
              } else if (ok) {
                *reinterpret_cast<f32x4*>((float*)g.C + orow[i] * g.ldc + n + j * 32 + 8 * gq + c4) =
                    v[ii][j][gq];
              }
              bf16x4 u;
#pragma unroll
              for (int e = 0; e < 4; ++e) {
                u[e] = f2bf(v[ii][j][gq][e] * w[j][gq][e]);
                ssum[j / 2] += v[ii][j][gq][e] * v[ii][j][gq][e];
              }
              const int c16 = j * 4 + gq, hh = fh ^ ((r >> 4) & 1);
              *reinterpret_cast<bf16x4*>(st + r * UROWB + ((c16 ^ sw) << 4) + (hh << 3)) = u;
            }
#pragma unroll
          for (int q = 0; q < TN / 64; ++q) {
            const float sq = xor32_sum(ssum[q]);
            if (ok && fh == 0) g.ss_out[(int64_t)m * ld_ss + n / 64 + q] = sq;
          }
        }
        sched_fence();
      }
    };
    if (has_rowmap)
      produce(std::true_type{}, std::false_type{});
    else if (kPre && pre_on)
      produce(std::false_type{}, std::bool_constant<kPre>{});
    else
      produce(std::false_type{}, std::false_type{});
    __builtin_amdgcn_s_waitcnt(0xC07F);  // lgkmcnt(0): staged writes done
    asm volatile("" ::: "memory");
    if (kStageX && !has_rowmap) {
      constexpr int XRPI = 64 / XCPR;  // staged x rows per read instruction
      const int xcl = lane % XCPR;
#pragma unroll 4
      for (int it = 0; it < TM / XRPI; ++it) {
        const int R = it * XRPI + lane / XCPR;
        const int m = m0 + wm * TM + R;
        const f32x4 xv =
            *reinterpret_cast<const f32x4*>(xs + R * XROWB + ((xcl ^ (R & 15)) << 4));
        if (!cols_ok || m >= M) continue;
        *reinterpret_cast<f32x4*>((float*)g.C + (int64_t)m * g.ldc + n + xcl * 4) = xv;
      }
    }
    constexpr int URPI = 64 / UCPR;  // staged rows per read instruction
    const int cl = lane % UCPR;
#pragma unroll 4
    for (int it = 0; it < TM / URPI; ++it) {
      const int R = it * URPI + lane / UCPR;
      const int m = m0 + wm * TM + R;
      u32x4 dd = *reinterpret_cast<const u32x4*>(st + R * UROWB + ((cl ^ ((R / URPL) % UCPR)) << 4));
      if ((R >> 4) & 1) {
        const uint32_t t0 = dd[0], t1 = dd[1];
        dd[0] = dd[2]; dd[1] = dd[3]; dd[2] = t0; dd[3] = t1;
      }
      if (!cols_ok || m >= M) continue;
      *reinterpret_cast<u32x4*>((bf16*)g.norm_out + (int64_t)m * ld_nout + n + cl * 8) = dd;
    }
    return;
  }
  if constexpr (EPI == VIT_EPI_STORE_ROPE || EPI == VIT_EPI_QKV_VT) {
    // each pair of 32-wide blocks (2h, 2h+1) is one 64-wide head: block 2h
    // holds the row-angle half, block 2h+1 the column-angle half; the
    // rotate_half partners (columns c and c+16 of a block) sit in one lane.
    // The lane's table entries (16 cos/sin pairs per row: its 4-column groups
    // c4 + 8 gq + 16 half) for a group of RG row blocks are all loaded before
    // any is used, so those loads are in flight together. RG is every row
    // block when a wave has 512 registers per lane (one wave per SIMD) and two
    // with 256 (the 8-wave tiles, whose accumulators already take half).
    if (n0 + wn * TN < g.rope_cols) {
      constexpr int RG = (WM * WN > 4 && BI > 2) ? 2 : BI;
      static_assert(BI % RG == 0, "row block groups");
#pragma unroll
      for (int i0 = 0; i0 < BI; i0 += RG) {
        f32x4 cs[RG][2][2][2];
#pragma unroll
        for (int ii = 0; ii < RG; ++ii) {
          const int m = min(m0 + wm * TM + (i0 + ii) * 32 + fr, M - 1);
          const float* tab = (const float*)g.rope_table + (int64_t)m * 64;
#pragma unroll
          for (int half = 0; half < 2; ++half)
#pragma unroll
            for (int gq = 0; gq < 2; ++gq)
#pragma unroll
              for (int q = 0; q < 2; ++q)
                cs[ii][half][gq][q] = *reinterpret_cast<const f32x4*>(
                    tab + 2 * (half * 16 + 8 * gq + c4) + 4 * q);
        }
#pragma unroll
        for (int ii = 0; ii < RG; ++ii) {
          const int i = i0 + ii;
#pragma unroll
          for (int h = 0; h < BJ / 2; ++h) {
            if (n0 + wn * TN + h * 64 >= g.rope_cols) continue;
#pragma unroll
            for (int half = 0; half < 2; ++half)
#pragma unroll
              for (int gq = 0; gq < 2; ++gq)
#pragma unroll
                for (int r = 0; r < 4; ++r) {
                  const float c = cs[ii][half][gq][r / 2][2 * (r % 2)];
                  const float sn = cs[ii][half][gq][r / 2][2 * (r % 2) + 1];
                  const float a1 = acc[i][2 * h + half][4 * gq + r];
                  const float a2 = acc[i][2 * h + half][4 * (gq + 2) + r];
                  acc[i][2 * h + half][4 * gq + r] = a1 * c - a2 * sn;
                  acc[i][2 * h + half][4 * (gq + 2) + r] = a2 * c + a1 * sn;
                }
          }
        }
        sched_fence();  // one group's table entries live at a time
      }
    }
  }

  // Staged store: the wave writes its output sub-tile into its own quarter of
  // the (now idle) LDS ring, then reads it back one 16-byte chunk per lane in
  // row order, so every global store instruction covers whole 128-byte lines
  // (direct stores from the MFMA layout touch 32 rows per instruction).
  constexpr bool kF32 = kF32Out;
  constexpr int OB = kF32 ? 4 : 2;             // output bytes per element
  constexpr int OTN = DUAL ? TN / 2 : TN;      // output columns per wave
  constexpr int ROWB = OTN * OB;               // bytes per staged row
  constexpr int CPRW = ROWB / 16;              // 16-byte chunks per staged row
  constexpr int RPL = ROWB <= 256 ? 256 / ROWB : 1;  // staged rows per 256-byte bank line
  constexpr int EPC = 16 / OB;                 // elements per chunk
  constexpr bool kStaged = EPI != VIT_EPI_ADD_F32 && (ROWB == 64 || ROWB == 128 || ROWB == 256) &&
                           TM * ROWB * NW <= STAGES * ROWS * BK * 2;
  const bool v_wave = (EPI == VIT_EPI_QKV_VT) && (n0 + wn * TN >= g.rope_cols);
  const bool staged = kStaged && (g.ldc * OB) % 16 == 0;  // 16-byte aligned output rows
  constexpr bool kBias = EPI == VIT_EPI_BIAS || EPI == VIT_EPI_BIAS_GELU;
  // bias of the lane's 4-column groups: loaded once, before any store, when the
  // wave tile is at most 64 columns wide; wider tiles (whose accumulators fill
  // the register file) read each group where it is used
  constexpr bool kBiasHoist = kBias && BJ <= 2;
  f32x4 bias_v[kBiasHoist ? BJ : 1][4];
  auto bias_ld = [&](int j, int gq) __attribute__((always_inline)) {
    return *reinterpret_cast<const f32x4*>(g.bias +
                                           min(n0 + wn * TN + j * 32 + 8 * gq + c4, N - 4));
  };
  if constexpr (kBiasHoist) {
#pragma unroll
    for (int j = 0; j < BJ; ++j)
#pragma unroll
      for (int gq = 0; gq < 4; ++gq) bias_v[j][gq] = bias_ld(j, gq);
  }
  auto bias_group = [&](int j, int gq) __attribute__((always_inline)) {
    if constexpr (kBiasHoist) return bias_v[j][gq];
    else if constexpr (kBias) return bias_ld(j, gq);
    else return f32x4{};
  };
  auto bias_act = [&](float v, float bias) __attribute__((always_inline)) {
    if constexpr (kBias) {
      v += bias;
      if constexpr (EPI == VIT_EPI_BIAS_GELU) v = gelu_f(v);
    }
    return v;
  };
  if (staged) {
    lds_barrier();  // every wave is done reading the ring
    if (!v_wave) {
      char* st = (char*)smem + wave * (TM * ROWB);
      // chunk c16 (and 8-byte half h for bf16) of staged row r goes to
      // chunk c16 ^ ((r / RPL) % CPRW), half h ^ ((r >> 4) & 1): conflict-free
      // writes from the MFMA layout and conflict-free row-order reads
#pragma unroll
      for (int i = 0; i < BI; ++i) {
        const int r = i * 32 + fr;
        const int sw = (r / RPL) % CPRW;
        char* row = st + r * ROWB;
#pragma unroll
        for (int j = 0; j < (DUAL ? BJ / 2 : BJ); ++j)
#pragma unroll
          for (int gq = 0; gq < 4; ++gq) {
            if constexpr (kF32) {
              const int c16 = j * 8 + 2 * gq + fh;
              f32x4 v;
#pragma unroll
              for (int e = 0; e < 4; ++e) v[e] = acc[i][j][4 * gq + e];
              *reinterpret_cast<f32x4*>(row + ((c16 ^ sw) << 4)) = v;
            } else {
              const int c16 = j * 4 + gq;
              const int hh = fh ^ ((r >> 4) & 1);
              const f32x4 bq = bias_group(j, gq);
              bf16x4 b;
#pragma unroll
              for (int e = 0; e < 4; ++e) {
                if constexpr (DUAL)
                  b[e] = f2bf(silu_f(acc[i][j][4 * gq + e]) * acc[i][j + BJ / 2][4 * gq + e]);
                else
                  b[e] = f2bf(bias_act(acc[i][j][4 * gq + e], bq[e]));
              }
              *reinterpret_cast<bf16x4*>(row + ((c16 ^ sw) << 4) + (hh << 3)) = b;
            }
          }
      }
      __builtin_amdgcn_s_waitcnt(0xC07F);  // lgkmcnt(0): staged writes done
      asm volatile("" ::: "memory");
      constexpr int RPI = 64 / CPRW;  // staged rows per read instruction
      const int cl = lane % CPRW;
      const int n = n0 + wn * OTN + cl * EPC;
      auto flush = [&](auto with_rowmap) __attribute__((always_inline)) {
        // with a row map, every map entry is read before the first store
        int64_t dst_row[with_rowmap ? TM / RPI : 1];
        if constexpr (with_rowmap) {
#pragma unroll
          for (int it = 0; it < TM / RPI; ++it)
            dst_row[it] = g.rowmap[min(m0 + wm * TM + it * RPI + lane / CPRW, M - 1)];
        }
        auto row_out = [&](int it) __attribute__((always_inline)) {
          const int R = it * RPI + lane / CPRW;
          const int m = m0 + wm * TM + R;
          u32x4 d = *reinterpret_cast<const u32x4*>(st + R * ROWB +
                                                    ((cl ^ ((R / RPL) % CPRW)) << 4));
          if (!kF32 && ((R >> 4) & 1)) {
            const uint32_t t0 = d[0], t1 = d[1];
            d[0] = d[2]; d[1] = d[3]; d[2] = t0; d[3] = t1;
          }
          if (m >= M || n >= N) return;
          int64_t drow = m;
          if constexpr (with_rowmap) drow = dst_row[it];
          char* dst = (char*)g.C + (drow * g.ldc + n) * OB;
          if (n + EPC <= N)
            *reinterpret_cast<u32x4*>(dst) = d;
          else  // N % 8 == 4 tail of a bf16 row: the first 8 bytes
            *reinterpret_cast<uint2*>(dst) = make_uint2(d[0], d[1]);
        };
        // fully unrolled with a row map, so that dst_row stays in registers
        if constexpr (with_rowmap) {
#pragma unroll
          for (int it = 0; it < TM / RPI; ++it) row_out(it);
        } else {
#pragma unroll 4
          for (int it = 0; it < TM / RPI; ++it) row_out(it);
        }
      };
      if (has_rowmap)
        flush(std::true_type{});
      else
        flush(std::false_type{});
      return;
    }
  }

  // direct stores (fp32 residual add, outputs too wide to stage, the
  // transposed v columns); all loads first, then all stores
  auto direct = [&](auto with_rowmap, auto with_pre) __attribute__((always_inline)) {
    int64_t orow[BI];
    int vpos_i[BI];
#pragma unroll
    for (int i = 0; i < BI; ++i) {
      const int m = min(m0 + wm * TM + i * 32 + fr, M - 1);
      if constexpr (with_rowmap) orow[i] = g.rowmap[m]; else orow[i] = m;
      if constexpr (EPI == VIT_EPI_QKV_VT) vpos_i[i] = g.vpos[m];
    }
    if constexpr (EPI == VIT_EPI_ADD_F32) {
      constexpr int GI = BI % 2 == 0 ? 2 : 1;  // row blocks per load/store group (divides BI)
#pragma unroll
      for (int i0 = 0; i0 < BI; i0 += GI) {
        // loads of the group (unconditional, clamped in bounds) before its stores
        f32x4 c[GI][BJ][4];
#pragma unroll
        for (int ii = 0; ii < GI; ++ii)
#pragma unroll
          for (int j = 0; j < BJ; ++j)
#pragma unroll
            for (int gq = 0; gq < 4; ++gq) {
              const int n = min(n0 + wn * TN + j * 32 + 8 * gq + c4, N - 4);
              if constexpr (with_pre)
                c[ii][j][gq] = pre[kPre ? i0 + ii : 0][kPre ? j : 0][gq];
              else
                c[ii][j][gq] =
                    *reinterpret_cast<const f32x4*>((const float*)g.C + orow[i0 + ii] * g.ldc + n);
            }
#pragma unroll
        for (int ii = 0; ii < GI; ++ii)
#pragma unroll
          for (int j = 0; j < BJ; ++j)
#pragma unroll
            for (int gq = 0; gq < 4; ++gq) {
              const int i = i0 + ii;
              const int m = m0 + wm * TM + i * 32 + fr;
              const int n = n0 + wn * TN + j * 32 + 8 * gq + c4;
              if (m >= M || n >= N) continue;
              f32x4 v = c[ii][j][gq];
#pragma unroll
              for (int r = 0; r < 4; ++r) v[r] += acc[i][j][4 * gq + r];
              *reinterpret_cast<f32x4*>((float*)g.C + orow[i] * g.ldc + n) = v;
            }
        sched_fence();
      }
      return;
    }
#pragma unroll
    for (int i = 0; i < BI; ++i) {
      const int m = m0 + wm * TM + i * 32 + fr;
      if (m >= M) continue;
      if constexpr (DUAL) {
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
            *reinterpret_cast<bf16x4*>((bf16*)g.C + orow[i] * g.ldc + n) = v;
          }
      } else {
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
              bf16* vt = (bf16*)g.vt + (int64_t)(n - g.rope_cols) * g.vt_ld + vpos_i[i];
#pragma unroll
              for (int r = 0; r < 4; ++r) vt[r * g.vt_ld] = f2bf(v[r]);
            } else if (EPI == VIT_EPI_STORE_F32) {
              *reinterpret_cast<f32x4*>((float*)g.C + orow[i] * g.ldc + n) = v;
            } else {
              const f32x4 bq = bias_group(j, gq);
              bf16x4 b;
#pragma unroll
              for (int r = 0; r < 4; ++r) b[r] = f2bf(bias_act(v[r], bq[r]));
              *reinterpret_cast<bf16x4*>((bf16*)g.C + orow[i] * g.ldc + n) = b;
            }
          }
      }
      sched_fence();  // one row block at a time (bounds live registers)
    }
  };
  if (has_rowmap)
    direct(std::true_type{}, std::false_type{});
  else if (kPre && pre_on)
    direct(std::false_type{}, std::bool_constant<kPre>{});
  else
    direct(std::false_type{}, std::false_type{});
}

// One launch computes one GEMM, or two independent GEMMs of the same tile
// configuration and epilogue (a grouped launch: workgroups below tiles0 take
// g0, the rest g1), which fills the CUs when each alone would leave many idle.
template <int BM, int BN, int BK, int WM, int WN, int STAGES, int EPI, bool DUAL>
__global__ __launch_bounds__(WM * WN * 64, 1) void gemm_mfma_kernel(GemmArgs g0, GemmArgs g1,
                                                                    int tiles0) {
  if ((int)blockIdx.x < tiles0)
    gemm_tile<BM, BN, BK, WM, WN, STAGES, EPI, DUAL>(g0, (int)blockIdx.x);
  else
    gemm_tile<BM, BN, BK, WM, WN, STAGES, EPI, DUAL>(g1, (int)blockIdx.x - tiles0);
}

// The two launches of a column split as one launch with two tile
// configurations of the same thread count: workgroups below tiles0 run tiles of
// configuration 0 over g0's columns, the rest tiles of configuration 1 over
// g1's.  The dispatcher starts workgroups in id order, so the many short tiles
// go first and their CUs then take the remaining long ones; the launch saves
// the boundary between the two launches.
template <int BM0, int BN0, int BK0, int WM0, int WN0, int S0, int BM1, int BN1, int BK1, int WM1,
          int WN1, int S1, int EPI, bool DUAL>
__global__ __launch_bounds__(WM0 * WN0 * 64, 1) void gemm_mfma_pair_kernel(GemmArgs g0, GemmArgs g1,
                                                                         int tiles0) {
  static_assert(WM0 * WN0 == WM1 * WN1, "one workgroup size");
  if ((int)blockIdx.x < tiles0)
    gemm_tile<BM0, BN0, BK0, WM0, WN0, S0, EPI, DUAL>(g0, (int)blockIdx.x);
  else
    gemm_tile<BM1, BN1, BK1, WM1, WN1, S1, EPI, DUAL>(g1, (int)blockIdx.x - tiles0);
}

template <int BM, int BN, int BK, int WM, int WN, int STAGES, int EPI, bool DUAL>
hipError_t mfma_cfg(const GemmArgs& g, hipStream_t s, const GemmArgs* g1 = nullptr) {
  constexpr int BNO = DUAL ? BN / 2 : BN;
  // the ring, then BM floats of per-row RMSNorm scale
  constexpr size_t lds = (size_t)STAGES * (BM + BN) * BK * sizeof(bf16) + BM * sizeof(float);
  auto kern = gemm_mfma_kernel<BM, BN, BK, WM, WN, STAGES, EPI, DUAL>;
  static bool attr = false;
  if (!attr) {
    hipError_t e = hipFuncSetAttribute((const void*)kern,
                                       hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
    if (e != hipSuccess) return e;
    attr = true;
  }
  const int64_t tiles = ((g.M + BM - 1) / BM) * ((g.N + BNO - 1) / BNO);
  const int64_t tiles1 = g1 ? ((g1->M + BM - 1) / BM) * ((g1->N + BNO - 1) / BNO) : 0;
  kern<<<dim3((unsigned)(tiles + tiles1)), dim3(WM * WN * 64), lds, s>>>(g, g1 ? *g1 : g,
                                                                          (int)tiles);
  return hipGetLastError();
}

template <int BM, int BN, int BK, int WM, int WN, int STAGES>
hipError_t mfma_epi(int epi, const GemmArgs& g, hipStream_t s, const GemmArgs* g1 = nullptr) {
  switch (epi) {
    case VIT_EPI_STORE: return mfma_cfg<BM, BN, BK, WM, WN, STAGES, VIT_EPI_STORE, false>(g, s, g1);
    case VIT_EPI_STORE_GATHER:
      return mfma_cfg<BM, BN, BK, WM, WN, STAGES, VIT_EPI_STORE_GATHER, false>(g, s, g1);
    case VIT_EPI_STORE_F32:
      return mfma_cfg<BM, BN, BK, WM, WN, STAGES, VIT_EPI_STORE_F32, false>(g, s, g1);
    case VIT_EPI_ADD_F32:
      // not built for the 256x256 tile (it spills; the dispatcher never picks it)
      if constexpr (!(BM == 256 && BN == 256))
        return mfma_cfg<BM, BN, BK, WM, WN, STAGES, VIT_EPI_ADD_F32, false>(g, s, g1);
      return hipErrorInvalidValue;
    case VIT_EPI_SWIGLU: return mfma_cfg<BM, BN, BK, WM, WN, STAGES, VIT_EPI_SWIGLU, true>(g, s, g1);
    case VIT_EPI_BIAS: return mfma_cfg<BM, BN, BK, WM, WN, STAGES, VIT_EPI_BIAS, false>(g, s, g1);
    case VIT_EPI_BIAS_GELU:
      return mfma_cfg<BM, BN, BK, WM, WN, STAGES, VIT_EPI_BIAS_GELU, false>(g, s, g1);
    case VIT_EPI_STORE_ROPE:
      if constexpr ((BN / WN) % 64 == 0)
        return mfma_cfg<BM, BN, BK, WM, WN, STAGES, VIT_EPI_STORE_ROPE, false>(g, s, g1);
      return hipErrorInvalidValue;
    case VIT_EPI_QKV_VT:
      if constexpr ((BN / WN) % 64 == 0)
        return mfma_cfg<BM, BN, BK, WM, WN, STAGES, VIT_EPI_QKV_VT, false>(g, s, g1);
      return hipErrorInvalidValue;
  }
  return hipErrorInvalidValue;
}

}  // namespace

hipError_t launch_gemm_mfma(int cfg, int epi, const GemmArgs& g, hipStream_t s,
                            const GemmArgs* g1) {
  switch (cfg) {
    case GEMM_MFMA_128x128: return mfma_epi<128, 128, 64, 4, 2, 4>(epi, g, s, g1);
    case GEMM_MFMA_256x128_W8: return mfma_epi<256, 128, 64, 4, 2, 3>(epi, g, s, g1);
    case GEMM_MFMA_256x256_W8: return mfma_epi<256, 256, 32, 2, 4, 4>(epi, g, s, g1);
    case GEMM_MFMA_192x256: return mfma_epi<192, 256, 32, 2, 2, 4>(epi, g, s, g1);
    case GEMM_MFMA_64x64_W2: return mfma_epi<64, 64, 64, 2, 1, 4>(epi, g, s, g1);
  }
  return hipErrorInvalidValue;
}

namespace {

template <int BM, int BN, int BK, int STAGES, bool DUAL>
constexpr size_t gemm_lds_bytes(int epi) {
  return (size_t)STAGES * (BM + BN) * BK * sizeof(bf16) +
         ((epi == VIT_EPI_STORE_F32 || epi == VIT_EPI_ADD_F32) ? 0 : BM * sizeof(float));
}

template <int BM0, int BN0, int BK0, int WM0, int WN0, int S0, int BM1, int BN1, int BK1, int WM1,
          int WN1, int S1, int EPI, bool DUAL>
hipError_t mfma_pair_cfg(const GemmArgs& g0, const GemmArgs& g1, hipStream_t s) {
  constexpr int BNO0 = DUAL ? BN0 / 2 : BN0, BNO1 = DUAL ? BN1 / 2 : BN1;
  constexpr size_t l0 = gemm_lds_bytes<BM0, BN0, BK0, S0, DUAL>(EPI);
  constexpr size_t l1 = gemm_lds_bytes<BM1, BN1, BK1, S1, DUAL>(EPI);
  constexpr size_t lds = l0 > l1 ? l0 : l1;
  auto kern = gemm_mfma_pair_kernel<BM0, BN0, BK0, WM0, WN0, S0, BM1, BN1, BK1, WM1, WN1, S1, EPI,
                                    DUAL>;
  static bool attr = false;
  if (!attr) {
    hipError_t e = hipFuncSetAttribute((const void*)kern,
                                       hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
    if (e != hipSuccess) return e;
    attr = true;
  }
  const int64_t tiles0 = ((g0.M + BM0 - 1) / BM0) * ((g0.N + BNO0 - 1) / BNO0);
  const int64_t tiles1 = ((g1.M + BM1 - 1) / BM1) * ((g1.N + BNO1 - 1) / BNO1);
  kern<<<dim3((unsigned)(tiles0 + tiles1)), dim3(WM0 * WN0 * 64), lds, s>>>(g0, g1, (int)tiles0);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_gemm_mfma_pair(int cfg0, int cfg1, int epi, const GemmArgs& g0,
                                 const GemmArgs& g1, hipStream_t s) {
  // the SwiGLU split of the encoder (short 128x128 tiles first, then 256x256)
  if (cfg0 == GEMM_MFMA_128x128 && cfg1 == GEMM_MFMA_256x256_W8 && epi == VIT_EPI_SWIGLU)
    return mfma_pair_cfg<128, 128, 64, 4, 2, 4, 256, 256, 32, 2, 4, 4, VIT_EPI_SWIGLU, true>(g0, g1,
                                                                                           s);
  return hipErrorNotSupported;
}
