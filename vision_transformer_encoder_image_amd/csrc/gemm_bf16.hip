// bf16 MFMA GEMM for gfx950: C[M,N] = epilogue(A[M,K] . B[N,K]^T).
//
// Both operands are K-contiguous (activations [tokens, in], weights [out, in]),
// so every lane fetches 16-byte runs along K for both MFMA operands.  Tile
// 128x128x64, 256 threads = 4 waves in a 2x2 arrangement, each wave owning a
// 64x64 sub-tile as 4x4 v_mfma_f32_16x16x32_bf16 blocks with fp32 accumulators.
// A and B tiles are double-buffered in LDS (XOR-swizzled 16-byte chunks) and the
// next K-tile is prefetched into registers while the current one is multiplied.
// Workgroups are remapped so that the tiles running on one XCD (workgroup ids
// are dealt round-robin over the 8 XCDs) form a contiguous band of the grouped
// tile order, which keeps shared A rows / B panels inside that XCD's L2.
//
// Epilogues: store bf16, store fp32, fp32 residual add in place, and the SwiGLU
// pair (two B matrices; the B tile holds 32 gate rows then 32 up rows for each
// wave column so that silu(gate) * up meets in the same lane).
#include "common.h"
#include "gemm_mfma.h"

namespace {

constexpr int BM = 128, BN = 128, BK = 64;
constexpr int kThreads = 256;
constexpr int kGroupM = 8;              // m-tiles per band of the grouped order
constexpr int kXcds = 8;

VIT_DEV int swz(int row, int kc) { return row * BK + ((kc ^ (row & 7)) << 3); }

VIT_DEV float silu(float g) { return g / (1.0f + __expf(-g)); }

// Logical tile index of this workgroup after the XCD remap.
VIT_DEV int xcd_remap(int bid, int ntiles) {
  const int per = ntiles / kXcds, rem = ntiles % kXcds;
  const int xcd = bid % kXcds, idx = bid / kXcds;
  return xcd * per + min(xcd, rem) + idx;
}

// Source of LDS B-tile row r.  SwiGLU tiles interleave the two weight matrices:
// rows 64c..64c+31 are gate rows n0+32c.., rows 64c+32..64c+63 the matching up rows.
template <bool DUAL>
VIT_DEV const bf16* b_row_src(const bf16* B, const bf16* B2, int n0, int N, int64_t ldb, int r,
                              int kc) {
  int brow = n0 + r;
  const bf16* base = B;
  if (DUAL) {
    const int wc = r >> 6, within = r & 63;
    brow = n0 + wc * 32 + (within & 31);
    base = (within >> 5) ? B2 : B;
  }
  return base + (int64_t)min(brow, N - 1) * ldb + kc * 8;
}

template <int EPI, bool DUAL>
__global__ __launch_bounds__(kThreads, 2) void gemm_bf16_kernel(GemmArgs g) {
  __shared__ __attribute__((aligned(16))) bf16 sA[2][BM * BK];
  __shared__ __attribute__((aligned(16))) bf16 sB[2][BN * BK];

  const bf16* __restrict__ A = (const bf16*)g.A;
  const bf16* __restrict__ B = (const bf16*)g.B;
  const bf16* __restrict__ B2 = (const bf16*)g.B2;
  const int M = (int)g.M, N = (int)g.N, K = (int)g.K, KB = (int)g.kb;
  constexpr int BNO = DUAL ? BN / 2 : BN;  // output columns per tile
  const int tiles_m = (M + BM - 1) / BM;
  const int tiles_n = (N + BNO - 1) / BNO;
  const int ntiles = tiles_m * tiles_n;

  // grouped order: bands of kGroupM m-tiles, n-major inside a band
  const int L = xcd_remap(blockIdx.x, ntiles);
  const int band = kGroupM * tiles_n;
  const int first_m = (L / band) * kGroupM;
  const int gm = min(tiles_m - first_m, kGroupM);
  const int tm = first_m + (L % band) % gm;
  const int tn = (L % band) / gm;
  const int m0 = tm * BM, n0 = tn * BNO;

  const int tid = threadIdx.x;
  const int lane = tid & 63, wave = tid >> 6;
  const int wm = wave >> 1, wn = wave & 1;

  // global -> register staging: each thread moves 4 chunks of A and 4 of B per
  // K-tile (rows ld_row + 32 i, 16-byte chunk ld_kc)
  const int ld_row = tid >> 3;
  const int ld_kc = tid & 7;
  const bf16* a_src0 = A + (int64_t)min(m0 + ld_row, M - 1) * g.lda + ld_kc * 8;
  const bf16* a_src1 = A + (int64_t)min(m0 + ld_row + 32, M - 1) * g.lda + ld_kc * 8;
  const bf16* a_src2 = A + (int64_t)min(m0 + ld_row + 64, M - 1) * g.lda + ld_kc * 8;
  const bf16* a_src3 = A + (int64_t)min(m0 + ld_row + 96, M - 1) * g.lda + ld_kc * 8;
  const bf16* b_src0 = b_row_src<DUAL>(B, B2, n0, N, g.ldb, ld_row, ld_kc);
  const bf16* b_src1 = b_row_src<DUAL>(B, B2, n0, N, g.ldb, ld_row + 32, ld_kc);
  const bf16* b_src2 = b_row_src<DUAL>(B, B2, n0, N, g.ldb, ld_row + 64, ld_kc);
  const bf16* b_src3 = b_row_src<DUAL>(B, B2, n0, N, g.ldb, ld_row + 96, ld_kc);
  const int s_off0 = swz(ld_row, ld_kc), s_off1 = swz(ld_row + 32, ld_kc);
  const int s_off2 = swz(ld_row + 64, ld_kc), s_off3 = swz(ld_row + 96, ld_kc);
  u32x4 ra0, ra1, ra2, ra3, rb0, rb1, rb2, rb3;

#define VIT_LOAD_TILE(k0)                                      \
  do {                                                         \
    if (((k0) + ld_kc * 8) < K) {                              \
      ra0 = ld16(a_src0 + (k0));                               \
      ra1 = ld16(a_src1 + (k0));                               \
      ra2 = ld16(a_src2 + (k0));                               \
      ra3 = ld16(a_src3 + (k0));                               \
    } else {                                                   \
      ra0 = ra1 = ra2 = ra3 = u32x4{0, 0, 0, 0};               \
    }                                                          \
    if (((k0) + ld_kc * 8) < KB) {                             \
      rb0 = ld16(b_src0 + (k0));                               \
      rb1 = ld16(b_src1 + (k0));                               \
      rb2 = ld16(b_src2 + (k0));                               \
      rb3 = ld16(b_src3 + (k0));                               \
    } else {                                                   \
      rb0 = rb1 = rb2 = rb3 = u32x4{0, 0, 0, 0};               \
    }                                                          \
  } while (0)
#define VIT_STORE_TILE(buf)                                       \
  do {                                                            \
    st16(&sA[buf][s_off0], ra0);            \
    st16(&sA[buf][s_off1], ra1);            \
    st16(&sA[buf][s_off2], ra2);            \
    st16(&sA[buf][s_off3], ra3);            \
    st16(&sB[buf][s_off0], rb0);            \
    st16(&sB[buf][s_off1], rb1);            \
    st16(&sB[buf][s_off2], rb2);            \
    st16(&sB[buf][s_off3], rb3);            \
  } while (0)

  f32x4 acc[4][4];
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j) acc[i][j] = f32x4{0.f, 0.f, 0.f, 0.f};

  const int nk = (K + BK - 1) / BK;
  VIT_LOAD_TILE(0);
  VIT_STORE_TILE(0);
  __syncthreads();

  const int fr = lane & 15;   // fragment row inside a 16-row block
  const int fk = lane >> 4;   // 8-element k-chunk inside a 32-wide k step
  for (int kt = 0; kt < nk; ++kt) {
    const int cur = kt & 1;
    if (kt + 1 < nk) VIT_LOAD_TILE((kt + 1) * BK);
#pragma unroll
    for (int ks = 0; ks < BK / 32; ++ks) {
      bf16x8 af[4], bfr[4];
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int r = wm * 64 + i * 16 + fr;
        af[i] = *reinterpret_cast<const bf16x8*>(&sA[cur][swz(r, ks * 4 + fk)]);
      }
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const int r = wn * 64 + j * 16 + fr;
        bfr[j] = *reinterpret_cast<const bf16x8*>(&sB[cur][swz(r, ks * 4 + fk)]);
      }
#pragma unroll
      for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j)
          acc[i][j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(af[i], bfr[j], acc[i][j], 0, 0, 0);
    }
    if (kt + 1 < nk) VIT_STORE_TILE(cur ^ 1);
    __syncthreads();
  }
#undef VIT_LOAD_TILE
#undef VIT_STORE_TILE

  // epilogue: lane holds column (lane & 15) and rows 4*(lane >> 4) + r of each block
  const int col_in = lane & 15;
  const int row_in = (lane >> 4) * 4;
  if (DUAL) {
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
      for (int j = 0; j < 2; ++j) {
        const int n = n0 + wn * 32 + j * 16 + col_in;
        if (n >= N) continue;
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          const int m = m0 + wm * 64 + i * 16 + row_in + r;
          if (m >= M) continue;
          const float v = silu(acc[i][j][r]) * acc[i][j + 2][r];
          ((bf16*)g.C)[(int64_t)m * g.ldc + n] = f2bf(v);
        }
      }
  } else {
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const int n = n0 + wn * 64 + j * 16 + col_in;
        if (n >= N) continue;
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          const int m = m0 + wm * 64 + i * 16 + row_in + r;
          if (m >= M) continue;
          const int64_t orow = g.rowmap ? (int64_t)g.rowmap[m] : (int64_t)m;
          const float v = acc[i][j][r];
          if (EPI == VIT_EPI_STORE) {
            ((bf16*)g.C)[orow * g.ldc + n] = f2bf(v);
          } else if (EPI == VIT_EPI_STORE_F32) {
            ((float*)g.C)[orow * g.ldc + n] = v;
          } else {  // VIT_EPI_ADD_F32
            float* c = (float*)g.C + orow * g.ldc + n;
            *c = *c + v;
          }
        }
      }
  }
}

}  // namespace

namespace {

hipError_t launch_simple(int epilogue, const GemmArgs& g, hipStream_t s) {
  const bool dual = epilogue == VIT_EPI_SWIGLU;
  const int64_t bno = dual ? BN / 2 : BN;
  const int64_t tiles = ((g.M + BM - 1) / BM) * ((g.N + bno - 1) / bno);
  const dim3 grid((unsigned)tiles);
  switch (epilogue) {
    case VIT_EPI_STORE:
      gemm_bf16_kernel<VIT_EPI_STORE, false><<<grid, kThreads, 0, s>>>(g);
      break;
    case VIT_EPI_STORE_F32:
      gemm_bf16_kernel<VIT_EPI_STORE_F32, false><<<grid, kThreads, 0, s>>>(g);
      break;
    case VIT_EPI_ADD_F32:
      gemm_bf16_kernel<VIT_EPI_ADD_F32, false><<<grid, kThreads, 0, s>>>(g);
      break;
    case VIT_EPI_SWIGLU:
      gemm_bf16_kernel<VIT_EPI_SWIGLU, true><<<grid, kThreads, 0, s>>>(g);
      break;
    default:
      return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

bool pipe_eligible(const GemmArgs& g) {
  const uintptr_t al = (uintptr_t)g.A | (uintptr_t)g.B | (uintptr_t)(g.B2 ? g.B2 : g.B) |
                       (uintptr_t)g.C;
  // the copies address A and B with 32-bit byte offsets from the matrix base
  const int64_t lim = (int64_t)1 << 32;
  // a gathered A operand: four source segments of a_seg columns (multiples of the
  // K-tile), rows addressed inside its a_src_rows x lda source matrix
  const bool gather_ok = !g.a_rows || (g.a_seg > 0 && g.a_seg % 64 == 0 && g.K == 4 * g.a_seg &&
                                       g.lda >= g.a_seg && ((uintptr_t)g.a_rows & 15) == 0 &&
                                       g.a_src_rows > 0 && g.a_src_rows * g.lda * 2 < lim);
  return g.K % 64 == 0 && g.kb % 8 == 0 && g.kb <= g.K && g.N % 4 == 0 && g.ldc % 4 == 0 &&
         g.lda % 8 == 0 && g.ldb % 8 == 0 && (al & 15) == 0 &&
         (g.a_rows || g.M * g.lda * 2 < lim) && g.N * g.ldb * 2 < lim && gather_ok;
}

}  // namespace

// Tile configuration by a wave-quantisation cost model: cost ~ (rounds of one
// workgroup per CU) x (tile area / relative efficiency per flop).  Fitted to
// gfx950 timings of the encoder's GEMM shapes (with the folded-RMSNorm work):
// per flop, relative to a 4-wave 128x128 tile, the 8-wave 128x128 tile is
// ~1.13x, the 8-wave 256x128 tile ~1.18x, the 4-wave 192x256 tile ~1.26x and
// the 8-wave 256x256 tile ~1.57x as efficient; with the fp32 read-modify-write
// epilogue, whose traffic grows with the tile, 1.04x / 1.1x / 1.2x, and the
// 256x256 tile (which spills with it) is not used.  The 4-wave 128x128 tile is
// not built: the 8-wave one was never slower.  Every tile takes the
// folded-RMSNorm producer (its wave sub-tiles are whole 64-column groups).
namespace {

struct TileOpt {
  int cfg, bm, bn;
  double eff;
  bool ok;
  int per_cu;  // workgroups that fit on one CU at once (LDS)
};

constexpr int kCUs = 256;
constexpr int kTileOpts = 5;

// The 2-wave 64x64 tile (64 KB of LDS, two workgroups per CU) is ~0.33x as
// efficient per flop, fitted to the 784-row encoder GEMMs of one 28x28 image:
// out-projection 15.8 -> 12.4 us, down-projection 27.0 -> 20.9 us, aligner
// (196 x 4096 x 4096) 29.2 -> 24.0 us, patch embedding 11.6 -> 10.2 us against
// the 128x128 tile; on the ragged batch's shapes it loses (out-projection 25.4
// against 20.7 us), which the model reproduces.
int tile_opts(int epilogue, TileOpt* o) {
  const bool rmw = epilogue == VIT_EPI_ADD_F32;
  o[0] = {GEMM_MFMA_128x128, 128, 128, rmw ? 1.04 : 1.13, true, 1};
  o[1] = {GEMM_MFMA_256x128_W8, 256, 128, rmw ? 1.1 : 1.18, true, 1};
  o[2] = {GEMM_MFMA_256x256_W8, 256, 256, 1.57, !rmw, 1};
  o[3] = {GEMM_MFMA_192x256, 192, 256, rmw ? 1.2 : 1.26, true, 1};
  o[4] = {GEMM_MFMA_64x64_W2, 64, 64, rmw ? 0.33 : 0.34, true, 2};
  return kTileOpts;
}

// output columns of one tile (the SwiGLU tile holds gate and up halves)
int64_t tile_cols(const TileOpt& o, int epilogue) {
  return epilogue == VIT_EPI_SWIGLU ? o.bn / 2 : o.bn;
}

double tile_cost(const TileOpt& o, int epilogue, int64_t M, int64_t N) {
  const int64_t bno = tile_cols(o, epilogue);
  const int64_t tiles = ((M + o.bm - 1) / o.bm) * ((N + bno - 1) / bno);
  const int64_t slots = (int64_t)kCUs * o.per_cu;
  return (double)((tiles + slots - 1) / slots) * o.bm * o.bn / o.eff;
}

int best_tile(int epilogue, int64_t M, int64_t N, double* cost) {
  TileOpt opts[kTileOpts];
  const int n = tile_opts(epilogue, opts);
  int best = GEMM_MFMA_128x128;
  double best_cost = 1e300;
  for (int i = 0; i < n; ++i) {
    if (!opts[i].ok) continue;
    const double c = tile_cost(opts[i], epilogue, M, N);
    if (c < best_cost) {
      best_cost = c;
      best = opts[i].cfg;
    }
  }
  if (cost) *cost = best_cost;
  return best;
}

// A split adds a launch whose own ramp-up and drain are not hidden by the
// first one's; in the model's units (a 128x128 round ~ 14.5e3 ~ 11 us) ~1 us.
constexpr double kSplitPenalty = 1.3e3;

}  // namespace

int gemm_mfma_choice(int epilogue, int64_t M, int64_t N) {
  return best_tile(epilogue, M, N, nullptr);
}

// Column split: when a wide GEMM's best single tile leaves a ragged last round
// (e.g. SwiGLU gate/up at M = 3,562: five rounds of 128x128 tiles, or a
// second 256x256 round holding 52 of 308 tiles), one launch of large tiles
// covers the columns that fill exactly one round and a second launch of
// smaller tiles covers the rest.  Only epilogues whose arithmetic does not
// depend on the absolute column take it (not the rotary or transposed-V forms;
// the folded-norm producer's second launch gets its columns' norm weights and
// its columns of u and of the partial sums, with the full rows' strides).
GemmSplit gemm_mfma_split(int epilogue, int64_t M, int64_t N) {
  GemmSplit best{};
  double best_cost;
  best.cfg_main = best_tile(epilogue, M, N, &best_cost);
  best.n_main = N;
  best.cfg_tail = -1;
  const bool col_free = epilogue == VIT_EPI_STORE || epilogue == VIT_EPI_STORE_GATHER ||
                        epilogue == VIT_EPI_STORE_F32 ||
                        epilogue == VIT_EPI_ADD_F32 || epilogue == VIT_EPI_SWIGLU ||
                        epilogue == VIT_EPI_BIAS || epilogue == VIT_EPI_BIAS_GELU;
  if (!col_free) return best;
  TileOpt opts[kTileOpts];
  tile_opts(epilogue, opts);
  // largest tiles first: at equal cost the large-tile launch is the main one
  for (const int i : {2, 3, 1, 0}) {
    const TileOpt& o = opts[i];
    if (!o.ok) continue;
    const int64_t bno = tile_cols(o, epilogue);
    const int64_t row_tiles = (M + o.bm - 1) / o.bm;
    const int64_t n_main = (kCUs / row_tiles) * bno;
    if (n_main <= 0 || n_main >= N) continue;
    double tail_cost;
    const int tail = best_tile(epilogue, M, N - n_main, &tail_cost);
    const double c = o.bm * o.bn / o.eff + tail_cost + kSplitPenalty;
    if (c < best_cost) {
      best_cost = c;
      best.cfg_main = o.cfg;
      best.n_main = n_main;
      best.cfg_tail = tail;
    }
  }
  return best;
}

// Two independent GEMMs of one epilogue in one launch (e.g. weight gradients
// whose tiles together fill the CUs once): the tile configuration is chosen by
// the same cost model over the combined tile count.  Plain epilogues only (no
// folded norm, rotary or row map); otherwise, or when either GEMM cannot take
// the MFMA path, two ordinary launches.
hipError_t launch_gemm_bf16_pair(int epilogue, const GemmArgs& g0, const GemmArgs& g1,
                                 hipStream_t s) {
  const bool plain = epilogue == VIT_EPI_STORE || epilogue == VIT_EPI_STORE_F32;
  const bool simple = !g0.norm_w && !g0.ss_in && !g1.norm_w && !g1.ss_in && !g0.rowmap &&
                      !g1.rowmap;
  if (!plain || !simple || !pipe_eligible(g0) || !pipe_eligible(g1) || g0.M == 0 || g0.N == 0 ||
      g1.M == 0 || g1.N == 0) {
    const hipError_t e = launch_gemm_bf16(epilogue, g0, s);
    if (e != hipSuccess) return e;
    return launch_gemm_bf16(epilogue, g1, s);
  }
  TileOpt opts[kTileOpts];
  tile_opts(epilogue, opts);
  int best = GEMM_MFMA_128x128;
  double best_cost = 1e300;
  for (const TileOpt& o : opts) {
    if (!o.ok) continue;
    const int64_t bno = tile_cols(o, epilogue);
    const int64_t tiles = ((g0.M + o.bm - 1) / o.bm) * ((g0.N + bno - 1) / bno) +
                          ((g1.M + o.bm - 1) / o.bm) * ((g1.N + bno - 1) / bno);
    const int64_t slots = (int64_t)kCUs * o.per_cu;
    const double c = (double)((tiles + slots - 1) / slots) * o.bm * o.bn / o.eff;
    if (c < best_cost) {
      best_cost = c;
      best = o.cfg;
    }
  }
  return launch_gemm_mfma(best, epilogue, g0, s, &g1);
}

bool gemm_bf16_can_fuse_rope(const GemmArgs& g) { return pipe_eligible(g); }

bool gemm_bf16_mfma_eligible(const GemmArgs& g) { return pipe_eligible(g); }

hipError_t launch_gemm_bf16(int epilogue, const GemmArgs& g, hipStream_t s) {
  if (g.M == 0 || g.N == 0) return hipSuccess;
  const bool rope = epilogue == VIT_EPI_STORE_ROPE || epilogue == VIT_EPI_QKV_VT;
  const bool norm = g.norm_w != nullptr || g.ss_in != nullptr;
  const bool bias = epilogue == VIT_EPI_BIAS || epilogue == VIT_EPI_BIAS_GELU;
  const bool gather = epilogue == VIT_EPI_STORE_GATHER;
  if (gather != (g.a_rows != nullptr)) return hipErrorInvalidValue;
  if ((rope || norm || bias || gather) && !pipe_eligible(g)) return hipErrorInvalidValue;
  if (bias && (!g.bias || norm)) return hipErrorInvalidValue;
  if (g.ss_in && (g.ss_groups < 1 || g.ss_groups > kMaxNormGroups)) return hipErrorInvalidValue;
  if (g.norm_w && (g.N % 64 != 0 || !g.norm_out || !g.ss_out ||
                   (epilogue != VIT_EPI_STORE_F32 && epilogue != VIT_EPI_ADD_F32)))
    return hipErrorInvalidValue;
  if (pipe_eligible(g)) {
    if (rope) {
      const int cfg = gemm_mfma_choice(VIT_EPI_STORE, g.M, g.N);
      return launch_gemm_mfma(cfg, epilogue, g, s);
    }
    const GemmSplit sp = gemm_mfma_split(epilogue, g.M, g.N);
    if (sp.n_main == g.N) return launch_gemm_mfma(sp.cfg_main, epilogue, g, s);
    GemmArgs a = g, b = g;
    a.N = sp.n_main;
    b.N = g.N - sp.n_main;
    const int64_t out_bytes =
        epilogue == VIT_EPI_STORE_F32 || epilogue == VIT_EPI_ADD_F32 ? 4 : 2;
    b.B = (const bf16*)g.B + sp.n_main * g.ldb;
    if (g.B2) b.B2 = (const bf16*)g.B2 + sp.n_main * g.ldb;
    b.C = (char*)g.C + sp.n_main * out_bytes;
    if (g.bias) b.bias = g.bias + sp.n_main;
    if (g.norm_w) {  // folded-norm producer: the tail writes its columns of u and ss
      a.ld_norm_out = b.ld_norm_out = g.ld_norm_out ? g.ld_norm_out : g.N;
      a.ld_ss_out = b.ld_ss_out = g.ld_ss_out ? g.ld_ss_out : (g.N / 64 + 3) & ~3;
      b.norm_w = g.norm_w + sp.n_main;
      b.norm_out = (bf16*)g.norm_out + sp.n_main;
      b.ss_out = g.ss_out + sp.n_main / 64;
    }
    // one launch when that pair of tile configurations is built, whichever of the
    // two covers the main columns (the built pair puts the 128x128 tiles first)
    hipError_t ep = launch_gemm_mfma_pair(sp.cfg_tail, sp.cfg_main, epilogue, b, a, s);
    if (ep == hipErrorNotSupported)
      ep = launch_gemm_mfma_pair(sp.cfg_main, sp.cfg_tail, epilogue, a, b, s);
    if (ep != hipErrorNotSupported) return ep;
    const hipError_t e = launch_gemm_mfma(sp.cfg_main, epilogue, a, s);
    if (e != hipSuccess) return e;
    return launch_gemm_mfma(sp.cfg_tail, epilogue, b, s);
  }
  return launch_simple(epilogue, g, s);
}
