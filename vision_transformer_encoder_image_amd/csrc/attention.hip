// Full bidirectional patch attention over packed images of different grids
// (NeMo Automodel vision page, DeepseekV4VisionAttention: every patch of an image
// attends to every patch of the same image; images are independent, i.e. the
// batch is block-diagonal).  Flash-style single pass with an online softmax, so
// the P_i x P_i score matrix never leaves registers.
//
// head_dim 72 bf16 kernel (gfx950 MFMA; head_dim 64 takes attn_vt_kernel below).
// One workgroup = 256 queries of one (image, head), 8 waves x 32 queries.  V
// comes transposed per head, [H*72, kv_total] with images at 64-aligned
// columns, keys ordered inside each 64-key tile by vt16_slot_key and zero past
// the image (a pack pass before the kernel).  Per 64-key tile:
//   S^T = K . Q^T  on v_mfma_f32_16x16x32_bf16 with K from LDS (A operand, rows =
//        keys) and Q held in registers for the whole kernel (B operand, columns =
//        queries).  Transposing S puts one query per lane column, so the row max
//        of the online softmax is a serial max over the lane's 16 values plus two
//        cross-lane steps, and the running sum needs no cross-lane work until the
//        end.
//   O^T += V^T . P^T  with P^T taken straight from the S^T accumulators (the
//        MFMA k-slots are permuted identically in both operands, so no shuffle
//        is needed) and V^T read from its LDS tile, one 16-byte read per
//        fragment.
// Softmax in base 2 with the 1/sqrt(D) scale folded into log2(e); fp32 state.
// K and V^T tiles are DMA'd into a 4-stage LDS ring two tiles ahead; one
// barrier per tile; waves 4-7 run each tile's O^T MFMAs one step late, out of
// phase with waves 0-3 on the same SIMDs.
//
// fp32 kernel (vector ALU): one thread per query, K/V tiles in LDS, same online
// softmax in base e.  Used by the single-precision mode.
#include <math.h>

#include <type_traits>

#include "common.h"

namespace {

constexpr int BQ = 256, BKV = 64;
// q-tile of the bf16 varlen descriptor: one workgroup (8 waves x 32 queries) of
// either bf16 kernel
constexpr int BQ_DESC = 256;
constexpr int kThreads = 512;

template <int D>
__global__ __launch_bounds__(kThreads, 1) void attn_bf16_kernel(const bf16* __restrict__ qkv,
                                                                const bf16* __restrict__ vt,
                                                                int64_t vt_ld, VarlenDesc desc,
                                                                int H, bf16* __restrict__ out,
                                                                float scale_log2,
                                                                float* __restrict__ lse2) {
  constexpr int DP = (D + 31) / 32 * 32;  // QK contraction length padded to the MFMA k
  constexpr int DO = (D + 15) / 16 * 16;  // output rows padded to the MFMA block
  constexpr int NDS = DP / 32;
  constexpr int NDB = DO / 16;
  // K and V^T tiles are DMA'd global -> LDS (global_load_lds_dwordx4) into a
  // ring of STAGES buffers.  K tile: 64 keys x D/8 16-byte chunks, rows of D
  // elements (an odd number of 16-byte chunks, so 16 lanes reading 16 rows hit
  // distinct banks); V^T tile: D rows x 8 chunks, chunk c of row r stored at
  // c ^ (r & 7).  Both are D/8 copies of 64 lanes; wave w issues copies w,
  // w + 8, ... of the NB per tile.
  static_assert(D % 8 == 0, "16-byte chunks");
  constexpr int STAGES = 4;  // tiles t-1 .. t+2 (see the late waves below)
  constexpr int KCH = D / 8;         // 16-byte chunks per K row
  constexpr int VOFF = BKV * D;      // V^T after K inside a stage (elements)
  constexpr int NB = D / 4;          // 64-lane copies per tile (K and V^T)
  constexpr int WAVES = kThreads / 64;
  __shared__ __attribute__((aligned(16))) bf16 sKV[STAGES][2 * BKV * D];

  // 1D grid over (head, q-tile), dealt so that every XCD gets a contiguous
  // range: the q-tiles of one (image, head) then share that XCD's L2 copy of
  // the image's K and V^T
  const int ntiles = desc.cu_tiles[desc.n_images];
  const int nitems = ntiles * H;
  const int per = nitems / 8, rem = nitems % 8;
  const int xcd = blockIdx.x % 8;
  const int item = xcd * per + min(xcd, rem) + (int)blockIdx.x / 8;
  const int h = item / ntiles, tile = item % ntiles;
  int img = 0;
  while (img + 1 < desc.n_images && tile >= desc.cu_tiles[img + 1]) ++img;
  const int seq0 = desc.cu_seqlens[img], seq1 = desc.cu_seqlens[img + 1];
  const int q0 = seq0 + (tile - desc.cu_tiles[img]) * BQ;
  const int64_t ld = 3 * (int64_t)H * D;
  const bf16* Qb = qkv + h * D;
  const bf16* Kb = qkv + (int64_t)H * D + h * D;
  const bf16* Vb = vt + (int64_t)h * D * vt_ld + desc.kv_off[img] - seq0;  // key kidx at Vb[kidx]

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int fr = lane & 15, fk = lane >> 4;

  bf16x8 qf[2][NDS];
#pragma unroll
  for (int qb = 0; qb < 2; ++qb) {
    const int qrow = q0 + wave * 32 + qb * 16 + fr;
#pragma unroll
    for (int ds = 0; ds < NDS; ++ds) {
      const int d0 = ds * 32 + fk * 8;
      u32x4 v = u32x4{0, 0, 0, 0};
      if (qrow < seq1 && d0 < D) v = ld16(Qb + qrow * ld + d0);
      qf[qb][ds] = __builtin_bit_cast(bf16x8, v);
    }
  }

  const int ncp = NB / WAVES + (wave < NB % WAVES ? 1 : 0);  // copies per tile, this wave
#define VIT_ISSUE(t)                                                                  \
  do {                                                                                \
    const int kv0_ = seq0 + (t) * BKV;                                                \
    bf16* st_ = sKV[(t) % STAGES];                                                    \
    _Pragma("unroll") for (int i = 0; i < (NB + WAVES - 1) / WAVES; ++i) {            \
      const int j_ = wave + WAVES * i;                                                \
      if (j_ < NB) {                                                                  \
        const bf16* src_;                                                             \
        if (j_ < NB / 2) {                                                            \
          const int c_ = j_ * 64 + lane, key_ = c_ / KCH;                             \
          src_ = Kb + (int64_t)min(kv0_ + key_, seq1 - 1) * ld + (c_ % KCH) * 8;       \
        } else {                                                                      \
          const int c_ = (j_ - NB / 2) * 64 + lane, r_ = c_ >> 3;                     \
          src_ = Vb + r_ * vt_ld + kv0_ + (((c_ & 7) ^ (r_ & 7)) << 3);               \
        }                                                                             \
        copy16_to_lds(src_, st_ + j_ * 512);                                          \
      }                                                                               \
    }                                                                                 \
  } while (0)
  // all of tile t's copies of this wave done; the next tile's may be in flight
  auto wait_tile = [&](bool next_in_flight) {
    if (!next_in_flight)
      wait_vmcnt<0>();
    else if (ncp == NB / WAVES + 1)
      wait_vmcnt<NB / WAVES + 1>();
    else
      wait_vmcnt<NB / WAVES>();
  };

  f32x4 o[NDB][2];
#pragma unroll
  for (int db = 0; db < NDB; ++db)
#pragma unroll
    for (int qb = 0; qb < 2; ++qb) o[db][qb] = f32x4{0.f, 0.f, 0.f, 0.f};
  float mrow[2] = {-INFINITY, -INFINITY};
  float lsum[2] = {0.f, 0.f};

  // The two waves that share a SIMD (w and w + 4) run out of phase: waves 4-7
  // ("late") add tile t-1's O^T MFMAs at the start of step t, before tile t's
  // S^T MFMAs, so their softmax meets the other wave's MFMAs.  Tile t-1's stage
  // stays intact through step t (tile t+2 lands in a different one of the 4).
  const bool late = wave >= WAVES / 2;
  bf16x8 pf[BKV / 32][2];
#define VIT_PV(sV_)                                                                   \
  do {                                                                                \
    const bf16* sv_ = (sV_);                                                          \
    _Pragma("unroll") for (int ks = 0; ks < BKV / 32; ++ks)                           \
    _Pragma("unroll") for (int db = 0; db < NDB; ++db) {                              \
      /* V^T slots 8 fk .. 8 fk + 7 of this 32-key half hold keys 4 fk .. 4 fk + 3    \
         and 16 + 4 fk .. 16 + 4 fk + 3, the k-slots of pf (vt16_slot_key); rows     \
         past D (padding of the last 16-row block, discarded) reread row D-1 */      \
      const int vr = min(db * 16 + fr, D - 1);                                        \
      const bf16x8 vf = *reinterpret_cast<const bf16x8*>(                             \
          &sv_[vr * BKV + (((ks * 4 + fk) ^ (vr & 7)) << 3)]);                        \
      _Pragma("unroll") for (int qb = 0; qb < 2; ++qb) o[db][qb] =                    \
          __builtin_amdgcn_mfma_f32_16x16x32_bf16(vf, pf[ks][qb], o[db][qb], 0, 0, 0); \
    }                                                                                 \
  } while (0)

  const int nkv = (seq1 - seq0 + BKV - 1) / BKV;
  VIT_ISSUE(0);
  if (nkv > 1) VIT_ISSUE(1);
  for (int t = 0; t < nkv; ++t) {
    const int kv0 = seq0 + t * BKV;
    wait_tile(t + 1 < nkv);
    // tile t in LDS for every wave, and every wave is done with tile t-2, whose
    // stage tile t+2 reuses
    lds_barrier();
    if (t + 2 < nkv) VIT_ISSUE(t + 2);
    if (late && t > 0) VIT_PV(sKV[(t - 1) % STAGES] + VOFF);
    const bf16* sK = sKV[t % STAGES];

    f32x4 s[4][2];
#pragma unroll
    for (int kb = 0; kb < 4; ++kb)
#pragma unroll
      for (int qb = 0; qb < 2; ++qb) s[kb][qb] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int ds = 0; ds < NDS; ++ds)
#pragma unroll
      for (int kb = 0; kb < 4; ++kb) {
        // chunks past D/8 (the zero-padded part of Q) reread the last one: finite
        // K values times zero Q fragments
        const bf16x8 kf = *reinterpret_cast<const bf16x8*>(
            &sK[(kb * 16 + fr) * D + min(ds * 4 + fk, KCH - 1) * 8]);
#pragma unroll
        for (int qb = 0; qb < 2; ++qb)
          s[kb][qb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(kf, qf[qb][ds], s[kb][qb], 0, 0, 0);
      }

    // online softmax in base 2 with the scale folded into one FMA per score;
    // keys past the image only in the image's last tile; the reference max
    // (mrow, scaled) is raised only when some lane's max grows by more than 2^8,
    // so most tiles skip the rescale of o and of the sum (p then stays <= 2^8)
    if (kv0 + BKV > seq1) {
#pragma unroll
      for (int kb = 0; kb < 4; ++kb)
#pragma unroll
        for (int qb = 0; qb < 2; ++qb)
#pragma unroll
          for (int i = 0; i < 4; ++i)
            if (kv0 + kb * 16 + fk * 4 + i >= seq1) s[kb][qb][i] = -INFINITY;
    }
#pragma unroll
    for (int qb = 0; qb < 2; ++qb) {
      float mx = -INFINITY;
#pragma unroll
      for (int kb = 0; kb < 4; ++kb)
#pragma unroll
        for (int i = 0; i < 4; ++i) mx = fmaxf(mx, s[kb][qb][i]);
      mx = fmaxf(mx, __shfl_xor(mx, 16, 64));
      mx = fmaxf(mx, __shfl_xor(mx, 32, 64));
      const float mxs = mx * scale_log2;
      if (__any(mxs - mrow[qb] > 8.0f)) {
        const float mnew = fmaxf(mrow[qb], mxs);
        const float alpha = __builtin_amdgcn_exp2f(mrow[qb] - mnew);
        mrow[qb] = mnew;
        lsum[qb] *= alpha;
#pragma unroll
        for (int db = 0; db < NDB; ++db)
#pragma unroll
          for (int i = 0; i < 4; ++i) o[db][qb][i] *= alpha;
      }
      const float nm = -mrow[qb];
#pragma unroll
      for (int kb = 0; kb < 4; ++kb)
#pragma unroll
        for (int i = 0; i < 4; ++i)
          s[kb][qb][i] = __builtin_amdgcn_exp2f(fmaf(s[kb][qb][i], scale_log2, nm));
    }

    // probabilities as the bf16 B operand of O^T += V^T P^T; the sum adds the
    // bf16 values the MFMAs use, two per dot2
#pragma unroll
    for (int ks = 0; ks < BKV / 32; ++ks)
#pragma unroll
      for (int qb = 0; qb < 2; ++qb) {
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          pf[ks][qb][i] = f2bf(s[2 * ks][qb][i]);
          pf[ks][qb][4 + i] = f2bf(s[2 * ks + 1][qb][i]);
        }
        const bf16x2 one2 = {(bf16)1.0f, (bf16)1.0f};
        const bf16x8 q8 = pf[ks][qb];
        float u = lsum[qb];
        u = __builtin_amdgcn_fdot2_f32_bf16(__builtin_shufflevector(q8, q8, 0, 1), one2, u, false);
        u = __builtin_amdgcn_fdot2_f32_bf16(__builtin_shufflevector(q8, q8, 2, 3), one2, u, false);
        u = __builtin_amdgcn_fdot2_f32_bf16(__builtin_shufflevector(q8, q8, 4, 5), one2, u, false);
        u = __builtin_amdgcn_fdot2_f32_bf16(__builtin_shufflevector(q8, q8, 6, 7), one2, u, false);
        lsum[qb] = u;
      }
    if (!late) VIT_PV(sKV[t % STAGES] + VOFF);
  }
  if (late && nkv > 0) VIT_PV(sKV[(nkv - 1) % STAGES] + VOFF);
#undef VIT_PV

  const int64_t ldo = (int64_t)H * D;
#pragma unroll
  for (int qb = 0; qb < 2; ++qb) {
    float l = lsum[qb];
    l += __shfl_xor(l, 16, 64);
    l += __shfl_xor(l, 32, 64);
    const float inv = 1.0f / l;
    const int query = q0 + wave * 32 + qb * 16 + fr;
    if (query >= seq1) continue;
    // base-2 log-sum-exp of the scaled scores (mrow is already scaled), for the backward
    if (lse2 && fk == 0) lse2[(int64_t)h * desc.total + query] = mrow[qb] + __log2f(l);
#pragma unroll
    for (int db = 0; db < NDB; ++db) {
      const int d = db * 16 + fk * 4;
      if (d >= D) continue;
      bf16x4 v;
#pragma unroll
      for (int i = 0; i < 4; ++i) v[i] = f2bf(o[db][qb][i] * inv);
      *reinterpret_cast<bf16x4*>(out + query * ldo + h * D + d) = v;
    }
  }
#undef VIT_ISSUE
}


// ---------------------------------------------------------------------------
// bf16 kernel for head_dim 64 with V supplied transposed ([H*64, ld], each
// image's keys starting 64-aligned, padding zero, and the keys of every
// 16-key group stored in the order 0-3, 8-11, 4-7, 12-15: see vt_key_slot).
// K tiles ([key][64]) and V^T tiles ([d][64 key slots]) are plain 128-byte rows,
// copied straight into a 4-stage LDS ring with global_load_lds_dwordx4 (16-byte
// chunks XOR-swizzled per row) with exact vmcnt waits, as in the GEMM.
// Math on v_mfma_f32_32x32x16_bf16: each wave owns 32 queries; per 64-key tile
//   S^T (2 blocks of 32 keys x 32 queries) = K . Q^T   (Q fragments in registers)
//   O^T (2 blocks of 32 dims x 32 queries) += V^T . P^T
// A lane holds one query (column) and 32 of the tile's 64 keys, so the row max
// needs one exchange with lane ^ 32 and the running sum none until the end.
// The k-slot order of P^T is the S^T accumulator order; the V^T key-slot
// permutation makes the matching 8 keys of a lane one contiguous 16-byte read.
// Software pipelining: every step reads the K fragments of tile t+1 and the V^T
// fragments of tile t from LDS and runs the softmax of one tile and the MFMAs
// (S^T of tile t+1, O^T of tile t).  The one barrier per tile keeps the waves in
// step, so the two waves that share a SIMD take opposite orders (softmax first /
// MFMAs first): while one works on the vector ALU the other feeds the matrix
// core.  The softmax reference max is raised only when some lane's max grows by
// more than 2^8 (exact after the final 1/sum; p stays <= 256).
constexpr int VT_BQ = 256, VT_BKV = 64, VT_STAGES = 4, VT_WAVES = 8;
constexpr float VT_RESCALE_LOG2 = 8.0f;

VIT_DEV int vt_swz(int row) { return (row >> 1) & 7; }

__global__ __launch_bounds__(64 * VT_WAVES, 1) void attn_vt_kernel(const bf16* __restrict__ qk, int64_t ldq,
                                                         const bf16* __restrict__ vt,
                                                         int64_t vt_ld, VarlenDesc desc, int H,
                                                         bf16* __restrict__ out, float c,
                                                         float* __restrict__ lse2) {
  __shared__ __attribute__((aligned(16))) bf16 sm[VT_STAGES][2][VT_BKV * 64];
  // 1D grid over (head, q-tile); workgroup ids are dealt round-robin to the 8
  // XCDs, so give every XCD a contiguous range of work items: the q-tiles of one
  // (image, head) then share that XCD's L2 copy of the image's K and V^T
  const int ntiles = desc.cu_tiles[desc.n_images];
  const int nitems = ntiles * H;
  const int per = nitems / 8, rem = nitems % 8;
  const int xcd = blockIdx.x % 8;
  const int item = xcd * per + min(xcd, rem) + (int)blockIdx.x / 8;
  const int h = item / ntiles, tile = item % ntiles;
  int img = 0;
  while (img + 1 < desc.n_images && tile >= desc.cu_tiles[img + 1]) ++img;
  const int seq0 = desc.cu_seqlens[img];
  const int P = desc.cu_seqlens[img + 1] - seq0;
  const int q0 = (tile - desc.cu_tiles[img]) * VT_BQ;  // local query offset
  const int kvo = desc.kv_off[img];
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int fr = lane & 31, fh = lane >> 5;
  const int64_t dm = (int64_t)H * 64;

  // copies per stage: 8 x 1 KB of K rows then 8 x 1 KB of V^T rows; wave w
  // issues copies w and w+8 (one K-row copy, one V^T-row copy)
  const int crow = lane >> 3;
  const int cpc = lane & 7;
#define VIT_ATT_ISSUE(t)                                                                 \
  do {                                                                                   \
    const int kv0_ = (t) * VT_BKV;                                                       \
    _Pragma("unroll") for (int i = 0; i < 16 / VT_WAVES; ++i) {                          \
      const int q_ = wave + VT_WAVES * i;                                                \
      const int r_ = 8 * (q_ & 7) + crow;                                                \
      const int kc_ = cpc ^ vt_swz(r_);                                                  \
      const bf16* src_;                                                                  \
      if (q_ < 8)                                                                        \
        src_ = qk + (int64_t)(seq0 + min(kv0_ + r_, P - 1)) * ldq + dm + h * 64 + kc_ * 8; \
      else                                                                               \
        src_ = vt + (int64_t)(h * 64 + r_) * vt_ld + kvo + kv0_ + kc_ * 8;               \
      copy16_to_lds(src_, &sm[(t) % VT_STAGES][q_ >> 3][(q_ & 7) * 512]);                \
    }                                                                                    \
  } while (0)
  // fragments of one tile: kf[2 ks + kb] = K rows 32 kb + (lane & 31), dims
  // 16 ks + 8 fh .. +7; vf[4 kb + 2 ks2 + db] = V^T rows (dims) 32 db + (lane & 31),
  // key slots 32 kb + 16 ks2 + 8 fh .. +7
#define VIT_ATT_LOADK(stage)                                                             \
  do {                                                                                   \
    const bf16* sK_ = sm[stage][0];                                                      \
    _Pragma("unroll") for (int ks = 0; ks < 4; ++ks)                                     \
    _Pragma("unroll") for (int kb = 0; kb < 2; ++kb) {                                   \
      const int r_ = kb * 32 + fr;                                                       \
      kf[2 * ks + kb] = *reinterpret_cast<const bf16x8*>(                                \
          sK_ + r_ * 64 + (((2 * ks + fh) ^ vt_swz(r_)) << 3));                          \
    }                                                                                    \
  } while (0)
#define VIT_ATT_LOADV(stage)                                                             \
  do {                                                                                   \
    const bf16* sV_ = sm[stage][1];                                                      \
    _Pragma("unroll") for (int kb = 0; kb < 2; ++kb)                                     \
    _Pragma("unroll") for (int ks2 = 0; ks2 < 2; ++ks2)                                  \
    _Pragma("unroll") for (int db = 0; db < 2; ++db) {                                   \
      const int vr_ = db * 32 + fr;                                                      \
      const int ch_ = kb * 4 + ks2 * 2 + fh;                                             \
      vf[4 * kb + 2 * ks2 + db] =                                                        \
          *reinterpret_cast<const bf16x8*>(sV_ + vr_ * 64 + ((ch_ ^ vt_swz(vr_)) << 3)); \
    }                                                                                    \
  } while (0)

  // Q^T fragments (B operand): query q0 + wave*32 + fr, dims 16 ks + 8 fh .. +7
  bf16x8 qf[4];
  {
    const int qi = min(q0 + wave * 32 + fr, P - 1);
    const bf16* qrow = qk + (int64_t)(seq0 + qi) * ldq + h * 64 + fh * 8;
#pragma unroll
    for (int ks = 0; ks < 4; ++ks) qf[ks] = __builtin_bit_cast(bf16x8, ld16(qrow + ks * 16));
  }

  f32x16 o[2] = {f32x16{}, f32x16{}};
  f32x16 sc[2];
  bf16x8 kf[8], vf[8], pf[4];
  float mref = -INFINITY, lsum = 0.f;
  const int nkv = (P + VT_BKV - 1) / VT_BKV;
  constexpr int CPS = 16 / VT_WAVES;  // copies per stage per wave
  VIT_ATT_ISSUE(0);
  if (nkv > 1) VIT_ATT_ISSUE(1);
  if (nkv > 2) VIT_ATT_ISSUE(2);
  if (nkv > 2)
    wait_vmcnt<2 * CPS>();
  else if (nkv > 1)
    wait_vmcnt<CPS>();
  else
    wait_vmcnt<0>();
  lds_barrier();
  VIT_ATT_LOADK(0);
  // consume the scale here: its kernel-argument load would otherwise be waited
  // for (lgkmcnt(0), which also drains the LDS reads) inside the loop
  asm volatile("" : "+s"(c));
  wait_lgkmcnt<0>();
  sched_fence();
  sc[0] = f32x16{};
  sc[1] = f32x16{};
#pragma unroll
  for (int ks = 0; ks < 4; ++ks)
#pragma unroll
    for (int kb = 0; kb < 2; ++kb)
      sc[kb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(kf[2 * ks + kb], qf[ks], sc[kb], 0, 0, 0);

  // online softmax of the scores in sc (keys kv0 .. kv0+63) into pf; rescales
  // o and lsum when the reference max moves
  auto softmax_tile = [&](int kv0) __attribute__((always_inline)) {
    if (kv0 + VT_BKV > P) {  // ragged last tile of the image
#pragma unroll
      for (int kb = 0; kb < 2; ++kb)
#pragma unroll
        for (int i = 0; i < 16; ++i)
          if (kv0 + kb * 32 + (i >> 2) * 8 + fh * 4 + (i & 3) >= P) sc[kb][i] = -INFINITY;
    }
    float mx = -INFINITY;
#pragma unroll
    for (int kb = 0; kb < 2; ++kb)
#pragma unroll
      for (int i = 0; i < 16; ++i) mx = fmaxf(mx, sc[kb][i]);
    mx = xor32_max(mx);
    if (__any((mx - mref) * c > VT_RESCALE_LOG2)) {
      const float mnew = fmaxf(mref, mx);
      const float alpha = __builtin_amdgcn_exp2f((mref - mnew) * c);
      mref = mnew;
      lsum *= alpha;
#pragma unroll
      for (int db = 0; db < 2; ++db) o[db] *= alpha;
    }
    const float nmc = -mref * c;
    // P^T fragment of key slots 32 kb + 16 ks2 + 8 fh .. +7
#pragma unroll
    for (int kb = 0; kb < 2; ++kb)
#pragma unroll
      for (int ks2 = 0; ks2 < 2; ++ks2)
#pragma unroll
        for (int j = 0; j < 8; ++j) {
          const float p = __builtin_amdgcn_exp2f(fmaf(sc[kb][8 * ks2 + j], c, nmc));
          pf[2 * kb + ks2][j] = f2bf(p);
        }
    // the running sum adds the bf16 probabilities that the P.V MFMAs use, two
    // per v_dot2c_f32_bf16 (half the vector-ALU adds), in two chains
    const bf16x2 one2 = {(bf16)1.0f, (bf16)1.0f};
    float s0 = 0.f, s1 = 0.f;
#pragma unroll
    for (int x = 0; x < 4; ++x) {
      s0 = __builtin_amdgcn_fdot2_f32_bf16(__builtin_shufflevector(pf[x], pf[x], 0, 1), one2, s0, false);
      s1 = __builtin_amdgcn_fdot2_f32_bf16(__builtin_shufflevector(pf[x], pf[x], 2, 3), one2, s1, false);
      s0 = __builtin_amdgcn_fdot2_f32_bf16(__builtin_shufflevector(pf[x], pf[x], 4, 5), one2, s0, false);
      s1 = __builtin_amdgcn_fdot2_f32_bf16(__builtin_shufflevector(pf[x], pf[x], 6, 7), one2, s1, false);
    }
    lsum += s0 + s1;
  };
  // S^T of the next tile (K fragments kf) into sc, and O^T += V^T . P^T of
  // this tile (V fragments vf, P^T fragments pf); the S^T MFMAs go first so
  // that their results are ready while the O^T ones still run
  auto mfma_tile = [&]() __attribute__((always_inline)) {
    f32x16 sn[2] = {f32x16{}, f32x16{}};
#pragma unroll
    for (int x = 0; x < 4; ++x) {
      sn[0] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(kf[2 * x], qf[x], sn[0], 0, 0, 0);
      sn[1] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(kf[2 * x + 1], qf[x], sn[1], 0, 0, 0);
    }
#pragma unroll
    for (int x = 0; x < 4; ++x) {
      const int kb = x >> 1, ks2 = x & 1;
      o[0] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(vf[4 * kb + 2 * ks2], pf[x], o[0], 0, 0, 0);
      o[1] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(vf[4 * kb + 2 * ks2 + 1], pf[x], o[1], 0, 0,
                                                     0);
    }
    sc[0] = sn[0];
    sc[1] = sn[1];
  };

  // Two phases, one per half of the workgroup (waves w and w + 4 share a SIMD):
  // waves 0-3 run the softmax of tile t and then its MFMAs; waves 4-7 run the
  // MFMAs of tile t first and the softmax of tile t+1 after them.  Both halves
  // meet at the one barrier per tile, after which one wave of every SIMD works
  // on the vector ALU while the other keeps the matrix cores busy.
  auto run = [&](auto mfma_first) __attribute__((always_inline)) {
    if constexpr (mfma_first) softmax_tile(0);
    for (int t = 0; t < nkv; ++t) {
      // tile t+1 must have landed; the barrier also retires all reads of tile
      // t-1, whose buffer the next copy overwrites
      if (t + 1 < nkv) {
        if (t + 2 < nkv)
          wait_vmcnt<CPS>();
        else
          wait_vmcnt<0>();
      }
      lds_barrier();
      if (t + 3 < nkv) VIT_ATT_ISSUE(t + 3);
      // K of tile t+1 (after the last tile a stale, in-bounds buffer whose
      // products are discarded) and V of tile t
      VIT_ATT_LOADK((t + 1) % VT_STAGES);
      VIT_ATT_LOADV(t % VT_STAGES);
      sched_fence();
      if constexpr (mfma_first) {
        wait_lgkmcnt<0>();
        sched_fence();
        mfma_tile();
        sched_fence();
        if (t + 1 < nkv) softmax_tile((t + 1) * VT_BKV);
      } else {
        softmax_tile(t * VT_BKV);  // covers the latency of the LDS reads
        wait_lgkmcnt<0>();
        sched_fence();
        mfma_tile();
      }
      sched_fence();
    }
  };
  if (wave < VT_WAVES / 2)
    run(std::false_type{});
  else
    run(std::true_type{});
#undef VIT_ATT_ISSUE
#undef VIT_ATT_LOADK
#undef VIT_ATT_LOADV

  const float l = lsum + __shfl_xor(lsum, 32, 64);
  const float inv = 1.0f / l;
  const int qi = q0 + wave * 32 + fr;
  if (qi < P) {
    // base-2 log-sum-exp of the scaled scores, log2(sum 2^(s c)), for the backward
    if (lse2 && fh == 0) lse2[(int64_t)h * desc.total + seq0 + qi] = mref * c + __log2f(l);
    bf16* orow = out + (int64_t)(seq0 + qi) * dm + h * 64;
#pragma unroll
    for (int db = 0; db < 2; ++db)
#pragma unroll
      for (int grp = 0; grp < 4; ++grp) {
        bf16x4 v;
#pragma unroll
        for (int r = 0; r < 4; ++r) v[r] = f2bf(o[db][4 * grp + r] * inv);
        *reinterpret_cast<bf16x4*>(orow + db * 32 + grp * 8 + fh * 4) = v;
      }
  }
}

// ---------------------------------------------------------------------------
constexpr int FQ = 64, FKV = 32;

template <int D>
__global__ __launch_bounds__(FQ) void attn_f32_kernel(const float* __restrict__ qkv,
                                                      VarlenDesc desc, int H,
                                                      float* __restrict__ out, float scale) {
  __shared__ float sK[FKV][D];
  __shared__ float sV[FKV][D];
  const int tile = blockIdx.x, h = blockIdx.y;
  int img = 0;
  while (img + 1 < desc.n_images && tile >= desc.cu_tiles[img + 1]) ++img;
  const int seq0 = desc.cu_seqlens[img], seq1 = desc.cu_seqlens[img + 1];
  const int query = seq0 + (tile - desc.cu_tiles[img]) * FQ + threadIdx.x;
  const int64_t ld = 3 * (int64_t)H * D;
  const bool valid = query < seq1;
  float q[D], o[D];
#pragma unroll
  for (int e = 0; e < D; ++e) {
    q[e] = valid ? qkv[query * ld + h * D + e] : 0.f;
    o[e] = 0.f;
  }
  float m = -INFINITY, l = 0.f;
  for (int kv0 = seq0; kv0 < seq1; kv0 += FKV) {
    for (int idx = threadIdx.x; idx < FKV * D; idx += FQ) {
      const int j = idx / D, e = idx % D;
      const int key = kv0 + j;
      sK[j][e] = key < seq1 ? qkv[key * ld + (int64_t)H * D + h * D + e] : 0.f;
      sV[j][e] = key < seq1 ? qkv[key * ld + 2 * (int64_t)H * D + h * D + e] : 0.f;
    }
    __syncthreads();
    const int nj = min(FKV, seq1 - kv0);
    for (int j = 0; j < nj; ++j) {
      float sdot = 0.f;
#pragma unroll
      for (int e = 0; e < D; ++e) sdot = fmaf(q[e], sK[j][e], sdot);
      const float sc = sdot * scale;
      const float mnew = fmaxf(m, sc);
      const float a = expf(m - mnew);
      const float p = expf(sc - mnew);
      l = l * a + p;
#pragma unroll
      for (int e = 0; e < D; ++e) o[e] = o[e] * a + p * sV[j][e];
      m = mnew;
    }
    __syncthreads();
  }
  if (!valid) return;
  const float inv = 1.0f / l;
#pragma unroll
  for (int e = 0; e < D; ++e) out[query * (int64_t)H * D + h * D + e] = o[e] * inv;
}

}  // namespace

int attention_q_tile(int dtype, int /*head_dim*/) { return dtype == VIT_BF16 ? BQ_DESC : FQ; }

hipError_t launch_attention_vt(const void* qk, int64_t ld_qk, const void* vt, int64_t vt_ld,
                               const VarlenDesc& d, int n_heads, void* out, hipStream_t s,
                               float* lse2) {
  static_assert(VT_BQ == BQ_DESC && BQ == BQ_DESC, "both bf16 kernels share the q-tile descriptor");
  const int tiles = d.cu_tiles[d.n_images];
  if (tiles == 0) return hipSuccess;
  const float c = (float)(1.4426950408889634 / 8.0);  // log2(e) / sqrt(64)
  attn_vt_kernel<<<dim3((unsigned)(tiles * n_heads)), 64 * VT_WAVES, 0, s>>>(
      (const bf16*)qk, ld_qk, (const bf16*)vt, vt_ld, d, n_heads, (bf16*)out, c, lse2);
  return hipGetLastError();
}

hipError_t launch_attention(int dtype, const void* qkv, const void* vt, int64_t vt_ld,
                            const VarlenDesc& d, int n_heads, int head_dim, void* out,
                            hipStream_t s, float* lse2) {
  const int tiles = d.cu_tiles[d.n_images];
  if (tiles == 0) return hipSuccess;
  if (dtype == VIT_BF16) {
    const float sl2 = (float)(1.4426950408889634 / sqrt((double)head_dim));
    if (head_dim != 72 || !vt || vt_ld < d.kv_off[d.n_images] || vt_ld % 8)
      return hipErrorInvalidValue;
    attn_bf16_kernel<72><<<dim3((unsigned)(tiles * n_heads)), kThreads, 0, s>>>(
        (const bf16*)qkv, (const bf16*)vt, vt_ld, d, n_heads, (bf16*)out, sl2, lse2);
  } else {
    if (lse2) return hipErrorInvalidValue;
    const dim3 grid((unsigned)tiles, (unsigned)n_heads);
    const float sc = (float)(1.0 / sqrt((double)head_dim));
    if (head_dim == 64)
      attn_f32_kernel<64><<<grid, FQ, 0, s>>>((const float*)qkv, d, n_heads, (float*)out, sc);
    else if (head_dim == 72)
      attn_f32_kernel<72><<<grid, FQ, 0, s>>>((const float*)qkv, d, n_heads, (float*)out, sc);
    else
      return hipErrorInvalidValue;
  }
  return hipGetLastError();
}
