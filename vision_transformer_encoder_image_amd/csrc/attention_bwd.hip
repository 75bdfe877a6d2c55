// Backward of the full bidirectional patch attention (NeMo Automodel vision
// page, DeepseekV4VisionAttention: per image and head, O = softmax(Q K^T /
// sqrt(D)) V), bf16 with head_dim 64 (and 72, below), varlen (block-diagonal).  With each
// query's log-sum-exp saved by the forward (base 2, lse2), P is recomputed
// tile by tile; with Dq = rowsum(dO * O):
//   dS = P (dO V^T - Dq),  dQ = dS K / sqrt(D),  dK = dS^T Q / sqrt(D),  dV = P^T dO.
// Two kernels, no atomics (deterministic):
//   attn_dq_kernel   32 queries per wave; per 64-key tile: S^T = K Q^T,
//                    dP^T = V dO^T (Q, dO fragments in registers), then
//                    dQ^T += K^T dS^T with dS^T straight from the accumulators;
//   attn_dkv_kernel  32 keys per wave; per 64-query tile: S = Q K^T, dP = dO V^T
//                    (K, V fragments in registers), then dV^T += dO^T P and
//                    dK^T += Q^T dS.
// The transposed operands (K^T, Q^T, dO^T) use the layout of the forward's V^T:
// [H*64, sum of 64-aligned image spans], the 16-key groups permuted as
// vt_key_slot, so a lane's 8 contraction slots match the 8 accumulator rows it
// holds.  Tiles are copied into LDS with global_load_lds_dwordx4 (16-byte chunks
// XOR-swizzled per 128-byte row), double-buffered, one barrier per tile.
#include <type_traits>

#include "common.h"

namespace {

constexpr int AB_WAVES = 4;              // waves per workgroup
constexpr int AB_ROWS = 32 * AB_WAVES;   // queries (dQ) or keys (dK, dV) per workgroup
constexpr int AB_T = 64;                 // inner tile: keys (dQ) or queries (dK, dV)
constexpr int kThreads = 256;

VIT_DEV int ab_swz(int row) { return (row >> 1) & 7; }

// Dq[h * total + p] = sum over e < D of dO[p, h*D + e] * O[p, h*D + e]
template <int D>
__global__ __launch_bounds__(kThreads) void rowdot_kernel(const bf16* __restrict__ dO,
                                                          const bf16* __restrict__ O, int64_t P,
                                                          int H, float* __restrict__ Dq) {
  static_assert(D % 8 == 0, "16-byte chunks");
  const int64_t i = (int64_t)blockIdx.x * kThreads + threadIdx.x;
  if (i >= P * H) return;
  const int64_t p = i / H;
  const int h = (int)(i % H);
  const int64_t base = p * (int64_t)H * D + h * D;
  float t = 0.f;
#pragma unroll
  for (int c = 0; c < D / 8; ++c) {
    const bf16x8 a = __builtin_bit_cast(bf16x8, ld16(dO + base + 8 * c));
    const bf16x8 b = __builtin_bit_cast(bf16x8, ld16(O + base + 8 * c));
#pragma unroll
    for (int e = 0; e < 8; ++e) t += bf2f(a[e]) * bf2f(b[e]);
  }
  Dq[(int64_t)h * P + p] = t;
}

// work item -> (head, tile), every XCD a contiguous range (as the forward)
struct Item {
  int h, img, seq0, P, r0;
};
VIT_DEV Item ab_item(const VarlenDesc& desc, int H) {
  const int ntiles = desc.cu_tiles[desc.n_images];
  const int nitems = ntiles * H;
  const int per = nitems / 8, rem = nitems % 8;
  const int xcd = blockIdx.x % 8;
  const int item = xcd * per + min(xcd, rem) + (int)blockIdx.x / 8;
  Item it;
  it.h = item / ntiles;
  const int tile = item % ntiles;
  int img = 0;
  while (img + 1 < desc.n_images && tile >= desc.cu_tiles[img + 1]) ++img;
  it.img = img;
  it.seq0 = desc.cu_seqlens[img];
  it.P = desc.cu_seqlens[img + 1] - it.seq0;
  it.r0 = (tile - desc.cu_tiles[img]) * AB_ROWS;
  return it;
}

// one 1 KB copy (8 rows of 128 bytes) of a row-major [rows][64] tile whose rows
// r = 8*q .. 8*q+7 are taken from row_ptr(r); chunk position lane % 8 of row
// lane / 8 holds the row's chunk (lane % 8) ^ ab_swz(row)
template <typename RowPtr>
VIT_DEV void ab_copy(RowPtr row_ptr, int q, int lane, bf16* lds_tile) {
  const int r = 8 * q + (lane >> 3);
  const int kc = (lane & 7) ^ ab_swz(r);
  copy16_to_lds(row_ptr(r) + kc * 8, lds_tile + q * 512);
}

// fragment of row r (16-byte chunk ch) of a swizzled [64][64] tile
VIT_DEV bf16x8 ab_frag(const bf16* tile, int r, int ch) {
  return *reinterpret_cast<const bf16x8*>(tile + r * 64 + ((ch ^ ab_swz(r)) << 3));
}

// The rotary's gradient on a lane's accumulator column: dims 32 db + 8 g + 4 fh + r
// (acc[db][4 g + r]) of the row at position p; dims i and i + 16 of each
// 32-dim half (g and g + 2) are rotation partners and sit in the same lane.
// Rotation by the opposite angles, times `scale`, rounded to bf16 once.
VIT_DEV void rope_inv_store(const f32x16 (&acc)[2], const float2* __restrict__ table, int64_t p,
                            int fh, float scale, bf16* row) {
#pragma unroll
  for (int db = 0; db < 2; ++db)
#pragma unroll
    for (int g = 0; g < 2; ++g) {
      bf16x4 lo, hi;
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const float2 cs = table[p * 32 + db * 16 + 8 * g + 4 * fh + r];
        const float a1 = acc[db][4 * g + r] * scale, a2 = acc[db][4 * (g + 2) + r] * scale;
        lo[r] = f2bf(a1 * cs.x + a2 * cs.y);
        hi[r] = f2bf(a2 * cs.x - a1 * cs.y);
      }
      *reinterpret_cast<bf16x4*>(row + db * 32 + g * 8 + fh * 4) = lo;
      *reinterpret_cast<bf16x4*>(row + db * 32 + (g + 2) * 8 + fh * 4) = hi;
    }
}

// ---------------------------------------------------------------------------
__global__ __launch_bounds__(64 * AB_WAVES, 2) void attn_dq_kernel(
    const bf16* __restrict__ qkv, int64_t ldq, const bf16* __restrict__ dO,
    const bf16* __restrict__ kt, int64_t t_ld, const float* __restrict__ lse2,
    const float* __restrict__ Dq, VarlenDesc desc, int H, float c,
    const float2* __restrict__ table, bf16* __restrict__ dq_out, int64_t ld_out) {
  __shared__ __attribute__((aligned(16))) bf16 sm[2][3][AB_T * 64];  // K, V, K^T
  const Item it = ab_item(desc, H);
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int fr = lane & 31, fh = lane >> 5;
  const int64_t dm = (int64_t)H * 64;
  const int h = it.h, P = it.P, seq0 = it.seq0;
  const int kvo = desc.kv_off[it.img];

  // this lane's query (column of S^T): Q and dO fragments, lse, Dq
  const int qi = min(it.r0 + wave * 32 + fr, P - 1);
  bf16x8 qf[4], df[4];
  {
    const bf16* qrow = qkv + (int64_t)(seq0 + qi) * ldq + h * 64 + fh * 8;
    const bf16* drow = dO + (int64_t)(seq0 + qi) * dm + h * 64 + fh * 8;
#pragma unroll
    for (int ks = 0; ks < 4; ++ks) {
      qf[ks] = __builtin_bit_cast(bf16x8, ld16(qrow + ks * 16));
      df[ks] = __builtin_bit_cast(bf16x8, ld16(drow + ks * 16));
    }
  }
  const float lse = lse2[(int64_t)h * desc.total + seq0 + qi];
  const float dq_ref = Dq[(int64_t)h * desc.total + seq0 + qi];

  auto issue = [&](int t, int st) __attribute__((always_inline)) {
    const int kv0 = t * AB_T;
    // 24 copies: 8 of K rows, 8 of V rows, 8 of K^T rows; wave w takes w, w+4, ...
#pragma unroll
    for (int i = 0; i < 24 / AB_WAVES; ++i) {
      const int q = wave + AB_WAVES * i;
      const int sub = q >> 3;
      if (sub == 0)
        ab_copy([&](int r) { return qkv + (int64_t)(seq0 + min(kv0 + r, P - 1)) * ldq + dm + h * 64; },
                q & 7, lane, sm[st][0]);
      else if (sub == 1)
        ab_copy([&](int r) { return qkv + (int64_t)(seq0 + min(kv0 + r, P - 1)) * ldq + 2 * dm + h * 64; },
                q & 7, lane, sm[st][1]);
      else
        ab_copy([&](int r) { return kt + (int64_t)(h * 64 + r) * t_ld + kvo + kv0; }, q & 7, lane,
                sm[st][2]);
    }
  };

  f32x16 acc[2] = {f32x16{}, f32x16{}};  // dQ^T: dims 32*db .. +31 x this wave's queries
  const int nkv = (P + AB_T - 1) / AB_T;
  asm volatile("" : "+s"(c));
  issue(0, 0);
  for (int t = 0; t < nkv; ++t) {
    const int st = t & 1;
    wait_vmcnt<0>();
    __syncthreads();  // tile t landed; every wave is done with the other buffer
    if (t + 1 < nkv) issue(t + 1, st ^ 1);
    // S^T = K Q^T and dP^T = V dO^T: rows = keys (2 blocks of 32), columns = queries
    f32x16 s[2] = {f32x16{}, f32x16{}}, dp[2] = {f32x16{}, f32x16{}};
#pragma unroll
    for (int ks = 0; ks < 4; ++ks)
#pragma unroll
      for (int kb = 0; kb < 2; ++kb) {
        const bf16x8 kf = ab_frag(sm[st][0], kb * 32 + fr, 2 * ks + fh);
        const bf16x8 vf = ab_frag(sm[st][1], kb * 32 + fr, 2 * ks + fh);
        s[kb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(kf, qf[ks], s[kb], 0, 0, 0);
        dp[kb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(vf, df[ks], dp[kb], 0, 0, 0);
      }
    // dS^T = P^T (dP^T - Dq), P^T = 2^(S^T c - lse); keys past the image give 0
    const int kv0 = t * AB_T;
    bf16x8 dsf[4];
#pragma unroll
    for (int kb = 0; kb < 2; ++kb)
#pragma unroll
      for (int ks2 = 0; ks2 < 2; ++ks2)
#pragma unroll
        for (int j = 0; j < 8; ++j) {
          const int i = 8 * ks2 + j;
          const int key = kv0 + kb * 32 + (i >> 2) * 8 + fh * 4 + (i & 3);
          const float p = key < P ? __builtin_amdgcn_exp2f(fmaf(s[kb][i], c, -lse)) : 0.f;
          dsf[2 * kb + ks2][j] = f2bf(p * (dp[kb][i] - dq_ref));
        }
    // dQ^T += K^T dS^T: K^T rows = dims, key slots 32 kb + 16 ks2 + 8 fh .. +7
#pragma unroll
    for (int x = 0; x < 4; ++x) {
      const int kb = x >> 1, ks2 = x & 1;
#pragma unroll
      for (int db = 0; db < 2; ++db) {
        const bf16x8 tf = ab_frag(sm[st][2], db * 32 + fr, kb * 4 + ks2 * 2 + fh);
        acc[db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(tf, dsf[x], acc[db], 0, 0, 0);
      }
    }
  }
  // dq (rotated space) x 1/sqrt(64), rotated back to the space of wqkv's output
  const int q = it.r0 + wave * 32 + fr;
  if (q < P)
    rope_inv_store(acc, table, seq0 + q, fh, 0.125f, dq_out + (int64_t)(seq0 + q) * ld_out + h * 64);
}

// ---------------------------------------------------------------------------
__global__ __launch_bounds__(64 * AB_WAVES, 2) void attn_dkv_kernel(
    const bf16* __restrict__ qkv, int64_t ldq, const bf16* __restrict__ dO,
    const bf16* __restrict__ qt, const bf16* __restrict__ dot, int64_t t_ld,
    const float* __restrict__ lse2, const float* __restrict__ Dq, VarlenDesc desc, int H, float c,
    const float2* __restrict__ table, bf16* __restrict__ dkv_out, int64_t ld_out) {
  // dynamic LDS (65 KB, above the static limit): Q, dO, Q^T, dO^T tiles of two
  // stages, then the lse and Dq of the tile
  extern __shared__ __attribute__((aligned(16))) char dkv_smem[];
  auto sm = reinterpret_cast<bf16 (*)[4][AB_T * 64]>(dkv_smem);
  auto sl = reinterpret_cast<float (*)[2][AB_T]>(dkv_smem + 2 * 4 * AB_T * 64 * sizeof(bf16));
  const Item it = ab_item(desc, H);
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int fr = lane & 31, fh = lane >> 5;
  const int64_t dm = (int64_t)H * 64;
  const int h = it.h, P = it.P, seq0 = it.seq0;
  const int kvo = desc.kv_off[it.img];

  // this lane's key (column of S): K and V fragments
  const int ki = min(it.r0 + wave * 32 + fr, P - 1);
  bf16x8 kf[4], vf[4];
  {
    const bf16* krow = qkv + (int64_t)(seq0 + ki) * ldq + dm + h * 64 + fh * 8;
    const bf16* vrow = qkv + (int64_t)(seq0 + ki) * ldq + 2 * dm + h * 64 + fh * 8;
#pragma unroll
    for (int ks = 0; ks < 4; ++ks) {
      kf[ks] = __builtin_bit_cast(bf16x8, ld16(krow + ks * 16));
      vf[ks] = __builtin_bit_cast(bf16x8, ld16(vrow + ks * 16));
    }
  }

  auto issue = [&](int t, int st) __attribute__((always_inline)) {
    const int q0 = t * AB_T;
    // 32 copies: Q rows, dO rows, Q^T rows, dO^T rows (8 each); wave w takes w, w+4, ...
#pragma unroll
    for (int i = 0; i < 32 / AB_WAVES; ++i) {
      const int q = wave + AB_WAVES * i;
      const int sub = q >> 3;
      if (sub == 0)
        ab_copy([&](int r) { return qkv + (int64_t)(seq0 + min(q0 + r, P - 1)) * ldq + h * 64; },
                q & 7, lane, sm[st][0]);
      else if (sub == 1)
        ab_copy([&](int r) { return dO + (int64_t)(seq0 + min(q0 + r, P - 1)) * dm + h * 64; },
                q & 7, lane, sm[st][1]);
      else if (sub == 2)
        ab_copy([&](int r) { return qt + (int64_t)(h * 64 + r) * t_ld + kvo + q0; }, q & 7, lane,
                sm[st][2]);
      else
        ab_copy([&](int r) { return dot + (int64_t)(h * 64 + r) * t_ld + kvo + q0; }, q & 7, lane,
                sm[st][3]);
    }
  };
  // lse and Dq of tile t, one value per thread of the first 128, into registers
  auto load_stats = [&](int t) __attribute__((always_inline)) {
    float v = 0.f;
    if (threadIdx.x < 2 * AB_T) {
      const int qq = min(t * AB_T + (int)(threadIdx.x & (AB_T - 1)), P - 1);
      const float* src = threadIdx.x < AB_T ? lse2 : Dq;
      v = src[(int64_t)h * desc.total + seq0 + qq];
    }
    return v;
  };

  f32x16 dv[2] = {f32x16{}, f32x16{}}, dk[2] = {f32x16{}, f32x16{}};  // dims x keys
  const int nq = (P + AB_T - 1) / AB_T;
  asm volatile("" : "+s"(c));
  issue(0, 0);
  float stat = load_stats(0);
  for (int t = 0; t < nq; ++t) {
    const int st = t & 1;
    wait_vmcnt<0>();
    if (threadIdx.x < 2 * AB_T) sl[st][threadIdx.x >> 6][threadIdx.x & (AB_T - 1)] = stat;
    __syncthreads();  // tile t (and its lse, Dq) landed; every wave is done with the other buffer
    if (t + 1 < nq) {
      issue(t + 1, st ^ 1);
      stat = load_stats(t + 1);
    }
    // S = Q K^T and dP = dO V^T: rows = queries (2 blocks of 32), columns = keys
    f32x16 s[2] = {f32x16{}, f32x16{}}, dp[2] = {f32x16{}, f32x16{}};
#pragma unroll
    for (int ks = 0; ks < 4; ++ks)
#pragma unroll
      for (int qb = 0; qb < 2; ++qb) {
        const bf16x8 qf = ab_frag(sm[st][0], qb * 32 + fr, 2 * ks + fh);
        const bf16x8 of = ab_frag(sm[st][1], qb * 32 + fr, 2 * ks + fh);
        s[qb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(qf, kf[ks], s[qb], 0, 0, 0);
        dp[qb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(of, vf[ks], dp[qb], 0, 0, 0);
      }
    // P = 2^(S c - lse[q]) (0 for queries past the image), dS = P (dP - Dq[q])
    const int q0 = t * AB_T;
    bf16x8 pf[4], dsf[4];
#pragma unroll
    for (int qb = 0; qb < 2; ++qb)
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        const int row = qb * 32 + g * 8 + fh * 4;  // this lane's rows row .. row+3
        const f32x4 l4 = *reinterpret_cast<const f32x4*>(&sl[st][0][row]);
        const f32x4 d4 = *reinterpret_cast<const f32x4*>(&sl[st][1][row]);
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          const int i = 4 * g + r;
          const float p =
              q0 + row + r < P ? __builtin_amdgcn_exp2f(fmaf(s[qb][i], c, -l4[r])) : 0.f;
          pf[2 * qb + (i >> 3)][i & 7] = f2bf(p);
          dsf[2 * qb + (i >> 3)][i & 7] = f2bf(p * (dp[qb][i] - d4[r]));
        }
      }
    // dV^T += dO^T P, dK^T += Q^T dS: rows = dims, query slots 32 qb + 16 ks2 + 8 fh .. +7
#pragma unroll
    for (int x = 0; x < 4; ++x) {
      const int qb = x >> 1, ks2 = x & 1;
#pragma unroll
      for (int db = 0; db < 2; ++db) {
        const bf16x8 of = ab_frag(sm[st][3], db * 32 + fr, qb * 4 + ks2 * 2 + fh);
        const bf16x8 qtf = ab_frag(sm[st][2], db * 32 + fr, qb * 4 + ks2 * 2 + fh);
        dv[db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(of, pf[x], dv[db], 0, 0, 0);
        dk[db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(qtf, dsf[x], dk[db], 0, 0, 0);
      }
    }
  }
  // dk x 1/sqrt(64) rotated back like dq; dv as is
  const int k = it.r0 + wave * 32 + fr;
  if (k < P) {
    bf16* krow = dkv_out + (int64_t)(seq0 + k) * ld_out + h * 64;
    bf16* vrow = krow + dm;
    rope_inv_store(dk, table, seq0 + k, fh, 0.125f, krow);
#pragma unroll
    for (int db = 0; db < 2; ++db)
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        bf16x4 b;
#pragma unroll
        for (int r = 0; r < 4; ++r) b[r] = f2bf(dv[db][4 * g + r]);
        *reinterpret_cast<bf16x4*>(vrow + db * 32 + g * 8 + fh * 4) = b;
      }
  }
}

// ---------------------------------------------------------------------------
// head_dim 72 (D not a multiple of 32): the same two kernels on 32x32x16 MFMAs
// with the head dimension padded.  The contractions over it (S, dP) take
// ceil(D/16) k-steps: the fragments held in registers are zero past D, and the
// LDS operand rereads its last real chunk against those zeros.  The outputs
// over it (dQ^T, dK^T, dV^T) take ceil(D/32) blocks of 32 dims whose rows past
// D reread row D-1 and are never stored.  Row tiles [64][D] in LDS keep the
// natural 2D-byte row stride (144 bytes: 9 chunks, an odd number, so 16
// consecutive rows of one chunk fall in distinct banks); transposed tiles
// [D][64 slots] are 128-byte rows swizzled as above.  Inside one 64-row (or
// 64-key) step the S / dP products of each 32-row half feed that half's
// output MFMAs before the next half starts, which bounds the live registers
// within 256 (two workgroups per CU).  dq and dk are written in the rotated
// space, scaled by 1/sqrt(D); launch_rope_inverse maps them back.
template <int D>
struct BwdDims {
  static_assert(D % 8 == 0 && D <= 96, "head dim");
  static constexpr int KS = (D + 15) / 16;  // 16-deep k-steps over the head dim
  static constexpr int DB = (D + 31) / 32;  // 32-dim blocks of the outputs over it
  static constexpr int CH = D / 8;          // 16-byte chunks per row-tile row
  static constexpr int TILE = AB_T * D;     // elements of a [64][D] or [D][64] tile
  static constexpr int NCP = TILE / 512;    // 1 KB copies per tile
  static_assert(TILE % 512 == 0, "whole copies");
};

// copy cq (0 .. NCP-1, one 1 KB copy per wave) of a row tile [64][D] whose row r
// is row_ptr(r): 16-byte chunk 64 cq + lane of the tile, row-major
template <int D, typename RowPtr>
VIT_DEV void row_tile_copy(RowPtr row_ptr, int cq, int lane, bf16* tile) {
  const int q = cq * 64 + lane;
  const int r = q / BwdDims<D>::CH, ch = q % BwdDims<D>::CH;
  copy16_to_lds(row_ptr(r) + ch * 8, tile + cq * 512);
}
// 16-byte fragment: row r, dims 16 ks + 8 fh .. +7 of a row tile (the chunk past
// the last real one rereads the last)
template <int D>
VIT_DEV bf16x8 row_frag(const bf16* tile, int r, int ks, int fh) {
  const int ch = min(2 * ks + fh, BwdDims<D>::CH - 1);
  return *reinterpret_cast<const bf16x8*>(tile + r * D + ch * 8);
}
// fragment of a transposed tile: row (dim) r clamped to D-1, slot chunk ch
template <int D>
VIT_DEV bf16x8 t_frag(const bf16* tile, int r, int ch) {
  r = min(r, D - 1);
  return *reinterpret_cast<const bf16x8*>(tile + r * 64 + ((ch ^ ab_swz(r)) << 3));
}
// head-dim fragments of one row in registers: dims 16 ks + 8 fh .. +7, zero past D
template <int D>
VIT_DEV void row_regs(const bf16* row, int fh, bf16x8 (&f)[BwdDims<D>::KS]) {
#pragma unroll
  for (int ks = 0; ks < BwdDims<D>::KS; ++ks) {
    const int e = 16 * ks + 8 * fh;
    u32x4 v = u32x4{0u, 0u, 0u, 0u};
    if (e < D) v = ld16(row + e);
    f[ks] = __builtin_bit_cast(bf16x8, v);
  }
}
// lane's output dims 32 db + 8 g + 4 fh .. +3 of acc, times scale, into row (bf16)
template <int D>
VIT_DEV void store_dims(const f32x16 (&acc)[BwdDims<D>::DB], float scale, int fh, bf16* row) {
#pragma unroll
  for (int db = 0; db < BwdDims<D>::DB; ++db)
#pragma unroll
    for (int g = 0; g < 4; ++g) {
      const int e = 32 * db + 8 * g + 4 * fh;
      if (e >= D) continue;
      bf16x4 b;
#pragma unroll
      for (int r = 0; r < 4; ++r) b[r] = f2bf(acc[db][4 * g + r] * scale);
      *reinterpret_cast<bf16x4*>(row + e) = b;
    }
}

template <int D>
__global__ __launch_bounds__(64 * AB_WAVES, 2) void attn_dq_pad_kernel(
    const bf16* __restrict__ qkv, int64_t ldq, const bf16* __restrict__ dO,
    const bf16* __restrict__ kt, int64_t t_ld, const float* __restrict__ lse2,
    const float* __restrict__ Dq, VarlenDesc desc, int H, float c, float scale,
    bf16* __restrict__ dq_out, int64_t ld_out) {
  using B = BwdDims<D>;
  __shared__ __attribute__((aligned(16))) bf16 sm[2][3][B::TILE];  // K, V rows; K^T
  const Item it = ab_item(desc, H);
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int fr = lane & 31, fh = lane >> 5;
  const int64_t dm = (int64_t)H * D;
  const int h = it.h, P = it.P, seq0 = it.seq0;
  const int kvo = desc.kv_off[it.img];

  // this lane's query (column of S^T): Q and dO fragments, lse, Dq
  const int qi = min(it.r0 + wave * 32 + fr, P - 1);
  bf16x8 qf[B::KS], df[B::KS];
  row_regs<D>(qkv + (int64_t)(seq0 + qi) * ldq + h * D, fh, qf);
  row_regs<D>(dO + (int64_t)(seq0 + qi) * dm + h * D, fh, df);
  const float lse = lse2[(int64_t)h * desc.total + seq0 + qi];
  const float dq_ref = Dq[(int64_t)h * desc.total + seq0 + qi];

  // 3 NCP copies per tile (K rows, V rows, K^T rows); wave w takes w, w+4, ...
  auto issue = [&](int t, int st) __attribute__((always_inline)) {
    const int kv0 = t * AB_T;
#pragma unroll
    for (int i = 0; i < (3 * B::NCP + AB_WAVES - 1) / AB_WAVES; ++i) {
      const int q = wave + AB_WAVES * i;
      if (q >= 3 * B::NCP) break;
      const int sub = q / B::NCP, cq = q % B::NCP;
      if (sub < 2) {
        const bf16* base = qkv + (sub + 1) * dm + h * D;
        row_tile_copy<D>([&](int r) { return base + (int64_t)(seq0 + min(kv0 + r, P - 1)) * ldq; },
                         cq, lane, sm[st][sub]);
      } else {
        ab_copy([&](int r) { return kt + (int64_t)(h * D + r) * t_ld + kvo + kv0; }, cq, lane,
                sm[st][2]);
      }
    }
  };

  f32x16 acc[B::DB];  // dQ^T: dims 32 db .. +31 x this wave's queries
#pragma unroll
  for (int db = 0; db < B::DB; ++db) acc[db] = f32x16{};
  const int nkv = (P + AB_T - 1) / AB_T;
  asm volatile("" : "+s"(c));
  issue(0, 0);
  for (int t = 0; t < nkv; ++t) {
    const int st = t & 1;
    wait_vmcnt<0>();
    __syncthreads();  // tile t landed; every wave is done with the other buffer
    if (t + 1 < nkv) issue(t + 1, st ^ 1);
    const int kv0 = t * AB_T;
#pragma unroll
    for (int kb = 0; kb < 2; ++kb) {
      // S^T = K Q^T and dP^T = V dO^T for keys 32 kb .. +31
      f32x16 s = f32x16{}, dp = f32x16{};
#pragma unroll
      for (int ks = 0; ks < B::KS; ++ks) {
        s = __builtin_amdgcn_mfma_f32_32x32x16_bf16(row_frag<D>(sm[st][0], kb * 32 + fr, ks, fh),
                                                    qf[ks], s, 0, 0, 0);
        dp = __builtin_amdgcn_mfma_f32_32x32x16_bf16(row_frag<D>(sm[st][1], kb * 32 + fr, ks, fh),
                                                     df[ks], dp, 0, 0, 0);
      }
      // dS^T = P^T (dP^T - Dq), P^T = 2^(S^T c - lse); keys past the image give 0
      bf16x8 dsf[2];
#pragma unroll
      for (int ks2 = 0; ks2 < 2; ++ks2)
#pragma unroll
        for (int j = 0; j < 8; ++j) {
          const int i = 8 * ks2 + j;
          const int key = kv0 + kb * 32 + (i >> 2) * 8 + fh * 4 + (i & 3);
          const float p = key < P ? __builtin_amdgcn_exp2f(fmaf(s[i], c, -lse)) : 0.f;
          dsf[ks2][j] = f2bf(p * (dp[i] - dq_ref));
        }
      // dQ^T += K^T dS^T: K^T rows = dims, key slots 32 kb + 16 ks2 + 8 fh .. +7
#pragma unroll
      for (int ks2 = 0; ks2 < 2; ++ks2)
#pragma unroll
        for (int db = 0; db < B::DB; ++db)
          acc[db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(
              t_frag<D>(sm[st][2], db * 32 + fr, kb * 4 + ks2 * 2 + fh), dsf[ks2], acc[db], 0, 0, 0);
    }
  }
  const int q = it.r0 + wave * 32 + fr;
  if (q < P) store_dims<D>(acc, scale, fh, dq_out + (int64_t)(seq0 + q) * ld_out + h * D);
}

template <int D>
__global__ __launch_bounds__(64 * AB_WAVES, 2) void attn_dkv_pad_kernel(
    const bf16* __restrict__ qkv, int64_t ldq, const bf16* __restrict__ dO,
    const bf16* __restrict__ qt, const bf16* __restrict__ dot, int64_t t_ld,
    const float* __restrict__ lse2, const float* __restrict__ Dq, VarlenDesc desc, int H, float c,
    float scale, bf16* __restrict__ dkv_out, int64_t ld_out) {
  using B = BwdDims<D>;
  // dynamic LDS: Q, dO rows and Q^T, dO^T tiles of two stages, then the lse and
  // Dq of the tile
  extern __shared__ __attribute__((aligned(16))) char dkv_pad_smem[];
  auto sm = reinterpret_cast<bf16 (*)[4][B::TILE]>(dkv_pad_smem);
  auto sl = reinterpret_cast<float (*)[2][AB_T]>(dkv_pad_smem + 2 * 4 * B::TILE * sizeof(bf16));
  const Item it = ab_item(desc, H);
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int fr = lane & 31, fh = lane >> 5;
  const int64_t dm = (int64_t)H * D;
  const int h = it.h, P = it.P, seq0 = it.seq0;
  const int kvo = desc.kv_off[it.img];

  // this lane's key (column of S): K and V fragments
  const int ki = min(it.r0 + wave * 32 + fr, P - 1);
  bf16x8 kf[B::KS], vf[B::KS];
  row_regs<D>(qkv + (int64_t)(seq0 + ki) * ldq + dm + h * D, fh, kf);
  row_regs<D>(qkv + (int64_t)(seq0 + ki) * ldq + 2 * dm + h * D, fh, vf);

  // 4 NCP copies per tile (Q rows, dO rows, Q^T, dO^T); wave w takes w, w+4, ...
  auto issue = [&](int t, int st) __attribute__((always_inline)) {
    const int q0 = t * AB_T;
#pragma unroll
    for (int i = 0; i < (4 * B::NCP + AB_WAVES - 1) / AB_WAVES; ++i) {
      const int q = wave + AB_WAVES * i;
      if (q >= 4 * B::NCP) break;
      const int sub = q / B::NCP, cq = q % B::NCP;
      if (sub == 0)
        row_tile_copy<D>(
            [&](int r) { return qkv + (int64_t)(seq0 + min(q0 + r, P - 1)) * ldq + h * D; }, cq,
            lane, sm[st][0]);
      else if (sub == 1)
        row_tile_copy<D>(
            [&](int r) { return dO + (int64_t)(seq0 + min(q0 + r, P - 1)) * dm + h * D; }, cq,
            lane, sm[st][1]);
      else
        ab_copy([&](int r) { return (sub == 2 ? qt : dot) + (int64_t)(h * D + r) * t_ld + kvo + q0; },
                cq, lane, sm[st][sub]);
    }
  };
  // lse and Dq of tile t, one value per thread of the first 128, into registers
  auto load_stats = [&](int t) __attribute__((always_inline)) {
    float v = 0.f;
    if (threadIdx.x < 2 * AB_T) {
      const int qq = min(t * AB_T + (int)(threadIdx.x & (AB_T - 1)), P - 1);
      const float* src = threadIdx.x < AB_T ? lse2 : Dq;
      v = src[(int64_t)h * desc.total + seq0 + qq];
    }
    return v;
  };

  f32x16 dv[B::DB], dk[B::DB];  // dims x keys
#pragma unroll
  for (int db = 0; db < B::DB; ++db) dv[db] = dk[db] = f32x16{};
  const int nq = (P + AB_T - 1) / AB_T;
  asm volatile("" : "+s"(c));
  issue(0, 0);
  float stat = load_stats(0);
  for (int t = 0; t < nq; ++t) {
    const int st = t & 1;
    wait_vmcnt<0>();
    if (threadIdx.x < 2 * AB_T) sl[st][threadIdx.x >> 6][threadIdx.x & (AB_T - 1)] = stat;
    __syncthreads();  // tile t (and its lse, Dq) landed; every wave is done with the other buffer
    if (t + 1 < nq) {
      issue(t + 1, st ^ 1);
      stat = load_stats(t + 1);
    }
    const int q0 = t * AB_T;
#pragma unroll
    for (int qb = 0; qb < 2; ++qb) {
      // S = Q K^T and dP = dO V^T for queries 32 qb .. +31
      f32x16 s = f32x16{}, dp = f32x16{};
#pragma unroll
      for (int ks = 0; ks < B::KS; ++ks) {
        s = __builtin_amdgcn_mfma_f32_32x32x16_bf16(row_frag<D>(sm[st][0], qb * 32 + fr, ks, fh),
                                                    kf[ks], s, 0, 0, 0);
        dp = __builtin_amdgcn_mfma_f32_32x32x16_bf16(row_frag<D>(sm[st][1], qb * 32 + fr, ks, fh),
                                                     vf[ks], dp, 0, 0, 0);
      }
      // P = 2^(S c - lse[q]) (0 for queries past the image), dS = P (dP - Dq[q])
      bf16x8 pf[2], dsf[2];
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        const int row = qb * 32 + g * 8 + fh * 4;  // this lane's rows row .. row+3
        const f32x4 l4 = *reinterpret_cast<const f32x4*>(&sl[st][0][row]);
        const f32x4 d4 = *reinterpret_cast<const f32x4*>(&sl[st][1][row]);
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          const int i = 4 * g + r;
          const float p = q0 + row + r < P ? __builtin_amdgcn_exp2f(fmaf(s[i], c, -l4[r])) : 0.f;
          pf[i >> 3][i & 7] = f2bf(p);
          dsf[i >> 3][i & 7] = f2bf(p * (dp[i] - d4[r]));
        }
      }
      // dV^T += dO^T P, dK^T += Q^T dS: rows = dims, query slots 32 qb + 16 ks2 + 8 fh .. +7
#pragma unroll
      for (int ks2 = 0; ks2 < 2; ++ks2)
#pragma unroll
        for (int db = 0; db < B::DB; ++db) {
          const int ch = qb * 4 + ks2 * 2 + fh;
          dv[db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(t_frag<D>(sm[st][3], db * 32 + fr, ch),
                                                           pf[ks2], dv[db], 0, 0, 0);
          dk[db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(t_frag<D>(sm[st][2], db * 32 + fr, ch),
                                                           dsf[ks2], dk[db], 0, 0, 0);
        }
    }
  }
  const int k = it.r0 + wave * 32 + fr;
  if (k < P) {
    bf16* krow = dkv_out + (int64_t)(seq0 + k) * ld_out + h * D;
    store_dims<D>(dk, scale, fh, krow);
    store_dims<D>(dv, 1.0f, fh, krow + dm);
  }
}

unsigned blocks_of(int64_t n) { return (unsigned)((n + kThreads - 1) / kThreads); }

}  // namespace

int attention_bwd_tile() { return AB_ROWS; }

hipError_t launch_rowdot(const void* dO, const void* O, int64_t P, int n_heads, int head_dim,
                         float* Dq, hipStream_t s) {
  if (P == 0) return hipSuccess;
  if (head_dim == 64)
    rowdot_kernel<64><<<blocks_of(P * n_heads), kThreads, 0, s>>>((const bf16*)dO, (const bf16*)O,
                                                                  P, n_heads, Dq);
  else if (head_dim == 72)
    rowdot_kernel<72><<<blocks_of(P * n_heads), kThreads, 0, s>>>((const bf16*)dO, (const bf16*)O,
                                                                  P, n_heads, Dq);
  else
    return hipErrorInvalidValue;
  return hipGetLastError();
}

namespace {
template <int D>
hipError_t launch_attention_bwd_pad(const void* qkv, int64_t ldq, const void* dO, const void* qt,
                                    const void* kt, const void* dot, int64_t t_ld,
                                    const float* lse2, const float* Dq, const VarlenDesc& d,
                                    int n_heads, void* dqkv, int64_t ld_out, hipStream_t s) {
  const int tiles = d.cu_tiles[d.n_images];
  if (tiles == 0) return hipSuccess;
  const float c = (float)(1.4426950408889634 / sqrt((double)D));  // log2(e) / sqrt(D)
  const float scale = (float)(1.0 / sqrt((double)D));
  const dim3 grid((unsigned)(tiles * n_heads));
  attn_dq_pad_kernel<D><<<grid, 64 * AB_WAVES, 0, s>>>(
      (const bf16*)qkv, ldq, (const bf16*)dO, (const bf16*)kt, t_ld, lse2, Dq, d, n_heads, c, scale,
      (bf16*)dqkv, ld_out);
  constexpr size_t lds = 2 * 4 * BwdDims<D>::TILE * sizeof(bf16) + 2 * 2 * AB_T * sizeof(float);
  static bool attr = false;
  if (!attr) {
    const hipError_t e = hipFuncSetAttribute((const void*)attn_dkv_pad_kernel<D>,
                                             hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
    if (e != hipSuccess) return e;
    attr = true;
  }
  attn_dkv_pad_kernel<D><<<grid, 64 * AB_WAVES, lds, s>>>(
      (const bf16*)qkv, ldq, (const bf16*)dO, (const bf16*)qt, (const bf16*)dot, t_ld, lse2, Dq, d,
      n_heads, c, scale, (bf16*)dqkv + (int64_t)n_heads * D, ld_out);
  return hipGetLastError();
}
}  // namespace

hipError_t launch_attention_bwd(const void* qkv, int64_t ldq, const void* dO, const void* qt,
                                const void* kt, const void* dot, int64_t t_ld, const float* lse2,
                                const float* Dq, const void* table, const VarlenDesc& d,
                                int n_heads, int head_dim, void* dqkv, int64_t ld_out,
                                hipStream_t s) {
  if (head_dim == 72)
    return launch_attention_bwd_pad<72>(qkv, ldq, dO, qt, kt, dot, t_ld, lse2, Dq, d, n_heads, dqkv,
                                        ld_out, s);
  if (head_dim != 64) return hipErrorInvalidValue;
  const int tiles = d.cu_tiles[d.n_images];
  if (tiles == 0) return hipSuccess;
  const float c = (float)(1.4426950408889634 / 8.0);  // log2(e) / sqrt(64)
  const dim3 grid((unsigned)(tiles * n_heads));
  attn_dq_kernel<<<grid, 64 * AB_WAVES, 0, s>>>((const bf16*)qkv, ldq, (const bf16*)dO,
                                                (const bf16*)kt, t_ld, lse2, Dq, d, n_heads, c,
                                                (const float2*)table, (bf16*)dqkv, ld_out);
  constexpr size_t dkv_lds = 2 * 4 * AB_T * 64 * sizeof(bf16) + 2 * 2 * AB_T * sizeof(float);
  static bool attr = false;
  if (!attr) {
    const hipError_t e = hipFuncSetAttribute((const void*)attn_dkv_kernel,
                                             hipFuncAttributeMaxDynamicSharedMemorySize,
                                             (int)dkv_lds);
    if (e != hipSuccess) return e;
    attr = true;
  }
  attn_dkv_kernel<<<grid, 64 * AB_WAVES, dkv_lds, s>>>(
      (const bf16*)qkv, ldq, (const bf16*)dO, (const bf16*)qt, (const bf16*)dot, t_ld, lse2, Dq, d,
      n_heads, c, (const float2*)table, (bf16*)dqkv + (int64_t)n_heads * 64, ld_out);
  return hipGetLastError();
}
