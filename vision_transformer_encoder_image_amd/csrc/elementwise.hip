// Bandwidth-bound passes of the encoder on gfx950: RMSNorm, rotary table and
// rotary application, 2x2 aligner gather, row padding, layout index arrays.
#include <math.h>

#include <cmath>

#include "common.h"

namespace {

constexpr int kThreads = 256;

// ---------------------------------------------------------------------------
// ss + v.x^2 + v.y^2 + v.z^2 + v.w^2 as four FMAs in this order (spelled out so
// that both RMSNorm kernels round the sum of squares identically)
VIT_DEV float sumsq4(float4 v, float ss) {
  ss = fmaf(v.x, v.x, ss);
  ss = fmaf(v.y, v.y, ss);
  ss = fmaf(v.z, v.z, ss);
  return fmaf(v.w, v.w, ss);
}

// RMSNorm (NeMo Automodel vision page, DeepseekV4VisionRMSNorm: fp32 scale,
// eps 1e-6): one wavefront per row, fp32 sum of squares reduced across the
// wave, then y = w * (x * rsqrt(mean + eps)) cast once to the output type.
template <typename TO>
__global__ __launch_bounds__(kThreads) void rmsnorm_kernel(const float* __restrict__ x,
                                                           const float* __restrict__ w, float eps,
                                                           int64_t rows, int dim,
                                                           TO* __restrict__ out) {
  const int lane = threadIdx.x & 63;
  const int64_t row = (int64_t)blockIdx.x * (kThreads / 64) + (threadIdx.x >> 6);
  if (row >= rows) return;
  const float4* xr = reinterpret_cast<const float4*>(x + row * dim);
  const float4* w4 = reinterpret_cast<const float4*>(w);
  const int n4 = dim >> 2;
  float ss = 0.f;
  for (int c = lane; c < n4; c += 64) {
    float4 v = xr[c];
    ss = sumsq4(v, ss);
  }
  ss = wave_sum(ss);
  const float rstd = 1.0f / sqrtf(ss / (float)dim + eps);
  for (int c = lane; c < n4; c += 64) {
    float4 v = xr[c];
    float4 s = w4[c];
    TO* o = out + row * dim + 4 * c;
    o[0] = from_f32<TO>(s.x * (v.x * rstd));
    o[1] = from_f32<TO>(s.y * (v.y * rstd));
    o[2] = from_f32<TO>(s.z * (v.z * rstd));
    o[3] = from_f32<TO>(s.w * (v.w * rstd));
  }
}

// The same for dim <= 256 * NV: the lane's NV float4s of the row stay in
// registers between the two passes (x is read once), and each float4 of output
// leaves as one vector store.  Same arithmetic, in the same order.
template <typename TO, int NV>
__global__ __launch_bounds__(kThreads) void rmsnorm_reg_kernel(const float* __restrict__ x,
                                                               const float* __restrict__ w,
                                                               float eps, int64_t rows, int dim,
                                                               TO* __restrict__ out) {
  typedef TO TO4 __attribute__((ext_vector_type(4)));
  const int lane = threadIdx.x & 63;
  const int64_t row = (int64_t)blockIdx.x * (kThreads / 64) + (threadIdx.x >> 6);
  if (row >= rows) return;
  const float4* xr = reinterpret_cast<const float4*>(x + row * dim);
  const float4* w4 = reinterpret_cast<const float4*>(w);
  const int n4 = dim >> 2;
  float4 v[NV];
#pragma unroll
  for (int i = 0; i < NV; ++i) {
    const int c = lane + 64 * i;
    v[i] = c < n4 ? xr[c] : make_float4(0.f, 0.f, 0.f, 0.f);
  }
  float ss = 0.f;
#pragma unroll
  for (int i = 0; i < NV; ++i)
    if (lane + 64 * i < n4) ss = sumsq4(v[i], ss);
  ss = wave_sum(ss);
  const float rstd = 1.0f / sqrtf(ss / (float)dim + eps);
#pragma unroll
  for (int i = 0; i < NV; ++i) {
    const int c = lane + 64 * i;
    if (c >= n4) continue;
    const float4 s = w4[c];
    TO4 o;
    o[0] = from_f32<TO>(s.x * (v[i].x * rstd));
    o[1] = from_f32<TO>(s.y * (v[i].y * rstd));
    o[2] = from_f32<TO>(s.z * (v[i].z * rstd));
    o[3] = from_f32<TO>(s.w * (v[i].w * rstd));
    *reinterpret_cast<TO4*>(out + row * dim + 4 * c) = o;
  }
}

// ---------------------------------------------------------------------------
// Rotary table (vision page, get_vision_cos_sin): entry (p, k), k < D/2, holds
// (cos, sin) of row * theta^(-k/(D/4)) for k < D/4 and of
// col * theta^(-(k-D/4)/(D/4)) otherwise; row/col restart at every image.
// Built in double precision, stored as float2.
VIT_DEV void rope_table_elem(const VarlenDesc& d, int head_dim, const RopeFreqs& fr,
                             float2* table, int64_t idx) {
  const int half = head_dim / 2, q4 = head_dim / 4;
  if (idx >= (int64_t)d.total * half) return;
  const int p = (int)(idx / half);
  const int k = (int)(idx % half);
  const int img = find_image(d, p);
  const int local = p - d.cu_seqlens[img];
  const int gw = d.grid_w[img];
  const int pos = (k < q4) ? local / gw : local % gw;
  const int kk = (k < q4) ? k : k - q4;
  double s, c;
  sincos((double)pos * fr.f[kk], &s, &c);
  table[idx] = make_float2((float)c, (float)s);
}

__global__ void rope_table_kernel(VarlenDesc d, int head_dim, RopeFreqs fr, float2* table) {
  rope_table_elem(d, head_dim, fr, table, (int64_t)blockIdx.x * blockDim.x + threadIdx.x);
}

// ---------------------------------------------------------------------------
// Half-split 2D rotary (vision page, apply_vision_rotary) on the q and k parts of
// a packed [P, 3*H*D] qkv buffer, in place, fp32 math.  One thread per V
// consecutive rotated pairs (i, i + D/4) inside one half of one head, so the
// two operands and the V table entries move as V-wide vectors (the host picks
// the widest V that divides D/4 and the pointers' alignment).
template <typename T, int V>
struct alignas(sizeof(T) * V) RopeVec {
  T v[V];
};

// With INV the rotation is by the opposite angles (the transpose), which maps a
// gradient with respect to the rotated q, k back to one with respect to q, k.
template <typename T, int V, bool INV>
__global__ void rope_kernel(T* qkv, const float2* __restrict__ table, int64_t P, int H, int D) {
  const int q4 = D / 4, qv = q4 / V;
  const int per_row = 4 * H * qv;  // 2 parts * H heads * 2 halves * D/(4V)
  const int64_t idx = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (idx >= P * per_row) return;
  const int64_t p = idx / per_row;
  int j = (int)(idx % per_row);
  const int kk = (j % qv) * V;
  j /= qv;
  const int half = j & 1;
  j >>= 1;
  const int h = j % H;
  const int part = j / H;  // 0 = q, 1 = k
  const int d = H * D;
  T* row = qkv + p * (3 * (int64_t)d) + part * d + h * D + half * (D / 2);
  const float2* cs = table + p * (D / 2) + half * q4 + kk;
  RopeVec<T, V> x1 = *reinterpret_cast<const RopeVec<T, V>*>(row + kk);
  RopeVec<T, V> x2 = *reinterpret_cast<const RopeVec<T, V>*>(row + kk + q4);
  RopeVec<float2, V> c = *reinterpret_cast<const RopeVec<float2, V>*>(cs);
#pragma unroll
  for (int e = 0; e < V; ++e) {
    const float a1 = to_f32(x1.v[e]), a2 = to_f32(x2.v[e]);
    const float sn = INV ? -c.v[e].y : c.v[e].y;
    x1.v[e] = from_f32<T>(a1 * c.v[e].x - a2 * sn);
    x2.v[e] = from_f32<T>(a2 * c.v[e].x + a1 * sn);
  }
  *reinterpret_cast<RopeVec<T, V>*>(row + kk) = x1;
  *reinterpret_cast<RopeVec<T, V>*>(row + kk + q4) = x2;
}

// ---------------------------------------------------------------------------
// 2x2 aligner gather (vision page, DeepseekV4VisionAligner): merged token t of
// image i concatenates patches TL, TR, BL, BR of its group.  One thread per
// 16-byte chunk of the output.
template <typename T>
__global__ void gather_kernel(const T* __restrict__ x, VarlenDesc d, int dim, int merge,
                              T* __restrict__ G) {
  constexpr int V = 16 / sizeof(T);
  const int m2 = merge * merge;
  const int64_t row_chunks = (int64_t)m2 * dim / V;
  const int64_t tokens = d.cu_tokens[d.n_images];
  const int64_t idx = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (idx >= tokens * row_chunks) return;
  const int64_t t = idx / row_chunks;
  const int col = (int)(idx % row_chunks) * V;
  const int s = col / dim;
  const int e = col % dim;
  // image of merged token t
  int img = 0;
  while (img + 1 < d.n_images && t >= d.cu_tokens[img + 1]) ++img;
  const int tl = (int)(t - d.cu_tokens[img]);
  const int gw = d.grid_w[img];
  const int gh = (d.cu_seqlens[img + 1] - d.cu_seqlens[img]) / gw;
  const int wq = (gw + merge - 1) / merge;  // merged columns (odd grids zero-padded)
  const int gi = tl / wq, gj = tl % wq;
  const int r = merge * gi + s / merge, c = merge * gj + s % merge;
  u32x4 v = {0u, 0u, 0u, 0u};
  if (r < gh && c < gw) v = ld16(x + ((int64_t)d.cu_seqlens[img] + r * gw + c) * dim + e);
  st16(G + t * (int64_t)m2 * dim + col, v);
}

// Copy rows [rows, cols] into [rows, ld_dst] zero-padding columns cols..ld_dst-1.
// cols and ld_dst multiples of 4; one thread per 4 elements.
template <typename T>
VIT_DEV void pad_rows_elem(const T* __restrict__ src, int64_t rows, int64_t cols, int64_t ld_dst,
                           T* __restrict__ dst, int64_t idx) {
  const int64_t q = ld_dst / 4;
  if (idx >= rows * q) return;
  const int64_t r = idx / q;
  const int64_t c = (idx % q) * 4;
  T* o = dst + r * ld_dst + c;
  if constexpr (sizeof(T) == 2) {
    // bf16 with 4-element aligned rows: one 8-byte load and store per thread
    if (cols % 4 == 0 && ((uintptr_t)src & 7) == 0 && ((uintptr_t)dst & 7) == 0 &&
        ld_dst % 4 == 0) {
      uint2 v = make_uint2(0u, 0u);
      if (c < cols) v = *reinterpret_cast<const uint2*>(src + r * cols + c);
      *reinterpret_cast<uint2*>(o) = v;
      return;
    }
  }
  T v[4];
  for (int k = 0; k < 4; ++k) v[k] = c + k < cols ? src[r * cols + c + k] : from_f32<T>(0.f);
  for (int k = 0; k < 4; ++k) o[k] = v[k];
}

template <typename T>
__global__ void pad_rows_kernel(const T* __restrict__ src, int64_t rows, int64_t cols,
                                int64_t ld_dst, T* __restrict__ dst) {
  pad_rows_elem(src, rows, cols, ld_dst, dst, (int64_t)blockIdx.x * blockDim.x + threadIdx.x);
}

// Column of every patch in the transposed-V layout (images start 64-aligned).
VIT_DEV void vpos_elem(const VarlenDesc& d, int32_t* vpos, int64_t idx) {
  const int p = (int)idx;
  if (idx >= d.total) return;
  const int img = find_image(d, p);
  vpos[p] = d.kv_off[img] + vt_key_slot(p - d.cu_seqlens[img]);
}

__global__ void vpos_kernel(VarlenDesc d, int32_t* vpos) {
  vpos_elem(d, vpos, (int64_t)blockIdx.x * blockDim.x + threadIdx.x);
}

// Zero the slots of vt that hold no key: in image i, every slot from the start
// of the 16-key group containing key P_i up to kv_off_{i+1} whose key is >= P_i.
VIT_DEV void vt_zero_pads_elem(const VarlenDesc& d, int64_t rows, bf16* vt, int64_t ld,
                               int64_t row, int c) {
  // c: offset from the start of the 16-key group holding key P_i
  if (row >= rows || c >= VT_ALIGN + 16) return;
  for (int i = 0; i < d.n_images; ++i) {
    const int P = d.cu_seqlens[i + 1] - d.cu_seqlens[i];
    const int j = (P & ~15) + c;  // local slot
    if (d.kv_off[i] + j < d.kv_off[i + 1] && vt_key_slot(j) >= P)
      vt[row * ld + d.kv_off[i] + j] = f2bf(0.f);
  }
}

__global__ void vt_zero_pads_kernel(VarlenDesc d, int64_t rows, bf16* vt, int64_t ld) {
  vt_zero_pads_elem(d, rows, vt, ld, blockIdx.y, blockIdx.x * blockDim.x + threadIdx.x);
}

// Patch (p, k) of a packed batch of pixel images (image i: [3, ps*gh_i, ps*gw_i]
// C order, images back to back, so image i starts at element patch_dim *
// cu_seqlens[i]): patch p = r*gw + c of its image holds pixel rows ps*r.., cols
// ps*c.. flattened in [3, ps, ps] C order (the layout DeepseekV4VisionTransformer
// .forward expects).  Columns k >= patch_dim of the padded row are zero.
template <typename T>
VIT_DEV void patchify_elem(const T* __restrict__ pix, const VarlenDesc& d, int ps, int64_t ld_dst,
                           T* __restrict__ dst, int64_t idx) {
  if (idx >= (int64_t)d.total * ld_dst) return;
  const int p = (int)(idx / ld_dst);
  const int k = (int)(idx % ld_dst);
  const int pd = 3 * ps * ps;
  T v = from_f32<T>(0.f);
  if (k < pd) {
    int lo = 0, hi = d.n_images - 1;  // image of patch p: last i with cu_seqlens[i] <= p
    while (lo < hi) {
      const int mid = (lo + hi + 1) >> 1;
      if (d.cu_seqlens[mid] <= p) lo = mid; else hi = mid - 1;
    }
    const int start = d.cu_seqlens[lo];
    const int gw = d.grid_w[lo];
    const int gh = (d.cu_seqlens[lo + 1] - start) / gw;
    const int local = p - start, r = local / gw, c = local % gw;
    const int ch = k / (ps * ps), y = (k % (ps * ps)) / ps, x = k % ps;
    const int64_t W = (int64_t)gw * ps, Hh = (int64_t)gh * ps;
    v = pix[(int64_t)pd * start + (ch * Hh + (int64_t)r * ps + y) * W + (int64_t)c * ps + x];
  }
  dst[idx] = v;
}

// bf16 pixels with an even patch size and 4-byte aligned rows: one thread per
// (patch, channel, pixel row of the patch) copies the ps contiguous pixels of
// that row as ps/2 32-bit words into the patch row; unit 3*ps of a patch zeroes
// the padding columns pd .. ld_dst-1.  Same result as patchify_elem.
VIT_DEV void patchify_rows_elem(const bf16* __restrict__ pix, const VarlenDesc& d, int ps,
                                int64_t ld_dst, bf16* __restrict__ dst, int64_t idx) {
  const int units = 3 * ps + 1;
  if (idx >= (int64_t)d.total * units) return;
  const int p = (int)(idx / units);
  const int u = (int)(idx % units);
  const int pd = 3 * ps * ps;
  uint32_t* o = reinterpret_cast<uint32_t*>(dst + (int64_t)p * ld_dst);
  if (u == 3 * ps) {
    for (int k = pd / 2; k < ld_dst / 2; ++k) o[k] = 0u;
    return;
  }
  const int img = find_image(d, p);
  const int start = d.cu_seqlens[img], gw = d.grid_w[img];
  const int gh = (d.cu_seqlens[img + 1] - start) / gw;
  const int local = p - start, r = local / gw, c = local % gw;
  const int ch = u / ps, y = u % ps;
  const int64_t W = (int64_t)gw * ps, Hh = (int64_t)gh * ps;
  const uint32_t* src = reinterpret_cast<const uint32_t*>(
      pix + (int64_t)pd * start + (ch * Hh + (int64_t)r * ps + y) * W + (int64_t)c * ps);
  uint32_t* out = o + (ch * ps * ps + y * ps) / 2;
  for (int k = 0; k < ps / 2; ++k) out[k] = src[k];
}

template <typename T>
__global__ void patchify_kernel(const T* __restrict__ pix, VarlenDesc d, int ps, int64_t ld_dst,
                                T* __restrict__ dst) {
  patchify_elem(pix, d, ps, ld_dst, dst, (int64_t)blockIdx.x * blockDim.x + threadIdx.x);
}

// Source rows of merged token t's 2x2 group for the aligner's gathered A
// operand: a_rows[4t + s] = patch row of the group's s-th patch (TL, TR, BL, BR;
// the aligner's row-major order inside the group), or `zero_row` where an odd
// grid is zero-padded to even (VIT_ALIGN_PAD).
VIT_DEV void aligner_rows_elem(const VarlenDesc& d, int32_t zero_row, int32_t* a_rows,
                               int64_t idx) {
  const int64_t tokens = d.cu_tokens[d.n_images];
  if (idx >= tokens * 4) return;
  const int64_t t = idx / 4;
  const int s = (int)(idx % 4);
  int img = 0;
  while (img + 1 < d.n_images && t >= d.cu_tokens[img + 1]) ++img;
  const int tl = (int)(t - d.cu_tokens[img]);
  const int gw = d.grid_w[img];
  const int gh = (d.cu_seqlens[img + 1] - d.cu_seqlens[img]) / gw;
  const int wq = (gw + 1) / 2;  // merged columns (odd grids zero-padded)
  const int r = 2 * (tl / wq) + s / 2, c = 2 * (tl % wq) + s % 2;
  a_rows[idx] = (r < gh && c < gw) ? d.cu_seqlens[img] + r * gw + c : zero_row;
}

// Everything an encode call prepares before the patch embedding, in one
// launch: block ranges [0, b[0]) pad the patches, [b[0], b[1]) pad the
// patch-embedding weight, [b[1], b[2]) build the rotary table, [b[2], b[3])
// the transposed-V positions, [b[3], b[4]) zero the transposed-V padding,
// [b[4], b[5]) the aligner's merged-token source rows and [b[5], b[6]) zero the
// row those name for padding.
__global__ __launch_bounds__(kThreads) void encode_prep_kernel(PrepArgs a) {
  const int64_t b = blockIdx.x;
  const int t = threadIdx.x;
  if (b < a.b[0]) {
    if (a.pixel_ps > 0 && a.pix_rows)
      patchify_rows_elem((const bf16*)a.patches, a.desc, a.pixel_ps, a.Kp, (bf16*)a.xpad,
                         b * kThreads + t);
    else if (a.pixel_ps > 0)
      patchify_elem((const bf16*)a.patches, a.desc, a.pixel_ps, a.Kp, (bf16*)a.xpad,
                    b * kThreads + t);
    else
      pad_rows_elem((const bf16*)a.patches, a.P, a.patch_dim, a.Kp, (bf16*)a.xpad,
                    b * kThreads + t);
  } else if (b < a.b[1]) {
    pad_rows_elem((const bf16*)a.w_pe, a.d, a.patch_dim, a.Kp, (bf16*)a.wpe,
                  (b - a.b[0]) * kThreads + t);
  } else if (b < a.b[2]) {
    rope_table_elem(a.desc, a.head_dim, a.freqs, (float2*)a.table, (b - a.b[1]) * kThreads + t);
  } else if (b < a.b[3]) {
    vpos_elem(a.desc, a.vpos, (b - a.b[2]) * kThreads + t);
  } else if (b < a.b[4]) {
    const int64_t i = (b - a.b[3]) * kThreads + t;
    vt_zero_pads_elem(a.desc, a.vt_rows, (bf16*)a.vt, a.vt_ld, i / (VT_ALIGN + 16),
                      (int)(i % (VT_ALIGN + 16)));
  } else if (b < a.b[5]) {
    aligner_rows_elem(a.desc, (int32_t)a.P, a.a_rows, (b - a.b[4]) * kThreads + t);
  } else if (b < a.b[6]) {
    const int64_t i = (b - a.b[5]) * kThreads + t;  // 8 bf16 per thread
    if (i < a.d / 8) reinterpret_cast<u32x4*>(a.zrow)[i] = u32x4{0u, 0u, 0u, 0u};
  }
}

// Columns col0 .. col0 + H*D of src [P, ld_src] transposed into a V^T layout:
// dst[h*D + e][kv_off[img] + slot] = src[cu[img] + key(slot)][col0 + h*D + e],
// zero past the image, where key() orders the keys of a 64-key tile for the
// MFMA that reads them (vt_key_slot for the 32x32x16 layout of head_dim 64,
// vt16_slot_key for the 16x16x32 layout of head_dim 72).  One block per
// (64-key tile of an image span, head): 64 source rows of D elements into
// LDS, then D destination rows of 64 slots.
// With a rotary table (head_dim 72 encode, src = the packed qkv buffer, col0 =
// its V part), the block also applies the half-split 2D rotary to the q and k
// rows of its keys and head in place, as rope_kernel does (fp32 math, pairs
// (i, i + D/4) of each half, two pairs per access).
template <int D, bool K16>
__global__ __launch_bounds__(256) void tpack_kernel(const bf16* __restrict__ src, int64_t ld_src,
                                                    int64_t col0, VarlenDesc d,
                                                    bf16* __restrict__ dst, int64_t ld,
                                                    const float2* __restrict__ rope_table) {
  constexpr int CH = D / 8;  // 16-byte chunks per source row
  constexpr int N = 64 * CH;  // chunks per tile, both ways
  __shared__ bf16 tile[64][D + 2];
  const int col = blockIdx.x * 64;  // first destination column (a 64-aligned span start + 64 j)
  const int h = blockIdx.y;
  int img = 0;
  while (img + 1 < d.n_images && col >= d.kv_off[img + 1]) ++img;
  const int k0 = col - d.kv_off[img];  // first key of the tile
  const int P = d.cu_seqlens[img + 1] - d.cu_seqlens[img];
#pragma unroll
  for (int k = 0; k < (N + 255) / 256; ++k) {
    const int q = threadIdx.x + 256 * k;
    if (q >= N) break;
    const int r = q / CH, ch = q % CH;  // key row, 8-element chunk
    bf16x8 v;
    if (k0 + r < P) {
      v = __builtin_bit_cast(bf16x8, ld16(src + (int64_t)(d.cu_seqlens[img] + k0 + r) * ld_src +
                                          col0 + h * D + ch * 8));
    } else {
#pragma unroll
      for (int e = 0; e < 8; ++e) v[e] = f2bf(0.f);
    }
#pragma unroll
    for (int e = 0; e < 8; ++e) tile[r][ch * 8 + e] = v[e];
  }
  if (rope_table) {
    static_assert(D % 8 == 0, "two pairs per access");
    constexpr int q4 = D / 4, qv = q4 / 2;
    const int64_t dm = (int64_t)gridDim.y * D;
    for (int it = threadIdx.x; it < 64 * 4 * qv; it += 256) {
      const int r = it / (4 * qv);
      int j = it % (4 * qv);
      const int kk = (j % qv) * 2;
      j /= qv;
      const int half = j & 1, part = j >> 1;  // part 0 = q, 1 = k
      if (k0 + r >= P) continue;
      const int64_t p = d.cu_seqlens[img] + k0 + r;
      bf16* row = const_cast<bf16*>(src) + p * ld_src + part * dm + h * D + half * (D / 2);
      const float4 cs = *reinterpret_cast<const float4*>(rope_table + p * (D / 2) + half * q4 + kk);
      bf16x2 x1 = *reinterpret_cast<const bf16x2*>(row + kk);
      bf16x2 x2 = *reinterpret_cast<const bf16x2*>(row + kk + q4);
      const float a0 = bf2f(x1[0]), a1 = bf2f(x1[1]), b0 = bf2f(x2[0]), b1 = bf2f(x2[1]);
      x1[0] = f2bf(a0 * cs.x - b0 * cs.y);
      x2[0] = f2bf(b0 * cs.x + a0 * cs.y);
      x1[1] = f2bf(a1 * cs.z - b1 * cs.w);
      x2[1] = f2bf(b1 * cs.z + a1 * cs.w);
      *reinterpret_cast<bf16x2*>(row + kk) = x1;
      *reinterpret_cast<bf16x2*>(row + kk + q4) = x2;
    }
  }
  __syncthreads();
#pragma unroll
  for (int k = 0; k < (N + 255) / 256; ++k) {
    const int q = threadIdx.x + 256 * k;
    if (q >= N) break;
    const int e = q >> 3, ch = q & 7;  // destination row (dim), chunk of 8 slots
    bf16x8 v;
#pragma unroll
    for (int j = 0; j < 8; ++j)
      v[j] = tile[K16 ? vt16_slot_key(ch * 8 + j) : vt_key_slot(ch * 8 + j)][e];
    st16(dst + (int64_t)(h * D + e) * ld + col + ch * 8, __builtin_bit_cast(u32x4, v));
  }
}

// Zero columns [c0, c1) of every row of a [rows, ld] buffer.
template <typename T>
__global__ void zero_cols_kernel(T* buf, int64_t rows, int64_t ld, int64_t c0, int64_t c1) {
  const int64_t w = c1 - c0;
  const int64_t idx = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (idx >= rows * w) return;
  buf[(idx / w) * ld + c0 + idx % w] = from_f32<T>(0.f);
}

// Aligner layout arrays of one image (permutation and newline layout).
__global__ void layout_kernel(int gh, int gw, int merge, int32_t* perm, int32_t* nl_type,
                              int32_t* nl_src) {
  const int idx = blockIdx.x * blockDim.x + threadIdx.x;
  const int m2 = merge * merge;
  const int hq = gh / merge, wq = gw / merge;
  if (perm && idx < gh * gw) {
    const int t = idx / m2, s = idx % m2;
    const int gi = t / wq, gj = t % wq;
    perm[idx] = (merge * gi + s / merge) * gw + merge * gj + s % merge;
  }
  const int L = hq * (wq + 1) + 2;
  if (idx < L) {
    int type, src;
    if (idx == 0) {
      type = 0; src = -1;
    } else if (idx == L - 1) {
      type = 3; src = -1;
    } else {
      const int q = idx - 1;
      const int r = q / (wq + 1), c = q % (wq + 1);
      if (c == wq) { type = 2; src = -1; } else { type = 1; src = r * wq + c; }
    }
    if (nl_type) nl_type[idx] = type;
    if (nl_src) nl_src[idx] = src;
  }
}

// Output row of every merged token when the aligner writes newline-layout spans.
__global__ void nl_rowmap_kernel(VarlenDesc d, int merge, int32_t* rowmap) {
  const int t = blockIdx.x * blockDim.x + threadIdx.x;
  if (t >= d.cu_tokens[d.n_images]) return;
  int img = 0, base = 0;
  while (img + 1 < d.n_images && t >= d.cu_tokens[img + 1]) {
    const int wq = (d.grid_w[img] + merge - 1) / merge;
    const int hq = (d.cu_tokens[img + 1] - d.cu_tokens[img]) / wq;
    base += hq * (wq + 1) + 2;
    ++img;
  }
  const int tl = t - d.cu_tokens[img];
  const int wq = (d.grid_w[img] + merge - 1) / merge;
  rowmap[t] = base + 1 + (tl / wq) * (wq + 1) + tl % wq;
}

inline unsigned blocks_for(int64_t n, int t = kThreads) { return (unsigned)((n + t - 1) / t); }

}  // namespace

hipError_t launch_rmsnorm(const float* x, const float* w, float eps, int64_t rows, int dim,
                          int out_dtype, void* out, hipStream_t s) {
  if (rows == 0) return hipSuccess;
  const unsigned grid = (unsigned)((rows + 3) / 4);
  const size_t osz = out_dtype == VIT_BF16 ? 2 : 4;
  // register-resident rows for dim <= 2048 when the output takes 4-element stores
  const int nv = dim <= 256 ? 1 : dim <= 512 ? 2 : dim <= 1024 ? 4 : dim <= 2048 ? 8 : 0;
  if (nv && (uintptr_t)out % (4 * osz) == 0) {
#define VIT_RMS_REG(NV_)                                                                        \
  if (out_dtype == VIT_BF16)                                                                    \
    rmsnorm_reg_kernel<bf16, NV_><<<grid, kThreads, 0, s>>>(x, w, eps, rows, dim, (bf16*)out);  \
  else                                                                                          \
    rmsnorm_reg_kernel<float, NV_><<<grid, kThreads, 0, s>>>(x, w, eps, rows, dim, (float*)out)
    switch (nv) {
      case 1: VIT_RMS_REG(1); break;
      case 2: VIT_RMS_REG(2); break;
      case 4: VIT_RMS_REG(4); break;
      default: VIT_RMS_REG(8); break;
    }
#undef VIT_RMS_REG
    return hipGetLastError();
  }
  if (out_dtype == VIT_BF16)
    rmsnorm_kernel<bf16><<<grid, kThreads, 0, s>>>(x, w, eps, rows, dim, (bf16*)out);
  else
    rmsnorm_kernel<float><<<grid, kThreads, 0, s>>>(x, w, eps, rows, dim, (float*)out);
  return hipGetLastError();
}

RopeFreqs rope_freqs(int head_dim, double theta) {
  RopeFreqs fr{};
  const int q4 = head_dim / 4;
  for (int k = 0; k < q4 && k < kRopeMaxFreqs; ++k) fr.f[k] = std::pow(theta, -(double)k / q4);
  return fr;
}

hipError_t launch_rope_table(const VarlenDesc& d, int head_dim, float theta, void* table,
                             hipStream_t s) {
  const int64_t n = (int64_t)d.total * (head_dim / 2);
  if (n == 0) return hipSuccess;
  if (head_dim / 4 > kRopeMaxFreqs) return hipErrorInvalidValue;
  rope_table_kernel<<<blocks_for(n), kThreads, 0, s>>>(d, head_dim, rope_freqs(head_dim, theta),
                                                        (float2*)table);
  return hipGetLastError();
}

template <typename T, bool INV = false>
hipError_t launch_rope_t(T* qkv, const float2* table, int64_t P, int H, int D, hipStream_t s) {
  const int q4 = D / 4;
  auto fits = [&](int v) {
    return q4 % v == 0 && (uintptr_t)qkv % (v * sizeof(T)) == 0 &&
           (uintptr_t)table % (v * sizeof(float2)) == 0;
  };
  const int64_t pairs = P * H * D;  // 2 parts * 2 halves * D/4 pairs per head
  if (fits(4))
    rope_kernel<T, 4, INV><<<blocks_for(pairs / 4), kThreads, 0, s>>>(qkv, table, P, H, D);
  else if (fits(2))
    rope_kernel<T, 2, INV><<<blocks_for(pairs / 2), kThreads, 0, s>>>(qkv, table, P, H, D);
  else
    rope_kernel<T, 1, INV><<<blocks_for(pairs), kThreads, 0, s>>>(qkv, table, P, H, D);
  return hipGetLastError();
}

hipError_t launch_rope(int dtype, void* qkv, const void* table, int64_t P, int n_heads,
                       int head_dim, hipStream_t s) {
  if (P * n_heads * head_dim == 0) return hipSuccess;
  if (dtype == VIT_BF16)
    return launch_rope_t((bf16*)qkv, (const float2*)table, P, n_heads, head_dim, s);
  return launch_rope_t((float*)qkv, (const float2*)table, P, n_heads, head_dim, s);
}
hipError_t launch_rope_inverse(void* qkv, const void* table, int64_t P, int n_heads, int head_dim,
                               hipStream_t s) {
  if (P * n_heads * head_dim == 0) return hipSuccess;
  return launch_rope_t<bf16, true>((bf16*)qkv, (const float2*)table, P, n_heads, head_dim, s);
}

hipError_t launch_gather(int dtype, const void* x, const VarlenDesc& d, int dim, int merge,
                         void* G, hipStream_t s) {
  const int esz = dtype == VIT_BF16 ? 2 : 4;
  const int64_t n = (int64_t)d.cu_tokens[d.n_images] * merge * merge * dim * esz / 16;
  if (n == 0) return hipSuccess;
  if (dtype == VIT_BF16)
    gather_kernel<bf16><<<blocks_for(n), kThreads, 0, s>>>((const bf16*)x, d, dim, merge,
                                                           (bf16*)G);
  else
    gather_kernel<float><<<blocks_for(n), kThreads, 0, s>>>((const float*)x, d, dim, merge,
                                                            (float*)G);
  return hipGetLastError();
}

hipError_t launch_pad_rows(int dtype, const void* src, int64_t rows, int64_t cols, int64_t ld_dst,
                           void* dst, hipStream_t s) {
  const int64_t n = rows * (ld_dst / 4);
  if (n == 0) return hipSuccess;
  if (dtype == VIT_BF16)
    pad_rows_kernel<bf16><<<blocks_for(n), kThreads, 0, s>>>((const bf16*)src, rows, cols,
                                                             ld_dst, (bf16*)dst);
  else
    pad_rows_kernel<float><<<blocks_for(n), kThreads, 0, s>>>((const float*)src, rows, cols,
                                                              ld_dst, (float*)dst);
  return hipGetLastError();
}

hipError_t launch_zero_cols(int dtype, void* buf, int64_t rows, int64_t ld, int64_t c0, int64_t c1,
                            hipStream_t s) {
  const int64_t n = rows * (c1 - c0);
  if (n <= 0) return hipSuccess;
  if (dtype == VIT_BF16)
    zero_cols_kernel<bf16><<<blocks_for(n), kThreads, 0, s>>>((bf16*)buf, rows, ld, c0, c1);
  else
    zero_cols_kernel<float><<<blocks_for(n), kThreads, 0, s>>>((float*)buf, rows, ld, c0, c1);
  return hipGetLastError();
}

hipError_t launch_encode_prep(PrepArgs a, hipStream_t s) {
  if (a.table && a.head_dim / 4 > kRopeMaxFreqs) return hipErrorInvalidValue;
  a.pix_rows = a.pixel_ps > 0 && a.pixel_ps % 2 == 0 && a.Kp % 2 == 0 &&
               ((uintptr_t)a.patches & 3) == 0 && ((uintptr_t)a.xpad & 3) == 0;
  const int64_t n[7] = {a.patches ? a.P * (a.pix_rows ? 3 * a.pixel_ps + 1
                                           : a.pixel_ps > 0 ? a.Kp : a.Kp / 4) : 0,
                        a.w_pe ? a.d * (a.Kp / 4) : 0,
                        a.table ? (int64_t)a.desc.total * (a.head_dim / 2) : 0,
                        a.vpos ? (int64_t)a.desc.total : 0,
                        a.vt ? a.vt_rows * (VT_ALIGN + 16) : 0,
                        a.a_rows ? a.tokens * 4 : 0,
                        a.zrow ? a.d / 8 : 0};
  if (a.zrow && (a.d % 8 || ((uintptr_t)a.zrow & 15))) return hipErrorInvalidValue;
  int64_t acc = 0;
  for (int i = 0; i < 7; ++i) {
    acc += (n[i] + kThreads - 1) / kThreads;
    a.b[i] = acc;
  }
  if (acc == 0) return hipSuccess;
  encode_prep_kernel<<<dim3((unsigned)acc), kThreads, 0, s>>>(a);
  return hipGetLastError();
}

hipError_t launch_patchify(int dtype, const void* pix, const VarlenDesc& d, int ps, int64_t ld_dst,
                           void* dst, hipStream_t s) {
  const int64_t n = (int64_t)d.total * ld_dst;
  if (n == 0) return hipSuccess;
  if (dtype == VIT_BF16)
    patchify_kernel<bf16><<<blocks_for(n), kThreads, 0, s>>>((const bf16*)pix, d, ps, ld_dst,
                                                             (bf16*)dst);
  else
    patchify_kernel<float><<<blocks_for(n), kThreads, 0, s>>>((const float*)pix, d, ps, ld_dst,
                                                              (float*)dst);
  return hipGetLastError();
}

hipError_t launch_vpos(const VarlenDesc& d, int32_t* vpos, hipStream_t s) {
  if (d.total == 0) return hipSuccess;
  vpos_kernel<<<blocks_for(d.total), kThreads, 0, s>>>(d, vpos);
  return hipGetLastError();
}

hipError_t launch_vt_zero_pads(const VarlenDesc& d, int64_t rows, void* vt, int64_t vt_ld,
                               hipStream_t s) {
  if (rows == 0) return hipSuccess;
  vt_zero_pads_kernel<<<dim3(1, (unsigned)rows), VT_ALIGN + 16, 0, s>>>(d, rows, (bf16*)vt,
                                                                        vt_ld);
  return hipGetLastError();
}

hipError_t launch_tpack(const void* src, int64_t ld_src, int64_t col0, const VarlenDesc& d,
                        int n_heads, int head_dim, void* dst, int64_t ld, hipStream_t s) {
  const int cols = d.kv_off[d.n_images];
  if (cols == 0) return hipSuccess;
  if (ld_src % 8 || col0 % 8 || ld % 8) return hipErrorInvalidValue;
  const dim3 grid((unsigned)(cols / 64), (unsigned)n_heads);
  if (head_dim == 64)
    tpack_kernel<64, false><<<grid, 256, 0, s>>>((const bf16*)src, ld_src, col0, d, (bf16*)dst, ld,
                                                 nullptr);
  else if (head_dim == 72)
    tpack_kernel<72, false><<<grid, 256, 0, s>>>((const bf16*)src, ld_src, col0, d, (bf16*)dst, ld,
                                                 nullptr);
  else
    return hipErrorInvalidValue;
  return hipGetLastError();
}

hipError_t launch_vt_pack(const void* qkv, const VarlenDesc& d, int n_heads, int head_dim,
                          void* vt, int64_t vt_ld, hipStream_t s, const void* rope_table) {
  const int64_t dm = (int64_t)n_heads * head_dim;
  if (head_dim == 64 && !rope_table) return launch_tpack(qkv, 3 * dm, 2 * dm, d, n_heads, 64, vt, vt_ld, s);
  if (head_dim != 72 || vt_ld % 8) return hipErrorInvalidValue;
  if (rope_table && (((uintptr_t)qkv & 3) || ((uintptr_t)rope_table & 15)))
    return hipErrorInvalidValue;
  const int cols = d.kv_off[d.n_images];
  if (cols == 0) return hipSuccess;
  tpack_kernel<72, true><<<dim3((unsigned)(cols / 64), (unsigned)n_heads), 256, 0, s>>>(
      (const bf16*)qkv, 3 * dm, 2 * dm, d, (bf16*)vt, vt_ld, (const float2*)rope_table);
  return hipGetLastError();
}

hipError_t launch_layout(int grid_h, int grid_w, int merge, int32_t* perm, int32_t* nl_type,
                         int32_t* nl_src, hipStream_t s) {
  const int n = grid_h * grid_w + 2 * grid_h + 2;  // >= both array lengths
  layout_kernel<<<blocks_for(n), kThreads, 0, s>>>(grid_h, grid_w, merge, perm, nl_type, nl_src);
  return hipGetLastError();
}

hipError_t launch_nl_rowmap(const VarlenDesc& d, int merge, int32_t* rowmap, hipStream_t s) {
  const int n = d.cu_tokens[d.n_images];
  if (n == 0) return hipSuccess;
  nl_rowmap_kernel<<<blocks_for(n), kThreads, 0, s>>>(d, merge, rowmap);
  return hipGetLastError();
}
