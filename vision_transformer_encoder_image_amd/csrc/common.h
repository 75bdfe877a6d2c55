// Shared device/host helpers of the gfx950 encoder library.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "vitenc.h"

#define VIT_DEV __device__ __forceinline__

typedef __bf16 bf16;
typedef __attribute__((__vector_size__(8 * sizeof(__bf16)))) __bf16 bf16x8;
typedef __attribute__((__vector_size__(4 * sizeof(__bf16)))) __bf16 bf16x4;
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef __attribute__((__vector_size__(4 * sizeof(float)))) float f32x4;
typedef __attribute__((__vector_size__(16 * sizeof(float)))) float f32x16;
typedef __attribute__((__vector_size__(4 * sizeof(uint32_t)))) uint32_t u32x4;

// 16-byte global load of a native vector (no HIP struct temporaries).
VIT_DEV u32x4 ld16(const void* p) { return *reinterpret_cast<const u32x4*>(p); }
VIT_DEV void st16(void* p, u32x4 v) { *reinterpret_cast<u32x4*>(p) = v; }

// Round-to-nearest-even float -> bf16 (finite values; NaN stays NaN).
VIT_DEV bf16 f2bf(float f) { return (bf16)f; }
VIT_DEV float bf2f(bf16 b) { return (float)b; }

template <typename T> VIT_DEV T from_f32(float v);
template <> VIT_DEV float from_f32<float>(float v) { return v; }
template <> VIT_DEV bf16 from_f32<bf16>(float v) { return f2bf(v); }
VIT_DEV float to_f32(float v) { return v; }
VIT_DEV float to_f32(bf16 v) { return bf2f(v); }

// Wave-wide (64 lanes) reductions through cross-lane shuffles.
VIT_DEV float wave_sum(float v) {
#pragma unroll
  for (int m = 32; m >= 1; m >>= 1) v += __shfl_xor(v, m, 64);
  return v;
}
VIT_DEV float wave_max(float v) {
#pragma unroll
  for (int m = 32; m >= 1; m >>= 1) v = fmaxf(v, __shfl_xor(v, m, 64));
  return v;
}

// s_waitcnt with only vmcnt constrained (gfx9 encoding: vmcnt[3:0] | expcnt[6:4]
// | lgkmcnt[11:8] | vmcnt[5:4] << 14).
template <int N>
VIT_DEV void wait_vmcnt() {
  static_assert(N >= 0 && N < 64, "vmcnt range");
  __builtin_amdgcn_s_waitcnt((N & 15) | (0x7 << 4) | (0xF << 8) | ((N >> 4) << 14));
}

// 16-byte global -> LDS copy per lane (global_load_lds_dwordx4): lane i writes
// bytes [16 i, 16 i + 16) after the wave-uniform LDS address.  The builtin only
// exists for the gfx950 device pass, so the host pass sees an empty body.
VIT_DEV void copy16_to_lds(const void* gptr, void* lptr) {
#if defined(__HIP_DEVICE_COMPILE__)
  __builtin_amdgcn_global_load_lds(gptr, (__attribute__((address_space(3))) void*)lptr, 16, 0, 0);
#else
  (void)gptr;
  (void)lptr;
#endif
}

// s_waitcnt with only lgkmcnt (LDS) constrained: at most N LDS operations of
// this wave may still be outstanding.
template <int N>
VIT_DEV void wait_lgkmcnt() {
  static_assert(N >= 0 && N < 16, "lgkmcnt range");
  __builtin_amdgcn_s_waitcnt(0xF | (0x7 << 4) | (N << 8) | (0x3 << 14));
}

// max over lanes l and l ^ 32 without the LDS crossbar (a ds_bpermute would
// count against lgkmcnt and wait for every LDS read issued before it):
// v_permlane32_swap exchanges the upper half of one operand with the lower half
// of the other, so with both operands = v the two results hold v[l] and v[l^32].
VIT_DEV float xor32_max(float v) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v), false,
                                                  false);
  return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}

// v[l] + v[l ^ 32] (identical in both lanes), through v_permlane32_swap.
VIT_DEV float xor32_sum(float v) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v), false,
                                                  false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}

// Scheduling fence: the compiler may not move any instruction across it.  Used
// to keep the LDS fragment reads of the next k-step ahead of the MFMAs of the
// current one (otherwise they are sunk below the MFMAs and their latency is
// exposed by an immediate wait).
VIT_DEV void sched_fence() { __builtin_amdgcn_sched_barrier(0); }

// Workgroup barrier that keeps LDS accesses in program order without draining
// the outstanding global->LDS copies (the exact vmcnt waits do that).
VIT_DEV void lds_barrier() {
  asm volatile("" ::: "memory");
  __builtin_amdgcn_s_barrier();
  asm volatile("" ::: "memory");
}

// Per-image descriptors of a packed batch, passed by value as kernel arguments.
struct VarlenDesc {
  int32_t n_images;
  int32_t total;                       // sum of P_i
  int32_t cu_seqlens[VIT_MAX_IMAGES + 1];
  int32_t grid_w[VIT_MAX_IMAGES];
  int32_t cu_tiles[VIT_MAX_IMAGES + 1];  // prefix sum of q-tiles per image (attention)
  int32_t kv_off[VIT_MAX_IMAGES + 1];    // image starts in the transposed-V layout (64-aligned)
  // merged-token starts of the 2x2 merge: ceil(gh/2) * ceil(gw/2) tokens per image
  // (gh*gw/4 on even grids; odd grids only with VIT_ALIGN_PAD)
  int32_t cu_tokens[VIT_MAX_IMAGES + 1];
};

// Keys of one image start at a multiple of this in the transposed-V layout.
constexpr int VT_ALIGN = 64;

// Slot of key j inside its 16-key group of the transposed-V layout: the groups
// of four keys are stored in the order 0-3, 8-11, 4-7, 12-15 (bits 2 and 3 of j
// swapped), so that the 8 keys one MFMA lane needs for P.V are contiguous.  The
// map is its own inverse.
VIT_DEV int vt_key_slot(int j) { return (j & ~12) | ((j & 4) << 1) | ((j & 8) >> 1); }

// The same for the 16x16x32 MFMA layout of the head_dim-72 attention kernel:
// inside each 32-slot group, lane group g (0..3) reads slots 8g .. 8g+7, which
// hold keys 4g .. 4g+3 and 16+4g .. 16+4g+3 (the k-slots of its P^T operand).
// Returns the key (inside the 64-key tile) stored in slot s.
VIT_DEV int vt16_slot_key(int s) { return (s & 35) | ((s >> 1) & 12) | ((s & 4) << 2); }

VIT_DEV int find_image(const VarlenDesc& d, int p) {
  int i = 0;
  while (i + 1 < d.n_images && p >= d.cu_seqlens[i + 1]) ++i;
  return i;
}

// Host-side launch helpers (defined in the .hip files, called by api.cpp).
struct GemmArgs {
  const void* A;
  const void* B;
  const void* B2;
  void* C;
  const int32_t* rowmap;  // optional output row remap (aligner newline layout)
  int64_t lda, ldb, ldc;
  int64_t M, N, K;
  int64_t kb;  // valid K of B (< K when A is zero-padded past B's width)
  const void* rope_table;  // float2 [M, 32] (head_dim 64) for the rotary epilogue
  int64_t rope_cols;       // columns [0, rope_cols) get the rotary (q and k)
  void* vt;                // transposed V [n_heads*64, vt_ld] (VIT_EPI_QKV_VT)
  const int32_t* vpos;     // column of every row m in vt
  int64_t vt_ld;
  // RMSNorm folded into the GEMMs around it.  Producer (fp32 store / add
  // epilogues, N a multiple of 64): besides the fp32 row x_new, write
  // u = bf16(x_new * norm_w) to norm_out [M, N] and the sum of x_new^2 over each
  // 64-column group k to ss_out[m * G4 + k] (G4 = N/64 rounded up to 4).
  // Consumer (bf16 epilogues, ss_groups <= kMaxNormGroups): scale output row m by
  // rstd = (sum over k < ss_groups of ss_in[m * G4 + k] * rms_inv_dim +
  // rms_eps)^-1/2 before anything else, so u . W^T * rstd equals the GEMM of the
  // normalised row.
  const float* norm_w;
  void* norm_out;
  float* ss_out;
  // row strides of norm_out (elements) and ss_out (floats) when they differ from
  // this launch's N and round4(N/64): a launch over a column range of a wider
  // GEMM (norm_w, norm_out and ss_out then point at the range's first column)
  int64_t ld_norm_out, ld_ss_out;
  const float* ss_in;
  int32_t ss_groups;
  float rms_eps;
  float rms_inv_dim;
  // fp32 per-column bias of VIT_EPI_BIAS / VIT_EPI_BIAS_GELU ([N])
  const float* bias;
  // Gathered A rows (VIT_EPI_STORE_GATHER): A is a [a_src_rows, lda] source
  // matrix and logical row m of the GEMM's A operand is the concatenation of
  // source rows a_rows[4m + s], s = 0..3, each a_seg columns wide (K = 4 a_seg).
  const int32_t* a_rows;
  int64_t a_seg;
  int64_t a_src_rows;
};

// Largest number of 64-column groups (vision_dim / 64) the folded RMSNorm takes.
constexpr int kMaxNormGroups = 24;

// Internal epilogue: bf16 store with the half-split 2D rotary applied to the
// q and k columns (head_dim 64 only; each wave owns whole heads).
constexpr int VIT_EPI_STORE_ROPE = 16;
// Internal epilogue: as VIT_EPI_STORE_ROPE for the q, k columns (C holds [M, rope_cols])
// while the v columns are written transposed, one row per (head, dim), into vt.
constexpr int VIT_EPI_QKV_VT = 17;
// Internal epilogue: bf16 store (as VIT_EPI_STORE) of a GEMM whose A operand is
// gathered row by row from four source rows (the aligner's 2x2 merge read
// straight from the normed patch rows; GemmArgs::a_rows).
constexpr int VIT_EPI_STORE_GATHER = 18;

hipError_t launch_gemm_bf16(int epilogue, const GemmArgs& g, hipStream_t s);
// two independent GEMMs with one epilogue, in one launch when both take the MFMA path
hipError_t launch_gemm_bf16_pair(int epilogue, const GemmArgs& g0, const GemmArgs& g1,
                                 hipStream_t s);
hipError_t launch_gemm_f32(int epilogue, const GemmArgs& g, hipStream_t s);
bool gemm_bf16_can_fuse_rope(const GemmArgs& g);
// the MFMA GEMM path (rotary, transposed-V and RMSNorm epilogues) takes these arguments
bool gemm_bf16_mfma_eligible(const GemmArgs& g);
hipError_t launch_rmsnorm(const float* x, const float* w, float eps, int64_t rows, int dim,
                          int out_dtype, void* out, hipStream_t s);
hipError_t launch_rope_table(const VarlenDesc& d, int head_dim, float theta, void* table,
                             hipStream_t s);
hipError_t launch_rope(int dtype, void* qkv, const void* table, int64_t P, int n_heads,
                       int head_dim, hipStream_t s);
// the rotation by the opposite angles on the q and k parts (bf16): gradients with
// respect to the rotated q, k back to gradients with respect to q, k
hipError_t launch_rope_inverse(void* qkv, const void* table, int64_t P, int n_heads, int head_dim,
                               hipStream_t s);
// fp32: vt unused.  bf16: head_dim 72 only, with vt from launch_vt_pack; lse2
// (optional, bf16 only, [n_heads, total] fp32): each query's log2(sum over keys of
// 2^(s c)), s the raw q.k score and c = log2(e)/sqrt(72)
hipError_t launch_attention(int dtype, const void* qkv, const void* vt, int64_t vt_ld,
                            const VarlenDesc& d, int n_heads, int head_dim, void* out,
                            hipStream_t s, float* lse2 = nullptr);
int attention_q_tile(int dtype, int head_dim);
// lse2 (optional, [n_heads, total] fp32): each query's log2(sum over keys of 2^(s c)),
// s the raw q.k score and c = log2(e)/sqrt(64)
hipError_t launch_attention_vt(const void* qk, int64_t ld_qk, const void* vt, int64_t vt_ld,
                               const VarlenDesc& d, int n_heads, void* out, hipStream_t s,
                               float* lse2 = nullptr);
// Per-call preparation of an encode (bf16): zero-padded patches and patch
// weight (K padded to Kp), rotary table, transposed-V positions and padding.
// A null destination skips its part; b[] is filled in by the launcher.
// Rotary frequencies theta^(-k / (head_dim/4)), k < head_dim/4 (computed on the
// host in double, passed by value to the table kernels).
constexpr int kRopeMaxFreqs = 32;
struct RopeFreqs {
  double f[kRopeMaxFreqs];
};
RopeFreqs rope_freqs(int head_dim, double theta);

struct PrepArgs {
  VarlenDesc desc;
  const void* patches;  // [P, patch_dim] -> xpad [P, Kp]; pixel images if pixel_ps > 0
  int32_t pixel_ps;     // patch size of pixel input (0: `patches` holds patches)
  int32_t pix_rows;     // set by the launcher: pixel rows copied as 32-bit words
  void* xpad;
  const void* w_pe;     // [d, patch_dim] -> wpe [d, Kp]
  void* wpe;
  int64_t P, d, patch_dim, Kp;
  void* table;          // float2 [P, head_dim / 2]
  int32_t head_dim;
  RopeFreqs freqs;
  int32_t* vpos;        // [P]
  void* vt;             // [vt_rows, vt_ld]
  int64_t vt_rows, vt_ld;
  // merged-token source rows for the aligner's gathered A operand ([tokens, 4],
  // source row P = the zero row zrow) and that zero row ([d] bf16)
  int32_t* a_rows;
  int64_t tokens;
  void* zrow;
  int64_t b[7];
};
hipError_t launch_encode_prep(PrepArgs a, hipStream_t s);
// pixel images (see VIT_IN_PIXELS) -> patches [P, ld_dst] (zero past 3*ps^2)
hipError_t launch_patchify(int dtype, const void* pix, const VarlenDesc& d, int ps, int64_t ld_dst,
                           void* dst, hipStream_t s);
hipError_t launch_vpos(const VarlenDesc& d, int32_t* vpos, hipStream_t s);
hipError_t launch_vt_zero_pads(const VarlenDesc& d, int64_t rows, void* vt, int64_t vt_ld,
                               hipStream_t s);
// V of a packed qkv buffer transposed into the attention kernels' V^T layout
// (head_dim 64 or 72); for head_dim 72 with rope_table, the same launch also
// applies the rotary to q and k in place.
hipError_t launch_vt_pack(const void* qkv, const VarlenDesc& d, int n_heads, int head_dim,
                          void* vt, int64_t vt_ld, hipStream_t s,
                          const void* rope_table = nullptr);
hipError_t launch_gather(int dtype, const void* x, const VarlenDesc& d, int dim, int merge,
                         void* G, hipStream_t s);
hipError_t launch_pad_rows(int dtype, const void* src, int64_t rows, int64_t cols, int64_t ld_dst,
                           void* dst, hipStream_t s);
hipError_t launch_zero_cols(int dtype, void* buf, int64_t rows, int64_t ld, int64_t c0, int64_t c1,
                            hipStream_t s);
hipError_t launch_layout(int grid_h, int grid_w, int merge, int32_t* perm, int32_t* nl_type,
                         int32_t* nl_src, hipStream_t s);
hipError_t launch_nl_rowmap(const VarlenDesc& d, int merge, int32_t* rowmap, hipStream_t s);
// PatchMerger projector: LayerNorm of every patch row into its 2x2-merged slot
// of G [sum P/4, 4*dim] (projector.hip); dim % 8 == 0, dim <= 4096
hipError_t launch_ln_gather(const void* x, const VarlenDesc& d, int dim, const float* w,
                            const float* b, float eps, void* G, hipStream_t s);
// backward of the MLP half of a block (backward.hip)
hipError_t launch_cast_bf16(const float* src, int64_t n, void* dst, hipStream_t s);
// dst [C, ld_dst] = src [R, C]^T, columns R .. cols_out-1 zero (bf16, ld % 8 == 0)
hipError_t launch_transpose_bf16(const void* src, int64_t R, int64_t C, int64_t ld_src, void* dst,
                                 int64_t cols_out, int64_t ld_dst, hipStream_t s);
// fp32 src [R, C] -> bf16 copy [R, C] and its transpose dst [C, ld_dst] (columns
// R .. cols_out-1 zero) in one pass; C % 8 == 0
hipError_t launch_cast_transpose(const float* src, int64_t R, int64_t C, void* copy, void* dst,
                                 int64_t cols_out, int64_t ld_dst, hipStream_t s);
// measured dense-MFMA peak (microbench.hip)
int64_t mfma_peak_out_floats();
double mfma_peak_flops(int iters);
hipError_t launch_mfma_peak(int iters, float* out, hipStream_t s);
// gu [rows, 2 hp] (g, u at columns 0 and hp), dgdu [rows, 2 hp] likewise, its
// columns h .. hp-1 of each half zero
hipError_t launch_swiglu_bwd(const float* gu, const float* da, int64_t rows, int h, int hp,
                             void* a, void* dgdu, hipStream_t s);
int rmsnorm_bwd_blocks(int64_t rows);
hipError_t launch_rmsnorm_bwd(const float* x, const float* w, const float* dn, const float* dy,
                              int64_t rows, int d, float eps, float* dx, float* partial,
                              float* dw, hipStream_t s);
// backward of the attention (attention_bwd.hip), bf16, head_dim D = 64 or 72
int attention_bwd_tile();  // queries / keys per workgroup: the q-tile of its descriptor
// dst [H*D, ld] = columns col0 .. col0+H*D of src, transposed into the V^T layout
// of the 32x32x16 MFMAs (64-aligned image spans, keys permuted by vt_key_slot,
// zero padding)
hipError_t launch_tpack(const void* src, int64_t ld_src, int64_t col0, const VarlenDesc& d,
                        int n_heads, int head_dim, void* dst, int64_t ld, hipStream_t s);
hipError_t launch_rowdot(const void* dO, const void* O, int64_t P, int n_heads, int head_dim,
                         float* Dq, hipStream_t s);
// dq -> columns [0, H*D) of dqkv, dk, dv -> [H*D, 3*H*D); q, k, v read from qkv
// ([P, ldq], rotated q, k); qt, kt, dot in the tpack layout.  D = 64: dq and dk
// rotated back with the rotary table in the kernels (the gradients before the
// rotary); D = 72: dq and dk left in the rotated space (table unused), for
// launch_rope_inverse.
hipError_t launch_attention_bwd(const void* qkv, int64_t ldq, const void* dO, const void* qt,
                                const void* kt, const void* dot, int64_t t_ld, const float* lse2,
                                const float* Dq, const void* table, const VarlenDesc& d,
                                int n_heads, int head_dim, void* dqkv, int64_t ld_out,
                                hipStream_t s);
// image tokens and sentinel rows into a text embedding stream (merge.hip)
size_t merge_workspace_bytes(int64_t positions);
// group counts of IMAGE positions, scanned in place in ws; total to n_image (optional)
hipError_t launch_merge_rank(const int32_t* types, int64_t positions, int32_t* n_image, void* ws,
                             hipStream_t s);
// the row copies, using the scanned counts left in ws by launch_merge_rank
hipError_t launch_merge_copy(void* embeds, int64_t positions, int64_t row_bytes,
                             const int32_t* types, const void* tokens, int64_t n_tokens,
                             const void* sentinels, const void* ws, hipStream_t s);
