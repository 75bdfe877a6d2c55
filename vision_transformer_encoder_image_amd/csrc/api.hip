// C ABI of the encoder library: argument validation, workspace plan, launch
// sequence of the vision tower + aligner, per-step entry points, event timing.
#include <hip/hip_runtime.h>

#include <cstdarg>
#include <cstdio>
#include <cstring>
#include <mutex>
#include <string>
#include <utility>
#include <vector>

#include "common.h"

namespace {

thread_local std::string g_last_error;

vit_status fail(vit_status st, const char* fmt, ...) __attribute__((format(printf, 2, 3)));
vit_status fail(vit_status st, const char* fmt, ...) {
  char buf[512];
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(buf, sizeof(buf), fmt, ap);
  va_end(ap);
  g_last_error = buf;
  return st;
}

vit_status hip_check(hipError_t e, const char* what) {
  if (e == hipSuccess) return VIT_OK;
  return fail(VIT_E_HIP, "%s: %s", what, hipGetErrorString(e));
}

#define VIT_TRY(expr)                    \
  do {                                   \
    vit_status _st = (expr);             \
    if (_st != VIT_OK) return _st;       \
  } while (0)
#define VIT_HIP(expr, what) VIT_TRY(hip_check((expr), (what)))

// ---------------------------------------------------------------- event timing
struct Prof {
  std::mutex mu;
  bool on[VIT_K_COUNT] = {};
  std::vector<std::pair<hipEvent_t, hipEvent_t>> ev[VIT_K_COUNT];
  size_t used[VIT_K_COUNT] = {};
};
Prof& prof() {
  static Prof p;
  return p;
}

struct ProfScope {
  int cls;
  hipStream_t s;
  hipEvent_t end = nullptr;
  ProfScope(int c, hipStream_t st) : cls(c), s(st) {
    Prof& p = prof();
    std::lock_guard<std::mutex> lk(p.mu);
    if (cls < 0 || cls >= VIT_K_COUNT || !p.on[cls]) return;  // -1: not timed
    if (p.used[cls] == p.ev[cls].size()) {
      // timing events without the system-scope release/acquire fence an
      // ordinary event adds around its timestamp (which writes back the caches
      // at every record and would slow the timed work down)
      hipEvent_t a, b;
      if (hipEventCreateWithFlags(&a, hipEventDisableSystemFence) != hipSuccess) return;
      if (hipEventCreateWithFlags(&b, hipEventDisableSystemFence) != hipSuccess) {
        (void)hipEventDestroy(a);
        return;
      }
      p.ev[cls].emplace_back(a, b);
    }
    auto& pr = p.ev[cls][p.used[cls]++];
    (void)hipEventRecord(pr.first, s);
    end = pr.second;
  }
  ~ProfScope() {
    if (end) (void)hipEventRecord(end, s);
  }
};

// ---------------------------------------------------------------- shapes
size_t align_up(size_t v, size_t a = 256) { return (v + a - 1) / a * a; }
int64_t round_up(int64_t v, int64_t a) { return (v + a - 1) / a * a; }

size_t esize(int dtype) { return dtype == VIT_BF16 ? 2 : 4; }

vit_status check_config(const vit_config* c) {
  if (!c) return fail(VIT_E_ARG, "config is NULL");
  if (c->dtype != VIT_BF16 && c->dtype != VIT_F32) return fail(VIT_E_ARG, "bad dtype %d", c->dtype);
  if (c->vision_dim <= 0 || c->n_heads <= 0 || c->head_dim <= 0 || c->mlp_hidden <= 0 ||
      c->n_blocks < 0 || c->patch_dim <= 0 || c->merge <= 0)
    return fail(VIT_E_SHAPE, "non-positive dimension in config");
  if (c->vision_dim != c->n_heads * c->head_dim)
    return fail(VIT_E_SHAPE, "vision_dim %d != n_heads %d * head_dim %d", c->vision_dim,
                c->n_heads, c->head_dim);
  if (c->head_dim % 4) return fail(VIT_E_SHAPE, "head_dim %d not a multiple of 4", c->head_dim);
  if (c->head_dim != 64 && c->head_dim != 72)
    return fail(VIT_E_SHAPE, "head_dim %d unsupported (64 or 72)", c->head_dim);
  if (c->vision_dim % 8 || c->mlp_hidden % 8 || c->patch_dim % 4)
    return fail(VIT_E_SHAPE, "vision_dim and mlp_hidden must be multiples of 8, patch_dim of 4");
  if (c->merge != 2) return fail(VIT_E_SHAPE, "merge %d unsupported (2)", c->merge);
  if (!(c->rms_eps >= 0.f) || !(c->rope_theta > 0.f)) return fail(VIT_E_SHAPE, "bad eps/theta");
  return VIT_OK;
}

// Patch size ps with patch_dim = 3 * ps^2, or 0 if there is none.
int patch_size_of(const vit_config& c) {
  for (int ps = 1; 3 * ps * ps <= c.patch_dim; ++ps)
    if (3 * ps * ps == c.patch_dim) return ps;
  return 0;
}

vit_status build_desc(const int32_t* grid_hw, int32_t n_images, int q_tile, bool need_even,
                      int merge, VarlenDesc* d, bool pad_odd = false) {
  if (!grid_hw) return fail(VIT_E_ARG, "grid_hw is NULL");
  if (n_images < 1 || n_images > VIT_MAX_IMAGES)
    return fail(VIT_E_SHAPE, "n_images %d outside [1, %d]", n_images, VIT_MAX_IMAGES);
  std::memset(d, 0, sizeof(*d));
  d->n_images = n_images;
  int64_t total = 0, tiles = 0, kv = 0, toks = 0;
  for (int i = 0; i < n_images; ++i) {
    const int gh = grid_hw[2 * i], gw = grid_hw[2 * i + 1];
    if (gh <= 0 || gw <= 0) return fail(VIT_E_SHAPE, "image %d has grid %dx%d", i, gh, gw);
    if (need_even && !pad_odd && (gh % merge || gw % merge))
      return fail(VIT_E_ODD_GRID, "image %d grid %dx%d not divisible by merge %d", i, gh, gw,
                  merge);
    d->cu_seqlens[i] = (int32_t)total;
    d->cu_tokens[i] = (int32_t)toks;
    toks += (int64_t)((gh + merge - 1) / merge) * ((gw + merge - 1) / merge);
    d->cu_tiles[i] = (int32_t)tiles;
    d->kv_off[i] = (int32_t)kv;
    d->grid_w[i] = gw;
    total += (int64_t)gh * gw;
    kv += ((int64_t)gh * gw + VT_ALIGN - 1) / VT_ALIGN * VT_ALIGN;
    tiles += ((int64_t)gh * gw + q_tile - 1) / q_tile;
    if (total > (1 << 24)) return fail(VIT_E_SHAPE, "more than 2^24 patches in one call");
  }
  d->cu_seqlens[n_images] = (int32_t)total;
  d->cu_tiles[n_images] = (int32_t)tiles;
  d->kv_off[n_images] = (int32_t)kv;
  d->cu_tokens[n_images] = (int32_t)toks;
  d->total = (int32_t)total;
  return VIT_OK;
}

struct Plan {
  int64_t P = 0, tokens = 0, Kp = 0, hp = 0;
  size_t table = 0, xpad = 0, wpe = 0, x = 0, n = 0, qkv = 0, act = 0, G = 0, rowmap = 0;
  size_t vt = 0, vpos = 0, u = 0, ss = 0, arows = 0;
  int64_t kv_total = 0;
  bool fuse_gather = false;  // bf16 aligner reads its 2x2 groups straight from n
  bool use_vt = false;  // bf16, head_dim 64: V written transposed by the wqkv GEMM
  bool pack_vt = false;  // bf16, head_dim 72: V transposed by a pack pass after the rotary
  bool fuse_norm = false;  // bf16, vision_dim % 64 == 0: RMSNorm folded into the GEMMs
  size_t total = 0;
};

Plan make_plan(const vit_config& c, const VarlenDesc& desc, int flags) {
  const int64_t P = desc.total;
  Plan p;
  const size_t es = esize(c.dtype);
  const bool aligner = !(flags & VIT_NO_ALIGNER);
  const int64_t d = c.vision_dim, h = c.mlp_hidden, m2 = (int64_t)c.merge * c.merge;
  p.P = P;
  p.tokens = aligner ? desc.cu_tokens[desc.n_images] : 0;
  (void)m2;
  p.Kp = c.dtype == VIT_BF16 ? round_up(c.patch_dim, 64) : c.patch_dim;
  const bool pixels = (flags & VIT_IN_PIXELS) != 0;
  // MLP activations keep a 64-multiple row stride in bf16 so the down GEMM runs
  // whole 64-wide K tiles (the pad columns are zero)
  p.hp = c.dtype == VIT_BF16 ? round_up(h, 64) : h;
  size_t off = 0;
  auto take = [&](size_t bytes) {
    const size_t o = off;
    off += align_up(bytes);
    return o;
  };
  p.table = take((size_t)P * (c.head_dim / 2) * sizeof(float2));
  if (c.dtype == VIT_BF16) {
    p.xpad = take((size_t)P * p.Kp * es);
    p.wpe = take((size_t)d * p.Kp * es);
  } else if (pixels) {
    p.xpad = take((size_t)P * p.Kp * es);  // fp32 patches cut from the pixels
  }
  p.x = take((size_t)P * d * sizeof(float));
  // also holds the attention output; one more row stays zero for the padded
  // 2x2 groups of the aligner's gathered operand
  p.n = take((size_t)(P + 1) * d * es);
  p.qkv = take((size_t)P * 3 * d * es);
  p.act = take((size_t)P * p.hp * es);
  p.use_vt = c.dtype == VIT_BF16 && c.head_dim == 64;
  p.pack_vt = c.dtype == VIT_BF16 && c.head_dim == 72;
  if (p.use_vt || p.pack_vt) {
    p.kv_total = desc.kv_off[desc.n_images];
    p.vt = take((size_t)d * p.kv_total * es);
  }
  if (p.use_vt) p.vpos = take((size_t)P * sizeof(int32_t));
  p.fuse_norm = c.dtype == VIT_BF16 && d % 64 == 0 && d / 64 <= kMaxNormGroups && c.n_blocks > 0;
  if (p.fuse_norm) {
    p.u = take((size_t)P * d * es);                     // bf16(x * norm weight)
    p.ss = take((size_t)P * round_up(d / 64, 4) * sizeof(float));  // partial sums of x^2
  }
  // bf16 with 64-multiple widths: the aligner GEMM gathers each merged token's
  // four patch rows itself (source rows per token); otherwise a gather pass
  // writes G [tokens, 4d] first
  // (G stays reserved for operands the GEMM's loader cannot take: unaligned
  // aligner weight or output)
  p.fuse_gather = aligner && c.dtype == VIT_BF16 && c.merge == 2 && d % 64 == 0;
  if (p.fuse_gather) p.arows = take((size_t)p.tokens * 4 * sizeof(int32_t));
  if (aligner) p.G = take((size_t)p.tokens * m2 * d * es);
  if (aligner && (flags & VIT_OUT_NLAYOUT)) p.rowmap = take((size_t)p.tokens * sizeof(int32_t));
  p.total = off;
  return p;
}

GemmArgs gemm_args(const void* A, int64_t lda, const void* B, const void* B2, int64_t ldb, void* C,
                   int64_t ldc, int64_t M, int64_t N, int64_t K, const int32_t* rowmap) {
  GemmArgs g{};
  g.A = A;
  g.B = B;
  g.B2 = B2;
  g.C = C;
  g.rowmap = rowmap;
  g.lda = lda;
  g.ldb = ldb;
  g.ldc = ldc;
  g.M = M;
  g.N = N;
  g.K = K;
  g.kb = K;
  g.rope_table = nullptr;
  g.rope_cols = 0;
  return g;
}

vit_status gemm(int dtype, int epi, const void* A, int64_t lda, const void* B, const void* B2,
                int64_t ldb, void* C, int64_t ldc, int64_t M, int64_t N, int64_t K,
                const int32_t* rowmap, hipStream_t s) {
  GemmArgs g{};
  g.A = A;
  g.B = B;
  g.B2 = B2;
  g.C = C;
  g.rowmap = rowmap;
  g.lda = lda;
  g.ldb = ldb;
  g.ldc = ldc;
  g.M = M;
  g.N = N;
  g.K = K;
  g.kb = K;
  g.rope_table = nullptr;
  g.rope_cols = 0;
  const hipError_t e = dtype == VIT_BF16 ? launch_gemm_bf16(epi, g, s) : launch_gemm_f32(epi, g, s);
  return hip_check(e, "gemm launch");
}

vit_status check_weights(const vit_config& c, const vit_weights* w, bool aligner) {
  if (!w) return fail(VIT_E_ARG, "weights is NULL");
  if (!w->patch_embed || !w->final_norm) return fail(VIT_E_ARG, "patch_embed/final_norm NULL");
  if (c.n_blocks > 0 &&
      (!w->wqkv || !w->wo || !w->w_gate || !w->w_up || !w->w_down || !w->norm1 || !w->norm2))
    return fail(VIT_E_ARG, "per-block weight array NULL");
  for (int b = 0; b < c.n_blocks; ++b)
    if (!w->wqkv[b] || !w->wo[b] || !w->w_gate[b] || !w->w_up[b] || !w->w_down[b] ||
        !w->norm1[b] || !w->norm2[b])
      return fail(VIT_E_ARG, "block %d has a NULL weight", b);
  if (aligner && !w->aligner) return fail(VIT_E_ARG, "aligner weight NULL");
  return VIT_OK;
}

// ckpt (optional, fp32 [2 n_blocks + 1][P][d]): the residual stream at the input
// of every residual branch and after the last block, copied out as it is formed
// (used by the backward of the tower)
vit_status encode_impl(const vit_config* cfg, const vit_weights* w, const void* in,
                       const int32_t* grid_hw, int32_t n_images, int32_t flags, void* out,
                       void* ws, size_t ws_bytes, hipStream_t s, float* ckpt = nullptr) {
  VIT_TRY(check_config(cfg));
  const vit_config& c = *cfg;
  if (flags & ~(VIT_NO_ALIGNER | VIT_OUT_NLAYOUT | VIT_IN_PIXELS | VIT_ALIGN_PAD))
    return fail(VIT_E_ARG, "unknown flags %d", flags);
  const int pixel_ps = (flags & VIT_IN_PIXELS) ? patch_size_of(*cfg) : 0;
  if ((flags & VIT_IN_PIXELS) && pixel_ps == 0)
    return fail(VIT_E_SHAPE, "pixel input needs patch_dim = 3*ps^2 (got %d)", cfg->patch_dim);
  const bool aligner = !(flags & VIT_NO_ALIGNER);
  if (aligner && c.llm_dim <= 0) return fail(VIT_E_SHAPE, "llm_dim must be positive with aligner");
  if (aligner && c.llm_dim % 8 && c.dtype == VIT_BF16)
    return fail(VIT_E_SHAPE, "llm_dim must be a multiple of 8");
  if (!in || !out) return fail(VIT_E_ARG, "in/out is NULL");
  VIT_TRY(check_weights(c, w, aligner));
  VarlenDesc desc;
  VIT_TRY(build_desc(grid_hw, n_images, attention_q_tile(c.dtype, c.head_dim), aligner, c.merge,
                     &desc, (flags & VIT_ALIGN_PAD) != 0));
  const Plan p = make_plan(c, desc, flags);
  if (!ws || ws_bytes < p.total)
    return fail(VIT_E_WORKSPACE, "workspace %zu bytes < %zu needed", ws ? ws_bytes : (size_t)0,
                p.total);
  char* base = (char*)ws;
  void* table = base + p.table;
  float* x = (float*)(base + p.x);
  void* n = base + p.n;
  void* qkv = base + p.qkv;
  void* act = base + p.act;
  const int dt = c.dtype;
  const int64_t P = p.P, d = c.vision_dim, h = c.mlp_hidden;
  const bool final_to_out = !aligner;

  // RMSNorm folded into the GEMMs: the GEMM that writes the residual stream x
  // (patch embedding, out-projection, down-projection) also writes
  // u = bf16(x * w_norm) and per-row partial sums of x^2; the GEMM that reads
  // the normalised row (wqkv, gate/up) takes u and scales its output rows by
  // 1/rms.  Only the final norm remains a pass of its own.
  void* u = p.fuse_norm ? base + p.u : nullptr;
  float* ss = p.fuse_norm ? (float*)(base + p.ss) : nullptr;
  auto producer = [&](GemmArgs& g, const float* wn) {
    g.norm_w = wn;
    g.norm_out = u;
    g.ss_out = ss;
  };
  auto consumer = [&](GemmArgs& g) {
    g.ss_in = ss;
    g.ss_groups = (int32_t)(d / 64);
    g.rms_eps = c.rms_eps;
    g.rms_inv_dim = 1.0f / (float)d;
  };
  bool fuse = p.fuse_norm;
  if (fuse) {  // every GEMM of the stack must take the MFMA path
    const GemmArgs chk[] = {
        gemm_args(base + p.xpad, p.Kp, base + p.wpe, nullptr, p.Kp, x, d, P, d, p.Kp, nullptr),
        gemm_args(u, d, w->wqkv[0], nullptr, d, qkv, 3 * d, P, 3 * d, d, nullptr),
        gemm_args(n, d, w->wo[0], nullptr, d, x, d, P, d, d, nullptr),
        gemm_args(u, d, w->w_gate[0], w->w_up[0], d, act, p.hp, P, h, d, nullptr),
        gemm_args(act, p.hp, w->w_down[0], nullptr, h, x, d, P, d, p.hp, nullptr)};
    for (const GemmArgs& g : chk) fuse = fuse && gemm_bf16_mfma_eligible(g);
  }

  void* vt = (p.use_vt || p.pack_vt) ? base + p.vt : nullptr;
  int32_t* vpos = p.use_vt ? (int32_t*)(base + p.vpos) : nullptr;
  // patch embedding: x (fp32 residual stream) = patches . Wpe^T
  {
    ProfScope ps(VIT_K_EMBED, s);
    if (dt == VIT_BF16) {
      // one launch prepares everything the call needs before the first GEMM:
      // patches and weight zero-padded to Kp, rotary table, transposed-V
      // positions and padding
      void* xpad = base + p.xpad;
      void* wpe = base + p.wpe;
      PrepArgs pa{};
      pa.desc = desc;
      pa.patches = in;
      pa.pixel_ps = pixel_ps;
      pa.xpad = xpad;
      pa.w_pe = w->patch_embed;
      pa.wpe = wpe;
      pa.P = P;
      pa.d = d;
      pa.patch_dim = c.patch_dim;
      pa.Kp = p.Kp;
      pa.table = table;
      pa.head_dim = c.head_dim;
      pa.freqs = rope_freqs(c.head_dim, (double)c.rope_theta);
      pa.vpos = vpos;
      pa.vt = vt;
      pa.vt_rows = p.use_vt ? d : 0;
      pa.vt_ld = p.kv_total;
      pa.a_rows = p.fuse_gather ? (int32_t*)(base + p.arows) : nullptr;
      pa.tokens = p.tokens;
      pa.zrow = p.fuse_gather ? (char*)n + (size_t)P * d * 2 : nullptr;
      VIT_HIP(launch_encode_prep(pa, s), "encode preparation");
      GemmArgs g = gemm_args(xpad, p.Kp, wpe, nullptr, p.Kp, x, d, P, d, p.Kp, nullptr);
      if (fuse) producer(g, w->norm1[0]);
      VIT_HIP(launch_gemm_bf16(VIT_EPI_STORE_F32, g, s), "patch embedding gemm");
    } else {
      const void* patches = in;
      if (pixel_ps > 0) {
        VIT_HIP(launch_patchify(dt, in, desc, pixel_ps, c.patch_dim, base + p.xpad, s), "patchify");
        patches = base + p.xpad;
      }
      VIT_TRY(gemm(dt, VIT_EPI_STORE_F32, patches, c.patch_dim, w->patch_embed, nullptr,
                   c.patch_dim, x, d, P, d, c.patch_dim, nullptr, s));
      VIT_HIP(launch_rope_table(desc, c.head_dim, c.rope_theta, table, s), "rope table");
    }
  }
  auto save = [&](int k) -> vit_status {
    if (!ckpt) return VIT_OK;
    return hip_check(hipMemcpyAsync(ckpt + (int64_t)k * P * d, x, (size_t)P * d * sizeof(float),
                                    hipMemcpyDeviceToDevice, s),
                     "residual checkpoint");
  };
  VIT_TRY(save(0));
  if (p.hp > h)
    VIT_HIP(launch_zero_cols(dt, act, P, p.hp, h, p.hp, s), "zero MLP pad columns");
  void* a_in = fuse ? u : n;  // A operand of the GEMMs after a norm

  for (int b = 0; b < c.n_blocks; ++b) {
    if (!fuse) {
      ProfScope ps(VIT_K_RMSNORM, s);
      VIT_HIP(launch_rmsnorm(x, w->norm1[b], c.rms_eps, P, (int)d, dt, n, s), "norm1");
    }
    // wqkv: with head_dim 64 in bf16 the epilogue applies the rotary to q, k
    // (stored [P, 2d]) and writes v transposed per head for the attention
    // kernel; otherwise plain [P, 3d] output and a separate rotary pass
    GemmArgs g = gemm_args(a_in, d, w->wqkv[b], nullptr, d, qkv, 2 * d, P, 3 * d, d, nullptr);
    g.rope_table = table;
    g.rope_cols = 2 * d;
    g.vt = vt;
    g.vpos = vpos;
    g.vt_ld = p.kv_total;
    if (fuse) consumer(g);
    const bool fuse_rope = p.use_vt && gemm_bf16_can_fuse_rope(g);
    {
      ProfScope ps(VIT_K_QKV, s);
      if (fuse_rope) {
        VIT_HIP(launch_gemm_bf16(VIT_EPI_QKV_VT, g, s), "qkv+rope gemm");
      } else if (dt == VIT_BF16) {
        GemmArgs gp = gemm_args(a_in, d, w->wqkv[b], nullptr, d, qkv, 3 * d, P, 3 * d, d, nullptr);
        if (fuse) consumer(gp);
        VIT_HIP(launch_gemm_bf16(VIT_EPI_STORE, gp, s), "qkv gemm");
      } else {
        VIT_TRY(gemm(dt, VIT_EPI_STORE, n, d, w->wqkv[b], nullptr, d, qkv, 3 * d, P, 3 * d, d,
                     nullptr, s));
      }
    }
    if (!fuse_rope) {
      ProfScope ps(VIT_K_ROPE, s);
      if (p.pack_vt) {  // one launch: rotary of q, k and the V^T pack
        VIT_HIP(launch_vt_pack(qkv, desc, c.n_heads, c.head_dim, vt, p.kv_total, s, table),
                "rope + pack V");
      } else {
        VIT_HIP(launch_rope(dt, qkv, table, P, c.n_heads, c.head_dim, s), "rope");
        if (vt)
          VIT_HIP(launch_vt_pack(qkv, desc, c.n_heads, c.head_dim, vt, p.kv_total, s), "pack V");
      }
    }
    {
      ProfScope ps(VIT_K_ATTN, s);
      if (p.use_vt)  // q, k rows of stride 2d after the fused epilogue, else 3d
        VIT_HIP(launch_attention_vt(qkv, fuse_rope ? 2 * d : 3 * d, vt, p.kv_total, desc,
                                    c.n_heads, n, s),
                "attention");
      else
        VIT_HIP(launch_attention(dt, qkv, vt, p.kv_total, desc, c.n_heads, c.head_dim, n, s),
                "attention");
    }
    {
      ProfScope ps(VIT_K_OUTPROJ, s);
      if (dt == VIT_BF16) {
        GemmArgs go = gemm_args(n, d, w->wo[b], nullptr, d, x, d, P, d, d, nullptr);
        if (fuse) producer(go, w->norm2[b]);
        VIT_HIP(launch_gemm_bf16(VIT_EPI_ADD_F32, go, s), "out-projection gemm");
      } else {
        VIT_TRY(gemm(dt, VIT_EPI_ADD_F32, n, d, w->wo[b], nullptr, d, x, d, P, d, d, nullptr, s));
      }
    }
    VIT_TRY(save(2 * b + 1));
    if (!fuse) {
      ProfScope ps(VIT_K_RMSNORM, s);
      VIT_HIP(launch_rmsnorm(x, w->norm2[b], c.rms_eps, P, (int)d, dt, n, s), "norm2");
    }
    {
      ProfScope ps(VIT_K_GATEUP, s);
      if (dt == VIT_BF16) {
        GemmArgs gg = gemm_args(a_in, d, w->w_gate[b], w->w_up[b], d, act, p.hp, P, h, d, nullptr);
        if (fuse) consumer(gg);
        VIT_HIP(launch_gemm_bf16(VIT_EPI_SWIGLU, gg, s), "gate/up gemm");
      } else {
        VIT_TRY(gemm(dt, VIT_EPI_SWIGLU, n, d, w->w_gate[b], w->w_up[b], d, act, p.hp, P, h, d,
                     nullptr, s));
      }
    }
    {
      ProfScope ps(VIT_K_DOWN, s);
      GemmArgs gd = gemm_args(act, p.hp, w->w_down[b], nullptr, h, x, d, P, d, p.hp, nullptr);
      gd.kb = h;  // act is zero past column h; W_down rows are h wide
      if (fuse && b + 1 < c.n_blocks) producer(gd, w->norm1[b + 1]);
      VIT_HIP(dt == VIT_BF16 ? launch_gemm_bf16(VIT_EPI_ADD_F32, gd, s)
                             : launch_gemm_f32(VIT_EPI_ADD_F32, gd, s),
              "down gemm");
    }
    VIT_TRY(save(2 * b + 2));
  }
  {
    ProfScope ps(VIT_K_RMSNORM, s);
    VIT_HIP(launch_rmsnorm(x, w->final_norm, c.rms_eps, P, (int)d, dt, final_to_out ? out : n, s),
            "final norm");
  }
  if (!aligner) return VIT_OK;

  const int64_t m2 = (int64_t)c.merge * c.merge;
  int32_t* rowmap = nullptr;
  if (flags & VIT_OUT_NLAYOUT) {
    rowmap = (int32_t*)(base + p.rowmap);
    VIT_HIP(launch_nl_rowmap(desc, c.merge, rowmap, s), "newline row map");
  }
  if (p.fuse_gather) {
    // the A operand's row t is the final-normed patch rows a_rows[4t .. 4t+3]
    // (TL, TR, BL, BR; row P of n is zero for padded groups), read by the GEMM's
    // own loader: no G buffer and no gather pass
    GemmArgs g = gemm_args(n, d, w->aligner, nullptr, m2 * d, out, c.llm_dim, p.tokens,
                           c.llm_dim, m2 * d, rowmap);
    g.a_rows = (const int32_t*)(base + p.arows);
    g.a_seg = d;
    g.a_src_rows = P + 1;
    if (gemm_bf16_mfma_eligible(g)) {
      ProfScope ps(VIT_K_ALIGNER, s);
      VIT_HIP(launch_gemm_bf16(VIT_EPI_STORE_GATHER, g, s), "aligner gemm");
      return VIT_OK;
    }
  }
  void* G = base + p.G;
  {
    ProfScope ps(VIT_K_GATHER, s);
    VIT_HIP(launch_gather(dt, n, desc, (int)d, c.merge, G, s), "aligner gather");
  }
  {
    ProfScope ps(VIT_K_ALIGNER, s);
    VIT_TRY(gemm(dt, VIT_EPI_STORE, G, m2 * d, w->aligner, nullptr, m2 * d, out, c.llm_dim,
                 p.tokens, c.llm_dim, m2 * d, rowmap, s));
  }
  return VIT_OK;
}

// Backward of the MLP half: workspace layout.  The gate and up halves of g|u,
// dg|du and the transposed weights sit hp = round64(h) columns apart, the
// columns between zero, so the dn GEMM's K (2 hp) is whole K-tiles.
struct MlpGradPlan {
  int64_t Pp = 0;  // rows rounded up to 64 (K of the weight-gradient GEMMs)
  int64_t hp = 0;  // hidden width rounded up to 64
  size_t n = 0, dy16 = 0, gu = 0, da = 0, a = 0, dgdu = 0, dn = 0, wdT = 0, wguT = 0;
  size_t dyT = 0, aT = 0, dgduT = 0, nT = 0, partial = 0, total = 0;
};

MlpGradPlan mlp_grad_plan(int64_t P, int64_t d, int64_t h) {
  MlpGradPlan p;
  p.Pp = round_up(P, 64);
  p.hp = round_up(h, 64);
  const int64_t hp = p.hp;
  size_t off = 0;
  auto take = [&](size_t bytes) {
    const size_t o = off;
    off += (size_t)round_up((int64_t)bytes, 256);
    return o;
  };
  p.n = take(P * d * 2);
  p.dy16 = take(P * d * 2);
  p.gu = take(P * 2 * hp * 4);
  p.da = take(P * h * 4);
  p.a = take(P * h * 2);
  p.dgdu = take(P * 2 * hp * 2);
  p.dn = take(P * d * 4);
  p.wdT = take(h * d * 2);
  p.wguT = take(d * 2 * hp * 2);
  p.dyT = take(d * p.Pp * 2);
  p.aT = take(h * p.Pp * 2);
  p.dgduT = take(2 * hp * p.Pp * 2);
  p.nT = take(d * p.Pp * 2);
  p.partial = take((size_t)rmsnorm_bwd_blocks(P) * d * 4);
  p.total = off;
  return p;
}

vit_status check_mlp_grad_sizes(int64_t rows, int32_t dim, int32_t hidden) {
  if (rows < 1 || rows > (1 << 24)) return fail(VIT_E_SHAPE, "rows %lld out of range", (long long)rows);
  if (dim <= 0 || dim % 64 || dim > 2048)
    return fail(VIT_E_SHAPE, "dim %d: need a multiple of 64, at most 2048", dim);
  if (hidden <= 0 || hidden % 16) return fail(VIT_E_SHAPE, "hidden %d: need a multiple of 16", hidden);
  return VIT_OK;
}

// Backward of the attention half: workspace layout
struct AttnGradPlan {
  int64_t P = 0, Pp = 0, kv = 0;
  size_t n = 0, qkv = 0, table = 0, vt = 0, o = 0, lse = 0, dy16 = 0, dO = 0, Dq = 0, qt = 0,
         kt = 0, dot = 0, dqkv = 0, woT = 0, wqkvT = 0, dn = 0, dyT = 0, oT = 0, dqkvT = 0,
         nT = 0, partial = 0, total = 0;
};

AttnGradPlan attn_grad_plan(const VarlenDesc& desc, int64_t d, int64_t H) {
  const int64_t D = d / H;
  AttnGradPlan p;
  p.P = desc.total;
  p.Pp = round_up(p.P, 64);
  p.kv = desc.kv_off[desc.n_images];
  const int64_t P = p.P;
  size_t off = 0;
  auto take = [&](size_t bytes) {
    const size_t o = off;
    off += (size_t)round_up((int64_t)bytes, 256);
    return o;
  };
  p.n = take(P * d * 2);
  p.qkv = take(P * 3 * d * 2);
  p.table = take(P * (D / 2) * 8);
  p.vt = take(d * p.kv * 2);
  p.o = take(P * d * 2);
  p.lse = take(H * P * 4);
  p.dy16 = take(P * d * 2);
  p.dO = take(P * d * 2);
  p.Dq = take(H * P * 4);
  p.qt = take(d * p.kv * 2);
  p.kt = take(d * p.kv * 2);
  p.dot = take(d * p.kv * 2);
  p.dqkv = take(P * 3 * d * 2);
  p.woT = take(d * d * 2);
  p.wqkvT = take(d * 3 * d * 2);
  p.dn = take(P * d * 4);
  p.dyT = take(d * p.Pp * 2);
  p.oT = take(d * p.Pp * 2);
  p.dqkvT = take(3 * d * p.Pp * 2);
  p.nT = take(d * p.Pp * 2);
  p.partial = take((size_t)rmsnorm_bwd_blocks(P) * d * 4);
  p.total = off;
  return p;
}

vit_status check_attn_grad(const vit_attn_grad* a) {
  if (!a) return fail(VIT_E_ARG, "arguments are NULL");
  if (a->n_heads <= 0 || (a->dim != 64 * a->n_heads && a->dim != 72 * a->n_heads) ||
      a->dim > 2048 || a->dim % 64)
    return fail(VIT_E_SHAPE,
                "dim %d, n_heads %d: need head_dim 64 or 72, dim a multiple of 64, dim <= 2048",
                a->dim, a->n_heads);
  if (!(a->eps >= 0.f) || !(a->rope_theta > 0.f)) return fail(VIT_E_ARG, "bad eps / theta");
  return VIT_OK;
}

// Backward of the whole tower: workspace layout.  The forward's own workspace
// comes first (its zero-padded patches are the B operand of the patch
// embedding's gradient), then the residual checkpoints, two gradient buffers,
// and one region that each half's backward reuses in turn (afterwards the
// operands of the patch embedding's gradient).
struct TowerGradPlan {
  Plan fwd;
  int64_t P = 0, Pp = 0;
  size_t out = 0, ckpt = 0, dxa = 0, dxb = 0, partial = 0, half = 0, half_bytes = 0, total = 0;
  size_t dx16 = 0, dxT = 0, xT = 0;  // offsets inside the half region
};

vit_status tower_setup(const vit_config* cfg, const int32_t* grid_hw, int32_t n_images,
                       TowerGradPlan* t) {
  VIT_TRY(check_config(cfg));
  const vit_config& c = *cfg;
  if (c.dtype != VIT_BF16) return fail(VIT_E_ARG, "tower backward: bf16 only");
  if ((c.head_dim != 64 && c.head_dim != 72) || c.vision_dim % 64 || c.vision_dim > 2048)
    return fail(VIT_E_SHAPE,
                "tower backward: head_dim 64 or 72, vision_dim a multiple of 64 and <= 2048 "
                "(got %d, %d)",
                c.head_dim, c.vision_dim);
  if (c.mlp_hidden % 16)
    return fail(VIT_E_SHAPE, "tower backward: mlp_hidden %d not a multiple of 16", c.mlp_hidden);
  if (c.patch_dim % 4)
    return fail(VIT_E_SHAPE, "tower backward: patch_dim %d not a multiple of 4", c.patch_dim);
  VarlenDesc fdesc, bdesc;
  VIT_TRY(build_desc(grid_hw, n_images, attention_q_tile(c.dtype, c.head_dim), false, c.merge,
                     &fdesc));
  VIT_TRY(build_desc(grid_hw, n_images, attention_bwd_tile(), false, 2, &bdesc));
  const int64_t P = fdesc.total, d = c.vision_dim;
  t->fwd = make_plan(c, fdesc, VIT_NO_ALIGNER);
  t->P = P;
  t->Pp = round_up(P, 64);
  size_t off = t->fwd.total;
  auto take = [&](size_t bytes) {
    const size_t o = off;
    off += (size_t)round_up((int64_t)bytes, 256);
    return o;
  };
  t->out = take(P * d * 2);
  t->ckpt = take((2 * (int64_t)c.n_blocks + 1) * P * d * 4);
  t->dxa = take(P * d * 4);
  t->dxb = take(P * d * 4);
  t->partial = take((size_t)rmsnorm_bwd_blocks(P) * d * 4);
  size_t half = 0;
  if (c.n_blocks > 0) {
    half = std::max(mlp_grad_plan(P, d, c.mlp_hidden).total,
                    attn_grad_plan(bdesc, d, c.n_heads).total);
  }
  t->dx16 = 0;
  t->dxT = (size_t)round_up(P * d * 2, 256);
  t->xT = t->dxT + (size_t)round_up(d * t->Pp * 2, 256);
  const size_t pe = t->xT + (size_t)round_up(t->fwd.Kp * t->Pp * 2, 256);
  t->half_bytes = std::max(half, pe);
  t->half = take(t->half_bytes);
  t->total = off;
  return VIT_OK;
}

// PatchMerger projector: argument checks and workspace layout
vit_status check_merger(const vit_merger* m) {
  if (!m) return fail(VIT_E_ARG, "merger is NULL");
  if (m->dim <= 0 || m->dim % 16 || m->dim > 4096)
    return fail(VIT_E_SHAPE, "merger dim %d: need a multiple of 16, at most 4096", m->dim);
  if (m->hidden <= 0 || m->hidden % 64)
    return fail(VIT_E_SHAPE, "merger hidden %d: need a positive multiple of 64", m->hidden);
  if (m->out_dim <= 0 || m->out_dim % 8)
    return fail(VIT_E_SHAPE, "merger out_dim %d: need a positive multiple of 8", m->out_dim);
  if (!(m->eps >= 0.f)) return fail(VIT_E_ARG, "merger eps must be >= 0");
  return VIT_OK;
}

bool misaligned16(const void* p) { return ((uintptr_t)p & 15) != 0; }

struct MergerPlan {
  int64_t T = 0;
  size_t G = 0, H = 0, total = 0;
};

MergerPlan merger_plan(const vit_merger& m, const VarlenDesc& d) {
  MergerPlan p;
  p.T = d.total / 4;
  p.G = 0;
  p.H = round_up((int64_t)(p.T * 4 * m.dim * 2), 256);
  p.total = p.H + round_up((int64_t)(p.T * m.hidden * 2), 256);
  return p;
}

}  // namespace

// Workspace of vit_encode_varlen_noalloc: one array in the library's device
// image, so every GPU the library runs on holds its own copy (from module load
// until the process ends) and no call allocates.  Host code never uses the
// array's name as a device address: its address on each device is taken once
// with hipGetSymbolAddress (device current) and kept per device.
static constexpr size_t kScratchBytes = (size_t)160 << 20;
static_assert(kScratchBytes == VIT_NOALLOC_WORKSPACE_MAX, "header and library agree");
static __device__ __attribute__((aligned(256))) char scratch[kScratchBytes];

static constexpr int kMaxDevices = 64;
static std::mutex g_scratch_mu;
static void* g_scratch_ptr[kMaxDevices] = {};

// Device address of the current device's scratch array (looked up on the first
// call on that device).
static vit_status scratch_on_current_device(void** out) {
  int dev = -1;
  VIT_TRY(hip_check(hipGetDevice(&dev), "hipGetDevice"));
  if (dev < 0 || dev >= kMaxDevices) return fail(VIT_E_ARG, "device %d out of range", dev);
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (!g_scratch_ptr[dev]) {
    void* p = nullptr;
    VIT_TRY(hip_check(hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)), "scratch address"));
    if (!p) return fail(VIT_E_HIP, "scratch address is NULL on device %d", dev);
    g_scratch_ptr[dev] = p;
  }
  *out = g_scratch_ptr[dev];
  return VIT_OK;
}

extern "C" {

const char* vit_status_str(int32_t st) {
  switch (st) {
    case VIT_OK: return "ok";
    case VIT_E_ARG: return "invalid argument";
    case VIT_E_SHAPE: return "invalid or unsupported shape";
    case VIT_E_ODD_GRID: return "grid not divisible by the aligner merge size";
    case VIT_E_WORKSPACE: return "workspace too small";
    case VIT_E_HIP: return "HIP runtime error";
    default: return "unknown status";
  }
}

const char* vit_last_error(void) { return g_last_error.c_str(); }

size_t vit_workspace_bytes(const vit_config* cfg, const int32_t* grid_hw_host, int32_t n_images,
                           int32_t flags) {
  if (check_config(cfg) != VIT_OK) return 0;
  if (flags & ~(VIT_NO_ALIGNER | VIT_OUT_NLAYOUT | VIT_IN_PIXELS | VIT_ALIGN_PAD)) {
    fail(VIT_E_ARG, "unknown flags %d", flags);
    return 0;
  }
  if ((flags & VIT_IN_PIXELS) && patch_size_of(*cfg) == 0) {
    fail(VIT_E_SHAPE, "pixel input needs patch_dim = 3*ps^2 (got %d)", cfg->patch_dim);
    return 0;
  }
  VarlenDesc d;
  const bool aligner = !(flags & VIT_NO_ALIGNER);
  if (build_desc(grid_hw_host, n_images, attention_q_tile(cfg->dtype, cfg->head_dim), aligner,
                 cfg->merge, &d, (flags & VIT_ALIGN_PAD) != 0) != VIT_OK)
    return 0;
  return make_plan(*cfg, d, flags).total;
}

vit_status vit_encode(const vit_config* cfg, const vit_weights* w, const void* in, int32_t grid_h,
                      int32_t grid_w, int32_t flags, void* out, void* ws, size_t ws_bytes,
                      void* stream) {
  const int32_t g[2] = {grid_h, grid_w};
  return encode_impl(cfg, w, in, g, 1, flags, out, ws, ws_bytes, (hipStream_t)stream);
}

vit_status vit_encode_varlen(const vit_config* cfg, const vit_weights* w, const void* in,
                             const int32_t* grid_hw_host, int32_t n_images, int32_t flags,
                             void* out, void* ws, size_t ws_bytes, void* stream) {
  return encode_impl(cfg, w, in, grid_hw_host, n_images, flags, out, ws, ws_bytes,
                     (hipStream_t)stream);
}

vit_status vit_encode_varlen_noalloc(const vit_config* cfg, const vit_weights* w, const void* in,
                                     const int32_t* grid_hw_host, int32_t n_images,
                                     int32_t flags, void* out, void* stream) {
  const size_t need = vit_workspace_bytes(cfg, grid_hw_host, n_images, flags);
  if (need == 0)  // invalid arguments: encode_impl reports which
    return encode_impl(cfg, w, in, grid_hw_host, n_images, flags, out, nullptr, 0,
                       (hipStream_t)stream);
  if (need > kScratchBytes)
    return fail(VIT_E_WORKSPACE,
                "this call needs %zu bytes of workspace; vit_encode_varlen_noalloc holds at "
                "most %zu (call vit_encode_varlen with a workspace instead)",
                need, kScratchBytes);
  void* ws = nullptr;
  VIT_TRY(scratch_on_current_device(&ws));
  return encode_impl(cfg, w, in, grid_hw_host, n_images, flags, out, ws, kScratchBytes,
                     (hipStream_t)stream);
}

size_t vit_noalloc_workspace_limit(void) { return kScratchBytes; }

vit_status vit_aligner_layout(int32_t grid_h, int32_t grid_w, int32_t merge, int32_t* perm,
                              int32_t* nl_type, int32_t* nl_src, void* stream) {
  if (merge != 2) return fail(VIT_E_SHAPE, "merge %d unsupported (2)", merge);
  if (grid_h <= 0 || grid_w <= 0 || (int64_t)grid_h * grid_w > (1 << 24))
    return fail(VIT_E_SHAPE, "bad grid %dx%d", grid_h, grid_w);
  if (grid_h % merge || grid_w % merge)
    return fail(VIT_E_ODD_GRID, "grid %dx%d not divisible by %d", grid_h, grid_w, merge);
  return hip_check(launch_layout(grid_h, grid_w, merge, perm, nl_type, nl_src,
                                 (hipStream_t)stream),
                   "layout");
}

vit_status vit_rmsnorm(const float* x, const float* w, float eps, int64_t rows, int32_t dim,
                       int32_t out_dtype, void* out, void* stream) {
  if (!x || !w || !out) return fail(VIT_E_ARG, "NULL pointer");
  if (out_dtype != VIT_BF16 && out_dtype != VIT_F32) return fail(VIT_E_ARG, "bad dtype");
  if (rows < 0 || dim <= 0 || dim % 4) return fail(VIT_E_SHAPE, "bad rows/dim");
  return hip_check(launch_rmsnorm(x, w, eps, rows, dim, out_dtype, out, (hipStream_t)stream),
                   "rmsnorm");
}

vit_status vit_rope_table(const int32_t* grid_hw_host, int32_t n_images, int32_t head_dim,
                          float theta, void* table, void* stream) {
  if (!table) return fail(VIT_E_ARG, "table is NULL");
  if (head_dim <= 0 || head_dim % 4 || head_dim / 4 > kRopeMaxFreqs)
    return fail(VIT_E_SHAPE, "head_dim %d: need a multiple of 4, at most %d", head_dim,
                4 * kRopeMaxFreqs);
  VarlenDesc d;
  VIT_TRY(build_desc(grid_hw_host, n_images, 1, false, 2, &d));
  return hip_check(launch_rope_table(d, head_dim, theta, table, (hipStream_t)stream), "rope table");
}

vit_status vit_rope(int32_t dtype, void* qkv, const void* table, int64_t P, int32_t n_heads,
                    int32_t head_dim, void* stream) {
  if (!qkv || !table) return fail(VIT_E_ARG, "NULL pointer");
  if (dtype != VIT_BF16 && dtype != VIT_F32) return fail(VIT_E_ARG, "bad dtype");
  if (P < 0 || n_heads <= 0 || head_dim <= 0 || head_dim % 4) return fail(VIT_E_SHAPE, "bad dims");
  return hip_check(launch_rope(dtype, qkv, table, P, n_heads, head_dim, (hipStream_t)stream),
                   "rope");
}

size_t vit_attention_workspace_bytes(int32_t dtype, const int32_t* grid_hw_host,
                                     int32_t n_images, int32_t n_heads, int32_t head_dim) {
  if (dtype != VIT_BF16 || (head_dim != 64 && head_dim != 72)) return 0;
  VarlenDesc d;
  if (build_desc(grid_hw_host, n_images, attention_q_tile(dtype, head_dim), false, 2, &d) != VIT_OK)
    return 0;
  return (size_t)n_heads * head_dim * d.kv_off[n_images] * 2;
}

vit_status vit_attention_varlen(int32_t dtype, const void* qkv, const int32_t* grid_hw_host,
                                int32_t n_images, int32_t n_heads, int32_t head_dim, void* out,
                                void* ws, size_t ws_bytes, void* stream) {
  if (!qkv || !out) return fail(VIT_E_ARG, "NULL pointer");
  if (dtype != VIT_BF16 && dtype != VIT_F32) return fail(VIT_E_ARG, "bad dtype");
  if (n_heads <= 0 || (head_dim != 64 && head_dim != 72))
    return fail(VIT_E_SHAPE, "head_dim %d unsupported (64 or 72)", head_dim);
  VarlenDesc d;
  VIT_TRY(build_desc(grid_hw_host, n_images, attention_q_tile(dtype, head_dim), false, 2, &d));
  hipStream_t s = (hipStream_t)stream;
  if (dtype == VIT_BF16) {
    const size_t need = (size_t)n_heads * head_dim * d.kv_off[n_images] * 2;
    if (!ws || ws_bytes < need)
      return fail(VIT_E_WORKSPACE, "attention workspace %zu < %zu", ws ? ws_bytes : (size_t)0, need);
    VIT_HIP(launch_vt_pack(qkv, d, n_heads, head_dim, ws, d.kv_off[n_images], s), "pack V");
    if (head_dim == 64)
      return hip_check(launch_attention_vt(qkv, 3 * (int64_t)n_heads * head_dim, ws,
                                           d.kv_off[n_images], d, n_heads, out, s),
                       "attention");
    return hip_check(launch_attention(dtype, qkv, ws, d.kv_off[n_images], d, n_heads, head_dim,
                                      out, s),
                     "attention");
  }
  return hip_check(launch_attention(dtype, qkv, nullptr, 0, d, n_heads, head_dim, out, s),
                   "attention");
}

vit_status vit_gemm(int32_t dtype, int32_t epilogue, const void* A, int64_t lda, const void* B,
                    const void* B2, int64_t ldb, void* C, int64_t ldc, int64_t M, int64_t N,
                    int64_t K, void* stream) {
  if (dtype != VIT_BF16 && dtype != VIT_F32) return fail(VIT_E_ARG, "bad dtype");
  if (epilogue < VIT_EPI_STORE || epilogue > VIT_EPI_SWIGLU) return fail(VIT_E_ARG, "bad epilogue");
  if (!A || !B || !C || (epilogue == VIT_EPI_SWIGLU && !B2)) return fail(VIT_E_ARG, "NULL pointer");
  if (M < 0 || N < 0 || K <= 0 || lda < K || ldb < K || ldc < N)
    return fail(VIT_E_SHAPE, "bad GEMM dims");
  if (M >= (1LL << 31) || N >= (1LL << 31) || K >= (1LL << 31))
    return fail(VIT_E_SHAPE, "GEMM dims must stay below 2^31");
  if (dtype == VIT_BF16) {
    if (K % 8 || lda % 8 || ldb % 8) return fail(VIT_E_SHAPE, "bf16 GEMM needs K, lda, ldb multiples of 8");
    if (((uintptr_t)A | (uintptr_t)B | (uintptr_t)(B2 ? B2 : B)) & 15)
      return fail(VIT_E_ARG, "bf16 GEMM operands must be 16-byte aligned");
  }
  return gemm(dtype, epilogue, A, lda, B, B2, ldb, C, ldc, M, N, K, nullptr, (hipStream_t)stream);
}

vit_status vit_aligner_gather(int32_t dtype, const void* x, const int32_t* grid_hw_host,
                              int32_t n_images, int32_t d, void* G, void* stream) {
  if (!x || !G) return fail(VIT_E_ARG, "NULL pointer");
  if (dtype != VIT_BF16 && dtype != VIT_F32) return fail(VIT_E_ARG, "bad dtype");
  if (d <= 0 || (d * (int)esize(dtype)) % 16) return fail(VIT_E_SHAPE, "row bytes must be a multiple of 16");
  VarlenDesc desc;
  VIT_TRY(build_desc(grid_hw_host, n_images, 1, true, 2, &desc));
  return hip_check(launch_gather(dtype, x, desc, d, 2, G, (hipStream_t)stream), "gather");
}

size_t vit_merge_workspace_bytes(int64_t positions) {
  if (positions < 0 || positions >= (1LL << 31)) {
    fail(VIT_E_SHAPE, "positions %lld out of range [0, 2^31)", (long long)positions);
    return 0;
  }
  return merge_workspace_bytes(positions);
}

vit_status vit_merge_image_embeddings(int32_t dtype, void* embeds, int64_t positions,
                                      int32_t hidden, const int32_t* types, const void* tokens,
                                      int64_t n_tokens, const void* sentinels, int32_t* n_image,
                                      void* ws, size_t ws_bytes, void* stream) {
  if (dtype != VIT_BF16 && dtype != VIT_F32) return fail(VIT_E_ARG, "bad dtype");
  if (positions < 0 || positions >= (1LL << 31) || n_tokens < 0 || n_tokens >= (1LL << 31))
    return fail(VIT_E_SHAPE, "positions / n_tokens out of range [0, 2^31)");
  const int64_t row_bytes = (int64_t)hidden * (int64_t)esize(dtype);
  if (hidden <= 0 || row_bytes % 16) return fail(VIT_E_SHAPE, "hidden %d: row bytes must be %% 16", hidden);
  if (positions > 0 && (!embeds || !types || !sentinels))
    return fail(VIT_E_ARG, "NULL pointer");
  if (n_tokens > 0 && !tokens) return fail(VIT_E_ARG, "tokens is NULL");
  if (((uintptr_t)embeds | (uintptr_t)tokens | (uintptr_t)sentinels) & 15)
    return fail(VIT_E_ARG, "rows must be 16-byte aligned");
  const size_t need = merge_workspace_bytes(positions);
  if (!ws || ws_bytes < need)
    return fail(VIT_E_WORKSPACE, "merge workspace %zu < %zu", ws ? ws_bytes : (size_t)0, need);
  hipStream_t s = (hipStream_t)stream;
  VIT_HIP(launch_merge_rank(types, positions, n_image, ws, s), "merge ranks");
  ProfScope ps(VIT_K_MERGE, s);
  return hip_check(launch_merge_copy(embeds, positions, row_bytes, types, tokens, n_tokens,
                                     sentinels, ws, s),
                   "merge copy");
}

size_t vit_patch_merger_workspace_bytes(const vit_merger* m, const int32_t* grid_hw_host,
                                        int32_t n_images) {
  if (check_merger(m) != VIT_OK) return 0;
  VarlenDesc d;
  if (build_desc(grid_hw_host, n_images, 1, true, 2, &d) != VIT_OK) return 0;
  return merger_plan(*m, d).total;
}

vit_status vit_patch_merger(const vit_merger* m, const void* x, const int32_t* grid_hw_host,
                            int32_t n_images, void* out, void* ws, size_t ws_bytes, void* stream) {
  VIT_TRY(check_merger(m));
  if (!x || !out || !m->ln_w || !m->ln_b || !m->w1 || !m->b1 || !m->w2 || !m->b2)
    return fail(VIT_E_ARG, "NULL pointer");
  if (misaligned16(x) || misaligned16(out) || misaligned16(ws) || misaligned16(m->ln_w) ||
      misaligned16(m->ln_b) || misaligned16(m->w1) || misaligned16(m->b1) || misaligned16(m->w2) ||
      misaligned16(m->b2))
    return fail(VIT_E_ARG, "merger buffers must be 16-byte aligned");
  VarlenDesc d;
  VIT_TRY(build_desc(grid_hw_host, n_images, 1, true, 2, &d));
  const MergerPlan p = merger_plan(*m, d);
  if (!ws || ws_bytes < p.total)
    return fail(VIT_E_WORKSPACE, "merger workspace %zu < %zu", ws ? ws_bytes : (size_t)0, p.total);
  char* base = (char*)ws;
  void* G = base + p.G;
  void* H = base + p.H;
  const int64_t K1 = 4 * (int64_t)m->dim;
  GemmArgs g1 = gemm_args(G, K1, m->w1, nullptr, K1, H, m->hidden, p.T, m->hidden, K1, nullptr);
  g1.bias = m->b1;
  GemmArgs g2 = gemm_args(H, m->hidden, m->w2, nullptr, m->hidden, out, m->out_dim, p.T,
                          m->out_dim, m->hidden, nullptr);
  g2.bias = m->b2;
  if (!gemm_bf16_mfma_eligible(g1) || !gemm_bf16_mfma_eligible(g2))
    return fail(VIT_E_SHAPE, "merger GEMMs too large for 32-bit operand offsets");
  hipStream_t s = (hipStream_t)stream;
  {
    ProfScope ps(VIT_K_LNGATHER, s);
    VIT_HIP(launch_ln_gather(x, d, m->dim, m->ln_w, m->ln_b, m->eps, G, s), "merger norm + gather");
  }
  {
    ProfScope ps(VIT_K_PROJ1, s);
    VIT_HIP(launch_gemm_bf16(VIT_EPI_BIAS_GELU, g1, s), "merger first linear");
  }
  ProfScope ps(VIT_K_PROJ2, s);
  return hip_check(launch_gemm_bf16(VIT_EPI_BIAS, g2, s), "merger second linear");
}

vit_status vit_layernorm_gather(const void* x, const int32_t* grid_hw_host, int32_t n_images,
                                int32_t dim, const float* ln_w, const float* ln_b, float eps,
                                void* G, void* stream) {
  if (!x || !ln_w || !ln_b || !G) return fail(VIT_E_ARG, "NULL pointer");
  if (dim <= 0 || dim % 8 || dim > 4096)
    return fail(VIT_E_SHAPE, "dim %d: need a multiple of 8, at most 4096", dim);
  if (!(eps >= 0.f)) return fail(VIT_E_ARG, "eps must be >= 0");
  if (misaligned16(x) || misaligned16(G) || misaligned16(ln_w) || misaligned16(ln_b))
    return fail(VIT_E_ARG, "buffers must be 16-byte aligned");
  VarlenDesc d;
  VIT_TRY(build_desc(grid_hw_host, n_images, 1, true, 2, &d));
  return hip_check(launch_ln_gather(x, d, dim, ln_w, ln_b, eps, G, (hipStream_t)stream),
                   "layernorm gather");
}

vit_status vit_gemm_bias(int32_t epilogue, const void* A, int64_t lda, const void* B, int64_t ldb,
                         const float* bias, void* C, int64_t ldc, int64_t M, int64_t N, int64_t K,
                         void* stream) {
  if (epilogue != VIT_EPI_BIAS && epilogue != VIT_EPI_BIAS_GELU)
    return fail(VIT_E_ARG, "bad bias epilogue %d", epilogue);
  if (!A || !B || !bias || !C) return fail(VIT_E_ARG, "NULL pointer");
  if (M < 0 || N <= 0 || K <= 0 || lda < K || ldb < K || ldc < N || M >= (1LL << 31) ||
      N >= (1LL << 31) || K >= (1LL << 31))
    return fail(VIT_E_SHAPE, "bad GEMM dims");
  if (misaligned16(bias)) return fail(VIT_E_ARG, "bias must be 16-byte aligned");
  GemmArgs g = gemm_args(A, lda, B, nullptr, ldb, C, ldc, M, N, K, nullptr);
  g.bias = bias;
  if (!gemm_bf16_mfma_eligible(g))
    return fail(VIT_E_SHAPE, "bias GEMM needs K %% 64 == 0, N %% 4 == 0, 16-byte aligned rows");
  return hip_check(launch_gemm_bf16(epilogue, g, (hipStream_t)stream), "bias gemm");
}

size_t vit_mlp_backward_workspace_bytes(int64_t rows, int32_t dim, int32_t hidden) {
  if (check_mlp_grad_sizes(rows, dim, hidden) != VIT_OK) return 0;
  return mlp_grad_plan(rows, dim, hidden).total;
}

vit_status vit_mlp_backward(const vit_mlp_grad* a, void* ws, size_t ws_bytes, void* stream) {
  if (!a) return fail(VIT_E_ARG, "arguments are NULL");
  VIT_TRY(check_mlp_grad_sizes(a->rows, a->dim, a->hidden));
  if (!(a->eps >= 0.f)) return fail(VIT_E_ARG, "eps must be >= 0");
  const void* ptrs[] = {a->x, a->norm_w, a->w_gate, a->w_up, a->w_down, a->dy, a->dx,
                        a->d_norm_w, a->d_w_gate, a->d_w_up, a->d_w_down};
  for (const void* q : ptrs) {
    if (!q) return fail(VIT_E_ARG, "NULL pointer");
    if (misaligned16(q)) return fail(VIT_E_ARG, "buffers must be 16-byte aligned");
  }
  const int64_t P = a->rows, d = a->dim, h = a->hidden;
  const MlpGradPlan p = mlp_grad_plan(P, d, h);
  const int64_t hp = p.hp;
  if (!ws || ws_bytes < p.total || misaligned16(ws))
    return fail(VIT_E_WORKSPACE, "workspace %zu < %zu (or misaligned)", ws ? ws_bytes : (size_t)0,
                p.total);
  char* base = (char*)ws;
  bf16* n = (bf16*)(base + p.n);
  bf16* dy16 = (bf16*)(base + p.dy16);
  float* gu = (float*)(base + p.gu);
  float* da = (float*)(base + p.da);
  bf16* act = (bf16*)(base + p.a);
  bf16* dgdu = (bf16*)(base + p.dgdu);
  float* dn = (float*)(base + p.dn);
  bf16* wdT = (bf16*)(base + p.wdT);
  bf16* wguT = (bf16*)(base + p.wguT);
  bf16* dyT = (bf16*)(base + p.dyT);
  bf16* aT = (bf16*)(base + p.aT);
  bf16* dgduT = (bf16*)(base + p.dgduT);
  bf16* nT = (bf16*)(base + p.nT);
  float* partial = (float*)(base + p.partial);
  hipStream_t s = (hipStream_t)stream;
  auto mm = [&](const void* A, int64_t lda, const void* B, int64_t ldb, void* C, int64_t ldc,
                int64_t M, int64_t N, int64_t K, bool dn_gemm = false) -> vit_status {
    GemmArgs g = gemm_args(A, lda, B, nullptr, ldb, C, ldc, M, N, K, nullptr);
    if (!gemm_bf16_mfma_eligible(g)) return fail(VIT_E_SHAPE, "backward GEMM %lldx%lldx%lld too large",
                                                 (long long)M, (long long)N, (long long)K);
    ProfScope all(VIT_K_BWD_GEMM, s);
    ProfScope one(dn_gemm ? VIT_K_BWD_DN : -1, s);
    return hip_check(launch_gemm_bf16(VIT_EPI_STORE_F32, g, s), "backward gemm");
  };
  // the memory-bound passes below are each timed as VIT_K_BWD_PASS
  // forward recomputation: n = bf16(norm2(x)), g and u (fp32, side by side)
  {
    ProfScope ps(VIT_K_BWD_PASS, s);
    VIT_HIP(launch_rmsnorm(a->x, a->norm_w, a->eps, P, (int)d, VIT_BF16, n, s), "norm");
  }
  VIT_TRY(mm(n, d, a->w_gate, d, gu, 2 * hp, P, h, d));
  VIT_TRY(mm(n, d, a->w_up, d, gu + hp, 2 * hp, P, h, d));
  // da = dy . W_down
  {
    ProfScope ps(VIT_K_BWD_PASS, s);
    VIT_HIP(launch_cast_transpose(a->dy, P, d, dy16, dyT, p.Pp, p.Pp, s), "cast + transpose dy");
  }
  {
    ProfScope ps(VIT_K_BWD_PASS, s);
    VIT_HIP(launch_transpose_bf16(a->w_down, d, h, h, wdT, d, d, s), "transpose W_down");
  }
  VIT_TRY(mm(dy16, d, wdT, d, da, h, P, h, d));
  // SwiGLU gradient (and the activation for dW_down)
  {
    ProfScope ps(VIT_K_BWD_PASS, s);
    VIT_HIP(launch_swiglu_bwd(gu, da, P, (int)h, (int)hp, act, dgdu, s), "swiglu backward");
  }
  // dn = dg . W_gate + du . W_up (columns h .. hp-1 of each half zero on both sides)
  {
    ProfScope ps(VIT_K_BWD_PASS, s);
    VIT_HIP(launch_transpose_bf16(a->w_gate, h, d, d, wguT, hp, 2 * hp, s), "transpose W_gate");
  }
  {
    ProfScope ps(VIT_K_BWD_PASS, s);
    VIT_HIP(launch_transpose_bf16(a->w_up, h, d, d, wguT + hp, hp, 2 * hp, s), "transpose W_up");
  }
  VIT_TRY(mm(dgdu, 2 * hp, wguT, 2 * hp, dn, d, P, d, 2 * hp, true));
  // RMSNorm gradient + residual, and the norm scale gradient
  {
    ProfScope ps(VIT_K_BWD_PASS, s);
    VIT_HIP(launch_rmsnorm_bwd(a->x, a->norm_w, dn, a->dy, P, (int)d, a->eps, a->dx, partial,
                               a->d_norm_w, s),
            "norm backward");
  }
  // weight gradients: contractions over the rows (zero-padded to Pp)
  {
    ProfScope ps(VIT_K_BWD_PASS, s);
    VIT_HIP(launch_transpose_bf16(act, P, h, h, aT, p.Pp, p.Pp, s), "transpose a");
  }
  {
    ProfScope ps(VIT_K_BWD_PASS, s);
    VIT_HIP(launch_transpose_bf16(dgdu, P, 2 * hp, 2 * hp, dgduT, p.Pp, p.Pp, s), "transpose dg, du");
  }
  {
    ProfScope ps(VIT_K_BWD_PASS, s);
    VIT_HIP(launch_transpose_bf16(n, P, d, d, nT, p.Pp, p.Pp, s), "transpose n");
  }
  VIT_TRY(mm(dyT, p.Pp, aT, p.Pp, a->d_w_down, h, d, h, p.Pp));
  VIT_TRY(mm(dgduT, p.Pp, nT, p.Pp, a->d_w_gate, d, h, d, p.Pp));
  return mm(dgduT + hp * p.Pp, p.Pp, nT, p.Pp, a->d_w_up, d, h, d, p.Pp);
}

size_t vit_attn_backward_workspace_bytes(const vit_attn_grad* a, const int32_t* grid_hw_host,
                                         int32_t n_images) {
  if (check_attn_grad(a) != VIT_OK) return 0;
  VarlenDesc d;
  if (build_desc(grid_hw_host, n_images, attention_bwd_tile(), false, 2, &d) != VIT_OK) return 0;
  return attn_grad_plan(d, a->dim, a->n_heads).total;
}

vit_status vit_attn_backward(const vit_attn_grad* a, const int32_t* grid_hw_host,
                             int32_t n_images, void* ws, size_t ws_bytes, void* stream) {
  VIT_TRY(check_attn_grad(a));
  const void* ptrs[] = {a->x, a->norm_w, a->wqkv, a->wo, a->dy, a->dx, a->d_norm_w, a->d_wqkv,
                        a->d_wo};
  for (const void* q : ptrs) {
    if (!q) return fail(VIT_E_ARG, "NULL pointer");
    if (misaligned16(q)) return fail(VIT_E_ARG, "buffers must be 16-byte aligned");
  }
  const int64_t d = a->dim, H = a->n_heads;
  const int D = (int)(d / H);  // head_dim, 64 or 72
  VarlenDesc fwd, bwd;  // q-tiles of the forward attention and of the backward kernels
  VIT_TRY(build_desc(grid_hw_host, n_images, attention_q_tile(VIT_BF16, D), false, 2, &fwd));
  VIT_TRY(build_desc(grid_hw_host, n_images, attention_bwd_tile(), false, 2, &bwd));
  const AttnGradPlan p = attn_grad_plan(bwd, d, H);
  const int64_t P = p.P;
  if (!ws || ws_bytes < p.total || misaligned16(ws))
    return fail(VIT_E_WORKSPACE, "workspace %zu < %zu (or misaligned)", ws ? ws_bytes : (size_t)0,
                p.total);
  char* base = (char*)ws;
  bf16* n = (bf16*)(base + p.n);
  bf16* qkv = (bf16*)(base + p.qkv);
  void* table = base + p.table;
  bf16* vt = (bf16*)(base + p.vt);
  bf16* o = (bf16*)(base + p.o);
  float* lse = (float*)(base + p.lse);
  bf16* dy16 = (bf16*)(base + p.dy16);
  bf16* dO = (bf16*)(base + p.dO);
  float* Dq = (float*)(base + p.Dq);
  bf16* qt = (bf16*)(base + p.qt);
  bf16* kt = (bf16*)(base + p.kt);
  bf16* dot = (bf16*)(base + p.dot);
  bf16* dqkv = (bf16*)(base + p.dqkv);
  bf16* woT = (bf16*)(base + p.woT);
  bf16* wqkvT = (bf16*)(base + p.wqkvT);
  float* dn = (float*)(base + p.dn);
  bf16* dyT = (bf16*)(base + p.dyT);
  bf16* oT = (bf16*)(base + p.oT);
  bf16* dqkvT = (bf16*)(base + p.dqkvT);
  bf16* nT = (bf16*)(base + p.nT);
  float* partial = (float*)(base + p.partial);
  hipStream_t s = (hipStream_t)stream;
  auto mm = [&](int epi, const void* A, int64_t lda, const void* B, int64_t ldb, void* C,
                int64_t ldc, int64_t M, int64_t N, int64_t K) -> vit_status {
    GemmArgs g = gemm_args(A, lda, B, nullptr, ldb, C, ldc, M, N, K, nullptr);
    if (!gemm_bf16_mfma_eligible(g)) return fail(VIT_E_SHAPE, "backward GEMM %lldx%lldx%lld too large",
                                                 (long long)M, (long long)N, (long long)K);
    ProfScope all(VIT_K_BWD_GEMM, s);
    return hip_check(launch_gemm_bf16(epi, g, s), "backward gemm");
  };
  // forward recomputation: n, rotated q, k and v, attention output and lse
  VIT_HIP(launch_rmsnorm(a->x, a->norm_w, a->eps, P, (int)d, VIT_BF16, n, s), "norm");
  VIT_HIP(launch_rope_table(fwd, D, a->rope_theta, table, s), "rope table");
  if (D == 64) {
    // qkv = n . Wqkv^T with the rotary applied to the q and k columns in the epilogue
    GemmArgs g = gemm_args(n, d, a->wqkv, nullptr, d, qkv, 3 * d, P, 3 * d, d, nullptr);
    g.rope_table = table;
    g.rope_cols = 2 * d;
    if (!gemm_bf16_can_fuse_rope(g)) return fail(VIT_E_SHAPE, "wqkv GEMM too large");
    {
      ProfScope all(VIT_K_BWD_GEMM, s);
      VIT_HIP(launch_gemm_bf16(VIT_EPI_STORE_ROPE, g, s), "qkv + rotary gemm");
    }
    VIT_HIP(launch_vt_pack(qkv, fwd, (int)H, 64, vt, p.kv, s), "pack V");
    ProfScope ps(VIT_K_ATTN, s);
    VIT_HIP(launch_attention_vt(qkv, 3 * d, vt, p.kv, fwd, (int)H, o, s, lse), "attention");
  } else {
    // as the encoder's head_dim-72 path: qkv = n . Wqkv^T, then one launch rotates
    // q and k in place and packs V^T for the 16x16x32 attention kernel
    VIT_TRY(mm(VIT_EPI_STORE, n, d, a->wqkv, d, qkv, 3 * d, P, 3 * d, d));
    VIT_HIP(launch_vt_pack(qkv, fwd, (int)H, D, vt, p.kv, s, table), "rotary + pack V");
    ProfScope ps(VIT_K_ATTN, s);
    VIT_HIP(launch_attention(VIT_BF16, qkv, vt, p.kv, fwd, (int)H, D, o, s, lse), "attention");
  }
  // dO = dy . Wo, Dq = rowsum(dO o), transposed operands of the attention gradient
  VIT_HIP(launch_cast_transpose(a->dy, P, d, dy16, dyT, p.Pp, p.Pp, s), "cast + transpose dy");
  VIT_HIP(launch_transpose_bf16(a->wo, d, d, d, woT, d, d, s), "transpose wo");
  VIT_TRY(mm(VIT_EPI_STORE, dy16, d, woT, d, dO, d, P, d, d));
  VIT_HIP(launch_rowdot(dO, o, P, (int)H, D, Dq, s), "rowsum(dO o)");
  VIT_HIP(launch_tpack(qkv, 3 * d, 0, fwd, (int)H, D, qt, p.kv, s), "pack Q^T");
  VIT_HIP(launch_tpack(qkv, 3 * d, d, fwd, (int)H, D, kt, p.kv, s), "pack K^T");
  VIT_HIP(launch_tpack(dO, d, 0, fwd, (int)H, D, dot, p.kv, s), "pack dO^T");
  {
    ProfScope ps(VIT_K_BWD_ATTN, s);
    VIT_HIP(launch_attention_bwd(qkv, 3 * d, dO, qt, kt, dot, p.kv, lse, Dq, table, bwd, (int)H, D,
                                 dqkv, 3 * d, s),
            "attention backward");
  }
  // head_dim 72: dq and dk come out in the rotated space; the rotation by the
  // opposite angles gives the gradients with respect to wqkv's q and k outputs
  if (D != 64) VIT_HIP(launch_rope_inverse(dqkv, table, P, (int)H, D, s), "rotary backward");
  // dn = dqkv . Wqkv, then the norm gradient and the residual
  VIT_HIP(launch_transpose_bf16(a->wqkv, 3 * d, d, d, wqkvT, 3 * d, 3 * d, s), "transpose wqkv");
  VIT_TRY(mm(VIT_EPI_STORE_F32, dqkv, 3 * d, wqkvT, 3 * d, dn, d, P, d, 3 * d));
  VIT_HIP(launch_rmsnorm_bwd(a->x, a->norm_w, dn, a->dy, P, (int)d, a->eps, a->dx, partial,
                             a->d_norm_w, s),
          "norm backward");
  // weight gradients: contractions over the rows (zero-padded to Pp)
  VIT_HIP(launch_transpose_bf16(o, P, d, d, oT, p.Pp, p.Pp, s), "transpose o");
  VIT_HIP(launch_transpose_bf16(dqkv, P, 3 * d, 3 * d, dqkvT, p.Pp, p.Pp, s), "transpose dqkv");
  VIT_HIP(launch_transpose_bf16(n, P, d, d, nT, p.Pp, p.Pp, s), "transpose n");
  // dWqkv (3d x d) and dWo (d x d) in one grouped launch: 192 + 64 tiles of 128x128
  // fill the 256 CUs once where the two alone would take two launches
  GemmArgs gq = gemm_args(dqkvT, p.Pp, nT, nullptr, p.Pp, a->d_wqkv, d, 3 * d, d, p.Pp, nullptr);
  GemmArgs go = gemm_args(dyT, p.Pp, oT, nullptr, p.Pp, a->d_wo, d, d, d, p.Pp, nullptr);
  if (!gemm_bf16_mfma_eligible(gq) || !gemm_bf16_mfma_eligible(go))
    return fail(VIT_E_SHAPE, "weight-gradient GEMMs too large");
  ProfScope all(VIT_K_BWD_GEMM, s);
  return hip_check(launch_gemm_bf16_pair(VIT_EPI_STORE_F32, gq, go, s), "weight gradients");
}

size_t vit_tower_backward_workspace_bytes(const vit_config* cfg, const int32_t* grid_hw_host,
                                          int32_t n_images) {
  TowerGradPlan t;
  if (tower_setup(cfg, grid_hw_host, n_images, &t) != VIT_OK) return 0;
  return t.total;
}

vit_status vit_tower_backward(const vit_config* cfg, const vit_weights* w, const void* patches,
                              const int32_t* grid_hw_host, int32_t n_images, const float* dy,
                              const vit_tower_grads* gr, void* ws, size_t ws_bytes, void* stream) {
  TowerGradPlan t;
  VIT_TRY(tower_setup(cfg, grid_hw_host, n_images, &t));
  const vit_config& c = *cfg;
  VIT_TRY(check_weights(c, w, false));
  if (!patches || !dy || !gr) return fail(VIT_E_ARG, "NULL pointer");
  const int L = c.n_blocks;
  if (L > 0 && (!gr->d_wqkv || !gr->d_wo || !gr->d_w_gate || !gr->d_w_up || !gr->d_w_down ||
                !gr->d_norm1 || !gr->d_norm2))
    return fail(VIT_E_ARG, "per-block gradient array NULL");
  {
    const void* ptrs[] = {dy, gr->d_patch_embed, gr->d_final_norm};
    for (const void* q : ptrs) {
      if (!q) return fail(VIT_E_ARG, "NULL pointer");
      if (misaligned16(q)) return fail(VIT_E_ARG, "buffers must be 16-byte aligned");
    }
    // every block's gradient buffers before any work is enqueued
    for (int b = 0; b < L; ++b) {
      const void* blk[] = {gr->d_wqkv[b], gr->d_wo[b], gr->d_w_gate[b], gr->d_w_up[b],
                           gr->d_w_down[b], gr->d_norm1[b], gr->d_norm2[b]};
      for (const void* q : blk) {
        if (!q) return fail(VIT_E_ARG, "block %d has a NULL gradient pointer", b);
        if (misaligned16(q)) return fail(VIT_E_ARG, "block %d: gradients must be 16-byte aligned", b);
      }
    }
  }
  if (!ws || ws_bytes < t.total || misaligned16(ws))
    return fail(VIT_E_WORKSPACE, "workspace %zu < %zu (or misaligned)", ws ? ws_bytes : (size_t)0,
                t.total);
  hipStream_t s = (hipStream_t)stream;
  char* base = (char*)ws;
  const int64_t P = t.P, d = c.vision_dim;
  float* ckpt = (float*)(base + t.ckpt);
  float* cur = (float*)(base + t.dxa);
  float* other = (float*)(base + t.dxb);
  char* half = base + t.half;
  // forward with the residual stream kept at the input of every residual branch
  VIT_TRY(encode_impl(cfg, w, patches, grid_hw_host, n_images, VIT_NO_ALIGNER, base + t.out, base,
                      t.fwd.total, s, ckpt));
  // final norm (no residual around it)
  VIT_HIP(launch_rmsnorm_bwd(ckpt + 2 * (int64_t)L * P * d, w->final_norm, dy, nullptr, P, (int)d,
                             c.rms_eps, cur, (float*)(base + t.partial), gr->d_final_norm, s),
          "final norm backward");
  // blocks in reverse: the MLP half, then the attention half
  for (int b = L - 1; b >= 0; --b) {
    vit_mlp_grad m{};
    m.rows = P;
    m.dim = (int32_t)d;
    m.hidden = c.mlp_hidden;
    m.eps = c.rms_eps;
    m.x = ckpt + (2 * (int64_t)b + 1) * P * d;
    m.norm_w = w->norm2[b];
    m.w_gate = w->w_gate[b];
    m.w_up = w->w_up[b];
    m.w_down = w->w_down[b];
    m.dy = cur;
    m.dx = other;
    m.d_norm_w = gr->d_norm2[b];
    m.d_w_gate = gr->d_w_gate[b];
    m.d_w_up = gr->d_w_up[b];
    m.d_w_down = gr->d_w_down[b];
    VIT_TRY(vit_mlp_backward(&m, half, t.half_bytes, stream));
    vit_attn_grad a{};
    a.dim = (int32_t)d;
    a.n_heads = c.n_heads;
    a.rope_theta = c.rope_theta;
    a.eps = c.rms_eps;
    a.x = ckpt + 2 * (int64_t)b * P * d;
    a.norm_w = w->norm1[b];
    a.wqkv = w->wqkv[b];
    a.wo = w->wo[b];
    a.dy = other;
    a.dx = cur;
    a.d_norm_w = gr->d_norm1[b];
    a.d_wqkv = gr->d_wqkv[b];
    a.d_wo = gr->d_wo[b];
    VIT_TRY(vit_attn_backward(&a, grid_hw_host, n_images, half, t.half_bytes, stream));
  }
  // patch embedding: dWpe [d, patch_dim] = dx0^T . patches, a contraction over
  // the rows (zero-padded to Pp) of the transposed gradient and of the forward's
  // zero-padded patches
  bf16* dx16 = (bf16*)(half + t.dx16);
  bf16* dxT = (bf16*)(half + t.dxT);
  bf16* xT = (bf16*)(half + t.xT);
  VIT_HIP(launch_cast_transpose(cur, P, d, dx16, dxT, t.Pp, t.Pp, s), "cast + transpose dx0");
  VIT_HIP(launch_transpose_bf16(base + t.fwd.xpad, P, t.fwd.Kp, t.fwd.Kp, xT, t.Pp, t.Pp, s),
          "transpose patches");
  GemmArgs g = gemm_args(dxT, t.Pp, xT, nullptr, t.Pp, gr->d_patch_embed, c.patch_dim, d,
                         c.patch_dim, t.Pp, nullptr);
  if (!gemm_bf16_mfma_eligible(g)) return fail(VIT_E_SHAPE, "patch embedding gradient GEMM");
  return hip_check(launch_gemm_bf16(VIT_EPI_STORE_F32, g, s), "patch embedding gradient");
}

int64_t vit_mfma_peak_out_floats(void) { return mfma_peak_out_floats(); }

vit_status vit_mfma_peak(int32_t iters, float* out, double* flops, void* stream) {
  if (!out || !flops) return fail(VIT_E_ARG, "NULL pointer");
  if (iters <= 0 || iters > (1 << 24)) return fail(VIT_E_ARG, "iters %d out of range", iters);
  *flops = mfma_peak_flops(iters);
  return hip_check(launch_mfma_peak(iters, out, (hipStream_t)stream), "mfma peak probe");
}

vit_status vit_profile_enable(int32_t cls, int32_t on) {
  if (cls < 0 || cls >= VIT_K_COUNT) return fail(VIT_E_ARG, "bad kernel class %d", cls);
  Prof& p = prof();
  std::lock_guard<std::mutex> lk(p.mu);
  p.on[cls] = on != 0;
  p.used[cls] = 0;
  return VIT_OK;
}

vit_status vit_profile_read(int32_t cls, double* total_ms, int64_t* launches) {
  if (cls < 0 || cls >= VIT_K_COUNT) return fail(VIT_E_ARG, "bad kernel class %d", cls);
  if (!total_ms || !launches) return fail(VIT_E_ARG, "NULL pointer");
  Prof& p = prof();
  std::lock_guard<std::mutex> lk(p.mu);
  double sum = 0.0;
  for (size_t i = 0; i < p.used[cls]; ++i) {
    auto& pr = p.ev[cls][i];
    VIT_HIP(hipEventSynchronize(pr.second), "event sync");
    float ms = 0.f;
    VIT_HIP(hipEventElapsedTime(&ms, pr.first, pr.second), "event elapsed");
    sum += ms;
  }
  *total_ms = sum;
  *launches = (int64_t)p.used[cls];
  p.used[cls] = 0;
  return VIT_OK;
}

}  // extern "C"
