// api.cpp -- the C ABI of libdit.so (declared in include/dit.h): argument
// validation, the workspace plan, and the kernel sequence of one DiT block and
// one denoise step on a single HIP stream.
//
// The sequence follows the denoiser as the SGLang-Diffusion pages frame it:
// the DiT forward over patchified latents conditioned on the prompt
// embeddings and the timestep ("Support New Diffusion Models", section
// "2. Pipeline Config"), followed by the flow update driven by the sigma
// schedule ("Disaggregated Diffusion Pipeline", section "Quick Start";
// "Model Configuration Conventions", section "Sampling And Geometry").
#include <hip/hip_runtime.h>

#include <algorithm>
#include <cmath>
#include <cstdint>
#include <mutex>
#include <new>
#include <vector>

#include "dit.h"
#include "kernels.h"

using namespace dit;

namespace dit {
LaunchTiming &launch_timing() {
  static thread_local LaunchTiming t;
  return t;
}
}  // namespace dit

namespace {

constexpr size_t WS_ALIGN = 256;

size_t round_up(size_t v, size_t a) { return (v + a - 1) / a * a; }

// Workspace plan: every buffer the step needs, at 256-byte aligned offsets.
struct Plan {
  int64_t S, S_pad, L_pad, P, D, F, H, d;
  int64_t NB;  // sequences the activation buffers hold: 2 with guidance, else 1
  size_t es;  // element size
  // kc, vct hold the cross K / V^T of every block: [B][L_max][D], [B][D][L_pad];
  // gtab is a device table of weight pointers: ckv_w[0..B), ckv_b[0..B) (the
  // grouped cross K/V projection), table[0..B) (per-block modulation tables),
  // then the two rows of the head table
  size_t cos_t, sin_t, x, y, q, k, vt, o, h, c, kc, vct, patches, u, h1, temb, e, bmod, hmod,
      gtab;
  // layerwise offload: every block's modulation table stays resident; the
  // other block weights stream through two slots, field f of a slot at
  // slot[s] + wofs[f] (fields in dit_block_weights order; table unused)
  size_t tables, slot[2], wofs[15], wbytes[15];
  // block caching across steps (float, NB S D elements each): h_0 and then
  // h_fn of the current step, the probes of the current and the reference
  // step (two buffers that swap roles), three Taylor factors of the middle
  // residual, and the probe's per-workgroup partial sums (double)
  size_t ch0, cprobe[2], ctf, cpart;
  size_t total;
};

// Elements of each dit_block_weights field, in declaration order.
void block_field_elems(const dit_config &c, int64_t n[15]) {
  const int64_t D = c.hidden, F = c.mlp_hidden;
  const int64_t v[15] = {6 * D, 3 * D * D, 3 * D, D * D, D, D * D, D, 2 * D * D, 2 * D,
                         D * D, D, F * D, F, D * F, D};
  for (int i = 0; i < 15; ++i) n[i] = v[i];
}

bool plan_layout(const dit_config &c, Plan &p) {
  p.es = c.dtype == DIT_BF16 ? 2 : 4;
  p.D = c.hidden;
  p.F = c.mlp_hidden;
  p.H = c.heads;
  p.d = c.head_dim;
  p.S = (int64_t)(c.lat_f / c.patch_f) * (c.lat_h / c.patch_h) * (c.lat_w / c.patch_w);
  p.S_pad = (int64_t)round_up((size_t)p.S, 64);
  p.L_pad = (int64_t)round_up((size_t)c.ctx_len_max, 64);
  p.P = (int64_t)c.in_channels * c.patch_f * c.patch_h * c.patch_w;
  p.NB = c.guidance ? 2 : 1;
  size_t off = 0;
  auto take = [&](size_t bytes) {
    size_t at = off;
    off = round_up(off + bytes, WS_ALIGN);
    return at;
  };
  const size_t f4 = 4, es = p.es, NB = (size_t)p.NB;
  // sequences stacked: rows [n S, (n+1) S) of x, y, q, k, o, h, u are sequence
  // n; vt columns [n S_pad, (n+1) S_pad); c, kc, vct hold context n at n times
  // their one-context size
  p.cos_t = take(f4 * p.S * (p.d / 2));
  p.sin_t = take(f4 * p.S * (p.d / 2));
  p.x = take(f4 * NB * p.S * p.D);
  p.y = take(es * NB * p.S * p.D);
  p.q = take(es * NB * p.S * p.D);
  p.k = take(es * NB * p.S * p.D);
  p.vt = take(es * p.D * NB * p.S_pad);
  p.o = take(es * NB * p.S * p.D);
  p.h = take(es * NB * p.S * p.F);
  p.c = take(es * NB * (size_t)c.ctx_len_max * p.D);
  p.kc = take(es * NB * (size_t)c.num_blocks * c.ctx_len_max * p.D);
  p.vct = take(es * NB * (size_t)c.num_blocks * p.D * p.L_pad);
  p.patches = take(es * p.S * p.P);
  p.u = take(f4 * NB * p.S * p.P);
  p.h1 = take(f4 * p.D);
  p.temb = take(f4 * p.D);
  p.e = take(f4 * 6 * p.D);
  p.bmod = take(f4 * 6 * p.D * c.num_blocks);
  p.hmod = take(f4 * 2 * p.D);
  p.gtab = take(sizeof(void *) * (3 * (size_t)c.num_blocks + 2));
  p.tables = p.slot[0] = p.slot[1] = 0;
  if (c.offload) {
    p.tables = take(es * (size_t)c.num_blocks * 6 * p.D);
    int64_t n[15];
    block_field_elems(c, n);
    size_t sb = 0;
    for (int f = 0; f < 15; ++f) {
      p.wbytes[f] = es * (size_t)n[f];
      p.wofs[f] = sb;
      if (f > 0) sb = round_up(sb + p.wbytes[f], WS_ALIGN);  // field 0 (table) stays resident
    }
    p.slot[0] = take(sb);
    p.slot[1] = take(sb);
  }
  p.ch0 = p.cprobe[0] = p.cprobe[1] = p.ctf = p.cpart = 0;
  if (c.cache) {
    const size_t n = f4 * NB * p.S * p.D;
    p.ch0 = take(n);
    p.cprobe[0] = take(n);
    p.cprobe[1] = take(n);
    p.ctf = take(3 * n);
    p.cpart = take(2 * sizeof(double) * CACHE_PROBE_MAX_WG);
  }
  p.total = off;
  return true;
}

// The attention kernel addresses keys and transposed values through buffer
// resources with 32-bit byte offsets and ranges: every key row of the last
// (partial) 64-key tile and the whole value matrix must lie below 2^31 bytes.
bool attention_offsets_fit(int64_t es, int64_t D, int64_t sk, int64_t ldk, int64_t ldv) {
  const int64_t lim = (int64_t)1 << 31;
  return ((sk + 63) / 64 * 64 + 64) * ldk * es < lim && D * ldv * es < lim;
}

dit_status check_config(const dit_config *c) {
  if (!c) return DIT_ERR_INVALID_ARG;
  if (c->dtype != DIT_F32 && c->dtype != DIT_BF16) return DIT_ERR_INVALID_ARG;
  const int32_t pos[] = {c->num_blocks, c->hidden,  c->heads,   c->head_dim, c->mlp_hidden,
                         c->freq_dim,   c->in_channels, c->patch_f, c->patch_h, c->patch_w,
                         c->lat_f,      c->lat_h,   c->lat_w,   c->ctx_len_max, c->text_dim};
  for (int32_t v : pos)
    if (v <= 0) return DIT_ERR_SHAPE;
  if (c->rope_f < 0 || c->rope_h < 0 || c->rope_w < 0) return DIT_ERR_SHAPE;
  if (!(c->ln_eps > 0.0f) || !(c->rope_theta > 0.0f)) return DIT_ERR_INVALID_ARG;
  if ((int64_t)c->heads * c->head_dim != c->hidden) return DIT_ERR_SHAPE;
  if (c->lat_f % c->patch_f || c->lat_h % c->patch_h || c->lat_w % c->patch_w) return DIT_ERR_SHAPE;
  if ((c->rope_f | c->rope_h | c->rope_w) & 1) return DIT_ERR_SHAPE;
  if (c->rope_f + c->rope_h + c->rope_w != c->head_dim) return DIT_ERR_SHAPE;
  if (c->freq_dim & 1) return DIT_ERR_SHAPE;
  if (c->head_dim != 32 && c->head_dim != 64 && c->head_dim != 128) return DIT_ERR_UNSUPPORTED;
  // 16-byte vector moves along every contracted dimension and row.
  const int64_t P = (int64_t)c->in_channels * c->patch_f * c->patch_h * c->patch_w;
  if (c->hidden % 8 || c->mlp_hidden % 8 || c->text_dim % 8 || c->freq_dim % 8 || P % 8)
    return DIT_ERR_UNSUPPORTED;
  // the LayerNorm keeps a row in registers (at most 5120 wide)
  if (c->hidden > 5120 || c->freq_dim > 8192) return DIT_ERR_UNSUPPORTED;
  const int64_t S = (int64_t)(c->lat_f / c->patch_f) * (c->lat_h / c->patch_h) *
                    (c->lat_w / c->patch_w);
  if (S > (int64_t)1 << 30) return DIT_ERR_UNSUPPORTED;
  if (c->guidance != 0 && c->guidance != 1) return DIT_ERR_INVALID_ARG;
  if (c->offload != 0 && c->offload != 1) return DIT_ERR_INVALID_ARG;
  if (c->cache != 0 && c->cache != 1) return DIT_ERR_INVALID_ARG;
  // guided steps stack two sequences; the transposed values are written in
  // runs of 8 rows, which must not straddle them
  if (c->guidance && S % 8) return DIT_ERR_UNSUPPORTED;
  const int64_t rows = c->guidance ? 2 * S : S;
  const DType dt = c->dtype == DIT_BF16 ? DT_BF16 : DT_F32;
  // every projection of the step: activations [rows, D | F | P] and weights
  // with up to max(3D, F) rows of width D or F; the context projection's
  // [L, text_dim] and [D, text_dim]
  const int64_t wide = std::max<int64_t>(std::max<int64_t>(c->hidden, c->mlp_hidden), P);
  const int64_t wrows = std::max<int64_t>(3 * (int64_t)c->hidden, c->mlp_hidden);
  if (!gemm_offsets_fit(dt, rows, wide, wrows, std::max(c->hidden, c->mlp_hidden)) ||
      !gemm_offsets_fit(dt, c->ctx_len_max, std::max(c->text_dim, c->hidden),
                        std::max(c->hidden, c->mlp_hidden), c->text_dim))
    return DIT_ERR_UNSUPPORTED;
  // self-attention keys [S, D] and values [D, S_pad per sequence]; cross keys
  // [L, D] and values [D, L_pad per context]
  const int64_t es = dt == DT_BF16 ? 2 : 4, seqs = c->guidance ? 2 : 1;
  if (!attention_offsets_fit(es, c->hidden, S, c->hidden, seqs * (int64_t)round_up((size_t)S, 64)) ||
      !attention_offsets_fit(es, c->hidden, c->ctx_len_max, c->hidden,
                             seqs * (int64_t)round_up((size_t)c->ctx_len_max, 64)))
    return DIT_ERR_UNSUPPORTED;
  return DIT_OK;
}

bool aligned16(const void *p) { return ((uintptr_t)p & 15u) == 0; }
bool ok_ptr(const void *p) { return p != nullptr && aligned16(p); }

dit_status hip_status(hipError_t e) { return e == hipSuccess ? DIT_OK : DIT_ERR_HIP; }

#define DIT_TRY(expr)                        \
  do {                                       \
    hipError_t _e = (expr);                  \
    if (_e != hipSuccess) return DIT_ERR_HIP; \
  } while (0)

// Launch `expr` (one kernel) on stream s; with profiling on, its launch
// records two events at the kernel's own start and end (dit_launch).  A
// launcher that enqueued no kernel leaves them pending: they are then
// recorded back to back, a zero-length interval.
#define DIT_RUN(m, kind, s, expr)                                        \
  do {                                                                   \
    if ((m)->prof.on) {                                                  \
      hipEvent_t _e0 = (m)->prof.get(), _e1 = (m)->prof.get();           \
      if (!_e0 || !_e1) return DIT_ERR_HIP;                              \
      launch_timing() = LaunchTiming{_e0, _e1};                          \
      const hipError_t _r = (expr);                                      \
      const bool _pending = launch_timing().start != nullptr;            \
      launch_timing() = LaunchTiming{};                                  \
      DIT_TRY(_r);                                                       \
      if (_pending) {                                                    \
        DIT_TRY(hipEventRecord(_e0, s));                                 \
        DIT_TRY(hipEventRecord(_e1, s));                                 \
      }                                                                  \
      (m)->prof.recs.push_back({(int)(kind), (m)->prof.next - 2});       \
    } else {                                                             \
      DIT_TRY(expr);                                                     \
    }                                                                    \
  } while (0)

// Kinds of timed launches (dit_profile_* report per kind).
enum ProfKind {
  PK_LN = 0, PK_GEMM_QKV, PK_ATTN_SELF, PK_GEMM_O, PK_GEMM_CQ, PK_GEMM_CKV,
  PK_ATTN_CROSS, PK_GEMM_CO, PK_GEMM_MLP1, PK_GEMM_MLP2, PK_TIME, PK_GEMM_TXT, PK_PATCHIFY,
  PK_GEMM_PE, PK_GEMM_OUT, PK_EULER, PK_CACHE_PROBE, PK_CACHE_APPLY, PK_CACHE_UPDATE, PK_COUNT
};
const char *const kProfNames[PK_COUNT] = {
    "layernorm_modulate", "gemm_qkv_rope", "attention_self", "gemm_o", "gemm_cross_q",
    "gemm_cross_kv", "attention_cross", "gemm_cross_o", "gemm_mlp1_gelu", "gemm_mlp2",
    "time_embedding", "gemm_text_proj", "patchify", "gemm_patch_embed", "gemm_head",
    "unpatchify_euler", "cache_probe", "cache_apply", "cache_update"};

// Optional per-launch timing: a start and an end event recorded on the launch
// stream around each kernel.  Events are created on demand and reused.
struct Profiler {
  bool on = false;
  std::vector<hipEvent_t> events;
  size_t next = 0;
  std::vector<std::pair<int, size_t>> recs;  // (kind, index of the start event)
  hipEvent_t get() {
    if (next == events.size()) {
      hipEvent_t e;
      if (hipEventCreate(&e) != hipSuccess) return nullptr;
      events.push_back(e);
    }
    return events[next++];
  }
  ~Profiler() {
    for (hipEvent_t e : events) (void)hipEventDestroy(e);
  }
};

}  // namespace

struct dit_model {
  dit_config cfg{};
  DType dt = DT_F32;
  dit_global_weights g{};                 // unused by block calls made without a handle
  std::vector<dit_block_weights> blocks;  // device pointers, or host ones with offload
  char *ws = nullptr;
  Plan plan;
  Profiler prof;
  // layerwise offload: block copies run on their own stream; ready[s] marks
  // slot s filled, freed[s] the end of the last block that read it
  hipStream_t copy_stream = nullptr;
  hipEvent_t ready[2] = {nullptr, nullptr}, freed[2] = {nullptr, nullptr};
  // block caching: the knobs and decision state of the current run (valid
  // while cache_ok), the probe buffer holding the reference, the sequence
  // count of the run, and host room for the probe's partial sums
  dit_cache_params cache_params{};
  dit_cache_state cache_state{};
  bool cache_ok = false;
  int cache_ref = 0, cache_nb = 0;
  std::vector<double> cache_part;
  template <typename U> U *buf(size_t off) const { return reinterpret_cast<U *>(ws + off); }
  ~dit_model() {
    for (int i = 0; i < 2; ++i) {
      if (ready[i]) (void)hipEventDestroy(ready[i]);
      if (freed[i]) (void)hipEventDestroy(freed[i]);
    }
    if (copy_stream) (void)hipStreamDestroy(copy_stream);
  }
};

namespace {

dit_status check_global(const dit_config &c, const dit_global_weights &g) {
  const void *req[] = {g.t1_w, g.t1_b, g.t2_w, g.t2_b, g.mod_w, g.mod_b,
                       g.pe_w, g.pe_b, g.head_table, g.out_w, g.out_b};
  for (const void *p : req)
    if (!ok_ptr(p)) return DIT_ERR_INVALID_ARG;
  if (c.text_dim != c.hidden && (!ok_ptr(g.txt_w) || !ok_ptr(g.txt_b))) return DIT_ERR_INVALID_ARG;
  return DIT_OK;
}

dit_status check_block(const dit_block_weights &b) {
  const void *req[] = {b.table, b.qkv_w, b.qkv_b, b.o_w, b.o_b, b.cq_w, b.cq_b, b.ckv_w,
                       b.ckv_b, b.co_w,  b.co_b,  b.w1,  b.b1,  b.w2,   b.b2};
  for (const void *p : req)
    if (!ok_ptr(p)) return DIT_ERR_INVALID_ARG;
  return DIT_OK;
}

GemmArgs gemm(const void *A, int64_t lda, const void *W, int64_t ldw, int M, int N, int K,
              const void *bias) {
  GemmArgs a{};
  a.A = A;
  a.lda = lda;
  a.W = W;
  a.ldw = ldw;
  a.M = M;
  a.N = N;
  a.K = K;
  a.bias = bias;
  return a;
}

// One block (weights w, device pointers) on the residual stream x [nb S, D]
// (nb stacked sequences sharing the modulation) with the projected contexts
// ctx[n] [L, D], whose cross K / V^T this block computes into slot n of kc /
// vct, or, with ckv_ready, finds there already.
dit_status run_block(dit_model *m, const dit_block_weights &w, int b, float *x,
                     const void *const *ctx, int L, const float *mod, hipStream_t s,
                     bool ckv_ready, int nb) {
  const dit_config &c = m->cfg;
  const Plan &p = m->plan;
  const int S = (int)p.S, D = (int)p.D, F = (int)p.F, R = nb * S;
  const int B = c.num_blocks;
  void *y = m->buf<void>(p.y), *q = m->buf<void>(p.q), *k = m->buf<void>(p.k);
  void *vt = m->buf<void>(p.vt), *o = m->buf<void>(p.o), *h = m->buf<void>(p.h);
  // this block's cross K / V^T slots (context 0; context n at n * ctx_k / ctx_v)
  void *kc = m->buf<char>(p.kc) + p.es * (size_t)b * c.ctx_len_max * p.D;
  void *vct = m->buf<char>(p.vct) + p.es * (size_t)b * p.D * p.L_pad;
  const int64_t ctx_k = (int64_t)B * c.ctx_len_max * D, ctx_v = (int64_t)B * D * p.L_pad;
  const int64_t vt_ld = nb * p.S_pad;  // the sequences' values side by side
  const float scale_log2 = (float)(1.4426950408889634 / std::sqrt((double)c.head_dim));

  // self-attention branch: y = LN(x)(1 + scale_a) + shift_a
  DIT_RUN(m, PK_LN, s, launch_ln_modulate(m->dt, x, R, D, c.ln_eps, mod + 0 * D, mod + 1 * D, y, s));
  {
    GemmArgs a = gemm(y, D, w.qkv_w, D, R, 3 * D, D, w.qkv_b);
    a.seg_width = D;
    a.seg_ptr[0] = q; a.seg_ld[0] = D; a.seg_trans[0] = 0;
    a.seg_ptr[1] = k; a.seg_ld[1] = D; a.seg_trans[1] = 0;
    a.seg_ptr[2] = vt; a.seg_ld[2] = vt_ld; a.seg_trans[2] = 1;
    // RoPE on q and k inside the projection's epilogue
    a.seg_rope[0] = 1; a.seg_rope[1] = 1;
    a.rope_cos = m->buf<float>(p.cos_t); a.rope_sin = m->buf<float>(p.sin_t);
    a.rope_half_d = c.head_dim / 2;
    if (nb > 1) {
      a.seg_rows = S;
      a.seg_bstride = p.S_pad;
    }
    DIT_RUN(m, PK_GEMM_QKV, s, launch_gemm(m->dt, EPI_SPLIT, a, s));
  }
  {
    AttnArgs a{q, D, k, D, vt, vt_ld, o, D, S, S, c.heads, c.head_dim, scale_log2};
    a.batch = nb;
    a.bq = a.bk = a.bo = (int64_t)S * D;
    a.bvt = p.S_pad;
    DIT_RUN(m, PK_ATTN_SELF, s, launch_attention(m->dt, a, s));
  }
  {
    GemmArgs a = gemm(o, D, w.o_w, D, R, D, D, w.o_b);
    a.out = x; a.ldo = D; a.gate = mod + 2 * D;
    DIT_RUN(m, PK_GEMM_O, s, launch_gemm(m->dt, EPI_RESIDUAL, a, s));
  }
  // cross-attention branch (plain LN, ungated)
  DIT_RUN(m, PK_LN, s, launch_ln_modulate(m->dt, x, R, D, c.ln_eps, nullptr, nullptr, y, s));
  {
    GemmArgs a = gemm(y, D, w.cq_w, D, R, D, D, w.cq_b);
    a.out = q; a.ldo = D;
    DIT_RUN(m, PK_GEMM_CQ, s, launch_gemm(m->dt, EPI_STORE, a, s));
  }
  for (int n = 0; n < nb && !ckv_ready; ++n) {
    GemmArgs a = gemm(ctx[n], D, w.ckv_w, D, L, 2 * D, D, w.ckv_b);
    a.seg_width = D;
    a.seg_ptr[0] = static_cast<char *>(kc) + p.es * n * ctx_k;
    a.seg_ld[0] = D; a.seg_trans[0] = 0;
    a.seg_ptr[1] = static_cast<char *>(vct) + p.es * n * ctx_v;
    a.seg_ld[1] = p.L_pad; a.seg_trans[1] = 1;
    DIT_RUN(m, PK_GEMM_CKV, s, launch_gemm(m->dt, EPI_SPLIT, a, s));
  }
  {
    AttnArgs a{q, D, kc, D, vct, p.L_pad, o, D, S, L, c.heads, c.head_dim, scale_log2};
    a.batch = nb;
    a.bq = a.bo = (int64_t)S * D;
    a.bk = ctx_k;
    a.bvt = ctx_v;
    DIT_RUN(m, PK_ATTN_CROSS, s, launch_attention(m->dt, a, s));
  }
  {
    GemmArgs a = gemm(o, D, w.co_w, D, R, D, D, w.co_b);
    a.out = x; a.ldo = D; a.gate = nullptr;
    DIT_RUN(m, PK_GEMM_CO, s, launch_gemm(m->dt, EPI_RESIDUAL, a, s));
  }
  // MLP branch: y = LN(x)(1 + scale_f) + shift_f; x += gate_f * W2 gelu(W1 y + b1) + b2
  DIT_RUN(m, PK_LN, s, launch_ln_modulate(m->dt, x, R, D, c.ln_eps, mod + 3 * D, mod + 4 * D, y, s));
  {
    GemmArgs a = gemm(y, D, w.w1, D, R, F, D, w.b1);
    a.out = h; a.ldo = F;
    DIT_RUN(m, PK_GEMM_MLP1, s, launch_gemm(m->dt, EPI_GELU, a, s));
  }
  {
    GemmArgs a = gemm(h, F, w.w2, F, R, D, F, w.b2);
    a.out = x; a.ldo = D; a.gate = mod + 5 * D;
    DIT_RUN(m, PK_GEMM_MLP2, s, launch_gemm(m->dt, EPI_RESIDUAL, a, s));
  }
  return DIT_OK;
}

// Device view of block b's weights in offload slot `slot` (its modulation
// table from the resident copy).
dit_block_weights slot_weights(const dit_model *m, int slot, int b) {
  const Plan &p = m->plan;
  const void **f = nullptr;
  dit_block_weights w{};
  f = reinterpret_cast<const void **>(&w);
  char *base = m->ws + p.slot[slot];
  for (int i = 1; i < 15; ++i) f[i] = base + p.wofs[i];
  f[0] = m->ws + p.tables + p.es * (size_t)b * 6 * p.D;
  return w;
}

// Block b's weights (pinned host memory) into slot `slot` on stream cs; the
// caller orders cs after the slot's previous reader.  Fields that sit in host
// memory exactly as in the slot (each at the previous one's offset plus the
// distance between their slot offsets) go over in one transfer.
hipError_t copy_block(const dit_model *m, int b, int slot, hipStream_t cs) {
  const Plan &p = m->plan;
  const char *const *src = reinterpret_cast<const char *const *>(&m->blocks[b]);
  char *base = m->ws + p.slot[slot];
  for (int i = 1; i < 15;) {
    int j = i + 1;
    while (j < 15 && src[j] == src[i] + (p.wofs[j] - p.wofs[i])) ++j;
    const size_t n = p.wofs[j - 1] + p.wbytes[j - 1] - p.wofs[i];
    hipError_t e = hipMemcpyAsync(base + p.wofs[i], src[i], n, hipMemcpyHostToDevice, cs);
    if (e != hipSuccess) return e;
    i = j;
  }
  return hipSuccess;
}

dit_status run_time_path(dit_model *m, float t, float *bmod, float *hmod, float *temb,
                         hipStream_t s) {
  const dit_config &c = m->cfg;
  const Plan &p = m->plan;
  const int D = (int)p.D;
  float *h1 = m->buf<float>(p.h1), *e = m->buf<float>(p.e);
  const void *const *tab = m->buf<const void *>(p.gtab);
  const int B = c.num_blocks;
  // h1 = W1 sinusoid(t) + b1 (sinusoid formed inside the launch)
  DIT_RUN(m, PK_TIME, s, launch_gemv(m->dt, m->g.t1_w, m->g.t1_b, nullptr, t, h1, D, c.freq_dim,
                                     false, nullptr, 0, nullptr, s));
  // temb = W2 SiLU(h1) + b2; head modulation = head table rows + temb
  DIT_RUN(m, PK_TIME, s, launch_gemv(m->dt, m->g.t2_w, m->g.t2_b, h1, 0.0f, temb, D, D, true,
                                     tab + 3 * B, 2, hmod, s));
  // e = Wm SiLU(temb) + bm; block b modulation = table_b + e
  DIT_RUN(m, PK_TIME, s, launch_gemv(m->dt, m->g.mod_w, m->g.mod_b, temb, 0.0f, e, 6 * D, D, true,
                                     tab + 2 * B, B, bmod, s));
  return DIT_OK;
}

}  // namespace

extern "C" {

dit_status dit_workspace_size(const dit_config *cfg, size_t *bytes) {
  if (!bytes) return DIT_ERR_INVALID_ARG;
  *bytes = 0;
  dit_status st = check_config(cfg);
  if (st != DIT_OK) return st;
  Plan p;
  plan_layout(*cfg, p);
  *bytes = p.total;
  return DIT_OK;
}

dit_status dit_create(const dit_config *cfg, const dit_weights *weights, void *workspace,
                      size_t workspace_bytes, void *stream, dit_model **out) {
  if (!out) return DIT_ERR_INVALID_ARG;
  *out = nullptr;
  dit_status st = check_config(cfg);
  if (st != DIT_OK) return st;
  if (!weights || !weights->blocks) return DIT_ERR_INVALID_ARG;
  if ((st = check_global(*cfg, weights->global)) != DIT_OK) return st;
  for (int b = 0; b < cfg->num_blocks; ++b)
    if ((st = check_block(weights->blocks[b])) != DIT_OK) return st;
  if (!workspace || ((uintptr_t)workspace & (WS_ALIGN - 1))) return DIT_ERR_INVALID_ARG;
  Plan p;
  plan_layout(*cfg, p);
  if (workspace_bytes < p.total) return DIT_ERR_WORKSPACE;

  dit_model *m = new (std::nothrow) dit_model;
  if (!m) return DIT_ERR_INVALID_ARG;
  m->cfg = *cfg;
  m->dt = cfg->dtype == DIT_BF16 ? DT_BF16 : DT_F32;
  m->g = weights->global;
  m->blocks.assign(weights->blocks, weights->blocks + cfg->num_blocks);
  m->ws = static_cast<char *>(workspace);
  m->plan = p;
  hipStream_t s = static_cast<hipStream_t>(stream);
  // device table of the per-block cross K/V weights and biases (grouped launch)
  const int B = cfg->num_blocks;
  std::vector<const void *> tab(3 * (size_t)B + 2);
  for (int b = 0; b < B; ++b) {
    // with offload the block weights are host pointers: no grouped cross K/V,
    // and the modulation tables are read from their resident copies
    tab[b] = cfg->offload ? nullptr : weights->blocks[b].ckv_w;
    tab[B + b] = cfg->offload ? nullptr : weights->blocks[b].ckv_b;
    tab[2 * B + b] = cfg->offload ? m->ws + p.tables + p.es * (size_t)b * 6 * cfg->hidden
                                  : weights->blocks[b].table;
  }
  const size_t es = cfg->dtype == DIT_BF16 ? 2 : 4;
  tab[3 * B] = weights->global.head_table;
  tab[3 * B + 1] = static_cast<const char *>(weights->global.head_table) + es * cfg->hidden;
  hipError_t e = hipMemcpyAsync(m->ws + p.gtab, tab.data(), tab.size() * sizeof(void *),
                                hipMemcpyHostToDevice, s);
  if (cfg->offload) {
    for (int b = 0; b < B && e == hipSuccess; ++b)
      e = hipMemcpyAsync(m->ws + p.tables + p.es * (size_t)b * 6 * cfg->hidden,
                         weights->blocks[b].table, p.es * 6 * (size_t)cfg->hidden,
                         hipMemcpyHostToDevice, s);
    if (e == hipSuccess) e = hipStreamCreateWithFlags(&m->copy_stream, hipStreamNonBlocking);
    for (int i = 0; i < 2 && e == hipSuccess; ++i) {
      e = hipEventCreateWithFlags(&m->ready[i], hipEventDisableTiming);
      if (e == hipSuccess) e = hipEventCreateWithFlags(&m->freed[i], hipEventDisableTiming);
    }
  }
  if (e == hipSuccess) e = hipStreamSynchronize(s);  // `tab` is released on return
  if (e == hipSuccess)
    e = launch_rope_tables(m->buf<float>(p.cos_t), m->buf<float>(p.sin_t),
                                    cfg->lat_f / cfg->patch_f, cfg->lat_h / cfg->patch_h,
                                    cfg->lat_w / cfg->patch_w, cfg->head_dim, cfg->rope_f,
                                    cfg->rope_h, cfg->rope_w, cfg->rope_theta, s);
  if (e != hipSuccess) {
    delete m;
    return DIT_ERR_HIP;
  }
  *out = m;
  return DIT_OK;
}

dit_status dit_destroy(dit_model *model) {
  delete model;
  return DIT_OK;
}

}  // extern "C"

namespace {

// Library-owned scratch of dit_block_forward_static, one copy per device (the
// code object's own global).  In host code `scratch` names a host-side stand-in,
// never the device memory: kernels and copies get the address that
// hipGetSymbolAddress returns for the current device, kept in scratch_ptr.
static __device__ __align__(256) unsigned char scratch[DIT_STATIC_SCRATCH_BYTES];
constexpr int kMaxDevices = 64;
std::mutex scratch_mutex;
void *scratch_ptr[kMaxDevices] = {};

// The device address of the scratch array on the current device, looked up
// once per device with that device current; nullptr on failure.
void *scratch_on_current_device() {
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return nullptr;
  std::lock_guard<std::mutex> lock(scratch_mutex);
  if (!scratch_ptr[dev]) {
    void *ptr = nullptr;
    if (hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch)) != hipSuccess || !ptr) return nullptr;
    scratch_ptr[dev] = ptr;
  }
  return scratch_ptr[dev];
}

}  // namespace

extern "C" {

dit_status dit_block_forward_static(const dit_config *cfg, const dit_block_weights *w, float *x,
                                    const void *ctx, int32_t ctx_len, const float *mod,
                                    void *stream) {
  dit_status st = check_config(cfg);
  if (st != DIT_OK) return st;
  if (cfg->guidance || cfg->offload || cfg->cache) return DIT_ERR_UNSUPPORTED;
  if (!w || !ok_ptr(x) || !ok_ptr(ctx) || !ok_ptr(mod)) return DIT_ERR_INVALID_ARG;
  if ((st = check_block(*w)) != DIT_OK) return st;
  if (ctx_len < 1 || ctx_len > cfg->ctx_len_max) return DIT_ERR_SHAPE;
  // the plan of a one-block model: rotary tables, activations, one block's
  // cross K / V^T
  dit_config one = *cfg;
  one.num_blocks = 1;
  Plan p;
  plan_layout(one, p);
  if (p.total > DIT_STATIC_SCRATCH_BYTES) return DIT_ERR_WORKSPACE;
  char *ws = static_cast<char *>(scratch_on_current_device());
  if (!ws) return DIT_ERR_HIP;
  // a handle on the stack: no heap memory, profiling off, no offload or cache
  dit_model m;
  m.cfg = one;
  m.dt = one.dtype == DIT_BF16 ? DT_BF16 : DT_F32;
  m.ws = ws;
  m.plan = p;
  hipStream_t s = static_cast<hipStream_t>(stream);
  DIT_TRY(launch_rope_tables(m.buf<float>(p.cos_t), m.buf<float>(p.sin_t),
                             one.lat_f / one.patch_f, one.lat_h / one.patch_h,
                             one.lat_w / one.patch_w, one.head_dim, one.rope_f, one.rope_h,
                             one.rope_w, one.rope_theta, s));
  const void *ctxs[1] = {ctx};
  return run_block(&m, *w, 0, x, ctxs, ctx_len, mod, s, false, 1);
}

dit_status dit_block_forward(dit_model *m, int32_t block, float *x, const void *ctx,
                             int32_t ctx_len, const float *mod, void *stream) {
  if (!m || !ok_ptr(x) || !ok_ptr(ctx) || !ok_ptr(mod)) return DIT_ERR_INVALID_ARG;
  if (block < 0 || block >= m->cfg.num_blocks) return DIT_ERR_SHAPE;
  if (ctx_len < 1 || ctx_len > m->cfg.ctx_len_max) return DIT_ERR_SHAPE;
  hipStream_t s = static_cast<hipStream_t>(stream);
  const void *ctxs[1] = {ctx};
  if (!m->cfg.offload) return run_block(m, m->blocks[block], block, x, ctxs, ctx_len, mod, s, false, 1);
  // offload: the block's weights into slot 0 on the call's own stream first
  DIT_TRY(copy_block(m, block, 0, s));
  return run_block(m, slot_weights(m, 0, block), block, x, ctxs, ctx_len, mod, s, false, 1);
}

}  // extern "C"

namespace {

// The start of a denoise step over nb sequences that share the latents X and
// the timestep and differ in their context ctx[n]: time path, context
// projection (cproj[n] receives where sequence n's projected context sits),
// patch embedding into every sequence's rows of x, and the cross K / V^T of
// every block.  nb = 2 is the guided step: sequence 0 takes the positive
// embeddings, 1 the negative ones.
dit_status step_prologue(dit_model *m, float *X, const void *const *ctx, int nb, int ctx_len,
                         float t, const void **cproj, hipStream_t s) {
  const dit_config &c = m->cfg;
  const Plan &p = m->plan;
  const int S = (int)p.S, D = (int)p.D, P = (int)p.P, B = c.num_blocks;
  float *x = m->buf<float>(p.x);
  dit_status st = run_time_path(m, t, m->buf<float>(p.bmod), m->buf<float>(p.hmod),
                                m->buf<float>(p.temb), s);
  if (st != DIT_OK) return st;

  // projected context n at c + n * L_max * D (or the caller's tokens)
  cproj[0] = ctx[0];
  cproj[1] = nb > 1 ? ctx[1] : nullptr;
  if (c.text_dim != c.hidden) {
    for (int n = 0; n < nb; ++n) {
      void *cn = m->buf<char>(p.c) + p.es * (size_t)n * c.ctx_len_max * D;
      GemmArgs a = gemm(ctx[n], c.text_dim, m->g.txt_w, c.text_dim, ctx_len, D, c.text_dim,
                        m->g.txt_b);
      a.out = cn;
      a.ldo = D;
      DIT_RUN(m, PK_GEMM_TXT, s, launch_gemm(m->dt, EPI_STORE, a, s));
      cproj[n] = cn;
    }
  }
  DIT_RUN(m, PK_PATCHIFY, s, launch_patchify(m->dt, X, m->buf<void>(p.patches), c.in_channels, c.lat_f, c.lat_h,
                          c.lat_w, c.patch_f, c.patch_h, c.patch_w, s));
  {
    GemmArgs a = gemm(m->buf<void>(p.patches), P, m->g.pe_w, P, S, D, P, m->g.pe_b);
    a.out = x;
    a.ldo = D;
    DIT_RUN(m, PK_GEMM_PE, s, launch_gemm(m->dt, EPI_STORE_F32, a, s));
  }
  // every sequence starts from the same embedded latents
  for (int n = 1; n < nb; ++n)
    DIT_TRY(hipMemcpyAsync(x + (size_t)n * S * D, x, sizeof(float) * (size_t)S * D,
                           hipMemcpyDeviceToDevice, s));
  // cross K / V^T of every block in one grouped launch per context: they
  // depend on the context only, not on the residual stream (with offload each
  // block computes its own from the streamed weights)
  for (int n = 0; n < nb && !c.offload; ++n) {
    GemmArgs a = gemm(cproj[n], D, nullptr, D, ctx_len, 2 * D, D, nullptr);
    a.seg_width = D;
    a.seg_ptr[0] = m->buf<char>(p.kc) + p.es * (size_t)n * B * c.ctx_len_max * D;
    a.seg_ld[0] = D; a.seg_trans[0] = 0;
    a.seg_ptr[1] = m->buf<char>(p.vct) + p.es * (size_t)n * B * D * p.L_pad;
    a.seg_ld[1] = p.L_pad; a.seg_trans[1] = 1;
    a.groups = B;
    a.gw = m->buf<const void *>(p.gtab);
    a.gbias = m->buf<const void *>(p.gtab) + B;
    a.seg_gstride[0] = (int64_t)c.ctx_len_max * D;
    a.seg_gstride[1] = (int64_t)D * p.L_pad;
    DIT_RUN(m, PK_GEMM_CKV, s, launch_gemm(m->dt, EPI_SPLIT, a, s));
  }
  return DIT_OK;
}

// Blocks [lo, hi) on the residual stream x of nb sequences.
dit_status run_blocks(dit_model *m, int lo, int hi, const void *const *cproj, int ctx_len,
                      hipStream_t s, int nb) {
  const Plan &p = m->plan;
  const int64_t D = p.D;
  float *x = m->buf<float>(p.x);
  const float *bmod = m->buf<float>(p.bmod);
  dit_status st = DIT_OK;
  if (!m->cfg.offload) {
    for (int b = lo; b < hi; ++b) {
      st = run_block(m, m->blocks[b], b, x, cproj, ctx_len, bmod + b * 6 * D, s, true, nb);
      if (st != DIT_OK) return st;
    }
    return DIT_OK;
  }
  // Layerwise offload: block lo + i runs from slot i & 1 while the next block
  // is copied into the other; the copy two blocks ahead waits for the end of
  // the block that last read its slot.  Both slots are free once the stream
  // reaches this point.
  hipStream_t cs = m->copy_stream;
  for (int k = 0; k < 2; ++k) DIT_TRY(hipEventRecord(m->freed[k], s));
  for (int i = 0; i < 2 && lo + i < hi; ++i) {
    DIT_TRY(hipStreamWaitEvent(cs, m->freed[i], 0));
    DIT_TRY(copy_block(m, lo + i, i, cs));
    DIT_TRY(hipEventRecord(m->ready[i], cs));
  }
  for (int b = lo; b < hi; ++b) {
    const int sl = (b - lo) & 1;
    DIT_TRY(hipStreamWaitEvent(s, m->ready[sl], 0));
    st = run_block(m, slot_weights(m, sl, b), b, x, cproj, ctx_len, bmod + b * 6 * D, s, false,
                   nb);
    if (st != DIT_OK) return st;
    if (b + 2 < hi) {
      DIT_TRY(hipEventRecord(m->freed[sl], s));
      DIT_TRY(hipStreamWaitEvent(cs, m->freed[sl], 0));
      DIT_TRY(copy_block(m, b + 2, sl, cs));
      DIT_TRY(hipEventRecord(m->ready[sl], cs));
    }
  }
  return DIT_OK;
}

// The end of a step: final layer on every sequence, then the Euler update with
// the velocity of sequence 0 or, for nb = 2, v_neg + g (v_pos - v_neg).
dit_status step_epilogue(dit_model *m, float *X, int nb, float sigma, float sigma_next, float g,
                         float *v_out, hipStream_t s) {
  const dit_config &c = m->cfg;
  const Plan &p = m->plan;
  const int S = (int)p.S, D = (int)p.D, P = (int)p.P, R = nb * S;
  float *hmod = m->buf<float>(p.hmod), *x = m->buf<float>(p.x), *u = m->buf<float>(p.u);
  DIT_RUN(m, PK_LN, s, launch_ln_modulate(m->dt, x, R, D, c.ln_eps, hmod, hmod + D, m->buf<void>(p.y), s));
  {
    GemmArgs a = gemm(m->buf<void>(p.y), D, m->g.out_w, D, R, P, D, m->g.out_b);
    a.out = u;
    a.ldo = P;
    DIT_RUN(m, PK_GEMM_OUT, s, launch_gemm(m->dt, EPI_STORE_F32, a, s));
  }
  DIT_RUN(m, PK_EULER, s, launch_unpatchify_euler(u, nb > 1 ? u + (size_t)S * P : nullptr, g, X, v_out,
                                  sigma_next - sigma, c.in_channels, c.lat_f, c.lat_h, c.lat_w,
                                  c.patch_f, c.patch_h, c.patch_w, s));
  return DIT_OK;
}

dit_status run_step(dit_model *m, float *X, const void *const *ctx, int nb, int ctx_len, float t,
                    float sigma, float sigma_next, float g, float *v_out, hipStream_t s) {
  const void *cproj[2];
  dit_status st = step_prologue(m, X, ctx, nb, ctx_len, t, cproj, s);
  if (st == DIT_OK) st = run_blocks(m, 0, m->cfg.num_blocks, cproj, ctx_len, s, nb);
  if (st == DIT_OK) st = step_epilogue(m, X, nb, sigma, sigma_next, g, v_out, s);
  return st;
}

// A step with block caching (the rules are stated with dit_cache_params).
// The first fn blocks run, then the probe kernel writes P = h_fn - h_0 and,
// when the step may reuse the cache, the partial sums of its difference to
// the reference probe, which the host reads back to decide.  A cached step
// adds the Taylor stand-in for the middle residual; a full step runs the
// middle blocks and refreshes the factors, and its probe becomes the
// reference.  The last bn blocks and the final layer always run.
dit_status run_step_cached(dit_model *m, float *X, const void *const *ctx, int nb, int ctx_len,
                           float t, float sigma, float sigma_next, float g, float *v_out,
                           hipStream_t s) {
  const Plan &p = m->plan;
  const dit_cache_params &cp = m->cache_params;
  dit_cache_state &cs = m->cache_state;
  const int B = m->cfg.num_blocks;
  const int64_t n = (int64_t)nb * p.S * p.D;
  float *x = m->buf<float>(p.x), *h0 = m->buf<float>(p.ch0), *tf = m->buf<float>(p.ctf);
  float *probe_ref = m->buf<float>(p.cprobe[m->cache_ref]);
  float *probe_cur = m->buf<float>(p.cprobe[1 - m->cache_ref]);
  double *part = m->buf<double>(p.cpart);
  m->cache_ok = false;  // until the step has been enqueued whole

  const void *cproj[2];
  dit_status st = step_prologue(m, X, ctx, nb, ctx_len, t, cproj, s);
  if (st != DIT_OK) return st;
  DIT_TRY(hipMemcpyAsync(h0, x, sizeof(float) * n, hipMemcpyDeviceToDevice, s));
  st = run_blocks(m, 0, cp.fn, cproj, ctx_len, s, nb);
  if (st != DIT_OK) return st;
  const bool eligible = cs.step >= cp.warmup && cs.factors >= 1 &&
                        cs.consecutive < cp.max_consecutive;
  DIT_RUN(m, PK_CACHE_PROBE, s,
          launch_cache_probe(x, h0, probe_cur, eligible ? probe_ref : nullptr, n, part, s));
  bool hit = false;
  double diff = -1.0;
  if (eligible) {
    const int G = cache_probe_groups(n);
    m->cache_part.resize(2 * (size_t)G);
    DIT_TRY(hipMemcpyAsync(m->cache_part.data(), part, 2 * sizeof(double) * G,
                           hipMemcpyDeviceToHost, s));
    DIT_TRY(hipStreamSynchronize(s));
    double num = 0.0, den = 0.0;
    for (int w = 0; w < G; ++w) {
      num += m->cache_part[2 * w];
      den += m->cache_part[2 * w + 1];
    }
    diff = den > 0.0 ? num / den : (num == 0.0 ? 0.0 : HUGE_VAL);
    hit = diff < (double)cp.rdt;
  }
  const int k = cs.step - cs.last_full;  // steps since the last full one
  const int order = cp.taylorseer ? cp.ts_order : 0;
  const int nnew = cs.factors + 1 < order + 1 ? cs.factors + 1 : order + 1;
  if (hit) {
    DIT_RUN(m, PK_CACHE_APPLY, s,
            launch_cache_apply(x, tf, n, cs.factors, (float)k, 0.5f * (float)k * (float)k, s));
  } else {
    st = run_blocks(m, cp.fn, B - cp.bn, cproj, ctx_len, s, nb);
    if (st != DIT_OK) return st;
    DIT_RUN(m, PK_CACHE_UPDATE, s, launch_cache_update(x, h0, tf, n, nnew, (float)k, s));
  }
  st = run_blocks(m, B - cp.bn, B, cproj, ctx_len, s, nb);
  if (st == DIT_OK) st = step_epilogue(m, X, nb, sigma, sigma_next, g, v_out, s);
  if (st != DIT_OK) return st;

  if (hit) {
    cs.consecutive += 1;
    cs.cached_total += 1;
  } else {
    cs.consecutive = 0;
    cs.last_full = cs.step;
    cs.factors = nnew;
    m->cache_ref = 1 - m->cache_ref;  // this step's probe is the new reference
  }
  cs.hit = hit ? 1 : 0;
  cs.diff = diff;
  cs.step += 1;
  m->cache_ok = true;
  return DIT_OK;
}

dit_status check_step(dit_model *m, float *X, int32_t ctx_len, float t, float sigma,
                      float sigma_next, float *v_out) {
  if (!m || !ok_ptr(X)) return DIT_ERR_INVALID_ARG;
  if (v_out && !aligned16(v_out)) return DIT_ERR_INVALID_ARG;
  if (!std::isfinite(t) || !std::isfinite(sigma) || !std::isfinite(sigma_next))
    return DIT_ERR_INVALID_ARG;
  if (ctx_len < 1 || ctx_len > m->cfg.ctx_len_max) return DIT_ERR_SHAPE;
  return DIT_OK;
}

}  // namespace

extern "C" {

dit_status dit_denoise_step(dit_model *m, float *X, const void *ctx, int32_t ctx_len, float t,
                            float sigma, float sigma_next, float *v_out, void *stream) {
  dit_status st = check_step(m, X, ctx_len, t, sigma, sigma_next, v_out);
  if (st != DIT_OK) return st;
  if (!ok_ptr(ctx)) return DIT_ERR_INVALID_ARG;
  const void *ctxs[1] = {ctx};
  return run_step(m, X, ctxs, 1, ctx_len, t, sigma, sigma_next, 1.0f, v_out,
                  static_cast<hipStream_t>(stream));
}

dit_status dit_denoise_step_cfg(dit_model *m, float *X, const void *ctx, const void *ctx_neg,
                                int32_t ctx_len, float t, float sigma, float sigma_next,
                                float guidance_scale, float *v_out, void *stream) {
  dit_status st = check_step(m, X, ctx_len, t, sigma, sigma_next, v_out);
  if (st != DIT_OK) return st;
  if (!ok_ptr(ctx) || !ok_ptr(ctx_neg) || !std::isfinite(guidance_scale))
    return DIT_ERR_INVALID_ARG;
  if (!m->cfg.guidance) return DIT_ERR_WORKSPACE;
  const void *ctxs[2] = {ctx, ctx_neg};
  return run_step(m, X, ctxs, 2, ctx_len, t, sigma, sigma_next, guidance_scale, v_out,
                  static_cast<hipStream_t>(stream));
}

dit_status dit_cache_begin(dit_model *m, const dit_cache_params *cp) {
  if (!m || !cp) return DIT_ERR_INVALID_ARG;
  if (!m->cfg.cache) return DIT_ERR_WORKSPACE;
  if (cp->warmup < 0 || cp->max_consecutive < 0 || !(cp->rdt >= 0.0f) ||
      (cp->taylorseer != 0 && cp->taylorseer != 1) || cp->ts_order < 0)
    return DIT_ERR_INVALID_ARG;
  if (cp->fn < 1 || cp->bn < 0 || (int64_t)cp->fn + cp->bn > m->cfg.num_blocks) return DIT_ERR_SHAPE;
  if (cp->taylorseer && cp->ts_order > 2) return DIT_ERR_UNSUPPORTED;
  m->cache_params = *cp;
  m->cache_state = dit_cache_state{};
  m->cache_state.last_full = -1;
  m->cache_state.diff = -1.0;
  m->cache_ref = 0;
  m->cache_nb = 0;
  m->cache_ok = true;
  return DIT_OK;
}

dit_status dit_cache_state_get(const dit_model *m, dit_cache_state *out) {
  if (!m || !out) return DIT_ERR_INVALID_ARG;
  if (!m->cfg.cache) return DIT_ERR_WORKSPACE;
  *out = m->cache_state;
  return DIT_OK;
}

dit_status dit_cache_factor_get(const dit_model *m, int32_t q, float *dst, void *stream) {
  if (!m || !ok_ptr(dst)) return DIT_ERR_INVALID_ARG;
  if (!m->cfg.cache) return DIT_ERR_WORKSPACE;
  if (m->cache_nb == 0 || q < 0 || q >= m->cache_state.factors) return DIT_ERR_SHAPE;
  const Plan &p = m->plan;
  const int64_t n = (int64_t)m->cache_nb * p.S * p.D;
  const float *tf = m->buf<float>(p.ctf);
  return hip_status(hipMemcpyAsync(dst, tf + q * n, sizeof(float) * n, hipMemcpyDeviceToDevice,
                                   static_cast<hipStream_t>(stream)));
}

dit_status dit_denoise_step_cached(dit_model *m, float *X, const void *ctx, const void *ctx_neg,
                                   int32_t ctx_len, float t, float sigma, float sigma_next,
                                   float guidance_scale, float *v_out, void *stream) {
  dit_status st = check_step(m, X, ctx_len, t, sigma, sigma_next, v_out);
  if (st != DIT_OK) return st;
  if (!ok_ptr(ctx) || (ctx_neg && !aligned16(ctx_neg)) || !std::isfinite(guidance_scale))
    return DIT_ERR_INVALID_ARG;
  if (!m->cfg.cache || (ctx_neg && !m->cfg.guidance)) return DIT_ERR_WORKSPACE;
  if (!m->cache_ok) return DIT_ERR_INVALID_ARG;  // no run begun, or the last step failed
  const int nb = ctx_neg ? 2 : 1;
  // the cached residuals are per sequence: one run keeps one sequence count
  if (m->cache_nb != 0 && m->cache_nb != nb) return DIT_ERR_SHAPE;
  m->cache_nb = nb;
  const void *ctxs[2] = {ctx, ctx_neg};
  return run_step_cached(m, X, ctxs, nb, ctx_len, t, sigma, sigma_next, guidance_scale, v_out,
                         static_cast<hipStream_t>(stream));
}

dit_status dit_euler_step(float *X, const float *v, int64_t n, float sigma, float sigma_next,
                          void *stream) {
  if (n < 0) return DIT_ERR_SHAPE;
  if (n == 0) return DIT_OK;
  if (!ok_ptr(X) || !ok_ptr(v)) return DIT_ERR_INVALID_ARG;
  if (!std::isfinite(sigma) || !std::isfinite(sigma_next)) return DIT_ERR_INVALID_ARG;
  return hip_status(launch_euler(X, v, n, sigma_next - sigma, static_cast<hipStream_t>(stream)));
}

dit_status dit_flow_sigmas(int32_t n_steps, double shift, double *sigmas) {
  if (!sigmas || !(shift > 0.0) || !std::isfinite(shift)) return DIT_ERR_INVALID_ARG;
  if (n_steps < 1) return DIT_ERR_SHAPE;
  for (int32_t k = 0; k <= n_steps; ++k) {
    const double s = 1.0 - (double)k / (double)n_steps;
    sigmas[k] = shift * s / (1.0 + (shift - 1.0) * s);
  }
  return DIT_OK;
}

dit_status dit_attention(int32_t dtype, int32_t heads, int32_t head_dim, const void *q,
                         int64_t ldq, const void *k, int64_t ldk, const void *vt, int64_t ldv,
                         void *o, int64_t ldo, int32_t sq, int32_t sk, void *stream) {
  if (dtype != DIT_F32 && dtype != DIT_BF16) return DIT_ERR_INVALID_ARG;
  if (!ok_ptr(q) || !ok_ptr(k) || !ok_ptr(vt) || !ok_ptr(o)) return DIT_ERR_INVALID_ARG;
  if (heads < 1 || sq < 1 || sk < 1) return DIT_ERR_SHAPE;
  if (head_dim != 32 && head_dim != 64 && head_dim != 128) return DIT_ERR_UNSUPPORTED;
  const int64_t D = (int64_t)heads * head_dim;
  if (ldq < D || ldk < D || ldo < D || ldv < (int64_t)round_up((size_t)sk, 64)) return DIT_ERR_SHAPE;
  if ((ldq | ldk | ldv | ldo) & 7) return DIT_ERR_INVALID_ARG;
  if (!attention_offsets_fit(dtype == DIT_BF16 ? 2 : 4, D, sk, ldk, ldv)) return DIT_ERR_UNSUPPORTED;
  const float scale_log2 = (float)(1.4426950408889634 / std::sqrt((double)head_dim));
  AttnArgs a{q, ldq, k, ldk, vt, ldv, o, ldo, sq, sk, heads, head_dim, scale_log2};
  return hip_status(launch_attention(dtype == DIT_BF16 ? DT_BF16 : DT_F32, a,
                                     static_cast<hipStream_t>(stream)));
}

dit_status dit_gemm(int32_t dtype, int32_t epilogue, const void *A, int64_t lda, const void *W,
                    int64_t ldw, int32_t M, int32_t N, int32_t K, const void *bias, void *out,
                    int64_t ldo, const float *gate, int32_t tile, void *stream) {
  if (dtype != DIT_F32 && dtype != DIT_BF16) return DIT_ERR_INVALID_ARG;
  if (epilogue < DIT_EPI_STORE || epilogue > DIT_EPI_STORE_F32) return DIT_ERR_INVALID_ARG;
  if (!ok_ptr(A) || !ok_ptr(W) || !ok_ptr(out)) return DIT_ERR_INVALID_ARG;
  if ((bias && !aligned16(bias)) || (gate && !aligned16(gate))) return DIT_ERR_INVALID_ARG;
  if (tile < 0 || tile > 5) return DIT_ERR_INVALID_ARG;
  if (M < 1 || N < 1 || K < 1 || lda < K || ldw < K || ldo < N) return DIT_ERR_SHAPE;
  if ((K | lda | ldw) & 7) return DIT_ERR_UNSUPPORTED;
  if (!gemm_offsets_fit(dtype == DIT_BF16 ? DT_BF16 : DT_F32, M, lda, N, ldw))
    return DIT_ERR_UNSUPPORTED;
  GemmArgs a = gemm(A, lda, W, ldw, M, N, K, bias);
  a.out = out;
  a.ldo = ldo;
  a.gate = gate;
  const Epilogue e = epilogue == DIT_EPI_STORE ? EPI_STORE
                     : epilogue == DIT_EPI_GELU ? EPI_GELU
                     : epilogue == DIT_EPI_RESIDUAL ? EPI_RESIDUAL : EPI_STORE_F32;
  return hip_status(launch_gemm(dtype == DIT_BF16 ? DT_BF16 : DT_F32, e, a,
                                static_cast<hipStream_t>(stream), tile));
}

dit_status dit_layernorm_modulate(int32_t dtype, int32_t D, float eps, const float *x,
                                  int32_t rows, const float *shift, const float *scale, void *y,
                                  void *stream) {
  if (dtype != DIT_F32 && dtype != DIT_BF16) return DIT_ERR_INVALID_ARG;
  if (!ok_ptr(x) || !ok_ptr(y)) return DIT_ERR_INVALID_ARG;
  if ((shift == nullptr) != (scale == nullptr)) return DIT_ERR_INVALID_ARG;
  if (shift && (!aligned16(shift) || !aligned16(scale))) return DIT_ERR_INVALID_ARG;
  if (!(eps > 0.0f)) return DIT_ERR_INVALID_ARG;
  if (rows < 0 || D < 4) return DIT_ERR_SHAPE;
  if (D % 4 || D > 5120) return DIT_ERR_UNSUPPORTED;
  return hip_status(launch_ln_modulate(dtype == DIT_BF16 ? DT_BF16 : DT_F32, x, rows, D, eps,
                                       shift, scale, y, static_cast<hipStream_t>(stream)));
}

dit_status dit_time_embedding(dit_model *m, float t, float *block_mod, float *head_mod,
                              float *temb, void *stream) {
  if (!m || !ok_ptr(block_mod) || !ok_ptr(head_mod) || !ok_ptr(temb)) return DIT_ERR_INVALID_ARG;
  if (!std::isfinite(t)) return DIT_ERR_INVALID_ARG;
  return run_time_path(m, t, block_mod, head_mod, temb, static_cast<hipStream_t>(stream));
}

dit_status dit_profile_enable(dit_model *m, int32_t enable) {
  if (!m) return DIT_ERR_INVALID_ARG;
  m->prof.on = enable != 0;
  if (m->prof.on) {
    m->prof.next = 0;
    m->prof.recs.clear();
  }
  return DIT_OK;
}

dit_status dit_profile_read(dit_model *m, int32_t kind, int64_t *launches, double *total_ms) {
  if (!m || !launches || !total_ms) return DIT_ERR_INVALID_ARG;
  if (kind < 0 || kind >= PK_COUNT) return DIT_ERR_SHAPE;
  int64_t n = 0;
  double ms = 0.0;
  for (const auto &r : m->prof.recs) {
    if (r.first != kind) continue;
    hipEvent_t e0 = m->prof.events[r.second], e1 = m->prof.events[r.second + 1];
    DIT_TRY(hipEventSynchronize(e1));
    float t = 0.0f;
    DIT_TRY(hipEventElapsedTime(&t, e0, e1));
    ms += t;
    ++n;
  }
  *launches = n;
  *total_ms = ms;
  return DIT_OK;
}

int32_t dit_profile_kind_count(void) { return PK_COUNT; }

const char *dit_profile_kind_name(int32_t kind) {
  return (kind >= 0 && kind < PK_COUNT) ? kProfNames[kind] : nullptr;
}

const char *dit_status_string(dit_status s) {
  switch (s) {
    case DIT_OK: return "DIT_OK";
    case DIT_ERR_INVALID_ARG: return "DIT_ERR_INVALID_ARG";
    case DIT_ERR_SHAPE: return "DIT_ERR_SHAPE";
    case DIT_ERR_UNSUPPORTED: return "DIT_ERR_UNSUPPORTED";
    case DIT_ERR_WORKSPACE: return "DIT_ERR_WORKSPACE";
    case DIT_ERR_HIP: return "DIT_ERR_HIP";
  }
  return "DIT_ERR_UNKNOWN";
}

}  // extern "C"
