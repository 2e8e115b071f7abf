// C-ABI layer: argument validation, handles, workspace layout and the order in
// which a step's kernels are enqueued.  Declarations and contracts are in
// include/llama_mi355x.h.
#include "llama_mi355x.h"

#include <hip/hip_runtime.h>

#include <algorithm>
#include <cstdarg>
#include <cstdio>
#include <cstring>
#include <string>
#include <vector>

#include "launch.h"

__attribute__((visibility("hidden"))) __thread LaunchTimer* launch_timer = nullptr;

namespace {

thread_local std::string g_err;

int fail(int code, const char* fmt, ...) {
  char buf[512];
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(buf, sizeof buf, fmt, ap);
  va_end(ap);
  g_err = buf;
  return code;
}

size_t align256(size_t x) { return (x + 255) & ~(size_t)255; }

// Device workspace carved into fixed regions.
struct Layout {
  size_t h, x, qkv, q, att, m, rope, logits, amx_v, amx_i, part, smp_v, smp_i, smp_bad, draft, flag,
      total;
};

struct Dims {
  int H, nq, nkv, d, qd, kvd, F, V, nexec;
  int M;      // largest number of rows one pass carries
  int Mdec;   // rows of one decode step (seqs * window)
  int Llog;   // rows of the internal logits buffer
};

Dims dims_of(const llama_config& c, int max_positions) {
  Dims d{};
  d.H = c.hidden;
  d.nq = c.n_q_heads;
  d.nkv = c.n_kv_heads;
  d.d = c.head_dim;
  d.qd = c.n_q_heads * c.head_dim;
  d.kvd = c.n_kv_heads * c.head_dim;
  d.F = c.ffn;
  d.V = c.vocab;
  d.nexec = c.n_blocks * c.n_loops;
  d.Mdec = c.max_seqs * c.max_window_rows;
  d.M = std::max(d.Mdec, c.max_chunk_rows);
  d.Llog = std::max(d.Mdec, 16);
  (void)max_positions;  // decode attention keeps at most attn_max_blocks() partials per row
  return d;
}

Layout layout_of(const Dims& d) {
  Layout L{};
  size_t off = 0;
  auto take = [&](size_t bytes) {
    size_t o = off;
    off += align256(bytes);
    return o;
  };
  L.h = take((size_t)d.M * d.H * 2);
  L.x = take((size_t)d.M * std::max(d.H, d.qd) * 2);
  L.qkv = take((size_t)d.M * (d.qd + 2 * d.kvd) * 2);
  L.q = take((size_t)d.M * d.qd * 2);
  L.att = take((size_t)d.M * d.qd * 2);
  L.m = take((size_t)d.M * d.F * 2);
  L.rope = take((size_t)d.M * (d.d / 2) * 8);
  int nch = d.V ? argmax_chunks(d.V) : 1;
  L.logits = take((size_t)d.Llog * std::max(d.V, 1) * 2);
  L.amx_v = take((size_t)d.Llog * nch * 4);
  L.amx_i = take((size_t)d.Llog * nch * 4);
  L.part = take((size_t)d.Mdec * d.nq * attn_max_blocks() * (d.d + 2) * 4);
  int nsc = d.V ? sample_chunks(d.V) : 1;
  L.smp_v = take((size_t)LLAMA_SAMPLE_MAX_ROWS * nsc * LLAMA_SAMPLE_MAX_TOP_K * 4);
  L.smp_i = take((size_t)LLAMA_SAMPLE_MAX_ROWS * nsc * LLAMA_SAMPLE_MAX_TOP_K * 4);
  L.smp_bad = take((size_t)LLAMA_SAMPLE_MAX_ROWS * nsc * 4);
  L.draft = take(3 * 32 * 4);  // a drafted round's window inputs, target tokens, count
  L.flag = take(256);
  L.total = off;
  return L;
}

int check_config(const llama_config* c) {
  if (!c) return fail(LLAMA_E_ARG, "config is NULL");
  if (c->n_blocks < 1 || c->n_loops < 1)
    return fail(LLAMA_E_GEOMETRY, "n_blocks and n_loops must be at least 1");
  if (c->head_dim != 64 && c->head_dim != 128)
    return fail(LLAMA_E_GEOMETRY, "head_dim %d is not served (64 or 128)", c->head_dim);
  if (c->hidden <= 0 || c->hidden % 128)
    return fail(LLAMA_E_GEOMETRY, "hidden %d is not a positive multiple of 128", c->hidden);
  if (c->ffn <= 0 || c->ffn % 128)
    return fail(LLAMA_E_GEOMETRY, "ffn %d is not a positive multiple of 128", c->ffn);
  if (c->n_kv_heads < 1 || c->n_q_heads < 1 || c->n_q_heads % c->n_kv_heads)
    return fail(LLAMA_E_GEOMETRY, "%d query heads do not split over %d KV heads", c->n_q_heads,
                c->n_kv_heads);
  if (c->n_q_heads / c->n_kv_heads > 8)
    return fail(LLAMA_E_GEOMETRY, "more than 8 query heads per KV head");
  if ((c->n_q_heads * c->head_dim) % 128 || (c->n_kv_heads * c->head_dim) % 128)
    return fail(LLAMA_E_GEOMETRY, "head widths must total multiples of 128");
  if (c->vocab < 0 || c->vocab % 128)
    return fail(LLAMA_E_GEOMETRY, "vocab %d is not a multiple of 128", c->vocab);
  if (!(c->rope_theta > 0.0)) return fail(LLAMA_E_GEOMETRY, "rope_theta must be positive");
  if (!(c->rms_eps >= 0.0f)) return fail(LLAMA_E_GEOMETRY, "rms_eps must be non-negative");
  if (c->max_chunk_rows < 1 || c->max_chunk_rows > 2048)
    return fail(LLAMA_E_GEOMETRY, "max_chunk_rows must be 1..2048");
  if (c->max_window_rows < 1 || c->max_window_rows > 16)
    return fail(LLAMA_E_GEOMETRY, "max_window_rows must be 1..16");
  if (c->max_seqs < 1 || c->max_seqs > LLAMA_MAX_SEQS)
    return fail(LLAMA_E_GEOMETRY, "max_seqs must be 1..%d", LLAMA_MAX_SEQS);
  if (c->prompt_exact != 0 && c->prompt_exact != 1)
    return fail(LLAMA_E_ARG, "prompt_exact must be 0 or 1");
  return LLAMA_OK;
}

}  // namespace

struct llama_model {
  llama_config cfg;
  Dims d;
  Layout L;
  std::vector<llama_block_weights> blocks;
  const void* embed;
  const void* final_norm;
  const void* lm_head;
  uint8_t* ws;
  int max_positions;
  void* cap;
  size_t cap_bytes;
  // parity probe of one execution (test hook)
  int probe_exec = -1;
  int probe_rows = 0;
  llama_probe probe{};
  bool flag_ready;  // the non-finite flag has been cleared on the device
  // measurement hook
  int timing_kernel = 0;
  std::vector<hipEvent_t> tev;  // pairs
  size_t tused = 0;
  template <typename T>
  T* at(size_t off) const {
    return (T*)(ws + off);
  }
};

struct llama_kv {
  llama_model* model;
  uint8_t* buf;
  int max_positions;
  int length;
  size_t slab;  // bytes of one execution's keys (or values)
};

namespace {

int dev_check(const char* what) {
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return fail(LLAMA_E_DEVICE, "%s: %s", what, hipGetErrorString(e));
  return LLAMA_OK;
}

// Rows [row0, row0 + rows) of the pass over sequences kvs[0..nseq) with
// `rows_per_seq` rows each, starting at positions pos0[s].
struct Pass {
  llama_model* m;
  llama_kv* const* kvs;
  int nseq;
  int rows_per_seq;
  int pos0[LLAMA_MAX_SEQS];
  hipStream_t s;
};

RowTable table_for(const Pass& p, int exec) {
  RowTable t{};
  for (int i = 0; i < p.nseq; ++i) {
    uint8_t* base = p.kvs[i]->buf + (size_t)exec * 2 * p.kvs[i]->slab;
    t.k[i] = (uint16_t*)base;
    t.v[i] = (uint16_t*)(base + p.kvs[i]->slab);
    t.pos0[i] = p.pos0[i];
  }
  t.rows_per_seq = p.rows_per_seq;
  return t;
}

// While in scope for the measured kernel class, the kernels launched record
// their own execution time in the model's event pool.
struct Timed {
  LaunchTimer lt;
  LaunchTimer* prev;
  bool on;
  Timed(llama_model* m, int cls, hipStream_t) : prev(launch_timer) {
    on = m->timing_kernel == cls;
    if (on) {
      lt = LaunchTimer{m->tev.data(), m->tev.size(), &m->tused};
      launch_timer = &lt;
    }
  }
  ~Timed() {
    if (on) launch_timer = prev;
  }
};

// Projection over all rows in launches of at most 16 rows.
void gemv_rows(int epi, const GemvSeg* seg, int nseg, int N, int K, const void* x, int ldx,
               int rows, void* out, int ldo, float* out32, int ld32, hipStream_t s,
               const void* normw = nullptr, float eps = 0.f) {
  for (int r0 = 0; r0 < rows; r0 += 16) {
    int n = std::min(16, rows - r0);
    launch_gemv(epi, seg, nseg, N, K, (const uint16_t*)x + (size_t)r0 * ldx, ldx, n,
                (uint16_t*)out + (size_t)r0 * ldo, ldo, out32 ? out32 + (size_t)r0 * ld32 : nullptr,
                ld32, normw, eps, s);
  }
}

// Decode windows of up to GEMV_NORM_ROWS rows normalise inside the
// projections (q/k/v, gate/up, lm_head) instead of running rmsnorm_kernel;
// both use one canonical order, so the bits are the same either way.
bool norm_fused(bool chunk, int rows) { return !chunk && rows <= GEMV_NORM_ROWS; }

// Runs the block stack over the pass's rows.  On return ws.h holds the
// residual after the last execution and, when the model has a vocabulary and
// the norm is not fused, ws.x the final-normed rows.  cap_row0 / cap_rows
// place these rows in the capture buffer.  While the parity probe is set,
// its execution also writes the probe's intermediate values (extra launches
// of the same kernels with storing epilogues, into the caller's buffers;
// their bf16 outputs land in workspace regions that are dead at that point).
void run_stack(const Pass& p, const int32_t* tok, const void* hin, void* hout, int cap_row0,
               int cap_rows, bool chunk) {
  llama_model* m = p.m;
  const Dims& d = m->d;
  const llama_config& c = m->cfg;
  const int rows = p.nseq * p.rows_per_seq;
  uint16_t* h = m->at<uint16_t>(m->L.h);
  uint16_t* x = m->at<uint16_t>(m->L.x);
  uint16_t* qkv = m->at<uint16_t>(m->L.qkv);
  uint16_t* q = m->at<uint16_t>(m->L.q);
  uint16_t* att = m->at<uint16_t>(m->L.att);
  uint16_t* mm = m->at<uint16_t>(m->L.m);
  float* part = m->at<float>(m->L.part);
  void* rope = m->ws + m->L.rope;
  const size_t rowb = (size_t)d.H * 2;
  const bool fuse = norm_fused(chunk, rows);
  const bool ex = c.prompt_exact != 0;
  const int nqkv = d.qd + 2 * d.kvd;

  if (tok) launch_embed(m->embed, d.V, d.H, tok, h, rows, p.s);
  else (void)hipMemcpyAsync(h, hin, rows * rowb, hipMemcpyDeviceToDevice, p.s);
  launch_rope_table(table_for(p, 0), rows, d.d, (float)c.rope_theta, rope, p.s);

  for (int loop = 0; loop < c.n_loops; ++loop) {
    for (int b = 0; b < c.n_blocks; ++b) {
      const int e = loop * c.n_blocks + b;
      const llama_block_weights& w = m->blocks[b];
      RowTable tab = table_for(p, e);
      const bool pr = m->probe_exec == e;
      const llama_probe& P = m->probe;
      auto pcopy = [&](void* dst, const void* src, size_t width_bytes) {
        if (pr && dst)
          (void)hipMemcpyAsync(dst, src, rows * width_bytes, hipMemcpyDeviceToDevice, p.s);
      };
      // the normed input of a projection, into the probe: copied when the
      // step normalises into ws.x, else by the same norm kernel
      auto pnorm = [&](void* dst, const void* normw) {
        if (!pr || !dst) return;
        if (fuse) launch_rmsnorm(h, normw, dst, rows, d.H, c.rms_eps, p.s);
        else pcopy(dst, x, rowb);
      };
      pcopy(P.h_in, h, rowb);

      if (!fuse) launch_rmsnorm(h, w.attn_norm, x, rows, d.H, c.rms_eps, p.s);
      pnorm(P.x_attn, w.attn_norm);
      GemvSeg qkvseg[3] = {{(const uint16_t*)w.q, 0, d.qd},
                           {(const uint16_t*)w.k, d.qd, d.qd + d.kvd},
                           {(const uint16_t*)w.v, d.qd + d.kvd, d.qd + 2 * d.kvd}};
      GemvSeg oseg[1] = {{(const uint16_t*)w.o, 0, d.H}};
      if (chunk) {
        {
          Timed t(m, LLAMA_TIMING_PREFILL_GEMM, p.s);
          launch_gemm(GEMV_STORE, x, d.H, rows, d.H, qkvseg, 3, nullptr, nullptr, qkv, nqkv,
                      pr ? P.qkv32 : nullptr, nqkv, nqkv, ex, p.s);
        }
        launch_rope_kv(qkv, q, tab, rows, d.nq, d.nkv, d.d, rope, p.s);
        pcopy(P.q_rope, q, (size_t)d.qd * 2);
        {
          Timed t(m, LLAMA_TIMING_PREFILL_ATTN, p.s);
          launch_attn_prefill(q, tab.k[0], tab.v[0], rows, p.pos0[0], d.nq, d.nkv, d.d, att,
                              pr ? P.attn32 : nullptr, ex, p.s);
        }
        pcopy(P.attn, att, (size_t)d.qd * 2);
        if (pr && P.o32)
          launch_gemm(GEMV_STORE, att, d.qd, rows, d.qd, oseg, 1, nullptr, nullptr, x, d.H, P.o32,
                      d.H, d.H, ex, p.s);
        {
          Timed t(m, LLAMA_TIMING_PREFILL_GEMM, p.s);
          launch_gemm(GEMV_RESIDUAL, att, d.qd, rows, d.qd, oseg, 1, nullptr, nullptr, h, d.H,
                      nullptr, 0, d.H, ex, p.s);
        }
      } else {
        const uint16_t* in = fuse ? h : x;
        if (pr && P.qkv32)  // same sums as the fused launch; bf16 results unused
          gemv_rows(GEMV_STORE, qkvseg, 3, nqkv, d.H, in, d.H, rows, qkv, nqkv, P.qkv32, nqkv,
                    p.s, fuse ? w.attn_norm : nullptr, c.rms_eps);
        {
          Timed t(m, LLAMA_TIMING_QKV, p.s);
          for (int r0 = 0; r0 < rows; r0 += 16)
            launch_gemv_qkv_rope(qkvseg, d.H, in + (size_t)r0 * d.H, d.H, std::min(16, rows - r0),
                                 r0, q, tab, rope, d.nq, d.nkv, d.d, fuse ? w.attn_norm : nullptr,
                                 c.rms_eps, p.s);
        }
        pcopy(P.q_rope, q, (size_t)d.qd * 2);
        {
          Timed t(m, LLAMA_TIMING_ATTN, p.s);
          launch_attn_decode(q, tab, rows, d.nq, d.nkv, d.d, part, att, pr ? P.attn32 : nullptr,
                             p.s);
        }
        pcopy(P.attn, att, (size_t)d.qd * 2);
        if (pr && P.o32)
          gemv_rows(GEMV_STORE, oseg, 1, d.H, d.qd, att, d.qd, rows, x, d.H, P.o32, d.H, p.s);
        {
          Timed t(m, LLAMA_TIMING_O, p.s);
          gemv_rows(GEMV_RESIDUAL, oseg, 1, d.H, d.qd, att, d.qd, rows, h, d.H, nullptr, 0, p.s);
        }
      }
      if (m->cap)
        (void)hipMemcpy2DAsync((uint8_t*)m->cap + (((size_t)e * 2 + 0) * cap_rows + cap_row0) * rowb,
                         rowb, h, rowb, rowb, rows, hipMemcpyDeviceToDevice, p.s);

      if (!fuse) launch_rmsnorm(h, w.mlp_norm, x, rows, d.H, c.rms_eps, p.s);
      pnorm(P.x_mlp, w.mlp_norm);
      GemvSeg gseg[1] = {{(const uint16_t*)w.gate, 0, d.F}};
      GemvSeg useg[1] = {{(const uint16_t*)w.up, 0, d.F}};
      GemvSeg gu[2] = {gseg[0], useg[0]};
      GemvSeg dseg[1] = {{(const uint16_t*)w.down, 0, d.H}};
      const bool pgu = pr && P.gate_up32;
      if (chunk) {
        if (pgu) {  // bf16 results land in ws.m before the SwiGLU launch rewrites it
          launch_gemm(GEMV_STORE, x, d.H, rows, d.H, gseg, 1, nullptr, nullptr, mm, d.F,
                      P.gate_up32, 2 * d.F, d.F, ex, p.s);
          launch_gemm(GEMV_STORE, x, d.H, rows, d.H, useg, 1, nullptr, nullptr, mm, d.F,
                      P.gate_up32 + d.F, 2 * d.F, d.F, ex, p.s);
        }
        {
          Timed t(m, LLAMA_TIMING_PREFILL_GEMM, p.s);
          launch_gemm(GEMV_SWIGLU, x, d.H, rows, d.H, nullptr, 0, w.gate, w.up, mm, d.F, nullptr,
                      0, 2 * d.F, ex, p.s);
          launch_gemm(GEMV_RESIDUAL, mm, d.F, rows, d.F, dseg, 1, nullptr, nullptr, h, d.H,
                      nullptr, 0, d.H, ex, p.s);
        }
        if (pr && P.down32)
          launch_gemm(GEMV_STORE, mm, d.F, rows, d.F, dseg, 1, nullptr, nullptr, x, d.H, P.down32,
                      d.H, d.H, ex, p.s);
      } else {
        const uint16_t* in = fuse ? h : x;
        if (pgu) {
          gemv_rows(GEMV_STORE, gseg, 1, d.F, d.H, in, d.H, rows, mm, d.F, P.gate_up32, 2 * d.F,
                    p.s, fuse ? w.mlp_norm : nullptr, c.rms_eps);
          gemv_rows(GEMV_STORE, useg, 1, d.F, d.H, in, d.H, rows, mm, d.F, P.gate_up32 + d.F,
                    2 * d.F, p.s, fuse ? w.mlp_norm : nullptr, c.rms_eps);
        }
        {
          Timed t(m, LLAMA_TIMING_GATE_UP, p.s);
          gemv_rows(GEMV_SWIGLU, gu, 2, d.F, d.H, in, d.H, rows, mm, d.F, nullptr, 0, p.s,
                    fuse ? w.mlp_norm : nullptr, c.rms_eps);
        }
        {
          Timed t(m, LLAMA_TIMING_DOWN, p.s);
          gemv_rows(GEMV_RESIDUAL, dseg, 1, d.H, d.F, mm, d.F, rows, h, d.H, nullptr, 0, p.s);
        }
        if (pr && P.down32)
          gemv_rows(GEMV_STORE, dseg, 1, d.H, d.F, mm, d.F, rows, x, d.H, P.down32, d.H, p.s);
      }
      pcopy(P.act, mm, (size_t)d.F * 2);
      if (m->cap)
        (void)hipMemcpy2DAsync((uint8_t*)m->cap + (((size_t)e * 2 + 1) * cap_rows + cap_row0) * rowb,
                         rowb, h, rowb, rowb, rows, hipMemcpyDeviceToDevice, p.s);
    }
    const bool last = loop == c.n_loops - 1;
    if (last && hout) (void)hipMemcpyAsync(hout, h, rows * rowb, hipMemcpyDeviceToDevice, p.s);
    if (d.V && !(last && fuse)) {
      // final norm at the end of every loop; it replaces the residual between
      // loops (after the last, a fused head normalises its rows itself)
      launch_rmsnorm(h, m->final_norm, last ? x : h, rows, d.H, c.rms_eps, p.s);
    }
  }
}

// lm_head over `rows` rows starting at x, then the greedy draw.  The rows
// are final-normed, or with normw raw residuals the projection normalises.
void run_head(llama_model* m, const uint16_t* x, int rows, void* logits_bf16, float* logits_f32,
              int32_t* next, hipStream_t s, const void* normw = nullptr) {
  const Dims& d = m->d;
  GemvSeg seg[1] = {{(const uint16_t*)m->lm_head, 0, d.V}};
  for (int r0 = 0; r0 < rows; r0 += d.Llog) {
    int n = std::min(d.Llog, rows - r0);
    uint16_t* lb = logits_bf16 ? (uint16_t*)logits_bf16 + (size_t)r0 * d.V
                               : m->at<uint16_t>(m->L.logits);
    {
      Timed t(m, LLAMA_TIMING_LM_HEAD, s);
      gemv_rows(GEMV_STORE, seg, 1, d.V, d.H, x + (size_t)r0 * d.H, d.H, n, lb, d.V,
                logits_f32 ? logits_f32 + (size_t)r0 * d.V : nullptr, d.V, s, normw,
                m->cfg.rms_eps);
    }
    if (next)
      launch_argmax(lb, d.V, d.V, n, m->at<float>(m->L.amx_v), m->at<int>(m->L.amx_i), next + r0,
                    m->at<int>(m->L.flag), s);
  }
}

// The first step on a model clears its non-finite flag (a fill kernel, so the
// clearing can sit inside a captured graph).
// It also clears any error an unrelated earlier runtime call left behind, so
// that the check after the step's launches reports the step's own.
void ready_flag(llama_model* m, hipStream_t s) {
  (void)hipGetLastError();
  if (!m->flag_ready) {
    launch_fill_zero(m->at<int>(m->L.flag), 64, s);
    m->flag_ready = true;
  }
}

// Rows enter as token ids (through the embedding) or as hidden rows; a
// blocks-only model has neither embedding nor logits.
int check_inputs(const llama_model* m, const void* tok, const void* hin, const void* lb,
                 const void* l32, const void* next) {
  if (!tok == !hin) return fail(LLAMA_E_ARG, "give exactly one of token ids and hidden rows");
  if (!m->d.V) {
    if (tok) return fail(LLAMA_E_ARG, "a blocks-only model takes hidden rows");
    if (lb || l32 || next) return fail(LLAMA_E_ARG, "a blocks-only model has no logits");
  }
  return LLAMA_OK;
}

int check_kv(const llama_model* m, const llama_kv* kv) {
  if (!kv) return fail(LLAMA_E_ARG, "cache handle is NULL");
  if (kv->model != m) return fail(LLAMA_E_ARG, "cache belongs to another model");
  return LLAMA_OK;
}

}  // namespace

extern "C" {

size_t llama_workspace_bytes(const llama_config* cfg, int32_t max_positions) {
  if (check_config(cfg) != LLAMA_OK || max_positions < 1) return 0;
  return layout_of(dims_of(*cfg, max_positions)).total;
}

int llama_load_weights(const llama_config* cfg, const llama_block_weights* blocks,
                       const void* embed, const void* final_norm, const void* lm_head,
                       void* workspace_dev, size_t workspace_bytes, int32_t max_positions,
                       llama_model** out) {
  int rc = check_config(cfg);
  if (rc) return rc;
  if (!out) return fail(LLAMA_E_ARG, "out is NULL");
  if (!blocks) return fail(LLAMA_E_ARG, "blocks is NULL");
  if (max_positions < 1) return fail(LLAMA_E_ARG, "max_positions must be positive");
  for (int b = 0; b < cfg->n_blocks; ++b) {
    const llama_block_weights& w = blocks[b];
    if (!w.attn_norm || !w.q || !w.k || !w.v || !w.o || !w.mlp_norm || !w.gate || !w.up || !w.down)
      return fail(LLAMA_E_ARG, "block %d has a NULL weight", b);
  }
  if (cfg->vocab) {
    if (!embed || !final_norm || !lm_head)
      return fail(LLAMA_E_ARG, "embed, final_norm and lm_head are required with a vocabulary");
    if (lm_head == embed)
      return fail(LLAMA_E_GEOMETRY, "tied heads are refused: lm_head is the embedding");
  } else if (embed || final_norm || lm_head) {
    return fail(LLAMA_E_ARG, "a blocks-only model (vocab 0) takes no embed/final_norm/lm_head");
  }
  Dims d = dims_of(*cfg, max_positions);
  Layout L = layout_of(d);
  if (!workspace_dev) return fail(LLAMA_E_ARG, "workspace is NULL");
  if (workspace_bytes < L.total)
    return fail(LLAMA_E_WORKSPACE, "workspace of %zu bytes, %zu needed", workspace_bytes, L.total);
  llama_model* m = new llama_model();
  m->cfg = *cfg;
  m->d = d;
  m->L = L;
  m->blocks.assign(blocks, blocks + cfg->n_blocks);
  m->embed = embed;
  m->final_norm = final_norm;
  m->lm_head = lm_head;
  m->ws = (uint8_t*)workspace_dev;
  m->max_positions = max_positions;
  m->cap = nullptr;
  m->cap_bytes = 0;
  m->flag_ready = false;
  *out = m;
  g_err.clear();
  return LLAMA_OK;
}

size_t llama_kv_bytes(const llama_model* m, int32_t max_positions) {
  if (!m || max_positions < 1) return 0;
  return (size_t)m->d.nexec * max_positions * m->d.kvd * 2 * 2;
}

int llama_kv_alloc(llama_model* m, int32_t max_positions, void* device_buf, size_t bytes,
                   llama_kv** out) {
  if (!m || !out || !device_buf) return fail(LLAMA_E_ARG, "NULL argument");
  if (max_positions < 1 || max_positions > m->max_positions)
    return fail(LLAMA_E_CAPACITY, "max_positions %d outside 1..%d", max_positions,
                m->max_positions);
  size_t need = llama_kv_bytes(m, max_positions);
  if (bytes < need) return fail(LLAMA_E_WORKSPACE, "cache of %zu bytes, %zu needed", bytes, need);
  llama_kv* kv = new llama_kv();
  kv->model = m;
  kv->buf = (uint8_t*)device_buf;
  kv->max_positions = max_positions;
  kv->length = 0;
  kv->slab = (size_t)max_positions * m->d.kvd * 2;
  *out = kv;
  return LLAMA_OK;
}

int32_t llama_kv_length(const llama_kv* kv) { return kv ? kv->length : -1; }

int llama_kv_truncate(llama_kv* kv, int32_t n) {
  if (!kv) return fail(LLAMA_E_ARG, "cache handle is NULL");
  if (n < 0 || n > kv->length)
    return fail(LLAMA_E_POSITION, "cannot keep %d positions of a cache holding %d", n, kv->length);
  kv->length = n;
  return LLAMA_OK;
}

int llama_test_kv_declare(llama_kv* kv, int32_t n) {
  if (!kv) return fail(LLAMA_E_ARG, "cache handle is NULL");
  if (n < 0 || n > kv->max_positions)
    return fail(LLAMA_E_CAPACITY, "length %d outside 0..%d", n, kv->max_positions);
  kv->length = n;
  return LLAMA_OK;
}

void* llama_kv_slab(const llama_kv* kv, int32_t exec, int32_t which) {
  if (!kv || exec < 0 || exec >= kv->model->d.nexec || (which != 0 && which != 1)) return nullptr;
  return kv->buf + ((size_t)exec * 2 + which) * kv->slab;
}

int llama_set_capture(llama_model* m, void* buf, size_t bytes) {
  if (!m) return fail(LLAMA_E_ARG, "model is NULL");
  m->cap = buf;
  m->cap_bytes = buf ? bytes : 0;
  return LLAMA_OK;
}

int llama_set_probe(llama_model* m, int32_t exec, const llama_probe* probe, int32_t max_rows) {
  if (!m) return fail(LLAMA_E_ARG, "model is NULL");
  if (!probe) {
    m->probe_exec = -1;
    m->probe_rows = 0;
    m->probe = llama_probe{};
    return LLAMA_OK;
  }
  if (exec < 0 || exec >= m->d.nexec)
    return fail(LLAMA_E_ARG, "execution %d outside 0..%d", exec, m->d.nexec - 1);
  if (max_rows < 1) return fail(LLAMA_E_ARG, "max_rows must be positive");
  m->probe_exec = exec;
  m->probe_rows = max_rows;
  m->probe = *probe;
  return LLAMA_OK;
}

static int check_capture(llama_model* m, int rows) {
  if (m->probe_exec >= 0 && rows > m->probe_rows)
    return fail(LLAMA_E_WORKSPACE, "probe buffers hold %d rows, the step has %d", m->probe_rows,
                rows);
  if (!m->cap) return LLAMA_OK;
  size_t need = (size_t)m->d.nexec * 2 * rows * m->d.H * 2;
  if (m->cap_bytes < need)
    return fail(LLAMA_E_WORKSPACE, "capture buffer of %zu bytes, %zu needed", m->cap_bytes, need);
  return LLAMA_OK;
}

int llama_prefill_chunk(llama_model* m, llama_kv* kv, const int32_t* tokens_dev,
                        const void* hidden_in_dev, int32_t n_rows, int32_t pos0,
                        void* hidden_out_dev, void* logits_bf16_dev, float* logits_f32_dev,
                        int32_t all_rows, int32_t* next_token_dev, void* hip_stream) {
  if (!m) return fail(LLAMA_E_ARG, "model is NULL");
  int rc = check_kv(m, kv);
  if (rc) return rc;
  if (n_rows < 1 || n_rows > m->cfg.max_chunk_rows)
    return fail(LLAMA_E_ARG, "n_rows %d outside 1..%d", n_rows, m->cfg.max_chunk_rows);
  if (pos0 != kv->length)
    return fail(LLAMA_E_POSITION, "pos0 %d differs from the cache length %d", pos0, kv->length);
  if ((int64_t)pos0 + n_rows > kv->max_positions)
    return fail(LLAMA_E_CAPACITY, "positions %d..%d pass the cache's %d", pos0, pos0 + n_rows - 1,
                kv->max_positions);
  rc = check_inputs(m, tokens_dev, hidden_in_dev, logits_bf16_dev, logits_f32_dev, next_token_dev);
  if (rc) return rc;
  rc = check_capture(m, n_rows);
  if (rc) return rc;
  hipStream_t s = (hipStream_t)hip_stream;
  ready_flag(m, s);
  Pass p{m, &kv, 1, n_rows, {0}, s};
  p.pos0[0] = pos0;
  run_stack(p, tokens_dev, hidden_in_dev, hidden_out_dev, 0, n_rows, true);
  if (m->d.V) {
    const uint16_t* x = m->at<uint16_t>(m->L.x);
    if (all_rows)
      run_head(m, x, n_rows, logits_bf16_dev, logits_f32_dev, next_token_dev, s);
    else
      run_head(m, x + (size_t)(n_rows - 1) * m->d.H, 1, logits_bf16_dev, logits_f32_dev,
               next_token_dev, s);
  }
  rc = dev_check("prefill launch");
  if (rc) return rc;
  kv->length += n_rows;
  return LLAMA_OK;
}

int llama_decode_step(llama_model* m, llama_kv* const* kvs, int32_t n_seq,
                      const int32_t* tokens_dev, const void* hidden_in_dev, int32_t rows,
                      void* hidden_out_dev, void* logits_bf16_dev, float* logits_f32_dev,
                      int32_t* next_tokens_dev, void* hip_stream) {
  if (!m) return fail(LLAMA_E_ARG, "model is NULL");
  if (!kvs) return fail(LLAMA_E_ARG, "kvs is NULL");
  if (n_seq < 1 || n_seq > m->cfg.max_seqs)
    return fail(LLAMA_E_ARG, "n_seq %d outside 1..%d", n_seq, m->cfg.max_seqs);
  if (rows < 1 || rows > m->cfg.max_window_rows)
    return fail(LLAMA_E_ARG, "rows %d outside 1..%d", rows, m->cfg.max_window_rows);
  for (int i = 0; i < n_seq; ++i) {
    int rc = check_kv(m, kvs[i]);
    if (rc) return rc;
    for (int j = 0; j < i; ++j)
      if (kvs[j] == kvs[i]) return fail(LLAMA_E_ARG, "sequence %d repeats sequence %d's cache", i, j);
    if ((int64_t)kvs[i]->length + rows > kvs[i]->max_positions)
      return fail(LLAMA_E_CAPACITY, "sequence %d: positions %d..%d pass the cache's %d", i,
                  kvs[i]->length, kvs[i]->length + rows - 1, kvs[i]->max_positions);
  }
  int rc = check_inputs(m, tokens_dev, hidden_in_dev, logits_bf16_dev, logits_f32_dev,
                        next_tokens_dev);
  if (rc) return rc;
  const int total = n_seq * rows;
  rc = check_capture(m, total);
  if (rc) return rc;
  hipStream_t s = (hipStream_t)hip_stream;
  ready_flag(m, s);
  Pass p{m, kvs, n_seq, rows, {0}, s};
  for (int i = 0; i < n_seq; ++i) p.pos0[i] = kvs[i]->length;
  run_stack(p, tokens_dev, hidden_in_dev, hidden_out_dev, 0, total, false);
  if (m->d.V && (logits_bf16_dev || logits_f32_dev || next_tokens_dev)) {
    const bool fuse = norm_fused(false, total);
    run_head(m, m->at<uint16_t>(fuse ? m->L.h : m->L.x), total, logits_bf16_dev, logits_f32_dev,
             next_tokens_dev, s, fuse ? m->final_norm : nullptr);
  }
  rc = dev_check("decode launch");
  if (rc) return rc;
  for (int i = 0; i < n_seq; ++i) kvs[i]->length += rows;
  return LLAMA_OK;
}

}  // extern "C"

namespace {

struct DraftSampling {
  float temperature;
  int32_t top_k;
  float top_p;
  const float* u;
};

int check_sampling(const llama_model* m, float temperature, int32_t top_k, float top_p) {
  const int V = m->d.V;
  if (!(temperature > 0.0f) || !(temperature < INFINITY))
    return fail(LLAMA_E_ARG, "temperature must be positive and finite (greedy draws take "
                "next_tokens in the step calls)");
  if (top_k < 1 || top_k > LLAMA_SAMPLE_MAX_TOP_K || top_k > V)
    return fail(LLAMA_E_ARG, "top_k %d outside 1..%d", top_k, std::min(LLAMA_SAMPLE_MAX_TOP_K, V));
  if (!(top_p > 0.0f) || !(top_p <= 1.0f)) return fail(LLAMA_E_ARG, "top_p must lie in (0, 1]");
  if (sample_chunks(V) * top_k > 4096)
    return fail(LLAMA_E_ARG, "top_k %d too large for a vocabulary of %d", top_k, V);
  return LLAMA_OK;
}

// One drafted round; sp == NULL: the target's greedy tokens, else its
// seeded draws (sp->u[i] for the token after window row i).
int draft_round(llama_model* target, llama_kv* target_kv, llama_model* draft, llama_kv* draft_kv,
                int32_t n_draft, const int32_t* last_token_dev, const DraftSampling* sp,
                int32_t* tokens_out_dev, int32_t* n_out, void* hip_stream) {
  if (!target || !draft) return fail(LLAMA_E_ARG, "model is NULL");
  if (target == draft) return fail(LLAMA_E_ARG, "the draft model is the target model");
  int rc = check_kv(target, target_kv);
  if (rc) return rc;
  rc = check_kv(draft, draft_kv);
  if (rc) return rc;
  if (!last_token_dev || !tokens_out_dev || !n_out) return fail(LLAMA_E_ARG, "NULL argument");
  if (!target->d.V || target->d.V != draft->d.V)
    return fail(LLAMA_E_ARG, "vocabularies differ (%d and %d)", target->d.V, draft->d.V);
  if (n_draft < 1 || n_draft + 1 > target->cfg.max_window_rows)
    return fail(LLAMA_E_ARG, "n_draft %d outside 1..%d (the target's window less one)", n_draft,
                target->cfg.max_window_rows - 1);
  if (sp) {
    if (!sp->u) return fail(LLAMA_E_ARG, "uniforms are NULL");
    rc = check_sampling(target, sp->temperature, sp->top_k, sp->top_p);
    if (rc) return rc;
  }
  const int p = target_kv->length;
  if (draft_kv->length != p)
    return fail(LLAMA_E_POSITION, "the draft cache holds %d positions, the target's %d",
                draft_kv->length, p);
  if ((int64_t)p + n_draft + 1 > target_kv->max_positions)
    return fail(LLAMA_E_CAPACITY, "positions %d..%d pass the target cache's %d", p, p + n_draft,
                target_kv->max_positions);
  if ((int64_t)p + n_draft + 1 > draft_kv->max_positions)
    return fail(LLAMA_E_CAPACITY, "positions %d..%d pass the draft cache's %d", p, p + n_draft,
                draft_kv->max_positions);
  rc = check_capture(target, n_draft + 1);
  if (rc) return rc;
  rc = check_capture(draft, 1);
  if (rc) return rc;
  hipStream_t s = (hipStream_t)hip_stream;
  int32_t* win = target->at<int32_t>(target->L.draft);  // [0..k]: last, d_1 .. d_k
  int32_t* tt = win + 32;                                 // the target's tokens
  int32_t* cnt = win + 64;
  if (hipMemcpyAsync(win, last_token_dev, 4, hipMemcpyDeviceToDevice, s) != hipSuccess)
    return dev_check("drafted round copy");
  // the draft's greedy proposals, one row at a time, each fed back
  for (int i = 0; i < n_draft; ++i) {
    rc = llama_decode_step(draft, &draft_kv, 1, win + i, nullptr, 1, nullptr, nullptr, nullptr,
                           win + i + 1, s);
    if (rc) return rc;
  }
  // the target's verdict on all of them in one window
  if (!sp) {
    rc = llama_decode_step(target, &target_kv, 1, win, nullptr, n_draft + 1, nullptr, nullptr,
                           nullptr, tt, s);
    if (rc) return rc;
  } else {
    void* lg = target->ws + target->L.logits;  // room for max(16, decode rows) rows
    rc = llama_decode_step(target, &target_kv, 1, win, nullptr, n_draft + 1, nullptr, lg, nullptr,
                           nullptr, s);
    if (rc) return rc;
    launch_sample(lg, target->d.V, target->d.V, n_draft + 1, sp->top_k, sp->temperature, sp->top_p,
                  sp->u, target->at<float>(target->L.smp_v), target->at<int>(target->L.smp_i),
                  target->at<int>(target->L.smp_bad), tt, target->at<int>(target->L.flag), s);
  }
  launch_draft_accept(win, tt, n_draft, tokens_out_dev, cnt, s);
  rc = dev_check("drafted round acceptance");
  if (rc) return rc;
  int32_t a = 0;
  if (hipMemcpyAsync(&a, cnt, 4, hipMemcpyDeviceToHost, s) != hipSuccess ||
      hipStreamSynchronize(s) != hipSuccess)
    return dev_check("drafted round count");
  // both caches keep the inputs last, d_1 .. d_a; with every proposal taken
  // the draft has not yet read d_k, so it reads it now (its token unused)
  target_kv->length = p + a + 1;
  if (a == n_draft) {
    rc = llama_decode_step(draft, &draft_kv, 1, win + n_draft, nullptr, 1, nullptr, nullptr,
                           nullptr, tt, s);
    if (rc) return rc;
  } else {
    draft_kv->length = p + a + 1;
  }
  *n_out = a + 1;
  return LLAMA_OK;
}

}  // namespace

extern "C" {

int llama_draft_round(llama_model* target, llama_kv* target_kv, llama_model* draft,
                      llama_kv* draft_kv, int32_t n_draft, const int32_t* last_token_dev,
                      int32_t* tokens_out_dev, int32_t* n_out, void* hip_stream) {
  return draft_round(target, target_kv, draft, draft_kv, n_draft, last_token_dev, nullptr,
                     tokens_out_dev, n_out, hip_stream);
}

int llama_draft_round_sampled(llama_model* target, llama_kv* target_kv, llama_model* draft,
                              llama_kv* draft_kv, int32_t n_draft, const int32_t* last_token_dev,
                              float temperature, int32_t top_k, float top_p, const float* u_dev,
                              int32_t* tokens_out_dev, int32_t* n_out, void* hip_stream) {
  const DraftSampling sp{temperature, top_k, top_p, u_dev};
  return draft_round(target, target_kv, draft, draft_kv, n_draft, last_token_dev, &sp,
                     tokens_out_dev, n_out, hip_stream);
}

int llama_sample(llama_model* m, const void* logits_bf16_dev, int32_t rows, int64_t ld,
                 float temperature, int32_t top_k, float top_p, const float* u_dev,
                 int32_t* tokens_dev, void* hip_stream) {
  if (!m) return fail(LLAMA_E_ARG, "model is NULL");
  const int V = m->d.V;
  if (!V) return fail(LLAMA_E_ARG, "a blocks-only model has no logits to sample");
  if (!logits_bf16_dev || !u_dev || !tokens_dev) return fail(LLAMA_E_ARG, "NULL buffer");
  if (rows < 1 || rows > LLAMA_SAMPLE_MAX_ROWS)
    return fail(LLAMA_E_ARG, "rows %d outside 1..%d", rows, LLAMA_SAMPLE_MAX_ROWS);
  if (ld < V) return fail(LLAMA_E_ARG, "row stride %lld below the vocabulary %d", (long long)ld, V);
  int rc = check_sampling(m, temperature, top_k, top_p);
  if (rc) return rc;
  hipStream_t s = (hipStream_t)hip_stream;
  ready_flag(m, s);
  launch_sample(logits_bf16_dev, V, ld, rows, top_k, temperature, top_p, u_dev,
                m->at<float>(m->L.smp_v), m->at<int>(m->L.smp_i), m->at<int>(m->L.smp_bad),
                tokens_dev, m->at<int>(m->L.flag), s);
  return dev_check("sample launch");
}

int llama_test_linear(llama_model* m, int32_t prompt_kernel, const void* x, int32_t rows,
                      const void* w, int32_t n, int32_t k, void* y, float* y32, void* hip_stream) {
  if (!m) return fail(LLAMA_E_ARG, "model is NULL");
  if (!x || !w || !y || !y32) return fail(LLAMA_E_ARG, "NULL buffer");
  if (n < 128 || k < 128 || n % 128 || k % 128)
    return fail(LLAMA_E_ARG, "n %d and k %d must be positive multiples of 128", n, k);
  if (prompt_kernel < 0 || prompt_kernel > 2)
    return fail(LLAMA_E_ARG, "prompt_kernel %d is not 0, 1 or 2", prompt_kernel);
  const int maxr = prompt_kernel ? 2048 : 16;
  if (rows < 1 || rows > maxr) return fail(LLAMA_E_ARG, "rows %d outside 1..%d", rows, maxr);
  hipStream_t s = (hipStream_t)hip_stream;
  (void)hipGetLastError();
  GemvSeg seg[1] = {{(const uint16_t*)w, 0, n}};
  if (prompt_kernel)
    launch_gemm(GEMV_STORE, x, k, rows, k, seg, 1, nullptr, nullptr, y, n, y32, n, n,
                prompt_kernel == 2, s);
  else
    launch_gemv(GEMV_STORE, seg, 1, n, k, x, k, rows, y, n, y32, n, nullptr, 0.f, s);
  return dev_check("test linear launch");
}

int llama_test_attention(llama_model* m, int32_t prompt_kernel, llama_kv* kv, int32_t exec,
                         const void* q, int32_t rows, int32_t pos0, void* out, float* out32,
                         void* hip_stream) {
  if (!m) return fail(LLAMA_E_ARG, "model is NULL");
  int rc = check_kv(m, kv);
  if (rc) return rc;
  if (!q || !out) return fail(LLAMA_E_ARG, "NULL buffer");
  if (exec < 0 || exec >= m->d.nexec)
    return fail(LLAMA_E_ARG, "execution %d outside 0..%d", exec, m->d.nexec - 1);
  if (prompt_kernel < 0 || prompt_kernel > 2)
    return fail(LLAMA_E_ARG, "prompt_kernel %d is not 0, 1 or 2", prompt_kernel);
  const int maxr = prompt_kernel ? m->cfg.max_chunk_rows : m->d.Mdec;
  if (rows < 1 || rows > maxr) return fail(LLAMA_E_ARG, "rows %d outside 1..%d", rows, maxr);
  if (pos0 < 0 || (int64_t)pos0 + rows > kv->length)
    return fail(LLAMA_E_POSITION, "positions %d..%d are not all in the cache (%d)", pos0,
                pos0 + rows - 1, kv->length);
  hipStream_t s = (hipStream_t)hip_stream;
  (void)hipGetLastError();
  Pass p{m, &kv, 1, rows, {0}, s};
  p.pos0[0] = pos0;
  RowTable tab = table_for(p, exec);
  const Dims& d = m->d;
  if (prompt_kernel)
    launch_attn_prefill(q, tab.k[0], tab.v[0], rows, pos0, d.nq, d.nkv, d.d, out, out32,
                        prompt_kernel == 2, s);
  else
    launch_attn_decode(q, tab, rows, d.nq, d.nkv, d.d, m->at<float>(m->L.part), out, out32, s);
  return dev_check("test attention launch");
}

int llama_sample_noalloc(const void* logits, int32_t vocab, int32_t rows, int64_t ld,
                         float temperature, int32_t top_k, float top_p, const float* u,
                         int32_t* tokens, void* hip_stream) {
  static_assert(LLAMA_SAMPLE_MAX_ROWS <= SAMPLE_NOALLOC_MAX_ROWS, "scratch rows");
  static_assert((size_t)(LLAMA_SAMPLE_NOALLOC_MAX_VOCAB + 4095) / 4096 <= SAMPLE_NOALLOC_MAX_CHUNKS,
                "scratch chunks");
  if (!logits || !u || !tokens) return fail(LLAMA_E_ARG, "NULL buffer");
  if (vocab < 1 || vocab > LLAMA_SAMPLE_NOALLOC_MAX_VOCAB)
    return fail(LLAMA_E_ARG, "vocab %d outside 1..%d", vocab, LLAMA_SAMPLE_NOALLOC_MAX_VOCAB);
  if (rows < 1 || rows > LLAMA_SAMPLE_MAX_ROWS)
    return fail(LLAMA_E_ARG, "rows %d outside 1..%d", rows, LLAMA_SAMPLE_MAX_ROWS);
  if (ld < vocab) return fail(LLAMA_E_ARG, "row stride %lld below the vocabulary %d", (long long)ld, vocab);
  if (!(temperature > 0.0f) || !(temperature < INFINITY))
    return fail(LLAMA_E_ARG, "temperature must be positive and finite");
  if (top_k < 1 || top_k > LLAMA_SAMPLE_MAX_TOP_K || top_k > vocab)
    return fail(LLAMA_E_ARG, "top_k %d outside 1..%d", top_k, std::min(LLAMA_SAMPLE_MAX_TOP_K, vocab));
  if (!(top_p > 0.0f) || !(top_p <= 1.0f)) return fail(LLAMA_E_ARG, "top_p must lie in (0, 1]");
  if ((int64_t)sample_chunks(vocab) * top_k > SAMPLE_NOALLOC_MAX_CAND)
    return fail(LLAMA_E_ARG, "top_k %d too large for a vocabulary of %d (scratch holds %d candidates per row)",
                top_k, vocab, SAMPLE_NOALLOC_MAX_CAND);
  if (sample_noalloc_scratch_bytes() != LLAMA_SAMPLE_NOALLOC_SCRATCH_BYTES)
    return fail(LLAMA_E_DEVICE, "scratch size mismatch");
  (void)hipGetLastError();
  const hipError_t e = launch_sample_noalloc(logits, vocab, ld, rows, top_k, temperature, top_p, u,
                                             tokens, (hipStream_t)hip_stream);
  if (e != hipSuccess) return fail(LLAMA_E_DEVICE, "sampling without allocation: %s", hipGetErrorString(e));
  return LLAMA_OK;
}

int llama_check_finite(llama_model* m, void* hip_stream) {
  if (!m) return fail(LLAMA_E_ARG, "model is NULL");
  hipStream_t s = (hipStream_t)hip_stream;
  int flag = 0;
  if (hipMemcpyAsync(&flag, m->ws + m->L.flag, sizeof(int), hipMemcpyDeviceToHost, s) !=
          hipSuccess ||
      hipStreamSynchronize(s) != hipSuccess)
    return fail(LLAMA_E_DEVICE, "reading the non-finite flag failed");
  if (flag) {
    launch_fill_zero(m->at<int>(m->L.flag), 64, s);
    (void)hipStreamSynchronize(s);
    return fail(LLAMA_E_NONFINITE, "a greedy or sampled draw met a logit row holding NaN or Inf");
  }
  return LLAMA_OK;
}

static void release_timing(llama_model* m) {
  for (hipEvent_t e : m->tev) (void)hipEventDestroy(e);
  m->tev.clear();
  m->tused = 0;
  m->timing_kernel = 0;
}

int llama_set_timing(llama_model* m, int32_t kernel, int32_t max_launches) {
  if (!m) return fail(LLAMA_E_ARG, "model is NULL");
  if (kernel < LLAMA_TIMING_OFF || kernel > LLAMA_TIMING_PREFILL_ATTN)
    return fail(LLAMA_E_ARG, "unknown kernel class %d", kernel);
  release_timing(m);
  if (kernel == LLAMA_TIMING_OFF) return LLAMA_OK;
  if (max_launches < 1 || max_launches > (1 << 20))
    return fail(LLAMA_E_ARG, "max_launches %d outside 1..2^20", max_launches);
  m->tev.resize((size_t)max_launches * 2);
  for (auto& e : m->tev) {
    if (hipEventCreate(&e) != hipSuccess) {
      e = nullptr;
      release_timing(m);
      return fail(LLAMA_E_DEVICE, "hipEventCreate failed");
    }
  }
  m->timing_kernel = kernel;
  return LLAMA_OK;
}

int llama_timing_read(llama_model* m, double* total_ms, int64_t* launches) {
  if (!m || !total_ms || !launches) return fail(LLAMA_E_ARG, "NULL argument");
  double sum = 0.0;
  for (size_t i = 0; i + 1 < m->tused; i += 2) {
    float ms = 0.f;
    if (hipEventSynchronize(m->tev[i + 1]) != hipSuccess ||
        hipEventElapsedTime(&ms, m->tev[i], m->tev[i + 1]) != hipSuccess)
      return fail(LLAMA_E_DEVICE, "reading timing events failed");
    sum += ms;
  }
  *total_ms = sum;
  *launches = (int64_t)(m->tused / 2);
  m->tused = 0;
  return LLAMA_OK;
}

void llama_kv_free(llama_kv* kv) { delete kv; }
void llama_free(llama_model* m) {
  if (m) release_timing(m);
  delete m;
}
const char* llama_last_error(void) { return g_err.c_str(); }

}  // extern "C"
