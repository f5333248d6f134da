// C-ABI entry points: host-side validation, decoder state and the launch
// sequence of a step.  Every check runs before any HIP call, so a refused
// call leaves the decoder unchanged and touches no device.
#include <dlfcn.h>
#include <hip/hip_runtime_api.h>

#include <algorithm>
#include <cmath>
#include <cstdarg>
#include <cstdio>
#include <cstdlib>
#include <cstring>
#include <map>
#include <mutex>
#include <string>
#include <vector>

#include "../../include/atd.h"
#include "internal.h"

using namespace atd;

struct atd_decoder {
  atd_config cfg{};
  std::vector<atd_layer_weights> layers;
  const float* final_norm = nullptr;
  const void* in_proj = nullptr;       // [hidden, in_dim] or null
  const float* in_proj_bias = nullptr;
  int in_dim = 0;                      // width of the input rows
  float* xin = nullptr;                // input rows before the projection [max_rows, in_dim]
  std::vector<const void*> heads, tables;
  std::vector<int32_t> table_vocab;
  // host mirror of every slot
  std::vector<int32_t> pos, cap;
  std::vector<char> attached;
  std::vector<std::vector<void*>> kp, vp;
  int device = 0;
  // device scratch, one allocation
  void* mem = nullptr;
  float *cos_t = nullptr, *sin_t = nullptr;
  float *rcos = nullptr, *rsin = nullptr;  // RoPE rows of an *_mrope call [max_rows, D/2]
  float *x = nullptr, *qkv = nullptr, *q = nullptr, *o = nullptr, *act = nullptr;
  float *pml = nullptr, *pacc = nullptr;
  int* attn_ticket = nullptr;  // [max_rows, Hkv] ticket counters of the attention
  void** kv_tab = nullptr;
  int *slot_pos = nullptr, *slot_cap = nullptr;
  float* part = nullptr;       // argmax partials [max_rows, nblk, 3]
  uint2* samp = nullptr;       // sampler chunk candidates [sample_blocks(V), kTopKMax]
  bool mma = false;            // MFMA path for chunks of >= kMmaMinRows rows
  float* mpart = nullptr;      // split-K partials of the MFMA GEMMs
  int mma_rows = 0;            // most rows of one MFMA chunk (multiple of kMmaRows)
  float* mss = nullptr;        // row sums of squares [mma_rows, ceil(h / kSsCols)]
  uint16_t *mhi = nullptr, *mlo = nullptr;  // GEMM input as bf16 hi/lo [mma_rows, Kmax]
  // second hi/lo pair of a <= 64-row chunk [kMmaRows, Kmax]: a GEMM whose
  // epilogue writes the next input reads the other pair
  uint16_t *mhi2 = nullptr, *mlo2 = nullptr;
  int* mticket = nullptr;      // [max column tiles] tickets of the decode GEMMs
  // the MFMA decode path's copy of the weights in B-operand order (one
  // allocation, made at decoder_create): per layer q/k/v, o, gate/up
  // interleaved, down; per head
  void* bmem = nullptr;
  std::vector<const uint16_t*> bq_sw, bo_sw, bgu_sw, bdown_sw, bhead_sw;
  int32_t* slot_list = nullptr;  // device [max_rows]: slots of a decoder_step_slots call
  std::vector<int32_t> step_slots;  // host copy of that list while its call enqueues
  int32_t* counter = nullptr;  // token counter of decoder_generate
  int32_t* ctl_base = nullptr; // first choice index of a controlled generate call
  size_t part_floats = 0;      // capacity of pacc in floats / D
  bool dry = false;  // ATD_FLAG_DRY_RUN: host state only, no HIP calls
  // stage timing (decoder_time_stage): layers to enqueue, -1 = all
  int only_stage = -1;
  // L2 prefetch from the step attention launch: bytes of the O projection
  // and gate/up weights to pull ahead (0 = none)
  size_t pf_budget = 0;
  // dense bf16 weights streamed with the nontemporal cache policy (weights
  // larger than the memory-side cache, which they could not stay in anyway)
  bool stream_nt = false;
  // graph cache of decoder_generate
  hipStream_t cap_stream = nullptr;
  struct GraphEntry {
    std::vector<int64_t> key;
    hipGraphExec_t exec;
  };
  std::vector<GraphEntry> graphs;
  std::string err;
};

namespace {

thread_local std::string g_err;

// ROCTx ranges around the enqueue of each entry point (and each layer of a
// step), for timelines: on only when ATD_ROCTX=1.  The ROCTx library is
// opened on first use, so a default build depends on nothing beyond HIP.
struct Roctx {
  int (*push)(const char*) = nullptr;
  int (*pop)() = nullptr;
};
const Roctx& roctx() {
  static Roctx r;
  static std::once_flag once;
  std::call_once(once, [] {
    const char* on = getenv("ATD_ROCTX");
    if (!on || strcmp(on, "1") != 0) return;
    void* h = dlopen("librocprofiler-sdk-roctx.so.1", RTLD_NOW | RTLD_GLOBAL);
    if (!h) h = dlopen("libroctx64.so", RTLD_NOW | RTLD_GLOBAL);
    if (!h) return;
    r.push = reinterpret_cast<int (*)(const char*)>(dlsym(h, "roctxRangePushA"));
    r.pop = reinterpret_cast<int (*)()>(dlsym(h, "roctxRangePop"));
    if (!r.push || !r.pop) r = Roctx{};
  });
  return r;
}
struct Range {
  bool on;
  explicit Range(const char* name) : on(roctx().push != nullptr) {
    if (on) roctx().push(name);
  }
  ~Range() {
    if (on) roctx().pop();
  }
  Range(const Range&) = delete;
  Range& operator=(const Range&) = delete;
};

int fail(atd_decoder* d, int code, const char* fmt, ...) {
  char buf[512];
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(buf, sizeof buf, fmt, ap);
  va_end(ap);
  if (d)
    d->err = buf;
  else
    g_err = buf;
  return code;
}

int hip_fail(atd_decoder* d, hipError_t e, const char* what) {
  return fail(d, ATD_ERR_DEVICE, "%s failed: %s (%s)", what, hipGetErrorName(e),
              hipGetErrorString(e));
}

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

int kv_elem_bytes(const atd_config& c) { return c.kv_dtype == ATD_BF16 ? 2 : 4; }

size_t align256(size_t n) { return (n + 255) & ~size_t(255); }

int check_config(const atd_config* c) {
  if (!c) return fail(nullptr, ATD_ERR_INVALID_ARG, "cfg is NULL");
  if (c->dtype != ATD_F32 && c->dtype != ATD_BF16)
    return fail(nullptr, ATD_ERR_DTYPE, "dtype %d is not ATD_F32 (0) or ATD_BF16 (1)", c->dtype);
  if (c->kv_dtype != ATD_F32 && c->kv_dtype != ATD_BF16)
    return fail(nullptr, ATD_ERR_DTYPE, "kv_dtype %d is not ATD_F32 (0) or ATD_BF16 (1)",
                c->kv_dtype);
  if (c->n_layers < 1 || c->n_layers > kMaxLayers)
    return fail(nullptr, ATD_ERR_UNSUPPORTED, "n_layers %d outside [1, %d]", c->n_layers,
                kMaxLayers);
  if (c->hidden < 8 || c->hidden % 8 || c->hidden > 8192)
    return fail(nullptr, ATD_ERR_UNSUPPORTED, "hidden %d: must be a multiple of 8 in [8, 8192]",
                c->hidden);
  if (c->ffn < 8 || c->ffn % 8 || c->ffn > 8192)
    return fail(nullptr, ATD_ERR_UNSUPPORTED, "ffn %d: must be a multiple of 8 in [8, 8192]",
                c->ffn);
  if (c->head_dim != 64 && c->head_dim != 128)
    return fail(nullptr, ATD_ERR_UNSUPPORTED, "head_dim %d: only 64 and 128 are implemented",
                c->head_dim);
  if (c->n_q_heads < 1 || c->n_kv_heads < 1 || c->n_q_heads % c->n_kv_heads)
    return fail(nullptr, ATD_ERR_SHAPE, "n_q_heads %d is not a multiple of n_kv_heads %d",
                c->n_q_heads, c->n_kv_heads);
  {
    const int r = c->n_q_heads / c->n_kv_heads;
    if (r != 1 && r != 2 && r != 4 && r != 8)
      return fail(nullptr, ATD_ERR_UNSUPPORTED, "n_q_heads / n_kv_heads = %d not in {1,2,4,8}",
                  r);
  }
  if ((long)c->n_q_heads * c->head_dim > 8192)
    return fail(nullptr, ATD_ERR_UNSUPPORTED, "n_q_heads * head_dim %d > 8192",
                c->n_q_heads * c->head_dim);
  if (c->dtype == ATD_F32 &&
      (c->hidden > 4096 || c->ffn > 4096 || c->n_q_heads * c->head_dim > 4096))
    return fail(nullptr, ATD_ERR_UNSUPPORTED,
                "float32 weights need hidden, ffn and n_q_heads*head_dim <= 4096");
  if (c->vocab < 2)
    return fail(nullptr, ATD_ERR_SHAPE, "vocab %d < 2", c->vocab);
  if (c->n_lm_heads < 1)
    return fail(nullptr, ATD_ERR_SHAPE, "n_lm_heads %d < 1", c->n_lm_heads);
  if (c->n_tables < 1 || c->n_tables > kMaxTables)
    return fail(nullptr, ATD_ERR_UNSUPPORTED, "n_tables %d outside [1, %d]", c->n_tables,
                kMaxTables);
  if (c->qk_norm != 0 && c->qk_norm != 1)
    return fail(nullptr, ATD_ERR_INVALID_ARG, "qk_norm %d is not 0 or 1", c->qk_norm);
  if (c->qkv_bias != 0 && c->qkv_bias != 1)
    return fail(nullptr, ATD_ERR_INVALID_ARG, "qkv_bias %d is not 0 or 1", c->qkv_bias);
  if (!(c->rope_theta > 0.0) || !std::isfinite(c->rope_theta))
    return fail(nullptr, ATD_ERR_INVALID_ARG, "rope_theta %g is not positive", c->rope_theta);
  if (!(c->rms_eps >= 0.0f) || !std::isfinite(c->rms_eps))
    return fail(nullptr, ATD_ERR_INVALID_ARG, "rms_eps %g is negative", (double)c->rms_eps);
  if (c->max_slots < 1 || c->max_slots > 65536)
    return fail(nullptr, ATD_ERR_CAPACITY, "max_slots %d outside [1, 65536]", c->max_slots);
  if (c->max_rows < 1 || c->max_rows > 65536)
    return fail(nullptr, ATD_ERR_CAPACITY, "max_rows %d outside [1, 65536]", c->max_rows);
  if (c->max_ctx < 1 || c->max_ctx > (1 << 20))
    return fail(nullptr, ATD_ERR_CAPACITY, "max_ctx %d outside [1, 2^20]", c->max_ctx);
  if (c->flags & ~(ATD_FLAG_DRY_RUN | ATD_FLAG_NO_MFMA | ATD_FLAG_NO_L2_PREFETCH))
    return fail(nullptr, ATD_ERR_INVALID_ARG, "unknown flags 0x%x", (unsigned)c->flags);
  {
    const int* ms = c->mrope_sections;
    const int half = c->head_dim / 2;
    const bool none = ms[0] == 0 && ms[1] == 0 && ms[2] == 0;
    if (!none && (ms[0] < 0 || ms[1] < 0 || ms[2] < 0 || ms[0] + ms[1] + ms[2] != half ||
                  3 * std::max(ms[1], ms[2]) > half))
      return fail(nullptr, ATD_ERR_INVALID_ARG,
                  "mrope_sections {%d, %d, %d}: need s_t + s_h + s_w = D/2 = %d and "
                  "3 max(s_h, s_w) <= D/2",
                  ms[0], ms[1], ms[2], half);
  }
  if (c->weight_format != ATD_WFMT_DENSE && c->weight_format != ATD_WFMT_Q8 &&
      c->weight_format != ATD_WFMT_Q4)
    return fail(nullptr, ATD_ERR_DTYPE, "weight_format %d is not ATD_WFMT_DENSE/Q8/Q4",
                c->weight_format);
  if (c->input_dim != 0 &&
      (c->input_dim < 8 || c->input_dim % 8 || c->input_dim > (c->dtype == ATD_F32 ? 4096 : 8192)))
    return fail(nullptr, ATD_ERR_UNSUPPORTED,
                "input_dim %d: must be 0 or a multiple of 8 in [8, %d]", c->input_dim,
                c->dtype == ATD_F32 ? 4096 : 8192);
  if (c->weight_format != ATD_WFMT_DENSE &&
      (c->hidden % kQBlock || c->ffn % kQBlock || (c->n_q_heads * c->head_dim) % kQBlock))
    return fail(nullptr, ATD_ERR_SHAPE,
                "quantized weights need hidden %d, ffn %d and n_q_heads*head_dim %d to be "
                "multiples of %d",
                c->hidden, c->ffn, c->n_q_heads * c->head_dim, kQBlock);
  return ATD_OK;
}

// Weight type of the seven per-layer matrices (dense bf16 of a decoder whose
// weights exceed the memory-side cache: streamed nontemporally).
int layer_wtype(const atd_decoder* d) {
  const atd_config& c = d->cfg;
  if (c.weight_format == ATD_WFMT_Q8) return kWQ8;
  if (c.weight_format == ATD_WFMT_Q4) return kWQ4;
  return c.dtype != ATD_BF16 ? kWF32 : d->stream_nt ? kWBF16NT : kWBF16;
}
// ... and of the LM heads (always dense)
int head_wtype(const atd_decoder* d) {
  return d->cfg.dtype != ATD_BF16 ? kWF32 : d->stream_nt ? kWBF16NT : kWBF16;
}

// Bytes of a decoder's dense matrices: the seven per layer, the LM heads and
// the input projection (when the input rows are narrower or wider than h).
size_t dense_weight_bytes(const atd_config& c) {
  const size_t h = c.hidden, nq = (size_t)c.n_q_heads * c.head_dim,
               nkv = (size_t)c.n_kv_heads * c.head_dim, F = c.ffn;
  const size_t per_layer = (nq + 2 * nkv) * h + h * nq + 3 * F * h;
  const size_t in_proj = c.input_dim && c.input_dim != c.hidden ? (size_t)c.input_dim * h : 0;
  const size_t el = c.dtype == ATD_BF16 ? 2 : 4;
  return (per_layer * c.n_layers + (size_t)c.n_lm_heads * c.vocab * h + in_proj) * el;
}

#define NEED(ptr, name)                                                                    \
  do {                                                                                     \
    if (!(ptr)) return fail(nullptr, ATD_ERR_INVALID_ARG, "%s is NULL", name);              \
    if (!aligned16(ptr)) return fail(nullptr, ATD_ERR_INVALID_ARG, "%s %p not 16-byte aligned", \
                                     name, (const void*)(ptr));                             \
  } while (0)

int check_weights(const atd_config* c, const atd_weights* w) {
  if (!w) return fail(nullptr, ATD_ERR_INVALID_ARG, "weights is NULL");
  if (!w->layers || !w->lm_heads || !w->tables || !w->table_vocab)
    return fail(nullptr, ATD_ERR_INVALID_ARG, "weights has a NULL host array");
  char name[64];
  for (int l = 0; l < c->n_layers; ++l) {
    const atd_layer_weights& L = w->layers[l];
#define LW(field)                                                 \
  snprintf(name, sizeof name, "layers[%d]." #field, l);           \
  NEED(L.field, name);
    LW(attn_norm) LW(wq) LW(wk) LW(wv) LW(wo) LW(mlp_norm) LW(w_gate) LW(w_up) LW(w_down)
    {
      const void* sc[7] = {L.wq_scale, L.wk_scale, L.wv_scale, L.wo_scale,
                           L.w_gate_scale, L.w_up_scale, L.w_down_scale};
      static const char* const sn[7] = {"wq_scale", "wk_scale", "wv_scale", "wo_scale",
                                        "w_gate_scale", "w_up_scale", "w_down_scale"};
      for (int j = 0; j < 7; ++j) {
        if (c->weight_format == ATD_WFMT_DENSE) {
          if (sc[j])
            return fail(nullptr, ATD_ERR_INVALID_ARG,
                        "layers[%d].%s is set but weight_format is dense", l, sn[j]);
        } else if (!sc[j] || ((uintptr_t)sc[j] & 1)) {
          return fail(nullptr, ATD_ERR_INVALID_ARG, "layers[%d].%s %p is NULL or odd", l, sn[j],
                      sc[j]);
        }
      }
    }
    if (c->qkv_bias) {
      LW(bq) LW(bk) LW(bv)
    } else if (L.bq || L.bk || L.bv) {
      return fail(nullptr, ATD_ERR_INVALID_ARG,
                  "layers[%d] has q/k/v bias pointers but qkv_bias = 0", l);
    }
    if (c->qk_norm) {
      LW(q_norm) LW(k_norm)
    } else if (L.q_norm || L.k_norm) {
      return fail(nullptr, ATD_ERR_INVALID_ARG,
                  "layers[%d] has QK-norm gains but qk_norm = 0", l);
    }
#undef LW
  }
  NEED(w->final_norm, "final_norm");
  if (w->in_proj) {
    NEED(w->in_proj, "in_proj");
    if (w->in_proj_bias) NEED(w->in_proj_bias, "in_proj_bias");
  } else if (c->input_dim != 0 && c->input_dim != c->hidden) {
    return fail(nullptr, ATD_ERR_INVALID_ARG,
                "input_dim %d differs from hidden %d but in_proj is NULL", c->input_dim,
                c->hidden);
  } else if (w->in_proj_bias) {
    return fail(nullptr, ATD_ERR_INVALID_ARG, "in_proj_bias is set but in_proj is NULL");
  }
  for (int j = 0; j < c->n_lm_heads; ++j) {
    snprintf(name, sizeof name, "lm_heads[%d]", j);
    NEED(w->lm_heads[j], name);
  }
  for (int g = 0; g < c->n_tables; ++g) {
    snprintf(name, sizeof name, "tables[%d]", g);
    NEED(w->tables[g], name);
    if (w->table_vocab[g] < 1)
      return fail(nullptr, ATD_ERR_SHAPE, "table_vocab[%d] = %d < 1", g, w->table_vocab[g]);
  }
  return ATD_OK;
}

SlotTables slots_of(const atd_decoder* d) {
  SlotTables st;
  st.kv = d->kv_tab;
  st.pos = d->slot_pos;
  st.cap = d->slot_cap;
  st.L = d->cfg.n_layers;
  return st;
}


// Split-count target of the attention for M rows: enough waves to spread the
// KV stream over the chip, few enough that each split carries real work.
int attn_waves(int M) { return M <= 4 ? kAttnWavesFew : kAttnWavesMax; }

// Launch a stage unless decoder_time_stage restricts the sequence to another.
#define STAGE(stage, call)                                              \
  do {                                                                  \
    if (d->only_stage < 0 || d->only_stage == (stage))                  \
      if ((e = (call)) != hipSuccess) return e;                         \
  } while (0)

// The per-layer launch sequence for M rows (decode step or prefill block).
AttnArgs attn_args(const atd_decoder* d, RowMap rows, int l, int M, int max_len_bound,
                   bool fused) {
  const atd_config& c = d->cfg;
  const atd_layer_weights& W = d->layers[l];
  const int waves = attn_waves(M);
  AttnArgs a{};
  a.fused = fused;
  a.qkv = d->qkv;
  a.q_norm = (const float*)W.q_norm;
  a.k_norm = (const float*)W.k_norm;
  a.qk_norm = c.qk_norm;
  a.eps = c.rms_eps;
  a.cos_t = rows.rope_rows ? d->rcos : d->cos_t;
  a.sin_t = rows.rope_rows ? d->rsin : d->sin_t;
  a.q = d->q;
  a.st = slots_of(d);
  a.rows = rows;
  a.layer = l;
  a.M = M;
  a.Hq = c.n_q_heads;
  a.Hkv = c.n_kv_heads;
  a.nsplit_max = attn_max_splits(max_len_bound, M, c.n_kv_heads, waves);
  a.waves = waves;
  if (rows.mode == kRowsPrefill || M == 1) {  // one slot: pass its rows directly
    const int slot = rows.mode == kRowsPrefill ? rows.slot0
                     : rows.slot_list               ? d->step_slots[rows.row0]
                                                    : rows.slot0 + rows.row0;
    a.k_direct = d->kp[slot][l];
    a.v_direct = d->vp[slot][l];
    a.cap_direct = d->cap[slot];
  }
  a.scale = 1.0f / std::sqrt((float)c.head_dim);
  a.pml = d->pml;
  a.pacc = d->pacc;
  a.ticket = d->attn_ticket;
  a.o = d->o;
  return a;
}

// Attention launch; its partials must fit the buffer sized at creation (a
// broken sizing invariant is reported, never written past).
hipError_t attention(const atd_decoder* d, const AttnArgs& a, hipStream_t s) {
  if ((size_t)a.M * a.Hq * a.nsplit_max > d->part_floats) return hipErrorInvalidValue;
  return launch_attention(a, d->cfg.kv_dtype == ATD_BF16, d->cfg.head_dim, a.Hq / a.Hkv, s);
}

RopeArgs rope_args(const atd_decoder* d, RowMap rows, int l, int M) {
  const atd_config& c = d->cfg;
  const atd_layer_weights& W = d->layers[l];
  RopeArgs r{};
  r.qkv = d->qkv;
  r.q_out = d->q;
  r.q_norm = (const float*)W.q_norm;
  r.k_norm = (const float*)W.k_norm;
  r.eps = c.rms_eps;
  r.cos_t = rows.rope_rows ? d->rcos : d->cos_t;
  r.sin_t = rows.rope_rows ? d->rsin : d->sin_t;
  r.st = slots_of(d);
  r.rows = rows;
  r.layer = l;
  r.M = M;
  r.Hq = c.n_q_heads;
  r.Hkv = c.n_kv_heads;
  r.D = c.head_dim;
  r.qk_norm = c.qk_norm;
  return r;
}

// The prefetch plan of layer l's step attention: the O projection's weights,
// then as many gate/up blocks as the budget leaves, then down blocks if gate/up
// fit whole (whole blocks only, so no load passes the end of a matrix).
L2Prefetch prefetch_plan(const atd_decoder* d, const atd_layer_weights& W, int wt, int wgs) {
  L2Prefetch p{};
  const size_t budget = d->pf_budget * std::min(wgs, kPfWorkgroups) / kPfWorkgroups;
  if (budget == 0) return p;
  const atd_config& c = d->cfg;
  const int h = c.hidden, nq = c.n_q_heads * c.head_dim;
  int br;
  size_t rb;
  gemv_block_rows(h, nq, wt, br, rb);
  // no slice unless it can take the whole O projection (the next launch): a
  // part of it leaves that launch waiting on HBM all the same, while the
  // slice's loads lengthen a short attention launch (measured on the 0.6B
  // Talker, 256-row buckets: 404 frames/s without the slice, 385 with 3 MiB)
  if (budget < (size_t)h / br * br * rb) return p;
  p.base[0] = (const char*)W.wo;
  p.bb[0] = (size_t)br * rb;
  p.nblk[0] = h / br;
  size_t left = budget - (size_t)p.nblk[0] * p.bb[0];
  gemv_block_rows(c.ffn, h, wt, br, rb);
  const size_t bb = (size_t)br * rb;
  const int ng = (int)std::min<size_t>(c.ffn / br, left / (2 * bb));
  p.nreg = 1;
  if (ng > 0) {
    p.base[1] = (const char*)W.w_gate;
    p.base[2] = (const char*)W.w_up;
    p.bb[1] = p.bb[2] = bb;
    p.nblk[1] = p.nblk[2] = ng;
    p.nreg = 3;
    left -= 2 * (size_t)ng * bb;
  }
  if (ng == c.ffn / br) {
    gemv_block_rows(h, c.ffn, wt, br, rb);
    p.bb[3] = (size_t)br * rb;
    const int nd = (int)std::min<size_t>(h / br, left / p.bb[3]);
    if (nd > 0) {
      p.base[3] = (const char*)W.w_down;
      p.nblk[3] = nd;
      p.nreg = 4;
    }
  }
  return p;
}

// GEMV path: the per-layer launch sequence for fewer than kMmaMinRows rows (or any
// rows without the matrix-core path: float32 or quantized weights, ATD_FLAG_NO_MFMA).
hipError_t run_layers_gemv(atd_decoder* d, RowMap rows, int M, int max_len_bound, float* x,
                           hipStream_t s) {
  const atd_config& c = d->cfg;
  const int h = c.hidden, D = c.head_dim, Hq = c.n_q_heads, Hkv = c.n_kv_heads;
  const int nq = Hq * D, nkv = Hkv * D, nqkv = nq + 2 * nkv;
  const int wt = layer_wtype(d);
  const int kv_bf16 = c.kv_dtype == ATD_BF16;
  const bool fused = rows.mode == kRowsStep;
  hipError_t e = hipSuccess;
  for (int l = 0; l < c.n_layers; ++l) {
    const Range range("layer");
    const atd_layer_weights& W = d->layers[l];
    GemvArgs g{};
    g.W[0] = W.wq;
    g.W[1] = W.wk;
    g.W[2] = W.wv;
    g.S[0] = (const uint16_t*)W.wq_scale;
    g.S[1] = (const uint16_t*)W.wk_scale;
    g.S[2] = (const uint16_t*)W.wv_scale;
    g.bias[0] = (const float*)W.bq;
    g.bias[1] = (const float*)W.bk;
    g.bias[2] = (const float*)W.bv;
    g.seg_end[0] = nq;
    g.seg_end[1] = nq + nkv;
    g.seg_end[2] = nqkv;
    g.x = x;
    g.ldx = h;
    g.gain = (const float*)W.attn_norm;
    g.eps = c.rms_eps;
    g.out = d->qkv;
    g.ldo = nqkv;
    g.K = h;
    g.N = nqkv;
    g.M = M;
    STAGE(ATD_STAGE_QKV, launch_gemv(g, kEpiStore, true, wt, s));
    // prefill rows of one slot read each other's keys: append them all first
    if (!fused) STAGE(ATD_STAGE_ROPE, launch_rope_append(rope_args(d, rows, l, M), kv_bf16, s));
    {
      AttnArgs aa = attn_args(d, rows, l, M, max_len_bound, fused);
      // only where a row's keys can span several blocks: their ticket merge
      // makes the launch long enough to hide the loads (a one-block launch,
      // e.g. over the Code Predictor's 16-row cache, would only be lengthened);
      // the prefetch slice has one workgroup per (block, KV head)
      const int gx = (aa.nsplit_max + 3) / 4;
      if (fused && gx > 1) aa.pf = prefetch_plan(d, W, wt, gx * c.n_kv_heads);
      STAGE(ATD_STAGE_ATTN, attention(d, aa, s));
    }

    GemvArgs op{};
    op.W[0] = W.wo;
    op.S[0] = (const uint16_t*)W.wo_scale;
    op.seg_end[0] = op.seg_end[1] = op.seg_end[2] = h;
    op.x = d->o;
    op.ldx = nq;
    op.out = x;
    op.ldo = h;
    op.K = nq;
    op.N = h;
    op.M = M;
    STAGE(ATD_STAGE_OPROJ, launch_gemv(op, kEpiResidual, false, wt, s));

    GemvArgs gu{};
    gu.W[0] = W.w_gate;
    gu.W2 = W.w_up;
    gu.S[0] = (const uint16_t*)W.w_gate_scale;
    gu.S2 = (const uint16_t*)W.w_up_scale;
    gu.seg_end[0] = gu.seg_end[1] = gu.seg_end[2] = c.ffn;
    gu.x = x;
    gu.ldx = h;
    gu.gain = (const float*)W.mlp_norm;
    gu.eps = c.rms_eps;
    gu.out = d->act;
    gu.ldo = c.ffn;
    gu.K = h;
    gu.N = c.ffn;
    gu.M = M;
    STAGE(ATD_STAGE_GATEUP, launch_gemv(gu, kEpiSwiglu, true, wt, s));

    GemvArgs dn{};
    dn.W[0] = W.w_down;
    dn.S[0] = (const uint16_t*)W.w_down_scale;
    dn.seg_end[0] = dn.seg_end[1] = dn.seg_end[2] = h;
    dn.x = d->act;
    dn.ldx = c.ffn;
    dn.out = x;
    dn.ldo = h;
    dn.K = c.ffn;
    dn.N = h;
    dn.M = M;
    STAGE(ATD_STAGE_DOWN, launch_gemv(dn, kEpiResidual, false, wt, s));
  }
  return e;
}

// GEMV path: final RMSNorm + LM head for M rows.
hipError_t run_head_gemv(atd_decoder* d, const float* xrows, int M, int head, float* y_out,
                         float* logits, hipStream_t s) {
  const atd_config& c = d->cfg;
  hipError_t e = hipSuccess;
  GemvArgs g{};
  g.W[0] = d->heads[head];
  g.seg_end[0] = g.seg_end[1] = g.seg_end[2] = c.vocab;
  g.x = xrows;
  g.ldx = c.hidden;
  g.gain = d->final_norm;
  g.eps = c.rms_eps;
  g.out = logits;
  g.ldo = c.vocab;
  g.y_out = y_out;
  g.K = c.hidden;
  g.N = c.vocab;
  g.M = M;
  STAGE(ATD_STAGE_HEAD, launch_gemv(g, kEpiStore, true, head_wtype(d), s));
  return e;
}

// MFMA path pieces -----------------------------------------------------------
// GEMM of the chunk's activations (d->mhi / d->mlo, [kMmaRows, K]) with an
// [N, K] weight given as up to three row segments; split partials into d->mpart.
hipError_t mma_gemm(atd_decoder* d, const void* w0, const void* w1, const void* w2, int e0,
                    int e1, int N, int K, int M, hipStream_t s) {
  const int tiles = (M + kMmaRows - 1) / kMmaRows;
  GemmArgs g{};
  g.hi = d->mhi;
  g.lo = d->mlo;
  g.W[0] = w0;
  g.W[1] = w1;
  g.W[2] = w2;
  g.seg_end[0] = e0;
  g.seg_end[1] = e1;
  g.seg_end[2] = N;
  g.K = K;
  g.N = N;
  g.kc = mma_kc(N, K, tiles);
  g.ks = mma_ks(N, K, tiles);
  g.mrows = tiles * kMmaRows;
  g.part = d->mpart;
  // several row tiles (prefill chunks): 128 x 128 output tiles share each
  // operand tile over more MFMAs, when they still give every compute unit a
  // workgroup (measured at 512 rows of the 1.7B shape: gate/up 92 -> 65 us,
  // QKV 33 -> 26, down 49 -> 46; the O projection's 128 workgroups: 18 -> 24,
  // so it stays on 64 x 64 tiles); one tile (decode streams) streams weights
  const long big = (long)((N + 127) / 128) * g.ks * ((g.mrows + 127) / 128);
  return tiles > 1 && big >= kMmaCUs ? launch_gemm_tile(g, s) : launch_gemm(g, s);
}

// Splits of the GEMM of an [N, K] weight over M rows (as mma_gemm takes them).
int mma_splits(int N, int K, int M) { return mma_ks(N, K, (M + kMmaRows - 1) / kMmaRows); }

// Reductions of the splits of the last GEMM (N columns, ks splits) over M rows.
ReduceArgs mma_red(atd_decoder* d, int N, int ks, int M, float* out, int ldo) {
  ReduceArgs r{};
  r.part = d->mpart;
  r.ks = ks;
  r.N = N;
  r.M = M;
  r.mrows = (M + kMmaRows - 1) / kMmaRows * kMmaRows;
  r.seg_end[0] = r.seg_end[1] = r.seg_end[2] = N;
  r.out = out;
  r.ldo = ldo;
  r.nss = (d->cfg.hidden + kSsCols - 1) / kSsCols;
  r.hn = d->cfg.hidden;
  r.eps = d->cfg.rms_eps;
  return r;
}

// x += splits (ks = 0: none), then x * gain as the next GEMM's hi/lo input
// and the row sums of squares for its norm factor
hipError_t mma_residual(atd_decoder* d, int ks, int M, float* x, const float* gain,
                        hipStream_t s, int frag = 0) {
  const int h = d->cfg.hidden;
  ReduceArgs r = mma_red(d, h, ks, M, x, h);
  r.frag = frag;
  r.ss = d->mss;
  r.gain = gain;
  r.hi = d->mhi;
  r.lo = d->mlo;
  return launch_reduce(r, kRedResidual, s);
}

// GEMM of a chunk of <= kMmaRows rows with its reduction and epilogue in
// one launch (k_gemm_dec): input hi / lo (64 x K, fragment order), an
// [N, K] weight in B-operand order (wb, made at decoder_create; kDecSwiglu:
// gate and up interleaved), bias segments ending at e0, e1, N; the
// epilogue's own fields of `g` are set by the caller.
hipError_t dec_gemm(atd_decoder* d, DecGemmArgs g, const uint16_t* hi, const uint16_t* lo,
                    const uint16_t* wb, int e0, int e1, int N, int K, int M, int epi,
                    hipStream_t s) {
  g.hi = hi;
  g.lo = lo;
  g.Wb = wb;
  g.nblk = (int)bfrag_blocks(N, epi == kDecSwiglu);
  g.seg_end[0] = e0;
  g.seg_end[1] = e1;
  g.seg_end[2] = N;
  g.K = K;
  g.N = N;
  g.M = M;
  g.cb = dec_cb(epi, K);
  g.kc = dec_kc(dec_tiles(N, epi, K), K);
  g.ks = (K + g.kc - 1) / g.kc;
  g.part = d->mpart;
  g.ticket = d->mticket;
  g.hn = d->cfg.hidden;
  g.eps = d->cfg.rms_eps;
  g.nss_in = (d->cfg.hidden + kSsCols - 1) / kSsCols;
  return launch_gemm_dec(g, epi, s);
}

// LM-head outputs of a call's rows (row 0 of the span the pointers address).
struct HeadOut {
  int head;
  float* y_out;    // [rows, h] or null
  float* logits;   // [rows, V]
};

// MFMA path for one chunk of 3..kMmaRows rows: every layer, then (if asked)
// the final norm and LM head.  Steps per layer: GEMM q/k/v of x*g, norm
// factor + bias -> attention (o as hi/lo) -> GEMM o, residual (+ x*g as
// hi/lo, sums of squares) -> GEMM gate/up, norm factor + SwiGLU (as hi/lo) ->
// GEMM down, residual (+ x*g for the next norm).  A chunk of one row tile
// (decode streams, short prefills) takes each step in one launch (k_gemm_dec);
// larger chunks run each GEMM's reduction as a launch of its own.
hipError_t run_chunk_mma(atd_decoder* d, RowMap rows, int M, int max_len_bound, float* x,
                         const HeadOut* ho, hipStream_t s) {
  const atd_config& c = d->cfg;
  const int h = c.hidden, D = c.head_dim, Hq = c.n_q_heads, Hkv = c.n_kv_heads;
  const int nq = Hq * D, nkv = Hkv * D, nqkv = nq + 2 * nkv, F = c.ffn;
  const int kv_bf16 = c.kv_dtype == ATD_BF16;
  const bool fused = rows.mode == kRowsStep;
  hipError_t e = hipSuccess;
  // one row tile: GEMMs with the reduction and epilogue in the same launch,
  // the hi / lo input (in MFMA-fragment order) alternating between two
  // buffers (a GEMM's epilogue writes the next GEMM's input while its other
  // workgroups still read)
  const bool one_tile = M <= kMmaRows;
  STAGE(ATD_STAGE_QKV,
        mma_residual(d, 0, M, x, (const float*)d->layers[0].attn_norm, s, one_tile ? 1 : 0));
  for (int l = 0; l < c.n_layers && one_tile; ++l) {
    const Range range("layer");
    const atd_layer_weights& W = d->layers[l];
    const float* next_gain =
        l + 1 < c.n_layers ? (const float*)d->layers[l + 1].attn_norm : d->final_norm;
    DecGemmArgs gq{};
    gq.out = d->qkv;
    gq.ldo = nqkv;
    gq.bias[0] = (const float*)W.bq;
    gq.bias[1] = (const float*)W.bk;
    gq.bias[2] = (const float*)W.bv;
    gq.ss_in = d->mss;
    STAGE(ATD_STAGE_QKV, dec_gemm(d, gq, d->mhi, d->mlo, d->bq_sw[l], nq, nq + nkv, nqkv, h,
                                  M, kDecStore, s));
    if (!fused) STAGE(ATD_STAGE_ROPE, launch_rope_append(rope_args(d, rows, l, M), kv_bf16, s));
    AttnArgs aa = attn_args(d, rows, l, M, max_len_bound, fused);
    aa.o_hi = d->mhi2;
    aa.o_lo = d->mlo2;
    aa.o_frag = 1;
    // many rows: the blocks' states are merged by a second launch, so no
    // block holds its compute unit through the ticket's round trips
    aa.defer = 1;
    if (fused)
      STAGE(ATD_STAGE_ATTN, attention(d, aa, s));
    else
      STAGE(ATD_STAGE_ATTN, launch_attn_prefill(aa, kv_bf16, D, Hq / Hkv, s));
    DecGemmArgs go{};
    go.out = x;
    go.ldo = h;
    go.ohi = d->mhi;
    go.olo = d->mlo;
    go.gain = (const float*)W.mlp_norm;
    go.ss_out = d->mss;
    STAGE(ATD_STAGE_OPROJ, dec_gemm(d, go, d->mhi2, d->mlo2, d->bo_sw[l], h, h, h, nq, M,
                                    kDecResidual, s));
    DecGemmArgs gg{};
    gg.ohi = d->mhi2;
    gg.olo = d->mlo2;
    gg.ss_in = d->mss;
    STAGE(ATD_STAGE_GATEUP, dec_gemm(d, gg, d->mhi, d->mlo, d->bgu_sw[l], 2 * F, 2 * F, 2 * F,
                                     h, M, kDecSwiglu, s));
    DecGemmArgs gd{};
    gd.out = x;
    gd.ldo = h;
    gd.ohi = d->mhi;
    gd.olo = d->mlo;
    gd.gain = next_gain;
    gd.ss_out = d->mss;
    STAGE(ATD_STAGE_DOWN, dec_gemm(d, gd, d->mhi2, d->mlo2, d->bdown_sw[l], h, h, h,
                                   F, M, kDecResidual, s));
  }
  for (int l = 0; l < c.n_layers && !one_tile; ++l) {
    const Range range("layer");
    const atd_layer_weights& W = d->layers[l];
    const float* next_gain =
        l + 1 < c.n_layers ? (const float*)d->layers[l + 1].attn_norm : d->final_norm;
    STAGE(ATD_STAGE_QKV, mma_gemm(d, W.wq, W.wk, W.wv, nq, nq + nkv, nqkv, h, M, s));
    ReduceArgs rq = mma_red(d, nqkv, mma_splits(nqkv, h, M), M, d->qkv, nqkv);
    rq.bias[0] = (const float*)W.bq;
    rq.bias[1] = (const float*)W.bk;
    rq.bias[2] = (const float*)W.bv;
    rq.seg_end[0] = nq;
    rq.seg_end[1] = nq + nkv;
    rq.ss = d->mss;
    STAGE(ATD_STAGE_QKV, launch_reduce(rq, kRedStore, s));
    if (!fused) STAGE(ATD_STAGE_ROPE, launch_rope_append(rope_args(d, rows, l, M), kv_bf16, s));
    AttnArgs aa = attn_args(d, rows, l, M, max_len_bound, fused);
    aa.o_hi = d->mhi;
    aa.o_lo = d->mlo;
    // a prefill chunk's rows share one slot: one pass over key tiles per
    // query tile; decode streams each read their own cache (split kernel)
    if (fused)
      STAGE(ATD_STAGE_ATTN, attention(d, aa, s));
    else
      STAGE(ATD_STAGE_ATTN, launch_attn_prefill(aa, kv_bf16, D, Hq / Hkv, s));
    STAGE(ATD_STAGE_OPROJ, mma_gemm(d, W.wo, W.wo, W.wo, h, h, h, nq, M, s));
    STAGE(ATD_STAGE_OPROJ, mma_residual(d, mma_splits(h, nq, M), M, x, (const float*)W.mlp_norm, s));
    STAGE(ATD_STAGE_GATEUP, mma_gemm(d, W.w_gate, W.w_up, W.w_up, F, 2 * F, 2 * F, h, M, s));
    ReduceArgs rg = mma_red(d, 2 * F, mma_splits(2 * F, h, M), M, nullptr, 0);
    rg.ss = d->mss;
    rg.hi = d->mhi;
    rg.lo = d->mlo;
    STAGE(ATD_STAGE_GATEUP, launch_reduce(rg, kRedSwiglu, s));
    STAGE(ATD_STAGE_DOWN, mma_gemm(d, W.w_down, W.w_down, W.w_down, h, h, h, F, M, s));
    STAGE(ATD_STAGE_DOWN, mma_residual(d, mma_splits(h, F, M), M, x, next_gain, s));
  }
  if (ho && one_tile) {
    // split partials of the head from the fragment-order input, then the
    // norm factor (and y_out) in the reduction
    DecGemmArgs gh{};
    STAGE(ATD_STAGE_HEAD, dec_gemm(d, gh, d->mhi, d->mlo, d->bhead_sw[ho->head], c.vocab,
                                   c.vocab, c.vocab, h, M, kDecParts, s));
    const int kch = dec_kc(dec_tiles(c.vocab, kDecParts, h), h);
    ReduceArgs rh = mma_red(d, c.vocab, (h + kch - 1) / kch, M, ho->logits, c.vocab);
    rh.ss = d->mss;
    rh.x = x;
    rh.gain = d->final_norm;
    rh.y_out = ho->y_out;
    STAGE(ATD_STAGE_HEAD, launch_reduce(rh, kRedStore, s));
  } else if (ho) {
    const void* Wh = d->heads[ho->head];
    STAGE(ATD_STAGE_HEAD, mma_gemm(d, Wh, Wh, Wh, c.vocab, c.vocab, c.vocab, h, M, s));
    ReduceArgs rh = mma_red(d, c.vocab, mma_splits(c.vocab, h, M), M, ho->logits, c.vocab);
    rh.ss = d->mss;
    rh.x = x;
    rh.gain = d->final_norm;
    rh.y_out = ho->y_out;
    STAGE(ATD_STAGE_HEAD, launch_reduce(rh, kRedStore, s));
  }
  return e;
}

// Rows of a call run through the stack (and the LM head when `ho` is set):
// chunks on the MFMA path, one after the other (which keeps a prefill causal:
// a chunk's rows only read keys of earlier rows, already appended), otherwise
// the GEMV path.
hipError_t run_layers(atd_decoder* d, RowMap rows, int M, int max_len_bound, float* x,
                      const HeadOut* ho, hipStream_t s) {
  const int h = d->cfg.hidden, V = d->cfg.vocab;
  hipError_t e = hipSuccess;
  // chunks of up to d->mma_rows rows (decode streams, or prefill rows), each
  // taken layer by layer: the GEMMs stream the weights once per chunk over its
  // 64-row tiles (a prefill chunk's rows read the keys of earlier chunks and
  // their own, appended first)
  const int step = d->mma && M >= kMmaMinRows ? d->mma_rows : M;
  for (int c0 = 0; c0 < M && e == hipSuccess; c0 += step) {
    RowMap r = rows;
    r.row0 = rows.row0 + c0;
    const int cm = std::min(step, M - c0);
    const int bound = rows.mode == kRowsPrefill ? std::min(max_len_bound, r.row0 + cm)
                                                : max_len_bound;
    float* xc = x + (size_t)c0 * h;
    HeadOut hc{};
    if (ho) {
      hc.head = ho->head;
      hc.y_out = ho->y_out ? ho->y_out + (size_t)c0 * h : nullptr;
      hc.logits = ho->logits + (size_t)c0 * V;
    }
    if (d->mma && cm >= kMmaMinRows) {
      e = run_chunk_mma(d, r, cm, bound, xc, ho ? &hc : nullptr, s);
    } else {
      e = run_layers_gemv(d, r, cm, bound, xc, s);
      if (e == hipSuccess && ho) e = run_head_gemv(d, xc, cm, hc.head, hc.y_out, hc.logits, s);
    }
  }
  return e;
}

int check_tables(atd_decoder* d, int G, const int32_t* table_ids, const int32_t* tok,
                 const float* extra) {
  if (G < 0 || G > kMaxTables)
    return fail(d, ATD_ERR_INVALID_ARG, "G = %d outside [0, %d]", G, kMaxTables);
  if (G == 0 && !extra)
    return fail(d, ATD_ERR_INVALID_ARG, "G = 0 needs extra input rows");
  if (G > 0 && (!tok || !table_ids))
    return fail(d, ATD_ERR_INVALID_ARG, "tok or table_ids is NULL with G = %d", G);
  for (int g = 0; g < G; ++g)
    if (table_ids[g] < 0 || table_ids[g] >= d->cfg.n_tables)
      return fail(d, ATD_ERR_INVALID_ARG, "table_ids[%d] = %d outside [0, %d)", g, table_ids[g],
                  d->cfg.n_tables);
  return ATD_OK;
}

EmbedArgs embed_args(atd_decoder* d, int B, const int32_t* tok, int G,
                     const int32_t* table_ids, const float* extra, float* out) {
  EmbedArgs e{};
  for (int g = 0; g < G; ++g) {
    e.tab[g] = d->tables[table_ids[g]];
    e.vocab[g] = d->table_vocab[table_ids[g]];
  }
  e.G = G;
  e.tok = tok;
  e.extra = extra;
  e.out = out;
  e.h = d->in_dim;
  e.M = B;
  return e;
}

// Where input rows are built: the projection's input, or the residual stream.
float* in_rows(const atd_decoder* d) { return d->in_proj ? d->xin : d->x; }

// With an input projection: the M rows in d->xin into d->x (in_proj r + bias).
hipError_t project_rows(atd_decoder* d, int M, hipStream_t s) {
  if (!d->in_proj) return hipSuccess;
  const atd_config& c = d->cfg;
  GemvArgs g{};
  g.W[0] = d->in_proj;
  g.bias[0] = d->in_proj_bias;
  g.seg_end[0] = g.seg_end[1] = g.seg_end[2] = c.hidden;
  g.x = d->xin;
  g.ldx = d->in_dim;
  g.out = d->x;
  g.ldo = c.hidden;
  g.K = d->in_dim;
  g.N = c.hidden;
  g.M = M;
  return launch_gemv(g, kEpiStore, false, head_wtype(d), s);
}

// Input rows of M tokens / extra rows built and projected into d->x.
hipError_t build_inputs(atd_decoder* d, EmbedArgs ea, hipStream_t s) {
  ea.out = in_rows(d);
  hipError_t e = launch_embed(ea, d->cfg.dtype == ATD_BF16, s);
  if (e == hipSuccess) e = project_rows(d, ea.M, s);
  return e;
}

// RoPE rows of an *_mrope call from its rotary positions (device [M, 3]).
hipError_t mrope_rows(atd_decoder* d, const int32_t* rope_pos, int M, hipStream_t s) {
  const atd_config& c = d->cfg;
  return launch_mrope_rows(rope_pos, M, c.head_dim / 2, c.mrope_sections[1],
                           c.mrope_sections[2], c.max_ctx, d->cos_t, d->sin_t, d->rcos,
                           d->rsin, s);
}

// Launch sequence of one decode step of B rows (slots slot0..slot0+B-1, or
// the slots of d->step_slots when `listed`); rope_pos: rotary positions
// [B, 3] of the rows, or null (cache positions).
hipError_t enqueue_step(atd_decoder* d, int slot0, int B, const int32_t* tok, int G,
                        const int32_t* table_ids, const float* extra, int head, float* y_out,
                        float* logits_out, int max_cap, hipStream_t s,
                        const int32_t* rope_pos = nullptr, bool listed = false) {
  RowMap rows{kRowsStep, slot0, 0, rope_pos ? 1 : 0};
  hipError_t e = hipSuccess;
  if (listed) {
    rows.slot_list = d->slot_list;
    e = launch_slot_list(d->slot_list, d->step_slots.data(), B, s);
  }
  if (e == hipSuccess && rope_pos) e = mrope_rows(d, rope_pos, B, s);
  if (e == hipSuccess) e = build_inputs(d, embed_args(d, B, tok, G, table_ids, extra, d->x), s);
  const HeadOut ho{head, y_out, logits_out};
  if (e == hipSuccess) e = run_layers(d, rows, B, max_cap, d->x, &ho, s);
  if (e == hipSuccess) e = launch_advance(slots_of(d), rows, B, s);
  return e;
}

// Byte offsets of the decoder's device scratch (one allocation) for a config.
struct ScratchPlan {
  size_t o_cos, o_sin, o_rcos, o_rsin, o_x, o_xin, o_qkv, o_q, o_o, o_act, o_pml, o_pacc, o_kv,
      o_pos, o_cap, o_part, o_cnt, o_list, o_ticket, o_samp, o_mss = 0, o_mhi = 0, o_mlo = 0,
      o_mpart = 0, o_mhi2 = 0, o_mlo2 = 0, o_mticket = 0, o_bw = 0;
  size_t bw_layer = 0, bw_head = 0;   // elements of one layer's / head's B-order copy
  size_t total = 0;
  size_t part_floats = 0;  // attention partials capacity, in floats per head dim
  bool mma = false;
  int mma_rows = 0;
};

void plan_scratch(const atd_config& c, bool in_proj, ScratchPlan& p) {
  const int R = c.max_rows, S = c.max_slots, h = c.hidden, D = c.head_dim;
  const int nq = c.n_q_heads * D, nqkv = nq + 2 * c.n_kv_heads * D;
  const int in_dim = c.input_dim ? c.input_dim : h;
  const size_t half = D / 2;
  size_t off = 0;
  auto carve = [&](size_t bytes) {
    size_t o = off;
    off += align256(bytes);
    return o;
  };
  p.o_cos = carve((size_t)c.max_ctx * half * 4);
  p.o_sin = carve((size_t)c.max_ctx * half * 4);
  p.o_rcos = carve((size_t)R * half * 4);
  p.o_rsin = carve((size_t)R * half * 4);
  p.o_x = carve((size_t)R * h * 4);
  p.o_xin = carve(in_proj ? (size_t)R * in_dim * 4 : 0);
  p.o_qkv = carve((size_t)R * nqkv * 4);
  p.o_q = carve((size_t)R * nq * 4);
  p.o_o = carve((size_t)R * nq * 4);
  p.o_act = carve((size_t)R * c.ffn * 4);
  // attention partials: M * Hq * attn_max_splits(L, M, Hkv) <= this many per head dim
  p.part_floats = (size_t)c.n_q_heads *
                  std::min((size_t)R * ((c.max_ctx + kAttnMinChunk - 1) / kAttnMinChunk),
                           (size_t)(kAttnWavesMax / c.n_kv_heads + R));
  p.o_pml = carve(p.part_floats * 2 * 4);
  p.o_pacc = carve(p.part_floats * D * 4);
  // MFMA path (bf16 dense weights, chunks of >= kMmaMinRows rows possible)
  p.mma = c.dtype == ATD_BF16 && c.weight_format == ATD_WFMT_DENSE &&
          !(c.flags & ATD_FLAG_NO_MFMA) && h % 32 == 0 && nq % 32 == 0 && c.ffn % 32 == 0 &&
          std::max(R, S) >= kMmaMinRows;
  if (p.mma) {
    // the decode GEMMs' weights in B-operand order: q/k/v, o, gate/up, down
    // per layer, then the heads (filled at creation, outside the zeroed part)
    p.bw_layer = (bfrag_blocks(nqkv, false) * h + bfrag_blocks(h, false) * nq +
                  bfrag_blocks(2 * c.ffn, true) * h + bfrag_blocks(h, false) * c.ffn) * 16;
    p.bw_head = bfrag_blocks(c.vocab, false) * h * 16;
    p.o_bw = carve((p.bw_layer * c.n_layers + p.bw_head * c.n_lm_heads) * 2);
  }
  p.o_kv = carve((size_t)S * c.n_layers * 2 * sizeof(void*));
  p.o_pos = carve((size_t)S * 4);
  p.o_cap = carve((size_t)S * 4);
  const int nblk_v = (c.vocab + kArgmaxChunk - 1) / kArgmaxChunk;
  p.o_part = carve((size_t)R * nblk_v * 3 * 4);
  p.o_cnt = carve(8);
  p.o_list = carve((size_t)R * 4);
  p.o_ticket = carve((size_t)R * c.n_kv_heads * 4);   // zeroed with the tables above
  const int nblk_s = sample_blocks(c.vocab);
  p.o_samp = carve(nblk_s > 1 ? (size_t)nblk_s * kTopKMax * sizeof(uint2) : 0);
  // MFMA path: hi/lo activations of one 64-row chunk and split-K partials of
  // the largest GEMM (q/k/v, o, gate/up, down, LM head)
  if (p.mma) {
    // chunks of up to kMmaPrefillRows rows (row tiles of kMmaRows)
    p.mma_rows = std::max(kMmaRows, (std::min(R, kMmaPrefillRows) + kMmaRows - 1) / kMmaRows *
                                        kMmaRows);
    // partials of the largest GEMM at every row-tile count a chunk can have
    size_t pmax = 0;
    for (int t = 1; t <= p.mma_rows / kMmaRows; ++t) {
      auto parts = [t](int n, int k) { return (size_t)mma_ks(n, k, t) * t * kMmaRows * n; };
      pmax = std::max({pmax, parts(nqkv, h), parts(h, nq), parts(2 * c.ffn, h),
                       parts(h, c.ffn), parts(c.vocab, h)});
    }
    // the decode GEMMs (one row tile): per-split 64 x 64 tiles of each GEMM
    auto dparts = [](int n, int k, int epi) {
      const int t = dec_tiles(n, epi, k), kc = dec_kc(t, k);
      return (size_t)t * ((k + kc - 1) / kc) * kMmaRows * 16 * dec_cb(epi, k);
    };
    pmax = std::max({pmax, dparts(nqkv, h, kDecStore), dparts(h, nq, kDecResidual),
                     dparts(2 * c.ffn, h, kDecSwiglu), dparts(h, c.ffn, kDecResidual),
                     dparts(c.vocab, h, kDecParts)});
    p.o_mss = carve((size_t)p.mma_rows * ((h + kSsCols - 1) / kSsCols) * 4);
    const size_t kmax = std::max({(size_t)h, (size_t)nq, (size_t)c.ffn});
    p.o_mhi = carve((size_t)p.mma_rows * kmax * 2);
    p.o_mlo = carve((size_t)p.mma_rows * kmax * 2);
    p.o_mpart = carve(pmax * 4);
    p.o_mhi2 = carve((size_t)kMmaRows * kmax * 2);
    p.o_mlo2 = carve((size_t)kMmaRows * kmax * 2);
    const int tmax = std::max({dec_tiles(nqkv, kDecStore, h), dec_tiles(h, kDecResidual, nq),
                               dec_tiles(h, kDecResidual, c.ffn),
                               dec_tiles(2 * c.ffn, kDecSwiglu, h)});
    p.o_mticket = carve((size_t)tmax * 4);   // zeroed with the rest
  }
  p.total = off;
}

}  // namespace

// ====================================================================== ABI

extern "C" int decoder_create(const atd_config* cfg, const atd_weights* w, atd_decoder** out) {
  if (!out) return fail(nullptr, ATD_ERR_INVALID_ARG, "out is NULL");
  int rc = check_config(cfg);
  if (rc) return rc;
  if ((rc = check_weights(cfg, w))) return rc;

  atd_decoder* d = new atd_decoder();
  d->cfg = *cfg;
  d->layers.assign(w->layers, w->layers + cfg->n_layers);
  d->final_norm = (const float*)w->final_norm;
  d->in_proj = w->in_proj;
  d->in_proj_bias = (const float*)w->in_proj_bias;
  d->in_dim = cfg->input_dim ? cfg->input_dim : cfg->hidden;
  d->heads.assign(w->lm_heads, w->lm_heads + cfg->n_lm_heads);
  d->tables.assign(w->tables, w->tables + cfg->n_tables);
  d->table_vocab.assign(w->table_vocab, w->table_vocab + cfg->n_tables);
  const int S = cfg->max_slots;
  d->pos.assign(S, 0);
  d->cap.assign(S, 0);
  d->attached.assign(S, 0);
  d->kp.assign(S, std::vector<void*>(cfg->n_layers, nullptr));
  d->vp.assign(S, std::vector<void*>(cfg->n_layers, nullptr));

  d->dry = (cfg->flags & ATD_FLAG_DRY_RUN) != 0;
  if (d->dry) {
    *out = d;
    return ATD_OK;
  }
  ScratchPlan sp;
  plan_scratch(*cfg, w->in_proj != nullptr, sp);
  d->part_floats = sp.part_floats;
  d->mma = sp.mma;
  d->mma_rows = sp.mma_rows;
  d->pf_budget = cfg->flags & ATD_FLAG_NO_L2_PREFETCH ? 0 : kL2PrefetchBytes;
  d->stream_nt = cfg->weight_format == ATD_WFMT_DENSE && cfg->dtype == ATD_BF16 &&
                 dense_weight_bytes(*cfg) > kMallBytes;
  const size_t off = sp.total;
  const size_t o_cos = sp.o_cos, o_sin = sp.o_sin, o_rcos = sp.o_rcos, o_rsin = sp.o_rsin,
               o_x = sp.o_x, o_xin = sp.o_xin, o_qkv = sp.o_qkv, o_q = sp.o_q, o_o = sp.o_o,
               o_act = sp.o_act, o_pml = sp.o_pml, o_pacc = sp.o_pacc, o_kv = sp.o_kv,
               o_pos = sp.o_pos, o_cap = sp.o_cap, o_part = sp.o_part, o_cnt = sp.o_cnt,
               o_list = sp.o_list, o_ticket = sp.o_ticket, o_samp = sp.o_samp,
               o_mss = sp.o_mss, o_mhi = sp.o_mhi,
               o_mlo = sp.o_mlo, o_mpart = sp.o_mpart, o_mhi2 = sp.o_mhi2,
               o_mlo2 = sp.o_mlo2, o_mticket = sp.o_mticket;
  const int D = cfg->head_dim;
  const size_t half = D / 2;

  hipError_t e = hipGetDevice(&d->device);
  if (e == hipSuccess) e = hipMalloc(&d->mem, off);
  if (e != hipSuccess) {
    rc = hip_fail(nullptr, e, "hipMalloc of decoder scratch");
    delete d;
    return rc;
  }
  char* base = static_cast<char*>(d->mem);
  d->cos_t = (float*)(base + o_cos);
  d->sin_t = (float*)(base + o_sin);
  d->rcos = (float*)(base + o_rcos);
  d->rsin = (float*)(base + o_rsin);
  d->x = (float*)(base + o_x);
  d->xin = w->in_proj ? (float*)(base + o_xin) : nullptr;
  d->qkv = (float*)(base + o_qkv);
  d->q = (float*)(base + o_q);
  d->o = (float*)(base + o_o);
  d->act = (float*)(base + o_act);
  d->pml = (float*)(base + o_pml);
  d->pacc = (float*)(base + o_pacc);
  d->kv_tab = (void**)(base + o_kv);
  d->slot_pos = (int*)(base + o_pos);
  d->slot_cap = (int*)(base + o_cap);
  d->part = (float*)(base + o_part);
  d->counter = (int32_t*)(base + o_cnt);
  d->slot_list = (int32_t*)(base + o_list);
  d->attn_ticket = (int*)(base + o_ticket);
  d->ctl_base = d->counter + 1;
  d->samp = (uint2*)(base + o_samp);
  if (d->mma) {
    d->mss = (float*)(base + o_mss);
    d->mhi = (uint16_t*)(base + o_mhi);
    d->mlo = (uint16_t*)(base + o_mlo);
    d->mpart = (float*)(base + o_mpart);
    d->mhi2 = (uint16_t*)(base + o_mhi2);
    d->mlo2 = (uint16_t*)(base + o_mlo2);
    d->mticket = (int*)(base + o_mticket);
  }

  // RoPE table: phi = p * theta^(-2i/D) in double, cos/sin rounded to float.
  std::vector<float> ct((size_t)cfg->max_ctx * half), sn((size_t)cfg->max_ctx * half);
  for (int p = 0; p < cfg->max_ctx; ++p)
    for (size_t i = 0; i < half; ++i) {
      const double omega = std::pow(cfg->rope_theta, -2.0 * (double)i / (double)D);
      const double phi = (double)p * omega;
      ct[(size_t)p * half + i] = (float)std::cos(phi);
      sn[(size_t)p * half + i] = (float)std::sin(phi);
    }
  e = hipMemcpy(d->cos_t, ct.data(), ct.size() * 4, hipMemcpyHostToDevice);
  if (e == hipSuccess) e = hipMemcpy(d->sin_t, sn.data(), sn.size() * 4, hipMemcpyHostToDevice);
  if (e == hipSuccess) e = hipMemset(base + o_kv, 0, off - o_kv);
  if (e == hipSuccess && d->mma) {
    // the decode GEMMs' weights in B-operand order
    const int h = cfg->hidden, nq = cfg->n_q_heads * D, nkv = cfg->n_kv_heads * D;
    const int nqkv = nq + 2 * nkv, F = cfg->ffn;
    uint16_t* bw = (uint16_t*)(base + sp.o_bw);
    auto swz = [&](const void* a0, const void* a1, const void* a2, int e0, int e1, int N, int K,
                   bool sw) {
      SwizzleArgs z{};
      z.src[0] = (const uint16_t*)a0;
      z.src[1] = (const uint16_t*)a1;
      z.src[2] = (const uint16_t*)a2;
      z.seg_end[0] = e0;
      z.seg_end[1] = e1;
      z.seg_end[2] = N;
      z.N = N;
      z.K = K;
      z.swiglu = sw;
      z.dst = bw;
      bw += bfrag_blocks(N, sw) * (size_t)K * 16;
      if (e == hipSuccess) e = launch_swizzle_b(z, nullptr);
      return (const uint16_t*)z.dst;
    };
    for (int l = 0; l < cfg->n_layers; ++l) {
      const atd_layer_weights& W = d->layers[l];
      d->bq_sw.push_back(swz(W.wq, W.wk, W.wv, nq, nq + nkv, nqkv, h, false));
      d->bo_sw.push_back(swz(W.wo, W.wo, W.wo, h, h, h, nq, false));
      d->bgu_sw.push_back(swz(W.w_gate, W.w_up, W.w_up, 2 * F, 2 * F, 2 * F, h, true));
      d->bdown_sw.push_back(swz(W.w_down, W.w_down, W.w_down, h, h, h, F, false));
    }
    for (int j = 0; j < cfg->n_lm_heads; ++j)
      d->bhead_sw.push_back(swz(d->heads[j], d->heads[j], d->heads[j], cfg->vocab, cfg->vocab,
                                cfg->vocab, h, false));
  }
  if (e == hipSuccess) e = hipDeviceSynchronize();
  if (e != hipSuccess) {
    rc = hip_fail(nullptr, e, "decoder scratch initialisation");
    (void)hipFree(d->mem);
    delete d;
    return rc;
  }
  *out = d;
  return ATD_OK;
}

extern "C" int atd_workspace_bytes(const atd_config* cfg, int32_t input_projection,
                                   size_t* out) {
  if (!out) return fail(nullptr, ATD_ERR_INVALID_ARG, "out is NULL");
  const int rc = check_config(cfg);
  if (rc) return rc;
  if (cfg->flags & ATD_FLAG_DRY_RUN) {
    *out = 0;
    return ATD_OK;
  }
  ScratchPlan sp;
  plan_scratch(*cfg, input_projection != 0, sp);
  *out = sp.total;
  return ATD_OK;
}

extern "C" int decoder_destroy(atd_decoder* d) {
  if (!d) return ATD_OK;
  hipError_t e = hipSuccess;
  if (d->mem && !d->dry) {
    e = hipDeviceSynchronize();
    for (auto& g : d->graphs) (void)hipGraphExecDestroy(g.exec);
    if (d->cap_stream) (void)hipStreamDestroy(d->cap_stream);
    hipError_t e2 = hipFree(d->mem);
    if (e == hipSuccess) e = e2;
  }
  delete d;
  return e == hipSuccess ? ATD_OK : hip_fail(nullptr, e, "decoder_destroy");
}

extern "C" const char* decoder_last_error(const atd_decoder* d) {
  return d ? d->err.c_str() : g_err.c_str();
}

extern "C" int kv_bucket_grow(atd_decoder* d, int32_t slot, void* const* k_new,
                              void* const* v_new, int32_t s_new, void* stream) {
  const Range range("kv_bucket_grow");
  if (!d) return fail(nullptr, ATD_ERR_INVALID_ARG, "decoder is NULL");
  const atd_config& c = d->cfg;
  if (slot < 0 || slot >= c.max_slots)
    return fail(d, ATD_ERR_INVALID_ARG, "slot %d outside [0, %d)", slot, c.max_slots);
  if (!k_new || !v_new) return fail(d, ATD_ERR_INVALID_ARG, "k_new or v_new is NULL");
  if (s_new < 1 || s_new > c.max_ctx)
    return fail(d, ATD_ERR_CAPACITY, "s_new %d outside [1, max_ctx %d]", s_new, c.max_ctx);
  const bool first = !d->attached[slot];
  if (!first && s_new <= d->pos[slot])
    return fail(d, ATD_ERR_CAPACITY, "s_new %d does not exceed the %d valid rows of slot %d",
                s_new, d->pos[slot], slot);
  for (int l = 0; l < c.n_layers; ++l) {
    if (!k_new[l] || !v_new[l] || !aligned16(k_new[l]) || !aligned16(v_new[l]))
      return fail(d, ATD_ERR_INVALID_ARG, "layer %d K/V buffer NULL or not 16-byte aligned", l);
    for (int j = 0; j < c.n_layers && !first; ++j)
      if (k_new[l] == d->kp[slot][j] || v_new[l] == d->vp[slot][j] ||
          k_new[l] == d->vp[slot][j] || v_new[l] == d->kp[slot][j])
        return fail(d, ATD_ERR_INVALID_ARG, "layer %d new buffer aliases a buffer in use", l);
  }
  hipStream_t s = (hipStream_t)stream;
  hipError_t e = hipSuccess;
  if (!d->dry && !first && d->pos[slot] > 0) {
    KvCopyArgs a{};
    for (int l = 0; l < c.n_layers; ++l) {
      a.src[2 * l] = d->kp[slot][l];
      a.src[2 * l + 1] = d->vp[slot][l];
      a.dst[2 * l] = k_new[l];
      a.dst[2 * l + 1] = v_new[l];
    }
    a.n = 2 * c.n_layers;
    a.Hkv = c.n_kv_heads;
    a.D = c.head_dim;
    a.rows = d->pos[slot];
    a.s_old = d->cap[slot];
    a.s_new = s_new;
    a.elem_bytes = kv_elem_bytes(c);
    e = launch_kv_copy(a, s);
  }
  if (e == hipSuccess && !d->dry)
    e = launch_set_slot(slots_of(d), slot, k_new, v_new, s_new, first ? 0 : -1, 1, s);
  if (e != hipSuccess) return hip_fail(d, e, "kv_bucket_grow");
  // captured steps hold the slot's cache rows as kernel arguments; their keys
  // name the buckets (bucket_key), so graphs of the old buckets stop matching
  for (int l = 0; l < c.n_layers; ++l) {
    d->kp[slot][l] = k_new[l];
    d->vp[slot][l] = v_new[l];
  }
  d->cap[slot] = s_new;
  if (first) d->pos[slot] = 0;
  d->attached[slot] = 1;
  return ATD_OK;
}

extern "C" int decoder_set_position(atd_decoder* d, int32_t slot, int32_t pos, void* stream) {
  if (!d) return fail(nullptr, ATD_ERR_INVALID_ARG, "decoder is NULL");
  if (slot < 0 || slot >= d->cfg.max_slots)
    return fail(d, ATD_ERR_INVALID_ARG, "slot %d outside [0, %d)", slot, d->cfg.max_slots);
  if (!d->attached[slot])
    return fail(d, ATD_ERR_INVALID_ARG, "slot %d has no KV buffers attached", slot);
  if (pos < 0 || pos > d->cap[slot])
    return fail(d, ATD_ERR_CAPACITY, "pos %d outside [0, capacity %d]", pos, d->cap[slot]);
  hipError_t e = d->dry ? hipSuccess
                        : launch_set_slot(slots_of(d), slot, nullptr, nullptr, -1, pos, 0,
                                          (hipStream_t)stream);
  if (e != hipSuccess) return hip_fail(d, e, "decoder_set_position");
  d->pos[slot] = pos;
  return ATD_OK;
}

extern "C" int decoder_get_position(const atd_decoder* d, int32_t slot, int32_t* pos,
                                    int32_t* capacity) {
  if (!d) return fail(nullptr, ATD_ERR_INVALID_ARG, "decoder is NULL");
  if (slot < 0 || slot >= d->cfg.max_slots)
    return fail(const_cast<atd_decoder*>(d), ATD_ERR_INVALID_ARG, "slot %d outside [0, %d)",
                slot, d->cfg.max_slots);
  if (pos) *pos = d->pos[slot];
  if (capacity) *capacity = d->cap[slot];
  return ATD_OK;
}

extern "C" int decoder_embed(atd_decoder* d, int32_t B, const int32_t* tok, int32_t G,
                             const int32_t* table_ids, const float* extra, float* x_out,
                             void* stream) {
  const Range range("decoder_embed");
  if (!d) return fail(nullptr, ATD_ERR_INVALID_ARG, "decoder is NULL");
  if (B < 1 || B > d->cfg.max_rows)
    return fail(d, ATD_ERR_CAPACITY, "B = %d outside [1, max_rows %d]", B, d->cfg.max_rows);
  if (!x_out) return fail(d, ATD_ERR_INVALID_ARG, "x_out is NULL");
  int rc = check_tables(d, G, table_ids, tok, extra);
  if (rc) return rc;
  if (d->dry) return ATD_OK;
  EmbedArgs a = embed_args(d, B, tok, G, table_ids, extra, x_out);
  hipError_t e = launch_embed(a, d->cfg.dtype == ATD_BF16, (hipStream_t)stream);
  return e == hipSuccess ? ATD_OK : hip_fail(d, e, "decoder_embed");
}

namespace {

int prefill_impl(atd_decoder* d, int32_t slot, const float* x, int32_t T,
                 const int32_t* rope_pos, int32_t head, float* y_out, float* logits_out,
                 void* stream, const char* name) {
  if (!d) return fail(nullptr, ATD_ERR_INVALID_ARG, "decoder is NULL");
  const atd_config& c = d->cfg;
  if (slot < 0 || slot >= c.max_slots)
    return fail(d, ATD_ERR_INVALID_ARG, "slot %d outside [0, %d)", slot, c.max_slots);
  if (!d->attached[slot])
    return fail(d, ATD_ERR_INVALID_ARG, "slot %d has no KV buffers attached", slot);
  if (!x || !logits_out) return fail(d, ATD_ERR_INVALID_ARG, "x or logits_out is NULL");
  if (y_out && !aligned16(y_out))
    return fail(d, ATD_ERR_INVALID_ARG, "y_out %p not 16-byte aligned", (void*)y_out);
  if (head < 0 || head >= c.n_lm_heads)
    return fail(d, ATD_ERR_INVALID_ARG, "head %d outside [0, %d)", head, c.n_lm_heads);
  if (T < 1) return fail(d, ATD_ERR_INVALID_ARG, "T = %d < 1", T);
  if (T > c.max_rows || T > c.max_ctx)
    return fail(d, ATD_ERR_CAPACITY, "T = %d beyond max_rows %d / max_ctx %d", T, c.max_rows,
                c.max_ctx);
  if (T > d->cap[slot])
    return fail(d, ATD_ERR_KV_FULL, "T = %d rows exceed slot %d capacity %d", T, slot,
                d->cap[slot]);
  if (d->dry) {
    d->pos[slot] = T;
    return ATD_OK;
  }
  hipStream_t s = (hipStream_t)stream;
  RowMap rows{kRowsPrefill, slot, 0, rope_pos ? 1 : 0};
  hipError_t e = rope_pos ? mrope_rows(d, rope_pos, T, s) : hipSuccess;
  if (e == hipSuccess) e = build_inputs(d, embed_args(d, T, nullptr, 0, nullptr, x, d->x), s);
  if (e == hipSuccess) e = run_layers(d, rows, T, T, d->x, nullptr, s);
  if (e == hipSuccess)
    e = run_head_gemv(d, d->x + (size_t)(T - 1) * c.hidden, 1, head, y_out, logits_out, s);
  if (e == hipSuccess) e = launch_advance(slots_of(d), rows, T, s);
  if (e != hipSuccess) return hip_fail(d, e, name);
  d->pos[slot] = T;
  return ATD_OK;
}

// slots: host list of the B rows' slots, or null for slot0 .. slot0 + B - 1.
int step_impl(atd_decoder* d, int32_t slot0, int32_t B, const int32_t* slots,
              const int32_t* tok, int32_t G, const int32_t* table_ids, const float* extra,
              const int32_t* rope_pos, int32_t head, float* y_out, float* logits_out,
              void* stream, const char* name) {
  if (!d) return fail(nullptr, ATD_ERR_INVALID_ARG, "decoder is NULL");
  const atd_config& c = d->cfg;
  if (B < 1 || B > c.max_rows)
    return fail(d, ATD_ERR_CAPACITY, "B = %d outside [1, max_rows %d]", B, c.max_rows);
  std::vector<int32_t> list(B);
  if (slots) {
    std::vector<char> used(c.max_slots, 0);
    for (int b = 0; b < B; ++b) {
      if (slots[b] < 0 || slots[b] >= c.max_slots)
        return fail(d, ATD_ERR_INVALID_ARG, "slots[%d] = %d outside [0, %d)", b, slots[b],
                    c.max_slots);
      if (used[slots[b]])
        return fail(d, ATD_ERR_INVALID_ARG, "slots[%d] = %d appears twice in one step", b,
                    slots[b]);
      used[slots[b]] = 1;
      list[b] = slots[b];
    }
  } else {
    if (slot0 < 0 || slot0 + B > c.max_slots)
      return fail(d, ATD_ERR_INVALID_ARG, "slots [%d, %d) outside [0, %d)", slot0, slot0 + B,
                  c.max_slots);
    for (int b = 0; b < B; ++b) list[b] = slot0 + b;
  }
  if (!logits_out) return fail(d, ATD_ERR_INVALID_ARG, "logits_out is NULL");
  if (y_out && !aligned16(y_out))
    return fail(d, ATD_ERR_INVALID_ARG, "y_out %p not 16-byte aligned", (void*)y_out);
  if (head < 0 || head >= c.n_lm_heads)
    return fail(d, ATD_ERR_INVALID_ARG, "head %d outside [0, %d)", head, c.n_lm_heads);
  int rc = check_tables(d, G, table_ids, tok, extra);
  if (rc) return rc;
  int max_cap = 0;
  for (int b = 0; b < B; ++b) {
    const int sl = list[b];
    if (!d->attached[sl])
      return fail(d, ATD_ERR_INVALID_ARG, "slot %d has no KV buffers attached", sl);
    if (d->pos[sl] >= d->cap[sl])
      return fail(d, ATD_ERR_KV_FULL, "slot %d is full: position %d, capacity %d", sl,
                  d->pos[sl], d->cap[sl]);
    if (d->pos[sl] + 1 > c.max_ctx)
      return fail(d, ATD_ERR_CAPACITY, "slot %d position %d reaches max_ctx %d", sl, d->pos[sl],
                  c.max_ctx);
    max_cap = std::max(max_cap, std::min(d->cap[sl], c.max_ctx));
  }
  if (d->dry) {
    for (int b = 0; b < B; ++b) d->pos[list[b]] += 1;
    return ATD_OK;
  }
  if (slots) d->step_slots = list;
  hipError_t e = enqueue_step(d, slot0, B, tok, G, table_ids, extra, head, y_out, logits_out,
                              max_cap, (hipStream_t)stream, rope_pos, slots != nullptr);
  d->step_slots.clear();
  if (e != hipSuccess) return hip_fail(d, e, name);
  for (int b = 0; b < B; ++b) d->pos[list[b]] += 1;
  return ATD_OK;
}

}  // namespace

extern "C" int decoder_prefill(atd_decoder* d, int32_t slot, const float* x, int32_t T,
                               int32_t head, float* y_out, float* logits_out, void* stream) {
  const Range range("decoder_prefill");
  return prefill_impl(d, slot, x, T, nullptr, head, y_out, logits_out, stream,
                      "decoder_prefill");
}

extern "C" int decoder_prefill_mrope(atd_decoder* d, int32_t slot, const float* x, int32_t T,
                                     const int32_t* rope_pos, int32_t head, float* y_out,
                                     float* logits_out, void* stream) {
  const Range range("decoder_prefill_mrope");
  if (!rope_pos) return fail(d, ATD_ERR_INVALID_ARG, "rope_pos is NULL");
  return prefill_impl(d, slot, x, T, rope_pos, head, y_out, logits_out, stream,
                      "decoder_prefill_mrope");
}

extern "C" int decoder_step(atd_decoder* d, int32_t slot0, int32_t B, const int32_t* tok,
                            int32_t G, const int32_t* table_ids, const float* extra,
                            int32_t head, float* y_out, float* logits_out, void* stream) {
  const Range range("decoder_step");
  return step_impl(d, slot0, B, nullptr, tok, G, table_ids, extra, nullptr, head, y_out,
                   logits_out, stream, "decoder_step");
}

extern "C" int decoder_step_slots(atd_decoder* d, int32_t B, const int32_t* slots,
                                  const int32_t* tok, int32_t G, const int32_t* table_ids,
                                  const float* extra, int32_t head, float* y_out,
                                  float* logits_out, void* stream) {
  const Range range("decoder_step_slots");
  if (!slots) return fail(d, ATD_ERR_INVALID_ARG, "slots is NULL");
  return step_impl(d, 0, B, slots, tok, G, table_ids, extra, nullptr, head, y_out, logits_out,
                   stream, "decoder_step_slots");
}

extern "C" int decoder_step_mrope(atd_decoder* d, int32_t slot0, int32_t B, const int32_t* tok,
                                  int32_t G, const int32_t* table_ids, const float* extra,
                                  const int32_t* rope_pos, int32_t head, float* y_out,
                                  float* logits_out, void* stream) {
  const Range range("decoder_step_mrope");
  if (!rope_pos) return fail(d, ATD_ERR_INVALID_ARG, "rope_pos is NULL");
  return step_impl(d, slot0, B, nullptr, tok, G, table_ids, extra, rope_pos, head, y_out,
                   logits_out, stream, "decoder_step_mrope");
}

// ---------------------------------------------------------------- argmax

namespace {
struct ChoiceScratch {
  void* p = nullptr;
  size_t bytes = 0;
  std::vector<void*> retired;   // smaller buffers, never freed
};
std::mutex g_choice_mu;
std::map<int, ChoiceScratch> g_choice_scratch;

// Device scratch of greedy_argmax / sample_topk, one per device (calls that
// overlap on one device share it).  A call that needs more space gets a new,
// larger buffer; the old one is kept allocated until the process ends, since
// work already queued, or a graph a caller captured around an earlier call,
// may still use its address.
int choice_scratch(size_t need, void** out) {
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return hip_fail(nullptr, e, "hipGetDevice");
  std::lock_guard<std::mutex> lk(g_choice_mu);
  ChoiceScratch& sc = g_choice_scratch[dev];
  if (sc.bytes < need) {
    const size_t bytes = std::max(need, std::max(2 * sc.bytes, size_t(1) << 16));
    void* p = nullptr;
    e = hipMalloc(&p, bytes);
    if (e != hipSuccess) return hip_fail(nullptr, e, "hipMalloc of token-choice scratch");
    if (sc.p) sc.retired.push_back(sc.p);
    sc.p = p;
    sc.bytes = bytes;
  }
  *out = sc.p;
  return ATD_OK;
}

// Validates sampling settings for a vocabulary of V (d may be NULL).
int check_sampling(atd_decoder* d, const atd_sampling* sp, int V) {
  if (!sp->uniforms) return fail(d, ATD_ERR_INVALID_ARG, "sampling uniforms is NULL");
  if (sp->top_k < 1 || sp->top_k > kTopKMax || sp->top_k > V)
    return fail(d, ATD_ERR_INVALID_ARG, "top_k %d outside [1, min(%d, V = %d)]", sp->top_k,
                kTopKMax, V);
  if (!(sp->temperature > 0.0f) || !std::isfinite(sp->temperature))
    return fail(d, ATD_ERR_INVALID_ARG, "temperature %g is not a positive number",
                (double)sp->temperature);
  if (!(sp->top_p > 0.0f && sp->top_p <= 1.0f))
    return fail(d, ATD_ERR_INVALID_ARG, "top_p %g outside (0, 1]", (double)sp->top_p);
  const int nblk = sample_blocks(V);
  if (nblk > 1 && (int64_t)nblk * sp->top_k > kSampleChunk)
    return fail(d, ATD_ERR_UNSUPPORTED,
                "V = %d in %d chunks of %d keeps %d candidates, above the %d one workgroup "
                "selects from",
                V, nblk, kSampleChunk, nblk * sp->top_k, kSampleChunk);
  return ATD_OK;
}

SampleArgs sample_args(const float* z, int B, int V, uint32_t* seen, float penalty,
                       const atd_sampling& sp, int32_t* tok, uint2* part) {
  SampleArgs a{};
  a.z = z;
  a.B = B;
  a.V = V;
  a.seen = seen;
  a.nwords = (V + 31) / 32;
  a.penalty = penalty;
  a.k = sp.top_k;
  a.temperature = sp.temperature;
  a.top_p = sp.top_p;
  a.u = sp.uniforms;
  a.u_row = nullptr;
  a.u_stride = 0;
  a.tok = tok;
  a.part = part;
  a.nblk = sample_blocks(V);
  return a;
}
}  // namespace

namespace {
// Validates generation controls for rows of V tokens (d may be NULL).
int check_controls(atd_decoder* d, const atd_controls* c, int V) {
  if (c->eos < -1 || c->eos >= V)
    return fail(d, ATD_ERR_INVALID_ARG, "eos %d outside [-1, %d)", c->eos, V);
  if (c->min_new_tokens < 0 || c->first_index < 0)
    return fail(d, ATD_ERR_INVALID_ARG, "min_new_tokens %d or first_index %d is negative",
                c->min_new_tokens, c->first_index);
  if (((uintptr_t)c->suppress & 3) || ((uintptr_t)c->eos_step & 3))
    return fail(d, ATD_ERR_INVALID_ARG, "suppress %p or eos_step %p not 4-byte aligned",
                (const void*)c->suppress, (void*)c->eos_step);
  return ATD_OK;
}

ChoiceCtl choice_ctl(const atd_controls* c, const int32_t* base, const int32_t* ctr) {
  ChoiceCtl k{};
  if (!c) return k;
  k.suppress = c->suppress;
  k.eos = c->eos;
  k.min_new = c->min_new_tokens;
  k.step0 = base ? 0 : c->first_index;
  k.step_base = base;
  k.step_ctr = ctr;
  k.eos_step = c->eos >= 0 ? c->eos_step : nullptr;
  return k;
}

// Controls as graph-key entries (first_index is read from the device).
void key_controls(std::vector<int64_t>& key, const atd_controls* c) {
  if (!c) {
    key.push_back(0);
    return;
  }
  key.insert(key.end(), {1, (int64_t)(uintptr_t)c->suppress, c->eos, c->min_new_tokens,
                         (int64_t)(uintptr_t)c->eos_step});
}
}  // namespace

namespace {
// Checks and arguments of a greedy_argmax call (partials not yet assigned).
int argmax_args(const float* logits, int32_t B, int32_t V, uint32_t* seen, float penalty,
                const atd_controls* controls, int32_t* tok_out, float* margin_out,
                ArgmaxArgs& a) {
  if (!logits || !tok_out) return fail(nullptr, ATD_ERR_INVALID_ARG, "logits or tok_out is NULL");
  if (B < 1) return fail(nullptr, ATD_ERR_INVALID_ARG, "B = %d < 1", B);
  if (V < 2) return fail(nullptr, ATD_ERR_INVALID_ARG, "V = %d < 2", V);
  if (!(penalty > 0.0f) || !std::isfinite(penalty))
    return fail(nullptr, ATD_ERR_INVALID_ARG, "penalty %g is not a positive number",
                (double)penalty);
  if (controls) {
    const int rc = check_controls(nullptr, controls, V);
    if (rc) return rc;
  }
  a = ArgmaxArgs{};
  a.ctl = choice_ctl(controls, nullptr, nullptr);
  a.z = logits;
  a.B = B;
  a.V = V;
  a.seen = seen;
  a.nwords = (V + 31) / 32;
  a.penalty = penalty;
  a.tok = tok_out;
  a.margin = margin_out;
  a.nblk = (V + kArgmaxChunk - 1) / kArgmaxChunk;
  return ATD_OK;
}
}  // namespace

extern "C" int greedy_argmax(const float* logits, int32_t B, int32_t V, uint32_t* seen,
                             float penalty, const atd_controls* controls, int32_t* tok_out,
                             float* margin_out, void* stream) {
  const Range range("greedy_argmax");
  ArgmaxArgs a;
  int rc = argmax_args(logits, B, V, seen, penalty, controls, tok_out, margin_out, a);
  if (rc) return rc;
  void* p = nullptr;
  rc = choice_scratch((size_t)B * a.nblk * 3 * sizeof(float), &p);
  if (rc) return rc;
  a.part = (float*)p;
  hipError_t e = launch_argmax(a, (hipStream_t)stream);
  return e == hipSuccess ? ATD_OK : hip_fail(nullptr, e, "greedy_argmax");
}

extern "C" int greedy_argmax_noalloc(const float* logits, int32_t B, int32_t V, uint32_t* seen,
                                     float penalty, const atd_controls* controls,
                                     int32_t* tok_out, float* margin_out, void* stream) {
  const Range range("greedy_argmax_noalloc");
  ArgmaxArgs a;
  const int rc = argmax_args(logits, B, V, seen, penalty, controls, tok_out, margin_out, a);
  if (rc) return rc;
  const size_t need = (size_t)B * a.nblk * 3;
  if (need > kNoAllocScratchFloats)
    return fail(nullptr, ATD_ERR_CAPACITY,
                "B = %d rows of V = %d need %zu floats of partials, beyond the fixed %zu", B, V,
                need, kNoAllocScratchFloats);
  float* p = nullptr;
  hipError_t e = noalloc_scratch(&p);
  if (e != hipSuccess) return hip_fail(nullptr, e, "greedy_argmax_noalloc scratch address");
  a.part = p;
  e = launch_argmax(a, (hipStream_t)stream);
  return e == hipSuccess ? ATD_OK : hip_fail(nullptr, e, "greedy_argmax_noalloc");
}

extern "C" int sample_topk(const float* logits, int32_t B, int32_t V, uint32_t* seen,
                           float penalty, const atd_sampling* sampling,
                           const atd_controls* controls, int32_t* tok_out, void* stream) {
  const Range range("sample_topk");
  if (!logits || !tok_out || !sampling)
    return fail(nullptr, ATD_ERR_INVALID_ARG, "logits, sampling or tok_out is NULL");
  if (B < 1) return fail(nullptr, ATD_ERR_INVALID_ARG, "B = %d < 1", B);
  if (V < 1) return fail(nullptr, ATD_ERR_INVALID_ARG, "V = %d < 1", V);
  if (!(penalty > 0.0f) || !std::isfinite(penalty))
    return fail(nullptr, ATD_ERR_INVALID_ARG, "penalty %g is not a positive number",
                (double)penalty);
  int rc = check_sampling(nullptr, sampling, V);
  if (rc) return rc;
  if (controls && (rc = check_controls(nullptr, controls, V)) != ATD_OK) return rc;
  SampleArgs a = sample_args(logits, B, V, seen, penalty, *sampling, tok_out, nullptr);
  a.ctl = choice_ctl(controls, nullptr, nullptr);
  if (a.nblk > 1) {
    void* p = nullptr;
    rc = choice_scratch((size_t)B * a.nblk * a.k * sizeof(uint2), &p);
    if (rc) return rc;
    a.part = (uint2*)p;
  }
  hipError_t e = launch_sample(a, (hipStream_t)stream);
  return e == hipSuccess ? ATD_OK : hip_fail(nullptr, e, "sample_topk");
}

// ---------------------------------------------------------------- quantization

extern "C" int quantize_blocks(const void* w, int32_t dtype, int64_t rows, int32_t cols,
                               int32_t format, void* codes, uint16_t* scales, void* stream) {
  const Range range("quantize_blocks");
  if (!w || !codes || !scales)
    return fail(nullptr, ATD_ERR_INVALID_ARG, "w, codes or scales is NULL");
  if (!aligned16(w) || !aligned16(codes) || ((uintptr_t)scales & 1))
    return fail(nullptr, ATD_ERR_INVALID_ARG,
                "w %p and codes %p must be 16-byte aligned, scales %p 2-byte aligned", w, codes,
                (void*)scales);
  if (dtype != ATD_F32 && dtype != ATD_BF16)
    return fail(nullptr, ATD_ERR_DTYPE, "dtype %d is not ATD_F32 (0) or ATD_BF16 (1)", dtype);
  if (format != ATD_WFMT_Q8 && format != ATD_WFMT_Q4)
    return fail(nullptr, ATD_ERR_DTYPE, "format %d is not ATD_WFMT_Q8 or ATD_WFMT_Q4", format);
  if (rows < 1 || cols < kQBlock || cols % kQBlock)
    return fail(nullptr, ATD_ERR_SHAPE, "rows %lld, cols %d: cols must be a positive multiple of %d",
                (long long)rows, cols, kQBlock);
  if (rows * (int64_t)(cols / kQBlock) > ((int64_t)1 << 40))
    return fail(nullptr, ATD_ERR_SHAPE, "rows %lld x cols %d is too large", (long long)rows,
                cols);
  QuantArgs a{};
  a.w = w;
  a.bf16 = dtype == ATD_BF16;
  a.rows = rows;
  a.cols = cols;
  a.q4 = format == ATD_WFMT_Q4;
  a.codes = codes;
  a.scales = scales;
  const hipError_t e = launch_quantize(a, (hipStream_t)stream);
  return e == hipSuccess ? ATD_OK : hip_fail(nullptr, e, "quantize_blocks");
}

// ---------------------------------------------------------------- codec convolutions

namespace {
int check_conv_ptrs(const void* a, const void* b, const void* c) {
  if (!a || !b || !c) return fail(nullptr, ATD_ERR_INVALID_ARG, "a NULL tensor pointer");
  if (((uintptr_t)a | (uintptr_t)b | (uintptr_t)c) & 3)
    return fail(nullptr, ATD_ERR_INVALID_ARG, "tensor pointers must be 4-byte aligned");
  return ATD_OK;
}
bool too_big(int64_t a, int64_t b) { return a * b >= ((int64_t)1 << 31); }
}  // namespace

extern "C" int codec_conv1d_causal(const float* x, const float* w, const float* bias,
                                   int32_t cin, int32_t cout, int32_t T, int32_t K,
                                   int32_t dilation, int32_t accumulate, float* y, void* stream) {
  const Range range("codec_conv1d_causal");
  int rc = check_conv_ptrs(x, w, y);
  if (rc) return rc;
  if (bias && ((uintptr_t)bias & 3))
    return fail(nullptr, ATD_ERR_INVALID_ARG, "bias %p not 4-byte aligned", (const void*)bias);
  if (cin < 1 || cout < 1 || T < 1 || K < 1 || dilation < 1)
    return fail(nullptr, ATD_ERR_INVALID_ARG, "cin %d, cout %d, T %d, K %d, dilation %d: all >= 1",
                cin, cout, T, K, dilation);
  if (too_big(cin, K) || too_big(cin, T) || too_big(cout, T) || too_big((int64_t)cout * cin, K))
    return fail(nullptr, ATD_ERR_INVALID_ARG, "tensor beyond 2^31 elements");
  ConvArgs a{};
  a.x = x;
  a.w = w;
  a.bias = bias;
  a.y = y;
  a.cin = cin;
  a.cout = cout;
  a.T = T;
  a.K = K;
  a.dil = dilation;
  a.ldy = T;
  a.ystride = 1;
  a.P = 1;
  a.accumulate = accumulate != 0;
  const hipError_t e = launch_conv(a, (hipStream_t)stream);
  return e == hipSuccess ? ATD_OK : hip_fail(nullptr, e, "codec_conv1d_causal");
}

extern "C" int codec_transconv1d_pack(const float* w, int32_t cin, int32_t cout, int32_t stride,
                                      float* packed, void* stream) {
  const Range range("codec_transconv1d_pack");
  int rc = check_conv_ptrs(w, packed, packed);
  if (rc) return rc;
  if (cin < 1 || cout < 1 || stride < 1)
    return fail(nullptr, ATD_ERR_INVALID_ARG, "cin %d, cout %d, stride %d: all >= 1", cin, cout,
                stride);
  if (too_big((int64_t)cin * cout, 2 * (int64_t)stride))
    return fail(nullptr, ATD_ERR_INVALID_ARG, "tensor beyond 2^31 elements");
  const hipError_t e = launch_pack_transconv(w, cin, cout, stride, packed, (hipStream_t)stream);
  return e == hipSuccess ? ATD_OK : hip_fail(nullptr, e, "codec_transconv1d_pack");
}

extern "C" int codec_transconv1d(const float* x, const float* packed, const float* bias,
                                 int32_t cin, int32_t cout, int32_t T, int32_t stride, float* y,
                                 void* stream) {
  const Range range("codec_transconv1d");
  int rc = check_conv_ptrs(x, packed, y);
  if (rc) return rc;
  if (bias && ((uintptr_t)bias & 3))
    return fail(nullptr, ATD_ERR_INVALID_ARG, "bias %p not 4-byte aligned", (const void*)bias);
  if (cin < 1 || cout < 1 || T < 1 || stride < 1)
    return fail(nullptr, ATD_ERR_INVALID_ARG, "cin %d, cout %d, T %d, stride %d: all >= 1", cin,
                cout, T, stride);
  if (too_big(cin, T) || too_big((int64_t)cout * T, stride) ||
      too_big((int64_t)cin * cout, 2 * (int64_t)stride))
    return fail(nullptr, ATD_ERR_INVALID_ARG, "tensor beyond 2^31 elements");
  ConvArgs a{};
  a.x = x;
  a.w = packed;
  a.bias = bias;
  a.y = y;
  a.cin = cin;
  a.cout = cout;
  a.T = T;
  a.K = 2;
  a.dil = 1;
  a.ldy = T * stride;
  a.ystride = stride;
  a.P = stride;
  const hipError_t e = launch_conv(a, (hipStream_t)stream);
  return e == hipSuccess ? ATD_OK : hip_fail(nullptr, e, "codec_transconv1d");
}

// ---------------------------------------------------------------- generation

namespace {

// Identifies the cache rows a captured graph was recorded with.
int64_t bucket_key(const atd_decoder* d, int slot) {
  uint64_t h = 1469598103934665603ull;
  for (size_t l = 0; l < d->kp[slot].size(); ++l) {
    h = (h ^ (uint64_t)(uintptr_t)d->kp[slot][l]) * 1099511628211ull;
    h = (h ^ (uint64_t)(uintptr_t)d->vp[slot][l]) * 1099511628211ull;
  }
  return (int64_t)h;
}

// Adds a graph to the cache; evicting the oldest first waits for the device
// (an evicted graph may still be in flight on the caller's stream).
hipError_t cache_graph(atd_decoder* d, std::vector<int64_t> key, hipGraphExec_t exec) {
  if (d->graphs.size() >= 8) {
    const hipError_t e = hipDeviceSynchronize();
    if (e != hipSuccess) return e;
    (void)hipGraphExecDestroy(d->graphs.front().exec);
    d->graphs.erase(d->graphs.begin());
  }
  d->graphs.push_back({std::move(key), exec});
  return hipSuccess;
}

uint32_t float_bits(float f) {
  uint32_t b;
  std::memcpy(&b, &f, 4);
  return b;
}

// Sampling settings as graph-key entries (a single 0 for greedy).
void key_sampling(std::vector<int64_t>& key, const atd_sampling* sp) {
  if (!sp) {
    key.push_back(0);
    return;
  }
  key.insert(key.end(), {1, sp->top_k, float_bits(sp->temperature), float_bits(sp->top_p),
                         (int64_t)(uintptr_t)sp->uniforms});
}

// Token choice of one row of d's logits inside a captured step: the
// penalised argmax (sp NULL) or the draw with
// u = sp->uniforms[u_off + (*u_row) * u_stride].
hipError_t enqueue_choice(atd_decoder* d, const float* z, uint32_t* seen, float penalty,
                          const atd_sampling* sp, const int32_t* u_row, int u_stride, int u_off,
                          int32_t* tok, hipStream_t s, const ChoiceCtl& ctl = ChoiceCtl{}) {
  const int V = d->cfg.vocab;
  if (!sp) {
    ArgmaxArgs a{};
    a.ctl = ctl;
    a.z = z;
    a.B = 1;
    a.V = V;
    a.seen = seen;
    a.nwords = (V + 31) / 32;
    a.penalty = penalty;
    a.tok = tok;
    a.margin = nullptr;
    a.part = d->part;
    a.nblk = (V + kArgmaxChunk - 1) / kArgmaxChunk;
    return launch_argmax(a, s);
  }
  SampleArgs a = sample_args(z, 1, V, seen, penalty, *sp, tok, d->samp);
  a.ctl = ctl;
  a.u = sp->uniforms + u_off;
  a.u_row = u_row;
  a.u_stride = u_stride;
  return launch_sample(a, s);
}

}  // namespace

extern "C" int decoder_generate(atd_decoder* d, int32_t slot, int32_t n_steps, int32_t* tok_io,
                                int32_t G, const int32_t* table_ids, const float* extra,
                                int32_t head, uint32_t* seen, float penalty,
                                const atd_sampling* sampling, const atd_controls* controls,
                                int32_t* tokens_out, float* y_out, float* logits_out,
                                void* stream) {
  const Range range("decoder_generate");
  if (!d) return fail(nullptr, ATD_ERR_INVALID_ARG, "decoder is NULL");
  const atd_config& c = d->cfg;
  if (slot < 0 || slot >= c.max_slots)
    return fail(d, ATD_ERR_INVALID_ARG, "slot %d outside [0, %d)", slot, c.max_slots);
  if (!d->attached[slot])
    return fail(d, ATD_ERR_INVALID_ARG, "slot %d has no KV buffers attached", slot);
  if (n_steps < 0) return fail(d, ATD_ERR_INVALID_ARG, "n_steps %d < 0", n_steps);
  if (!tok_io || !logits_out) return fail(d, ATD_ERR_INVALID_ARG, "tok_io or logits_out is NULL");
  if (G < 1) return fail(d, ATD_ERR_INVALID_ARG, "G = %d < 1", G);
  int rc = check_tables(d, G, table_ids, tok_io, extra);
  if (rc) return rc;
  if (y_out && !aligned16(y_out))
    return fail(d, ATD_ERR_INVALID_ARG, "y_out %p not 16-byte aligned", (void*)y_out);
  if (head < 0 || head >= c.n_lm_heads)
    return fail(d, ATD_ERR_INVALID_ARG, "head %d outside [0, %d)", head, c.n_lm_heads);
  if (!(penalty > 0.0f) || !std::isfinite(penalty))
    return fail(d, ATD_ERR_INVALID_ARG, "penalty %g is not a positive number", (double)penalty);
  if (sampling && (rc = check_sampling(d, sampling, c.vocab)) != ATD_OK) return rc;
  if (controls && (rc = check_controls(d, controls, c.vocab)) != ATD_OK) return rc;
  if ((int64_t)d->pos[slot] + n_steps > d->cap[slot])
    return fail(d, ATD_ERR_KV_FULL, "slot %d: %d steps from position %d exceed capacity %d",
                slot, n_steps, d->pos[slot], d->cap[slot]);
  if ((int64_t)d->pos[slot] + n_steps > c.max_ctx)
    return fail(d, ATD_ERR_CAPACITY, "slot %d: %d steps from position %d exceed max_ctx %d", slot,
                n_steps, d->pos[slot], c.max_ctx);
  if (n_steps == 0) return ATD_OK;
  if (d->dry) {
    d->pos[slot] += n_steps;
    return ATD_OK;
  }
  hipStream_t s = (hipStream_t)stream;
  const int max_cap = std::min(d->cap[slot], c.max_ctx);

  std::vector<int64_t> key = {slot, G, (int64_t)(uintptr_t)extra, head,
                              (int64_t)(uintptr_t)tok_io, (int64_t)(uintptr_t)seen,
                              (int64_t)(uintptr_t)tokens_out, (int64_t)(uintptr_t)y_out,
                              (int64_t)(uintptr_t)logits_out, max_cap, bucket_key(d, slot)};
  key.push_back(float_bits(penalty));
  for (int g = 0; g < G; ++g) key.push_back(table_ids[g]);
  key_sampling(key, sampling);
  key_controls(key, controls);
  // the step index lives in d->counter
  const bool count = tokens_out || sampling || controls;
  hipGraphExec_t exec = nullptr;
  for (auto& ge : d->graphs)
    if (ge.key == key) exec = ge.exec;
  hipError_t e = hipSuccess;
  if (!exec) {
    if (!d->cap_stream) {
      e = hipStreamCreateWithFlags(&d->cap_stream, hipStreamNonBlocking);
      if (e != hipSuccess) return hip_fail(d, e, "hipStreamCreate (capture stream)");
    }
    hipStream_t cs = d->cap_stream;
    e = hipStreamBeginCapture(cs, hipStreamCaptureModeThreadLocal);
    if (e != hipSuccess) return hip_fail(d, e, "hipStreamBeginCapture");
    hipError_t le = enqueue_step(d, slot, 1, tok_io, G, table_ids, extra, head, y_out, logits_out,
                                 max_cap, cs);
    if (le == hipSuccess)
      le = enqueue_choice(d, logits_out, seen, penalty, sampling, d->counter, 1, 0, tok_io, cs,
                          choice_ctl(controls, d->ctl_base, d->counter));
    if (le == hipSuccess && count) le = launch_record_token(tok_io, tokens_out, d->counter, cs);
    hipGraph_t graph = nullptr;
    e = hipStreamEndCapture(cs, &graph);
    if (le != hipSuccess || e != hipSuccess) {
      if (graph) (void)hipGraphDestroy(graph);
      return hip_fail(d, le != hipSuccess ? le : e, "capture of a decode step");
    }
    e = hipGraphInstantiate(&exec, graph, nullptr, nullptr, 0);
    (void)hipGraphDestroy(graph);
    if (e != hipSuccess) return hip_fail(d, e, "hipGraphInstantiate");
    e = cache_graph(d, key, exec);
    if (e != hipSuccess) return hip_fail(d, e, "graph cache");
  }
  if (count) e = launch_fill_i32(d->counter, 1, 0, s);
  if (controls && e == hipSuccess) e = launch_fill_i32(d->ctl_base, 1, controls->first_index, s);
  for (int k = 0; k < n_steps && e == hipSuccess; ++k) e = hipGraphLaunch(exec, s);
  if (e != hipSuccess) return hip_fail(d, e, "decoder_generate replay");
  d->pos[slot] += n_steps;
  return ATD_OK;
}

// ---------------------------------------------------------------- Talker frame loop

namespace {

constexpr int kCodeGroups = 16;   // codes per Talker frame (c0 and 15 Code Predictor groups)

// The Code Predictor pass of one frame, then the record of its 16 codes:
// rows [y, table_0[c0]] -> 2-row prefill, head 0 -> c1; steps j = 1..14 fed
// table_j[c_j], head j -> c_{j+1}.  Choices greedy (sp NULL) or drawn with
// u = sp->uniforms[(*counter) * 15 + j] for c_{j+1}.
hipError_t enqueue_cp_pass(atd_decoder* cp, int cp_slot, int32_t* codes, const float* y,
                           float* cp_logits, int32_t* codes_out, int32_t* counter,
                           const atd_sampling* sp, hipStream_t s) {
  const atd_config& c = cp->cfg;
  const int cp_cap = std::min(cp->cap[cp_slot], c.max_ctx);
  const int G = kCodeGroups - 1;
  // prefill rows: the Talker's output and the embedding of c0 (table 0)
  const int32_t t0 = 0;
  EmbedArgs r0 = embed_args(cp, 1, nullptr, 0, nullptr, y, in_rows(cp));
  EmbedArgs r1 = embed_args(cp, 1, codes, 1, &t0, nullptr, in_rows(cp) + cp->in_dim);
  hipError_t e = launch_embed(r0, c.dtype == ATD_BF16, s);
  if (e == hipSuccess) e = launch_embed(r1, c.dtype == ATD_BF16, s);
  if (e == hipSuccess) e = project_rows(cp, 2, s);
  const RowMap pre{kRowsPrefill, cp_slot, 0};
  if (e == hipSuccess) e = run_layers(cp, pre, 2, 2, cp->x, nullptr, s);
  if (e == hipSuccess) e = run_head_gemv(cp, cp->x + c.hidden, 1, 0, nullptr, cp_logits, s);
  if (e == hipSuccess) e = launch_advance(slots_of(cp), pre, 2, s);
  if (e == hipSuccess)
    e = enqueue_choice(cp, cp_logits, nullptr, 1.0f, sp, counter, G, 0, codes + 1, s);
  for (int j = 1; j < G && e == hipSuccess; ++j) {
    const int32_t tj = j;
    e = enqueue_step(cp, cp_slot, 1, codes + j, 1, &tj, nullptr, j, nullptr, cp_logits, cp_cap, s);
    if (e == hipSuccess)
      e = enqueue_choice(cp, cp_logits, nullptr, 1.0f, sp, counter, G, j, codes + j + 1, s);
  }
  if (e == hipSuccess) e = launch_record_tokens(codes, kCodeGroups, codes_out, counter, s);
  return e;
}

// One Talker step of the frame loop: input sum_g table_g[c_g] + text[*counter],
// head 0 -> y and logits, penalised choice -> c0 (greedy, or drawn with
// u = sp->uniforms[*counter]).
hipError_t enqueue_talker_step(atd_decoder* tk, int tk_slot, int32_t* codes, const float* text,
                               int32_t* counter, uint32_t* seen, float penalty,
                               const atd_sampling* sp, const atd_controls* ctl, float* y,
                               float* tk_logits, hipStream_t s) {
  const atd_config& c = tk->cfg;
  int32_t tabs[kCodeGroups];
  for (int g = 0; g < kCodeGroups; ++g) tabs[g] = g;
  RowMap rows{kRowsStep, tk_slot, 0};
  EmbedArgs ea = embed_args(tk, 1, codes, kCodeGroups, tabs, text, tk->x);
  ea.extra_row = counter;
  hipError_t e = build_inputs(tk, ea, s);
  const HeadOut ho{0, y, tk_logits};
  const int max_cap = std::min(tk->cap[tk_slot], c.max_ctx);
  if (e == hipSuccess) e = run_layers(tk, rows, 1, max_cap, tk->x, &ho, s);
  if (e == hipSuccess) e = launch_advance(slots_of(tk), rows, 1, s);
  if (e == hipSuccess)
    e = enqueue_choice(tk, tk_logits, seen, penalty, sp, counter, 1, 0, codes, s,
                       choice_ctl(ctl, tk->ctl_base, counter));
  return e;
}

}  // namespace

extern "C" int talker_generate_frames(atd_decoder* tk, int32_t tk_slot, atd_decoder* cp,
                                      int32_t cp_slot, int32_t n_frames, int32_t* codes_io,
                                      float* y_io, const float* text, uint32_t* seen,
                                      float penalty, const atd_sampling* tk_sampling,
                                      const atd_sampling* cp_sampling,
                                      const atd_controls* tk_controls, int32_t* codes_out,
                                      float* tk_logits, float* cp_logits, void* stream) {
  const Range range("talker_generate_frames");
  if (!tk) return fail(nullptr, ATD_ERR_INVALID_ARG, "Talker decoder is NULL");
  if (!cp || cp == tk) return fail(tk, ATD_ERR_INVALID_ARG, "Code Predictor decoder is NULL or the Talker's");
  const atd_config &tc = tk->cfg, &cc = cp->cfg;
  if (tk->dry != cp->dry) return fail(tk, ATD_ERR_INVALID_ARG, "one decoder is a dry run, the other not");
  if (n_frames < 1) return fail(tk, ATD_ERR_INVALID_ARG, "n_frames %d < 1", n_frames);
  if (tc.hidden != cp->in_dim)
    return fail(tk, ATD_ERR_SHAPE,
                "the Code Predictor's input width %d is not the Talker's hidden size %d",
                cp->in_dim, tc.hidden);
  if (tk->in_dim != tc.hidden)
    return fail(tk, ATD_ERR_SHAPE, "the Talker of a frame loop takes no input projection");
  if (tc.n_tables < kCodeGroups)
    return fail(tk, ATD_ERR_SHAPE, "the Talker has %d tables, a frame input needs %d", tc.n_tables,
                kCodeGroups);
  if (cc.n_tables < kCodeGroups - 1 || cc.n_lm_heads < kCodeGroups - 1)
    return fail(tk, ATD_ERR_SHAPE, "the Code Predictor has %d tables / %d heads, needs %d each",
                cc.n_tables, cc.n_lm_heads, kCodeGroups - 1);
  if (tk_slot < 0 || tk_slot >= tc.max_slots || !tk->attached[tk_slot])
    return fail(tk, ATD_ERR_INVALID_ARG, "Talker slot %d is not an attached slot", tk_slot);
  if (cp_slot < 0 || cp_slot >= cc.max_slots || !cp->attached[cp_slot])
    return fail(tk, ATD_ERR_INVALID_ARG, "Code Predictor slot %d is not an attached slot", cp_slot);
  if (cc.max_rows < 2)
    return fail(tk, ATD_ERR_CAPACITY, "the Code Predictor's max_rows %d < 2", cc.max_rows);
  if (std::min(cp->cap[cp_slot], cc.max_ctx) < kCodeGroups)
    return fail(tk, ATD_ERR_KV_FULL, "Code Predictor slot %d holds %d rows, a pass needs %d",
                cp_slot, std::min(cp->cap[cp_slot], cc.max_ctx), kCodeGroups);
  const int steps = n_frames - 1;
  if ((int64_t)tk->pos[tk_slot] + steps > std::min(tk->cap[tk_slot], tc.max_ctx))
    return fail(tk, ATD_ERR_KV_FULL, "Talker slot %d: %d steps from position %d exceed %d rows",
                tk_slot, steps, tk->pos[tk_slot], std::min(tk->cap[tk_slot], tc.max_ctx));
  if (!codes_io || !y_io || !tk_logits || !cp_logits || !seen)
    return fail(tk, ATD_ERR_INVALID_ARG, "codes_io, y_io, seen or a logits buffer is NULL");
  if (steps > 0 && !text) return fail(tk, ATD_ERR_INVALID_ARG, "text is NULL");
  if (!aligned16(y_io)) return fail(tk, ATD_ERR_INVALID_ARG, "y_io %p not 16-byte aligned", (void*)y_io);
  if (!(penalty > 0.0f) || !std::isfinite(penalty))
    return fail(tk, ATD_ERR_INVALID_ARG, "penalty %g is not a positive number", (double)penalty);
  int rc = ATD_OK;
  if (tk_sampling && (rc = check_sampling(tk, tk_sampling, tc.vocab)) != ATD_OK) return rc;
  if (cp_sampling && (rc = check_sampling(tk, cp_sampling, cc.vocab)) != ATD_OK) return rc;
  if (tk_controls && (rc = check_controls(tk, tk_controls, tc.vocab)) != ATD_OK) return rc;
  if (tk->dry) {
    tk->pos[tk_slot] += steps;
    cp->pos[cp_slot] = kCodeGroups;
    return ATD_OK;
  }
  hipStream_t s = (hipStream_t)stream;
  const uint32_t pb = float_bits(penalty);
  const int64_t tag = 0x46524d;   // frame graphs in the Talker decoder's cache
  auto graph_for = [&](int full, hipGraphExec_t* out) -> hipError_t {
    std::vector<int64_t> key = {tag, full, tk_slot, (int64_t)(uintptr_t)cp, cp_slot,
                                (int64_t)(uintptr_t)codes_io, (int64_t)(uintptr_t)y_io,
                                (int64_t)(uintptr_t)text, (int64_t)(uintptr_t)seen, pb,
                                (int64_t)(uintptr_t)codes_out, (int64_t)(uintptr_t)tk_logits,
                                (int64_t)(uintptr_t)cp_logits,
                                std::min(tk->cap[tk_slot], tc.max_ctx),
                                std::min(cp->cap[cp_slot], cc.max_ctx), bucket_key(tk, tk_slot),
                                bucket_key(cp, cp_slot)};
    key_sampling(key, tk_sampling);
    key_sampling(key, cp_sampling);
    key_controls(key, tk_controls);
    for (auto& ge : tk->graphs)
      if (ge.key == key) {
        *out = ge.exec;
        return hipSuccess;
      }
    hipError_t e = hipSuccess;
    if (!tk->cap_stream) {
      e = hipStreamCreateWithFlags(&tk->cap_stream, hipStreamNonBlocking);
      if (e != hipSuccess) return e;
    }
    hipStream_t cs = tk->cap_stream;
    e = hipStreamBeginCapture(cs, hipStreamCaptureModeThreadLocal);
    if (e != hipSuccess) return e;
    hipError_t le = hipSuccess;
    if (full)
      le = enqueue_talker_step(tk, tk_slot, codes_io, text, tk->counter, seen, penalty,
                               tk_sampling, tk_controls, y_io, tk_logits, cs);
    if (le == hipSuccess)
      le = enqueue_cp_pass(cp, cp_slot, codes_io, y_io, cp_logits, codes_out, tk->counter,
                           cp_sampling, cs);
    hipGraph_t graph = nullptr;
    e = hipStreamEndCapture(cs, &graph);
    if (le != hipSuccess || e != hipSuccess) {
      if (graph) (void)hipGraphDestroy(graph);
      return le != hipSuccess ? le : e;
    }
    hipGraphExec_t exec = nullptr;
    e = hipGraphInstantiate(&exec, graph, nullptr, nullptr, 0);
    (void)hipGraphDestroy(graph);
    if (e != hipSuccess) return e;
    e = cache_graph(tk, key, exec);
    if (e != hipSuccess) return e;
    *out = exec;
    return hipSuccess;
  };
  hipGraphExec_t first = nullptr, rest = nullptr;
  hipError_t e = graph_for(0, &first);
  if (e == hipSuccess && steps > 0) e = graph_for(1, &rest);
  if (e != hipSuccess) return hip_fail(tk, e, "capture of the frame loop");
  e = launch_fill_i32(tk->counter, 1, 0, s);
  if (tk_controls && e == hipSuccess)
    e = launch_fill_i32(tk->ctl_base, 1, tk_controls->first_index, s);
  if (e == hipSuccess) e = hipGraphLaunch(first, s);
  for (int f = 1; f < n_frames && e == hipSuccess; ++f) e = hipGraphLaunch(rest, s);
  if (e != hipSuccess) return hip_fail(tk, e, "talker_generate_frames replay");
  tk->pos[tk_slot] += steps;
  cp->pos[cp_slot] = kCodeGroups;
  return ATD_OK;
}

// ---------------------------------------------------------------- read-stream bandwidth

extern "C" int atd_read_stream(const void* buf, size_t bytes, int32_t reps, uint32_t* sink,
                               void* stream, double* us_per_read) {
  if (!buf || !sink || !us_per_read)
    return fail(nullptr, ATD_ERR_INVALID_ARG, "buf, sink or us_per_read is NULL");
  if (!aligned16(buf)) return fail(nullptr, ATD_ERR_INVALID_ARG, "buf %p not 16-byte aligned", buf);
  if (bytes < 16 || bytes % 16)
    return fail(nullptr, ATD_ERR_INVALID_ARG, "bytes %zu not a positive multiple of 16", bytes);
  if (reps < 1) return fail(nullptr, ATD_ERR_INVALID_ARG, "reps %d < 1", reps);
  hipStream_t s = (hipStream_t)stream;
  hipEvent_t e0 = nullptr, e1 = nullptr;
  hipError_t e = hipEventCreate(&e0);
  if (e == hipSuccess) e = hipEventCreate(&e1);
  if (e == hipSuccess) e = launch_read_stream(buf, bytes, sink, s);   // warm-up pass
  if (e == hipSuccess) e = hipEventRecord(e0, s);
  for (int r = 0; r < reps && e == hipSuccess; ++r) e = launch_read_stream(buf, bytes, sink, s);
  if (e == hipSuccess) e = hipEventRecord(e1, s);
  if (e == hipSuccess) e = hipEventSynchronize(e1);
  float ms = 0.f;
  if (e == hipSuccess) e = hipEventElapsedTime(&ms, e0, e1);
  if (e0) (void)hipEventDestroy(e0);
  if (e1) (void)hipEventDestroy(e1);
  if (e != hipSuccess) return hip_fail(nullptr, e, "atd_read_stream");
  *us_per_read = (double)ms * 1e3 / reps;
  return ATD_OK;
}

// ---------------------------------------------------------------- stage timing

extern "C" int decoder_time_stage(atd_decoder* d, int32_t stage, int32_t slot0, int32_t B,
                                  int32_t reps, void* stream, double* us_per_layer) {
  if (!d) return fail(nullptr, ATD_ERR_INVALID_ARG, "decoder is NULL");
  if (stage != ATD_STAGE_QKV && stage != ATD_STAGE_ATTN && stage != ATD_STAGE_OPROJ &&
      stage != ATD_STAGE_GATEUP && stage != ATD_STAGE_DOWN)
    return fail(d, ATD_ERR_INVALID_ARG, "stage %d is not a per-layer decode stage", stage);
  if (B < 1 || B > d->cfg.max_rows)
    return fail(d, ATD_ERR_CAPACITY, "B = %d outside [1, max_rows = %d]", B, d->cfg.max_rows);
  if (slot0 < 0 || slot0 + B > d->cfg.max_slots)
    return fail(d, ATD_ERR_INVALID_ARG, "slots %d..%d outside [0, %d)", slot0, slot0 + B - 1,
                d->cfg.max_slots);
  int bound = 1;
  for (int b = slot0; b < slot0 + B; ++b) {
    if (!d->attached[b]) return fail(d, ATD_ERR_INVALID_ARG, "slot %d is not attached", b);
    if (stage == ATD_STAGE_ATTN && d->pos[b] >= d->cap[b])   // it writes the row at pos
      return fail(d, ATD_ERR_KV_FULL, "slot %d: position %d at capacity %d", b, d->pos[b],
                  d->cap[b]);
    bound = std::max(bound, std::min(d->pos[b] + 1, d->cap[b]));
  }
  if (reps < 1) return fail(d, ATD_ERR_INVALID_ARG, "reps %d < 1", reps);
  if (!us_per_layer) return fail(d, ATD_ERR_INVALID_ARG, "us_per_layer is NULL");
  if (d->dry) return fail(d, ATD_ERR_DEVICE, "dry-run decoder has no device");
  hipStream_t s = (hipStream_t)stream;
  hipEvent_t e0 = nullptr, e1 = nullptr;
  hipError_t e = hipEventCreate(&e0);
  if (e == hipSuccess) e = hipEventCreate(&e1);
  const RowMap rows{kRowsStep, slot0, 0};
  d->only_stage = stage;
  if (e == hipSuccess) e = hipEventRecord(e0, s);
  for (int r = 0; r < reps && e == hipSuccess; ++r)
    e = run_layers(d, rows, B, bound, d->x, nullptr, s);
  d->only_stage = -1;
  if (e == hipSuccess) e = hipEventRecord(e1, s);
  if (e == hipSuccess) e = hipEventSynchronize(e1);
  float ms = 0.f;
  if (e == hipSuccess) e = hipEventElapsedTime(&ms, e0, e1);
  if (e0) (void)hipEventDestroy(e0);
  if (e1) (void)hipEventDestroy(e1);
  if (e != hipSuccess) return hip_fail(d, e, "decoder_time_stage");
  *us_per_layer = (double)ms * 1e3 / ((double)reps * d->cfg.n_layers);
  return ATD_OK;
}
