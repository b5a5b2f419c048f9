// Host runtime behind the C ABI declared in include/pmk.h.
//
// Pages: "Netra Kernel" summary, details (a runtime with a C ABI binds persistent and boundary
// buffers and launches fixed kernels, or replays a prepared HIP graph, on a caller-owned stream;
// requests outside the exact operation contract are rejected rather than approximated) and
// "AutoMegaKernel" explainer, Safety Gate (an invalid schedule is rejected before any launch).
#include <hip/hip_runtime.h>

#include <algorithm>
#include <cmath>
#include <map>
#include <cstdio>
#include <cstring>
#include <mutex>
#include <string>
#include <vector>

#include "../../include/pmk.h"
#include "pmk_device.h"
#include "schedule.h"

namespace pmk {
const void* persistent_kernel(int wdt, int kvdt, int o_copy);
const void* phase_kernel(int wdt, int kvdt);
const void* prefill_kernel(int wdt, int kvdt);
hipError_t launch_begin_call(const KParams& P, const CallParams& cp, hipStream_t st);
hipError_t launch_reset(const KParams& P, int n_flags, int n_counters, int pos, int token, const int32_t* d_token,
                        hipStream_t st);
hipError_t launch_set_pos(const KParams& P, int pos, const int32_t* d_token, hipStream_t st);
hipError_t launch_copy_token(const KParams& P, int32_t* dst, hipStream_t st);
hipError_t launch_load_kv_rows(const KParams& P, const void* k, const void* v, int npos, int es, hipStream_t st);
hipError_t launch_read_kv_rows(const KParams& P, void* k, void* v, int npos, int es, hipStream_t st);
hipError_t launch_repack_qkv(uint8_t* dst, const void* wq, const void* wk, const void* wv, int nq, int nkv, int hd,
                             int64_t rowb, hipStream_t st);
hipError_t launch_repack_gu(uint8_t* dst, const void* wg, const void* wu, int F, int64_t rowb, hipStream_t st);
hipError_t launch_widen(float* dst, const void* src, int n, int bf16, hipStream_t st);
hipError_t launch_int_recode(uint8_t* p, int64_t bytes, int wdt, hipStream_t st);
hipError_t launch_kv_calib(const KParams& P, int finish, hipStream_t st);
hipError_t static_workspace_address(int device, void** out);
}  // namespace pmk

using namespace pmk;

namespace {

thread_local std::string g_err;

int64_t align256(int64_t v) { return (v + 255) & ~(int64_t)255; }

constexpr int kMaxTuneSteps = 64;  // steps of one measured run of the tuning search
int64_t nblk(int64_t n) { return (n + 127) / 128; }

// Scale elements of the 7 linear tensors of one layer (q k v o gate up down) and of the LM head:
// fp8 one per 128x128 block, int8 / int4 one per row and 128-column group.
void scale_counts(const ModelDims& m, int64_t sz[7]) {
  const int64_t H = m.H, F = m.F, qd = m.qdim(), kvd = (int64_t)m.nkv * m.hd;
  const int64_t rows[7] = {qd, kvd, kvd, H, F, F, H}, cols[7] = {H, H, H, qd, H, H, F};
  for (int i = 0; i < 7; ++i) sz[i] = (m.wdt == PMK_DT_FP8_E4M3 ? nblk(rows[i]) : rows[i]) * nblk(cols[i]);
}
// LDS of the batched prefill: the attention's eight wave records of 16 queries x (hd + 2) floats,
// or the GEMM's three 256-row x 64-byte weight buffers
size_t prefill_lds_bytes(const ModelDims& m) {
  return std::max((size_t)kWaves * 16 * (m.hd + 2) * 4, (size_t)3 * 256 * 64);
}
int64_t lm_scale_count(const ModelDims& m) { return (m.wdt == PMK_DT_FP8_E4M3 ? nblk(m.V) : m.V) * nblk(m.H); }

struct Phase {
  int first, count;
};

}  // namespace

struct pmk_ctx {
  pmk_model_config cfg;
  pmk_schedule_config sc;
  ModelDims m;
  Schedule sched;
  DeviceTables tabs;
  int device = -1;
  int n_cus = 0;
  int kves = 2;
  pmk_sizes sizes{};
  // arena layout (bytes)
  int64_t a_embed = 0, a_lm = 0, a_layers = 0, layer_bytes = 0, off_qkv = 0, off_o = 0, off_gu = 0, off_d = 0;
  int64_t a_gains = 0, a_final = 0, a_scales = 0, sc_layer = 0, sc_off[7] = {}, a_sclm = 0, a_rope = 0;
  // workspace layout (bytes)
  int64_t w_ctrl = 0, w_call = 0, w_flags = 0, w_counters = 0, w_keys = 0, w_tune = 0, w_kvscale = 0, w_kvamax = 0, w_x = 0,
          w_xm = 0, w_q = 0, w_kvcur = 0, w_part = 0, w_o = 0, w_h = 0, w_trace = 0, w_tasks = 0, w_qoff = 0, w_qtasks = 0,
          w_cprod = 0, w_cflag = 0;
  // batched prefill: tokens per chunk (0: none) and its chunk buffers
  int pf_chunk = 0;
  int64_t w_pfx = 0, w_pfxm = 0, w_pfx2 = 0, w_pfxm2 = 0, w_pfq = 0, w_pfbn = 0, w_pfbo = 0, w_pfbh = 0, w_pfbar = 0;
  uint8_t* arena = nullptr;
  uint8_t* kv = nullptr;
  uint8_t* ws = nullptr;
  bool bound = false, weights = false, kv_ready = false;
  bool ws_static = false;  // the workspace is the device's static array (pmk_bind_static_workspace)
  int32_t pos_host = 0;
  bool pos_exact = true;   // false after a decode call with an eos id: pos_host is then an upper bound
  int mode = PMK_MODE_MEGAKERNEL;
  int trace_on = 0;
  int xs_floats = 0;
  int epi_floats = 0, epi_off = 0, yp_off = 0, y_off = 0, xh_off = 0, gs_off = 0;
  int o_epi_off = 0, o_yp_off = 0, o_y_off = 0, pf_off = 0, pf_units = 0, attn_g2_off = -1;
  size_t lds_bytes = 0;     // per-op kernels
  size_t lds_bytes_pk = 0;  // persistent kernel (adds the O-projection tile area)
  KParams kp{};
  std::vector<Phase> phases;
  hipStream_t cap_stream = nullptr;
  hipGraph_t graph = nullptr;
  hipGraphExec_t graph_exec = nullptr;
  std::string err;
  std::vector<float> rope_host;
  uint64_t hash = 0;
  RowWeights rw;  // per-queue GEMV row shares set by pmk_tune (empty: even split)
  // workspace capacity, fixed at creation: schedules the tuner installs later (other combine parts,
  // O shares, fewer attention splits) must fit it, so no buffer moves when a schedule changes
  int64_t cap_flags = 0, cap_tasks = 0;
  int cap_splits = 0;
};

namespace {

pmk_status fail(pmk_ctx* c, pmk_status s, const std::string& msg) {
  if (c) c->err = msg;
  g_err = msg;
  return s;
}

#define HIPCHK(ctx, call)                                                                        \
  do {                                                                                           \
    hipError_t e_ = (call);                                                                      \
    if (e_ != hipSuccess)                                                                        \
      return fail(ctx, PMK_ERR_HIP, std::string(#call) + ": " + hipGetErrorString(e_));          \
  } while (0)

std::string contract_check(const pmk_model_config& c) {
  if (c.has_bias) return "biased projections are outside the contract";
  if (c.tie_embeddings) return "tied embeddings are outside the contract";
  if (c.n_layers < 1 || c.hidden < 1 || c.n_q_heads < 1 || c.n_kv_heads < 1 || c.ffn < 1 || c.vocab < 1 || c.max_seq < 1)
    return "every dimension must be positive";
  if (c.head_dim != 64 && c.head_dim != 128) return "head_dim must be 64 or 128";
  if (c.n_q_heads % c.n_kv_heads) return "n_q_heads must be a multiple of n_kv_heads";
  if (c.n_q_heads / c.n_kv_heads > 8) return "at most 8 query heads per kv head";
  const bool ok_pair = (c.weight_dtype == PMK_DT_F16 && c.kv_dtype == PMK_DT_F16) ||
                       (c.weight_dtype == PMK_DT_BF16 && c.kv_dtype == PMK_DT_BF16) ||
                       (c.weight_dtype == PMK_DT_FP8_E4M3 && c.kv_dtype == PMK_DT_FP8_E4M3) ||
                       (c.weight_dtype == PMK_DT_INT8 && c.kv_dtype == PMK_DT_BF16) ||
                       (c.weight_dtype == PMK_DT_INT4 && c.kv_dtype == PMK_DT_BF16);
  if (!ok_pair)
    return "supported (weight, kv) formats: (f16, f16), (bf16, bf16), (fp8, fp8), (int8, bf16), (int4, bf16)";
  const int epl = weight_epl(c.weight_dtype);
  if (c.hidden % epl || c.ffn % epl || (c.n_q_heads * c.head_dim) % epl)
    return "hidden, ffn and n_q_heads*head_dim must be multiples of 8 (16 for fp8 and int8, 32 for int4 weights)";
  const int kves = c.kv_dtype == PMK_DT_FP8_E4M3 ? 1 : 2;
  if (c.head_dim * kves < 128) return "a KV row (head_dim * element size) must cover at least 128 bytes";
  if (!(c.rms_eps > 0.f) || !(c.rope_theta > 0.f)) return "rms_eps and rope_theta must be positive";
  if (c.ffn > 36864 || c.hidden > 36864) return "hidden and ffn above 36864 exceed the staged-activation LDS budget";
  return "";
}

ModelDims dims_of(const pmk_model_config& c) {
  ModelDims m;
  m.L = c.n_layers;
  m.H = c.hidden;
  m.nq = c.n_q_heads;
  m.nkv = c.n_kv_heads;
  m.hd = c.head_dim;
  m.F = c.ffn;
  m.V = c.vocab;
  m.max_seq = c.max_seq;
  m.wdt = c.weight_dtype;
  m.kvdt = c.kv_dtype;
  m.eps = c.rms_eps;
  m.theta = c.rope_theta;
  return m;
}

pmk_schedule_config defaults(const pmk_schedule_config* s) {
  pmk_schedule_config d{};
  if (s) d = *s;
  if (d.spin_limit <= 0) d.spin_limit = 1ll << 22;
  d.prefetch = d.prefetch < 0 ? 0 : d.prefetch == 1 ? 1 : 2;
  return d;
}

// KV cache positions per head: the V cache is stored in blocks of 32 positions
int64_t seqcap_of(const ModelDims& m) { return ((int64_t)m.max_seq + 31) / 32 * 32; }

void compute_layout(pmk_ctx* c) {
  const ModelDims& m = c->m;
  const int64_t H = m.H, F = m.F, V = m.V, qd = m.qdim(), L = m.L;
  auto rb = [&](int64_t K) { return weight_row_bytes(m.wdt, K); };
  int64_t a = 0;
  c->a_embed = a; a = align256(a + V * H * 2);
  c->a_lm = a; a = align256(a + V * rb(H));
  int64_t lb = 0;
  c->off_qkv = lb; lb = align256(lb + (int64_t)m.qkv_rows() * rb(H));
  c->off_o = lb; lb = align256(lb + H * rb(qd));
  c->off_gu = lb; lb = align256(lb + 2 * F * rb(H));
  c->off_d = lb; lb = align256(lb + H * rb(F));
  c->layer_bytes = lb;
  c->a_layers = a; a = align256(a + L * lb);
  c->a_gains = a; a = align256(a + L * 2 * H * 4);
  c->a_final = a; a = align256(a + H * 4);
  c->a_scales = a;
  if (weight_scale_bytes(m.wdt) > 0) {
    int64_t sz[7];
    scale_counts(m, sz);
    int64_t off = 0;
    for (int i = 0; i < 7; ++i) { c->sc_off[i] = off; off += sz[i]; }
    c->sc_layer = off;
    const int es = weight_scale_bytes(m.wdt);
    a = align256(a + L * off * es);
    c->a_sclm = a;
    a = align256(a + lm_scale_count(m) * es);
  } else {
    c->sc_layer = 0;
    c->a_sclm = a;
  }
  c->a_rope = a; a = align256(a + (int64_t)m.max_seq * (m.hd / 2) * 8);
  c->sizes.arena_bytes = a;
  c->sizes.kv_bytes = 2 * align256((int64_t)L * m.nkv * seqcap_of(m) * m.hd * c->kves);

  const Schedule& s = c->sched;
  const int64_t NT = std::max<int64_t>(c->cap_tasks, (int64_t)s.tasks.size());
  int64_t w = 0;
  c->w_ctrl = w; w = align256(w + CTRL_WORDS * 4);
  c->w_call = w; w = align256(w + sizeof(CallParams));
  c->w_flags = w; w = align256(w + std::max<int64_t>(c->cap_flags, s.n_flags) * 4);
  c->w_counters = w; w = align256(w + (int64_t)s.counters.size() * 4);
  c->w_keys = w; w = align256(w + ((int64_t)std::max(m.max_seq, kMaxTuneSteps) + 1) * 8);
  c->w_tune = w; w = align256(w + (int64_t)kMaxTuneSteps * 4);
  c->w_kvscale = w; w = align256(w + L * m.nkv * 2 * 4);
  c->w_kvamax = w; w = align256(w + L * m.nkv * 2 * 4);
  c->w_x = w; w = align256(w + (L + 1) * H * 8);  // (tag, value) pairs
  c->w_xm = w; w = align256(w + L * H * 8);
  c->w_q = w; w = align256(w + L * qd * 8);  // (tag, value) pairs
  c->w_kvcur = w; w = align256(w + L * m.nkv * 2 * m.hd * 8);
  c->w_part = w; w = align256(w + L * m.nkv * std::max(c->cap_splits, s.attn_splits) * m.grp() * (m.hd + 4) * 4);
  c->w_o = w; w = align256(w + L * qd * 8);  // (tag, value) pairs
  c->w_h = w; w = align256(w + L * F * 4);
  c->w_trace = w; w = align256(w + (int64_t)std::max(0, c->sc.trace_steps) * NT * 64);
  c->w_tasks = w; w = align256(w + NT * (int64_t)sizeof(pmk_task));
  c->w_qoff = w; w = align256(w + ((int64_t)s.n_queues + 1) * 4);
  c->w_qtasks = w; w = align256(w + NT * 4);
  c->w_cprod = w; w = align256(w + (int64_t)s.counters.size() * 4);
  c->w_cflag = w; w = align256(w + (int64_t)s.counters.size() * 4);
  if (c->pf_chunk > 0) {
    const int64_t ch = c->pf_chunk;
    c->w_pfx = w; w = align256(w + ch * H * 4);
    c->w_pfxm = w; w = align256(w + ch * H * 4);
    c->w_pfq = w; w = align256(w + ch * qd * 4);
    c->w_pfx2 = w; w = align256(w + ch * H * 4);
    c->w_pfxm2 = w; w = align256(w + ch * H * 4);
    c->w_pfbn = w; w = align256(w + 2 * ch * H * 2);  // two 16-bit terms per activation
    c->w_pfbo = w; w = align256(w + 2 * ch * qd * 2);
    c->w_pfbh = w; w = align256(w + 2 * ch * F * 2);
    c->w_pfbar = w; w = align256(w + (int64_t)std::max(c->n_cus, 1) * 4);  // one barrier flag per workgroup
  }
  c->sizes.workspace_bytes = w;

  // LDS: staged activation vectors, or the attention scratch
  const int epl = weight_epl(m.wdt);
  auto padn = [&](int64_t n) { const int64_t sl = 64 * epl; return (n + sl - 1) / sl * sl; };
  const int64_t grp = m.grp();
  // attention: q [grp][hd], per-wave P.V partials [8][grp][hd], per-wave (max, sum) [8][grp][2]
  const int64_t attn = grp * m.hd + kWaves * grp * m.hd + kWaves * grp * 2 + 2 * m.hd;
  const int64_t xs = std::max({padn(H), padn(qd), padn(F), attn});
  c->xs_floats = (int)((xs + 63) / 64 * 64);
  // epilogue inputs staged behind the scratch words: the RoPE row (+ fp8 K/V scales) of QKV tasks,
  // the residual rows of OPROJ and DOWN tasks
  int64_t epi = m.hd + 4 * (int64_t)m.nkv, rmax = 1;
  for (const pmk_task& t : s.tasks) {
    if (t.op == PMK_OP_OPROJ || t.op == PMK_OP_DOWN) epi = std::max<int64_t>(epi, t.a1 - t.a0);
    if (t.op != PMK_OP_ATTN && t.op != PMK_OP_TOKEN && t.op != PMK_OP_COMBINE) rmax = std::max<int64_t>(rmax, t.a1 - t.a0);
  }
  c->epi_floats = (int)((epi + 63) / 64 * 64);
  c->epi_off = c->xs_floats + 64;
  c->yp_off = c->epi_off + c->epi_floats;
  c->y_off = c->yp_off + (int)((kWaves * rmax + 63) / 64 * 64);
  c->xh_off = c->y_off + (int)((rmax + 63) / 64 * 64);
  // integer weight formats: the normalised vector of an RMSNorm prologue as binary16 (the fp32
  // source stays in the staging area while it is rounded), and the prologue's gains in fp32
  const int64_t xh_floats = weight_is_int(m.wdt) ? (padn(H) / 2 + 63) / 64 * 64 : 0;
  const int64_t gs_floats = weight_is_int(m.wdt) ? padn(H) : 0;
  c->gs_off = c->xh_off + (int)xh_floats;
  c->lds_bytes = (size_t)(c->gs_off + gs_floats) * 4;
  // OPROJ tasks keep o, their residual rows, partial sums and results in a compact block; the rest
  // of LDS (persistent kernel only) holds the O-projection tile, copied before the task's wait.
  int64_t ormax = 1;
  for (const pmk_task& t : s.tasks)
    if (t.op == PMK_OP_OPROJ) ormax = std::max<int64_t>(ormax, t.a1 - t.a0);
  auto r64 = [](int64_t n) { return (n + 63) / 64 * 64; };
  c->o_epi_off = (int)r64(padn(qd));
  c->o_yp_off = c->o_epi_off + (int)r64(ormax);
  c->o_y_off = c->o_yp_off + (int)r64(kWaves * ormax);
  const int64_t o_end = c->o_y_off + r64(ormax);
  c->pf_off = (int)((std::max(o_end, r64(attn)) + 255) / 256 * 256);
  const int64_t lds_floats = kLdsBytes / 4;
  c->pf_units = c->sc.prefetch == 2 ? (int)std::max<int64_t>(0, (lds_floats - c->pf_off) / 256) : 0;
  c->lds_bytes_pk = c->pf_units > 0 ? std::max(c->lds_bytes, (size_t)(c->pf_off + (int64_t)c->pf_units * 256) * 4)
                                    : c->lds_bytes;
  // attention splits longer than 8 groups of 32 positions: per-wave buffers for the second group
  // (its K rows and V block), behind the attention scratch, when they fit
  c->attn_g2_off = -1;
  if (((int64_t)m.max_seq + s.attn_splits - 1) / s.attn_splits > 32 * kWaves) {
    const int64_t kes = m.kvdt == PMK_DT_FP8_E4M3 ? 1 : 2;
    const int64_t g2_floats = kWaves * (32 * m.hd * kes + m.hd * 32 * kes) / 4;
    const int64_t off = r64(attn);
    if (off + g2_floats <= lds_floats) {
      c->attn_g2_off = (int)off;
      c->lds_bytes_pk = std::max(c->lds_bytes_pk, (size_t)(off + g2_floats) * 4);
    }
  }
}

void fill_params(pmk_ctx* c) {
  KParams& P = c->kp;
  const ModelDims& m = c->m;
  P = KParams{};
  P.L = m.L; P.H = m.H; P.nq = m.nq; P.nkv = m.nkv; P.hd = m.hd; P.F = m.F; P.V = m.V;
  P.grp = m.grp(); P.qkv_rows = m.qkv_rows(); P.qdim = m.qdim(); P.max_seq = m.max_seq; P.S = c->sched.attn_splits;
  P.o_copy = c->sched.o_copy;
  P.seqcap = (int)seqcap_of(m);
  P.wdt = m.wdt; P.kvdt = m.kvdt; P.eps = m.eps;
  P.attn_scale = (float)(1.0 / std::sqrt((double)m.hd));
  uint8_t* A = c->arena;
  P.embed = reinterpret_cast<const uint16_t*>(A + c->a_embed);
  P.gains = reinterpret_cast<const float*>(A + c->a_gains);
  P.final_gain = reinterpret_cast<const float*>(A + c->a_final);
  P.wbase = A + c->a_layers;
  P.layer_bytes = c->layer_bytes;
  P.off_qkv = c->off_qkv; P.off_o = c->off_o; P.off_gu = c->off_gu; P.off_d = c->off_d;
  P.lm = A + c->a_lm;
  P.scales = A + c->a_scales;
  P.sc_layer = c->sc_layer;
  for (int i = 0; i < 7; ++i) P.sc_off[i] = c->sc_off[i];
  P.sc_lm = A + c->a_sclm;
  P.rope = reinterpret_cast<const float2*>(A + c->a_rope);
  P.kc = c->kv;
  P.vc = c->kv + c->sizes.kv_bytes / 2;
  uint8_t* W = c->ws;
  P.ctrl = reinterpret_cast<uint32_t*>(W + c->w_ctrl);
  P.call = reinterpret_cast<CallParams*>(W + c->w_call);
  P.flags = reinterpret_cast<uint32_t*>(W + c->w_flags);
  P.counters = reinterpret_cast<uint32_t*>(W + c->w_counters);
  P.keys = reinterpret_cast<unsigned long long*>(W + c->w_keys);
  P.kv_scale = reinterpret_cast<float*>(W + c->w_kvscale);
  P.kv_amax = reinterpret_cast<uint32_t*>(W + c->w_kvamax);
  P.x = reinterpret_cast<unsigned long long*>(W + c->w_x);
  P.xm = reinterpret_cast<unsigned long long*>(W + c->w_xm);
  P.q = reinterpret_cast<unsigned long long*>(W + c->w_q);
  P.kvcur = reinterpret_cast<unsigned long long*>(W + c->w_kvcur);
  P.part = reinterpret_cast<float*>(W + c->w_part);
  P.o = reinterpret_cast<unsigned long long*>(W + c->w_o);
  P.h = reinterpret_cast<float*>(W + c->w_h);
  P.trace = reinterpret_cast<unsigned long long*>(W + c->w_trace);
  P.tasks = reinterpret_cast<const pmk_task*>(W + c->w_tasks);
  P.qoff = reinterpret_cast<const int32_t*>(W + c->w_qoff);
  P.qtasks = reinterpret_cast<const int32_t*>(W + c->w_qtasks);
  P.ctr_prod = reinterpret_cast<const int32_t*>(W + c->w_cprod);
  P.ctr_flag = reinterpret_cast<const int32_t*>(W + c->w_cflag);
  P.n_queues = c->sched.n_queues;
  P.n_tasks = (int)c->sched.tasks.size();
  P.sync_mode = c->sched.sync_mode;
  P.prefetch = c->sc.prefetch;
  P.trace_steps = std::max(0, c->sc.trace_steps);
  P.spin_limit = c->sc.spin_limit;
  P.xs_floats = c->xs_floats;
  P.epi_off = c->epi_off;
  P.yp_off = c->yp_off;
  P.y_off = c->y_off;
  P.xh_off = c->xh_off;
  P.gs_off = c->gs_off;
  P.o_epi_off = c->o_epi_off;
  P.o_yp_off = c->o_yp_off;
  P.o_y_off = c->o_y_off;
  P.pf_off = c->pf_off;
  P.attn_g2_off = c->attn_g2_off;
  P.pf_units = c->pf_units;
}

void compute_phases(pmk_ctx* c) {
  c->phases.clear();
  const auto& T = c->sched.tasks;
  for (int i = 0; i < (int)T.size();) {
    int j = i;
    while (j < (int)T.size() && T[j].op == T[i].op && T[j].layer == T[i].layer) ++j;
    c->phases.push_back({i, j - i});
    i = j;
  }
}

// The context bound to each device's static workspace (one at a time: a later bind takes it over).
std::mutex g_static_mu;
pmk_ctx* g_static_owner[kMaxDevices] = {};

bool owns_static(const pmk_ctx* c) {
  std::lock_guard<std::mutex> lock(g_static_mu);
  return c->device >= 0 && c->device < kMaxDevices && g_static_owner[c->device] == c;
}

void release_static(pmk_ctx* c) {
  std::lock_guard<std::mutex> lock(g_static_mu);
  if (c->device >= 0 && c->device < kMaxDevices && g_static_owner[c->device] == c) g_static_owner[c->device] = nullptr;
  c->ws_static = false;
}

pmk_status need_device(pmk_ctx* c) {
  if (!c) return PMK_ERR_INVALID_ARG;
  if (c->device < 0) return fail(c, PMK_ERR_NOT_BOUND, "context was created without a device");
  if (!c->bound) return fail(c, PMK_ERR_NOT_BOUND, "buffers are not bound (pmk_bind)");
  if (c->ws_static && !owns_static(c))
    return fail(c, PMK_ERR_NOT_BOUND, "another context has since bound this device's static workspace; bind again");
  HIPCHK(c, hipSetDevice(c->device));
  return PMK_OK;
}

// After a decode call with an eos id the device's position word is the exact position: read it.
pmk_status sync_position(pmk_ctx* c) {
  if (c->pos_exact) return PMK_OK;
  HIPCHK(c, hipSetDevice(c->device));
  HIPCHK(c, hipDeviceSynchronize());
  uint32_t pos = 0;
  HIPCHK(c, hipMemcpy(&pos, c->ws + c->w_ctrl + CTRL_POS * 4, 4, hipMemcpyDeviceToHost));
  c->pos_host = (int32_t)pos;
  c->pos_exact = true;
  return PMK_OK;
}

pmk_status launch_persistent(pmk_ctx* c, hipStream_t st) {
  const void* fn = persistent_kernel(c->m.wdt, c->m.kvdt, c->sched.o_copy);
  void* args[] = {&c->kp};
  HIPCHK(c, hipLaunchCooperativeKernel(fn, dim3(c->n_cus), dim3(kThreads), args, (unsigned)c->lds_bytes_pk, st));
  return PMK_OK;
}

pmk_status launch_step_per_op(pmk_ctx* c, hipStream_t st) {
  const void* fn = phase_kernel(c->m.wdt, c->m.kvdt);
  for (const Phase& ph : c->phases) {
    int first = ph.first;
    void* args[] = {&c->kp, &first};
    HIPCHK(c, hipLaunchKernel(fn, dim3(ph.count), dim3(kThreads), args, c->lds_bytes, st));
  }
  return PMK_OK;
}

pmk_status ensure_graph(pmk_ctx* c) {
  if (c->graph_exec) return PMK_OK;
  if (!c->cap_stream) HIPCHK(c, hipStreamCreateWithFlags(&c->cap_stream, hipStreamNonBlocking));
  HIPCHK(c, hipStreamBeginCapture(c->cap_stream, hipStreamCaptureModeThreadLocal));
  pmk_status s = launch_step_per_op(c, c->cap_stream);
  hipGraph_t g = nullptr;
  hipError_t e = hipStreamEndCapture(c->cap_stream, &g);
  if (s != PMK_OK) return s;
  if (e != hipSuccess) return fail(c, PMK_ERR_HIP, std::string("hipStreamEndCapture: ") + hipGetErrorString(e));
  c->graph = g;
  HIPCHK(c, hipGraphInstantiate(&c->graph_exec, g, nullptr, nullptr, 0));
  return PMK_OK;
}

// Run `n` steps of the current call (begin_call already issued) in the context's mode.
pmk_status run_steps(pmk_ctx* c, int n, hipStream_t st) {
  if (c->mode == PMK_MODE_MEGAKERNEL) return launch_persistent(c, st);
  if (c->mode == PMK_MODE_GRAPH) {
    pmk_status s = ensure_graph(c);
    if (s != PMK_OK) return s;
    for (int i = 0; i < n; ++i) HIPCHK(c, hipGraphLaunch(c->graph_exec, st));
    return PMK_OK;
  }
  for (int i = 0; i < n; ++i) {
    pmk_status s = launch_step_per_op(c, st);
    if (s != PMK_OK) return s;
  }
  return PMK_OK;
}

pmk_status begin_call(pmk_ctx* c, const CallParams& cp, hipStream_t st) {
  HIPCHK(c, launch_begin_call(c->kp, cp, st));
  return PMK_OK;
}

pmk_status run_prefill(pmk_ctx* c, const int32_t* d_tokens, int32_t P, int calib, hipStream_t st) {
  HIPCHK(c, launch_reset(c->kp, c->sched.n_flags, (int)c->sched.counters.size(), 0, 0, nullptr, st));
  const int chunk = 256;
  for (int off = 0; off < P; off += chunk) {
    const int n = std::min(chunk, P - off);
    CallParams cp{};
    cp.forced = d_tokens + off;
    cp.n_steps = n;
    cp.eos = -1;
    cp.calib = calib;
    pmk_status s = begin_call(c, cp, st);
    if (s != PMK_OK) return s;
    s = run_steps(c, n, st);
    if (s != PMK_OK) return s;
  }
  return PMK_OK;
}

pmk_status set_kv_scales(pmk_ctx* c, const float* d_kv_scales, hipStream_t st) {
  const size_t bytes = (size_t)c->m.L * c->m.nkv * 2 * 4;
  if (c->m.kvdt == PMK_DT_FP8_E4M3) {
    if (!d_kv_scales) return fail(c, PMK_ERR_INVALID_ARG, "an fp8 KV cache needs d_kv_scales [n_layers][n_kv][2]");
    HIPCHK(c, hipMemcpyAsync(c->ws + c->w_kvscale, d_kv_scales, bytes, hipMemcpyDeviceToDevice, st));
  }
  return PMK_OK;
}

// Teacher-forced run of positions 0..P-1 from d_tokens (launches of at most 256 steps), from a
// reset synchronisation state.
pmk_status run_prefill(pmk_ctx* c, const int32_t* d_tokens, int32_t P, int calib, hipStream_t st);

}  // namespace

// =================================================================================================
// C ABI
// =================================================================================================
extern "C" {

int pmk_abi_version(void) { return PMK_ABI_VERSION; }

const char* pmk_status_str(pmk_status s) {
  switch (s) {
    case PMK_OK: return "ok";
    case PMK_ERR_INVALID_ARG: return "invalid argument";
    case PMK_ERR_UNSUPPORTED: return "outside the operation contract";
    case PMK_ERR_SCHEDULE_INVALID: return "schedule rejected by the static validator";
    case PMK_ERR_CAPACITY: return "KV capacity exceeded";
    case PMK_ERR_NOT_BOUND: return "not bound or not loaded";
    case PMK_ERR_HIP: return "HIP runtime error";
    case PMK_ERR_TIMEOUT: return "device wait timed out";
    case PMK_ERR_NAN: return "NaN logits";
    case PMK_ERR_DEVICE: return "unsupported device";
  }
  return "unknown status";
}

const char* pmk_last_error(const pmk_ctx* ctx) { return ctx ? ctx->err.c_str() : g_err.c_str(); }
const char* pmk_last_global_error(void) { return g_err.c_str(); }

pmk_status pmk_create(const pmk_model_config* cfg, const pmk_schedule_config* sched, int hip_device, pmk_ctx** out) {
  g_err.clear();
  if (!cfg || !out) return fail(nullptr, PMK_ERR_INVALID_ARG, "cfg and out must not be NULL");
  *out = nullptr;
  const std::string why = contract_check(*cfg);
  if (!why.empty()) return fail(nullptr, PMK_ERR_UNSUPPORTED, why);
  pmk_ctx* c = new pmk_ctx();
  c->cfg = *cfg;
  c->sc = defaults(sched);
  c->m = dims_of(*cfg);
  c->kves = cfg->kv_dtype == PMK_DT_FP8_E4M3 ? 1 : 2;
  c->device = hip_device;
  int n_cus = c->sc.n_cus;
  if (hip_device >= 0) {
    hipDeviceProp_t p;
    hipError_t e = hipGetDeviceProperties(&p, hip_device);
    if (e != hipSuccess) { delete c; return fail(nullptr, PMK_ERR_HIP, std::string("hipGetDeviceProperties: ") + hipGetErrorString(e)); }
    if (std::strncmp(p.gcnArchName, "gfx950", 6) != 0) {
      delete c;
      return fail(nullptr, PMK_ERR_DEVICE, std::string("device is ") + p.gcnArchName + ", the kernels are built for gfx950");
    }
    if (!p.cooperativeLaunch) { delete c; return fail(nullptr, PMK_ERR_DEVICE, "device lacks cooperative launch"); }
    if (n_cus <= 0 || n_cus > p.multiProcessorCount) n_cus = p.multiProcessorCount;
  } else if (n_cus <= 0) {
    n_cus = 256;
  }
  c->n_cus = n_cus;
  {
    // batched prefill: tokens per chunk
    const int ch = c->sc.prefill_chunk;
    if (ch < -1 || (ch > 0 && (ch % 128 != 0 || ch > 1024))) {
      delete c;
      return fail(nullptr, PMK_ERR_INVALID_ARG, "prefill_chunk must be 0, -1 or a multiple of 128 up to 1024");
    }
    if (c->sc.prefill_ksplit < 0 || c->sc.prefill_ksplit > 2) {
      delete c;
      return fail(nullptr, PMK_ERR_INVALID_ARG, "prefill_ksplit must be 0, 1 or 2");
    }
    if (c->sc.combine_o_copy < 0 || c->sc.combine_o_copy > 2) {
      delete c;
      return fail(nullptr, PMK_ERR_INVALID_ARG, "combine_o_copy must be 0, 1 or 2");
    }
    const int cap = (c->m.max_seq + 127) / 128 * 128;
    c->pf_chunk = ch == -1 ? 0 : std::min(ch == 0 ? 512 : ch, cap);
  }
  std::string e = build_schedule(c->m, c->sc, n_cus, &c->sched);
  if (!e.empty()) { delete c; return fail(nullptr, PMK_ERR_SCHEDULE_INVALID, e); }
  e = validate_schedule(c->sched);
  if (!e.empty()) { delete c; return fail(nullptr, PMK_ERR_SCHEDULE_INVALID, e); }
  c->tabs = flatten(c->sched);
  c->hash = schedule_hash(c->sched);
  {
    // capacity for the schedules tuning may install: as many combines per kv head as q heads, full
    // O-projection shares on their queues, at most the default attention splits
    c->cap_flags = c->sched.n_flags;
    c->cap_tasks = (int64_t)c->sched.tasks.size();
    c->cap_splits = c->sched.attn_splits;
    pmk_schedule_config cap_sc = c->sc;
    cap_sc.combine_parts = c->m.grp();
    cap_sc.combine_o_share = 3;
    Schedule cap;
    if (build_schedule(c->m, cap_sc, n_cus, &cap).empty()) {
      c->cap_flags = std::max<int64_t>(c->cap_flags, cap.n_flags);
      c->cap_tasks = std::max<int64_t>(c->cap_tasks, (int64_t)cap.tasks.size());
    }
  }
  compute_layout(c);
  if (c->lds_bytes > (size_t)kLdsBytes || c->lds_bytes_pk > (size_t)kLdsBytes) {
    delete c;
    return fail(nullptr, PMK_ERR_UNSUPPORTED, "the staged activations and attention scratch exceed 160 KiB of LDS");
  }
  compute_phases(c);
  if (hip_device >= 0) {
    hipError_t he = hipSetDevice(hip_device);
    const void* fns[3] = {persistent_kernel(c->m.wdt, c->m.kvdt, c->sched.o_copy), phase_kernel(c->m.wdt, c->m.kvdt),
                          persistent_kernel(c->m.wdt, c->m.kvdt, !c->sched.o_copy)};
    // the attribute is an upper bound shared by every context: allow all of a CU's LDS
    for (const void* fn : fns) {
      if (he == hipSuccess) he = hipFuncSetAttribute(fn, hipFuncAttributeMaxDynamicSharedMemorySize, kLdsBytes);
    }
    int per_cu = 0;
    if (he == hipSuccess) he = hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, fns[0], kThreads, c->lds_bytes_pk);
    if (he != hipSuccess) { delete c; return fail(nullptr, PMK_ERR_HIP, std::string("kernel setup: ") + hipGetErrorString(he)); }
    if (per_cu < 1) { delete c; return fail(nullptr, PMK_ERR_DEVICE, "the persistent kernel cannot be resident on a CU"); }
    if (c->pf_chunk > 0) {
      per_cu = 0;
      const void* pf = prefill_kernel(c->m.wdt, c->m.kvdt);
      he = hipFuncSetAttribute(pf, hipFuncAttributeMaxDynamicSharedMemorySize, kLdsBytes);
      if (he == hipSuccess)
        he = hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, pf, kThreads, prefill_lds_bytes(c->m));
      if (he != hipSuccess || per_cu < 1) c->pf_chunk = 0;  // step-by-step prefill then
    }
  }
  *out = c;
  return PMK_OK;
}

void pmk_destroy(pmk_ctx* c) {
  if (!c) return;
  release_static(c);
  if (c->device >= 0) (void)hipSetDevice(c->device);
  if (c->graph_exec) (void)hipGraphExecDestroy(c->graph_exec);
  if (c->graph) (void)hipGraphDestroy(c->graph);
  if (c->cap_stream) (void)hipStreamDestroy(c->cap_stream);
  delete c;
}

pmk_status pmk_buffer_sizes(const pmk_ctx* c, pmk_sizes* out) {
  if (!c || !out) return PMK_ERR_INVALID_ARG;
  *out = c->sizes;
  return PMK_OK;
}

static pmk_status bind_impl(pmk_ctx* c, void* d_arena, void* d_kv, void* d_ws) {
  c->arena = (uint8_t*)d_arena;
  c->kv = (uint8_t*)d_kv;
  c->ws = (uint8_t*)d_ws;
  fill_params(c);
  // schedule tables and a clean synchronisation state
  HIPCHK(c, hipMemcpy(c->ws + c->w_tasks, c->tabs.tasks.data(), c->tabs.tasks.size() * sizeof(pmk_task), hipMemcpyHostToDevice));
  HIPCHK(c, hipMemcpy(c->ws + c->w_qoff, c->tabs.qoff.data(), c->tabs.qoff.size() * 4, hipMemcpyHostToDevice));
  HIPCHK(c, hipMemcpy(c->ws + c->w_qtasks, c->tabs.qtasks.data(), c->tabs.qtasks.size() * 4, hipMemcpyHostToDevice));
  HIPCHK(c, hipMemcpy(c->ws + c->w_cprod, c->tabs.ctr_producers.data(), c->tabs.ctr_producers.size() * 4, hipMemcpyHostToDevice));
  HIPCHK(c, hipMemcpy(c->ws + c->w_cflag, c->tabs.ctr_flag_base.data(), c->tabs.ctr_flag_base.size() * 4, hipMemcpyHostToDevice));
  HIPCHK(c, hipMemset(c->ws + c->w_kvscale, 0, (size_t)c->m.L * c->m.nkv * 2 * 4));
  HIPCHK(c, hipMemset(c->ws + c->w_kvamax, 0, (size_t)c->m.L * c->m.nkv * 2 * 4));
  HIPCHK(c, launch_reset(c->kp, c->sched.n_flags, (int)c->sched.counters.size(), 0, 0, nullptr, nullptr));
  HIPCHK(c, hipDeviceSynchronize());
  if (c->graph_exec) { (void)hipGraphExecDestroy(c->graph_exec); c->graph_exec = nullptr; }
  if (c->graph) { (void)hipGraphDestroy(c->graph); c->graph = nullptr; }
  c->bound = true;
  c->weights = false;
  c->kv_ready = false;
  c->pos_host = 0;
  c->pos_exact = true;
  return PMK_OK;
}

pmk_status pmk_bind(pmk_ctx* c, void* d_arena, void* d_kv, void* d_ws) {
  if (!c) return PMK_ERR_INVALID_ARG;
  if (c->device < 0) return fail(c, PMK_ERR_NOT_BOUND, "context was created without a device");
  if (!d_arena || !d_kv || !d_ws) return fail(c, PMK_ERR_INVALID_ARG, "buffers must not be NULL");
  if (((uintptr_t)d_arena | (uintptr_t)d_kv | (uintptr_t)d_ws) & 255)
    return fail(c, PMK_ERR_INVALID_ARG, "buffers must be 256-byte aligned");
  HIPCHK(c, hipSetDevice(c->device));
  release_static(c);
  c->bound = false;
  return bind_impl(c, d_arena, d_kv, d_ws);
}

pmk_status pmk_bind_static_workspace(pmk_ctx* c, void* d_arena, void* d_kv) {
  if (!c) return PMK_ERR_INVALID_ARG;
  if (c->sizes.workspace_bytes > kStaticWorkspaceBytes)
    return fail(c, PMK_ERR_CAPACITY,
                "this schedule's workspace needs " + std::to_string(c->sizes.workspace_bytes) +
                    " bytes; the static workspace holds at most " + std::to_string(kStaticWorkspaceBytes) +
                    " (use pmk_bind with a caller-allocated workspace, or a schedule without a trace ring)");
  if (c->device < 0) return fail(c, PMK_ERR_NOT_BOUND, "context was created without a device");
  if (c->device >= kMaxDevices) return fail(c, PMK_ERR_DEVICE, "device index beyond the static workspace table");
  if (!d_arena || !d_kv) return fail(c, PMK_ERR_INVALID_ARG, "buffers must not be NULL");
  if (((uintptr_t)d_arena | (uintptr_t)d_kv) & 255) return fail(c, PMK_ERR_INVALID_ARG, "buffers must be 256-byte aligned");
  HIPCHK(c, hipSetDevice(c->device));
  void* ws = nullptr;
  HIPCHK(c, static_workspace_address(c->device, &ws));
  {
    std::lock_guard<std::mutex> lock(g_static_mu);
    g_static_owner[c->device] = c;  // a context bound before loses it (its device calls then fail)
  }
  c->ws_static = true;
  c->bound = false;
  return bind_impl(c, d_arena, d_kv, ws);
}

pmk_status pmk_load_weights(pmk_ctx* c, const pmk_weight_ptrs* w, void* stream) {
  pmk_status s = need_device(c);
  if (s != PMK_OK) return s;
  hipStream_t st = (hipStream_t)stream;
  const ModelDims& m = c->m;
  const int ses = weight_scale_bytes(m.wdt);  // scale element bytes, 0 for unscaled formats
  if (!w || !w->embed || !w->final_norm || !w->lm_head || !w->layers) return fail(c, PMK_ERR_INVALID_ARG, "missing weight pointers");
  if (ses && (!w->lm_head_scale || !w->layer_scales))
    return fail(c, PMK_ERR_INVALID_ARG, "fp8, int8 and int4 weights need their scales");
  const int64_t H = m.H, F = m.F, V = m.V, qd = m.qdim();
  auto rb = [&](int64_t K) { return weight_row_bytes(m.wdt, K); };
  const int gbf16 = m.wdt == PMK_DT_F16 ? 0 : 1;
  for (int l = 0; l < m.L; ++l)
    for (int k = 0; k < 9; ++k)
      if (!w->layers[l * 9 + k]) return fail(c, PMK_ERR_INVALID_ARG, "missing layer weight pointer");
  HIPCHK(c, hipMemcpyAsync(c->arena + c->a_embed, w->embed, V * H * 2, hipMemcpyDeviceToDevice, st));
  HIPCHK(c, hipMemcpyAsync(c->arena + c->a_lm, w->lm_head, V * rb(H), hipMemcpyDeviceToDevice, st));
  for (int l = 0; l < m.L; ++l) {
    const void* const* L9 = w->layers + l * 9;
    uint8_t* base = c->arena + c->a_layers + l * c->layer_bytes;
    HIPCHK(c, launch_repack_qkv(base + c->off_qkv, L9[0], L9[1], L9[2], m.nq, m.nkv, m.hd, rb(H), st));
    HIPCHK(c, hipMemcpyAsync(base + c->off_o, L9[3], H * rb(qd), hipMemcpyDeviceToDevice, st));
    HIPCHK(c, launch_repack_gu(base + c->off_gu, L9[4], L9[5], m.F, rb(H), st));
    HIPCHK(c, hipMemcpyAsync(base + c->off_d, L9[6], H * rb(F), hipMemcpyDeviceToDevice, st));
    float* g = reinterpret_cast<float*>(c->arena + c->a_gains) + (int64_t)l * 2 * H;
    HIPCHK(c, launch_widen(g, L9[7], (int)H, gbf16, st));
    HIPCHK(c, launch_widen(g + H, L9[8], (int)H, gbf16, st));
    if (ses) {
      const void* const* S7 = w->layer_scales + l * 7;
      int64_t sz[7];
      scale_counts(m, sz);
      uint8_t* sb = c->arena + c->a_scales + l * c->sc_layer * ses;
      for (int k = 0; k < 7; ++k) {
        if (!S7[k]) return fail(c, PMK_ERR_INVALID_ARG, "missing scale pointer");
        HIPCHK(c, hipMemcpyAsync(sb + c->sc_off[k] * ses, S7[k], sz[k] * ses, hipMemcpyDeviceToDevice, st));
      }
    }
  }
  HIPCHK(c, launch_widen(reinterpret_cast<float*>(c->arena + c->a_final), w->final_norm, (int)H, gbf16, st));
  if (ses)
    HIPCHK(c, hipMemcpyAsync(c->arena + c->a_sclm, w->lm_head_scale, lm_scale_count(m) * ses, hipMemcpyDeviceToDevice,
                             st));
  if (weight_is_int(m.wdt)) {  // every code of the LM head and the layer blocks (padding included)
    HIPCHK(c, launch_int_recode(c->arena + c->a_lm, V * rb(H), m.wdt, st));
    HIPCHK(c, launch_int_recode(c->arena + c->a_layers, m.L * c->layer_bytes, m.wdt, st));
  }
  // RoPE table: angle p * theta^(-2i/hd) in double, cos and sin rounded to fp32
  const int half = m.hd / 2;
  c->rope_host.resize((size_t)m.max_seq * half * 2);
  for (int p = 0; p < m.max_seq; ++p)
    for (int i = 0; i < half; ++i) {
      const double ang = (double)p * std::pow((double)m.theta, -2.0 * i / (double)m.hd);
      c->rope_host[((size_t)p * half + i) * 2] = (float)std::cos(ang);
      c->rope_host[((size_t)p * half + i) * 2 + 1] = (float)std::sin(ang);
    }
  HIPCHK(c, hipMemcpyAsync(c->arena + c->a_rope, c->rope_host.data(), c->rope_host.size() * 4, hipMemcpyHostToDevice, st));
  c->weights = true;
  return PMK_OK;
}

pmk_status pmk_prefill_kv(pmk_ctx* c, const int32_t* d_tokens, int32_t P, const float* d_kv_scales, int32_t* d_first_token,
                          void* stream) {
  pmk_status s = need_device(c);
  if (s != PMK_OK) return s;
  if (!c->weights) return fail(c, PMK_ERR_NOT_BOUND, "weights are not loaded");
  if (!d_tokens || P <= 0) return fail(c, PMK_ERR_INVALID_ARG, "prefill needs P > 0 device tokens");
  if (P > c->m.max_seq) return fail(c, PMK_ERR_CAPACITY, "prompt longer than max_seq");
  hipStream_t st = (hipStream_t)stream;
  // one prefill pass: batched (positions 0..P-2 in one launch, then the last position as a
  // teacher-forced decode step, whose logits give the first token) or step by step
  auto pass = [&](int calib) -> pmk_status {
    if (c->pf_chunk <= 0 || P < 2) return run_prefill(c, d_tokens, P, calib, st);
    PrefillArgs a{};
    a.tokens = d_tokens;
    a.n = P - 1;
    a.chunk = c->pf_chunk;
    a.x = reinterpret_cast<float*>(c->ws + c->w_pfx);
    a.xm = reinterpret_cast<float*>(c->ws + c->w_pfxm);
    a.x2 = reinterpret_cast<float*>(c->ws + c->w_pfx2);
    a.xm2 = reinterpret_cast<float*>(c->ws + c->w_pfxm2);
    a.q = reinterpret_cast<float*>(c->ws + c->w_pfq);
    a.bn = reinterpret_cast<uint16_t*>(c->ws + c->w_pfbn);
    a.bo = reinterpret_cast<uint16_t*>(c->ws + c->w_pfbo);
    a.bh = reinterpret_cast<uint16_t*>(c->ws + c->w_pfbh);
    a.bar = reinterpret_cast<uint32_t*>(c->ws + c->w_pfbar);
    a.calib = calib;
    a.ksplit = c->sc.prefill_ksplit;
    HIPCHK(c, launch_reset(c->kp, c->sched.n_flags, (int)c->sched.counters.size(), P - 1, 0, d_tokens + P - 1, st));
    HIPCHK(c, hipMemsetAsync(a.bar, 0, (size_t)c->n_cus * 4, st));
    void* args[] = {&c->kp, &a};
    HIPCHK(c, hipLaunchCooperativeKernel(prefill_kernel(c->m.wdt, c->m.kvdt), dim3(c->n_cus), dim3(kThreads), args,
                                         (unsigned)prefill_lds_bytes(c->m), st));
    CallParams cp{};
    cp.forced = d_tokens + P - 1;
    cp.n_steps = 1;
    cp.eos = -1;
    cp.calib = calib;
    pmk_status r = begin_call(c, cp, st);
    if (r == PMK_OK) r = run_steps(c, 1, st);
    return r;
  };
  if (c->m.kvdt == PMK_DT_FP8_E4M3 && !d_kv_scales) {
    // static scales from this prompt: a calibration pass with every scale 1 records max |k|, |v|
    // per (layer, kv head); each scale becomes that maximum / 448; then the real prefill
    HIPCHK(c, launch_kv_calib(c->kp, 0, st));
    s = pass(1);
    if (s != PMK_OK) return s;
    HIPCHK(c, launch_kv_calib(c->kp, 1, st));
  } else {
    s = set_kv_scales(c, d_kv_scales, st);
    if (s != PMK_OK) return s;
  }
  s = pass(0);
  if (s != PMK_OK) return s;
  if (d_first_token) HIPCHK(c, launch_copy_token(c->kp, d_first_token, st));
  c->pos_host = P;
  c->pos_exact = true;
  c->kv_ready = true;
  return PMK_OK;
}

pmk_status pmk_get_kv_scales(pmk_ctx* c, float* d_out, void* stream) {
  pmk_status s = need_device(c);
  if (s != PMK_OK) return s;
  if (!d_out) return fail(c, PMK_ERR_INVALID_ARG, "d_out must not be NULL");
  if (c->m.kvdt != PMK_DT_FP8_E4M3) return fail(c, PMK_ERR_INVALID_ARG, "only an fp8 KV cache has scales");
  HIPCHK(c, hipMemcpyAsync(d_out, c->ws + c->w_kvscale, (size_t)c->m.L * c->m.nkv * 2 * 4, hipMemcpyDeviceToDevice,
                           (hipStream_t)stream));
  return PMK_OK;
}

pmk_status pmk_load_kv(pmk_ctx* c, const void* d_k, const void* d_v, int32_t P, int32_t next_token, const float* d_kv_scales,
                       void* stream) {
  pmk_status s = need_device(c);
  if (s != PMK_OK) return s;
  if (P < 0 || P > c->m.max_seq) return fail(c, PMK_ERR_CAPACITY, "P exceeds max_seq");
  if (P > 0 && (!d_k || !d_v)) return fail(c, PMK_ERR_INVALID_ARG, "missing KV pointers");
  if (next_token < 0 || next_token >= c->m.V) return fail(c, PMK_ERR_INVALID_ARG, "next_token out of range");
  hipStream_t st = (hipStream_t)stream;
  s = set_kv_scales(c, d_kv_scales, st);
  if (s != PMK_OK) return s;
  HIPCHK(c, launch_reset(c->kp, c->sched.n_flags, (int)c->sched.counters.size(), P, next_token, nullptr, st));
  if (P > 0) HIPCHK(c, launch_load_kv_rows(c->kp, d_k, d_v, P, c->kves, st));
  c->pos_host = P;
  c->pos_exact = true;
  c->kv_ready = true;
  return PMK_OK;
}

pmk_status pmk_read_kv(pmk_ctx* c, void* d_k, void* d_v, int32_t P, void* stream) {
  pmk_status s = need_device(c);
  if (s != PMK_OK) return s;
  if (!c->kv_ready) return fail(c, PMK_ERR_NOT_BOUND, "no KV state to read");
  s = sync_position(c);
  if (s != PMK_OK) return s;
  if (P < 0 || P > c->pos_host) return fail(c, PMK_ERR_INVALID_ARG, "P must be within the written positions");
  if (P > 0 && (!d_k || !d_v)) return fail(c, PMK_ERR_INVALID_ARG, "missing KV pointers");
  if (P > 0) HIPCHK(c, launch_read_kv_rows(c->kp, d_k, d_v, P, c->kves, (hipStream_t)stream));
  return PMK_OK;
}

pmk_status pmk_rewind(pmk_ctx* c, int32_t pos, const int32_t* d_token, void* stream) {
  pmk_status s = need_device(c);
  if (s != PMK_OK) return s;
  if (!c->kv_ready) return fail(c, PMK_ERR_NOT_BOUND, "no KV state to rewind");
  s = sync_position(c);  // only positions whose KV rows were written are valid targets
  if (s != PMK_OK) return s;
  if (pos <= 0 || pos > c->pos_host || !d_token) return fail(c, PMK_ERR_INVALID_ARG, "rewind needs 0 < pos <= position and a token");
  HIPCHK(c, launch_set_pos(c->kp, pos, d_token, (hipStream_t)stream));
  c->pos_host = pos;
  return PMK_OK;
}

pmk_status pmk_decode_n_tokens(pmk_ctx* c, int32_t n, int32_t* d_out_tokens, float* d_out_logits, int32_t eos_id,
                               int32_t* d_n_done, void* stream) {
  pmk_status s = need_device(c);
  if (s != PMK_OK) return s;
  if (!c->weights || !c->kv_ready) return fail(c, PMK_ERR_NOT_BOUND, "weights and KV state must be loaded first");
  if (n <= 0 || !d_out_tokens) return fail(c, PMK_ERR_INVALID_ARG, "n > 0 and d_out_tokens are required");
  s = sync_position(c);
  if (s != PMK_OK) return s;
  if ((int64_t)c->pos_host + n > c->m.max_seq) return fail(c, PMK_ERR_CAPACITY, "position + n exceeds max_seq");
  hipStream_t st = (hipStream_t)stream;
  CallParams cp{};
  cp.out_tokens = d_out_tokens;
  cp.out_logits = d_out_logits;
  cp.n_done = d_n_done;
  cp.forced = nullptr;
  cp.n_steps = n;
  cp.eos = eos_id;
  cp.trace = c->trace_on;
  s = begin_call(c, cp, st);
  if (s != PMK_OK) return s;
  s = run_steps(c, n, st);
  if (s != PMK_OK) return s;
  c->pos_host += n;
  if (eos_id >= 0) c->pos_exact = false;  // the device stops after the eos step: it keeps the exact position
  return PMK_OK;
}

pmk_status pmk_set_mode(pmk_ctx* c, int32_t mode) {
  if (!c || mode < PMK_MODE_MEGAKERNEL || mode > PMK_MODE_PER_OP) return PMK_ERR_INVALID_ARG;
  c->mode = mode;
  return PMK_OK;
}

pmk_status pmk_get_position(const pmk_ctx* cc, int32_t* pos) {
  if (!cc || !pos) return PMK_ERR_INVALID_ARG;
  pmk_ctx* c = const_cast<pmk_ctx*>(cc);  // the exact position may have to be read from the device
  if (!c->pos_exact) {
    pmk_status s = need_device(c);
    if (s != PMK_OK) return s;
    s = sync_position(c);
    if (s != PMK_OK) return s;
  }
  *pos = c->pos_host;
  return PMK_OK;
}

pmk_status pmk_poll_error(pmk_ctx* c, pmk_device_error* err) {
  pmk_status s = need_device(c);
  if (s != PMK_OK) return s;
  uint32_t w[6];
  HIPCHK(c, hipMemcpy(w, c->ws + c->w_ctrl + CTRL_ERR * 4, sizeof w, hipMemcpyDeviceToHost));
  if (err) {
    err->code = (int32_t)w[0];
    err->cu = (int32_t)w[1];
    err->task = (int32_t)w[2];
    err->counter = (int32_t)w[3];
    err->expected = w[4];
    err->seen = w[5];
  }
  return (pmk_status)w[0];
}

pmk_status pmk_set_trace(pmk_ctx* c, int32_t on) {
  if (!c) return PMK_ERR_INVALID_ARG;
  if (on && c->sc.trace_steps <= 0) return fail(c, PMK_ERR_INVALID_ARG, "the schedule has no trace buffer (trace_steps = 0)");
  if (on && c->bound) {
    HIPCHK(c, hipSetDevice(c->device));
    HIPCHK(c, hipMemset(c->ws + c->w_trace, 0, (size_t)c->sc.trace_steps * c->sched.tasks.size() * 64));
  }
  c->trace_on = on ? 1 : 0;
  return PMK_OK;
}

static pmk_status read_trace(pmk_ctx* c, std::vector<unsigned long long>& t) {
  pmk_status s = need_device(c);
  if (s != PMK_OK) return s;
  if (c->sc.trace_steps <= 0) return fail(c, PMK_ERR_INVALID_ARG, "no trace buffer");
  HIPCHK(c, hipDeviceSynchronize());
  t.resize((size_t)c->sc.trace_steps * c->sched.tasks.size() * 8);
  HIPCHK(c, hipMemcpy(t.data(), c->ws + c->w_trace, t.size() * 8, hipMemcpyDeviceToHost));
  return PMK_OK;
}

// Replace the context's schedule by `s`: validate, check it fits the workspace capacity and LDS,
// re-derive the tables and the LDS layout, upload the tables, and discard the synchronisation state
// of the previous schedule (flags, counters and step tags cleared, epoch restarted) while keeping the
// position `pos` and next input token `token`.  Synchronous on `st`.
static pmk_status install_schedule(pmk_ctx* c, Schedule&& s, int32_t pos, int32_t token, hipStream_t st) {
  const std::string e = validate_schedule(s);
  if (!e.empty()) return fail(c, PMK_ERR_SCHEDULE_INVALID, e);
  if (s.counters.size() != c->sched.counters.size() || s.n_flags > c->cap_flags ||
      (int64_t)s.tasks.size() > c->cap_tasks || s.attn_splits > c->cap_splits)
    return fail(c, PMK_ERR_SCHEDULE_INVALID, "tune: the schedule exceeds the workspace capacity fixed at creation");
  const pmk_sizes old_sizes = c->sizes;
  Schedule prev = std::move(c->sched);
  c->sched = std::move(s);
  compute_layout(c);
  if (c->sizes.workspace_bytes != old_sizes.workspace_bytes || c->lds_bytes > (size_t)kLdsBytes || c->lds_bytes_pk > (size_t)kLdsBytes) {
    c->sched = std::move(prev);
    compute_layout(c);
    return fail(c, PMK_ERR_SCHEDULE_INVALID, "tune: the schedule does not fit the bound buffers or LDS");
  }
  c->tabs = flatten(c->sched);
  c->hash = schedule_hash(c->sched);
  compute_phases(c);
  fill_params(c);
  HIPCHK(c, hipStreamSynchronize(st));
  HIPCHK(c, hipMemcpy(c->ws + c->w_tasks, c->tabs.tasks.data(), c->tabs.tasks.size() * sizeof(pmk_task), hipMemcpyHostToDevice));
  HIPCHK(c, hipMemcpy(c->ws + c->w_qoff, c->tabs.qoff.data(), c->tabs.qoff.size() * 4, hipMemcpyHostToDevice));
  HIPCHK(c, hipMemcpy(c->ws + c->w_qtasks, c->tabs.qtasks.data(), c->tabs.qtasks.size() * 4, hipMemcpyHostToDevice));
  HIPCHK(c, hipMemcpy(c->ws + c->w_cprod, c->tabs.ctr_producers.data(), c->tabs.ctr_producers.size() * 4, hipMemcpyHostToDevice));
  HIPCHK(c, hipMemcpy(c->ws + c->w_cflag, c->tabs.ctr_flag_base.data(), c->tabs.ctr_flag_base.size() * 4, hipMemcpyHostToDevice));
  if (c->graph_exec) { (void)hipGraphExecDestroy(c->graph_exec); c->graph_exec = nullptr; }
  if (c->graph) { (void)hipGraphDestroy(c->graph); c->graph = nullptr; }
  HIPCHK(c, launch_reset(c->kp, c->sched.n_flags, (int)c->sched.counters.size(), pos, token, nullptr, st));
  HIPCHK(c, hipStreamSynchronize(st));
  return PMK_OK;
}

namespace {

// One measured configuration of the tuning search.
struct TuneRun {
  double us = 0;                         // µs per step of the timed steps
  std::vector<unsigned long long> keys;  // per step: orderable max logit << 32 | ~argmax
};

float key_value(unsigned long long k) {
  const uint32_t ov = (uint32_t)(k >> 32);
  const uint32_t u = (ov & 0x80000000u) ? (ov & 0x7fffffffu) : ~ov;
  float f;
  std::memcpy(&f, &u, 4);
  return f;
}

}  // namespace

// `steps` megakernel steps from (pos, token), after an untimed pass of the same steps from the same
// state; timed with HIP events on `st`; the steps' argmax keys are read back for the correctness
// gate.  The state is back at (pos, token) afterwards.
static pmk_status tune_timed_run(pmk_ctx* c, int steps, int32_t pos, int32_t token, hipStream_t st, TuneRun* r) {
  hipEvent_t e0 = nullptr, e1 = nullptr;
  HIPCHK(c, hipEventCreate(&e0));
  HIPCHK(c, hipEventCreate(&e1));
  pmk_status s = PMK_OK;
  for (int pass = 0; pass < 2 && s == PMK_OK; ++pass) {
    CallParams cp{};
    cp.out_tokens = reinterpret_cast<int32_t*>(c->ws + c->w_tune);
    cp.n_steps = steps;
    cp.eos = -1;
    if (pass == 1) HIPCHK(c, hipEventRecord(e0, st));
    s = begin_call(c, cp, st);
    if (s == PMK_OK) s = launch_persistent(c, st);
    if (s == PMK_OK && pass == 1) HIPCHK(c, hipEventRecord(e1, st));
    if (s == PMK_OK) HIPCHK(c, hipStreamSynchronize(st));
    if (s == PMK_OK && pass == 1) {
      float ms = 0;
      HIPCHK(c, hipEventElapsedTime(&ms, e0, e1));
      r->us = ms * 1e3 / steps;
      r->keys.resize(steps);
      HIPCHK(c, hipMemcpy(r->keys.data(), c->ws + c->w_keys, steps * 8, hipMemcpyDeviceToHost));
    }
    if (s == PMK_OK) HIPCHK(c, launch_reset(c->kp, c->sched.n_flags, (int)c->sched.counters.size(), pos, token, nullptr, st));
  }
  (void)hipEventDestroy(e0);
  (void)hipEventDestroy(e1);
  if (s != PMK_OK) return s;
  uint32_t err = 0;
  HIPCHK(c, hipMemcpy(&err, c->ws + c->w_ctrl + CTRL_ERR * 4, 4, hipMemcpyDeviceToHost));
  if (err) return fail(c, (pmk_status)err, "tune: a device error during a measured run");
  return PMK_OK;
}

// Per-queue streaming rate (bytes per tick, after the pre-wait prefetch) of a GEMV op, and each
// queue's XCD, from a traced run of the installed schedule.
static pmk_status tune_rates(pmk_ctx* c, int steps, int32_t pos, int32_t token, hipStream_t st,
                             std::vector<double> rate[8], std::vector<int>* xcd) {
  pmk_status s = pmk_set_trace(c, 1);
  if (s != PMK_OK) return s;
  CallParams cp{};
  cp.out_tokens = reinterpret_cast<int32_t*>(c->ws + c->w_tune);
  cp.n_steps = steps;
  cp.eos = -1;
  cp.trace = 1;
  s = begin_call(c, cp, st);
  if (s == PMK_OK) s = launch_persistent(c, st);
  if (s != PMK_OK) return s;
  std::vector<unsigned long long> t;
  s = read_trace(c, t);
  c->trace_on = 0;
  if (s != PMK_OK) return s;
  HIPCHK(c, launch_reset(c->kp, c->sched.n_flags, (int)c->sched.counters.size(), pos, token, nullptr, st));
  HIPCHK(c, hipStreamSynchronize(st));
  const size_t NT = c->sched.tasks.size();
  const int NQ = c->sched.n_queues;
  std::vector<int> queue_of(NT, 0);
  for (int q = 0; q < NQ; ++q)
    for (int32_t ti : c->sched.queues[q]) queue_of[ti] = q;
  xcd->assign(NQ, -1);
  std::vector<double> bytes(8 * (size_t)NQ, 0.0), ticks(8 * (size_t)NQ, 0.0);
  const ModelDims& m = c->m;
  const double es = weight_bits(m.wdt) / 8.0;
  for (int sp = 1; sp < steps; ++sp)  // the first step also pays the launch
    for (size_t i = 0; i < NT; ++i) {
      const pmk_task& k = c->sched.tasks[i];
      const unsigned long long* r = &t[((size_t)sp * NT + i) * 8];
      if (r[2]) (*xcd)[queue_of[i]] = (int)(r[3] >> 32);
      if (k.op == PMK_OP_ATTN || k.op == PMK_OP_TOKEN || k.op == PMK_OP_COMBINE) continue;
      if (!r[4] || !r[5] || r[5] <= r[4]) continue;
      const double K = k.op == PMK_OP_DOWN ? m.F : k.op == PMK_OP_OPROJ ? m.qdim() : m.H;
      const size_t at = (size_t)k.op * NQ + queue_of[i];
      bytes[at] += std::max(0.0, (k.a1 - k.a0) * K * es - (double)kPrefetchBytes);
      ticks[at] += (double)(r[5] - r[4]);
    }
  for (int op = 0; op < 8; ++op) {
    rate[op].assign(NQ, 0.0);
    for (int q = 0; q < NQ; ++q)
      if (ticks[(size_t)op * NQ + q] > 0) rate[op][q] = bytes[(size_t)op * NQ + q] / ticks[(size_t)op * NQ + q];
  }
  return PMK_OK;
}

// Row weights for op from measured rates: per queue, or the mean of each queue's XCD; moved from
// even toward proportional by `damp`.  Empty when some queue has no rate.
static std::vector<double> tune_weights(const std::vector<double>& rate, const std::vector<int>& xcd, bool by_xcd,
                                        double damp) {
  const int NQ = (int)rate.size();
  std::vector<double> r = rate;
  for (int q = 0; q < NQ; ++q)
    if (!(rate[q] > 0)) return {};
  if (by_xcd) {
    std::map<int, std::pair<double, int>> acc;
    for (int q = 0; q < NQ; ++q) { acc[xcd[q]].first += rate[q]; acc[xcd[q]].second += 1; }
    for (int q = 0; q < NQ; ++q) r[q] = acc[xcd[q]].first / acc[xcd[q]].second;
  }
  double mean = 0;
  for (double x : r) mean += x;
  mean /= NQ;
  std::vector<double> w(NQ);
  for (int q = 0; q < NQ; ++q) w[q] = std::min(std::max(1.0 + damp * (r[q] / mean - 1.0), 0.5), 2.0);
  return w;
}

pmk_status pmk_tune(pmk_ctx* c, int32_t steps, pmk_tune_result* res, void* stream) {
  pmk_status s = need_device(c);
  if (s != PMK_OK) return s;
  if (res) std::memset(res, 0, sizeof *res);
  if (!c->weights || !c->kv_ready) return fail(c, PMK_ERR_NOT_BOUND, "weights and KV state must be loaded first");
  s = sync_position(c);
  if (s != PMK_OK) return s;
  if (steps <= 0) steps = 32;
  steps = std::max(4, std::min(steps, kMaxTuneSteps));
  if ((int64_t)c->pos_host + steps > c->m.max_seq) return fail(c, PMK_ERR_CAPACITY, "position + steps exceeds max_seq");
  hipStream_t st = (hipStream_t)stream;
  HIPCHK(c, hipSetDevice(c->device));
  HIPCHK(c, hipStreamSynchronize(st));
  const int32_t pos0 = c->pos_host;
  uint32_t tok = 0;
  HIPCHK(c, hipMemcpy(&tok, c->ws + c->w_ctrl + CTRL_TOKEN * 4, 4, hipMemcpyDeviceToHost));
  const int32_t token0 = (int32_t)tok;
  const int NQ = c->sched.n_queues;
  // the starting point: the schedule in force, from a clean state
  pmk_schedule_config best_sc = c->sc;
  RowWeights best_rw = c->rw;
  {
    Schedule cur;
    std::string e = build_schedule(c->m, best_sc, NQ, &cur, &best_rw);
    if (!e.empty()) return fail(c, PMK_ERR_SCHEDULE_INVALID, e);
    s = install_schedule(c, std::move(cur), pos0, token0, st);
    if (s != PMK_OK) return s;
  }
  TuneRun ref;
  s = tune_timed_run(c, steps, pos0, token0, st, &ref);
  if (s != PMK_OK) return s;
  double best_us = ref.us;
  if (res) res->us_before = ref.us;
  std::string desc;
  int tried = 0, kept = 0, gated = 0, invalid = 0;
  // install and time a candidate; keep it if it passes the gate and is faster by more than 0.2%
  auto attempt = [&](const pmk_schedule_config& sc, const RowWeights& rw, const std::string& what) -> pmk_status {
    Schedule ns;
    ++tried;
    if (!build_schedule(c->m, sc, NQ, &ns, &rw).empty() || !validate_schedule(ns).empty()) { ++invalid; return PMK_OK; }
    if (install_schedule(c, std::move(ns), pos0, token0, st) != PMK_OK) { ++invalid; c->err.clear(); }
    else {
      TuneRun r;
      pmk_status s2 = tune_timed_run(c, steps, pos0, token0, st, &r);
      if (s2 != PMK_OK) return s2;
      // correctness gate against the starting schedule's run from the same state: the same greedy
      // token at every step, and the same largest logit within 1e-3 (a row split changes only the
      // grouping of a row's partial sums).  The integer weight formats round every GEMV operand to
      // binary16, where a regrouped fp32 sum moves some elements by a whole binary16 step: 2e-2 there.
      const float gate_tol = weight_is_int(c->m.wdt) ? 2e-2f : 1e-3f;
      bool same = true;
      for (int i = 0; i < steps; ++i) {
        const float a = key_value(ref.keys[i]), b = key_value(r.keys[i]);
        same = same && (uint32_t)ref.keys[i] == (uint32_t)r.keys[i] &&
               std::fabs(a - b) <= gate_tol * std::max(1.0f, std::fabs(a));
      }
      if (!same) ++gated;
      if (same && r.us < best_us * (1.0 - 0.002)) {
        best_us = r.us;
        best_sc = sc;
        best_rw = rw;
        ++kept;
        desc += (desc.empty() ? "" : "; ") + what;
        return PMK_OK;
      }
    }
    // revert to the best so far
    Schedule bs;
    std::string e = build_schedule(c->m, best_sc, NQ, &bs, &best_rw);
    if (!e.empty()) return fail(c, PMK_ERR_SCHEDULE_INVALID, e);
    return install_schedule(c, std::move(bs), pos0, token0, st);
  };
  // 1. speed-weighted row shares of gate/up, then of the down projection, from measured rates
  if (c->sc.trace_steps >= 2) {
    std::vector<double> rate[8];
    std::vector<int> xcd;
    s = tune_rates(c, std::min(steps, c->sc.trace_steps), pos0, token0, st, rate, &xcd);
    if (s != PMK_OK) return s;
    for (int op : {PMK_OP_GATEUP, PMK_OP_DOWN})
      for (bool by_xcd : {true, false})
        for (double damp : {1.0, 0.5}) {
          std::vector<double> w = tune_weights(rate[op], xcd, by_xcd, damp);
          if (w.empty()) continue;
          RowWeights rw = best_rw;
          rw.w[op] = w;
          char what[96];
          std::snprintf(what, sizeof what, "%s rows %s x%.1f", op == PMK_OP_GATEUP ? "gate/up" : "down",
                        by_xcd ? "per XCD" : "per queue", damp);
          s = attempt(best_sc, rw, what);
          if (s != PMK_OK) return s;
        }
  }
  // 2. O-projection rows on the combine queues, combines per kv head, attention splits
  for (int share : {1, 2, 3}) {
    if (share == best_sc.combine_o_share) continue;
    pmk_schedule_config sc = best_sc;
    sc.combine_o_share = share;
    s = attempt(sc, best_rw, std::string("combine_o_share ") + std::to_string(share));
    if (s != PMK_OK) return s;
  }
  {
    pmk_schedule_config sc = best_sc;
    sc.combine_o_copy = c->sched.o_copy ? 1 : 2;
    s = attempt(sc, best_rw, std::string("combine_o_copy ") + std::to_string(sc.combine_o_copy));
    if (s != PMK_OK) return s;
  }
  for (int cp = 1; cp <= c->m.grp(); ++cp) {
    if (c->m.grp() % cp || cp == c->sched.combine_parts) continue;
    pmk_schedule_config sc = best_sc;
    sc.combine_parts = cp;
    s = attempt(sc, best_rw, std::string("combine_parts ") + std::to_string(cp));
    if (s != PMK_OK) return s;
  }
  for (int frac : {3, 2}) {  // 3/4 and 1/2 of the capacity splits
    const int S = c->cap_splits * frac / 4;
    if (S < 1 || S == c->sched.attn_splits) continue;
    pmk_schedule_config sc = best_sc;
    sc.attn_splits = S;
    s = attempt(sc, best_rw, std::string("attn_splits ") + std::to_string(S));
    if (s != PMK_OK) return s;
  }
  c->sc = best_sc;
  c->rw = best_rw;
  if (res) {
    res->tried = tried;
    res->kept = kept;
    res->gate_rejected = gated;
    res->invalid = invalid;
    res->us_after = best_us;
    res->chosen = best_sc;
    res->chosen.combine_parts = c->sched.combine_parts;
    res->chosen.attn_splits = c->sched.attn_splits;
    std::snprintf(res->desc, sizeof res->desc, "%s", desc.empty() ? "default" : desc.c_str());
  }
  c->pos_host = pos0;
  c->pos_exact = true;
  return PMK_OK;
}

pmk_status pmk_trace_stats(pmk_ctx* c, double* wait_share, double* step_us) {
  std::vector<unsigned long long> t;
  pmk_status s = read_trace(c, t);
  if (s != PMK_OK) return s;
  const size_t NT = c->sched.tasks.size();
  double wait = 0, wall = 0, steps_us = 0;
  int nsteps = 0;
  for (int st = 0; st < c->sc.trace_steps; ++st) {
    unsigned long long lo = ~0ull, hi = 0;
    bool any = false;
    for (size_t i = 0; i < NT; ++i) {
      const unsigned long long* r = &t[((size_t)st * NT + i) * 8];
      if (!r[0] || !r[2] || r[2] < r[0]) continue;
      any = true;
      const unsigned long long t1 = (r[1] >= r[0] && r[1] <= r[2]) ? r[1] : r[0];
      wait += (double)(t1 - r[0]);
      wall += (double)(r[2] - r[0]);
      lo = std::min(lo, r[0]);
      hi = std::max(hi, r[2]);
    }
    if (any) { steps_us += (hi - lo) * 0.01; ++nsteps; }
  }
  if (wait_share) *wait_share = wall > 0 ? wait / wall : 0.0;
  if (step_us) *step_us = nsteps ? steps_us / nsteps : 0.0;
  return PMK_OK;
}

pmk_status pmk_trace_export(pmk_ctx* c, const char* path) {
  if (!path) return PMK_ERR_INVALID_ARG;
  std::vector<unsigned long long> t;
  pmk_status s = read_trace(c, t);
  if (s != PMK_OK) return s;
  FILE* f = std::fopen(path, "w");
  if (!f) return fail(c, PMK_ERR_INVALID_ARG, std::string("cannot open ") + path);
  static const char* names[] = {"?", "qkv", "attn", "oproj", "gateup", "down", "lmhead", "token", "combine"};
  const size_t NT = c->sched.tasks.size();
  unsigned long long t0 = ~0ull;
  for (size_t i = 0; i < t.size(); i += 8)
    if (t[i]) t0 = std::min(t0, t[i]);
  std::fprintf(f, "{\"traceEvents\":[\n");
  bool first = true;
  for (int st = 0; st < c->sc.trace_steps; ++st)
    for (size_t i = 0; i < NT; ++i) {
      const unsigned long long* r = &t[((size_t)st * NT + i) * 8];
      if (!r[0] || !r[2]) continue;
      const pmk_task& k = c->sched.tasks[i];
      const unsigned long long t1 = (r[1] >= r[0] && r[1] <= r[2]) ? r[1] : r[0];
      std::fprintf(f, "%s{\"name\":\"wait\",\"ph\":\"X\",\"pid\":%d,\"tid\":%llu,\"ts\":%.2f,\"dur\":%.2f}", first ? "" : ",\n",
                   st, r[3] & 0xffffffffull, (r[0] - t0) * 0.01, (t1 - r[0]) * 0.01);
      std::fprintf(f, ",\n{\"name\":\"%s L%d\",\"ph\":\"X\",\"pid\":%d,\"tid\":%llu,\"ts\":%.2f,\"dur\":%.2f,\"args\":{\"xcd\":%llu,\"m4\":%.2f,\"m5\":%.2f,\"m6\":%.2f,\"m7\":%.2f}}",
                   names[k.op >= 1 && k.op <= 8 ? k.op : 0], k.layer, st, r[3] & 0xffffffffull, (t1 - t0) * 0.01, (r[2] - t1) * 0.01, r[3] >> 32,
                   r[4] >= t1 ? (r[4] - t1) * 0.01 : -1.0, r[5] >= t1 ? (r[5] - t1) * 0.01 : -1.0,
                   r[6] >= t1 ? (r[6] - t1) * 0.01 : -1.0, r[7] >= t1 ? (r[7] - t1) * 0.01 : -1.0);
      first = false;
    }
  std::fprintf(f, "\n]}\n");
  std::fclose(f);
  return PMK_OK;
}

pmk_status pmk_schedule_get_info(const pmk_ctx* c, pmk_schedule_info* info) {
  if (!c || !info) return PMK_ERR_INVALID_ARG;
  info->n_tasks = (int32_t)c->sched.tasks.size();
  info->n_counters = (int32_t)c->sched.counters.size();
  info->n_cus = c->sched.n_queues;
  info->attn_splits = c->sched.attn_splits;
  int mx = 0;
  for (auto& q : c->sched.queues) mx = std::max(mx, (int)q.size());
  info->max_tasks_per_cu = mx;
  info->sync_mode = c->sched.sync_mode;
  info->hash = c->hash;
  return PMK_OK;
}

// ---- schedule IR API ----
pmk_status pmk_schedule_build_weighted(const pmk_model_config* cfg, const pmk_schedule_config* sched, int32_t n_cus,
                                       const float* weights, pmk_schedule** out) {
  g_err.clear();
  if (!cfg || !out || n_cus <= 0) return fail(nullptr, PMK_ERR_INVALID_ARG, "bad arguments");
  *out = nullptr;
  const std::string why = contract_check(*cfg);
  if (!why.empty()) return fail(nullptr, PMK_ERR_UNSUPPORTED, why);
  RowWeights rw;
  if (weights) {
    for (int op : {PMK_OP_QKV, PMK_OP_OPROJ, PMK_OP_GATEUP, PMK_OP_DOWN, PMK_OP_LMHEAD}) {
      rw.w[op].assign(weights + (size_t)op * n_cus, weights + (size_t)(op + 1) * n_cus);
      for (double x : rw.w[op])
        if (!(x > 0)) return fail(nullptr, PMK_ERR_INVALID_ARG, "row weights must be positive");
    }
  }
  pmk_schedule* s = new pmk_schedule();
  const pmk_schedule_config sc = defaults(sched);
  const std::string e = build_schedule(dims_of(*cfg), sc, n_cus, &s->s, weights ? &rw : nullptr);
  if (!e.empty()) { delete s; return fail(nullptr, PMK_ERR_SCHEDULE_INVALID, e); }
  *out = s;
  return PMK_OK;
}

pmk_status pmk_schedule_build(const pmk_model_config* cfg, const pmk_schedule_config* sched, int32_t n_cus, pmk_schedule** out) {
  return pmk_schedule_build_weighted(cfg, sched, n_cus, nullptr, out);
}

void pmk_schedule_free(pmk_schedule* s) { delete s; }
int32_t pmk_schedule_num_tasks(const pmk_schedule* s) { return s ? (int32_t)s->s.tasks.size() : 0; }
int32_t pmk_schedule_num_counters(const pmk_schedule* s) { return s ? (int32_t)s->s.counters.size() : 0; }
int32_t pmk_schedule_num_queues(const pmk_schedule* s) { return s ? s->s.n_queues : 0; }

pmk_status pmk_schedule_get_task(const pmk_schedule* s, int32_t i, pmk_task* t) {
  if (!s || !t || i < 0 || i >= (int32_t)s->s.tasks.size()) return PMK_ERR_INVALID_ARG;
  *t = s->s.tasks[i];
  return PMK_OK;
}

pmk_status pmk_schedule_set_task(pmk_schedule* s, int32_t i, const pmk_task* t) {
  if (!s || !t || i < 0 || i >= (int32_t)s->s.tasks.size()) return PMK_ERR_INVALID_ARG;
  s->s.tasks[i] = *t;
  return PMK_OK;
}

const int32_t* pmk_schedule_queue(const pmk_schedule* s, int32_t q, int32_t* len) {
  if (!s || q < 0 || q >= s->s.n_queues) { if (len) *len = 0; return nullptr; }
  if (len) *len = (int32_t)s->s.queues[q].size();
  return s->s.queues[q].data();
}

pmk_status pmk_schedule_set_queue(pmk_schedule* s, int32_t q, const int32_t* tasks, int32_t len) {
  if (!s || q < 0 || q >= s->s.n_queues || len < 0 || (len && !tasks)) return PMK_ERR_INVALID_ARG;
  s->s.queues[q].assign(tasks, tasks + len);
  return PMK_OK;
}

int32_t pmk_schedule_counter_producers(const pmk_schedule* s, int32_t c) {
  if (!s || c < 0 || c >= (int32_t)s->s.counters.size()) return -1;
  return s->s.counters[c].producers;
}

pmk_status pmk_schedule_set_counter_producers(pmk_schedule* s, int32_t c, int32_t producers) {
  if (!s || c < 0 || c >= (int32_t)s->s.counters.size()) return PMK_ERR_INVALID_ARG;
  s->s.counters[c].producers = producers;
  return PMK_OK;
}

pmk_status pmk_schedule_validate(const pmk_schedule* s, char* report, size_t cap) {
  if (!s) return PMK_ERR_INVALID_ARG;
  const std::string e = validate_schedule(s->s);
  if (report && cap) {
    std::strncpy(report, e.c_str(), cap - 1);
    report[cap - 1] = 0;
  }
  return e.empty() ? PMK_OK : PMK_ERR_SCHEDULE_INVALID;
}

pmk_status pmk_schedule_simulate(const pmk_schedule* s, int32_t steps, uint64_t seed, char* report, size_t cap) {
  if (!s || steps <= 0) return PMK_ERR_INVALID_ARG;
  std::string r;
  const pmk_status st = simulate_schedule(s->s, steps, seed, &r);
  if (report && cap) {
    std::strncpy(report, r.c_str(), cap - 1);
    report[cap - 1] = 0;
  }
  return st;
}

uint64_t pmk_schedule_hash(const pmk_schedule* s) { return s ? schedule_hash(s->s) : 0; }

}  // extern "C"
