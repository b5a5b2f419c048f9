// Parameters shared by the host runtime and the gfx950 kernels.
#pragma once

#include <cstdint>

#include "../../include/pmk.h"
#include "pmk_limits.h"

namespace pmk {

constexpr int kThreads = 512;   // one workgroup per CU: 8 wave64s (2 per SIMD)
constexpr int kWaves = kThreads / 64;
constexpr int kLdsBytes = 160 * 1024;  // LDS of one gfx950 CU

// The static workspace (pmk_bind_static_workspace): bytes per device, and devices supported.
constexpr size_t kStaticWorkspaceBytes = (size_t)32 << 20;
constexpr int kMaxDevices = 64;

// control words (workspace, uint32) -------------------------------------------------------------
enum Ctrl : int {
  CTRL_EPOCH = 0,    // global decode steps since the last reset (counters / flags are relative to it)
  CTRL_POS = 1,      // next position to write
  CTRL_TOKEN = 2,    // next input token
  CTRL_STEP = 3,     // per-op modes: step index within the current call
  CTRL_STOPPED = 4,  // per-op modes: eos seen in this call
  CTRL_ABORT = 5,    // watchdog: a wait gave up; every wait exits
  CTRL_ERR = 8,      // pmk_device_error: code, cu, task, counter, expected, seen (6 words)
  CTRL_SAVED = 16,   // next input token saved while the schedule is tuned
  CTRL_WORDS = 64
};

// per-call parameters kept in device memory so a captured graph can read them
struct CallParams {
  int32_t* out_tokens;
  float* out_logits;
  int32_t* n_done;
  const int32_t* forced;  // teacher-forced input tokens (prefill), or null
  int32_t n_steps;
  int32_t eos;
  int32_t trace;
  int32_t calib;  // FP8 KV: record max |k|, |v| per (layer, kv head) while the steps run (scale calibration)
};

// Batched prefill: chunk buffers in the workspace.
struct PrefillArgs {
  const int32_t* tokens;  // prompt tokens (device)
  int32_t n;              // positions 0..n-1 go through the batched path
  int32_t chunk;          // tokens per chunk (a multiple of 128)
  float* x;               // [chunk][H] residual stream
  float* xm;              // [chunk][H] residual after attention
  float* x2;              // [chunk][H] second K-half of the down projection (x = x + x2 at the next RMSNorm)
  float* xm2;             // [chunk][H] second K-half of the O projection (xm = xm + xm2 at the RMSNorm)
  float* q;               // [chunk][qdim] queries after RoPE
  uint16_t* bn;           // [terms][chunk][H] normalised activations (two 16-bit terms, or the
                          // one binary16 value of the integer formats)
  uint16_t* bo;           // [terms][chunk][qdim] attention output
  uint16_t* bh;           // [terms][chunk][F] SwiGLU output
  uint32_t* bar;          // grid barrier: one flag word per workgroup (zero at launch)
  int32_t calib;          // FP8 KV scale calibration: record max |k|, |v| of every appended row
  int32_t ksplit;         // K-halves of the O and down projections: 0 automatic, 1 never, 2 always
};

struct KParams {
  // model
  int L, H, nq, nkv, hd, F, V, grp, qkv_rows, qdim, max_seq, S;
  int seqcap;             // KV cache positions per head: max_seq rounded up to 32
  int wdt, kvdt;
  float eps;
  float attn_scale;  // 1/sqrt(hd)
  // arena
  const uint16_t* embed;  // [V][H] 16-bit
  const float* gains;     // [L][2][H]
  const float* final_gain;
  const uint8_t* wbase;   // layer l block at wbase + l*layer_bytes
  int64_t layer_bytes;
  int64_t off_qkv, off_o, off_gu, off_d;
  const uint8_t* lm;      // [V][H]
  const void* scales;     // fp8 / int8 / int4: per layer [q k v o g u d] scale arrays (fp8: fp32 per
                          // 128x128 block; int: bf16 per row and 128-column group)
  int64_t sc_layer;       // scale elements per layer
  int64_t sc_off[7];      // offsets (scale elements) of the 7 arrays inside a layer
  const void* sc_lm;      // the LM head's scales
  const float2* rope;     // [max_seq][hd/2] (cos, sin)
  // kv cache: K [L][nkv][seqcap][hd], V [L][nkv][seqcap / 32][hd][32]
  uint8_t* kc;
  uint8_t* vc;
  // workspace
  uint32_t* ctrl;
  CallParams* call;
  uint32_t* flags;
  uint32_t* counters;
  unsigned long long* keys;  // [max_seq + 1]
  float* kv_scale;        // [L][nkv][2]
  uint32_t* kv_amax;      // [L][nkv][2] calibration: fp32 bits of max |k|, |v| (non-negative: ordered as integers)
  unsigned long long* x;   // [L+1][H] residual stream entering each layer (and the final norm), tagged
  unsigned long long* xm;  // [L][H] residual after the attention block, tagged
  unsigned long long* q;      // [L][qdim] roped queries, tagged
  unsigned long long* kvcur;  // [L][nkv][2][hd] the step's K row and V column as 16-bit operand bits, tagged
  float* part;            // [L][nkv][S][grp][hd+4]: m, l, 2 pad, acc[hd]
  unsigned long long* o;  // [L][qdim] attention output, each value tagged: (step + 1) << 32 | fp32 bits
  float* h;               // [L][F]
  unsigned long long* trace;  // [trace_steps][n_tasks][4]
  // schedule tables
  const pmk_task* tasks;
  const int32_t* qoff;
  const int32_t* qtasks;
  const int32_t* ctr_prod;
  const int32_t* ctr_flag;
  int n_queues, n_tasks, sync_mode, prefetch, trace_steps;
  int64_t spin_limit;
  int xs_floats;          // LDS floats reserved for staged activation vectors (or attention scratch)
  int epi_off;            // LDS float offset of staged epilogue inputs (RoPE row, residual rows)
  int yp_off;             // LDS float offset of per-slice GEMV partial sums [8 * rows]
  int y_off;              // LDS float offset of GEMV row results [rows]
  int xh_off;             // LDS float offset of the binary16 normalised vector (integer weight formats)
  int gs_off;             // LDS float offset of the staged RMSNorm gains (integer weight formats)
  int o_epi_off, o_yp_off, o_y_off;  // the same three areas for OPROJ tasks, packed below pf_off
  int attn_g2_off;        // LDS float offset of the attention's per-wave second-group buffers (-1: none)
  int pf_off;             // LDS float offset of the O-projection weight tile (copied before the task's wait)
  int pf_units;           // 1 KiB units in that area (0: the copy is off)
  int32_t o_copy;  // a COMBINE copies its queue's next O-projection tile to LDS before its wait
};

}  // namespace pmk
