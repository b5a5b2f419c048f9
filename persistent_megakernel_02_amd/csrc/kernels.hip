// gfx950 (CDNA4) kernels of the persistent batch-1 decode path.
//
// One workgroup of 512 threads (8 wave64s) per CU executes that CU's static task queue for n
// decode steps (the persistent kernel), or one task per workgroup (the per-op kernels that the
// hipGraph baseline captures).  Both run the same task functions below.
//
// Pages: "AutoMegaKernel" explainer, Method: Layer 0 (one cooperative block per compute unit
// running wait -> dispatch -> signal over a local queue with monotonic counters) and Layer 1
// (GEMV, attention and RMSNorm instructions).  "Kog AI MI300X monokernel tutorial": batch-1
// projections are GEMV on the vector ALUs (not matrix cores), the decode loop with LM-head
// sampling and the EOS check stays inside one resident kernel, and sync moved from atomic
// arrival counters to polling of the producers' own words.  "Netra Kernel" summary, details:
// FP8 E4M3 block-scale weights and GQA attention over an FP8 KV cache.
//
// Memory ordering.  Data exchanged between CUs (activations, q, attention partials, the current
// K/V row, flags) is written with agent-scope coherent stores (sc1) and read with agent-scope
// coherent loads, so no L2 write-back or invalidate is needed.  A producer drains its stores
// (s_waitcnt vmcnt(0) in every wave, then a workgroup barrier) before one thread publishes the
// flag or counter; a consumer polls that word and only then issues its coherent data loads.
// Weights and the KV rows of positions written before this launch are read with plain
// non-temporal loads (kernel boundaries order them).  KV rows of positions written during this
// launch are read with coherent loads by the splits that hold them (a V-cache line holds 32
// positions, so it is read before all of its slots are written), and the position written in the
// current step is never read from the cache but from its step-tagged copy.
#include <hip/hip_runtime.h>

#include <cstdint>
#include <mutex>
#include <type_traits>

#include "pmk_device.h"

namespace pmk {

typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));
typedef float f32x2 __attribute__((ext_vector_type(2)));

enum { WF16 = 0, WBF16 = 1, WFP8 = 2, WI8 = 3, WI4 = 4 };

// ------------------------------------------------------------------------------------------------
// coherent (agent scope) accesses
// ------------------------------------------------------------------------------------------------
__device__ __forceinline__ float ldc(const float* p) {
  return __hip_atomic_load(const_cast<float*>(p), __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ uint32_t ldc(const uint32_t* p) {
  return __hip_atomic_load(const_cast<uint32_t*>(p), __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ unsigned long long ldc(const unsigned long long* p) {
  return __hip_atomic_load(const_cast<unsigned long long*>(p), __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ void stc(float* p, float v) {
  __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ void stc(uint32_t* p, uint32_t v) {
  __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ void stc(uint16_t* p, uint16_t v) {
  __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ void stc(uint8_t* p, uint8_t v) {
  __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ void stc(unsigned long long* p, unsigned long long v) {
  __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
// A value that carries its own readiness: the step tag (global step + 1) in the high word and the
// fp32 bits in the low word, written with one 8-byte atomic store (single-copy atomic), so a
// reader that sees the tag of its step sees that step's value.
__device__ __forceinline__ unsigned long long tagged(float v, int e) {
  return ((unsigned long long)(uint32_t)(e + 1) << 32) | __float_as_uint(v);
}
// wait until every memory access this wave issued has completed
__device__ __forceinline__ void drain() {
  __atomic_signal_fence(__ATOMIC_SEQ_CST);
  __builtin_amdgcn_s_waitcnt(0);
  __atomic_signal_fence(__ATOMIC_SEQ_CST);
}

// Agent-coherent 16-byte load through a buffer resource (cache policy sc1).  Reads at or past
// `bytes` return zero (hardware range check), which also zero-fills padding.
__device__ __forceinline__ __amdgpu_buffer_rsrc_t coherent_rsrc(const void* base, uint32_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, (int)bytes, 0x00020000);
}
__device__ __forceinline__ u32x4 ldc16(__amdgpu_buffer_rsrc_t r, uint32_t byte_off) {
  return __builtin_amdgcn_raw_buffer_load_b128(r, byte_off, 0, 16);
}
__device__ __forceinline__ float4 as_f4(u32x4 v) {
  return make_float4(__uint_as_float(v.x), __uint_as_float(v.y), __uint_as_float(v.z), __uint_as_float(v.w));
}

// ------------------------------------------------------------------------------------------------
// reductions
// ------------------------------------------------------------------------------------------------
// Sum over the 64 lanes with DPP row operations; every lane receives the total.
__device__ __forceinline__ float wave_sum(float v) {
  int x = __float_as_int(v);
  v += __int_as_float(__builtin_amdgcn_update_dpp(0, x, 0xB1, 0xF, 0xF, false));  // quad_perm [1,0,3,2]
  x = __float_as_int(v);
  v += __int_as_float(__builtin_amdgcn_update_dpp(0, x, 0x4E, 0xF, 0xF, false));  // quad_perm [2,3,0,1]
  x = __float_as_int(v);
  v += __int_as_float(__builtin_amdgcn_update_dpp(0, x, 0x141, 0xF, 0xF, false));  // row_half_mirror
  x = __float_as_int(v);
  v += __int_as_float(__builtin_amdgcn_update_dpp(0, x, 0x140, 0xF, 0xF, false));  // row_mirror
  x = __float_as_int(v);
  v += __int_as_float(__builtin_amdgcn_update_dpp(0, x, 0x142, 0xA, 0xF, false));  // row_bcast15 -> rows 1,3
  x = __float_as_int(v);
  v += __int_as_float(__builtin_amdgcn_update_dpp(0, x, 0x143, 0xC, 0xF, false));  // row_bcast31 -> rows 2,3
  return __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), 63));
}

// One DPP max step: a lane's value against the lane the DPP control CTRL selects (rows ROWS).
template <int CTRL, int ROWS>
__device__ __forceinline__ float dpp_max(float a) {
  const int x = __float_as_int(a);
  return fmaxf(a, __int_as_float(__builtin_amdgcn_update_dpp(x, x, CTRL, ROWS, 0xF, false)));
}

// ------------------------------------------------------------------------------------------------
// storage formats
// ------------------------------------------------------------------------------------------------
template <int DT>
__device__ __forceinline__ float dec16(uint16_t b) {
  if (DT == WBF16) return __uint_as_float((uint32_t)b << 16);
  return (float)__builtin_bit_cast(_Float16, b);
}
template <int DT>
__device__ __forceinline__ uint16_t enc16(float v) {
  if (DT == WBF16) {
    uint32_t u = __float_as_uint(v);
    if ((u & 0x7fffffffu) > 0x7f800000u) return (uint16_t)((u >> 16) | 0x40);
    u += 0x7fffu + ((u >> 16) & 1u);
    return (uint16_t)(u >> 16);
  }
  return __builtin_bit_cast(uint16_t, (_Float16)v);  // round to nearest even
}
// OCP E4M3FN: nearest even, saturating to +-448
__device__ __forceinline__ uint8_t enc_e4m3(float v) {
  if (v != v) return 0x7f;
  const uint8_t sign = (__float_as_uint(v) >> 24) & 0x80;
  const float a = fabsf(v);
  if (a >= 448.f) return sign | 0x7e;
  if (a < 0.015625f) return sign | (uint8_t)rintf(a * 512.f);  // subnormal grid 2^-9
  int ex;
  const float m = frexpf(a, &ex);               // a = m * 2^ex, m in [0.5, 1)
  float q = rintf(ldexpf(m, 4));                 // significand in [8, 16]
  int e = ex - 1;
  if (q == 16.f) { q = 8.f; e += 1; }
  int code = ((e + 7) << 3) | ((int)q - 8);
  return sign | (uint8_t)(code > 0x7e ? 0x7e : code);
}
__device__ __forceinline__ float dec_e4m3(uint32_t word, int byte) {
  // hardware OCP E4M3 -> f32 (gfx950)
  const f32x2 lo = __builtin_amdgcn_cvt_pk_f32_fp8(word, false);
  const f32x2 hi = __builtin_amdgcn_cvt_pk_f32_fp8(word, true);
  return byte == 0 ? lo.x : byte == 1 ? lo.y : byte == 2 ? hi.x : hi.y;
}

// ------------------------------------------------------------------------------------------------
// synchronisation: waits (wave 0 polls, then a workgroup barrier) and signals
// ------------------------------------------------------------------------------------------------
__device__ __noinline__ void report_error(uint32_t* ctrl, uint32_t code, int cu, int task, int ctr, uint32_t expected,
                                          uint32_t seen) {
  if (atomicCAS(&ctrl[CTRL_ERR], 0u, code) == 0u) {
    stc(&ctrl[CTRL_ERR + 1], (uint32_t)cu);
    stc(&ctrl[CTRL_ERR + 2], (uint32_t)task);
    stc(&ctrl[CTRL_ERR + 3], (uint32_t)ctr);
    stc(&ctrl[CTRL_ERR + 4], expected);
    stc(&ctrl[CTRL_ERR + 5], seen);
  }
  stc(&ctrl[CTRL_ABORT], 1u);
}

// Executed by the 64 lanes of wave 0.  Returns when the dependency is met, the launch was
// aborted, or the spin limit ran out (which aborts the launch).
__device__ __noinline__ void wave_wait(uint32_t* ctrl, const uint32_t* word, int prod, int count, int lag, int e,
                                       int counters_mode, int64_t spin_limit, int cu, int task, int ctr) {
  const int lane = threadIdx.x & 63;
  int64_t spins = 0;
  // Every poll issues all of its loads (the watched words and the abort word) before it waits for
  // any of them, so one poll costs one memory round trip.
  if (counters_mode) {
    const int64_t need = (int64_t)(e - lag) * prod + count;
    if (need <= 0) return;
    while (true) {
      const uint32_t ab = ldc(&ctrl[CTRL_ABORT]);
      const uint32_t v = ldc(word);
      if ((int64_t)v >= need) return;
      if (ab) return;
      if (++spins > spin_limit) {
        if (lane == 0) report_error(ctrl, PMK_ERR_TIMEOUT, cu, task, ctr, (uint32_t)need, v);
        return;
      }
    }
  } else {
    const int target = e - lag + 1;
    if (target <= 0) return;
    constexpr int MW = 8;  // flag words per lane in one batch (512 producers per round trip)
    // the address is wave uniform: move it to scalar registers so the resource is too
    const uint64_t wa = (uint64_t)word;
    const uint64_t wu = (uint64_t)(uint32_t)__builtin_amdgcn_readfirstlane((int)(uint32_t)wa) |
                        ((uint64_t)(uint32_t)__builtin_amdgcn_readfirstlane((int)(uint32_t)(wa >> 32)) << 32);
    const int produ = __builtin_amdgcn_readfirstlane(prod);
    const __amdgpu_buffer_rsrc_t r = coherent_rsrc((const void*)wu, (uint32_t)produ * 4);  // words past prod read 0
    while (true) {
      const uint32_t ab = ldc(&ctrl[CTRL_ABORT]);
      int have = 0;
      for (int base = 0; base < prod; base += 64 * MW) {
        uint32_t v[MW];
#pragma unroll
        for (int k = 0; k < MW; ++k)
          v[k] = __builtin_amdgcn_raw_buffer_load_b32(r, (uint32_t)(base + k * 64 + lane) * 4, 0, 16);
#pragma unroll
        for (int k = 0; k < MW; ++k) have += __popcll(__ballot((int)v[k] >= target));
      }
      if (have >= count) return;
      if (ab) return;
      if (++spins > spin_limit) {
        if (lane == 0) report_error(ctrl, PMK_ERR_TIMEOUT, cu, task, ctr, (uint32_t)target, (uint32_t)have);
        return;
      }
    }
  }
}

__device__ __forceinline__ void block_wait(const KParams& P, int ctr, int count, int lag, int e, int cu, int task) {
  if (ctr >= 0 && threadIdx.x < 64) {
    const bool cm = P.sync_mode == PMK_SYNC_COUNTERS;
    const uint32_t* word = cm ? P.counters + ctr : P.flags + P.ctr_flag[ctr];
    wave_wait(P.ctrl, word, P.ctr_prod[ctr], count, lag, e, cm ? 1 : 0, P.spin_limit, cu, task, ctr);
  }
  __syncthreads();
}

// All waves drain their stores, then thread 0 publishes.
__device__ __forceinline__ void block_signal(const KParams& P, int ctr, int slot, int e) {
  drain();
  __syncthreads();
  if (threadIdx.x == 0 && ctr >= 0) {
    if (P.sync_mode == PMK_SYNC_COUNTERS)
      __hip_atomic_fetch_add(&P.counters[ctr], 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    else
      stc(&P.flags[P.ctr_flag[ctr] + slot], (uint32_t)(e + 1));
  }
}

// ------------------------------------------------------------------------------------------------
// GEMV: rows [r0, r1) of W (row-major [rows][K]) against the activation vector staged in LDS.
// Each wave owns a contiguous block of row groups (PAIR rows each).  A lane reads 16-byte
// chunks c = j*64 + lane of a row (j = slice), so one wave instruction streams 1 KiB.  Weight
// loads run through a ring of D registers per lane; the first D are issued BEFORE the task's
// dependency wait (weights do not depend on it), then each consumed slot is refilled with the
// chunk D units ahead.  Past the end the refill re-reads the tile's first chunk (a cache hit).
// ------------------------------------------------------------------------------------------------
template <int WDT>
struct WFmt {
  static constexpr int EPL = weight_epl(WDT);      // elements per 16-byte chunk
  static constexpr bool SCALED = WDT >= WFP8;      // a scale per 128-column group of a chunk's row
  static constexpr bool H16 = weight_is_int(WDT);  // the GEMV's activation vector is staged as binary16
  static constexpr int CPG = 128 / EPL;            // chunks per 128-column scale group
  static constexpr int EDT = WDT >= WFP8 ? WBF16 : WDT;  // format of the embedding (and gains)
  // scale element: fp32 per 128x128 block (fp8), bf16 bits per row and 128-column group (int)
  using ST = typename std::conditional<WDT == WFP8, float, uint16_t>::type;
  static __device__ __forceinline__ int64_t row_bytes(int K) { return (int64_t)(K / EPL) * 16; }
};

template <int WDT>
__device__ __forceinline__ float scale_value(typename WFmt<WDT>::ST s) {
  if constexpr (WDT == WFP8) return s;
  else return __uint_as_float((uint32_t)s << 16);
}

// The activation elements of chunk c (EPL of them) in the staged vector: fp32, or binary16 pairs
// packed two to a 32-bit word for the integer formats.
template <int WDT>
__device__ __forceinline__ const float* xchunk(const float* xs, int c) {
  return WFmt<WDT>::H16 ? xs + c * (WFmt<WDT>::EPL / 2) : xs + c * WFmt<WDT>::EPL;
}

typedef _Float16 h16x2 __attribute__((ext_vector_type(2)));
__device__ __forceinline__ h16x2 as_h2(uint32_t u) { return __builtin_bit_cast(h16x2, u); }

// Integer weight codes (stored offset binary: int8 q + 128 per byte; int4 q + 8 per nibble, the
// nibbles of each 32-bit word holding columns 0 2 4 6 1 3 5 7 from the low end) -> binary16 pairs
// of consecutive columns, exactly: a code u placed in the low mantissa bits of 1024.0 (0x6400)
// is the binary16 value 1024 + u, and one packed add (or fma, for a nibble sitting 4 bits up)
// removes 1024 and the offset.  Each pair then goes through one v_dot2_f32_f16 with the matching
// pair of binary16 activations: exact products, accumulated in fp32 (measured on gfx950: within 2
// fp32 ulps of the largest term of the exact sum, as a chain of two fp32 fmas).
__device__ __forceinline__ float dot_i8_word(uint32_t w, uint32_t x01, uint32_t x23, float acc) {
  const h16x2 bias = {(_Float16)-1152.0f, (_Float16)-1152.0f};
  const h16x2 lo = as_h2(__builtin_amdgcn_perm(0x64646464u, w, 0x04010400u)) + bias;  // columns 0, 1
  const h16x2 hi = as_h2(__builtin_amdgcn_perm(0x64646464u, w, 0x04030402u)) + bias;  // columns 2, 3
  acc = __builtin_amdgcn_fdot2(lo, as_h2(x01), acc, false);
  return __builtin_amdgcn_fdot2(hi, as_h2(x23), acc, false);
}

// (w & mask) | magic in one instruction (the compiler splits it in two: neither constant fits a
// 32-bit operand of the three-operand form, so one comes from an SGPR and one from a VGPR)
__device__ __forceinline__ uint32_t and_or(uint32_t w, uint32_t mask, uint32_t magic) {
  uint32_t r;
  asm("v_and_or_b32 %0, %1, %2, %3" : "=v"(r) : "v"(w), "s"(mask), "v"(magic));
  return r;
}

__device__ __forceinline__ float dot_i4_word(uint32_t w, u32x4 x, float acc) {
  const h16x2 b1 = {(_Float16)-1032.0f, (_Float16)-1032.0f};
  const h16x2 m16 = {(_Float16)0.0625f, (_Float16)0.0625f};
  const h16x2 b2 = {(_Float16)-72.0f, (_Float16)-72.0f};
  const uint32_t magic = 0x64006400u, w8 = w >> 8;
  const h16x2 p0 = as_h2(and_or(w, 0x000F000Fu, magic)) + b1;                                  // columns 0, 1
  const h16x2 p1 = __builtin_elementwise_fma(as_h2(and_or(w, 0x00F000F0u, magic)), m16, b2);   // columns 2, 3
  const h16x2 p2 = as_h2(and_or(w8, 0x000F000Fu, magic)) + b1;                                 // columns 4, 5
  const h16x2 p3 = __builtin_elementwise_fma(as_h2(and_or(w8, 0x00F000F0u, magic)), m16, b2);  // columns 6, 7
  acc = __builtin_amdgcn_fdot2(p0, as_h2(x.x), acc, false);
  acc = __builtin_amdgcn_fdot2(p1, as_h2(x.y), acc, false);
  acc = __builtin_amdgcn_fdot2(p2, as_h2(x.z), acc, false);
  return __builtin_amdgcn_fdot2(p3, as_h2(x.w), acc, false);
}

template <int WDT>
__device__ __forceinline__ float chunk_dot(u32x4 w, const float* __restrict__ x) {
  if constexpr (WDT == WI8) {  // 16 columns; x: 16 binary16 (two 16-byte LDS reads)
    const u32x4 xa = *reinterpret_cast<const u32x4*>(x);
    const u32x4 xb = *reinterpret_cast<const u32x4*>(x + 4);
    float a = 0.f, b = 0.f;
    a = dot_i8_word(w.x, xa.x, xa.y, a);
    b = dot_i8_word(w.y, xa.z, xa.w, b);
    a = dot_i8_word(w.z, xb.x, xb.y, a);
    b = dot_i8_word(w.w, xb.z, xb.w, b);
    return a + b;
  } else if constexpr (WDT == WI4) {  // 32 columns; x: 32 binary16 (four 16-byte LDS reads)
    const u32x4* xv = reinterpret_cast<const u32x4*>(x);
    float a = 0.f, b = 0.f;
    a = dot_i4_word(w.x, xv[0], a);
    b = dot_i4_word(w.y, xv[1], b);
    a = dot_i4_word(w.z, xv[2], a);
    b = dot_i4_word(w.w, xv[3], b);
    return a + b;
  } else if constexpr (WDT == WFP8) {
    const float4 x0 = *reinterpret_cast<const float4*>(x);
    const float4 x1 = *reinterpret_cast<const float4*>(x + 4);
    const float4 x2 = *reinterpret_cast<const float4*>(x + 8);
    const float4 x3 = *reinterpret_cast<const float4*>(x + 12);
    float a = 0.f, b = 0.f;
    f32x2 p;
    p = __builtin_amdgcn_cvt_pk_f32_fp8(w.x, false); a = fmaf(p.x, x0.x, a); b = fmaf(p.y, x0.y, b);
    p = __builtin_amdgcn_cvt_pk_f32_fp8(w.x, true);  a = fmaf(p.x, x0.z, a); b = fmaf(p.y, x0.w, b);
    p = __builtin_amdgcn_cvt_pk_f32_fp8(w.y, false); a = fmaf(p.x, x1.x, a); b = fmaf(p.y, x1.y, b);
    p = __builtin_amdgcn_cvt_pk_f32_fp8(w.y, true);  a = fmaf(p.x, x1.z, a); b = fmaf(p.y, x1.w, b);
    p = __builtin_amdgcn_cvt_pk_f32_fp8(w.z, false); a = fmaf(p.x, x2.x, a); b = fmaf(p.y, x2.y, b);
    p = __builtin_amdgcn_cvt_pk_f32_fp8(w.z, true);  a = fmaf(p.x, x2.z, a); b = fmaf(p.y, x2.w, b);
    p = __builtin_amdgcn_cvt_pk_f32_fp8(w.w, false); a = fmaf(p.x, x3.x, a); b = fmaf(p.y, x3.y, b);
    p = __builtin_amdgcn_cvt_pk_f32_fp8(w.w, true);  a = fmaf(p.x, x3.z, a); b = fmaf(p.y, x3.w, b);
    return a + b;
  } else {
    const float4 x0 = *reinterpret_cast<const float4*>(x);
    const float4 x1 = *reinterpret_cast<const float4*>(x + 4);
    float a = 0.f, b = 0.f;
    a = fmaf(dec16<WDT>((uint16_t)(w.x & 0xffffu)), x0.x, a);
    b = fmaf(dec16<WDT>((uint16_t)(w.x >> 16)), x0.y, b);
    a = fmaf(dec16<WDT>((uint16_t)(w.y & 0xffffu)), x0.z, a);
    b = fmaf(dec16<WDT>((uint16_t)(w.y >> 16)), x0.w, b);
    a = fmaf(dec16<WDT>((uint16_t)(w.z & 0xffffu)), x1.x, a);
    b = fmaf(dec16<WDT>((uint16_t)(w.z >> 16)), x1.y, b);
    a = fmaf(dec16<WDT>((uint16_t)(w.w & 0xffffu)), x1.z, a);
    b = fmaf(dec16<WDT>((uint16_t)(w.w >> 16)), x1.w, b);
    return a + b;
  }
}

// chunk_dot with the activations already in registers (the same order of operations, so the same
// result): x[k] holds elements 4k .. 4k+3 of the chunk
template <int WDT>
__device__ __forceinline__ float chunk_dot_regs(u32x4 w, const float4* x) {
  if constexpr (WDT == WFP8) {
    float a = 0.f, b = 0.f;
    f32x2 p;
    p = __builtin_amdgcn_cvt_pk_f32_fp8(w.x, false); a = fmaf(p.x, x[0].x, a); b = fmaf(p.y, x[0].y, b);
    p = __builtin_amdgcn_cvt_pk_f32_fp8(w.x, true);  a = fmaf(p.x, x[0].z, a); b = fmaf(p.y, x[0].w, b);
    p = __builtin_amdgcn_cvt_pk_f32_fp8(w.y, false); a = fmaf(p.x, x[1].x, a); b = fmaf(p.y, x[1].y, b);
    p = __builtin_amdgcn_cvt_pk_f32_fp8(w.y, true);  a = fmaf(p.x, x[1].z, a); b = fmaf(p.y, x[1].w, b);
    p = __builtin_amdgcn_cvt_pk_f32_fp8(w.z, false); a = fmaf(p.x, x[2].x, a); b = fmaf(p.y, x[2].y, b);
    p = __builtin_amdgcn_cvt_pk_f32_fp8(w.z, true);  a = fmaf(p.x, x[2].z, a); b = fmaf(p.y, x[2].w, b);
    p = __builtin_amdgcn_cvt_pk_f32_fp8(w.w, false); a = fmaf(p.x, x[3].x, a); b = fmaf(p.y, x[3].y, b);
    p = __builtin_amdgcn_cvt_pk_f32_fp8(w.w, true);  a = fmaf(p.x, x[3].z, a); b = fmaf(p.y, x[3].w, b);
    return a + b;
  } else {
    float a = 0.f, b = 0.f;
    a = fmaf(dec16<WDT>((uint16_t)(w.x & 0xffffu)), x[0].x, a);
    b = fmaf(dec16<WDT>((uint16_t)(w.x >> 16)), x[0].y, b);
    a = fmaf(dec16<WDT>((uint16_t)(w.y & 0xffffu)), x[0].z, a);
    b = fmaf(dec16<WDT>((uint16_t)(w.y >> 16)), x[0].w, b);
    a = fmaf(dec16<WDT>((uint16_t)(w.z & 0xffffu)), x[1].x, a);
    b = fmaf(dec16<WDT>((uint16_t)(w.z >> 16)), x[1].y, b);
    a = fmaf(dec16<WDT>((uint16_t)(w.w & 0xffffu)), x[1].z, a);
    b = fmaf(dec16<WDT>((uint16_t)(w.w >> 16)), x[1].w, b);
    return a + b;
  }
}

// register ring depth (16-byte weight loads in flight per lane); fp8 slots also carry a block scale
#ifndef PMK_RING_UNITS
#define PMK_RING_UNITS 10
#endif
template <int WDT>
constexpr int ring_depth() { return WDT == WFP8 && PMK_RING_UNITS > 16 ? 16 : PMK_RING_UNITS; }
// of which issued before a task's dependency wait
#ifndef PMK_PREFETCH_UNITS
#define PMK_PREFETCH_UNITS 10
#endif
template <int WDT>
constexpr int prefetch_depth() { return PMK_PREFETCH_UNITS < ring_depth<WDT>() ? PMK_PREFETCH_UNITS : ring_depth<WDT>(); }

// Split of one GEMV tile over the 8 waves: KS slices of every row's K times 8/KS groups of rows;
// KS minimises the busiest wave's cost, units plus row_cost per row (a row ends in a wave-wide
// reduction; short tiles then still keep all waves streaming).  KS never exceeds the row's slice
// count: every wave of a row group then owns at least one slice, so every partial sum the
// reduction reads (one per row and slice range) is written.  Wave w takes row group w / KS
// and slice range w % KS; its units (one 16-byte chunk per lane of one row and one 64-chunk
// slice) run row by row, slices in order within a row.
struct TileSplit {
  int R, KS, gi, si, wr0, wr1, s0, s1, nunits;
  __device__ __forceinline__ TileSplit(int r0, int r1, int nsl, int wave, int row_cost = 0) {
    R = r1 - r0;
    int best = 0x7fffffff;
    KS = 1;
#pragma unroll
    for (int ks = 1; ks <= kWaves; ks <<= 1) {
      const int g = kWaves / ks;
      const int cost = ((R + g - 1) / g) * ((nsl + ks - 1) / ks + row_cost);
      if (ks <= nsl && cost < best) { best = cost; KS = ks; }
    }
    const int G = kWaves / KS;
    gi = wave / KS;
    si = wave % KS;
    wr0 = r0 + (int)((int64_t)R * gi / G);
    wr1 = r0 + (int)((int64_t)R * (gi + 1) / G);
    s0 = (int)((int64_t)nsl * si / KS);
    s1 = (int)((int64_t)nsl * (si + 1) / KS);
    nunits = (wr1 - wr0) * (s1 - s0);
  }
};

// GEMV over rows [r0, r1) of W (row-major [rows][K]) against the vector staged in LDS by `sync`.
// On return (after a workgroup barrier) y[r - r0] holds row r's fp32 dot product.  yp is LDS
// scratch of 8 * (r1 - r0) floats for the per-slice partial sums (summed in slice order).
// A lane reads 16-byte chunks c = j*64 + lane of a row (slice j), so one wave instruction streams
// 1 KiB.  Weight loads run through a ring of kRing registers per lane (10 x 16 B: 80 KiB in flight
// per workgroup; measured on the 8B-class decode, deeper rings stream more slowly and shallower
// ones cannot cover the latency); the first kPre (the whole ring by default) are issued BEFORE the
// dependency wait (weights do not depend on it); each consumed slot is refilled with the chunk
// kRing units ahead, until the wave's units are all issued.  The loop issues no other global load.
template <int WDT, class Sync, class ScaleRow>
__device__ __forceinline__ void gemv_rows(const uint8_t* __restrict__ W, int K, int r0, int r1, const float* xs,
                                          float* yp, float* y, bool prefetch, Sync sync, ScaleRow srow,
                                          int row_cost = 0) {
  constexpr int EPL = WFmt<WDT>::EPL;
  const int lane = threadIdx.x & 63;
  // int4 takes the wave index as a scalar: the split, the issue cursor and the unit branches are
  // then scalar, ~87 vector instructions per unit instead of ~108, for a loop that is vector-ALU
  // bound (8B int4 482 -> 500 tok/s in an A/B).  For the other formats the scalar cursor costs
  // reloads from the full scalar file instead and runs no faster (bf16, int8) or slower (fp8).
  const int wave = WDT == WI4 ? __builtin_amdgcn_readfirstlane(threadIdx.x >> 6) : threadIdx.x >> 6;
  const int64_t rb = WFmt<WDT>::row_bytes(K);
  const int nch = K / EPL, nsl = (nch + 63) >> 6;
  const TileSplit sp(r0, r1, nsl, wave, row_cost);
  const int R = sp.R, KS = sp.KS, si = sp.si, wr0 = sp.wr0, wr1 = sp.wr1, s0 = sp.s0, s1 = sp.s1;
  const int nunits = sp.nunits;

  constexpr int kRing = ring_depth<WDT>();
  u32x4 ring[kRing];
  float rsc[kRing];
  // The tile's rows go through a buffer resource: an offset past the tile (units after the wave's
  // last one, the unused lanes of a partial last slice) reads zeros without touching memory, so
  // no loaded value is ever selected on and every load stays in flight until it is consumed.
  const __amdgpu_buffer_rsrc_t wr = __builtin_amdgcn_make_buffer_rsrc(
      const_cast<uint8_t*>(W + (int64_t)r0 * rb), (short)0, (int)((int64_t)R * rb), 0x00020000);
  constexpr uint32_t kOut = (uint32_t)kMaxTileBytes;  // past any tile the validator accepts
  // The issue cursor (row, slice) moves row by row; the row's byte offset in the tile and (scaled
  // formats) its scale row are updated when the row changes, not recomputed per unit: the fp8 loops
  // run close to the vector-ALU issue limit, and the per-unit index arithmetic was most of it.
  int lrow = wr0, lj = s0;
  uint32_t roff = (uint32_t)((int64_t)(wr0 - r0) * rb);
  const typename WFmt<WDT>::ST* srp = nullptr;
  // a wave without rows reads the tile's first row's scales (a row that exists) for its zero units
  const int srow0 = wr0 < wr1 ? wr0 : r0;
  if constexpr (WFmt<WDT>::SCALED) srp = srow(srow0);
  // The chunk count lives in a vector register: the issue's compare then needs no scalar register.
  // The scalar file of this kernel is full, and without this the count was reloaded from a spill
  // slot at every unit (8B decode 324 -> 337 tok/s in an A/B; pinning the row stride the same way
  // as well moved other values into spills and was slower).
  int nch_v = nch;
  asm volatile("" : "+v"(nch_v));
  auto issue = [&](int d) {
    const int c = lj * 64 + lane;
    const bool ok = lrow < wr1 && c < nch_v;
    const uint32_t off = ok ? roff + (uint32_t)c * 16u : kOut;
    ring[d] = __builtin_amdgcn_raw_buffer_load_b128(wr, off, 0, 2);  // nontemporal
    if constexpr (WFmt<WDT>::SCALED) rsc[d] = scale_value<WDT>(srp[(uint32_t)(c < nch ? c : 0) / WFmt<WDT>::CPG]);
    if (++lj == s1) {
      lj = s0;
      ++lrow;
      roff += (uint32_t)rb;
      if constexpr (WFmt<WDT>::SCALED) srp = srow(lrow < wr1 ? lrow : srow0);
    }
  };
  // kPre units per lane are issued before the dependency wait (when prefetching), the rest of the
  // ring after it: loads leave a workgroup in issue order, so a deep pre-wait backlog would delay
  // the wait's polls and the input staging behind it.  Both branches issue the same number of
  // loads, which keeps the compiler's load counting exact for the first pass of the ring.
  constexpr int kPre = prefetch_depth<WDT>();
  if (prefetch) {
#pragma unroll
    for (int d = 0; d < kPre; ++d) issue(d);
    sync();
  } else {
    sync();
#pragma unroll
    for (int d = 0; d < kPre; ++d) issue(d);
  }
#pragma unroll
  for (int d = kPre; d < kRing; ++d) issue(d);
  if (nunits > 0) {
    float acc = 0.f;
    int crow = wr0, cj = s0;
    for (int base = 0; base < nunits; base += kRing) {
#pragma unroll
      for (int d = 0; d < kRing; ++d) {
        // consume slot d, then refill it: the refill lands in the slot's own registers, so the
        // ring never needs copying (a copy would have to wait for every load in flight)
        if (base + d < nunits) {
          const float part = chunk_dot<WDT>(ring[d], xchunk<WDT>(xs, cj * 64 + lane));
          if constexpr (WFmt<WDT>::SCALED) acc = fmaf(part, rsc[d], acc);
          else acc += part;
          if (++cj == s1) {
            cj = s0;
            const float v = wave_sum(acc);
            acc = 0.f;
            if (lane == 0) yp[(crow - r0) * KS + si] = v;
            ++crow;
          }
        }
        issue(d);
      }
    }
  }
  __syncthreads();
  for (int i = threadIdx.x; i < R; i += kThreads) {
    float v = 0.f;
    for (int k = 0; k < KS; ++k) v += yp[i * KS + k];
    y[i] = v;
  }
  __syncthreads();
}

typedef __attribute__((address_space(3))) void lds_void;

// Copy a GEMV tile (rows [r0, r1) of W) into LDS with LDS-DMA buffer loads: no registers, and an
// out-of-range lane (past the last chunk of a row) writes zeros.  Unit (row, slice) lands at
// pf + ((row - r0) * nsl + slice) KiB; each wave copies the units gemv_rows_lds has it consume
// (same split), so its own load counter orders the copy before its reads (the compiler waits on
// outstanding LDS-DMA before an LDS access that may alias it).
template <int WDT>
__device__ __forceinline__ void tile_to_lds(const uint8_t* __restrict__ W, int K, int r0, int r1, float* pf,
                                            int row_cost) {
  const int lane = threadIdx.x & 63, wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int64_t rb = WFmt<WDT>::row_bytes(K);
  const int nch = K / WFmt<WDT>::EPL, nsl = (nch + 63) >> 6;
  const TileSplit sp(r0, r1, nsl, wave, row_cost);
  const __amdgpu_buffer_rsrc_t wr = __builtin_amdgcn_make_buffer_rsrc(
      const_cast<uint8_t*>(W + (int64_t)r0 * rb), (short)0, (int)((int64_t)sp.R * rb), 0x00020000);
  constexpr uint32_t kOut = (uint32_t)kMaxTileBytes;
  int lrow = sp.wr0, lj = sp.s0;
  for (int u = 0; u < sp.nunits; ++u) {
    const int c = lj * 64 + lane;
    const uint32_t off = c < nch ? (uint32_t)((int64_t)(lrow - r0) * rb + (int64_t)c * 16) : kOut;
    __builtin_amdgcn_raw_ptr_buffer_load_lds(wr, (lds_void*)(pf + ((lrow - r0) * nsl + lj) * 256), 16, off, 0, 0,
                                             2);  // nontemporal
    if (++lj == sp.s1) { lj = sp.s0; ++lrow; }
  }
}

// gemv_rows over a tile that tile_to_lds copies into LDS (issued before this call, so the copy
// overlaps `sync`, the dependency wait and input staging): the same split, the same per-lane
// chunk order and the same summation order, so the results are bitwise those of gemv_rows.
template <int WDT, class Sync, class ScaleRow>
__device__ __forceinline__ void gemv_rows_lds(int K, int r0, int r1, const float* xs, const float* pf, float* yp,
                                              float* y, Sync sync, ScaleRow srow, int row_cost) {
  constexpr int EPL = WFmt<WDT>::EPL;
  const int lane = threadIdx.x & 63, wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int nch = K / EPL, nsl = (nch + 63) >> 6;
  const TileSplit sp(r0, r1, nsl, wave, row_cost);
  const int R = sp.R, KS = sp.KS, si = sp.si, s0 = sp.s0, s1 = sp.s1;
  sync();
  // FP8: the activation chunks a lane multiplies are the same for every row of its slices, so with
  // up to 4 slices per wave they are read from LDS once, into registers (+0.4% on the 8B FP8 decode
  // in an A/B; for 16-bit weights the same change measured -0.15%, so they keep the LDS reads)
  constexpr int MAXS = WDT == WFP8 ? 64 / EPL : 0;
  const int ns = s1 - s0;
  if (MAXS > 0 && sp.nunits > 0 && ns >= 1 && ns <= MAXS) {
    constexpr int F4 = EPL / 4;  // float4 per chunk
    float4 xr[MAXS > 0 ? MAXS : 1][F4];
#pragma unroll
    for (int k = 0; k < MAXS; ++k)
      if (k < ns)
#pragma unroll
        for (int f = 0; f < F4; ++f) xr[k][f] = *reinterpret_cast<const float4*>(xs + ((s0 + k) * 64 + lane) * EPL + 4 * f);
    for (int row = sp.wr0; row < sp.wr1; ++row) {
      const float* src = pf + (row - r0) * nsl * 256 + lane * 4;
      float acc = 0.f;
      u32x4 w[MAXS > 0 ? MAXS : 1];
#pragma unroll
      for (int k = 0; k < MAXS; ++k)
        if (k < ns) w[k] = *reinterpret_cast<const u32x4*>(src + (s0 + k) * 256);
#pragma unroll
      for (int k = 0; k < MAXS; ++k)
        if (k < ns) {
          const float part = chunk_dot_regs<WDT>(w[k], xr[k]);
          if constexpr (WDT == WFP8) {
            const int c = (s0 + k) * 64 + lane;
            acc = fmaf(part, srow(row)[(c < nch ? c : 0) >> 3], acc);
          } else {
            acc += part;
          }
        }
      const float v = wave_sum(acc);
      if (lane == 0) yp[(row - r0) * KS + si] = v;
    }
  } else if (sp.nunits > 0) {
    for (int row = sp.wr0; row < sp.wr1; ++row) {
      const float* src = pf + (row - r0) * nsl * 256 + lane * 4;
      int u = s0;
      float acc = 0.f;
      auto step = [&](const u32x4& w, int j) {
        const int c = j * 64 + lane;
        const float part = chunk_dot<WDT>(w, xchunk<WDT>(xs, c));
        if constexpr (WFmt<WDT>::SCALED)
          acc = fmaf(part, scale_value<WDT>(srow(row)[(uint32_t)(c < nch ? c : 0) / WFmt<WDT>::CPG]), acc);
        else
          acc += part;
      };
      int j = s0;
      for (; j + 4 <= s1; j += 4, u += 4) {  // four units' LDS reads in flight
        u32x4 w[4];
#pragma unroll
        for (int k = 0; k < 4; ++k) w[k] = *reinterpret_cast<const u32x4*>(src + (u + k) * 256);
#pragma unroll
        for (int k = 0; k < 4; ++k) step(w[k], j + k);
      }
      for (; j < s1; ++j, ++u) step(*reinterpret_cast<const u32x4*>(src + u * 256), j);
      const float v = wave_sum(acc);
      if (lane == 0) yp[(row - r0) * KS + si] = v;
    }
  }
  __syncthreads();
  for (int i = threadIdx.x; i < R; i += kThreads) {
    float v = 0.f;
    for (int k = 0; k < KS; ++k) v += yp[i * KS + k];
    y[i] = v;
  }
  __syncthreads();
}

// ------------------------------------------------------------------------------------------------
// input staging (RMSNorm prologue fused into the consuming GEMV)
// ------------------------------------------------------------------------------------------------
// Two fp32 values as a binary16 pair (nearest even), the lower element in the low half.
__device__ __forceinline__ uint32_t pack_h2(float a, float b) {
  return __builtin_bit_cast(uint32_t, __builtin_convertvector((f32x2){a, b}, h16x2));
}

// Store staged elements i, i+1 of the activation vector: fp32, or one binary16 pair (H16).
template <bool H16>
__device__ __forceinline__ void put2(float* xs, int i, float a, float b) {
  if constexpr (H16) reinterpret_cast<uint32_t*>(xs)[i >> 1] = pack_h2(a, b);
  else *reinterpret_cast<float2*>(xs + i) = make_float2(a, b);
}

// Load n fp32 values from a coherent buffer into xs[0..pad) (zeros past n), every load of a
// batch issued before any is consumed.  H16 stores them as binary16.
template <bool H16 = false, int B = 8>
__device__ __forceinline__ void load_vector(const float* src, int n, int pad, float* xs) {
  const __amdgpu_buffer_rsrc_t r = coherent_rsrc(src, (uint32_t)n * 4);
  for (int base = 0; base < pad; base += B * 4 * kThreads) {
    u32x4 v[B];
#pragma unroll
    for (int k = 0; k < B; ++k) {
      const int i = base + (k * kThreads + (int)threadIdx.x) * 4;
      v[k] = i < pad ? ldc16(r, (uint32_t)i * 4) : u32x4{0u, 0u, 0u, 0u};
    }
#pragma unroll
    for (int k = 0; k < B; ++k) {
      const int i = base + (k * kThreads + (int)threadIdx.x) * 4;
      if (i < pad) {
        const float4 f = as_f4(v[k]);
        if constexpr (H16)
          *reinterpret_cast<uint2*>(xs + (i >> 1)) = make_uint2(pack_h2(f.x, f.y), pack_h2(f.z, f.w));
        else
          *reinterpret_cast<float4*>(xs + i) = f;
      }
    }
  }
}

// RMSNorm prologue, split in two.  The staging writes xs[0..H) = src * gain (xs[H..pad) = 0)
// and red[w] = wave w's share of sum(src^2), with one batch of loads and one barrier; the factor
// 1/sqrt(mean(src^2) + eps) (rms_factor) then scales the GEMV results, since every row's dot
// product with (src * gain) times that factor is its dot product with the normalised input.
// With RAW (the integer weight formats) xs holds src itself and gs the gains, and norm_to_h16 then
// forms the normalised vector (src * r) * gain and rounds it to binary16, the activation operand
// those formats define.
// This one stages a 16-bit embedding row (the first layer's input); stage_rmsnorm_tagged stages
// the tagged residual stream.
template <int EDT, bool RAW = false>
__device__ __forceinline__ void stage_rmsnorm_embed(const uint16_t* emb, const float* gain, int H, int pad, float* xs,
                                                    float* red, float* gs = nullptr) {
  float ss = 0.f;
  for (int i = 8 * threadIdx.x; i < pad; i += 8 * kThreads) {
    float f[8], g[8];
    if (i < H) {
      const u32x4 w = *reinterpret_cast<const u32x4*>(emb + i);
      const float4 g0 = *reinterpret_cast<const float4*>(gain + i);
      const float4 g1 = *reinterpret_cast<const float4*>(gain + i + 4);
      g[0] = g0.x; g[1] = g0.y; g[2] = g0.z; g[3] = g0.w;
      g[4] = g1.x; g[5] = g1.y; g[6] = g1.z; g[7] = g1.w;
      const uint32_t wd[4] = {w.x, w.y, w.z, w.w};
#pragma unroll
      for (int k = 0; k < 4; ++k) {
        f[2 * k] = dec16<EDT>((uint16_t)(wd[k] & 0xffff));
        f[2 * k + 1] = dec16<EDT>((uint16_t)(wd[k] >> 16));
      }
    } else {
#pragma unroll
      for (int k = 0; k < 8; ++k) f[k] = g[k] = 0.f;
    }
#pragma unroll
    for (int k = 0; k < 8; ++k) {
      xs[i + k] = RAW ? f[k] : f[k] * g[k];
      if constexpr (RAW) gs[i + k] = g[k];
      ss = fmaf(f[k], f[k], ss);
    }
  }
  ss = wave_sum(ss);
  if ((threadIdx.x & 63) == 0) red[threadIdx.x >> 6] = ss;
  __syncthreads();
}

__device__ __forceinline__ float rms_factor(const float* red, int H, float eps) {
  float t = 0.f;
#pragma unroll
  for (int w = 0; w < kWaves; ++w) t += red[w];
  return 1.0f / sqrtf(t / (float)H + eps);
}

// Integer weight formats: after an RMSNorm staging with RAW / H16 (xs = src and gs = the gains in
// fp32, red = the wave sums, behind a barrier), xh[0..pad) = binary16((src * r) * gain) with r =
// 1 / sqrt(mean(src^2) + eps) (zeros past H), the normalised vector in the order of operations of
// its definition; ends with a barrier.  The GEMV results then need no factor.
__device__ __forceinline__ void norm_to_h16(const float* xs, const float* gs, int H, int pad, const float* red,
                                            float eps, float* xh) {
  const float r = rms_factor(red, H, eps);
  for (int i = 2 * (int)threadIdx.x; i < pad; i += 2 * kThreads) {
    float a = 0.f, b = 0.f;
    if (i < H) {
      const float2 x = *reinterpret_cast<const float2*>(xs + i);
      const float2 g = *reinterpret_cast<const float2*>(gs + i);
      a = (x.x * r) * g.x;
      b = (x.y * r) * g.y;
    }
    reinterpret_cast<uint32_t*>(xh)[i >> 1] = pack_h2(a, b);
  }
  __syncthreads();
}

__device__ __forceinline__ int pad_len(int n, int epl) {
  const int slice = 64 * epl;
  return (n + slice - 1) / slice * slice;
}

// ------------------------------------------------------------------------------------------------
// step context and token handling
// ------------------------------------------------------------------------------------------------
struct StepCtx {
  int e;        // global step (since the last reset)
  int s;        // step within this call
  int pos;      // position written by this step
  int pos0;     // first position written by this kernel launch (KV rows from pos0 on are read coherently)
  int tok;      // input token if already known, else -1
  bool per_op;  // per-op kernels: no waits (kernel boundaries order the tasks)
  bool calib;   // FP8 KV scale calibration: QKV records max |k|, |v| of every appended row
};

// Stage a tagged vector src[0..n) of step e into xs (zero padding to pad): every thread re-reads
// its 16-byte pairs until both tags show step e (bounded by the watchdog; the abort word is
// checked on every retry).  The reads are the wait; the caller's barrier ends it.  With NORM, xs
// holds src * gain and the return value is this thread's share of sum(src^2) (the gains are
// loaded before the first read, since they do not depend on the wait).
template <bool NORM = false, bool H16 = false>
__device__ __forceinline__ float stage_tagged(const KParams& P, const unsigned long long* src, int n, int pad,
                                              float* xs, int e, bool poll, int cu, int task,
                                              const float* gain = nullptr, float* gs = nullptr) {
  constexpr int B = 4;  // 16-byte loads (two values) per thread per batch
  const __amdgpu_buffer_rsrc_t r = coherent_rsrc(src, (uint32_t)n * 8);
  const uint32_t want = (uint32_t)(e + 1);
  float ss = 0.f;
  for (int base = 0; base < pad; base += B * 2 * kThreads) {
    u32x4 v[B];
    bool ok[B];
    float2 g[B];
#pragma unroll
    for (int k = 0; k < B; ++k) {
      ok[k] = false;
      const int i = base + (k * kThreads + (int)threadIdx.x) * 2;
      if constexpr (NORM) g[k] = i < n ? *reinterpret_cast<const float2*>(gain + i) : make_float2(0.f, 0.f);
    }
    int64_t spins = 0;
    while (true) {
      __atomic_signal_fence(__ATOMIC_SEQ_CST);  // each retry reads memory again
#pragma unroll
      for (int k = 0; k < B; ++k) {
        const int i = base + (k * kThreads + (int)threadIdx.x) * 2;
        if (!ok[k]) v[k] = i < n ? ldc16(r, (uint32_t)i * 8) : u32x4{0u, want, 0u, want};
      }
      bool all = true;
#pragma unroll
      for (int k = 0; k < B; ++k) {
        ok[k] = ok[k] || !poll || (v[k].y == want && v[k].w == want);
        all = all && ok[k];
      }
      if (all) break;
      if (ldc(&P.ctrl[CTRL_ABORT]) != 0u) break;
      if (++spins > P.spin_limit) {
        report_error(P.ctrl, PMK_ERR_TIMEOUT, cu, task, -1, want, v[0].y);
        break;
      }
    }
#pragma unroll
    for (int k = 0; k < B; ++k) {
      const int i = base + (k * kThreads + (int)threadIdx.x) * 2;
      float a = __uint_as_float(v[k].x), b = __uint_as_float(v[k].z);
      if constexpr (NORM) {
        ss = fmaf(a, a, ss);
        ss = fmaf(b, b, ss);
        if constexpr (!H16) {  // H16 with NORM: src itself and the gains, normalised by norm_to_h16
          a *= g[k].x;
          b *= g[k].y;
        } else {
          if (i < pad) *reinterpret_cast<float2*>(gs + i) = g[k];
        }
      }
      if (i < pad) put2<H16 && !NORM>(xs, i, a, b);
    }
  }
  return ss;
}

// RMSNorm prologue from a tagged vector (as stage_rmsnorm): xs = src * gain (H16: src), red[w] =
// wave w's share of sum(src^2), one barrier.
template <bool H16 = false>
__device__ __forceinline__ void stage_rmsnorm_tagged(const KParams& P, const unsigned long long* src, const float* gain,
                                                     int H, int pad, float* xs, float* red, int e, bool poll, int cu,
                                                     int task, float* gs = nullptr) {
  float ss = stage_tagged<true, H16>(P, src, H, pad, xs, e, poll, cu, task, gain, gs);
  ss = wave_sum(ss);
  if ((threadIdx.x & 63) == 0) red[threadIdx.x >> 6] = ss;
  __syncthreads();
}

// One tagged value of step e (re-read until its tag shows e, like stage_tagged).
__device__ __forceinline__ float ld_tagged(const KParams& P, const unsigned long long* p, int e, bool poll, int cu,
                                           int task) {
  const uint32_t want = (uint32_t)(e + 1);
  int64_t spins = 0;
  while (true) {
    const unsigned long long v = ldc(p);
    if (!poll || (uint32_t)(v >> 32) == want) return __uint_as_float((uint32_t)v);
    if (ldc(&P.ctrl[CTRL_ABORT]) != 0u || ++spins > P.spin_limit) {
      if (spins > P.spin_limit) report_error(P.ctrl, PMK_ERR_TIMEOUT, cu, task, -1, want, (uint32_t)(v >> 32));
      return __uint_as_float((uint32_t)v);
    }
  }
}

// In flags mode a consumer of a tagged vector (x, xm, o) polls the tags instead of its producers'
// flags, and those producers publish no flag; counters mode keeps counter waits and signals.
__device__ __forceinline__ bool polls_tags(const KParams& P, const StepCtx& sc) {
  return !sc.per_op && P.sync_mode != PMK_SYNC_COUNTERS;
}

// An O projection tile that fits the LDS tile area is copied there whole (LDS-DMA) before the
// task's dependency wait, instead of the register ring's first units: the wait for the attention
// combine is long enough for all of it to land, and the GEMV then runs from LDS.
__device__ __forceinline__ bool oproj_tile_in_lds(const KParams& P, const pmk_task& t, const StepCtx& sc, int nsl) {
  return P.prefetch == 2 && !sc.per_op && (t.a1 - t.a0) * nsl <= P.pf_units;
}

// O-projection tiles are short (a few rows per CU): the split weighs each row's reduction like
// four units, the same in every mode, so the LDS path and the streaming path agree bitwise
constexpr int kOprojRowCost = 4;
// LM-head tiles are long (~500 rows per CU on a 128K vocabulary) and short-rowed (4 or 8 slices):
// with no row cost the split gave every wave one slice of every row, so each unit ended in a
// wave-wide reduction, which made the fp8 head vector-ALU bound (~20 GB/s per CU against ~28 for
// the other phases).  Weighing a row end like one unit keeps whole rows in one wave.
constexpr int kLmheadRowCost = 1;

__device__ __forceinline__ int key_token(unsigned long long key) { return (int)(0xFFFFFFFFu - (uint32_t)key); }

__device__ __forceinline__ int input_token(const KParams& P, const StepCtx& sc) {
  int tok = sc.tok;
  if (tok < 0) tok = key_token(ldc(&P.keys[sc.s - 1]));
  return tok < 0 ? 0 : (tok >= P.V ? P.V - 1 : tok);
}

__device__ __forceinline__ void trace_mark(const KParams& P, int s, int ti, int slot, uint64_t value) {
  if (threadIdx.x == 0 && P.trace_steps > 0 && P.call->trace && s < P.trace_steps)
    P.trace[((int64_t)s * P.n_tasks + ti) * 8 + slot] = value;
}

// sub-phase timestamp of the running task (trace slots 4..7)
__device__ __forceinline__ void mark(const KParams& P, const StepCtx& sc, int ti, int slot) {
  if (!sc.per_op) trace_mark(P, sc.s, ti, slot, __builtin_amdgcn_s_memrealtime());
}

__device__ __forceinline__ void maybe_wait(const KParams& P, const pmk_task& t, const StepCtx& sc, int cu, int ti) {
  if (sc.per_op) return;
  block_wait(P, t.wait_ctr, t.wait_count, t.wait_lag, sc.e, cu, ti);
  trace_mark(P, sc.s, ti, 1, __builtin_amdgcn_s_memrealtime());
}

// ------------------------------------------------------------------------------------------------
// tasks
// ------------------------------------------------------------------------------------------------
// Scale array of linear tensor `which` (q k v o gate up down) of layer l, and the scale row of
// its (unpacked) row orow: one row per 128 rows for fp8 blocks, one per row for the integer groups.
template <int WDT>
__device__ __forceinline__ const typename WFmt<WDT>::ST* scale_rows(const KParams& P, int l, int which) {
  return reinterpret_cast<const typename WFmt<WDT>::ST*>(P.scales) + (int64_t)l * P.sc_layer + P.sc_off[which];
}
template <int WDT>
__device__ __forceinline__ const typename WFmt<WDT>::ST* scale_row(const typename WFmt<WDT>::ST* base, int orow,
                                                                   int nbc) {
  return base + (int64_t)(WDT == WFP8 ? orow / 128 : orow) * nbc;
}

// QKV: RMSNorm(x) -> packed QKV rows [a0, a1) -> RoPE on q/k pairs -> q to the workspace,
// k and v appended to the cache at `pos`.  The RoPE row of this position (and the fp8 K/V scales)
// are staged in LDS with the input, so the epilogue reads no global memory.
template <int WDT, int KVDT>
__device__ __forceinline__ void task_qkv(const KParams& P, const pmk_task& t, int ti, const StepCtx& sc, float* lds,
                                         int cu) {
  constexpr int EDT = WFmt<WDT>::EDT;
  constexpr bool H16 = WFmt<WDT>::H16;
  const int l = t.layer, H = P.H, hd = P.hd, half = hd / 2;
  const int pad = pad_len(H, WFmt<WDT>::EPL);
  float* xs = lds;
  float* red = lds + P.xs_floats;
  float2* rope = reinterpret_cast<float2*>(lds + P.epi_off);  // [hd/2] (cos, sin), then [2*nkv] (scale, -)
  float* yp = lds + P.yp_off;
  float* y = lds + P.y_off;
  const uint8_t* W = P.wbase + (int64_t)l * P.layer_bytes + P.off_qkv;
  auto sync = [&]() {
    // the RoPE row of this position and the K/V scales do not depend on the wait: loaded before it
    // (half <= 64 < kThreads and 2 * nkv <= kThreads: one value per thread)
    const float2 cs = threadIdx.x < half ? P.rope[(int64_t)sc.pos * half + threadIdx.x] : make_float2(0.f, 0.f);
    float ks8 = 0.f;
    if constexpr (KVDT == WFP8)
      if (threadIdx.x < 2 * P.nkv) ks8 = P.kv_scale[(int64_t)l * P.nkv * 2 + threadIdx.x];
    const bool poll_x = l > 0 && polls_tags(P, sc);
    if (!poll_x) maybe_wait(P, t, sc, cu, ti);
    if (threadIdx.x < half) rope[threadIdx.x] = cs;
    if constexpr (KVDT == WFP8)
      if (threadIdx.x < 2 * P.nkv) rope[half + threadIdx.x] = make_float2(ks8, 0.f);
    if (l == 0) {
      const int tok = input_token(P, sc);
      stage_rmsnorm_embed<EDT, H16>(P.embed + (int64_t)tok * H, P.gains, H, pad, xs, red, lds + P.gs_off);
    } else {
      stage_rmsnorm_tagged<H16>(P, P.x + (int64_t)l * H, P.gains + (int64_t)l * 2 * H, H, pad, xs, red, sc.e,
                                !sc.per_op, cu, ti, lds + P.gs_off);
    }
    if constexpr (H16) norm_to_h16(xs, lds + P.gs_off, H, pad, red, P.eps, lds + P.xh_off);
    if (poll_x) trace_mark(P, sc.s, ti, 1, __builtin_amdgcn_s_memrealtime());
    mark(P, sc, ti, 4);
  };
  const int qrows = P.qdim, krows = P.nkv * hd;
  const int nbc = (H + 127) / 128;
  // scale-array bases taken before the loop (a dynamically indexed kernel argument would be
  // re-read from memory for every weight unit, behind a full wait)
  using ST = typename WFmt<WDT>::ST;
  const ST* const sq = scale_rows<WDT>(P, l, 0);
  const ST* const sk = scale_rows<WDT>(P, l, 1);
  const ST* const sv = scale_rows<WDT>(P, l, 2);
  auto srow = [=](int r) -> const ST* {
    const ST* base;
    int orow;
    if (r < qrows) { base = sq; orow = r; }
    else if (r < qrows + krows) { base = sk; orow = r - qrows; }
    else { base = sv; orow = r - qrows - krows; }
    const int head = orow / hd, pr = orow % hd;
    const int dim = (pr >> 1) + (pr & 1) * half;
    return scale_row<WDT>(base, head * hd + dim, nbc);
  };
  // integer formats: the GEMV reads the normalised binary16 vector, whose results need no factor
  gemv_rows<WDT>(W, H, t.a0, t.a1, H16 ? lds + P.xh_off : xs, yp, y, P.prefetch != 0, sync, srow);
  mark(P, sc, ti, 5);
  const float rn = H16 ? 1.0f : rms_factor(red, H, P.eps);
  const int npairs = (t.a1 - t.a0) >> 1;
  for (int p = threadIdx.x; p < npairs; p += kThreads) {
    const int r = t.a0 + 2 * p;
    float a = y[2 * p] * rn, b = y[2 * p + 1] * rn;
    int sec, base;
    if (r < qrows) { sec = 0; base = 0; }
    else if (r < qrows + krows) { sec = 1; base = qrows; }
    else { sec = 2; base = qrows + krows; }
    const int head = (r - base) / hd, i = ((r - base) % hd) >> 1;
    if (sec < 2) {
      const float2 cs = rope[i];
      const float a2 = a * cs.x - b * cs.y;
      const float b2 = b * cs.x + a * cs.y;
      a = a2;
      b = b2;
    }
    if (sec == 0) {
      unsigned long long* q = P.q + (int64_t)l * P.qdim + head * hd;
      stc(q + i, tagged(a, sc.e));
      stc(q + i + half, tagged(b, sc.e));
      continue;
    }
    // element index of dims i and i + hd/2 at this position: K [pos][hd] rows; V in blocks of 32
    // positions, [pos / 32][hd][pos % 32]
    const int64_t hb = (int64_t)l * P.nkv + head;
    const int64_t ia = sec == 1 ? (hb * P.seqcap + sc.pos) * hd + i
                                : ((hb * (P.seqcap / 32) + sc.pos / 32) * hd + i) * 32 + sc.pos % 32;
    const int64_t ib = sec == 1 ? ia + half : ia + (int64_t)half * 32;
    uint8_t* cache = sec == 1 ? P.kc : P.vc;
    uint32_t ba, bb;  // the stored elements as 16-bit matrix-core operands (fp8: its bf16 value)
    if constexpr (KVDT == WFP8) {
      if (sc.calib)
        __hip_atomic_fetch_max(&P.kv_amax[hb * 2 + (sec - 1)], __float_as_uint(fmaxf(fabsf(a), fabsf(b))),
                               __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      const float s8 = rope[half + 2 * head + (sec - 1)].x;
      const uint8_t ca = enc_e4m3(a / s8), cb = enc_e4m3(b / s8);
      stc(cache + ia, ca);
      stc(cache + ib, cb);
      ba = __float_as_uint(dec_e4m3(ca, 0)) >> 16;  // exact: E4M3 values are bf16 values
      bb = __float_as_uint(dec_e4m3(cb, 0)) >> 16;
    } else {
      uint16_t* c16 = reinterpret_cast<uint16_t*>(cache);
      const uint16_t ca = enc16<KVDT>(a), cb = enc16<KVDT>(b);
      stc(c16 + ia, ca);
      stc(c16 + ib, cb);
      ba = ca;
      bb = cb;
    }
    // this step's attention takes the current position from here (tagged), not from the cache
    unsigned long long* cur = P.kvcur + ((int64_t)hb * 2 + (sec - 1)) * hd;
    stc(cur + i, tagged(__uint_as_float(ba), sc.e));
    stc(cur + i + half, tagged(__uint_as_float(bb), sc.e));
  }
  if (!polls_tags(P, sc)) block_signal(P, t.signal_ctr, t.signal_slot, sc.e);
}

// Max / sum over the four lanes of a quad (quad_perm DPP); every lane of the quad receives it.
__device__ __forceinline__ float quad_max(float v) {
  v = dpp_max<0xB1, 0xF>(v);     // quad_perm [1,0,3,2]
  return dpp_max<0x4E, 0xF>(v);  // quad_perm [2,3,0,1]
}
__device__ __forceinline__ float quad_sum(float v) {
  v += __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), 0xB1, 0xF, 0xF, false));
  return v + __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), 0x4E, 0xF, 0xF, false));
}

// Sum / max over the lanes that share `lane % N` (N = 8 or 16 lanes per row): the other half of
// the DPP row for N = 8, then across the four rows with the gfx950 row-swap moves.  Every lane
// receives its column's result.
template <int N>
__device__ __forceinline__ float column_sum(float v) {
  if constexpr (N == 8) v += __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), 0x128, 0xF, 0xF, false));  // row_ror:8
  const uint32_t u = __float_as_uint(v);
  const auto r16 = __builtin_amdgcn_permlane16_swap(u, u, false, false);
  v = __uint_as_float(r16[0]) + __uint_as_float(r16[1]);
  const uint32_t w = __float_as_uint(v);
  const auto r32 = __builtin_amdgcn_permlane32_swap(w, w, false, false);
  return __uint_as_float(r32[0]) + __uint_as_float(r32[1]);
}
template <int N>
__device__ __forceinline__ float column_max(float v) {
  if constexpr (N == 8)
    v = fmaxf(v, __int_as_float(__builtin_amdgcn_update_dpp(__float_as_int(v), __float_as_int(v), 0x128, 0xF, 0xF, false)));
  const uint32_t u = __float_as_uint(v);
  const auto r16 = __builtin_amdgcn_permlane16_swap(u, u, false, false);
  v = fmaxf(__uint_as_float(r16[0]), __uint_as_float(r16[1]));
  const uint32_t w = __float_as_uint(v);
  const auto r32 = __builtin_amdgcn_permlane32_swap(w, w, false, false);
  return fmaxf(__uint_as_float(r32[0]), __uint_as_float(r32[1]));
}

// ---- 16-bit matrix-core operands (v_mfma_f32_16x16x32_{f16,bf16}) ----
// A (16 x 32): lane l holds row l % 16, k = 8 (l / 16) .. + 8; B (32 x 16): lane l holds column
// l % 16, k = 8 (l / 16) .. + 8; C (16 x 16): lane l holds rows 4 (l / 16) + i, column l % 16.
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef unsigned int u32x2 __attribute__((ext_vector_type(2)));

// the MFMA input type for a KV cache format: f16 for an f16 cache, bf16 otherwise (FP8 E4M3
// values are exact in bf16)
template <int KVDT>
__device__ __forceinline__ f32x4 mfma16(u32x4 a, u32x4 b, f32x4 c) {
  if constexpr (KVDT == WF16)
    return __builtin_amdgcn_mfma_f32_16x16x32_f16(__builtin_bit_cast(f16x8, a), __builtin_bit_cast(f16x8, b), c, 0, 0, 0);
  else
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, a), __builtin_bit_cast(bf16x8, b), c, 0, 0,
                                                   0);
}

// fp32 x[8] as two 16-bit vectors with x = hi + lo to ~2^-17 relative: an fp32 operand of a
// 16-bit matrix product costs two products (hi, then lo) accumulated in fp32.
template <int KVDT>
__device__ __forceinline__ void split16(const float* x, u32x4& hi, u32x4& lo) {
  uint32_t h[4], o[4];
#pragma unroll
  for (int k = 0; k < 4; ++k) {
    const float a = x[2 * k], b = x[2 * k + 1];
    if constexpr (KVDT == WF16) {
      const auto hp = __builtin_amdgcn_cvt_pkrtz(a, b);
      const auto lp = __builtin_amdgcn_cvt_pkrtz(a - (float)hp[0], b - (float)hp[1]);
      h[k] = __builtin_bit_cast(uint32_t, hp);
      o[k] = __builtin_bit_cast(uint32_t, lp);
    } else {
      const uint32_t hb = __builtin_bit_cast(uint32_t, __builtin_convertvector((f32x2){a, b}, bf16x2));
      const float ha = __uint_as_float(hb << 16), hbv = __uint_as_float(hb & 0xFFFF0000u);
      h[k] = hb;
      o[k] = __builtin_bit_cast(uint32_t, __builtin_convertvector((f32x2){a - ha, b - hbv}, bf16x2));
    }
  }
  hi = u32x4{h[0], h[1], h[2], h[3]};
  lo = u32x4{o[0], o[1], o[2], o[3]};
}

// fp32 x[8] as three bf16 vectors with x = hi + mid + lo to ~2^-24 relative (three products).
// The integer weight formats take this one: their GEMVs round the attention output to binary16,
// which turns a difference of ~2^-17 in it into a whole binary16 step in some elements, so the
// attention is computed to fp32 accuracy there.
__device__ __forceinline__ void split16x3(const float* x, u32x4& hi, u32x4& mid, u32x4& lo) {
  uint32_t h[4], m[4], o[4];
#pragma unroll
  for (int k = 0; k < 4; ++k) {
    const float a = x[2 * k], b = x[2 * k + 1];
    const uint32_t hb = __builtin_bit_cast(uint32_t, __builtin_convertvector((f32x2){a, b}, bf16x2));
    const float ra = a - __uint_as_float(hb << 16), rb = b - __uint_as_float(hb & 0xFFFF0000u);
    const uint32_t mb = __builtin_bit_cast(uint32_t, __builtin_convertvector((f32x2){ra, rb}, bf16x2));
    h[k] = hb;
    m[k] = mb;
    o[k] = __builtin_bit_cast(uint32_t, __builtin_convertvector(
                                            (f32x2){ra - __uint_as_float(mb << 16), rb - __uint_as_float(mb & 0xFFFF0000u)},
                                            bf16x2));
  }
  hi = u32x4{h[0], h[1], h[2], h[3]};
  mid = u32x4{m[0], m[1], m[2], m[3]};
  lo = u32x4{o[0], o[1], o[2], o[3]};
}

// 8 FP8 E4M3 values -> 8 bf16 (exact: every E4M3 value is a bf16 value).  gfx950's scaled
// conversion with scale 1 writes a bf16 pair in one instruction (checked on the device against the
// upper halves of the fp32 conversion for every pair of finite codes); converting to fp32 and
// packing took two per pair (8B FP8 prefill of 8192 tokens 1269 -> 1223 ms).
__device__ __forceinline__ u32x4 fp8x8_bf16(u32x2 w) {
#define PMK_FP8_BF16(v, hi) __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(v, 1.0f, hi))
  return u32x4{PMK_FP8_BF16(w.x, false), PMK_FP8_BF16(w.x, true), PMK_FP8_BF16(w.y, false), PMK_FP8_BF16(w.y, true)};
#undef PMK_FP8_BF16
}

// KV cache element loads through a buffer resource (out of range: zeros): 8 elements per lane as
// 16-bit matrix-core operands.  Rows of positions written before this launch are streamed
// (nontemporal); a split that holds positions written during this launch (COH) reads every row with
// agent-coherent loads (sc1), as it reads any other value another CU stored in this launch: a
// V-cache line holds 32 positions, so it is read at the steps before all of its slots are written.
// The current position is never read from the cache: it comes from its tagged copy.
template <int KVDT, bool COH>
__device__ __forceinline__ u32x4 kv_load8(__amdgpu_buffer_rsrc_t r, uint32_t off) {
  constexpr int kPol = COH ? 16 : 2;  // sc1 : nt
  if constexpr (KVDT == WFP8) {
    const u32x2 w = __builtin_amdgcn_raw_buffer_load_b64(r, off, 0, kPol);
    return fp8x8_bf16(w);
  } else {
    return __builtin_amdgcn_raw_buffer_load_b128(r, off, 0, kPol);
  }
}

// Zero the 16-bit elements j >= nv of an 8-element operand (0 <= nv < 8).
__device__ __forceinline__ u32x4 keep_first(u32x4 v, int nv) {
  uint32_t w[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
  for (int k = 0; k < 4; ++k) w[k] &= (2 * k < nv ? 0x0000FFFFu : 0u) | (2 * k + 1 < nv ? 0xFFFF0000u : 0u);
  return u32x4{w[0], w[1], w[2], w[3]};
}

// Split-KV attention for kv head g, split j over positions [t0, t1) of T = pos + 1, for the grp
// query heads of the group (grp <= 16); the partial (m, l, acc[hd]) of each head goes to the
// workspace, and the group's COMBINE task merges the splits into o.
// Partial record per (split, head): m, l, two pad words, acc[hd] (hd + 4 floats).
// On the matrix cores: the split is cut into 32-position groups (chunks are whole groups, at most
// 16) and each wave takes one or two of them.  Scores are two 16 x 16 products per 32-dim slice,
// K rows (A, from the [pos][hd] cache) times q (B, heads as columns); the A rows are the positions
// in the order p0 + 8 (r / 4) + r % 4 (block 0) and + 4 (block 1), so that lane l ends up holding
// the scores of positions p0 + 8 (l / 16) .. + 8 of head l % 16, which is exactly its B operand of
// P.V.  P.V is V^T (A: 8 positions of one dim per lane) times P, one 16 x 16 product per 16 dims
// (V is stored in blocks of 32 positions, [pos / 32][hd][pos % 32], so one wave instruction reads
// 1 KiB of contiguous cache).  q and P enter as 16-bit hi + lo pairs (two products each), so the
// result keeps about fp32 precision.  K/V rows are loaded from the cache before the dependency
// wait; the current position (written this step) comes from its tagged copy, which wave 0 stages
// with q.  The wave's softmax (max and sum across the four lanes of a head column with
// column_max / column_sum) runs on the 8 scores a lane holds; the eight waves' (max, sum, acc)
// are then merged in LDS with the usual rescaling, exactly as the splits are merged by the
// combine.
template <int WDT, int KVDT, int HD, int NGW, bool G2LDS, bool COH>
__device__ __forceinline__ void task_attn(const KParams& P, const pmk_task& t, int ti, const StepCtx& sc, float* lds,
                                          int cu) {
  constexpr int KES = KVDT == WFP8 ? 1 : 2;
  constexpr bool X3 = weight_is_int(WDT) && KVDT == WBF16;  // q and P in three bf16 terms (split16x3)
  constexpr int ROWB = HD * KES;      // K row bytes
  constexpr int NC = HD / 32;         // 32-dim slices of the score product
  constexpr int NT = HD / 16;         // 16-dim tiles of P.V
  constexpr int PSTR = HD + 4;        // partial record: m, l, 2 pad, acc[hd] (16-byte aligned)
  constexpr uint32_t kOut = (uint32_t)kMaxTileBytes;
  const int l = t.layer, g = t.a0, split = t.a1, S = P.S, grp = P.grp;
  const int T = sc.pos + 1;
  const int chunk = ((T + S - 1) / S + 31) & ~31;
  const int t0 = min(T, split * chunk), t1 = min(T, t0 + chunk);
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int col = lane & 15, grp4 = lane >> 4;  // MFMA column / row-group of this lane
  const int64_t head = (int64_t)l * P.nkv + g;
  const __amdgpu_buffer_rsrc_t kr = __builtin_amdgcn_make_buffer_rsrc(
      P.kc + head * P.seqcap * ROWB, (short)0, (int)((int64_t)P.seqcap * ROWB), 0x00020000);
  const __amdgpu_buffer_rsrc_t vr = __builtin_amdgcn_make_buffer_rsrc(
      P.vc + head * HD * P.seqcap * KES, (short)0, (int)((int64_t)HD * P.seqcap * KES), 0x00020000);
  float* qs = lds;                      // [grp][HD]
  float* red = qs + grp * HD;           // [kWaves][grp][HD] per-wave P.V partials
  float* wml = red + kWaves * grp * HD; // [kWaves][grp][2] per-wave (max, sum)
  uint32_t* kvs = reinterpret_cast<uint32_t*>(wml + kWaves * grp * 2);  // [2][HD] current K row, V column
  float kscale = 1.f, vscale = 1.f;
  if constexpr (KVDT == WFP8) {
    kscale = P.kv_scale[head * 2];
    vscale = P.kv_scale[head * 2 + 1];
  }
  // Wave w takes the 32-position groups v, v + 8, ... (NGW of them) with v = (w + 7) mod 8: wave 0
  // takes the last group of each round (used only when the split needs it), so its dependency
  // poll is normally not queued behind K/V loads, and it alone stages q.  The first group's rows
  // of past positions are loaded before the dependency wait; a second group reuses the same
  // registers, its K rows loaded once the first group's scores are done and its V^T rows once the
  // first group's P.V is, with an online rescale of the wave's (max, sum, acc).
  const int wv = __builtin_amdgcn_readfirstlane((wave + kWaves - 1) % kWaves);
  // the current position's row is not read from the cache (it is written in this step): zeros,
  // replaced from the tagged copy before use
  auto koff = [&](int p, int c) {
    return p < t1 && p != sc.pos ? (uint32_t)(p * ROWB + (32 * c + 8 * grp4) * KES) : kOut;
  };
  auto voff = [&](int pv, int tt) {
    return pv < t1 ? (uint32_t)((((pv >> 5) * HD + 16 * tt + col) * 32 + (pv & 31)) * KES) : kOut;
  };
  // K rows of this lane (score blocks 0 and 1) and V^T positions of this lane, for group k
  auto pk_of = [&](int k) { return t0 + 32 * (wv + kWaves * k) + 8 * (col >> 2) + (col & 3); };
  auto pv_of = [&](int k) { return t0 + 32 * (wv + kWaves * k) + 8 * grp4; };
  u32x4 ka[NC], kb[NC], vt[NT];
  // K rows and V^T positions of group k from the cache; the current position's slot (written
  // this step) is replaced from the tagged copy staged in LDS before it is used
  auto load_k = [&](int k) {
    const int pk0 = pk_of(k);
#pragma unroll
    for (int c = 0; c < NC; ++c) {
      ka[c] = kv_load8<KVDT, COH>(kr, koff(pk0, c));
      kb[c] = kv_load8<KVDT, COH>(kr, koff(pk0 + 4, c));
    }
  };
  auto load_v = [&](int k) {
    const int pv = pv_of(k);
#pragma unroll
    for (int tt = 0; tt < NT; ++tt) vt[tt] = kv_load8<KVDT, COH>(vr, voff(pv, tt));
  };
  auto patch_k = [&](int k) {
    const int pk0 = pk_of(k);
    const bool c0 = pk0 == sc.pos, c1 = pk0 + 4 == sc.pos;
    if (c0 || c1) {
#pragma unroll
      for (int c = 0; c < NC; ++c) {
        const uint32_t* e = kvs + 32 * c + 8 * grp4;
        const u32x4 v = {e[0] | (e[1] << 16), e[2] | (e[3] << 16), e[4] | (e[5] << 16), e[6] | (e[7] << 16)};
        if (c0) ka[c] = v;
        else kb[c] = v;
      }
    }
  };
  auto patch_v = [&](int k) {
    const int pv = pv_of(k);
    if (pv <= sc.pos && sc.pos < pv + 8) {
      const int e = sc.pos - pv, wi = e >> 1;
      const uint32_t keep = (e & 1) ? 0x0000FFFFu : 0xFFFF0000u;
      const int sh = (e & 1) ? 16 : 0;
#pragma unroll
      for (int tt = 0; tt < NT; ++tt) {
        const uint32_t b = kvs[HD + 16 * tt + col] << sh;
        vt[tt].x = wi == 0 ? (vt[tt].x & keep) | b : vt[tt].x;
        vt[tt].y = wi == 1 ? (vt[tt].y & keep) | b : vt[tt].y;
        vt[tt].z = wi == 2 ? (vt[tt].z & keep) | b : vt[tt].z;
        vt[tt].w = wi == 3 ? (vt[tt].w & keep) | b : vt[tt].w;
      }
    }
  };
  // group 0: before the dependency wait
  load_k(0);
  load_v(0);
  // A second group (splits of more than 8 groups), in the persistent kernel when LDS has room: its
  // K rows and V block (contiguous in the cache) are copied to this wave's LDS buffer before the
  // wait too, so its loads are not issued only after the first group's products (two exposed
  // memory round trips); per-op kernels load them into registers as below.  Rows past the
  // split's end are zeroed as the buffer-resource path does.
  constexpr int G2K = 32 * ROWB, G2B = G2K + HD * 32 * KES;  // bytes: K rows, + V block
  constexpr bool g2_lds = NGW == 2 && G2LDS;  // the caller checked: persistent kernel, buffers present
  const int p1 = t0 + 32 * (wv + kWaves);  // the second group's first position
  const uint8_t* g2 = reinterpret_cast<const uint8_t*>(lds + (P.attn_g2_off < 0 ? 0 : P.attn_g2_off)) + wave * G2B;
  if (g2_lds && p1 < t1) {
    constexpr int kPol = COH ? 16 : 2;  // sc1 : nt (as kv_load8)
#pragma unroll
    for (int u = 0; u < G2K / 1024; ++u)
      __builtin_amdgcn_raw_ptr_buffer_load_lds(kr, (lds_void*)(g2 + u * 1024), 16,
                                               (uint32_t)(p1 * ROWB + u * 1024 + lane * 16), 0, 0, kPol);
#pragma unroll
    for (int u = 0; u < (G2B - G2K) / 1024; ++u)
      __builtin_amdgcn_raw_ptr_buffer_load_lds(vr, (lds_void*)(g2 + G2K + u * 1024), 16,
                                               (uint32_t)((p1 >> 5) * HD * 32 * KES + u * 1024 + lane * 16), 0,
                                               0, kPol);
  }
  auto lds8 = [&](int off) -> u32x4 {  // 8 elements of the second group's buffer as 16-bit operands
    if constexpr (KVDT == WFP8) return fp8x8_bf16(*reinterpret_cast<const u32x2*>(g2 + off));
    else return *reinterpret_cast<const u32x4*>(g2 + off);
  };
  auto lds_group2 = [&]() {
    const int pk0 = pk_of(1), pv = pv_of(1);
#pragma unroll
    for (int c = 0; c < NC; ++c) {
      ka[c] = pk0 < t1 ? lds8((pk0 - p1) * ROWB + (32 * c + 8 * grp4) * KES) : u32x4{0u, 0u, 0u, 0u};
      kb[c] = pk0 + 4 < t1 ? lds8((pk0 + 4 - p1) * ROWB + (32 * c + 8 * grp4) * KES) : u32x4{0u, 0u, 0u, 0u};
    }
#pragma unroll
    for (int tt = 0; tt < NT; ++tt)
      vt[tt] = pv < t1 ? lds8(G2K + ((16 * tt + col) * 32 + (pv & 31)) * KES) : u32x4{0u, 0u, 0u, 0u};
  };
  // Wave 0 stages q of the group's heads and, in the split that holds the current position, that
  // position's K row and V column (16-bit operand bits), all tagged with the step.  In flags mode
  // the tagged reads are the wait; otherwise the counter wait comes first.
  const bool poll = polls_tags(P, sc);
  if (!poll) maybe_wait(P, t, sc, cu, ti);
  if (wave == 0) {
    constexpr int QB = 4, CB = HD / 64;  // 16-byte pairs per lane per round: q; current K and V
    const uint32_t want = (uint32_t)(sc.e + 1);
    const int nq = grp * HD;
    const bool has_cur = t0 <= sc.pos && sc.pos < t1;
    const __amdgpu_buffer_rsrc_t qr = coherent_rsrc(P.q + (int64_t)l * P.qdim + (int64_t)g * grp * HD, nq * 8);
    const __amdgpu_buffer_rsrc_t cr = coherent_rsrc(P.kvcur + head * 2 * HD, 2 * HD * 8);
    for (int base = 0; base < nq; base += QB * 128) {
      const bool first = base == 0;
      u32x4 v[QB], c[CB];
      bool okv[QB], okc[CB];
#pragma unroll
      for (int k = 0; k < QB; ++k) okv[k] = false;
#pragma unroll
      for (int k = 0; k < CB; ++k) okc[k] = false;
      int64_t spins = 0;
      while (true) {
        __atomic_signal_fence(__ATOMIC_SEQ_CST);  // each retry reads memory again
#pragma unroll
        for (int k = 0; k < QB; ++k) {
          const int i = base + (k * 64 + lane) * 2;
          if (!okv[k]) v[k] = i < nq ? ldc16(qr, (uint32_t)i * 8) : u32x4{0u, want, 0u, want};
        }
#pragma unroll
        for (int k = 0; k < CB; ++k)
          if (!okc[k]) c[k] = first && has_cur ? ldc16(cr, (uint32_t)(k * 64 + lane) * 16) : u32x4{0u, want, 0u, want};
        bool all = true;
#pragma unroll
        for (int k = 0; k < QB; ++k) {
          okv[k] = okv[k] || sc.per_op || (v[k].y == want && v[k].w == want);
          all = all && okv[k];
        }
#pragma unroll
        for (int k = 0; k < CB; ++k) {
          okc[k] = okc[k] || sc.per_op || (c[k].y == want && c[k].w == want);
          all = all && okc[k];
        }
        if (__ballot(!all) == 0ull) break;
        if (ldc(&P.ctrl[CTRL_ABORT]) != 0u) break;
        if (++spins > P.spin_limit) {
          report_error(P.ctrl, PMK_ERR_TIMEOUT, cu, ti, -1, want, v[0].y);
          break;
        }
      }
#pragma unroll
      for (int k = 0; k < QB; ++k) {
        const int i = base + (k * 64 + lane) * 2;
        if (i < nq) *reinterpret_cast<float2*>(qs + i) = make_float2(__uint_as_float(v[k].x), __uint_as_float(v[k].z));
      }
      if (first && has_cur) {
#pragma unroll
        for (int k = 0; k < CB; ++k) {
          const int i = (k * 64 + lane) * 2;
          kvs[i] = c[k].x;
          kvs[i + 1] = c[k].z;
        }
      }
    }
    if (poll) trace_mark(P, sc.s, ti, 1, __builtin_amdgcn_s_memrealtime());
  }
  __syncthreads();
  const float qk_scale = kscale * P.attn_scale;
  float m = -INFINITY, sum = 0.f;
  f32x4 acc[NT];
#pragma unroll
  for (int tt = 0; tt < NT; ++tt) acc[tt] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
  for (int k = 0; k < NGW; ++k) {
    if (t0 + 32 * (wv + kWaves * k) >= t1) break;  // wave-uniform: no positions left
    const int pv = pv_of(k);
    if (k > 0 && g2_lds) lds_group2();
    patch_k(k);
    // positions past the split's end (the last V^T group may straddle it) contribute nothing
    if (pv < t1 && pv + 8 > t1) {
#pragma unroll
      for (int tt = 0; tt < NT; ++tt) vt[tt] = keep_first(vt[tt], t1 - pv);
    }
    // ---- scores: blocks 0 and 1 of 16 positions x 16 head columns ----
    f32x4 s0 = {0.f, 0.f, 0.f, 0.f}, s1 = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int c = 0; c < NC; ++c) {
      float qv[8];
#pragma unroll
      for (int e = 0; e < 8; ++e) qv[e] = col < grp ? qs[col * HD + 32 * c + 8 * grp4 + e] : 0.f;
      u32x4 qh, ql;
      if constexpr (X3) {
        u32x4 qm;
        split16x3(qv, qh, qm, ql);
        s0 = mfma16<KVDT>(ka[c], qm, s0);
        s1 = mfma16<KVDT>(kb[c], qm, s1);
      } else {
        split16<KVDT>(qv, qh, ql);
      }
      s0 = mfma16<KVDT>(ka[c], qh, s0);
      s0 = mfma16<KVDT>(ka[c], ql, s0);
      s1 = mfma16<KVDT>(kb[c], qh, s1);
      s1 = mfma16<KVDT>(kb[c], ql, s1);
    }
    const bool next = k + 1 < NGW && t0 + 32 * (wv + kWaves * (k + 1)) < t1;
    if (next && !g2_lds) load_k(k + 1);
    // ---- softmax: the lane holds positions pv + 0..7 of head column col ----
    float sc8[8];
    float mk = -INFINITY;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      sc8[i] = pv + i < t1 ? s0[i] * qk_scale : -INFINITY;
      sc8[4 + i] = pv + 4 + i < t1 ? s1[i] * qk_scale : -INFINITY;
      mk = fmaxf(mk, fmaxf(sc8[i], sc8[4 + i]));
    }
    const float mn = fmaxf(m, column_max<16>(mk));
    float ps = 0.f;
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      sc8[i] = mn == -INFINITY ? 0.f : expf(sc8[i] - mn);
      ps += sc8[i];
    }
    ps = column_sum<16>(ps);
    if (k > 0) {
      const float alpha = m == -INFINITY ? 0.f : expf(m - mn);
      sum *= alpha;
#pragma unroll
      for (int tt = 0; tt < NT; ++tt)
#pragma unroll
        for (int i = 0; i < 4; ++i) acc[tt][i] *= alpha;
    }
    sum += ps;
    m = mn;
    // ---- P.V: 16 dims x 16 head columns per tile ----
    patch_v(k);
    u32x4 ph, pl;
    if constexpr (X3) {
      u32x4 pm;
      split16x3(sc8, ph, pm, pl);
#pragma unroll
      for (int tt = 0; tt < NT; ++tt) acc[tt] = mfma16<KVDT>(vt[tt], pm, acc[tt]);
    } else {
      split16<KVDT>(sc8, ph, pl);
    }
#pragma unroll
    for (int tt = 0; tt < NT; ++tt) {
      acc[tt] = mfma16<KVDT>(vt[tt], ph, acc[tt]);
      acc[tt] = mfma16<KVDT>(vt[tt], pl, acc[tt]);
    }
    if (next && !g2_lds) load_v(k + 1);
  }
  if (col < grp) {
    float* dst = red + ((int64_t)wave * grp + col) * HD + 4 * grp4;
#pragma unroll
    for (int tt = 0; tt < NT; ++tt)
      *reinterpret_cast<float4*>(dst + 16 * tt) =
          make_float4(acc[tt][0] * vscale, acc[tt][1] * vscale, acc[tt][2] * vscale, acc[tt][3] * vscale);
    if (grp4 == 0) {
      wml[(wave * grp + col) * 2] = m;
      wml[(wave * grp + col) * 2 + 1] = sum;
    }
  }
  __syncthreads();
  mark(P, sc, ti, 4);
  // ---- merge the eight waves into this split's partial ----
  float* partp = P.part + ((((int64_t)l * P.nkv + g) * S + split) * grp) * PSTR;
  for (int i = tid; i < grp * HD; i += kThreads) {
    const int j = i / HD, d = i % HD;
    float M = -INFINITY;
#pragma unroll
    for (int w = 0; w < kWaves; ++w) M = fmaxf(M, wml[(w * grp + j) * 2]);
    float o = 0.f, lsum = 0.f;
#pragma unroll
    for (int w = 0; w < kWaves; ++w) {
      const float mwv = wml[(w * grp + j) * 2];
      const float sc_w = mwv == -INFINITY ? 0.f : expf(mwv - M);
      o = fmaf(sc_w, red[((int64_t)w * grp + j) * HD + d], o);
      lsum = fmaf(sc_w, wml[(w * grp + j) * 2 + 1], lsum);
    }
    stc(partp + (int64_t)j * PSTR + 4 + d, o);
    if (d == 0) {
      stc(partp + (int64_t)j * PSTR, M);
      stc(partp + (int64_t)j * PSTR + 1, lsum);
    }
  }
  mark(P, sc, ti, 5);
  block_signal(P, t.signal_ctr, t.signal_slot, sc.e);
}

// Combine of the attention splits of kv head g for the group's q heads [j0, j1) (a1 = j0 | j1 << 8;
// a group is split over several combines when one would read too many partials): waits for all
// S partials of the head group, then o = sum_s exp(m_s - M) acc_s / sum_s exp(m_s - M) l_s per
// head, M = max_s m_s.
template <int HD>
__device__ __forceinline__ void task_combine(const KParams& P, const pmk_task& t, int ti, const StepCtx& sc, int cu) {
  constexpr int PSTR = HD + 4;  // partial record: m, l, 2 pad, acc[hd]
  const int l = t.layer, g = t.a0, S = P.S, grp = P.grp, tid = threadIdx.x;
  maybe_wait(P, t, sc, cu, ti);
  // In registers: a quad of threads owns four consecutive dims of one head; its threads take every
  // fourth split and merge them online in batches of coherent loads (header m, l and the four acc
  // values), then the quad merges its four (max, sum, acc) with DPP and each thread stores one dim.
  {
    constexpr int QPH = HD / 4;  // dim quads per head
    constexpr int CB = 8;        // splits per thread per batch
    constexpr uint32_t kOut = (uint32_t)kMaxTileBytes;
    const float* pg = P.part + (((int64_t)l * P.nkv + g) * S) * grp * PSTR;
    const __amdgpu_buffer_rsrc_t pr = coherent_rsrc(pg, (uint32_t)((int64_t)S * grp * PSTR * 4));
    unsigned long long* o = P.o + (int64_t)l * P.qdim + (int64_t)g * grp * HD;
    const int r = tid & 3;
    const int j0 = t.a1 & 255, j1 = t.a1 >> 8;  // this task's q heads of the group
    for (int qd = tid >> 2; qd < (j1 - j0) * QPH; qd += kThreads / 4) {
      const int j = j0 + qd / QPH, d0 = (qd % QPH) * 4;
      float M = -INFINITY, den = 0.f, a0 = 0.f, a1 = 0.f, a2 = 0.f, a3 = 0.f;
      for (int sb = 0; sb < S; sb += 4 * CB) {
        u32x4 hv[CB], av[CB];
#pragma unroll
        for (int k = 0; k < CB; ++k) {
          const int s2 = sb + 4 * k + r;
          const uint32_t off = s2 < S ? (uint32_t)((s2 * grp + j) * PSTR) * 4u : kOut;
          hv[k] = ldc16(pr, off);
          av[k] = ldc16(pr, off + (uint32_t)(4 + d0) * 4u);
        }
        float mb = -INFINITY;
#pragma unroll
        for (int k = 0; k < CB; ++k)
          if (sb + 4 * k + r < S) mb = fmaxf(mb, __uint_as_float(hv[k].x));
        const float Mn = fmaxf(M, mb);
        if (Mn != -INFINITY) {
          const float f = M == -INFINITY ? 0.f : expf(M - Mn);
          den *= f; a0 *= f; a1 *= f; a2 *= f; a3 *= f;
#pragma unroll
          for (int k = 0; k < CB; ++k) {
            const float m = __uint_as_float(hv[k].x);
            if (sb + 4 * k + r < S && m != -INFINITY) {
              const float w = expf(m - Mn);
              den = fmaf(w, __uint_as_float(hv[k].y), den);
              a0 = fmaf(w, __uint_as_float(av[k].x), a0);
              a1 = fmaf(w, __uint_as_float(av[k].y), a1);
              a2 = fmaf(w, __uint_as_float(av[k].z), a2);
              a3 = fmaf(w, __uint_as_float(av[k].w), a3);
            }
          }
          M = Mn;
        }
      }
      const float Mq = quad_max(M);  // finite: every head has at least the current position
      const float f = M == -INFINITY ? 0.f : expf(M - Mq);
      den = quad_sum(den * f);
      a0 = quad_sum(a0 * f);
      a1 = quad_sum(a1 * f);
      a2 = quad_sum(a2 * f);
      a3 = quad_sum(a3 * f);
      const float v = r == 0 ? a0 : r == 1 ? a1 : r == 2 ? a2 : a3;
      stc(o + j * HD + d0 + r, tagged(v / den, sc.e));
    }
  }
  mark(P, sc, ti, 4);
  // With flags, the O projection polls the tags of o itself (no drain, no flag); counters keep
  // the drained signal.
  if (!polls_tags(P, sc)) block_signal(P, t.signal_ctr, t.signal_slot, sc.e);
}

// O projection + residual: xm[r] = x[r] + Wo[r].o  (residual rows staged in LDS with the input)
template <int WDT>
__device__ __forceinline__ void task_oproj(const KParams& P, const pmk_task& t, int ti, const StepCtx& sc, float* lds,
                                           int cu, bool tile_copied = false) {
  constexpr int EDT = WFmt<WDT>::EDT;
  const int l = t.layer, K = P.qdim, R = t.a1 - t.a0;
  // compact LDS layout (o, residual rows, partial sums, results) below the LDS tile area
  float* xs = lds;
  float* res = lds + P.o_epi_off;
  float* yp = lds + P.o_yp_off;
  float* y = lds + P.o_y_off;
  const uint8_t* W = P.wbase + (int64_t)l * P.layer_bytes + P.off_o;
  // flags mode: the wait on the combines is the tag poll of o below
  const bool poll_o = polls_tags(P, sc);
  auto sync = [&]() {
    if (!poll_o) maybe_wait(P, t, sc, cu, ti);
    const int tok = l == 0 ? input_token(P, sc) : 0;
    float rv = 0.f;  // first kThreads residual rows ride with the input loads
    if ((int)threadIdx.x < R)
      rv = l == 0 ? dec16<EDT>(P.embed[(int64_t)tok * P.H + t.a0 + threadIdx.x])
                  : ld_tagged(P, P.x + (int64_t)l * P.H + t.a0 + threadIdx.x, sc.e, !sc.per_op, cu, ti);
    for (int i = threadIdx.x + kThreads; i < R; i += kThreads)
      res[i] = l == 0 ? dec16<EDT>(P.embed[(int64_t)tok * P.H + t.a0 + i])
                      : ld_tagged(P, P.x + (int64_t)l * P.H + t.a0 + i, sc.e, !sc.per_op, cu, ti);
    stage_tagged<false, WFmt<WDT>::H16>(P, P.o + (int64_t)l * K, K, pad_len(K, WFmt<WDT>::EPL), xs, sc.e, !sc.per_op,
                                        cu, ti);
    if ((int)threadIdx.x < R) res[threadIdx.x] = rv;
    __syncthreads();
    if (poll_o) trace_mark(P, sc.s, ti, 1, __builtin_amdgcn_s_memrealtime());
    mark(P, sc, ti, 4);
  };
  const int nbc = (K + 127) / 128;
  using ST = typename WFmt<WDT>::ST;
  const ST* const so = scale_rows<WDT>(P, l, 3);
  auto srow = [=](int r) -> const ST* { return scale_row<WDT>(so, r, nbc); };
  if (oproj_tile_in_lds(P, t, sc, (K / WFmt<WDT>::EPL + 63) >> 6)) {
    if (!tile_copied) tile_to_lds<WDT>(W, K, t.a0, t.a1, lds + P.pf_off, kOprojRowCost);
    gemv_rows_lds<WDT>(K, t.a0, t.a1, xs, lds + P.pf_off, yp, y, sync, srow, kOprojRowCost);
  } else
    gemv_rows<WDT>(W, K, t.a0, t.a1, xs, yp, y, P.prefetch != 0, sync, srow, kOprojRowCost);
  mark(P, sc, ti, 5);
  for (int i = threadIdx.x; i < R; i += kThreads) stc(P.xm + (int64_t)l * P.H + t.a0 + i, tagged(res[i] + y[i], sc.e));
  if (!polls_tags(P, sc)) block_signal(P, t.signal_ctr, t.signal_slot, sc.e);
}

// RMSNorm(xm) -> interleaved gate/up rows [a0, a1) -> h[n] = silu(gate_n) * up_n
template <int WDT>
__device__ __forceinline__ void task_gateup(const KParams& P, const pmk_task& t, int ti, const StepCtx& sc, float* lds,
                                            int cu) {
  constexpr bool H16 = WFmt<WDT>::H16;
  const int l = t.layer, H = P.H, pad = pad_len(H, WFmt<WDT>::EPL);
  float* xs = lds;
  float* red = lds + P.xs_floats;
  float* yp = lds + P.yp_off;
  float* y = lds + P.y_off;
  const uint8_t* W = P.wbase + (int64_t)l * P.layer_bytes + P.off_gu;
  auto sync = [&]() {
    const bool poll = polls_tags(P, sc);
    if (!poll) maybe_wait(P, t, sc, cu, ti);
    stage_rmsnorm_tagged<H16>(P, P.xm + (int64_t)l * H, P.gains + (int64_t)l * 2 * H + H, H, pad, xs, red, sc.e,
                              !sc.per_op, cu, ti, lds + P.gs_off);
    if constexpr (H16) norm_to_h16(xs, lds + P.gs_off, H, pad, red, P.eps, lds + P.xh_off);
    if (poll) trace_mark(P, sc.s, ti, 1, __builtin_amdgcn_s_memrealtime());
    mark(P, sc, ti, 4);
  };
  const int nbc = (H + 127) / 128;
  using ST = typename WFmt<WDT>::ST;
  const ST* const sg = scale_rows<WDT>(P, l, 4);
  const ST* const su = scale_rows<WDT>(P, l, 5);
  auto srow = [=](int r) -> const ST* { return scale_row<WDT>((r & 1) ? su : sg, r >> 1, nbc); };
  gemv_rows<WDT>(W, H, t.a0, t.a1, H16 ? lds + P.xh_off : xs, yp, y, P.prefetch != 0, sync, srow);
  mark(P, sc, ti, 5);
  const int npairs = (t.a1 - t.a0) >> 1;
  const float rn = H16 ? 1.0f : rms_factor(red, H, P.eps);
  for (int p = threadIdx.x; p < npairs; p += kThreads) {
    const float gte = y[2 * p] * rn, up = y[2 * p + 1] * rn;
    stc(P.h + (int64_t)l * P.F + (t.a0 >> 1) + p, gte / (1.0f + expf(-gte)) * up);
  }
  block_signal(P, t.signal_ctr, t.signal_slot, sc.e);
}

// down projection + residual: x[l+1][r] = xm[r] + Wd[r].h  (residual rows staged in LDS)
template <int WDT>
__device__ __forceinline__ void task_down(const KParams& P, const pmk_task& t, int ti, const StepCtx& sc, float* lds,
                                          int cu) {
  const int l = t.layer, K = P.F, R = t.a1 - t.a0;
  float* xs = lds;
  float* res = lds + P.epi_off;
  float* yp = lds + P.yp_off;
  float* y = lds + P.y_off;
  const uint8_t* W = P.wbase + (int64_t)l * P.layer_bytes + P.off_d;
  auto sync = [&]() {
    maybe_wait(P, t, sc, cu, ti);
    float rv = 0.f;
    if ((int)threadIdx.x < R) rv = ld_tagged(P, P.xm + (int64_t)l * P.H + t.a0 + threadIdx.x, sc.e, !sc.per_op, cu, ti);
    for (int i = threadIdx.x + kThreads; i < R; i += kThreads)
      res[i] = ld_tagged(P, P.xm + (int64_t)l * P.H + t.a0 + i, sc.e, !sc.per_op, cu, ti);
    load_vector<WFmt<WDT>::H16>(P.h + (int64_t)l * K, K, pad_len(K, WFmt<WDT>::EPL), xs);
    if ((int)threadIdx.x < R) res[threadIdx.x] = rv;
    __syncthreads();
    mark(P, sc, ti, 4);
  };
  const int nbc = (K + 127) / 128;
  using ST = typename WFmt<WDT>::ST;
  const ST* const sd = scale_rows<WDT>(P, l, 6);
  auto srow = [=](int r) -> const ST* { return scale_row<WDT>(sd, r, nbc); };
  gemv_rows<WDT>(W, K, t.a0, t.a1, xs, yp, y, P.prefetch != 0, sync, srow);
  mark(P, sc, ti, 5);
  for (int i = threadIdx.x; i < R; i += kThreads)
    stc(P.x + (int64_t)(l + 1) * P.H + t.a0 + i, tagged(res[i] + y[i], sc.e));
  if (!polls_tags(P, sc)) block_signal(P, t.signal_ctr, t.signal_slot, sc.e);
}

// final RMSNorm + LM-head rows [a0, a1); tile argmax folded into the step's 64-bit key
// (orderable value in the high word, inverted index in the low word: max value, lowest index)
__device__ __forceinline__ uint32_t orderable(float v) {
  const uint32_t u = __float_as_uint(v);
  return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}

__device__ __forceinline__ unsigned long long wave_max_u64(unsigned long long k) {
  for (int o = 32; o > 0; o >>= 1) {
    const unsigned long long other = ((unsigned long long)(uint32_t)__shfl_xor((int)(k >> 32), o) << 32) |
                                     (uint32_t)__shfl_xor((int)(uint32_t)k, o);
    k = other > k ? other : k;
  }
  return k;
}

template <int WDT>
__device__ __forceinline__ void task_lmhead(const KParams& P, const pmk_task& t, int ti, const StepCtx& sc, float* lds,
                                            int cu) {
  constexpr bool H16 = WFmt<WDT>::H16;
  const int H = P.H, R = t.a1 - t.a0, pad = pad_len(H, WFmt<WDT>::EPL);
  float* xs = lds;
  float* red = lds + P.xs_floats;
  float* yp = lds + P.yp_off;
  float* y = lds + P.y_off;
  float* out_logits = P.call->out_logits;
  auto sync = [&]() {
    const bool poll = polls_tags(P, sc);
    if (!poll) maybe_wait(P, t, sc, cu, ti);
    stage_rmsnorm_tagged<H16>(P, P.x + (int64_t)P.L * H, P.final_gain, H, pad, xs, red, sc.e,
                              !sc.per_op, cu, ti, lds + P.gs_off);
    if constexpr (H16) norm_to_h16(xs, lds + P.gs_off, H, pad, red, P.eps, lds + P.xh_off);
    if (poll) trace_mark(P, sc.s, ti, 1, __builtin_amdgcn_s_memrealtime());
    mark(P, sc, ti, 4);
  };
  const int nbc = (H + 127) / 128;
  using ST = typename WFmt<WDT>::ST;
  const ST* const sl = reinterpret_cast<const ST*>(P.sc_lm);
  auto srow = [=](int r) -> const ST* { return scale_row<WDT>(sl, r, nbc); };
  gemv_rows<WDT>(P.lm, H, t.a0, t.a1, H16 ? lds + P.xh_off : xs, yp, y, P.prefetch != 0, sync, srow, kLmheadRowCost);
  mark(P, sc, ti, 5);
  const float rn = H16 ? 1.0f : rms_factor(red, H, P.eps);
  unsigned long long key = 0ull;
  bool nan_seen = false;
  for (int i = threadIdx.x; i < R; i += kThreads) {
    const float v = y[i] * rn;
    if (v != v) nan_seen = true;
    const unsigned long long k = ((unsigned long long)orderable(v) << 32) | (0xFFFFFFFFu - (uint32_t)(t.a0 + i));
    key = k > key ? k : key;
    if (out_logits) out_logits[(int64_t)sc.s * P.V + t.a0 + i] = v;
  }
  key = wave_max_u64(key);
  unsigned long long* kred = reinterpret_cast<unsigned long long*>(red + 16);
  const int wave = threadIdx.x >> 6;
  if ((threadIdx.x & 63) == 0) kred[wave] = key;
  if (nan_seen) report_error(P.ctrl, PMK_ERR_NAN, cu, ti, -1, 0, 0);
  __syncthreads();
  if (threadIdx.x == 0) {
    unsigned long long k = 0;
    for (int w = 0; w < kWaves; ++w) k = kred[w] > k ? kred[w] : k;
    __hip_atomic_fetch_max(&P.keys[sc.s], k, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  }
  block_signal(P, t.signal_ctr, t.signal_slot, sc.e);
}

// greedy token of the step: output, next-input slot; per-op kernels also advance the step state
__device__ __forceinline__ void task_token(const KParams& P, const pmk_task& t, int ti, const StepCtx& sc, float* lds, int cu) {
  maybe_wait(P, t, sc, cu, ti);
  if (threadIdx.x == 0) {
    CallParams* cp = P.call;
    const unsigned long long key = ldc(&P.keys[sc.s]);
    int tok = key_token(key);
    const uint32_t ov = (uint32_t)(key >> 32);
    const float best = __uint_as_float((ov & 0x80000000u) ? (ov & 0x7fffffffu) : ~ov);
    if (key == 0ull || best != best) {
      report_error(P.ctrl, PMK_ERR_NAN, cu, ti, -1, 0, 0);
      tok = 0;
    }
    if (cp->out_tokens) cp->out_tokens[sc.s] = tok;
    stc(&P.ctrl[CTRL_TOKEN], (uint32_t)tok);
    if (sc.per_op) {
      const bool stop = cp->eos >= 0 && tok == cp->eos && cp->forced == nullptr;
      stc(&P.ctrl[CTRL_POS], (uint32_t)(sc.pos + 1));
      stc(&P.ctrl[CTRL_EPOCH], (uint32_t)(sc.e + 1));
      stc(&P.ctrl[CTRL_STEP], (uint32_t)(sc.s + 1));
      if (stop) stc(&P.ctrl[CTRL_STOPPED], 1u);
      if (cp->n_done) cp->n_done[0] = sc.s + 1;
    }
  }
  (void)lds;
  (void)t;
}

template <int WDT, int KVDT, int NGW, bool G2LDS, bool COH>
__device__ __forceinline__ void attn_hd(const KParams& P, const pmk_task& t, int ti, const StepCtx& sc, float* lds,
                                        int cu) {
  if (P.hd == 128) task_attn<WDT, KVDT, 128, NGW, G2LDS, COH>(P, t, ti, sc, lds, cu);
  else task_attn<WDT, KVDT, 64, NGW, G2LDS, COH>(P, t, ti, sc, lds, cu);
}

// An O-projection task that follows a COMBINE on the same queue has its LDS tile copied by the
// combine, before the combine's wait: the combine uses no LDS, and otherwise the copy would start
// only once the combine ends, which put those queues' O projections last on the chip's critical path.
// Both tasks evaluate the same predicate on their own (no state is carried from one task to the
// next): the combine to issue the copy, the O projection to skip its own.
template <int WDT>
__device__ __forceinline__ bool combine_copies_tile(const KParams& P, const StepCtx& sc, const pmk_task& o, int layer) {
  const int nsl = (P.qdim / WFmt<WDT>::EPL + 63) >> 6;
  return P.o_copy && o.op == PMK_OP_OPROJ && o.layer == layer && oproj_tile_in_lds(P, o, sc, nsl);
}

template <int WDT, int KVDT, bool OCOPY = false>
__device__ __forceinline__ void run_task(const KParams& P, const pmk_task& t, int ti, const StepCtx& sc, float* lds,
                                         int cu, int qi = -1, int q0 = 0, int q1 = 0) {
  switch (t.op) {
    case PMK_OP_QKV: task_qkv<WDT, KVDT>(P, t, ti, sc, lds, cu); break;
    case PMK_OP_ATTN: {
      // splits longer than 8 groups of 32 positions give each wave a second group; a split that
      // reaches the 32-position block of this launch's first position reads coherently
      const int T = sc.pos + 1;
      const int chunk = ((T + P.S - 1) / P.S + 31) & ~31;
      const bool coh = min(T, (t.a1 + 1) * chunk) > (sc.pos0 & ~31);
      if (chunk / 32 > kWaves) {
        if (!sc.per_op && P.attn_g2_off >= 0) {
          if (coh) attn_hd<WDT, KVDT, 2, true, true>(P, t, ti, sc, lds, cu);
          else attn_hd<WDT, KVDT, 2, true, false>(P, t, ti, sc, lds, cu);
        } else {
          if (coh) attn_hd<WDT, KVDT, 2, false, true>(P, t, ti, sc, lds, cu);
          else attn_hd<WDT, KVDT, 2, false, false>(P, t, ti, sc, lds, cu);
        }
      } else {
        if (coh) attn_hd<WDT, KVDT, 1, false, true>(P, t, ti, sc, lds, cu);
        else attn_hd<WDT, KVDT, 1, false, false>(P, t, ti, sc, lds, cu);
      }
      break;
    }
    case PMK_OP_COMBINE:
      if (OCOPY && qi >= 0 && qi + 1 < q1) {
        const pmk_task tn = P.tasks[P.qtasks[qi + 1]];
        if (combine_copies_tile<WDT>(P, sc, tn, t.layer))
          tile_to_lds<WDT>(P.wbase + (int64_t)t.layer * P.layer_bytes + P.off_o, P.qdim, tn.a0, tn.a1, lds + P.pf_off,
                           kOprojRowCost);
      }
      if (P.hd == 128) task_combine<128>(P, t, ti, sc, cu);
      else task_combine<64>(P, t, ti, sc, cu);
      break;
    case PMK_OP_OPROJ: {
      bool copied = false;
      if (OCOPY && qi > q0) {
        const pmk_task tp = P.tasks[P.qtasks[qi - 1]];
        copied = tp.op == PMK_OP_COMBINE && combine_copies_tile<WDT>(P, sc, t, tp.layer);
      }
      task_oproj<WDT>(P, t, ti, sc, lds, cu, copied);
      break;
    }
    case PMK_OP_GATEUP: task_gateup<WDT>(P, t, ti, sc, lds, cu); break;
    case PMK_OP_DOWN: task_down<WDT>(P, t, ti, sc, lds, cu); break;
    case PMK_OP_LMHEAD: task_lmhead<WDT>(P, t, ti, sc, lds, cu); break;
    case PMK_OP_TOKEN: task_token(P, t, ti, sc, lds, cu); break;
    default: break;
  }
  __syncthreads();  // LDS is reused by the next task
}

// ------------------------------------------------------------------------------------------------
// the persistent kernel: one workgroup per CU, n steps of this CU's queue
// ------------------------------------------------------------------------------------------------
// OCOPY: the instance whose COMBINE tasks copy the next O-projection tile early (schedules with
// o_copy set); the other instance has none of that code, which the register allocation of the
// rest of the kernel also benefits from
template <int WDT, int KVDT, bool OCOPY>
__global__ __launch_bounds__(kThreads, 1) void pmk_persistent(KParams P) {
  extern __shared__ float lds[];
  const int cu = blockIdx.x;
  const CallParams cp = *P.call;
  const int epoch0 = (int)P.ctrl[CTRL_EPOCH];
  const int pos0 = (int)P.ctrl[CTRL_POS];
  const int tok0 = (int)P.ctrl[CTRL_TOKEN];
  const int q0 = P.qoff[cu], q1 = P.qoff[cu + 1];
  const int lm_ctr = P.tasks[P.qtasks[P.qoff[1] - 1]].wait_ctr;  // queue 0 ends with the TOKEN task
  // the trace records which XCD (hardware XCC id) ran each queue, for XCD-aware row shares
  unsigned xcc;
  asm volatile("s_getreg_b32 %0, hwreg(HW_REG_XCC_ID)" : "=s"(xcc));
  const uint64_t who = ((uint64_t)(xcc & 0xfu) << 32) | (uint32_t)cu;
  int steps = 0;
  for (int s = 0; s < cp.n_steps; ++s) {
    const int e = epoch0 + s;
    if (s > 0 && cp.eos >= 0 && cp.forced == nullptr) {
      block_wait(P, lm_ctr, P.ctr_prod[lm_ctr], 1, e, cu, -1);
      if (key_token(ldc(&P.keys[s - 1])) == cp.eos) break;
    }
    StepCtx sc;
    sc.e = e;
    sc.s = s;
    sc.pos = pos0 + s;
    sc.pos0 = pos0;
    sc.tok = cp.forced ? cp.forced[s] : (s == 0 ? tok0 : -1);
    if (sc.tok >= P.V) sc.tok = P.V - 1;
    sc.per_op = false;
    sc.calib = cp.calib != 0;
    for (int qi = q0; qi < q1; ++qi) {
      const int ti = P.qtasks[qi];
      const pmk_task t = P.tasks[ti];
      trace_mark(P, s, ti, 0, __builtin_amdgcn_s_memrealtime());
      run_task<WDT, KVDT, OCOPY>(P, t, ti, sc, lds, cu, qi, q0, q1);
      trace_mark(P, s, ti, 2, __builtin_amdgcn_s_memrealtime());
      trace_mark(P, s, ti, 3, who);
    }
    steps = s + 1;
  }
  if (cu == 0 && threadIdx.x == 0) {
    stc(&P.ctrl[CTRL_EPOCH], (uint32_t)(epoch0 + steps));
    stc(&P.ctrl[CTRL_POS], (uint32_t)(pos0 + steps));
    if (cp.n_done) cp.n_done[0] = steps;
  }
}

// ------------------------------------------------------------------------------------------------
// per-op kernels (hipGraph baseline): one workgroup per task of one phase, no waits
// ------------------------------------------------------------------------------------------------
template <int WDT, int KVDT>
__global__ __launch_bounds__(kThreads, 1) void pmk_phase(KParams P, int first_task) {
  extern __shared__ float lds[];
  const CallParams* cp = P.call;
  const int s = (int)P.ctrl[CTRL_STEP];
  if (P.ctrl[CTRL_STOPPED] || s >= cp->n_steps) return;
  StepCtx sc;
  sc.e = (int)P.ctrl[CTRL_EPOCH];
  sc.s = s;
  sc.pos = (int)P.ctrl[CTRL_POS];
  sc.pos0 = sc.pos;  // every step is its own set of launches
  sc.tok = cp->forced ? cp->forced[s] : (int)P.ctrl[CTRL_TOKEN];
  if (sc.tok >= P.V) sc.tok = P.V - 1;
  if (sc.tok < 0) sc.tok = 0;
  sc.per_op = true;
  sc.calib = cp->calib != 0;
  const int ti = first_task + blockIdx.x;
  const pmk_task t = P.tasks[ti];
  run_task<WDT, KVDT>(P, t, ti, sc, lds, blockIdx.x);
}

// ------------------------------------------------------------------------------------------------
// small service kernels
// ------------------------------------------------------------------------------------------------
__global__ void pmk_begin_call(KParams P, CallParams cp) {
  const int i = blockIdx.x * blockDim.x + threadIdx.x;
  if (i == 0) {
    *P.call = cp;
    P.ctrl[CTRL_STEP] = 0;
    P.ctrl[CTRL_STOPPED] = 0;
    if (cp.n_done) cp.n_done[0] = 0;
  }
  for (int k = i; k <= cp.n_steps; k += gridDim.x * blockDim.x) P.keys[k] = 0ull;
}

// zero flags, counters, control words and the step tags of the attention output; set position
// and next token
// ------------------------------------------------------------------------------------------------
// Batched prefill.  The prompt's positions go through the model in chunks of up to `chunk`
// tokens; each layer of a chunk is a sequence of grid-wide phases of ONE cooperative launch:
// RMSNorm (four waves per token), the QKV GEMM with RoPE and the KV append in its epilogue, causal
// attention, the O GEMM + residual, RMSNorm, the gate/up GEMM + SwiGLU, the down GEMM + residual.
// The GEMMs are dense contractions over the chunk's tokens and run on the matrix cores
// (v_mfma_f32_16x16x32): the weights are the A operand, converted exactly to a 16-bit format where
// they are not one (FP8 -> bf16, int8 / int4 codes -> binary16) and scaled per 128-column group
// after the products (FP8 block scales, integer group scales); the activations are the B operand,
// as two 16-bit terms (x = t0 + t1 to within 2^-18 |x| for bf16 terms, 2^-22 for binary16; each
// product accumulated in fp32: about the rounding an fp32 dot product of a few thousand terms
// accumulates anyway) or, for the integer formats, as the one binary16 value the format defines.  A phase reads only what earlier phases wrote; phases are separated by a grid
// barrier, so there is no schedule to validate.
// ------------------------------------------------------------------------------------------------
constexpr int kPfTokens = 128;  // GEMM tile tokens (16 per wave)
// 16-bit terms of an fp32 activation operand (GEMM inputs, attention q and probabilities) for the
// 16-bit and FP8 weight formats (the integer formats take one binary16 term in the GEMMs and three
// in the attention)
constexpr int kPfTerms = 2;

// Element (t, k) of an activation plane of K columns (the GEMMs' B operand): 16-token blocks of
// 8-column groups of 16 tokens x 8 columns, so that a wave's operand load of one step (16 tokens x
// 32 columns) is one contiguous KiB
__device__ __forceinline__ int64_t pf_b_index(int t, int k, int K) {
  return ((((int64_t)(t >> 4) * (K >> 3)) + (k >> 3)) << 7) + ((t & 15) << 3) + (k & 7);
}

template <int WDT>
struct PfFmt {
  static constexpr bool INT = weight_is_int(WDT);
  static constexpr int ADT = WDT == WF16 || INT ? WF16 : WBF16;  // matrix-core operand format
  static constexpr int NTERM = INT ? 1 : kPfTerms;                // activation terms
  static constexpr bool SCALED = WDT >= WFP8;
};

// fp32 x[8] -> NT 16-bit terms of format DT per element (nearest even at each step): term 0 is x
// rounded, term 1 the rounded remainder
template <int DT, int NT>
__device__ __forceinline__ void split_terms8(const float* x, u32x4 (&t)[NT]) {
  uint32_t w[NT][4];
#pragma unroll
  for (int k = 0; k < 4; ++k) {
    uint16_t h[NT][2];
#pragma unroll
    for (int e = 0; e < 2; ++e) {
      float r = x[2 * k + e];
#pragma unroll
      for (int n = 0; n < NT; ++n) {
        h[n][e] = enc16<DT>(r);
        if (n + 1 < NT) r -= dec16<DT>(h[n][e]);
      }
    }
#pragma unroll
    for (int n = 0; n < NT; ++n) w[n][k] = h[n][0] | ((uint32_t)h[n][1] << 16);
  }
#pragma unroll
  for (int n = 0; n < NT; ++n) t[n] = u32x4{w[n][0], w[n][1], w[n][2], w[n][3]};
}

// Store v as NT 16-bit terms of format DT at element idx of NT planes `plane` elements apart (one
// term: v rounded to DT, the binary16 activation of the integer formats).
template <int DT, int NT>
__device__ __forceinline__ void put_terms(uint16_t* planes, int64_t plane, int64_t idx, float v) {
#pragma unroll
  for (int n = 0; n < NT; ++n) {
    const uint16_t h = enc16<DT>(v);
    planes[n * plane + idx] = h;
    if (n + 1 < NT) v -= dec16<DT>(h);
  }
}

// Grid barrier number `k` (1-based) of the launch.  Each workgroup owns one flag word (bar[b],
// zero at launch): it drains its stores, publishes them (agent-scope release) and stores k into
// its flag; then wave 0 polls all the flags, one coherent load per lane per 64 workgroups, until
// every one shows k (a single shared counter serialised 256 atomics, ~50 us per barrier).  The
// acquire fence then makes the other workgroups' stores visible to later loads.  The wait is
// bounded like every other wait (watchdog: the abort word ends all of them).
__device__ __forceinline__ void pf_barrier(const KParams& P, uint32_t* bar, uint32_t k) {
  drain();
  __syncthreads();
  if (threadIdx.x == 0) {
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "agent");
    stc(&bar[blockIdx.x], k);
  }
  if (threadIdx.x < 64) {
    const int n = (int)gridDim.x;
    int64_t spins = 0;
    while (true) {
      __atomic_signal_fence(__ATOMIC_SEQ_CST);  // each round reads the flags again
      bool ok = true;
      for (int b = (int)threadIdx.x; b < n; b += 64) ok = ok && ldc(&bar[b]) >= k;
      if (__all(ok)) break;
      if (ldc(&P.ctrl[CTRL_ABORT]) != 0u) break;
      if (++spins > P.spin_limit) {
        if (threadIdx.x == 0) report_error(P.ctrl, PMK_ERR_TIMEOUT, (int)blockIdx.x, -1, -1, k, 0);
        break;
      }
    }
  }
  __syncthreads();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "agent");
}

// RMSNorm of `ntok` rows of src [chunk][H] (or, with emb_tok, of the embedding rows of those tokens,
// written to src first) into the activation planes bn: (x * r) * g with r = 1 / sqrt(mean(x^2) +
// eps), as NT terms of format DT.  One wave per token.
template <int DT, int NT, int EDT>
__device__ __forceinline__ void pf_rmsnorm(const KParams& P, const PrefillArgs& A, float* src, const float* add,
                                           const int32_t* emb_tok, const float* gain, int ntok, float* red) {
  // four waves per token (a quarter of the columns each; their sums of squares meet in LDS), two
  // tokens per workgroup and round
  constexpr int WPT = 4, TPR = kWaves / WPT;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6, sub = wave % WPT, H = P.H, Hq = H / WPT;
  const int64_t plane = (int64_t)A.chunk * H;
  for (int t0 = (int)blockIdx.x * TPR; t0 < ntok; t0 += (int)gridDim.x * TPR) {
    const int t = t0 + wave / WPT;
    const bool ok = t < ntok;
    float* x = src + (int64_t)t * H;
    // a projection computed in two K-halves: the residual stream is the sum of both planes (stored
    // back, for the residual the next GEMM's epilogue adds)
    const float* x2 = add ? add + (int64_t)t * H : nullptr;
    float ss = 0.f;
    if (ok) {
      if (emb_tok) {
        int tok = emb_tok[t];
        tok = tok < 0 ? 0 : (tok >= P.V ? P.V - 1 : tok);
        const uint16_t* e = P.embed + (int64_t)tok * H;
        for (int k = sub * Hq + 2 * lane; k < (sub + 1) * Hq; k += 128) {
          const uint32_t w = *reinterpret_cast<const uint32_t*>(e + k);
          *reinterpret_cast<float2*>(x + k) = make_float2(dec16<EDT>((uint16_t)(w & 0xffffu)),
                                                          dec16<EDT>((uint16_t)(w >> 16)));
        }
      }
      for (int k = sub * Hq + 2 * lane; k < (sub + 1) * Hq; k += 128) {
        float2 v = *reinterpret_cast<const float2*>(x + k);
        if (x2) {
          const float2 u = *reinterpret_cast<const float2*>(x2 + k);
          v = make_float2(v.x + u.x, v.y + u.y);
          *reinterpret_cast<float2*>(x + k) = v;
        }
        ss = fmaf(v.x, v.x, ss);
        ss = fmaf(v.y, v.y, ss);
      }
    }
    ss = wave_sum(ss);
    if (lane == 0) red[wave] = ss;
    __syncthreads();
    float tot = 0.f;
#pragma unroll
    for (int q = 0; q < WPT; ++q) tot += red[(wave / WPT) * WPT + q];
    __syncthreads();  // red is written again in the next round
    if (!ok) continue;
    const float r = 1.0f / sqrtf(tot / (float)H + P.eps);
    for (int k = sub * Hq + 2 * lane; k < (sub + 1) * Hq; k += 128) {
      const float2 v = *reinterpret_cast<const float2*>(x + k);
      const float2 g = *reinterpret_cast<const float2*>(gain + k);
      put_terms<DT, NT>(A.bn, plane, pf_b_index(t, k, H), (v.x * r) * g.x);
      put_terms<DT, NT>(A.bn, plane, pf_b_index(t, k + 1, H), (v.y * r) * g.y);
    }
  }
}

// 8 columns of one weight row as 8 exact 16-bit matrix-core operands (format PfFmt::ADT), from
// their bytes in the arena: 16-bit formats as stored; FP8 E4M3 to bf16; int8 / int4 codes (offset
// binary, int4 nibbles of the word in the order 0 2 4 6 1 3 5 7) to binary16.
// A weight piece of 8 columns as loaded (16 B of a 16-bit format, 8 B of FP8 or int8, 4 B of
// int4), and its conversion to eight 16-bit matrix-core operands (done when the piece is stored to
// LDS, so a load in flight holds only the raw bytes)
template <int WDT>
struct PfRaw {
  using T = u32x4;
};
template <>
struct PfRaw<WFP8> {
  using T = u32x2;
};
template <>
struct PfRaw<WI8> {
  using T = u32x2;
};
template <>
struct PfRaw<WI4> {
  using T = uint32_t;
};

template <int WDT>
__device__ __forceinline__ typename PfRaw<WDT>::T pf_load_raw(__amdgpu_buffer_rsrc_t r, uint32_t off) {
  if constexpr (WDT == WF16 || WDT == WBF16) return __builtin_amdgcn_raw_buffer_load_b128(r, off, 0, 0);
  else if constexpr (WDT == WFP8 || WDT == WI8) return __builtin_amdgcn_raw_buffer_load_b64(r, off, 0, 0);
  else return __builtin_amdgcn_raw_buffer_load_b32(r, off, 0, 0);
}

template <int WDT>
__device__ __forceinline__ u32x4 pf_a16(typename PfRaw<WDT>::T w) {
  if constexpr (WDT == WF16 || WDT == WBF16) {
    return w;
  } else if constexpr (WDT == WFP8) {
    return fp8x8_bf16(w);
  } else if constexpr (WDT == WI8) {
    const h16x2 bias = {(_Float16)-1152.0f, (_Float16)-1152.0f};
    auto cv = [&](uint32_t v, uint32_t sel) {
      return __builtin_bit_cast(uint32_t, as_h2(__builtin_amdgcn_perm(0x64646464u, v, sel)) + bias);
    };
    return u32x4{cv(w.x, 0x04010400u), cv(w.x, 0x04030402u), cv(w.y, 0x04010400u), cv(w.y, 0x04030402u)};
  } else {
    const h16x2 b1 = {(_Float16)-1032.0f, (_Float16)-1032.0f};
    const h16x2 m16 = {(_Float16)0.0625f, (_Float16)0.0625f};
    const h16x2 b2 = {(_Float16)-72.0f, (_Float16)-72.0f};
    const uint32_t magic = 0x64006400u, w8 = w >> 8;
    const h16x2 p0 = as_h2(and_or(w, 0x000F000Fu, magic)) + b1;
    const h16x2 p1 = __builtin_elementwise_fma(as_h2(and_or(w, 0x00F000F0u, magic)), m16, b2);
    const h16x2 p2 = as_h2(and_or(w8, 0x000F000Fu, magic)) + b1;
    const h16x2 p3 = __builtin_elementwise_fma(as_h2(and_or(w8, 0x00F000F0u, magic)), m16, b2);
    return u32x4{__builtin_bit_cast(uint32_t, p0), __builtin_bit_cast(uint32_t, p1), __builtin_bit_cast(uint32_t, p2),
                 __builtin_bit_cast(uint32_t, p3)};
  }
}

// Byte offset of the 16-byte piece (row, 8-column group kg) of a step's A block in LDS: rows of 64
// bytes, the four pieces of a row permuted by row bits 1..3.  The matrix-core operand reads take one
// kg for 16 consecutive rows of a block, and the stores four kg of consecutive rows: both then fall
// on distinct banks in every group of 8 (or 16) lanes, where the plain row-major order put four of
// every eight lanes' reads on the same banks.
__device__ __forceinline__ uint32_t pf_a_offset(int row, int kg) {
  return (uint32_t)row * 64u + (uint32_t)((kg ^ ((row >> 1) & 3) ^ ((row >> 3) & 1)) * 16);
}

// Steps of weight loads in flight ahead of the LDS store (raw pieces in registers; it divides the
// activation ring's depth): two, one for the scaled formats, whose per-group accumulators leave no
// registers for more
template <int WDT>
constexpr int pf_a_depth() { return WDT >= WFP8 ? 1 : 2; }

// One GEMM tile: rows [row0, row0 + MR) of W ([N][K] in format WDT) against tokens
// [tok0, tok0 + 128) of the activation planes B ([NTERM] planes of chunk x K, layout pf_b_index),
// over the 32-column steps [step0, step1).  Wave w takes tile rows (w / 4) MR / 2 .. + MR / 2 - 1
// and tokens tok0 + 32 (w % 4) .. + 31 (two 16-token column blocks): per step it reads MR / 2 rows
// of the weight block from LDS (half of what a wave taking all rows would) and its tokens' terms
// from global memory (a 2-step register ring).  The weight block of a step goes through LDS once
// for the workgroup (converted to 16-bit operands on the way, three buffers) and each wave reads its
// operands of the next step while its matrix-core products of this step run.  Scaled formats
// accumulate each 128-column group apart and add it times scale(row, group).
// epi(r, t, v, ks) receives rows r .. r + 3 (r = a 16-row block's first row + 4 (lane / 16)) of token
// t (its 16-token block's first token + lane % 16); rows past N are garbage the epilogues skip.
template <int WDT, int MR, class ScaleF, class Epi>
__device__ __forceinline__ void pf_gemm_tile(const uint8_t* W, int N, int K, const uint16_t* B, int chunk, int row0,
                                             int tok0, int step0, int step1, int ks, float* lds, ScaleF scale,
                                             Epi epi) {
  using F = PfFmt<WDT>;
  constexpr int NT = F::NTERM;
  constexpr int RB = MR / 32;                   // 16-row blocks per wave
  constexpr int AW = MR >= 128 ? MR / 128 : 1;  // 8-column A pieces per thread per step (MR x 4 pieces)
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6, r16 = lane & 15, kg = lane >> 4;
  const int wrow = (wave >> 2) * (MR / 2);      // the wave's first tile row
  const int tb0 = (tok0 >> 4) + 2 * (wave & 3);  // the wave's two 16-token blocks
  const int rows = N - row0 < MR ? N - row0 : MR;
  const int64_t rbytes = weight_row_bytes(WDT, K);
  const __amdgpu_buffer_rsrc_t wr = __builtin_amdgcn_make_buffer_rsrc(
      const_cast<uint8_t*>(W + (int64_t)row0 * rbytes), (short)0, (int)(rows * rbytes), 0x00020000);
  const __amdgpu_buffer_rsrc_t br = __builtin_amdgcn_make_buffer_rsrc(
      const_cast<uint16_t*>(B), (short)0, (int)((int64_t)NT * chunk * K * 2), 0x00020000);
  constexpr uint32_t kOut = 0x7FFFFFF0u;
  const uint32_t bplane = (uint32_t)chunk * (uint32_t)K * 2u;
  const uint32_t bblk = (uint32_t)K * 32u;                 // bytes of a 16-token block
  const uint32_t bbase = (uint32_t)tb0 * bblk + (uint32_t)r16 * 16u;
  const int nsteps = step1 - step0, kofs = 32 * step0;  // this tile's columns: [kofs, 32 step1)
  // A: each thread's pieces of a step are loaded DA steps before they are stored (raw bytes in a
  // register ring, slot = step % DA), converted on the store two steps ahead of their use; step s
  // goes to LDS buffer s % 3 (MR x 64 bytes, pf_a_offset), which is read one step ahead of its use,
  // so the buffer written at a step was last read two barriers earlier.
  // Piece p = thread + 512 a -> row p / 4, columns 8 (p % 4) ..
  constexpr int DA = pf_a_depth<WDT>();
  using RawT = typename PfRaw<WDT>::T;
  uint8_t* abuf = reinterpret_cast<uint8_t*>(lds);
  RawT ar[DA][AW];
  auto load_a = [&](int slot, int step) {
#pragma unroll
    for (int a = 0; a < AW; ++a) {
      const int p = (int)threadIdx.x + kThreads * a, r = p >> 2, k = kofs + step * 32 + 8 * (p & 3);
      const uint32_t off = (uint32_t)(r * rbytes + (int64_t)k * weight_bits(WDT) / 8);
      ar[slot][a] = pf_load_raw<WDT>(wr, k < K && p < MR * 4 ? off : kOut);
    }
  };
  auto store_a = [&](int slot, int step) {
    uint8_t* dst = abuf + (step % 3) * MR * 64;
#pragma unroll
    for (int a = 0; a < AW; ++a) {
      const int p = (int)threadIdx.x + kThreads * a;
      if (p < MR * 4) *reinterpret_cast<u32x4*>(dst + pf_a_offset(p >> 2, p & 3)) = pf_a16<WDT>(ar[slot][a]);
    }
  };
  // the wave's operands of one step: RB 16-row blocks
  u32x4 ao[2][RB];
  auto read_a = [&](int buf, int step) {
    const uint8_t* src = abuf + (step % 3) * MR * 64 + wrow * 64 + pf_a_offset(r16, kg);
#pragma unroll
    for (int b = 0; b < RB; ++b) ao[buf][b] = *reinterpret_cast<const u32x4*>(src + b * 16 * 64);
  };
  // B: a ring of D steps of this lane's terms (two token blocks) in flight; a step past the end
  // reads zeros without touching memory
  constexpr int D = 2;  // 4 measured slower: the registers it takes spill elsewhere in the kernel
  static_assert(D % DA == 0 && D % 2 == 0, "the rings' slots follow the step");
  u32x4 rb[D][2][NT];
  auto issue = [&](int d, int step) {
    const int k = kofs + step * 32 + 8 * kg;
    const bool ok = k < K;  // K is a multiple of 8: a lane's 8 columns are all in or all out
    const uint32_t ko = bbase + (uint32_t)(k >> 3) * 256u;
#pragma unroll
    for (int c = 0; c < 2; ++c)
#pragma unroll
      for (int t = 0; t < NT; ++t)
        rb[d][c][t] = __builtin_amdgcn_raw_buffer_load_b128(br, ok ? ko + (uint32_t)c * bblk + (uint32_t)t * bplane : kOut,
                                                            0, 0);
  };
#pragma unroll
  for (int s = 0; s < DA; ++s) load_a(s, s);
  store_a(0, 0);
  load_a(0, DA);
#pragma unroll
  for (int d = 0; d < D; ++d) issue(d, d);
  store_a(1 % DA, 1);
  load_a(1 % DA, 1 + DA);
  __syncthreads();
  read_a(0, 0);
  f32x4 acc[RB][2], accg[F::SCALED ? RB : 1][2];
#pragma unroll
  for (int b = 0; b < RB; ++b) acc[b][0] = acc[b][1] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
  for (int b = 0; b < (F::SCALED ? RB : 1); ++b) accg[b][0] = accg[b][1] = f32x4{0.f, 0.f, 0.f, 0.f};
  for (int base = 0; base < nsteps; base += D) {
#pragma unroll
    for (int d = 0; d < D; ++d) {
      const int step = base + d;
      if (step < nsteps) {
        if (step + 1 < nsteps) read_a((d + 1) & 1, step + 1);
        // the low terms first (each accumulator sums its products smallest first), all of a term's
        // products before the next term's: consecutive products never share an accumulator
#pragma unroll
        for (int t = NT - 1; t >= 0; --t)
#pragma unroll
          for (int b = 0; b < RB; ++b)
#pragma unroll
            for (int c = 0; c < 2; ++c) {
              f32x4& cc = F::SCALED ? accg[b][c] : acc[b][c];
              cc = mfma16<F::ADT>(ao[d & 1][b], rb[d][c][t], cc);
            }
        if constexpr (F::SCALED) {
          if ((step & 3) == 3 || step == nsteps - 1) {  // end of a 128-column group (step0 % 4 == 0)
            const int g = (step0 + step) >> 2;
#pragma unroll
            for (int b = 0; b < RB; ++b)
#pragma unroll
              for (int i = 0; i < 4; ++i) {
                const float sv = scale(row0 + wrow + 16 * b + 4 * kg + i, g);
#pragma unroll
                for (int c = 0; c < 2; ++c) {
                  acc[b][c][i] = fmaf(accg[b][c][i], sv, acc[b][c][i]);
                  accg[b][c][i] = 0.f;
                }
              }
          }
        }
      }
      issue(d, step + D);
      // step + 2's weights into the buffer read two barriers ago, then their slot refilled with the
      // loads DA steps after them
      if (step + 2 < nsteps) store_a((d + 2) % DA, step + 2);
      load_a((d + 2) % DA, step + 2 + DA);
      __syncthreads();
    }
  }
#pragma unroll
  for (int b = 0; b < RB; ++b)
#pragma unroll
    for (int c = 0; c < 2; ++c) epi(row0 + wrow + 16 * b + 4 * kg, (tb0 + c) * 16 + r16, acc[b][c], ks);
}

// K-halves of a GEMM phase: 2 where K has at least eight 32-column steps (the halves split at a
// 128-column group boundary) and `mode` asks for it (2) or, automatic (0), its tiles would fill at
// most half the grid; else 1
__device__ __forceinline__ int pf_ksplit(int N, int K, int MR, int ntok, int mode) {
  const int tiles = ((N + MR - 1) / MR) * ((ntok + kPfTokens - 1) / kPfTokens);
  const bool can = (((K + 31) / 32 / 2) & ~3) > 0;
  return can && (mode == 2 || (mode == 0 && 2 * tiles <= (int)gridDim.x)) ? 2 : 1;
}

// Run the tiles of one GEMM phase: rows [0, N) x tokens [0, ntok) x ksplit K-parts (epi gets the
// part's index: part 1 of two adds its products to a plane of its own), tiles of MR rows spread over
// the grid.
template <int WDT, int MR, class ScaleF, class Epi>
__device__ __forceinline__ void pf_gemm(const uint8_t* W, int N, int K, const uint16_t* B, int chunk, int ntok,
                                        int ksplit, float* lds, ScaleF scale, Epi epi) {
  const int nr = (N + MR - 1) / MR, nt = (ntok + kPfTokens - 1) / kPfTokens, total = nr * nt * ksplit;
  const int ns = (K + 31) / 32, mid = ksplit == 2 ? ((ns / 2) & ~3) : ns;
  // workgroup b runs on XCD b % 8: each round of G tiles gives XCD x the consecutive tiles
  // x G / 8 .. (x + 1) G / 8 - 1, so the token tiles of a row block (and K-part) share its weight
  // reads in one L2
  const int G = (int)gridDim.x, rounds = (total + G - 1) / G;
  for (int k = 0; k < rounds; ++k) {
    const int b = (int)blockIdx.x;
    const int ti = k * G + ((G & 7) == 0 ? (b & 7) * (G >> 3) + (b >> 3) : b);
    if (ti >= total) continue;
    const int part = ti / (nr * nt), rt = ti % (nr * nt);
    const int row0 = (rt / nt) * MR, tok0 = (rt % nt) * kPfTokens;
    pf_gemm_tile<WDT, MR>(W, N, K, B, chunk, row0, tok0, part == 0 ? 0 : mid, part == 0 ? mid : ns, part, lds,
                          scale, epi);
  }
}

// 8 cache elements (K row piece or V^T piece) as 16-bit matrix-core operands: FP8 to bf16 (exact).
template <int KVDT>
__device__ __forceinline__ u32x4 pf_kv8(const uint8_t* base, int64_t elem) {
  if constexpr (KVDT == WFP8) return fp8x8_bf16(*reinterpret_cast<const u32x2*>(base + elem));
  else return *reinterpret_cast<const u32x4*>(base + elem * 2);
}

// Causal attention of the chunk's queries (positions p0 .. p0 + ntok - 1) over the cache
// positions 0 .. p0 + ntok - 1 (this chunk's rows were appended by the QKV phase).  One workgroup
// per (q head j, block of 16 queries); its eight waves split the key positions, wave w taking the
// 32-position groups w, w + 8, ... up to the block's last query, with the decode attention's
// matrix-core layout and the 16 queries of the head as the B columns: scores = K rows (A) x q
// (B, two 16-bit terms; three for the integer formats), online softmax per query, P.V = V^T (A,
// from the blocked V cache) x P (B, the same terms); an FP8 cache is read as bf16 operands and
// scaled (K on the scores, V on the output).  The waves' (max, sum, acc) are merged in LDS
// (8 x 16 x (hd + 2) floats) and the output goes to the activation planes bo as ONT terms of
// format ODT.
template <int KVDT, int ODT, int ONT, int HD>
__device__ __forceinline__ void pf_attn(const KParams& P, const PrefillArgs& A, int l, int p0, int ntok, float* lds) {
  constexpr int KDT = KVDT == WF16 ? WF16 : WBF16;  // operand format of the cache values
  constexpr int KES = KVDT == WFP8 ? 1 : 2;
  constexpr int NC = HD / 32, NT = HD / 16, REC = HD + 2;
  // q and P as 16-bit terms: three where the output is rounded to one binary16 term (the integer
  // formats' A16 operand of the O projection, whose rounding turns a two-term error into whole
  // binary16 steps in some elements), else two
  constexpr int QT = ONT == 1 ? 3 : kPfTerms;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6, c16 = lane & 15, kg = lane >> 4;
  const int nqb = (ntok + 15) / 16, ntasks = P.nq * nqb, qd = P.qdim;
  const int pend = p0 + ntok;  // cache positions [0, pend) are written
  const int64_t oplane = (int64_t)A.chunk * qd;
  float* rec = lds + (wave * 16 + c16) * REC;  // this lane's column record: acc[HD], m, sum
  for (int task = blockIdx.x; task < ntasks; task += gridDim.x) {
    const int j = task % P.nq, qb = task / P.nq;
    const int g = j / P.grp;
    const int64_t hb = (int64_t)l * P.nkv + g;
    float kscale = 1.f, vscale = 1.f;
    if constexpr (KVDT == WFP8) {
      kscale = P.kv_scale[hb * 2];
      vscale = P.kv_scale[hb * 2 + 1];
    }
    const float scale = kscale * P.attn_scale;
    const int tq = qb * 16 + c16;                  // this lane's query (column)
    const int tqc = tq < ntok ? tq : ntok - 1;     // padding columns repeat the last query
    const int qpos = p0 + tqc;
    const int qlast = p0 + ((qb * 16 + 15) < ntok ? qb * 16 + 15 : ntok - 1);
    float m = -INFINITY, sum = 0.f;
    f32x4 acc[NT];
#pragma unroll
    for (int tt = 0; tt < NT; ++tt) acc[tt] = f32x4{0.f, 0.f, 0.f, 0.f};
    if (32 * wave <= qlast) {
      u32x4 qt[NC][QT];
#pragma unroll
      for (int s = 0; s < NC; ++s) {
        float qv[8];
        const float* src = A.q + (int64_t)tqc * qd + j * HD + 32 * s + 8 * kg;
#pragma unroll
        for (int e = 0; e < 8; ++e) qv[e] = src[e];
        split_terms8<KDT, QT>(qv, qt[s]);
      }
      for (int kb = 32 * wave; kb <= qlast; kb += 32 * kWaves) {
        // A rows: block 0 row r -> position kb + 8 (r / 4) + r % 4, block 1 the same + 4, so that
        // each lane ends up with the scores of positions kb + 8 kg .. + 7 of its query
        const int pr0 = kb + 8 * (c16 >> 2) + (c16 & 3);
        f32x4 s0 = {0.f, 0.f, 0.f, 0.f}, s1 = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int s = 0; s < NC; ++s) {
          const u32x4 ka = pf_kv8<KVDT>(P.kc, (hb * P.seqcap + pr0) * HD + 32 * s + 8 * kg);
          const u32x4 kb4 = pf_kv8<KVDT>(P.kc, (hb * P.seqcap + pr0 + 4) * HD + 32 * s + 8 * kg);
#pragma unroll
          for (int n = QT - 1; n >= 0; --n) {
            s0 = mfma16<KDT>(ka, qt[s][n], s0);
            s1 = mfma16<KDT>(kb4, qt[s][n], s1);
          }
        }
        const int pv = kb + 8 * kg;  // this lane's 8 positions
        u32x4 vt[NT];
        const int nv = pend - pv;  // positions of this lane's group that are written (others: zero V)
#pragma unroll
        for (int tt = 0; tt < NT; ++tt) {
          vt[tt] = pf_kv8<KVDT>(P.vc, ((hb * (P.seqcap / 32) + kb / 32) * HD + 16 * tt + c16) * 32 + 8 * kg);
          if (nv < 8) vt[tt] = keep_first(vt[tt], nv < 0 ? 0 : nv);
        }
        float sc8[8];
        float mk = -INFINITY;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          sc8[i] = pv + i <= qpos ? s0[i] * scale : -INFINITY;
          sc8[4 + i] = pv + 4 + i <= qpos ? s1[i] * scale : -INFINITY;
          mk = fmaxf(mk, fmaxf(sc8[i], sc8[4 + i]));
        }
        const float mn = fmaxf(m, column_max<16>(mk));
        float ps = 0.f;
#pragma unroll
        for (int i = 0; i < 8; ++i) {
          sc8[i] = mn == -INFINITY ? 0.f : expf(sc8[i] - mn);
          ps += sc8[i];
        }
        ps = column_sum<16>(ps);
        const float alpha = m == -INFINITY ? 0.f : expf(m - mn);
        sum = sum * alpha + ps;
#pragma unroll
        for (int tt = 0; tt < NT; ++tt)
#pragma unroll
          for (int i = 0; i < 4; ++i) acc[tt][i] *= alpha;
        m = mn;
        u32x4 pt[QT];
        split_terms8<KDT, QT>(sc8, pt);
#pragma unroll
        for (int tt = 0; tt < NT; ++tt)
#pragma unroll
          for (int n = QT - 1; n >= 0; --n) acc[tt] = mfma16<KDT>(vt[tt], pt[n], acc[tt]);
      }
    }
    // merge the eight waves' records in LDS (a wave without positions left m = -inf, sum = 0)
#pragma unroll
    for (int tt = 0; tt < NT; ++tt)
#pragma unroll
      for (int i = 0; i < 4; ++i) rec[16 * tt + 4 * kg + i] = acc[tt][i];
    if (kg == 0) {
      rec[HD] = m;
      rec[HD + 1] = sum;
    }
    __syncthreads();
    for (int idx = threadIdx.x; idx < 16 * HD; idx += kThreads) {
      const int c = idx / HD, d = idx % HD, t = qb * 16 + c;
      if (t >= ntok) continue;
      float mx = -INFINITY;
#pragma unroll
      for (int w = 0; w < kWaves; ++w) mx = fmaxf(mx, lds[(w * 16 + c) * REC + HD]);
      float num = 0.f, den = 0.f;
#pragma unroll
      for (int w = 0; w < kWaves; ++w) {
        const float* r = lds + (w * 16 + c) * REC;
        const float f = r[HD] == -INFINITY ? 0.f : expf(r[HD] - mx);
        num = fmaf(r[d], f, num);
        den = fmaf(r[HD + 1], f, den);
      }
      put_terms<ODT, ONT>(A.bo, oplane, pf_b_index(t, j * HD + d, qd), num / den * vscale);
    }
    __syncthreads();
  }
}

template <int WDT, int KVDT>
__global__ void __launch_bounds__(kThreads, 1) pmk_prefill_batch(KParams P, PrefillArgs A) {
  extern __shared__ float lds_pf[];  // the attention's wave records, or the GEMM's weight blocks
  using F = PfFmt<WDT>;
  constexpr int ADT = F::ADT, NT = F::NTERM, EDT = WFmt<WDT>::EDT;
  using ST = typename WFmt<WDT>::ST;
  const int H = P.H, qd = P.qdim, F_ = P.F, hd = P.hd, half = P.hd / 2, chunk = A.chunk;
  const int qrows = P.qdim, krows = P.nkv * P.hd;
  uint32_t nbar = 0;
  for (int p0 = 0; p0 < A.n; p0 += chunk) {
    const int ntok = A.n - p0 < chunk ? A.n - p0 : chunk;
    pf_rmsnorm<ADT, NT, EDT>(P, A, A.x, nullptr, A.tokens + p0, P.gains, ntok, lds_pf);
    // K-halves of the O and down projections for this chunk (their partial planes are summed by
    // the RMSNorm that reads them)
    const int ks_o = pf_ksplit(H, qd, 128, ntok, A.ksplit), ks_d = pf_ksplit(H, F_, 128, ntok, A.ksplit);
    pf_barrier(P, A.bar, ++nbar);
    for (int l = 0; l < P.L; ++l) {
      const uint8_t* Wl = P.wbase + (int64_t)l * P.layer_bytes;
      // scale of (packed) row r, 128-column group g of each linear tensor (unscaled formats: unused)
      const int nbh = (H + 127) / 128, nbq = (qd + 127) / 128, nbf = (F_ + 127) / 128;
      const ST* const sq = scale_rows<WDT>(P, l, 0);
      const ST* const sk = scale_rows<WDT>(P, l, 1);
      const ST* const sv = scale_rows<WDT>(P, l, 2);
      auto s_qkv = [&](int r, int g) -> float {
        if constexpr (!F::SCALED) return 1.f;
        else {
          const ST* base;
          int orow;
          if (r < qrows) { base = sq; orow = r; }
          else if (r < qrows + krows) { base = sk; orow = r - qrows; }
          else { base = sv; orow = r - qrows - krows; }
          const int head = orow / hd, pr = orow % hd;
          return scale_value<WDT>(scale_row<WDT>(base, head * hd + (pr >> 1) + (pr & 1) * half, nbh)[g]);
        }
      };
      // QKV: rows 2m, 2m + 1 are a RoPE pair (q, k) or two v dims; q to A.q, k and v to the cache
      pf_gemm<WDT, 128>(Wl + P.off_qkv, P.qkv_rows, H, A.bn, chunk, ntok, 1, lds_pf, s_qkv,
                        [&](int r4, int t, f32x4 v, int) {
        // the 16 rows of this lane's block lie in one section and one head (sections and heads are
        // multiples of 16 rows), so the calibration's max reduces over the wave first
        float amax = 0.f;
        if (t < ntok && r4 < P.qkv_rows) {
        const int pos = p0 + t;
#pragma unroll
        for (int pp = 0; pp < 2; ++pp) {
          const int r = r4 + 2 * pp;
          float a = v[2 * pp], b = v[2 * pp + 1];
          int sec, base;
          if (r < qrows) { sec = 0; base = 0; }
          else if (r < qrows + krows) { sec = 1; base = qrows; }
          else { sec = 2; base = qrows + krows; }
          const int head = (r - base) / hd, i = ((r - base) % hd) >> 1;
          if (sec < 2) {
            const float2 cs = P.rope[(int64_t)pos * half + i];
            const float a2 = a * cs.x - b * cs.y;
            const float b2 = b * cs.x + a * cs.y;
            a = a2;
            b = b2;
          }
          if (sec == 0) {
            float* q = A.q + (int64_t)t * qd + head * hd;
            q[i] = a;
            q[i + half] = b;
            continue;
          }
          const int64_t hb = (int64_t)l * P.nkv + head;
          const int64_t ia = sec == 1 ? (hb * P.seqcap + pos) * hd + i
                                      : ((hb * (P.seqcap / 32) + pos / 32) * hd + i) * 32 + pos % 32;
          const int64_t ib = sec == 1 ? ia + half : ia + (int64_t)half * 32;
          if constexpr (KVDT == WFP8) {
            amax = fmaxf(amax, fmaxf(fabsf(a), fabsf(b)));
            const float s8 = P.kv_scale[hb * 2 + (sec - 1)];
            uint8_t* c8 = sec == 1 ? P.kc : P.vc;
            c8[ia] = enc_e4m3(a / s8);
            c8[ib] = enc_e4m3(b / s8);
          } else {
            uint16_t* c16 = reinterpret_cast<uint16_t*>(sec == 1 ? P.kc : P.vc);
            c16[ia] = enc16<KVDT>(a);
            c16[ib] = enc16<KVDT>(b);
          }
        }
        }
        if constexpr (KVDT == WFP8) {
          const int rb = r4 & ~15;  // the block's first row (the same on every lane)
          if (A.calib && rb >= qrows && rb < P.qkv_rows) {
#pragma unroll
            for (int o = 32; o >= 1; o >>= 1) amax = fmaxf(amax, __shfl_xor(amax, o));
            const int sec = rb < qrows + krows ? 1 : 2, head = (rb - (sec == 1 ? qrows : qrows + krows)) / hd;
            if ((threadIdx.x & 63) == 0)
              __hip_atomic_fetch_max(&P.kv_amax[((int64_t)l * P.nkv + head) * 2 + (sec - 1)], __float_as_uint(amax),
                                     __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
          }
        }
      });
      pf_barrier(P, A.bar, ++nbar);
      if (hd == 128) pf_attn<KVDT, ADT, NT, 128>(P, A, l, p0, ntok, lds_pf);
      else pf_attn<KVDT, ADT, NT, 64>(P, A, l, p0, ntok, lds_pf);
      pf_barrier(P, A.bar, ++nbar);
      // O projection + residual
      const ST* const so = scale_rows<WDT>(P, l, 3);
      auto s_o = [&](int r, int g) -> float {
        if constexpr (!F::SCALED) return 1.f;
        else return scale_value<WDT>(scale_row<WDT>(so, r, nbq)[g]);
      };
      pf_gemm<WDT, 128>(Wl + P.off_o, H, qd, A.bo, chunk, ntok, ks_o, lds_pf, s_o, [&](int r4, int t, f32x4 v, int ks) {
        if (t >= ntok) return;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const int r = r4 + i;
          if (r >= H) continue;
          const int64_t e = (int64_t)t * H + r;
          if (ks == 0) A.xm[e] = A.x[e] + v[i];
          else A.xm2[e] = v[i];
        }
      });
      pf_barrier(P, A.bar, ++nbar);
      pf_rmsnorm<ADT, NT, EDT>(P, A, A.xm, ks_o == 2 ? A.xm2 : nullptr, nullptr, P.gains + (int64_t)l * 2 * H + H,
                               ntok, lds_pf);
      pf_barrier(P, A.bar, ++nbar);
      // gate/up (interleaved rows 2n, 2n + 1) + SwiGLU
      const int64_t hplane = (int64_t)chunk * F_;
      const ST* const sg = scale_rows<WDT>(P, l, 4);
      const ST* const su = scale_rows<WDT>(P, l, 5);
      auto s_gu = [&](int r, int g) -> float {
        if constexpr (!F::SCALED) return 1.f;
        else return scale_value<WDT>(scale_row<WDT>((r & 1) ? su : sg, r >> 1, nbh)[g]);
      };
      // 256-row tiles (128 where the per-group accumulators of a scaled format would not fit)
      pf_gemm<WDT, F::SCALED ? 128 : 256>(Wl + P.off_gu, 2 * F_, H, A.bn, chunk, ntok, 1, lds_pf, s_gu,
                                          [&](int r4, int t, f32x4 v, int) {
        if (t >= ntok) return;
#pragma unroll
        for (int pp = 0; pp < 2; ++pp) {
          const int n = (r4 >> 1) + pp;
          if (n >= F_) continue;
          const float gte = v[2 * pp], up = v[2 * pp + 1];
          put_terms<ADT, NT>(A.bh, hplane, pf_b_index(t, n, F_), gte / (1.0f + expf(-gte)) * up);
        }
      });
      pf_barrier(P, A.bar, ++nbar);
      // down projection + residual
      const ST* const sd = scale_rows<WDT>(P, l, 6);
      auto s_d = [&](int r, int g) -> float {
        if constexpr (!F::SCALED) return 1.f;
        else return scale_value<WDT>(scale_row<WDT>(sd, r, nbf)[g]);
      };
      pf_gemm<WDT, 128>(Wl + P.off_d, H, F_, A.bh, chunk, ntok, ks_d, lds_pf, s_d, [&](int r4, int t, f32x4 v, int ks) {
        if (t >= ntok) return;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const int r = r4 + i;
          if (r >= H) continue;
          const int64_t e = (int64_t)t * H + r;
          if (ks == 0) A.x[e] = A.xm[e] + v[i];
          else A.x2[e] = v[i];
        }
      });
      pf_barrier(P, A.bar, ++nbar);
      if (l + 1 < P.L) {
        pf_rmsnorm<ADT, NT, EDT>(P, A, A.x, ks_d == 2 ? A.x2 : nullptr, nullptr, P.gains + (int64_t)(l + 1) * 2 * H,
                                 ntok, lds_pf);
        pf_barrier(P, A.bar, ++nbar);
      }
    }
  }
}

__global__ void pmk_reset(KParams P, int n_flags, int n_counters, int pos, int token, const int32_t* d_token) {
  const int i = blockIdx.x * blockDim.x + threadIdx.x, n = gridDim.x * blockDim.x;
  for (int k = i; k < n_flags; k += n) P.flags[k] = 0u;
  for (int k = i; k < n_counters; k += n) P.counters[k] = 0u;
  for (int64_t k = i; k < (int64_t)P.L * P.qdim; k += n) P.o[k] = 0ull;
  for (int64_t k = i; k < (int64_t)(P.L + 1) * P.H; k += n) P.x[k] = 0ull;
  for (int64_t k = i; k < (int64_t)P.L * P.H; k += n) P.xm[k] = 0ull;
  for (int64_t k = i; k < (int64_t)P.L * P.qdim; k += n) P.q[k] = 0ull;
  for (int64_t k = i; k < (int64_t)P.L * P.nkv * 2 * P.hd; k += n) P.kvcur[k] = 0ull;
  for (int k = i; k < CTRL_WORDS; k += n) P.ctrl[k] = 0u;
  __syncthreads();
  if (i == 0) {
    P.ctrl[CTRL_POS] = (uint32_t)pos;
    P.ctrl[CTRL_TOKEN] = (uint32_t)(d_token ? *d_token : token);
  }
}

// rewind: position and next token only (counters keep counting from the current epoch)
__global__ void pmk_set_pos(KParams P, int pos, const int32_t* d_token) {
  if (threadIdx.x == 0 && blockIdx.x == 0) {
    P.ctrl[CTRL_POS] = (uint32_t)pos;
    P.ctrl[CTRL_TOKEN] = (uint32_t)*d_token;
  }
}

// FP8 KV scale calibration: before, every scale is 1 and every recorded maximum 0; after, each
// (layer, kv head, K|V) scale is its recorded max |value| / 448 (1 where that maximum is 0), which
// maps the largest calibrated value to the largest E4M3 magnitude
__global__ void pmk_kv_calib(KParams P, int finish) {
  const int n = P.L * P.nkv * 2;
  for (int i = blockIdx.x * blockDim.x + threadIdx.x; i < n; i += gridDim.x * blockDim.x) {
    if (!finish) {
      P.kv_scale[i] = 1.0f;
      P.kv_amax[i] = 0u;
    } else {
      const float a = __uint_as_float(P.kv_amax[i]);
      P.kv_scale[i] = a > 0.f ? a / 448.0f : 1.0f;
    }
  }
}

__global__ void pmk_copy_token(const KParams P, int32_t* dst) {
  if (threadIdx.x == 0 && blockIdx.x == 0) *dst = (int32_t)P.ctrl[CTRL_TOKEN];
}

// KV rows [L][nkv][P][hd] (element bytes es) -> K cache [L][nkv][seqcap][hd] and the V cache in
// blocks of 32 positions, [L][nkv][seqcap / 32][hd][32]
__global__ void pmk_load_kv_rows(KParams P, const uint8_t* src_k, const uint8_t* src_v, int npos, int es) {
  const int64_t rowb = (int64_t)P.hd * es;
  const int64_t total = (int64_t)P.L * P.nkv * npos * rowb / 16;
  for (int64_t i = blockIdx.x * (int64_t)blockDim.x + threadIdx.x; i < total; i += (int64_t)gridDim.x * blockDim.x) {
    const int64_t byte = i * 16;
    const int64_t row = byte / rowb, off = byte % rowb;
    const int64_t lg = row / npos, p = row % npos;
    const int64_t dst = (lg * P.seqcap + p) * rowb + off;
    *reinterpret_cast<u32x4*>(P.kc + dst) = *reinterpret_cast<const u32x4*>(src_k + byte);
  }
  const int64_t nel = (int64_t)P.L * P.nkv * npos * P.hd;
  for (int64_t i = blockIdx.x * (int64_t)blockDim.x + threadIdx.x; i < nel; i += (int64_t)gridDim.x * blockDim.x) {
    const int64_t d = i % P.hd, p = (i / P.hd) % npos, lg = i / ((int64_t)P.hd * npos);
    const int64_t dst = ((lg * (P.seqcap / 32) + p / 32) * P.hd + d) * 32 + p % 32;
    if (es == 1) P.vc[dst] = src_v[i];
    else reinterpret_cast<uint16_t*>(P.vc)[dst] = reinterpret_cast<const uint16_t*>(src_v)[i];
  }
}

// The inverse: positions 0..npos-1 of both caches -> canonical rows [L][nkv][npos][hd]
__global__ void pmk_read_kv_rows(KParams P, uint8_t* dst_k, uint8_t* dst_v, int npos, int es) {
  const int64_t rowb = (int64_t)P.hd * es;
  const int64_t total = (int64_t)P.L * P.nkv * npos * rowb / 16;
  for (int64_t i = blockIdx.x * (int64_t)blockDim.x + threadIdx.x; i < total; i += (int64_t)gridDim.x * blockDim.x) {
    const int64_t byte = i * 16;
    const int64_t row = byte / rowb, off = byte % rowb;
    const int64_t lg = row / npos, p = row % npos;
    *reinterpret_cast<u32x4*>(dst_k + byte) = *reinterpret_cast<const u32x4*>(P.kc + (lg * P.seqcap + p) * rowb + off);
  }
  const int64_t nel = (int64_t)P.L * P.nkv * npos * P.hd;
  for (int64_t i = blockIdx.x * (int64_t)blockDim.x + threadIdx.x; i < nel; i += (int64_t)gridDim.x * blockDim.x) {
    const int64_t d = i % P.hd, p = (i / P.hd) % npos, lg = i / ((int64_t)P.hd * npos);
    const int64_t src = ((lg * (P.seqcap / 32) + p / 32) * P.hd + d) * 32 + p % 32;
    if (es == 1) dst_v[i] = P.vc[src];
    else reinterpret_cast<uint16_t*>(dst_v)[i] = reinterpret_cast<const uint16_t*>(P.vc)[src];
  }
}

// Repack: packed QKV row r of layer l <- wq/wk/wv row (head*hd + pair + half*hd/2)
__global__ void pmk_repack_qkv(uint8_t* dst, const uint8_t* wq, const uint8_t* wk, const uint8_t* wv, int nq, int nkv,
                               int hd, int64_t rowb) {
  const int r = blockIdx.x;
  const int qrows = nq * hd, krows = nkv * hd;
  const uint8_t* src;
  int base;
  if (r < qrows) { src = wq; base = 0; }
  else if (r < qrows + krows) { src = wk; base = qrows; }
  else { src = wv; base = qrows + krows; }
  const int head = (r - base) / hd, pr = (r - base) % hd;
  const int orow = head * hd + (pr >> 1) + (pr & 1) * (hd / 2);
  const u32x4* s = reinterpret_cast<const u32x4*>(src + (int64_t)orow * rowb);
  u32x4* d = reinterpret_cast<u32x4*>(dst + (int64_t)r * rowb);
  for (int i = threadIdx.x; i < rowb / 16; i += blockDim.x) d[i] = s[i];
}

// Repack: packed gate/up row r <- gate row r/2 (r even) or up row r/2 (r odd)
__global__ void pmk_repack_gu(uint8_t* dst, const uint8_t* wg, const uint8_t* wu, int64_t rowb) {
  const int r = blockIdx.x;
  const uint8_t* src = (r & 1) ? wu : wg;
  const u32x4* s = reinterpret_cast<const u32x4*>(src + (int64_t)(r >> 1) * rowb);
  u32x4* d = reinterpret_cast<u32x4*>(dst + (int64_t)r * rowb);
  for (int i = threadIdx.x; i < rowb / 16; i += blockDim.x) d[i] = s[i];
}

// Integer weight codes, two's complement as loaded -> the kernels' encoding, in place over n 32-bit
// words: int8 bytes to offset binary (q + 128); int4 nibbles to offset binary (q + 8) with the
// nibbles of each word reordered so that positions 0..7 hold columns 0 2 4 6 1 3 5 7.
__global__ void pmk_int_recode(uint32_t* p, int64_t n, int wdt) {
  const int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (i >= n) return;
  const uint32_t w = p[i];
  if (wdt == WI8) {
    p[i] = w ^ 0x80808080u;
    return;
  }
  uint32_t o = 0;
#pragma unroll
  for (int pos = 0; pos < 8; ++pos) {
    const int col = pos < 4 ? 2 * pos : 2 * (pos - 4) + 1;
    o |= ((w >> (4 * col)) & 15u) << (4 * pos);
  }
  p[i] = o ^ 0x88888888u;
}

// 16-bit gain -> fp32
__global__ void pmk_widen(float* dst, const uint16_t* src, int n, int bf16) {
  const int i = blockIdx.x * blockDim.x + threadIdx.x;
  if (i < n) dst[i] = bf16 ? dec16<WBF16>(src[i]) : dec16<WF16>(src[i]);
}

// ------------------------------------------------------------------------------------------------
// static workspace, for callers that cannot allocate device memory
// ------------------------------------------------------------------------------------------------
// One array per device (each device that loads this library holds its own copy until the process
// ends).  Host code never passes the array's name to a kernel or a copy (on the host it names a
// stand-in, not device memory): it takes the device address from hipGetSymbolAddress, once per
// device, with that device current, and uses that address from then on.
static __device__ __align__(256) uint8_t scratch[kStaticWorkspaceBytes];

hipError_t static_workspace_address(int device, void** out) {
  static std::mutex mu;
  static void* addr[kMaxDevices] = {};
  if (device < 0 || device >= kMaxDevices) return hipErrorInvalidDevice;
  std::lock_guard<std::mutex> lock(mu);
  if (!addr[device]) {
    void* p = nullptr;
    const hipError_t e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return e;
    if (p == nullptr || ((uintptr_t)p & 255u)) return hipErrorInvalidSymbol;
    addr[device] = p;
  }
  *out = addr[device];
  return hipSuccess;
}

// ------------------------------------------------------------------------------------------------
// host-visible launch helpers
// ------------------------------------------------------------------------------------------------
typedef void (*KernelFn)(KParams);
typedef void (*PhaseFn)(KParams, int);

template <bool OCOPY>
static const void* persistent_instance(int wdt, int kvdt) {
  if (wdt == WF16 && kvdt == WF16) return (const void*)pmk_persistent<WF16, WF16, OCOPY>;
  if (wdt == WBF16 && kvdt == WBF16) return (const void*)pmk_persistent<WBF16, WBF16, OCOPY>;
  if (wdt == WFP8 && kvdt == WFP8) return (const void*)pmk_persistent<WFP8, WFP8, OCOPY>;
  if (wdt == WI8 && kvdt == WBF16) return (const void*)pmk_persistent<WI8, WBF16, OCOPY>;
  if (wdt == WI4 && kvdt == WBF16) return (const void*)pmk_persistent<WI4, WBF16, OCOPY>;
  return nullptr;
}
const void* persistent_kernel(int wdt, int kvdt, int o_copy) {
  return o_copy ? persistent_instance<true>(wdt, kvdt) : persistent_instance<false>(wdt, kvdt);
}

// batched prefill kernel of a (weight, KV) format pair
const void* prefill_kernel(int wdt, int kvdt) {
  if (wdt == WF16 && kvdt == WF16) return (const void*)pmk_prefill_batch<WF16, WF16>;
  if (wdt == WBF16 && kvdt == WBF16) return (const void*)pmk_prefill_batch<WBF16, WBF16>;
  if (wdt == WFP8 && kvdt == WFP8) return (const void*)pmk_prefill_batch<WFP8, WFP8>;
  if (wdt == WI8 && kvdt == WBF16) return (const void*)pmk_prefill_batch<WI8, WBF16>;
  if (wdt == WI4 && kvdt == WBF16) return (const void*)pmk_prefill_batch<WI4, WBF16>;
  return nullptr;
}

const void* phase_kernel(int wdt, int kvdt) {
  if (wdt == WF16 && kvdt == WF16) return (const void*)pmk_phase<WF16, WF16>;
  if (wdt == WBF16 && kvdt == WBF16) return (const void*)pmk_phase<WBF16, WBF16>;
  if (wdt == WFP8 && kvdt == WFP8) return (const void*)pmk_phase<WFP8, WFP8>;
  if (wdt == WI8 && kvdt == WBF16) return (const void*)pmk_phase<WI8, WBF16>;
  if (wdt == WI4 && kvdt == WBF16) return (const void*)pmk_phase<WI4, WBF16>;
  return nullptr;
}

hipError_t launch_begin_call(const KParams& P, const CallParams& cp, hipStream_t st) {
  hipLaunchKernelGGL(pmk_begin_call, dim3(16), dim3(256), 0, st, P, cp);
  return hipGetLastError();
}
hipError_t launch_reset(const KParams& P, int n_flags, int n_counters, int pos, int token, const int32_t* d_token,
                        hipStream_t st) {
  hipLaunchKernelGGL(pmk_reset, dim3(1), dim3(1024), 0, st, P, n_flags, n_counters, pos, token, d_token);
  return hipGetLastError();
}
hipError_t launch_set_pos(const KParams& P, int pos, const int32_t* d_token, hipStream_t st) {
  hipLaunchKernelGGL(pmk_set_pos, dim3(1), dim3(64), 0, st, P, pos, d_token);
  return hipGetLastError();
}
hipError_t launch_kv_calib(const KParams& P, int finish, hipStream_t st) {
  hipLaunchKernelGGL(pmk_kv_calib, dim3(1), dim3(256), 0, st, P, finish);
  return hipGetLastError();
}
hipError_t launch_copy_token(const KParams& P, int32_t* dst, hipStream_t st) {
  hipLaunchKernelGGL(pmk_copy_token, dim3(1), dim3(64), 0, st, P, dst);
  return hipGetLastError();
}
hipError_t launch_load_kv_rows(const KParams& P, const void* k, const void* v, int npos, int es, hipStream_t st) {
  hipLaunchKernelGGL(pmk_load_kv_rows, dim3(2048), dim3(256), 0, st, P, (const uint8_t*)k, (const uint8_t*)v, npos, es);
  return hipGetLastError();
}
hipError_t launch_read_kv_rows(const KParams& P, void* k, void* v, int npos, int es, hipStream_t st) {
  hipLaunchKernelGGL(pmk_read_kv_rows, dim3(2048), dim3(256), 0, st, P, (uint8_t*)k, (uint8_t*)v, npos, es);
  return hipGetLastError();
}
hipError_t launch_repack_qkv(uint8_t* dst, const void* wq, const void* wk, const void* wv, int nq, int nkv, int hd,
                             int64_t rowb, hipStream_t st) {
  hipLaunchKernelGGL(pmk_repack_qkv, dim3((nq + 2 * nkv) * hd), dim3(256), 0, st, dst, (const uint8_t*)wq,
                     (const uint8_t*)wk, (const uint8_t*)wv, nq, nkv, hd, rowb);
  return hipGetLastError();
}
hipError_t launch_repack_gu(uint8_t* dst, const void* wg, const void* wu, int F, int64_t rowb, hipStream_t st) {
  hipLaunchKernelGGL(pmk_repack_gu, dim3(2 * F), dim3(256), 0, st, dst, (const uint8_t*)wg, (const uint8_t*)wu, rowb);
  return hipGetLastError();
}
hipError_t launch_int_recode(uint8_t* p, int64_t bytes, int wdt, hipStream_t st) {
  const int64_t n = bytes / 4;
  if (n <= 0) return hipSuccess;
  hipLaunchKernelGGL(pmk_int_recode, dim3((unsigned)((n + 255) / 256)), dim3(256), 0, st, reinterpret_cast<uint32_t*>(p),
                     n, wdt);
  return hipGetLastError();
}
hipError_t launch_widen(float* dst, const void* src, int n, int bf16, hipStream_t st) {
  hipLaunchKernelGGL(pmk_widen, dim3((n + 255) / 256), dim3(256), 0, st, dst, (const uint16_t*)src, n, bf16);
  return hipGetLastError();
}

}  // namespace pmk
