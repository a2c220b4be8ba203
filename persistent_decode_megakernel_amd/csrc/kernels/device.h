// Device-side task bodies shared by the persistent megakernel and the unfused ablation kernels.
// gfx950 only: wave64, kWaves (8) waves per workgroup in the megakernel.
//
// Numerics: weights are bf16 (or int8 with per-row fp32 scales) and are converted exactly to
// fp32; activations, accumulations, norms, softmax and residuals are fp32. The exception is the
// batch-1 int8 GEMV, which takes its input as a 23-bit fixed-point integer (one power-of-two
// scale per vector, see stage_digits) and sums the products exactly in int32. Appended K/V rows
// are rounded to bf16 (round to nearest even). Every reduction runs in a fixed order, so results
// do not depend on which CU ran a tile or when.
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "../sched/layout.h"

namespace amk {

struct DevLayer {
  const void *qkv, *o, *gu, *dn;           // packed weights (bf16 bits or int8)
  const float *s_qkv, *s_o, *s_gu, *s_dn;  // scales: per row (int8), per row and group (int4)
  const uint16_t *attn_norm, *mlp_norm;
};

struct DevModel {
  int32_t L, d, nq, nkv, hd, F, V, qkvr, qd, qpg;
  int32_t wtype, tied, max_batch, max_seq;
  int32_t gs;  // int4: inputs per scale group
  int32_t tiled;  // layer matrices (and an untied LM head) are tile-major (weight_tiled_bytes)
  int32_t nblk, n_lm;
  uint32_t n_tasks;
  uint32_t argmax_id;  // the step's last task: every other task of the step precedes it
  float eps, attn_scale;
  const DevLayer *layers;
  const uint16_t *embed, *final_norm;
  const void *lm;
  const float *lm_scale;
  const float2 *rope;  // [max_seq][hd/2] (cos, sin) of pos * theta^(-2j/hd)
  float *h;            // [2L+1][B][d] residual stream (slot 0 unused: the embedding row)
  float *q;            // [L][B][qd]
  float *part;         // [L][B][nq][nblk][hd+2]
  float *ao;           // [L][B][qd] attention output, merged over the KV blocks
  // batch-1 instances: the same activations as tagged fp32 words (tag_word)
  uint32_t *ht;        // [2L+1][d] residual stream
  uint32_t *at;        // [L][F] SwiGLU output
  uint32_t *aot;       // [L][qd] merged attention output
  uint32_t *qt;        // [L][qd] q after RoPE
  uint32_t *kvt;       // [L][2][nkv][hd] the K/V row appended at pos: bf16 bits << 16 | tag
  float *a;            // [L][B][F]
  float *logits;       // [B][V] used when the caller passes no logits buffer
  float2 *amax;        // [n_lm][B] (value, index bits)
  uint32_t *flags;     // [n_tasks]
  // The epoch of the last completed step. A launch reads it once per workgroup at its start and
  // runs step i at epoch + 1 + i; the last step's argmax stores epoch + n_steps. Kept on the
  // device (not a launch argument) so that a captured and replayed launch still advances it.
  uint32_t *ectr;
  uint32_t *err;       // [0] status, [1] abort, [2] task, [3] detail
  const Task *tasks;
  const uint32_t *offsets;
  // unfused-path scratch
  float *xn;    // [B][max(d, qd, F)]
  float *y;     // [B][max(qkvr, 2F, V, d)]
  float *o;     // [B][qd]
  uint64_t timeout_ticks;  // bound of one dependency wait (s_memrealtime ticks, 100 MHz)
  uint64_t *trace;         // optional: [n_tasks][4] timestamps, then [n_cu] XCC ids; null = off
};

// One decode step: tokens at their positions in, next tokens (and optionally logits) out.
// Sequence b is at position pos_in[b] + step (pos = pos_in[0]; positions may differ between
// sequences). A launch may run n_steps consecutive steps (step = 0 .. n_steps-1): step i takes the
// tokens step i-1 wrote, at positions pos_in[b] + i, with flag epoch epoch + i. The device reads
// the positions through posp, which each kernel entry points at its own kernel-argument copy of
// pos_in (a run-time index into a private copy would put the whole struct in scratch memory).
struct StepArgs {
  const int32_t *tokens;
  float *logits;
  int32_t *next;
  uint16_t *kv;
  int32_t kv_batch, kv_max_seq;
  int32_t pos, batch;
  uint32_t epoch;
  int32_t step, n_steps;
  int32_t pos_in[kMaxBatch];
  const int32_t *posp;
  // -1: column b is KV sequence b. Otherwise every column is a position of KV sequence kv_seq
  // (prompt processing: the columns are consecutive tokens of one sequence).
  int32_t kv_seq;
};

constexpr uint32_t ERR_TIMEOUT = 7;
constexpr uint32_t ERR_TOKEN = 8;

// ------------------------------------------------------------------------------------------
// small helpers
// ------------------------------------------------------------------------------------------
__device__ __forceinline__ float bf_lo(uint32_t v) { return __uint_as_float(v << 16); }
__device__ __forceinline__ float bf_hi(uint32_t v) { return __uint_as_float(v & 0xffff0000u); }
__device__ __forceinline__ float bf16_to_f32(uint16_t v) { return __uint_as_float((uint32_t)v << 16); }

// round to nearest even (inputs are finite)
__device__ __forceinline__ uint16_t f32_to_bf16(float f) {
  uint32_t u = __float_as_uint(f);
  u += 0x7fffu + ((u >> 16) & 1u);
  return (uint16_t)(u >> 16);
}

__device__ __forceinline__ int lane_id() { return (int)(threadIdx.x & 63); }

// A wave-uniform value moved to a scalar register (the builtin takes and returns int).
__device__ __forceinline__ uint32_t uniform_u32(uint32_t v) {
  return (uint32_t)__builtin_amdgcn_readfirstlane((int)v);
}
__device__ __forceinline__ int wave_id() { return (int)(threadIdx.x >> 6); }

// butterfly sum over the 64 lanes; every lane receives the total
__device__ __forceinline__ float wave_sum(float v) {
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) v += __shfl_xor(v, o, 64);
  return v;
}
__device__ __forceinline__ float wave_max(float v) {
#pragma unroll
  for (int o = 32; o >= 1; o >>= 1) v = fmaxf(v, __shfl_xor(v, o, 64));
  return v;
}

// a lane's value from another lane of its 16-lane row (DPP control CTRL, every lane active)
template <int CTRL>
__device__ __forceinline__ float dpp_f(float v) {
  return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), CTRL, 0xF, 0xF, false));
}
// sum over aligned groups of G lanes (G = 2, 4, 8 or 16, within a 16-lane row), every lane of a
// group receiving it: lane ^ 1 and lane ^ 2 (quad_perm), then the mirrored half-row and row,
// which pair groups already summed. No LDS round trip, unlike a shuffle.
template <int G>
__device__ __forceinline__ float group_sum(float v) {
  static_assert(G == 2 || G == 4 || G == 8 || G == 16, "group of 2 to 16 lanes");
  v += dpp_f<0xB1>(v);                    // quad_perm(1,0,3,2)
  if constexpr (G >= 4) v += dpp_f<0x4E>(v);   // quad_perm(2,3,0,1)
  if constexpr (G >= 8) v += dpp_f<0x141>(v);  // row_half_mirror
  if constexpr (G >= 16) v += dpp_f<0x140>(v); // row_mirror
  return v;
}

// the value of lane ^ o (o a power of two below 64, known at compile time after unrolling): DPP
// row_ror:8 for o = 8, a shuffle otherwise
__device__ __forceinline__ float xor_lanes(float v, int o) {
  return o == 8 ? dpp_f<0x128>(v) : __shfl_xor(v, o, 64);
}

// max over the 64 lanes of non-negative values, every lane receives it: DPP within rows of 16
// lanes (float bits of non-negative values order as integers), then the four row maxima
__device__ __forceinline__ float wave_max_nonneg(float v) {
  int x = __float_as_int(v);
  x = max(x, __builtin_amdgcn_update_dpp(0, x, 0xB1, 0xF, 0xF, false));   // quad_perm(1,0,3,2)
  x = max(x, __builtin_amdgcn_update_dpp(0, x, 0x4E, 0xF, 0xF, false));   // quad_perm(2,3,0,1)
  x = max(x, __builtin_amdgcn_update_dpp(0, x, 0x141, 0xF, 0xF, false));  // row_half_mirror
  x = max(x, __builtin_amdgcn_update_dpp(0, x, 0x140, 0xF, 0xF, false));  // row_mirror
  const int a = max(__builtin_amdgcn_readlane(x, 0), __builtin_amdgcn_readlane(x, 16));
  const int b = max(__builtin_amdgcn_readlane(x, 32), __builtin_amdgcn_readlane(x, 48));
  return __int_as_float(max(a, b));
}

// sum over the threads of a workgroup of nw waves; red = LDS scratch of >= nw floats.
// Every thread receives the total (fixed order: waves summed 0..nw-1).
__device__ __forceinline__ float block_sum(float v, float *red, int nw) {
  v = wave_sum(v);
  __syncthreads();
  if (lane_id() == 0) red[wave_id()] = v;
  __syncthreads();
  float t = 0.f;
  for (int w = 0; w < nw; ++w) t += red[w];
  return t;
}

__device__ __forceinline__ float silu(float z) { return z / (1.0f + __expf(-z)); }

__device__ __forceinline__ float dot8_bf16(const uint4 w, const float *x) {
  const float4 x0 = *reinterpret_cast<const float4 *>(x);
  const float4 x1 = *reinterpret_cast<const float4 *>(x + 4);
  float a = bf_lo(w.x) * x0.x;
  float b = bf_hi(w.x) * x0.y;
  a = fmaf(bf_lo(w.y), x0.z, a);
  b = fmaf(bf_hi(w.y), x0.w, b);
  a = fmaf(bf_lo(w.z), x1.x, a);
  b = fmaf(bf_hi(w.z), x1.y, b);
  a = fmaf(bf_lo(w.w), x1.z, a);
  b = fmaf(bf_hi(w.w), x1.w, b);
  return a + b;
}

// 16 int8 weights (two's complement) dotted with 16 floats.
__device__ __forceinline__ float dot16_i8(const uint4 w, const float *x) {
  float a = 0.f, b = 0.f;
  const uint32_t ws[4] = {w.x, w.y, w.z, w.w};
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const float4 xv = *reinterpret_cast<const float4 *>(x + 4 * i);
    const int32_t v = (int32_t)ws[i];
    a = fmaf((float)((v << 24) >> 24), xv.x, a);
    b = fmaf((float)((v << 16) >> 24), xv.y, b);
    a = fmaf((float)((v << 8) >> 24), xv.z, a);
    b = fmaf((float)(v >> 24), xv.w, b);
  }
  return a + b;
}

// 32 int4 weights (one 16-byte unit) dotted with 32 floats. Nibble order within each 32-bit word
// (the library's repacked layout): byte j holds input j in its low and input j + 4 in its high
// nibble, so word i covers inputs 8i .. 8i + 7.
__device__ __forceinline__ float dot32_i4(const uint4 w, const float *x) {
  float a = 0.f, b = 0.f;
  const uint32_t ws[4] = {w.x, w.y, w.z, w.w};
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int32_t v = (int32_t)ws[i];
    const float4 xl = *reinterpret_cast<const float4 *>(x + 8 * i);
    const float4 xh = *reinterpret_cast<const float4 *>(x + 8 * i + 4);
    a = fmaf((float)((v << 28) >> 28), xl.x, a);
    b = fmaf((float)((v << 24) >> 28), xh.x, b);
    a = fmaf((float)((v << 20) >> 28), xl.y, a);
    b = fmaf((float)((v << 16) >> 28), xh.y, b);
    a = fmaf((float)((v << 12) >> 28), xl.z, a);
    b = fmaf((float)((v << 8) >> 28), xh.z, b);
    a = fmaf((float)((v << 4) >> 28), xl.w, a);
    b = fmaf((float)(v >> 28), xh.w, b);
  }
  return a + b;
}

// Global-memory accesses. Pointers held in DevModel are generic (flat) to the compiler; flat
// accesses count against both vmcnt and lgkmcnt, so every LDS access would also wait for all
// outstanding global loads. Casting to the global address space keeps the two counters apart.
#define AMK_GAS __attribute__((address_space(1)))
typedef uint32_t u32x4_t __attribute__((ext_vector_type(4)));
template <typename T>
__device__ __forceinline__ const AMK_GAS T *gptr(const T *p) {
  return (const AMK_GAS T *)p;
}
template <typename T>
__device__ __forceinline__ AMK_GAS T *gptr(T *p) {
  return (AMK_GAS T *)p;
}
template <typename T>
__device__ __forceinline__ T gld(const T *p) { return *gptr(p); }
template <typename T>
__device__ __forceinline__ void gst(T *p, T v) { *gptr(p) = v; }
// Device-coherent accesses for data that another CU reads or wrote within the same launch
// (residual stream, q, the appended KV row, attention partials, SwiGLU output, argmax partials).
// They are device-scope ("sc1") loads and stores: they do not hit a possibly stale copy in
// another XCD's L2 and stores write through, so a producer only has to wait for its own stores
// to complete before publishing its flag, and a consumer needs no cache invalidation after
// observing it. This replaces whole-L2 writeback/invalidate fences at every dependency.
template <typename T>
__device__ __forceinline__ T cld(const T *p) {
  return __hip_atomic_load(gptr(p), __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
template <typename T>
__device__ __forceinline__ void cst(T *p, T v) {
  __hip_atomic_store(gptr(p), v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ float cldf(const float *p) {
  return __uint_as_float(cld(reinterpret_cast<const uint32_t *>(p)));
}
__device__ __forceinline__ void cstf(float *p, float v) {
  cst(reinterpret_cast<uint32_t *>(p), __float_as_uint(v));
}
__device__ __forceinline__ uint4 load_nt(const uint4 *p) {
  const u32x4_t v = __builtin_nontemporal_load((const AMK_GAS u32x4_t *)p);
  return make_uint4(v.x, v.y, v.z, v.w);
}
__device__ __forceinline__ uint4 gld4(const uint4 *p) {
  const u32x4_t v = *(const AMK_GAS u32x4_t *)p;
  return make_uint4(v.x, v.y, v.z, v.w);
}
// 16-byte device-coherent loads go through a raw buffer resource: the buffer intrinsics take a
// cache-policy operand, plain pointer loads of 16 bytes cannot carry the device-scope bit.
// Word 3 of the resource selects the 32-bit data format (the only field untyped loads use);
// offsets at or beyond `bytes` read as zero instead of faulting.
typedef float f32x4_t __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2_t __attribute__((ext_vector_type(2)));
// 4 bf16 values (8 bytes) at p[i4 * 4 ..] as two packed words
__device__ __forceinline__ uint2 gld_bf16x4(const uint16_t *p, int i4) {
  const u32x2_t v = *((const AMK_GAS u32x2_t *)p + i4);
  return make_uint2(v.x, v.y);
}
constexpr int kRsrcWord3 = 0x00020000;
constexpr int kCachePolicyNt = 2;
constexpr int kCachePolicySc1 = 16;
// s_waitcnt immediates (gfx9 layout: vmcnt[3:0] | expcnt[6:4] | lgkmcnt[11:8] | vmcnt[5:4] at
// [15:14]) waiting on vector memory only
constexpr int kWaitVm0 = 0x0F70;
constexpr int kWaitVm8 = 0x0F78;
constexpr int kWaitVm16 = 0x4F70;  // vmcnt 16: its bits 5:4 sit in bits 15:14
#define AMK_LDS __attribute__((address_space(3)))
// A buffer resource must sit in scalar registers: every caller passes wave-uniform values, and
// taking them from the first lane lets the compiler see that (otherwise it may keep the resource in
// vector registers and wrap every load in a loop over its distinct values).
__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc(const void *base, uint32_t bytes) {
  // (the builtin returns a signed int: address_from_words widens each half without sign extension)
  const uint64_t a = reinterpret_cast<uint64_t>(base);
  const uint64_t u = address_from_words(__builtin_amdgcn_readfirstlane((int)(uint32_t)(a >> 32)),
                                        __builtin_amdgcn_readfirstlane((int)(uint32_t)a));
  return __builtin_amdgcn_make_buffer_rsrc(reinterpret_cast<void *>(u), 0,
                                           __builtin_amdgcn_readfirstlane((int)bytes), kRsrcWord3);
}
__device__ __forceinline__ float4 cld4(__amdgpu_buffer_rsrc_t r, uint32_t off_bytes) {
  const f32x4_t v = __builtin_bit_cast(
      f32x4_t, __builtin_amdgcn_raw_buffer_load_b128(r, (int)off_bytes, 0, kCachePolicySc1));
  return make_float4(v.x, v.y, v.z, v.w);
}

// The per-CU task tables do not change during a launch: read them through the constant address
// space, so the (uniform) loads are scalar. A vector load here would have to wait until the
// previous task's outstanding stores complete (loads and stores share the vector memory count),
// delaying every task start by the store latency.
#define AMK_CAS __attribute__((address_space(4)))
typedef uint32_t u32x4c_t __attribute__((ext_vector_type(4)));
__device__ __forceinline__ Task load_task(const Task *p) {
  static_assert(sizeof(Task) == 48, "task record size");
  const AMK_CAS u32x4c_t *q = (const AMK_CAS u32x4c_t *)p;
  const u32x4c_t w[3] = {q[0], q[1], q[2]};
  Task t;
  __builtin_memcpy(&t, w, sizeof t);
  return t;
}
__device__ __forceinline__ uint32_t load_const(const uint32_t *p) { return *(const AMK_CAS uint32_t *)p; }

// position of sequence b in this step
__device__ __forceinline__ int pos_of(const StepArgs &s, int b) {
  return (int)load_const(reinterpret_cast<const uint32_t *>(s.posp + b)) + s.step;
}
// a kernel's arguments with posp pointing at their own positions
__device__ __forceinline__ StepArgs with_positions(const StepArgs &s) {
  StepArgs t = s;
  t.posp = &s.pos_in[0];
  return t;
}

// ------------------------------------------------------------------------------------------
// dependency flags
// ------------------------------------------------------------------------------------------
__device__ __forceinline__ uint32_t flag_load(const uint32_t *p) {
  return __hip_atomic_load(gptr(p), __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

__device__ __forceinline__ void record_error(uint32_t *err, uint32_t code, uint32_t task,
                                             uint32_t detail) {
  uint32_t expected = 0;
  if (__hip_atomic_compare_exchange_strong(gptr(&err[0]), &expected, code, __ATOMIC_RELAXED,
                                           __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT)) {
    __hip_atomic_store(gptr(&err[2]), task, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    __hip_atomic_store(gptr(&err[3]), detail, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  }
}

// Called by one whole wave. Spins until flags[lo..hi) all reached `epoch`. Each poll round
// issues the loads for up to 512 flags (8 per lane, indices clamped into the range) before
// testing any of them, so a round costs one memory latency whatever the range's size. Returns
// false (after recording the error and raising the abort flag) when the wait exceeds the timeout
// or another workgroup has aborted.
__device__ bool wait_range(const DevModel &m, uint32_t lo, uint32_t hi, uint32_t epoch,
                           uint32_t task) {
  constexpr int kPer = 8;
  const uint32_t lane = (uint32_t)lane_id();
  uint64_t t0 = 0;
  for (uint32_t g = lo; g < hi; g += 64 * kPer) {
    const uint32_t last = min(hi, g + 64 * kPer) - 1;
    uint32_t spins = 0;
    while (true) {
      uint32_t v[kPer];
#pragma unroll
      for (int j = 0; j < kPer; ++j) v[j] = flag_load(&m.flags[min(g + lane + 64u * j, last)]);
      bool ok = true;
#pragma unroll
      for (int j = 0; j < kPer; ++j) ok = ok && (int32_t)(v[j] - epoch) >= 0;
      if (__all(ok)) break;
      if (spins == 0) t0 = wall_clock64();
      ++spins;
      if ((spins & 15) == 0) {
        if (flag_load(&m.err[1]) != 0) return false;
        if (wall_clock64() - t0 > m.timeout_ticks) {
          if (lane == 0) {
            record_error(m.err, ERR_TIMEOUT, task, g);
            __hip_atomic_store(gptr(&m.err[1]), 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
          }
          return false;
        }
      }
      __builtin_amdgcn_s_sleep(1);
    }
  }
  // No acquire fence: everything a task reads that was produced in this launch is read with
  // device-coherent loads, ordered after the flag observation.
  return true;
}

// Dependency wait of a task in two halves: wait_poll (wave 0 spins on the task's flag ranges;
// other waves return at once) and wait_join (the workgroup meets at a barrier; false on every
// thread when the wait timed out or the step was aborted). Work placed between the two runs on
// waves 1.. before the flags are seen and on wave 0 after.
__device__ __forceinline__ void wait_poll(const DevModel &m, const Task &t, uint32_t epoch,
                                          int *abort_slot) {
  if (wave_id() == 0) {
    bool ok = true;
    if (t.w0_hi > t.w0_lo) ok = wait_range(m, t.w0_lo, t.w0_hi, epoch, t.id);
    if (ok && t.w1_hi > t.w1_lo) ok = wait_range(m, t.w1_lo, t.w1_hi, epoch, t.id);
    if (lane_id() == 0) *abort_slot = ok ? 0 : 1;
  }
}
__device__ __forceinline__ bool wait_join(const DevModel &m, const Task &t, int *abort_slot) {
  __syncthreads();
  if (m.trace && threadIdx.x == 0) gst(&m.trace[(uint64_t)t.id * 4 + 1], (uint64_t)wall_clock64());
  return *abort_slot == 0;
}
__device__ __forceinline__ bool wait_task(const DevModel &m, const Task &t, uint32_t epoch,
                                          int *abort_slot) {
  wait_poll(m, t, epoch, abort_slot);
  return wait_join(m, t, abort_slot);
}

// ------------------------------------------------------------------------------------------
// GEMV core: ys[r - r0] = sum_k W[r, k] * xs[k] for r in [r0, r1), one wave per row in turn.
// W row-major [rows, K]; xs in LDS (K floats). Rows are dealt to waves round-robin. The K loop
// issues U 16-byte loads per lane before consuming them.
// ------------------------------------------------------------------------------------------
template <int U>
__device__ __forceinline__ float row_dot_bf16(const uint16_t *__restrict__ W, int64_t row, int K,
                                              const float *xs) {
  const uint4 *wr = reinterpret_cast<const uint4 *>(W + row * (int64_t)K);
  const int n16 = K >> 3;
  const int lane = lane_id();
  float acc = 0.f;
  for (int u0 = 0; u0 < n16; u0 += 64 * U) {
    uint4 w[U];
#pragma unroll
    for (int j = 0; j < U; ++j) {
      const int u = u0 + j * 64 + lane;
      w[j] = (u < n16) ? load_nt(wr + u) : make_uint4(0, 0, 0, 0);
    }
#pragma unroll
    for (int j = 0; j < U; ++j) {
      const int u = u0 + j * 64 + lane;
      if (u < n16) acc += dot8_bf16(w[j], xs + 8 * u);
    }
  }
  return wave_sum(acc);
}

template <int U>
__device__ __forceinline__ float row_dot_i8(const int8_t *__restrict__ W, int64_t row, int K,
                                            const float *xs) {
  const uint4 *wr = reinterpret_cast<const uint4 *>(W + row * (int64_t)K);
  const int n16 = K >> 4;
  const int lane = lane_id();
  float acc = 0.f;
  for (int u0 = 0; u0 < n16; u0 += 64 * U) {
    uint4 w[U];
#pragma unroll
    for (int j = 0; j < U; ++j) {
      const int u = u0 + j * 64 + lane;
      w[j] = (u < n16) ? load_nt(wr + u) : make_uint4(0, 0, 0, 0);
    }
#pragma unroll
    for (int j = 0; j < U; ++j) {
      const int u = u0 + j * 64 + lane;
      if (u < n16) acc += dot16_i8(w[j], xs + 16 * u);
    }
  }
  return wave_sum(acc);
}

// int4 row: each 16-byte unit (32 inputs) times its group's scale
__device__ __forceinline__ float row_dot_i4(const uint8_t *__restrict__ W, const float *scale,
                                            int gs, int64_t row, int K, const float *xs) {
  const uint4 *wr = reinterpret_cast<const uint4 *>(W + row * (int64_t)(K / 2));
  const float *sr = scale + row * (int64_t)(K / gs);
  const int n32 = K >> 5, upg = gs >> 5;
  const int lane = lane_id();
  float acc = 0.f;
  for (int u = lane; u < n32; u += 64) acc = fmaf(gld(&sr[u / upg]), dot32_i4(load_nt(wr + u), xs + 32 * u), acc);
  return wave_sum(acc);
}

// rows [r0, r1) of a matrix for B staged vectors (xs + b*K); ys[b*(r1-r0) + r - r0].
// WT = 0: bf16 weights; WT = 1: int8 weights times scale[r]; WT = 2: int4 weights, scale[r][g]
// per group of gs inputs.
template <int WT>
__device__ void gemv_rows(const void *W, const float *scale, int K, int r0, int r1,
                          const float *xs, float *ys, int B, int nw, int gs = 0) {
  const int n = r1 - r0;
  for (int i = wave_id(); i < n; i += nw) {
    const int64_t r = r0 + i;
    for (int b = 0; b < B; ++b) {
      float v;
      if constexpr (WT == 2)
        v = row_dot_i4(static_cast<const uint8_t *>(W), scale, gs, r, K, xs + (int64_t)b * K);
      else if constexpr (WT == 1)
        v = row_dot_i8<4>(static_cast<const int8_t *>(W), r, K, xs + (int64_t)b * K) * gld(&scale[r]);
      else
        v = row_dot_bf16<8>(static_cast<const uint16_t *>(W), r, K, xs + (int64_t)b * K);
      if (lane_id() == 0) ys[b * n + i] = v;
    }
  }
}

// ------------------------------------------------------------------------------------------
// Batch-1 GEMV as a per-wave stream of 8 KB chunks (64 lanes x 8 units of 16 bytes). A wave owns
// rows r0 + wave, r0 + wave + nw, ...; each row is nch chunks. Two register buffers alternate so
// one chunk is always in flight while the other is consumed, and the first chunk can be issued
// before the task's dependency wait (weights never depend on the step's activations).
// WT = 0: bf16 (8 weights per unit); WT = 1: int8 (16 weights per unit, times scale[row]).
// ------------------------------------------------------------------------------------------
constexpr int kChunkUnits = 8;

template <int WT>
struct GemvStream {
  const uint8_t *W;
  int K, r0, r1, nw, n16, nch, S;
  int wave, lane;

  __device__ __forceinline__ void init(const void *w, int k, int a, int b, int nwaves) {
    constexpr int EPU = WT ? 16 : 8;
    W = static_cast<const uint8_t *>(w);
    K = k;
    r0 = a;
    r1 = b;
    nw = nwaves;
    wave = __builtin_amdgcn_readfirstlane(wave_id());  // uniform: keeps the loop scalar
    lane = lane_id();
    n16 = K / EPU;
    nch = (n16 + 64 * kChunkUnits - 1) / (64 * kChunkUnits);
    const int n = r1 - r0;
    const int rows_w = (n > wave) ? (n - wave + nw - 1) / nw : 0;
    S = rows_w * nch;
  }
  __device__ __forceinline__ int row_of(int s) const { return r0 + wave + (s / nch) * nw; }
  // Loads are unconditional (the ragged tail re-reads the row's last unit and is discarded in
  // consume): a per-lane branch here would make the compiler wait for every outstanding load
  // before each use, which serialises the two buffers.
  __device__ __forceinline__ void load(uint4 (&buf)[kChunkUnits], int s) const {
    const int row = row_of(s), c = s % nch;
    const uint4 *rp = reinterpret_cast<const uint4 *>(W + (int64_t)row * K * (WT ? 1 : 2));
    const int base = c * 64 * kChunkUnits + lane;
#pragma unroll
    for (int j = 0; j < kChunkUnits; ++j) buf[j] = load_nt(rp + min(base + j * 64, n16 - 1));
  }
  // chunk s straight into LDS, bypassing registers: 16 bytes per lane per instruction, lane i's
  // bytes at dst + 16 i (dst: this wave's 8 KB slot)
  __device__ __forceinline__ void load_lds(int s, uint4 *dst) const {
    const int row = row_of(s), c = s % nch;
    const uint4 *rp = reinterpret_cast<const uint4 *>(W + (int64_t)row * K * (WT ? 1 : 2));
    const int base = c * 64 * kChunkUnits + lane;
#pragma unroll
    for (int j = 0; j < kChunkUnits; ++j)
      __builtin_amdgcn_global_load_lds((const AMK_GAS void *)(rp + min(base + j * 64, n16 - 1)),
                                       (AMK_LDS void *)(dst + j * 64), 16, 0, kCachePolicyNt);
  }
  // accumulate chunk s; at the end of a row reduce over the wave and store ys[row - r0]
  __device__ __forceinline__ void consume(const uint4 (&buf)[kChunkUnits], int s, float &acc,
                                          const float *xs, float *ys, const float *scale) const {
    constexpr int EPU = WT ? 16 : 8;
    const int c = s % nch;
    const int base = c * 64 * kChunkUnits + lane;
#pragma unroll
    for (int j = 0; j < kChunkUnits; ++j) {
      const int u = base + j * 64;
      const float *xp = xs + EPU * min(u, n16 - 1);
      float d;
      if constexpr (WT == 1)
        d = dot16_i8(buf[j], xp);
      else
        d = dot8_bf16(buf[j], xp);
      acc += (u < n16) ? d : 0.f;
    }
    if (c == nch - 1) {
      const int row = row_of(s);
      float v = wave_sum(acc);
      if constexpr (WT == 1) v *= gld(&scale[row]);
      if (lane == 0) ys[row - r0] = v;
      acc = 0.f;
    }
  }
  // Run the stream with two chunks issued before the dependency wait: chunk 0 in this wave's LDS
  // slot pf (load_lds), chunk 1 in P. Chunk 2 is issued first, then the LDS chunk is consumed
  // once the vector-memory count shows its copy done (loads complete in issue order).
  __device__ __forceinline__ void run_pf(const uint4 *pf, const uint4 (&P)[kChunkUnits],
                                         const float *xs, float *ys, const float *scale) const {
    if (S == 0) return;
    float acc = 0.f;
    uint4 A[kChunkUnits], Bf[kChunkUnits];
    if (S > 2) {
      load(A, 2);
      __builtin_amdgcn_s_waitcnt(kWaitVm8);
    } else {
      __builtin_amdgcn_s_waitcnt(kWaitVm0);
    }
#pragma unroll
    for (int j = 0; j < kChunkUnits; ++j) Bf[j] = pf[j * 64 + lane];
    consume(Bf, 0, acc, xs, ys, scale);
    if (S == 1) return;
    consume(P, 1, acc, xs, ys, scale);
    if (S == 2) return;
    int s = 2;
    for (; s + 2 < S; s += 2) {
      load(Bf, s + 1);
      consume(A, s, acc, xs, ys, scale);
      load(A, s + 2);
      consume(Bf, s + 1, acc, xs, ys, scale);
    }
    if (s + 1 < S) {
      load(Bf, s + 1);
      consume(A, s, acc, xs, ys, scale);
      consume(Bf, s + 1, acc, xs, ys, scale);
    } else {
      consume(A, s, acc, xs, ys, scale);
    }
  }
  // Run the stream. P holds chunk 0, loaded before the task's dependency wait and complete by
  // now. It is consumed before the steady-state loop, which then starts (and loops back) with
  // exactly one buffer of loads in flight: the compiler's wait-count tracking stays exact across
  // the back edge only when entry and back edge carry the same pending loads.
  __device__ __forceinline__ void run(const uint4 (&P)[kChunkUnits], const float *xs, float *ys,
                                      const float *scale) const {
    if (S == 0) return;
    float acc = 0.f;
    if (S == 1) {
      consume(P, 0, acc, xs, ys, scale);
      return;
    }
    uint4 A[kChunkUnits], Bf[kChunkUnits];
    load(A, 1);
    consume(P, 0, acc, xs, ys, scale);
    int s = 1;
    for (; s + 2 < S; s += 2) {
      load(Bf, s + 1);
      consume(A, s, acc, xs, ys, scale);
      load(A, s + 2);
      consume(Bf, s + 1, acc, xs, ys, scale);
    }
    if (s + 1 < S) {
      load(Bf, s + 1);
      consume(A, s, acc, xs, ys, scale);
      consume(Bf, s + 1, acc, xs, ys, scale);
    } else {
      consume(A, s, acc, xs, ys, scale);
    }
  }
};

// ------------------------------------------------------------------------------------------
// Batch-1 int8 GEMV over integer digits of the input
// ------------------------------------------------------------------------------------------
// The staged input x (K fp32 values in LDS) is rounded once per task to fixed-point integers
// X_k = rint(x_k 2^(22-e)), with 2^e > max|x| so that |X_k| <= 2^22, and each X_k is split into
// balanced base-256 digits X = 65536 d2 + 256 d1 + d0, every digit in [-128, 127]. A row's dot
// product with its int8 weights q is then three exact int32 sums A_p = sum_k q_k d_p,k (v_dot4:
// four int8 products per instruction, no conversion of the weights) and
//   sum_k q_k x_k  ~=  2^(e-22) (65536 A2 + 256 A1 + A0),
// where |x_k - X_k 2^(e-22)| <= 2^(e-23) <= 2^-22 max|x|: the input is rounded 14 bits finer
// than bf16. |A_p| <= 128 * 127 * K stays within int32 for K <= 2^17.
// LDS layout, unit-interleaved: unit u (elements 16u .. 16u+15) holds d2[16], d1[16], d0[16] at
// byte 48u, so a lane's three 16-byte reads share one address and lanes 48 bytes apart fall on
// distinct banks; the 96 bytes after the last unit are zero, and lanes past a row's end read them.
// The digits overwrite the fp32 input (3K + 96 <= 4K bytes); every thread holds its share in
// registers across a barrier before any digit is written, which bounds K by kDigitMaxK.
constexpr int kDigitRedSlot = kRedFloats - kWaves;  // red[] floats that hold the per-wave maxima

// The digit scale from the per-wave maxima of |x| in red (published before a barrier): returns
// 2^(22-e), the factor that takes x to its digit integer.
__device__ __forceinline__ float digit_up(const float *red, int *e_out) {
  const AMK_LDS float *rm = (const AMK_LDS float *)red + kDigitRedSlot;
  float top = 0.f;
#pragma unroll
  for (int w = 0; w < kWaves; ++w) top = fmaxf(top, rm[w]);
  int e;
  frexpf(top, &e);  // top < 2^e (top = 0: e = 0)
  *e_out = e;
  return ldexpf(1.0f, 22 - e);
}
// The digits of four consecutive elements 4i .. 4i+3 into the digit layout.
__device__ __forceinline__ void put_digits(float *xs, int i, float a, float b, float c, float d,
                                           float up) {
  const float f[4] = {a, b, c, d};
  uint32_t w2 = 0, w1 = 0, w0 = 0;
#pragma unroll
  for (int k = 0; k < 4; ++k) {
    const int X = (int)rintf(f[k] * up);
    const int d0 = (int)(int8_t)(X & 0xff);
    const int X1 = (X - d0) >> 8;  // exact: X - d0 is a multiple of 256
    const int d1 = (int)(int8_t)(X1 & 0xff);
    const int d2 = (X1 - d1) >> 8;  // |d2| <= 65
    w0 |= (uint32_t)(d0 & 0xff) << (8 * k);
    w1 |= (uint32_t)(d1 & 0xff) << (8 * k);
    w2 |= (uint32_t)(d2 & 0xff) << (8 * k);
  }
  AMK_LDS uint32_t *p = (AMK_LDS uint32_t *)((AMK_LDS uint8_t *)xs + 48 * (i >> 2) + 4 * (i & 3));
  p[0] = w2;
  p[4] = w1;
  p[8] = w0;
}
// 96 zero bytes after the last unit: one int8 digit unit of 16 inputs, or the int4 one of 32
__device__ __forceinline__ void put_zero_unit(float *xs, int K) {
  if (threadIdx.x < 24) ((AMK_LDS uint32_t *)((AMK_LDS uint8_t *)xs + 48 * (K >> 4)))[threadIdx.x] = 0u;
}

// In place, for an input already staged as fp32 in xs: returns 2^(e-22), the weight of one unit
// of the digit integers.
__device__ __forceinline__ float stage_digits(float *xs, int K, float *red) {
  constexpr int R = kDigitMaxK / 4 / kThreads;
  const int n4 = K >> 2;
  const AMK_LDS u32x4_t *x4 = (const AMK_LDS u32x4_t *)xs;
  float4 v[R];
  float mx = 0.f;
#pragma unroll
  for (int j = 0; j < R; ++j) {
    const int i = (int)threadIdx.x + j * kThreads;
    v[j] = make_float4(0.f, 0.f, 0.f, 0.f);
    if (i < n4) {
      const u32x4_t r = x4[i];
      v[j] = make_float4(__uint_as_float(r.x), __uint_as_float(r.y), __uint_as_float(r.z),
                         __uint_as_float(r.w));
    }
    mx = fmaxf(mx, fmaxf(fmaxf(fabsf(v[j].x), fabsf(v[j].y)), fmaxf(fabsf(v[j].z), fabsf(v[j].w))));
  }
  mx = wave_max_nonneg(mx);
  if (lane_id() == 0) ((AMK_LDS float *)red)[kDigitRedSlot + wave_id()] = mx;
  __syncthreads();
  int e;
  const float up = digit_up(red, &e);
#pragma unroll
  for (int j = 0; j < R; ++j) {
    const int i = (int)threadIdx.x + j * kThreads;
    if (i < n4) put_digits(xs, i, v[j].x, v[j].y, v[j].z, v[j].w, up);
  }
  put_zero_unit(xs, K);
  __syncthreads();
  return ldexpf(1.0f, e - 22);
}

// The int8 stream itself: the same per-wave chunks, register double buffering and LDS prefetch as
// GemvStream, with RPC rows per chunk. RPC = 1: a row is nch chunks and lanes past its end read
// the zero digit unit. RPC > 1 (rows of exactly 64 * kChunkUnits / RPC units, e.g. K = 4096 with
// RPC = 2): unit slot j of a lane belongs to row slot j / UPL, so no chunk is half empty.
template <int RPC>
struct GemvStreamI8 {
  static constexpr int UPL = kChunkUnits / RPC;  // units per lane per row in one chunk
  const uint8_t *W;
  int K, r0, nw, n16, nch, S, rows_w;
  int wave, lane;

  __device__ __forceinline__ void init(const void *w, const float *, int, int k, int a, int b,
                                       int nwaves) {
    W = static_cast<const uint8_t *>(w);
    K = k;
    r0 = a;
    nw = nwaves;
    wave = __builtin_amdgcn_readfirstlane(wave_id());
    lane = lane_id();
    n16 = K / 16;
    nch = RPC == 1 ? (n16 + 64 * kChunkUnits - 1) / (64 * kChunkUnits) : 1;
    const int n = b - a;
    rows_w = (n > wave) ? (n - wave + nw - 1) / nw : 0;
    S = RPC == 1 ? rows_w * nch : (rows_w + RPC - 1) / RPC;
  }
  // index, in this wave's row list, of row slot q of chunk s, and the row an index names (an
  // index past the wave's last row re-reads that row; its result is dropped)
  __device__ __forceinline__ int slot_idx(int s, int q) const { return RPC == 1 ? s / nch : s * RPC + q; }
  __device__ __forceinline__ int row_at(int i) const { return r0 + wave + min(i, rows_w - 1) * nw; }
  __device__ __forceinline__ int unit_of(int s, int j) const {
    return RPC == 1 ? (s % nch) * 64 * kChunkUnits + lane + 64 * j : lane + 64 * (j % UPL);
  }
  __device__ __forceinline__ const uint4 *unit_ptr(int s, int j) const {
    const int row = row_at(slot_idx(s, j / UPL));
    return reinterpret_cast<const uint4 *>(W + (int64_t)row * K) + min(unit_of(s, j), n16 - 1);
  }
  __device__ __forceinline__ void load(uint4 (&buf)[kChunkUnits], int s) const {
#pragma unroll
    for (int j = 0; j < kChunkUnits; ++j) buf[j] = load_nt(unit_ptr(s, j));
  }
  __device__ __forceinline__ void load_lds(int s, uint4 *dst) const {
#pragma unroll
    for (int j = 0; j < kChunkUnits; ++j)
      __builtin_amdgcn_global_load_lds((const AMK_GAS void *)unit_ptr(s, j),
                                       (AMK_LDS void *)(dst + j * 64), 16, 0, kCachePolicyNt);
  }
  __device__ __forceinline__ void consume(const uint4 (&buf)[kChunkUnits], int s, int (&acc)[RPC][3],
                                          const uint8_t *xd, float sx, float *ys,
                                          const float *scale) const {
#pragma unroll
    for (int j = 0; j < kChunkUnits; ++j) {
      const int q = j / UPL;
      const int u = unit_of(s, j);
      const AMK_LDS u32x4_t *dp =
          (const AMK_LDS u32x4_t *)((const AMK_LDS uint8_t *)xd + 48 * (RPC == 1 ? min(u, n16) : u));
      const u32x4_t d2 = dp[0], d1 = dp[1], d0 = dp[2];
      const uint4 w = buf[j];
      acc[q][0] = __builtin_amdgcn_sdot4((int)w.x, (int)d2.x, acc[q][0], false);
      acc[q][1] = __builtin_amdgcn_sdot4((int)w.x, (int)d1.x, acc[q][1], false);
      acc[q][2] = __builtin_amdgcn_sdot4((int)w.x, (int)d0.x, acc[q][2], false);
      acc[q][0] = __builtin_amdgcn_sdot4((int)w.y, (int)d2.y, acc[q][0], false);
      acc[q][1] = __builtin_amdgcn_sdot4((int)w.y, (int)d1.y, acc[q][1], false);
      acc[q][2] = __builtin_amdgcn_sdot4((int)w.y, (int)d0.y, acc[q][2], false);
      acc[q][0] = __builtin_amdgcn_sdot4((int)w.z, (int)d2.z, acc[q][0], false);
      acc[q][1] = __builtin_amdgcn_sdot4((int)w.z, (int)d1.z, acc[q][1], false);
      acc[q][2] = __builtin_amdgcn_sdot4((int)w.z, (int)d0.z, acc[q][2], false);
      acc[q][0] = __builtin_amdgcn_sdot4((int)w.w, (int)d2.w, acc[q][0], false);
      acc[q][1] = __builtin_amdgcn_sdot4((int)w.w, (int)d1.w, acc[q][1], false);
      acc[q][2] = __builtin_amdgcn_sdot4((int)w.w, (int)d0.w, acc[q][2], false);
    }
    if (RPC > 1 || s % nch == nch - 1) {
#pragma unroll
      for (int q = 0; q < RPC; ++q) {
        const int i = slot_idx(s, q);
        float v = fmaf((float)acc[q][0], 65536.0f, fmaf((float)acc[q][1], 256.0f, (float)acc[q][2]));
        v = wave_sum(v);
        if (lane == 0 && i < rows_w) {
          const int row = row_at(i);
          ys[row - r0] = v * sx * gld(&scale[row]);
        }
        acc[q][0] = acc[q][1] = acc[q][2] = 0;
      }
    }
  }
  // as GemvStream::run_pf: chunk 0 in this wave's LDS slot pf, chunk 1 in P
  __device__ __forceinline__ void run_pf(const uint4 *pf, const uint4 (&P)[kChunkUnits],
                                         const uint8_t *xd, float sx, float *ys,
                                         const float *scale) const {
    if (S == 0) return;
    int acc[RPC][3];
#pragma unroll
    for (int q = 0; q < RPC; ++q) acc[q][0] = acc[q][1] = acc[q][2] = 0;
    uint4 A[kChunkUnits], Bf[kChunkUnits];
    if (S > 2) {
      load(A, 2);
      __builtin_amdgcn_s_waitcnt(kWaitVm8);
    } else {
      __builtin_amdgcn_s_waitcnt(kWaitVm0);
    }
#pragma unroll
    for (int j = 0; j < kChunkUnits; ++j) Bf[j] = pf[j * 64 + lane];
    consume(Bf, 0, acc, xd, sx, ys, scale);
    if (S == 1) return;
    consume(P, 1, acc, xd, sx, ys, scale);
    if (S == 2) return;
    int s = 2;
    for (; s + 2 < S; s += 2) {
      load(Bf, s + 1);
      consume(A, s, acc, xd, sx, ys, scale);
      load(A, s + 2);
      consume(Bf, s + 1, acc, xd, sx, ys, scale);
    }
    if (s + 1 < S) {
      load(Bf, s + 1);
      consume(A, s, acc, xd, sx, ys, scale);
      consume(Bf, s + 1, acc, xd, sx, ys, scale);
    } else {
      consume(A, s, acc, xd, sx, ys, scale);
    }
  }
};

// The int4 stream: as GemvStreamI8, with 16-byte units of 32 inputs (rows of K / 2 bytes) and
// one fp32 scale per row and group of gs inputs (a multiple of 32, so a unit lies in one group).
// A unit's nibbles go to the integer dot products as int8 lanes holding 16 q: for word i (inputs
// 8i .. 8i + 7), (w << 4) & 0xF0F0F0F0 holds inputs 8i .. 8i + 3 and w & 0xF0F0F0F0 inputs
// 8i + 4 .. 8i + 7. Each unit's exact int32 sums are scaled by its group's scale into an fp32
// accumulator; the row's sum carries a factor 16 that the end of the row removes. A unit's digits
// are two consecutive int8 digit units (96 bytes). RPC > 1: rows of exactly 64 * kChunkUnits / RPC
// units (K = 4096 with RPC = 4).
template <int RPC>
struct GemvStreamI4 {
  static constexpr int UPL = kChunkUnits / RPC;
  const uint8_t *W;
  const float *scale;
  int K, r0, nw, n32, nch, S, rows_w, ng, upg;
  int wave, lane;
  float sc0[kChunkUnits], scP[kChunkUnits];  // scales of the chunks issued before the wait

  __device__ __forceinline__ void init(const void *w, const float *sc, int gs, int k, int a, int b,
                                       int nwaves) {
    W = static_cast<const uint8_t *>(w);
    scale = sc;
    K = k;
    r0 = a;
    nw = nwaves;
    wave = __builtin_amdgcn_readfirstlane(wave_id());
    lane = lane_id();
    n32 = K / 32;
    ng = K / gs;
    upg = gs / 32;
    nch = RPC == 1 ? (n32 + 64 * kChunkUnits - 1) / (64 * kChunkUnits) : 1;
    const int n = b - a;
    rows_w = (n > wave) ? (n - wave + nw - 1) / nw : 0;
    S = RPC == 1 ? rows_w * nch : (rows_w + RPC - 1) / RPC;
  }
  __device__ __forceinline__ int slot_idx(int s, int q) const { return RPC == 1 ? s / nch : s * RPC + q; }
  __device__ __forceinline__ int row_at(int i) const { return r0 + wave + min(i, rows_w - 1) * nw; }
  __device__ __forceinline__ int unit_of(int s, int j) const {
    return RPC == 1 ? (s % nch) * 64 * kChunkUnits + lane + 64 * j : lane + 64 * (j % UPL);
  }
  __device__ __forceinline__ void addr(int s, int j, const uint4 **wp, const float **sp) const {
    const int row = row_at(slot_idx(s, j / UPL));
    const int u = min(unit_of(s, j), n32 - 1);
    *wp = reinterpret_cast<const uint4 *>(W + (int64_t)row * (K / 2)) + u;
    *sp = scale + (int64_t)row * ng + u / upg;
  }
  __device__ __forceinline__ void load2(uint4 (&buf)[kChunkUnits], float (&sb)[kChunkUnits], int s) const {
#pragma unroll
    for (int j = 0; j < kChunkUnits; ++j) {
      const uint4 *wp;
      const float *sp;
      addr(s, j, &wp, &sp);
      buf[j] = load_nt(wp);
      sb[j] = gld(sp);
    }
  }
  // the register chunk issued before the wait (its scales kept in scP)
  __device__ __forceinline__ void load(uint4 (&buf)[kChunkUnits], int s) { load2(buf, scP, s); }
  // chunk s straight into LDS (its scales into sc0)
  __device__ __forceinline__ void load_lds(int s, uint4 *dst) {
#pragma unroll
    for (int j = 0; j < kChunkUnits; ++j) {
      const uint4 *wp;
      const float *sp;
      addr(s, j, &wp, &sp);
      __builtin_amdgcn_global_load_lds((const AMK_GAS void *)wp, (AMK_LDS void *)(dst + j * 64), 16,
                                       0, kCachePolicyNt);
      sc0[j] = gld(sp);
    }
  }
  __device__ __forceinline__ void consume(const uint4 (&buf)[kChunkUnits], const float (&sb)[kChunkUnits],
                                          int s, float (&acc)[RPC], const uint8_t *xd, float sx,
                                          float *ys) const {
#pragma unroll
    for (int j = 0; j < kChunkUnits; ++j) {
      const int q = j / UPL;
      const int u = unit_of(s, j);
      const AMK_LDS u32x4_t *dp =
          (const AMK_LDS u32x4_t *)((const AMK_LDS uint8_t *)xd + 96 * (RPC == 1 ? min(u, n32) : u));
      const u32x4_t d2a = dp[0], d1a = dp[1], d0a = dp[2], d2b = dp[3], d1b = dp[4], d0b = dp[5];
      const uint4 w = buf[j];
      const uint32_t ws[4] = {w.x, w.y, w.z, w.w};
      int a2 = 0, a1 = 0, a0 = 0;
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int lo = (int)((ws[i] << 4) & 0xF0F0F0F0u), hi = (int)(ws[i] & 0xF0F0F0F0u);
        const u32x4_t &D2 = i < 2 ? d2a : d2b, &D1 = i < 2 ? d1a : d1b, &D0 = i < 2 ? d0a : d0b;
        const int wl = 2 * (i & 1);
        a2 = __builtin_amdgcn_sdot4(lo, (int)D2[wl], a2, false);
        a1 = __builtin_amdgcn_sdot4(lo, (int)D1[wl], a1, false);
        a0 = __builtin_amdgcn_sdot4(lo, (int)D0[wl], a0, false);
        a2 = __builtin_amdgcn_sdot4(hi, (int)D2[wl + 1], a2, false);
        a1 = __builtin_amdgcn_sdot4(hi, (int)D1[wl + 1], a1, false);
        a0 = __builtin_amdgcn_sdot4(hi, (int)D0[wl + 1], a0, false);
      }
      // |a_p| <= 32 * 128 * 128: exact in fp32
      const float v = fmaf((float)a2, 65536.0f, fmaf((float)a1, 256.0f, (float)a0));
      acc[q] = fmaf(v, sb[j], acc[q]);
    }
    if (RPC > 1 || s % nch == nch - 1) {
#pragma unroll
      for (int q = 0; q < RPC; ++q) {
        const int i = slot_idx(s, q);
        const float v = wave_sum(acc[q]);
        if (lane == 0 && i < rows_w) ys[row_at(i) - r0] = v * (sx * 0.0625f);
        acc[q] = 0.f;
      }
    }
  }
  __device__ __forceinline__ void run_pf(const uint4 *pf, const uint4 (&P)[kChunkUnits],
                                         const uint8_t *xd, float sx, float *ys,
                                         const float *) const {
    if (S == 0) return;
    float acc[RPC];
#pragma unroll
    for (int q = 0; q < RPC; ++q) acc[q] = 0.f;
    uint4 A[kChunkUnits], Bf[kChunkUnits];
    float sA[kChunkUnits], sB[kChunkUnits];
    if (S > 2) {
      load2(A, sA, 2);
      __builtin_amdgcn_s_waitcnt(kWaitVm16);
    } else {
      __builtin_amdgcn_s_waitcnt(kWaitVm0);
    }
#pragma unroll
    for (int j = 0; j < kChunkUnits; ++j) Bf[j] = pf[j * 64 + lane];
    consume(Bf, sc0, 0, acc, xd, sx, ys);
    if (S == 1) return;
    consume(P, scP, 1, acc, xd, sx, ys);
    if (S == 2) return;
    int s = 2;
    for (; s + 2 < S; s += 2) {
      load2(Bf, sB, s + 1);
      consume(A, sA, s, acc, xd, sx, ys);
      load2(A, sA, s + 2);
      consume(Bf, sB, s + 1, acc, xd, sx, ys);
    }
    if (s + 1 < S) {
      load2(Bf, sB, s + 1);
      consume(A, sA, s, acc, xd, sx, ys);
      consume(Bf, sB, s + 1, acc, xd, sx, ys);
    } else {
      consume(A, sA, s, acc, xd, sx, ys);
    }
  }
};

// ------------------------------------------------------------------------------------------
// input staging (LDS)
// ------------------------------------------------------------------------------------------
// token of sequence b, validated (an out-of-range id is recorded as a device error and read as 0)
__device__ __forceinline__ int32_t token_of(const DevModel &m, const StepArgs &s, int b) {
  int32_t t = cld(&s.tokens[b]);  // device-coherent: a previous step of the launch may have written it
  if (t < 0 || t >= m.V) {
    if (threadIdx.x == 0) record_error(m.err, ERR_TOKEN, 0xffffffffu, (uint32_t)t);
    t = 0;
  }
  return t;
}

// RMSNorm staging, split around the GEMV. The norm's scale 1/rms(src_b) is one number per batch
// row, so W (src_b * gain) scaled afterwards equals W rmsnorm(src_b) * gain: the input is staged
// as xs[b][i] = src_b[i] * gain[i] in one round of loads, and the per-wave partial sums of
// squares go to red[b * nw + wave]; norm_scale_ys applies the scale to the GEMV outputs.
// src = h slot `slot` or, for slot 0, the embedding row of the token. Needs d % 4 == 0.
constexpr int kStageVec = 4;  // float4 groups per thread per round (d <= 8192 in one round)
__device__ void stage_norm(const DevModel &m, const StepArgs &s, int slot, const uint16_t *gain,
                           float *xs, float *red, int nw) {
  const int d = m.d, n4 = d / 4;
  const int lane = lane_id(), wave = wave_id();
  for (int b = 0; b < s.batch; ++b) {
    float *x = xs + (int64_t)b * d;
    const uint16_t *e = (slot == 0) ? m.embed + (int64_t)token_of(m, s, b) * d : nullptr;
    const float *src = m.h + ((int64_t)slot * m.max_batch + b) * d;
    const __amdgpu_buffer_rsrc_t rs = make_rsrc(src, (uint32_t)d * 4u);
    float ss = 0.f;
    for (int base = 0; base < n4; base += kStageVec * nw * 64) {
      float4 hv[kStageVec];
      uint2 gv[kStageVec];
#pragma unroll
      for (int j = 0; j < kStageVec; ++j) {
        const int i4 = min(base + (int)threadIdx.x + j * nw * 64, n4 - 1);
        if (e) {
          const uint2 ev = gld_bf16x4(e, i4);
          hv[j] = make_float4(bf_lo(ev.x), bf_hi(ev.x), bf_lo(ev.y), bf_hi(ev.y));
        } else {
          hv[j] = cld4(rs, (uint32_t)i4 * 16u);
        }
        gv[j] = gld_bf16x4(gain, i4);
      }
#pragma unroll
      for (int j = 0; j < kStageVec; ++j) {
        const int i4 = base + (int)threadIdx.x + j * nw * 64;
        if (i4 < n4) {
          const float4 v = hv[j];
          ss += v.x * v.x + v.y * v.y + v.z * v.z + v.w * v.w;
          *reinterpret_cast<float4 *>(x + 4 * i4) =
              make_float4(v.x * bf_lo(gv[j].x), v.y * bf_hi(gv[j].x), v.z * bf_lo(gv[j].y),
                          v.w * bf_hi(gv[j].y));
        }
      }
    }
    ss = wave_sum(ss);
    if (lane == 0) red[b * nw + wave] = ss;
  }
  __syncthreads();
}

// ys[b][i] *= 1 / sqrt(mean(src_b^2) + eps) with the partial sums stage_norm left in red (read
// after the workgroup barrier that follows the GEMV). Ends with a barrier.
__device__ __forceinline__ void norm_scale_ys(const DevModel &m, const StepArgs &s, int n, float *ys,
                              const float *red, int nw) {
  for (int b = 0; b < s.batch; ++b) {
    float tot = 0.f;
    for (int w = 0; w < nw; ++w) tot += red[b * nw + w];
    const float inv = 1.0f / sqrtf(tot / (float)m.d + m.eps);
    for (int i = threadIdx.x; i < n; i += nw * 64) ys[b * n + i] *= inv;
  }
  __syncthreads();
}

// xs[b][i] = src[b * src_stride + i], i < K (K % 4 == 0, src rows 16-byte aligned): device-
// coherent 16-byte loads, kStageVec * 2 per thread in flight per round.
__device__ void stage_plain(const float *src, int64_t src_stride, int K, int B, float *xs, int nw) {
  const int n4 = K / 4;
  constexpr int V = 2 * kStageVec;
  for (int b = 0; b < B; ++b) {
    const __amdgpu_buffer_rsrc_t rs = make_rsrc(src + b * src_stride, (uint32_t)K * 4u);
    float *x = xs + (int64_t)b * K;
    for (int base = 0; base < n4; base += V * nw * 64) {
      float4 v[V];
#pragma unroll
      for (int j = 0; j < V; ++j)
        v[j] = cld4(rs, (uint32_t)min(base + (int)threadIdx.x + j * nw * 64, n4 - 1) * 16u);
#pragma unroll
      for (int j = 0; j < V; ++j) {
        const int i4 = base + (int)threadIdx.x + j * nw * 64;
        if (i4 < n4) *reinterpret_cast<float4 *>(x + 4 * i4) = v[j];
      }
    }
  }
  __syncthreads();
}

// Tagged activations (batch 1). A value that crosses CUs within a step is stored as one fp32
// word whose two lowest mantissa bits are replaced by the low bits of the step's epoch (the value
// moves by at most 3 ulp). One aligned 32-bit store carries value and tag together, so the
// consumer's staging loads are its dependency wait: it reloads until every tag matches, and the
// producer needs neither to wait for its stores nor to publish a flag.
//
// Two tag bits suffice because every slot is written exactly once by every step that completes,
// so a slot holds either this step's word or the previous step's, whose tag differs. A step that
// fails leaves the device abort word set until the host resets the model, which also clears every
// slot; a consumer reads the abort word in its first round, so it never accepts an older word.
constexpr uint32_t kTagMask = 3u;
__device__ __forceinline__ uint32_t tag_word(float v, uint32_t epoch) {
  return (__float_as_uint(v) & ~kTagMask) | (epoch & kTagMask);
}
// The value a tagged word carries, with its tag bits cleared: the value the producer computed
// truncated to 21 mantissa bits, whatever the epoch. Results therefore do not depend on the step
// count, and two runs of the same inputs agree bit for bit at any epochs.
__device__ __forceinline__ float untag(uint32_t w) { return __uint_as_float(w & ~kTagMask); }

// xs[i] = v_i * gain[i] (gain may be null) for the n tagged words at src (n % 4 == 0), once every
// tag matches `epoch`; with a gain the per-wave sums of v^2 go to red[wave]. Each thread owns up
// to eight 16-byte units per round and reloads only those whose tags were stale. Returns false
// after a timeout (recorded as a device error) or when the abort word is set.
// DIGITS: the input of a batch-1 int8 GEMV. The values stay in registers until all have arrived
// (one round: n <= kDigitMaxK), then go to LDS as integer digits (see stage_digits) instead of
// fp32; *sx receives the weight of one digit unit.
template <bool DIGITS>
__device__ __forceinline__ bool stage_tagged(const DevModel &m, const uint32_t *src, int n, const uint16_t *gain,
                             uint32_t epoch, float *xs, float *red, uint32_t task,
                             float *sx = nullptr) {
  constexpr int V = 8;
  static_assert(!DIGITS || kDigitMaxK <= 4 * V * kThreads, "digit staging takes one round");
  const int nu = n >> 2;
  const uint32_t tag = epoch & kTagMask;
  const __amdgpu_buffer_rsrc_t rs = make_rsrc(src, (uint32_t)n * 4u);
  uint32_t *const err = m.err;  // read here, in uniform code, so they come from scalar loads
  const uint64_t tmo = m.timeout_ticks;
  float ss = 0.f, mx = 0.f;
  uint64_t t0 = 0;
  uint32_t spins = 0;
  u32x4_t keep[DIGITS ? V : 1];  // DIGITS: the staged values, until all have arrived
  for (int base = 0; base < nu; base += V * kThreads) {
    uint32_t need = 0;
#pragma unroll
    for (int j = 0; j < V; ++j)
      if (base + (int)threadIdx.x + j * kThreads < nu) need |= 1u << j;
    while (true) {
      u32x4_t v[V];
#pragma unroll
      for (int j = 0; j < V; ++j)
        if (need & (1u << j))
          v[j] = __builtin_amdgcn_raw_buffer_load_b128(
              rs, (int)((uint32_t)(base + (int)threadIdx.x + j * kThreads) * 16u), 0,
              kCachePolicySc1);
      // thread 0: the abort word on the first round and every eighth retry; the timeout
      int ab = 0;
      if (threadIdx.x == 0 && (spins == 0 || (spins & 7) == 7)) {
        ab = flag_load(&err[1]) != 0;
        if (!ab && spins && wall_clock64() - t0 > tmo) {
          record_error(err, ERR_TIMEOUT, task, 0xfffffff0u);
          __hip_atomic_store(gptr(&err[1]), 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
          ab = 1;
        }
      }
#pragma unroll
      for (int j = 0; j < V; ++j) {
        if (need & (1u << j)) {
          const u32x4_t w = v[j];
          if ((((w.x ^ tag) | (w.y ^ tag) | (w.z ^ tag) | (w.w ^ tag)) & kTagMask) == 0) {
            need &= ~(1u << j);
            const int u = base + (int)threadIdx.x + j * kThreads;
            float a = untag(w.x), b = untag(w.y), c = untag(w.z), d = untag(w.w);
            if (gain) {
              ss = fmaf(a, a, fmaf(b, b, fmaf(c, c, fmaf(d, d, ss))));
              const uint2 g = gld_bf16x4(gain, u);
              a *= bf_lo(g.x);
              b *= bf_hi(g.x);
              c *= bf_lo(g.y);
              d *= bf_hi(g.y);
            }
            if constexpr (DIGITS) {
              mx = fmaxf(mx, fmaxf(fmaxf(fabsf(a), fabsf(b)), fmaxf(fabsf(c), fabsf(d))));
              keep[j] = u32x4_t{__float_as_uint(a), __float_as_uint(b), __float_as_uint(c),
                                __float_as_uint(d)};
            } else {
              *reinterpret_cast<float4 *>(xs + 4 * u) = make_float4(a, b, c, d);
            }
          }
        }
      }
      const int pending = __syncthreads_or(need != 0);
      if (__syncthreads_or(ab)) return false;
      if (!pending) break;
      if (spins == 0) t0 = wall_clock64();
      ++spins;
      __builtin_amdgcn_s_sleep(1);
    }
  }
  if (gain) {
    ss = wave_sum(ss);
    if (lane_id() == 0) *(AMK_LDS float *)(red + wave_id()) = ss;
  }
  if constexpr (DIGITS) {
    mx = wave_max_nonneg(mx);
    if (lane_id() == 0) ((AMK_LDS float *)red)[kDigitRedSlot + wave_id()] = mx;
  }
  __syncthreads();
  if constexpr (DIGITS) {
    int e;
    const float up = digit_up(red, &e);
#pragma unroll
    for (int j = 0; j < V; ++j) {
      const int u = (int)threadIdx.x + j * kThreads;
      if (u < nu)
        put_digits(xs, u, __uint_as_float(keep[j].x), __uint_as_float(keep[j].y),
                   __uint_as_float(keep[j].z), __uint_as_float(keep[j].w), up);
    }
    put_zero_unit(xs, n);
    __syncthreads();
    *sx = ldexpf(1.0f, e - 22);
  }
  return true;
}

// ------------------------------------------------------------------------------------------
// Batch GEMV (B = 2..16 sequences) on the matrix cores:
//   ys[b * n + (r - r0)] = sum_k X_b[k] W[r][k]  (times scale[r] for int8), r in [r0, r1).
// v_mfma_f32_16x16x32_bf16 computes a 16 x 16 tile C = A B over 32 k. Lane l supplies
// A[l % 16][8 (l/16) + e] and B[8 (l/16) + e][l % 16], e < 8, and receives C[4 (l/16) + i][l % 16],
// i < 4. A holds 16 weight rows. The inputs are split into two bf16 halves, x = hi + lo, and the
// 16 columns of B carry hi of sequence c (c < 8) and lo of sequence c - 8 (c >= 8), so one
// instruction multiplies both halves and y_b = C[.][b] + C[.][b + 8] keeps about 16 bits of the
// fp32 input; columns of sequences >= B are zero. Wide (B > 8): column c carries sequence c, and
// two instructions, one per half, accumulate into the same tile. K is split over the workgroup's waves
// (contiguous runs of 32-k steps); their partial tiles are summed in LDS (mred). Inputs are read
// straight from the device-coherent buffers (no LDS staging). Each wave issues the loads of U
// k-steps (GP 16-row groups each) before using any of them.
// Weights and inputs are addressed through buffer resources: out-of-range lanes read zeros.
// ------------------------------------------------------------------------------------------
typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
constexpr int kMfmaGroups = 4;
static_assert(kMfmaRedFloats == kWaves * kMfmaGroups * 16 * 16, "LDS for the partial tiles");

struct BatchInput {
  const float *x;        // fp32 rows, `stride` floats apart (null when emb is set)
  int32_t stride;
  const uint16_t *emb;   // bf16 embedding [V][K]: sequence b reads row tokens[b]
  const uint16_t *gain;  // bf16 [K] multiplied into the input, or null
  bool sumsq;            // leave sum_k x^2 of sequence b's partial range in red[b * nw + wave]
};

__device__ __forceinline__ bf16x8_t bf16x8_of_bits(uint32_t a, uint32_t b, uint32_t c, uint32_t d) {
  const u32x4_t v = {a, b, c, d};
  return __builtin_bit_cast(bf16x8_t, v);
}
// eight int8 weights (two words) as eight bf16 (exact: |q| <= 127)
__device__ __forceinline__ bf16x8_t bf16x8_of_i8(uint32_t w0, uint32_t w1) {
  uint32_t o[4];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int32_t v = (int32_t)(i < 2 ? w0 : w1);
    const int sh = (i & 1) * 16;
    const float f0 = (float)((v << (24 - sh)) >> 24), f1 = (float)((v << (16 - sh)) >> 24);
    o[i] = (__float_as_uint(f0) >> 16) | (__float_as_uint(f1) & 0xffff0000u);
  }
  return bf16x8_of_bits(o[0], o[1], o[2], o[3]);
}

// eight int4 weights (one word, inputs k .. k + 7 in the library's nibble order) as the eight bf16
// values q + 136 (exact: 128 + (q + 8) with q + 8 in [0, 15] is the bf16 0x4300 | (q + 8)); the
// caller subtracts 136 times the column sums of the input
__device__ __forceinline__ bf16x8_t bf16x8_of_i4_offset(uint32_t w) {
  const uint32_t lo = (w & 0x0F0F0F0Fu) ^ 0x08080808u, hi = ((w >> 4) & 0x0F0F0F0Fu) ^ 0x08080808u;
  // byte selectors 0-3 take the second operand's bytes, 4 the first's (0x43)
  return bf16x8_of_bits(__builtin_amdgcn_perm(0x43434343u, lo, 0x04010400u),
                        __builtin_amdgcn_perm(0x43434343u, lo, 0x04030402u),
                        __builtin_amdgcn_perm(0x43434343u, hi, 0x04010400u),
                        __builtin_amdgcn_perm(0x43434343u, hi, 0x04030402u));
}

// per-lane view of one batched GEMV tile
struct MfmaTile {
  __amdgpu_buffer_rsrc_t rw, rx, rg;
  int K, rb, n, t0, t1;
  const float *sc;  // int4: the tile's scale rows [n][ng]
  int ng, gs;
  // byte offset of this lane's weights for 16-row group g and k step t: wl + g wg + t wt
  uint32_t wl, wg, wt;
  int B;           // sequences
  uint32_t xrow;   // byte offset of this lane's input row (kNoRow: loads nothing, reads zeros)
  int col, kq;     // B/C column (l % 16) and k quarter (l / 16)
  bool emb, gain, lo_half;
};

// An input offset no k step brings back inside the input resource (its loads return zeros and
// touch no memory).
constexpr uint32_t kNoRow = 0x80000000u;

// one pass: groups [g0, g0 + gn) (gn <= GP) over this wave's k steps, the loads of U steps
// issued before any of them is used; returns the partial tiles
template <int WT, int GP, int U, bool GAIN, bool WIDE>
__device__ __forceinline__ void mfma_pass(const MfmaTile &T, int g0, int gn, bool sumsq, float &ss,
                                          f32x4_t (&acc)[kMfmaGroups]) {
#pragma unroll
  for (int g = 0; g < kMfmaGroups; ++g) acc[g] = f32x4_t{0.f, 0.f, 0.f, 0.f};
  for (int t = T.t0; t < T.t1; t += U) {
    uint32_t xw[U][8];
    uint32_t gw[GAIN ? U : 1][4];
    uint32_t wf[U][GP][4];
#pragma unroll
    for (int u = 0; u < U; ++u) {
      if (t + u < T.t1) {
        const int k = 32 * (t + u) + 8 * T.kq;
        if (T.emb) {
          const u32x4_t e = __builtin_amdgcn_raw_buffer_load_b128(T.rx, (int)(T.xrow + (uint32_t)k * 2u), 0, 0);
          xw[u][0] = e.x; xw[u][1] = e.y; xw[u][2] = e.z; xw[u][3] = e.w;
        } else {
          const u32x4_t a = __builtin_amdgcn_raw_buffer_load_b128(T.rx, (int)(T.xrow + (uint32_t)k * 4u), 0, kCachePolicySc1);
          const u32x4_t b = __builtin_amdgcn_raw_buffer_load_b128(T.rx, (int)(T.xrow + (uint32_t)k * 4u + 16u), 0, kCachePolicySc1);
          xw[u][0] = a.x; xw[u][1] = a.y; xw[u][2] = a.z; xw[u][3] = a.w;
          xw[u][4] = b.x; xw[u][5] = b.y; xw[u][6] = b.z; xw[u][7] = b.w;
        }
        if constexpr (GAIN) {
          const u32x4_t gv = __builtin_amdgcn_raw_buffer_load_b128(T.rg, k * 2, 0, 0);
          gw[u][0] = gv.x; gw[u][1] = gv.y; gw[u][2] = gv.z; gw[u][3] = gv.w;
        }
#pragma unroll
        for (int g = 0; g < GP; ++g) {
          if (g < gn) {
            const uint32_t off = T.wl + (uint32_t)(g0 + g) * T.wg + (uint32_t)(t + u) * T.wt;
            if constexpr (WT == 2) {
              wf[u][g][0] = __builtin_amdgcn_raw_buffer_load_b32(T.rw, (int)off, 0, kCachePolicyNt);
              wf[u][g][1] = wf[u][g][2] = wf[u][g][3] = 0;
            } else if constexpr (WT == 0) {
              const u32x4_t w = __builtin_amdgcn_raw_buffer_load_b128(T.rw, (int)off, 0, kCachePolicyNt);
              wf[u][g][0] = w.x; wf[u][g][1] = w.y; wf[u][g][2] = w.z; wf[u][g][3] = w.w;
            } else {
              const u32x2_t w = __builtin_amdgcn_raw_buffer_load_b64(T.rw, (int)off, 0, kCachePolicyNt);
              wf[u][g][0] = w.x; wf[u][g][1] = w.y; wf[u][g][2] = 0; wf[u][g][3] = 0;
            }
          }
        }
      }
    }
#pragma unroll
    for (int u = 0; u < U; ++u) {
      if (t + u < T.t1) {
        const int k = 32 * (t + u) + 8 * T.kq;
        if constexpr (!WIDE) {
          // packed: the lo-half lanes (columns 8..15, banks 2 and 3 of each 16-lane row) loaded
          // nothing; they take their sequence's inputs from the hi-half lane 8 columns away
#pragma unroll
          for (int i = 0; i < 8; ++i)
            xw[u][i] = (uint32_t)__builtin_amdgcn_update_dpp((int)xw[u][i], (int)xw[u][i], 0x128, 0xF,
                                                             0xC, false);
        }
        float xv[8];
        if (T.emb) {
#pragma unroll
          for (int i = 0; i < 4; ++i) { xv[2 * i] = bf_lo(xw[u][i]); xv[2 * i + 1] = bf_hi(xw[u][i]); }
        } else {
#pragma unroll
          for (int i = 0; i < 8; ++i) xv[i] = __uint_as_float(xw[u][i]);
        }
        // x * gain as bf16 halves: packed, the hi half for columns < 8 and the lo half for the
        // others; wide, both halves of the column's sequence. Inputs past K are 0.
        uint32_t hx[4], lx[4];
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          float v0 = k + 2 * i < T.K ? xv[2 * i] : 0.f, v1 = k + 2 * i + 1 < T.K ? xv[2 * i + 1] : 0.f;
          if (sumsq && (WIDE || !T.lo_half)) ss = fmaf(v0, v0, fmaf(v1, v1, ss));
          if constexpr (GAIN) {
            v0 *= bf_lo(gw[u][i]);
            v1 *= bf_hi(gw[u][i]);
          }
          const uint16_t h0 = f32_to_bf16(v0), h1 = f32_to_bf16(v1);
          const uint16_t l0 = f32_to_bf16(v0 - bf16_to_f32(h0)), l1 = f32_to_bf16(v1 - bf16_to_f32(h1));
          if (!WIDE && T.lo_half)
            hx[i] = (uint32_t)l0 | ((uint32_t)l1 << 16);
          else
            hx[i] = (uint32_t)h0 | ((uint32_t)h1 << 16);
          lx[i] = (uint32_t)l0 | ((uint32_t)l1 << 16);
        }
        const bf16x8_t xb = bf16x8_of_bits(hx[0], hx[1], hx[2], hx[3]);
        const bf16x8_t xl = bf16x8_of_bits(lx[0], lx[1], lx[2], lx[3]);  // wide only
        if constexpr (WT == 2) {
          // int4: each k step's products, less 136 times the input column sums, times the
          // step's group scale of each row (a k step of 32 inputs lies in one group)
          const uint32_t c136 = 0x43084308u;  // bf16 136.0, twice
          const bf16x8_t a136 = bf16x8_of_bits(c136, c136, c136, c136);
          f32x4_t corr = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a136, xb, f32x4_t{0.f, 0.f, 0.f, 0.f}, 0, 0, 0);
          if constexpr (WIDE) corr = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a136, xl, corr, 0, 0, 0);
          const f32x4_t ncorr = -corr;
          const int grp = (32 * (t + u)) / T.gs;
#pragma unroll
          for (int g = 0; g < GP; ++g) {
            if (g < gn) {
              const bf16x8_t a = bf16x8_of_i4_offset(wf[u][g][0]);
              f32x4_t p = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, xb, ncorr, 0, 0, 0);
              if constexpr (WIDE) p = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, xl, p, 0, 0, 0);
#pragma unroll
              for (int i = 0; i < 4; ++i) {
                const int r = min(16 * (g0 + g) + 4 * T.kq + i, T.n - 1);
                acc[g][i] = fmaf(p[i], gld(&T.sc[(int64_t)r * T.ng + grp]), acc[g][i]);
              }
            }
          }
        } else {
#pragma unroll
          for (int g = 0; g < GP; ++g) {
            if (g < gn) {
              const bf16x8_t a = WT == 0 ? bf16x8_of_bits(wf[u][g][0], wf[u][g][1], wf[u][g][2], wf[u][g][3])
                                         : bf16x8_of_i8(wf[u][g][0], wf[u][g][1]);
              acc[g] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, xb, acc[g], 0, 0, 0);
              if constexpr (WIDE) acc[g] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, xl, acc[g], 0, 0, 0);
            }
          }
        }
      }
    }
  }
}

template <int WT, bool WIDE>
__device__ __forceinline__ void mfma_dispatch(const MfmaTile &T, int g0, int gn, bool sq, float &ss,
                                              f32x4_t (&acc)[kMfmaGroups]) {
  if (T.gain) {
    if (gn <= 1)
      mfma_pass<WT, 1, 4, true, WIDE>(T, g0, gn, sq, ss, acc);
    else if (gn == 2)
      mfma_pass<WT, 2, 4, true, WIDE>(T, g0, gn, sq, ss, acc);
    else
      mfma_pass<WT, 4, 2, true, WIDE>(T, g0, gn, sq, ss, acc);
  } else {
    if (gn <= 1)
      mfma_pass<WT, 1, 4, false, WIDE>(T, g0, gn, sq, ss, acc);
    else if (gn == 2)
      mfma_pass<WT, 2, 4, false, WIDE>(T, g0, gn, sq, ss, acc);
    else
      mfma_pass<WT, 4, 2, false, WIDE>(T, g0, gn, sq, ss, acc);
  }
}

// ------------------------------------------------------------------------------------------
// Batched GEMV over tile-major weights, streamed through a per-wave LDS ring (megakernel
// instances). A round is one k step of a pass: the step's tile of each of the GP row groups (one
// 64-lane copy of 16 bytes per lane; int8 and int4 tiles fill the first 32 or 16 lanes), the
// step's inputs of every sequence, the norm gain and, for int4, the step's group scale of each
// row, all copied from memory straight into the round's LDS slot. Every round issues the same
// copies; lanes and rounds with nothing to fetch address past their buffer resource, which moves
// no data. D rounds are issued ahead (in steady state round r is in LDS once the vector-memory
// count is down to D times the copies per round; wait_round has the prologue's counts), and no
// registers wait on loads in flight. A copy writes 16 (or 4)
// bytes of LDS for each active lane whether or not it fetched anything, so each copy's slot area
// holds 64 lanes' worth, except the gain's, which only lanes 0..3 copy.
// ------------------------------------------------------------------------------------------
template <int WT, int GP, bool GAIN, bool WIDE>
struct RingShape {
  static constexpr int NX = WIDE ? 2 : 1;             // input copies (8 fp32 or 16 bf16 rows each)
  static constexpr int XO = GP * 1024;                // inputs [b][32]: fp32, or bf16 embedding rows
  static constexpr int GO = XO + NX * 1024;           // gain [32] bf16
  static constexpr int SO = GO + (GAIN ? 64 : 0);     // int4: scales [16 GP] fp32
  static constexpr int SB = (SO + (WT == 2 ? 256 : 0) + 63) / 64 * 64;  // slot bytes
  static constexpr int NS = kRingBytes / SB;          // slots
  static constexpr int D = NS - 1;                    // rounds in flight
  static constexpr int NI = GP + NX + (GAIN ? 1 : 0) + (WT == 2 ? 1 : 0);  // copies per round
  static_assert(D >= 1 && D * NI <= 63, "the vector-memory count has 6 bits");
};

// this lane's part of the ring copies
struct RingLanes {
  AMK_LDS uint8_t *ring;        // this wave's ring
  __amdgpu_buffer_rsrc_t rs;    // int4: scale rows of the tile
  uint32_t woff;                // lane's 16 bytes of a weight tile (kNoRow: none)
  uint32_t xoff[2], xstep;      // input copies: bytes at k step 0, bytes per k step
  uint32_t goff;                // gain: lanes 0..3
  uint32_t soff;                // int4 scales: lane's row in the pass (kNoRow: none)
};

// the copies of round r that do not depend on the step's activations: weight tiles, gain, scales
template <int WT, int GP, bool GAIN, bool WIDE>
__device__ __forceinline__ void ring_issue_w(const MfmaTile &T, const RingLanes &L, int g0, int gn,
                                             bool live, int r, int slot) {
  using RS = RingShape<WT, GP, GAIN, WIDE>;
  const uint32_t t = (uint32_t)(T.t0 + r);
  AMK_LDS uint8_t *p = L.ring + slot * RS::SB;
#pragma unroll
  for (int g = 0; g < GP; ++g) {
    const uint32_t off = (live && g < gn) ? L.woff + (uint32_t)(g0 + g) * T.wg + t * T.wt : kNoRow;
    __builtin_amdgcn_raw_ptr_buffer_load_lds(T.rw, (AMK_LDS void *)(p + g * 1024), 16, (int)off, 0, 0,
                                             kCachePolicyNt);
  }
  if constexpr (GAIN) {
    // only lanes 0..3 run this copy: an LDS copy writes 16 bytes for every active lane, fetched
    // or not, and the slot holds 64 bytes of gain
    if (lane_id() < 4) {
      const uint32_t off = live ? L.goff + t * 64u : kNoRow;
      __builtin_amdgcn_raw_ptr_buffer_load_lds(T.rg, (AMK_LDS void *)(p + RS::GO), 16, (int)off, 0, 0, 0);
    }
  }
  if constexpr (WT == 2) {
    const uint32_t off = live ? L.soff + (uint32_t)((32 * (int)t) / T.gs) * 4u : kNoRow;
    __builtin_amdgcn_raw_ptr_buffer_load_lds(L.rs, (AMK_LDS void *)(p + RS::SO), 4, (int)off, 0, 0, 0);
  }
}

// the input copies of round r (written by other tasks of this step)
template <int WT, int GP, bool GAIN, bool WIDE>
__device__ __forceinline__ void ring_issue_x(const MfmaTile &T, const RingLanes &L, bool live, int r,
                                             int slot) {
  using RS = RingShape<WT, GP, GAIN, WIDE>;
  const uint32_t t = (uint32_t)(T.t0 + r);
  AMK_LDS uint8_t *p = L.ring + slot * RS::SB;
#pragma unroll
  for (int j = 0; j < RS::NX; ++j) {
    const uint32_t off = live ? L.xoff[j] + t * L.xstep : kNoRow;
    if (T.emb)
      __builtin_amdgcn_raw_ptr_buffer_load_lds(T.rx, (AMK_LDS void *)(p + RS::XO + j * 1024), 16,
                                               (int)off, 0, 0, 0);
    else  // produced this step by other CUs: device-coherent
      __builtin_amdgcn_raw_ptr_buffer_load_lds(T.rx, (AMK_LDS void *)(p + RS::XO + j * 1024), 16,
                                               (int)off, 0, 0, kCachePolicySc1);
  }
}

// A pass's prologue, part one: the weight copies of its first D rounds. On a task's first pass
// this is issued before the task's dependency wait.
template <int WT, int GP, bool GAIN, bool WIDE>
__device__ __forceinline__ void ring_prefetch(const MfmaTile &T, RingLanes &L, int g0, int gn) {
  using RS = RingShape<WT, GP, GAIN, WIDE>;
  const int NR = T.t1 - T.t0;
  if constexpr (WT == 2) L.soff = lane_id() < 16 * gn ? (uint32_t)((16 * g0 + lane_id()) * T.ng) * 4u : kNoRow;
#pragma unroll
  for (int r = 0; r < RS::D; ++r) ring_issue_w<WT, GP, GAIN, WIDE>(T, L, g0, gn, r < NR, r, r);
}

template <int N>
__device__ __forceinline__ void wait_vm() {
  asm volatile("s_waitcnt vmcnt(%0)" ::"n"(N) : "memory");
}
// Round r is in LDS. Issue order: the first D rounds' weight copies (ring_prefetch), their input
// copies, then one whole round per iteration. For r < D the copies issued after round r are the
// later prologue rounds' inputs plus r + 1 whole rounds; after that, D whole rounds.
template <int D, int NX, int NI, int I = 0>
__device__ __forceinline__ void wait_round(int r) {
  if constexpr (I < D) {
    if (r == I) {
      wait_vm<(D - 1 - I) * NX + (I + 1) * NI>();
      return;
    }
    wait_round<D, NX, NI, I + 1>(r);
  } else {
    wait_vm<D * NI>();
  }
}

// One pass (groups [g0, g0 + gn)) of the ring stream; `prefetched`: ring_prefetch already ran.
template <int WT, int GP, bool GAIN, bool WIDE>
__device__ __forceinline__ void mfma_ring_pass(const MfmaTile &T, RingLanes &L, int g0, int gn,
                                               bool sumsq, float &ss, f32x4_t (&acc)[kMfmaGroups],
                                               bool prefetched) {
  using RS = RingShape<WT, GP, GAIN, WIDE>;
#pragma unroll
  for (int g = 0; g < kMfmaGroups; ++g) acc[g] = f32x4_t{0.f, 0.f, 0.f, 0.f};
  const int NR = T.t1 - T.t0, lane = lane_id();
  const int b = WIDE ? T.col : (T.col & 7);  // this lane's sequence (packed: hi or lo half of it)
  const bool xlive = b < T.B;
  if (!prefetched) ring_prefetch<WT, GP, GAIN, WIDE>(T, L, g0, gn);
#pragma unroll
  for (int r = 0; r < RS::D; ++r) ring_issue_x<WT, GP, GAIN, WIDE>(T, L, r < NR, r, r);
  int wslot = RS::D, rslot = 0;
  for (int r = 0; r < NR; ++r) {
    // the slot refilled now was read in the previous round: let those reads finish first
    asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
    const bool live = r + RS::D < NR;
    ring_issue_w<WT, GP, GAIN, WIDE>(T, L, g0, gn, live, r + RS::D, wslot);
    ring_issue_x<WT, GP, GAIN, WIDE>(T, L, live, r + RS::D, wslot);
    wslot = wslot + 1 == RS::NS ? 0 : wslot + 1;
    wait_round<RS::D, RS::NX, RS::NI>(r);
    const AMK_LDS uint8_t *p = L.ring + rslot * RS::SB;
    rslot = rslot + 1 == RS::NS ? 0 : rslot + 1;
    const int k = 32 * (T.t0 + r) + 8 * T.kq;
    float xv[8];
    if (T.emb) {
      const u32x4_t e = *(const AMK_LDS u32x4_t *)(p + RS::XO + (b * 32 + 8 * T.kq) * 2);
      xv[0] = bf_lo(e.x); xv[1] = bf_hi(e.x); xv[2] = bf_lo(e.y); xv[3] = bf_hi(e.y);
      xv[4] = bf_lo(e.z); xv[5] = bf_hi(e.z); xv[6] = bf_lo(e.w); xv[7] = bf_hi(e.w);
    } else {
      const AMK_LDS u32x4_t *xp = (const AMK_LDS u32x4_t *)(p + RS::XO + (b * 32 + 8 * T.kq) * 4);
      const u32x4_t a = xp[0], c = xp[1];
      xv[0] = __uint_as_float(a.x); xv[1] = __uint_as_float(a.y);
      xv[2] = __uint_as_float(a.z); xv[3] = __uint_as_float(a.w);
      xv[4] = __uint_as_float(c.x); xv[5] = __uint_as_float(c.y);
      xv[6] = __uint_as_float(c.z); xv[7] = __uint_as_float(c.w);
    }
    u32x4_t gw = {0u, 0u, 0u, 0u};
    if constexpr (GAIN) gw = *(const AMK_LDS u32x4_t *)(p + RS::GO + T.kq * 16);
    uint32_t hx[4], lx[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      float v0 = (xlive && k + 2 * i < T.K) ? xv[2 * i] : 0.f;
      float v1 = (xlive && k + 2 * i + 1 < T.K) ? xv[2 * i + 1] : 0.f;
      if (sumsq && (WIDE || !T.lo_half)) ss = fmaf(v0, v0, fmaf(v1, v1, ss));
      if constexpr (GAIN) {
        v0 *= bf_lo(gw[i]);
        v1 *= bf_hi(gw[i]);
      }
      const uint16_t h0 = f32_to_bf16(v0), h1 = f32_to_bf16(v1);
      const uint16_t l0 = f32_to_bf16(v0 - bf16_to_f32(h0)), l1 = f32_to_bf16(v1 - bf16_to_f32(h1));
      if (!WIDE && T.lo_half)
        hx[i] = (uint32_t)l0 | ((uint32_t)l1 << 16);
      else
        hx[i] = (uint32_t)h0 | ((uint32_t)h1 << 16);
      lx[i] = (uint32_t)l0 | ((uint32_t)l1 << 16);
    }
    const bf16x8_t xb = bf16x8_of_bits(hx[0], hx[1], hx[2], hx[3]);
    const bf16x8_t xl = bf16x8_of_bits(lx[0], lx[1], lx[2], lx[3]);  // wide only
    if constexpr (WT == 2) {
      const uint32_t c136 = 0x43084308u;  // bf16 136.0, twice
      const bf16x8_t a136 = bf16x8_of_bits(c136, c136, c136, c136);
      f32x4_t corr = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a136, xb, f32x4_t{0.f, 0.f, 0.f, 0.f}, 0, 0, 0);
      if constexpr (WIDE) corr = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a136, xl, corr, 0, 0, 0);
      const f32x4_t ncorr = -corr;
#pragma unroll
      for (int g = 0; g < GP; ++g) {
        if (g < gn) {
          const uint32_t w = *(const AMK_LDS uint32_t *)(p + g * 1024 + lane * 4);
          const f32x4_t sc = *(const AMK_LDS f32x4_t *)(p + RS::SO + (16 * g + 4 * T.kq) * 4);
          const bf16x8_t a = bf16x8_of_i4_offset(w);
          f32x4_t q = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, xb, ncorr, 0, 0, 0);
          if constexpr (WIDE) q = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, xl, q, 0, 0, 0);
#pragma unroll
          for (int i = 0; i < 4; ++i) acc[g][i] = fmaf(q[i], sc[i], acc[g][i]);
        }
      }
    } else {
#pragma unroll
      for (int g = 0; g < GP; ++g) {
        if (g < gn) {
          bf16x8_t a;
          if constexpr (WT == 0) {
            const u32x4_t w = *(const AMK_LDS u32x4_t *)(p + g * 1024 + lane * 16);
            a = bf16x8_of_bits(w.x, w.y, w.z, w.w);
          } else {
            const u32x2_t w = *(const AMK_LDS u32x2_t *)(p + g * 1024 + lane * 8);
            a = bf16x8_of_i8(w.x, w.y);
          }
          acc[g] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, xb, acc[g], 0, 0, 0);
          if constexpr (WIDE) acc[g] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, xl, acc[g], 0, 0, 0);
        }
      }
    }
  }
  // the rounds issued past the end land in the ring too: drain them before the LDS is reused
  asm volatile("s_waitcnt vmcnt(0)" ::: "memory");
}

template <int WT, bool WIDE>
__device__ __forceinline__ void ring_dispatch(const MfmaTile &T, RingLanes &L, int g0, int gn, bool sq,
                                              float &ss, f32x4_t (&acc)[kMfmaGroups], bool prefetched) {
  if (T.gain) {
    if (gn <= 1) mfma_ring_pass<WT, 1, true, WIDE>(T, L, g0, gn, sq, ss, acc, prefetched);
    else if (gn == 2) mfma_ring_pass<WT, 2, true, WIDE>(T, L, g0, gn, sq, ss, acc, prefetched);
    else if (gn == 3) mfma_ring_pass<WT, 3, true, WIDE>(T, L, g0, gn, sq, ss, acc, prefetched);
    else mfma_ring_pass<WT, 4, true, WIDE>(T, L, g0, gn, sq, ss, acc, prefetched);
  } else {
    if (gn <= 1) mfma_ring_pass<WT, 1, false, WIDE>(T, L, g0, gn, sq, ss, acc, prefetched);
    else if (gn == 2) mfma_ring_pass<WT, 2, false, WIDE>(T, L, g0, gn, sq, ss, acc, prefetched);
    else if (gn == 3) mfma_ring_pass<WT, 3, false, WIDE>(T, L, g0, gn, sq, ss, acc, prefetched);
    else mfma_ring_pass<WT, 4, false, WIDE>(T, L, g0, gn, sq, ss, acc, prefetched);
  }
}

template <int WT, bool WIDE>
__device__ __forceinline__ void ring_prefetch_dispatch(const MfmaTile &T, RingLanes &L, int g0, int gn) {
  if (T.gain) {
    if (gn <= 1) ring_prefetch<WT, 1, true, WIDE>(T, L, g0, gn);
    else if (gn == 2) ring_prefetch<WT, 2, true, WIDE>(T, L, g0, gn);
    else if (gn == 3) ring_prefetch<WT, 3, true, WIDE>(T, L, g0, gn);
    else ring_prefetch<WT, 4, true, WIDE>(T, L, g0, gn);
  } else {
    if (gn <= 1) ring_prefetch<WT, 1, false, WIDE>(T, L, g0, gn);
    else if (gn == 2) ring_prefetch<WT, 2, false, WIDE>(T, L, g0, gn);
    else if (gn == 3) ring_prefetch<WT, 3, false, WIDE>(T, L, g0, gn);
    else ring_prefetch<WT, 4, false, WIDE>(T, L, g0, gn);
  }
}

// Row groups of the pass that starts at group g0: the tile's G groups in ceil(G / kMfmaGroups)
// passes of nearly equal size, the larger first (5 groups: 3 + 2; 6: 3 + 3; 7: 4 + 3). A pass of
// three keeps three rounds in flight in the ring against two for a pass of four.
__device__ __forceinline__ int pass_groups(int G, int g0) {
  const int np = (G + kMfmaGroups - 1) / kMfmaGroups;
  const int base = G / np, big = (G % np) * (base + 1);  // the first G % np passes have base + 1
  return g0 < big ? base + 1 : base;
}

// A batched GEMV tile in two parts. gemv_mfma_begin sets the tile up and, on the ring path,
// issues the first pass's weight copies; it reads nothing the step produces, so a task calls it
// before its dependency wait and gemv_mfma_end (inputs, passes, reduction) after.
// `tiled`: W is in the tile-major layout (weight_tiled_bytes) and r0 a multiple of 16; else
// row-major. RING (megakernel instances, whose LDS region `mred` holds kRingBytes per wave): a
// tile-major matrix is streamed through the waves' LDS rings, and each wave's partial tiles sit at
// the start of its own ring; otherwise the loads go to registers.
struct MfmaJob {
  MfmaTile T;
  RingLanes L;
  int G, NC, wave, lane;
  bool wide, ring;
};

template <int WT, bool RING>
__device__ __forceinline__ void gemv_mfma_begin(MfmaJob &J, const DevModel &m, const StepArgs &s,
                                                const void *W, bool tiled, const float *scale, int K,
                                                int r0, int r1, const BatchInput &in, float *mred) {
  constexpr int NW = kWaves;
  MfmaTile &T = J.T;
  const int B = s.batch, n = r1 - r0, G = (n + 15) / 16;
  const int lane = lane_id(), wave = (int)uniform_u32((uint32_t)wave_id());
  J.G = G;
  J.lane = lane;
  J.wave = wave;
  T.K = K;
  T.n = n;
  T.rb = WT == 2 ? K / 2 : K * (WT ? 1 : 2);
  T.gs = WT == 2 ? m.gs : 32;
  T.ng = K / T.gs;
  T.sc = WT == 2 ? scale + (int64_t)r0 * T.ng : nullptr;
  const int steps = (K + 31) / 32;
  T.t0 = (int)((int64_t)steps * wave / NW);
  T.t1 = (int)((int64_t)steps * (wave + 1) / NW);
  T.col = lane & 15;
  T.kq = lane >> 4;
  J.wide = B > 8;  // one column per sequence, both halves by two instructions
  J.NC = J.wide ? 16 : 8;  // columns of the partial tiles in LDS
  T.lo_half = !J.wide && T.col >= 8;
  T.emb = in.emb != nullptr;
  T.gain = in.gain != nullptr;
  T.B = B;
  const uint32_t lb = WT == 0 ? 16u : (WT == 1 ? 8u : 4u);  // one lane's 8 weights, bytes
  if (tiled) {  // a k step of a 16-row group is one 64-lane run
    T.wl = (uint32_t)lane * lb;
    T.wt = 64u * lb;
    T.wg = (uint32_t)steps * T.wt;
    T.rw = make_rsrc(static_cast<const uint8_t *>(W) + (int64_t)(r0 / 16) * T.wg, (uint32_t)G * T.wg);
  } else {
    T.wl = (uint32_t)T.col * (uint32_t)T.rb + (uint32_t)T.kq * lb;
    T.wt = 4u * lb;
    T.wg = 16u * (uint32_t)T.rb;
    T.rw = make_rsrc(static_cast<const uint8_t *>(W) + (int64_t)r0 * T.rb, (uint32_t)n * (uint32_t)T.rb);
  }
  T.rx = in.emb ? make_rsrc(in.emb, (uint32_t)m.V * (uint32_t)K * 2u)
                : make_rsrc(in.x, (uint32_t)B * (uint32_t)in.stride * 4u);
  T.rg = make_rsrc(in.gain ? in.gain : m.final_norm, (uint32_t)K * 2u);
  J.ring = RING && tiled;
  if constexpr (RING) {
    if (J.ring) {
      RingLanes &L = J.L;
      L.ring = (AMK_LDS uint8_t *)(mred) + wave * kRingBytes;
      L.rs = make_rsrc(WT == 2 ? T.sc : scale, WT == 2 ? (uint32_t)(n * T.ng) * 4u : 0u);
      L.woff = (uint32_t)lane < T.wt / 16u ? (uint32_t)lane * 16u : kNoRow;  // a tile is T.wt bytes
      L.goff = lane < 4 ? (uint32_t)lane * 16u : kNoRow;
      L.soff = kNoRow;
      const int gn = pass_groups(G, 0);
      if (J.wide)
        ring_prefetch_dispatch<WT, true>(T, L, 0, gn);
      else
        ring_prefetch_dispatch<WT, false>(T, L, 0, gn);
    }
  }
}

// After gemv_mfma_begin with the ring prefetch in flight, a task that abandons the tile (its
// dependency wait failed) lets the copies land before it leaves.
__device__ __forceinline__ void gemv_mfma_abandon() { asm volatile("s_waitcnt vmcnt(0)" ::: "memory"); }

template <int WT, bool RING>
__device__ __forceinline__ void gemv_mfma_end(MfmaJob &J, const DevModel &m, const StepArgs &s,
                                              const float *scale, int r0, const BatchInput &in,
                                              float *ys, float *red, float *mred) {
  constexpr int NW = kWaves;
  MfmaTile &T = J.T;
  RingLanes &L = J.L;
  const int B = s.batch, n = T.n, G = J.G, K = T.K, NC = J.NC, lane = J.lane, wave = J.wave;
  const bool wide = J.wide, ring = J.ring;
  // where the inputs come from (the tokens of a later step of a multi-step launch are written by
  // the previous step, so only now)
  const int b = wide ? T.col : (T.col & 7);
  // register path: one load per sequence and k; packed lo-half lanes receive the inputs from
  // their hi-half lane
  T.xrow = kNoRow;
  if (b < B && !T.lo_half)
    T.xrow = in.emb ? (uint32_t)token_of(m, s, b) * (uint32_t)K * 2u : (uint32_t)b * (uint32_t)in.stride * 4u;
  if (ring) {
    if (in.emb) {  // bf16 rows: 4 lanes of 16 bytes per sequence and k step, 16 sequences
      const int bx = lane >> 2;
      L.xoff[0] = bx < B ? (uint32_t)token_of(m, s, bx) * (uint32_t)K * 2u + (uint32_t)(lane & 3) * 16u : kNoRow;
      L.xoff[1] = kNoRow;
      L.xstep = 64u;
    } else {  // fp32 rows: 8 lanes per sequence and k step, 8 sequences per copy
#pragma unroll
      for (int j = 0; j < 2; ++j) {
        const int bx = 8 * j + (lane >> 3);
        L.xoff[j] = bx < B ? (uint32_t)bx * (uint32_t)in.stride * 4u + (uint32_t)(lane & 7) * 16u : kNoRow;
      }
      L.xstep = 128u;
    }
  }
  // partial tiles: wave w's at mred + w * wstride, [group][16 rows][NC]
  const int wstride = ring ? kRingBytes / 4 : kMfmaGroups * 16 * NC;
  float ss = 0.f;
  for (int g0 = 0, gn = 0; g0 < G; g0 += gn) {
    gn = pass_groups(G, g0);
    const bool sq = in.sumsq && g0 == 0;
    f32x4_t acc[kMfmaGroups];
    if constexpr (RING) {
      if (ring) {
        if (wide)
          ring_dispatch<WT, true>(T, L, g0, gn, sq, ss, acc, g0 == 0);
        else
          ring_dispatch<WT, false>(T, L, g0, gn, sq, ss, acc, g0 == 0);
      }
    }
    if (!ring) {
      if (wide)
        mfma_dispatch<WT, true>(T, g0, gn, sq, ss, acc);
      else
        mfma_dispatch<WT, false>(T, g0, gn, sq, ss, acc);
    }
    // partial tiles of all waves (16 columns: hi and lo halves) -> ys
#pragma unroll
    for (int g = 0; g < kMfmaGroups; ++g)
      if (g < gn)
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          // column c of row 4 kq + i: hi and lo of one sequence land in the same float
          const int row = 4 * T.kq + i;
          float v = acc[g][i];
          if (!wide) v += __shfl_xor(v, 8, 64);  // lanes c and c ^ 8: the halves of sequence c & 7
          if (T.col < NC) mred[wave * wstride + (g * 16 + row) * NC + T.col] = v;
        }
    __syncthreads();
    for (int e = threadIdx.x; e < gn * 16 * NC; e += NW * 64) {
      const int g = e / (16 * NC), row = (e / NC) & 15, bb = e % NC;
      const int r = 16 * (g0 + g) + row;
      if (bb < B && r < n) {
        float t = 0.f;
        for (int w = 0; w < NW; ++w) t += mred[w * wstride + (g * 16 + row) * NC + bb];
        if constexpr (WT == 1) t *= gld(&scale[r0 + r]);
        ys[bb * n + r] = t;
      }
    }
    __syncthreads();
  }
  if (in.sumsq) {
    ss += __shfl_xor(ss, 16, 64);
    ss += __shfl_xor(ss, 32, 64);
    if (T.kq == 0 && T.col < B && (wide || T.col < 8)) red[T.col * NW + wave] = ss;
  }
}

template <int WT, bool RING = false>
__device__ __forceinline__ void gemv_mfma(const DevModel &m, const StepArgs &s, const void *W, bool tiled,
                                          const float *scale, int K, int r0, int r1, const BatchInput &in,
                                          float *ys, float *red, float *mred) {
  MfmaJob J;
  gemv_mfma_begin<WT, RING>(J, m, s, W, tiled, scale, K, r0, r1, in, mred);
  gemv_mfma_end<WT, RING>(J, m, s, scale, r0, in, ys, red, mred);
}

// ------------------------------------------------------------------------------------------
// epilogues (ys in LDS, n = r1 - r0 rows per batch row)
// ------------------------------------------------------------------------------------------
__device__ __forceinline__ int64_t kv_index(const DevModel &m, const StepArgs &s, int l, int kvi,
                                            int b, int g, int p, int dim) {
  const int64_t kb = s.kv_seq >= 0 ? s.kv_seq : b;  // the KV sequence of column b
  return (((((int64_t)l * 2 + kvi) * s.kv_batch + kb) * m.nkv + g) * s.kv_max_seq + p) *
             (int64_t)m.hd + dim;
}

// QKV rows: RoPE on pairs of rotary rows, q -> q buffer (fp32), k/v -> KV cache slot pos (bf16).
__device__ __forceinline__ void epi_qkv(const DevModel &m, const StepArgs &s, int l, int r0, int r1,
                        const float *ys, int nw) {
  const int n = r1 - r0, hd = m.hd, half = hd / 2;
  for (int b = 0; b < s.batch; ++b) {
    const int pb = pos_of(s, b);
    const float2 *cs = m.rope + (int64_t)pb * half;
    for (int pi = threadIdx.x; pi < n / 2; pi += nw * 64) {
      const int r = r0 + 2 * pi;
      const QkvRow q0 = qkv_decode(r, m.nq, m.nkv, hd);
      const QkvRow q1 = qkv_decode(r + 1, m.nq, m.nkv, hd);
      float v0 = ys[b * n + 2 * pi], v1 = ys[b * n + 2 * pi + 1];
      if (q0.kind != KIND_V) {  // rotary pair (dim j, dim j + hd/2)
        const u32x2_t cw = *(const AMK_GAS u32x2_t *)&cs[q0.dim];
        const float2 c = make_float2(__uint_as_float(cw.x), __uint_as_float(cw.y));
        const float a = v0, bb = v1;
        v0 = a * c.x - bb * c.y;
        v1 = bb * c.x + a * c.y;
      }
      if (q0.kind == KIND_Q) {
        if (m.max_batch == 1) {  // batch 1: q only as tagged words, for the attention blocks
          uint32_t *qb = m.qt + (int64_t)l * m.qd;
          cst(&qb[q0.head * hd + q0.dim], tag_word(v0, s.epoch));
          cst(&qb[q1.head * hd + q1.dim], tag_word(v1, s.epoch));
        } else {
          float *qb = m.q + ((int64_t)l * m.max_batch + b) * m.qd;
          cstf(&qb[q0.head * hd + q0.dim], v0);
          cstf(&qb[q1.head * hd + q1.dim], v1);
        }
      } else {
        const int kvi = (q0.kind == KIND_K) ? 0 : 1;
        const uint16_t k0 = f32_to_bf16(v0), k1 = f32_to_bf16(v1);
        uint16_t *c0 = &s.kv[kv_index(m, s, l, kvi, b, q0.head, pb, q0.dim)];
        uint16_t *c1 = &s.kv[kv_index(m, s, l, kvi, b, q1.head, pb, q1.dim)];
        if (m.max_batch == 1) {
          // This step's attention blocks take the row from tagged words. A single-step launch's
          // cache row is read only by later launches (the kernel boundary makes it visible), so
          // plain stores do: device-coherent 2-byte stores are slow to complete, and any later
          // load in this workgroup would wait for them (loads and stores share one counter). In
          // a multi-step launch the next step reads it as history, from any XCD.
          if (s.n_steps > 1) {
            cst(c0, k0);
            cst(c1, k1);
          } else {
            gst(c0, k0);
            gst(c1, k1);
          }
          uint32_t *kb = m.kvt + (((int64_t)l * 2 + kvi) * m.nkv + q0.head) * hd;
          const uint32_t tg = s.epoch & kTagMask;
          cst(&kb[q0.dim], ((uint32_t)k0 << 16) | tg);
          cst(&kb[q1.dim], ((uint32_t)k1 << 16) | tg);
        } else {
          cst(c0, k0);
          cst(c1, k1);
        }
      }
    }
  }
}

// out[b][r] = res[b][r] + ys (res slot 0 = the embedding row of the token)
__device__ __forceinline__ void epi_residual(const DevModel &m, const StepArgs &s, int res_slot, int out_slot,
                             int r0, int r1, const float *ys, int nw) {
  const int n = r1 - r0, d = m.d;
  for (int b = 0; b < s.batch; ++b) {
    float *out = m.h + ((int64_t)out_slot * m.max_batch + b) * d;
    const float *res = m.h + ((int64_t)res_slot * m.max_batch + b) * d;
    const uint16_t *e = (res_slot == 0) ? m.embed + (int64_t)token_of(m, s, b) * d : nullptr;
    for (int i = threadIdx.x; i < n; i += nw * 64) {
      const int r = r0 + i;
      const float base = e ? bf16_to_f32(gld(&e[r])) : cldf(&res[r]);
      cstf(&out[r], base + ys[b * n + i]);
    }
  }
}

__device__ __forceinline__ void epi_swiglu(const DevModel &m, const StepArgs &s, int l, int r0, int r1,
                           const float *ys, int nw) {
  const int n = r1 - r0;
  for (int b = 0; b < s.batch; ++b) {
    float *a = m.a + ((int64_t)l * m.max_batch + b) * m.F;
    for (int i = threadIdx.x; i < n / 2; i += nw * 64)
      cstf(&a[r0 / 2 + i], silu(ys[b * n + 2 * i]) * ys[b * n + 2 * i + 1]);
  }
}

// batch-1 (tagged) forms of the residual and SwiGLU epilogues. The residual word is read untagged:
// the tile has already staged a complete tagged input whose producers had read that same residual
// slot, so the slot is current.
__device__ void epi_residual_tagged(const DevModel &m, const StepArgs &s, int res_slot,
                                    int out_slot, int r0, int r1, const float *ys, int nw) {
  const int n = r1 - r0, d = m.d;
  uint32_t *out = m.ht + (int64_t)out_slot * d;
  const uint32_t *res = m.ht + (int64_t)res_slot * d;
  const uint16_t *e = (res_slot == 0) ? m.embed + (int64_t)token_of(m, s, 0) * d : nullptr;
  for (int i = threadIdx.x; i < n; i += nw * 64) {
    const int r = r0 + i;
    const float base = e ? bf16_to_f32(gld(&e[r])) : untag(cld(&res[r]));
    cst(&out[r], tag_word(base + ys[i], s.epoch));
  }
}
__device__ void epi_swiglu_tagged(const DevModel &m, const StepArgs &s, int l, int r0, int r1,
                                  const float *ys, int nw) {
  const int n = r1 - r0;
  uint32_t *a = m.at + (int64_t)l * m.F;
  for (int i = threadIdx.x; i < n / 2; i += nw * 64)
    cst(&a[r0 / 2 + i], tag_word(silu(ys[2 * i]) * ys[2 * i + 1], s.epoch));
}

// logits rows + (max, lowest index of max) of this tile into amax[slot][b]
__device__ __forceinline__ void epi_logits(const DevModel &m, const StepArgs &s, int r0, int r1, int slot,
                           const float *ys, float *red, int nw) {
  const int n = r1 - r0;
  float *lg = s.logits ? s.logits : m.logits;
  for (int b = 0; b < s.batch; ++b) {
    float best = -INFINITY;
    int bi = 0x7fffffff;
    for (int i = threadIdx.x; i < n; i += nw * 64) {
      const float v = ys[b * n + i];
      gst(&lg[(int64_t)b * m.V + r0 + i], v);
      if (v > best) { best = v; bi = r0 + i; }
    }
#pragma unroll
    for (int o = 32; o >= 1; o >>= 1) {
      const float ov = __shfl_xor(best, o, 64);
      const int oi = __shfl_xor(bi, o, 64);
      if (ov > best || (ov == best && oi < bi)) { best = ov; bi = oi; }
    }
    __syncthreads();
    if (lane_id() == 0) {
      red[2 * wave_id()] = best;
      red[2 * wave_id() + 1] = __int_as_float(bi);
    }
    __syncthreads();
    if (threadIdx.x == 0) {
      float bv = red[0];
      int bj = __float_as_int(red[1]);
      for (int w = 1; w < nw; ++w) {
        const float v = red[2 * w];
        const int j = __float_as_int(red[2 * w + 1]);
        if (v > bv || (v == bv && j < bj)) { bv = v; bj = j; }
      }
      cst(reinterpret_cast<uint64_t *>(&m.amax[(int64_t)slot * m.max_batch + b]),
          (uint64_t)__float_as_uint(bv) | ((uint64_t)(uint32_t)bj << 32));
    }
  }
}

// next[b] = argmax over the LM tiles' partials (value desc, index asc); one wave.
__device__ __forceinline__ void argmax_combine(const DevModel &m, const StepArgs &s, int n_slots) {
  if (wave_id() != 0) return;
  for (int b = 0; b < s.batch; ++b) {
    float best = -INFINITY;
    int bi = 0x7fffffff;
    for (int k = lane_id(); k < n_slots; k += 64) {
      const uint64_t p = cld(reinterpret_cast<const uint64_t *>(&m.amax[(int64_t)k * m.max_batch + b]));
      const float v = __uint_as_float((uint32_t)p);
      const int j = (int)(uint32_t)(p >> 32);
      if (v > best || (v == best && j < bi)) { best = v; bi = j; }
    }
#pragma unroll
    for (int o = 32; o >= 1; o >>= 1) {
      const float ov = __shfl_xor(best, o, 64);
      const int oi = __shfl_xor(bi, o, 64);
      if (ov > best || (ov == best && oi < bi)) { best = ov; bi = oi; }
    }
    if (lane_id() == 0) cst(&s.next[b], (bi == 0x7fffffff) ? 0 : bi);
  }
}

// ------------------------------------------------------------------------------------------
// attention partial for (layer l, kv group g, KV block blk) over positions [lo, hi) of ctx.
// LDS: q [qpg][hd] | scores [qpg][chunk] | acc [nw][qpg*hd] | appended K/V row [2][hd] bf16.
// Lane layout: LPR = hd/8 lanes per KV row (8 dims each), 64/LPR rows per wave per load.
// ------------------------------------------------------------------------------------------
// An empty KV block's partial: (m, l, acc) = (kEmptyBlockM, 0, 0). The value is finite (tagged
// words replace its low mantissa bits) and so far below any score that its merge weight
// e^{m - M} is exactly 0.
constexpr float kEmptyBlockM = -3.0e38f;

// q of heads [h0, h0 + qn) of KV group g (scaled by 1/sqrt(hd)) into qs [qn][hd] and the appended
// K/V row's bf16 values into kvrow [2][hd], from the QKV tiles' tagged words, reloaded until every
// tag is current (this is the wait for those tiles). Every query head of the group is polled,
// whichever heads this pass keeps: the task's declared wait is the QKV tiles of the whole group,
// and reading all their words keeps that exact. The words go in rounds of V per thread
// ((qpg + 2) * hd words: one round up to V * kThreads). Returns false after a timeout (recorded)
// or when the abort word is set.
__device__ bool attn_stage_tagged(const DevModel &m, const StepArgs &s, int l, int g, int h0,
                                  int qn, float *qs, uint16_t *kvrow, uint32_t task) {
  constexpr int V = 4;
  const int hd = m.hd, nqw = m.qpg * hd, n = nqw + 2 * hd, q0 = h0 * hd, q1 = (h0 + qn) * hd;
  const uint32_t tag = s.epoch & kTagMask;
  const uint32_t *qsrc = m.qt + (int64_t)l * m.qd + (int64_t)g * m.qpg * hd;
  const uint32_t *ksrc = m.kvt + ((int64_t)l * 2 * m.nkv + g) * hd;
  const uint32_t *vsrc = m.kvt + ((int64_t)(l * 2 + 1) * m.nkv + g) * hd;
  uint32_t *const err = m.err;
  const uint64_t tmo = m.timeout_ticks;
  uint64_t t0 = 0;
  uint32_t spins = 0;
  for (int base = 0; base < n; base += V * kThreads) {
    uint32_t need = 0;
#pragma unroll
    for (int j = 0; j < V; ++j)
      if (base + (int)threadIdx.x + j * kThreads < n) need |= 1u << j;
    while (true) {
      uint32_t w[V];
#pragma unroll
      for (int j = 0; j < V; ++j) {
        const int i = base + (int)threadIdx.x + j * kThreads;
        if (need & (1u << j))
          w[j] = cld(i < nqw ? &qsrc[i] : (i < nqw + hd ? &ksrc[i - nqw] : &vsrc[i - nqw - hd]));
      }
      int ab = 0;
      if (threadIdx.x == 0 && (spins == 0 || (spins & 7) == 7)) {
        ab = flag_load(&err[1]) != 0;
        if (!ab && spins && wall_clock64() - t0 > tmo) {
          record_error(err, ERR_TIMEOUT, task, 0xfffffff1u);
          __hip_atomic_store(gptr(&err[1]), 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
          ab = 1;
        }
      }
#pragma unroll
      for (int j = 0; j < V; ++j) {
        const int i = base + (int)threadIdx.x + j * kThreads;
        if ((need & (1u << j)) && (w[j] & kTagMask) == tag) {
          need &= ~(1u << j);
          if (i < nqw) {
            if (i >= q0 && i < q1) qs[i - q0] = untag(w[j]) * m.attn_scale;
          } else {
            kvrow[i - nqw] = (uint16_t)(w[j] >> 16);
          }
        }
      }
      const int pending = __syncthreads_or(need != 0);
      if (__syncthreads_or(ab)) return false;
      if (!pending) break;
      if (spins == 0) t0 = wall_clock64();
      ++spins;
      __builtin_amdgcn_s_sleep(1);
    }
  }
  return true;
}

// Attention partials, on every path (batch-1 and batched megakernel instances, the operator
// kernels): heads [h0, h0 + qn) of KV group g, KV block blk, for every sequence of the step.
// Each wave streams its own rows, like a GEMV tile: sequence b's block is cut into chunks of
// kWaves * U * RPW rows, wave w takes U * RPW consecutive rows of each chunk, and the wave walks
// its chunks of all sequences in order with two register buffers, the next chunk's loads issued
// before the current one is folded. The softmax is online per row slot of the wave (running
// max, sum and weighted V), so nothing but the end of a sequence synchronises the waves: there
// each wave folds its row slots together, writes (acc, m, l) to LDS, and after one barrier all
// threads merge the waves' partials into the sequence's partial. q and the appended K/V row of
// every sequence (written by this step's QKV tiles) are read once after the wait, into LDS; the
// first chunk is issued before it. Partials stay in LDS until every sequence is done and then
// go out in one burst (a store in the loop would hold up the next chunk's wait: vector loads and
// stores complete under one counter). wait_for (batched megakernel): the QKV tiles' flags,
// polled by wave 0. TAGGED (batch 1, one sequence): q and the appended row are read from the QKV
// tiles' tagged words (attn_stage_tagged, which is also the wait), the first chunk is issued
// before and the second after that staging, and the partial goes out as tagged words straight
// from the merge over waves. LDS: q [B][qn][HD] | appended rows [B][2][HD] bf16 | partials
// [B][qn][HD + 2] | wave partials [2][NW][qn][HD + 2].
template <int HD, int QMAX, bool TAGGED>
__device__ __forceinline__ bool attn_block_seqs(const DevModel &m, const StepArgs &s, int l,
                                                int g, int blk, int h0, int qn, float *lds,
                                                float *red, const Task *wait_for,
                                                int *abort_slot) {
  (void)red;
  constexpr int NW = kWaves;
  constexpr int LPR = HD / 8;       // lanes per row (8 bf16 each)
  constexpr int RPW = 64 / LPR;     // row slots of a wave
  // loads of K (and of V) per chunk: more for one-head batch-1 passes (their registers allow it)
  constexpr bool LONG = TAGGED && QMAX == 1;
  constexpr int U = LONG ? kAttnSeqItersB1 : kAttnSeqIters;
  constexpr int CR = U * RPW;       // rows of a wave's chunk
  constexpr int WR = NW * CR;       // rows of a workgroup chunk
  static_assert(WR == attn_seq_chunk_rows(HD, LONG), "chunk rows");
  const int B = s.batch, nblk = m.nblk, nq = m.nq;
  if (B <= 0) return true;
  const int lane = lane_id(), wave = __builtin_amdgcn_readfirstlane(wave_id());
  const int sub = lane % LPR, rs = lane / LPR;
  float *qall = lds;                                                   // [B][qn][HD]
  uint16_t *rows = reinterpret_cast<uint16_t *>(qall + B * qn * HD);   // [B][2][HD]
  float *parts = qall + B * qn * HD + B * HD;                          // [B][qn][HD + 2]
  float *wpart = parts + B * qn * (HD + 2);                            // [2][NW][qn][HD + 2]

  // a position in the stream of (sequence, chunk) pairs; sequences without rows in this block
  // are skipped. Every field is wave-uniform.
  struct Cur {
    int b, c, lo, hi, nch, pos;
  };
  auto seq_at = [&](int b, Cur &cu) __attribute__((always_inline)) {
    cu.b = b;
    cu.c = 0;
    cu.pos = pos_of(s, b);
    attn_block_range(cu.pos + 1, nblk, blk, &cu.lo, &cu.hi);
    cu.nch = cu.hi > cu.lo ? (cu.hi - cu.lo + WR - 1) / WR : 0;
  };
  auto from = [&](int b, Cur &cu) __attribute__((always_inline)) {
    cu.nch = 0;
    for (; b < B && cu.nch == 0; ++b) seq_at(b, cu);
  };
  auto advance = [&](Cur &cu) __attribute__((always_inline)) {
    if (++cu.c == cu.nch) from(cu.b + 1, cu);
  };
  int S = 0;
  for (int b = 0; b < B; ++b) {
    int lo, hi;
    attn_block_range(pos_of(s, b) + 1, nblk, blk, &lo, &hi);
    if (hi > lo) S += (hi - lo + WR - 1) / WR;
  }

  // the wave's rows of a chunk. Loads are unconditional: rows past the block re-read its last
  // row (skipped when folded); a per-lane branch or select here would make the compiler wait
  // for every outstanding load at the first use, i.e. for the next chunk too.
  auto load = [&](const Cur &cu, uint4 (&kr)[U], uint4 (&vr)[U]) __attribute__((always_inline)) {
    const uint16_t *Kb = s.kv + kv_index(m, s, l, 0, cu.b, g, 0, 0);
    const uint16_t *Vb = s.kv + kv_index(m, s, l, 1, cu.b, g, 0, 0);
    const int j0 = cu.lo + cu.c * WR + wave * CR + rs;
#pragma unroll
    for (int it = 0; it < U; ++it) {
      const int j = min(j0 + it * RPW, cu.hi - 1);
      kr[it] = load_nt(reinterpret_cast<const uint4 *>(Kb + (int64_t)j * HD + sub * 8));
      vr[it] = load_nt(reinterpret_cast<const uint4 *>(Vb + (int64_t)j * HD + sub * 8));
    }
  };

  float acc[QMAX][8], lsum[QMAX], mrun[QMAX];
  auto reset = [&]() __attribute__((always_inline)) {
#pragma unroll
    for (int h = 0; h < QMAX; ++h) {
      lsum[h] = 0.f;
      mrun[h] = kEmptyBlockM;
#pragma unroll
      for (int e = 0; e < 8; ++e) acc[h][e] = 0.f;
    }
  };
  int ended = 0;  // sequences finished so far: picks the wave-partial buffer
  // fold one chunk into the row slot's (acc, lsum, mrun); at the sequence's last chunk, merge
  auto fold = [&](const Cur &cu, const uint4 (&kr)[U], const uint4 (&vr)[U]) __attribute__((always_inline)) {
    const int b = cu.b, pos = cu.pos;
    const float *qs = qall + b * qn * HD + sub * 8;
    const uint16_t *row = rows + b * 2 * HD;
    // the appended row as register values: the empty asm keeps the compiler from turning the
    // choice below into a choice of addresses, which would move kr / vr to the stack
    uint4 rk = *reinterpret_cast<const uint4 *>(row + sub * 8);
    uint4 rv = *reinterpret_cast<const uint4 *>(row + HD + sub * 8);
    asm("" : "+v"(rk.x), "+v"(rk.y), "+v"(rk.z), "+v"(rk.w), "+v"(rv.x), "+v"(rv.y), "+v"(rv.z), "+v"(rv.w));
    const int j0 = cu.lo + cu.c * WR + wave * CR + rs;
    float sc[U][QMAX];
#pragma unroll
    for (int it = 0; it < U; ++it) {
      const int j = j0 + it * RPW;
      const uint4 k = (j == pos) ? rk : kr[it];
#pragma unroll
      for (int h = 0; h < QMAX; ++h) {
        float p = 0.f;
        if (h < qn) {
          p = group_sum<LPR>(dot8_bf16(k, qs + h * HD));
        }
        sc[it][h] = p;
      }
    }
#pragma unroll
    for (int h = 0; h < QMAX; ++h) {
      if (h < qn) {
        float mc = mrun[h];
#pragma unroll
        for (int it = 0; it < U; ++it)
          if (j0 + it * RPW < cu.hi) mc = fmaxf(mc, sc[it][h]);
        const float f = __expf(mrun[h] - mc);
        mrun[h] = mc;
        lsum[h] *= f;
#pragma unroll
        for (int e = 0; e < 8; ++e) acc[h][e] *= f;
#pragma unroll
        for (int it = 0; it < U; ++it) sc[it][h] = (j0 + it * RPW < cu.hi) ? __expf(sc[it][h] - mc) : 0.f;
      }
    }
#pragma unroll
    for (int it = 0; it < U; ++it) {
      const int j = j0 + it * RPW;
      const uint4 v = (j == pos) ? rv : vr[it];
      const float vv[8] = {bf_lo(v.x), bf_hi(v.x), bf_lo(v.y), bf_hi(v.y),
                           bf_lo(v.z), bf_hi(v.z), bf_lo(v.w), bf_hi(v.w)};
#pragma unroll
      for (int h = 0; h < QMAX; ++h) {
        if (h < qn) {
          lsum[h] += sc[it][h];
#pragma unroll
          for (int e = 0; e < 8; ++e) acc[h][e] = fmaf(sc[it][h], vv[e], acc[h][e]);
        }
      }
    }
    if (cu.c != cu.nch - 1) return;
    // end of sequence b: fold the wave's row slots (lanes with equal sub), then the waves
    float *wp = wpart + (ended & 1) * NW * qn * (HD + 2) + wave * qn * (HD + 2);
#pragma unroll
    for (int h = 0; h < QMAX; ++h) {
      if (h < qn) {
        float mx = mrun[h];
#pragma unroll
        for (int o = LPR; o < 64; o <<= 1) mx = fmaxf(mx, xor_lanes(mx, o));
        const float f = __expf(mrun[h] - mx);
        float t = lsum[h] * f;
#pragma unroll
        for (int e = 0; e < 8; ++e) acc[h][e] *= f;
#pragma unroll
        for (int o = LPR; o < 64; o <<= 1) {
          t += xor_lanes(t, o);
#pragma unroll
          for (int e = 0; e < 8; ++e) acc[h][e] += xor_lanes(acc[h][e], o);
        }
        if (rs == 0) {
#pragma unroll
          for (int e = 0; e < 8; ++e) wp[h * (HD + 2) + sub * 8 + e] = acc[h][e];
        }
        if (lane == 0) {
          wp[h * (HD + 2) + HD] = mx;
          wp[h * (HD + 2) + HD + 1] = t;
        }
      }
    }
    reset();
    __syncthreads();
    const float *w0 = wpart + (ended & 1) * NW * qn * (HD + 2);
    float *pl = parts + b * qn * (HD + 2);
    for (int i = threadIdx.x; i < qn * (HD + 2); i += NW * 64) {
      const int h = i / (HD + 2), e = i - h * (HD + 2);
      float mx = kEmptyBlockM;
      for (int w = 0; w < NW; ++w) mx = fmaxf(mx, w0[w * qn * (HD + 2) + h * (HD + 2) + HD]);
      float t = 0.f;
      if (e == HD) {
        t = mx;
      } else {
        for (int w = 0; w < NW; ++w)
          t += __expf(w0[w * qn * (HD + 2) + h * (HD + 2) + HD] - mx) * w0[w * qn * (HD + 2) + i];
      }
      if constexpr (TAGGED) {
        // batch 1: the only sequence's partial goes out at once, as tagged words
        float *pout = m.part + ((((int64_t)l * m.max_batch + b) * nq + (int64_t)g * m.qpg + h0 + h) * nblk + blk) * (HD + 2);
        cst(reinterpret_cast<uint32_t *>(&pout[e]), tag_word(t, s.epoch));
      } else {
        pl[i] = t;
      }
    }
    ++ended;
  };

  reset();
  Cur lc, cc;
  from(0, lc);
  cc = lc;
  uint4 P[2][U], A[2][U], Bf[2][U];
  // the first chunk goes out before the wait (the KV history does not depend on it), the second
  // after the staging: a CU's loads return in order, and the staging polls would otherwise wait
  // behind both chunks (7B, 64 KB per chunk: 2.643 -> 2.605 ms per step)
  if constexpr (TAGGED) {
    if (S > 0) load(lc, P[0], P[1]);
    asm volatile("" ::: "memory");  // issue it before the staging loads, not at its first use
    // q (scaled) and the appended K/V row: epoch-tagged words, the staging loads are the wait
    if (!attn_stage_tagged(m, s, l, g, h0, qn, qall, rows, wait_for ? wait_for->id : 0u)) {
      __builtin_amdgcn_s_waitcnt(0);
      return false;
    }
    if (m.trace && wait_for && h0 == 0 && threadIdx.x == 0)
      gst(&m.trace[(uint64_t)wait_for->id * 4 + 1], (uint64_t)wall_clock64());
  } else {
    // wave 0 polls the flags and a wave's loads return in order, so it issues its first chunk
    // after polling; the other waves issue theirs before the join. Chunk 1 goes out after the
    // join: q is read behind whatever is in flight.
    if (wait_for) wait_poll(m, *wait_for, s.epoch, abort_slot);
    if (S > 0) load(lc, P[0], P[1]);
    asm volatile("" ::: "memory");  // issue them before the join, not at their first use
    if (wait_for && !wait_join(m, *wait_for, abort_slot)) return false;
    // q (scaled by 1/sqrt(hd)) and the appended K/V rows of every sequence: one round of
    // device-coherent 4-byte loads (this step's QKV tiles wrote them)
    for (int i = threadIdx.x; i < B * qn * HD; i += NW * 64) {
      const int b = i / (qn * HD), r = i - b * (qn * HD);
      qall[i] = cldf(&m.q[((int64_t)l * m.max_batch + b) * m.qd + ((int64_t)g * m.qpg + h0) * HD + r]) *
                m.attn_scale;
    }
    for (int i = threadIdx.x; i < B * HD; i += NW * 64) {  // 32-bit words: [B][2][HD / 2]
      const int b = i / HD, r = i - b * HD, kvi = r / (HD / 2), w = r - kvi * (HD / 2);
      const uint32_t *src = reinterpret_cast<const uint32_t *>(
          s.kv + kv_index(m, s, l, kvi, b, g, pos_of(s, b), 0));
      reinterpret_cast<uint32_t *>(rows)[i] = cld(&src[w]);
    }
  }
  // every thread's loads so far (chunk 0 too), also where a thread staged nothing: the wait
  // counts of the stream below then start from no pending loads on every path
  __builtin_amdgcn_s_waitcnt(kWaitVm0);
  __syncthreads();
  {  // chunk 1, for both paths
    if (S > 1) {
      advance(lc);
      load(lc, A[0], A[1]);
    }
    asm volatile("" ::: "memory");
  }
  // the stream: P (chunk 0, complete by now) is folded while A (chunk 1) arrives; the steady loop
  // enters and loops back with exactly one buffer of loads in flight, so the compiler's wait
  // for a buffer leaves the other buffer's loads outstanding. The empty asm statements keep each
  // chunk's loads issued ahead of the previous chunk's arithmetic.
  if (S > 0) {
    fold(cc, P[0], P[1]);
    if (S > 1) {
      advance(cc);
      int t = 1;
      for (; t + 2 < S; t += 2) {
        advance(lc);
        load(lc, Bf[0], Bf[1]);
        asm volatile("" ::: "memory");
        fold(cc, A[0], A[1]);
        advance(cc);
        advance(lc);
        load(lc, A[0], A[1]);
        asm volatile("" ::: "memory");
        fold(cc, Bf[0], Bf[1]);
        advance(cc);
      }
      if (t + 1 < S) {
        advance(lc);
        load(lc, Bf[0], Bf[1]);
        asm volatile("" ::: "memory");
        fold(cc, A[0], A[1]);
        advance(cc);
        fold(cc, Bf[0], Bf[1]);
      } else {
        fold(cc, A[0], A[1]);
      }
    }
  }
  // a batch-1 partial went out from the merge (the caller's barrier ends the task)
  if (TAGGED && S > 0) return true;
  __syncthreads();
  // every sequence's partial of this block, [b][h][HD + 2]: device-coherent stores; a sequence
  // without rows here gives the empty partial
  const int per = qn * (HD + 2);
  for (int i = threadIdx.x; i < B * per; i += NW * 64) {
    const int b = i / per, r = i - b * per, h = r / (HD + 2), e = r - h * (HD + 2);
    int lo, hi;
    attn_block_range(pos_of(s, b) + 1, nblk, blk, &lo, &hi);
    const float v = hi > lo ? parts[i] : (e == HD ? kEmptyBlockM : 0.f);
    float *pout = m.part + ((((int64_t)l * m.max_batch + b) * nq + (int64_t)g * m.qpg + h0 + h) * nblk + blk) * (HD + 2);
    if constexpr (TAGGED)
      cst(reinterpret_cast<uint32_t *>(&pout[e]), tag_word(v, s.epoch));
    else
      cstf(&pout[e], v);
  }
  return true;
}

// Attention tasks always run with kWaves waves (kThreads threads). The task covers query heads
// [hs, hs + hn) of KV group g (a megakernel task's aux2 / aux3; the whole group when aux3 is 0 and
// for the operator kernels); more heads than QMAX are processed QMAX heads at a time (the KV block
// is re-read from cache for each pass). wait_for (megakernel) is waited on inside the first pass,
// after the KV-history prefetch.
template <int HD, int QMAX, bool TAGGED>
__device__ __forceinline__ bool attn_task(const DevModel &m, const StepArgs &s, int l, int g,
                                          int blk, float *lds, float *red, const Task *wait_for,
                                          int *abort_slot) {
  const int hs = (wait_for && wait_for->aux3) ? (int)wait_for->aux2 : 0;
  const int hn = (wait_for && wait_for->aux3) ? (int)wait_for->aux3 : m.qpg;
  // the partial waits for the QKV tiles only; a merger's wait for its group's other blocks (the
  // second range) comes in attn_merge
  Task first{};
  if (wait_for) {
    first = *wait_for;
    first.w1_lo = first.w1_hi = 0;
  }
  for (int h0 = hs; h0 < hs + hn; h0 += QMAX) {
    const Task *w = (wait_for && (TAGGED || h0 == hs)) ? &first : nullptr;
    {
      if (!attn_block_seqs<HD, QMAX, TAGGED>(m, s, l, g, blk, h0, min(QMAX, hs + hn - h0), lds, red, w,
                                     abort_slot))
        return false;
    }
  }
  return true;
}

// Merge of KV group g's nblk partials into the attention output, run by the group's last block
// (the designated merger) after its own partial:
//   o[h][e] = sum_k e^{m_k - M} acc_k[e] / sum_k e^{m_k - M} l_k,  M = max_k m_k
// (log-sum-exp over the blocks; an empty block's weight is exactly 0). TAGGED (batch 1): the other
// blocks store no flag, their partials are tagged words reloaded until every tag matches, and
// the output is written tagged. Otherwise the other blocks' flags (the task's second wait range)
// are waited on first. The merger's own partial is read back like the others once its stores
// are complete. Each thread merges whole output elements, eight blocks' loads at a time.
template <bool TAGGED>
__device__ __forceinline__ bool attn_merge(const DevModel &m, const StepArgs &s, const Task &t, int *abort_slot) {
  const int l = t.layer, g = (int)t.a0;
  if constexpr (!TAGGED) {
    Task others = t;  // the group's other blocks (the QKV tiles were waited on for the partial)
    others.w0_lo = others.w0_hi = 0;
    if (!wait_task(m, others, s.epoch, abort_slot)) return false;
  }
  __builtin_amdgcn_s_waitcnt(0);  // this block's own partial stores are complete
  __syncthreads();
  constexpr int KB = 8;
  const int hd = m.hd, nblk = m.nblk, qpg = m.qpg, nq = m.nq;
  // the task's query heads [hs, hs + hn) of the group (the whole group when aux3 is 0)
  const int hs = t.aux3 ? (int)t.aux2 : 0, hn = t.aux3 ? (int)t.aux3 : qpg;
  const int per_b = hn * hd, total = s.batch * per_b;
  const uint32_t tag = s.epoch & kTagMask;
  uint32_t *const err = m.err;
  const uint64_t tmo = m.timeout_ticks;
  uint32_t done = 0;  // elements (one bit per loop iteration of this thread) already written
  uint64_t t0 = 0;
  uint32_t spins = 0;
  while (true) {
    int stale = 0;
    int it = 0;
    for (int i = threadIdx.x; i < total; i += kThreads, ++it) {
      if (TAGGED && (done & (1u << it))) continue;  // TAGGED: at most 8 elements per thread
      const int b = i / per_b, r = i - b * per_b, h = g * qpg + hs + r / hd, e = r % hd;
      const uint32_t *ph = reinterpret_cast<const uint32_t *>(m.part) +
                           (((int64_t)l * m.max_batch + b) * nq + h) * nblk * (hd + 2);
      float M = kEmptyBlockM, den = 0.f, num = 0.f;
      uint32_t bad = 0;
      for (int k0 = 0; k0 < nblk; k0 += KB) {
        uint32_t wm[KB], wl[KB], wa[KB];
#pragma unroll
        for (int j = 0; j < KB; ++j) {
          const uint32_t *pk = ph + (int64_t)min(k0 + j, nblk - 1) * (hd + 2);
          wm[j] = cld(pk + hd);
          wl[j] = cld(pk + hd + 1);
          wa[j] = cld(pk + e);
        }
        // tagged partials are read with their tag bits cleared
        auto val = [](uint32_t w) { return TAGGED ? untag(w) : __uint_as_float(w); };
        float Mb = M;
#pragma unroll
        for (int j = 0; j < KB; ++j) {
          if (TAGGED) bad |= ((wm[j] ^ tag) | (wl[j] ^ tag) | (wa[j] ^ tag)) & kTagMask;
          if (k0 + j < nblk) Mb = fmaxf(Mb, val(wm[j]));
        }
        const float f = __expf(M - Mb);
        den *= f;
        num *= f;
#pragma unroll
        for (int j = 0; j < KB; ++j) {
          if (k0 + j < nblk) {
            const float w = __expf(val(wm[j]) - Mb);
            den = fmaf(w, val(wl[j]), den);
            num = fmaf(w, val(wa[j]), num);
          }
        }
        M = Mb;
      }
      if (bad) {
        stale = 1;
        continue;
      }
      if constexpr (TAGGED) done |= 1u << it;
      if constexpr (TAGGED)
        cst(&m.aot[(int64_t)l * m.qd + (int64_t)h * hd + e], tag_word(num / den, s.epoch));
      else
        cstf(&m.ao[((int64_t)l * m.max_batch + b) * m.qd + (int64_t)h * hd + e], num / den);
    }
    if constexpr (!TAGGED) return true;
    int ab = 0;
    if (threadIdx.x == 0 && (spins & 7) == 7) {
      ab = flag_load(&err[1]) != 0;
      if (!ab && wall_clock64() - t0 > tmo) {
        record_error(err, ERR_TIMEOUT, t.id, 0xfffffff2u);
        __hip_atomic_store(gptr(&err[1]), 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        ab = 1;
      }
    }
    const int pending = __syncthreads_or(stale);
    if (__syncthreads_or(ab)) return false;
    if (!pending) return true;
    if (spins == 0) t0 = wall_clock64();
    ++spins;
    __builtin_amdgcn_s_sleep(1);
  }
}

// ------------------------------------------------------------------------------------------
// weights of a GEMV matrix
// ------------------------------------------------------------------------------------------
__device__ __forceinline__ void gemv_matrix(const DevModel &m, int mat, int l, const void **W,
                                            const float **scale, int *K, int *wtype) {
  *wtype = m.wtype;
  switch (mat) {
    case M_QKV: *W = gld(&m.layers[l].qkv); *scale = gld(&m.layers[l].s_qkv); *K = m.d; break;
    case M_O: *W = gld(&m.layers[l].o); *scale = gld(&m.layers[l].s_o); *K = m.qd; break;
    case M_GU: *W = gld(&m.layers[l].gu); *scale = gld(&m.layers[l].s_gu); *K = m.d; break;
    case M_D: *W = gld(&m.layers[l].dn); *scale = gld(&m.layers[l].s_dn); *K = m.F; break;
    default:
      *W = m.lm;
      *scale = m.lm_scale;
      *K = m.d;
      if (m.tied) *wtype = 0;
      break;
  }
}

}  // namespace amk
