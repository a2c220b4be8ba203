// The persistent decode megakernel: one workgroup per CU walks its frozen task list.
//
// Ada-MK technical summary ("Methodology", Phase I and II): the whole decode step runs as one
// persistent kernel whose execution order was fixed offline and serialised, so the device makes
// no decision about what to run where. Each workgroup reads its own list of tile tasks; before a
// task it waits (one wave spinning on device-scope flags), runs the task body with all of its
// waves, and publishes its own flag once its stores have completed. Dependencies between CUs are
// point-to-point flags; there is no grid-wide barrier.
//
// The kernel is instantiated per (weight type, head_dim, query heads per pass) so that each
// instance carries a single GEMV and a single attention body.
#include <hip/hip_runtime.h>

#include "device.h"

namespace amk {

// Task t waiting instead on the previous step's argmax (multi-step launches).
__device__ __forceinline__ Task prev_step(const DevModel &m, const Task &t) {
  Task w = t;
  w.w0_lo = m.argmax_id;
  w.w0_hi = m.argmax_id + 1;
  w.w1_lo = w.w1_hi = 0;
  return w;
}

// Batch-1 staging of an int8 GEMV's input from its epoch-tagged producer words (which doubles as
// the dependency wait; the first layer's QKV tiles read the embedding and have no producer): the
// input goes to LDS as integer digits and *sx receives their unit weight.
__device__ __forceinline__ bool stage_b1_digits(const DevModel &m, const StepArgs &s, const Task &t,
                                                int K, float *xs, float *red, float *sx) {
  const int l = t.layer;
  switch (t.mat) {
    case M_QKV:
      if (l == 0) {
        stage_norm(m, s, 0, gld(&m.layers[0].attn_norm), xs, red, kWaves);
        *sx = stage_digits(xs, K, red);
        return true;
      }
      return stage_tagged<true>(m, m.ht + (int64_t)2 * l * m.d, m.d, gld(&m.layers[l].attn_norm),
                                  s.epoch, xs, red, t.id, sx);
    case M_O:
      return stage_tagged<true>(m, m.aot + (int64_t)l * m.qd, m.qd, nullptr, s.epoch, xs, red,
                                  t.id, sx);
    case M_GU:
      return stage_tagged<true>(m, m.ht + (int64_t)(2 * l + 1) * m.d, m.d,
                                  gld(&m.layers[l].mlp_norm), s.epoch, xs, red, t.id, sx);
    case M_D:
      return stage_tagged<true>(m, m.at + (int64_t)l * m.F, m.F, nullptr, s.epoch, xs, red, t.id,
                                  sx);
    default:
      return stage_tagged<true>(m, m.ht + (int64_t)2 * m.L * m.d, m.d, m.final_norm, s.epoch, xs,
                                  red, t.id, sx);
  }
}

// Batch-1 int8 / int4 GEMV body: as the bf16 body in gemv_task, with one of two stream shapes
// (SA one row per chunk, SB several) and the input staged as digits.
template <class SA, class SB>
__device__ __forceinline__ bool gemv_b1_q(const DevModel &m, const StepArgs &s, const Task &t,
                                           const void *W, const float *scale, int K, bool use_b,
                                           float *xs, float *ys, float *red, uint4 *pf,
                                           int *abort_slot) {
  SA sa;
  SB sb;
  uint4 P[kChunkUnits];
  uint4 *slot;
  if (use_b) {
    sb.init(W, scale, m.gs, K, (int)t.a0, (int)t.a1, kWaves);
    slot = pf + sb.wave * (64 * kChunkUnits);
  } else {
    sa.init(W, scale, m.gs, K, (int)t.a0, (int)t.a1, kWaves);
    slot = pf + sa.wave * (64 * kChunkUnits);
  }
  const bool tagged = !(t.mat == M_QKV && t.layer == 0);
  if (!tagged) wait_poll(m, s.step > 0 ? prev_step(m, t) : t, s.epoch - (s.step > 0), abort_slot);
  if (use_b) {
    if (sb.S > 0) sb.load_lds(0, slot);
    if (sb.S > 1) sb.load(P, 1);
  } else {
    if (sa.S > 0) sa.load_lds(0, slot);
    if (sa.S > 1) sa.load(P, 1);
  }
  asm volatile("" ::: "memory");
  if (!tagged && !wait_join(m, t, abort_slot)) return false;
  if (m.trace && threadIdx.x == 0) gst(&m.trace[(uint64_t)t.id * 4 + 1], (uint64_t)wall_clock64());
  float sx = 0.f;
  if (!stage_b1_digits(m, s, t, K, xs, red, &sx)) {
    __builtin_amdgcn_s_waitcnt(0);  // no copy into LDS may outlive the workgroup
    return false;
  }
  if (m.trace && threadIdx.x == 0) gst(&m.trace[(uint64_t)t.id * 4 + 2], (uint64_t)wall_clock64());
  const uint8_t *xd = reinterpret_cast<const uint8_t *>(xs);
  if (use_b)
    sb.run_pf(slot, P, xd, sx, ys, scale);
  else
    sa.run_pf(slot, P, xd, sx, ys, scale);
  return true;
}

// GEMV tile task. Batch 1: the first two weight chunks of every wave (one into its LDS slot, one
// into registers) are issued at once, then the input is staged from its epoch-tagged producer
// words, which is also the dependency wait (int8, int4: gemv_b1_q). Batched: a flag wait (wave 0 polls), then the matrix-core GEMV reads its inputs
// straight from memory. The RMSNorm scale is applied to the outputs and the epilogue writes them
// (tagged for batch 1).
// pre0 (batch-1 bf16): the previous task on this CU already issued chunk 0 of every wave into
// its LDS slot (gemv_issue_chunk0).
template <int WT, bool BATCHED>
__device__ __forceinline__ bool gemv_task(const DevModel &m, const StepArgs &s, const Task &t,
                                          float *xs, float *ys, float *red, uint4 *pf,
                                          int *abort_slot, bool pre0 = false) {
  constexpr int NW = kWaves;
  const int l = t.layer;
  const void *W;
  const float *scale;
  int K, wtype;
  gemv_matrix(m, t.mat, l, &W, &scale, &K, &wtype);
  const int r0 = (int)t.a0, r1 = (int)t.a1;
  // The kernel instance (and its LDS layout: staged input and prefetch slots, or the matrix
  // cores' partial tiles) follows the model's batch capacity; a smaller step batch runs the
  // batched GEMV with zero columns.
  constexpr bool b1 = !BATCHED;
  if (b1) {
    if constexpr (WT == 0) {
      GemvStream<0> st;
      uint4 P[kChunkUnits];
      st.init(W, K, r0, r1, NW);
      uint4 *slot = pf + st.wave * (64 * kChunkUnits);
      // inputs produced in this step by other tiles are tagged with the epoch, so their staging
      // loads are the dependency wait (no flags): the weight prefetch is issued at once
      const bool tagged = !(t.mat == M_QKV && l == 0);
      // the first layer's QKV tiles read the token: in a later step of a multi-step launch they
      // wait for the previous step's argmax (which every task of that step precedes)
      if (!tagged) wait_poll(m, s.step > 0 ? prev_step(m, t) : t, s.epoch - (s.step > 0), abort_slot);
      if (st.S > 0 && !pre0) st.load_lds(0, slot);
      if (st.S > 1) st.load(P, 1);
      // keep the register prefetch issued here, ahead of the staging loads, not at its first use
      asm volatile("" ::: "memory");
      if (!tagged && !wait_join(m, t, abort_slot)) return false;
      if (m.trace && threadIdx.x == 0) gst(&m.trace[(uint64_t)t.id * 4 + 1], (uint64_t)wall_clock64());
      bool ok = true;
      switch (t.mat) {
        case M_QKV:
          if (l == 0)
            stage_norm(m, s, 0, gld(&m.layers[0].attn_norm), xs, red, NW);
          else
            ok = stage_tagged<false>(m, m.ht + (int64_t)2 * l * m.d, m.d,
                                     gld(&m.layers[l].attn_norm), s.epoch, xs, red, t.id);
          break;
        case M_O:
          ok = stage_tagged<false>(m, m.aot + (int64_t)l * m.qd, m.qd, nullptr, s.epoch, xs, red,
                                   t.id);
          break;
        case M_GU:
          ok = stage_tagged<false>(m, m.ht + (int64_t)(2 * l + 1) * m.d, m.d,
                                   gld(&m.layers[l].mlp_norm), s.epoch, xs, red, t.id);
          break;
        case M_D:
          ok = stage_tagged<false>(m, m.at + (int64_t)l * m.F, m.F, nullptr, s.epoch, xs, red, t.id);
          break;
        default:
          ok = stage_tagged<false>(m, m.ht + (int64_t)2 * m.L * m.d, m.d, m.final_norm, s.epoch, xs,
                                   red, t.id);
          break;
      }
      if (!ok) {
        __builtin_amdgcn_s_waitcnt(0);  // no copy into LDS may outlive the workgroup
        return false;
      }
      if (m.trace && threadIdx.x == 0) gst(&m.trace[(uint64_t)t.id * 4 + 2], (uint64_t)wall_clock64());
      st.run_pf(slot, P, xs, ys, scale);
    } else if constexpr (WT == 1) {
      // int8 rows of 256 units (K = 4096) fill half a chunk: two rows per chunk
      if (!gemv_b1_q<GemvStreamI8<1>, GemvStreamI8<2>>(m, s, t, W, scale, K,
                                                       K == 16 * 32 * kChunkUnits, xs, ys, red,
                                                       pf, abort_slot))
        return false;
    } else {
      // int4 rows of 128 units (K = 4096): four rows per chunk
      if (!gemv_b1_q<GemvStreamI4<1>, GemvStreamI4<4>>(m, s, t, W, scale, K,
                                                       K == 32 * 16 * kChunkUnits, xs, ys, red,
                                                       pf, abort_slot))
        return false;
    }
  } else {
    // batched: inputs straight from memory into the matrix cores (RMSNorm scale applied after)
    BatchInput in{nullptr, m.d, nullptr, nullptr, true};
    const int64_t hb = (int64_t)m.max_batch * m.d;
    switch (t.mat) {
      case M_QKV:
        if (l == 0) in.emb = m.embed; else in.x = m.h + 2 * l * hb;
        in.gain = gld(&m.layers[l].attn_norm);
        break;
      case M_O: in = BatchInput{m.ao + (int64_t)l * m.max_batch * m.qd, m.qd, nullptr, nullptr, false}; break;
      case M_GU: in.x = m.h + (2 * l + 1) * hb; in.gain = gld(&m.layers[l].mlp_norm); break;
      case M_D: in = BatchInput{m.a + (int64_t)l * m.max_batch * m.F, m.F, nullptr, nullptr, false}; break;
      default: in.x = m.h + 2 * (int64_t)m.L * hb; in.gain = m.final_norm; break;
    }
    // the first weight copies go out before the dependency wait (weights do not depend on it)
    MfmaJob job;
    gemv_mfma_begin<WT, true>(job, m, s, W, m.tiled && !(t.mat == M_LM && m.tied), scale, K, r0, r1, in, xs);
    if ((s.step > 0 && t.mat == M_QKV && l == 0 && !wait_task(m, prev_step(m, t), s.epoch - 1, abort_slot)) ||
        !wait_task(m, t, s.epoch, abort_slot)) {
      gemv_mfma_abandon();
      return false;
    }
    if (m.trace && threadIdx.x == 0) gst(&m.trace[(uint64_t)t.id * 4 + 2], (uint64_t)wall_clock64());
    gemv_mfma_end<WT, true>(job, m, s, scale, r0, in, ys, red, xs);
  }
  __syncthreads();
  if (t.mat != M_O && t.mat != M_D) norm_scale_ys(m, s, r1 - r0, ys, red, NW);
  switch (t.mat) {
    case M_QKV: epi_qkv(m, s, l, r0, r1, ys, NW); break;
    case M_O:
      if (b1) epi_residual_tagged(m, s, 2 * l, 2 * l + 1, r0, r1, ys, NW);
      else epi_residual(m, s, 2 * l, 2 * l + 1, r0, r1, ys, NW);
      break;
    case M_GU:
      if (b1) epi_swiglu_tagged(m, s, l, r0, r1, ys, NW);
      else epi_swiglu(m, s, l, r0, r1, ys, NW);
      break;
    case M_D:
      if (b1) epi_residual_tagged(m, s, 2 * l + 1, 2 * l + 2, r0, r1, ys, NW);
      else epi_residual(m, s, 2 * l + 1, 2 * l + 2, r0, r1, ys, NW);
      break;
    default: epi_logits(m, s, r0, r1, (int)t.aux0, ys, red, NW); break;
  }
  return true;
}

// Chunk 0 of every wave of batch-1 bf16 GEMV task t into its LDS slot, issued by the task before
// it on this CU once that task has no loads left to wait for (an attention block after its
// partial, a merger after its merge): the copy then overlaps the end of that task instead of
// following it, and gemv_task (pre0) issues the rest. Returns whether it issued.
template <int WT, bool BATCHED>
__device__ __forceinline__ bool gemv_issue_chunk0(const DevModel &m, const Task &t, uint4 *pf) {
  if constexpr (WT != 0 || BATCHED) {
    return false;
  } else {
    if (t.type != T_GEMV) return false;
    const void *W;
    const float *scale;
    int K, wtype;
    gemv_matrix(m, t.mat, t.layer, &W, &scale, &K, &wtype);
    GemvStream<0> st;
    st.init(W, K, (int)t.a0, (int)t.a1, kWaves);
    if (st.S > 0) st.load_lds(0, pf + st.wave * (64 * kChunkUnits));
    return true;
  }
}

// Whether a finished task's consumers learn of it from its flag. In batch-1 instances only the LM
// tiles (for the argmax) and the argmax do: every other task publishes tagged data (QKV: q and the
// appended K/V row; attention blocks: partials and the merged output; O, gate/up, down: their
// outputs) and neither waits for its stores nor stores a flag. The schedule validator's
// stores_flag is the same rule.
template <bool BATCHED>
__device__ __forceinline__ bool publishes_flag(const Task &t) {
  return BATCHED || t.type == T_ARGMAX || (t.type == T_GEMV && t.mat == M_LM);
}

template <int WT, int HD, int QMAX, bool BATCHED>
__device__ __forceinline__ void megakernel_body(const DevModel &m, const StepArgs &s0) {
  extern __shared__ __attribute__((aligned(16))) float lds[];  // 16-byte reads of xs need it
  const int32_t xa = lds_xs_floats(m.max_batch, m.d, m.qd, m.F);
  const int32_t xb = lds_attn_floats(m.max_batch, m.qpg, m.hd);
  float *xs = lds;
  float *red = lds + (xa > xb ? xa : xb);  // kRedFloats floats
  uint4 *pf = reinterpret_cast<uint4 *>(red + kRedFloats);  // lds_prefetch_floats(max_batch)
  float *ys = red + kRedFloats + lds_prefetch_floats(m.max_batch);  // batch * max_tile_rows
  __shared__ int abort_flag;
  if (threadIdx.x == 0) abort_flag = 0;
  __syncthreads();
  const uint32_t t0 = load_const(&m.offsets[blockIdx.x]), t1 = load_const(&m.offsets[blockIdx.x + 1]);
  uint64_t *const trace = m.trace;
  if (trace && threadIdx.x == 0) {
    // XCC (XCD) that runs this workgroup: HW_REG_XCC_ID, bits [3:0]
    const uint32_t xcc = __builtin_amdgcn_s_getreg((3 << 11) | (0 << 6) | 20);
    gst(&trace[(uint64_t)m.n_tasks * 4 + blockIdx.x], (uint64_t)xcc);
  }
  // Epoch of the last completed step, read once per workgroup. Every workgroup with tasks reads
  // it before its first task, and the store below comes after the last step's argmax, which
  // every task follows, so all of them see the same value. A workgroup without tasks may read
  // either value and uses neither.
  const uint32_t e0 = uniform_u32(flag_load(m.ectr));
  for (int step = 0; step < s0.n_steps; ++step) {
    StepArgs s = s0;
    s.step = step;
    s.epoch = e0 + 1u + (uint32_t)step;
    s.pos = s0.pos + step;
    s.posp = &s0.pos_in[0];
    if (step > 0) s.tokens = s0.next + (int64_t)(step - 1) * s0.batch;
    s.next = s0.next + (int64_t)step * s0.batch;
    if (s0.logits) s.logits = s0.logits + (int64_t)step * s0.batch * m.V;
    bool pre0 = false;  // the current task's chunk 0 was issued by the task before it
    for (uint32_t ti = t0; ti < t1; ++ti) {
      const Task t = load_task(&m.tasks[ti]);
      if (trace && threadIdx.x == 0) gst(&trace[(uint64_t)t.id * 4 + 0], (uint64_t)wall_clock64());
      bool ok;
      if (t.type == T_GEMV) {
        ok = gemv_task<WT, BATCHED>(m, s, t, xs, ys, red, pf, &abort_flag, pre0);
        pre0 = false;
      } else if (t.type == T_ATTN) {
        ok = attn_task<HD, QMAX, !BATCHED>(m, s, t.layer, (int)t.a0, (int)t.a1, xs, red, &t, &abort_flag);
        if (trace && threadIdx.x == 0) gst(&trace[(uint64_t)t.id * 4 + 2], (uint64_t)wall_clock64());
        if (ok && t.aux1) ok = attn_merge<!BATCHED>(m, s, t, &abort_flag);
        // the next task's first weight chunk, into the GEMV prefetch slots (unused by attention)
        if (ok && ti + 1 < t1) pre0 = gemv_issue_chunk0<WT, BATCHED>(m, load_task(&m.tasks[ti + 1]), pf);
      } else {
        ok = wait_task(m, t, s.epoch, &abort_flag);
        if (ok) argmax_combine(m, s, (int)t.aux0);
        // the launch's last step is complete: the next launch starts from its epoch
        if (ok && step == s0.n_steps - 1 && threadIdx.x == 0)
          __hip_atomic_store(gptr(m.ectr), s.epoch, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      }
      // a failed task leaves no copy into LDS in flight when the workgroup ends
      if (!ok) {
        __builtin_amdgcn_s_waitcnt(0);
        return;
      }
      // Publish: every wave waits for its own (device-coherent) stores to complete, the workgroup
      // meets, then one thread stores the flag. Data that crosses CUs is written with device-scope
      // stores, so no L2 writeback is needed before the flag.
      if (publishes_flag<BATCHED>(t)) {
        __builtin_amdgcn_s_waitcnt(0);
        __syncthreads();
        if (threadIdx.x == 0) {
          if (trace) gst(&trace[(uint64_t)t.id * 4 + 3], (uint64_t)wall_clock64());
          __hip_atomic_store(gptr(&m.flags[t.id]), s.epoch, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        }
      } else {
        __syncthreads();
        if (trace && threadIdx.x == 0) gst(&trace[(uint64_t)t.id * 4 + 3], (uint64_t)wall_clock64());
      }
    }
  }
}

}  // namespace amk

using namespace amk;

#define AMK_MK(WT, HD, Q)                                                                     \
  extern "C" __global__ void __launch_bounds__(kThreads, 1)                                   \
      amk_megakernel_w##WT##_h##HD##_q##Q(const DevModel *__restrict__ mp, StepArgs s) {      \
    megakernel_body<WT, HD, Q, false>(*mp, s);                                                \
  }                                                                                           \
  extern "C" __global__ void __launch_bounds__(kThreads, 1)                                   \
      amk_megakernel_w##WT##_h##HD##_q##Q##_b(const DevModel *__restrict__ mp, StepArgs s) {  \
    megakernel_body<WT, HD, Q, true>(*mp, s);                                                 \
  }

// batch-1 instances (weight stream with LDS prefetch) and batched ones (suffix _b: matrix cores).
// The build compiles this file once per (weight type, head_dim) pair, selected by AMK_MK_WT and
// AMK_MK_HD, so the instances compile in parallel; each object holds that pair's three instances.
#if !defined(AMK_MK_WT) || !defined(AMK_MK_HD)
#error "compile with -DAMK_MK_WT=<0|1|2> -DAMK_MK_HD=<64|128>"
#endif
#define AMK_MK_CAT(a, b, c) AMK_MK(a, b, c)
AMK_MK_CAT(AMK_MK_WT, AMK_MK_HD, 1)
AMK_MK_CAT(AMK_MK_WT, AMK_MK_HD, 2)
AMK_MK_CAT(AMK_MK_WT, AMK_MK_HD, 4)
