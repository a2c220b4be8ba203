// The persistent decode megakernel: one workgroup per CU walks its frozen task list.
//
// Ada-MK technical summary ("Methodology", Phase I and II): the whole decode step runs as one
// persistent kernel whose execution order was fixed offline and serialised, so the device makes
// no decision about what to run where. Each workgroup reads its own list of tile tasks; before a
// task it waits (one wave spinning on agent-scope flags, then an acquire), runs the task body
// with all 16 waves, and publishes its own flag with an agent-scope release. Dependencies between
// CUs are point-to-point flags; there is no grid-wide barrier.
//
// The kernel is instantiated per (weight type, head_dim, query heads per pass) so that each
// instance carries a single GEMV and a single attention body.
#include <hip/hip_runtime.h>

#include "device.h"

namespace amk {

template <int WT>
__device__ __forceinline__ void run_gemv_task(const DevModel &m, const StepArgs &s, const Task &t,
                                              float *xs, float *ys, float *red) {
  constexpr int NW = kWaves;
  const int l = t.layer;
  const void *W;
  const float *scale;
  int K, wtype;
  gemv_matrix(m, t.mat, l, &W, &scale, &K, &wtype);
  switch (t.mat) {
    case M_QKV: stage_norm(m, s, 2 * l, m.layers[l].attn_norm, xs, red, NW); break;
    case M_O: stage_combine(m, s, l, xs, NW); break;
    case M_GU: stage_norm(m, s, 2 * l + 1, m.layers[l].mlp_norm, xs, red, NW); break;
    case M_D: stage_plain(m.a + (int64_t)l * m.max_batch * m.F, m.F, m.F, s.batch, xs, NW); break;
    default: stage_norm(m, s, 2 * m.L, m.final_norm, xs, red, NW); break;
  }
  const int r0 = (int)t.a0, r1 = (int)t.a1;
  if (WT == 1 && wtype == 1)
    gemv_rows<1>(W, scale, K, r0, r1, xs, ys, s.batch, NW);
  else
    gemv_rows<0>(W, scale, K, r0, r1, xs, ys, s.batch, NW);
  __syncthreads();
  switch (t.mat) {
    case M_QKV: epi_qkv(m, s, l, r0, r1, ys, NW); break;
    case M_O: epi_residual(m, s, 2 * l, 2 * l + 1, r0, r1, ys, NW); break;
    case M_GU: epi_swiglu(m, s, l, r0, r1, ys, NW); break;
    case M_D: epi_residual(m, s, 2 * l + 1, 2 * l + 2, r0, r1, ys, NW); break;
    default: epi_logits(m, s, r0, r1, (int)t.aux0, ys, red, NW); break;
  }
}

template <int WT, int HD, int QMAX>
__device__ __forceinline__ void megakernel_body(const DevModel &m, const StepArgs &s) {
  extern __shared__ float lds[];
  const int32_t xa = lds_xs_floats(m.max_batch, m.d, m.qd, m.F);
  const int32_t xb = lds_attn_floats(m.max_batch, m.qpg, m.hd);
  float *xs = lds;
  float *red = lds + (xa > xb ? xa : xb);  // 64 * 8 floats
  float *ys = red + 64 * 8;                // batch * max_tile_rows floats
  __shared__ int abort_flag;
  const uint32_t t0 = m.offsets[blockIdx.x], t1 = m.offsets[blockIdx.x + 1];
  for (uint32_t ti = t0; ti < t1; ++ti) {
    const Task t = m.tasks[ti];
    if (wave_id() == 0) {
      bool ok = true;
      if (t.w0_hi > t.w0_lo) ok = wait_range(m, t.w0_lo, t.w0_hi, s.epoch, t.id);
      if (ok && t.w1_hi > t.w1_lo) ok = wait_range(m, t.w1_lo, t.w1_hi, s.epoch, t.id);
      if (lane_id() == 0) abort_flag = ok ? 0 : 1;
    }
    __syncthreads();
    if (abort_flag) return;
    if (t.type == T_GEMV)
      run_gemv_task<WT>(m, s, t, xs, ys, red);
    else if (t.type == T_ATTN)
      attn_task<HD, QMAX>(m, s, t.layer, (int)t.a0, (int)t.a1, xs, red);
    else
      argmax_combine(m, s, (int)t.aux0);
    __syncthreads();
    if (threadIdx.x == 0)
      __hip_atomic_store(&m.flags[t.id], s.epoch, __ATOMIC_RELEASE, __HIP_MEMORY_SCOPE_AGENT);
  }
}

}  // namespace amk

using namespace amk;

#define AMK_MK(WT, HD, Q)                                                          \
  extern "C" __global__ void __launch_bounds__(kThreads, 1)                        \
      amk_megakernel_w##WT##_h##HD##_q##Q(const DevModel *__restrict__ mp, StepArgs s) { \
    megakernel_body<WT, HD, Q>(*mp, s);                                            \
  }

AMK_MK(0, 64, 1)
AMK_MK(0, 64, 2)
AMK_MK(0, 64, 4)
AMK_MK(0, 128, 1)
AMK_MK(0, 128, 2)
AMK_MK(0, 128, 4)
AMK_MK(1, 64, 1)
AMK_MK(1, 64, 2)
AMK_MK(1, 64, 4)
AMK_MK(1, 128, 1)
AMK_MK(1, 128, 2)
AMK_MK(1, 128, 4)
