// Unfused ablation: the same decode step issued as one kernel launch per operator
// (embed, then per layer rmsnorm, QKV GEMV, RoPE + KV append, attention partials, attention
// combine, O GEMV + residual, rmsnorm, gate/up GEMV, SwiGLU, down GEMV + residual, then final
// rmsnorm, LM-head GEMV with per-workgroup argmax partials, argmax): 1 + 10 L + 3 launches.
// Kernel boundaries order the operators; intermediate vectors round-trip through HBM. The GEMV
// and attention bodies are the megakernel's.
#include <hip/hip_runtime.h>

#include "device.h"

namespace amk {
constexpr int kUfWaves = 8;          // GEMV workgroups: 8 waves
constexpr int kUfRowsPerBlock = 32;  // 4 rows per wave
}  // namespace amk

using namespace amk;

extern "C" __global__ void __launch_bounds__(256) amk_uf_embed(const DevModel *__restrict__ mp,
                                                               StepArgs s) {
  const DevModel &m = *mp;
  const int b = blockIdx.y;
  const uint16_t *e = m.embed + (int64_t)token_of(m, s, b) * m.d;
  float *h0 = m.h + (int64_t)b * m.d;
  for (int i = blockIdx.x * 256 + threadIdx.x; i < m.d; i += gridDim.x * 256) h0[i] = bf16_to_f32(e[i]);
}

// dst[b] = rmsnorm(src[b]) * gain, one workgroup per sequence
extern "C" __global__ void __launch_bounds__(1024) amk_uf_rmsnorm(const DevModel *__restrict__ mp,
                                                                  const float *src, const uint16_t *gain,
                                                                  float *dst) {
  const DevModel &m = *mp;
  __shared__ float red[16];
  const int b = blockIdx.x, d = m.d;
  const float *x = src + (int64_t)b * d;
  float ss = 0.f;
  for (int i = threadIdx.x; i < d; i += 1024) ss += x[i] * x[i];
  const float tot = block_sum(ss, red, 16);
  const float inv = 1.0f / sqrtf(tot / (float)d + m.eps);
  for (int i = threadIdx.x; i < d; i += 1024) dst[(int64_t)b * d + i] = x[i] * inv * bf16_to_f32(gain[i]);
}

// mode 0: y[b][r] = W x ; mode 1: out[b][r] = res[b][r] + W x ; mode 2: logits + argmax partial
template <int WT, int MODE>
__device__ void uf_gemv(const DevModel &m, const StepArgs &s, const void *W, const float *scale,
                        int K, int rows, const float *x, float *y, const float *res, float *out) {
  extern __shared__ __attribute__((aligned(16))) float lds[];  // 16-byte reads of xs need it
  float *red = lds;                       // 64 * 8
  float *ys = red + 64 * 8;               // batch * kUfRowsPerBlock
  float *xs = ys + kMaxBatch * kUfRowsPerBlock;  // K (batch 1) or the matrix cores' partial tiles
  const int r0 = blockIdx.x * kUfRowsPerBlock, r1 = min(rows, r0 + kUfRowsPerBlock);
  // tile-major weights (batched models; a tied LM head stays the row-major embedding) are read
  // by the matrix-core GEMV at any batch
  const bool tiled = m.tiled && !(MODE == 2 && m.tied);
  if (s.batch == 1 && !tiled) {
    stage_plain(x, K, K, 1, xs, kUfWaves);
    gemv_rows<WT>(W, scale, K, r0, r1, xs, ys, 1, kUfWaves, m.gs);
  } else {
    gemv_mfma<WT>(m, s, W, tiled, scale, K, r0, r1, BatchInput{x, K, nullptr, nullptr, false}, ys, red, xs);
  }
  __syncthreads();
  const int n = r1 - r0;
  if (MODE == 0) {
    for (int b = 0; b < s.batch; ++b)
      for (int i = threadIdx.x; i < n; i += kUfWaves * 64) y[(int64_t)b * rows + r0 + i] = ys[b * n + i];
  } else if (MODE == 1) {
    for (int b = 0; b < s.batch; ++b)
      for (int i = threadIdx.x; i < n; i += kUfWaves * 64)
        out[(int64_t)b * m.d + r0 + i] = res[(int64_t)b * m.d + r0 + i] + ys[b * n + i];
  } else {
    epi_logits(m, s, r0, r1, blockIdx.x, ys, red, kUfWaves);
  }
}

#define AMK_UF_GEMV(WT, MODE)                                                                 \
  extern "C" __global__ void __launch_bounds__(kUfWaves * 64)                                \
      amk_uf_gemv_w##WT##_m##MODE(const DevModel *__restrict__ mp, StepArgs s, const void *W, \
                                  const float *scale, int K, int rows, const float *x, float *y, \
                                  const float *res, float *out) {                            \
    uf_gemv<WT, MODE>(*mp, s, W, scale, K, rows, x, y, res, out);                            \
  }
AMK_UF_GEMV(0, 0)
AMK_UF_GEMV(0, 1)
AMK_UF_GEMV(0, 2)
AMK_UF_GEMV(1, 0)
AMK_UF_GEMV(1, 1)
AMK_UF_GEMV(1, 2)
AMK_UF_GEMV(2, 0)
AMK_UF_GEMV(2, 1)
AMK_UF_GEMV(2, 2)

// RoPE + KV append from the raw packed QKV outputs y[b][qkvr]; one thread per row pair
extern "C" __global__ void __launch_bounds__(256) amk_uf_rope_kv(const DevModel *__restrict__ mp,
                                                                 StepArgs s, int l) {
  const DevModel &m = *mp;
  const StepArgs sp = with_positions(s);
  const int b = blockIdx.y;
  const int pi = blockIdx.x * 256 + threadIdx.x;
  if (pi >= m.qkvr / 2) return;
  const int hd = m.hd, r = 2 * pi;
  const float *y = m.y + (int64_t)b * m.qkvr;
  const QkvRow q0 = qkv_decode(r, m.nq, m.nkv, hd);
  const QkvRow q1 = qkv_decode(r + 1, m.nq, m.nkv, hd);
  float v0 = y[r], v1 = y[r + 1];
  if (q0.kind != KIND_V) {
    const float2 c = m.rope[(int64_t)pos_of(sp, b) * (hd / 2) + q0.dim];
    const float a = v0, bb = v1;
    v0 = a * c.x - bb * c.y;
    v1 = bb * c.x + a * c.y;
  }
  if (q0.kind == KIND_Q) {
    float *qb = m.q + ((int64_t)l * m.max_batch + b) * m.qd;
    qb[q0.head * hd + q0.dim] = v0;
    qb[q1.head * hd + q1.dim] = v1;
  } else {
    const int kvi = (q0.kind == KIND_K) ? 0 : 1;
    s.kv[kv_index(m, s, l, kvi, b, q0.head, pos_of(sp, b), q0.dim)] = f32_to_bf16(v0);
    s.kv[kv_index(m, s, l, kvi, b, q1.head, pos_of(sp, b), q1.dim)] = f32_to_bf16(v1);
  }
}

template <int HD, int QMAX>
__device__ void uf_attn(const DevModel &m, const StepArgs &s, int l) {
  extern __shared__ __attribute__((aligned(16))) float lds[];  // 16-byte reads of xs need it
  float *red = lds;
  float *work = lds + 64 * 8;
  attn_task<HD, QMAX, false>(m, with_positions(s), l, blockIdx.x, blockIdx.y, work, red, nullptr,
                             nullptr);
}

#define AMK_UF_ATTN(HD, Q)                                                                   \
  extern "C" __global__ void __launch_bounds__(kThreads, 1)                                  \
      amk_uf_attn_h##HD##_q##Q(const DevModel *__restrict__ mp, StepArgs s, int l) {         \
    uf_attn<HD, Q>(*mp, s, l);                                                               \
  }
AMK_UF_ATTN(64, 1)
AMK_UF_ATTN(64, 2)
AMK_UF_ATTN(64, 4)
AMK_UF_ATTN(128, 1)
AMK_UF_ATTN(128, 2)
AMK_UF_ATTN(128, 4)

// o[b][h*hd + j] from the KV-block partials of layer l; one workgroup per (head, sequence)
extern "C" __global__ void __launch_bounds__(128) amk_uf_combine(const DevModel *__restrict__ mp,
                                                                 int l) {
  const DevModel &m = *mp;
  const int h = blockIdx.x, b = blockIdx.y, hd = m.hd, nblk = m.nblk;
  const float *ph = m.part + ((((int64_t)l * m.max_batch + b) * m.nq + h) * nblk) * (hd + 2);
  for (int j = threadIdx.x; j < hd; j += blockDim.x) {
    float M = -INFINITY;
    for (int k = 0; k < nblk; ++k) M = fmaxf(M, ph[k * (hd + 2) + hd]);
    float num = 0.f, den = 0.f;
    for (int k = 0; k < nblk; ++k) {
      const float *p = ph + k * (hd + 2);
      const float w = __expf(p[hd] - M);
      num = fmaf(w, p[j], num);
      den = fmaf(w, p[hd + 1], den);
    }
    m.o[(int64_t)b * m.qd + h * hd + j] = num / den;
  }
}

// a[l][b][i] = silu(gate_i) * up_i from the packed (interleaved) gate/up outputs y[b][2F]
extern "C" __global__ void __launch_bounds__(256) amk_uf_swiglu(const DevModel *__restrict__ mp,
                                                                int l, int batch) {
  const DevModel &m = *mp;
  const int64_t n = (int64_t)batch * m.F;
  for (int64_t k = blockIdx.x * 256 + threadIdx.x; k < n; k += (int64_t)gridDim.x * 256) {
    const int64_t b = k / m.F, i = k - b * m.F;
    const float *y = m.y + b * 2 * m.F;
    m.a[((int64_t)l * m.max_batch + b) * m.F + i] = silu(y[2 * i]) * y[2 * i + 1];
  }
}

extern "C" __global__ void __launch_bounds__(64) amk_uf_argmax(const DevModel *__restrict__ mp,
                                                               StepArgs s, int n_slots) {
  argmax_combine(*mp, s, n_slots);
}
