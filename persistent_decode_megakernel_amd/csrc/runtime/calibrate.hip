// Measured cost model of the schedule search: microbenchmarks on the device, and the fit of
// amk_cost_model from them (amk_calibrate).
//
// The pages solidify the execution path by profiling candidate schedules offline (Ada-MK
// technical summary, "Methodology", Phase I; "Key Contributions" item 2). The search here ranks
// candidates with a cost model of four rates and latencies; these kernels measure them with the
// megakernel's own device code paths:
//   * stream: n_active workgroups (one per CU) each stream a private slice with the batch-1 GEMV
//     body (GemvStream: per-wave 8 KB chunks of nontemporal 16-byte loads, two in flight); the
//     per-CU rate as a function of how many CUs stream at once;
//   * relay: a ring of workgroups hands a vector of K fp32 words from one to the next with the
//     batch-1 protocol (epoch-tagged words; the consumer's staging loads are its wait) or with the
//     batched one (a device-scope flag published after the data's stores complete, polled by one
//     wave; then the data staged with device-coherent loads). Each hop is one dependency of the
//     frozen schedule: wait, stage the input, write the output. The ring's workgroups sit on one
//     XCD or on different XCDs (workgroup w of a launch runs on XCD w mod 8), and the other CUs
//     either idle or stream memory meanwhile (the loaded case is the one inside a decode step).
//   * phase: every workgroup of the launch at once stages a K-word vector that all of them wrote a
//     share of in the previous phase (batch-1 protocol), then writes its share of the next one:
//     the all-to-all dependency of consecutive phases of a decode step, where each task waits for
//     the last of the many tiles that produced its input.
// The cost model's hop is the phase: hop_us + K * 4 bytes / l2_gbs, fitted over three vector
// lengths. The relays (one producer per consumer) are reported beside it: the difference is the
// wait for the slowest of many producers.
#include <hip/hip_runtime.h>

#include <algorithm>
#include <cmath>
#include <cstdio>
#include <cstring>
#include <string>
#include <vector>

#include "../kernels/device.h"
#include "../sched/sched_internal.h"
#include "errors.h"

namespace amk {

constexpr int kCalibK = 4096;        // inputs per streamed row (one 8 KB bf16 row per chunk)
constexpr int kCalibLds = 96 * 1024; // dynamic LDS: keeps one workgroup per CU
constexpr uint32_t kCalibMaxPasses = 64;

// Stream rows [row0, row0 + rows) of a bf16 [.., kCalibK] region with the batch-1 GEMV body.
__device__ __forceinline__ void calib_stream_rows(const uint8_t *buf, int64_t row0, int rows,
                                                  float *xs, float *ys) {
  GemvStream<0> st;
  st.init(buf + row0 * kCalibK * 2, kCalibK, 0, rows, kWaves);
  uint4 P[kChunkUnits];
  if (st.S > 0) st.load(P, 0);
  st.run(P, xs, ys, nullptr);
}

// Per-CU stream rate: workgroups w < n_active each stream rows_per_wg rows of their own slice;
// thread 0 stamps the start and end (after a workgroup barrier) into stamps[2w], [2w + 1].
extern "C" __global__ void __launch_bounds__(kThreads, 1)
amk_calib_stream(const uint8_t *buf, int rows_per_wg, int n_active, uint64_t *stamps) {
  extern __shared__ __attribute__((aligned(16))) float lds[];
  const int w = blockIdx.x;
  if (w >= n_active) return;
  float *xs = lds, *ys = lds + kCalibK;
  for (int i = threadIdx.x; i < kCalibK; i += kThreads) xs[i] = 0.f;
  __syncthreads();
  if (threadIdx.x == 0) gst(&stamps[2 * w], (uint64_t)wall_clock64());
  calib_stream_rows(buf, (int64_t)w * rows_per_wg, rows_per_wg, xs, ys);
  __syncthreads();
  if (threadIdx.x == 0) gst(&stamps[2 * w + 1], (uint64_t)wall_clock64());
}

struct RelayArgs {
  uint32_t *slots;      // hops + 1 vectors of K words (tagged) or K floats (flag protocol)
  uint32_t *flags;      // flag protocol: one word per hop (= dm.flags)
  uint32_t *stop;       // raised by the ring when it is done: the streaming workgroups stop
  int32_t ring[8];      // workgroup ids of the ring, in hop order
  int32_t n_ring;
  int32_t hops;
  int32_t K;
  int32_t use_flags;
  int32_t load;         // 1: workgroups outside the ring stream memory until the ring is done
  const uint8_t *buf;   // streamed by the others
  int32_t rows_per_pass;
  uint64_t *stamps;     // [0] first hop start, [1] last hop end
  uint32_t *progress;   // hops completed (diagnostics when a relay stops)
};

// A ring of workgroups relays a K-word vector: hop i is run by ring[i % n_ring], which waits for
// hop i - 1's vector (slot i), stages it, and writes slot i + 1. Every slot is written once and
// read once (epoch 1; the host fills slot 0 with words of that epoch and leaves the others zero),
// so no reader meets a location again whose two-bit tag could repeat. Every wait is bounded by
// the model's watchdog (dm.timeout_ticks); a timeout raises the abort word, which ends every
// other wait.
extern "C" __global__ void __launch_bounds__(kThreads, 1)
amk_calib_relay(const DevModel *__restrict__ mp, RelayArgs a) {
  extern __shared__ __attribute__((aligned(16))) float lds[];
  const DevModel &m = *mp;
  __shared__ int abort_flag;
  float *xs = lds, *red = lds + 11264;
  const int w = blockIdx.x;
  int me = -1;
  for (int r = 0; r < a.n_ring; ++r)
    if (a.ring[r] == w) me = r;
  if (me < 0) {
    if (!a.load) return;
    float *ys = lds + kCalibK;
    for (int i = threadIdx.x; i < kCalibK; i += kThreads) xs[i] = 0.f;
    __syncthreads();
    // stream this workgroup's slice again and again until the ring is done (bounded)
    for (uint32_t pass = 0; pass < kCalibMaxPasses; ++pass) {
      calib_stream_rows(a.buf, (int64_t)w * a.rows_per_pass, a.rows_per_pass, xs, ys);
      __syncthreads();
      if (flag_load(a.stop) != 0 || flag_load(&m.err[1]) != 0) break;
    }
    return;
  }
  if (threadIdx.x == 0) abort_flag = 0;
  __syncthreads();
  const int K = a.K;
  for (int i = me; i < a.hops; i += a.n_ring) {
    const uint32_t *src = a.slots + (size_t)i * K;
    uint32_t *dst = a.slots + (size_t)(i + 1) * K;
    if (i == 0 && threadIdx.x == 0) gst(&a.stamps[0], (uint64_t)wall_clock64());
    if (a.use_flags) {
      // batched protocol: wave 0 polls the previous hop's flag, then the data is staged
      Task t{};
      t.id = (uint32_t)i;
      if (i > 0) {
        t.w0_lo = (uint32_t)(i - 1);
        t.w0_hi = t.w0_lo + 1;
      }
      if (!wait_task(m, t, 1u, &abort_flag)) return;  // m.flags is a.flags
      stage_plain(reinterpret_cast<const float *>(src), 0, K, 1, xs, kWaves);
      for (int k = threadIdx.x; k < K; k += kThreads) cstf(reinterpret_cast<float *>(dst) + k, xs[k] + 1.f);
      __builtin_amdgcn_s_waitcnt(0);
      __syncthreads();
      if (threadIdx.x == 0)
        __hip_atomic_store(gptr(&a.flags[i]), 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    } else {
      // batch-1 protocol: the staging loads are the wait
      if (!stage_tagged<false>(m, src, K, nullptr, 1u, xs, red, (uint32_t)i)) return;
      for (int k = threadIdx.x; k < K; k += kThreads) cst(&dst[k], tag_word(xs[k] + 1.f, 1u));
      __syncthreads();
    }
    if (threadIdx.x == 0) __hip_atomic_fetch_add(gptr(a.progress), 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    if (i == a.hops - 1 && threadIdx.x == 0) {
      __builtin_amdgcn_s_waitcnt(0);
      gst(&a.stamps[1], (uint64_t)wall_clock64());
      __hip_atomic_store(gptr(a.stop), 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    }
  }
}

struct PhaseArgs {
  uint32_t *slots;      // (phases + 1) vectors of K tagged words; slot 0 holds epoch-1 words
  int32_t phases;
  int32_t K;
  uint64_t *stamps;     // [0] workgroup 0's start, [1] workgroup 0 has staged the last vector
  uint32_t *progress;   // phases workgroup 0 completed (diagnostics when a run stops)
};

// Phase i: every workgroup stages slot i (its staging loads wait until every word carries epoch
// 1), then writes its share of slot i + 1. Each slot is written once, so no reader meets a word
// whose two-bit tag could repeat; every wait is bounded by the watchdog, whose timeout raises the
// abort word and so ends every other wait.
extern "C" __global__ void __launch_bounds__(kThreads, 1)
amk_calib_phase(const DevModel *__restrict__ mp, PhaseArgs a) {
  extern __shared__ __attribute__((aligned(16))) float lds[];
  const DevModel &m = *mp;
  float *xs = lds, *red = lds + 11264;
  const int n = gridDim.x, w = blockIdx.x, K = a.K;
  const int per = (K + n - 1) / n, lo = min(K, w * per), hi = min(K, lo + per);
  if (w == 0 && threadIdx.x == 0) gst(&a.stamps[0], (uint64_t)wall_clock64());
  for (int i = 0; i < a.phases; ++i) {
    if (!stage_tagged<false>(m, a.slots + (size_t)i * K, K, nullptr, 1u, xs, red, (uint32_t)i)) return;
    uint32_t *dst = a.slots + (size_t)(i + 1) * K;
    for (int k = lo + (int)threadIdx.x; k < hi; k += kThreads) cst(&dst[k], tag_word(xs[k] + 1.f, 1u));
    __syncthreads();
    if (w == 0 && threadIdx.x == 0)
      __hip_atomic_fetch_add(gptr(a.progress), 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  }
  if (w == 0) {
    if (!stage_tagged<false>(m, a.slots + (size_t)a.phases * K, K, nullptr, 1u, xs, red, (uint32_t)a.phases))
      return;
    if (threadIdx.x == 0) gst(&a.stamps[1], (uint64_t)wall_clock64());
  }
}

namespace {

struct HipErr : std::runtime_error {
  explicit HipErr(const std::string &m) : std::runtime_error(m) {}
};
void ck(hipError_t e, const char *what) {
  if (e != hipSuccess) throw HipErr(std::string(what) + ": " + hipGetErrorString(e));
}

struct DevBuf {
  void *p = nullptr;
  explicit DevBuf(size_t n) { ck(hipMalloc(&p, n), "hipMalloc"); }
  ~DevBuf() {
    if (p) (void)hipFree(p);
  }
  DevBuf(const DevBuf &) = delete;
  DevBuf &operator=(const DevBuf &) = delete;
};

// least-squares line y = a + b x
void fit_line(const std::vector<double> &x, const std::vector<double> &y, double *a, double *b) {
  const double n = (double)x.size();
  double sx = 0, sy = 0, sxx = 0, sxy = 0;
  for (size_t i = 0; i < x.size(); ++i) {
    sx += x[i];
    sy += y[i];
    sxx += x[i] * x[i];
    sxy += x[i] * y[i];
  }
  const double d = n * sxx - sx * sx;
  *b = d != 0 ? (n * sxy - sx * sy) / d : 0.0;
  *a = (sy - *b * sx) / n;
}

}  // namespace
}  // namespace amk

using namespace amk;

extern "C" amk_status amk_calibrate(amk_cost_model *out, char *report, size_t report_cap,
                                    void *stream) {
  AMK_API_BEGIN
  if (!out) return set_error(AMK_E_INVALID, "amk_calibrate: null output");
  hipStream_t st = static_cast<hipStream_t>(stream);
  try {
    int dev = 0;
    ck(hipGetDevice(&dev), "hipGetDevice");
    hipDeviceProp_t prop;
    ck(hipGetDeviceProperties(&prop, dev), "hipGetDeviceProperties");
    const int n_cu = prop.multiProcessorCount;
    int clock_khz = 100000;
    if (hipDeviceGetAttribute(&clock_khz, hipDeviceAttributeWallClockRate, dev) != hipSuccess ||
        clock_khz <= 0)
      clock_khz = 100000;
    const double us_per_tick = 1000.0 / clock_khz;
    ck(hipFuncSetAttribute((const void *)amk_calib_stream, hipFuncAttributeMaxDynamicSharedMemorySize,
                           kCalibLds), "hipFuncSetAttribute");
    ck(hipFuncSetAttribute((const void *)amk_calib_relay, hipFuncAttributeMaxDynamicSharedMemorySize,
                           kCalibLds), "hipFuncSetAttribute");
    ck(hipFuncSetAttribute((const void *)amk_calib_phase, hipFuncAttributeMaxDynamicSharedMemorySize,
                           kCalibLds), "hipFuncSetAttribute");
    // 2 GiB streamed per pass at most: far beyond every cache, 8 MiB per workgroup
    const int rows_per_wg = 1024;  // 8 MiB of bf16 rows
    const size_t buf_bytes = (size_t)n_cu * rows_per_wg * kCalibK * 2;
    DevBuf buf(buf_bytes);
    ck(hipMemsetAsync(buf.p, 0, buf_bytes, st), "hipMemsetAsync");
    DevBuf stamps(sizeof(uint64_t) * 2 * (size_t)n_cu);
    std::vector<uint64_t> hs(2 * (size_t)n_cu);
    std::string js = "{\"n_cu\": " + std::to_string(n_cu) + ", \"stream\": [";

    // ---- stream rate vs active CUs -------------------------------------------------------
    std::vector<int> actives;
    for (int a = 8; a < n_cu; a *= 2) actives.push_back(a);
    actives.push_back(n_cu);
    double full_rate = 0.0;
    for (size_t ai = 0; ai < actives.size(); ++ai) {
      const int na = actives[ai];
      double best = 0.0;
      for (int rep = 0; rep < 3; ++rep) {  // the first run of a size warms up; keep the best
        hipLaunchKernelGGL(amk_calib_stream, dim3(n_cu), dim3(kThreads), kCalibLds, st,
                           (const uint8_t *)buf.p, rows_per_wg, na, (uint64_t *)stamps.p);
        ck(hipGetLastError(), "amk_calib_stream");
        ck(hipMemcpyAsync(hs.data(), stamps.p, hs.size() * 8, hipMemcpyDeviceToHost, st), "hipMemcpyAsync");
        ck(hipStreamSynchronize(st), "hipStreamSynchronize");
        uint64_t t0 = ~0ull, t1 = 0;
        for (int w = 0; w < na; ++w) {
          t0 = std::min(t0, hs[2 * w]);
          t1 = std::max(t1, hs[2 * w + 1]);
        }
        const double us = (double)(t1 - t0) * us_per_tick;
        const double gbs = (double)na * rows_per_wg * kCalibK * 2 / (us * 1e3);
        best = std::max(best, gbs);
      }
      if (na == n_cu) full_rate = best;
      char tmp[128];
      std::snprintf(tmp, sizeof tmp, "%s{\"active_cus\": %d, \"gbs\": %.1f, \"per_cu_gbs\": %.2f}",
                    ai ? ", " : "", na, best, best / na);
      js += tmp;
    }
    js += "], \"relay\": [";

    // ---- hand-off relays ----------------------------------------------------------------
    const int kmax = 11264, kHops = 400;
    DevBuf slots(sizeof(uint32_t) * (size_t)kmax * (kHops + 1));
    DevBuf flags(sizeof(uint32_t) * kHops);
    DevBuf err(16);
    DevBuf stop(256);
    DevBuf progress(256);
    DevModel dm{};
    dm.err = (uint32_t *)err.p;
    dm.flags = (uint32_t *)flags.p;
    dm.timeout_ticks = (uint64_t)(2000.0 * clock_khz);  // 2 s
    DevBuf d_dm(sizeof(DevModel));
    ck(hipMemcpyAsync(d_dm.p, &dm, sizeof dm, hipMemcpyHostToDevice, st), "hipMemcpyAsync");
    const int Ks[3] = {1024, 4096, 11008};
    double fit_hop = 0.0, fit_l2 = 0.0, flag_hop = 0.0;
    bool first = true;
    for (int use_flags = 0; use_flags < 2; ++use_flags)
      for (int cross = 0; cross < 2; ++cross)
        for (int load = 0; load < 2; ++load) {
          std::vector<double> xk, yus;
          for (int K : Ks) {
            if (use_flags && K != 4096) continue;
            RelayArgs a{};
            a.slots = (uint32_t *)slots.p;
            a.flags = (uint32_t *)flags.p;
            a.stop = (uint32_t *)stop.p;
            a.n_ring = 4;
            for (int r = 0; r < 4; ++r) a.ring[r] = cross ? r : 8 * r;  // XCDs 0..3, or XCD 0
            a.hops = kHops;
            a.K = K;
            a.use_flags = use_flags;
            a.load = load;
            a.buf = (const uint8_t *)buf.p;
            a.rows_per_pass = 256;  // 2 MiB per pass per streaming workgroup
            a.stamps = (uint64_t *)stamps.p;
            a.progress = (uint32_t *)progress.p;
            ck(hipMemsetAsync(slots.p, 0, sizeof(uint32_t) * (size_t)kmax * (kHops + 1), st), "hipMemsetAsync");
            ck(hipMemsetD32Async((hipDeviceptr_t)slots.p, 1, (size_t)K, st), "hipMemsetD32Async");  // slot 0: epoch 1
            ck(hipMemsetAsync(flags.p, 0, sizeof(uint32_t) * kHops, st), "hipMemsetAsync");
            ck(hipMemsetAsync(err.p, 0, 16, st), "hipMemsetAsync");
            ck(hipMemsetAsync(stop.p, 0, 256, st), "hipMemsetAsync");
            ck(hipMemsetAsync(progress.p, 0, 256, st), "hipMemsetAsync");
            const DevModel *g = (const DevModel *)d_dm.p;
            void *args[] = {(void *)&g, (void *)&a};
            ck(hipLaunchCooperativeKernel((const void *)amk_calib_relay, dim3(n_cu), dim3(kThreads),
                                          args, kCalibLds, st), "amk_calib_relay");
            uint32_t herr[4] = {0, 0, 0, 0}, done = 0;
            ck(hipMemcpyAsync(hs.data(), stamps.p, 16, hipMemcpyDeviceToHost, st), "hipMemcpyAsync");
            ck(hipMemcpyAsync(herr, err.p, 16, hipMemcpyDeviceToHost, st), "hipMemcpyAsync");
            ck(hipMemcpyAsync(&done, progress.p, 4, hipMemcpyDeviceToHost, st), "hipMemcpyAsync");
            ck(hipStreamSynchronize(st), "hipStreamSynchronize");
            if (herr[0]) {
              char msg[256];
              std::snprintf(msg, sizeof msg,
                            "relay (%s, %s XCD, others %s, K %d) stopped after %u of %d hops: "
                            "device error %u at hop %u (detail 0x%x)",
                            use_flags ? "flag" : "tagged", cross ? "cross" : "same",
                            load ? "streaming" : "idle", K, done, a.hops, herr[0], herr[2], herr[3]);
              throw std::runtime_error(msg);
            }
            const double us = (double)(hs[1] - hs[0]) * us_per_tick / a.hops;
            xk.push_back(4.0 * K);
            yus.push_back(us);
            char tmp[200];
            std::snprintf(tmp, sizeof tmp,
                          "%s{\"protocol\": \"%s\", \"xcd\": \"%s\", \"others\": \"%s\", \"K\": %d, "
                          "\"us_per_hop\": %.3f}",
                          first ? "" : ", ", use_flags ? "flag" : "tagged", cross ? "cross" : "same",
                          load ? "streaming" : "idle", K, us);
            js += tmp;
            first = false;
          }
          if (cross && load) {
            if (!use_flags) {
              double a0, b0;
              fit_line(xk, yus, &a0, &b0);
              fit_hop = a0;
              fit_l2 = b0 > 0 ? 1.0 / (b0 * 1e3) : 0.0;  // bytes per us -> GB/s
            } else {
              flag_hop = yus[0];
            }
          }
        }
    js += "], \"phase\": [";

    // ---- all-to-all phases ---------------------------------------------------------------
    const int kPhases = 128;
    double phase_hop = 0.0, phase_l2 = 0.0;
    {
      std::vector<double> xk, yus;
      for (int ki = 0; ki < 3; ++ki) {
        const int K = Ks[ki];
        double best = 1e30;
        for (int rep = 0; rep < 2; ++rep) {
          PhaseArgs a{};
          a.slots = (uint32_t *)slots.p;
          a.phases = kPhases;
          a.K = K;
          a.stamps = (uint64_t *)stamps.p;
          a.progress = (uint32_t *)progress.p;
          const size_t words = (size_t)K * (kPhases + 1);
          ck(hipMemsetAsync(slots.p, 0, sizeof(uint32_t) * words, st), "hipMemsetAsync");
          ck(hipMemsetD32Async((hipDeviceptr_t)slots.p, 1, (size_t)K, st), "hipMemsetD32Async");
          ck(hipMemsetAsync(err.p, 0, 16, st), "hipMemsetAsync");
          ck(hipMemsetAsync(progress.p, 0, 256, st), "hipMemsetAsync");
          const DevModel *g = (const DevModel *)d_dm.p;
          void *args[] = {(void *)&g, (void *)&a};
          ck(hipLaunchCooperativeKernel((const void *)amk_calib_phase, dim3(n_cu), dim3(kThreads),
                                        args, kCalibLds, st), "amk_calib_phase");
          uint32_t herr[4] = {0, 0, 0, 0}, done = 0;
          ck(hipMemcpyAsync(hs.data(), stamps.p, 16, hipMemcpyDeviceToHost, st), "hipMemcpyAsync");
          ck(hipMemcpyAsync(herr, err.p, 16, hipMemcpyDeviceToHost, st), "hipMemcpyAsync");
          ck(hipMemcpyAsync(&done, progress.p, 4, hipMemcpyDeviceToHost, st), "hipMemcpyAsync");
          ck(hipStreamSynchronize(st), "hipStreamSynchronize");
          if (herr[0]) {
            char msg[200];
            std::snprintf(msg, sizeof msg,
                          "phases (K %d) stopped after %u of %d: device error %u at phase %u (detail 0x%x)",
                          K, done, kPhases, herr[0], herr[2], herr[3]);
            throw std::runtime_error(msg);
          }
          best = std::min(best, (double)(hs[1] - hs[0]) * us_per_tick / kPhases);
        }
        xk.push_back(4.0 * K);
        yus.push_back(best);
        char tmp[120];
        std::snprintf(tmp, sizeof tmp, "%s{\"K\": %d, \"us_per_phase\": %.3f}", ki ? ", " : "", K, best);
        js += tmp;
      }
      double a0, b0;
      fit_line(xk, yus, &a0, &b0);
      phase_hop = a0;
      phase_l2 = b0 > 0 ? 1.0 / (b0 * 1e3) : 0.0;
    }
    amk_cost_model cm{};
    cm.cu_stream_gbs = full_rate / n_cu;
    cm.hop_us = std::max(0.0, phase_hop);
    cm.l2_gbs = phase_l2 > 0 ? phase_l2 : 100.0;
    cm.task_us = 0.0;  // a phase's fixed time already holds the task's wait, barrier and epilogue
    cm.attn_us = 0.0;
    cm.prefetch_kb = builtin_cost_model().prefetch_kb;
    char tmp[400];
    std::snprintf(tmp, sizeof tmp,
                  "], \"fit\": {\"cu_stream_gbs\": %.3f, \"hop_us\": %.3f, \"l2_gbs\": %.2f, "
                  "\"task_us\": %.3f, \"relay_hop_us\": %.3f, \"relay_l2_gbs\": %.2f, "
                  "\"flag_hop_us_k4096\": %.3f}}",
                  cm.cu_stream_gbs, cm.hop_us, cm.l2_gbs, cm.task_us, fit_hop, fit_l2, flag_hop);
    js += tmp;
    *out = cm;
    if (report && report_cap) {
      std::strncpy(report, js.c_str(), report_cap - 1);
      report[report_cap - 1] = 0;
    }
  } catch (const HipErr &ex) {
    return set_error(AMK_E_HIP, std::string("amk_calibrate: ") + ex.what());
  } catch (const std::runtime_error &ex) {
    return set_error(AMK_E_DEVICE_TIMEOUT, std::string("amk_calibrate: ") + ex.what());
  }
  clear_error();
  return AMK_OK;
  AMK_API_END
}
