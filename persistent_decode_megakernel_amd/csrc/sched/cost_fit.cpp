// The cost model against task traces of one model's steps: the simulation's timeline in the trace
// format (amk_schedule_predict_trace), and the fit of the model's fixed costs to measured traces
// (amk_cost_model_fit).
//
// The pages profile the model that is to be served, offline, and freeze the schedule that the
// measurements favour (Ada-MK technical summary, "Methodology", Phase I). The microbenchmarks of
// amk_calibrate give the rates; what a real task adds beyond its bytes and its hop (the epilogue
// of a GEMV tile, the softmax and reductions of an attention block, the wait for the slowest of
// many producers) depends on the model's shapes, so it is read off a traced step of that model:
//   hop     : median over GEMV tiles that waited of  staged - act / l2_gbs - (producers' median end)
//   task_us : median over GEMV tiles of  end - [max(start + pre / rate, staged) + (hbm - pre) / rate]
//   attn_us : median over attention blocks of  partial_end - [max(start + pre / rate,
//             max(start, producers' median end + hop) + act / l2_gbs) + (hbm - pre) / rate]
// with the byte counts and prefetch rules of the simulation itself. hop_us is then set so that the
// simulated step of the traced schedule lasts as long as the measured one; the model so fitted
// predicts the schedule search's other candidates for the same model.
#include <algorithm>
#include <cmath>
#include <cstdio>
#include <cstring>
#include <string>
#include <vector>

#include "../runtime/errors.h"
#include "sched_internal.h"

namespace amk {
namespace {

constexpr double kTickUs = 0.01;  // trace stamps: 100 MHz wall clock

double median(std::vector<double> v) {
  if (v.empty()) return NAN;
  const size_t k = v.size() / 2;
  std::nth_element(v.begin(), v.begin() + (long)k, v.end());
  double m = v[k];
  if (v.size() % 2 == 0) {
    std::nth_element(v.begin(), v.begin() + (long)k - 1, v.end());
    m = 0.5 * (m + v[k - 1]);
  }
  return m;
}

struct Stamp {
  double start, mid, end;
  bool ok;
};

// one trace's stamps in us from its earliest task start; tasks whose stamps are out of order are
// marked unusable (a task that did not run leaves stale words)
std::vector<Stamp> read_trace(const Schedule &s, const uint64_t *tr, double *span) {
  const uint32_t n = s.hdr.n_tasks;
  uint64_t t0 = UINT64_MAX, t1 = 0;
  for (uint32_t i = 0; i < n; ++i) {
    t0 = std::min(t0, tr[4 * (size_t)i]);
    t1 = std::max(t1, tr[4 * (size_t)i + 3]);
  }
  std::vector<Stamp> v(n);
  for (uint32_t i = 0; i < n; ++i) {
    const uint64_t a = tr[4 * (size_t)i], m = tr[4 * (size_t)i + 2], e = tr[4 * (size_t)i + 3];
    v[i].ok = a >= t0 && m >= a && e >= m;
    v[i].start = (double)(a - t0) * kTickUs;
    v[i].mid = (double)(m - t0) * kTickUs;
    v[i].end = (double)(e - t0) * kTickUs;
  }
  *span = t1 > t0 ? (double)(t1 - t0) * kTickUs : 0.0;
  return v;
}

}  // namespace
}  // namespace amk

using namespace amk;

extern "C" amk_status amk_schedule_predict_trace(const void *blob, size_t bytes,
                                                 const amk_cost_model *cost, int32_t ctx,
                                                 uint64_t *trace, size_t trace_words) {
  AMK_API_BEGIN
  if (!trace) return set_error(AMK_E_INVALID, "amk_schedule_predict_trace: null output");
  Schedule s;
  std::string e;
  if (!parse(blob, bytes, &s, &e)) return set_error(AMK_E_INVALID, e);
  if (ctx < 1) return set_error(AMK_E_INVALID, "amk_schedule_predict_trace: ctx must be >= 1");
  const size_t need = 4 * (size_t)s.hdr.n_tasks + s.per_cu.size();
  if (trace_words < need)
    return set_error(AMK_E_INVALID, "amk_schedule_predict_trace: trace holds fewer than "
                                    "4 * n_tasks + n_cu words");
  std::vector<TaskTimes> tt;
  const double span = predict_times(s, fill_cost(cost, (int32_t)s.hdr.n_cu), ctx, &tt);
  if (!std::isfinite(span)) return set_error(AMK_E_SCHEDULE_REJECTED, "amk_schedule_predict_trace: the schedule does not complete");
  auto tick = [](double us) { return (uint64_t)std::llround(us / kTickUs); };
  for (size_t i = 0; i < tt.size(); ++i) {
    trace[4 * i + 0] = tick(tt[i].start);
    trace[4 * i + 1] = tick(tt[i].start);
    trace[4 * i + 2] = tick(tt[i].mid);
    trace[4 * i + 3] = tick(tt[i].end);
  }
  for (size_t c = 0; c < s.per_cu.size(); ++c) trace[4 * (size_t)s.hdr.n_tasks + c] = 0;
  clear_error();
  return AMK_OK;
  AMK_API_END
}

extern "C" amk_status amk_cost_model_fit(const void *blob, size_t bytes, const uint64_t *traces,
                                         int32_t n_traces, int32_t ctx, const amk_cost_model *base,
                                         amk_cost_model *out, char *report, size_t report_cap) {
  AMK_API_BEGIN
  if (!traces || !out || n_traces < 1)
    return set_error(AMK_E_INVALID, "amk_cost_model_fit: null argument or no traces");
  Schedule s;
  std::string e;
  if (!parse(blob, bytes, &s, &e)) return set_error(AMK_E_INVALID, e);
  if (!validate_schedule(s, &e)) return set_error(AMK_E_SCHEDULE_REJECTED, e);
  if (ctx < 1) return set_error(AMK_E_INVALID, "amk_cost_model_fit: ctx must be >= 1");
  amk_cost_model cm = fill_cost(base, (int32_t)s.hdr.n_cu);
  const uint32_t n = s.hdr.n_tasks;
  const size_t words = 4 * (size_t)n + s.per_cu.size();
  const double rate = cm.cu_stream_gbs * 1e3, l2 = cm.l2_gbs * 1e3, pf = cm.prefetch_kb * 1024.0;
  const double B = std::max<uint32_t>(1, s.hdr.batch);
  std::vector<const Task *> by_id(n, nullptr);
  for (auto &v : s.per_cu)
    for (auto &t : v) by_id[t.id] = &t;
  std::vector<std::vector<Stamp>> st((size_t)n_traces);
  std::vector<double> spans((size_t)n_traces);
  for (int32_t k = 0; k < n_traces; ++k) st[(size_t)k] = read_trace(s, traces + (size_t)k * words, &spans[(size_t)k]);
  // the median end of a task's first-range producers, or -1 if one is unusable. The simulation
  // finishes a phase's tiles together; measured from their median end, the hop also holds the
  // wait for the slowest of them.
  std::vector<double> ends;
  auto last_producer = [&](const std::vector<Stamp> &v, const Task &t) {
    ends.clear();
    for (uint32_t i = t.w0_lo; i < t.w0_hi && i < n; ++i) {
      if (!v[i].ok) return -1.0;
      ends.push_back(v[i].end);
    }
    return ends.empty() ? -INFINITY : median(ends);
  };
  std::vector<double> hops, gemv, attn;
  for (auto &v : st)
    for (uint32_t i = 0; i < n; ++i) {
      const Task &t = *by_id[i];
      if (!v[i].ok || t.type != T_GEMV || t.w0_hi <= t.w0_lo) continue;
      double hbm, act;
      task_bytes(s.hdr, t, ctx, &hbm, &act);
      const double d = last_producer(v, t);
      const double waited = v[i].mid - act / l2 - v[i].start;
      if (d >= 0 && waited > 0.25) hops.push_back(v[i].mid - act / l2 - d);
    }
  const double hop = hops.empty() ? cm.hop_us : std::max(0.0, median(hops));
  for (auto &v : st)
    for (uint32_t i = 0; i < n; ++i) {
      const Task &t = *by_id[i];
      if (!v[i].ok) continue;
      double hbm, act;
      task_bytes(s.hdr, t, ctx, &hbm, &act);
      if (t.type == T_GEMV) {
        const double pre = std::min(hbm, pf);
        gemv.push_back(v[i].end - (std::max(v[i].start + pre / rate, v[i].mid) + (hbm - pre) / rate));
      } else if (t.type == T_ATTN) {
        double d = last_producer(v, t);
        if (d < 0) continue;
        if (t.w0_hi <= t.w0_lo) d = v[i].start;
        const double pre = hbm / B;
        const double staged = std::max(v[i].start, d + hop) + act / l2;
        attn.push_back(v[i].mid - (std::max(v[i].start + pre / rate, staged) + (hbm - pre) / rate));
      }
    }
  if (!gemv.empty()) cm.task_us = std::max(0.0, median(gemv));
  if (!attn.empty()) cm.attn_us = std::max(0.0, median(attn));
  double meas = 0.0;
  for (double x : spans) meas += x;
  meas /= (double)n_traces;
  // The hop then takes the value at which the simulated step of the traced schedule lasts as
  // long as the measured one (the makespan grows with the hop; bisection over [0, 64] us): the
  // in-situ median misses how the slowest of many producers stretches a phase.
  double lo = 0.0, hi = 64.0;
  cm.hop_us = lo;
  const double p_lo = predict_makespan(s, cm, ctx);
  cm.hop_us = hi;
  const double p_hi = predict_makespan(s, cm, ctx);
  if (meas <= p_lo) {
    hi = lo;
  } else if (meas >= p_hi) {
    lo = hi;
  } else {
    for (int it = 0; it < 50; ++it) {
      cm.hop_us = 0.5 * (lo + hi);
      (predict_makespan(s, cm, ctx) < meas ? lo : hi) = cm.hop_us;
    }
  }
  cm.hop_us = 0.5 * (lo + hi);
  const double pred = predict_makespan(s, cm, ctx);
  *out = cm;
  if (report && report_cap) {
    char buf[512];
    std::snprintf(buf, sizeof buf,
                  "{\"n_cu\": %u, \"samples\": {\"hop\": %zu, \"gemv\": %zu, \"attn\": %zu}, "
                  "\"hop_in_situ_us\": %.3f, \"measured_us\": %.2f, \"predicted_us\": %.2f, "
                  "\"fit\": {\"cu_stream_gbs\": %.3f, "
                  "\"hop_us\": %.3f, \"task_us\": %.3f, \"l2_gbs\": %.3f, \"prefetch_kb\": %.1f, "
                  "\"attn_us\": %.3f}}",
                  (unsigned)s.per_cu.size(), hops.size(), gemv.size(), attn.size(), hop, meas, pred,
                  cm.cu_stream_gbs, cm.hop_us, cm.task_us, cm.l2_gbs, cm.prefetch_kb, cm.attn_us);
    std::strncpy(report, buf, report_cap - 1);
    report[report_cap - 1] = 0;
  }
  clear_error();
  return AMK_OK;
  AMK_API_END
}
