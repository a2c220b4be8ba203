// Profile-guided re-tiling of a frozen schedule.
//
// The pages' method fixes the execution path offline: a search that profiles candidates on the
// device and solidifies the best one, so that nothing is decided at run time (Ada-MK summary,
// "Fine-Grained DAG-Based Automatic Search"; AutoMegaKernel abstract, frozen schedule IR). Here
// the measured quantity is how long each GEMV tile of a phase takes on the CU it is placed on,
// and the free parameters are the row boundaries between the tiles of a phase. Every phase of
// the decode graph is all-to-all (a tile of the next phase needs the whole output vector), so a
// phase ends with its slowest tile; the rows are moved until the tiles of each phase would finish
// together given when each one could start. Task ids, placement and the phase-range waits stay
// as they are; the attention waits, which name the QKV tiles covering a KV group's rows, follow
// the new QKV boundaries.
#include <algorithm>
#include <cmath>
#include <cstdlib>
#include <cstring>
#include <map>
#include <string>
#include <utility>
#include <vector>

#include "../runtime/errors.h"
#include "sched_internal.h"

namespace amk {

namespace {

constexpr double kTickUs = 0.01;  // task-trace stamps count a 100 MHz clock

// Row boundaries (multiples of align except the last, which is `rows`; every tile holds at least
// one align unit) closest to the real-valued target sizes w[i] scaled to `rows` in total.
std::vector<uint32_t> boundaries(const std::vector<double> &w, uint32_t rows, uint32_t align) {
  const size_t n = w.size();
  const int64_t units = ((int64_t)rows + align - 1) / align;
  double tot = 0;
  for (double x : w) tot += x;
  std::vector<uint32_t> b(n + 1, 0);
  b[n] = rows;
  double cum = 0;
  int64_t prev = 0;  // previous boundary in align units
  for (size_t i = 1; i < n; ++i) {
    cum += w[i - 1];
    const double want = (double)rows * (cum / tot);
    int64_t u = (int64_t)std::llround(want / align);
    u = std::min(std::max(u, prev + 1), units - (int64_t)(n - i));
    b[i] = (uint32_t)(u * align);
    prev = u;
  }
  return b;
}

}  // namespace

bool rebalance_schedule(Schedule *s, const uint64_t *traces, int n_traces, double gain,
                        std::string *err) {
  const BlobHeader &h = s->hdr;
  const uint32_t n = h.n_tasks;
  const size_t stride = 4ull * n + h.n_cu;
  auto fail = [&](const std::string &m) {
    if (err) *err = m;
    return false;
  };
  if (n_traces < 1 || !traces) return fail("rebalance: no traces");
  if (!(gain > 0.0 && gain <= 1.0)) return fail("rebalance: gain must be in (0, 1]");
  std::vector<Task *> by_id(n, nullptr);
  for (auto &v : s->per_cu)
    for (Task &t : v) {
      if (t.id >= n) return fail("rebalance: task id out of range");
      by_id[t.id] = &t;
    }
  // GEMV phases (matrix, layer), tiles in row order
  std::map<std::pair<int, int>, std::vector<Task *>> phases;
  for (Task *t : by_id) {
    if (!t) return fail("rebalance: missing task id");
    if (t->type == T_GEMV) phases[{(int)t->mat, (int)t->layer}].push_back(t);
  }
  const uint32_t cap_rows = 4096u / std::max<uint32_t>(1, h.batch);
  uint32_t max_rows = 1;
  for (auto &ph : phases) {
    std::vector<Task *> &v = ph.second;
    std::sort(v.begin(), v.end(), [](const Task *a, const Task *b) { return a->a0 < b->a0; });
    const size_t k = v.size();
    const int mat = ph.first.first;
    const uint32_t align = gemv_row_align(mat, h.cfg.max_batch);
    const uint32_t rows = v.back()->a1;
    bool ok = k >= 2 && v.front()->a0 == 0;
    // staged and end times relative to the phase's first staged stamp, averaged over the traces
    std::vector<double> st(k, 0.0), en(k, 0.0);
    for (int r = 0; r < n_traces && ok; ++r) {
      const uint64_t *tr = traces + (size_t)r * stride;
      uint64_t ref = ~0ull;
      for (const Task *t : v) {
        const uint64_t *a = tr + 4ull * t->id;
        if (a[2] == 0 || a[3] < a[2]) ok = false;
        ref = std::min(ref, a[2]);
      }
      if (!ok) break;
      for (size_t i = 0; i < k; ++i) {
        const uint64_t *a = tr + 4ull * v[i]->id;
        st[i] += (double)(a[2] - ref) * kTickUs / n_traces;
        en[i] += (double)(a[3] - ref) * kTickUs / n_traces;
      }
    }
    if (ok) {
      // cost per row of each tile's body on its CU; find the common finish time T at which the
      // tiles, each starting when it did, would cover the phase's rows
      std::vector<double> c(k);
      for (size_t i = 0; i < k; ++i)
        c[i] = std::max(en[i] - st[i], 0.05) / (double)(v[i]->a1 - v[i]->a0);
      auto rows_at = [&](double T, size_t i) { return std::max(T - st[i], c[i] * align) / c[i]; };
      double lo = 0.0, hi = 0.0;
      for (size_t i = 0; i < k; ++i) hi = std::max(hi, en[i]);
      hi = hi * 2.0 + 1.0;
      for (int it = 0; it < 100; ++it) {
        const double mid = 0.5 * (lo + hi);
        double tot = 0;
        for (size_t i = 0; i < k; ++i) tot += rows_at(mid, i);
        (tot < rows ? lo : hi) = mid;
      }
      std::vector<double> w(k);
      for (size_t i = 0; i < k; ++i) {
        const double cur = (double)(v[i]->a1 - v[i]->a0);
        w[i] = std::max((double)align, cur + gain * (rows_at(hi, i) - cur));
      }
      std::vector<uint32_t> b = boundaries(w, rows, align);
      bool fits = true;
      for (size_t i = 0; i < k; ++i) fits &= b[i + 1] - b[i] <= cap_rows;
      if (fits)
        for (size_t i = 0; i < k; ++i) {
          v[i]->a0 = b[i];
          v[i]->a1 = b[i + 1];
        }
    }
    for (const Task *t : v) max_rows = std::max(max_rows, t->a1 - t->a0);
  }
  // attention tasks wait on the QKV tiles that cover their KV group's packed rows
  const BlobConfig &c = h.cfg;
  const uint32_t grows = (uint32_t)qkv_group_rows(c.n_heads, c.n_kv_heads, c.head_dim);
  for (Task *t : by_id) {
    if (t->type != T_ATTN) continue;
    auto it = phases.find({(int)M_QKV, (int)t->layer});
    if (it == phases.end()) return fail("rebalance: attention task without QKV tiles");
    const uint32_t r0 = t->a0 * grows, r1 = (t->a0 + 1) * grows;
    uint32_t lo = ~0u, hi = 0;
    for (const Task *q : it->second)
      if (q->a0 < r1 && q->a1 > r0) {
        lo = std::min(lo, q->id);
        hi = std::max(hi, q->id + 1);
      }
    if (hi <= lo) return fail("rebalance: KV group not covered by QKV tiles");
    t->w0_lo = lo;
    t->w0_hi = hi;
  }
  s->hdr.lds_bytes = (uint32_t)lds_bytes_for((int32_t)h.batch, c.hidden, c.n_heads * c.head_dim,
                                             c.ffn, c.n_heads / c.n_kv_heads, c.head_dim,
                                             (int32_t)max_rows);
  s->hdr.predicted_us = predict_makespan(*s, default_cost_model((int32_t)h.n_cu), (int32_t)h.ctx_hint);
  return true;
}

}  // namespace amk

using namespace amk;

extern "C" amk_status amk_schedule_rebalance(const void *blob, size_t bytes, const uint64_t *traces,
                                             int32_t n_traces, double gain, void **out_blob,
                                             size_t *out_bytes) {
  AMK_API_BEGIN
  if (!blob || !traces || !out_blob || !out_bytes)
    return set_error(AMK_E_INVALID, "amk_schedule_rebalance: null argument");
  Schedule s;
  std::string e, rep;
  if (!parse(blob, bytes, &s, &e)) return set_error(AMK_E_INVALID, e);
  if (!validate_schedule(s, &rep)) return set_error(AMK_E_SCHEDULE_REJECTED, rep);
  if (!rebalance_schedule(&s, traces, n_traces, gain, &e)) return set_error(AMK_E_INVALID, e);
  if (!validate_schedule(s, &rep)) return set_error(AMK_E_SCHEDULE_REJECTED, rep);
  std::vector<uint8_t> out = serialize(s);
  void *mem = std::malloc(out.size());
  if (!mem) return set_error(AMK_E_OOM, "amk_schedule_rebalance: out of host memory");
  std::memcpy(mem, out.data(), out.size());
  *out_blob = mem;
  *out_bytes = out.size();
  clear_error();
  return AMK_OK;
  AMK_API_END
}
