// C entry points of the host-only schedule layer.
#include <cmath>
#include <cstdlib>
#include <cstring>
#include <new>
#include <stdexcept>
#include <string>
#include <vector>

#include "../runtime/errors.h"
#include "sched_internal.h"

namespace amk {

// the caller's model with its zero (or invalid) fields taken from the default model
amk_cost_model fill_cost(const amk_cost_model *c, int32_t n_cu) {
  amk_cost_model d = default_cost_model(n_cu);
  if (!c) return d;
  amk_cost_model m = *c;
  if (!(m.cu_stream_gbs > 0)) m.cu_stream_gbs = d.cu_stream_gbs;
  if (!(m.hop_us > 0)) m.hop_us = d.hop_us;
  if (!(m.task_us > 0)) m.task_us = d.task_us;
  if (!(m.l2_gbs > 0)) m.l2_gbs = d.l2_gbs;
  if (!(m.prefetch_kb > 0)) m.prefetch_kb = d.prefetch_kb;
  if (!(m.attn_us > 0)) m.attn_us = d.attn_us;
  return m;
}

// Exhaustive search over the discrete parameters left free (zero) in `base`; the cost model
// ranks candidates by predicted makespan at the context hint.
Schedule search_schedule(const amk_config &cfg, int32_t batch, int32_t n_cu,
                         const amk_sched_params &base, const amk_cost_model &cost) {
  std::vector<int32_t> placements = {base.placement};
  std::vector<int32_t> rotates = {base.rotate};
  std::vector<int32_t> blocks = {base.attn_blocks};
  std::vector<int32_t> tiles = {base.min_tile_kb > 0 ? base.min_tile_kb : 4};
  if (base.search) {
    placements = {0, 1};
    rotates = {0, 1};
    if (base.attn_blocks == 0) {
      amk_sched_params p = base;
      Schedule s0 = build_schedule(cfg, batch, n_cu, p);
      int32_t a = (int32_t)s0.hdr.attn_blocks;
      blocks = {a};
      if (a / 2 >= 1) blocks.push_back(a / 2);
      blocks.push_back(a * 2);
    }
    if (base.min_tile_kb == 0) tiles = {4, 16, 64};
  }
  Schedule best;
  double best_t = INFINITY;
  bool have = false;
  const int32_t ctx = base.ctx_hint > 0 ? base.ctx_hint : cfg.max_seq;
  for (int32_t pl : placements)
    for (int32_t ro : rotates)
      for (int32_t bl : blocks)
        for (int32_t tk : tiles) {
          amk_sched_params p = base;
          p.placement = pl;
          p.rotate = ro;
          p.attn_blocks = bl;
          p.min_tile_kb = tk;
          Schedule s = build_schedule(cfg, batch, n_cu, p);
          if (s.hdr.lds_bytes > kMaxLdsBytes) continue;
          double t = predict_makespan(s, cost, ctx);
          if (!have || t < best_t) {
            best_t = t;
            best = std::move(s);
            have = true;
          }
        }
  if (!have) throw std::runtime_error("no schedule candidate fits the LDS budget");
  best.hdr.predicted_us = best_t;
  return best;
}

// Build stamp of the schedule search (this file and the builder): part of the key under which
// model creation caches built schedules, so a rebuilt library never reuses older builds' blobs.
const char *schedule_build_stamp() {
  static const std::string stamp = std::string(__DATE__ " " __TIME__) + "/" + builder_stamp();
  return stamp.c_str();
}

}  // namespace amk

using namespace amk;

extern "C" amk_status amk_schedule_build(const amk_config *cfg, int32_t batch, int32_t n_cu,
                                         const amk_sched_params *params,
                                         const amk_cost_model *cost, void **blob, size_t *bytes) {
  AMK_API_BEGIN
  if (!cfg || !blob || !bytes) return set_error(AMK_E_INVALID, "amk_schedule_build: null argument");
  std::string e;
  if (!config_ok(*cfg, &e)) return set_error(AMK_E_INVALID, e);
  if (batch < 1 || batch > cfg->max_batch)
    return set_error(AMK_E_INVALID, "amk_schedule_build: batch outside [1, max_batch]");
  if (n_cu < 1 || n_cu > 4096) return set_error(AMK_E_INVALID, "amk_schedule_build: bad n_cu");
  amk_sched_params p{};
  if (params) p = *params;
  else p.search = 1;
  if (p.attn_blocks < 0 || p.min_block < 0 || p.rotate < 0 || p.ctx_hint < 0 || p.min_tile_kb < 0 ||
      p.placement < 0 || p.placement > 1)
    return set_error(AMK_E_INVALID, "amk_schedule_build: negative or unknown parameter");
  amk_cost_model cm = fill_cost(cost, n_cu);
  Schedule s = search_schedule(*cfg, batch, n_cu, p, cm);
  std::vector<uint8_t> out = serialize(s);
  void *mem = std::malloc(out.size());
  if (!mem) return set_error(AMK_E_OOM, "amk_schedule_build: out of host memory");
  std::memcpy(mem, out.data(), out.size());
  *blob = mem;
  *bytes = out.size();
  clear_error();
  return AMK_OK;
  AMK_API_END
}

extern "C" amk_status amk_schedule_validate(const void *blob, size_t bytes, char *report,
                                            size_t report_cap) {
  AMK_API_BEGIN
  Schedule s;
  std::string e, rep;
  bool ok = parse(blob, bytes, &s, &e) ? validate_schedule(s, &rep) : (rep = "REJECTED: " + e, false);
  if (report && report_cap) {
    std::strncpy(report, rep.c_str(), report_cap - 1);
    report[report_cap - 1] = 0;
  }
  if (!ok) return set_error(AMK_E_SCHEDULE_REJECTED, rep);
  clear_error();
  return AMK_OK;
  AMK_API_END
}

extern "C" amk_status amk_schedule_simulate(const void *blob, size_t bytes, char *report,
                                            size_t report_cap) {
  AMK_API_BEGIN
  Schedule s;
  std::string e, rep;
  bool ok = parse(blob, bytes, &s, &e) ? simulate_schedule(s, &rep, 64) : (rep = "UNSAFE: " + e, false);
  if (report && report_cap) {
    std::strncpy(report, rep.c_str(), report_cap - 1);
    report[report_cap - 1] = 0;
  }
  if (!ok) return set_error(AMK_E_SCHEDULE_REJECTED, rep);
  clear_error();
  return AMK_OK;
  AMK_API_END
}

extern "C" amk_status amk_schedule_predict(const void *blob, size_t bytes,
                                           const amk_cost_model *cost, int32_t ctx,
                                           double *makespan_us) {
  AMK_API_BEGIN
  if (!makespan_us) return set_error(AMK_E_INVALID, "amk_schedule_predict: null output");
  Schedule s;
  std::string e;
  if (!parse(blob, bytes, &s, &e)) return set_error(AMK_E_INVALID, e);
  if (ctx < 1) return set_error(AMK_E_INVALID, "amk_schedule_predict: ctx must be >= 1");
  *makespan_us = predict_makespan(s, fill_cost(cost, (int32_t)s.hdr.n_cu), ctx);
  clear_error();
  return AMK_OK;
  AMK_API_END
}

extern "C" void amk_blob_free(void *blob) { std::free(blob); }
