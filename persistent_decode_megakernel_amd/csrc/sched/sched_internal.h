// Host-side schedule layer: in-memory schedule, blob (de)serialisation, task footprints.
#pragma once
#include <cstddef>
#include <cstdint>
#include <string>
#include <vector>

#include "amk.h"
#include "layout.h"

namespace amk {

// Dynamic LDS a schedule may ask for per workgroup (bytes): the CU's 160 KiB less a reserve for
// what the kernels declare statically (272 bytes today: control words and the block-wide vote of
// __syncthreads_or); model creation checks that the workgroup still fits.
constexpr uint32_t kMaxLdsBytes = 160 * 1024 - 1024;

struct Schedule {
  BlobHeader hdr{};
  std::vector<std::vector<Task>> per_cu;  // program order per CU

  uint32_t n_tasks() const;
};

// Serialise / parse. parse() checks only framing (magic, version, sizes); validate() the rest.
std::vector<uint8_t> serialize(const Schedule &s);
bool parse(const void *blob, size_t bytes, Schedule *out, std::string *err);

// Buffers whose contents a decode step produces (all other inputs are read-only for a step).
enum BufId : int32_t {
  BUF_H = 0,       // residual stream h[s], s = 0..2L: [B][d]; h[0] is the embedding gather
  BUF_Q = 1,       // q after RoPE, per layer: [B][nq*hd]
  BUF_KVNEW = 2,   // the KV cache slot being appended, per layer: [2][B][nkv][hd]
  BUF_PART = 3,    // attention partials, per layer: [B][nq][nblk][hd+2]
  BUF_A = 4,       // SwiGLU output, per layer: [B][F]
  BUF_LOGITS = 5,  // [B][V]
  BUF_AMAX = 6,    // argmax partials [slots][B]
  BUF_NEXT = 7,    // [B]
  BUF_AO = 8,      // attention output merged over the KV blocks, per layer: [B][nq*hd]
};

struct Access {
  int32_t buf;    // BufId
  int32_t index;  // layer (BUF_Q/KVNEW/PART/A/AO) or residual slot (BUF_H); 0 otherwise
  int64_t lo, hi; // element range [lo, hi)
  bool write;
  bool staged;    // read as the task's staged input: the dependency of a tagged hand-off
};

// Batch-1 megakernel instances (max_batch == 1) hand every step-local value over as epoch-tagged
// words: a task with staged inputs (GEMV input vectors; the attention blocks' q and appended K/V
// row; the merger's other partials) waits by reloading them until every tag is current (its flag
// waits are not consulted), and only the LM tiles and the argmax store flags. These two
// predicates mirror the kernel's choice.
bool tagged_handoff(const BlobHeader &h);
bool stores_flag(const BlobHeader &h, const Task &t);

// Read/write footprint of a task, derived from the task's own fields and the config. Reads of
// the embedding row (h[0]), weights and KV history are not listed: nothing in a step writes them.
// Returns false (and err) if the task's fields are malformed for the config.
bool footprint(const BlobHeader &h, const Task &t, std::vector<Access> *acc, std::string *err);

// Algorithmic HBM bytes a task streams (weights, scales, KV rows) at context length ctx, and the
// activation bytes it re-reads from cache. Used by the cost model.
void task_bytes(const BlobHeader &h, const Task &t, int32_t ctx, double *hbm, double *act);

double predict_makespan(const Schedule &s, const amk_cost_model &cost, int32_t ctx);
// The same simulation, with each task's times (us): picked up by its CU, its input staged (an
// attention block: its partial done), finished.
struct TaskTimes {
  double start, mid, end;
  uint32_t cu;
};
double predict_times(const Schedule &s, const amk_cost_model &cost, int32_t ctx,
                     std::vector<TaskTimes> *times);

// Built-in cost model values, and the model the search uses when given none: the calibrated
// one stored beside the library for this CU count, else the built-in one (*source says which).
amk_cost_model builtin_cost_model();
amk_cost_model default_cost_model(int32_t n_cu, std::string *source = nullptr);
bool parse_cost_model(const std::string &text, int32_t n_cu, amk_cost_model *out);
// The caller's model with its zero (or invalid) fields taken from default_cost_model(n_cu).
amk_cost_model fill_cost(const amk_cost_model *c, int32_t n_cu);

Schedule build_schedule(const amk_config &cfg, int32_t batch, int32_t n_cu,
                        const amk_sched_params &p);

// Compile stamps of the builder and of the search (cache keys of built schedules).
const char *builder_stamp();
const char *schedule_build_stamp();

bool validate_schedule(const Schedule &s, std::string *report);
bool simulate_schedule(const Schedule &s, std::string *report, int32_t max_delay_runs);

bool config_ok(const amk_config &c, std::string *err);

// Move the GEMV tile boundaries of *s towards equal finish times measured in task traces (see
// amk_schedule_rebalance). Keeps ids, placement and waits; attention waits follow the QKV tiles.
bool rebalance_schedule(Schedule *s, const uint64_t *traces, int n_traces, double gain,
                        std::string *err);

}  // namespace amk
