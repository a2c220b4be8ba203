// Static validation and dynamic simulation of a frozen schedule.
//
// Follows the AutoMegaKernel abstract (page 5 of the set): a frozen schedule is certified free of
// deadlock and races by static graph checks before it is launched, and unsafe schedules are
// rejected. Here the checks are:
//   * structure: every task id appears once, fields are in range for the config, wait ranges
//     name existing tasks and never the task itself, LDS and batch limits hold;
//   * deadlock freedom: the graph of flag waits plus per-CU program order is acyclic. With every
//     workgroup co-resident (the runtime launches cooperatively) and flags that only grow, an
//     acyclic graph means every wait is eventually satisfied;
//   * race freedom and coverage: every element a task reads from a buffer written during the
//     step is written by exactly one task, and that writer happens-before the reader;
//   * tagged hand-offs (batch-1 instances): a tile that waits by reloading its tagged input
//     declares exactly that input's writers as its waits, so the graph checked above is the one
//     the kernel enforces, and no task waits on the flag of a tile that stores none;
//   * step ordering: exactly one argmax task, and every task precedes it (through waits and
//     program order). A multi-step launch starts a step's first-layer QKV tiles after the
//     previous step's argmax, so no task of a step can overlap the next step's writes.
// The simulator is an independent dynamic check: it executes the tasks under several
// interleavings (greedy, and one run per delayed CU) with shadow memory, flagging stale reads,
// double writes and stuck states.
#include <algorithm>
#include <cstdio>
#include <cstring>
#include <map>
#include <string>
#include <vector>

#include "sched_internal.h"

namespace amk {
namespace {

std::string fmt(const char *f, long long a = 0, long long b = 0, long long c = 0) {
  char buf[256];
  std::snprintf(buf, sizeof buf, f, a, b, c);
  return buf;
}

void add_range(std::vector<Access> *acc, int buf, int index, int64_t lo, int64_t hi, bool w,
               bool staged = false) {
  if (hi > lo) acc->push_back(Access{buf, index, lo, hi, w, staged});
}

// the GEMV input vector: read whole, staged into LDS
void add_staged(std::vector<Access> *acc, int buf, int index, int64_t n) {
  add_range(acc, buf, index, 0, n, false, true);
}

// Merge sorted element indices into intervals.
void add_elems(std::vector<Access> *acc, int buf, int index, std::vector<int64_t> &e, bool w) {
  std::sort(e.begin(), e.end());
  size_t i = 0;
  while (i < e.size()) {
    size_t j = i + 1;
    while (j < e.size() && e[j] == e[j - 1] + 1) ++j;
    add_range(acc, buf, index, e[i], e[j - 1] + 1, w);
    i = j;
  }
}

}  // namespace

bool tagged_handoff(const BlobHeader &h) { return h.cfg.max_batch == 1; }

bool stores_flag(const BlobHeader &h, const Task &t) {
  return !tagged_handoff(h) || t.type == T_ARGMAX || (t.type == T_GEMV && t.mat == M_LM);
}

bool footprint(const BlobHeader &h, const Task &t, std::vector<Access> *acc, std::string *err) {
  const BlobConfig &c = h.cfg;
  const int64_t B = h.batch, L = c.n_layers, d = c.hidden, nq = c.n_heads, nkv = c.n_kv_heads,
                hd = c.head_dim, F = c.ffn, V = c.vocab, qd = nq * hd, qpg = nq / nkv,
                nblk = h.attn_blocks;
  auto bad = [&](const char *m) {
    if (err) *err = fmt("task %lld: ", t.id) + m;
    return false;
  };
  acc->clear();
  if (t.type == T_GEMV) {
    if (t.a0 >= t.a1) return bad("empty or inverted row range");
    const int64_t l = t.layer;
    if (t.mat != M_LM && l >= L) return bad("layer out of range");
    int64_t rows, K;
    switch (t.mat) {
      case M_QKV: rows = qkv_rows((int32_t)nq, (int32_t)nkv, (int32_t)hd); K = d; break;
      case M_O: rows = d; K = qd; break;
      case M_GU: rows = 2 * F; K = d; break;
      case M_D: rows = d; K = F; break;
      case M_LM: rows = V; K = d; break;
      default: return bad("unknown matrix");
    }
    if (t.a1 > rows) return bad("rows beyond the matrix");
    // the kernel instance, and with it the weight layout, follows the model's batch capacity
    const int64_t align = gemv_row_align(t.mat, c.max_batch);
    if (t.a0 % align || (t.a1 % align && t.a1 != rows))
      return bad(c.max_batch > 1 ? "tile boundary off the weights' 16-row groups" : "tile splits a row pair");
    if (t.aux1 != 0 || (int64_t)t.aux2 != K) return bad("K range must be the full row");
    if ((int64_t)t.a1 - t.a0 > 4096 / B) return bad("tile too tall for the output staging");
    const int64_t a0 = t.a0, a1 = t.a1;
    switch (t.mat) {
      case M_QKV: {
        if (l > 0) add_staged(acc, BUF_H, (int)(2 * l), B * d);
        std::vector<int64_t> qe, ke;
        for (int64_t r = a0; r < a1; ++r) {
          QkvRow q = qkv_decode((int32_t)r, (int32_t)nq, (int32_t)nkv, (int32_t)hd);
          for (int64_t b = 0; b < B; ++b) {
            if (q.kind == KIND_Q)
              qe.push_back(b * qd + q.head * hd + q.dim);
            else
              ke.push_back((((q.kind == KIND_K ? 0 : 1) * B + b) * nkv + q.head) * hd + q.dim);
          }
        }
        add_elems(acc, BUF_Q, (int)l, qe, true);
        add_elems(acc, BUF_KVNEW, (int)l, ke, true);
        break;
      }
      case M_O:
        add_staged(acc, BUF_AO, (int)l, B * qd);
        for (int64_t b = 0; b < B; ++b) {
          if (l > 0) add_range(acc, BUF_H, (int)(2 * l), b * d + a0, b * d + a1, false);
          add_range(acc, BUF_H, (int)(2 * l + 1), b * d + a0, b * d + a1, true);
        }
        break;
      case M_GU:
        add_staged(acc, BUF_H, (int)(2 * l + 1), B * d);
        for (int64_t b = 0; b < B; ++b) add_range(acc, BUF_A, (int)l, b * F + a0 / 2, b * F + a1 / 2, true);
        break;
      case M_D:
        add_staged(acc, BUF_A, (int)l, B * F);
        for (int64_t b = 0; b < B; ++b) {
          add_range(acc, BUF_H, (int)(2 * l + 1), b * d + a0, b * d + a1, false);
          add_range(acc, BUF_H, (int)(2 * l + 2), b * d + a0, b * d + a1, true);
        }
        break;
      case M_LM:
        if (t.layer != 0) return bad("LM tile must carry layer 0");
        if (t.aux0 >= h.n_lm_tiles) return bad("argmax slot out of range");
        add_staged(acc, BUF_H, (int)(2 * L), B * d);
        for (int64_t b = 0; b < B; ++b) add_range(acc, BUF_LOGITS, 0, b * V + a0, b * V + a1, true);
        add_range(acc, BUF_AMAX, 0, (int64_t)t.aux0 * B, (int64_t)t.aux0 * B + B, true);
        break;
    }
    return true;
  }
  if (t.type == T_ATTN) {
    const int64_t l = t.layer, g = t.a0, blk = t.a1;
    if (l >= L) return bad("layer out of range");
    if (g >= nkv) return bad("kv group out of range");
    if (blk >= nblk || t.aux0 != h.attn_blocks) return bad("KV block out of range");
    // query heads [hs, hs + hn) of the group (aux3 = 0: the whole group)
    const int64_t hs = t.aux3 ? (int64_t)t.aux2 : 0, hn = t.aux3 ? (int64_t)t.aux3 : qpg;
    if (hn < 1 || hs < 0 || hs + hn > qpg) return bad("query head range outside the KV group");
    // the range's last block merges the range's partials (and only it)
    const bool merger = blk == nblk - 1;
    if (t.aux1 != (merger ? 1u : 0u)) return bad("the merger must be the group's last KV block");
    for (int64_t b = 0; b < B; ++b) {
      add_range(acc, BUF_Q, (int)l, b * qd + g * qpg * hd, b * qd + (g + 1) * qpg * hd, false, true);
      for (int64_t kvi = 0; kvi < 2; ++kvi) {
        int64_t base = ((kvi * B + b) * nkv + g) * hd;
        add_range(acc, BUF_KVNEW, (int)l, base, base + hd, false, true);
      }
      for (int64_t hh = g * qpg + hs; hh < g * qpg + hs + hn; ++hh) {
        int64_t base = ((b * nq + hh) * nblk + blk) * (hd + 2);
        add_range(acc, BUF_PART, (int)l, base, base + hd + 2, true);
      }
    }
    if (merger) {
      // every other block's partials of the range in (its own it reads back after its stores),
      // the range's merged heads out
      for (int64_t b = 0; b < B; ++b) {
        for (int64_t hh = g * qpg + hs; hh < g * qpg + hs + hn; ++hh) {
          int64_t base = (b * nq + hh) * nblk * (hd + 2);
          add_range(acc, BUF_PART, (int)l, base, base + blk * (hd + 2), false, true);
        }
        add_range(acc, BUF_AO, (int)l, b * qd + (g * qpg + hs) * hd, b * qd + (g * qpg + hs + hn) * hd, true);
      }
    }
    return true;
  }
  if (t.type == T_ARGMAX) {
    if (t.aux0 != h.n_lm_tiles) return bad("argmax must read every LM slot");
    add_range(acc, BUF_AMAX, 0, 0, (int64_t)t.aux0 * B, false);
    add_range(acc, BUF_NEXT, 0, 0, B, true);
    return true;
  }
  return bad("unknown task type");
}

namespace {

struct Graph {
  uint32_t n = 0;
  std::vector<uint32_t> cu, pos;          // by id
  std::vector<const Task *> task;         // by id
  std::vector<int64_t> prev_same_cu;      // by id: id of the previous task on the CU or -1
  std::vector<uint32_t> topo_index;       // by id
  std::vector<uint32_t> stamp;
  uint32_t cur_stamp = 0;

  bool waits_on(const Task &r, uint32_t w) const {
    return (w >= r.w0_lo && w < r.w0_hi) || (w >= r.w1_lo && w < r.w1_hi);
  }

  // does task w happen-before task r?
  bool hb(uint32_t w, uint32_t r) {
    if (w == r) return false;
    if (cu[w] == cu[r]) return pos[w] < pos[r];
    if (waits_on(*task[r], w)) return true;
    if (topo_index[w] >= topo_index[r]) return false;
    // backward search from r over predecessors, pruned by topological index
    ++cur_stamp;
    std::vector<uint32_t> stack{r};
    stamp[r] = cur_stamp;
    const uint32_t tw = topo_index[w];
    while (!stack.empty()) {
      uint32_t x = stack.back();
      stack.pop_back();
      auto visit = [&](uint32_t y) -> bool {
        if (y == w) return true;
        if (stamp[y] == cur_stamp || topo_index[y] < tw) return false;
        stamp[y] = cur_stamp;
        stack.push_back(y);
        return false;
      };
      if (prev_same_cu[x] >= 0 && visit((uint32_t)prev_same_cu[x])) return true;
      const Task &t = *task[x];
      for (int k = 0; k < 2; ++k) {
        uint32_t lo = k ? t.w1_lo : t.w0_lo, hi = k ? t.w1_hi : t.w0_hi;
        for (uint32_t y = lo; y < hi; ++y)
          if (visit(y)) return true;
      }
    }
    return false;
  }
};

struct BufKey {
  int32_t buf, index;
  bool operator<(const BufKey &o) const { return buf != o.buf ? buf < o.buf : index < o.index; }
};

struct Span {
  int64_t lo, hi;
  uint32_t id;
};

}  // namespace

bool validate_schedule(const Schedule &s, std::string *report) {
  std::string r;
  auto fail = [&](const std::string &m) {
    if (report) *report = "REJECTED: " + m;
    return false;
  };
  const BlobHeader &h = s.hdr;
  amk_config cfg;
  std::memcpy(&cfg, &h.cfg, sizeof cfg);
  std::string e;
  if (!config_ok(cfg, &e)) return fail(e);
  if (h.batch < 1 || (int32_t)h.batch > cfg.max_batch) return fail("batch outside [1, max_batch]");
  if (h.attn_blocks < 1) return fail("attn_blocks must be >= 1");
  if (h.n_lm_tiles < 1) return fail("no LM tiles");
  if (s.per_cu.size() != h.n_cu) return fail("CU table size mismatch");
  if (h.lds_bytes > kMaxLdsBytes) return fail(fmt("LDS %lld bytes exceeds %lld", h.lds_bytes, kMaxLdsBytes));
  const uint32_t n = s.n_tasks();
  if (n != h.n_tasks) return fail("task count mismatch");

  Graph g;
  g.n = n;
  g.cu.assign(n, 0);
  g.pos.assign(n, 0);
  g.task.assign(n, nullptr);
  g.prev_same_cu.assign(n, -1);
  uint32_t max_rows = 1;
  for (uint32_t c = 0; c < h.n_cu; ++c) {
    int64_t prev = -1;
    for (uint32_t i = 0; i < s.per_cu[c].size(); ++i) {
      const Task &t = s.per_cu[c][i];
      if (t.id >= n) return fail(fmt("task id %lld out of range", t.id));
      if (g.task[t.id]) return fail(fmt("task id %lld appears twice", t.id));
      g.task[t.id] = &t;
      g.cu[t.id] = c;
      g.pos[t.id] = i;
      g.prev_same_cu[t.id] = prev;
      prev = t.id;
      for (int k = 0; k < 2; ++k) {
        uint32_t lo = k ? t.w1_lo : t.w0_lo, hi = k ? t.w1_hi : t.w0_hi;
        if (lo > hi || hi > n) return fail(fmt("task %lld: wait range [%lld, %lld) invalid", t.id, lo, hi));
        if (t.id >= lo && t.id < hi) return fail(fmt("task %lld waits on itself", t.id));
      }
      if (t.type == T_GEMV) max_rows = std::max(max_rows, t.a1 - t.a0);
    }
  }
  const uint32_t need_lds = (uint32_t)lds_bytes_for((int32_t)h.batch, cfg.hidden,
                                                    cfg.n_heads * cfg.head_dim, cfg.ffn,
                                                    cfg.n_heads / cfg.n_kv_heads, cfg.head_dim,
                                                    (int32_t)max_rows);
  if (h.lds_bytes < need_lds) return fail(fmt("LDS %lld bytes below the %lld the tiles need", h.lds_bytes, need_lds));

  // deadlock freedom: Kahn's algorithm over waits + program order
  std::vector<uint32_t> indeg(n, 0);
  std::vector<uint32_t> succ_off(n + 1, 0);
  for (uint32_t id = 0; id < n; ++id) {
    const Task &t = *g.task[id];
    if (g.prev_same_cu[id] >= 0) { ++indeg[id]; ++succ_off[g.prev_same_cu[id] + 1]; }
    for (int k = 0; k < 2; ++k) {
      uint32_t lo = k ? t.w1_lo : t.w0_lo, hi = k ? t.w1_hi : t.w0_hi;
      for (uint32_t y = lo; y < hi; ++y) { ++indeg[id]; ++succ_off[y + 1]; }
    }
  }
  for (uint32_t i = 0; i < n; ++i) succ_off[i + 1] += succ_off[i];
  std::vector<uint32_t> succ(succ_off[n]);
  std::vector<uint32_t> fill(succ_off.begin(), succ_off.end() - 1);
  for (uint32_t id = 0; id < n; ++id) {
    const Task &t = *g.task[id];
    if (g.prev_same_cu[id] >= 0) succ[fill[g.prev_same_cu[id]]++] = id;
    for (int k = 0; k < 2; ++k) {
      uint32_t lo = k ? t.w1_lo : t.w0_lo, hi = k ? t.w1_hi : t.w0_hi;
      for (uint32_t y = lo; y < hi; ++y) succ[fill[y]++] = id;
    }
  }
  std::vector<uint32_t> q;
  q.reserve(n);
  for (uint32_t i = 0; i < n; ++i)
    if (!indeg[i]) q.push_back(i);
  g.topo_index.assign(n, 0);
  for (size_t k = 0; k < q.size(); ++k) {
    uint32_t x = q[k];
    g.topo_index[x] = (uint32_t)k;
    for (uint32_t j = succ_off[x]; j < succ_off[x + 1]; ++j)
      if (--indeg[succ[j]] == 0) q.push_back(succ[j]);
  }
  if (q.size() != n) return fail(fmt("dependency cycle: %lld of %lld tasks can never start", n - q.size(), n));
  g.stamp.assign(n, 0);

  // footprints grouped by buffer instance
  std::map<BufKey, std::vector<Span>> writes, reads;
  std::vector<Access> acc;
  for (uint32_t id = 0; id < n; ++id) {
    if (!footprint(h, *g.task[id], &acc, &e)) return fail(e);
    for (const Access &a : acc)
      (a.write ? writes : reads)[BufKey{a.buf, a.index}].push_back(Span{a.lo, a.hi, id});
  }
  size_t checked = 0;
  for (auto &kv : writes) {
    auto &w = kv.second;
    std::sort(w.begin(), w.end(), [](const Span &a, const Span &b) { return a.lo < b.lo; });
    for (size_t i = 1; i < w.size(); ++i)
      if (w[i].lo < w[i - 1].hi)
        return fail(fmt("tasks %lld and %lld write the same elements of buffer %lld", w[i - 1].id, w[i].id, kv.first.buf));
  }
  for (auto &kv : reads) {
    auto it = writes.find(kv.first);
    for (const Span &rd : kv.second) {
      if (it == writes.end())
        return fail(fmt("task %lld reads buffer %lld/%lld that no task writes", rd.id, kv.first.buf, kv.first.index));
      const auto &w = it->second;
      // first write whose hi > rd.lo
      size_t i = std::lower_bound(w.begin(), w.end(), rd.lo,
                                  [](const Span &a, int64_t v) { return a.hi <= v; }) - w.begin();
      int64_t covered = rd.lo;
      for (; i < w.size() && w[i].lo < rd.hi; ++i) {
        if (w[i].lo > covered)
          return fail(fmt("task %lld reads element %lld that no task writes", rd.id, covered));
        covered = w[i].hi;
        ++checked;
        if (!g.hb(w[i].id, rd.id))
          return fail(fmt("race: task %lld reads data of task %lld without waiting for it (buffer %lld)", rd.id, w[i].id, kv.first.buf));
      }
      if (covered < rd.hi)
        return fail(fmt("task %lld reads element %lld that no task writes", rd.id, covered));
    }
  }
  // tagged hand-offs: the kernel's wait for a task with staged inputs is those inputs' writers;
  // a flag wait must name tasks that store flags
  if (tagged_handoff(h)) {
    std::vector<uint32_t> want, have;
    for (uint32_t id = 0; id < n; ++id) {
      const Task &t = *g.task[id];
      if (!footprint(h, t, &acc, &e)) return fail(e);
      have.clear();
      for (int k = 0; k < 2; ++k)
        for (uint32_t y = k ? t.w1_lo : t.w0_lo; y < (k ? t.w1_hi : t.w0_hi); ++y) have.push_back(y);
      want.clear();
      bool staged = false;
      for (const Access &a : acc) {
        if (!a.staged) continue;
        staged = true;
        auto it = writes.find(BufKey{a.buf, a.index});
        if (it == writes.end()) continue;
        for (const Span &w : it->second)
          if (w.hi > a.lo && w.lo < a.hi) want.push_back(w.id);
      }
      if (!staged) {
        for (uint32_t y : have)
          if (!stores_flag(h, *g.task[y]))
            return fail(fmt("task %lld waits on the flag of task %lld, which stores none", id, y));
        continue;
      }
      std::sort(want.begin(), want.end());
      want.erase(std::unique(want.begin(), want.end()), want.end());
      std::sort(have.begin(), have.end());
      have.erase(std::unique(have.begin(), have.end()), have.end());
      if (want != have)
        return fail(fmt("task %lld: declared waits (%lld tasks) differ from the writers of its tagged inputs (%lld tasks)",
                        id, (long long)have.size(), (long long)want.size()));
    }
  }
  // step ordering: one argmax, and every task an ancestor of it
  {
    int64_t am = -1;
    for (uint32_t id = 0; id < n; ++id)
      if (g.task[id]->type == T_ARGMAX) {
        if (am >= 0) return fail("more than one argmax task");
        am = id;
      }
    if (am < 0) return fail("no argmax task");
    std::vector<uint8_t> seen(n, 0);
    std::vector<uint32_t> st{(uint32_t)am};
    seen[am] = 1;
    size_t reached = 1;
    while (!st.empty()) {
      const uint32_t x = st.back();
      st.pop_back();
      auto visit = [&](uint32_t y) {
        if (y < n && !seen[y]) {
          seen[y] = 1;
          ++reached;
          st.push_back(y);
        }
      };
      if (g.prev_same_cu[x] >= 0) visit((uint32_t)g.prev_same_cu[x]);
      const Task &t = *g.task[x];
      for (int k = 0; k < 2; ++k)
        for (uint32_t y = k ? t.w1_lo : t.w0_lo; y < (k ? t.w1_hi : t.w0_hi); ++y) visit(y);
    }
    if (reached != n)
      return fail(fmt("%lld tasks do not precede the argmax (steps of one launch could overlap)",
                      (long long)(n - reached)));
  }
  // outputs must be complete
  {
    auto need = [&](int buf, int64_t total) -> bool {
      auto it = writes.find(BufKey{buf, 0});
      if (it == writes.end()) return total == 0;
      int64_t covered = 0;
      for (const Span &sp : it->second) {
        if (sp.lo > covered) return false;
        covered = std::max(covered, sp.hi);
      }
      return covered >= total;
    };
    if (!need(BUF_LOGITS, (int64_t)h.batch * cfg.vocab)) return fail("logits not fully written");
    if (!need(BUF_NEXT, h.batch)) return fail("next tokens not written");
  }
  if (report)
    *report = fmt("OK: %lld tasks on %lld CUs, %lld producer/consumer pairs checked", n, h.n_cu, (long long)checked);
  return true;
}

// ---------------------------------------------------------------------------------------------
// simulator
// ---------------------------------------------------------------------------------------------
namespace {

struct Shadow {
  std::map<BufKey, std::map<int64_t, int64_t>> written;  // merged written intervals lo -> hi

  bool covered(const Access &a) {
    auto &m = written[BufKey{a.buf, a.index}];
    auto it = m.upper_bound(a.lo);
    if (it == m.begin()) return false;
    --it;
    return it->first <= a.lo && it->second >= a.hi;
  }
  bool overlaps(const Access &a) {
    auto &m = written[BufKey{a.buf, a.index}];
    auto it = m.lower_bound(a.hi);
    if (it == m.begin()) return false;
    --it;
    return it->second > a.lo;
  }
  void add(const Access &a) {
    auto &m = written[BufKey{a.buf, a.index}];
    int64_t lo = a.lo, hi = a.hi;
    auto it = m.lower_bound(lo);
    if (it != m.begin()) {
      auto p = std::prev(it);
      if (p->second >= lo) { lo = p->first; hi = std::max(hi, p->second); it = m.erase(p); }
    }
    while (it != m.end() && it->first <= hi) { hi = std::max(hi, it->second); it = m.erase(it); }
    m[lo] = hi;
  }
};

// One run. delayed < 0: greedy in CU order. Otherwise CU `delayed` only advances when no other
// CU can. Returns false with a message on deadlock, stale read or double write.
bool sim_run(const Schedule &s, int64_t delayed, std::string *msg) {
  const uint32_t n = s.n_tasks(), ncu = (uint32_t)s.per_cu.size();
  std::vector<uint8_t> done(n, 0);
  std::vector<size_t> head(ncu, 0);
  Shadow sh;
  std::vector<Access> acc;
  std::string e;
  size_t left = n;
  auto ready = [&](const Task &t) {
    for (int k = 0; k < 2; ++k) {
      uint32_t lo = k ? t.w1_lo : t.w0_lo, hi = k ? t.w1_hi : t.w0_hi;
      for (uint32_t y = lo; y < hi; ++y)
        if (y >= n || !done[y]) return false;
    }
    return true;
  };
  auto exec = [&](const Task &t) -> bool {
    if (!footprint(s.hdr, t, &acc, &e)) { *msg = e; return false; }
    for (const Access &a : acc)
      if (!a.write && !sh.covered(a)) {
        *msg = fmt("stale read: task %lld ran before the data it reads (buffer %lld) was written", t.id, a.buf);
        return false;
      }
    for (const Access &a : acc)
      if (a.write) {
        if (sh.overlaps(a)) { *msg = fmt("double write by task %lld (buffer %lld)", t.id, a.buf); return false; }
        sh.add(a);
      }
    if (t.id < n) done[t.id] = 1;
    --left;
    return true;
  };
  while (left) {
    bool progress = false;
    for (uint32_t c = 0; c < ncu; ++c) {
      if ((int64_t)c == delayed) continue;
      while (head[c] < s.per_cu[c].size() && ready(s.per_cu[c][head[c]])) {
        if (!exec(s.per_cu[c][head[c]])) return false;
        ++head[c];
        progress = true;
      }
    }
    if (progress) continue;
    if (delayed >= 0 && head[delayed] < s.per_cu[delayed].size() &&
        ready(s.per_cu[delayed][head[delayed]])) {
      if (!exec(s.per_cu[delayed][head[delayed]])) return false;
      ++head[delayed];
      continue;
    }
    *msg = fmt("deadlock: %lld tasks can never start", (long long)left);
    return false;
  }
  return true;
}

}  // namespace

bool simulate_schedule(const Schedule &s, std::string *report, int32_t max_delay_runs) {
  std::string msg;
  const uint32_t n = s.n_tasks();
  std::vector<uint8_t> seen(n, 0);
  for (auto &v : s.per_cu)
    for (auto &t : v) {
      if (t.id >= n || seen[t.id]) {
        if (report) *report = "UNSAFE: task ids are not a permutation";
        return false;
      }
      seen[t.id] = 1;
    }
  if (!sim_run(s, -1, &msg)) {
    if (report) *report = "UNSAFE (greedy run): " + msg;
    return false;
  }
  const uint32_t ncu = (uint32_t)s.per_cu.size();
  const uint32_t runs = (max_delay_runs < 0 || (uint32_t)max_delay_runs >= ncu) ? ncu : (uint32_t)max_delay_runs;
  for (uint32_t k = 0; k < runs; ++k) {
    uint32_t c = (runs == ncu) ? k : (uint32_t)(((uint64_t)k * ncu) / runs);
    if (!sim_run(s, c, &msg)) {
      if (report) *report = fmt("UNSAFE (CU %lld delayed): ", c) + msg;
      return false;
    }
  }
  if (report) *report = fmt("SAFE: %lld tasks, %lld interleavings", n, runs + 1);
  return true;
}

}  // namespace amk
