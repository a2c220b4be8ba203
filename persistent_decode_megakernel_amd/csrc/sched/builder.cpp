// Offline schedule construction: decompose one decode step into tile tasks, place them on CUs,
// order each CU's list, and search the free parameters against a cost model.
//
// Method (Ada-MK technical summary, "Methodology", Phase I): the execution path is fixed for a
// given deployment configuration, so every decision about what runs where is taken here, before
// any launch, and serialised; the device only walks its frozen list. The decomposition works on
// tile tasks with explicit dependencies rather than an instruction-level graph.
#include <algorithm>
#include <cmath>
#include <cstring>
#include <string>
#include <vector>

#include "sched_internal.h"

namespace amk {

const char *builder_stamp() { return __DATE__ " " __TIME__; }

uint32_t Schedule::n_tasks() const {
  uint32_t n = 0;
  for (auto &v : per_cu) n += (uint32_t)v.size();
  return n;
}

uint32_t weight_bits(int wtype) {
  return wtype == AMK_WT_INT4 ? 4u : (wtype == AMK_WT_INT8 ? 8u : 16u);
}

bool config_ok(const amk_config &c, std::string *err) {
  auto fail = [&](const char *m) {
    if (err) *err = m;
    return false;
  };
  if (c.n_layers < 1 || c.hidden < 8 || c.n_heads < 1 || c.n_kv_heads < 1 || c.head_dim < 8 ||
      c.ffn < 8 || c.vocab < 2)
    return fail("config: non-positive dimension");
  if (c.n_heads % c.n_kv_heads) return fail("config: n_heads must be a multiple of n_kv_heads");
  if (c.head_dim % 8) return fail("config: head_dim must be a multiple of 8");
  if (c.hidden % 8 || c.ffn % 8) return fail("config: hidden and ffn must be multiples of 8");
  if ((int64_t)c.n_heads * c.head_dim != c.hidden)
    return fail("config: hidden must equal n_heads * head_dim");
  if (c.head_dim > 256) return fail("config: head_dim > 256 unsupported");
  if (c.n_heads / c.n_kv_heads > 16) return fail("config: more than 16 query heads per KV head");
  if (c.max_batch < 1 || c.max_batch > kMaxBatch) return fail("config: max_batch must be in [1, 16]");
  if (c.max_seq < 1) return fail("config: max_seq must be >= 1");
  if (c.wtype != AMK_WT_BF16 && c.wtype != AMK_WT_INT8 && c.wtype != AMK_WT_INT4)
    return fail("config: unknown wtype");
  if (c.wtype != AMK_WT_BF16 && c.tied_lm_head)
    return fail("config: int8/int4 weights with a tied LM head are unsupported");
  // batch-1 int8/int4 tiles write their input's digits and a 96-byte zero unit over its fp32
  // staging area: 3K + 96 <= 4 max(hidden, ffn) bytes
  if (c.wtype != AMK_WT_BF16 && c.hidden < 128)
    return fail("config: int8/int4 weights need hidden >= 128");
  if ((c.wtype == AMK_WT_INT4) != (c.group_size != 0))
    return fail("config: group_size is set for int4 weights and only for them");
  if (c.wtype == AMK_WT_INT4) {
    const int g = c.group_size;
    if (g < 32 || g % 32 || c.hidden % g || c.ffn % g || (c.n_heads * c.head_dim) % g)
      return fail("config: int4 group_size must be a multiple of 32 dividing hidden and ffn");
    if (std::max(c.hidden, c.ffn) > kDigitMaxK)
      return fail("config: int4 weights need hidden and ffn <= 16384");
  }
  if (c.wtype == AMK_WT_INT8 && (c.hidden % 16 || c.ffn % 16))
    return fail("config: int8 weights need hidden and ffn multiples of 16");
  if (c.wtype == AMK_WT_INT8 &&
      std::max(std::max(c.hidden, c.n_heads * c.head_dim), c.ffn) > kDigitMaxK)
    return fail("config: int8 weights need hidden, n_heads * head_dim and ffn <= 16384");
  if (!(c.rms_eps > 0.f) || !(c.rope_theta > 0.f)) return fail("config: eps/theta must be > 0");
  return true;
}

namespace {

struct Tiling {
  std::vector<uint32_t> bounds;  // n_tiles + 1 row boundaries
  uint32_t n() const { return (uint32_t)bounds.size() - 1; }
};

// Cut `rows` rows into at most `max_tiles` balanced tiles whose boundaries are multiples of
// `align` (the last tile ends at `rows`, which need not be one), with at least `min_rows` rows per
// tile when possible.
Tiling cut_rows(uint32_t rows, uint32_t align, uint32_t max_tiles, uint32_t min_rows) {
  uint32_t units = (rows + align - 1) / align;
  uint32_t n = std::min<uint32_t>(max_tiles, units);
  if (min_rows > align) n = std::min<uint32_t>(n, std::max<uint32_t>(1, rows / min_rows));
  n = std::max<uint32_t>(n, 1);
  Tiling t;
  for (uint32_t i = 0; i <= n; ++i)
    t.bounds.push_back(std::min<uint32_t>(rows, align * (uint32_t)(((uint64_t)i * units) / n)));
  return t;
}

// CU receiving placement slot s (0 <= s < n_cu). Workgroups of a launch are dealt to the XCDs
// round-robin (workgroup w runs on XCD w % n_xcd), so the XCD-blocked placement maps consecutive
// slots to workgroups of the same XCD.
uint32_t cu_of_slot(uint32_t s, uint32_t n_cu, int placement) {
  const uint32_t n_xcd = (n_cu % 8 == 0) ? 8 : 1;
  if (placement == 1 || n_xcd == 1) return s % n_cu;
  const uint32_t per = n_cu / n_xcd;
  s %= n_cu;
  return (s % per) * n_xcd + (s / per);
}

struct Builder {
  amk_config c;
  int32_t batch;
  uint32_t n_cu;
  amk_sched_params p;
  Schedule s;
  uint32_t next_id = 0;
  uint32_t phase = 0;
  uint32_t max_tile_rows = 1;

  uint32_t place(uint32_t i, uint32_t n_tasks) {
    // spread n_tasks over the CUs, then rotate by phase
    uint32_t slot = (uint32_t)(((uint64_t)i * n_cu) / std::max<uint32_t>(n_tasks, 1));
    slot = (slot + (uint32_t)p.rotate * phase) % n_cu;
    return cu_of_slot(slot, n_cu, p.placement);
  }

  // Emit a GEMV phase; returns [first id, last id + 1) and the tiling.
  std::pair<uint32_t, uint32_t> gemv(uint8_t mat, uint16_t layer, uint32_t rows, uint32_t K,
                                     uint32_t wbits, uint32_t w_lo, uint32_t w_hi, Tiling *out_tiling) {
    const uint32_t align = gemv_row_align(mat, c.max_batch);
    const uint32_t min_bytes = (uint32_t)std::max(1, p.min_tile_kb) * 1024u;
    uint32_t row_bytes = std::max<uint32_t>(1, K * wbits / 8);
    uint32_t min_rows = (min_bytes + row_bytes - 1) / row_bytes;
    min_rows = (min_rows + align - 1) / align * align;
    // keep ys (batch x tile rows floats) bounded
    const uint32_t cap_rows = 4096u / (uint32_t)batch;
    uint32_t max_tiles = n_cu;
    Tiling t = cut_rows(rows, align, max_tiles, min_rows);
    while (true) {
      uint32_t mx = 0;
      for (uint32_t i = 0; i < t.n(); ++i) mx = std::max(mx, t.bounds[i + 1] - t.bounds[i]);
      if (mx <= cap_rows || t.n() >= (rows + align - 1) / align) break;
      t = cut_rows(rows, align, t.n() * 2, align);
    }
    uint32_t first = next_id;
    for (uint32_t i = 0; i < t.n(); ++i) {
      Task k{};
      k.type = T_GEMV;
      k.mat = mat;
      k.layer = layer;
      k.id = next_id++;
      k.a0 = t.bounds[i];
      k.a1 = t.bounds[i + 1];
      k.w0_lo = w_lo;
      k.w0_hi = w_hi;
      k.aux0 = (mat == M_LM) ? i : 0;
      k.aux1 = 0;
      k.aux2 = K;
      max_tile_rows = std::max(max_tile_rows, k.a1 - k.a0);
      s.per_cu[place(i, t.n())].push_back(k);
    }
    ++phase;
    if (out_tiling) *out_tiling = t;
    return {first, next_id};
  }

  void run() {
    const uint32_t L = c.n_layers, d = c.hidden, nq = c.n_heads, nkv = c.n_kv_heads,
                   hd = c.head_dim, F = c.ffn, V = c.vocab;
    const uint32_t wb = weight_bits(c.wtype);
    const uint32_t qkvr = qkv_rows(nq, nkv, hd);
    const uint32_t grows = qkv_group_rows(nq, nkv, hd);
    const uint32_t ctx_hint = p.ctx_hint > 0 ? (uint32_t)p.ctx_hint : (uint32_t)c.max_seq;
    const uint32_t min_block = p.min_block > 0 ? (uint32_t)p.min_block : 64u;
    uint32_t nblk = (uint32_t)p.attn_blocks;
    if (nblk == 0) {
      uint32_t by_cu = std::max<uint32_t>(1, n_cu / nkv);
      uint32_t by_ctx = std::max<uint32_t>(1, ctx_hint / min_block);
      nblk = std::min(by_cu, by_ctx);
    }
    // query heads per attention task: the group's heads split into `ranges` tasks per KV block
    const uint32_t qpg = nq / nkv;
    uint32_t hp = qpg;
    if (p.heads_per_task > 0 && qpg % (uint32_t)p.heads_per_task == 0) {
      hp = (uint32_t)p.heads_per_task;
    } else if (p.heads_per_task == 0 && c.max_batch == 1) {
      for (uint32_t r = qpg; r >= 1; --r)
        if (qpg % r == 0 && nkv * r * nblk <= 2 * n_cu) {
          hp = qpg / r;
          break;
        }
    }
    const uint32_t ranges = qpg / hp;
    s.per_cu.assign(n_cu, {});
    uint32_t d_lo = 0, d_hi = 0;  // tasks producing the residual entering the layer
    for (uint32_t l = 0; l < L; ++l) {
      Tiling qt;
      auto qkv = gemv(M_QKV, (uint16_t)l, qkvr, d, wb, d_lo, d_hi, &qt);
      // attention: one task per (kv group, range of its query heads, KV block); waits on the QKV
      // tiles of its whole group (it reads every q word of the group). The range's last block
      // also merges the range's partials and so waits on the range's other blocks too. Mergers
      // are numbered after all other blocks of the layer, so the O tiles wait on the id range of
      // the mergers and each merger on the id range of its head range's other blocks.
      const uint32_t a_first = next_id;
      const uint32_t n_rng = nkv * ranges;
      const uint32_t n_attn = n_rng * nblk;
      const uint32_t m_first = a_first + n_rng * (nblk - 1);
      for (uint32_t g = 0; g < nkv; ++g) {
        uint32_t r0 = g * grows, r1 = (g + 1) * grows;
        uint32_t lo = qkv.second, hi = qkv.first;
        for (uint32_t i = 0; i < qt.n(); ++i) {
          if (qt.bounds[i] < r1 && qt.bounds[i + 1] > r0) {
            lo = std::min(lo, qkv.first + i);
            hi = std::max(hi, qkv.first + i + 1);
          }
        }
        for (uint32_t hr = 0; hr < ranges; ++hr) {
          const uint32_t rg = g * ranges + hr;  // this head range's index in the layer
          for (uint32_t b = 0; b < nblk; ++b) {
            const bool merger = b + 1 == nblk;
            Task k{};
            k.type = T_ATTN;
            k.layer = (uint16_t)l;
            k.id = merger ? m_first + rg : a_first + rg * (nblk - 1) + b;
            k.a0 = g;
            k.a1 = b;
            k.w0_lo = lo;
            k.w0_hi = hi;
            if (merger) {
              k.w1_lo = a_first + rg * (nblk - 1);
              k.w1_hi = k.w1_lo + (nblk - 1);
            }
            k.aux0 = nblk;
            k.aux1 = merger ? 1u : 0u;
            k.aux2 = hr * hp;  // first query head of the range within the group
            k.aux3 = hp;       // heads in the range
            s.per_cu[place(rg * nblk + b, n_attn)].push_back(k);
          }
        }
      }
      next_id = a_first + n_attn;
      ++phase;
      auto o = gemv(M_O, (uint16_t)l, d, nq * hd, wb, m_first, next_id, nullptr);
      auto gu = gemv(M_GU, (uint16_t)l, 2 * F, d, wb, o.first, o.second, nullptr);
      auto dn = gemv(M_D, (uint16_t)l, d, F, wb, gu.first, gu.second, nullptr);
      d_lo = dn.first;
      d_hi = dn.second;
    }
    const uint32_t lmwb = c.tied_lm_head ? 16 : wb;
    Tiling lt;
    auto lm = gemv(M_LM, 0, V, d, lmwb, d_lo, d_hi, &lt);
    Task k{};
    k.type = T_ARGMAX;
    k.id = next_id++;
    k.w0_lo = lm.first;
    k.w0_hi = lm.second;
    k.aux0 = lt.n();
    s.per_cu[cu_of_slot(0, n_cu, p.placement)].push_back(k);

    BlobHeader &h = s.hdr;
    h.magic = kBlobMagic;
    h.version = kBlobVersion;
    h.n_cu = n_cu;
    h.n_tasks = next_id;
    h.batch = (uint32_t)batch;
    h.attn_blocks = nblk;
    h.n_lm_tiles = lt.n();
    h.lds_bytes = (uint32_t)lds_bytes_for(batch, d, nq * hd, F, nq / nkv, hd, max_tile_rows);
    h.ctx_hint = ctx_hint;
    h.placement = (uint32_t)p.placement;
    h.rotate = (uint32_t)p.rotate;
    static_assert(sizeof(BlobConfig) == sizeof(amk_config), "config copy layout");
    std::memcpy(&h.cfg, &c, sizeof(BlobConfig));
  }
};

}  // namespace

amk_cost_model builtin_cost_model() {
  amk_cost_model m{};
  m.cu_stream_gbs = 8000.0 * 0.8 / 256.0;  // 80% of 8 TB/s shared by 256 CUs
  m.hop_us = 2.0;
  m.task_us = 1.0;
  m.attn_us = 1.0;
  m.l2_gbs = 100.0;
  m.prefetch_kb = 128.0;  // two 8 KB chunks per wave, eight waves
  return m;
}

void task_bytes(const BlobHeader &h, const Task &t, int32_t ctx, double *hbm, double *act) {
  const BlobConfig &c = h.cfg;
  const double B = h.batch;
  *hbm = 0;
  *act = 0;
  if (t.type == T_GEMV) {
    const double rows = (double)t.a1 - t.a0;
    const double K = (double)t.aux2 - t.aux1;
    const int wt = (t.mat == M_LM && c.tied_lm_head) ? (int)AMK_WT_BF16 : c.wtype;
    // weights plus their fp32 scales: one per row (int8) or per row and group (int4)
    *hbm = rows * K * weight_bits(wt) / 8.0;
    if (wt == AMK_WT_INT8) *hbm += rows * 4.0;
    if (wt == AMK_WT_INT4) *hbm += rows * (K / c.group_size) * 4.0;
    *act = B * K * 4.0;
  } else if (t.type == T_ATTN) {
    int32_t lo, hi;
    attn_block_range(ctx, (int32_t)h.attn_blocks, (int32_t)t.a1, &lo, &hi);
    *hbm = B * 2.0 * (double)(hi - lo) * c.head_dim * 2.0;
    // q of the group, plus (by the merger) the partials of its head range
    const double qpg = c.n_heads / c.n_kv_heads;
    const double hn = t.aux3 ? (double)t.aux3 : qpg;
    *act = B * qpg * c.head_dim * 4.0 + B * hn * (c.head_dim + 2) * 4.0;
  } else if (t.type == T_ARGMAX) {
    *act = (double)t.aux0 * B * 8.0;
  }
}

// List-schedule simulation of one step: every CU runs its tasks in order; a task's inputs are
// seen hop_us after the last of its producers finished. Bytes stream at cu_stream_gbs per CU.
// What a task can do before its inputs are there is overlapped with the wait, as the kernel does:
// a GEMV tile streams its first prefetch_kb of weights (batch 1; the batched ring, its first
// rounds) from the moment its CU is free; an attention block issues the KV history of its first
// sequence. Staging an input costs its activation bytes at l2_gbs. Beyond hop and bytes, a task
// takes task_us (an attention block's partial, attn_us).
double predict_times(const Schedule &s, const amk_cost_model &cm, int32_t ctx,
                     std::vector<TaskTimes> *times) {
  const uint32_t n = s.hdr.n_tasks;
  std::vector<double> finish(n, -1.0);
  std::vector<size_t> head(s.per_cu.size(), 0);
  std::vector<double> cu_free(s.per_cu.size(), 0.0);
  size_t done = 0, total = 0;
  for (auto &v : s.per_cu) total += v.size();
  const double rate = cm.cu_stream_gbs * 1e3, l2 = cm.l2_gbs * 1e3;  // bytes per us
  const double pf = cm.prefetch_kb * 1024.0;
  const double B = std::max<uint32_t>(1, s.hdr.batch);
  if (times) times->assign(n, TaskTimes{});
  // repeated sweeps; tasks become ready once all producers have finished
  bool progress = true;
  while (done < total && progress) {
    progress = false;
    for (size_t c = 0; c < s.per_cu.size(); ++c) {
      while (head[c] < s.per_cu[c].size()) {
        const Task &t = s.per_cu[c][head[c]];
        // dep[r]: when the producers of wait range r have finished and been seen
        double dep[2] = {0.0, 0.0};
        bool ok = true;
        for (int r = 0; r < 2 && ok; ++r) {
          uint32_t lo = r ? t.w1_lo : t.w0_lo, hi = r ? t.w1_hi : t.w0_hi;
          for (uint32_t i = lo; i < hi && i < n; ++i) {
            if (finish[i] < 0) {
              ok = false;
              break;
            }
            dep[r] = std::max(dep[r], finish[i] + cm.hop_us);
          }
        }
        if (!ok) break;
        const double free = cu_free[c];
        double hbm, act;
        task_bytes(s.hdr, t, ctx, &hbm, &act);
        const double staged = std::max(free, dep[0]) + act / l2;
        double end, mid = staged;
        if (t.type == T_GEMV) {
          const double pre = std::min(hbm, pf);
          end = std::max(free + pre / rate, staged) + (hbm - pre) / rate + cm.task_us;
        } else if (t.type == T_ATTN) {
          const double pre = hbm / B;  // the first sequence's rows, issued before the wait
          end = mid = std::max(free + pre / rate, staged) + (hbm - pre) / rate + cm.attn_us;
          // a merger then waits for its group's other blocks and merges their partials
          if (t.aux1) end = std::max(end, dep[1]) + act / l2 + cm.task_us;
        } else {
          end = staged + cm.task_us;
        }
        if (times && t.id < n) (*times)[t.id] = TaskTimes{free, mid, end, (uint32_t)c};
        finish[t.id] = end;
        cu_free[c] = end;
        ++head[c];
        ++done;
        progress = true;
      }
    }
  }
  if (done < total) return INFINITY;
  double m = 0;
  for (double f : cu_free) m = std::max(m, f);
  return m;
}

double predict_makespan(const Schedule &s, const amk_cost_model &cm, int32_t ctx) {
  return predict_times(s, cm, ctx, nullptr);
}

Schedule build_schedule(const amk_config &cfg, int32_t batch, int32_t n_cu,
                        const amk_sched_params &p) {
  Builder b;
  b.c = cfg;
  b.batch = batch;
  b.n_cu = (uint32_t)n_cu;
  b.p = p;
  b.run();
  return std::move(b.s);
}

std::vector<uint8_t> serialize(const Schedule &s) {
  BlobHeader h = s.hdr;
  const uint32_t n_cu = (uint32_t)s.per_cu.size();
  h.n_cu = n_cu;
  h.n_tasks = s.n_tasks();
  h.offsets_off = (uint32_t)sizeof(BlobHeader);
  h.tasks_off = (uint32_t)((h.offsets_off + 4u * (n_cu + 1) + 63u) & ~63u);
  h.total_bytes = h.tasks_off + (uint32_t)sizeof(Task) * h.n_tasks;
  std::vector<uint8_t> out(h.total_bytes, 0);
  std::memcpy(out.data(), &h, sizeof h);
  uint32_t *off = reinterpret_cast<uint32_t *>(out.data() + h.offsets_off);
  uint32_t k = 0;
  for (uint32_t c = 0; c < n_cu; ++c) {
    off[c] = k;
    for (const Task &t : s.per_cu[c]) {
      std::memcpy(out.data() + h.tasks_off + sizeof(Task) * k, &t, sizeof(Task));
      ++k;
    }
  }
  off[n_cu] = k;
  return out;
}

bool parse(const void *blob, size_t bytes, Schedule *out, std::string *err) {
  auto fail = [&](const std::string &m) {
    if (err) *err = m;
    return false;
  };
  if (!blob) return fail("blob: null");
  if (bytes < sizeof(BlobHeader)) return fail("blob: shorter than its header");
  BlobHeader h;
  std::memcpy(&h, blob, sizeof h);
  if (h.magic != kBlobMagic) return fail("blob: bad magic");
  if (h.version != kBlobVersion) return fail("blob: unsupported version");
  if (h.total_bytes != bytes) return fail("blob: size mismatch");
  if (h.n_cu == 0 || h.n_cu > 4096) return fail("blob: bad CU count");
  if (h.offsets_off < sizeof(BlobHeader) ||
      (uint64_t)h.offsets_off + 4ull * (h.n_cu + 1) > bytes)
    return fail("blob: offsets table out of range");
  if ((uint64_t)h.tasks_off + (uint64_t)sizeof(Task) * h.n_tasks != bytes)
    return fail("blob: task table size mismatch");
  if (h.tasks_off % 16) return fail("blob: task table misaligned");
  const uint8_t *b = static_cast<const uint8_t *>(blob);
  std::vector<uint32_t> off(h.n_cu + 1);
  std::memcpy(off.data(), b + h.offsets_off, 4u * (h.n_cu + 1));
  if (off[0] != 0 || off[h.n_cu] != h.n_tasks) return fail("blob: offsets do not span tasks");
  // every offset is checked before any task is copied: a single monotone, bounded sequence
  // keeps every CU's task range inside the task table
  for (uint32_t c = 0; c < h.n_cu; ++c)
    if (off[c + 1] < off[c] || off[c + 1] > h.n_tasks) return fail("blob: offsets not monotone");
  out->hdr = h;
  out->per_cu.assign(h.n_cu, {});
  for (uint32_t c = 0; c < h.n_cu; ++c) {
    for (uint32_t i = off[c]; i < off[c + 1]; ++i) {
      Task t;
      std::memcpy(&t, b + h.tasks_off + sizeof(Task) * i, sizeof t);
      out->per_cu[c].push_back(t);
    }
  }
  return true;
}

}  // namespace amk
