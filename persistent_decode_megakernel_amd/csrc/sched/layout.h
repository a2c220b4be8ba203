// Packed weight-row layouts and the frozen schedule format, shared by the host-side schedule
// layer, the runtime (repacking) and the device kernels.
//
// Packed QKV matrix (rows = (n_heads + 2 n_kv_heads) * head_dim, cols = hidden): KV-group major.
// Group g holds, in order, the rows of its q heads, then of k head g, then of v head g. Inside
// a rotary head (q or k) rows are pair-interleaved: packed row 2j is dimension j and packed row
// 2j+1 is dimension j + head_dim/2, so any tile that starts and ends on an even row holds whole
// RoPE pairs. V rows keep their natural order. Every row a KV group needs is therefore one
// contiguous packed range, which lets attention tasks wait on a contiguous range of tiles.
//
// Packed gate/up matrix (rows = 2 ffn): row 2i is gate row i, row 2i+1 is up row i, so an
// even-aligned tile can apply SwiGLU on its own outputs.
#pragma once
#include <stdint.h>

#ifdef __HIPCC__
#define AMK_HD __host__ __device__ __forceinline__
#else
#define AMK_HD inline
#endif

namespace amk {

// A 64-bit address from its two 32-bit halves as signed words (the form in which the device's
// first-lane broadcast returns them). Each half is widened as unsigned: converting a signed word
// with bit 31 set straight to 64 bits would sign-extend it into the upper half.
AMK_HD uint64_t address_from_words(int32_t hi, int32_t lo) {
  return ((uint64_t)(uint32_t)hi << 32) | (uint64_t)(uint32_t)lo;
}

enum QkvKind : int32_t { KIND_Q = 0, KIND_K = 1, KIND_V = 2 };

struct QkvRow {
  int32_t kind;  // QkvKind
  int32_t head;  // q head index (KIND_Q) or kv head index (KIND_K / KIND_V)
  int32_t dim;   // dimension inside the head
};

AMK_HD int32_t qkv_group_rows(int32_t nq, int32_t nkv, int32_t hd) { return (nq / nkv + 2) * hd; }
AMK_HD int32_t qkv_rows(int32_t nq, int32_t nkv, int32_t hd) { return (nq + 2 * nkv) * hd; }

AMK_HD QkvRow qkv_decode(int32_t r, int32_t nq, int32_t nkv, int32_t hd) {
  const int32_t qpg = nq / nkv;
  const int32_t grows = (qpg + 2) * hd;
  const int32_t g = r / grows;
  const int32_t rem = r - g * grows;
  const int32_t s = rem / hd;
  const int32_t t = rem - s * hd;
  QkvRow out;
  if (s < qpg) {
    out.kind = KIND_Q;
    out.head = g * qpg + s;
  } else {
    out.kind = (s == qpg) ? KIND_K : KIND_V;
    out.head = g;
  }
  out.dim = (out.kind == KIND_V) ? t : ((t & 1) ? (hd / 2 + t / 2) : (t / 2));
  return out;
}

// Source row (in the caller's wq / wk / wv matrix) of packed QKV row r.
AMK_HD int32_t qkv_source_row(int32_t r, int32_t nq, int32_t nkv, int32_t hd) {
  QkvRow q = qkv_decode(r, nq, nkv, hd);
  return q.head * hd + q.dim;
}

// ------------------------------------------------------------------------------------------
// Frozen schedule format
// ------------------------------------------------------------------------------------------
constexpr uint32_t kBlobMagic = 0x534b4d41u;  // "AMKS"
constexpr uint32_t kBlobVersion = 2;

enum TaskType : uint8_t { T_GEMV = 1, T_ATTN = 2, T_ARGMAX = 3 };
enum MatId : uint8_t { M_QKV = 0, M_O = 1, M_GU = 2, M_D = 3, M_LM = 4 };

// One tile task. The device reads these with scalar loads; the order of a CU's tasks in the
// blob is the order the CU executes them. A task may start once every task whose id lies in
// [w0_lo, w0_hi) or [w1_lo, w1_hi) has published flag >= the step's epoch; on completion it
// publishes flags[id] = epoch.
struct Task {
  uint8_t type;   // TaskType
  uint8_t mat;    // MatId (T_GEMV)
  uint16_t layer;
  uint32_t id;
  uint32_t a0, a1;  // T_GEMV: packed rows [a0, a1); T_ATTN: kv group a0, KV block a1
  uint32_t w0_lo, w0_hi;
  uint32_t w1_lo, w1_hi;
  uint32_t aux0;  // T_GEMV + M_LM: argmax partial slot; T_ATTN: blocks per group; T_ARGMAX: slots
  uint32_t aux1, aux2;  // T_GEMV: K range [aux1, aux2) (always the full row in this version)
  uint32_t aux3;
};
static_assert(sizeof(Task) == 48, "task record is 48 bytes");

struct BlobConfig {  // plain copy of amk_config (kept layout-stable inside the blob)
  int32_t n_layers, hidden, n_heads, n_kv_heads, head_dim, ffn, vocab;
  float rms_eps, rope_theta;
  int32_t tied_lm_head, wtype, max_batch, max_seq;
  int32_t group_size;
};

struct BlobHeader {
  uint32_t magic, version;
  uint32_t n_cu, n_tasks;
  uint32_t batch, attn_blocks;
  uint32_t n_lm_tiles, lds_bytes;
  uint32_t ctx_hint, placement;
  uint32_t offsets_off, tasks_off;  // byte offsets of uint32 offsets[n_cu+1] and Task[n_tasks]
  uint32_t total_bytes, rotate;
  BlobConfig cfg;
  double predicted_us;
};

// Row alignment of GEMV tiles. A model of batch capacity above 1 runs the batched kernel
// instance on tile-major weights (16-row groups, see weight_tiled_bytes), so its tile boundaries
// are multiples of 16 rows (the last tile may end at the matrix's ragged row count); batch-1 tiles
// only keep RoPE and SwiGLU row pairs whole.
AMK_HD uint32_t gemv_row_align(int32_t mat, int32_t max_batch) {
  return max_batch > 1 ? 16u : ((mat == M_QKV || mat == M_GU) ? 2u : 1u);
}

// Tile-major weight layout of the batched matrix-core GEMV: the matrix is cut into 16-row x
// 32-input tiles, stored group-major (tile (g, t) of the rows' group g and input step t at
// index g * ceil(K / 32) + t). Inside a tile, lane l = 16 q + c of the instruction's A operand
// holds row 16 g + c, inputs 32 t + 8 q .. 32 t + 8 q + 7 (16 bytes bf16, 8 int8, 4 int4) at byte
// l * lane_bytes, so one step of a 16-row group is one contiguous 64-lane load. Rows past the
// matrix and inputs past K are zero.
AMK_HD int32_t weight_lane_bytes(int32_t wbits) { return wbits; }  // 8 inputs of wbits bits
AMK_HD uint64_t weight_tiled_bytes(int64_t rows, int64_t K, int32_t wbits) {
  return (uint64_t)((rows + 15) / 16) * (uint64_t)((K + 31) / 32) * 64u * (uint64_t)weight_lane_bytes(wbits);
}

// Attention KV block b of nblk over a context of ctx positions: [lo, hi).
AMK_HD void attn_block_range(int32_t ctx, int32_t nblk, int32_t b, int32_t *lo, int32_t *hi) {
  *lo = (int32_t)(((int64_t)b * ctx) / nblk);
  *hi = (int32_t)(((int64_t)(b + 1) * ctx) / nblk);
}

}  // namespace amk

namespace amk {
// LDS layout of the megakernel workgroup (bytes), shared by the builder (recorded in the blob,
// checked by the validator) and the runtime (dynamic LDS at launch).
//   xs : batch x max(hidden, n_heads*head_dim, ffn) float  -- staged GEMV input vector(s)
//   ys : batch x max_tile_rows float                        -- GEMV tile outputs before epilogue
//   red: kRedFloats float                                   -- reductions, combine weights
// Attention tasks reuse the xs region (q, appended rows, partials).
constexpr int32_t kWaves = 8;
constexpr int32_t kThreads = kWaves * 64;
constexpr int32_t kAttnMaxHeads = 4;  // query heads per attention pass (larger groups take several)
// Query heads per attention pass of a KV group of qpg heads.
AMK_HD constexpr int32_t attn_qmax(int32_t qpg) { return qpg <= 1 ? 1 : (qpg <= 2 ? 2 : kAttnMaxHeads); }
// KV rows one loop iteration of the attention body covers: hd / 8 lanes per row, 8 waves.
AMK_HD constexpr int32_t attn_rows_per_iter(int32_t hd) { return 8 * (64 / (hd / 8)); }
// Attention blocks stream each wave's own KV rows in chunks of kAttnSeqIters loads of K (and of V)
// per lane, two chunks in flight per wave; a workgroup chunk is this many rows.
constexpr int32_t kAttnSeqIters = 4;
// one-head batch-1 passes: longer chunks (the first is issued before the staging wait)
constexpr int32_t kAttnSeqItersB1 = 6;
AMK_HD constexpr int32_t attn_seq_chunk_rows(int32_t hd, bool b1_one_head = false) {
  return attn_rows_per_iter(hd) * (b1_one_head ? kAttnSeqItersB1 : kAttnSeqIters);
}
constexpr int32_t kRedFloats = 2048;        // reduction scratch; holds n_heads x blocks weights
// Batch-1 int8 GEMV: the staged input is converted in place to integer digits, holding every
// thread's share in registers; that bounds the input length of an int8 matrix.
constexpr int32_t kDigitMaxK = 16384;

// Staged GEMV input (batch 1 only: batched GEMVs read their inputs straight from memory and use
// the region for the partial tiles of the matrix-core reduction instead).
constexpr int32_t kMaxBatch = 16;  // sequences per step
// partial 16-row tiles of the batched GEMV: waves x row groups x 16 rows x 16 columns
constexpr int32_t kMfmaRedFloats = kWaves * 4 * 16 * 16;
// Batched megakernel instances stream tile-major weights through an LDS ring per wave, which also
// holds that wave's partial tiles between passes: 16.25 KB, four slots of a three-group round
// (three 1 KB weight copies, 1 KB of inputs, 64 bytes of gain).
constexpr int32_t kRingBytes = 16640;
constexpr int32_t kRingFloats = kWaves * kRingBytes / 4;
AMK_HD int32_t lds_xs_floats(int32_t batch, int32_t hidden, int32_t qdim, int32_t ffn) {
  int32_t k = hidden > qdim ? hidden : qdim;
  k = k > ffn ? k : ffn;
  return batch == 1 ? (k + 63) / 64 * 64 : kRingFloats;
}
AMK_HD int32_t lds_attn_floats(int32_t batch, int32_t qpg, int32_t hd) {
  // at most kAttnMaxHeads heads per pass: q and the appended K/V rows of every sequence,
  // [batch][qn*hd] + [batch][2][hd] bf16, every sequence's partial until they are stored,
  // [batch][qn][hd + 2], and the waves' partials of two sequences, [2][waves][qn][hd + 2]
  // (rounded to 64 floats: the regions after it stay 256-byte aligned for 16-byte LDS copies)
  const int32_t qn = qpg < kAttnMaxHeads ? qpg : kAttnMaxHeads;
  const int32_t n = batch * (qn * hd + hd + qn * (hd + 2)) + 2 * kWaves * qn * (hd + 2);
  return (n + 63) / 64 * 64;
}
// Batch-1 GEMV tiles stage the first weight chunk of every wave in LDS (8 KB per wave).
constexpr int32_t kPrefetchFloats = kWaves * 2048;
AMK_HD int32_t lds_prefetch_floats(int32_t batch) { return batch == 1 ? kPrefetchFloats : 0; }
// LDS of the megakernel: [xs or attention scratch][red: kRedFloats][prefetch][ys]
AMK_HD int32_t lds_bytes_for(int32_t batch, int32_t hidden, int32_t qdim, int32_t ffn,
                             int32_t qpg, int32_t hd, int32_t max_tile_rows) {
  int32_t a = lds_xs_floats(batch, hidden, qdim, ffn);
  int32_t b = lds_attn_floats(batch, qpg, hd);
  int32_t region = a > b ? a : b;
  return 4 * (region + kRedFloats + lds_prefetch_floats(batch) + batch * max_tile_rows);
}
}  // namespace amk
