// Runtime behind the C ABI: model creation (weight repacking, schedule build/validation, device
// tables), KV caches, and the per-step launch of the megakernel or the unfused ablation.
#include <hip/hip_runtime.h>

#include <unistd.h>

#include <algorithm>
#include <cmath>
#include <cstdio>
#include <cstdlib>
#include <cstring>
#include <filesystem>
#include <mutex>
#include <new>
#include <stdexcept>
#include <string>
#include <vector>

#include "../kernels/device.h"
#include "../sched/sched_internal.h"
#include "errors.h"

using namespace amk;

// kernels defined in the other translation units
#define AMK_DECL_MK(WT, HD, Q)                                                         \
  extern "C" __global__ void amk_megakernel_w##WT##_h##HD##_q##Q(const DevModel *, StepArgs); \
  extern "C" __global__ void amk_megakernel_w##WT##_h##HD##_q##Q##_b(const DevModel *, StepArgs);
AMK_DECL_MK(0, 64, 1)
AMK_DECL_MK(0, 64, 2)
AMK_DECL_MK(0, 64, 4)
AMK_DECL_MK(0, 128, 1)
AMK_DECL_MK(0, 128, 2)
AMK_DECL_MK(0, 128, 4)
AMK_DECL_MK(1, 64, 1)
AMK_DECL_MK(1, 64, 2)
AMK_DECL_MK(1, 64, 4)
AMK_DECL_MK(1, 128, 1)
AMK_DECL_MK(1, 128, 2)
AMK_DECL_MK(1, 128, 4)
AMK_DECL_MK(2, 64, 1)
AMK_DECL_MK(2, 64, 2)
AMK_DECL_MK(2, 64, 4)
AMK_DECL_MK(2, 128, 1)
AMK_DECL_MK(2, 128, 2)
AMK_DECL_MK(2, 128, 4)
extern "C" __global__ void amk_uf_embed(const DevModel *, StepArgs);
extern "C" __global__ void amk_uf_rmsnorm(const DevModel *, const float *, const uint16_t *, float *);
#define AMK_DECL_UG(WT, MODE)                                                                  \
  extern "C" __global__ void amk_uf_gemv_w##WT##_m##MODE(const DevModel *, StepArgs, const void *, \
                                                         const float *, int, int, const float *,  \
                                                         float *, const float *, float *);
AMK_DECL_UG(0, 0)
AMK_DECL_UG(0, 1)
AMK_DECL_UG(0, 2)
AMK_DECL_UG(1, 0)
AMK_DECL_UG(1, 1)
AMK_DECL_UG(1, 2)
AMK_DECL_UG(2, 0)
AMK_DECL_UG(2, 1)
AMK_DECL_UG(2, 2)
extern "C" __global__ void amk_uf_rope_kv(const DevModel *, StepArgs, int);
#define AMK_DECL_UA(HD, Q) extern "C" __global__ void amk_uf_attn_h##HD##_q##Q(const DevModel *, StepArgs, int);
AMK_DECL_UA(64, 1)
AMK_DECL_UA(64, 2)
AMK_DECL_UA(64, 4)
AMK_DECL_UA(128, 1)
AMK_DECL_UA(128, 2)
AMK_DECL_UA(128, 4)
extern "C" __global__ void amk_uf_combine(const DevModel *, int);
extern "C" __global__ void amk_uf_swiglu(const DevModel *, int, int);
extern "C" __global__ void amk_uf_argmax(const DevModel *, StepArgs, int);

// row gather used for repacking: dst row pairs[i].x <- src row pairs[i].y (4-byte words)
extern "C" __global__ void __launch_bounds__(256)
amk_gather_rows(uint32_t *dst, const uint32_t *src, const int2 *pairs, int n, int row_words) {
  for (int i = blockIdx.x; i < n; i += gridDim.x) {
    const int2 p = pairs[i];
    const uint32_t *s = src + (int64_t)p.y * row_words;
    uint32_t *d = dst + (int64_t)p.x * row_words;
    for (int k = threadIdx.x; k < row_words; k += 256) d[k] = s[k];
  }
}

// int4 matrices: nibble order within each 32-bit word, from the interface's (byte j: inputs 2j in
// the low and 2j + 1 in the high nibble, so input e at bits 4e) to the kernels' (byte j: input j in
// the low and j + 4 in the high nibble), where one mask or a shift and a mask yield four inputs as
// the high nibbles of four bytes
extern "C" __global__ void __launch_bounds__(256) amk_int4_reorder(uint32_t *w, size_t n) {
  for (size_t i = (size_t)blockIdx.x * 256 + threadIdx.x; i < n; i += (size_t)gridDim.x * 256) {
    const uint32_t v = w[i];
    uint32_t o = 0;
#pragma unroll
    for (int e = 0; e < 8; ++e) o |= ((v >> (4 * e)) & 0xFu) << (8 * (e & 3) + 4 * (e >> 2));
    w[i] = o;
  }
}

// tile-major copy of a row-major matrix [rows][K] for the batched matrix-core GEMV (layout in
// weight_tiled_bytes): one thread per lane piece of lb bytes (8 inputs), zeros past the matrix
extern "C" __global__ void __launch_bounds__(256)
amk_tile_rows(uint8_t *dst, const uint8_t *src, int rows, int K, int lb) {
  const int S = (K + 31) / 32;
  const size_t row_bytes = (size_t)K * lb / 8, n = (size_t)((rows + 15) / 16) * S * 64;
  for (size_t i = (size_t)blockIdx.x * 256 + threadIdx.x; i < n; i += (size_t)gridDim.x * 256) {
    const int l = (int)(i % 64), t = (int)((i / 64) % S), g = (int)(i / 64 / S);
    const int r = 16 * g + (l & 15);
    const size_t b0 = (size_t)(32 * t + 8 * (l >> 4)) * lb / 8;  // byte of input 32 t + 8 q
    uint8_t *d = dst + i * lb;
    for (int j = 0; j < lb; ++j)
      d[j] = (r < rows && b0 + j < row_bytes) ? src[(size_t)r * row_bytes + b0 + j] : (uint8_t)0;
  }
}

// zero n 32-bit words: used instead of a memset node where the caller may be capturing a graph
extern "C" __global__ void __launch_bounds__(256) amk_zero_words(uint32_t *p, size_t n) {
  for (size_t i = (size_t)blockIdx.x * 256 + threadIdx.x; i < n; i += (size_t)gridDim.x * 256) p[i] = 0u;
}

namespace {

constexpr int kUfRowsPerBlock = 32;  // must match the unfused GEMV kernels
constexpr int kUfThreads = 8 * 64;

struct HipError : std::runtime_error {
  explicit HipError(const std::string &m) : std::runtime_error(m) {}
};

void hip_check(hipError_t e, const char *what) {
  if (e != hipSuccess) throw HipError(std::string(what) + ": " + hipGetErrorString(e));
}

using MkFn = void (*)(const DevModel *, StepArgs);

MkFn pick_megakernel(int wt, int hd, int qmax, bool batched) {
#define AMK_P(WT, HD, Q)                                                                    \
  if (wt == WT && hd == HD && qmax == Q)                                                    \
    return batched ? amk_megakernel_w##WT##_h##HD##_q##Q##_b : amk_megakernel_w##WT##_h##HD##_q##Q;
  AMK_P(0, 64, 1) AMK_P(0, 64, 2) AMK_P(0, 64, 4) AMK_P(0, 128, 1) AMK_P(0, 128, 2) AMK_P(0, 128, 4)
  AMK_P(1, 64, 1) AMK_P(1, 64, 2) AMK_P(1, 64, 4) AMK_P(1, 128, 1) AMK_P(1, 128, 2) AMK_P(1, 128, 4)
  AMK_P(2, 64, 1) AMK_P(2, 64, 2) AMK_P(2, 64, 4) AMK_P(2, 128, 1) AMK_P(2, 128, 2) AMK_P(2, 128, 4)
#undef AMK_P
  return nullptr;
}

using UaFn = void (*)(const DevModel *, StepArgs, int);
UaFn pick_uf_attn(int hd, int qmax) {
#define AMK_P(HD, Q) \
  if (hd == HD && qmax == Q) return amk_uf_attn_h##HD##_q##Q;
  AMK_P(64, 1) AMK_P(64, 2) AMK_P(64, 4) AMK_P(128, 1) AMK_P(128, 2) AMK_P(128, 4)
#undef AMK_P
  return nullptr;
}

using UgFn = void (*)(const DevModel *, StepArgs, const void *, const float *, int, int,
                      const float *, float *, const float *, float *);
UgFn pick_uf_gemv(int wt, int mode) {
  static const UgFn t[3][3] = {{amk_uf_gemv_w0_m0, amk_uf_gemv_w0_m1, amk_uf_gemv_w0_m2},
                               {amk_uf_gemv_w1_m0, amk_uf_gemv_w1_m1, amk_uf_gemv_w1_m2},
                               {amk_uf_gemv_w2_m0, amk_uf_gemv_w2_m1, amk_uf_gemv_w2_m2}};
  return t[wt][mode];
}

int qmax_for(int qpg) { return attn_qmax(qpg); }

// Query heads per pass of the megakernel instance that fits a schedule's attention tasks (a task
// may cover only some of its group's query heads, aux2 / aux3).
int mk_qmax_for(const Schedule &s, int qpg) {
  int task_heads = 1;
  for (const auto &v : s.per_cu)
    for (const Task &t : v)
      if (t.type == T_ATTN) task_heads = std::max(task_heads, t.aux3 ? (int)t.aux3 : qpg);
  return qmax_for(task_heads);
}

// The per-step scratch of a model as one block of device memory. It opens with the state region,
// which must hold zeros before a model's first step (and again after a reset or a schedule
// change): the epoch counter, the dependency flags and the tagged activation slots of batch-1
// instances (whose tags must not match any epoch yet). Plain scratch follows, written before it
// is read within every step. Offsets are 256-byte aligned; an absent buffer has kNone.
constexpr size_t kNone = ~(size_t)0;
struct ScratchPlan {
  size_t ectr = kNone, flags = kNone, ht = kNone, at = kNone, aot = kNone, qt = kNone,
         kvt = kNone, part = kNone;  // state region
  size_t h = kNone, q = kNone, ao = kNone, a = kNone, logits = kNone, amax = kNone, xn = kNone,
         y = kNone, o = kNone;
  size_t state_bytes = 0, total = 0;
};

ScratchPlan plan_scratch(const amk_config &c, int nblk, uint32_t n_tasks, int n_amax) {
  ScratchPlan p;
  size_t off = 0;
  auto take = [&](size_t bytes) {
    if (bytes == 0) return kNone;
    const size_t o = off;
    off += (bytes + 255) & ~(size_t)255;
    return o;
  };
  const size_t L = c.n_layers, d = c.hidden, nq = c.n_heads, nkv = c.n_kv_heads, hd = c.head_dim,
               F = c.ffn, V = c.vocab, B = c.max_batch, qd = nq * hd;
  const size_t qkvr = (size_t)qkv_rows(c.n_heads, c.n_kv_heads, c.head_dim);
  const bool tagged = B == 1;  // batch-1 instances hand activations over as tagged words
  p.ectr = take(4);
  p.flags = take(4 * (size_t)std::max<uint32_t>(1, n_tasks));
  p.ht = take(tagged ? 4 * (2 * L + 1) * d : 0);
  p.at = take(tagged ? 4 * L * F : 0);
  p.aot = take(tagged ? 4 * L * qd : 0);
  p.qt = take(tagged ? 4 * L * qd : 0);
  p.kvt = take(tagged ? 4 * L * 2 * nkv * hd : 0);
  p.part = take(4 * L * B * nq * (size_t)nblk * (hd + 2));
  p.state_bytes = off;
  const size_t kmax = std::max(std::max(d, qd), F);
  p.h = take(4 * (2 * L + 1) * B * d);
  p.q = take(4 * L * B * qd);
  p.ao = take(4 * L * B * qd);
  p.a = take(4 * L * B * F);
  p.logits = take(4 * B * V);
  p.amax = take(8 * (size_t)n_amax * B);
  p.xn = take(4 * B * kmax);
  p.y = take(4 * B * std::max(std::max(qkvr, 2 * F), std::max(V, d)));
  p.o = take(4 * B * qd);
  p.total = off;
  return p;
}

// Point the scratch fields of dm into the block at base, laid out by p.
void carve_scratch(DevModel &dm, uint8_t *base, const ScratchPlan &p) {
  auto at = [&](size_t off) -> uint8_t * { return off == kNone ? nullptr : base + off; };
  dm.ectr = reinterpret_cast<uint32_t *>(at(p.ectr));
  dm.flags = reinterpret_cast<uint32_t *>(at(p.flags));
  dm.ht = reinterpret_cast<uint32_t *>(at(p.ht));
  dm.at = reinterpret_cast<uint32_t *>(at(p.at));
  dm.aot = reinterpret_cast<uint32_t *>(at(p.aot));
  dm.qt = reinterpret_cast<uint32_t *>(at(p.qt));
  dm.kvt = reinterpret_cast<uint32_t *>(at(p.kvt));
  dm.part = reinterpret_cast<float *>(at(p.part));
  dm.h = reinterpret_cast<float *>(at(p.h));
  dm.q = reinterpret_cast<float *>(at(p.q));
  dm.ao = reinterpret_cast<float *>(at(p.ao));
  dm.a = reinterpret_cast<float *>(at(p.a));
  dm.logits = reinterpret_cast<float *>(at(p.logits));
  dm.amax = reinterpret_cast<float2 *>(at(p.amax));
  dm.xn = reinterpret_cast<float *>(at(p.xn));
  dm.y = reinterpret_cast<float *>(at(p.y));
  dm.o = reinterpret_cast<float *>(at(p.o));
}

// ---- cache of built schedules ------------------------------------------------------------
// Model creation without a caller's schedule keeps the schedule it builds on disk, keyed by all
// the builder reads (config, batch, CU count, the device's architecture, the cost model the search
// ranks with) and the build of the schedule layer; the next creation with the same key reads it
// back instead of searching again. A cached blob is parsed and validated like a caller's; one that
// fails, or was built for another configuration, is rebuilt and replaced. Directory:
// $AMK_CACHE_DIR, else ~/.cache/amk; AMK_CACHE_DIR=off disables the cache.
uint64_t fnv1a(const void *p, size_t n, uint64_t h = 1469598103934665603ull) {
  const uint8_t *b = static_cast<const uint8_t *>(p);
  for (size_t i = 0; i < n; ++i) h = (h ^ b[i]) * 1099511628211ull;
  return h;
}

std::string cache_dir() {
  const char *env = std::getenv("AMK_CACHE_DIR");
  if (env && std::strcmp(env, "off") == 0) return "";
  if (env && *env) return env;
  const char *home = std::getenv("HOME");
  return home && *home ? std::string(home) + "/.cache/amk" : "";
}

std::string cache_path(const amk_config &cfg, int n_cu, const char *arch) {
  const std::string dir = cache_dir();
  if (dir.empty()) return "";
  BlobConfig bc;
  std::memcpy(&bc, &cfg, sizeof bc);
  const amk_cost_model cm = default_cost_model(n_cu);
  uint64_t h = fnv1a(&bc, sizeof bc);
  h = fnv1a(&n_cu, sizeof n_cu, h);
  h = fnv1a(arch, std::strlen(arch), h);
  h = fnv1a(&cm, sizeof cm, h);
  const uint32_t version = kBlobVersion;
  h = fnv1a(&version, sizeof version, h);
  const char *stamp = schedule_build_stamp();
  h = fnv1a(stamp, std::strlen(stamp), h);
  char name[64];
  std::snprintf(name, sizeof name, "/schedule-%016llx.amks", (unsigned long long)h);
  return dir + name;
}

bool read_file(const std::string &path, std::vector<uint8_t> *out) {
  FILE *f = std::fopen(path.c_str(), "rb");
  if (!f) return false;
  out->clear();
  uint8_t buf[1 << 16];
  size_t n;
  while ((n = std::fread(buf, 1, sizeof buf, f)) > 0) out->insert(out->end(), buf, buf + n);
  std::fclose(f);
  return !out->empty();
}

// write by rename, so a reader never sees a partial file; failures leave no cache entry
void write_file(const std::string &path, const std::vector<uint8_t> &data) {
  std::error_code ec;
  std::filesystem::create_directories(std::filesystem::path(path).parent_path(), ec);
  const std::string tmp = path + ".tmp" + std::to_string((unsigned long)getpid());
  FILE *f = std::fopen(tmp.c_str(), "wb");
  if (!f) return;
  const bool ok = std::fwrite(data.data(), 1, data.size(), f) == data.size();
  if (std::fclose(f) != 0 || !ok || std::rename(tmp.c_str(), path.c_str()) != 0) std::remove(tmp.c_str());
}

// ---- scratch of the entry point that allocates nothing (amk_decode_steps_noalloc) ----------
// A file-scope device array, one copy per GPU the library runs on, held until the process ends.
// In host code its name is only a stand-in: kernels and copies use the address that
// hipGetSymbolAddress returns for the current device (static_scratch_base).
constexpr size_t kStaticScratchBytes = (size_t)AMK_STATIC_SCRATCH_BYTES;
static __device__ __align__(256) uint8_t scratch[kStaticScratchBytes];

constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
uint8_t *g_scratch_base[kMaxDevices] = {};

// Device address of `scratch` on device `dev`, which must be current. Looked up once per device
// (at the first model creation there) and kept.
uint8_t *static_scratch_base(int dev) {
  if (dev < 0 || dev >= kMaxDevices) throw std::runtime_error("device index beyond the scratch table");
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (!g_scratch_base[dev]) {
    void *p = nullptr;
    const hipError_t e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess || !p)
      throw std::runtime_error(std::string("hipGetSymbolAddress(scratch): ") + hipGetErrorString(e));
    g_scratch_base[dev] = static_cast<uint8_t *>(p);
  }
  return g_scratch_base[dev];
}

}  // namespace

struct amk_model {
  amk_config cfg{};
  int32_t path = 0;
  int device = 0;
  int n_cu = 0;
  Schedule sched;
  std::vector<uint8_t> blob;
  std::vector<void *> allocs;
  DevModel dm{};
  DevModel *d_dm = nullptr;
  // prompt processing (amk_prefill): the model's weights with scratch for kMaxBatch columns,
  // created by the first call
  DevModel dm_pf{};
  DevModel *d_dm_pf = nullptr;
  int32_t *pf_next = nullptr;  // device int32 [kMaxBatch]
  std::vector<DevLayer> layers;
  ScratchPlan plan;
  uint8_t *scratch = nullptr;  // the model's own per-step scratch block (plan.total bytes)
  // the same descriptor with its scratch in this device's static array (amk_decode_steps_noalloc);
  // null when plan.total exceeds the array
  DevModel dm_static{};
  DevModel *d_dm_static = nullptr;
  uint8_t *static_base = nullptr;
  uint32_t lds_bytes = 0;
  uint32_t uf_attn_lds = 0;
  uint64_t weight_bytes = 0;
  int n_lm_uf = 0;
  MkFn mk = nullptr;
  int mk_qmax = 0;  // query heads per attention pass of the megakernel instance
  UaFn uf_attn = nullptr;
  uint32_t *h_err = nullptr;  // pinned copy of the device error words
  hipEvent_t err_event = nullptr;
  bool err_pending = false;

  template <typename T>
  T *dalloc(size_t count) {
    void *p = nullptr;
    size_t bytes = count * sizeof(T);
    if (bytes == 0) bytes = 16;
    hipError_t e = hipMalloc(&p, bytes);
    if (e != hipSuccess) throw std::bad_alloc();
    allocs.push_back(p);
    return static_cast<T *>(p);
  }
};

struct amk_kv {
  amk_model *m = nullptr;
  void *data = nullptr;
  bool owned = false;
  int32_t batch = 0, max_seq = 0;
  size_t bytes = 0;
};

namespace {

void free_model(amk_model *m) {
  if (!m) return;
  for (void *p : m->allocs) (void)hipFree(p);
  if (m->h_err) (void)hipHostFree(m->h_err);
  if (m->err_event) (void)hipEventDestroy(m->err_event);
  delete m;
}

void gather(amk_model *m, void *dst, const void *src, const std::vector<int2> &pairs,
            size_t row_bytes, hipStream_t st) {
  if (pairs.empty()) return;
  if (row_bytes % 4) throw std::runtime_error("row size not a multiple of 4 bytes");
  int2 *d_pairs = nullptr;
  hip_check(hipMalloc(&d_pairs, pairs.size() * sizeof(int2)), "hipMalloc");
  hipError_t e = hipMemcpyAsync(d_pairs, pairs.data(), pairs.size() * sizeof(int2),
                                hipMemcpyHostToDevice, st);
  if (e == hipSuccess) {
    int blocks = (int)std::min<size_t>(pairs.size(), 65535);
    hipLaunchKernelGGL(amk_gather_rows, dim3(blocks), dim3(256), 0, st, (uint32_t *)dst,
                       (const uint32_t *)src, (const int2 *)d_pairs, (int)pairs.size(),
                       (int)(row_bytes / 4));
    e = hipGetLastError();
  }
  if (e == hipSuccess) e = hipStreamSynchronize(st);
  (void)hipFree(d_pairs);
  hip_check(e, "repack");
  (void)m;
}

// device buffer for the duration of a scope (repack staging)
struct DeviceTemp {
  void *p = nullptr;
  explicit DeviceTemp(size_t bytes) {
    if (bytes) hip_check(hipMalloc(&p, bytes), "hipMalloc");
  }
  ~DeviceTemp() {
    if (p) (void)hipFree(p);
  }
  DeviceTemp(const DeviceTemp &) = delete;
  DeviceTemp &operator=(const DeviceTemp &) = delete;
};

void copy_d2d(void *dst, const void *src, size_t bytes, hipStream_t st) {
  hip_check(hipMemcpyAsync(dst, src, bytes, hipMemcpyDeviceToDevice, st), "hipMemcpyAsync");
}

amk_status map_device_error(uint32_t code, uint32_t task, uint32_t detail) {
  if (code == ERR_TIMEOUT)
    return set_error(AMK_E_DEVICE_TIMEOUT, "device dependency wait timed out (task " +
                                               std::to_string(task) + " waiting on task " +
                                               std::to_string(detail) + ")");
  if (code == ERR_TOKEN)
    return set_error(AMK_E_DEVICE_FAULT,
                     "token id out of range: " + std::to_string((int32_t)detail));
  return set_error(AMK_E_DEVICE_FAULT, "device error code " + std::to_string(code));
}

void zero_async(void *p, size_t bytes, hipStream_t st) {
  const size_t n = bytes / 4;
  const unsigned blocks = (unsigned)std::min<size_t>(1024, (n + 255) / 256);
  if (n) hipLaunchKernelGGL(amk_zero_words, dim3(blocks), dim3(256), 0, st, static_cast<uint32_t *>(p), n);
}

// id of the schedule's argmax task (validated: exactly one, and every task precedes it)
uint32_t argmax_of(const Schedule &s) {
  for (const auto &v : s.per_cu)
    for (const Task &t : v)
      if (t.type == T_ARGMAX) return t.id;
  return 0;
}

// Zero the state region of the model's scratch (epoch counter, flags, tagged slots): the step
// after this starts at epoch 1 and no stale word can carry its tag.
void zero_state(amk_model *m, hipStream_t st) { zero_async(m->scratch, m->plan.state_bytes, st); }

// upload the host copy of the model's device descriptor (and of its static-scratch twin)
void upload_dm(amk_model *m) {
  hip_check(hipMemcpy(m->d_dm, &m->dm, sizeof(DevModel), hipMemcpyHostToDevice), "hipMemcpy");
  if (m->d_dm_static) {
    m->dm_static = m->dm;
    carve_scratch(m->dm_static, m->static_base, m->plan);
    hip_check(hipMemcpy(m->d_dm_static, &m->dm_static, sizeof(DevModel), hipMemcpyHostToDevice),
              "hipMemcpy");
  }
}

// reset device error words, flags, tagged slots and the epoch after a device-side failure
void reset_device_state(amk_model *m, hipStream_t st) {
  (void)hipMemsetAsync(m->dm.err, 0, 4 * sizeof(uint32_t), st);
  zero_state(m, st);
  (void)hipStreamSynchronize(st);
  m->err_pending = false;
}

}  // namespace

extern "C" amk_status amk_model_create(const amk_config *cfg, const amk_weights *w, int32_t path,
                                       const void *schedule_blob, size_t blob_bytes, void *stream,
                                       amk_model **out) {
  amk_model *m = nullptr;
  try {
    if (!cfg || !w || !out) return set_error(AMK_E_INVALID, "amk_model_create: null argument");
    *out = nullptr;
    std::string e;
    if (!config_ok(*cfg, &e)) return set_error(AMK_E_INVALID, e);
    if (path != AMK_PATH_MEGAKERNEL && path != AMK_PATH_UNFUSED)
      return set_error(AMK_E_INVALID, "amk_model_create: unknown path");
    if (cfg->head_dim != 64 && cfg->head_dim != 128)
      return set_error(AMK_E_UNSUPPORTED, "head_dim must be 64 or 128");
    if (cfg->wtype == AMK_WT_INT8 && (cfg->hidden % 16 || cfg->ffn % 16))
      return set_error(AMK_E_UNSUPPORTED, "int8 weights need hidden and ffn multiples of 16");
    if (!w->embed || !w->final_norm || !w->layers || (!cfg->tied_lm_head && !w->lm_head))
      return set_error(AMK_E_INVALID, "amk_model_create: missing weight pointer");
    const bool i8 = cfg->wtype == AMK_WT_INT8, i4 = cfg->wtype == AMK_WT_INT4;
    for (int l = 0; l < cfg->n_layers; ++l) {
      const amk_layer_weights &lw = w->layers[l];
      if (!lw.wq || !lw.wk || !lw.wv || !lw.wo || !lw.wg || !lw.wu || !lw.wd || !lw.attn_norm ||
          !lw.mlp_norm)
        return set_error(AMK_E_INVALID, "amk_model_create: missing layer weight pointer");
      if ((i8 || i4) && (!lw.sq || !lw.sk || !lw.sv || !lw.so || !lw.sg || !lw.su || !lw.sd))
        return set_error(AMK_E_INVALID, "amk_model_create: int8/int4 weights need scales");
    }
    if ((i8 || i4) && !cfg->tied_lm_head && !w->lm_head_scale)
      return set_error(AMK_E_INVALID, "amk_model_create: int8/int4 LM head needs scales");

    m = new amk_model();
    m->cfg = *cfg;
    m->path = path;
    hipStream_t st = static_cast<hipStream_t>(stream);
    hip_check(hipGetDevice(&m->device), "hipGetDevice");
    hipDeviceProp_t prop;
    hip_check(hipGetDeviceProperties(&prop, m->device), "hipGetDeviceProperties");
    m->n_cu = prop.multiProcessorCount;
    int clock_khz = 0;
    if (hipDeviceGetAttribute(&clock_khz, hipDeviceAttributeWallClockRate, m->device) != hipSuccess ||
        clock_khz <= 0)
      clock_khz = 100000;

    // ---- schedule -------------------------------------------------------------------------
    if (schedule_blob) {
      if (!parse(schedule_blob, blob_bytes, &m->sched, &e)) {
        free_model(m);
        return set_error(AMK_E_SCHEDULE_REJECTED, e);
      }
      m->blob.assign((const uint8_t *)schedule_blob, (const uint8_t *)schedule_blob + blob_bytes);
    } else {
      // a cached build of this configuration, if one validates; else build (and cache) it
      const std::string cpath = cache_path(*cfg, m->n_cu, prop.gcnArchName);
      bool cached = false;
      if (!cpath.empty() && read_file(cpath, &m->blob)) {
        Schedule cs;
        std::string ce, crep;
        if (parse(m->blob.data(), m->blob.size(), &cs, &ce) && validate_schedule(cs, &crep) &&
            std::memcmp(&cs.hdr.cfg, cfg, sizeof(BlobConfig)) == 0 &&
            (int32_t)cs.hdr.batch == cfg->max_batch && (int)cs.hdr.n_cu == m->n_cu) {
          m->sched = std::move(cs);
          cached = true;
        }
      }
      if (!cached) {
        void *b = nullptr;
        size_t n = 0;
        amk_status s2 = amk_schedule_build(cfg, cfg->max_batch, m->n_cu, nullptr, nullptr, &b, &n);
        if (s2 != AMK_OK) {
          free_model(m);
          return s2;
        }
        m->blob.assign((uint8_t *)b, (uint8_t *)b + n);
        amk_blob_free(b);
        parse(m->blob.data(), m->blob.size(), &m->sched, &e);
        if (!cpath.empty()) write_file(cpath, m->blob);
      }
    }
    std::string rep;
    if (!validate_schedule(m->sched, &rep)) {
      free_model(m);
      return set_error(AMK_E_SCHEDULE_REJECTED, rep);
    }
    const BlobHeader &h = m->sched.hdr;
    if (std::memcmp(&h.cfg, cfg, sizeof(BlobConfig)) != 0) {
      free_model(m);
      return set_error(AMK_E_SCHEDULE_REJECTED, "schedule was built for a different config");
    }
    if ((int32_t)h.batch != cfg->max_batch) {
      free_model(m);
      return set_error(AMK_E_SCHEDULE_REJECTED, "schedule batch differs from max_batch");
    }
    if (path == AMK_PATH_MEGAKERNEL && (int)h.n_cu != m->n_cu) {
      free_model(m);
      return set_error(AMK_E_SCHEDULE_REJECTED,
                       "schedule targets " + std::to_string(h.n_cu) + " CUs, device has " +
                           std::to_string(m->n_cu));
    }
    m->lds_bytes = h.lds_bytes;
    if (m->lds_bytes > (uint32_t)prop.sharedMemPerBlock && prop.sharedMemPerBlock > 0) {
      free_model(m);
      return set_error(AMK_E_SCHEDULE_REJECTED, "schedule LDS exceeds the device limit");
    }

    // ---- weights --------------------------------------------------------------------------
    const int L = cfg->n_layers, d = cfg->hidden, nq = cfg->n_heads, nkv = cfg->n_kv_heads,
              hd = cfg->head_dim, F = cfg->ffn, V = cfg->vocab, B = cfg->max_batch;
    const int qd = nq * hd, qkvr = qkv_rows(nq, nkv, hd);
    // bytes of a weight row of K inputs, and of its scales (one per row, or one per group)
    auto row_b = [&](int K) -> size_t { return i4 ? (size_t)K / 2 : (size_t)K * (i8 ? 1 : 2); };
    auto scale_b = [&](int K) -> size_t { return i4 ? (size_t)(K / cfg->group_size) * 4 : 4; };
    auto reorder = [&](void *w, size_t bytes) {
      if (!i4) return;
      const size_t n = bytes / 4;
      hipLaunchKernelGGL(amk_int4_reorder, dim3((unsigned)std::min<size_t>((n + 255) / 256, 65535)),
                         dim3(256), 0, st, (uint32_t *)w, n);
      hip_check(hipGetLastError(), "amk_int4_reorder");
    };
    // Batched models keep the layer matrices (and an untied LM head) tile-major: each matrix is
    // assembled row-major in `stage`, then tiled into its own allocation.
    const bool tiled = B > 1;
    const int wbits = i4 ? 4 : (i8 ? 8 : 16);
    size_t stage_bytes = 0;
    if (tiled) {
      const size_t mx = std::max(std::max((size_t)qkvr * row_b(d), (size_t)2 * F * row_b(d)),
                                 std::max((size_t)d * row_b(qd), (size_t)d * row_b(F)));
      stage_bytes = cfg->tied_lm_head ? mx : std::max(mx, (size_t)V * row_b(d));
    }
    DeviceTemp stage(stage_bytes);
    // where a matrix of `rows` x K is assembled, and its final home
    auto home = [&](int rows, int K) -> void * {
      return m->dalloc<uint8_t>(tiled ? (size_t)weight_tiled_bytes(rows, K, wbits) : (size_t)rows * row_b(K));
    };
    auto build = [&](void *dst) -> void * { return tiled ? stage.p : dst; };
    auto finish = [&](void *dst, int rows, int K) {
      if (!tiled) return;
      const size_t n = (size_t)((rows + 15) / 16) * ((K + 31) / 32) * 64;
      hipLaunchKernelGGL(amk_tile_rows, dim3((unsigned)std::min<size_t>((n + 255) / 256, 65535)),
                         dim3(256), 0, st, (uint8_t *)dst, (const uint8_t *)stage.p, rows, K,
                         weight_lane_bytes(wbits));
      hip_check(hipGetLastError(), "amk_tile_rows");
      hip_check(hipStreamSynchronize(st), "hipStreamSynchronize");  // `stage` is reused
    };
    DevModel &dm = m->dm;
    dm.L = L; dm.d = d; dm.nq = nq; dm.nkv = nkv; dm.hd = hd; dm.F = F; dm.V = V;
    dm.qkvr = qkvr; dm.qd = qd; dm.qpg = nq / nkv;
    dm.wtype = cfg->wtype; dm.tied = cfg->tied_lm_head; dm.max_batch = B; dm.max_seq = cfg->max_seq;
    dm.gs = cfg->group_size;
    dm.tiled = tiled;
    dm.nblk = (int32_t)h.attn_blocks;
    dm.n_lm = (int32_t)h.n_lm_tiles;
    dm.n_tasks = h.n_tasks;
    dm.trace = nullptr;
    dm.eps = cfg->rms_eps;
    dm.attn_scale = (float)(1.0 / std::sqrt((double)hd));
    m->layers.resize(L);
    m->weight_bytes = 0;
    for (int l = 0; l < L; ++l) {
      const amk_layer_weights &lw = w->layers[l];
      DevLayer &dl = m->layers[l];
      void *qkv = home(qkvr, d), *gu = home(2 * F, d), *o = home(d, qd), *dn = home(d, F);
      std::vector<int2> pq, pk, pv, pg, pu;
      for (int r = 0; r < qkvr; ++r) {
        QkvRow q = qkv_decode(r, nq, nkv, hd);
        int2 pr = make_int2(r, q.head * hd + q.dim);
        (q.kind == KIND_Q ? pq : (q.kind == KIND_K ? pk : pv)).push_back(pr);
      }
      for (int i = 0; i < F; ++i) {
        pg.push_back(make_int2(2 * i, i));
        pu.push_back(make_int2(2 * i + 1, i));
      }
      void *w_ = build(qkv);
      gather(m, w_, lw.wq, pq, row_b(d), st);
      gather(m, w_, lw.wk, pk, row_b(d), st);
      gather(m, w_, lw.wv, pv, row_b(d), st);
      reorder(w_, (size_t)qkvr * row_b(d));
      finish(qkv, qkvr, d);
      w_ = build(gu);
      gather(m, w_, lw.wg, pg, row_b(d), st);
      gather(m, w_, lw.wu, pu, row_b(d), st);
      reorder(w_, (size_t)2 * F * row_b(d));
      finish(gu, 2 * F, d);
      w_ = build(o);
      copy_d2d(w_, lw.wo, (size_t)d * row_b(qd), st);
      reorder(w_, (size_t)d * row_b(qd));
      finish(o, d, qd);
      w_ = build(dn);
      copy_d2d(w_, lw.wd, (size_t)d * row_b(F), st);
      reorder(w_, (size_t)d * row_b(F));
      finish(dn, d, F);
      dl.qkv = qkv; dl.gu = gu; dl.o = o; dl.dn = dn;
      dl.s_qkv = dl.s_gu = dl.s_o = dl.s_dn = nullptr;
      if (i8 || i4) {
        float *sqkv = (float *)m->dalloc<uint8_t>(qkvr * scale_b(d));
        float *sgu = (float *)m->dalloc<uint8_t>(2 * F * scale_b(d));
        float *so = (float *)m->dalloc<uint8_t>(d * scale_b(qd));
        float *sdn = (float *)m->dalloc<uint8_t>(d * scale_b(F));
        gather(m, sqkv, lw.sq, pq, scale_b(d), st);
        gather(m, sqkv, lw.sk, pk, scale_b(d), st);
        gather(m, sqkv, lw.sv, pv, scale_b(d), st);
        gather(m, sgu, lw.sg, pg, scale_b(d), st);
        gather(m, sgu, lw.su, pu, scale_b(d), st);
        copy_d2d(so, lw.so, (size_t)d * scale_b(qd), st);
        copy_d2d(sdn, lw.sd, (size_t)d * scale_b(F), st);
        dl.s_qkv = sqkv; dl.s_gu = sgu; dl.s_o = so; dl.s_dn = sdn;
        m->weight_bytes += (uint64_t)(qkvr + 2 * F) * scale_b(d) + (uint64_t)d * (scale_b(qd) + scale_b(F));
      }
      uint16_t *an = m->dalloc<uint16_t>(d), *mn = m->dalloc<uint16_t>(d);
      copy_d2d(an, lw.attn_norm, (size_t)d * 2, st);
      copy_d2d(mn, lw.mlp_norm, (size_t)d * 2, st);
      dl.attn_norm = an;
      dl.mlp_norm = mn;
      m->weight_bytes += (uint64_t)(qkvr + 2 * F) * row_b(d) + (uint64_t)d * (row_b(qd) + row_b(F)) + 4ull * d;
    }
    uint16_t *emb = m->dalloc<uint16_t>((size_t)V * d);
    copy_d2d(emb, w->embed, (size_t)V * d * 2, st);
    uint16_t *fn = m->dalloc<uint16_t>(d);
    copy_d2d(fn, w->final_norm, (size_t)d * 2, st);
    dm.embed = emb;
    dm.final_norm = fn;
    m->weight_bytes += 2ull * d;
    if (cfg->tied_lm_head) {
      dm.lm = emb;
      dm.lm_scale = nullptr;
      m->weight_bytes += 2ull * V * d;
    } else {
      void *lm = home(V, d);
      void *w_ = build(lm);
      copy_d2d(w_, w->lm_head, (size_t)V * row_b(d), st);
      reorder(w_, (size_t)V * row_b(d));
      finish(lm, V, d);
      dm.lm = lm;
      m->weight_bytes += (uint64_t)V * row_b(d);
      if (i8 || i4) {
        float *ls = (float *)m->dalloc<uint8_t>((size_t)V * scale_b(d));
        copy_d2d(ls, w->lm_head_scale, (size_t)V * scale_b(d), st);
        dm.lm_scale = ls;
        m->weight_bytes += (uint64_t)V * scale_b(d);
      }
    }
    DevLayer *d_layers = m->dalloc<DevLayer>(L);
    hip_check(hipMemcpyAsync(d_layers, m->layers.data(), sizeof(DevLayer) * L,
                             hipMemcpyHostToDevice, st), "hipMemcpyAsync");
    dm.layers = d_layers;

    // ---- tables and scratch ----------------------------------------------------------------
    std::vector<float2> rope((size_t)cfg->max_seq * (hd / 2));
    for (int p = 0; p < cfg->max_seq; ++p)
      for (int j = 0; j < hd / 2; ++j) {
        const double ang = (double)p * std::pow((double)cfg->rope_theta, -2.0 * j / hd);
        rope[(size_t)p * (hd / 2) + j] = make_float2((float)std::cos(ang), (float)std::sin(ang));
      }
    float2 *d_rope = m->dalloc<float2>(rope.size());
    hip_check(hipMemcpyAsync(d_rope, rope.data(), rope.size() * sizeof(float2),
                             hipMemcpyHostToDevice, st), "hipMemcpyAsync");
    dm.rope = d_rope;
    m->n_lm_uf = (V + kUfRowsPerBlock - 1) / kUfRowsPerBlock;
    m->plan = plan_scratch(*cfg, dm.nblk, h.n_tasks, std::max<int>(m->n_lm_uf, dm.n_lm));
    m->scratch = m->dalloc<uint8_t>(m->plan.total);
    carve_scratch(dm, m->scratch, m->plan);
    dm.err = m->dalloc<uint32_t>(4);
    const int kmax = std::max(std::max(d, qd), F);
    hip_check(hipMemsetAsync(dm.err, 0, 16, st), "hipMemsetAsync");
    zero_state(m, st);
    // task tables
    std::vector<uint32_t> offs(h.n_cu + 1);
    std::vector<Task> tasks;
    tasks.reserve(h.n_tasks);
    for (uint32_t c = 0; c < h.n_cu; ++c) {
      offs[c] = (uint32_t)tasks.size();
      for (const Task &t : m->sched.per_cu[c]) tasks.push_back(t);
    }
    offs[h.n_cu] = (uint32_t)tasks.size();
    Task *d_tasks = m->dalloc<Task>(tasks.size());
    uint32_t *d_offs = m->dalloc<uint32_t>(offs.size());
    hip_check(hipMemcpyAsync(d_tasks, tasks.data(), tasks.size() * sizeof(Task),
                             hipMemcpyHostToDevice, st), "hipMemcpyAsync");
    hip_check(hipMemcpyAsync(d_offs, offs.data(), offs.size() * 4, hipMemcpyHostToDevice, st),
              "hipMemcpyAsync");
    dm.tasks = d_tasks;
    dm.offsets = d_offs;
    dm.argmax_id = argmax_of(m->sched);
    double wd_ms = 2000.0;
    if (const char *env = std::getenv("AMK_WATCHDOG_MS")) wd_ms = std::atof(env);
    dm.timeout_ticks = (uint64_t)(wd_ms * clock_khz);
    m->d_dm = m->dalloc<DevModel>(1);
    // the static scratch array of this device: looked up here, once per device
    m->static_base = static_scratch_base(m->device);
    if (m->plan.total <= kStaticScratchBytes) m->d_dm_static = m->dalloc<DevModel>(1);
    hip_check(hipStreamSynchronize(st), "hipStreamSynchronize");
    upload_dm(m);

    // the megakernel instance fits the schedule's attention tasks (a task may cover only some of
    // its group's query heads); the operator kernels take whole groups
    const int qmax = qmax_for(dm.qpg);
    m->mk_qmax = mk_qmax_for(m->sched, dm.qpg);
    m->mk = pick_megakernel(cfg->wtype, hd, m->mk_qmax, B > 1);
    m->uf_attn = pick_uf_attn(hd, qmax);
    if (!m->mk || !m->uf_attn) throw std::runtime_error("no kernel instance for this shape");
    // the operator kernels may run prompt chunks of kMaxBatch columns
    m->uf_attn_lds = 4u * (64 * 8 + (uint32_t)lds_attn_floats(kMaxBatch, qmax, hd));
    if (path == AMK_PATH_MEGAKERNEL) {
      hip_check(hipFuncSetAttribute((const void *)m->mk, hipFuncAttributeMaxDynamicSharedMemorySize,
                                    (int)m->lds_bytes), "hipFuncSetAttribute");
      int per_cu = 0;
      hip_check(hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, (const void *)m->mk, kThreads,
                                                             m->lds_bytes), "occupancy");
      if (per_cu < 1) throw std::runtime_error("megakernel workgroup does not fit on a CU");
    } else {
      // a step may run any batch up to max_batch: allow the larger of the two GEMV layouts
      const uint32_t gl = 4u * (64 * 8 + kMaxBatch * kUfRowsPerBlock +
                                (uint32_t)std::max<int>(kmax, B > 1 ? kMfmaRedFloats : 0));
      for (int wt = 0; wt < 3; ++wt)
        for (int mode = 0; mode < 3; ++mode)
          hip_check(hipFuncSetAttribute((const void *)pick_uf_gemv(wt, mode),
                                        hipFuncAttributeMaxDynamicSharedMemorySize, (int)gl),
                    "hipFuncSetAttribute");
      hip_check(hipFuncSetAttribute((const void *)m->uf_attn,
                                    hipFuncAttributeMaxDynamicSharedMemorySize, (int)m->uf_attn_lds),
                "hipFuncSetAttribute");
    }
    hip_check(hipHostMalloc((void **)&m->h_err, 16, hipHostMallocDefault), "hipHostMalloc");
    std::memset(m->h_err, 0, 16);
    hip_check(hipEventCreateWithFlags(&m->err_event, hipEventDisableTiming), "hipEventCreate");
    hip_check(hipStreamSynchronize(st), "hipStreamSynchronize");
    *out = m;
    clear_error();
    return AMK_OK;
  } catch (const std::bad_alloc &) {
    free_model(m);
    return set_error(AMK_E_OOM, "amk_model_create: allocation failed");
  } catch (const HipError &ex) {
    free_model(m);
    return set_error(AMK_E_HIP, ex.what());
  } catch (const std::exception &ex) {
    free_model(m);
    return set_error(AMK_E_INVALID, std::string("amk_model_create: ") + ex.what());
  }
}

extern "C" amk_status amk_kv_bytes(const amk_model *m, int32_t batch, int32_t max_seq, size_t *bytes) {
  if (!m || !bytes) return set_error(AMK_E_INVALID, "amk_kv_bytes: null argument");
  if (batch < 1 || batch > m->cfg.max_batch) return set_error(AMK_E_INVALID, "amk_kv_bytes: bad batch");
  if (max_seq < 1 || max_seq > m->cfg.max_seq) return set_error(AMK_E_INVALID, "amk_kv_bytes: bad max_seq");
  *bytes = (size_t)m->cfg.n_layers * 2 * batch * m->cfg.n_kv_heads * (size_t)max_seq * m->cfg.head_dim * 2;
  clear_error();
  return AMK_OK;
}

extern "C" amk_status amk_kv_alloc(amk_model *m, int32_t batch, int32_t max_seq, void *d_buf,
                                   size_t buf_bytes, amk_kv **out) {
  AMK_API_BEGIN
  if (!out) return set_error(AMK_E_INVALID, "amk_kv_alloc: null output");
  *out = nullptr;
  size_t need = 0;
  amk_status st = amk_kv_bytes(m, batch, max_seq, &need);
  if (st != AMK_OK) return st;
  amk_kv *kv = new amk_kv();
  kv->m = m;
  kv->batch = batch;
  kv->max_seq = max_seq;
  kv->bytes = need;
  if (d_buf) {
    if (buf_bytes < need) {
      delete kv;
      return set_error(AMK_E_CAPACITY, "amk_kv_alloc: buffer smaller than amk_kv_bytes");
    }
    kv->data = d_buf;
  } else {
    if (hipMalloc(&kv->data, need) != hipSuccess) {
      delete kv;
      return set_error(AMK_E_OOM, "amk_kv_alloc: device allocation failed");
    }
    kv->owned = true;
    if (hipMemset(kv->data, 0, need) != hipSuccess) {
      (void)hipFree(kv->data);
      delete kv;
      return set_error(AMK_E_HIP, "amk_kv_alloc: hipMemset failed");
    }
  }
  *out = kv;
  clear_error();
  return AMK_OK;
  AMK_API_END
}

extern "C" amk_status amk_kv_data(const amk_kv *kv, void **d_ptr) {
  if (!kv || !d_ptr) return set_error(AMK_E_INVALID, "amk_kv_data: null argument");
  *d_ptr = kv->data;
  return AMK_OK;
}

extern "C" amk_status amk_kv_free(amk_kv *kv) {
  if (!kv) return set_error(AMK_E_INVALID, "amk_kv_free: null argument");
  if (kv->owned) (void)hipFree(kv->data);
  delete kv;
  return AMK_OK;
}

// One step as a sequence of operator launches, on the model's scratch (dm, g = its device copy):
// the unfused ablation, and prompt processing.
static void launch_unfused(amk_model *m, const DevModel &dm, const DevModel *g, const StepArgs &s,
                           hipStream_t st) {
  const int B = s.batch, L = dm.L, d = dm.d;
  const int wt = dm.wtype;
  // LDS: the staged input of a batch-1 row-major GEMV and/or the matrix cores' partial tiles (a
  // tile-major model runs those at batch 1 too, except for a tied LM head)
  const int kmx = std::max(std::max(d, dm.qd), dm.F);
  const uint32_t gl = 4u * (64 * 8 + kMaxBatch * kUfRowsPerBlock +
                            (uint32_t)(B > 1 ? kMfmaRedFloats : (dm.tiled ? std::max(kmx, kMfmaRedFloats) : kmx)));
  auto grid = [](int rows) { return dim3((rows + kUfRowsPerBlock - 1) / kUfRowsPerBlock); };
  float *h = dm.h;
  auto hslot = [&](int slot) { return h + (size_t)slot * dm.max_batch * d; };
  hipLaunchKernelGGL(amk_uf_embed, dim3((d + 255) / 256, B), dim3(256), 0, st, g, s);
  for (int l = 0; l < L; ++l) {
    const DevLayer &ly = m->layers[l];
    hipLaunchKernelGGL(amk_uf_rmsnorm, dim3(B), dim3(1024), 0, st, g, (const float *)hslot(2 * l), ly.attn_norm, dm.xn);
    hipLaunchKernelGGL(pick_uf_gemv(wt, 0), grid(dm.qkvr), dim3(kUfThreads), gl, st, g, s, ly.qkv, ly.s_qkv, d, dm.qkvr, (const float *)dm.xn, dm.y, (const float *)nullptr, (float *)nullptr);
    hipLaunchKernelGGL(amk_uf_rope_kv, dim3((dm.qkvr / 2 + 255) / 256, B), dim3(256), 0, st, g, s, l);
    hipLaunchKernelGGL(m->uf_attn, dim3(dm.nkv, dm.nblk), dim3(kThreads), m->uf_attn_lds, st, g, s, l);
    hipLaunchKernelGGL(amk_uf_combine, dim3(dm.nq, B), dim3(128), 0, st, g, l);
    hipLaunchKernelGGL(pick_uf_gemv(wt, 1), grid(d), dim3(kUfThreads), gl, st, g, s, ly.o, ly.s_o, dm.qd, d, (const float *)dm.o, (float *)nullptr, (const float *)hslot(2 * l), hslot(2 * l + 1));
    hipLaunchKernelGGL(amk_uf_rmsnorm, dim3(B), dim3(1024), 0, st, g, (const float *)hslot(2 * l + 1), ly.mlp_norm, dm.xn);
    hipLaunchKernelGGL(pick_uf_gemv(wt, 0), grid(2 * dm.F), dim3(kUfThreads), gl, st, g, s, ly.gu, ly.s_gu, d, 2 * dm.F, (const float *)dm.xn, dm.y, (const float *)nullptr, (float *)nullptr);
    hipLaunchKernelGGL(amk_uf_swiglu, dim3(std::min(1024, (B * dm.F + 255) / 256)), dim3(256), 0, st, g, l, B);
    hipLaunchKernelGGL(pick_uf_gemv(wt, 1), grid(d), dim3(kUfThreads), gl, st, g, s, ly.dn, ly.s_dn, dm.F, d, (const float *)(dm.a + (size_t)l * dm.max_batch * dm.F), (float *)nullptr, (const float *)hslot(2 * l + 1), hslot(2 * l + 2));
  }
  hipLaunchKernelGGL(amk_uf_rmsnorm, dim3(B), dim3(1024), 0, st, g, (const float *)hslot(2 * L), dm.final_norm, dm.xn);
  const int lm_wt = dm.tied ? 0 : wt;
  hipLaunchKernelGGL(pick_uf_gemv(lm_wt, 2), grid(dm.V), dim3(kUfThreads), gl, st, g, s, dm.lm, dm.lm_scale, d, dm.V, (const float *)dm.xn, (float *)nullptr, (const float *)nullptr, (float *)nullptr);
  hipLaunchKernelGGL(amk_uf_argmax, dim3(1), dim3(64), 0, st, g, s, m->n_lm_uf);
}

namespace {

// n_steps greedy steps of `batch` sequences, sequence b at position pos[b] in the first step
// Argument checks of a decode call (no allocation unless an error is reported).
amk_status check_decode(const amk_model *m, const amk_kv *kv, const int32_t *d_tokens,
                        const int32_t *pos, int32_t n_steps, int32_t batch, const int32_t *d_out,
                        const char *fn) {
  auto fail = [&](amk_status st, const char *why) { return set_error(st, std::string(fn) + why); };
  if (!m || !kv || !d_tokens || !d_out || !pos) return fail(AMK_E_INVALID, ": null argument");
  if (kv->m != m) return fail(AMK_E_INVALID, ": KV cache belongs to another model");
  if (n_steps < 1) return fail(AMK_E_INVALID, ": n_steps must be >= 1");
  if (n_steps > 0x100000) return fail(AMK_E_INVALID, ": n_steps too large");
  if (batch < 1 || batch > m->cfg.max_batch || batch > kv->batch)
    return fail(AMK_E_CAPACITY, ": batch exceeds max_batch or the KV cache");
  for (int32_t b = 0; b < batch; ++b)
    if (pos[b] < 0 || (int64_t)pos[b] + n_steps > std::min(kv->max_seq, m->cfg.max_seq))
      return fail(AMK_E_CAPACITY, ": positions beyond max_seq");
  return AMK_OK;
}

// n_steps greedy steps of `batch` sequences, sequence b at position pos[b] in the first step, on
// the scratch that descriptor dm (device copy g) points at. Launches only: no allocation.
amk_status decode_on(amk_model *m, const DevModel &dm, const DevModel *g, amk_kv *kv,
                     const int32_t *d_tokens, const int32_t *pos, int32_t n_steps, int32_t batch,
                     float *d_logits, int32_t *d_out, hipStream_t st) {
  StepArgs s;
  s.tokens = d_tokens;
  s.logits = d_logits;
  s.next = d_out;
  s.kv = static_cast<uint16_t *>(kv->data);
  s.kv_batch = kv->batch;
  s.kv_max_seq = kv->max_seq;
  s.pos = pos[0];
  for (int32_t b = 0; b < kMaxBatch; ++b) s.pos_in[b] = b < batch ? pos[b] : 0;
  s.kv_seq = -1;
  s.posp = nullptr;  // set on the device
  s.batch = batch;
  s.epoch = 0;  // the megakernel takes its epochs from the device counter
  s.step = 0;
  s.n_steps = n_steps;
  if (m->path == AMK_PATH_MEGAKERNEL) {
    void *args[] = {(void *)&g, (void *)&s};
    hipError_t e = hipLaunchCooperativeKernel((const void *)m->mk, dim3(m->n_cu), dim3(kThreads),
                                              args, m->lds_bytes, st);
    if (e != hipSuccess) return set_error(AMK_E_HIP, std::string("megakernel launch: ") + hipGetErrorString(e));
  } else {
    // the ablation runs each step as its own sequence of launches, chaining tokens on the device
    for (int32_t i = 0; i < n_steps; ++i) {
      StepArgs si = s;
      si.n_steps = 1;
      si.pos = pos[0] + i;
      for (int32_t b = 0; b < batch; ++b) si.pos_in[b] = pos[b] + i;
      si.tokens = i ? d_out + (int64_t)(i - 1) * batch : d_tokens;
      si.next = d_out + (int64_t)i * batch;
      si.logits = d_logits ? d_logits + (int64_t)i * batch * m->cfg.vocab : nullptr;
      launch_unfused(m, dm, g, si, st);
    }
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return set_error(AMK_E_HIP, std::string("unfused launch: ") + hipGetErrorString(e));
  }
  clear_error();
  return AMK_OK;
}

amk_status decode(amk_model *m, amk_kv *kv, const int32_t *d_tokens, const int32_t *pos,
                  int32_t n_steps, int32_t batch, float *d_logits, int32_t *d_out, void *stream,
                  const char *fn) {
  const amk_status c = check_decode(m, kv, d_tokens, pos, n_steps, batch, d_out, fn);
  if (c != AMK_OK) return c;
  return decode_on(m, m->dm, m->d_dm, kv, d_tokens, pos, n_steps, batch, d_logits, d_out,
                   static_cast<hipStream_t>(stream));
}

}  // namespace

extern "C" amk_status amk_decode_steps(amk_model *m, amk_kv *kv, const int32_t *d_tokens,
                                       int32_t pos, int32_t n_steps, int32_t batch,
                                       float *d_logits, int32_t *d_out, void *stream) {
  AMK_API_BEGIN
  int32_t pv[kMaxBatch];
  for (int32_t b = 0; b < kMaxBatch; ++b) pv[b] = pos;
  if (batch > kMaxBatch) return set_error(AMK_E_CAPACITY, "amk_decode_steps: batch exceeds max_batch");
  return decode(m, kv, d_tokens, pv, n_steps, batch, d_logits, d_out, stream, "amk_decode_steps");
  AMK_API_END
}

extern "C" amk_status amk_decode_steps_ragged(amk_model *m, amk_kv *kv, const int32_t *d_tokens,
                                              const int32_t *h_pos, int32_t n_steps, int32_t batch,
                                              float *d_logits, int32_t *d_out, void *stream) {
  AMK_API_BEGIN
  return decode(m, kv, d_tokens, h_pos, n_steps, batch, d_logits, d_out, stream,
                "amk_decode_steps_ragged");
  AMK_API_END
}

// The variant of amk_decode_steps that allocates nothing: the same kernels on this device's
// static scratch array instead of the model's scratch block. Every call first clears the array's
// state region (a fill kernel, so the call may be captured into a graph), since the array keeps
// whatever the last call on this GPU, of any model, left there.
extern "C" amk_status amk_decode_steps_noalloc(amk_model *m, amk_kv *kv, const int32_t *d_tokens,
                                               int32_t pos, int32_t n_steps, int32_t batch,
                                               float *d_logits, int32_t *d_out, void *stream) {
  AMK_API_BEGIN
  if (batch > kMaxBatch) return set_error(AMK_E_CAPACITY, "amk_decode_steps_noalloc: batch exceeds max_batch");
  int32_t pv[kMaxBatch];
  for (int32_t b = 0; b < kMaxBatch; ++b) pv[b] = pos;
  const amk_status c = check_decode(m, kv, d_tokens, pv, n_steps, batch, d_out, "amk_decode_steps_noalloc");
  if (c != AMK_OK) return c;
  if (!m->d_dm_static)
    return set_error(AMK_E_CAPACITY, "amk_decode_steps_noalloc: the model's step scratch (" +
                                         std::to_string(m->plan.total) + " bytes) exceeds the static array (" +
                                         std::to_string(kStaticScratchBytes) + " bytes)");
  hipStream_t st = static_cast<hipStream_t>(stream);
  if (m->path == AMK_PATH_MEGAKERNEL) zero_async(m->static_base, m->plan.state_bytes, st);
  return decode_on(m, m->dm_static, m->d_dm_static, kv, d_tokens, pv, n_steps, batch, d_logits,
                   d_out, st);
  AMK_API_END
}

extern "C" amk_status amk_decode_step(amk_model *m, amk_kv *kv, const int32_t *d_tokens,
                                      int32_t pos, int32_t batch, float *d_logits,
                                      int32_t *d_next, void *stream) {
  return amk_decode_steps(m, kv, d_tokens, pos, 1, batch, d_logits, d_next, stream);
}

namespace {

// The prompt-processing copy of the model: weights shared, scratch for kMaxBatch columns.
void prefill_init(amk_model *m, hipStream_t st) {
  if (m->d_dm_pf) return;
  DevModel dp = m->dm;
  const int L = dp.L, d = dp.d, qd = dp.qd, F = dp.F, V = dp.V, C = kMaxBatch;
  const int kmax = std::max(std::max(d, qd), F);
  dp.max_batch = C;
  dp.h = m->dalloc<float>((size_t)(2 * L + 1) * C * d);
  dp.q = m->dalloc<float>((size_t)L * C * qd);
  dp.part = m->dalloc<float>((size_t)L * C * dp.nq * dp.nblk * (dp.hd + 2));
  dp.ao = m->dalloc<float>((size_t)L * C * qd);
  dp.a = m->dalloc<float>((size_t)L * C * F);
  dp.logits = m->dalloc<float>((size_t)C * V);
  dp.amax = m->dalloc<float2>((size_t)std::max<int>(m->n_lm_uf, dp.n_lm) * C);
  dp.xn = m->dalloc<float>((size_t)C * kmax);
  dp.y = m->dalloc<float>((size_t)C * std::max(std::max(dp.qkvr, 2 * F), std::max(V, d)));
  dp.o = m->dalloc<float>((size_t)C * qd);
  m->pf_next = m->dalloc<int32_t>(C);
  DevModel *g = m->dalloc<DevModel>(1);
  hip_check(hipMemcpyAsync(g, &dp, sizeof dp, hipMemcpyHostToDevice, st), "hipMemcpyAsync");
  // the operator kernels at the widest layout (a megakernel model has not set them)
  const uint32_t gl = 4u * (64 * 8 + kMaxBatch * kUfRowsPerBlock + (uint32_t)std::max<int>(kmax, kMfmaRedFloats));
  for (int wt = 0; wt < 3; ++wt)
    for (int mode = 0; mode < 3; ++mode)
      hip_check(hipFuncSetAttribute((const void *)pick_uf_gemv(wt, mode),
                                    hipFuncAttributeMaxDynamicSharedMemorySize, (int)gl),
                "hipFuncSetAttribute");
  hip_check(hipFuncSetAttribute((const void *)m->uf_attn, hipFuncAttributeMaxDynamicSharedMemorySize,
                                (int)m->uf_attn_lds), "hipFuncSetAttribute");
  m->dm_pf = dp;
  m->d_dm_pf = g;
}

}  // namespace

extern "C" amk_status amk_prefill(amk_model *m, amk_kv *kv, int32_t seq, const int32_t *d_tokens,
                                  int32_t pos0, int32_t n_tokens, float *d_logits,
                                  int32_t *d_next, void *stream) {
  AMK_API_BEGIN
  if (!m || !kv || !d_tokens || !d_next) return set_error(AMK_E_INVALID, "amk_prefill: null argument");
  if (kv->m != m) return set_error(AMK_E_INVALID, "amk_prefill: KV cache belongs to another model");
  if (n_tokens < 1) return set_error(AMK_E_INVALID, "amk_prefill: n_tokens must be >= 1");
  if (seq < 0 || seq >= kv->batch) return set_error(AMK_E_CAPACITY, "amk_prefill: seq outside the KV cache");
  if (pos0 < 0 || (int64_t)pos0 + n_tokens > std::min(kv->max_seq, m->cfg.max_seq))
    return set_error(AMK_E_CAPACITY, "amk_prefill: positions beyond max_seq");
  hipStream_t st = static_cast<hipStream_t>(stream);
  try {
    prefill_init(m, st);
  } catch (const std::bad_alloc &) {
    return set_error(AMK_E_OOM, "amk_prefill: allocation failed");
  }
  const DevModel &dp = m->dm_pf;
  int32_t last = 0;
  for (int32_t c0 = 0; c0 < n_tokens; c0 += kMaxBatch) {
    const int32_t C = std::min<int32_t>(kMaxBatch, n_tokens - c0);
    StepArgs s;
    s.tokens = d_tokens + c0;
    s.logits = nullptr;  // the scratch logits of the prefill model
    s.next = m->pf_next;
    s.kv = static_cast<uint16_t *>(kv->data);
    s.kv_batch = kv->batch;
    s.kv_max_seq = kv->max_seq;
    s.pos = pos0 + c0;
    for (int32_t b = 0; b < kMaxBatch; ++b) s.pos_in[b] = pos0 + c0 + std::min(b, C - 1);
    s.posp = nullptr;
    s.kv_seq = seq;
    s.batch = C;
    s.epoch = 0;
    s.step = 0;
    s.n_steps = 1;
    launch_unfused(m, dp, m->d_dm_pf, s, st);
    last = C - 1;
  }
  hipError_t e = hipGetLastError();
  if (e == hipSuccess)
    e = hipMemcpyAsync(d_next, m->pf_next + last, sizeof(int32_t), hipMemcpyDeviceToDevice, st);
  if (e == hipSuccess && d_logits)
    e = hipMemcpyAsync(d_logits, dp.logits + (size_t)last * dp.V, sizeof(float) * dp.V,
                       hipMemcpyDeviceToDevice, st);
  if (e != hipSuccess) return set_error(AMK_E_HIP, std::string("amk_prefill: ") + hipGetErrorString(e));
  clear_error();
  return AMK_OK;
  AMK_API_END
}

extern "C" amk_status amk_sync(amk_model *m, void *stream) {
  AMK_API_BEGIN
  if (!m) return set_error(AMK_E_INVALID, "amk_sync: null model");
  hipStream_t st = static_cast<hipStream_t>(stream);
  hipError_t e = hipStreamSynchronize(st);
  if (e != hipSuccess) return set_error(AMK_E_HIP, std::string("amk_sync: ") + hipGetErrorString(e));
  uint32_t err[4];
  e = hipMemcpy(err, m->dm.err, 16, hipMemcpyDeviceToHost);
  if (e != hipSuccess) return set_error(AMK_E_HIP, std::string("amk_sync: ") + hipGetErrorString(e));
  m->err_pending = false;
  if (err[0]) {
    reset_device_state(m, st);
    std::memset(m->h_err, 0, 16);
    return map_device_error(err[0], err[2], err[3]);
  }
  clear_error();
  return AMK_OK;
  AMK_API_END
}

extern "C" amk_status amk_trace_enable(amk_model *m, uint64_t *d_trace, size_t bytes) {
  AMK_API_BEGIN
  if (!m) return set_error(AMK_E_INVALID, "amk_trace_enable: null model");
  const size_t need = 8ull * (4ull * m->sched.hdr.n_tasks + (size_t)m->n_cu);
  if (d_trace && bytes < need)
    return set_error(AMK_E_CAPACITY, "amk_trace_enable: buffer needs " + std::to_string(need) + " bytes");
  (void)hipDeviceSynchronize();
  m->dm.trace = d_trace;
  upload_dm(m);
  clear_error();
  return AMK_OK;
  AMK_API_END
}

extern "C" amk_status amk_model_get_info(const amk_model *m, amk_model_info *out) {
  if (!m || !out) return set_error(AMK_E_INVALID, "amk_model_get_info: null argument");
  out->n_cu = m->n_cu;
  out->n_tasks = (int32_t)m->sched.hdr.n_tasks;
  out->launches_per_step = m->path == AMK_PATH_MEGAKERNEL ? 1 : 1 + 10 * m->cfg.n_layers + 3;
  out->lds_bytes = (int32_t)m->lds_bytes;
  out->attn_blocks = (int32_t)m->sched.hdr.attn_blocks;
  out->path = m->path;
  out->weight_bytes = m->weight_bytes;
  out->predicted_us = m->sched.hdr.predicted_us;
  out->scratch_bytes = m->plan.total;
  out->heads_per_pass = m->path == AMK_PATH_MEGAKERNEL ? m->mk_qmax : qmax_for(m->dm.qpg);
  return AMK_OK;
}

extern "C" amk_status amk_model_get_schedule(const amk_model *m, void **blob, size_t *bytes) {
  if (!m || !blob || !bytes) return set_error(AMK_E_INVALID, "amk_model_get_schedule: null argument");
  void *p = std::malloc(m->blob.size());
  if (!p) return set_error(AMK_E_OOM, "amk_model_get_schedule: out of host memory");
  std::memcpy(p, m->blob.data(), m->blob.size());
  *blob = p;
  *bytes = m->blob.size();
  return AMK_OK;
}

namespace {

// Install an already validated schedule of the model's structure: upload its task tables over
// the current ones, set the kernel's LDS size, restart the flag epochs. Synchronises `st`.
amk_status install_schedule(amk_model *m, Schedule &&s, std::vector<uint8_t> &&blob,
                            hipStream_t st) {
  const BlobHeader &h = s.hdr, &c = m->sched.hdr;
  if (m->path != AMK_PATH_MEGAKERNEL)
    return set_error(AMK_E_UNSUPPORTED, "schedule replacement needs the megakernel path");
  if (std::memcmp(&h.cfg, &c.cfg, sizeof(BlobConfig)) != 0 || h.batch != c.batch ||
      h.n_cu != c.n_cu || h.n_tasks != c.n_tasks || h.attn_blocks != c.attn_blocks ||
      h.n_lm_tiles != c.n_lm_tiles)
    return set_error(AMK_E_UNSUPPORTED,
                     "schedule differs in structure (config, batch, CUs, tasks, KV blocks or LM "
                     "tiles): create a new model with it");
  hip_check(hipStreamSynchronize(st), "hipStreamSynchronize");
  std::vector<uint32_t> offs(h.n_cu + 1);
  std::vector<Task> tasks;
  tasks.reserve(h.n_tasks);
  for (uint32_t cu = 0; cu < h.n_cu; ++cu) {
    offs[cu] = (uint32_t)tasks.size();
    for (const Task &t : s.per_cu[cu]) tasks.push_back(t);
  }
  offs[h.n_cu] = (uint32_t)tasks.size();
  const int qmax = mk_qmax_for(s, m->dm.qpg);
  const MkFn mk = pick_megakernel(m->cfg.wtype, m->dm.hd, qmax, m->cfg.max_batch > 1);
  if (!mk) return set_error(AMK_E_UNSUPPORTED, "no megakernel instance for this schedule");
  if (h.lds_bytes != m->lds_bytes || mk != m->mk) {
    hip_check(hipFuncSetAttribute((const void *)mk, hipFuncAttributeMaxDynamicSharedMemorySize,
                                  (int)h.lds_bytes), "hipFuncSetAttribute");
    int per_cu = 0;
    hip_check(hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, (const void *)mk, kThreads,
                                                           h.lds_bytes), "occupancy");
    if (per_cu < 1) return set_error(AMK_E_SCHEDULE_REJECTED, "schedule LDS does not fit on a CU");
  }
  hip_check(hipMemcpy(const_cast<Task *>(m->dm.tasks), tasks.data(), tasks.size() * sizeof(Task),
                      hipMemcpyHostToDevice), "hipMemcpy");
  hip_check(hipMemcpy(const_cast<uint32_t *>(m->dm.offsets), offs.data(), offs.size() * 4,
                      hipMemcpyHostToDevice), "hipMemcpy");
  zero_state(m, st);
  hip_check(hipStreamSynchronize(st), "hipStreamSynchronize");
  m->lds_bytes = h.lds_bytes;
  m->mk = mk;
  m->mk_qmax = qmax;
  m->sched = std::move(s);
  m->blob = std::move(blob);
  m->dm.argmax_id = argmax_of(m->sched);
  upload_dm(m);
  return AMK_OK;
}

void set_trace(amk_model *m, uint64_t *d_trace) {
  m->dm.trace = d_trace;
  upload_dm(m);
}

}  // namespace

extern "C" amk_status amk_model_set_schedule(amk_model *m, const void *blob, size_t bytes,
                                             void *stream) {
  AMK_API_BEGIN
  if (!m || !blob) return set_error(AMK_E_INVALID, "amk_model_set_schedule: null argument");
  Schedule s;
  std::string e, rep;
  if (!parse(blob, bytes, &s, &e)) return set_error(AMK_E_SCHEDULE_REJECTED, e);
  if (!validate_schedule(s, &rep)) return set_error(AMK_E_SCHEDULE_REJECTED, rep);
  std::vector<uint8_t> copy((const uint8_t *)blob, (const uint8_t *)blob + bytes);
  amk_status r = install_schedule(m, std::move(s), std::move(copy), static_cast<hipStream_t>(stream));
  if (r == AMK_OK) clear_error();
  return r;
  AMK_API_END
}

extern "C" amk_status amk_model_tune(amk_model *m, amk_kv *kv, int32_t pos, int32_t rounds,
                                     int32_t steps, double gain, void *stream, double *best_us) {
  AMK_API_BEGIN
  if (!m || !kv) return set_error(AMK_E_INVALID, "amk_model_tune: null argument");
  if (kv->m != m) return set_error(AMK_E_INVALID, "amk_model_tune: KV cache belongs to another model");
  if (m->path != AMK_PATH_MEGAKERNEL) return set_error(AMK_E_UNSUPPORTED, "amk_model_tune: megakernel path only");
  if (rounds < 0 || steps < 1 || !(gain > 0.0 && gain <= 1.0))
    return set_error(AMK_E_INVALID, "amk_model_tune: rounds >= 0, steps >= 1, 0 < gain <= 1");
  if (pos < 0 || (int64_t)pos + steps > std::min(kv->max_seq, m->cfg.max_seq))
    return set_error(AMK_E_CAPACITY, "amk_model_tune: positions beyond max_seq");
  hipStream_t st = static_cast<hipStream_t>(stream);
  const int32_t batch = std::min(m->cfg.max_batch, kv->batch);
  const size_t stride = 4ull * m->sched.hdr.n_tasks + (size_t)m->n_cu;
  int32_t *d_tok = nullptr;
  uint64_t *d_trace = nullptr;
  hipEvent_t ev[2] = {nullptr, nullptr};
  amk_status status = AMK_OK;
  try {
    hip_check(hipMalloc(&d_tok, sizeof(int32_t) * batch), "hipMalloc");
    hip_check(hipMalloc(&d_trace, 8 * stride), "hipMalloc");
    hip_check(hipEventCreate(&ev[0]), "hipEventCreate");
    hip_check(hipEventCreate(&ev[1]), "hipEventCreate");
    set_trace(m, nullptr);
    // run the steps (token 0, greedy chaining); traced: collect one trace per step
    auto run = [&](std::vector<uint64_t> *traces, double *us) -> amk_status {
      hip_check(hipMemsetAsync(d_tok, 0, sizeof(int32_t) * batch, st), "hipMemsetAsync");
      if (traces) set_trace(m, d_trace);
      hip_check(hipEventRecord(ev[0], st), "hipEventRecord");
      for (int32_t i = 0; i < steps; ++i) {
        amk_status r = amk_decode_step(m, kv, d_tok, pos + i, batch, nullptr, d_tok, st);
        if (r != AMK_OK) return r;
        if (traces) {
          hip_check(hipStreamSynchronize(st), "hipStreamSynchronize");
          const size_t off = traces->size();
          traces->resize(off + stride);
          hip_check(hipMemcpy(traces->data() + off, d_trace, 8 * stride, hipMemcpyDeviceToHost), "hipMemcpy");
        }
      }
      hip_check(hipEventRecord(ev[1], st), "hipEventRecord");
      amk_status r = amk_sync(m, stream);
      if (traces) set_trace(m, nullptr);
      if (r != AMK_OK) return r;
      float ms = 0.f;
      hip_check(hipEventElapsedTime(&ms, ev[0], ev[1]), "hipEventElapsedTime");
      if (us) *us = 1000.0 * ms / steps;
      return AMK_OK;
    };
    double best = 0.0;
    if ((status = run(nullptr, nullptr)) == AMK_OK)  // warm-up
      status = run(nullptr, &best);
    Schedule best_s = m->sched;
    std::vector<uint8_t> best_blob = m->blob;
    for (int32_t r = 0; r < rounds && status == AMK_OK; ++r) {
      std::vector<uint64_t> traces;
      if ((status = run(&traces, nullptr)) != AMK_OK) break;
      Schedule s = m->sched;
      std::string e, rep;
      if (!rebalance_schedule(&s, traces.data(), steps, gain, &e)) {
        status = set_error(AMK_E_INVALID, "amk_model_tune: " + e);
        break;
      }
      if (!validate_schedule(s, &rep)) {
        status = set_error(AMK_E_SCHEDULE_REJECTED, rep);
        break;
      }
      std::vector<uint8_t> blob = serialize(s);
      if ((status = install_schedule(m, std::move(s), std::move(blob), st)) != AMK_OK) break;
      double us = 0.0;
      if ((status = run(nullptr, &us)) != AMK_OK) break;
      if (us < best) {
        best = us;
        best_s = m->sched;
        best_blob = m->blob;
      }
    }
    if (status == AMK_OK && best_blob != m->blob)
      status = install_schedule(m, std::move(best_s), std::move(best_blob), st);
    if (status == AMK_OK && best_us) *best_us = best;
  } catch (...) {
    (void)hipDeviceSynchronize();
    m->dm.trace = nullptr;
    try {
      upload_dm(m);
    } catch (...) {
    }
    if (d_tok) (void)hipFree(d_tok);
    if (d_trace) (void)hipFree(d_trace);
    for (hipEvent_t e : ev)
      if (e) (void)hipEventDestroy(e);
    throw;
  }
  (void)hipDeviceSynchronize();
  if (m->dm.trace) {
    m->dm.trace = nullptr;
    upload_dm(m);
  }
  (void)hipFree(d_tok);
  (void)hipFree(d_trace);
  for (hipEvent_t e : ev) (void)hipEventDestroy(e);
  if (status == AMK_OK) clear_error();
  return status;
  AMK_API_END
}

extern "C" amk_status amk_destroy(amk_model *m) {
  if (!m) return set_error(AMK_E_INVALID, "amk_destroy: null model");
  (void)hipDeviceSynchronize();
  free_model(m);
  return AMK_OK;
}
