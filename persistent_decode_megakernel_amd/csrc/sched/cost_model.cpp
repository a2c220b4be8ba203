// The cost model the schedule search uses when the caller passes none: the one amk_calibrate
// measured on the device, stored as JSON beside the library, when it was measured for the same
// number of compute units; otherwise built-in values.
//
// File: $AMK_COST_MODEL if set ("off": none), else cost_model.json in the directory of the shared
// library that holds this code. Its "fit" object carries the fields of amk_cost_model; "n_cu" the
// CU count it was measured on. A file that is missing, unreadable, for another CU count or without
// a complete fit is ignored.
#include <dlfcn.h>

#include <cstdio>
#include <cstdlib>
#include <cstring>
#include <fstream>
#include <sstream>
#include <string>

#include "../runtime/errors.h"
#include "sched_internal.h"

namespace amk {

namespace {

// value of the number after "key": inside text (from `from`), or false
bool json_number(const std::string &text, const char *key, size_t from, double *out) {
  const std::string k = std::string("\"") + key + "\"";
  size_t p = text.find(k, from);
  if (p == std::string::npos) return false;
  p = text.find(':', p + k.size());
  if (p == std::string::npos) return false;
  const char *b = text.c_str() + p + 1;
  char *e = nullptr;
  const double v = std::strtod(b, &e);
  if (e == b) return false;
  *out = v;
  return true;
}

std::string library_dir() {
  Dl_info info{};
  if (!dladdr(reinterpret_cast<void *>(&builtin_cost_model), &info) || !info.dli_fname) return "";
  std::string p(info.dli_fname);
  const size_t slash = p.rfind('/');
  return slash == std::string::npos ? std::string(".") : p.substr(0, slash);
}

}  // namespace

bool parse_cost_model(const std::string &text, int32_t n_cu, amk_cost_model *out) {
  double file_cu = 0;
  if (!json_number(text, "n_cu", 0, &file_cu) || (int32_t)file_cu != n_cu) return false;
  const size_t fit = text.find("\"fit\"");
  if (fit == std::string::npos) return false;
  amk_cost_model m = builtin_cost_model();
  double v;
  if (!json_number(text, "cu_stream_gbs", fit, &v) || !(v > 0)) return false;
  m.cu_stream_gbs = v;
  if (!json_number(text, "hop_us", fit, &v) || !(v >= 0)) return false;
  m.hop_us = v;
  if (!json_number(text, "l2_gbs", fit, &v) || !(v > 0)) return false;
  m.l2_gbs = v;
  if (json_number(text, "task_us", fit, &v) && v >= 0) m.task_us = v;
  if (json_number(text, "prefetch_kb", fit, &v) && v >= 0) m.prefetch_kb = v;
  if (json_number(text, "attn_us", fit, &v) && v >= 0) m.attn_us = v;
  *out = m;
  return true;
}

amk_cost_model default_cost_model(int32_t n_cu, std::string *source) {
  amk_cost_model m = builtin_cost_model();
  if (source) *source = "built-in";
  const char *env = std::getenv("AMK_COST_MODEL");
  if (env && std::strcmp(env, "off") == 0) return m;
  const std::string path = env && *env ? std::string(env) : library_dir() + "/cost_model.json";
  std::ifstream f(path);
  if (!f) return m;
  std::stringstream ss;
  ss << f.rdbuf();
  amk_cost_model c;
  if (parse_cost_model(ss.str(), n_cu, &c)) {
    m = c;
    if (source) *source = path;
  }
  return m;
}

}  // namespace amk

using namespace amk;

extern "C" amk_status amk_cost_model_default(int32_t n_cu, amk_cost_model *out, char *source,
                                             size_t source_cap) {
  AMK_API_BEGIN
  if (!out) return set_error(AMK_E_INVALID, "amk_cost_model_default: null output");
  std::string src;
  *out = default_cost_model(n_cu, &src);
  if (source && source_cap) {
    std::strncpy(source, src.c_str(), source_cap - 1);
    source[source_cap - 1] = 0;
  }
  clear_error();
  return AMK_OK;
  AMK_API_END
}
