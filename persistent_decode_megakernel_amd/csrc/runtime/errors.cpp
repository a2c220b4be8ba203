#include "errors.h"

namespace amk {
namespace {
thread_local std::string g_last;
}
amk_status set_error(amk_status st, const std::string &msg) {
  g_last = msg;
  return st;
}
void clear_error() { g_last.clear(); }
const char *last_error_text() { return g_last.c_str(); }
}  // namespace amk

extern "C" const char *amk_last_error(void) { return amk::last_error_text(); }
