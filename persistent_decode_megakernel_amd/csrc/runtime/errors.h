// Thread-local last-error text behind amk_last_error(), and the status helpers every C entry
// point uses so that no C++ exception crosses the ABI.
#pragma once
#include <string>

#include "amk.h"

namespace amk {
amk_status set_error(amk_status st, const std::string &msg);
void clear_error();
const char *last_error_text();
}  // namespace amk

#define AMK_API_BEGIN try {
#define AMK_API_END                                                          \
  }                                                                          \
  catch (const std::bad_alloc &) {                                           \
    return amk::set_error(AMK_E_OOM, "host allocation failed");             \
  }                                                                          \
  catch (const std::exception &ex) {                                         \
    return amk::set_error(AMK_E_INVALID, std::string("internal: ") + ex.what()); \
  }                                                                          \
  catch (...) {                                                              \
    return amk::set_error(AMK_E_INVALID, "internal: unknown exception");    \
  }
