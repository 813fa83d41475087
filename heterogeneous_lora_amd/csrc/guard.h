// Exception barrier for the C entry points (host code only).
#pragma once

#include <exception>
#include <new>

#include "internal.h"

namespace slora {

// Runs an entry point's body; a C++ exception (std::bad_alloc from host containers,
// above all) becomes SLORA_E_INVALID with a message instead of crossing the C ABI.
template <class F>
int guarded(const char* what, F&& body) {
  try {
    return body();
  } catch (const std::bad_alloc&) {
    return fail(SLORA_E_INVALID, "%s: host memory exhausted", what);
  } catch (const std::exception& e) {
    return fail(SLORA_E_INVALID, "%s: %s", what, e.what());
  } catch (...) {
    return fail(SLORA_E_INVALID, "%s: unexpected error", what);
  }
}

}  // namespace slora
