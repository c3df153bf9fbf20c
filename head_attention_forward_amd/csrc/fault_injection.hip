// Fault-injection hook for tests of the error path (compiled in only when
// MHA_FAULT_INJECTION is defined, i.e. in libmha_fault.so; the normal build
// contains nothing from this file).  mha_fault_inject(n) makes the next n
// kernel launches of the library fail in launch_kernel (kernels.h) before
// they reach the HIP runtime, so the entry point returns MHA_ERR_HIP -- on
// a machine without a GPU too.
#ifdef MHA_FAULT_INJECTION
#include <atomic>

#include "kernels.h"

namespace mha {
namespace {
std::atomic<int> g_armed{0};
}  // namespace

bool fault_injection_fires() {
  int n = g_armed.load();
  while (n > 0)
    if (g_armed.compare_exchange_weak(n, n - 1)) return true;
  return false;
}
}  // namespace mha

extern "C" void mha_fault_inject(int launches) { mha::g_armed.store(launches > 0 ? launches : 0); }
#endif
