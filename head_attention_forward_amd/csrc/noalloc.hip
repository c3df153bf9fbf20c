// sdpa_backward_noalloc: sdpa_backward for callers that cannot allocate
// device memory (code under HIP graph capture, serving loops, harnesses
// that forbid hipMalloc).  Its only scratch -- the two fp32 row terms per
// query row that the dQ kernel writes and the dK/dV kernel reads -- lives
// in the library's own device array below instead of a caller workspace.
//
// Every GPU the library runs this entry point on holds its own copy of the
// array until the process ends.  In host code `scratch` names a host-side
// stand-in, not device memory: its device address is looked up once per
// device (hipGetSymbolAddress, with that device current) and only that
// address is ever handed to kernels.  Calls on one GPU share its array:
// calls that overlap in time on one GPU (two streams) race.  Nothing needs
// clearing between calls: each call writes every row term it reads first.
#include <mutex>

#include "kernels.h"

namespace mha {
namespace {

constexpr int64_t kScratchRows = (int64_t)1 << 20;  // query rows B * h * n_q
constexpr int kMaxDevices = 64;

// Two fp32 arrays of kScratchRows each (8 MiB).
static __device__ __align__(256) float scratch[2 * kScratchRows];

std::once_flag g_once[kMaxDevices];
void* g_ptr[kMaxDevices];
hipError_t g_err[kMaxDevices];

// Device address of this device's `scratch`, looked up on first use.
hipError_t scratch_address(void** out) {
  int dev = -1;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
  std::call_once(g_once[dev], [dev] {
    void* p = nullptr;
    g_err[dev] = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    g_ptr[dev] = g_err[dev] == hipSuccess ? p : nullptr;
  });
  if (g_err[dev] != hipSuccess) return g_err[dev];
  *out = g_ptr[dev];
  return hipSuccess;
}

}  // namespace
}  // namespace mha

extern "C" int sdpa_backward_noalloc(const void* Q, const void* K, const void* V, const void* O,
                                     const void* dO, const float* lse, void* dQ, void* dK, void* dV,
                                     int B, int h, int n_q, int n_k, int d_k, int d_v, float scale,
                                     int mask_kind, const int32_t* key_lengths, int dtype,
                                     hipStream_t stream) {
  // Every argument check runs before the first HIP call.
  const int st = mha::check_backward_args(Q, K, V, O, dO, lse, dQ, dK, dV, B, h, n_q, n_k, d_k, d_v,
                                          scale, mask_kind, key_lengths, dtype);
  if (st != MHA_OK) return st;
  if ((int64_t)B * h * n_q > mha::kScratchRows) return MHA_ERR_WORKSPACE;
  const size_t need = sdpa_backward_workspace_bytes(B, h, n_q);
  if (need == 0 || need > sizeof(mha::scratch)) return MHA_ERR_WORKSPACE;
  void* ws = nullptr;
  if (mha::scratch_address(&ws) != hipSuccess) return MHA_ERR_HIP;
  return sdpa_backward(Q, K, V, O, dO, lse, dQ, dK, dV, B, h, n_q, n_k, d_k, d_v, scale, mask_kind,
                       key_lengths, dtype, ws, sizeof(mha::scratch), stream);
}
