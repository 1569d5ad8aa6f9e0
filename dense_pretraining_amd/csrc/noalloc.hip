// nc_decode_step_noalloc: the decode step with its scratch in a static device
// array instead of a caller workspace, for callers that cannot allocate.
#include <mutex>

#include "common.h"
#include "kernels.h"

namespace {

// The decode step's scratch (carve_decode's layout). Each GPU the library runs
// on holds its own copy from the load of the code object to the end of the
// process. In host code the name is a host-side stand-in, never a device
// address: the device address comes from hipGetSymbolAddress, per device.
static __device__ __align__(256) unsigned char scratch[NC_NOALLOC_SCRATCH_BYTES];

constexpr int kMaxDevices = 64;
std::mutex g_mu;
void* g_ptr[kMaxDevices];  // the array's address on each device, once looked up

// The current device's address of `scratch`: looked up once per device, with
// that device current, and kept.
nc_status scratch_address(void** out) {
  int dev = -1;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return nc::record_hip_error(e, "nc_decode_step_noalloc: hipGetDevice");
  if (dev < 0 || dev >= kMaxDevices) return NC_ERR_UNSUPPORTED;
  std::lock_guard<std::mutex> lock(g_mu);
  if (!g_ptr[dev]) {
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess || !p) return nc::record_hip_error(e, "nc_decode_step_noalloc: hipGetSymbolAddress");
    g_ptr[dev] = p;
  }
  *out = g_ptr[dev];
  return NC_OK;
}

}  // namespace

extern "C" nc_status nc_decode_step_noalloc(const nc_config* cfg, const void* params, const int32_t* tok, int pos,
                                            void* cache, int32_t* next_tok, uint32_t* status, void* stream) {
  // every argument check first (nothing touches the device), then the size
  size_t need = 0;
  NC_TRY(nc::decode_step_on(cfg, params, tok, pos, cache, next_tok, status, nullptr, 0, &need, nullptr));
  if (need > (size_t)NC_NOALLOC_SCRATCH_BYTES) return NC_ERR_WORKSPACE;
  void* ptr = nullptr;
  NC_TRY(scratch_address(&ptr));
  return nc::decode_step_on(cfg, params, tok, pos, cache, next_tok, status, ptr, (size_t)NC_NOALLOC_SCRATCH_BYTES,
                            &need, static_cast<hipStream_t>(stream));
}
