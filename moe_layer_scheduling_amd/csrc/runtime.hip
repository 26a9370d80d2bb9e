// Entry points shared by both kernels: status strings, workspace clearing, device
// status query, device checks.
#include <string.h>

#include "common.hpp"
#include "host.hpp"

namespace etc {
namespace host {

int current_gfx950_device() {
  static int checked[MAX_DEVICES] = {0};  // 0 unknown, 1 gfx950, 2 other
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= MAX_DEVICES) return -1;
  if (checked[dev] == 0) {
    hipDeviceProp_t prop;
    if (hipGetDeviceProperties(&prop, dev) != hipSuccess) return -1;
    checked[dev] = (strncmp(prop.gcnArchName, "gfx950", 6) == 0) ? 1 : 2;
  }
  return checked[dev] == 1 ? dev : -1;
}

int device_cus(int dev) {
  static int cus[MAX_DEVICES] = {0};
  if (dev < 0 || dev >= MAX_DEVICES) return 0;
  if (cus[dev] == 0) {
    int v = 0;
    if (hipDeviceGetAttribute(&v, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess) return 0;
    cus[dev] = v;
  }
  return cus[dev];
}

}  // namespace host
}  // namespace etc

using namespace etc;

ETC_API const char* etc_status_string(etc_status s) {
  switch (s) {
    case ETC_OK: return "ok";
    case ETC_ERR_INVALID_ARG: return "invalid argument";
    case ETC_ERR_UNSUPPORTED: return "unsupported shape";
    case ETC_ERR_WORKSPACE: return "workspace missing, misaligned or too small";
    case ETC_ERR_HIP: return "HIP runtime error";
    case ETC_ERR_TIMEOUT: return "device wait timed out";
    case ETC_ERR_NO_DEVICE: return "no gfx950 device is current";
  }
  return "unknown status";
}

ETC_API int32_t etc_abi_version(void) { return ETC_ABI_VERSION; }

ETC_API etc_status etc_workspace_init(void* workspace, size_t bytes, void* stream) {
  if (workspace == nullptr || bytes < 256 || (reinterpret_cast<uintptr_t>(workspace) & 255u))
    return ETC_ERR_WORKSPACE;
  if (host::current_gfx950_device() < 0) return ETC_ERR_NO_DEVICE;
  if (hipMemsetAsync(workspace, 0, bytes, static_cast<hipStream_t>(stream)) != hipSuccess)
    return ETC_ERR_HIP;
  return ETC_OK;
}

ETC_API etc_status etc_query_device_status(const void* workspace, void* stream) {
  if (workspace == nullptr) return ETC_ERR_WORKSPACE;
  if (host::current_gfx950_device() < 0) return ETC_ERR_NO_DEVICE;
  int32_t words[W_NWORDS];
  hipStream_t s = static_cast<hipStream_t>(stream);
  if (hipMemcpyAsync(words, workspace, sizeof(words), hipMemcpyDeviceToHost, s) != hipSuccess)
    return ETC_ERR_HIP;
  if (hipStreamSynchronize(s) != hipSuccess) return ETC_ERR_HIP;
  return words[W_STATUS] == 0 ? ETC_OK : static_cast<etc_status>(words[W_STATUS]);
}
