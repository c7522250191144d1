// chunked.hip -- chunkwise-parallel MFMA prefill (placeholder until the kernels land).
#include "device_common.hpp"
#include "launch.hpp"

namespace glah {

int device_cu_count() {
  int dev = 0, n = 0;
  if (hipGetDevice(&dev) != hipSuccess) return 256;
  if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || n <= 0) return 256;
  return n;
}

bool chunked_supported(const LayerArgs &, int) { return false; }
size_t chunked_workspace_bytes(const LayerArgs &, int) { return 0; }
hipError_t launch_chunked_prefill(const LayerArgs &, int) { return hipErrorNotSupported; }
bool swa_mfma_supported(const LayerArgs &) { return false; }
hipError_t launch_swa_mfma(const LayerArgs &) { return hipErrorNotSupported; }

}  // namespace glah
