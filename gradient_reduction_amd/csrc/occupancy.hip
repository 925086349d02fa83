// Occupancy caps for streaming launches on gfx950.  A launch that reserves
// dynamic LDS it never touches fits fewer of its workgroups into one compute
// unit's LDS, so fewer, longer streams of row accesses are in flight at once;
// for the row mixes of these kernels that measured faster than a full compute
// unit.  The reservation is computed once per kernel, device and cap.
#include <hip/hip_runtime.h>

#include <cstdint>
#include <map>
#include <mutex>
#include <tuple>

#include "internal.h"

namespace dc {

size_t occupancy_pad(const void* kernel, int cap) {
  if (cap <= 0) return 0;
  static std::mutex mu;
  static std::map<std::tuple<const void*, int, int>, size_t> cache;
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess) {
    (void)hipGetLastError();
    return 0;
  }
  const auto key = std::make_tuple(kernel, dev, cap);
  {
    std::lock_guard<std::mutex> g(mu);
    const auto it = cache.find(key);
    if (it != cache.end()) return it->second;
  }
  int lds_cu = 0;
  hipFuncAttributes fa;
  if (hipDeviceGetAttribute(&lds_cu, hipDeviceAttributeMaxSharedMemoryPerMultiprocessor, dev) !=
          hipSuccess ||
      hipFuncGetAttributes(&fa, kernel) != hipSuccess) {
    (void)hipGetLastError();
    return 0;
  }
  const int64_t per_wg = (int64_t)(lds_cu / cap) / 256 * 256;
  const int64_t pad = per_wg - (int64_t)fa.sharedSizeBytes;
  // a workgroup may reserve at most 64 KB: a smaller cap is not reachable
  const size_t v = (pad > 0 && per_wg <= 65536) ? (size_t)pad : 0;
  std::lock_guard<std::mutex> g(mu);
  cache[key] = v;
  return v;
}

int stream_cap(int rows, int u, int kb) {
  const int per_wg_kb = rows * u;  // 64 threads x 16 bytes = 1 KB per row access
  if (kb <= 0 || per_wg_kb <= 0) return 0;
  const int cap = kb / per_wg_kb;
  if (cap >= 32) return 0;
  return cap < 3 ? 3 : cap;
}

}  // namespace dc
