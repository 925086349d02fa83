// Partition lists and owner map for gfx950.
//
// DeepSpeed issue "[REQUEST] DeepCompile ZeRO-1: reduce-to-owner instead of
// AllReduce", Design points: the owner map costs nothing to build; a param
// listed in exactly one optimizer partition is owned by that partition's
// rank, a param straddling a partition boundary keeps AllReduce, and groups
// reduced over another communicator are left out.
//
// Both kernels run once at init on a single 1024-thread workgroup: sizes are
// scanned with wave64 shuffle scans whose wave totals are combined through
// LDS, and chunks of 1024 params are chained with a running carry.
#include "device_common.h"
#include "internal.h"

namespace dc {
namespace {

constexpr int kScanThreads = 1024;
constexpr int kWaves = kScanThreads / 64;

// Exclusive block-wide prefix sum of v; *total gets the block sum.  Every
// thread of the block must call it.
template <typename T>
__device__ T block_exclusive_scan(T v, T* lds, T* total) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  T x = v;
#pragma unroll
  for (int d = 1; d < 64; d <<= 1) {
    const T y = __shfl_up(x, d, 64);
    if (lane >= d) x += y;
  }
  if (lane == 63) lds[wave] = x;
  __syncthreads();
  if (wave == 0) {
    T w = lane < kWaves ? lds[lane] : T(0);
#pragma unroll
    for (int d = 1; d < kWaves; d <<= 1) {
      const T y = __shfl_up(w, d, 64);
      if (lane >= d) w += y;
    }
    if (lane < kWaves) lds[lane] = w;  // inclusive wave totals
  }
  __syncthreads();
  const T before = wave > 0 ? lds[wave - 1] : T(0);
  *total = lds[kWaves - 1];
  __syncthreads();  // lds is reused by the next call
  return before + x - v;
}

struct GroupArgs {
  GroupTable g;
};

__global__ __launch_bounds__(kScanThreads) void k_partition_ids(
    int32_t P, const int64_t* __restrict__ numel, GroupArgs ga, int64_t* __restrict__ flat_offset,
    int64_t* __restrict__ part_size, int32_t* __restrict__ pid_offsets,
    int32_t* __restrict__ pids, int64_t cap) {
  __shared__ int64_t lds64[kWaves];
  __shared__ int32_t lds32[kWaves];
  const GroupTable& g = ga.g;
  int64_t pid_carry = 0;
  for (int32_t grp = 0; grp < g.num_groups; ++grp) {
    const int32_t b = g.begin[grp], e = g.begin[grp + 1];
    // T_g: sum of the group's sizes (negative sizes count as 0)
    int64_t T = 0;
    for (int32_t i0 = b; i0 < e; i0 += kScanThreads) {
      const int32_t i = i0 + (int32_t)threadIdx.x;
      const int64_t n = i < e ? max(numel[i], (int64_t)0) : 0;
      int64_t chunk;
      block_exclusive_scan<int64_t>(n, lds64, &chunk);
      T += chunk;
    }
    const int64_t parts = g.parts[grp];
    const int64_t S = (T + parts - 1) / parts;
    if (threadIdx.x == 0) part_size[grp] = S;
    // offsets a_i, partition ranges, CSR
    int64_t carry = 0;
    for (int32_t i0 = b; i0 < e; i0 += kScanThreads) {
      const int32_t i = i0 + (int32_t)threadIdx.x;
      const int64_t n = i < e ? max(numel[i], (int64_t)0) : 0;
      int64_t chunk;
      const int64_t a = carry + block_exclusive_scan<int64_t>(n, lds64, &chunk);
      carry += chunk;
      int32_t cnt = 0;
      int64_t firstp = 0;
      if (i < e && n > 0) {
        firstp = a / S;
        cnt = (int32_t)((a + n - 1) / S - firstp + 1);
      }
      int32_t ctot;
      const int64_t off = pid_carry + block_exclusive_scan<int32_t>(cnt, lds32, &ctot);
      pid_carry += ctot;
      if (i < e) {
        flat_offset[i] = a;
        pid_offsets[i] = (int32_t)off;
        for (int32_t k = 0; k < cnt; ++k)
          if (off + k < cap) pids[off + k] = (int32_t)(firstp + k);
      }
    }
  }
  if (threadIdx.x == 0) pid_offsets[P] = (int32_t)pid_carry;
}

__global__ __launch_bounds__(kScanThreads) void k_owner_map(
    int32_t W, int32_t P, const int32_t* __restrict__ pid_offsets,
    const int32_t* __restrict__ pids, int64_t cap, GroupArgs ga, int32_t* __restrict__ owner,
    int32_t* __restrict__ counts) {
  __shared__ int32_t s_own, s_str;
  const GroupTable& g = ga.g;
  for (int32_t grp = 0; grp < g.num_groups; ++grp) {
    if (threadIdx.x == 0) {
      s_own = 0;
      s_str = 0;
    }
    __syncthreads();
    const int32_t b = g.begin[grp], e = g.begin[grp + 1];
    const bool elig = g.eligible[grp] != 0;
    for (int32_t i0 = b; i0 < e; i0 += kScanThreads) {
      const int32_t i = i0 + (int32_t)threadIdx.x;
      bool own = false, str = false;
      if (i < e) {
        const int32_t o0 = pid_offsets[i], o1 = pid_offsets[i + 1];
        const int32_t n = o1 - o0;
        int32_t o = -1;
        if (elig && n == 1 && o0 >= 0 && o0 < cap) {
          o = pids[o0];
          if (o < 0 || o >= W) o = -1;
        }
        owner[i] = o;
        own = o >= 0;
        str = n >= 2;
      }
      // one wave-wide ballot per predicate, one LDS atomic per wave
      const uint64_t bo = __ballot(own), bs = __ballot(str);
      if ((threadIdx.x & 63) == 0) {
        atomicAdd(&s_own, (int32_t)__popcll(bo));
        atomicAdd(&s_str, (int32_t)__popcll(bs));
      }
    }
    __syncthreads();
    if (threadIdx.x == 0) {
      counts[2 * grp] = s_own;
      counts[2 * grp + 1] = s_str;
    }
    __syncthreads();
  }
  (void)P;
}

// ZeRO-2 partition size of every param: its group's S when the group is on
// the data-parallel comm, else 0.  One thread per param; the group is found
// by a scan of the (at most DC_MAX_GROUPS) group starts.
__global__ __launch_bounds__(256) void k_param_part_size(int32_t P, GroupArgs ga,
                                                         const int64_t* __restrict__ part_size,
                                                         int64_t* __restrict__ out) {
  const int32_t i = (int32_t)(blockIdx.x * 256 + threadIdx.x);
  if (i >= P) return;
  const GroupTable& g = ga.g;
  int32_t grp = 0;
  for (int32_t k = 1; k < g.num_groups; ++k)
    if (g.begin[k] <= i) grp = k;
  out[i] = g.eligible[grp] ? part_size[grp] : 0;
}

}  // namespace

hipError_t launch_param_part_size(int32_t num_params, const GroupTable& g, const int64_t* part_size,
                                  int64_t* out, hipStream_t stream) {
  if (num_params <= 0) return hipSuccess;
  GroupArgs ga{g};
  hipLaunchKernelGGL(k_param_part_size, dim3((unsigned)((num_params + 255) / 256)), dim3(256), 0,
                     stream, num_params, ga, part_size, out);
  return hipGetLastError();
}

hipError_t launch_partition_ids(int32_t num_params, const int64_t* numel, const GroupTable& g,
                                int64_t* flat_offset, int64_t* part_size, int32_t* pid_offsets,
                                int32_t* pids, int64_t cap, hipStream_t stream) {
  GroupArgs ga{g};
  hipLaunchKernelGGL(k_partition_ids, dim3(1), dim3(kScanThreads), 0, stream, num_params, numel,
                     ga, flat_offset, part_size, pid_offsets, pids, cap);
  return hipGetLastError();
}

hipError_t launch_owner_map(int32_t W, int32_t num_params, const int32_t* pid_offsets,
                            const int32_t* pids, int64_t cap, const GroupTable& g, int32_t* owner,
                            int32_t* counts, hipStream_t stream) {
  GroupArgs ga{g};
  hipLaunchKernelGGL(k_owner_map, dim3(1), dim3(kScanThreads), 0, stream, W, num_params,
                     pid_offsets, pids, cap, ga, owner, counts);
  return hipGetLastError();
}

}  // namespace dc
