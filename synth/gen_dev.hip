// Seeded synthetic gradient values, GPU side (gfx950).
//
// Input generation only: none of the reduction's arithmetic lives here.  It is
// the device twin of synth/gen_host.c (same definition, integer operations
// only), so a slab filled here holds exactly the bytes the host generator
// produces for the same (seed, stream, column).  The definition is written out
// in gen_host.c's header.
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace {

constexpr uint64_t kG = 0x9E3779B97F4A7C15ULL;

__host__ __device__ inline uint64_t mix(uint64_t z) {
  z ^= z >> 30;
  z *= 0xBF58476D1CE4E5B9ULL;
  z ^= z >> 27;
  z *= 0x94D049BB133111EBULL;
  z ^= z >> 31;
  return z;
}

__device__ inline uint32_t value_bits(uint64_t key, uint64_t i, uint32_t C, uint32_t E, bool bf16) {
  uint64_t h = mix(key + (i + 1) * kG);
  uint64_t h2 = mix(h + kG);
  int64_t k = (int64_t)(h & 0xFFFF) + (int64_t)((h >> 16) & 0xFFFF) +
              (int64_t)((h >> 32) & 0xFFFF) + (int64_t)(h >> 48) - 131070;
  uint32_t neg = (k < 0) || (k == 0 && (h2 & 1));
  uint64_t mag = (uint64_t)(k < 0 ? -k : k);
  uint64_t n = ((mag << 24) | (h2 >> 40)) * (uint64_t)C;
  if (n == 0) return bf16 ? (neg << 15) : (neg << 31);
  int L = 64 - __builtin_clzll(n);
  uint32_t bexp = (uint32_t)(L - 1 - 24 - (int)E + 127);
  if (bf16) {
    uint64_t sig = L > 8 ? n >> (L - 8) : n << (8 - L);
    return (neg << 15) | (bexp << 7) | (uint32_t)(sig & 0x7F);
  }
  uint64_t sig = L > 24 ? n >> (L - 24) : n << (24 - L);
  return (neg << 31) | (bexp << 23) | (uint32_t)(sig & 0x7FFFFF);
}

// Row r of a [rows, ld] slab gets stream stream0 + r: position j of the row
// holds the value of column col0 + j, for j in [0, ncols).
__global__ void fill_slab(int bf16, uint64_t seed, uint64_t stream0, uint32_t C, uint32_t E,
                          int64_t ld, int64_t ncols, int64_t col0, void* base) {
  const int64_t r = blockIdx.y;
  const uint64_t key = mix(mix(seed + kG) + (stream0 + (uint64_t)r + 1) * kG);
  const int64_t step = (int64_t)gridDim.x * blockDim.x;
  for (int64_t j = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; j < ncols; j += step) {
    uint32_t v = value_bits(key, (uint64_t)(col0 + j), C, E, bf16 != 0);
    if (bf16)
      reinterpret_cast<uint16_t*>(base)[r * ld + j] = (uint16_t)v;
    else
      reinterpret_cast<uint32_t*>(base)[r * ld + j] = v;
  }
}

}  // namespace

// Fill a [rows, ld] slab (dtype 0 = bf16, 1 = fp32) on `stream` with columns
// [col0, col0 + ncols) of every row's stream.  Returns 0 on success, -1 on a
// bad argument, or the HIP error code of the launch.
extern "C" int synth_fill_slab_device_at(int dtype, uint64_t seed, uint64_t stream0, uint32_t C,
                                         uint32_t E, int32_t rows, int64_t ld, int64_t ncols,
                                         int64_t col0, void* base, hipStream_t stream) {
  if (base == nullptr || rows <= 0 || rows > 65535 || ncols < 0 || ld < ncols || col0 < 0 ||
      (dtype != 0 && dtype != 1))
    return -1;
  if (ncols == 0) return 0;
  int64_t blocks = (ncols + 255) / 256;
  if (blocks > 8192) blocks = 8192;
  hipLaunchKernelGGL(fill_slab, dim3((unsigned)blocks, (unsigned)rows), dim3(256), 0, stream,
                     dtype == 0 ? 1 : 0, seed, stream0, C, E, ld, ncols, col0, base);
  return (int)hipGetLastError();
}

extern "C" int synth_fill_slab_device(int dtype, uint64_t seed, uint64_t stream0, uint32_t C,
                                      uint32_t E, int32_t rows, int64_t ld, int64_t ncols,
                                      void* base, hipStream_t stream) {
  return synth_fill_slab_device_at(dtype, seed, stream0, C, E, rows, ld, ncols, 0, base, stream);
}
