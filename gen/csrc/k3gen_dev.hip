// Device side of the seeded input generator: the integer-only element rules
// of k3gen.h (packed E2M1 bytes and E8M0 scale bytes), so that a whole expert
// bank can be written straight into HBM.  Same stream definition as the host
// fills; a test compares the two byte for byte.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "k3gen.h"

namespace {

constexpr uint64_t kGamma = 0x9E3779B97F4A7C15ULL;

__device__ __forceinline__ uint64_t mix64(uint64_t z) {
  z = (z ^ (z >> 30)) * 0xBF58476D1CE4E5B9ULL;
  z = (z ^ (z >> 27)) * 0x94D049BB133111EBULL;
  return z ^ (z >> 31);
}

__device__ __forceinline__ uint64_t draw(uint64_t key, uint64_t i) {
  return mix64(key + (i + 1) * kGamma);
}

// One thread per output byte index j (grid-stride); byte (start+j) of the
// stream is byte ((start+j) mod 8) of draw (start+j)/8.
__global__ void fill_bytes(uint64_t key, uint64_t start, uint64_t n, uint8_t* out) {
  const uint64_t stride = (uint64_t)gridDim.x * blockDim.x;
  for (uint64_t j = (uint64_t)blockIdx.x * blockDim.x + threadIdx.x; j < n; j += stride) {
    const uint64_t g = start + j;
    out[j] = (uint8_t)(draw(key, g >> 3) >> (8 * (g & 7)));
  }
}

// Fast path when start and n are multiples of 8 and out is 8-byte aligned:
// one draw per thread, one 8-byte store.
__global__ void fill_bytes8(uint64_t key, uint64_t start8, uint64_t n8, uint64_t* out) {
  const uint64_t stride = (uint64_t)gridDim.x * blockDim.x;
  for (uint64_t j = (uint64_t)blockIdx.x * blockDim.x + threadIdx.x; j < n8; j += stride)
    out[j] = draw(key, start8 + j);
}

__global__ void fill_scales(uint64_t key, uint64_t start, uint64_t n, int lo, uint64_t span,
                            uint8_t* out) {
  const uint64_t stride = (uint64_t)gridDim.x * blockDim.x;
  for (uint64_t j = (uint64_t)blockIdx.x * blockDim.x + threadIdx.x; j < n; j += stride) {
    const uint64_t d = draw(key, start + j);
    out[j] = (uint8_t)(127 + lo + (int)(((d >> 32) * span) >> 32));
  }
}

unsigned grid_for(uint64_t n) {
  uint64_t blocks = (n + 255) / 256;
  if (blocks > 65536) blocks = 65536;
  if (blocks == 0) blocks = 1;
  return (unsigned)blocks;
}

}  // namespace

extern "C" int k3gen_dev_bytes(uint64_t key, uint64_t start, uint64_t n, uint8_t* out,
                               void* stream) {
  if (n == 0) return 0;
  hipStream_t s = (hipStream_t)stream;
  if ((start % 8) == 0 && (n % 8) == 0 && ((uintptr_t)out % 8) == 0) {
    fill_bytes8<<<grid_for(n / 8), 256, 0, s>>>(key, start / 8, n / 8, (uint64_t*)out);
  } else {
    fill_bytes<<<grid_for(n), 256, 0, s>>>(key, start, n, out);
  }
  return (int)hipGetLastError();
}

extern "C" int k3gen_dev_scales(uint64_t key, uint64_t start, uint64_t n, int lo, int hi,
                                uint8_t* out, void* stream) {
  if (n == 0) return 0;
  fill_scales<<<grid_for(n), 256, 0, (hipStream_t)stream>>>(key, start, n, lo,
                                                          (uint64_t)(hi - lo + 1), out);
  return (int)hipGetLastError();
}
