// Device-side filler for the seeded synthetic inputs: the same SplitMix64
// counter-based generator and value mappings as synth/__init__.py,
// implemented independently so multi-GiB tensors can be produced directly
// in HBM.  Nothing of the attention method is computed here.
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace {

constexpr uint64_t GAMMA = 0x9E3779B97F4A7C15ull;

__host__ __device__ inline uint64_t mix64(uint64_t z) {
  z = (z ^ (z >> 30)) * 0xBF58476D1CE4E5B9ull;
  z = (z ^ (z >> 27)) * 0x94D049BB133111EBull;
  return z ^ (z >> 31);
}

__device__ inline uint64_t word(uint64_t key, uint64_t j) { return mix64(key + (j + 1) * GAMMA); }

__device__ inline uint16_t f32_to_bf16_rne(float f) {
  uint32_t u = __float_as_uint(f);
  return (uint16_t)((u + 0x7FFFu + ((u >> 16) & 1u)) >> 16);
}

// kind 0: int8 in [-8, 7] (16 per word)
__global__ void k_fill_i8u4(int8_t* __restrict__ dst, uint64_t key, int64_t n) {
  const int64_t nw = (n + 15) / 16;
  for (int64_t w = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; w < nw;
       w += (int64_t)gridDim.x * blockDim.x) {
    uint64_t x = word(key, (uint64_t)w);
    const int64_t e0 = w * 16;
    if (e0 + 16 <= n) {
      uint32_t out[4];
      for (int q = 0; q < 4; ++q) {
        uint32_t v = 0;
        for (int b = 0; b < 4; ++b) {
          int nib = (int)((x >> (4 * (q * 4 + b))) & 15u) - 8;
          v |= ((uint32_t)(uint8_t)(int8_t)nib) << (8 * b);
        }
        out[q] = v;
      }
      *reinterpret_cast<uint4*>(dst + e0) = make_uint4(out[0], out[1], out[2], out[3]);
    } else {
      for (int i = 0; i < 16 && e0 + i < n; ++i) dst[e0 + i] = (int8_t)((int)((x >> (4 * i)) & 15u) - 8);
    }
  }
}

// kind 1: the same integers as bf16
__global__ void k_fill_bf16u4(uint16_t* __restrict__ dst, uint64_t key, int64_t n) {
  const int64_t nw = (n + 15) / 16;
  for (int64_t w = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; w < nw;
       w += (int64_t)gridDim.x * blockDim.x) {
    uint64_t x = word(key, (uint64_t)w);
    const int64_t e0 = w * 16;
    for (int i = 0; i < 16 && e0 + i < n; ++i)
      dst[e0 + i] = f32_to_bf16_rne((float)((int)((x >> (4 * i)) & 15u) - 8));
  }
}

// kind 2: Irwin-Hall(12) approximately N(0,1), rounded to bf16
__global__ void k_fill_bf16n(uint16_t* __restrict__ dst, uint64_t key, int64_t n) {
  for (int64_t e = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; e < n;
       e += (int64_t)gridDim.x * blockDim.x) {
    int64_t s = 0;
    for (int t = 0; t < 3; ++t) {
      uint64_t x = word(key, (uint64_t)e * 3 + t);
      for (int i = 0; i < 4; ++i) s += (int64_t)((x >> (16 * i)) & 0xFFFFu);
    }
    const int32_t d = (int32_t)(s - 6 * 65536);
    dst[e] = f32_to_bf16_rne((float)d * (1.0f / 65536.0f));
  }
}

}  // namespace

extern "C" {

// Fill `n` elements of `dst` (device memory) with generator kind `kind`
// (0 int8 [-8,7], 1 bf16 integers [-8,7], 2 bf16 ~N(0,1)) for tensor `tid`
// under run seed `seed`.  Returns 0 on success, 1 on a bad argument, 2 on a
// HIP error.
int synth_fill(void* dst, int kind, uint64_t seed, uint64_t tid, int64_t n, void* stream) {
  if (!dst || n < 0 || seed >= (1ull << 32) || tid >= (1ull << 32)) return 1;
  if (kind == 0 && ((uintptr_t)dst % 16) != 0) return 1;
  if (n == 0) return 0;
  const uint64_t key = mix64((seed | (tid << 32)) + GAMMA);
  hipStream_t st = reinterpret_cast<hipStream_t>(stream);
  const int threads = 256;
  int64_t work = kind == 2 ? n : (n + 15) / 16;
  int64_t blocks = (work + threads - 1) / threads;
  if (blocks > 65536) blocks = 65536;
  switch (kind) {
    case 0: k_fill_i8u4<<<(unsigned)blocks, threads, 0, st>>>((int8_t*)dst, key, n); break;
    case 1: k_fill_bf16u4<<<(unsigned)blocks, threads, 0, st>>>((uint16_t*)dst, key, n); break;
    case 2: k_fill_bf16n<<<(unsigned)blocks, threads, 0, st>>>((uint16_t*)dst, key, n); break;
    default: return 1;
  }
  return hipGetLastError() == hipSuccess ? 0 : 2;
}

}
