// Device helpers shared by the gfx950 kernels: vector types, bf16 and key
// conversions, wave/block reductions and scans (64-wide wavefronts).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#define LCT_DEV __device__ __forceinline__

namespace lct {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef short short4v __attribute__((ext_vector_type(4)));
typedef float floatx4 __attribute__((ext_vector_type(4)));
typedef int intx4 __attribute__((ext_vector_type(4)));
typedef uint32_t uintx4 __attribute__((ext_vector_type(4)));

constexpr int WAVE = 64;

// Index of the calling wave in its workgroup, as a scalar: the compiler then
// knows it is uniform across the wave (loop bounds and branches derived from
// it stay scalar instead of becoming per-lane masked loops).
LCT_DEV int wave_id() { return __builtin_amdgcn_readfirstlane((int)(threadIdx.x >> 6)); }

// Raw buffer resource over `bytes` bytes (bytes < 2^31).  Loads through it
// take a 32-bit per-lane offset and a wave-uniform offset; reads at or past
// `bytes` return zeros (hardware range check), so no clamping is needed.
constexpr int BUF_RSRC_WORD3 = 0x00020000;
constexpr int BUF_NT = 2;  // cache policy: non-temporal (streamed once)

LCT_DEV __amdgpu_buffer_rsrc_t make_rsrc(const void* base, int64_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, (int)bytes,
                                           BUF_RSRC_WORD3);
}

LCT_DEV float bf16_to_f32(uint32_t b16) { return __uint_as_float(b16 << 16); }

// Round-to-nearest-even fp32 -> bf16 bit pattern (finite values).
LCT_DEV uint32_t f32_to_bf16(float f) {
  uint32_t u = __float_as_uint(f);
  return (u + 0x7FFFu + ((u >> 16) & 1u)) >> 16;
}

// Order-preserving unsigned keys: a < b (as numbers) <=> key(a) < key(b).
LCT_DEV uint32_t key_of_i32(int32_t s) { return (uint32_t)s ^ 0x80000000u; }
LCT_DEV uint32_t key_of_f32(float f) {
  uint32_t b = __float_as_uint(f);
  if (b == 0x80000000u) b = 0u;  // -0.0 compares equal to +0.0
  return (b & 0x80000000u) ? ~b : (b | 0x80000000u);
}

template <typename T>
LCT_DEV T wave_max(T v) {
#pragma unroll
  for (int d = 32; d >= 1; d >>= 1) {
    T o = __shfl_xor(v, d, WAVE);
    v = v > o ? v : o;
  }
  return v;
}
template <typename T>
LCT_DEV T wave_min(T v) {
#pragma unroll
  for (int d = 32; d >= 1; d >>= 1) {
    T o = __shfl_xor(v, d, WAVE);
    v = v < o ? v : o;
  }
  return v;
}
template <typename T>
LCT_DEV T wave_sum(T v) {
#pragma unroll
  for (int d = 32; d >= 1; d >>= 1) v += __shfl_xor(v, d, WAVE);
  return v;
}

// Inclusive prefix sum across the 64 lanes of a wave.
LCT_DEV uint32_t wave_incl_scan(uint32_t x) {
  const int lane = threadIdx.x & 63;
#pragma unroll
  for (int d = 1; d < WAVE; d <<= 1) {
    uint32_t y = __shfl_up(x, d, WAVE);
    if (lane >= d) x += y;
  }
  return x;
}

// Block-wide exclusive prefix sum.  `lds` needs NT/64 + 1 words.  All threads
// of the block must call it.  Returns the exclusive prefix; `total` gets the
// block sum.
template <int NT>
LCT_DEV uint32_t block_excl_scan(uint32_t v, uint32_t* lds, uint32_t& total) {
  constexpr int NW = NT / WAVE;
  const int lane = threadIdx.x & 63, wid = wave_id();
  uint32_t x = wave_incl_scan(v);
  if (lane == WAVE - 1) lds[wid] = x;
  __syncthreads();
  if (wid == 0) {
    uint32_t w = lane < NW ? lds[lane] : 0u;
    uint32_t s = wave_incl_scan(w);
    if (lane < NW) lds[lane] = s - w;
    if (lane == NW - 1) lds[NW] = s;
  }
  __syncthreads();
  uint32_t r = lds[wid] + x - v;
  total = lds[NW];
  __syncthreads();
  return r;
}

// Block-wide min / max of uint32 (all threads call; result broadcast).
template <int NT>
LCT_DEV void block_minmax(uint32_t& mn, uint32_t& mx, uint32_t* lds /* 2*NT/64 */) {
  constexpr int NW = NT / WAVE;
  const int lane = threadIdx.x & 63, wid = wave_id();
  mn = wave_min(mn);
  mx = wave_max(mx);
  if (lane == 0) {
    lds[wid] = mn;
    lds[NW + wid] = mx;
  }
  __syncthreads();
  mn = lds[0];
  mx = lds[NW];
#pragma unroll
  for (int w = 1; w < NW; ++w) {
    mn = min(mn, lds[w]);
    mx = max(mx, lds[NW + w]);
  }
  __syncthreads();
}

// Number of low bits to drop so that (key - lo) >> shift fits in NB_LOG2 bits.
LCT_DEV uint32_t window_shift(uint32_t lo, uint32_t hi, int nb_log2) {
  uint32_t span = hi - lo;
  int bits = span ? 32 - __clz(span) : 0;
  return bits > nb_log2 ? (uint32_t)(bits - nb_log2) : 0u;
}

// Descending bitonic sort of n (power of two) 64-bit values in LDS by the
// NT threads of a block (every thread calls it).
template <int NT>
LCT_DEV void bitonic_sort_desc(uint64_t* a, int n) {
  for (int size = 2; size <= n; size <<= 1) {
    for (int stride = size >> 1; stride > 0; stride >>= 1) {
      for (int i = threadIdx.x; i < (n >> 1); i += NT) {
        int lo = 2 * i - (i & (stride - 1));
        int hi = lo + stride;
        bool desc = (lo & size) == 0;
        uint64_t x = a[lo], y = a[hi];
        if (desc ? (x < y) : (x > y)) {
          a[lo] = y;
          a[hi] = x;
        }
      }
      __syncthreads();
    }
  }
}

}  // namespace lct
