// Device-side pieces of the top-k select shared by the select kernels and
// by the causal prefill index (its rows that need a whole-row select):
// key conversion, histogram bins, the bitmap -> ascending list expansion, the
// exact threshold inside a bin, and the one-workgroup select of one row.
#pragma once

#include "common.h"

namespace lct {

template <int DT>
LCT_DEV uint32_t load_key(const void* p, int64_t i) {
  if (DT == 0) return key_of_i32(reinterpret_cast<const int32_t*>(p)[i]);
  return key_of_f32(reinterpret_cast<const float*>(p)[i]);
}

LCT_DEV uint32_t lane_rank(uint64_t mask) {
  return __builtin_amdgcn_mbcnt_hi((uint32_t)(mask >> 32),
                                   __builtin_amdgcn_mbcnt_lo((uint32_t)mask, 0u));
}

// Histogram bin of a key; keys outside the window are clamped into the end
// bins (cannot happen when the window was taken over the same keys).
LCT_DEV uint32_t bin_of(uint32_t key, uint32_t lo, uint32_t shift, uint32_t nb) {
  uint32_t b = key >= lo ? (key - lo) >> shift : 0u;
  return b < nb ? b : nb - 1u;
}

LCT_DEV uint32_t next_pow2(uint32_t x) { return x <= 1 ? 1u : 1u << (32 - __clz(x - 1)); }

// Ascending position list from a bitmap (all threads of the block).
template <int NT>
LCT_DEV void emit_bitmap(const uint32_t* bitmap, uint32_t nwords, int32_t* out, uint32_t k,
                         uint32_t* lds_scan) {
  constexpr int W = 4;
  uint32_t carry = 0;
  for (uint32_t base = 0; base < nwords; base += NT * W) {
    uint32_t w0 = base + threadIdx.x * W;
    uint32_t words[W];
    uint32_t cnt = 0;
#pragma unroll
    for (int j = 0; j < W; ++j) {
      words[j] = (w0 + j < nwords) ? bitmap[w0 + j] : 0u;
      cnt += __popc(words[j]);
    }
    uint32_t tot;
    uint32_t off = carry + block_excl_scan<NT>(cnt, lds_scan, tot);
#pragma unroll
    for (int j = 0; j < W; ++j) {
      uint32_t wv = words[j];
      while (wv) {
        uint32_t b = __ffs(wv) - 1;
        wv &= wv - 1;
        if (off < k) out[off] = (int32_t)((w0 + j) * 32 + b);
        ++off;
      }
    }
    carry += tot;
  }
  for (uint32_t j = carry + threadIdx.x; j < k; j += NT) out[j] = -1;
}

LCT_DEV uint32_t row_nvalid(const int32_t* valid_len, int row, int64_t n, int vl_div) {
  if (!valid_len) return (uint32_t)n;
  int32_t v = valid_len[row / vl_div];
  if (v < 0) v = 0;
  return (uint32_t)(v < n ? v : n);
}

// Exact threshold inside bin tb by 8-bit radix passes over the row (used when
// the bin holds more candidates than fit in LDS).  Returns the exact key T;
// need_eq gets how many keys equal to T are taken (the lowest positions).
template <int NT, int DT>
LCT_DEV uint32_t exact_threshold(const void* row, uint32_t nv, uint32_t lo, uint32_t shift,
                                 uint32_t nb, uint32_t tb, uint32_t need, uint32_t& need_eq,
                                 uint32_t* lds_hist, uint32_t* lds_scan) {
  uint32_t prefix = 0, rb = shift, need_rem = need;
  while (rb > 0) {
    const uint32_t w = rb < 8 ? rb : 8;
    const uint32_t ds = rb - w;
    for (int i = threadIdx.x; i < 256; i += NT) lds_hist[i] = 0;
    __syncthreads();
    for (uint32_t p = threadIdx.x; p < nv; p += NT) {
      const uint32_t key = load_key<DT>(row, p);
      if (bin_of(key, lo, shift, nb) != tb) continue;
      const uint32_t sub = (key - lo) & ((1u << shift) - 1u);
      if ((sub >> rb) != prefix) continue;
      atomicAdd(&lds_hist[(sub >> ds) & ((1u << w) - 1u)], 1u);
    }
    __syncthreads();
    if (threadIdx.x == 0) {
      uint32_t cum = 0, dsel = 0;
      for (int b = (1 << w) - 1; b >= 0; --b) {
        const uint32_t c = lds_hist[b];
        if (cum + c >= need_rem) {
          dsel = (uint32_t)b;
          break;
        }
        cum += c;
      }
      lds_scan[0] = dsel;
      lds_scan[1] = need_rem - cum;
    }
    __syncthreads();
    prefix = (prefix << w) | lds_scan[0];
    need_rem = lds_scan[1];
    rb = ds;
    __syncthreads();
  }
  need_eq = need_rem;
  return lo + (tb << shift) + prefix;
}


constexpr int ROW_NT = 512;
constexpr int ROW_NB_LOG2 = 11;
constexpr int ROW_NB = 1 << ROW_NB_LOG2;
constexpr int ROW_CAP = 2048;
constexpr int ROW_RC = 16;  // keys per thread kept in registers (rows up to 8192 keys)

// LDS of the one-row select; BMW bitmap words (rows of up to 32 * BMW keys).
template <int BMW>
struct RowSelSmem {
  uint32_t h[ROW_NB];
  uint64_t sc[ROW_CAP];
  uint32_t bm[BMW];
  uint32_t lds_scan[ROW_NT / 64 + 2];
  uint32_t lds[32];
  uint32_t s_fill;
};

// Top-k of one row by the ROW_NT threads of a workgroup (all call it): the
// row's keys are rp[0, nv) (int32 scores for DT = 0, fp32 for DT = 1); out
// gets the min(k, nv) chosen positions ascending, then -1 up to k.  Rows of up
// to ROW_NT * ROW_RC keys are read once into registers (key j*ROW_NT +
// threadIdx.x in kr[j]: the order every pass below walks the row in); longer
// rows are read again by each pass.  The caller separates two calls on the
// same LDS with a barrier.
template <int DT, int BMW>
LCT_DEV void row_select(const void* rp, uint32_t nv, int k, int32_t* __restrict__ out, RowSelSmem<BMW>& sm) {
  constexpr int NT = ROW_NT;
  uint32_t* const h = sm.h;
  uint64_t* const sc = sm.sc;
  uint32_t* const bm = sm.bm;
  uint32_t* const lds_scan = sm.lds_scan;
  uint32_t* const lds = sm.lds;
  uint32_t& s_fill = sm.s_fill;
  const uint32_t kk = (uint32_t)k < nv ? (uint32_t)k : nv;
  const uint32_t nwords = (nv + 31) / 32;
  const int lane = threadIdx.x & 63, wid = wave_id();
  if (kk == nv) {  // every valid position is chosen
    for (uint32_t j = threadIdx.x; j < (uint32_t)k; j += NT) out[j] = j < nv ? (int32_t)j : -1;
    return;
  }
  const bool cached = nv <= (uint32_t)(NT * ROW_RC);
  uint32_t kr[ROW_RC];
  if (cached) {
#pragma unroll
    for (int j = 0; j < ROW_RC; ++j) {
      const uint32_t p = (uint32_t)(j * NT) + threadIdx.x;
      kr[j] = p < nv ? load_key<DT>(rp, p) : 0u;
    }
  }
  // 1. window
  uint32_t mn = 0xFFFFFFFFu, mx = 0u;
  if (cached) {
#pragma unroll
    for (int j = 0; j < ROW_RC; ++j)
      if ((uint32_t)(j * NT) + threadIdx.x < nv) {
        mn = min(mn, kr[j]);
        mx = max(mx, kr[j]);
      }
  } else {
    for (uint32_t p = threadIdx.x; p < nv; p += NT) {
      uint32_t key = load_key<DT>(rp, p);
      mn = min(mn, key);
      mx = max(mx, key);
    }
  }
  block_minmax<NT>(mn, mx, lds);
  const uint32_t lo = mn, shift = window_shift(mn, mx, ROW_NB_LOG2);
  // 2. histogram
  for (int i = threadIdx.x; i < ROW_NB; i += NT) h[i] = 0;
  if (threadIdx.x == 0) s_fill = 0;
  __syncthreads();
  if (cached) {
#pragma unroll
    for (int j = 0; j < ROW_RC; ++j)
      if ((uint32_t)(j * NT) + threadIdx.x < nv) atomicAdd(&h[bin_of(kr[j], lo, shift, ROW_NB)], 1u);
  } else {
    for (uint32_t p = threadIdx.x; p < nv; p += NT)
      atomicAdd(&h[bin_of(load_key<DT>(rp, p), lo, shift, ROW_NB)], 1u);
  }
  __syncthreads();
  // 3. threshold bin: suffix sums, each thread owns ROW_NB / NT consecutive bins
  constexpr int BPT = ROW_NB / NT;
  uint32_t mine = 0;
#pragma unroll
  for (int j = 0; j < BPT; ++j) mine += h[threadIdx.x * BPT + j];
  // exclusive prefix from the top: reverse thread order
  uint32_t tot;
  uint32_t pre = block_excl_scan<NT>(mine, lds_scan, tot);  // count in lower bins
  // count strictly above this thread's bins = tot - pre - mine
  uint32_t above = tot - pre - mine;
  if (above < kk && above + mine >= kk) {
    uint32_t cum = above;
    for (int j = BPT - 1; j >= 0; --j) {
      uint32_t c = h[threadIdx.x * BPT + j];
      if (cum + c >= kk) {
        lds[0] = (uint32_t)(threadIdx.x * BPT + j);
        lds[1] = kk - cum;
        lds[2] = c;
        break;
      }
      cum += c;
    }
  }
  __syncthreads();
  const uint32_t tb = lds[0], need = lds[1], ccount = lds[2];
  __syncthreads();
  // 4. bitmap of bins above tb, candidates of bin tb (a wave takes 64
  // consecutive positions cb .. cb + 63)
  auto mark = [&](uint32_t cb, uint32_t key) {
    const uint32_t p = cb + lane;
    const bool valid = p < nv;
    const uint32_t bin = bin_of(key, lo, shift, ROW_NB);
    const bool ab = valid && bin > tb;
    const bool cand = valid && bin == tb;
    const uint64_t am = __ballot(ab);
    if (lane == 0) {
      bm[cb >> 5] = (uint32_t)am;
      if ((cb >> 5) + 1 < BMW) bm[(cb >> 5) + 1] = (uint32_t)(am >> 32);
    }
    const uint64_t cm = __ballot(cand);
    if (cm && ccount <= ROW_CAP) {
      uint32_t b0 = 0;
      if (lane == 0) b0 = atomicAdd(&s_fill, (uint32_t)__popcll(cm));
      b0 = __shfl(b0, 0, 64);
      if (cand) sc[b0 + lane_rank(cm)] = ((uint64_t)key << 32) | (uint32_t)(~p);
    }
  };
  if (cached) {
#pragma unroll
    for (int j = 0; j < ROW_RC; ++j) {
      const uint32_t cb = (uint32_t)(j * NT + wid * 64);
      if (cb < nv) mark(cb, kr[j]);  // wave-uniform
    }
  } else {
    for (uint32_t cb = wid * 64; cb < nv; cb += NT) {
      const uint32_t p = cb + lane;
      mark(cb, p < nv ? load_key<DT>(rp, p) : 0u);
    }
  }
  __syncthreads();
  if (ccount <= ROW_CAP) {
    uint32_t m = next_pow2(ccount);
    for (uint32_t i = ccount + threadIdx.x; i < m; i += NT) sc[i] = 0ull;
    __syncthreads();
    bitonic_sort_desc<NT>(sc, (int)m);
    for (uint32_t i = threadIdx.x; i < need; i += NT) {
      uint32_t p = ~(uint32_t)(sc[i] & 0xFFFFFFFFull);
      atomicOr(&bm[p >> 5], 1u << (p & 31));
    }
  } else {
    uint32_t need_eq;
    const uint32_t T = exact_threshold<NT, DT>(rp, nv, lo, shift, ROW_NB, tb, need, need_eq, h, lds_scan);
    uint32_t carry = 0;
    for (uint32_t base = 0; base < nv; base += NT) {
      const uint32_t p = base + threadIdx.x;
      const uint32_t key = p < nv ? load_key<DT>(rp, p) : 0u;
      const bool in = p < nv && bin_of(key, lo, shift, ROW_NB) == tb;
      const bool gt = in && key > T;
      const bool eq = in && key == T;
      uint32_t tot2;
      const uint32_t r = block_excl_scan<NT>(eq ? 1u : 0u, lds_scan, tot2);
      if (gt || (eq && carry + r < need_eq)) atomicOr(&bm[p >> 5], 1u << (p & 31));
      carry += tot2;
    }
  }
  __syncthreads();
  emit_bitmap<NT>(bm, nwords, out, (uint32_t)k, lds_scan);
}

}  // namespace lct
