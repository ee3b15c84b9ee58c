// Top-k position select for gfx950.
//
// Semantics (tutorial page, DSA section; CLSA explainer section 2.3): per
// row keep the k largest scores among the valid positions, equal scores
// going to the lower position, and list the chosen positions ascending,
// padded with -1.
//
// Both variants use the same exact scheme:
//   1. min/max of the row's keys -> a window of NB bins, bin = (key-lo)>>shift;
//   2. histogram -> the threshold bin tb that holds the k-th largest key;
//   3. keys in bins above tb are chosen outright (a position bitmap built
//      with wave ballots); keys in bin tb are candidates, sorted by
//      (key desc, position asc) and the first `need` of them chosen;
//      when there are too many candidates the bin is resolved exactly by
//      8-bit radix passes and an ordered scan (lowest positions first);
//   4. the bitmap is turned into the ascending position list by a
//      block-wide prefix sum of popcounts.
// The bitmap yields ascending order without any sort of the k outputs.
//
// Multi-workgroup variant (few long rows): K1 (a producer: the indexer
// scorer or k_topk_minmax) writes per-tile (min,max) and clears the row
// state; K2 builds per-tile 256-bin histograms and its last workgroup per
// row finds tb; K3 writes the bitmap and candidates and its last workgroup
// per row finishes the row.  Cross-workgroup hand-off uses device-scope
// fences and an atomic ticket; no workgroup ever waits on another.

#include "common.h"
#include "kernels.h"

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

// Descending bitonic sort of n (power of two) 64-bit values in LDS.
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

// Histogram bin of a key; keys outside the window are clamped into the end
// bins (cannot happen when the window was taken over the same keys).
LCT_DEV uint32_t bin_of(uint32_t key, uint32_t lo, uint32_t shift, uint32_t nb) {
  uint32_t b = key >= lo ? (key - lo) >> shift : 0u;
  return b < nb ? b : nb - 1u;
}

LCT_DEV uint32_t next_pow2(uint32_t x) { return x <= 1 ? 1u : 1u << (32 - __clz(x - 1)); }

// Resolve bin `tb` exactly by streaming the row (used when it holds more
// candidates than fit in LDS): radix passes over the low `shift` bits, then
// an ordered scan that takes the `need_eq` lowest positions among keys equal
// to the exact threshold.  Sets the chosen bits in `bitmap`.
template <int NT, int DT>
LCT_DEV void resolve_bin_exact(const void* row, uint32_t nv, uint32_t lo, uint32_t shift,
                               uint32_t nb, uint32_t tb, uint32_t need, uint32_t* bitmap,
                               uint32_t* lds_hist, uint32_t* lds_scan) {
  uint32_t prefix = 0, rb = shift, need_rem = need;
  while (rb > 0) {
    uint32_t w = rb < 8 ? rb : 8;
    uint32_t ds = rb - w;
    for (int i = threadIdx.x; i < 256; i += NT) lds_hist[i] = 0;
    __syncthreads();
    for (uint32_t p = threadIdx.x; p < nv; p += NT) {
      const uint32_t key = load_key<DT>(row, p);
      if (bin_of(key, lo, shift, nb) != tb) continue;
      uint32_t sub = (key - lo) & ((1u << shift) - 1u);
      if ((sub >> rb) != prefix) continue;
      atomicAdd(&lds_hist[(sub >> ds) & ((1u << w) - 1u)], 1u);
    }
    __syncthreads();
    // walk digits from the top (one thread: at most 256 bins)
    if (threadIdx.x == 0) {
      uint32_t cum = 0, dsel = 0;
      for (int b = (1 << w) - 1; b >= 0; --b) {
        uint32_t c = lds_hist[b];
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
  const uint32_t T = lo + (tb << shift) + prefix;  // exact threshold key
  uint32_t carry = 0;
  for (uint32_t base = 0; base < nv; base += NT) {
    uint32_t p = base + threadIdx.x;
    uint32_t key = p < nv ? load_key<DT>(row, p) : 0u;
    bool in = p < nv && bin_of(key, lo, shift, nb) == tb;
    bool gt = in && key > T;
    bool eq = in && key == T;
    uint32_t tot;
    uint32_t r = block_excl_scan<NT>(eq ? 1u : 0u, lds_scan, tot);
    bool sel = gt || (eq && carry + r < need_rem);
    if (sel) atomicOr(&bitmap[p >> 5], 1u << (p & 31));
    carry += tot;
  }
  __syncthreads();
}

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

// ====================================================== multi-workgroup ====

TopkMultiLayout topk_multi_layout(int rows, int64_t n, int t1) {
  TopkMultiLayout l;
  auto up = [](size_t x) { return (x + 255) & ~size_t(255); };
  l.t1 = t1;
  l.t2 = (int)((n + TOPK_K2_TILE - 1) / TOPK_K2_TILE);
  l.t3 = (int)((n + TOPK_K3_TILE - 1) / TOPK_K3_TILE);
  l.nwords = ((n + 63) / 64) * 2;
  size_t off = 0;
  l.state = off;
  off += up((size_t)rows * sizeof(TopkRowState));
  l.mm = off;
  off += up((size_t)rows * t1 * 2 * sizeof(uint32_t));
  l.hist = off;
  off += up((size_t)rows * l.t2 * TOPK_NB * sizeof(uint32_t));
  l.cands = off;
  off += up((size_t)rows * TOPK_CAP * sizeof(uint64_t));
  l.bitmap = off;
  off += up((size_t)rows * l.nwords * sizeof(uint32_t));
  l.total = off;
  return l;
}

LCT_DEV uint32_t row_nvalid(const int32_t* valid_len, int row, int64_t n, int vl_div) {
  if (!valid_len) return (uint32_t)n;
  int32_t v = valid_len[row / vl_div];
  if (v < 0) v = 0;
  return (uint32_t)(v < n ? v : n);
}

// K1 (generic producer): per-tile (min,max) of the valid keys; clears state.
template <int DT>
__global__ __launch_bounds__(256) void k_topk_minmax(const void* __restrict__ scores, int64_t n,
                                                     int64_t ld, const int32_t* valid_len,
                                                     int vl_div, uint32_t* __restrict__ mm, int t1,
                                                     TopkRowState* __restrict__ st) {
  __shared__ uint32_t lds[16];
  const int row = blockIdx.y, tile = blockIdx.x;
  const uint32_t nv = row_nvalid(valid_len, row, n, vl_div);
  const void* rp = reinterpret_cast<const char*>(scores) + (size_t)row * ld * 4;
  uint32_t mn = 0xFFFFFFFFu, mx = 0u;
  const int64_t base = (int64_t)tile * TOPK_MM_TILE;
  for (int j = 0; j < TOPK_MM_TILE / 256; ++j) {
    int64_t p = base + j * 256 + threadIdx.x;
    if (p < nv) {
      uint32_t key = load_key<DT>(rp, p);
      mn = min(mn, key);
      mx = max(mx, key);
    }
  }
  block_minmax<256>(mn, mx, lds);
  if (threadIdx.x == 0) {
    mm[((size_t)row * t1 + tile) * 2 + 0] = mn;
    mm[((size_t)row * t1 + tile) * 2 + 1] = mx;
    if (tile == 0) {
      st[row].cand_fill = 0;
      st[row].done2 = 0;
      st[row].done3 = 0;
    }
  }
}

// K2: window from the (min,max) partials, 256-bin histogram per tile; the last
// workgroup of a row sums the tile histograms and finds the threshold bin.
template <int DT>
__global__ __launch_bounds__(256) void k_topk_hist(const void* __restrict__ scores, int64_t n,
                                                   int64_t ld, int k, const int32_t* valid_len,
                                                   int vl_div, const uint32_t* __restrict__ mm, int t1,
                                                   uint32_t* __restrict__ hist, int t2,
                                                   TopkRowState* __restrict__ st) {
  __shared__ uint32_t h[TOPK_NB];
  __shared__ uint32_t lds[16];
  __shared__ uint32_t s_last;
  const int row = blockIdx.y, tile = blockIdx.x;
  const uint32_t nv = row_nvalid(valid_len, row, n, vl_div);
  const uint32_t kk = (uint32_t)k < nv ? (uint32_t)k : nv;
  // reduce the producer's partials
  uint32_t mn = 0xFFFFFFFFu, mx = 0u;
  for (int i = threadIdx.x; i < t1; i += 256) {
    mn = min(mn, mm[((size_t)row * t1 + i) * 2 + 0]);
    mx = max(mx, mm[((size_t)row * t1 + i) * 2 + 1]);
  }
  block_minmax<256>(mn, mx, lds);
  const uint32_t lo = mn;
  const uint32_t shift = nv ? window_shift(mn, mx, TOPK_NB_LOG2) : 0u;
  for (int i = threadIdx.x; i < TOPK_NB; i += 256) h[i] = 0;
  __syncthreads();
  const void* rp = reinterpret_cast<const char*>(scores) + (size_t)row * ld * 4;
  if (kk < nv) {
    const int64_t base = (int64_t)tile * TOPK_K2_TILE;
    for (int j = 0; j < TOPK_K2_TILE / 256; ++j) {
      int64_t p = base + j * 256 + threadIdx.x;
      if (p < nv) atomicAdd(&h[bin_of(load_key<DT>(rp, p), lo, shift, TOPK_NB)], 1u);
    }
  }
  __syncthreads();
  uint32_t* hp = hist + ((size_t)row * t2 + tile) * TOPK_NB;
  for (int i = threadIdx.x; i < TOPK_NB; i += 256) hp[i] = h[i];
  __threadfence();
  __syncthreads();
  if (threadIdx.x == 0) s_last = (atomicAdd(&st[row].done2, 1u) == (uint32_t)(t2 - 1));
  __syncthreads();
  if (!s_last) return;
  __threadfence();
  // last workgroup of this row: total histogram, threshold bin from the top
  for (int i = threadIdx.x; i < TOPK_NB; i += 256) {
    uint32_t c = 0;
    for (int t = 0; t < t2; ++t) c += hist[((size_t)row * t2 + t) * TOPK_NB + i];
    h[i] = c;
  }
  __syncthreads();
  if (threadIdx.x == 0) {
    TopkRowState s = st[row];
    s.lo = lo;
    s.shift = shift;
    s.nvalid = nv;
    s.kk = kk;
    if (kk >= nv) {
      s.tb = TOPK_ALL;
      s.need = 0;
      s.cand_count = 0;
    } else {
      uint32_t cum = 0;
      int b = TOPK_NB - 1;
      for (; b > 0; --b) {
        if (cum + h[b] >= kk) break;
        cum += h[b];
      }
      s.tb = (uint32_t)b;
      s.need = kk - cum;
      s.cand_count = h[b];
    }
    s.done2 = 0;
    st[row] = s;
  }
}

// K3: bitmap of positions above the threshold bin + candidate list; the last
// workgroup of a row selects among the candidates and writes the index row.
template <int DT>
__global__ __launch_bounds__(TOPK_K3_THREADS) void k_topk_emit(
    const void* __restrict__ scores, int64_t n, int64_t ld, int k, int32_t* __restrict__ idx,
    TopkRowState* __restrict__ st, uint64_t* __restrict__ cands, uint32_t* __restrict__ bitmap,
    int64_t nwords, int t3) {
  constexpr int NT = TOPK_K3_THREADS;
  __shared__ uint64_t sc[TOPK_CAP];
  __shared__ uint32_t lds_scan[NT / 64 + 2];
  __shared__ uint32_t lds_hist[256];
  __shared__ uint32_t s_last;
  const int row = blockIdx.y, tile = blockIdx.x;
  const TopkRowState s = st[row];
  const uint32_t nv = s.nvalid;
  const void* rp = reinterpret_cast<const char*>(scores) + (size_t)row * ld * 4;
  uint32_t* bm = bitmap + (size_t)row * nwords;
  uint64_t* cd = cands + (size_t)row * TOPK_CAP;
  const int lane = threadIdx.x & 63, wid = threadIdx.x >> 6;
  const int64_t tbase = (int64_t)tile * TOPK_K3_TILE;
  for (int c = wid; c < TOPK_K3_TILE / 64; c += NT / 64) {
    int64_t cb = tbase + (int64_t)c * 64;
    if (cb >= n) break;
    int64_t p = cb + lane;
    bool valid = p < nv;
    uint32_t key = valid ? load_key<DT>(rp, p) : 0u;
    uint32_t bin = bin_of(key, s.lo, s.shift, TOPK_NB);
    bool above = valid && (s.tb == TOPK_ALL || bin > s.tb);
    bool cand = valid && s.tb != TOPK_ALL && bin == s.tb;
    uint64_t am = __ballot(above);
    if (lane == 0) *reinterpret_cast<uint64_t*>(bm + (cb >> 5)) = am;
    uint64_t cm = __ballot(cand);
    if (cm && s.cand_count <= TOPK_CAP) {
      uint32_t b0 = 0;
      if (lane == 0) b0 = atomicAdd(&st[row].cand_fill, (uint32_t)__popcll(cm));
      b0 = __shfl(b0, 0, 64);
      if (cand) {
        uint32_t slot = b0 + lane_rank(cm);
        if (slot < TOPK_CAP) cd[slot] = ((uint64_t)key << 32) | (uint32_t)(~(uint32_t)p);
      }
    }
  }
  __threadfence();
  __syncthreads();
  if (threadIdx.x == 0) s_last = (atomicAdd(&st[row].done3, 1u) == (uint32_t)(t3 - 1));
  __syncthreads();
  if (!s_last) return;
  __threadfence();
  int32_t* out = idx + (size_t)row * k;
  if (s.tb != TOPK_ALL) {
    if (s.cand_count <= TOPK_CAP) {
      uint32_t m = next_pow2(s.cand_count);
      for (uint32_t i = threadIdx.x; i < m; i += NT) sc[i] = i < s.cand_count ? cd[i] : 0ull;
      __syncthreads();
      bitonic_sort_desc<NT>(sc, (int)m);
      for (uint32_t i = threadIdx.x; i < s.need; i += NT) {
        uint32_t p = ~(uint32_t)(sc[i] & 0xFFFFFFFFull);
        atomicOr(&bm[p >> 5], 1u << (p & 31));
      }
    } else {
      resolve_bin_exact<NT, DT>(rp, nv, s.lo, s.shift, TOPK_NB, s.tb, s.need, bm, lds_hist, lds_scan);
    }
    __threadfence();
    __syncthreads();
  }
  emit_bitmap<NT>(bm, (uint32_t)((nv + 31) / 32), out, (uint32_t)k, lds_scan);
  if (threadIdx.x == 0) st[row].done3 = 0;
}

hipError_t launch_topk_minmax(const void* scores, int dtype, int rows, int64_t n, int64_t ld,
                              const int32_t* valid_len, int vl_div, char* ws,
                              const TopkMultiLayout& lay, hipStream_t s) {
  dim3 grid(lay.t1, rows);
  auto st = reinterpret_cast<TopkRowState*>(ws + lay.state);
  auto mm = reinterpret_cast<uint32_t*>(ws + lay.mm);
  if (dtype == 0)
    k_topk_minmax<0><<<grid, 256, 0, s>>>(scores, n, ld, valid_len, vl_div, mm, lay.t1, st);
  else
    k_topk_minmax<1><<<grid, 256, 0, s>>>(scores, n, ld, valid_len, vl_div, mm, lay.t1, st);
  return hipGetLastError();
}

hipError_t launch_topk_hist(const void* scores, int dtype, int rows, int64_t n, int64_t ld,
                            int k, const int32_t* valid_len, int vl_div, char* ws,
                            const TopkMultiLayout& lay, hipStream_t s) {
  dim3 grid(lay.t2, rows);
  auto st = reinterpret_cast<TopkRowState*>(ws + lay.state);
  auto mm = reinterpret_cast<const uint32_t*>(ws + lay.mm);
  auto hist = reinterpret_cast<uint32_t*>(ws + lay.hist);
  if (dtype == 0)
    k_topk_hist<0><<<grid, 256, 0, s>>>(scores, n, ld, k, valid_len, vl_div, mm, lay.t1, hist, lay.t2, st);
  else
    k_topk_hist<1><<<grid, 256, 0, s>>>(scores, n, ld, k, valid_len, vl_div, mm, lay.t1, hist, lay.t2, st);
  return hipGetLastError();
}

hipError_t launch_topk_emit(const void* scores, int dtype, int32_t* idx, int rows, int64_t n,
                            int64_t ld, int k, char* ws, const TopkMultiLayout& lay,
                            hipStream_t s) {
  dim3 grid(lay.t3, rows);
  auto st = reinterpret_cast<TopkRowState*>(ws + lay.state);
  auto cands = reinterpret_cast<uint64_t*>(ws + lay.cands);
  auto bm = reinterpret_cast<uint32_t*>(ws + lay.bitmap);
  if (dtype == 0)
    k_topk_emit<0><<<grid, TOPK_K3_THREADS, 0, s>>>(scores, n, ld, k, idx, st, cands, bm,
                                                    lay.nwords, lay.t3);
  else
    k_topk_emit<1><<<grid, TOPK_K3_THREADS, 0, s>>>(scores, n, ld, k, idx, st, cands, bm,
                                                    lay.nwords, lay.t3);
  return hipGetLastError();
}

// ================================================== one workgroup per row ====

constexpr int ROW_NT = 512;
constexpr int ROW_NB_LOG2 = 11;
constexpr int ROW_NB = 1 << ROW_NB_LOG2;
constexpr int ROW_CAP = 2048;

template <int DT>
__global__ __launch_bounds__(ROW_NT) void k_topk_rows(const void* __restrict__ scores, int64_t n,
                                                      int64_t ld, int k,
                                                      const int32_t* valid_len, int vl_div,
                                                      int64_t causal_pos0,
                                                      int32_t* __restrict__ idx) {
  constexpr int NT = ROW_NT;
  __shared__ uint32_t h[ROW_NB];
  __shared__ uint64_t sc[ROW_CAP];
  __shared__ uint32_t bm[TOPK_ROW_MAX_N / 32];
  __shared__ uint32_t lds_scan[NT / 64 + 2];
  __shared__ uint32_t lds[32];
  __shared__ uint32_t s_fill;
  const int row = blockIdx.x;
  uint32_t nv;
  if (causal_pos0 >= 0) {
    int64_t v = causal_pos0 + row + 1;
    nv = (uint32_t)(v < n ? v : n);
  } else {
    nv = row_nvalid(valid_len, row, n, vl_div);
  }
  const uint32_t kk = (uint32_t)k < nv ? (uint32_t)k : nv;
  const void* rp = reinterpret_cast<const char*>(scores) + (size_t)row * ld * 4;
  int32_t* out = idx + (size_t)row * k;
  const uint32_t nwords = (nv + 31) / 32;
  const int lane = threadIdx.x & 63, wid = threadIdx.x >> 6;
  if (kk == nv) {  // every valid position is chosen
    for (uint32_t j = threadIdx.x; j < (uint32_t)k; j += NT) out[j] = j < nv ? (int32_t)j : -1;
    return;
  }
  // 1. window
  uint32_t mn = 0xFFFFFFFFu, mx = 0u;
  for (uint32_t p = threadIdx.x; p < nv; p += NT) {
    uint32_t key = load_key<DT>(rp, p);
    mn = min(mn, key);
    mx = max(mx, key);
  }
  block_minmax<NT>(mn, mx, lds);
  const uint32_t lo = mn, shift = window_shift(mn, mx, ROW_NB_LOG2);
  // 2. histogram
  for (int i = threadIdx.x; i < ROW_NB; i += NT) h[i] = 0;
  if (threadIdx.x == 0) s_fill = 0;
  __syncthreads();
  for (uint32_t p = threadIdx.x; p < nv; p += NT)
    atomicAdd(&h[bin_of(load_key<DT>(rp, p), lo, shift, ROW_NB)], 1u);
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
  // 4. bitmap of bins above tb, candidates of bin tb
  for (uint32_t cb = wid * 64; cb < nv; cb += NT) {
    uint32_t p = cb + lane;
    bool valid = p < nv;
    uint32_t key = valid ? load_key<DT>(rp, p) : 0u;
    uint32_t bin = bin_of(key, lo, shift, ROW_NB);
    bool ab = valid && bin > tb;
    bool cand = valid && bin == tb;
    uint64_t am = __ballot(ab);
    if (lane == 0) {
      bm[cb >> 5] = (uint32_t)am;
      if ((cb >> 5) + 1 < (TOPK_ROW_MAX_N / 32)) bm[(cb >> 5) + 1] = (uint32_t)(am >> 32);
    }
    uint64_t cm = __ballot(cand);
    if (cm && ccount <= ROW_CAP) {
      uint32_t b0 = 0;
      if (lane == 0) b0 = atomicAdd(&s_fill, (uint32_t)__popcll(cm));
      b0 = __shfl(b0, 0, 64);
      if (cand) sc[b0 + lane_rank(cm)] = ((uint64_t)key << 32) | (uint32_t)(~p);
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
    resolve_bin_exact<NT, DT>(rp, nv, lo, shift, ROW_NB, tb, need, bm, h, lds_scan);
  }
  __syncthreads();
  emit_bitmap<NT>(bm, nwords, out, (uint32_t)k, lds_scan);
}

hipError_t launch_topk_rows(const void* scores, int dtype, int32_t* idx, int rows, int64_t n,
                            int64_t ld, int k, const int32_t* valid_len, int vl_div,
                            int64_t causal_pos0, hipStream_t s) {
  if (dtype == 0)
    k_topk_rows<0><<<rows, ROW_NT, 0, s>>>(scores, n, ld, k, valid_len, vl_div, causal_pos0, idx);
  else
    k_topk_rows<1><<<rows, ROW_NT, 0, s>>>(scores, n, ld, k, valid_len, vl_div, causal_pos0, idx);
  return hipGetLastError();
}

}  // namespace lct
