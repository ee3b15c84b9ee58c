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
// Multi-workgroup variant (few long rows), four kernels whose boundaries are
// the only hand-offs between workgroups: K1 (a producer: the indexer scorer
// or k_topk_minmax) writes per-tile (min,max) and clears the row's candidate
// counter and 256-bin histogram; K2 adds each tile's histogram into the row
// histogram with atomics; K3 finds tb from it, writes the bitmap words, the
// candidates and per-tile chosen counts; K4 resolves the candidates and
// expands the bitmap into the ascending list.

#include "common.h"
#include "kernels.h"
#include "topk_dev.h"

namespace lct {

// ====================================================== multi-workgroup ====

TopkMultiLayout topk_multi_layout(int rows, int64_t n, int t1) {
  TopkMultiLayout l;
  auto up = [](size_t x) { return (x + 255) & ~size_t(255); };
  l.t1 = t1;
  l.k2_tile = TOPK_K2_TILE;
  l.t2 = (int)((n + l.k2_tile - 1) / l.k2_tile);
  l.t3 = (int)((n + TOPK_K3_TILE - 1) / TOPK_K3_TILE);
  l.t4 = (int)((n + TOPK_K4_TILE - 1) / TOPK_K4_TILE);
  l.nwords = ((n + 63) / 64) * 2;
  size_t off = 0;
  l.state = off;
  off += up((size_t)rows * sizeof(TopkRowState));
  l.mm = off;
  off += up((size_t)rows * t1 * 2 * sizeof(uint32_t));
  l.hist = off;
  off += up((size_t)rows * TOPK_NB * sizeof(uint32_t));
  l.cands = off;
  off += up((size_t)rows * TOPK_CAP * sizeof(uint64_t));
  l.bitmap = off;
  off += up((size_t)rows * l.nwords * sizeof(uint32_t));
  l.tilecnt = off;
  off += up((size_t)rows * l.t3 * sizeof(uint32_t));
  l.total = off;
  return l;
}

// K1 (generic producer): per-tile (min,max) of the valid keys; clears the
// row's candidate counter.  The indexer scorer does the same when it feeds
// the select directly.
template <int DT>
__global__ __launch_bounds__(256) void k_topk_minmax(const void* __restrict__ scores, int64_t n,
                                                     int64_t ld, const int32_t* valid_len,
                                                     int vl_div, uint32_t* __restrict__ mm, int t1,
                                                     TopkRowState* __restrict__ st,
                                                     uint32_t* __restrict__ hist) {
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
    if (tile == 0) st[row].cand_fill = 0;
  }
  if (tile == 0) hist[(size_t)row * TOPK_NB + threadIdx.x % TOPK_NB] = 0u;
}

// Window of a row from the producer's (min,max) partials.  The caller loads
// this thread's first partial (index threadIdx.x) before anything else, so
// that waiting for it does not also wait for loads issued later (vmcnt
// counts in issue order); further partials (t1 > NT) are read here.
LCT_DEV uint2 first_partial(const uint32_t* mm_row, int t1) {
  return (int)threadIdx.x < t1 ? reinterpret_cast<const uint2*>(mm_row)[threadIdx.x]
                               : uint2{0xFFFFFFFFu, 0u};
}
template <int NT>
LCT_DEV void row_window(const uint32_t* mm_row, int t1, uint2 first, uint32_t nv, uint32_t& lo,
                        uint32_t& shift, uint32_t* lds) {
  uint32_t mn = first.x, mx = first.y;
  for (int i = threadIdx.x + NT; i < t1; i += NT) {
    mn = min(mn, mm_row[2 * i]);
    mx = max(mx, mm_row[2 * i + 1]);
  }
  block_minmax<NT>(mn, mx, lds);
  lo = mn;
  shift = nv ? window_shift(mn, mx, TOPK_NB_LOG2) : 0u;
}

// K2: 256-bin histogram of one tile of a row (window from the partials).
template <int DT>
__global__ __launch_bounds__(256) void k_topk_hist(const void* __restrict__ scores, int64_t n,
                                                   int64_t ld, int k, const int32_t* valid_len,
                                                   int vl_div, const uint32_t* __restrict__ mm,
                                                   int t1, uint32_t* __restrict__ hist,
                                                   int64_t tile_len) {
  __shared__ uint32_t h[TOPK_NB];
  __shared__ uint32_t lds[16];
  const int row = blockIdx.y, tile = blockIdx.x;
  const uint32_t nv = row_nvalid(valid_len, row, n, vl_div);
  const uint32_t kk = (uint32_t)k < nv ? (uint32_t)k : nv;
  const void* rp = reinterpret_cast<const char*>(scores) + (size_t)row * ld * 4;
  const int64_t base = (int64_t)tile * tile_len;
  const int64_t end = base + tile_len < (int64_t)nv ? base + tile_len : (int64_t)nv;
  const uint32_t* mm_row = mm + (size_t)row * t1 * 2;
  const uint2 first = first_partial(mm_row, t1);
  // then the tile's keys; the window reduction overlaps them
  constexpr int PF = 16;
  uint32_t kbuf[PF];
#pragma unroll
  for (int j = 0; j < PF; ++j) {
    const int64_t p = base + j * 256 + threadIdx.x;
    kbuf[j] = load_key<DT>(rp, p < end ? p : (end > 0 ? end - 1 : 0));  // clamped, in bounds
  }
  uint32_t lo, shift;
  row_window<256>(mm_row, t1, first, nv, lo, shift, lds);
  for (int i = threadIdx.x; i < TOPK_NB; i += 256) h[i] = 0;
  __syncthreads();
  if (kk < nv) {
#pragma unroll
    for (int j = 0; j < PF; ++j)
      if (base + j * 256 + threadIdx.x < end) atomicAdd(&h[bin_of(kbuf[j], lo, shift, TOPK_NB)], 1u);
    for (int64_t p = base + PF * 256 + threadIdx.x; p < end; p += 256)
      atomicAdd(&h[bin_of(load_key<DT>(rp, p), lo, shift, TOPK_NB)], 1u);
  }
  __syncthreads();
  // accumulate into the row histogram (cleared by the producer kernel)
  uint32_t* hp = hist + (size_t)row * TOPK_NB;
  for (int i = threadIdx.x; i < TOPK_NB; i += 256)
    if (h[i]) atomicAdd(&hp[i], h[i]);
}

struct RowSel {
  uint32_t lo, shift, tb, need, ccount;
};

// Threshold bin of a row from its histogram (every caller derives the same
// values).  NT >= TOPK_NB.  `first` and `c` are loaded by the caller ahead of
// its other loads: first_partial(mm_row, t1) and hist_entry(hist_row).
LCT_DEV uint32_t hist_entry(const uint32_t* hist_row) {
  // thread t < NB owns bin NB-1-t
  return (int)threadIdx.x < TOPK_NB ? hist_row[TOPK_NB - 1 - threadIdx.x] : 0u;
}
template <int NT>
LCT_DEV RowSel row_select_params(const uint32_t* mm_row, int t1, uint2 first, uint32_t c,
                                 uint32_t nv, uint32_t kk, uint32_t* lds_scan,
                                 uint32_t* lds_small) {
  static_assert(NT >= TOPK_NB, "one thread per bin");
  RowSel r;
  row_window<NT>(mm_row, t1, first, nv, r.lo, r.shift, lds_small);
  if (kk >= nv) {
    r.tb = TOPK_ALL;
    r.need = 0;
    r.ccount = 0;
    return r;
  }
  // an exclusive scan in thread order counts the keys in higher bins
  uint32_t tot;
  const uint32_t higher = block_excl_scan<NT>(c, lds_scan, tot);
  if ((int)threadIdx.x < TOPK_NB && higher < kk && higher + c >= kk) {
    lds_small[0] = (uint32_t)(TOPK_NB - 1 - threadIdx.x);
    lds_small[1] = kk - higher;
    lds_small[2] = c;
  }
  __syncthreads();
  r.tb = lds_small[0];
  r.need = lds_small[1];
  r.ccount = lds_small[2];
  __syncthreads();
  return r;
}

// K3: bitmap words of positions above the threshold bin and the list of
// candidates in it, for one tile of a row.
template <int DT>
__global__ __launch_bounds__(TOPK_K3_THREADS) void k_topk_emit(
    const void* __restrict__ scores, int64_t n, int64_t ld, int k, const int32_t* valid_len,
    int vl_div, const uint32_t* __restrict__ mm, int t1, const uint32_t* __restrict__ hist,
    TopkRowState* __restrict__ st, uint64_t* __restrict__ cands,
    uint32_t* __restrict__ bitmap, int64_t nwords, uint32_t* __restrict__ tilecnt, int t3) {
  constexpr int NT = TOPK_K3_THREADS;
  __shared__ uint32_t lds_scan[NT / 64 + 2];
  __shared__ uint32_t lds_small[2 * (NT / 64) + 4];
  __shared__ uint32_t wave_cnt[NT / 64];
  __shared__ uint32_t wave_cand[NT / 64 + 2];
  const int row = blockIdx.y, tile = blockIdx.x;
  const uint32_t nv = row_nvalid(valid_len, row, n, vl_div);
  const uint32_t kk = (uint32_t)k < nv ? (uint32_t)k : nv;
  const void* rp = reinterpret_cast<const char*>(scores) + (size_t)row * ld * 4;
  const int lane = threadIdx.x & 63, wid = wave_id();
  const int64_t tbase = (int64_t)tile * TOPK_K3_TILE;
  constexpr int CH = TOPK_K3_TILE / NT;  // 64-position chunks per wave
  // the row's window partial and histogram entry first, then the keys of
  // this thread's chunks
  const uint32_t* mm_row = mm + (size_t)row * t1 * 2;
  const uint2 first = first_partial(mm_row, t1);
  const uint32_t hc = hist_entry(hist + (size_t)row * TOPK_NB);
  uint32_t kbuf[CH];
#pragma unroll
  for (int c = 0; c < CH; ++c) {
    const int64_t p = tbase + (int64_t)(c * (NT / 64) + wid) * 64 + lane;
    kbuf[c] = load_key<DT>(rp, p < nv ? p : (nv > 0 ? nv - 1 : 0));  // clamped, in bounds
  }
  const RowSel s = row_select_params<NT>(mm_row, t1, first, hc, nv, kk, lds_scan, lds_small);
  if (tile == 0 && threadIdx.x == 0) {
    TopkRowState w = st[row];
    w.lo = s.lo;
    w.shift = s.shift;
    w.tb = s.tb;
    w.need = s.need;
    w.cand_count = s.ccount;
    w.nvalid = nv;
    w.kk = kk;
    st[row] = w;
  }
  uint32_t* bm = bitmap + (size_t)row * nwords;
  uint64_t* cd = cands + (size_t)row * TOPK_CAP;
  // pass 1: bitmap words and this wave's counts (chosen keys, candidates)
  uint32_t nabove = 0, ncand = 0;
#pragma unroll
  for (int c = 0; c < CH; ++c) {
    const int64_t cb = tbase + (int64_t)(c * (NT / 64) + wid) * 64;
    if (cb >= n) break;
    const int64_t p = cb + lane;
    const bool valid = p < nv;
    const uint32_t bin = bin_of(kbuf[c], s.lo, s.shift, TOPK_NB);
    const uint64_t am = __ballot(valid && (s.tb == TOPK_ALL || bin > s.tb));
    if (lane == 0) *reinterpret_cast<uint64_t*>(bm + (cb >> 5)) = am;
    nabove += (uint32_t)__popcll(am);
    ncand += (uint32_t)__popcll(__ballot(valid && s.tb != TOPK_ALL && bin == s.tb));
  }
  if (lane == 0) {
    wave_cnt[wid] = nabove;
    wave_cand[wid] = ncand;
  }
  __syncthreads();
  if (threadIdx.x == 0) {
    uint32_t t = 0, cs = 0;
    for (int w = 0; w < NT / 64; ++w) {
      t += wave_cnt[w];
      const uint32_t x = wave_cand[w];
      wave_cand[w] = cs;
      cs += x;
    }
    tilecnt[(size_t)row * t3 + tile] = t;
    // one slot reservation per workgroup
    wave_cand[NT / 64] = (cs && s.ccount <= TOPK_CAP) ? atomicAdd(&st[row].cand_fill, cs) : 0u;
    wave_cand[NT / 64 + 1] = cs;
  }
  __syncthreads();
  if (wave_cand[NT / 64 + 1] == 0 || s.ccount > TOPK_CAP) return;  // uniform over the block
  // pass 2: candidates (key, ~position) into the reserved slots
  uint32_t slot = wave_cand[NT / 64] + wave_cand[wid];
#pragma unroll
  for (int c = 0; c < CH; ++c) {
    const int64_t cb = tbase + (int64_t)(c * (NT / 64) + wid) * 64;
    if (cb >= n) break;
    const int64_t p = cb + lane;
    const bool cand = p < nv && bin_of(kbuf[c], s.lo, s.shift, TOPK_NB) == s.tb;
    const uint64_t cm = __ballot(cand);
    if (cand) {
      const uint32_t at = slot + lane_rank(cm);
      if (at < TOPK_CAP) cd[at] = ((uint64_t)kbuf[c] << 32) | (uint32_t)(~(uint32_t)p);
    }
    slot += (uint32_t)__popcll(cm);
  }
}

// K4: the chosen candidates are decided (redundantly, by every workgroup of
// the row: rank counting when there are few, a bitonic sort otherwise); each
// workgroup then expands one tile of the bitmap into the ascending index row,
// at the offset given by the per-tile counts of K3 plus the chosen
// candidates below the tile.
constexpr int FIN_NT = 1024;
constexpr int TOPK_RANK_MAX = 512;  // rank counting up to this many candidates

template <int DT>
__global__ __launch_bounds__(FIN_NT) void k_topk_finalize(
    const void* __restrict__ scores, int64_t ld, int k, int32_t* __restrict__ idx,
    const TopkRowState* __restrict__ st, const uint64_t* __restrict__ cands,
    const uint32_t* __restrict__ bitmap, int64_t nwords, const uint32_t* __restrict__ tilecnt,
    int t3) {
  constexpr int NT = FIN_NT;
  static_assert(TOPK_K4_TILE == NT * 32, "one bitmap word per thread");
  static_assert(TOPK_RANK_MAX <= NT && TOPK_RANK_MAX / 64 <= NT / 64 / 2, "rank counting layout");
  __shared__ uint64_t sc[TOPK_CAP];
  __shared__ uint32_t tw[NT];
  __shared__ uint32_t lds_scan[NT / 64 + 2];
  __shared__ uint32_t lds_hist[256];
  __shared__ uint32_t rank[TOPK_RANK_MAX];
  __shared__ uint32_t s_below;
  const int row = blockIdx.y, tile = blockIdx.x;
  const uint32_t* bm = bitmap + (size_t)row * nwords;
  const uint32_t w0 = (uint32_t)tile * NT;             // first bitmap word of this tile
  // independent loads first: this tile's bitmap word, candidates, tile counts
  const uint32_t w = w0 + threadIdx.x;
  const uint32_t word_raw = bm[w < (uint32_t)nwords ? w : (uint32_t)nwords - 1];
  const uint64_t* cd = cands + (size_t)row * TOPK_CAP;
  const uint64_t cand_raw = cd[threadIdx.x % TOPK_RANK_MAX];
  uint32_t before = 0;
  {
    const int k3_per_k4 = TOPK_K4_TILE / TOPK_K3_TILE;
    const int lim = tile * k3_per_k4 < t3 ? tile * k3_per_k4 : t3;
    for (int t = threadIdx.x; t < lim; t += NT) before += tilecnt[(size_t)row * t3 + t];
  }
  const TopkRowState s = st[row];
  const uint32_t nv = s.nvalid;
  int32_t* out = idx + (size_t)row * k;
  const void* rp = reinterpret_cast<const char*>(scores) + (size_t)row * ld * 4;
  const uint32_t nw = (nv + 31) / 32;

  if (s.tb != TOPK_ALL && s.cand_count > TOPK_CAP) {
    // too many candidates in the threshold bin: tile 0 resolves the bin exactly
    // and writes the whole row with an ordered scan; the other tiles have nothing to do
    if (tile != 0) return;
    uint32_t need_eq;
    const uint32_t T = exact_threshold<NT, DT>(rp, nv, s.lo, s.shift, TOPK_NB, s.tb, s.need,
                                               need_eq, lds_hist, lds_scan);
    uint32_t carry_eq = 0, carry = 0;
    for (uint32_t base = 0; base < nv; base += NT) {
      const uint32_t p = base + threadIdx.x;
      const uint32_t key = p < nv ? load_key<DT>(rp, p) : 0u;
      const uint32_t bin = bin_of(key, s.lo, s.shift, TOPK_NB);
      const bool in = p < nv && bin == s.tb;
      const bool eq = in && key == T;
      uint32_t teq;
      const uint32_t req = block_excl_scan<NT>(eq ? 1u : 0u, lds_scan, teq);
      const bool sel = (p < nv && bin > s.tb) || (in && key > T) || (eq && carry_eq + req < need_eq);
      uint32_t tsel;
      const uint32_t rs = block_excl_scan<NT>(sel ? 1u : 0u, lds_scan, tsel);
      if (sel && carry + rs < (uint32_t)k) out[carry + rs] = (int32_t)p;
      carry_eq += teq;
      carry += tsel;
    }
    for (uint32_t j = carry + threadIdx.x; j < (uint32_t)k; j += NT) out[j] = -1;
    return;
  }

  tw[threadIdx.x] = w < nw ? word_raw : 0u;
  if (threadIdx.x == 0) s_below = 0;
  __syncthreads();
  uint32_t chosen_below = 0;
  if (s.tb != TOPK_ALL) {
    const uint32_t c = s.cand_count;
    if (c <= TOPK_RANK_MAX) {
      if (threadIdx.x < c) sc[threadIdx.x] = cand_raw;
      if (threadIdx.x < TOPK_RANK_MAX) rank[threadIdx.x] = 0u;
      __syncthreads();
      // rank of a candidate = how many candidates order before it.  The c*c
      // comparisons are spread over all waves: wave w compares candidate
      // group w / S (64 candidates, one per lane) with slice w % S of the list.
      // (wave_id() is a scalar, so the loop below has uniform bounds and is
      // unrolled with its LDS reads pipelined)
      const int lane = threadIdx.x & 63, wv = wave_id();
      const int ng = (int)(c + 63) / 64;  // <= TOPK_RANK_MAX / 64
      const int S = (NT / 64) / ng;
      if (wv < ng * S) {
        const int g = wv / S, sl = wv % S;
        const uint32_t i = (uint32_t)(g * 64 + lane);
        const uint32_t j0 = c * sl / S, j1 = c * (sl + 1) / S;
        if (i < c) {
          const uint64_t me = sc[i];
          uint32_t r = 0;
#pragma unroll 8
          for (uint32_t j = j0; j < j1; ++j) r += sc[j] > me ? 1u : 0u;
          if (r) atomicAdd(&rank[i], r);
        }
      }
      __syncthreads();
      if (threadIdx.x < c && rank[threadIdx.x] < s.need) {
        const uint32_t p = ~(uint32_t)(sc[threadIdx.x] & 0xFFFFFFFFull);
        const uint32_t pw = p >> 5;
        if (pw < w0) ++chosen_below;
        else if (pw < w0 + NT) atomicOr(&tw[pw - w0], 1u << (p & 31));
      }
    } else {
      const uint32_t m = next_pow2(c);
      for (uint32_t i = threadIdx.x; i < m; i += NT) sc[i] = i < c ? cd[i] : 0ull;
      __syncthreads();
      bitonic_sort_desc<NT>(sc, (int)m);
      for (uint32_t i = threadIdx.x; i < s.need; i += NT) {
        const uint32_t p = ~(uint32_t)(sc[i] & 0xFFFFFFFFull);
        const uint32_t pw = p >> 5;
        if (pw < w0) ++chosen_below;
        else if (pw < w0 + NT) atomicOr(&tw[pw - w0], 1u << (p & 31));
      }
    }
  }
  uint32_t tot;
  const uint32_t off0 = block_excl_scan<NT>(before + chosen_below, lds_scan, tot);
  (void)off0;
  const uint32_t offset = tot;  // everything before this tile
  const uint32_t word = tw[threadIdx.x];
  uint32_t tot2;
  uint32_t off = offset + block_excl_scan<NT>(__popc(word), lds_scan, tot2);
  uint32_t wv = word;
  while (wv) {
    const uint32_t bit = __ffs(wv) - 1;
    wv &= wv - 1;
    if (off < (uint32_t)k) out[off] = (int32_t)(w * 32 + bit);
    ++off;
  }
  if (tile == 0)
    for (uint32_t j = s.kk + threadIdx.x; j < (uint32_t)k; j += NT) out[j] = -1;
}

hipError_t launch_topk_minmax(const void* scores, int dtype, int rows, int64_t n, int64_t ld,
                              const int32_t* valid_len, int vl_div, char* ws,
                              const TopkMultiLayout& lay, hipStream_t s) {
  dim3 grid(lay.t1, rows);
  auto st = reinterpret_cast<TopkRowState*>(ws + lay.state);
  auto mm = reinterpret_cast<uint32_t*>(ws + lay.mm);
  auto hist = reinterpret_cast<uint32_t*>(ws + lay.hist);
  if (dtype == 0)
    k_topk_minmax<0><<<grid, 256, 0, s>>>(scores, n, ld, valid_len, vl_div, mm, lay.t1, st, hist);
  else
    k_topk_minmax<1><<<grid, 256, 0, s>>>(scores, n, ld, valid_len, vl_div, mm, lay.t1, st, hist);
  return hipGetLastError();
}

hipError_t launch_topk_select_multi(const void* scores, int dtype, int32_t* idx, int rows,
                                    int64_t n, int64_t ld, int k, const int32_t* valid_len,
                                    int vl_div, char* ws, const TopkMultiLayout& lay,
                                    hipStream_t s) {
  auto st = reinterpret_cast<TopkRowState*>(ws + lay.state);
  auto mm = reinterpret_cast<const uint32_t*>(ws + lay.mm);
  auto hist = reinterpret_cast<uint32_t*>(ws + lay.hist);
  auto cands = reinterpret_cast<uint64_t*>(ws + lay.cands);
  auto bm = reinterpret_cast<uint32_t*>(ws + lay.bitmap);
  auto tc = reinterpret_cast<uint32_t*>(ws + lay.tilecnt);
  const dim3 g2(lay.t2, rows), g3(lay.t3, rows), g4(lay.t4, rows);
  if (dtype == 0) {
    k_topk_hist<0><<<g2, 256, 0, s>>>(scores, n, ld, k, valid_len, vl_div, mm, lay.t1, hist, lay.k2_tile);
    k_topk_emit<0><<<g3, TOPK_K3_THREADS, 0, s>>>(scores, n, ld, k, valid_len, vl_div, mm, lay.t1, hist, st, cands, bm, lay.nwords, tc, lay.t3);
    k_topk_finalize<0><<<g4, FIN_NT, 0, s>>>(scores, ld, k, idx, st, cands, bm, lay.nwords, tc, lay.t3);
  } else {
    k_topk_hist<1><<<g2, 256, 0, s>>>(scores, n, ld, k, valid_len, vl_div, mm, lay.t1, hist, lay.k2_tile);
    k_topk_emit<1><<<g3, TOPK_K3_THREADS, 0, s>>>(scores, n, ld, k, valid_len, vl_div, mm, lay.t1, hist, st, cands, bm, lay.nwords, tc, lay.t3);
    k_topk_finalize<1><<<g4, FIN_NT, 0, s>>>(scores, ld, k, idx, st, cands, bm, lay.nwords, tc, lay.t3);
  }
  return hipGetLastError();
}

// ================================================== one workgroup per row ====

// One workgroup per row; BMW bitmap words in LDS (a short-row instance keeps
// LDS small so that more rows are resident per CU).
template <int DT, int BMW>
__global__ __launch_bounds__(ROW_NT) void k_topk_rows(const void* __restrict__ scores, int64_t n,
                                                      int64_t ld, int k,
                                                      const int32_t* valid_len, int vl_div,
                                                      int64_t causal_pos0,
                                                      int32_t* __restrict__ idx) {
  __shared__ RowSelSmem<BMW> sm;
  const int row = blockIdx.x;
  uint32_t nv;
  if (causal_pos0 >= 0) {
    int64_t v = causal_pos0 + row + 1;
    nv = (uint32_t)(v < n ? v : n);
  } else {
    nv = row_nvalid(valid_len, row, n, vl_div);
  }
  const void* rp = reinterpret_cast<const char*>(scores) + (size_t)row * ld * 4;
  row_select<DT, BMW>(rp, nv, k, idx + (size_t)row * k, sm);
}

hipError_t launch_topk_rows(const void* scores, int dtype, int32_t* idx, int rows, int64_t n,
                            int64_t ld, int k, const int32_t* valid_len, int vl_div,
                            int64_t causal_pos0, hipStream_t s) {
  constexpr int SHORT = ROW_NT * ROW_RC / 32;  // bitmap words of the register-cached rows
  if (n <= (int64_t)SHORT * 32) {
    if (dtype == 0)
      k_topk_rows<0, SHORT><<<rows, ROW_NT, 0, s>>>(scores, n, ld, k, valid_len, vl_div, causal_pos0, idx);
    else
      k_topk_rows<1, SHORT><<<rows, ROW_NT, 0, s>>>(scores, n, ld, k, valid_len, vl_div, causal_pos0, idx);
  } else if (dtype == 0) {
    k_topk_rows<0, TOPK_ROW_MAX_N / 32><<<rows, ROW_NT, 0, s>>>(scores, n, ld, k, valid_len, vl_div, causal_pos0,
                                                               idx);
  } else {
    k_topk_rows<1, TOPK_ROW_MAX_N / 32><<<rows, ROW_NT, 0, s>>>(scores, n, ld, k, valid_len, vl_div, causal_pos0,
                                                               idx);
  }
  return hipGetLastError();
}

}  // namespace lct
