// Fused causal prefill indexer: int8 MFMA scores filtered to short candidate
// lists per query row, then an exact top-k select per row, without storing
// the score matrix.
//
// Source: tutorial page, sections "DSA 与 IndexShare" and "两个阶段各付一笔"
// (prefill scores every earlier position of every query, then keeps the top
// k per query); CLSA explainer section 2.3 (the index set is a small integer
// array per query).  Result: the same set the plain definition gives (score
// desc, lowest position first among equal scores, ascending, -1 padded).
//
// Stored int32 scores cost 4 bytes per 512 int8 operations, which binds a
// plain scorer to HBM writes (8.6 GB per 64K-token group).  Instead:
//
// k_pf_filter: every workgroup owns whole query-row blocks of 128 rows
// (block i paired with block NB-1-i so that all workgroups do the same
// causal work) and runs, per block,
//   S1/S2  per-row min/max over every 64th key's score, then a 128-bin
//          histogram over that range of every 16th key's score -> a threshold
//          t_r with m_s samples at or above it, m_s = k/16 + 6 sqrt(k/16) + 4 (about
//          1.56 k keys expected above it at k = 2048);
//   M      one sweep over all keys <= the row: every score >= t_r is a
//          candidate (position << 16 | min(score - t_r, 65535)).  Candidates
//          go to a per-row ring in LDS; two flush waves (64 rows each) copy
//          whole 128-byte lines of it to the row's list in memory, so that
//          memory sees full lines, few store instructions and no partially
//          written lines.
// Rows with fewer than 32 m_s earlier positions (a dense candidate stream)
// are left to the plain path: one block of scores and a row select.
// k_pf_select (one workgroup per row): the entries sit in registers; a histogram
// of score - t_r names the bin holding the k-th largest; higher bins are all
// in; that bin is settled exactly (an exact-score histogram, then the ties
// by position).  Output through a position bitmap, ascending.
// Rows the lists cannot settle (a ring or list overflow, a crowded bin,
// fewer than k candidates) are listed and recomputed by the plain path.
//
// k_pf_filter waves: 0..7 compute (rows 32*(w%4).., keys 32*(w/4).. of
// each 64-key tile); wave 8 keeps three key tiles in flight by LDS DMA;
// waves 9 and 10 flush the candidate rings (64 rows each).  The compute
// waves issue no global memory operation inside a sweep.  Scores start from
// -t_r in the MFMA accumulator, so the threshold test and the entry come
// straight from the accumulated value.

#include <math.h>
#include <stddef.h>

#include <cmath>
#include <type_traits>

#include "common.h"
#include "kernels.h"
#include "topk_dev.h"

namespace lct {

constexpr int PF_HD = 256;                 // indexer features per row (int8)
constexpr int PF_KS = PF_HD / 64;          // 64-byte MFMA k-steps per row
constexpr int PF_RB = 128;                 // query rows per block
constexpr int PF_TK = 64;                  // keys per tile
constexpr int PF_NBUF = 4;                 // key-tile buffers: 3 tiles in flight
constexpr int PF_SS = 16;                  // sample stride (positions) of the histogram sweep
constexpr int PF_SS1 = 4 * PF_SS;          // sample stride of the min / max sweep
constexpr int PF_NBIN = 128;               // histogram bins
constexpr int PF_CW = 8;                   // compute waves
constexpr int PF_QB = 2;                   // 16-row blocks per compute wave
constexpr int PF_WROWS = 16 * PF_QB;       // rows per compute wave
constexpr int PF_WR = PF_RB / PF_WROWS;    // row groups
constexpr int PF_KL = PF_TK * PF_WR / (16 * PF_CW);  // 16-key blocks per compute wave and tile
static_assert(PF_WR * PF_WROWS == PF_RB && PF_CW % PF_WR == 0 && PF_KL * 16 * (PF_CW / PF_WR) == PF_TK,
              "compute waves tile the block's rows x the tile's keys");
constexpr int PF_DMA_W = PF_CW;            // the DMA wave
constexpr int PF_FL_W = PF_CW + 1;         // the first flush wave
constexpr int PF_NFL = 2;                  // flush waves
constexpr int PF_FH = PF_RB / (64 * PF_NFL);  // rows per flush lane
static_assert(PF_FH * 64 * PF_NFL == PF_RB && PF_FH <= 2, "one or two rows per flush lane");
constexpr int PF_NT = (PF_CW + 1 + PF_NFL) * 64;
constexpr int PF_CHUNKS = (PF_TK / 16) * PF_KS;  // 1 KiB fragments per key tile
constexpr int PF_RING = 128;               // candidate ring entries per row (LDS)
constexpr int PF_LCAP = 512;               // select: entries of the k-th bin a wave can hold
constexpr int PF_SEL_NT = 256;             // select: threads of the one workgroup per row
static_assert(PF_RB * PF_RING <= PF_RB * PF_NBIN, "the rings reuse the sample histogram");

typedef __attribute__((address_space(3))) void pf_lds_void;

#define PF_WAIT_VM0() __builtin_amdgcn_s_waitcnt(0x0F70)
#define PF_WAIT_LGKM0() __builtin_amdgcn_s_waitcnt(0xC07F)

// Workgroup barrier that does not wait for outstanding global stores (a
// __syncthreads() would): LDS operations are drained, then s_barrier.
LCT_DEV void pf_barrier() {
  PF_WAIT_LGKM0();
  __asm__ __volatile__("" ::: "memory");
  __builtin_amdgcn_s_barrier();
  __asm__ __volatile__("" ::: "memory");
}

// The key-tile buffers are objects of their own, apart from the rest and
// from each other: the compiler then sees that a DMA into one buffer does not
// touch the LDS data being read, and inserts no wait on the vector memory
// counter (which for the compute waves also counts their candidate stores).
struct PfShared {
  char (&kt0)[PF_CHUNKS][1024];
  char (&kt1)[PF_CHUNKS][1024];
  char (&kt2)[PF_CHUNKS][1024];
  char (&kt3)[PF_CHUNKS][1024];
  uint32_t (&hist)[PF_RB][PF_NBIN];  // sample histogram, then the candidate rings
  int32_t (&smax)[PF_RB];
  int32_t (&smin)[PF_RB];
  int32_t (&base)[PF_RB];
  int32_t (&thd)[PF_RB];
  uint32_t (&scnt)[3][PF_RB];  // candidates per row and step (steps mod 3)
};

// One sweep over key tiles [0, n_tiles) of keys at positions stride * j
// (j = tile * PF_TK + ..), in ascending or (desc) descending tile order.
// The helper wave keeps PF_NBUF - 1 tiles in flight by LDS DMA while the
// compute waves run `body(tile, buf)` on the current one.  Every wave calls
// this; the flush waves run `aux(step)` once per tile.  Key rows past the cache
// read as zeros (range-checked buffer loads; the whole offset is in the
// per-lane register).
#define PF_WAIT_VM(n) __builtin_amdgcn_s_waitcnt((((n)&15) | (((n) >> 4) << 14)) | 0x0F70)
template <typename Body, typename Aux>
LCT_DEV void pf_sweep(PfShared& sh, __amdgpu_buffer_rsrc_t krs, int n_tiles, int stride, bool desc,
                      int wid, int lane, Body body, Aux aux) {
  const int n = lane & 15, g = lane >> 4;
  typedef __attribute__((address_space(3))) char lds_char;
  typedef char Buf[PF_CHUNKS][1024];
  auto issue = [&](Buf& buf, int ts) {
    const int t = desc ? n_tiles - 1 - ts : ts;
    // opaque to the compiler, so that the per-chunk offsets are formed per
    // tile instead of being hoisted out of the sweep (and spilled)
    uint32_t vb = (uint32_t)((t * PF_TK + n) * stride) * PF_HD + g * 16;
    __asm__ volatile("" : "+v"(vb));
    lds_char* const dst = (lds_char*)&buf[0][0];
    // (the instruction's immediate offset would move the LDS destination
    // too, so every offset goes into the per-lane register)
#pragma unroll
    for (int c = 0; c < PF_CHUNKS; ++c) {
      const uint32_t voff = vb + (uint32_t)((c / PF_KS) * 16 * stride * PF_HD + (c % PF_KS) * 64);
      __builtin_amdgcn_raw_ptr_buffer_load_lds(krs, (pf_lds_void*)(dst + c * 1024), 16, voff, 0, 0, 0);
    }
  };
  static_assert(PF_NBUF == 4 && PF_CHUNKS == 16, "the waits below count 16 loads per tile, 2 tiles ahead");
  if (wid == PF_DMA_W) {
    if (n_tiles > 0) issue(sh.kt0, 0);
    if (n_tiles > 1) issue(sh.kt1, 1);
    if (n_tiles > 2) issue(sh.kt2, 2);
  }
  // step ts computes on `cur` (buffer ts % 4) while tile ts + 3 goes to
  // `ahead3` (buffer (ts + 3) % 4, last read in step ts - 1)
  auto step = [&](Buf& cur, Buf& ahead3, int ts) {
    if (wid == PF_DMA_W) {
      // tile ts has landed once at most the tiles issued after it are in flight
      const int ahead = n_tiles - 1 - ts;
      if (ahead >= 2) PF_WAIT_VM(32);
      else if (ahead == 1) PF_WAIT_VM(16);
      else PF_WAIT_VM(0);
    }
    pf_barrier();
    if (wid == PF_DMA_W) {
      if (ts + 3 < n_tiles) issue(ahead3, ts + 3);
    } else if (wid >= PF_FL_W) {
      aux(ts);
    } else {
      body(desc ? n_tiles - 1 - ts : ts, ts, cur);
    }
  };
  for (int ts = 0; ts < n_tiles; ts += 4) {
    step(sh.kt0, sh.kt3, ts);
    if (ts + 1 < n_tiles) step(sh.kt1, sh.kt0, ts + 1);
    if (ts + 2 < n_tiles) step(sh.kt2, sh.kt1, ts + 2);
    if (ts + 3 < n_tiles) step(sh.kt3, sh.kt2, ts + 3);
  }
  pf_barrier();  // every read of the last tile is done
}

// acc[qb][kl] = ini[qb] + scores of query rows 16qb + n (of the wave's 64)
// against keys PF_KL*16 wk + 16kl + 4g + e of the tile, e = vector element.
LCT_DEV void pf_tile_mfma(const char (&buf)[PF_CHUNKS][1024], const intx4 (&qf)[PF_QB][PF_KS], int wk,
                          int lane, const int32_t (&ini)[PF_QB], intx4 (&acc)[PF_QB][PF_KL]) {
#pragma unroll
  for (int i = 0; i < PF_QB; ++i)
#pragma unroll
    for (int j = 0; j < PF_KL; ++j) acc[i][j] = intx4{ini[i], ini[i], ini[i], ini[i]};
#pragma unroll
  for (int kl = 0; kl < PF_KL; ++kl) {
#pragma unroll
    for (int ks = 0; ks < PF_KS; ++ks) {
      const intx4 a = *reinterpret_cast<const intx4*>(&buf[(wk * PF_KL + kl) * PF_KS + ks][lane * 16]);
#pragma unroll
      for (int qb = 0; qb < PF_QB; ++qb)
        acc[qb][kl] = __builtin_amdgcn_mfma_i32_16x16x64_i8(a, qf[qb][ks], acc[qb][kl], 0, 0, 0);
    }
  }
}

// LDS accesses of the flush waves, written as inline assembly with the wait
// inside: the compiler would otherwise drain the vector memory counter before
// every LDS access (it cannot tell them from the key DMA), which for the flush
// wave means waiting for all of its earlier stores.
LCT_DEV uint32_t pf_lds_ld(uint32_t a) {
  uint32_t v;
  __asm__ volatile("ds_read_b32 %0, %1\n\ts_waitcnt lgkmcnt(0)" : "=v"(v) : "v"(a) : "memory");
  return v;
}
LCT_DEV void pf_lds_st(uint32_t a, uint32_t v) {
  __asm__ volatile("ds_write_b32 %0, %1" ::"v"(a), "v"(v) : "memory");
}
LCT_DEV void pf_lds_st4(uint32_t a, uintx4 v) {
  __asm__ volatile("ds_write_b128 %0, %1" ::"v"(a), "v"(v) : "memory");
}
// one 128-byte line of a ring (eight 16-byte LDS loads, one wait)
LCT_DEV void pf_lds_ld_line(uint32_t a, uintx4 (&v)[8]) {
  __asm__ volatile(
      "ds_read_b128 %0, %8\n\tds_read_b128 %1, %8 offset:16\n\tds_read_b128 %2, %8 offset:32\n\t"
      "ds_read_b128 %3, %8 offset:48\n\tds_read_b128 %4, %8 offset:64\n\tds_read_b128 %5, %8 offset:80\n\t"
      "ds_read_b128 %6, %8 offset:96\n\tds_read_b128 %7, %8 offset:112\n\ts_waitcnt lgkmcnt(0)"
      : "=&v"(v[0]), "=&v"(v[1]), "=&v"(v[2]), "=&v"(v[3]), "=&v"(v[4]), "=&v"(v[5]), "=&v"(v[6]), "=&v"(v[7])
      : "v"(a)
      : "memory");
}
// two 16-byte and two 4-byte LDS loads, one wait
LCT_DEV void pf_lds_ld_state(uint32_t a0, uint32_t a1, uint32_t b0, uint32_t b1, uintx4& s0,
                             uintx4& s1, uint32_t& c0, uint32_t& c1) {
  __asm__ volatile(
      "ds_read_b128 %0, %4\n\tds_read_b128 %1, %5\n\tds_read_b32 %2, %6\n\tds_read_b32 %3, %7\n\t"
      "s_waitcnt lgkmcnt(0)"
      : "=&v"(s0), "=&v"(s1), "=&v"(c0), "=&v"(c1)
      : "v"(a0), "v"(a1), "v"(b0), "v"(b1)
      : "memory");
}

// one 16-byte and one 4-byte LDS load, one wait
LCT_DEV void pf_lds_ld_state1(uint32_t a0, uint32_t b0, uintx4& s0, uint32_t& c0) {
  __asm__ volatile("ds_read_b128 %0, %2\n\tds_read_b32 %1, %3\n\ts_waitcnt lgkmcnt(0)"
                   : "=&v"(s0), "=&v"(c0)
                   : "v"(a0), "v"(b0)
                   : "memory");
}

// Sample-histogram bin of d = score - min over a span of `span` values:
// (d * M) >> 16 with M = floor((2^23 - 1) / span), so bins stay < 128.
// Scores lie within +-2^22, so d and M fit the 24-bit multiplier.
LCT_DEV uint32_t pf_sample_bin(uint32_t d, uint32_t M) {
  const uint32_t b = __umul24(d, M) >> 16;
  return b < PF_NBIN ? b : PF_NBIN - 1;
}

__global__ __launch_bounds__(PF_NT) void k_pf_filter(const int8_t* __restrict__ q,
                                                     const int8_t* __restrict__ k, int L, int kk,
                                                     int r_all, uint32_t* __restrict__ list,
                                                     uint32_t* __restrict__ meta, int m_s) {
  __shared__ __attribute__((aligned(16))) char kt0[PF_CHUNKS][1024];
  __shared__ __attribute__((aligned(16))) char kt1[PF_CHUNKS][1024];
  __shared__ __attribute__((aligned(16))) char kt2[PF_CHUNKS][1024];
  __shared__ __attribute__((aligned(16))) char kt3[PF_CHUNKS][1024];
  // (512-byte rows: a ring row's slot address is one and-or)
  __shared__ __attribute__((aligned(512))) uint32_t hist[PF_RB][PF_NBIN];
  __shared__ int32_t smax[PF_RB], smin[PF_RB], basev[PF_RB], thdv[PF_RB];
  __shared__ uint32_t scnt[3][PF_RB];
  __shared__ __attribute__((aligned(16))) uint32_t fst[PF_RB][4];  // flush state per row
  // a compute wave's non-candidate stores land on its one trash word (stores
  // to one address cost fewer LDS bank cycles than a word per lane)
  __shared__ uint32_t trash[PF_CW];
  PfShared sh{kt0, kt1, kt2, kt3, hist, smax, smin, basev, thdv, scnt};
  const int lane = threadIdx.x & 63, wid = wave_id();
  const int n = lane & 15, g = lane >> 4;
  const int wq = wid % PF_WR, wk = wid / PF_WR;  // compute waves: row group, key part
  const int NB = (L + PF_RB - 1) / PF_RB;
  const __amdgpu_buffer_rsrc_t krs = make_rsrc(k, (int64_t)L * PF_HD);
  const __amdgpu_buffer_rsrc_t lrs = make_rsrc(list, (int64_t)L * PF_CROW * 4);
  const int32_t zero[PF_QB] = {};
  auto no_aux = [](int) {};

  // The long block first, its sweeps ascending; then the short one, its
  // sweeps descending.  At any time the workgroups in their first block all
  // read tile t and those in their second block all read tile NB - t, so the
  // key tiles in flight are shared through L2 instead of being fetched once
  // per workgroup.
  for (int half = 0; half < 2; ++half) {
    const int rb = half == 0 ? NB - 1 - (int)blockIdx.x : (int)blockIdx.x;
    if (half == 1 && rb >= NB - 1 - (int)blockIdx.x) break;  // the middle block has no partner
    const bool desc = half == 1;
    const int r0 = rb * PF_RB;
    const int r_last = (r0 + PF_RB < L ? r0 + PF_RB : L) - 1;
    if (r_last < r_all) continue;  // shorter rows: every earlier position, or the plain path

    // ---- query fragments (compute waves): rows r0 + PF_WROWS wq + 16qb + n
    intx4 qf[PF_QB][PF_KS];
    if (wid < PF_CW) {
#pragma unroll
      for (int qb = 0; qb < PF_QB; ++qb) {
        const int row = r0 + wq * PF_WROWS + qb * 16 + n;
#pragma unroll
        for (int ks = 0; ks < PF_KS; ++ks)
          qf[qb][ks] = row <= r_last ? *reinterpret_cast<const intx4*>(
                                           q + (size_t)row * PF_HD + ks * 64 + g * 16)
                                     : intx4{0, 0, 0, 0};
      }
    }
    for (int i = threadIdx.x; i < PF_RB; i += PF_NT) {
      sh.smax[i] = INT32_MIN;
      sh.smin[i] = INT32_MAX;
      sh.scnt[0][i] = sh.scnt[1][i] = sh.scnt[2][i] = 0u;
    }
    for (int i = threadIdx.x; i < PF_RB * PF_NBIN; i += PF_NT) (&sh.hist[0][0])[i] = 0u;
    __syncthreads();

    // ---- S1: per-row min / max of every 64th key's score, the range of
    // the histogram below (rows past the block's end collect garbage that
    // nothing reads)
    const int n_samp = r_last / PF_SS + 1;  // sampled keys j: position 16 j <= r_last
    const int st_tiles = (n_samp + PF_TK - 1) / PF_TK;
    const int st_tiles1 = (r_last / PF_SS1 + 1 + PF_TK - 1) / PF_TK;
    {
      int32_t mx[PF_QB], mn[PF_QB];
#pragma unroll
      for (int i = 0; i < PF_QB; ++i) {
        mx[i] = INT32_MIN;
        mn[i] = INT32_MAX;
      }
      pf_sweep(sh, krs, st_tiles1, PF_SS1, desc, wid, lane, [&](int t, int, auto& buf) {
        intx4 acc[PF_QB][PF_KL];
        pf_tile_mfma(buf, qf, wk, lane, zero, acc);
        const bool diag = (t * PF_TK + PF_TK - 1) * PF_SS1 > r0;  // a sample past some row
#pragma unroll
        for (int qb = 0; qb < PF_QB; ++qb) {
          const int row = r0 + wq * PF_WROWS + qb * 16 + n;
#pragma unroll
          for (int kl = 0; kl < PF_KL; ++kl)
#pragma unroll
            for (int e = 0; e < 4; ++e) {
              const int pos = (t * PF_TK + wk * PF_KL * 16 + kl * 16 + g * 4 + e) * PF_SS1;
              if (!diag || pos <= row) {
                mx[qb] = max(mx[qb], acc[qb][kl][e]);
                mn[qb] = min(mn[qb], acc[qb][kl][e]);
              }
            }
        }
      }, no_aux);
      if (wid < PF_CW) {
#pragma unroll
        for (int qb = 0; qb < PF_QB; ++qb) {
          int32_t a = mx[qb], b = mn[qb];
          a = max(a, __shfl_xor(a, 16, 64));
          a = max(a, __shfl_xor(a, 32, 64));
          b = min(b, __shfl_xor(b, 16, 64));
          b = min(b, __shfl_xor(b, 32, 64));
          if (g == 0) {
            const int rl = wq * PF_WROWS + qb * 16 + n;
            atomicMax(&sh.smax[rl], a);
            atomicMin(&sh.smin[rl], b);
          }
        }
      }
      __syncthreads();
    }
    // ---- S2: 128-bin histogram of every 16th key's score over S1's
    // [min, max] (scores outside it are clamped into the end bins)
    {
      int32_t lo[PF_QB], hi[PF_QB];
      uint32_t M[PF_QB];
#pragma unroll
      for (int qb = 0; qb < PF_QB; ++qb) {
        const int rl = wq * PF_WROWS + qb * 16 + n;
        lo[qb] = sh.smin[rl];
        hi[qb] = sh.smax[rl] - lo[qb];
        const uint32_t span = (uint32_t)hi[qb] + 1u;
        M[qb] = span == 0u ? 1u : ((1u << 23) - 1u) / span;
      }
      pf_sweep(sh, krs, st_tiles, PF_SS, desc, wid, lane, [&](int t, int, auto& buf) {
        intx4 acc[PF_QB][PF_KL];
        pf_tile_mfma(buf, qf, wk, lane, zero, acc);
        const bool diag = (t * PF_TK + PF_TK - 1) * PF_SS > r0;
#pragma unroll
        for (int qb = 0; qb < PF_QB; ++qb) {
          const int rl = wq * PF_WROWS + qb * 16 + n;
          const int row = r0 + rl;
#pragma unroll
          for (int kl = 0; kl < PF_KL; ++kl)
#pragma unroll
            for (int e = 0; e < 4; ++e) {
              const int pos = (t * PF_TK + wk * PF_KL * 16 + kl * 16 + g * 4 + e) * PF_SS;
              if (!diag || pos <= row)
                atomicAdd(&sh.hist[rl][pf_sample_bin((uint32_t)min(max(acc[qb][kl][e] - lo[qb], 0), hi[qb]), M[qb])],
                          1u);
            }
        }
      }, no_aux);
    }
    // ---- threshold per row: the smallest score whose sample bin holds the
    // m_s-th largest sample; rows below r_all take no candidates here
    if (threadIdx.x < PF_RB) {
      const int rl = threadIdx.x;
      const int row = r0 + rl;
      int32_t thd = INT32_MAX, bs = 0;
      if (row <= r_last && row >= r_all) {
        const int32_t lo = sh.smin[rl];
        const uint32_t span = (uint32_t)(sh.smax[rl] - lo) + 1u;
        const uint32_t M = ((1u << 23) - 1u) / span;
        uint32_t acc = 0;
        int b = PF_NBIN - 1;
        for (; b > 0; --b) {
          acc += sh.hist[rl][b];
          if (acc >= (uint32_t)m_s) break;
        }
        bs = lo + (int32_t)(((uint32_t)b * 65536u + M - 1u) / M);
        thd = -1;  // candidate: score - bs >= 0
        // the select bins score - bs by this shift: the sampled range spans
        // fewer than 96 of its 128 bins
        int sf = 0;
        while ((((int64_t)sh.smax[rl] - bs) >> sf) >= 96) ++sf;
        meta[(size_t)row * PF_META + 3] = (uint32_t)sf;
      }
      sh.base[rl] = bs;
      sh.thd[rl] = thd;
    }
    __syncthreads();

    // ---- M: all keys <= the block's last row; candidates to the rings
    uint32_t* const ring = &sh.hist[0][0];  // [PF_RB][PF_RING]
    // flush-wave state per row, kept in LDS (not in registers across the
    // sweep): candidates of the steps before the current one (all written),
    // entries flushed, flushed count when the previous step began, overflow
    const uint32_t ring_lds = (uint32_t)(uintptr_t)(__attribute__((address_space(3))) uint32_t*)ring;
    const uint32_t scnt_lds = (uint32_t)(uintptr_t)(__attribute__((address_space(3))) uint32_t*)&sh.scnt[0][0];
    const uint32_t fst_lds = (uint32_t)(uintptr_t)(__attribute__((address_space(3))) uint32_t*)&fst[0][0];
    // flush wave f takes rows lane + 64 (PF_FH f + h), h < PF_FH
    const int frow = lane + 64 * PF_FH * (wid - PF_FL_W);
    if (wid >= PF_FL_W) {
#pragma unroll
      for (int h = 0; h < PF_FH; ++h) pf_lds_st4(fst_lds + 16 * (frow + 64 * h), uintx4{0u, 0u, 0u, 0u});
    }
    // whole lines [ff, lim) of the lane's rows: each lane copies its own rows'
    // lines, 128 bytes per line (one LDS round trip, eight 16-byte stores)
    auto flush_lines = [&](uintx4 (&st)[PF_FH], const uint32_t (&lim)[PF_FH]) {
#pragma unroll
      for (int h = 0; h < PF_FH; ++h) {
        const uint32_t rl = (uint32_t)(frow + 64 * h);
        while (st[h].y + 32u <= lim[h]) {
          uintx4 v[8];
          pf_lds_ld_line(ring_lds + 4 * (rl * PF_RING + (st[h].y & (PF_RING - 1))), v);
          const uint32_t dst = (((uint32_t)r0 + rl) * PF_CROW + st[h].y) * 4u;
#pragma unroll
          for (int j = 0; j < 8; ++j) __builtin_amdgcn_raw_buffer_store_b128(v[j], lrs, (int)(dst + 16 * j), 0, 0);
          st[h].y += 32u;
        }
      }
    };
    // state and the last finished step's counts of the lane's rows
    auto load_state = [&](int step, uintx4 (&st)[PF_FH], uint32_t (&c)[PF_FH]) {
      if constexpr (PF_FH == 2)
        pf_lds_ld_state(fst_lds + 16 * frow, fst_lds + 16 * (frow + 64),
                        scnt_lds + 4 * ((step % 3) * PF_RB + frow),
                        scnt_lds + 4 * ((step % 3) * PF_RB + frow + 64), st[0], st[1], c[0], c[1]);
      else
        pf_lds_ld_state1(fst_lds + 16 * frow, scnt_lds + 4 * ((step % 3) * PF_RB + frow), st[0], c[0]);
    };
    // step ts: the counts of step ts - 1 are final; the counters of step
    // ts + 1 (last read in step ts - 1) are cleared for it
    auto flush_step = [&](int ts) {
      uintx4 st[PF_FH];
      uint32_t c[PF_FH], lim[PF_FH] = {};
      load_state(ts > 0 ? ts - 1 : 0, st, c);
#pragma unroll
      for (int h = 0; h < PF_FH; ++h) {
        const int rl = frow + 64 * h;
        const int row = r0 + rl;
        pf_lds_st(scnt_lds + 4 * (((ts + 1) % 3) * PF_RB + rl), 0u);
        if (row > r_last || row < r_all) continue;
        if (ts > 0) st[h].x += c[h];
        // a slot written in the previous step may have wrapped onto a line
        // that step's flush was still reading
        if (st[h].x - st[h].z > (uint32_t)PF_RING) st[h].w = 1u;
        st[h].z = st[h].y;
        lim[h] = min(st[h].x, (uint32_t)PF_CROW);
      }
      flush_lines(st, lim);
#pragma unroll
      for (int h = 0; h < PF_FH; ++h) pf_lds_st4(fst_lds + 16 * (frow + 64 * h), st[h]);
    };
    int m_tiles;
    {
      int32_t ini[PF_QB], thd[PF_QB];
      uint32_t base[PF_QB];  // candidates of the row before the current step
#pragma unroll
      for (int qb = 0; qb < PF_QB; ++qb) {
        const int rl = wq * PF_WROWS + qb * 16 + n;
        ini[qb] = -sh.base[rl];
        thd[qb] = sh.thd[rl];
        base[qb] = 0u;
      }
      auto emit = [&](auto diag_c, int t, int ts, const intx4 (&acc)[PF_QB][PF_KL]) {
        constexpr bool DIAG = decltype(diag_c)::value;
        const int cs = ts % 3;
        // candidates of this lane per row: a bit per element, then one slot
        // reservation per row for all of them (the reservations are
        // unconditional, so their LDS round trips overlap), then the writes
        uint32_t bits[PF_QB], first[PF_QB];
#pragma unroll
        for (int qb = 0; qb < PF_QB; ++qb) {
          const int rl = wq * PF_WROWS + qb * 16 + n;
          uint32_t b = 0;
#pragma unroll
          for (int kl = 0; kl < PF_KL; ++kl)
#pragma unroll
            for (int e = 0; e < 4; ++e) {
              bool c = acc[qb][kl][e] > thd[qb];
              if (DIAG) c = c && t * PF_TK + wk * PF_KL * 16 + kl * 16 + g * 4 + e <= r0 + rl;
              b |= c ? 1u << (kl * 4 + e) : 0u;
            }
          bits[qb] = b;
        }
#pragma unroll
        for (int qb = 0; qb < PF_QB; ++qb)
          first[qb] = base[qb] + atomicAdd(&sh.scnt[cs][wq * PF_WROWS + qb * 16 + n], (uint32_t)__popc(bits[qb]));
        // entry = position << 16 | min(offset, 65535): one saturating pack
        // of the offset and the element's position (positions < 65536); the
        // slot (in bytes) advances by the candidate bit after each store, and
        // the row's 512-byte alignment makes its address one and-or
        static_assert(PF_RING * 4 == 512, "ring rows of 512 bytes");
        const uint32_t pos0 = (uint32_t)(t * PF_TK + wk * PF_KL * 16 + g * 4);
        uint32_t pj[PF_KL * 4];
#pragma unroll
        for (int j = 0; j < PF_KL * 4; ++j) pj[j] = pos0 + (uint32_t)((j >> 2) * 16 + (j & 3));
#pragma unroll
        for (int qb = 0; qb < PF_QB; ++qb) {
          const uint32_t rrow = ring_lds + 4u * (uint32_t)((wq * PF_WROWS + qb * 16 + n) * PF_RING);
          const uint32_t tr = (uint32_t)(uintptr_t)(__attribute__((address_space(3))) uint32_t*)&trash[wid];
          uint32_t s4 = first[qb] << 2;
#pragma unroll
          for (int kl = 0; kl < PF_KL; ++kl)
#pragma unroll
            for (int e = 0; e < 4; ++e) {
              const uint32_t c = (bits[qb] >> (kl * 4 + e)) & 1u;
              // every lane stores: a candidate to its slot, the others to the
              // wave's trash word (no exec-mask branch per element)
              *reinterpret_cast<__attribute__((address_space(3))) uint32_t*>((uintptr_t)(c ? (s4 & 508u) | rrow : tr)) =
                  __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_pk_u16((uint32_t)acc[qb][kl][e], pj[kl * 4 + e]));
              s4 += c << 2;
            }
        }
      };
      m_tiles = (r_last + 1 + PF_TK - 1) / PF_TK;
      pf_sweep(sh, krs, m_tiles, 1, desc, wid, lane, [&](int t, int ts, auto& buf) {
        intx4 acc[PF_QB][PF_KL];
        if (ts > 0) {
#pragma unroll
          for (int qb = 0; qb < PF_QB; ++qb) base[qb] += sh.scnt[(ts - 1) % 3][wq * PF_WROWS + qb * 16 + n];
        }
        pf_tile_mfma(buf, qf, wk, lane, ini, acc);
        if (t * PF_TK + PF_TK - 1 > r0) emit(std::true_type{}, t, ts, acc);
        else emit(std::false_type{}, t, ts, acc);
      }, flush_step);

    }
    // ---- the rest of every ring, the counts and the flags
    if (wid >= PF_FL_W) {
      uintx4 st[PF_FH];
      uint32_t c[PF_FH], lim[PF_FH] = {};
      load_state(m_tiles - 1, st, c);
#pragma unroll
      for (int h = 0; h < PF_FH; ++h) {
        const int rl = frow + 64 * h;
        const int row = r0 + rl;
        if (row > r_last || row < r_all) continue;
        st[h].x += c[h];
        if (st[h].x - st[h].z > (uint32_t)PF_RING || st[h].x > (uint32_t)PF_CROW) st[h].w = 1u;
        lim[h] = min(st[h].x, (uint32_t)PF_CROW);
      }
      flush_lines(st, lim);
#pragma unroll
      for (int h = 0; h < PF_FH; ++h) {
        const int rl = frow + 64 * h;
        const int row = r0 + rl;
        if (row > r_last || row < r_all) continue;
        for (uint32_t i = st[h].y; i < lim[h]; ++i)
          __builtin_amdgcn_raw_buffer_store_b32(pf_lds_ld(ring_lds + 4 * (rl * PF_RING + (i & (PF_RING - 1)))),
                                                lrs, (int)(((uint32_t)row * PF_CROW + i) * 4u), 0, 0);
        meta[(size_t)row * PF_META + 0] = st[h].x;
        meta[(size_t)row * PF_META + 1] = st[h].w;
        meta[(size_t)row * PF_META + 2] = (uint32_t)sh.base[rl];
      }
    }
    __syncthreads();  // LDS reuse by the next block
  }
}

// ---- exact select per row from the candidate lists ----------------------

struct PfSelShared {
  uint32_t bm[2048];  // position bitmap (65536 positions)
  union {
    struct {
      uint32_t lpos[PF_LCAP];  // the k-th bin's entries
      int32_t lsc[PF_LCAP];
    } l;
    uint16_t stage[PF_MAX_K];  // then the output row, before a coalesced copy
  } u;
  uint32_t hist[PF_NBIN];
  uint32_t sub[256];  // exact-score histogram of the k-th bin, then its ties
  uint32_t qrow[PF_HD / 4];
  uint32_t scan[PF_SEL_NT / 64 + 2];
  uint32_t v[8];  // bin, above, count, status, list fill, clamped, cut value, tie fill
};
static_assert(sizeof(uint16_t) * PF_MAX_K <= 2 * sizeof(uint32_t) * PF_LCAP, "output staging fits");

// LDS slot of bitmap word w: the words a thread expands (8 in a row) are
// spread over the banks
LCT_DEV uint32_t pf_bw(uint32_t w) { return w ^ ((w >> 3) & 31u); }

LCT_DEV uint32_t pf_mbcnt(uint64_t m) {
  return __builtin_amdgcn_mbcnt_hi((uint32_t)(m >> 32), __builtin_amdgcn_mbcnt_lo((uint32_t)m, 0u));
}

// Over the counts c(b) of bins b = top .. 0 held two per lane (lane l: bins
// top - 2l and top - 2l - 1), find the bin that holds the need-th largest
// entry.  Returns false if the counts sum to less than need.  One wave.
LCT_DEV bool pf_find_bin(uint32_t c_hi, uint32_t c_lo, int top, uint32_t need, int lane,
                         uint32_t& bin, uint32_t& above, uint32_t& cnt) {
  const uint32_t tot = c_hi + c_lo;
  const uint32_t incl = wave_incl_scan(tot);
  const uint32_t excl = incl - tot;
  uint32_t b = 0xFFFFFFFFu, ab = 0, cn = 0;
  if (excl < need && incl >= need) {
    if (excl + c_hi >= need) {
      b = top - 2 * lane;
      ab = excl;
      cn = c_hi;
    } else {
      b = top - 2 * lane - 1;
      ab = excl + c_hi;
      cn = c_lo;
    }
  }
  const uint64_t bal = __ballot(b != 0xFFFFFFFFu);
  const int src = bal ? __ffsll((unsigned long long)bal) - 1 : 0;
  bin = __shfl(b, src, 64);
  above = __shfl(ab, src, 64);
  cnt = __shfl(cn, src, 64);
  return bal != 0;
}

// Exact top-k of one row from its candidate list: one workgroup of
// PF_SEL_NT threads per row.  The list is read once into registers (entry
// 4 NT m + 4 t + u in element u of e[m] of thread t); a histogram of
// score - t_r names the bin holding the k-th largest; higher bins go to the
// position bitmap, that bin to an LDS list, which is settled exactly (an
// exact-score histogram and the ties at the cut ranked by position, or, for
// a top bin or clamped offsets, every entry ranked); the bitmap is expanded
// into the ascending row (a block-wide prefix sum of popcounts, eight words
// per thread).  Rows the list cannot settle are listed for the whole-row
// select.  The kernel is latency bound, so it is held to 64 VGPRs: eight
// waves per SIMD (eight rows per CU) instead of seven.
__global__ __launch_bounds__(PF_SEL_NT) __attribute__((amdgpu_waves_per_eu(8))) void k_pf_select(
    const int8_t* __restrict__ q, const int8_t* __restrict__ k, int L, int kk, int r_all,
    const uint32_t* __restrict__ list, const uint32_t* __restrict__ meta,
    int32_t* __restrict__ idx, int32_t* __restrict__ fails) {
  constexpr int NT = PF_SEL_NT;
  constexpr int EM = PF_CROW / (4 * NT);  // 16-byte loads per thread
  static_assert(EM * 4 * NT == PF_CROW, "the list fits the registers exactly");
  __shared__ __attribute__((aligned(16))) PfSelShared sh;
  const int tid = threadIdx.x, lane = tid & 63, wid = wave_id();
  const int row = blockIdx.x;
  int32_t* out = idx + (size_t)row * kk;
  if (row < kk) {
    for (int j = tid; j < kk; j += NT) out[j] = j <= row ? j : -1;
    return;
  }
  if (row < r_all) return;  // the plain path writes these rows
  const uint4 m4 = *reinterpret_cast<const uint4*>(meta + (size_t)row * PF_META);
  const uint32_t c = m4.x;
  const int32_t base = (int32_t)m4.z;
  const int sf = (int)m4.w;
  if (m4.y != 0u || c < (uint32_t)kk || c > (uint32_t)PF_CROW) {
    if (tid == 0) fails[1 + atomicAdd(&fails[0], 1)] = row;
    return;
  }
  // entry = position << 16 | min(score - base, 65535); bin = min(value >> sf, 127)
  const uint32_t* lp = list + (size_t)row * PF_CROW;
  auto bin_of = [&](uint32_t e) { return min((e & 0xFFFFu) >> sf, (uint32_t)(PF_NBIN - 1)); };
  uintx4 e[EM];
#pragma unroll
  for (int m = 0; m < EM; ++m) {
    const uint32_t i = 4u * NT * m + 4u * tid;
    e[m] = i < c ? *reinterpret_cast<const uintx4*>(lp + i) : uintx4{0xFFFFFFFFu, 0xFFFFFFFFu, 0xFFFFFFFFu, 0xFFFFFFFFu};
#pragma unroll
    for (int u = 0; u < 4; ++u)
      if (i + u >= c) e[m][u] = 0xFFFFFFFFu;
  }
  const uint32_t nwords = (uint32_t)((row + 1 + 31) / 32);
  for (int i = tid; i < PF_NBIN; i += NT) sh.hist[i] = 0u;
  for (uint32_t w = tid; w < nwords; w += NT) sh.bm[pf_bw(w)] = 0u;
  if (tid < 8) sh.v[tid] = 0u;
  __syncthreads();
  // the bin histogram
#pragma unroll
  for (int m = 0; m < EM; ++m)
#pragma unroll
    for (int u = 0; u < 4; ++u)
      if (e[m][u] != 0xFFFFFFFFu) atomicAdd(&sh.hist[bin_of(e[m][u])], 1u);
  __syncthreads();
  if (wid == 0) {
    const uint2 hw = reinterpret_cast<const uint2*>(sh.hist)[63 - lane];
    // hw.y = bin 127 - 2 lane, hw.x = bin 126 - 2 lane
    uint32_t bsel, above, nsel;
    const bool ok = pf_find_bin(hw.y, hw.x, PF_NBIN - 1, (uint32_t)kk, lane, bsel, above, nsel);
    if (lane == 0) {
      sh.v[0] = bsel;
      sh.v[1] = above;
      sh.v[2] = nsel;
      sh.v[3] = (!ok || nsel > (uint32_t)PF_LCAP) ? 1u : 0u;
    }
  }
  __syncthreads();
  if (sh.v[3]) {  // uniform
    if (tid == 0) fails[1 + atomicAdd(&fails[0], 1)] = row;
    return;
  }
  const uint32_t bsel = sh.v[0], nsel = sh.v[2];
  const uint32_t need1 = (uint32_t)kk - sh.v[1];  // taken from the k-th bin, 1..nsel
  uint32_t* lpos = sh.u.l.lpos;
  int32_t* lsc = sh.u.l.lsc;
  // bins above bsel are in; bin bsel goes to the list with its offset
  {
    bool clamped = false;
#pragma unroll
    for (int m = 0; m < EM; ++m)
#pragma unroll
      for (int u = 0; u < 4; ++u) {
        const uint32_t x = e[m][u];
        const bool valid = x != 0xFFFFFFFFu;
        const uint32_t b = bin_of(x), p = x >> 16, d = x & 0xFFFFu;
        if (valid && b > bsel) atomicOr(&sh.bm[pf_bw(p >> 5)], 1u << (p & 31));
        const bool inl = valid && b == bsel;
        const uint64_t bl = __ballot(inl);
        if (bl) {  // uniform over the wave
          uint32_t s0 = 0;
          if (lane == 0) s0 = atomicAdd(&sh.v[4], (uint32_t)__popcll(bl));
          s0 = __shfl(s0, 0, 64);
          if (inl) {
            const uint32_t slot = s0 + pf_mbcnt(bl);  // < nsel <= PF_LCAP
            lpos[slot] = p;
            lsc[slot] = (int32_t)d;
          }
        }
        clamped = clamped || (inl && d == 0xFFFFu);
      }
    if (__ballot(clamped) != 0 && lane == 0) sh.v[5] = 1u;
  }
  __syncthreads();
  const bool clamped = sh.v[5] != 0u;
  if (clamped) {
    // offsets clamped at 65535 are not exact: recompute the bin's scores
    if (tid < PF_HD / 4) sh.qrow[tid] = reinterpret_cast<const uint32_t*>(q + (size_t)row * PF_HD)[tid];
    __syncthreads();
    for (uint32_t j = tid; j < nsel; j += NT) {
      const int8_t* kp = k + (size_t)lpos[j] * PF_HD;
      int32_t sacc = 0;
#pragma unroll
      for (int w = 0; w < PF_HD / 16; ++w) {
        const uintx4 kv = *reinterpret_cast<const uintx4*>(kp + w * 16);
        const uintx4 qv = *reinterpret_cast<const uintx4*>(&sh.qrow[w * 4]);
        sacc = __builtin_amdgcn_sdot4((int)qv.x, (int)kv.x, sacc, false);
        sacc = __builtin_amdgcn_sdot4((int)qv.y, (int)kv.y, sacc, false);
        sacc = __builtin_amdgcn_sdot4((int)qv.z, (int)kv.z, sacc, false);
        sacc = __builtin_amdgcn_sdot4((int)qv.w, (int)kv.w, sacc, false);
      }
      lsc[j] = sacc - base;
    }
    __syncthreads();
  }
  // the need1 best of the bin by (score desc, position asc).  Below the top
  // bin and with sf <= 7 the bin spans 2^sf consecutive exact values from
  // bsel << sf: a 128-counter histogram finds the cut value T, and only the
  // ties at T are ranked by position.
  bool ranked = false;
  if (!clamped && sf <= 7 && bsel < (uint32_t)(PF_NBIN - 1)) {  // uniform
    const int32_t lo_b = (int32_t)(bsel << sf);
    for (int i = tid; i < 128; i += NT) sh.sub[i] = 0u;
    __syncthreads();
    for (uint32_t j = tid; j < nsel; j += NT) atomicAdd(&sh.sub[lsc[j] - lo_b], 1u);
    __syncthreads();
    if (wid == 0) {
      const uint2 hw = reinterpret_cast<const uint2*>(sh.sub)[63 - lane];
      uint32_t tb, ab2, n_eq;
      const bool found = pf_find_bin(hw.y, hw.x, 127, need1, lane, tb, ab2, n_eq);
      if (lane == 0) {
        sh.v[6] = (uint32_t)(lo_b + (int32_t)tb);
        sh.v[7] = need1 - ab2;                 // ties at T to take, 1..n_eq
        sh.v[3] = (found && n_eq <= 256) ? n_eq : 0xFFFFFFFFu;
        sh.v[4] = 0u;                           // tie fill
      }
    }
    __syncthreads();
    const uint32_t n_eq = sh.v[3];
    if (n_eq != 0xFFFFFFFFu) {  // uniform
      const int32_t T = (int32_t)sh.v[6];
      const uint32_t need_eq = sh.v[7];
      // ties at T compacted into sh.sub, the rest above T straight to the bitmap
      for (uint32_t j0 = 0; j0 < nsel; j0 += NT) {
        const uint32_t j = j0 + tid;
        const bool in = j < nsel;
        const int32_t sv = in ? lsc[j] : INT32_MIN;
        const uint32_t p = in ? lpos[j] : 0u;
        if (in && sv > T) atomicOr(&sh.bm[pf_bw(p >> 5)], 1u << (p & 31));
        const uint64_t bl = __ballot(in && sv == T);
        if (bl) {
          uint32_t s0 = 0;
          if (lane == 0) s0 = atomicAdd(&sh.v[4], (uint32_t)__popcll(bl));
          s0 = __shfl(s0, 0, 64);
          if (in && sv == T) sh.sub[s0 + pf_mbcnt(bl)] = p;
        }
      }
      __syncthreads();
      for (uint32_t j = tid; j < n_eq; j += NT) {
        const uint32_t p = sh.sub[j];
        uint32_t r = 0;
        for (uint32_t mm = 0; mm < n_eq; ++mm) r += sh.sub[mm] < p ? 1u : 0u;
        if (r < need_eq) atomicOr(&sh.bm[pf_bw(p >> 5)], 1u << (p & 31));
      }
      ranked = true;
    }
  }
  if (!ranked) {
    // any bin: rank every entry of the bin against all the others
    for (uint32_t j = tid; j < nsel; j += NT) {
      const int32_t sv = lsc[j];
      const uint32_t p = lpos[j];
      uint32_t r = 0;
      for (uint32_t mm = 0; mm < nsel; ++mm) {
        const int32_t sm = lsc[mm];
        const uint32_t pm = lpos[mm];
        r += (sm > sv || (sm == sv && pm < p)) ? 1u : 0u;
      }
      if (r < need1) atomicOr(&sh.bm[pf_bw(p >> 5)], 1u << (p & 31));
    }
  }
  __syncthreads();
  // ascending: thread t expands words [8t, 8t + 8) into the LDS stage (the
  // k-th bin's list is dead now), then the row goes out in coalesced stores
  constexpr int WPT = 2048 / NT;
  uint32_t wv[WPT], cnt = 0;
#pragma unroll
  for (int j = 0; j < WPT; ++j) {
    const uint32_t w = tid * WPT + j;
    wv[j] = w < nwords ? sh.bm[pf_bw(w)] : 0u;
    cnt += __popc(wv[j]);
  }
  uint32_t tot;
  uint32_t off = block_excl_scan<NT>(cnt, sh.scan, tot);
  uint16_t* stage = sh.u.stage;
#pragma unroll
  for (int j = 0; j < WPT; ++j) {
    const uint32_t w = tid * WPT + j;
    uint32_t x = wv[j];
    while (x) {
      const uint32_t b = __ffs(x) - 1;
      x &= x - 1;
      if (off < (uint32_t)kk) stage[off] = (uint16_t)(w * 32 + b);
      ++off;
    }
  }
  __syncthreads();
  if ((kk & 3) == 0 && (reinterpret_cast<uintptr_t>(out) & 15u) == 0) {
    // eight entries per thread: one 16-byte LDS read, 16-byte stores
    for (uint32_t j0 = 8u * tid; j0 < (uint32_t)kk; j0 += 8u * NT) {
      const uintx4 sv = *reinterpret_cast<const uintx4*>(&stage[j0]);  // j0 + 8 <= PF_MAX_K
      intx4 v[2];
#pragma unroll
      for (int u = 0; u < 8; ++u) {
        const uint32_t p = (sv[u >> 1] >> (16 * (u & 1))) & 0xFFFFu;
        v[u >> 2][u & 3] = j0 + u < tot ? (int32_t)p : -1;
      }
      *reinterpret_cast<intx4*>(out + j0) = v[0];
      if (j0 + 8 <= (uint32_t)kk) *reinterpret_cast<intx4*>(out + j0 + 4) = v[1];  // else j0 + 4 == kk
    }
  } else {
    for (uint32_t j = tid; j < (uint32_t)kk; j += NT) out[j] = j < tot ? (int32_t)stage[j] : -1;
  }
}

// ---- whole-row select for the rows the lists could not settle ----------

// A fixed grid takes the rows k_pf_select listed, in turn: workgroup w takes
// list slots w, w + grid, ... below the count the list holds on the device
// (the host never reads it, so the call stays asynchronous), scores its row
// against every earlier key into its own slice of the workspace (one key per
// lane, the query row broadcast from LDS) and runs the one-row select on it.
__global__ __launch_bounds__(ROW_NT) void k_pf_fallback(const int8_t* __restrict__ q,
                                                        const int8_t* __restrict__ k, int kk,
                                                        const int32_t* __restrict__ fails,
                                                        int32_t* __restrict__ scratch, int L,
                                                        int32_t* __restrict__ idx,
                                                        int32_t* __restrict__ n_out) {
  __shared__ RowSelSmem<PF_MAX_L / 32> sm;
  __shared__ uintx4 qrow[PF_HD / 16];
  const int nf = fails[0];
  if (n_out && blockIdx.x == 0 && threadIdx.x == 0) *n_out = nf;
  int32_t* const sc = scratch + (size_t)blockIdx.x * L;
  for (int slot = blockIdx.x; slot < nf; slot += gridDim.x) {
    const int row = fails[1 + slot];
    __syncthreads();  // the previous row is done with the LDS and the slice
    if (threadIdx.x < PF_HD / 16)
      qrow[threadIdx.x] = reinterpret_cast<const uintx4*>(q + (size_t)row * PF_HD)[threadIdx.x];
    __syncthreads();
    for (int t = threadIdx.x; t <= row; t += ROW_NT) {
      const uintx4* kp = reinterpret_cast<const uintx4*>(k + (size_t)t * PF_HD);
      int32_t acc = 0;
#pragma unroll
      for (int w = 0; w < PF_HD / 16; ++w) {
        const uintx4 kv = kp[w], qv = qrow[w];
        acc = __builtin_amdgcn_sdot4((int)qv.x, (int)kv.x, acc, false);
        acc = __builtin_amdgcn_sdot4((int)qv.y, (int)kv.y, acc, false);
        acc = __builtin_amdgcn_sdot4((int)qv.z, (int)kv.z, acc, false);
        acc = __builtin_amdgcn_sdot4((int)qv.w, (int)kv.w, acc, false);
      }
      sc[t] = acc;
    }
    __syncthreads();  // the whole row is stored (same workgroup, same L1)
    row_select<0, PF_MAX_L / 32>(sc, (uint32_t)row + 1u, kk, idx + (size_t)row * kk, sm);
  }
}

__global__ void k_pf_zero_fails(int32_t* fails) {
  if (threadIdx.x == 0) fails[0] = 0;
}

// Rows with fewer than 32 m_s earlier positions are left to the plain path.
static void pf_params(int64_t L, int kk, int* m_s, int* r_all) {
  // sampled keys (every 16th) wanted at or above the threshold: k/16 plus
  // six times the spread of that count, so that fewer than k candidates is rare
  const double ks = kk / (double)PF_SS;
  *m_s = (int)std::ceil(ks + 6.0 * std::sqrt(ks)) + 4;
  int64_t ra = 2 * PF_SS * (int64_t)*m_s;
  if (ra < kk) ra = kk;
  if (ra > L) ra = L;
  *r_all = (int)ra;
}

// Workgroups of the whole-row fallback (one row at a time each).
static int pf_fallback_grid(int64_t L) { return (int)(L < PF_FB_GRID ? L : PF_FB_GRID); }

size_t pf_workspace_layout(int64_t L, int HD, int kk, PfLayout* lay) {
  (void)HD;
  auto up = [](size_t x) { return (x + 255) & ~size_t(255); };
  int m_s, r_all;
  pf_params(L, kk, &m_s, &r_all);
  PfLayout l;
  size_t off = 0;
  l.list = off;
  off += up((size_t)L * PF_CROW * 4);
  l.meta = off;
  off += up((size_t)L * PF_META * 4);
  l.fails = off;
  off += up((size_t)(1 + L) * 4);
  l.short_scores = off;
  off += up((size_t)(r_all - kk > 0 ? r_all - kk : 0) * r_all * 4);
  l.fb_scores = off;
  off += up((size_t)pf_fallback_grid(L) * L * 4);
  l.total = off;
  if (lay) *lay = l;
  return off;
}

hipError_t launch_pf_fused(const int8_t* q, const int8_t* k, int64_t L, int HD, int kk,
                           int32_t* idx, char* ws, hipStream_t st, int32_t* n_failed) {
  if (HD != PF_HD || L < 1 || L > PF_MAX_L || kk < 1 || kk > PF_MAX_K) return hipErrorInvalidValue;
  PfLayout l;
  pf_workspace_layout(L, HD, kk, &l);
  int m_s, r_all;
  pf_params(L, kk, &m_s, &r_all);
  auto list = reinterpret_cast<uint32_t*>(ws + l.list);
  auto meta = reinterpret_cast<uint32_t*>(ws + l.meta);
  auto fails = reinterpret_cast<int32_t*>(ws + l.fails);
  hipError_t e;
  k_pf_zero_fails<<<1, 64, 0, st>>>(fails);
  if ((e = hipGetLastError()) != hipSuccess) return e;
  // rows [k, r_all): one block of plain scores against keys [0, r_all)
  if (r_all > kk) {
    auto ss = reinterpret_cast<int32_t*>(ws + l.short_scores);
    if ((e = launch_idx_score_mfma(q + (size_t)kk * PF_HD, k, ss, 1, r_all - kk, r_all, PF_HD, kk, st)) != hipSuccess)
      return e;
    if ((e = launch_topk_rows(ss, 0, idx + (size_t)kk * kk, r_all - kk, r_all, r_all, kk, nullptr, 1, kk, st)) !=
        hipSuccess)
      return e;
  }
  const int64_t NB = (L + PF_RB - 1) / PF_RB;
  k_pf_filter<<<dim3((unsigned)((NB + 1) / 2)), PF_NT, 0, st>>>(q, k, (int)L, kk, r_all, list, meta, m_s);
  if ((e = hipGetLastError()) != hipSuccess) return e;
  k_pf_select<<<dim3((unsigned)L), PF_SEL_NT, 0, st>>>(q, k, (int)L, kk, r_all, list, meta, idx, fails);
  if ((e = hipGetLastError()) != hipSuccess) return e;
  // rows the lists could not settle: a fixed grid reads their count on the device
  k_pf_fallback<<<pf_fallback_grid(L), ROW_NT, 0, st>>>(q, k, kk, fails, reinterpret_cast<int32_t*>(ws + l.fb_scores),
                                                       (int)L, idx, n_failed);
  if ((e = hipGetLastError()) != hipSuccess) return e;
  return hipSuccess;
}

}  // namespace lct
