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
//   S1/S2  two sweeps over every 16th key: per-row min/max of the sampled
//          scores, then a 128-bin histogram of them -> a threshold t_r with
//          m_s samples at or above it, m_s = k/16 + 6 sqrt(k/16) + 4 (about
//          1.56 k keys expected above it at k = 2048); rows with fewer
//          samples keep every key;
//   M      one sweep over all keys <= the row: every score >= t_r is a
//          candidate, stored as (position << 8 | bin), bin a monotone 7-bit
//          quantisation of the score, and counted in a per-row LDS histogram
//          of bins.  Each lane appends to its own sub-list of the row (16 per
//          row), so no slot is ever negotiated between lanes.
// k_pf_select (one wave per row): the bin histogram names the bin holding
// the k-th largest candidate; higher bins are all in; the exact scores of
// that bin's entries (recomputed, int32) settle the rest by (score desc,
// position asc).  Output through a position bitmap, ascending.
// Rows the lists cannot settle (a full sub-list, a crowded bin, fewer than
// k candidates) are listed and recomputed by the plain score + row select.
//
// k_pf_filter: waves 0..7 compute (rows 64*(w&1).., keys 32*(w>>1).. of each
// 128-key tile); wave 8 only brings key tiles into LDS by LDS DMA.  The
// compute waves never wait on a global memory operation inside a sweep, so
// their candidate stores are fire-and-forget; the helper's waits count only
// its own DMA.  Scores start from -base_r in the MFMA accumulator, so the
// threshold test and the bin come straight from the accumulated value.

#include <math.h>
#include <stddef.h>

#include <cmath>
#include <type_traits>

#include "common.h"
#include "kernels.h"

namespace lct {

constexpr int PF_HD = 256;                 // indexer features per row (int8)
constexpr int PF_KS = PF_HD / 64;          // 64-byte MFMA k-steps per row
constexpr int PF_RB = 128;                 // query rows per block
constexpr int PF_TK = 128;                 // keys per tile
constexpr int PF_SS = 16;                  // sample stride (positions)
constexpr int PF_NBIN = 128;               // histogram bins (sample and candidate)
constexpr int PF_BIN_FILL = 96;            // the sampled range spans < 96 candidate bins
constexpr int PF_CW = 8;                   // compute waves
constexpr int PF_NT = (PF_CW + 1) * 64;    // + one DMA wave
constexpr int PF_CHUNKS = 8 * PF_KS;       // 1 KiB fragments per key tile
constexpr int PF_SUB = PF_CROW / PF_NSUB;  // entries per sub-list; the last 8 are dump slots
constexpr int PF_LCAP = 512;               // select: entries of the k-th bin a wave can hold
constexpr int PF_SEL_W = 4;                // select: waves (rows) per workgroup
static_assert(PF_CROW % PF_NSUB == 0, "sub-lists tile the row list");

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

// The two key-tile buffers are objects of their own, apart from the rest:
// the compiler then sees that the LDS DMA writes only them and does not
// drain the (store-laden) vector memory counter before other LDS accesses.
struct PfShared {
  char (&kt_a)[PF_CHUNKS][1024];
  char (&kt_b)[PF_CHUNKS][1024];
  uint32_t (&hist)[PF_RB][PF_NBIN];  // sample histogram, then candidate bins
  int32_t (&smax)[PF_RB];
  int32_t (&smin)[PF_RB];
  int32_t (&base)[PF_RB];
  int32_t (&thd)[PF_RB];
  int32_t (&shf)[PF_RB];
};

// One sweep over key tiles [0, n_tiles) of keys at positions stride * j
// (j = tile * 128 + ..).  The helper wave DMAs tile t+1 while the compute
// waves run `body(tile, buf)` on tile t.  Every wave calls this.  Key rows
// past the cache read as zeros (range-checked buffer loads; the whole offset
// is in the per-lane register).
template <typename Body>
LCT_DEV void pf_sweep(PfShared& sh, __amdgpu_buffer_rsrc_t krs, int n_tiles, int stride, int wid,
                      int lane, Body body) {
  const int n = lane & 15, g = lane >> 4;
  // LDS addresses as 32-bit local pointers
  typedef __attribute__((address_space(3))) char lds_char;
  lds_char* const kta = (lds_char*)&sh.kt_a[0][0];
  lds_char* const ktb = (lds_char*)&sh.kt_b[0][0];
  auto issue = [&](int b, int t) {
    // opaque to the compiler, so that the 32 per-chunk offsets are formed
    // per tile instead of being hoisted out of the sweep (and spilled)
    uint32_t vb = (uint32_t)((t * PF_TK + n) * stride) * PF_HD + g * 16;
    __asm__ volatile("" : "+v"(vb));
    // (the instruction's immediate offset would move the LDS destination
    // too, so every offset goes into the per-lane register)
    auto go = [&](lds_char* dst) {
#pragma unroll
      for (int c = 0; c < PF_CHUNKS; ++c) {
        const uint32_t voff = vb + (uint32_t)((c / PF_KS) * 16 * stride * PF_HD + (c % PF_KS) * 64);
        __builtin_amdgcn_raw_ptr_buffer_load_lds(krs, (pf_lds_void*)(dst + c * 1024), 16, voff, 0, 0, 0);
      }
    };
    if (b) go(ktb);
    else go(kta);
  };
  if (wid == PF_CW && n_tiles > 0) issue(0, 0);
  auto step = [&](char (&cur)[PF_CHUNKS][1024], int nb, int t) {
    if (wid == PF_CW) PF_WAIT_VM0();  // tile t has landed (the helper issues nothing else)
    pf_barrier();
    if (wid == PF_CW) {
      if (t + 1 < n_tiles) issue(nb, t + 1);
    } else {
      body(t, cur);
    }
  };
  for (int t = 0; t < n_tiles; t += 2) {
    step(sh.kt_a, 1, t);
    if (t + 1 < n_tiles) step(sh.kt_b, 0, t + 1);
  }
  pf_barrier();  // every read of the last tile is done
}

// acc[qb][kl] = ini[qb] + scores of query rows 16qb + n (of the wave's 64)
// against keys 32wk + 16kl + 4g + e of the tile, e = vector element.
LCT_DEV void pf_tile_mfma(const char (&buf)[PF_CHUNKS][1024], const intx4 (&qf)[4][PF_KS], int wk,
                          int lane, const int32_t (&ini)[4], intx4 (&acc)[4][2]) {
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < 2; ++j) acc[i][j] = intx4{ini[i], ini[i], ini[i], ini[i]};
#pragma unroll
  for (int kl = 0; kl < 2; ++kl) {
#pragma unroll
    for (int ks = 0; ks < PF_KS; ++ks) {
      const intx4 a = *reinterpret_cast<const intx4*>(&buf[(wk * 2 + kl) * PF_KS + ks][lane * 16]);
#pragma unroll
      for (int qb = 0; qb < 4; ++qb)
        acc[qb][kl] = __builtin_amdgcn_mfma_i32_16x16x64_i8(a, qf[qb][ks], acc[qb][kl], 0, 0, 0);
    }
  }
}

// LDS counter increment written as inline assembly: the compiler would
// otherwise drain the vector memory counter before every LDS atomic (it
// cannot tell it from the key DMA), which for the compute waves means
// waiting for all of their candidate stores.  Only the counter updates go
// this way; reads of the counters follow an explicit LDS wait and barrier.
template <int OFF>
LCT_DEV void pf_lds_inc(uint32_t lds_addr) {
  __asm__ volatile("ds_add_u32 %0, %1 offset:%2" ::"v"(lds_addr), "v"(1u), "i"(OFF) : "memory");
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
                                                     uint32_t* __restrict__ strict_buf,
                                                     uint32_t* __restrict__ hist_out,
                                                     uint32_t* __restrict__ meta, int m_s) {
  __shared__ __attribute__((aligned(16))) char kt_a[PF_CHUNKS][1024];
  __shared__ __attribute__((aligned(16))) char kt_b[PF_CHUNKS][1024];
  __shared__ __attribute__((aligned(16))) uint32_t hist[PF_RB][PF_NBIN];
  __shared__ int32_t smax[PF_RB], smin[PF_RB], basev[PF_RB], thdv[PF_RB], shfv[PF_RB];
  PfShared sh{kt_a, kt_b, hist, smax, smin, basev, thdv, shfv};
  const int lane = threadIdx.x & 63, wid = wave_id();
  const int n = lane & 15, g = lane >> 4;
  const int wq = wid & 1, wk = wid >> 1;  // compute waves: row half, key quarter
  const int sub = wk * 4 + g;             // the lane's sub-list in each of its rows
  const int NB = (L + PF_RB - 1) / PF_RB;
  const __amdgpu_buffer_rsrc_t krs = make_rsrc(k, (int64_t)L * PF_HD);
  const __amdgpu_buffer_rsrc_t srs = make_rsrc(strict_buf, (int64_t)L * PF_CROW * 4);
  const int32_t zero[4] = {0, 0, 0, 0};

  for (int half = 0; half < 2; ++half) {
    const int rb = half == 0 ? (int)blockIdx.x : NB - 1 - (int)blockIdx.x;
    if (half == 1 && rb <= (int)blockIdx.x) break;  // the middle block has no partner
    const int r0 = rb * PF_RB;
    const int r_last = (r0 + PF_RB < L ? r0 + PF_RB : L) - 1;
    if (r_last < kk) continue;  // rows < k take every earlier position: nothing to score

    // ---- query fragments (compute waves): rows r0 + 64wq + 16qb + n
    intx4 qf[4][PF_KS];
    if (wid < PF_CW) {
#pragma unroll
      for (int qb = 0; qb < 4; ++qb) {
        const int row = r0 + wq * 64 + qb * 16 + n;
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
    }
    for (int i = threadIdx.x; i < PF_RB * PF_NBIN; i += PF_NT) (&sh.hist[0][0])[i] = 0u;
    __syncthreads();

    // ---- S1: per-row min / max of the sampled scores (rows past the
    // block's end collect garbage that nothing reads)
    const int n_samp = r_last / PF_SS + 1;  // sampled keys j: position 16 j <= r_last
    const int st_tiles = (n_samp + PF_TK - 1) / PF_TK;
    {
      int32_t mx[4], mn[4];
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        mx[i] = INT32_MIN;
        mn[i] = INT32_MAX;
      }
      pf_sweep(sh, krs, st_tiles, PF_SS, wid, lane, [&](int t, auto& buf) {
        intx4 acc[4][2];
        pf_tile_mfma(buf, qf, wk, lane, zero, acc);
        const bool diag = (t * PF_TK + PF_TK - 1) * PF_SS > r0;  // a sample past some row
#pragma unroll
        for (int qb = 0; qb < 4; ++qb) {
          const int row = r0 + wq * 64 + qb * 16 + n;
#pragma unroll
          for (int kl = 0; kl < 2; ++kl)
#pragma unroll
            for (int e = 0; e < 4; ++e) {
              const int pos = (t * PF_TK + wk * 32 + kl * 16 + g * 4 + e) * PF_SS;
              if (!diag || pos <= row) {
                mx[qb] = max(mx[qb], acc[qb][kl][e]);
                mn[qb] = min(mn[qb], acc[qb][kl][e]);
              }
            }
        }
      });
      if (wid < PF_CW) {
#pragma unroll
        for (int qb = 0; qb < 4; ++qb) {
          int32_t a = mx[qb], b = mn[qb];
          a = max(a, __shfl_xor(a, 16, 64));
          a = max(a, __shfl_xor(a, 32, 64));
          b = min(b, __shfl_xor(b, 16, 64));
          b = min(b, __shfl_xor(b, 32, 64));
          if (g == 0) {
            const int rl = wq * 64 + qb * 16 + n;
            atomicMax(&sh.smax[rl], a);
            atomicMin(&sh.smin[rl], b);
          }
        }
      }
      __syncthreads();
    }
    // ---- S2: 128-bin histogram of the sampled scores over [min, max]
    {
      int32_t lo[4];
      uint32_t M[4];
#pragma unroll
      for (int qb = 0; qb < 4; ++qb) {
        const int rl = wq * 64 + qb * 16 + n;
        lo[qb] = sh.smin[rl];
        const uint32_t span = (uint32_t)(sh.smax[rl] - lo[qb]) + 1u;
        M[qb] = span == 0u ? 1u : ((1u << 23) - 1u) / span;
      }
      pf_sweep(sh, krs, st_tiles, PF_SS, wid, lane, [&](int t, auto& buf) {
        intx4 acc[4][2];
        pf_tile_mfma(buf, qf, wk, lane, zero, acc);
        const bool diag = (t * PF_TK + PF_TK - 1) * PF_SS > r0;
#pragma unroll
        for (int qb = 0; qb < 4; ++qb) {
          const int rl = wq * 64 + qb * 16 + n;
          const int row = r0 + rl;
#pragma unroll
          for (int kl = 0; kl < 2; ++kl)
#pragma unroll
            for (int e = 0; e < 4; ++e) {
              const int pos = (t * PF_TK + wk * 32 + kl * 16 + g * 4 + e) * PF_SS;
              if (!diag || pos <= row)
                atomicAdd(&sh.hist[rl][pf_sample_bin((uint32_t)(acc[qb][kl][e] - lo[qb]), M[qb])], 1u);
            }
        }
      });
    }
    // ---- threshold, bin base and bin shift per row
    if (threadIdx.x < PF_RB) {
      const int rl = threadIdx.x;
      const int row = r0 + rl;
      int32_t thd = INT32_MAX, bs = 0, sf = 0;  // rows without candidates
      if (row <= r_last && row >= kk) {
        const int32_t lo = sh.smin[rl], hi = sh.smax[rl];
        const uint32_t span = (uint32_t)(hi - lo) + 1u;
        if (row / PF_SS + 1 >= m_s) {
          const uint32_t M = ((1u << 23) - 1u) / span;
          uint32_t acc = 0;
          int b = PF_NBIN - 1;
          for (; b > 0; --b) {
            acc += sh.hist[rl][b];
            if (acc >= (uint32_t)m_s) break;
          }
          // the smallest score whose sample bin is >= b: every score at or
          // above it is a candidate
          bs = lo + (int32_t)(((uint32_t)b * 65536u + M - 1u) / M);
          thd = -1;  // candidate: score - bs >= 0
        } else {
          bs = lo - (int32_t)(span >> 2) - 1;  // every key is a candidate
          thd = INT32_MIN;
        }
        while ((((int64_t)hi - bs) >> sf) >= PF_BIN_FILL) ++sf;
      }
      sh.base[rl] = bs;
      sh.thd[rl] = thd;
      sh.shf[rl] = sf;
      if (row <= r_last) {
        meta[(size_t)row * PF_META + PF_NSUB] = (uint32_t)bs;
        meta[(size_t)row * PF_META + PF_NSUB + 1] = (uint32_t)sf;
      }
    }
    __syncthreads();
    for (int i = threadIdx.x; i < PF_RB * PF_NBIN; i += PF_NT) (&sh.hist[0][0])[i] = 0u;
    __syncthreads();

    // ---- M: all keys <= the block's last row; candidates to the sub-lists
    {
      int32_t ini[4], thd[4], sf[4];
      uint32_t off[4];
      // byte offset of sub-list `sub` of row r0 + 64 wq + n; row 16 qb
      // further on starts 16 qb PF_CROW entries later
      const uint32_t off0 = ((uint32_t)(r0 + wq * 64 + n) * PF_CROW + sub * PF_SUB) * 4u;
#pragma unroll
      for (int qb = 0; qb < 4; ++qb) {
        const int rl = wq * 64 + qb * 16 + n;
        ini[qb] = -sh.base[rl];
        thd[qb] = sh.thd[rl];
        sf[qb] = sh.shf[rl];
        off[qb] = off0 + (uint32_t)(qb * 16 * PF_CROW * 4);
      }
      const uint32_t g8 = (uint32_t)(g * 4) << 8;
      // LDS byte address of hist[64 wq + n][0]; row 16 qb further on is the
      // instruction's immediate offset
      const uint32_t hrow = (uint32_t)(uintptr_t)(__attribute__((address_space(3))) uint32_t*)&hist[0][0] +
                            (uint32_t)((wq * 64 + n) * PF_NBIN * 4);
      auto emit = [&](auto diag_c, int t, const intx4 (&acc)[4][2]) {
        constexpr bool DIAG = decltype(diag_c)::value;
        // entry = position << 8 | bin; the position's tile / wave / element
        // part is uniform across the wave (one scalar per element)
        uint32_t pu[2][4];
#pragma unroll
        for (int kl = 0; kl < 2; ++kl)
#pragma unroll
          for (int e = 0; e < 4; ++e)
            pu[kl][e] = __builtin_amdgcn_readfirstlane((uint32_t)(t * PF_TK + wk * 32 + kl * 16 + e) << 8);
        auto per_qb = [&](auto qb_c) {
          constexpr int qb = decltype(qb_c)::value;
          const int rl = wq * 64 + qb * 16 + n;
#pragma unroll
          for (int kl = 0; kl < 2; ++kl)
#pragma unroll
            for (int e = 0; e < 4; ++e) {
              const int32_t d = acc[qb][kl][e];
              bool c = d > thd[qb];
              if (DIAG) c = c && t * PF_TK + wk * 32 + kl * 16 + g * 4 + e <= r0 + rl;
              if (c) {
                const int32_t bq = d >> sf[qb];
                const uint32_t bin = (uint32_t)(bq < 0 ? 0 : bq > PF_NBIN - 1 ? PF_NBIN - 1 : bq);
                pf_lds_inc<qb * 16 * PF_NBIN * 4>(hrow + bin * 4);
                __builtin_amdgcn_raw_buffer_store_b32(pu[kl][e] + g8 + bin, srs, (int)off[qb], 0, 0);
                off[qb] += 4u;
              }
            }
          // a lane adds at most 8 entries per row and tile: past the usable
          // slots, the next 8 writes land in the dump slots
          off[qb] = min(off[qb], off0 + (uint32_t)((qb * 16 * PF_CROW + PF_SUB - 8) * 4));
        };
        per_qb(std::integral_constant<int, 0>{});
        per_qb(std::integral_constant<int, 1>{});
        per_qb(std::integral_constant<int, 2>{});
        per_qb(std::integral_constant<int, 3>{});
      };
      const int m_tiles = (r_last + 1 + PF_TK - 1) / PF_TK;
      pf_sweep(sh, krs, m_tiles, 1, wid, lane, [&](int t, auto& buf) {
        intx4 acc[4][2];
        pf_tile_mfma(buf, qf, wk, lane, ini, acc);
        if (t * PF_TK + PF_TK - 1 > r0) emit(std::true_type{}, t, acc);
        else emit(std::false_type{}, t, acc);
      });
      // candidate counts per (row, sub-list); a count of PF_SUB - 8 means
      // the sub-list may have overflowed into its dump slots
      if (wid < PF_CW) {
#pragma unroll
        for (int qb = 0; qb < 4; ++qb) {
          const int row = r0 + wq * 64 + qb * 16 + n;
          if (row <= r_last && row >= kk)
            meta[(size_t)row * PF_META + sub] = (off[qb] - off0 - (uint32_t)(qb * 16 * PF_CROW * 4)) >> 2;
        }
      }
    }
    __syncthreads();
    // ---- per-row bin histogram for the select
    for (int i = threadIdx.x; i < PF_RB * PF_NBIN; i += PF_NT) {
      const int rl = i / PF_NBIN;
      if (r0 + rl <= r_last) hist_out[(size_t)r0 * PF_NBIN + i] = (&sh.hist[0][0])[i];
    }
    __syncthreads();  // LDS reuse by the next block
  }
}

// ---- exact select per row from the candidate lists ----------------------

struct PfSelShared {
  uint32_t bm[PF_SEL_W][2048];  // position bitmap (65536 positions)
  uint32_t lpos[PF_SEL_W][PF_LCAP];
  int32_t lsc[PF_SEL_W][PF_LCAP];
  uint32_t sub[PF_SEL_W][256];  // exact-score histogram of the k-th bin, then its ties
  uint32_t qrow[PF_SEL_W][PF_HD / 4];
};

LCT_DEV void pf_wave_sync() {
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
  __builtin_amdgcn_wave_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
}

LCT_DEV uint32_t pf_mbcnt(uint64_t m) {
  return __builtin_amdgcn_mbcnt_hi((uint32_t)(m >> 32), __builtin_amdgcn_mbcnt_lo((uint32_t)m, 0u));
}

// Over the counts c(b) of bins b = top .. 0 held two per lane (lane l: bins
// top - 2l and top - 2l - 1), find the bin that holds the need-th largest
// entry.  Returns false if the counts sum to less than need.
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

__global__ __launch_bounds__(PF_SEL_W * 64) void k_pf_select(
    const int8_t* __restrict__ q, const int8_t* __restrict__ k, int L, int kk,
    const uint32_t* __restrict__ strict_buf, const uint32_t* __restrict__ hist,
    const uint32_t* __restrict__ meta, int32_t* __restrict__ idx, int32_t* __restrict__ fails) {
  __shared__ __attribute__((aligned(16))) PfSelShared sh;
  const int lane = threadIdx.x & 63, wid = wave_id();
  const int row = blockIdx.x * PF_SEL_W + wid;
  if (row >= L) return;
  int32_t* out = idx + (size_t)row * kk;
  if (row < kk) {
    for (int j = lane; j < kk; j += 64) out[j] = j <= row ? j : -1;
    return;
  }
  // counts of the 16 sub-lists, the bin base and shift
  const uint32_t mw = lane < PF_NSUB + 2 ? meta[(size_t)row * PF_META + lane] : 0u;
  const uint32_t cnt_l = lane < PF_NSUB ? mw : 0u;
  const uint32_t total = wave_sum(cnt_l);
  const bool full = __ballot(lane < PF_NSUB && mw >= (uint32_t)(PF_SUB - 8)) != 0;
  const int32_t base = (int32_t)__shfl(mw, PF_NSUB, 64);
  const int sf = (int)__shfl(mw, PF_NSUB + 1, 64);
  bool fail = full || total < (uint32_t)kk;
  uint32_t bsel = 0, above = 0, nsel = 0;
  if (!fail) {
    const uint2 hw = reinterpret_cast<const uint2*>(hist + (size_t)row * PF_NBIN)[63 - lane];
    // hw.y = bin 127 - 2 lane, hw.x = bin 126 - 2 lane
    if (!pf_find_bin(hw.y, hw.x, PF_NBIN - 1, (uint32_t)kk, lane, bsel, above, nsel)) fail = true;
    if (nsel > (uint32_t)PF_LCAP) fail = true;
  }
  if (fail) {
    if (lane == 0) fails[1 + atomicAdd(&fails[0], 1)] = row;
    return;
  }
  const uint32_t need1 = (uint32_t)kk - above;  // taken from the k-th bin, 1..nsel
  uint32_t* bm = sh.bm[wid];
  uint32_t* lpos = sh.lpos[wid];
  int32_t* lsc = sh.lsc[wid];
  const uint32_t nwords = (uint32_t)((row + 1 + 31) / 32);
  for (uint32_t w = lane; w < nwords; w += 64) bm[w] = 0u;
  pf_wave_sync();
  // bins above bsel are in; bin bsel goes to the list (two sub-lists, ten
  // loads in flight per lane)
  {
    const uint32_t* sp = strict_buf + (size_t)row * PF_CROW;
    uint32_t lcount = 0;
    for (int s0 = 0; s0 < PF_NSUB; s0 += 2) {
      uint32_t e[2][5];
#pragma unroll
      for (int h = 0; h < 2; ++h) {
        const uint32_t c = __shfl(cnt_l, s0 + h, 64);
#pragma unroll
        for (int m = 0; m < 5; ++m) {
          const uint32_t i = m * 64 + lane;
          e[h][m] = i < c ? sp[(s0 + h) * PF_SUB + i] : 0xFFFFFFFFu;
        }
      }
#pragma unroll
      for (int h = 0; h < 2; ++h)
#pragma unroll
        for (int m = 0; m < 5; ++m) {
          const uint32_t b = e[h][m] & 255u, p = e[h][m] >> 8;
          const bool valid = e[h][m] != 0xFFFFFFFFu;
          if (valid && b > bsel) atomicOr(&bm[p >> 5], 1u << (p & 31));
          const bool inl = valid && b == bsel;
          const uint64_t bl = __ballot(inl);
          if (inl) {
            const uint32_t slot = lcount + pf_mbcnt(bl);
            if (slot < (uint32_t)PF_LCAP) lpos[slot] = p;  // the bin holds exactly nsel entries
          }
          lcount += (uint32_t)__popcll(bl);
        }
    }
  }
  // exact scores of the bin's entries
  sh.qrow[wid][lane] = reinterpret_cast<const uint32_t*>(q + (size_t)row * PF_HD)[lane];
  pf_wave_sync();
  for (uint32_t j = lane; j < nsel; j += 64) {
    const int8_t* kp = k + (size_t)lpos[j] * PF_HD;
    int32_t s = 0;
#pragma unroll
    for (int w = 0; w < PF_HD / 16; ++w) {
      const uintx4 kv = *reinterpret_cast<const uintx4*>(kp + w * 16);
      const uintx4 qv = *reinterpret_cast<const uintx4*>(&sh.qrow[wid][w * 4]);
      s = __builtin_amdgcn_sdot4((int)qv.x, (int)kv.x, s, false);
      s = __builtin_amdgcn_sdot4((int)qv.y, (int)kv.y, s, false);
      s = __builtin_amdgcn_sdot4((int)qv.z, (int)kv.z, s, false);
      s = __builtin_amdgcn_sdot4((int)qv.w, (int)kv.w, s, false);
    }
    lsc[j] = s;
  }
  pf_wave_sync();
  // the need1 best of the bin by (score desc, position asc).  Inner bins
  // span 2^sf consecutive scores from lo_b: with sf <= 7 a 128-counter
  // exact-score histogram finds the cut score T, and only the ties at T are
  // ranked.
  const int32_t lo_b = base + (int32_t)(bsel << sf);
  bool ranked = false;
  if (bsel > 0 && bsel < (uint32_t)(PF_NBIN - 1) && sf <= 7) {
    uint32_t* sh_sub = sh.sub[wid];
    for (int i = lane; i < 128; i += 64) sh_sub[i] = 0u;
    pf_wave_sync();
    for (uint32_t j = lane; j < nsel; j += 64) atomicAdd(&sh_sub[lsc[j] - lo_b], 1u);
    pf_wave_sync();
    const uint2 hw = reinterpret_cast<const uint2*>(sh_sub)[63 - lane];
    uint32_t tb, ab2, n_eq;
    const bool found = pf_find_bin(hw.y, hw.x, 127, need1, lane, tb, ab2, n_eq);
    const int32_t T = lo_b + (int32_t)tb;
    const uint32_t need_eq = need1 - ab2;  // ties at T to take, 1..n_eq
    pf_wave_sync();
    if (found && n_eq <= 256) {
      // ties at T compacted into sh_sub, then ranked by position
      uint32_t tcount = 0;
      for (uint32_t j0 = 0; j0 < nsel; j0 += 64) {
        const uint32_t j = j0 + lane;
        const bool in = j < nsel;
        const int32_t s = in ? lsc[j] : INT32_MIN;
        const uint32_t p = in ? lpos[j] : 0u;
        if (in && s > T) atomicOr(&bm[p >> 5], 1u << (p & 31));
        const uint64_t bl = __ballot(in && s == T);
        if (in && s == T) sh_sub[tcount + pf_mbcnt(bl)] = p;
        tcount += (uint32_t)__popcll(bl);
      }
      pf_wave_sync();
      for (uint32_t j = lane; j < n_eq; j += 64) {
        const uint32_t p = sh_sub[j];
        uint32_t r = 0;
        for (uint32_t m = 0; m < n_eq; ++m) r += sh_sub[m] < p ? 1u : 0u;
        if (r < need_eq) atomicOr(&bm[p >> 5], 1u << (p & 31));
      }
      ranked = true;
    }
  }
  if (!ranked) {
    // any bin: rank every entry of the bin against all the others
    for (uint32_t j = lane; j < nsel; j += 64) {
      const int32_t s = lsc[j];
      const uint32_t p = lpos[j];
      uint32_t r = 0;
      for (uint32_t m = 0; m < nsel; ++m) {
        const int32_t sm = lsc[m];
        const uint32_t pm = lpos[m];
        r += (sm > s || (sm == s && pm < p)) ? 1u : 0u;
      }
      if (r < need1) atomicOr(&bm[p >> 5], 1u << (p & 31));
    }
  }
  pf_wave_sync();
  // emit ascending: lane l expands words [32l, 32l + 32)
  uint32_t cnt = 0;
  for (int j = 0; j < 32; ++j) {
    const uint32_t w = lane * 32 + j;
    cnt += w < nwords ? __popc(bm[w]) : 0u;
  }
  const uint32_t incl = wave_incl_scan(cnt);
  uint32_t off = incl - cnt;
  for (int j = 0; j < 32; ++j) {
    const uint32_t w = lane * 32 + j;
    uint32_t v = w < nwords ? bm[w] : 0u;
    while (v) {
      const uint32_t b = __ffs(v) - 1;
      v &= v - 1;
      if (off < (uint32_t)kk) out[off] = (int32_t)(w * 32 + b);
      ++off;
    }
  }
  const uint32_t tot = __shfl(incl, 63, 64);
  for (uint32_t j = tot + lane; j < (uint32_t)kk; j += 64) out[j] = -1;
}

// ---- plain path for the rows the lists could not settle -----------------

// compact the queries of failed rows [b0, b0 + nb) of the list
__global__ __launch_bounds__(256) void k_pf_fb_gather(const int8_t* __restrict__ q,
                                                      const int32_t* __restrict__ rows,
                                                      int8_t* __restrict__ qc,
                                                      int32_t* __restrict__ vlen) {
  const int slot = blockIdx.x;
  const int64_t row = rows[slot];
  for (int i = threadIdx.x; i < PF_HD; i += 256) qc[(size_t)slot * PF_HD + i] = q[row * PF_HD + i];
  if (threadIdx.x == 0) vlen[slot] = (int32_t)(row + 1);
}

__global__ __launch_bounds__(256) void k_pf_fb_scatter(const int32_t* __restrict__ fidx, int kk,
                                                       const int32_t* __restrict__ rows,
                                                       int32_t* __restrict__ idx) {
  const int slot = blockIdx.x;
  const int64_t row = rows[slot];
  for (int j = threadIdx.x; j < kk; j += 256) idx[row * kk + j] = fidx[(size_t)slot * kk + j];
}

__global__ void k_pf_zero_fails(int32_t* fails) {
  if (threadIdx.x == 0) fails[0] = 0;
}

size_t pf_workspace_layout(int64_t L, int HD, int kk, PfLayout* lay) {
  (void)HD;
  auto up = [](size_t x) { return (x + 255) & ~size_t(255); };
  PfLayout l;
  size_t off = 0;
  l.strict = off;
  off += up((size_t)L * PF_CROW * 4);
  l.hist = off;
  off += up((size_t)L * PF_NBIN * 4);
  l.meta = off;
  off += up((size_t)L * PF_META * 4);
  l.fails = off;
  off += up((size_t)(1 + L) * 4);
  l.qc = off;
  off += up((size_t)PF_FAIL_CAP * PF_HD);
  l.vlen = off;
  off += up((size_t)PF_FAIL_CAP * 4);
  l.fscores = off;
  off += up((size_t)PF_FAIL_CAP * L * 4);
  l.fidx = off;
  off += up((size_t)PF_FAIL_CAP * kk * 4);
  l.total = off;
  if (lay) *lay = l;
  return off;
}

hipError_t launch_pf_fused(const int8_t* q, const int8_t* k, int64_t L, int HD, int kk,
                           int32_t* idx, char* ws, hipStream_t st, int* n_failed) {
  if (HD != PF_HD || L < 1 || L > PF_MAX_L || kk < 1 || kk > PF_MAX_K) return hipErrorInvalidValue;
  PfLayout l;
  pf_workspace_layout(L, HD, kk, &l);
  auto strict = reinterpret_cast<uint32_t*>(ws + l.strict);
  auto hist = reinterpret_cast<uint32_t*>(ws + l.hist);
  auto meta = reinterpret_cast<uint32_t*>(ws + l.meta);
  auto fails = reinterpret_cast<int32_t*>(ws + l.fails);
  hipError_t e;
  k_pf_zero_fails<<<1, 64, 0, st>>>(fails);
  if ((e = hipGetLastError()) != hipSuccess) return e;
  const int64_t NB = (L + PF_RB - 1) / PF_RB;
  // sampled keys (every 16th) wanted at or above the threshold: k/16 plus
  // six times the spread of that count, so that fewer than k candidates is rare
  const double ks = kk / (double)PF_SS;
  const int m_s = (int)std::ceil(ks + 6.0 * std::sqrt(ks)) + 4;
  k_pf_filter<<<dim3((unsigned)((NB + 1) / 2)), PF_NT, 0, st>>>(q, k, (int)L, kk, strict, hist,
                                                                meta, m_s);
  if ((e = hipGetLastError()) != hipSuccess) return e;
  k_pf_select<<<dim3((unsigned)((L + PF_SEL_W - 1) / PF_SEL_W)), PF_SEL_W * 64, 0, st>>>(
      q, k, (int)L, kk, strict, hist, meta, idx, fails);
  if ((e = hipGetLastError()) != hipSuccess) return e;
  // rows the lists could not settle: the count decides how much plain work follows
  int32_t nf = 0;
  if ((e = hipMemcpyAsync(&nf, fails, sizeof(nf), hipMemcpyDeviceToHost, st)) != hipSuccess) return e;
  if ((e = hipStreamSynchronize(st)) != hipSuccess) return e;
  if (n_failed) *n_failed = nf;
  auto qc = reinterpret_cast<int8_t*>(ws + l.qc);
  auto vlen = reinterpret_cast<int32_t*>(ws + l.vlen);
  auto fscores = reinterpret_cast<int32_t*>(ws + l.fscores);
  auto fidx = reinterpret_cast<int32_t*>(ws + l.fidx);
  for (int b0 = 0; b0 < nf; b0 += PF_FAIL_CAP) {
    const int nb = nf - b0 < PF_FAIL_CAP ? nf - b0 : PF_FAIL_CAP;
    const int32_t* rows = fails + 1 + b0;
    k_pf_fb_gather<<<nb, 256, 0, st>>>(q, rows, qc, vlen);
    if ((e = hipGetLastError()) != hipSuccess) return e;
    if ((e = launch_idx_score_mfma(qc, k, fscores, 1, nb, L, PF_HD, -1, st)) != hipSuccess) return e;
    if ((e = launch_topk_rows(fscores, 0, fidx, nb, L, L, kk, vlen, 1, -1, st)) != hipSuccess) return e;
    k_pf_fb_scatter<<<nb, 256, 0, st>>>(fidx, kk, rows, idx);
    if ((e = hipGetLastError()) != hipSuccess) return e;
  }
  return hipSuccess;
}

}  // namespace lct
