// Indexer scores for gfx950.
//
// Source: tutorial page, section "DSA 与 IndexShare": a lightweight indexer
// scores every history token for the current query.  Reading: the score is
// the sum over indexer heads of per-head int8 dot products, which equals one
// dot product over the row's H_idx * d_idx int8 features.
//
// Decode (few query rows): the key cache is streamed once from HBM with
// 16-byte loads.  P = HD/16 lanes share one key row; in each of P steps a
// wave reads 64/P consecutive rows (64*16 contiguous bytes), multiplies them
// with v_dot4_i32_i8 against the query bytes the lane holds, and keeps one
// partial per step.  A butterfly reduce-scatter over the P lanes (P-1
// shuffles) then leaves every lane with the full score of one position, so
// each wave ends a round of 64 positions with 64 scores to store.
// One workgroup per tile of SCORE_TILE positions of one row (4 waves, each
// taking every 4th round of the tile).  The same pass records the per-tile
// (min, max) of the keys a following top-k select needs.
//
// Prefill (many query rows): S = Qi * Ki^T is a dense int8 contraction, run
// on v_mfma_i32_16x16x64_i8 with 128x128 output tiles per workgroup; tiles
// strictly above the causal diagonal are skipped.

#include "common.h"
#include "kernels.h"

namespace lct {

ScorePlan score_plan(int B, int Lq, int64_t L, int HD) {
  ScorePlan p;
  p.qc = Lq <= 1 ? 1 : Lq <= 2 ? 2 : Lq <= 4 ? 4 : Lq <= 8 ? 8 : 16;
  if (HD >= 512 && p.qc > 4) p.qc = 4;  // register budget
  p.nqc = (Lq + p.qc - 1) / p.qc;
  p.tiles = (int)((L + SCORE_TILE - 1) / SCORE_TILE);
  return p;
}

LCT_DEV int dot16(intx4 a, intx4 b) {
  int acc = 0;
  acc = __builtin_amdgcn_sdot4(a.x, b.x, acc, false);
  acc = __builtin_amdgcn_sdot4(a.y, b.y, acc, false);
  acc = __builtin_amdgcn_sdot4(a.z, b.z, acc, false);
  acc = __builtin_amdgcn_sdot4(a.w, b.w, acc, false);
  return acc;
}

template <int P, int QC>
__global__ __launch_bounds__(256) void k_idx_score_stream(
    const int8_t* __restrict__ q, const int8_t* __restrict__ k, int32_t* __restrict__ s, int Lq,
    int64_t L, int64_t q_pos0, int n_qchunks, uint32_t* __restrict__ mm, int t1,
    TopkRowState* __restrict__ st, uint32_t* __restrict__ hist,
    const int32_t* __restrict__ valid_len) {
  constexpr int HD = P * 16;
  constexpr int G = 64 / P;  // consecutive rows read per step
  constexpr int ROUNDS = SCORE_TILE / (4 * 64);
  __shared__ uint32_t lds[2 * QC * 4];
  const int lane = threadIdx.x & 63, wid = wave_id();
  const int tile = blockIdx.x;
  const int b = blockIdx.y / n_qchunks;
  const int r0 = (blockIdx.y % n_qchunks) * QC;
  const int g = lane / P, j = lane % P;

  intx4 qv[QC];
#pragma unroll
  for (int i = 0; i < QC; ++i) {
    const int r = r0 + i < Lq ? r0 + i : Lq - 1;  // rows past Lq are computed, never stored
    qv[i] = *reinterpret_cast<const intx4*>(q + ((size_t)b * Lq + r) * HD + j * 16);
  }
  uint32_t nv = (uint32_t)L;
  if (valid_len) {
    int32_t v = valid_len[b];
    nv = v < 0 ? 0u : ((int64_t)v < L ? (uint32_t)v : (uint32_t)L);
  }
  uint32_t mn[QC], mx[QC];
#pragma unroll
  for (int i = 0; i < QC; ++i) {
    mn[i] = 0xFFFFFFFFu;
    mx[i] = 0u;
  }
  const __amdgpu_buffer_rsrc_t krs = make_rsrc(k + (size_t)b * L * HD, L * HD);
  const uint32_t lane_off = (uint32_t)(g * HD + j * 16);
  for (int rd = 0; rd < ROUNDS; ++rd) {
    const int64_t base = (int64_t)tile * SCORE_TILE + (int64_t)(rd * 4 + wid) * 64;
    if (base >= L) break;
    // All P loads are issued before any arithmetic, as buffer loads over the
    // key rows of this batch entry.  The whole byte offset is in the per-lane
    // operand, so the buffer range check covers it: rows past L read zeros
    // (their scores are never stored).
    intx4 kv[P];
    const uint32_t off = (uint32_t)(base * HD) + lane_off;
#pragma unroll
    for (int t = 0; t < P; ++t)
      kv[t] = __builtin_amdgcn_raw_buffer_load_b128(krs, (int)(off + (uint32_t)(t * G * HD)), 0, BUF_NT);
    // keep the loads ahead of the arithmetic (the scheduler would otherwise
    // trade memory-level parallelism for registers)
    __builtin_amdgcn_sched_barrier(0);
    const int64_t pos = base + j * G + g;  // the position this lane ends up owning
#pragma unroll
    for (int i = 0; i < QC; ++i) {
      int acc[P];
#pragma unroll
      for (int t = 0; t < P; ++t) acc[t] = dot16(kv[t], qv[i]);
#pragma unroll
      for (int d = P / 2; d >= 1; d >>= 1) {
        const bool upper = (j & d) != 0;
#pragma unroll
        for (int t = 0; t < d; ++t) {
          int send = upper ? acc[t] : acc[t + d];
          int keep = upper ? acc[t + d] : acc[t];
          acc[t] = keep + __shfl_xor(send, d, 64);
        }
      }
      const int r = r0 + i;
      if (r < Lq && pos < L) {
        int32_t v = acc[0];
        bool cand = pos < (int64_t)nv;
        if (q_pos0 >= 0 && pos > q_pos0 + r) {
          v = INT32_MIN;
          cand = false;
        }
        s[((size_t)b * Lq + r) * L + pos] = v;
        if (cand) {
          uint32_t key = key_of_i32(v);
          mn[i] = min(mn[i], key);
          mx[i] = max(mx[i], key);
        }
      }
    }
  }
  if (mm) {
#pragma unroll
    for (int i = 0; i < QC; ++i) {
      uint32_t a = wave_min(mn[i]), c = wave_max(mx[i]);
      if (lane == 0) {
        lds[(i * 4 + wid) * 2 + 0] = a;
        lds[(i * 4 + wid) * 2 + 1] = c;
      }
    }
    __syncthreads();
    if (threadIdx.x < QC && r0 + (int)threadIdx.x < Lq) {
      const int i = threadIdx.x;
      uint32_t a = lds[(i * 4) * 2], c = lds[(i * 4) * 2 + 1];
      for (int w = 1; w < 4; ++w) {
        a = min(a, lds[(i * 4 + w) * 2]);
        c = max(c, lds[(i * 4 + w) * 2 + 1]);
      }
      const size_t row = (size_t)b * Lq + r0 + i;
      mm[(row * t1 + tile) * 2 + 0] = a;
      mm[(row * t1 + tile) * 2 + 1] = c;
      if (tile == 0) st[row].cand_fill = 0;
    }
    if (tile == 0) {
      // clear the rows' select histograms (accumulated by the next kernel)
      for (int i = 0; i < QC; ++i)
        if (r0 + i < Lq) hist[((size_t)b * Lq + r0 + i) * TOPK_NB + threadIdx.x % TOPK_NB] = 0u;
    }
  }
}

template <int P>
static hipError_t stream_dispatch_qc(const ScorePlan& pl, int B, const int8_t* q, const int8_t* k,
                                     int32_t* s, int Lq, int64_t L, int64_t q_pos0, uint32_t* mm,
                                     TopkRowState* st, uint32_t* hist, const int32_t* vl,
                                     hipStream_t stream) {
  const dim3 grid(pl.tiles, B * pl.nqc);
#define LCT_SC(QC)                                                                             \
  k_idx_score_stream<P, QC><<<grid, 256, 0, stream>>>(q, k, s, Lq, L, q_pos0, pl.nqc, mm,      \
                                                      pl.tiles, st, hist, vl)
  switch (pl.qc) {
    case 1: LCT_SC(1); break;
    case 2: LCT_SC(2); break;
    case 4: LCT_SC(4); break;
    case 8: LCT_SC(8); break;
    default: LCT_SC(16); break;
  }
#undef LCT_SC
  return hipGetLastError();
}

hipError_t launch_idx_score_stream(const int8_t* q, const int8_t* k, int32_t* s, int B, int Lq,
                                   int64_t L, int HD, int64_t q_pos0, uint32_t* mm,
                                   TopkRowState* state, uint32_t* hist,
                                   const int32_t* valid_len, hipStream_t stream) {
  const ScorePlan pl = score_plan(B, Lq, L, HD);
  switch (HD) {
    case 16: return stream_dispatch_qc<1>(pl, B, q, k, s, Lq, L, q_pos0, mm, state, hist, valid_len, stream);
    case 32: return stream_dispatch_qc<2>(pl, B, q, k, s, Lq, L, q_pos0, mm, state, hist, valid_len, stream);
    case 64: return stream_dispatch_qc<4>(pl, B, q, k, s, Lq, L, q_pos0, mm, state, hist, valid_len, stream);
    case 128: return stream_dispatch_qc<8>(pl, B, q, k, s, Lq, L, q_pos0, mm, state, hist, valid_len, stream);
    case 256: return stream_dispatch_qc<16>(pl, B, q, k, s, Lq, L, q_pos0, mm, state, hist, valid_len, stream);
    case 512: return stream_dispatch_qc<32>(pl, B, q, k, s, Lq, L, q_pos0, mm, state, hist, valid_len, stream);
    default: return hipErrorInvalidValue;
  }
}

// ------------------------------------------------------------- prefill ----
// Dense scores S = Qi Ki^T on v_mfma_i32_16x16x64_i8, computed as S^T tiles
// (keys are the MFMA rows, queries the columns) so that every lane ends with
// 4 consecutive keys of one query row: 16-byte stores along the score rows.
// Workgroup: MF_Q queries x MF_KT key tiles of 128.  The query fragments stay
// in registers for the whole loop; each 128-key tile is brought into LDS by
// LDS DMA (global_load_lds_dwordx4, one 1 KiB MFMA fragment per instruction)
// while the previous tile is multiplied.  2*MF_NWR waves of 64 queries x 64
// keys; a key tile serves all MF_Q queries (fewer re-reads of the keys).
// Tiles strictly above the causal diagonal are skipped, entries above it in
// the diagonal tiles are written as INT32_MIN.  Scores go out as buffer
// stores over the workgroup's rows: out-of-range elements (rows past Lq,
// keys past L) get an offset past the buffer and are dropped, so every wave
// issues the same number of stores per tile and the wait for the next tile's
// DMA can count them.  With 16-byte stores, each 16-query slice of a wave's
// tile is first turned around in a 4 KiB LDS buffer (chunk index XOR row,
// conflict-free both ways) so that each store instruction writes 4 whole
// 256-byte row pieces instead of 16 pieces of 64 bytes.
constexpr int MF_NWR = 2;   // waves along the query dimension (x2 along keys)
constexpr int MF_Q = 64 * MF_NWR;  // queries per workgroup
constexpr int MF_K = 128;   // keys per tile
constexpr int MF_KT = 4;    // key tiles per workgroup (more, smaller workgroups write faster)

typedef __attribute__((address_space(3))) void mf_lds_void;
typedef const __attribute__((address_space(1))) void mf_global_cvoid;

// s_waitcnt vmcnt(n) with expcnt / lgkmcnt left at their maxima (n < 64)
#define MF_WAIT_VM(n) __builtin_amdgcn_s_waitcnt((((n) & 15) | (((n) >> 4) << 14)) | 0x0F70)

// KS = HD / 64 k-steps; VEC: 16-byte stores (L % 4 == 0), else 4-byte ones
template <int KS, bool VEC>
__global__ __launch_bounds__(128 * MF_NWR) void k_idx_score_mfma(const int8_t* __restrict__ q,
                                                        const int8_t* __restrict__ k,
                                                        int32_t* __restrict__ s, int Lq,
                                                        int64_t L, int64_t q_pos0) {
  constexpr int HD = KS * 64;
  constexpr int CHUNKS = 8 * KS;          // 1 KiB fragments per key tile
  constexpr int NWV = 2 * MF_NWR;         // waves
  constexpr int CPW = CHUNKS / NWV;       // per wave
  static_assert(CHUNKS % NWV == 0, "chunks per wave");
  // the two key-tile buffers are separate objects so that the compiler can
  // tell the DMA into one from the reads of the other (otherwise it drains
  // vmcnt before every LDS read, serialising DMA and compute)
  __shared__ __attribute__((aligned(16))) char kt_a[CHUNKS][1024];
  __shared__ __attribute__((aligned(16))) char kt_b[CHUNKS][1024];
  __shared__ __attribute__((aligned(16))) intx4 st_lds[NWV][16][16];  // [wave][row][16-byte chunk]
  const int lane = threadIdx.x & 63, wid = wave_id();
  const int wr = wid >> 1, wc = wid & 1;
  const int b = blockIdx.z;
  const int64_t q0 = (int64_t)blockIdx.y * MF_Q;           // first query of the workgroup
  const int64_t kt_first = (int64_t)blockIdx.x * MF_KT;     // first key tile
  int64_t n_kt = (L + MF_K - 1) / MF_K - kt_first;
  if (n_kt > MF_KT) n_kt = MF_KT;
  if (q_pos0 >= 0) {
    // key tiles beyond the last query's diagonal are not needed
    const int64_t last_q = q0 + MF_Q - 1 < Lq ? q0 + MF_Q - 1 : Lq - 1;
    const int64_t lim = (q_pos0 + last_q) / MF_K + 1 - kt_first;  // tiles that hold a key <= it
    if (lim < n_kt) n_kt = lim;
  }
  if (n_kt <= 0) return;  // uniform over the workgroup
  const int8_t* qb = q + (size_t)b * Lq * HD;
  const int8_t* kb = k + (size_t)b * L * HD;
  const int n = lane & 15, g = lane >> 4;

  // DMA of key tile t into a buffer: chunk c = (key block c / KS, k-step
  // c % KS); lane (n, g) brings key 16*block + n, bytes 64*ks + 16*g .. +15.
  // Keys past L read key L-1 (in bounds; their scores are never stored).
  auto issue_tile = [&](auto& buf, int64_t t) {
    const int64_t key0 = (kt_first + t) * MF_K;
#pragma unroll
    for (int i = 0; i < CPW; ++i) {
      const int c = wid * CPW + i;
      int64_t key = key0 + (c / KS) * 16 + n;
      if (key >= L) key = L - 1;
      __builtin_amdgcn_global_load_lds((mf_global_cvoid*)(kb + key * HD + (c % KS) * 64 + g * 16),
                                       (mf_lds_void*)&buf[c][0], 16, 0, 0);
    }
  };
  issue_tile(kt_a, 0);

  // query fragments (B operand): block qb, k-step ks: lane (n, g) holds query
  // q0 + 64 wr + 16 qb + n, bytes 64 ks + 16 g .. +15
  intx4 qf[4][KS];
#pragma unroll
  for (int qb4 = 0; qb4 < 4; ++qb4) {
    const int64_t row = q0 + wr * 64 + qb4 * 16 + n;
#pragma unroll
    for (int ks = 0; ks < KS; ++ks)
      qf[qb4][ks] = row < Lq ? *reinterpret_cast<const intx4*>(qb + row * HD + ks * 64 + g * 16)
                             : intx4{0, 0, 0, 0};
  }

  // the workgroup's score rows as one buffer (MF_Q * L * 4 < 2^31 bytes)
  const int64_t nrows = Lq - q0 < MF_Q ? Lq - q0 : MF_Q;
  const __amdgpu_buffer_rsrc_t srs =
      __builtin_amdgcn_make_buffer_rsrc(s + ((size_t)b * Lq + q0) * L, (short)0,
                                        (int)(nrows * L * 4), BUF_RSRC_WORD3);
  constexpr uint32_t DROP = 0x80000000u;  // an offset past the buffer

  auto step = [&](auto& cur, auto& nxt, int64_t t) {
    // this wave's DMA of tile t has landed once at most the score stores of
    // tile t-1 (issued after it) are outstanding; the barrier then makes
    // every wave's chunks visible and retires all reads of tile t-1
    if (t == 0 || !VEC) MF_WAIT_VM(0); else MF_WAIT_VM(16);
    // a plain barrier: __syncthreads() would also wait for the score stores
    __builtin_amdgcn_s_barrier();
    if (t + 1 < n_kt) issue_tile(nxt, t + 1);
    __asm__ __volatile__("" ::: "memory");
    intx4 acc[4][4];
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
      for (int j = 0; j < 4; ++j) acc[i][j] = intx4{0, 0, 0, 0};
#pragma unroll
    for (int kb4 = 0; kb4 < 4; ++kb4) {
#pragma unroll
      for (int ks = 0; ks < KS; ++ks) {
        const int c = (wc * 4 + kb4) * KS + ks;
        const intx4 a = *reinterpret_cast<const intx4*>(&cur[c][lane * 16]);
#pragma unroll
        for (int qb4 = 0; qb4 < 4; ++qb4)
          acc[qb4][kb4] = __builtin_amdgcn_mfma_i32_16x16x64_i8(a, qf[qb4][ks], acc[qb4][kb4], 0, 0, 0);
      }
    }
    // acc[qb][kb][e] = S[query q0 + 64wr + 16qb + n][key key0 + 16kb + 4g + e]
    const int64_t key0 = (kt_first + t) * MF_K + wc * 64;
#pragma unroll
    for (int qb4 = 0; qb4 < 4; ++qb4) {
      const int64_t rl = wr * 64 + qb4 * 16 + n;  // row within the workgroup
      const int64_t diag = q_pos0 >= 0 ? q_pos0 + q0 + rl : INT64_MAX;  // last unmasked key
      intx4 v[4];
#pragma unroll
      for (int kb4 = 0; kb4 < 4; ++kb4) {
        const int64_t col = key0 + kb4 * 16 + g * 4;
        v[kb4] = acc[qb4][kb4];
#pragma unroll
        for (int e = 0; e < 4; ++e)
          if (col + e > diag) v[kb4][e] = INT32_MIN;
      }
      if (VEC) {
        // turn the 16 x 64 slice around in LDS: chunk (row n, 4kb + g) ...
#pragma unroll
        for (int kb4 = 0; kb4 < 4; ++kb4) st_lds[wid][n][(kb4 * 4 + g) ^ n] = v[kb4];
        __asm__ __volatile__("" ::: "memory");
        // ... and read 4 rows x 16 chunks per instruction: lane -> row 4i + lane/16, chunk lane%16
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const int r = i * 4 + (lane >> 4), c = lane & 15;
          const intx4 w = st_lds[wid][r][c ^ r];
          const int64_t rr = wr * 64 + qb4 * 16 + r;
          const int64_t col = key0 + c * 4;
          const uint32_t off = (uint32_t)((rr * L + col) * 4);
          __builtin_amdgcn_raw_buffer_store_b128(w, srs, rr < nrows && col < L ? (int)off : (int)DROP, 0, 0);
        }
        __asm__ __volatile__("" ::: "memory");
      } else {
        const bool row_ok = rl < nrows;
#pragma unroll
        for (int kb4 = 0; kb4 < 4; ++kb4) {
          const int64_t col = key0 + kb4 * 16 + g * 4;
          const uint32_t off = (uint32_t)((rl * L + col) * 4);
#pragma unroll
          for (int e = 0; e < 4; ++e)
            __builtin_amdgcn_raw_buffer_store_b32(v[kb4][e], srs, row_ok && col + e < L ? (int)(off + 4 * e) : (int)DROP, 0, 0);
        }
      }
    }
  };
  for (int64_t t = 0; t < n_kt; t += 2) {
    step(kt_a, kt_b, t);
    if (t + 1 < n_kt) step(kt_b, kt_a, t + 1);
  }
}

hipError_t launch_idx_score_mfma(const int8_t* q, const int8_t* k, int32_t* s, int B, int Lq,
                                 int64_t L, int HD, int64_t q_pos0, hipStream_t st) {
  if ((int64_t)MF_Q * L * 4 >= ((int64_t)1 << 31)) return hipErrorInvalidValue;
  const int64_t kts = (L + MF_K - 1) / MF_K;
  dim3 grid((unsigned)((kts + MF_KT - 1) / MF_KT), (unsigned)((Lq + MF_Q - 1) / MF_Q), B);
  // 16-byte stores need 16-byte aligned score rows
  const bool vec = L % 4 == 0 && ((uintptr_t)s % 16) == 0;
#define LCT_MF(KS)                                                                             \
  if (vec) k_idx_score_mfma<KS, true><<<grid, 128 * MF_NWR, 0, st>>>(q, k, s, Lq, L, q_pos0);   \
  else k_idx_score_mfma<KS, false><<<grid, 128 * MF_NWR, 0, st>>>(q, k, s, Lq, L, q_pos0)
  switch (HD) {
    case 64: LCT_MF(1); break;
    case 128: LCT_MF(2); break;
    case 256: LCT_MF(4); break;
    case 512: LCT_MF(8); break;
    default: return hipErrorInvalidValue;
  }
#undef LCT_MF
  return hipGetLastError();
}

}  // namespace lct
