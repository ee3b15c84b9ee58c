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
// 128x128 output tile per workgroup, four waves of 64x64, each a 4x4 grid of
// 16x16 int8 MFMA blocks.  Operands are read straight from global memory in
// the MFMA lane layout (lane: row lane%16, 16 contiguous bytes at
// k = 16*(lane/16)); the 128-row panels are shared through L2.
constexpr int MF_TILE = 128;

__global__ __launch_bounds__(256) void k_idx_score_mfma(const int8_t* __restrict__ q,
                                                        const int8_t* __restrict__ k,
                                                        int32_t* __restrict__ s, int Lq,
                                                        int64_t L, int HD, int64_t q_pos0) {
  const int lane = threadIdx.x & 63, wid = wave_id();
  const int b = blockIdx.z;
  const int64_t row0 = (int64_t)blockIdx.y * MF_TILE + (wid >> 1) * 64;
  const int64_t col0 = (int64_t)blockIdx.x * MF_TILE + (wid & 1) * 64;
  if (q_pos0 >= 0) {
    // whole workgroup tile above the diagonal: nothing to compute
    const int64_t last_row_pos = q_pos0 + (int64_t)blockIdx.y * MF_TILE + MF_TILE - 1;
    if ((int64_t)blockIdx.x * MF_TILE > last_row_pos) return;
  }
  const int8_t* qb = q + (size_t)b * Lq * HD;
  const int8_t* kb = k + (size_t)b * L * HD;
  const int rl = lane & 15, kq = lane >> 4;
  intx4 acc[4][4];
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int c = 0; c < 4; ++c) acc[i][c] = intx4{0, 0, 0, 0};
  for (int kk = 0; kk < HD; kk += 64) {
    intx4 a[4], bb[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      int64_t r = row0 + i * 16 + rl;
      a[i] = r < Lq ? *reinterpret_cast<const intx4*>(qb + r * HD + kk + kq * 16)
                    : intx4{0, 0, 0, 0};
      int64_t c = col0 + i * 16 + rl;
      bb[i] = c < L ? *reinterpret_cast<const intx4*>(kb + c * HD + kk + kq * 16)
                    : intx4{0, 0, 0, 0};
    }
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
      for (int c = 0; c < 4; ++c)
        acc[i][c] = __builtin_amdgcn_mfma_i32_16x16x64_i8(a[i], bb[c], acc[i][c], 0, 0, 0);
  }
  // C layout: lane holds rows 4*(lane/16)+e, column lane%16 of each block
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int c = 0; c < 4; ++c)
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        int64_t r = row0 + i * 16 + kq * 4 + e;
        int64_t col = col0 + c * 16 + rl;
        if (r < Lq && col < L) {
          int32_t v = acc[i][c][e];
          if (q_pos0 >= 0 && col > q_pos0 + r) v = INT32_MIN;
          s[((size_t)b * Lq + r) * L + col] = v;
        }
      }
}

hipError_t launch_idx_score_mfma(const int8_t* q, const int8_t* k, int32_t* s, int B, int Lq,
                                 int64_t L, int HD, int64_t q_pos0, hipStream_t st) {
  dim3 grid((unsigned)((L + MF_TILE - 1) / MF_TILE), (unsigned)((Lq + MF_TILE - 1) / MF_TILE), B);
  k_idx_score_mfma<<<grid, 256, 0, st>>>(q, k, s, Lq, L, HD, q_pos0);
  return hipGetLastError();
}

}  // namespace lct
