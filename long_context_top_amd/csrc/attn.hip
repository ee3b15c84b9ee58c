// Sparse attention over gathered K/V rows for gfx950.
//
// Source: CLSA explainer section 1.1 (softmax(QK^T / sqrt(d_k)) V) evaluated
// over the selected keys only (section 2.3, selector; tutorial DSA section);
// split decode with a log-sum-exp merge of partial results and one KV-tile
// load serving every query head of its KV group (SSA article, section 6).
//
// Work unit: one (batch, query row, KV head).  Each wave owns one unit and a
// contiguous slice of its index row, and works through it 64 selected
// positions at a time; the waves of a workgroup are independent (no
// workgroup barrier, each wave has its own LDS region):
//   * the 16-byte pieces of the gathered K rows go straight into the A
//     operand of v_mfma_f32_16x16x32_bf16 (lane = row lane%16, 8 features at
//     8*(lane/16)); the G query heads of the KV group form the B operand, so
//     S^T[token][head] comes out in C layout (4 tokens x 1 head per lane);
//   * fp32 online softmax per head (running max and sum, exp2 domain);
//   * O^T += V^T P^T on the same MFMA: P^T from the C fragments is already in
//     B-operand layout (the k order inside the MFMA is a fixed permutation of
//     32 tokens); the gathered V pieces go from global memory straight into
//     LDS (global_load_lds_dwordx4, no registers) and are read back
//     transposed with ds_read_b64_tr_b16 (4 tokens x 4 features per lane).
// A wave that owns a whole index row writes the normalised output; otherwise
// it writes an (O, m, l) partial and k_split_merge combines the slices.

#include "common.h"
#include "kernels.h"

namespace lct {

constexpr int ATT_D = 128;
constexpr int ATT_STEP = 64;             // positions per wave iteration (4 blocks of 16)
constexpr int ATT_NW = 4;                // independent waves per workgroup
constexpr int ATT_PS = ATT_D + 4;        // partial row: O[D], m, l, 2 pad (16-byte rows)
constexpr int ATT_TARGET_WAVES = 1024;   // split short index rows until this many waves
constexpr float LOG2E = 1.4426950408889634f;

typedef __attribute__((address_space(3))) short4v lds_short4v;
typedef __attribute__((address_space(3))) void lds_void;
typedef const __attribute__((address_space(1))) void global_cvoid;

// s_waitcnt vmcnt(0) (expcnt, lgkmcnt left at their maxima): the LDS DMA
// writes are counted by vmcnt and the compiler does not track them
constexpr int WAITCNT_VM0 = 0x0F70;

AttnPlan attn_plan(int B, int Lq, int Hkv, int kk) {
  AttnPlan p;
  const int64_t units = (int64_t)B * Lq * Hkv;
  const int64_t pieces = (kk + 31) / 32;  // 32-position pieces of an index row
  int64_t splits = (ATT_TARGET_WAVES + units - 1) / units;
  if (splits > MERGE_MAX_SPLITS) splits = MERGE_MAX_SPLITS;
  if (splits > pieces) splits = pieces;
  if (splits < 1) splits = 1;
  int64_t per = (kk + splits - 1) / splits;
  per = ((per + 31) / 32) * 32;
  if (per < 32) per = 32;
  p.per_split = (int)per;
  p.splits = (int)((kk + per - 1) / per);
  if (p.splits < 1) p.splits = 1;
  p.part_bytes = p.splits > 1 ? (size_t)units * p.splits * 16 * ATT_PS * sizeof(float) : 0;
  return p;
}

LCT_DEV void compiler_fence() { __asm__ __volatile__("" ::: "memory"); }

template <int G>
__global__ __launch_bounds__(ATT_NW * 64) void k_sparse_attn(
    const uint16_t* __restrict__ q, const uint16_t* __restrict__ k,
    const uint16_t* __restrict__ v, const int32_t* __restrict__ idx, float* __restrict__ out,
    int64_t units, int Lq, int Hq, int Hkv, int64_t L, int kk, float scale_log2, int splits,
    int per_split, float* __restrict__ part) {
  constexpr int D = ATT_D;
  // per wave, per (16-token block j, 32-feature slice st): the 1 KiB that one
  // LDS DMA instruction writes, lane l's 16 bytes at 16*l
  __shared__ __attribute__((aligned(16))) char vt[ATT_NW][4][4][1024];
  const int lane = threadIdx.x & 63, wid = wave_id();
  // wave order: KV head fastest, then split, then (b, r): the waves of a
  // workgroup read the same selected positions of neighbouring KV heads, so
  // their row pieces are adjacent in memory
  const int64_t gw = (int64_t)blockIdx.x * ATT_NW + wid;
  if (gw >= units * splits) return;  // the whole wave; nothing below waits on other waves
  const int kvh = (int)(gw % Hkv);
  const int64_t rest = gw / Hkv;
  const int split = (int)(rest % splits);
  const int64_t br = rest / splits;  // b * Lq + r
  const int64_t unit = br * Hkv + kvh;
  const int64_t b = br / Lq;
  const int hl = lane & 15, kg = lane >> 4;
  const int e_begin = split * per_split;
  const int e_end = min(kk, e_begin + per_split);
  const int32_t* ix = idx + br * kk;
  char(*vw)[4][1024] = vt[wid];

  // index entries of the first iteration (they gate the gathers), then q
  int pos[4];
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    const int e = e_begin + 16 * j + hl;
    pos[j] = ix[e < e_end ? e : e_end - 1];
  }
  // query fragment (B operand): lanes of head slots >= G load head G-1, zeroed
  bf16x8 qf[4];
  {
    const int hq = hl < G ? hl : G - 1;
#pragma unroll
    for (int st = 0; st < 4; ++st) {
      qf[st] = *reinterpret_cast<const bf16x8*>(q + ((br * Hq) + kvh * G + hq) * D + st * 32 + kg * 8);
      if (hl >= G) qf[st] = bf16x8{};
    }
  }
  float m = -INFINITY, lsum = 0.f;
  floatx4 o[D / 16];
#pragma unroll
  for (int dt = 0; dt < D / 16; ++dt) o[dt] = floatx4{0.f, 0.f, 0.f, 0.f};

  const size_t row_stride = (size_t)Hkv * D;  // elements between positions
  const uint16_t* kbase = k + ((size_t)b * L * Hkv + kvh) * D;
  const uint16_t* vbase = v + ((size_t)b * L * Hkv + kvh) * D;
  // transposed read of 16-feature tile dt of block j: this lane supplies
  // token 4*kg + hl/4, features 16*dt + 4*(hl%4) .. +3, which the DMA put in
  // slice dt/2, lane (4*kg + hl/4) + 16*(2*(dt%2) + (hl%4)/2), byte 8*(hl%2)
  const int tr_off = 16 * ((4 * kg + (hl >> 2)) + 16 * ((hl & 3) >> 1)) + 8 * (hl & 1);

  for (int e0 = e_begin; e0 < e_end; e0 += ATT_STEP) {
    int pp[4];
    uint64_t msk[4];
    bool any = false;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int e = e0 + 16 * j + hl;
      int p = pos[j];
      if (e >= e_end || p < 0 || (int64_t)p >= L) p = -1;  // padding / out of range: skipped
      pp[j] = p;
      msk[j] = __ballot(p >= 0);
      any = any || msk[j] != 0;
    }
    // next iteration's index entries (clamped, so always in bounds)
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int e = e0 + ATT_STEP + 16 * j + hl;
      pos[j] = ix[e < e_end ? e : e_end - 1];
    }
    if (!any) continue;  // uniform over the wave
    // gathers; masked positions read row 0 (in bounds) and are masked below.
    // K pieces into registers (MFMA A operand), V pieces into LDS by DMA.
    bf16x8 kf[4][4];
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const size_t roff = (size_t)(pp[j] >= 0 ? pp[j] : 0) * row_stride + kg * 8;
#pragma unroll
      for (int st = 0; st < 4; ++st)
        kf[j][st] = *reinterpret_cast<const bf16x8*>(kbase + roff + st * 32);
    }
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const size_t roff = (size_t)(pp[j] >= 0 ? pp[j] : 0) * row_stride + kg * 8;
#pragma unroll
      for (int st = 0; st < 4; ++st)
        __builtin_amdgcn_global_load_lds((global_cvoid*)(vbase + roff + st * 32),
                                         (lds_void*)&vw[j][st][0], 16, 0, 0);
    }
    __builtin_amdgcn_sched_barrier(0);  // every load above is issued before any MFMA
    // S^T = K Q^T per 16-token block
    floatx4 sacc[4];
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      sacc[j] = floatx4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int st = 0; st < 4; ++st)
        sacc[j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(kf[j][st], qf[st], sacc[j], 0, 0, 0);
    }
    // sacc[j][e] = S^T[token 16j + 4kg + e][head hl]
    float z[4][4];
    float tmax = -INFINITY;
#pragma unroll
    for (int j = 0; j < 4; ++j)
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        z[j][e] = ((msk[j] >> (kg * 4 + e)) & 1) ? sacc[j][e] * scale_log2 : -INFINITY;
        tmax = fmaxf(tmax, z[j][e]);
      }
    tmax = fmaxf(tmax, __shfl_xor(tmax, 16, 64));
    tmax = fmaxf(tmax, __shfl_xor(tmax, 32, 64));
    const float mnew = fmaxf(m, tmax);  // finite: the iteration has a valid position
    const float alpha = exp2f(m - mnew);
    // the weights enter the PV product as bf16; the denominator sums the same
    // rounded weights so that the normalisation is consistent
    __bf16 pw[4][4];
    float psum = 0.f;
#pragma unroll
    for (int j = 0; j < 4; ++j)
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        pw[j][e] = (__bf16)exp2f(z[j][e] - mnew);
        psum += (float)pw[j][e];
      }
    lsum = lsum * alpha + psum;
    m = mnew;
    // the V pieces have landed in LDS once vmcnt drains
    __builtin_amdgcn_s_waitcnt(WAITCNT_VM0);
    compiler_fence();
    // O^T += V^T P^T, 32 tokens (blocks 2h, 2h+1) per MFMA: the MFMA's
    // k = 8kg + jj is token 4kg + jj of block 2h (jj < 4) or 4kg + jj - 4 of
    // block 2h+1, in both operands
#pragma unroll
    for (int dt = 0; dt < D / 16; ++dt) o[dt] = o[dt] * alpha;
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      bf16x8 pf;
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        pf[e] = pw[2 * h][e];
        pf[4 + e] = pw[2 * h + 1][e];
      }
#pragma unroll
      for (int dt = 0; dt < D / 16; ++dt) {
        const short4v lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
            (lds_short4v*)&vw[2 * h][dt >> 1][512 * (dt & 1) + tr_off]);
        const short4v hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
            (lds_short4v*)&vw[2 * h + 1][dt >> 1][512 * (dt & 1) + tr_off]);
        // whole-vector reinterpretation (element-wise bf16 casts of the
        // read results are mis-assembled by the compiler)
        const bf16x8 va = __builtin_bit_cast(bf16x8, __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7));
        o[dt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(va, pf, o[dt], 0, 0, 0);
      }
    }
    compiler_fence();
  }

  // o[dt][e] = O^T[d = 16dt + 4kg + e][head hl]; lsum: this lane's share
  lsum += __shfl_xor(lsum, 16, 64);
  lsum += __shfl_xor(lsum, 32, 64);
  if (hl >= G) return;
  if (splits == 1) {
    const float inv = lsum > 0.f ? 1.f / lsum : 0.f;
    float* op = out + ((br * Hq) + kvh * G + hl) * D + kg * 4;
#pragma unroll
    for (int dt = 0; dt < D / 16; ++dt) *reinterpret_cast<floatx4*>(op + dt * 16) = o[dt] * inv;
  } else {
    float* pp = part + ((unit * splits + split) * G + hl) * ATT_PS;
#pragma unroll
    for (int dt = 0; dt < D / 16; ++dt) *reinterpret_cast<floatx4*>(pp + dt * 16 + kg * 4) = o[dt];
    if (kg == 0) *reinterpret_cast<float2*>(pp + D) = float2{m, lsum};
  }
}

// Log-sum-exp merge of split partials (SSA article section 6, third stage):
// O = sum_s e^{m_s - M} O_s / sum_s e^{m_s - M} l_s with M = max_s m_s.
// One workgroup per (unit, head), one thread per output feature; all split
// partials of a thread are loaded at once (one memory round trip).

__global__ __launch_bounds__(256) void k_split_merge(const float* __restrict__ part,
                                                     float* __restrict__ out, int splits, int hs,
                                                     int G, int D, int rs) {
  __shared__ float wts[MERGE_MAX_SPLITS];
  __shared__ float s_inv;
  const int64_t unit = blockIdx.x;
  const int h = blockIdx.y;
  const int d = threadIdx.x < D ? threadIdx.x : D - 1;
  const size_t stride = (size_t)hs * rs;
  const float* base = part + ((size_t)unit * splits * hs + h) * rs;
  // all loads are issued together: this thread's feature of every split
  // (unconditional; split indices past `splits` re-read the last split and get
  // weight 0) and, in the first wave, one split's (m, l) per lane
  float o[MERGE_MAX_SPLITS];
#pragma unroll
  for (int s = 0; s < MERGE_MAX_SPLITS; ++s) o[s] = base[(size_t)(s < splits ? s : splits - 1) * stride + d];
  if (threadIdx.x < 64) {
    const int s = threadIdx.x < splits ? threadIdx.x : splits - 1;
    const float m = base[(size_t)s * stride + D];
    const float l = base[(size_t)s * stride + D + 1];
    const float M = wave_max(m);
    const float w = (M == -INFINITY || (int)threadIdx.x >= splits) ? 0.f : exp2f(m - M);
    const float L = wave_sum(w * l);
    if (threadIdx.x < MERGE_MAX_SPLITS) wts[threadIdx.x] = w;
    if (threadIdx.x == 0) s_inv = L > 0.f ? 1.f / L : 0.f;
  }
  __syncthreads();
  float acc = 0.f;
#pragma unroll
  for (int s = 0; s < MERGE_MAX_SPLITS; ++s) acc += wts[s] * o[s];
  if (threadIdx.x < D) out[((size_t)unit * G + h) * D + d] = acc * s_inv;
}

hipError_t launch_split_merge(const float* part, float* out, int64_t units, int splits, int hs,
                              int G, int D, int rs, hipStream_t st) {
  if (splits > MERGE_MAX_SPLITS || D > 256 || rs < D + 2) return hipErrorInvalidValue;
  const int threads = D < 64 ? 64 : D;
  k_split_merge<<<dim3((unsigned)units, G), threads, 0, st>>>(part, out, splits, hs, G, D, rs);
  return hipGetLastError();
}

hipError_t launch_sparse_attn(const uint16_t* q, const uint16_t* k, const uint16_t* v,
                              const int32_t* idx, float* out, int B, int Lq, int Hq, int Hkv,
                              int64_t L, int kk, float scale, const AttnPlan& plan,
                              float* partials, hipStream_t st) {
  const int G = Hq / Hkv;
  const int64_t units = (int64_t)B * Lq * Hkv;
  const int64_t waves = units * plan.splits;
  const dim3 grid((unsigned)((waves + ATT_NW - 1) / ATT_NW));
  const float sl2 = scale * LOG2E;
#define LCT_ATT(GG)                                                                          \
  k_sparse_attn<GG><<<grid, ATT_NW * 64, 0, st>>>(q, k, v, idx, out, units, Lq, Hq, Hkv, L, kk, \
                                                  sl2, plan.splits, plan.per_split, partials)
  switch (G) {
    case 1: LCT_ATT(1); break;
    case 2: LCT_ATT(2); break;
    case 4: LCT_ATT(4); break;
    case 8: LCT_ATT(8); break;
    case 16: LCT_ATT(16); break;
    default: return hipErrorInvalidValue;
  }
#undef LCT_ATT
  hipError_t e = hipGetLastError();
  if (e != hipSuccess || plan.splits == 1) return e;
  return launch_split_merge(partials, out, units, plan.splits, G, G, ATT_D, ATT_PS, st);
}

}  // namespace lct
