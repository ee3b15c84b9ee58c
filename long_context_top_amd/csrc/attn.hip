// Sparse attention over gathered K/V rows for gfx950.
//
// Source: CLSA explainer section 1.1 (softmax(QK^T / sqrt(d_k)) V) evaluated
// over the selected keys only (section 2.3, selector; tutorial DSA section);
// split decode with a log-sum-exp merge of partial results and one KV-tile
// load serving every query head of its KV group (SSA article, section 6).
//
// Work unit: one (batch, query row, KV head) and a contiguous slice of its
// index row.  Each wave takes 32 selected positions at a time:
//   * the 16-byte pieces of the 32 gathered K rows go straight into the A
//     operand of v_mfma_f32_16x16x32_bf16 (lane = row lane%16, 8 features at
//     8*(lane/16)); the G query heads of the KV group form the B operand, so
//     S^T[token][head] comes out in C layout (4 tokens x 1 head per lane);
//   * fp32 online softmax per head (running max and sum, exp2 domain);
//   * O^T += V^T P^T on the same MFMA: P^T from the C fragments is already in
//     B-operand layout (the k order inside the MFMA is a fixed permutation of
//     the 32 tokens), V is staged through LDS and read transposed.
// The 4 waves of a workgroup are merged in LDS; when several workgroups share
// a unit they write (O, m, l) partials and k_split_merge combines them.

#include "common.h"
#include "kernels.h"

namespace lct {

constexpr int ATT_D = 128;
constexpr int ATT_TOK = 32;      // positions per wave step
constexpr int ATT_VSTRIDE = ATT_D + 8;  // padded LDS row (bf16 elements)
constexpr float LOG2E = 1.4426950408889634f;

AttnPlan attn_plan(int B, int Lq, int Hkv, int kk) {
  AttnPlan p;
  const int64_t units = (int64_t)B * Lq * Hkv;
  // One pass per workgroup: each wave takes one 32-position step, so a
  // workgroup covers 32*NW positions of its unit.  4-wave workgroups when
  // that already gives >= 256 workgroups, else narrower ones (more splits,
  // at most MERGE_MAX_SPLITS); very long index rows take several passes.
  const int tok = ATT_TOK;
  auto nsplit = [&](int w) { return (kk + (int64_t)w * tok - 1) / ((int64_t)w * tok); };
  int nw = 4;
  int64_t splits = 1;
  if (units < 1024) {  // few units: split their index rows across workgroups
    while (nw > 1 && units * nsplit(nw) < 256 && nsplit(nw / 2) <= MERGE_MAX_SPLITS) nw /= 2;
    splits = nsplit(nw);
    if (splits > MERGE_MAX_SPLITS) splits = MERGE_MAX_SPLITS;
  }
  int64_t per = (kk + splits - 1) / splits;
  per = ((per + tok - 1) / tok) * tok;
  p.tok = tok;
  p.waves = nw;
  p.per_split = (int)per;
  p.splits = (int)((kk + per - 1) / per);
  if (p.splits < 1) p.splits = 1;
  p.part_bytes = p.splits > 1 ? (size_t)units * p.splits * 16 * (ATT_D + 2) * sizeof(float) : 0;
  return p;
}

template <int G, int NW, int TOK>
__global__ __launch_bounds__(NW * 64) void k_sparse_attn(
    const uint16_t* __restrict__ q, const uint16_t* __restrict__ k,
    const uint16_t* __restrict__ v, const int32_t* __restrict__ idx, float* __restrict__ out,
    int Lq, int Hq, int Hkv, int64_t L, int kk, float scale_log2, int splits, int per_split,
    float* __restrict__ part) {
  static_assert(TOK == 16 || TOK == 32, "16 or 32 positions per wave step");
  constexpr int D = ATT_D;
  constexpr int NB = TOK / 16;  // 16-position blocks per step
  __shared__ __attribute__((aligned(16))) uint16_t vt[NW][ATT_TOK][ATT_VSTRIDE];
  __shared__ float red_m[NW][16];
  __shared__ float red_l[NW][16];
  float* red_o = reinterpret_cast<float*>(&vt[0][0][0]);  // reused after the loop: [NW][16][D]
  static_assert(sizeof(vt) >= NW * 16 * D * sizeof(float), "LDS reuse");

  const int lane = threadIdx.x & 63, wid = threadIdx.x >> 6;
  const int split = blockIdx.x, kvh = blockIdx.z;
  const int64_t br = blockIdx.y;  // b * Lq + r
  const int64_t b = br / Lq;
  const int hl = lane & 15, kg = lane >> 4;
  const int e_begin = split * per_split;
  const int e_end = min(kk, e_begin + per_split);
  const int32_t* ix = idx + br * kk;

  // index rows of the first step (issued first: they gate the gather)
  int pre[NB];
#pragma unroll
  for (int j = 0; j < NB; ++j) {
    const int e = e_begin + wid * TOK + 16 * j + hl;
    pre[j] = ix[e < e_end ? e : e_end - 1];
  }
  // query fragment: lanes of head slots >= G load head G-1 and are zeroed
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
  const int n_iter = (e_end - e_begin + TOK * NW - 1) / (TOK * NW);

  for (int it = 0; it < n_iter; ++it) {
    const int e0 = e_begin + (it * NW + wid) * TOK;
    int pos[NB];
    uint64_t msk[NB];
    bool any = false;
#pragma unroll
    for (int j = 0; j < NB; ++j) {
      const int e = e0 + 16 * j + hl;
      int p = it == 0 ? pre[j] : ix[e < e_end ? e : e_end - 1];
      if (e >= e_end || (int64_t)p >= L) p = -1;  // padding and out-of-range positions are skipped
      pos[j] = p;
      msk[j] = __ballot(p >= 0);
      any = any || msk[j] != 0;
    }
    bf16x8 kf[NB][4];
    uintx4 vf[NB][4];
    if (any) {
      // masked positions read row 0 (in bounds); their logits are masked below
#pragma unroll
      for (int j = 0; j < NB; ++j) {
        const size_t roff = (size_t)(pos[j] >= 0 ? pos[j] : 0) * row_stride + kg * 8;
#pragma unroll
        for (int st = 0; st < 4; ++st) {
          kf[j][st] = *reinterpret_cast<const bf16x8*>(kbase + roff + st * 32);
          vf[j][st] = *reinterpret_cast<const uintx4*>(vbase + roff + st * 32);
        }
      }
#pragma unroll
      for (int j = 0; j < NB; ++j)
#pragma unroll
        for (int st = 0; st < 4; ++st)
          *reinterpret_cast<uintx4*>(&vt[wid][16 * j + hl][st * 32 + kg * 8]) = vf[j][st];
    }
    __syncthreads();
    if (any) {
      floatx4 sacc[NB];
#pragma unroll
      for (int j = 0; j < NB; ++j) {
        sacc[j] = floatx4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int st = 0; st < 4; ++st)
          sacc[j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(kf[j][st], qf[st], sacc[j], 0, 0, 0);
      }
      // sacc[j][e] = S^T[token 16j + 4kg + e][head hl]; mask positions without a row
      float z[NB][4];
      float tmax = -INFINITY;
#pragma unroll
      for (int j = 0; j < NB; ++j)
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          z[j][e] = ((msk[j] >> (kg * 4 + e)) & 1) ? sacc[j][e] * scale_log2 : -INFINITY;
          tmax = fmaxf(tmax, z[j][e]);
        }
      tmax = fmaxf(tmax, __shfl_xor(tmax, 16, 64));
      tmax = fmaxf(tmax, __shfl_xor(tmax, 32, 64));
      const float mnew = fmaxf(m, tmax);  // finite: the step has a valid position
      const float alpha = exp2f(m - mnew);
      // the weights enter the PV product as bf16; the denominator sums the
      // same rounded weights so that the normalisation is consistent
      __bf16 pw[NB][4];
      float psum = 0.f;
#pragma unroll
      for (int j = 0; j < NB; ++j)
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          pw[j][e] = (__bf16)exp2f(z[j][e] - mnew);
          psum += (float)pw[j][e];
        }
      lsum = lsum * alpha + psum;
      m = mnew;
      if constexpr (TOK == 32) {
        // O^T += V^T P^T on 16x16x32: the MFMA's k = 8kg + jj stands for
        // position (jj < 4 ? 4kg + jj : 16 + 4kg + jj - 4) in both operands
        bf16x8 pf;
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          pf[e] = pw[0][e];
          pf[4 + e] = pw[NB - 1][e];
        }
#pragma unroll
        for (int dt = 0; dt < D / 16; ++dt) {
          bf16x8 va;
          const int d = dt * 16 + hl;
#pragma unroll
          for (int jj = 0; jj < 4; ++jj) {
            va[jj] = __builtin_bit_cast(__bf16, vt[wid][kg * 4 + jj][d]);
            va[4 + jj] = __builtin_bit_cast(__bf16, vt[wid][16 + kg * 4 + jj][d]);
          }
          o[dt] = o[dt] * alpha;
          o[dt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(va, pf, o[dt], 0, 0, 0);
        }
      } else {
        // O^T += V^T P^T on 16x16x16: P^T is the C fragment of S^T as it stands
        short4v pf;
#pragma unroll
        for (int e = 0; e < 4; ++e) pf[e] = __builtin_bit_cast(short, pw[0][e]);
#pragma unroll
        for (int dt = 0; dt < D / 16; ++dt) {
          short4v va;
          const int d = dt * 16 + hl;
#pragma unroll
          for (int jj = 0; jj < 4; ++jj) va[jj] = (short)vt[wid][kg * 4 + jj][d];
          o[dt] = o[dt] * alpha;
          o[dt] = __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(va, pf, o[dt], 0, 0, 0);
        }
      }
    }
    __syncthreads();
  }

  // ---- merge the NW waves (per head hl; o[dt][e] is O^T[d = 16dt+4kg+e][hl]) ----
  lsum += __shfl_xor(lsum, 16, 64);
  lsum += __shfl_xor(lsum, 32, 64);
  if (kg == 0) {
    red_m[wid][hl] = m;
    red_l[wid][hl] = lsum;
  }
#pragma unroll
  for (int dt = 0; dt < D / 16; ++dt)
#pragma unroll
    for (int e = 0; e < 4; ++e) red_o[(wid * 16 + hl) * D + dt * 16 + kg * 4 + e] = o[dt][e];
  __syncthreads();
  // slot t (of 256): head t/16, 8 consecutive d's; each thread takes 256/(NW*64) slots
  float M[256 / (NW * 64)], Ls[256 / (NW * 64)], acc[256 / (NW * 64)][8];
#pragma unroll
  for (int si = 0; si < 256 / (NW * 64); ++si) {
    const int slot = si * NW * 64 + threadIdx.x;
    const int h = slot >> 4, d0 = (slot & 15) * 8;
    M[si] = -INFINITY;
#pragma unroll
    for (int w = 0; w < NW; ++w) M[si] = fmaxf(M[si], red_m[w][h]);
    Ls[si] = 0.f;
#pragma unroll
    for (int i = 0; i < 8; ++i) acc[si][i] = 0.f;
    if (M[si] != -INFINITY) {
#pragma unroll
      for (int w = 0; w < NW; ++w) {
        const float sc = exp2f(red_m[w][h] - M[si]);
        Ls[si] += sc * red_l[w][h];
#pragma unroll
        for (int i = 0; i < 8; ++i) acc[si][i] += sc * red_o[(w * 16 + h) * D + d0 + i];
      }
    }
  }
  const int64_t unit = br * Hkv + kvh;
#pragma unroll
  for (int si = 0; si < 256 / (NW * 64); ++si) {
    const int slot = si * NW * 64 + threadIdx.x;
    const int h = slot >> 4, d0 = (slot & 15) * 8;
    if (splits == 1) {
      if (h < G) {
        float* op = out + ((br * Hq) + kvh * G + h) * D + d0;
        const float inv = Ls[si] > 0.f ? 1.f / Ls[si] : 0.f;
        *reinterpret_cast<floatx4*>(op) =
            floatx4{acc[si][0] * inv, acc[si][1] * inv, acc[si][2] * inv, acc[si][3] * inv};
        *reinterpret_cast<floatx4*>(op + 4) =
            floatx4{acc[si][4] * inv, acc[si][5] * inv, acc[si][6] * inv, acc[si][7] * inv};
      }
    } else if (h < G) {
      // split-K: write the partial; the merge kernel combines the splits
      float* pp = part + ((unit * splits + split) * 16 + h) * (D + 2);
      *reinterpret_cast<floatx4*>(pp + d0) = floatx4{acc[si][0], acc[si][1], acc[si][2], acc[si][3]};
      *reinterpret_cast<floatx4*>(pp + d0 + 4) = floatx4{acc[si][4], acc[si][5], acc[si][6], acc[si][7]};
      if ((slot & 15) == 0) {
        pp[D] = M[si];
        pp[D + 1] = Ls[si];
      }
    }
  }
}

// Log-sum-exp merge of split partials (SSA article section 6, third stage):
// O = sum_s e^{m_s - M} O_s / sum_s e^{m_s - M} l_s with M = max_s m_s.
// One workgroup per (unit, head), one thread per output feature; all split
// partials of a thread are loaded at once (one memory round trip).

__global__ __launch_bounds__(256) void k_split_merge(const float* __restrict__ part,
                                                     float* __restrict__ out, int splits, int hs,
                                                     int G, int D) {
  __shared__ float wts[MERGE_MAX_SPLITS];
  __shared__ float s_inv;
  const int64_t unit = blockIdx.x;
  const int h = blockIdx.y;
  const int d = threadIdx.x < D ? threadIdx.x : D - 1;
  const size_t stride = (size_t)hs * (D + 2);
  const float* base = part + ((size_t)unit * splits * hs + h) * (D + 2);
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
                              int G, int D, hipStream_t st) {
  if (splits > MERGE_MAX_SPLITS || D > 256) return hipErrorInvalidValue;
  const int threads = D < 64 ? 64 : D;
  k_split_merge<<<dim3((unsigned)units, G), threads, 0, st>>>(part, out, splits, hs, G, D);
  return hipGetLastError();
}

hipError_t launch_sparse_attn(const uint16_t* q, const uint16_t* k, const uint16_t* v,
                              const int32_t* idx, float* out, int B, int Lq, int Hq, int Hkv,
                              int64_t L, int kk, float scale, const AttnPlan& plan,
                              float* partials, hipStream_t st) {
  const int G = Hq / Hkv;
  dim3 grid(plan.splits, (unsigned)((int64_t)B * Lq), Hkv);
  const float sl2 = scale * LOG2E;
#define LCT_ATT(GG, NWW, TT)                                                               \
  k_sparse_attn<GG, NWW, TT><<<grid, NWW * 64, 0, st>>>(q, k, v, idx, out, Lq, Hq, Hkv, L, kk, \
                                                        sl2, plan.splits, plan.per_split,       \
                                                        partials)
#define LCT_ATT_T(GG, NWW)                  \
  if (plan.tok == 32) {                     \
    LCT_ATT(GG, NWW, 32);                   \
  } else {                                  \
    LCT_ATT(GG, NWW, 16);                   \
  }
#define LCT_ATT_G(GG)                       \
  switch (plan.waves) {                     \
    case 1: LCT_ATT_T(GG, 1); break;        \
    case 2: LCT_ATT_T(GG, 2); break;        \
    default: LCT_ATT_T(GG, 4); break;       \
  }
  switch (G) {
    case 1: LCT_ATT_G(1); break;
    case 2: LCT_ATT_G(2); break;
    case 4: LCT_ATT_G(4); break;
    case 8: LCT_ATT_G(8); break;
    case 16: LCT_ATT_G(16); break;
    default: return hipErrorInvalidValue;
  }
#undef LCT_ATT_G
#undef LCT_ATT_T
#undef LCT_ATT
  hipError_t e = hipGetLastError();
  if (e != hipSuccess || plan.splits == 1) return e;
  return launch_split_merge(partials, out, (int64_t)B * Lq * Hkv, plan.splits, 16, G, ATT_D, st);
}

}  // namespace lct
