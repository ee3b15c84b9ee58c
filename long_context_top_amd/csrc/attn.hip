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
// The 4 waves of a workgroup are merged in LDS; several workgroups of one
// unit write (m, l, O) partials and the last one to finish merges them.

#include "common.h"
#include "kernels.h"

namespace lct {

constexpr int ATT_D = 128;
constexpr int ATT_TOK = 32;      // positions per wave step
constexpr int ATT_WAVES = 4;
constexpr int ATT_VSTRIDE = ATT_D + 8;  // padded LDS row (bf16 elements)
constexpr float LOG2E = 1.4426950408889634f;

AttnPlan attn_plan(int B, int Lq, int Hkv, int kk) {
  AttnPlan p;
  const int64_t units = (int64_t)B * Lq * Hkv;
  const int step = ATT_TOK * ATT_WAVES;  // entries one workgroup covers per pass
  int max_splits = (kk + step - 1) / step;
  if (max_splits < 1) max_splits = 1;
  // aim for >= 2048 workgroups in flight, never more than one pass per split
  int splits = (int)((2048 + units - 1) / units);
  if (splits > max_splits) splits = max_splits;
  if (splits < 1) splits = 1;
  if (units > (int64_t)(LCT_CONTROL_COUNTERS)) splits = 1;
  p.splits = splits;
  int per = (kk + splits - 1) / splits;
  per = ((per + ATT_TOK - 1) / ATT_TOK) * ATT_TOK;
  p.per_split = per < ATT_TOK ? ATT_TOK : per;
  p.splits = (kk + p.per_split - 1) / p.per_split;
  if (p.splits < 1) p.splits = 1;
  p.counters = p.splits > 1 ? (size_t)units : 0;
  p.part_bytes = p.splits > 1 ? (size_t)units * p.splits * 16 * (ATT_D + 2) * sizeof(float) : 0;
  return p;
}

template <int G>
__global__ __launch_bounds__(256) void k_sparse_attn(
    const uint16_t* __restrict__ q, const uint16_t* __restrict__ k,
    const uint16_t* __restrict__ v, const int32_t* __restrict__ idx, float* __restrict__ out,
    int Lq, int Hq, int Hkv, int64_t L, int kk, float scale_log2, int splits, int per_split,
    uint32_t* __restrict__ counters, float* __restrict__ part) {
  constexpr int D = ATT_D;
  __shared__ __attribute__((aligned(16))) uint16_t vt[ATT_WAVES][ATT_TOK][ATT_VSTRIDE];
  __shared__ float red_m[ATT_WAVES][16];
  __shared__ float red_l[ATT_WAVES][16];
  __shared__ uint32_t s_last;
  float* red_o = reinterpret_cast<float*>(&vt[0][0][0]);  // reused after the loop: [4][16][D]
  static_assert(sizeof(vt) >= ATT_WAVES * 16 * D * sizeof(float), "LDS reuse");

  const int lane = threadIdx.x & 63, wid = threadIdx.x >> 6;
  const int split = blockIdx.x, kvh = blockIdx.z;
  const int64_t br = blockIdx.y;  // b * Lq + r
  const int64_t b = br / Lq;
  const int hl = lane & 15, kg = lane >> 4;
  const int e_begin = split * per_split;
  const int e_end = min(kk, e_begin + per_split);
  const int32_t* ix = idx + br * kk;

  bf16x8 qf[4];
#pragma unroll
  for (int st = 0; st < 4; ++st) {
    if (hl < G)
      qf[st] = *reinterpret_cast<const bf16x8*>(q + ((br * Hq) + kvh * G + hl) * D + st * 32 + kg * 8);
    else
      qf[st] = bf16x8{};
  }
  float m = -INFINITY, lsum = 0.f;
  floatx4 o[D / 16];
#pragma unroll
  for (int dt = 0; dt < D / 16; ++dt) o[dt] = floatx4{0.f, 0.f, 0.f, 0.f};

  const size_t row_stride = (size_t)Hkv * D;  // elements between positions
  const uint16_t* kbase = k + ((size_t)b * L * Hkv + kvh) * D;
  const uint16_t* vbase = v + ((size_t)b * L * Hkv + kvh) * D;
  const int n_iter = (e_end - e_begin + ATT_TOK * ATT_WAVES - 1) / (ATT_TOK * ATT_WAVES);

  for (int it = 0; it < n_iter; ++it) {
    const int e0 = e_begin + (it * ATT_WAVES + wid) * ATT_TOK;
    const int ea = e0 + hl, eb = e0 + 16 + hl;
    int pa = ea < e_end ? ix[ea] : -1;
    int pb = eb < e_end ? ix[eb] : -1;
    if ((int64_t)pa >= L) pa = -1;  // out-of-range positions are skipped, never read
    if ((int64_t)pb >= L) pb = -1;
    const uint64_t ma = __ballot(pa >= 0), mb = __ballot(pb >= 0);
    const bool any = (ma | mb) != 0;
    bf16x8 kfa[4], kfb[4];
    uintx4 vfa[4], vfb[4];
    if (any) {
      const uint16_t* ka = kbase + (size_t)(pa >= 0 ? pa : 0) * row_stride;
      const uint16_t* kb2 = kbase + (size_t)(pb >= 0 ? pb : 0) * row_stride;
      const uint16_t* va = vbase + (size_t)(pa >= 0 ? pa : 0) * row_stride;
      const uint16_t* vb = vbase + (size_t)(pb >= 0 ? pb : 0) * row_stride;
#pragma unroll
      for (int st = 0; st < 4; ++st) {
        kfa[st] = *reinterpret_cast<const bf16x8*>(ka + st * 32 + kg * 8);
        kfb[st] = *reinterpret_cast<const bf16x8*>(kb2 + st * 32 + kg * 8);
        vfa[st] = *reinterpret_cast<const uintx4*>(va + st * 32 + kg * 8);
        vfb[st] = *reinterpret_cast<const uintx4*>(vb + st * 32 + kg * 8);
      }
#pragma unroll
      for (int st = 0; st < 4; ++st) {
        *reinterpret_cast<uintx4*>(&vt[wid][hl][st * 32 + kg * 8]) = vfa[st];
        *reinterpret_cast<uintx4*>(&vt[wid][16 + hl][st * 32 + kg * 8]) = vfb[st];
      }
    }
    __syncthreads();
    if (any) {
      floatx4 sa = {0.f, 0.f, 0.f, 0.f}, sb = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int st = 0; st < 4; ++st) {
        sa = __builtin_amdgcn_mfma_f32_16x16x32_bf16(kfa[st], qf[st], sa, 0, 0, 0);
        sb = __builtin_amdgcn_mfma_f32_16x16x32_bf16(kfb[st], qf[st], sb, 0, 0, 0);
      }
      // sa[e] = S^T[token kg*4+e][head hl]; mask tokens without a position
      float za[4], zb[4];
      float tmax = -INFINITY;
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const int t = kg * 4 + e;
        za[e] = ((ma >> t) & 1) ? sa[e] * scale_log2 : -INFINITY;
        zb[e] = ((mb >> t) & 1) ? sb[e] * scale_log2 : -INFINITY;
        tmax = fmaxf(tmax, fmaxf(za[e], zb[e]));
      }
      tmax = fmaxf(tmax, __shfl_xor(tmax, 16, 64));
      tmax = fmaxf(tmax, __shfl_xor(tmax, 32, 64));
      const float mnew = fmaxf(m, tmax);  // finite: the tile has a valid token
      const float alpha = exp2f(m - mnew);
      // the weights enter the PV product as bf16; the denominator sums the
      // same rounded weights so that the normalisation is consistent
      bf16x8 pf;
      float psum = 0.f;
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        pf[e] = (__bf16)exp2f(za[e] - mnew);
        pf[4 + e] = (__bf16)exp2f(zb[e] - mnew);
        psum += (float)pf[e] + (float)pf[4 + e];
      }
      lsum = lsum * alpha + psum;
      m = mnew;
#pragma unroll
      for (int dt = 0; dt < D / 16; ++dt) {
        // A = V^T[d][k]: k = kg*8 + jj <-> token (jj<4 ? kg*4+jj : 16+kg*4+jj-4)
        bf16x8 vf;
        const int d = dt * 16 + hl;
#pragma unroll
        for (int jj = 0; jj < 4; ++jj) {
          vf[jj] = __builtin_bit_cast(__bf16, vt[wid][kg * 4 + jj][d]);
          vf[4 + jj] = __builtin_bit_cast(__bf16, vt[wid][16 + kg * 4 + jj][d]);
        }
        o[dt] = o[dt] * alpha;
        o[dt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(vf, pf, o[dt], 0, 0, 0);
      }
    }
    __syncthreads();
  }

  // ---- merge the 4 waves (per head hl; o[dt][e] is O^T[d = 16dt+4kg+e][hl]) ----
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
  // thread t: head t/16, 8 consecutive d's
  const int h = threadIdx.x >> 4;          // 0..15
  const int d0 = (threadIdx.x & 15) * 8;   // 0..120
  float M = -INFINITY;
#pragma unroll
  for (int w = 0; w < ATT_WAVES; ++w) M = fmaxf(M, red_m[w][h]);
  float Ls = 0.f, acc[8];
#pragma unroll
  for (int i = 0; i < 8; ++i) acc[i] = 0.f;
  if (M != -INFINITY) {
#pragma unroll
    for (int w = 0; w < ATT_WAVES; ++w) {
      const float sc = exp2f(red_m[w][h] - M);
      Ls += sc * red_l[w][h];
#pragma unroll
      for (int i = 0; i < 8; ++i) acc[i] += sc * red_o[(w * 16 + h) * D + d0 + i];
    }
  }
  const int64_t unit = br * Hkv + kvh;
  if (splits == 1) {
    if (h < G) {
      float* op = out + ((br * Hq) + kvh * G + h) * D + d0;
      const float inv = Ls > 0.f ? 1.f / Ls : 0.f;
      floatx4 x0 = {acc[0] * inv, acc[1] * inv, acc[2] * inv, acc[3] * inv};
      floatx4 x1 = {acc[4] * inv, acc[5] * inv, acc[6] * inv, acc[7] * inv};
      *reinterpret_cast<floatx4*>(op) = x0;
      *reinterpret_cast<floatx4*>(op + 4) = x1;
    }
    return;
  }
  // ---- split-K: write the partial, the last workgroup of the unit merges ----
  float* pp = part + ((unit * splits + split) * 16 + h) * (D + 2);
#pragma unroll
  for (int i = 0; i < 8; ++i) pp[d0 + i] = acc[i];
  if ((threadIdx.x & 15) == 0) {
    pp[D] = M;
    pp[D + 1] = Ls;
  }
  __threadfence();
  __syncthreads();
  if (threadIdx.x == 0) s_last = (atomicAdd(&counters[unit], 1u) == (uint32_t)(splits - 1));
  __syncthreads();
  if (!s_last) return;
  __threadfence();
  if (h < G) {
    float Mx = -INFINITY;
    for (int s2 = 0; s2 < splits; ++s2)
      Mx = fmaxf(Mx, part[((unit * splits + s2) * 16 + h) * (D + 2) + D]);
    float L2 = 0.f, a2[8];
#pragma unroll
    for (int i = 0; i < 8; ++i) a2[i] = 0.f;
    if (Mx != -INFINITY) {
      for (int s2 = 0; s2 < splits; ++s2) {
        const float* p2 = part + ((unit * splits + s2) * 16 + h) * (D + 2);
        const float sc = exp2f(p2[D] - Mx);
        L2 += sc * p2[D + 1];
#pragma unroll
        for (int i = 0; i < 8; ++i) a2[i] += sc * p2[d0 + i];
      }
    }
    const float inv = L2 > 0.f ? 1.f / L2 : 0.f;
    float* op = out + ((br * Hq) + kvh * G + h) * D + d0;
    floatx4 x0 = {a2[0] * inv, a2[1] * inv, a2[2] * inv, a2[3] * inv};
    floatx4 x1 = {a2[4] * inv, a2[5] * inv, a2[6] * inv, a2[7] * inv};
    *reinterpret_cast<floatx4*>(op) = x0;
    *reinterpret_cast<floatx4*>(op + 4) = x1;
  }
  if (threadIdx.x == 0) counters[unit] = 0u;  // leave the control region zeroed
}

hipError_t launch_sparse_attn(const uint16_t* q, const uint16_t* k, const uint16_t* v,
                              const int32_t* idx, float* out, int B, int Lq, int Hq, int Hkv,
                              int64_t L, int kk, float scale, const AttnPlan& plan,
                              uint32_t* counters, float* partials, hipStream_t st) {
  const int G = Hq / Hkv;
  dim3 grid(plan.splits, (unsigned)((int64_t)B * Lq), Hkv);
  const float sl2 = scale * LOG2E;
#define LCT_ATT(GG)                                                                          \
  k_sparse_attn<GG><<<grid, 256, 0, st>>>(q, k, v, idx, out, Lq, Hq, Hkv, L, kk, sl2,        \
                                          plan.splits, plan.per_split, counters, partials)
  switch (G) {
    case 1: LCT_ATT(1); break;
    case 2: LCT_ATT(2); break;
    case 4: LCT_ATT(4); break;
    case 8: LCT_ATT(8); break;
    case 16: LCT_ATT(16); break;
    default: return hipErrorInvalidValue;
  }
#undef LCT_ATT
  return hipGetLastError();
}

}  // namespace lct
