// Gist-chunk routing and selective unfolding for gfx950.
//
// Sources: SSA article (arXiv 2604.20920) section 2 (one gist after every
// chunk of 16 tokens), section 3 (the query is compared with every gist, the
// top chunks are chosen and their raw tokens unfolded next to the chosen
// chunks' gists; unchosen gists are left out), section 6 (decode reads only
// the chosen segments plus a little metadata; split-K with a log-sum-exp
// merge); GSA summary page section 2.2.
//
// k_gist_score streams the gist keys once (same lane layout as the int8
// indexer: D/8 lanes per 256-byte row, butterfly reduce-scatter so every lane
// ends with one gist's score).  k_gsa_attn is a VALU kernel: there is one
// query per (batch, head) stream, so a matrix-core tile would be 1/16 used;
// each wave unfolds one chosen chunk at a time (16 raw K/V rows = 4 KiB
// contiguous each, plus the gist's V row) with an fp32 online softmax.  The
// gist's logit reuses the routing score (q . gist_key) instead of re-reading
// the gist key.

#include "common.h"
#include "kernels.h"

namespace lct {

constexpr int GS_TILE = 1024;   // gists per workgroup
constexpr int GSA_D = 128;
constexpr int GSA_MAX_SPLITS = 32;  // slices of one (b, head) row merged by k_split_merge
constexpr float GSA_LOG2E = 1.4426950408889634f;

template <int P>
__global__ __launch_bounds__(256) void k_gist_score(const uint16_t* __restrict__ q,
                                                   const uint16_t* __restrict__ gk,
                                                   float* __restrict__ s, int64_t Nc) {
  constexpr int D = P * 8, G = 64 / P;
  const int lane = threadIdx.x & 63, wid = wave_id();
  const int64_t bh = blockIdx.y;
  const int g = lane / P, j = lane % P;
  float qv[8];
  {
    uintx4 raw = *reinterpret_cast<const uintx4*>(q + bh * D + j * 8);
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      qv[2 * e] = bf16_to_f32(raw[e] & 0xFFFFu);
      qv[2 * e + 1] = bf16_to_f32(raw[e] >> 16);
    }
  }
  const uint16_t* kb = gk + (size_t)bh * Nc * D;
  for (int rd = 0; rd < GS_TILE / 256; ++rd) {
    const int64_t base = (int64_t)blockIdx.x * GS_TILE + (int64_t)(rd * 4 + wid) * 64;
    if (base >= Nc) break;
    uintx4 kv[P];
#pragma unroll
    for (int t = 0; t < P; ++t) {
      int64_t pos = base + t * G + g;
      kv[t] = pos < Nc ? __builtin_nontemporal_load(
                             reinterpret_cast<const uintx4*>(kb + pos * D + j * 8))
                       : uintx4{0u, 0u, 0u, 0u};
    }
    float acc[P];
#pragma unroll
    for (int t = 0; t < P; ++t) {
      float a = 0.f;
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        a = fmaf(bf16_to_f32(kv[t][e] & 0xFFFFu), qv[2 * e], a);
        a = fmaf(bf16_to_f32(kv[t][e] >> 16), qv[2 * e + 1], a);
      }
      acc[t] = a;
    }
#pragma unroll
    for (int d = P / 2; d >= 1; d >>= 1) {
      const bool upper = (j & d) != 0;
#pragma unroll
      for (int t = 0; t < d; ++t) {
        float send = upper ? acc[t] : acc[t + d];
        float keep = upper ? acc[t + d] : acc[t];
        acc[t] = keep + __shfl_xor(send, d, 64);
      }
    }
    const int64_t pos = base + j * G + g;
    if (pos < Nc) s[bh * Nc + pos] = acc[0];
  }
}

hipError_t launch_gist_score(const uint16_t* q, const uint16_t* gk, float* s, int BH, int64_t Nc,
                             int D, hipStream_t st) {
  dim3 grid((unsigned)((Nc + GS_TILE - 1) / GS_TILE), BH);
  switch (D) {
    case 64: k_gist_score<8><<<grid, 256, 0, st>>>(q, gk, s, Nc); break;
    case 128: k_gist_score<16><<<grid, 256, 0, st>>>(q, gk, s, Nc); break;
    case 256: k_gist_score<32><<<grid, 256, 0, st>>>(q, gk, s, Nc); break;
    default: return hipErrorInvalidValue;
  }
  return hipGetLastError();
}

GsaPlan gsa_plan(int BH, int kc, int tail_len) {
  GsaPlan p;
  const int items = kc + (tail_len > 0 ? 1 : 0);
  int max_splits = (items + 3) / 4;
  if (max_splits < 1) max_splits = 1;
  int splits = (512 + BH - 1) / BH;
  if (splits > max_splits) splits = max_splits;
  if (splits > GSA_MAX_SPLITS) splits = GSA_MAX_SPLITS;
  if (splits < 1) splits = 1;
  p.splits = splits;
  p.part_bytes = splits > 1 ? (size_t)BH * splits * (GSA_D + 2) * sizeof(float) : 0;
  return p;
}

__global__ __launch_bounds__(256) void k_gsa_attn(
    const uint16_t* __restrict__ q, const uint16_t* __restrict__ rk,
    const uint16_t* __restrict__ rv, const uint16_t* __restrict__ gv,
    const float* __restrict__ gscores, const int32_t* __restrict__ cidx, float* __restrict__ out,
    int64_t Nc, int64_t raw_cap, int kc, int tail_len, float scale_log2, int splits,
    float* __restrict__ part) {
  constexpr int D = GSA_D;
  __shared__ float red_o[4][D];
  __shared__ float red_m[4], red_l[4];
  const int lane = threadIdx.x & 63, wid = wave_id();
  const int g = lane >> 4, j = lane & 15;
  const int64_t bh = blockIdx.y;
  const int split = blockIdx.x;
  const int items = kc + (tail_len > 0 ? 1 : 0);
  const int ips = (items + splits - 1) / splits;
  const int i_begin = split * ips, i_end = min(items, i_begin + ips);

  float qv[8];
  {
    uintx4 raw = *reinterpret_cast<const uintx4*>(q + bh * D + j * 8);
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      qv[2 * e] = bf16_to_f32(raw[e] & 0xFFFFu);
      qv[2 * e + 1] = bf16_to_f32(raw[e] >> 16);
    }
  }
  float m = -INFINITY, l = 0.f, o[8];
#pragma unroll
  for (int e = 0; e < 8; ++e) o[e] = 0.f;
  const uint16_t* rkb = rk + (size_t)bh * raw_cap * D;
  const uint16_t* rvb = rv + (size_t)bh * raw_cap * D;

  for (int it = i_begin + wid; it < i_end; it += 4) {
    const bool tail = it == kc;
    const int64_t c = tail ? Nc : (int64_t)cidx[bh * kc + it];
    if (!tail && (c < 0 || c >= Nc)) continue;
    const int ntok = tail ? tail_len : 16;
    uintx4 kr[4], vr[4];
#pragma unroll
    for (int st = 0; st < 4; ++st) {
      const int t = st * 4 + g;
      const int64_t pos = c * 16 + (t < ntok ? t : 0);
      kr[st] = *reinterpret_cast<const uintx4*>(rkb + pos * D + j * 8);
      vr[st] = *reinterpret_cast<const uintx4*>(rvb + pos * D + j * 8);
    }
    uintx4 gvr = {0u, 0u, 0u, 0u};
    float zg = -INFINITY;
    if (!tail) {
      gvr = *reinterpret_cast<const uintx4*>(gv + ((size_t)bh * Nc + c) * D + j * 8);
      zg = gscores[bh * Nc + c] * scale_log2;
    }
    float z[4];
    float tmax = zg;
#pragma unroll
    for (int st = 0; st < 4; ++st) {
      float a = 0.f;
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        a = fmaf(bf16_to_f32(kr[st][e] & 0xFFFFu), qv[2 * e], a);
        a = fmaf(bf16_to_f32(kr[st][e] >> 16), qv[2 * e + 1], a);
      }
      a += __shfl_xor(a, 8, 64);
      a += __shfl_xor(a, 4, 64);
      a += __shfl_xor(a, 2, 64);
      a += __shfl_xor(a, 1, 64);
      z[st] = (st * 4 + g) < ntok ? a * scale_log2 : -INFINITY;
      tmax = fmaxf(tmax, z[st]);
    }
    tmax = fmaxf(tmax, __shfl_xor(tmax, 16, 64));
    tmax = fmaxf(tmax, __shfl_xor(tmax, 32, 64));
    const float mnew = fmaxf(m, tmax);
    const float alpha = exp2f(m - mnew);
    float psum = 0.f;
#pragma unroll
    for (int e = 0; e < 8; ++e) o[e] *= alpha;
#pragma unroll
    for (int st = 0; st < 4; ++st) {
      const float p = exp2f(z[st] - mnew);
      psum += p;
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        o[2 * e] = fmaf(p, bf16_to_f32(vr[st][e] & 0xFFFFu), o[2 * e]);
        o[2 * e + 1] = fmaf(p, bf16_to_f32(vr[st][e] >> 16), o[2 * e + 1]);
      }
    }
    if (g == 0 && !tail) {
      const float pg = exp2f(zg - mnew);
      psum += pg;
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        o[2 * e] = fmaf(pg, bf16_to_f32(gvr[e] & 0xFFFFu), o[2 * e]);
        o[2 * e + 1] = fmaf(pg, bf16_to_f32(gvr[e] >> 16), o[2 * e + 1]);
      }
    }
    l = l * alpha + psum;
    m = mnew;
  }
  // sum the four token groups of the wave (m is uniform across the wave)
  l += __shfl_xor(l, 16, 64);
  l += __shfl_xor(l, 32, 64);
#pragma unroll
  for (int e = 0; e < 8; ++e) {
    o[e] += __shfl_xor(o[e], 16, 64);
    o[e] += __shfl_xor(o[e], 32, 64);
  }
  if (g == 0) {
#pragma unroll
    for (int e = 0; e < 8; ++e) red_o[wid][j * 8 + e] = o[e];
  }
  if (lane == 0) {
    red_m[wid] = m;
    red_l[wid] = l;
  }
  __syncthreads();
  const int d = threadIdx.x;  // threads d < D own one output feature each
  float M = fmaxf(fmaxf(red_m[0], red_m[1]), fmaxf(red_m[2], red_m[3]));
  float Ls = 0.f, acc = 0.f;
  if (d < D && M != -INFINITY) {
#pragma unroll
    for (int w = 0; w < 4; ++w) {
      const float sc = exp2f(red_m[w] - M);
      Ls += sc * red_l[w];
      acc += sc * red_o[w][d];
    }
  }
  if (splits == 1) {
    if (d < D) out[bh * D + d] = Ls > 0.f ? acc / Ls : 0.f;
    return;
  }
  float* pp = part + ((size_t)bh * splits + split) * (D + 2);
  if (d < D) pp[d] = acc;
  if (d == 0) {
    pp[D] = M;
    pp[D + 1] = Ls;
  }
}

hipError_t launch_gsa_attn(const uint16_t* q, const uint16_t* rk, const uint16_t* rv,
                           const uint16_t* gv, const float* gscores, const int32_t* cidx,
                           float* out, int BH, int64_t Nc, int64_t raw_cap, int kc, int tail_len,
                           float scale, const GsaPlan& plan, float* partials, hipStream_t st) {
  dim3 grid(plan.splits, BH);
  k_gsa_attn<<<grid, 256, 0, st>>>(q, rk, rv, gv, gscores, cidx, out, Nc, raw_cap, kc, tail_len,
                                   scale * GSA_LOG2E, plan.splits, partials);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess || plan.splits == 1) return e;
  return launch_split_merge(partials, out, BH, plan.splits, 1, 1, GSA_D, GSA_D + 2, st);
}

}  // namespace lct
