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
//
// Hierarchical routing (SSA article section 5, H-SSA; GSA summary page
// section 2.4): k_hgsa_route, one workgroup per (batch, head), scores the
// meta-gists, keeps the best km groups, scores only the gists of those
// groups and keeps the best kc chunks; it reads (Nm + km*group) key rows
// instead of Nc, so the routing cost no longer grows with the whole context.

#include "common.h"
#include "kernels.h"

namespace lct {

constexpr int GS_TILE = 512;    // gists per workgroup (1024: 93-95 us, 2048: 106 us at 8192 x 256 rows)
constexpr int GSA_D = 128;
constexpr int GSA_MAX_SPLITS = 32;  // slices of one (b, head) row merged by k_split_merge
constexpr float GSA_LOG2E = 1.4426950408889634f;
constexpr int HG_RANK_MAX = 1024;  // items ranked by counting (else a bitonic sort)

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

// ------------------------------------------------------ hierarchical ----

// Dot products of n bf16 key rows (D = 128, 256 bytes each) with the query:
// 16 lanes per row, 16 bytes per lane (a wave reads 4 rows = 1 KiB
// contiguous pieces per instruction), partial sums reduced over the 16 lanes;
// the workgroup's 4 waves take rows 4w .. 4w+3, then every 16th, eight rows
// per lane loaded at once.  row_of(i) names the key row of item i (i < n);
// sink(i, score) is called by one lane per item.
template <class RowOf, class Sink>
LCT_DEV void hg_score_rows(const uint16_t* base, int n, const float (&qv)[8], RowOf row_of, Sink sink) {
  constexpr int BATCH = 8;  // rows per lane loaded before any is used (one memory round trip)
  const int lane = threadIdx.x & 63, wid = wave_id();
  const int sub = lane & 15, r4 = lane >> 4;
  for (int i0 = wid * 4; i0 < n; i0 += BATCH * (HG_NT / 16)) {
    uint4 raw[BATCH];
#pragma unroll
    for (int b = 0; b < BATCH; ++b) {
      const int i = i0 + b * (HG_NT / 16) + r4;
      raw[b] = *reinterpret_cast<const uint4*>(base + (size_t)row_of(i < n ? i : n - 1) * GSA_D + sub * 8);
    }
#pragma unroll
    for (int b = 0; b < BATCH; ++b) {
      const int i = i0 + b * (HG_NT / 16) + r4;
      const uint32_t w[4] = {raw[b].x, raw[b].y, raw[b].z, raw[b].w};
      float part = 0.f;
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        part = fmaf(bf16_to_f32(w[j] & 0xFFFFu), qv[2 * j], part);
        part = fmaf(bf16_to_f32(w[j] >> 16), qv[2 * j + 1], part);
      }
      part += __shfl_xor(part, 8, 16);
      part += __shfl_xor(part, 4, 16);
      part += __shfl_xor(part, 2, 16);
      part += __shfl_xor(part, 1, 16);
      if (sub == 0 && i < n) sink(i, part);
    }
  }
}

// Selection key: order-preserving score above, the inverted item id below,
// so a descending sort puts the higher score first and, among equal scores,
// the lower id; never 0 (that marks padding).
LCT_DEV uint64_t hg_key(float s, uint32_t id) { return ((uint64_t)key_of_f32(s) << 32) | (0xFFFFFFFFu - id); }
LCT_DEV uint32_t hg_id(uint64_t key) { return 0xFFFFFFFFu - (uint32_t)key; }

LCT_DEV int hg_pow2(int n) {
  int p = 1;
  while (p < n) p <<= 1;
  return p;
}

// Of the n items in keys[] (0 = not an item), the k with the largest keys,
// listed by item index ascending into sel[] (min(k, items) entries); returns
// how many.  Items' keys are distinct.  Up to HG_RANK_MAX items each thread
// ranks its items by counting (two short loops over LDS); beyond that a
// bitonic sort (keys[] padded to a power of two) and a rank among the first k.
LCT_DEV int hg_select(uint64_t* keys, uint8_t* flag, int n, int k, int32_t* sel) {
  __shared__ int s_cnt;
  if (threadIdx.x == 0) s_cnt = 0;
  if (n <= HG_RANK_MAX) {
    for (int i = threadIdx.x; i < n; i += HG_NT) {
      const uint64_t ki = keys[i];
      int r = 0;
      for (int j = 0; j < n; ++j) r += keys[j] > ki ? 1 : 0;
      flag[i] = (ki != 0 && r < k) ? 1 : 0;
    }
    __syncthreads();
    for (int i = threadIdx.x; i < n; i += HG_NT) {
      if (!flag[i]) continue;
      int pos = 0;
      for (int j = 0; j < i; ++j) pos += flag[j];
      sel[pos] = i;
      atomicAdd(&s_cnt, 1);
    }
  } else {
    const int n2 = hg_pow2(n);
    for (int i = n + threadIdx.x; i < n2; i += HG_NT) keys[i] = 0;
    // the sort orders keys, so the item index travels in the key's low bits
    __syncthreads();
    bitonic_sort_desc<HG_NT>(keys, n2);
    for (int t = threadIdx.x; t < k; t += HG_NT) {
      if (keys[t] == 0) continue;
      const uint32_t it = hg_id(keys[t]);
      int r = 0;
      for (int u = 0; u < k; ++u) r += (keys[u] != 0 && hg_id(keys[u]) < it) ? 1 : 0;
      sel[r] = (int32_t)it;
      atomicAdd(&s_cnt, 1);
    }
  }
  __syncthreads();
  return s_cnt;
}

__global__ __launch_bounds__(HG_NT) void k_hgsa_route(
    const uint16_t* __restrict__ q, const uint16_t* __restrict__ mk, const uint16_t* __restrict__ gk,
    float* __restrict__ gscores, int32_t* __restrict__ cidx, int64_t Nc, int Nm, int group, int km,
    int kc) {
  __shared__ uint64_t keys[HG_MAX_ITEMS];
  __shared__ uint8_t flag[HG_MAX_ITEMS];
  __shared__ int32_t gsel[HG_MAX_KM];
  __shared__ int32_t csel[HG_MAX_KC];
  const int64_t bh = blockIdx.x;
  const int sub = threadIdx.x & 15;
  float qv[8];
  {
    const uint4 raw = *reinterpret_cast<const uint4*>(q + bh * GSA_D + sub * 8);
    const uint32_t w[4] = {raw.x, raw.y, raw.z, raw.w};
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      qv[2 * j] = bf16_to_f32(w[j] & 0xFFFFu);
      qv[2 * j + 1] = bf16_to_f32(w[j] >> 16);
    }
  }
  // 1. the km best meta-gists (groups), ascending
  for (int i = threadIdx.x; i < Nm; i += HG_NT) keys[i] = 0;
  __syncthreads();
  hg_score_rows(mk + (size_t)bh * Nm * GSA_D, Nm, qv, [](int i) { return i; },
                [&](int i, float s) { keys[i] = hg_key(s, (uint32_t)i); });
  __syncthreads();
  hg_select(keys, flag, Nm, km, gsel);
  // 2. the kc best chunks among the chosen groups' gists; candidate p is
  // chunk gsel[p / group] * group + p % group (ascending in p; past Nc in a
  // short last group: no item)
  const int nc_items = km * group;
  for (int i = threadIdx.x; i < nc_items; i += HG_NT) keys[i] = 0;
  __syncthreads();
  auto chunk_of = [&](int p) -> int64_t { return (int64_t)gsel[p / group] * group + p % group; };
  hg_score_rows(gk + (size_t)bh * Nc * GSA_D, nc_items, qv,
                [&](int p) { const int64_t c = chunk_of(p); return c < Nc ? c : Nc - 1; },
                [&](int p, float s) {
                  const int64_t c = chunk_of(p);
                  if (c < Nc) {
                    keys[p] = hg_key(s, (uint32_t)p);  // ties: lower p = lower chunk
                    gscores[bh * Nc + c] = s;          // the gist logit of the attention
                  }
                });
  __syncthreads();
  const int nch = hg_select(keys, flag, nc_items, kc, csel);
  for (int t = threadIdx.x; t < kc; t += HG_NT)
    cidx[bh * kc + t] = t < nch ? (int32_t)chunk_of(csel[t]) : -1;
}

hipError_t launch_hgsa_route(const uint16_t* q, const uint16_t* mk, const uint16_t* gk, float* gscores,
                             int32_t* cidx, int BH, int64_t Nc, int Nm, int group, int km, int kc,
                             hipStream_t st) {
  if (Nm > HG_MAX_ITEMS || km > HG_MAX_KM || km > Nm || (int64_t)km * group > HG_MAX_ITEMS || kc > HG_MAX_KC)
    return hipErrorInvalidValue;
  k_hgsa_route<<<dim3((unsigned)BH), HG_NT, 0, st>>>(q, mk, gk, gscores, cidx, Nc, Nm, group, km, kc);
  return hipGetLastError();
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
