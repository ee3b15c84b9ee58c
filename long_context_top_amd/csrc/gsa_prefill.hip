// GSA prefill attention under the gist mask for gfx950.
//
// Sources: SSA article section 4 (the gist mask: a segment's raw tokens see
// one another and every earlier segment's gist tokens, never the raw tokens
// of earlier segments), section 6 (prefill kernel: the global key columns
// are moved in front, which leaves softmax unchanged, so the pattern becomes
// a dense thin block -- the gists -- plus a diagonal band -- the segment's
// own raw tokens).
//
// The keys arrive already in that order: the gist keys and values are their
// own arrays ([BH, Nc, D]) and so are the raw ones ([BH, raw_cap, D]).  A
// raw query of chunk c attends to gists [0, c) (a prefix of the gist array,
// no mask) and to its own chunk's raw tokens up to itself; a gist query of
// chunk c to gists [0, c] and its chunk's 16 raw tokens.
//
// Work: one workgroup of 4 waves per 128 queries (raw: 8 chunks, two per
// wave; gist: 128 gists, 32 per wave); each wave holds GP_QG = 2 groups of
// 16 queries as the columns of v_mfma_f32_16x16x32_bf16 (S^T = K Q^T,
// O^T += V^T P^T, as in the sparse attention kernel), every K or V fragment
// it reads from LDS feeding one MFMA per group.  The workgroup walks its key
// tiles of 64 rows (the gist prefix, then the band) through two LDS buffers
// filled by buffer loads to LDS, so each key row is read once per workgroup
// and serves its 4 waves; rows are stored with their 16-byte chunks
// XOR-swizzled by row so that the A-operand reads (K tiles) and the
// transposed reads (V tiles) hit distinct banks.  Raw queries and outputs are
// [BH, Nc*16, D], gist ones [BH, Nc, D].  Tiles a query group cannot see are
// skipped by it, tiles it sees whole take an unmasked softmax, the others
// mask one interval of rows per query.  The running softmax reference moves
// only when a tile's maximum exceeds it by 2^8, so the output is rarely
// rescaled.  One launch holds both kinds: the gist workgroups first, then the
// raw ones, each kind heaviest first over all heads (the gist prefix grows
// with the chunk index), so the light raw workgroups fill the tail.

#include "common.h"
#include "kernels.h"

namespace lct {

constexpr int GP_D = 128;
constexpr int GP_CHUNK = 16;
constexpr int GP_TILE = 64;                  // key rows per tile
constexpr int GP_NW = 4;                     // waves per workgroup
constexpr int GP_QG = 2;                     // query groups of 16 per wave: every K/V fragment
                                             // read from LDS feeds two MFMAs (two waves per
                                             // SIMD; one group measured 6.8 against 6.0 ms)
constexpr int GP_ROWB = GP_D * 2;            // bytes per key row
constexpr int GP_TILEB = GP_TILE * GP_ROWB;  // 16 KiB
constexpr float GP_LOG2E = 1.4426950408889634f;
constexpr float GP_SLACK = 8.f;              // log2 headroom of the softmax reference

typedef __attribute__((address_space(3))) short4v gp_lds_short4v;
typedef __attribute__((address_space(3))) void gp_lds_void;

// s_waitcnt vmcnt(0), lgkmcnt(0) (expcnt left at its maximum)
#define GP_WAIT_VM0() __builtin_amdgcn_s_waitcnt(0x0F70)
#define GP_WAIT_LGKM0() __builtin_amdgcn_s_waitcnt(0xC07F)

LCT_DEV void gp_fence() { __asm__ __volatile__("" ::: "memory"); }

typedef __bf16 gp_bf16x2 __attribute__((ext_vector_type(2)));
typedef float gp_floatx2 __attribute__((ext_vector_type(2)));

// Two weights rounded to bf16 and packed (one v_cvt_pk_bf16_f32).
LCT_DEV uint32_t gp_pack(float a, float b) {
  return __builtin_bit_cast(uint32_t, __builtin_convertvector((gp_floatx2){a, b}, gp_bf16x2));
}

// Maximum over the four lanes l, l ^ 16, l ^ 32, l ^ 48 (the 64 keys of a
// tile for one query): the permlane swaps pair every lane with lane ^ 32,
// then with lane ^ 16.
LCT_DEV float gp_max4(float t) {
  const auto a = __builtin_amdgcn_permlane32_swap(__float_as_uint(t), __float_as_uint(t), false, false);
  t = fmaxf(__uint_as_float(a[0]), __uint_as_float(a[1]));
  const auto b = __builtin_amdgcn_permlane16_swap(__float_as_uint(t), __float_as_uint(t), false, false);
  return fmaxf(__uint_as_float(b[0]), __uint_as_float(b[1]));
}

// Byte offset of 16-byte chunk c of tile row r: the chunk index is XORed
// with a permutation s(r) of 0..15 over 16 rows, one per array.  V tiles:
// s(r) = 2*(r % 8) + (r / 8) % 2 keeps the pairs of chunks (2i, 2i+1)
// together and gives 4 consecutive rows different pairs (the transposed V
// reads: 4 rows x 2 chunks per 16 lanes).  K tiles: s(r) = 8*(r % 2) +
// (r / 2) % 8 (the A-operand reads: 16 rows, one chunk per 16 lanes).  Both
// were measured free of LDS bank conflicts on gfx950 for their reads (bank
// conflict counter); the V form leaves the A-operand reads 2-way conflicted.
template <bool KT>
LCT_DEV int gp_s(int r) {
  return KT ? ((r & 1) << 3) | ((r >> 1) & 7) : ((r & 7) << 1) | ((r >> 3) & 1);
}
template <bool KT>
LCT_DEV int gp_swz(int r, int c) { return r * GP_ROWB + 16 * (c ^ gp_s<KT>(r)); }

// DMA of key/value rows [row0, row0 + n) (n <= 64; rows past n repeat the
// last one: finite data, masked out) into a tile.  16 instructions of 1 KiB
// per array, 4 per wave: instruction i holds tile rows 4i .. 4i+3, lane l
// the 16 bytes of row 4i + l/16 that the swizzle puts at slot l % 16.
template <bool KT>
LCT_DEV void gp_dma(__amdgpu_buffer_rsrc_t rs, int row0, int n, char* tile, int wid, int lane) {
#pragma unroll
  for (int u = 0; u < 4; ++u) {
    const int i = wid * 4 + u;
    const int r = 4 * i + (lane >> 4);
    const int c = (lane & 15) ^ gp_s<KT>(r);
    const int rg = row0 + (r < n ? r : n - 1);
    __builtin_amdgcn_raw_ptr_buffer_load_lds(rs, (gp_lds_void*)(tile + i * 1024), 16, rg * GP_ROWB + c * 16, 0, 0,
                                             0);
  }
}

// DMA of a whole tile (rows [row0, row0 + 64)): the same slots as gp_dma,
// the row base in the scalar offset and the lane part precomputed (off[u]).
LCT_DEV void gp_dma_whole(__amdgpu_buffer_rsrc_t rs, int row0, char* tile, int wid, const int* off) {
#pragma unroll
  for (int u = 0; u < 4; ++u)
    __builtin_amdgcn_raw_ptr_buffer_load_lds(rs, (gp_lds_void*)(tile + (wid * 4 + u) * 1024), 16, off[u],
                                             row0 * GP_ROWB, 0, 0);
}

// Tile t of a workgroup's key walk: the gist prefix [0, na) in tiles of 64,
// then the band rows [b0, b0 + nb).  seg 0: gist keys, 1: raw keys.  Row
// indices fit in 32 bits (a head's raw K array is < 2 GiB).
struct GpTile {
  int seg, n, r0;
};
LCT_DEV GpTile gp_tile(int t, int ta, int na, int b0, int nb) {
  GpTile x;
  if (t < ta) {
    x.seg = 0;
    x.r0 = t * GP_TILE;
    x.n = na - x.r0 < GP_TILE ? na - x.r0 : GP_TILE;
  } else {
    x.seg = 1;
    x.r0 = b0 + (t - ta) * GP_TILE;
    x.n = b0 + nb - x.r0 < GP_TILE ? b0 + nb - x.r0 : GP_TILE;
  }
  return x;
}

// The DMA of one tile's K and V rows; the buffer resources are made here from
// uniform pointers (passed through a lambda's captures or selected as values
// they are not known to be uniform and get re-made lane by lane).
LCT_DEV void gp_issue(const GpTile& x, const uint16_t* gkb, const uint16_t* gvb, const uint16_t* rkb,
                      const uint16_t* rvb, int64_t Nc, int64_t raw_cap, char* tk, char* tv, int wid, int lane,
                      const int* offk, const int* offv) {
  if (x.n == GP_TILE) {
    if (x.seg == 0) {
      gp_dma_whole(make_rsrc(gkb, Nc * GP_ROWB), x.r0, tk, wid, offk);
      gp_dma_whole(make_rsrc(gvb, Nc * GP_ROWB), x.r0, tv, wid, offv);
    } else {
      gp_dma_whole(make_rsrc(rkb, raw_cap * GP_ROWB), x.r0, tk, wid, offk);
      gp_dma_whole(make_rsrc(rvb, raw_cap * GP_ROWB), x.r0, tv, wid, offv);
    }
  } else if (x.seg == 0) {
    gp_dma<true>(make_rsrc(gkb, Nc * GP_ROWB), x.r0, x.n, tk, wid, lane);
    gp_dma<false>(make_rsrc(gvb, Nc * GP_ROWB), x.r0, x.n, tv, wid, lane);
  } else {
    gp_dma<true>(make_rsrc(rkb, raw_cap * GP_ROWB), x.r0, x.n, tk, wid, lane);
    gp_dma<false>(make_rsrc(rvb, raw_cap * GP_ROWB), x.r0, x.n, tv, wid, lane);
  }
}

// The keys of a tile that query hl of a wave sees form one interval of tile
// rows, [lo, hi) (empty when lo >= hi).  seg 0: gist keys, seg 1: raw keys;
// qid: raw -> the wave's chunk, gist -> the wave's first gist (query hl is
// gist qid + hl).
//   raw query, gists:  the earlier gists, key < qid
//   raw query, raws:   its chunk's tokens up to itself, 16 qid <= key <= 16 qid + hl
//   gist query, gists: the earlier gists and itself, key <= qid + hl
//   gist query, raws:  its chunk's 16 tokens, 16 (qid + hl) <= key < 16 (qid + hl + 1)
template <bool GQ>
LCT_DEV void gp_interval(int seg, int r0, int n, int qid, int hl, int& lo, int& hi) {
  int a, b;
  if (!GQ) {
    a = seg == 0 ? 0 : GP_CHUNK * qid;
    b = seg == 0 ? qid : GP_CHUNK * qid + hl + 1;
  } else {
    a = seg == 0 ? 0 : GP_CHUNK * (qid + hl);
    b = seg == 0 ? qid + hl + 1 : GP_CHUNK * (qid + hl + 1);
  }
  lo = a - r0 > 0 ? a - r0 : 0;
  hi = b - r0 < n ? b - r0 : n;
  hi = hi > lo ? hi : lo;
}

// 0: the wave sees no pair of the tile, 2: every pair, 1: some.
template <bool GQ>
LCT_DEV int gp_tile_class(int seg, int r0, int n, int qid) {
  if (!GQ) {
    if (seg == 0) return r0 >= qid ? 0 : (r0 + GP_TILE <= qid && n == GP_TILE ? 2 : 1);
    return (r0 + n <= qid * GP_CHUNK || r0 >= (qid + 1) * GP_CHUNK) ? 0 : 1;
  }
  if (seg == 0) return r0 > qid + 15 ? 0 : (r0 + GP_TILE - 1 <= qid && n == GP_TILE ? 2 : 1);
  return (r0 + n <= qid * GP_CHUNK || r0 >= (qid + 16) * GP_CHUNK) ? 0 : 1;
}

// One workgroup's work: workgroup `blk` of the raw (GQ false) or gist (GQ
// true) queries of nbh (batch, head) pairs, taken heaviest first over all
// pairs (blk / nbh counts down the query blocks, blk % nbh picks the pair);
// the four tile buffers are the kernel's LDS objects.
template <bool GQ>
LCT_DEV void gp_workgroup(const uint16_t* __restrict__ qr, const uint16_t* __restrict__ qg,
                          const uint16_t* __restrict__ rk, const uint16_t* __restrict__ rv,
                          const uint16_t* __restrict__ gk, const uint16_t* __restrict__ gv,
                          float* __restrict__ outr, float* __restrict__ outg, int64_t Nc, int64_t raw_cap,
                          float scale_log2, int blk, int wg_per_bh, char* tk0, char* tv0, char* tk1,
                          char* tv1, int nbh) {
  constexpr int D = GP_D;
  constexpr int NG = GP_QG;  // query groups of 16 per wave
  const int lane = threadIdx.x & 63, wid = wave_id();
  const int hl = lane & 15, kg = lane >> 4;
  const int64_t bh = blk % nbh;
  const int j = wg_per_bh - 1 - blk / nbh;  // heaviest first over all heads
  const int nc = (int)Nc;
  // queries of group g: raw -> chunk qid[g]'s 16 tokens; gist -> gists qid[g] .. qid[g]+15
  constexpr int QPW = GQ ? 16 * NG : NG;       // gists / chunks per wave
  constexpr int QPG = GP_NW * QPW;             // per workgroup
  int qid[NG];
#pragma unroll
  for (int g = 0; g < NG; ++g) qid[g] = QPG * j + QPW * wid + (GQ ? 16 * g : g);
  // key segments: the gist prefix the workgroup's last query sees, then the band
  const int na = GQ ? min(nc, QPG * j + QPG) : min(nc, QPG * j + QPG - 1);
  const int b0 = QPG * j * GP_CHUNK;
  const int nb = min(QPG * GP_CHUNK, (nc - QPG * j) * GP_CHUNK);
  const int ta = (int)((na + GP_TILE - 1) / GP_TILE);
  const int tb = (int)((nb + GP_TILE - 1) / GP_TILE);
  const int nt = ta + tb;
  const uint16_t* gkb = gk + bh * Nc * D;
  const uint16_t* gvb = gv + bh * Nc * D;
  const uint16_t* rkb = rk + bh * raw_cap * D;
  const uint16_t* rvb = rv + bh * raw_cap * D;

  // query fragments (B operands): lane (hl, kg) holds query hl of group g,
  // features st*32 + kg*8 ..
  bf16x8 qf[NG][4];
#pragma unroll
  for (int g = 0; g < NG; ++g) {
    const int qrow = GQ ? min(qid[g] + hl, nc - 1) : min(qid[g], nc - 1) * GP_CHUNK + hl;
    const uint16_t* qp = (GQ ? qg + (bh * Nc + qrow) * D : qr + (bh * Nc * GP_CHUNK + qrow) * D) + kg * 8;
#pragma unroll
    for (int st = 0; st < 4; ++st) qf[g][st] = *reinterpret_cast<const bf16x8*>(qp + st * 32);
  }
  bf16x8 ones;
#pragma unroll
  for (int i = 0; i < 8; ++i) ones[i] = (__bf16)1.0f;
  float m[NG];
  floatx4 lacc[NG];
  floatx4 o[NG][D / 16];
#pragma unroll
  for (int g = 0; g < NG; ++g) {
    m[g] = -INFINITY;
    lacc[g] = floatx4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int dt = 0; dt < D / 16; ++dt) o[g][dt] = floatx4{0.f, 0.f, 0.f, 0.f};
  }
  int doffk[4], doffv[4];  // this lane's byte offsets in a whole tile's DMA (gp_dma's slots)
#pragma unroll
  for (int u = 0; u < 4; ++u) {
    const int r = 4 * (wid * 4 + u) + (lane >> 4);
    doffk[u] = r * GP_ROWB + 16 * ((lane & 15) ^ gp_s<true>(r));
    doffv[u] = r * GP_ROWB + 16 * ((lane & 15) ^ gp_s<false>(r));
  }
  // transposed V read of this lane: token 4*kg + hl/4 of a block, features
  // 16*dt + 4*(hl%4) .. +3 -> chunk 2*dt + (hl%4)/2, byte 8*(hl%2)
  const int trt = 4 * kg + (hl >> 2);

  auto compute = [&](int t, const char* tk, const char* tv) {
    const GpTile x = gp_tile(t, ta, na, b0, nb);
    const int seg = x.seg, n = x.n, r0 = x.r0;
    int cls[NG];
    bool any = false;
#pragma unroll
    for (int g = 0; g < NG; ++g) {
      cls[g] = qid[g] < nc ? gp_tile_class<GQ>(seg, r0, n, qid[g]) : 0;
      any = any || cls[g] != 0;
    }
    if (!any) return;  // uniform over the wave
    // S^T = K Q^T: sacc[g][jb][e] = S^T[key 16jb + 4kg + e][query hl of group g];
    // each K fragment read from LDS serves every query group
    floatx4 sacc[NG][4];
#pragma unroll
    for (int jb = 0; jb < 4; ++jb) {
#pragma unroll
      for (int g = 0; g < NG; ++g) sacc[g][jb] = floatx4{0.f, 0.f, 0.f, 0.f};
      const int r = 16 * jb + hl;
#pragma unroll
      for (int st = 0; st < 4; ++st) {
        const bf16x8 kf = *reinterpret_cast<const bf16x8*>(tk + gp_swz<true>(r, st * 4 + kg));
#pragma unroll
        for (int g = 0; g < NG; ++g)
          sacc[g][jb] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(kf, qf[g][st], sacc[g][jb], 0, 0, 0);
      }
    }
    uint32_t pw[NG][4][2];  // bf16 weight pairs: keys 16 jb + 4 kg + (2i, 2i+1)
#pragma unroll
    for (int g = 0; g < NG; ++g) {
      // a tile the group sees whole takes the unmasked path (uniform branch)
      float tmax = -INFINITY;
      bool vis[4][4];
      int lo = 0, hi = 0;
      if (cls[g] == 1) {
        gp_interval<GQ>(seg, r0, n, qid[g], hl, lo, hi);
        lo -= 4 * kg;  // row 16 jb + 4 kg + e is visible iff lo <= 16 jb + e < hi
        hi = max(hi - 4 * kg, lo);
      }
      if (cls[g] == 2) {
#pragma unroll
        for (int jb = 0; jb < 4; ++jb)
#pragma unroll
          for (int e = 0; e < 4; ++e) tmax = fmaxf(tmax, sacc[g][jb][e]);
      } else {
#pragma unroll
        for (int jb = 0; jb < 4; ++jb)
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            vis[jb][e] = (unsigned)(16 * jb + e - lo) < (unsigned)(hi - lo);
            tmax = fmaxf(tmax, vis[jb][e] ? sacc[g][jb][e] : -INFINITY);
          }
      }
      tmax = gp_max4(tmax);
      // the reference maximum moves only when a score exceeds it by more
      // than 2^GP_SLACK: the weights stay <= 2^GP_SLACK (fine in fp32 and
      // bf16) and O is rescaled far less often
      const float cand = tmax * scale_log2;
      const bool grow = cand > m[g] + GP_SLACK;
      const float mnew = grow ? cand : m[g];
      const float mref = mnew == -INFINITY ? 0.f : mnew;  // a query with nothing visible yet
      const float alpha = __builtin_amdgcn_exp2f(m[g] - mref);
      m[g] = mnew;
      if (cls[g] == 2) {
#pragma unroll
        for (int jb = 0; jb < 4; ++jb) {
          float w[4];
#pragma unroll
          for (int e = 0; e < 4; ++e) w[e] = __builtin_amdgcn_exp2f(fmaf(sacc[g][jb][e], scale_log2, -mref));
          pw[g][jb][0] = gp_pack(w[0], w[1]);
          pw[g][jb][1] = gp_pack(w[2], w[3]);
        }
      } else {
#pragma unroll
        for (int jb = 0; jb < 4; ++jb) {
          float w[4];
#pragma unroll
          for (int e = 0; e < 4; ++e)
            w[e] = vis[jb][e] ? __builtin_amdgcn_exp2f(fmaf(sacc[g][jb][e], scale_log2, -mref)) : 0.f;
          pw[g][jb][0] = gp_pack(w[0], w[1]);
          pw[g][jb][1] = gp_pack(w[2], w[3]);
        }
      }
      if (__ballot(grow) != 0) {
#pragma unroll
        for (int dt = 0; dt < D / 16; ++dt) o[g][dt] = o[g][dt] * alpha;
        lacc[g] = lacc[g] * alpha;
      }
    }
    // O^T += V^T P^T, 32 keys (blocks 2h, 2h+1) per MFMA; each V fragment
    // read from LDS serves every query group
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      bf16x8 pf[NG];
#pragma unroll
      for (int g = 0; g < NG; ++g)
        pf[g] = __builtin_bit_cast(bf16x8, (uintx4){pw[g][2 * h][0], pw[g][2 * h][1], pw[g][2 * h + 1][0],
                                                     pw[g][2 * h + 1][1]});
#pragma unroll
      for (int dt = 0; dt < D / 16; ++dt) {
        const int c = 2 * dt + ((hl & 3) >> 1);
        const int rlo = 16 * (2 * h) + trt, rhi = 16 * (2 * h + 1) + trt;
        const short4v lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
            (gp_lds_short4v*)(tv + gp_swz<false>(rlo, c) + 8 * (hl & 1)));
        const short4v hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
            (gp_lds_short4v*)(tv + gp_swz<false>(rhi, c) + 8 * (hl & 1)));
        const bf16x8 va = __builtin_bit_cast(bf16x8, __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7));
#pragma unroll
        for (int g = 0; g < NG; ++g) o[g][dt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(va, pf[g], o[g][dt], 0, 0, 0);
      }
#pragma unroll
      for (int g = 0; g < NG; ++g) lacc[g] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(ones, pf[g], lacc[g], 0, 0, 0);
    }
  };

  // two LDS buffers, the loop unrolled by two so every access names one of
  // them; a tile's DMA is waited for by its issuing waves, then the barrier
  // makes it visible to all and frees the other buffer for the next tile
  if (nt > 0) gp_issue(gp_tile(0, ta, na, b0, nb), gkb, gvb, rkb, rvb, Nc, raw_cap, tk0, tv0, wid, lane, doffk, doffv);
  for (int t = 0; t < nt; t += 2) {
    GP_WAIT_VM0();
    __syncthreads();
    if (t + 1 < nt)
      gp_issue(gp_tile(t + 1, ta, na, b0, nb), gkb, gvb, rkb, rvb, Nc, raw_cap, tk1, tv1, wid, lane, doffk, doffv);
    gp_fence();
    compute(t, tk0, tv0);
    gp_fence();
    if (t + 1 >= nt) break;
    GP_WAIT_VM0();
    __syncthreads();
    if (t + 2 < nt)
      gp_issue(gp_tile(t + 2, ta, na, b0, nb), gkb, gvb, rkb, rvb, Nc, raw_cap, tk0, tv0, wid, lane, doffk, doffv);
    gp_fence();
    compute(t + 1, tk1, tv1);
    gp_fence();
  }

  // o[g][dt][e] = O^T[d = 16dt + 4kg + e][query hl of group g]; lacc: the denominator
#pragma unroll
  for (int g = 0; g < NG; ++g) {
    const float l = lacc[g][0];
    const float inv = l > 0.f ? 1.f / l : 0.f;
    float* op;
    if (GQ) {
      if (qid[g] + hl >= nc) continue;
      op = outg + (bh * Nc + qid[g] + hl) * D + kg * 4;
    } else {
      if (qid[g] >= nc) continue;
      op = outr + (bh * Nc * GP_CHUNK + qid[g] * GP_CHUNK + hl) * D + kg * 4;
    }
#pragma unroll
    for (int dt = 0; dt < D / 16; ++dt) *reinterpret_cast<floatx4*>(op + dt * 16) = o[g][dt] * inv;
  }
}

// Both query kinds in one launch: the gist workgroups (the heavier ones on
// average) first, then the raw ones, each kind heaviest first over all heads,
// so the light raw workgroups fill the tail.
__global__ __launch_bounds__(GP_NW * 64) void k_gsa_prefill(
    const uint16_t* __restrict__ qr, const uint16_t* __restrict__ qg, const uint16_t* __restrict__ rk,
    const uint16_t* __restrict__ rv, const uint16_t* __restrict__ gk, const uint16_t* __restrict__ gv,
    float* __restrict__ outr, float* __restrict__ outg, int64_t Nc, int64_t raw_cap, float scale_log2,
    int n_gist_wg, int wg_gist_per_bh, int wg_raw_per_bh) {
  __shared__ __attribute__((aligned(16))) char tk0[GP_TILEB];
  __shared__ __attribute__((aligned(16))) char tv0[GP_TILEB];
  __shared__ __attribute__((aligned(16))) char tk1[GP_TILEB];
  __shared__ __attribute__((aligned(16))) char tv1[GP_TILEB];
  const int blk = (int)blockIdx.x;
  if (blk < n_gist_wg)
    gp_workgroup<true>(qr, qg, rk, rv, gk, gv, outr, outg, Nc, raw_cap, scale_log2, blk, wg_gist_per_bh, tk0, tv0,
                       tk1, tv1, n_gist_wg / wg_gist_per_bh);
  else
    gp_workgroup<false>(qr, qg, rk, rv, gk, gv, outr, outg, Nc, raw_cap, scale_log2, blk - n_gist_wg,
                        wg_raw_per_bh, tk0, tv0, tk1, tv1, n_gist_wg / wg_gist_per_bh);
}

hipError_t launch_gsa_prefill(const uint16_t* qr, const uint16_t* qg, const uint16_t* rk, const uint16_t* rv,
                              const uint16_t* gk, const uint16_t* gv, float* outr, float* outg, int BH,
                              int64_t Nc, int64_t raw_cap, float scale, hipStream_t st) {
  const float sl2 = scale * GP_LOG2E;
  const int wr = (int)((Nc + GP_NW * GP_QG - 1) / (GP_NW * GP_QG));
  const int wgq = (int)((Nc + GP_NW * GP_QG * 16 - 1) / (GP_NW * GP_QG * 16));
  if ((int64_t)BH * (wr + wgq) >= ((int64_t)1 << 31)) return hipErrorInvalidValue;
  const int ngist = BH * wgq;
  k_gsa_prefill<<<dim3((unsigned)(ngist + BH * wr)), GP_NW * 64, 0, st>>>(qr, qg, rk, rv, gk, gv, outr, outg, Nc,
                                                                         raw_cap, sl2, ngist, wgq, wr);
  return hipGetLastError();
}

}  // namespace lct
