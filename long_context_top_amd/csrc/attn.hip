// Sparse attention over gathered K/V rows for gfx950.
//
// Source: CLSA explainer section 1.1 (softmax(QK^T / sqrt(d_k)) V) evaluated
// over the selected keys only (section 2.3, selector; tutorial DSA section);
// split decode with a log-sum-exp merge of partial results and one KV-tile
// load serving every query head of its KV group (SSA article, section 6).
//
// Work unit: one (batch, query row, KV head) and a run of its index entries.
// Each wave owns one unit and works through the run 64 selected positions at
// a time; the waves of a workgroup are independent (no workgroup barrier,
// each wave has its own LDS region):
//   * gathers read 16 tokens x 64 contiguous bytes per instruction (a quad
//     of lanes per token piece, the rate the address unit takes);
//   * the K pieces are moved by ds_bpermute into the A operand of
//     v_mfma_f32_16x16x32_bf16 (lane = row lane%16, 8 features at
//     8*(lane/16)); the G query heads of the KV group form the B operand, so
//     S^T[token][head] comes out in C layout (4 tokens x 1 head per lane);
//   * fp32 online softmax per head (running max and sum, exp2 domain);
//   * O^T += V^T P^T on the same MFMA: P^T from the C fragments is already in
//     B-operand layout (the k order inside the MFMA is a fixed permutation of
//     32 tokens); the V pieces go into the wave's LDS tile (decode: buffer
//     loads to LDS, no registers; many rows: through registers and LDS
//     stores) and are read back transposed with ds_read_b64_tr_b16 (4 tokens
//     x 4 features per lane);
//   * software pipelined: the next 64 positions' gathers are in flight while
//     this iteration's MFMA and softmax run.
// Few rows (decode): the index row is split over several waves, each writes
// an (O, m, l) partial and k_split_merge combines them.  Many rows over a
// long cache (prefill): the positions are cut into segments and the units
// ordered segment-major so the gathers hit L2 (k_sparse_attn_seg below).

#include "common.h"
#include "kernels.h"

namespace lct {

constexpr int ATT_D = 128;
constexpr int ATT_STEP = 64;             // positions per wave iteration (4 blocks of 16)
constexpr int ATT_NW = 4;                // independent waves per workgroup
constexpr int ATT_PS = ATT_D + 4;        // partial row: O[D], m, l, 2 pad (16-byte rows)
constexpr int ATT_TARGET_WAVES = 1024;   // split short index rows until this many waves
constexpr float LOG2E = 1.4426950408889634f;
#ifndef ATT_SEG_SHIFT
#define ATT_SEG_SHIFT 14                 // log2 positions per segment (segmented path)
#endif
constexpr int ATT_SEG_MAX = 64;          // segments per row at most (the segment grows)
constexpr int UA_R = 16;                 // rows per block of the block-union path
constexpr int64_t ATT_SEG_MIN_UNITS = 16384;  // (row, KV head) pairs that take the segmented path

typedef __attribute__((address_space(3))) short4v lds_short4v;
typedef __attribute__((address_space(3))) void lds_void;
typedef const __attribute__((address_space(1))) void global_cvoid;

// s_waitcnt vmcnt(0) (expcnt, lgkmcnt left at their maxima): the LDS DMA
// writes are counted by vmcnt and the compiler does not track them
constexpr int WAITCNT_VM0 = 0x0F70;
// s_waitcnt vmcnt(n): vmcnt is 6 bits, low 4 in [3:0], high 2 in [15:14]
constexpr int waitcnt_vm(int n) { return 0x0F70 | (n & 15) | ((n >> 4) << 14); }
constexpr int WAITCNT_VM8 = waitcnt_vm(8);
constexpr int WAITCNT_VM24 = waitcnt_vm(24);
// s_waitcnt lgkmcnt(0) (vmcnt, expcnt at their maxima)
constexpr int WAITCNT_LGKM0 = 0xC07F;

AttnPlan attn_plan(int B, int Lq, int Hq, int Hkv, int kk, int64_t L) {
  AttnPlan p;
  const int G = Hq / Hkv;
  const int64_t rows = (int64_t)B * Lq;
  const int64_t units = rows * Hkv;
  p.nseg = 0;
  p.seg_shift = 0;
  p.bnd_bytes = 0;
  p.ua_blocks = 0;
  // many rows over a long cache: position segments (see k_sparse_attn_seg)
  if (units >= ATT_SEG_MIN_UNITS && L > ((int64_t)2 << ATT_SEG_SHIFT)) {
    int shift = ATT_SEG_SHIFT;
    while (((L - 1) >> shift) + 1 > ATT_SEG_MAX) ++shift;
    p.seg_shift = shift;
    p.nseg = (int)(((L - 1) >> shift) + 1);
    p.splits = 1;
    p.per_split = kk;
    p.part_bytes = (size_t)units * p.nseg * G * ATT_PS * sizeof(float);
    p.bnd_bytes = (size_t)rows * (p.nseg + 1) * sizeof(int32_t);
    // blocks of UA_R rows that may take the block-union path (one flag each)
    p.ua_blocks = (G == 4 || G == 8 || G == 16) ? rows / UA_R : 0;
    return p;
  }
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

// Index entries [e0, e0 + 64) gate the gathers of one iteration: lane l
// holds entry e0 + 16j + l/4 for j < 4, the token whose row its gathers
// read (clamped into the slice, so in bounds; entries past the slice are
// masked by the caller).
LCT_DEV void attn_entries(const int32_t* ix, int e0, int e_end, int tk, int (&pos)[4]) {
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    const int e = e0 + 16 * j + tk;
    pos[j] = ix[e < e_end ? e : e_end - 1];
  }
}

LCT_DEV bf16x8 lane_permute(bf16x8 x, int src_byte) {
  const int4 w = __builtin_bit_cast(int4, x);
  int4 r;
  r.x = __builtin_amdgcn_ds_bpermute(src_byte, w.x);
  r.y = __builtin_amdgcn_ds_bpermute(src_byte, w.y);
  r.z = __builtin_amdgcn_ds_bpermute(src_byte, w.z);
  r.w = __builtin_amdgcn_ds_bpermute(src_byte, w.w);
  return __builtin_bit_cast(bf16x8, r);
}

// Query fragment (B operand): the G query heads of KV head kvh of query row
// br; lanes of head slots >= G load head G-1 and are zeroed.
template <int G>
LCT_DEV void attn_query(const uint16_t* q, int64_t br, int Hq, int kvh, int hl, int kg,
                        bf16x8 (&qf)[4]) {
  constexpr int D = ATT_D;
  const int hq = hl < G ? hl : G - 1;
#pragma unroll
  for (int st = 0; st < 4; ++st) {
    qf[st] = *reinterpret_cast<const bf16x8*>(q + ((br * Hq) + kvh * G + hq) * D + st * 32 + kg * 8);
    if (hl >= G) qf[st] = bf16x8{};
  }
}

// Gather roles.  Each load instruction reads 16 tokens x 64 bytes (a
// 32-feature slice st of each row), lane l taking 16-byte chunk ck = l%4 of
// token tk = l/4: the four lanes of a quad read one contiguous 64-byte
// piece, so the address unit takes a quad per cycle (one row per lane, as
// the MFMA operand layout would have it, costs a cycle per lane).  K chunks
// land in registers and are moved to the A-operand layout (lane (hl, kg):
// token hl, chunk kg) with ds_bpermute; V chunks go to LDS by DMA, lane l's
// 16 bytes at 16*l, the chunk order inside a quad swizzled (chunk
// ck ^ 2*(tk/4 % 2)) so the transposed reads of lanes 0-31 fall on distinct
// banks.

// Positions of one iteration's tokens: -1 where the entry is past the slice,
// -1 or outside [0, L); msk[j] bit 4t set <=> token t of block j is valid.
LCT_DEV bool attn_mask(int e0, int e_end, int64_t L, int tk, const int (&pos)[4], int (&pp)[4],
                       uint64_t (&msk)[4]) {
  bool any = false;
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    const int e = e0 + 16 * j + tk;
    int p = pos[j];
    if (e >= e_end || p < 0 || (int64_t)p >= L) p = -1;
    pp[j] = p;
    msk[j] = __ballot(p >= 0);
    any = any || msk[j] != 0;
  }
  return any;  // uniform over the wave
}

// K chunks of one iteration into registers; masked tokens read row 0 (in
// bounds) and are masked in the softmax.
LCT_DEV void attn_gather_k(__amdgpu_buffer_rsrc_t krs, int row_bytes, int ck, const int (&pp)[4],
                           bf16x8 (&kr)[4][4]) {
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    const int roff = (pp[j] >= 0 ? pp[j] : 0) * row_bytes + ck * 16;  // < 2 GiB
#pragma unroll
    for (int st = 0; st < 4; ++st)
      kr[j][st] = __builtin_bit_cast(bf16x8, __builtin_amdgcn_raw_buffer_load_b128(krs, roff + st * 64, 0, 0));
  }
}

// V chunks of blocks 2h, 2h+1 of one iteration into half h of the wave's
// LDS tile, lane l's 16 bytes of each 1 KiB piece at byte 16 l.  VREG = false:
// by DMA (no registers, the wave does not wait); the halves are separate LDS
// objects, so the compiler can tell that reads of one do not wait for DMA
// into the other.  (Buffer loads rather than global ones: the compiler counts
// a global load that writes LDS as touching both memories and then waits for
// every outstanding load whenever any register load result is needed.)
// VREG = true: loaded into registers and written to LDS by the wave, which
// waits for the data there; measured faster for the many-row kernel, whose
// gathers keep the address unit busy (16.3 -> 15.7-15.9 ms per 64K layer), and
// slower for the decode kernel, whose gathers are latency bound.
template <bool VREG>
LCT_DEV void attn_gather_v_half(__amdgpu_buffer_rsrc_t vrs, int row_bytes, int cv,
                                const int (&pp)[4], int h, char (*vh)[4][1024]) {
#pragma unroll
  for (int jj = 0; jj < 2; ++jj) {
    const int j = 2 * h + jj;
    // byte offset of the chunk inside the batch entry's V (< 2 GiB)
    const int roff = (pp[j] >= 0 ? pp[j] : 0) * row_bytes + cv * 16;  // < 2 GiB
#pragma unroll
    for (int st = 0; st < 4; ++st) {
      if (VREG) {
        const uintx4 t = __builtin_amdgcn_raw_buffer_load_b128(vrs, roff + st * 64, 0, 0);
        *reinterpret_cast<uintx4*>(&vh[jj][st][(threadIdx.x & 63) * 16]) = t;
      } else {
        __builtin_amdgcn_raw_ptr_buffer_load_lds(vrs, (lds_void*)&vh[jj][st][0], 16, roff + st * 64, 0, 0, 0);
      }
    }
  }
}

// Per-lane constants of the gather and transposed-read layouts.
struct AttnLanes {
  int hl, kg;  // MFMA layout: row / column lane%16, k-group lane/16
  int tk, ck;  // gather layout: token lane/4, chunk lane%4
  int cv;      // swizzled V chunk
  int bsrc;    // ds_bpermute byte address of the lane holding (token hl, chunk kg)
  int tr0, tr1;  // transposed-read byte offsets for even / odd feature tiles
};

LCT_DEV AttnLanes attn_lanes(int lane) {
  AttnLanes a;
  a.hl = lane & 15;
  a.kg = lane >> 4;
  a.tk = lane >> 2;
  // K chunk order inside a quad: tokens 8-15 take their chunks rotated by
  // two, so the 32 source lanes of each half of a ds_bpermute below are
  // distinct modulo 32
  a.ck = (lane & 3) ^ ((a.tk >> 3) << 1);
  a.cv = (lane & 3) ^ (((a.tk >> 2) & 1) << 1);
  a.bsrc = (4 * a.hl + (a.kg ^ ((a.hl >> 3) << 1))) * 4;
  // transposed read of 16-feature tile dt of block j: this lane supplies
  // token T = 4*kg + hl/4, features 16*dt + 4*(hl%4) .. +3: chunk
  // c = 2*(dt%2) + (hl%4)/2 of slice dt/2, stored at lane 4T + (c ^ 2*(kg%2)),
  // byte 8*(hl%2) of it
  const int trb = 64 * (4 * a.kg + (a.hl >> 2)) + 16 * ((a.hl & 3) >> 1) + 8 * (a.hl & 1);
  a.tr0 = trb + 32 * (a.kg & 1);
  a.tr1 = trb + 32 * ((a.kg & 1) ^ 1);
  return a;
}

// One iteration (64 index entries) of the online softmax.  On entry kr
// holds this iteration's K chunks (gather layout), the V tile is in flight
// or landed, pp/msk describe its tokens and pos holds the next iteration's
// entries.  With NEXT the next iteration's K gathers are issued once this
// iteration's K has gone through the MFMAs, its V gathers (two halves) once
// the matching half of this iteration's V tile has been read, so both
// overlap this iteration's MFMA and softmax work; on exit kr, pp, msk and
// pos describe the next iteration.
template <int G, bool NEXT, bool VREG>
LCT_DEV void attn_iter(const int32_t* ix, int e0, int e_end, int64_t L, const AttnLanes& a,
                       int (&pos)[4], int (&pp)[4], uint64_t (&msk)[4], bf16x8 (&kr)[4][4],
                       const bf16x8 (&qf)[4], __amdgpu_buffer_rsrc_t krs, __amdgpu_buffer_rsrc_t vrs,
                       int row_bytes, float scale_log2, char (*vta)[4][1024],
                       char (*vtb)[4][1024], float& m, floatx4& lacc, floatx4 (&o)[ATT_D / 16]) {
  constexpr int D = ATT_D;
  bf16x8 ones;
#pragma unroll
  for (int i = 0; i < 8; ++i) ones[i] = (__bf16)1.0f;
  // S^T = K Q^T per 16-token block; sacc[j][e] = S^T[token 16j + 4kg + e][head hl]
  floatx4 sacc[4];
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    sacc[j] = floatx4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int st = 0; st < 4; ++st)
      sacc[j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(lane_permute(kr[j][st], a.bsrc), qf[st], sacc[j],
                                                         0, 0, 0);
  }
  uint64_t mskc[4];
#pragma unroll
  for (int j = 0; j < 4; ++j) mskc[j] = msk[j];
  int ppn[4];
  if (NEXT) {
    attn_mask(e0 + ATT_STEP, e_end, L, a.tk, pos, ppn, msk);
    attn_gather_k(krs, row_bytes, a.ck, ppn, kr);
    attn_entries(ix, e0 + 2 * ATT_STEP, e_end, a.tk, pos);
  }
  // running maximum in the exp2 domain (scale_log2 > 0 commutes with max)
  const bool full = (mskc[0] & mskc[1] & mskc[2] & mskc[3]) == ~0ull;  // uniform
  uint32_t mk[4];  // this lane's tokens 4kg + e of block j: bit 4e
#pragma unroll
  for (int j = 0; j < 4; ++j) mk[j] = (uint32_t)(mskc[j] >> (16 * a.kg));
  float tmax = -INFINITY;
  if (full) {
#pragma unroll
    for (int j = 0; j < 4; ++j)
#pragma unroll
      for (int e = 0; e < 4; ++e) tmax = fmaxf(tmax, sacc[j][e]);
  } else {
#pragma unroll
    for (int j = 0; j < 4; ++j)
#pragma unroll
      for (int e = 0; e < 4; ++e) tmax = fmaxf(tmax, ((mk[j] >> (4 * e)) & 1) ? sacc[j][e] : -INFINITY);
  }
  tmax = fmaxf(tmax, __shfl_xor(tmax, 16, 64));
  tmax = fmaxf(tmax, __shfl_xor(tmax, 32, 64));
  const float mnew = fmaxf(m, tmax * scale_log2);
  // no valid token yet (a run of skipped entries): any finite reference
  // keeps alpha and the weights at 0 instead of NaN
  const float mref = mnew == -INFINITY ? 0.f : mnew;
  const float alpha = __builtin_amdgcn_exp2f(m - mref);
  m = mnew;
  // weights 2^(s * scale_log2 - m), rounded to bf16 for the PV product; the
  // denominator is the same MFMA over these rounded weights (a row of ones)
  __bf16 pw[4][4];
  if (full) {
#pragma unroll
    for (int j = 0; j < 4; ++j)
#pragma unroll
      for (int e = 0; e < 4; ++e) pw[j][e] = (__bf16)__builtin_amdgcn_exp2f(fmaf(sacc[j][e], scale_log2, -mref));
  } else {
#pragma unroll
    for (int j = 0; j < 4; ++j)
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const float w = __builtin_amdgcn_exp2f(fmaf(sacc[j][e], scale_log2, -mref));
        pw[j][e] = (__bf16)(((mk[j] >> (4 * e)) & 1) ? w : 0.f);
      }
  }
  // the running maximum moves ever more rarely: rescale only when it did
  if (__ballot(alpha != 1.f) != 0) {
#pragma unroll
    for (int dt = 0; dt < D / 16; ++dt) o[dt] = o[dt] * alpha;
    lacc = lacc * alpha;
  }
  // O^T += V^T P^T, 32 tokens (blocks 2h, 2h+1: half h of the tile) per
  // MFMA: the MFMA's k = 8kg + jj is token 4kg + jj of block 2h (jj < 4) or
  // 4kg + jj - 4 of block 2h+1, in both operands
#pragma unroll
  for (int h = 0; h < 2; ++h) {
    char(*vh)[4][1024] = h == 0 ? vta : vtb;
    // half h of this iteration's V tile has landed once at most 24 memory
    // operations issued after its DMA are outstanding: after half 0 come
    // half 1 (8) and, with NEXT, the next K gathers (16); after half 1 come,
    // with NEXT, the next K gathers and the next half 0 (24)
    if (NEXT) __builtin_amdgcn_s_waitcnt(WAITCNT_VM24);
    else if (h == 0) __builtin_amdgcn_s_waitcnt(WAITCNT_VM8);
    else __builtin_amdgcn_s_waitcnt(WAITCNT_VM0);
    compiler_fence();
    bf16x8 va[D / 16];
#pragma unroll
    for (int dt = 0; dt < D / 16; ++dt) {
      const int tro = (dt & 1) ? a.tr1 : a.tr0;
      const short4v lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_short4v*)&vh[0][dt >> 1][tro]);
      const short4v hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_short4v*)&vh[1][dt >> 1][tro]);
      // whole-vector reinterpretation (element-wise bf16 casts of the read
      // results are mis-assembled by the compiler)
      va[dt] = __builtin_bit_cast(bf16x8, __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7));
    }
    if (NEXT) {
      // half h is free once its reads have returned: the next iteration's
      // blocks 2h, 2h+1 go there
      __builtin_amdgcn_s_waitcnt(WAITCNT_LGKM0);
      compiler_fence();
      attn_gather_v_half<VREG>(vrs, row_bytes, a.cv, ppn, h, vh);
    }
    bf16x8 pf;
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      pf[e] = pw[2 * h][e];
      pf[4 + e] = pw[2 * h + 1][e];
    }
#pragma unroll
    for (int dt = 0; dt < D / 16; ++dt)
      o[dt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(va[dt], pf, o[dt], 0, 0, 0);
    lacc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(ones, pf, lacc, 0, 0, 0);
  }
  compiler_fence();
  if (NEXT) {
#pragma unroll
    for (int j = 0; j < 4; ++j) pp[j] = ppn[j];
  }
}

// Online softmax attention of one query row's G heads over the index
// entries [e_begin, e_end) of its row `ix`, 64 entries per iteration: on
// return m is the running maximum (exp2 domain), lsum the denominator of the
// lane's head and o = O^T (unnormalised); called with m = -inf, o = 0.  `pos` holds the first iteration's entries
// (attn_entries).  Entries that are -1 or outside [0, L) are skipped.
template <int G, bool VREG>
LCT_DEV void attn_span(const int32_t* ix, int e_begin, int e_end, int (&pos)[4],
                       const bf16x8 (&qf)[4], const uint16_t* kbase, const uint16_t* vbase,
                       size_t row_stride, int64_t L, float scale_log2, char (*vta)[4][1024],
                       char (*vtb)[4][1024], int lane, float& m, float& lsum,
                       floatx4 (&o)[ATT_D / 16]) {
  if (e_begin >= e_end) return;
  const AttnLanes a = attn_lanes(lane);
  int pp[4];
  uint64_t msk[4];
  attn_mask(e_begin, e_end, L, a.tk, pos, pp, msk);
  // K and V rows of this KV head (a batch entry's cache is < 2 GiB, so
  // 32-bit offsets; the range check only guards, every access is in bounds)
  const int row_bytes = (int)(row_stride * 2);
  const __amdgpu_buffer_rsrc_t krs = make_rsrc(kbase, L * (int64_t)row_bytes);
  const __amdgpu_buffer_rsrc_t vrs = make_rsrc(vbase, L * (int64_t)row_bytes);
  bf16x8 kr[4][4];
  attn_gather_k(krs, row_bytes, a.ck, pp, kr);
  attn_entries(ix, e_begin + ATT_STEP, e_end, a.tk, pos);  // the next iteration's entries
  attn_gather_v_half<VREG>(vrs, row_bytes, a.cv, pp, 0, vta);
  attn_gather_v_half<VREG>(vrs, row_bytes, a.cv, pp, 1, vtb);
  // the softmax denominator accumulates on the MFMA (every row of lacc holds
  // the sum of this lane's head)
  floatx4 lacc = floatx4{0.f, 0.f, 0.f, 0.f};
  int e0 = e_begin;
  for (; e0 + ATT_STEP < e_end; e0 += ATT_STEP)
    attn_iter<G, true, VREG>(ix, e0, e_end, L, a, pos, pp, msk, kr, qf, krs, vrs, row_bytes, scale_log2, vta,
                       vtb, m, lacc, o);
  attn_iter<G, false, VREG>(ix, e0, e_end, L, a, pos, pp, msk, kr, qf, krs, vrs, row_bytes, scale_log2, vta,
                      vtb, m, lacc, o);
  lsum = lacc[0];
}

template <int G>
__global__ __launch_bounds__(ATT_NW * 64) void k_sparse_attn(
    const uint16_t* __restrict__ q, const uint16_t* __restrict__ k,
    const uint16_t* __restrict__ v, const int32_t* __restrict__ idx, float* __restrict__ out,
    int64_t units, int Lq, int Hq, int Hkv, int64_t L, int kk, float scale_log2, int splits,
    int per_split, float* __restrict__ part) {
  constexpr int D = ATT_D;
  // per wave, per (16-token block j, 32-feature slice st): the 1 KiB that one
  // LDS DMA instruction writes, lane l's 16 bytes at 16*l; blocks 0-1 and
  // 2-3 in separate objects
  __shared__ __attribute__((aligned(16))) char vta[ATT_NW][2][4][1024];
  __shared__ __attribute__((aligned(16))) char vtb[ATT_NW][2][4][1024];
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

  // index entries of the first iteration (they gate the gathers), then q
  int pos[4];
  attn_entries(ix, e_begin, e_end, lane >> 2, pos);
  bf16x8 qf[4];
  attn_query<G>(q, br, Hq, kvh, hl, kg, qf);
  float m = -INFINITY, lsum = 0.f;
  floatx4 o[D / 16];
#pragma unroll
  for (int dt = 0; dt < D / 16; ++dt) o[dt] = floatx4{0.f, 0.f, 0.f, 0.f};
  const size_t row_stride = (size_t)Hkv * D;  // elements between positions
  attn_span<G, false>(ix, e_begin, e_end, pos, qf, k + ((size_t)b * L * Hkv + kvh) * D,
               v + ((size_t)b * L * Hkv + kvh) * D, row_stride, L, scale_log2, vta[wid], vtb[wid], lane, m,
               lsum, o);

  // o[dt][e] = O^T[d = 16dt + 4kg + e][head hl]; lsum: head hl's denominator
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

template <int SPL>
__global__ __launch_bounds__(256) void k_split_merge(const float* __restrict__ part,
                                                     float* __restrict__ out, int splits, int hs,
                                                     int G, int D, int rs) {
  static_assert(SPL <= 64, "one wave weighs the splits");
  __shared__ float wts[SPL];
  __shared__ float s_inv;
  const int64_t unit = blockIdx.x;
  const int h = blockIdx.y;
  const int d = threadIdx.x < D ? threadIdx.x : D - 1;
  const size_t stride = (size_t)hs * rs;
  const float* base = part + ((size_t)unit * splits * hs + h) * rs;
  // all loads are issued together: this thread's feature of every split
  // (unconditional; split indices past `splits` re-read the last split and get
  // weight 0) and, in the first wave, one split's (m, l) per lane
  float o[SPL];
#pragma unroll
  for (int s = 0; s < SPL; ++s) o[s] = base[(size_t)(s < splits ? s : splits - 1) * stride + d];
  if (threadIdx.x < 64) {
    const int s = threadIdx.x < splits ? threadIdx.x : splits - 1;
    const float m = base[(size_t)s * stride + D];
    const float l = base[(size_t)s * stride + D + 1];
    const float M = wave_max(m);
    const float w = (M == -INFINITY || (int)threadIdx.x >= splits) ? 0.f : exp2f(m - M);
    const float L = wave_sum(w * l);
    if (threadIdx.x < SPL) wts[threadIdx.x] = w;
    if (threadIdx.x == 0) s_inv = L > 0.f ? 1.f / L : 0.f;
  }
  __syncthreads();
  float acc = 0.f;
#pragma unroll
  for (int s = 0; s < SPL; ++s) acc += wts[s] * o[s];
  if (threadIdx.x < D) out[((size_t)unit * G + h) * D + d] = acc * s_inv;
}

hipError_t launch_split_merge(const float* part, float* out, int64_t units, int splits, int hs,
                              int G, int D, int rs, hipStream_t st) {
  if (splits > MERGE_MAX_SPLITS || D > 256 || rs < D + 2) return hipErrorInvalidValue;
  const int threads = D < 64 ? 64 : D;
  const dim3 grid((unsigned)units, G);
  // the load slots per thread: the next power of two of the split count
  if (splits <= 8) k_split_merge<8><<<grid, threads, 0, st>>>(part, out, splits, hs, G, D, rs);
  else if (splits <= 16) k_split_merge<16><<<grid, threads, 0, st>>>(part, out, splits, hs, G, D, rs);
  else if (splits <= 32) k_split_merge<32><<<grid, threads, 0, st>>>(part, out, splits, hs, G, D, rs);
  else k_split_merge<64><<<grid, threads, 0, st>>>(part, out, splits, hs, G, D, rs);
  return hipGetLastError();
}

// ---------------------------------------------------------------------------
// Segmented path for many query rows over a long cache (causal prefill).
//
// Every (row, position) pair of the index sets reads that position's K and V
// pieces; with many rows the same K/V rows are read again and again, and the
// rate is set by where they come from.  A layer's K/V (128 MiB at 64K
// positions, 4 KV heads) fits the last-level cache but not an XCD's 4 MiB L2.
// The positions are therefore cut into segments of 2^shift positions (a KV
// head's K and V of one segment: 8 MiB at 16384 positions; shorter segments
// hit L2 more often but cost more partials, and 16384 measured fastest at
// 64K positions), and the work units (row, KV head, segment) are ordered
// segment-major with the KV head
// fastest at workgroup granularity: workgroup w takes KV head w % Hkv, and
// since the dispatcher deals workgroups round-robin over the 8 XCDs, each XCD
// sees one KV head (Hkv dividing 8) and, at any time, the segment the grid
// has reached: the gathers hit its L2.  Each unit attends over the index
// entries of its row that fall in its segment (a contiguous run, index rows
// being ascending) and writes an (O, m, l) partial; a row whose entries all
// fall in one segment (short rows, or rows that are not ascending, which are
// given one segment covering the whole row) writes its output directly.
// k_seg_merge combines the partials (log-sum-exp merge, SSA article section 6).

// bnd[row][j] (j = 0..nseg) = index entries of the row whose position lies
// below segment j's start; bnd[row][nseg] = the row's valid entries.  Needs
// the row ascending over its valid entries (positions in [0, L)) followed
// only by -1; any other row gets {0, kk, ..., kk}: one segment, whole row.
// One wave per row, one pass: the shape check and the bounds (staged in LDS
// until the shape is known) over SB_LD x 64 entries per round, all loads of a
// round issued first.  Rows of blocks on the block-union path are skipped:
// nothing reads their bounds.
constexpr int SB_LD = 8;
__global__ __launch_bounds__(256) void k_seg_bounds(const int32_t* __restrict__ idx,
                                                    int32_t* __restrict__ bnd, int64_t rows, int kk,
                                                    int64_t L, int shift, int nseg,
                                                    const int32_t* __restrict__ uflag, int64_t nblk) {
  __shared__ int32_t sb[4][ATT_SEG_MAX + 1];
  const int lane = threadIdx.x & 63, w = wave_id();
  const int64_t br = (int64_t)blockIdx.x * 4 + w;
  if (br >= rows) return;
  if (uflag && br / UA_R < nblk && uflag[br / UA_R]) return;
  const int32_t* ix = idx + br * kk;
  int32_t* bb = bnd + br * (nseg + 1);
  int32_t* s = sb[w];
  bool bad = false;
  int carry = -2;   // the previous entry (-2: before the first)
  int kcarry = -1;  // its segment key (-1 before entry 0)
  for (int c0 = 0; c0 <= kk; c0 += 64 * SB_LD) {
    int pv[SB_LD];
#pragma unroll
    for (int j = 0; j < SB_LD; ++j) {
      const int e = c0 + 64 * j + lane;
      pv[j] = e < kk ? ix[e] : -1;
    }
#pragma unroll
    for (int j = 0; j < SB_LD; ++j) {
      const int e = c0 + 64 * j + lane;
      const int p = pv[j];
      int prv = __shfl(p, (lane + 63) & 63, 64);
      if (lane == 0) prv = carry;
      carry = __shfl(p, 63, 64);
      const bool valid = p >= 0 && (int64_t)p < L;
      bool ok;
      if (prv == -2) ok = valid || p == -1;
      else if (prv == -1) ok = p == -1;
      else ok = p == -1 || (valid && p > prv);
      bad = bad || (e < kk && !ok);
      // entry e opens segments (key(e-1), key(e)]; key = segment of the
      // position, nseg for -1 and for the virtual entry kk
      const int key = (e >= kk || p < 0) ? nseg : min(p >> shift, nseg);
      int kprv = __shfl(key, (lane + 63) & 63, 64);
      if (lane == 0) kprv = kcarry;
      kcarry = __shfl(key, 63, 64);
      if (e <= kk)
        for (int jj = kprv + 1; jj <= key; ++jj) s[jj] = e;
    }
  }
  __builtin_amdgcn_wave_barrier();
  const bool rbad = __ballot(bad) != 0;
  for (int j = lane; j <= nseg; j += 64) bb[j] = rbad ? (j == 0 ? 0 : kk) : s[j];
}

template <int G>
__global__ __launch_bounds__(ATT_NW * 64) void k_sparse_attn_seg(
    const uint16_t* __restrict__ q, const uint16_t* __restrict__ k,
    const uint16_t* __restrict__ v, const int32_t* __restrict__ idx,
    const int32_t* __restrict__ bnd, float* __restrict__ out, float* __restrict__ part,
    int64_t rows, int64_t groups, int Lq, int Hq, int Hkv, int64_t L, int kk, float scale_log2,
    int nseg, const int32_t* __restrict__ uflag, int64_t nblk) {
  constexpr int D = ATT_D;
  __shared__ __attribute__((aligned(16))) char vta[ATT_NW][2][4][1024];
  __shared__ __attribute__((aligned(16))) char vtb[ATT_NW][2][4][1024];
  const int lane = threadIdx.x & 63, wid = wave_id();
  // workgroup -> (segment, group of ATT_NW rows, KV head), KV head fastest
  const int64_t wg = blockIdx.x;
  const int kvh = (int)(wg % Hkv);
  const int64_t t = wg / Hkv;
  const int seg = (int)(t / groups);
  const int64_t br = (t % groups) * ATT_NW + wid;  // b * Lq + r
  if (br >= rows) return;  // the whole wave; nothing below waits on other waves
  if (uflag && br / UA_R < nblk && uflag[br / UA_R]) return;  // a union block's row
  const int32_t* bb = bnd + br * (nseg + 1);
  const int e_begin = bb[seg], e_end = bb[seg + 1], n = bb[nseg];
  const bool whole = e_end - e_begin == n;  // the row's only non-empty segment
  if (e_begin == e_end && !(n == 0 && seg == 0)) return;
  const int64_t b = br / Lq;
  const int hl = lane & 15, kg = lane >> 4;
  const int32_t* ix = idx + br * kk;

  int pos[4];
  attn_entries(ix, e_begin, e_end > e_begin ? e_end : e_begin + 1, lane >> 2, pos);
  bf16x8 qf[4];
  attn_query<G>(q, br, Hq, kvh, hl, kg, qf);
  float m = -INFINITY, lsum = 0.f;
  floatx4 o[D / 16];
#pragma unroll
  for (int dt = 0; dt < D / 16; ++dt) o[dt] = floatx4{0.f, 0.f, 0.f, 0.f};
  const size_t row_stride = (size_t)Hkv * D;
  attn_span<G, true>(ix, e_begin, e_end, pos, qf, k + ((size_t)b * L * Hkv + kvh) * D,
               v + ((size_t)b * L * Hkv + kvh) * D, row_stride, L, scale_log2, vta[wid], vtb[wid], lane, m,
               lsum, o);

  if (hl >= G) return;
  if (whole) {
    const float inv = lsum > 0.f ? 1.f / lsum : 0.f;
    float* op = out + ((br * Hq) + kvh * G + hl) * D + kg * 4;
#pragma unroll
    for (int dt = 0; dt < D / 16; ++dt) *reinterpret_cast<floatx4*>(op + dt * 16) = o[dt] * inv;
  } else {
    float* pp = part + (((br * Hkv + kvh) * nseg + seg) * G + hl) * ATT_PS;
#pragma unroll
    for (int dt = 0; dt < D / 16; ++dt) *reinterpret_cast<floatx4*>(pp + dt * 16 + kg * 4) = o[dt];
    if (kg == 0) *reinterpret_cast<float2*>(pp + D) = float2{m, lsum};
  }
}

// Merge of the segment partials of one row (one workgroup; wave w takes KV
// heads w, w + 4, ...): O = sum_j 2^(m_j - M) O_j / sum_j 2^(m_j - M) l_j over
// the row's non-empty segments, M = max_j m_j.  Rows written directly by
// their only non-empty segment are skipped.
template <int G>
__global__ __launch_bounds__(256) void k_seg_merge(const float* __restrict__ part,
                                                   const int32_t* __restrict__ bnd,
                                                   float* __restrict__ out, int Hq, int Hkv,
                                                   int nseg, const int32_t* __restrict__ uflag,
                                                   int64_t nblk) {
  constexpr int D = ATT_D;
  const int lane = threadIdx.x & 63, wid = wave_id();
  const int64_t br = blockIdx.x;
  if (uflag && br / UA_R < nblk && uflag[br / UA_R]) return;  // written by the union path
  const int32_t* bb = bnd + br * (nseg + 1);
  const int n = bb[nseg];
  const int cnt = lane < nseg ? bb[lane + 1] - bb[lane] : 0;
  if (__ballot(lane < nseg && cnt == n) != 0) return;  // settled by one unit
  const uint64_t live = __ballot(cnt > 0);
  for (int h = wid; h < Hkv; h += 4) {
    const float* pb = part + (br * Hkv + h) * (int64_t)nseg * G * ATT_PS;
    for (int c = lane; c < G * (D / 4); c += 64) {
      const int hq = c / (D / 4), d4 = 4 * (c % (D / 4));
      float M = -INFINITY;
      for (uint64_t w = live; w; w &= w - 1) {
        const int j = __builtin_ctzll(w);
        M = fmaxf(M, pb[(j * G + hq) * ATT_PS + D]);
      }
      floatx4 acc = floatx4{0.f, 0.f, 0.f, 0.f};
      float lt = 0.f;
      for (uint64_t w = live; w; w &= w - 1) {
        const int j = __builtin_ctzll(w);
        const float* pr = pb + (j * G + hq) * ATT_PS;
        const float wt = exp2f(pr[D] - M);
        lt += wt * pr[D + 1];
        acc += wt * *reinterpret_cast<const floatx4*>(pr + d4);
      }
      const float inv = lt > 0.f ? 1.f / lt : 0.f;
      *reinterpret_cast<floatx4*>(out + ((br * Hq) + h * G + hq) * D + d4) = acc * inv;
    }
  }
}

// ---------------------------------------------------------------------------
// Block-union path for rows whose index sets overlap (neighbouring queries of
// a causal prefill).  The per-row paths read every (row, selected position)
// pair's K and V through the address unit; when the sets of neighbouring
// rows overlap, a block of UA_R consecutive rows can instead gather the union
// of their sets once into LDS and attend with a membership mask (a key of the
// union counts for a row only if that row selected it), so each shared
// position is fetched once per block instead of once per row, at the price of
// MFMA work on the union for every row of the block.  k_union_plan decides per
// block from the union's size; k_union_attn does the union blocks; the
// segment path skips their rows.
constexpr int UA_WIN = 16384;  // positions per membership window (16 rows x 2 KiB of bits)
constexpr int UA_CH = 64;      // union positions per chunk
constexpr int UA_LD = 16;      // index entries per thread and round of the membership pass
constexpr int UA_NBUF = 4;     // staging buffers of the chunk ring (unions over UA_SMALL positions)
constexpr int UA_SMALL = 2048; // unions up to this size: two staging buffers, two workgroups per CU
constexpr int UA_SET = UA_CH * 256 * 2;  // one staging buffer: the chunk's K and V tiles
// Union mode when the block's rows select each union position UA_SHARE x G / 8
// times on average (sum of n_r >= that x |U|).  A union chunk costs its
// workgroup G waves of MFMA and softmax work whoever selected its positions,
// while the per-row path pays per (row, position) pair at the address unit:
// measured on the 64K causal prefill, about 5 pairs per union position at 8
// heads per KV head break even.
#ifndef UA_SHARE
#define UA_SHARE 6
#endif

// Workgroup barrier that drains LDS operations but not the vector memory
// counter (a __syncthreads() would also wait for the LDS DMA in flight).
LCT_DEV void ua_barrier() {
  __builtin_amdgcn_s_waitcnt(WAITCNT_LGKM0);
  __asm__ __volatile__("" ::: "memory");
  __builtin_amdgcn_s_barrier();
  __asm__ __volatile__("" ::: "memory");
}

// One workgroup (256 threads, 16 per row) per block of UA_R rows.  The rows
// must lie in one batch entry, each ascending over its valid entries (in
// [0, L)) followed only by -1.  Their union is built window by window
// (UA_WIN positions: per-row membership bitmaps, then the window's union in
// ascending order with a 16-bit row mask per position) into the block's list
// of UA_UCAP slots (lpos, lmask).  flag[block] = the union's size if the
// block takes the union path -- at most UA_UCAP positions, each selected
// UA_SHARE x G / 8 times on average (sum of n_r >= that x |U|) -- else 0.
__global__ __launch_bounds__(256) void k_union_plan(const int32_t* __restrict__ idx, int64_t rows, int Lq,
                                                    int kk, int64_t L, int G, int32_t* __restrict__ flag,
                                                    int32_t* __restrict__ lpos, uint16_t* __restrict__ lmask) {
  constexpr int NT = 256, RT = NT / UA_R;                 // 16 threads per row
  constexpr int BPT = 32, NPASS = UA_WIN / (NT * BPT);    // union bits per thread and pass
  __shared__ __attribute__((aligned(16))) uint32_t mem[UA_R][UA_WIN / 32];
  __shared__ int32_t s_n[UA_R], s_cur[UA_R];
  __shared__ uint32_t s_bad;
  __shared__ int32_t s_pmax;
  __shared__ uint32_t scan[NT / 64 + 2];
  const int64_t blk = blockIdx.x;
  const int64_t r0 = blk * UA_R;
  const int rr = threadIdx.x / RT, t = threadIdx.x % RT;
  const int gsh = (threadIdx.x & 63) / RT * RT;  // the row's first lane in its wave
  const uint64_t gm = ((1ull << RT) - 1ull) << gsh;
  if (threadIdx.x == 0) {
    s_bad = (r0 + UA_R > rows || r0 / Lq != (r0 + UA_R - 1) / Lq) ? 1u : 0u;
    s_pmax = -1;
  }
  __syncthreads();
  if (s_bad) {
    if (threadIdx.x == 0) flag[blk] = 0;
    return;
  }
  const int32_t* ix = idx + (r0 + rr) * kk;
  // shape and length of each row, UA_LD entries per thread and round
  bool bad = false;
  int n = 0, pmax = -1;
  for (int e0 = 0; e0 < kk; e0 += RT * UA_LD) {
    int pv[UA_LD], pr[UA_LD];
#pragma unroll
    for (int j = 0; j < UA_LD; ++j) {
      const int e = e0 + t + RT * j;
      pv[j] = e < kk ? ix[e] : -1;
      pr[j] = e == 0 ? -2 : (e < kk ? ix[e - 1] : -1);
    }
#pragma unroll
    for (int j = 0; j < UA_LD; ++j) {
      const int p = pv[j], prv = pr[j];
      bool ok;
      if (prv == -2) ok = p == -1 || (p >= 0 && (int64_t)p < L);
      else if (prv == -1) ok = p == -1;
      else ok = p == -1 || (p > prv && (int64_t)p < L);
      bad = bad || !ok;
      n += p >= 0 ? 1 : 0;
      pmax = max(pmax, p);
    }
  }
#pragma unroll
  for (int d = 1; d < RT; d <<= 1) {
    n += __shfl_xor(n, d, 64);
    pmax = max(pmax, __shfl_xor(pmax, d, 64));
    const int ob = __shfl_xor((int)bad, d, 64);  // every lane takes part in the shuffle
    bad = bad || ob != 0;
  }
  if (t == 0) {
    s_n[rr] = n;
    s_cur[rr] = 0;
    if (bad) atomicOr(&s_bad, 1u);
    atomicMax(&s_pmax, pmax);
  }
  __syncthreads();
  int64_t sum_n = 0;
#pragma unroll
  for (int r = 0; r < UA_R; ++r) sum_n += s_n[r];
  // the largest union the block may take the path with
  const int64_t lim = min((int64_t)UA_UCAP, sum_n * 8 / ((int64_t)UA_SHARE * G));
  if (s_bad || lim <= 0) {
    if (threadIdx.x == 0) flag[blk] = 0;
    return;
  }
  const int plast = s_pmax;
  int32_t* lp = lpos + blk * UA_UCAP;
  uint16_t* lm = lmask + blk * UA_UCAP;
  uint32_t ucount = 0;  // union entries so far (block-uniform)
  for (int p0 = 0; p0 <= plast; p0 += UA_WIN) {
    for (int i = threadIdx.x; i < UA_R * (UA_WIN / 128); i += NT)
      reinterpret_cast<uint4*>(&mem[0][0])[i] = uint4{0u, 0u, 0u, 0u};
    __syncthreads();
    {
      const int nr = s_n[rr];
      int c0 = s_cur[rr];
      int taken = 0;
      bool more = true;
      while (more) {
        // UA_LD entries per thread per round, all loads issued before any is used
        int pv[UA_LD];
#pragma unroll
        for (int j = 0; j < UA_LD; ++j) {
          const int e = c0 + t + j * RT;
          pv[j] = e < nr ? ix[e] : INT32_MAX;
        }
        uint32_t cnt = 0;
#pragma unroll
        for (int j = 0; j < UA_LD; ++j) {
          const int p = pv[j];
          const bool in = p < p0 + UA_WIN;
          if (in) atomicOr(&mem[rr][(p - p0) >> 5], 1u << ((p - p0) & 31));
          // entries are ascending: the run in the window is a prefix
          cnt += (uint32_t)__popcll(__ballot(in) & gm);
        }
        taken += (int)cnt;
        more = cnt == (uint32_t)(RT * UA_LD);
        c0 += RT * UA_LD;
      }
      __syncthreads();
      if (t == 0) s_cur[rr] += taken;
    }
    __syncthreads();
    // the window's union appended in ascending order, BPT bits per thread
    // and pass
#pragma unroll
    for (int pass = 0; pass < NPASS; ++pass) {
      const int wd = pass * NT + (int)threadIdx.x;
      uint32_t rw[UA_R], ubits = 0;
#pragma unroll
      for (int r = 0; r < UA_R; ++r) {
        rw[r] = mem[r][wd];
        ubits |= rw[r];
      }
      uint32_t nu;
      uint32_t o2 = ucount + block_excl_scan<NT>(__popc(ubits), scan, nu);
      if (ucount + nu > (uint64_t)lim) {  // uniform: too large a union
        if (threadIdx.x == 0) flag[blk] = 0;
        return;
      }
      uint32_t x = ubits;
      while (x) {
        const int bbit = __ffs(x) - 1;
        x &= x - 1;
        uint32_t msk = 0;
#pragma unroll
        for (int r = 0; r < UA_R; ++r) msk |= ((rw[r] >> bbit) & 1u) << r;
        lp[o2] = p0 + wd * 32 + bbit;
        lm[o2] = (uint16_t)msk;
        ++o2;
      }
      ucount += nu;
    }
    __syncthreads();  // the bitmaps are read before the next window clears them
  }
  if (threadIdx.x == 0) flag[blk] = (int32_t)ucount;
}

// P^T V^T product of one half (two 16-token blocks) of a landed V tile.
LCT_DEV void ua_pv_half(const char (&vh)[2][4][1024], const AttnLanes& a, const __bf16 (&pw)[4][4], int h,
                        floatx4 (&o)[ATT_D / 16], floatx4& lacc) {
  constexpr int D = ATT_D;
  bf16x8 ones;
#pragma unroll
  for (int i = 0; i < 8; ++i) ones[i] = (__bf16)1.0f;
  // the 16 transposed reads in one asm block with their wait: the compiler
  // cannot tell these LDS reads from the next chunk's DMA into the other
  // buffer set and would otherwise drain that DMA first (the chunk's own DMA
  // was waited for before the barrier that precedes this)
  short4v r[16];
  const uint32_t b0 = (uint32_t)(uintptr_t)(const __attribute__((address_space(3))) char*)&vh[0][0][a.tr0];
  const uint32_t b1 = (uint32_t)(uintptr_t)(const __attribute__((address_space(3))) char*)&vh[0][0][a.tr1];
  __asm__ volatile(
      "ds_read_b64_tr_b16 %0, %16 offset:0\n\t"
      "ds_read_b64_tr_b16 %1, %16 offset:4096\n\t"
      "ds_read_b64_tr_b16 %2, %17 offset:0\n\t"
      "ds_read_b64_tr_b16 %3, %17 offset:4096\n\t"
      "ds_read_b64_tr_b16 %4, %16 offset:1024\n\t"
      "ds_read_b64_tr_b16 %5, %16 offset:5120\n\t"
      "ds_read_b64_tr_b16 %6, %17 offset:1024\n\t"
      "ds_read_b64_tr_b16 %7, %17 offset:5120\n\t"
      "ds_read_b64_tr_b16 %8, %16 offset:2048\n\t"
      "ds_read_b64_tr_b16 %9, %16 offset:6144\n\t"
      "ds_read_b64_tr_b16 %10, %17 offset:2048\n\t"
      "ds_read_b64_tr_b16 %11, %17 offset:6144\n\t"
      "ds_read_b64_tr_b16 %12, %16 offset:3072\n\t"
      "ds_read_b64_tr_b16 %13, %16 offset:7168\n\t"
      "ds_read_b64_tr_b16 %14, %17 offset:3072\n\t"
      "ds_read_b64_tr_b16 %15, %17 offset:7168\n\t"
      "s_waitcnt lgkmcnt(0)"
      : "=&v"(r[0]), "=&v"(r[1]), "=&v"(r[2]), "=&v"(r[3]), "=&v"(r[4]), "=&v"(r[5]), "=&v"(r[6]),
        "=&v"(r[7]), "=&v"(r[8]), "=&v"(r[9]), "=&v"(r[10]), "=&v"(r[11]), "=&v"(r[12]), "=&v"(r[13]),
        "=&v"(r[14]), "=&v"(r[15])
      : "v"(b0), "v"(b1)
      : "memory");
  static_assert(sizeof(vh[0]) == 4096 && sizeof(vh[0][0]) == 1024, "offsets above: block 4096, slice 1024");
  bf16x8 vv[D / 16];
#pragma unroll
  for (int dt = 0; dt < D / 16; ++dt)
    vv[dt] = __builtin_bit_cast(bf16x8, __builtin_shufflevector(r[2 * dt], r[2 * dt + 1], 0, 1, 2, 3, 4, 5, 6, 7));
  bf16x8 pf;
#pragma unroll
  for (int e = 0; e < 4; ++e) {
    pf[e] = pw[2 * h][e];
    pf[4 + e] = pw[2 * h + 1][e];
  }
#pragma unroll
  for (int dt = 0; dt < D / 16; ++dt) o[dt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(vv[dt], pf, o[dt], 0, 0, 0);
  lacc = __builtin_amdgcn_mfma_f32_16x16x32_bf16(ones, pf, lacc, 0, 0, 0);
}

// Online-softmax attention of one wave's 16 columns over one landed chunk of
// 64 union positions (base: the chunk's first union slot): S^T = K Q^T from
// the swizzled K tile, the membership mask of each column's row (wrm: the
// wave's row bits in both 16-bit halves), weights, O^T += V^T P^T.
constexpr float UA_MSLACK = 8.f;  // log2 of the largest weight before a rescale
LCT_DEV void ua_chunk(int base, const char (&kt)[UA_CH * 256], const char (&va)[2][4][1024],
                      const char (&vb)[2][4][1024], const uint16_t* umask, const AttnLanes& a,
                      const bf16x8 (&qf)[4], int rbit, uint32_t wrm, float scale_log2, float& m,
                      floatx4& lacc, floatx4 (&o)[ATT_D / 16]) {
  constexpr int D = ATT_D;
  const int hl = a.hl, kg = a.kg;
  // K: lane (hl, kg) reads 16-byte chunk st*4 + kg of token 16j + hl, stored
  // as chunk (st*4 + kg) ^ hl = (st ^ (hl / 4))*4 + (kg ^ (hl % 4)).  The reads
  // are written out with their wait, two token blocks per asm block: the
  // compiler cannot tell them from the DMA into the other staging buffers and
  // would otherwise drain that DMA first.
  floatx4 sacc[4];
  const uint32_t kb = (uint32_t)(uintptr_t)(const __attribute__((address_space(3))) char*)&kt[0] + hl * 256 +
                      ((kg ^ (hl & 3)) << 4);
  const uint32_t k0 = kb + ((0 ^ (hl >> 2)) << 6), k1 = kb + ((1 ^ (hl >> 2)) << 6);
  const uint32_t k2 = kb + ((2 ^ (hl >> 2)) << 6), k3 = kb + ((3 ^ (hl >> 2)) << 6);
  static_assert(sizeof(kt) == 4 * 4096, "K tile: four 16-token blocks of 4096 bytes");
#pragma unroll
  for (int jp = 0; jp < 2; ++jp) {
    intx4 r[8];  // [token block jj][st]
    if (jp == 0)
      __asm__ volatile(
          "ds_read_b128 %0, %8 offset:0\n\t"
          "ds_read_b128 %1, %9 offset:0\n\t"
          "ds_read_b128 %2, %10 offset:0\n\t"
          "ds_read_b128 %3, %11 offset:0\n\t"
          "ds_read_b128 %4, %8 offset:4096\n\t"
          "ds_read_b128 %5, %9 offset:4096\n\t"
          "ds_read_b128 %6, %10 offset:4096\n\t"
          "ds_read_b128 %7, %11 offset:4096\n\t"
          "s_waitcnt lgkmcnt(0)"
          : "=&v"(r[0]), "=&v"(r[1]), "=&v"(r[2]), "=&v"(r[3]), "=&v"(r[4]), "=&v"(r[5]), "=&v"(r[6]),
            "=&v"(r[7])
          : "v"(k0), "v"(k1), "v"(k2), "v"(k3)
          : "memory");
    else
      __asm__ volatile(
          "ds_read_b128 %0, %8 offset:8192\n\t"
          "ds_read_b128 %1, %9 offset:8192\n\t"
          "ds_read_b128 %2, %10 offset:8192\n\t"
          "ds_read_b128 %3, %11 offset:8192\n\t"
          "ds_read_b128 %4, %8 offset:12288\n\t"
          "ds_read_b128 %5, %9 offset:12288\n\t"
          "ds_read_b128 %6, %10 offset:12288\n\t"
          "ds_read_b128 %7, %11 offset:12288\n\t"
          "s_waitcnt lgkmcnt(0)"
          : "=&v"(r[0]), "=&v"(r[1]), "=&v"(r[2]), "=&v"(r[3]), "=&v"(r[4]), "=&v"(r[5]), "=&v"(r[6]),
            "=&v"(r[7])
          : "v"(k0), "v"(k1), "v"(k2), "v"(k3)
          : "memory");
#pragma unroll
    for (int jj = 0; jj < 2; ++jj) {
      const int j = 2 * jp + jj;
      sacc[j] = floatx4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int st = 0; st < 4; ++st)
        sacc[j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, r[4 * jj + st]), qf[st],
                                                          sacc[j], 0, 0, 0);
    }
  }
  // membership of this lane's tokens 16j + 4kg + e (masks of tokens e = 0..3
  // in the halves of w2[j]) for its column's row; scores of other tokens
  // drop to -inf.  A chunk that every row of the wave takes whole skips the
  // per-token test (wave-uniform).
  uint2 w2[4];
  bool whole = true;
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    w2[j] = *reinterpret_cast<const uint2*>(&umask[base + 16 * j + 4 * kg]);  // padding: 0
    whole = whole && (w2[j].x & wrm) == wrm && (w2[j].y & wrm) == wrm;
  }
  float sm[4][4];
  if (__ballot(!whole) == 0) {
#pragma unroll
    for (int j = 0; j < 4; ++j)
#pragma unroll
      for (int e = 0; e < 4; ++e) sm[j][e] = sacc[j][e];
  } else {
#pragma unroll
    for (int j = 0; j < 4; ++j)
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const uint32_t w = e < 2 ? w2[j].x : w2[j].y;
        sm[j][e] = ((w >> (rbit + 16 * (e & 1))) & 1u) ? sacc[j][e] : -INFINITY;
      }
  }
  float tmax = -INFINITY;
#pragma unroll
  for (int j = 0; j < 4; ++j)
#pragma unroll
    for (int e = 0; e < 4; ++e) tmax = fmaxf(tmax, sm[j][e]);
  tmax = fmaxf(tmax, __shfl_xor(tmax, 16, 64));
  tmax = fmaxf(tmax, __shfl_xor(tmax, 32, 64));
  const float tm = tmax * scale_log2;
  // The reference max m moves (and O, l are rescaled) only when a column's
  // scores pass it by more than UA_MSLACK: the weights stay below
  // 2^UA_MSLACK, and numerator and denominator share the reference.
  if (__ballot(tm > m + UA_MSLACK) != 0) {
    const float mnew = fmaxf(m, tm);
    const float alpha = mnew == -INFINITY ? 1.f : __builtin_amdgcn_exp2f(m - mnew);
#pragma unroll
    for (int dt = 0; dt < D / 16; ++dt) o[dt] = o[dt] * alpha;
    lacc = lacc * alpha;
    m = mnew;
  }
  const float mref = m == -INFINITY ? 0.f : m;
  __bf16 pw[4][4];
#pragma unroll
  for (int j = 0; j < 4; ++j)
#pragma unroll
    for (int e = 0; e < 4; ++e) pw[j][e] = (__bf16)__builtin_amdgcn_exp2f(fmaf(sm[j][e], scale_log2, -mref));
  ua_pv_half(va, a, pw, 0, o, lacc);
  ua_pv_half(vb, a, pw, 1, o, lacc);
}

// Union attention of one (block, KV head) in union mode; G waves, wave w
// takes rows w*(16/G) .. (w+1)*(16/G) - 1 of the block with their G heads as
// its 16 MFMA columns (column c: row c / G, head c % G).
// Phase 1 builds the block's whole union: per window of UA_WIN positions, each
// row's entries in the window (a contiguous run of its ascending list, from a
// cursor) set its membership bits; the window's union is appended to a list of
// positions + 16-bit row masks (at most UA_UCAP entries: the plan flags no
// larger union).  The bitmaps live in the first staging buffer, free then.
// Phase 2 gathers chunks of 64 union positions into a ring of NBUF staging
// buffers (NBUF - 1 chunks in flight while one is attended) and every wave
// attends each chunk with its rows' masks.  K is stored 16-byte-chunk swizzled
// (chunk s of token t at s ^ (t % 16)), so the A-operand reads (16 tokens of
// one chunk) fall on distinct banks; V uses the layout of the per-row path
// for the transposed reads.
template <int G, bool SMALL>
__global__ __launch_bounds__(G * 64) __attribute__((amdgpu_waves_per_eu(SMALL && G == 8 ? 4 : 1))) void k_union_attn(
    const uint16_t* __restrict__ q, const uint16_t* __restrict__ k, const uint16_t* __restrict__ v,
    const int32_t* __restrict__ flag, const int32_t* __restrict__ lpos, const uint16_t* __restrict__ lmask,
    float* __restrict__ out, int Lq, int Hq, int Hkv, int64_t L, float scale_log2) {
  constexpr int D = ATT_D;
  constexpr int NT = G * 64;
  constexpr int RW = UA_R / G;  // rows per wave
  // SMALL: unions of up to UA_SMALL positions with two staging buffers (one
  // chunk in flight; 76 KiB of LDS, so two workgroups share a CU and run out
  // of step); else the larger unions with the deeper ring (152 KiB, one per CU)
  constexpr int NBUF = SMALL ? 2 : UA_NBUF;
  constexpr int CAP = SMALL ? UA_SMALL : UA_UCAP;
  static_assert(G >= 4 && G <= 16 && UA_R % G == 0, "union path for 4 to 16 heads per KV head");
  static_assert(CAP % UA_CH == 0 && UA_SMALL <= UA_UCAP, "the last chunk's padding stays in the list");
  __shared__ int32_t upos[CAP];
  __shared__ __attribute__((aligned(8))) uint16_t umask[CAP];
  __shared__ __attribute__((aligned(16))) char stage[NBUF][UA_SET];
  const int64_t blk = blockIdx.x / Hkv;
  const int kvh = (int)(blockIdx.x % Hkv);
  const int nu = min(flag[blk], UA_UCAP);
  // uniform: the segment path takes blocks with no union, each instance its sizes
  if (nu <= 0 || (SMALL ? nu > UA_SMALL : nu <= UA_SMALL)) return;
  const int lane = threadIdx.x & 63, wid = wave_id();
  const int64_t r0 = blk * UA_R;
  const int64_t b = r0 / Lq;
  const int hl = lane & 15, kg = lane >> 4;
  const AttnLanes a = attn_lanes(lane);
  // this wave's columns: row r0 + wid*RW + hl / G, head kvh*G + hl % G
  const int rbit = wid * RW + hl / G;
  const uint32_t wrm = (((1u << RW) - 1u) << (wid * RW)) * 0x10001u;
  bf16x8 qf[4];
  {
    const int64_t row = r0 + rbit;
    const uint16_t* qp = q + ((row * Hq) + kvh * G + hl % G) * D + kg * 8;
#pragma unroll
    for (int st = 0; st < 4; ++st) qf[st] = *reinterpret_cast<const bf16x8*>(qp + st * 32);
  }
  // ---- the block's union list (k_union_plan), padded to whole chunks with
  // masks no row takes
  const int nch = (nu + UA_CH - 1) / UA_CH;
  {
    const int32_t* lp = lpos + blk * UA_UCAP;
    const uint16_t* lm = lmask + blk * UA_UCAP;
    for (int i = threadIdx.x; i < nch * UA_CH; i += NT) {
      upos[i] = i < nu ? lp[i] : 0;
      umask[i] = i < nu ? lm[i] : (uint16_t)0;
    }
  }
  __syncthreads();

  // ---- phase 2: the chunks, NBUF - 1 in flight
  const int row_bytes = Hkv * D * 2;
  const __amdgpu_buffer_rsrc_t krs = make_rsrc(k + (size_t)b * L * Hkv * D + kvh * D, L * (int64_t)row_bytes);
  const __amdgpu_buffer_rsrc_t vrs = make_rsrc(v + (size_t)b * L * Hkv * D + kvh * D, L * (int64_t)row_bytes);
  float m = -INFINITY;
  floatx4 lacc = floatx4{0.f, 0.f, 0.f, 0.f};
  floatx4 o[D / 16];
#pragma unroll
  for (int dt = 0; dt < D / 16; ++dt) o[dt] = floatx4{0.f, 0.f, 0.f, 0.f};
  // staging buffer: K tile (64 x 256 B, swizzled), then the two V halves
  auto kt_of = [&](int sb) -> char (&)[UA_CH * 256] {
    return *reinterpret_cast<char (*)[UA_CH * 256]>(&stage[sb][0]);
  };
  auto va_of = [&](int sb) -> char (&)[2][4][1024] {
    return *reinterpret_cast<char (*)[2][4][1024]>(&stage[sb][UA_CH * 256]);
  };
  auto vb_of = [&](int sb) -> char (&)[2][4][1024] {
    return *reinterpret_cast<char (*)[2][4][1024]>(&stage[sb][UA_CH * 256 + 8192]);
  };
  // DMA of chunk c (union positions c*64 ..) into staging buffer c % NBUF:
  // 16 K and 16 V instructions per chunk, 32 / G per wave (i = wid + ii * G)
  auto issue = [&](int c) {
    const int sb = c % NBUF;
    char* kt = &kt_of(sb)[0];
    char (*va)[4][1024] = va_of(sb);
    char (*vb)[4][1024] = vb_of(sb);
    const int base = c * UA_CH;
#pragma unroll
    for (int ii = 0; ii < 32 / G; ++ii) {
      const int i = wid + ii * G;
      if (i < 16) {
        const int tok = 4 * i + (lane >> 4), s = lane & 15;
        const int up = base + tok < nu ? base + tok : base;
        const int roff = upos[up] * row_bytes + ((s ^ (tok & 15)) << 4);
        __builtin_amdgcn_raw_ptr_buffer_load_lds(krs, (lds_void*)(kt + i * 1024), 16, roff, 0, 0, 0);
      } else {
        const int j = (i - 16) >> 2, st = (i - 16) & 3;
        const int tok = 16 * j + a.tk;
        const int up = base + tok < nu ? base + tok : base;
        const int roff = upos[up] * row_bytes + st * 64 + a.cv * 16;
        char* dst = j < 2 ? &va[j][st][0] : &vb[j - 2][st][0];
        __builtin_amdgcn_raw_ptr_buffer_load_lds(vrs, (lds_void*)dst, 16, roff, 0, 0, 0);
      }
    }
  };
  constexpr int NDMA = 32 / G;  // DMA instructions per wave and chunk
  static_assert(NBUF >= 2 && (NBUF - 2) * NDMA <= 63, "vector memory counter range");
  // Plain barriers (ua_barrier): each wave waits for its own DMA with an
  // explicit count, so the barrier need not drain the DMA in flight.
  __builtin_amdgcn_s_waitcnt(WAITCNT_VM0);
#pragma unroll
  for (int c = 0; c < NBUF - 1; ++c)
    if (c < nch) issue(c);
  for (int c = 0; c < nch; ++c) {
    // this wave's DMA of chunk c has landed once at most min(NBUF - 2,
    // nch - 1 - c) later chunks are outstanding
    const int later = min(NBUF - 2, nch - 1 - c);
    if (later >= 2) __builtin_amdgcn_s_waitcnt(waitcnt_vm(2 * NDMA));
    else if (later == 1) __builtin_amdgcn_s_waitcnt(waitcnt_vm(NDMA));
    else __builtin_amdgcn_s_waitcnt(WAITCNT_VM0);
    // every wave's DMA of chunk c has landed, and every wave is done with
    // chunk c - 1, whose buffer takes chunk c + NBUF - 1
    ua_barrier();
    if (c + NBUF - 1 < nch) issue(c + NBUF - 1);
    const int sb = c % NBUF;
    ua_chunk(c * UA_CH, kt_of(sb), va_of(sb), vb_of(sb), umask, a, qf, rbit, wrm, scale_log2, m, lacc, o);
  }
  // o[dt][e] = O^T[d = 16dt + 4kg + e][column hl]; every row of lacc holds
  // the column's denominator
  const float inv = lacc[0] > 0.f ? 1.f / lacc[0] : 0.f;
  const int64_t row = r0 + rbit;
  float* op = out + ((row * Hq) + kvh * G + hl % G) * D + kg * 4;
#pragma unroll
  for (int dt = 0; dt < D / 16; ++dt) *reinterpret_cast<floatx4*>(op + dt * 16) = o[dt] * inv;
}

static hipError_t launch_sparse_attn_seg(const uint16_t* q, const uint16_t* k, const uint16_t* v,
                                         const int32_t* idx, float* out, int B, int Lq, int Hq,
                                         int Hkv, int64_t L, int kk, float sl2, const AttnPlan& plan,
                                         float* ws, hipStream_t st, bool reuse) {
  const int G = Hq / Hkv;
  const int64_t rows = (int64_t)B * Lq;
  const int64_t groups = (rows + ATT_NW - 1) / ATT_NW;
  float* part = ws;
  int32_t* bnd = reinterpret_cast<int32_t*>(reinterpret_cast<char*>(ws) + attn_bnd_offset(plan));
  int32_t* uflag = plan.ua_blocks > 0 ? reinterpret_cast<int32_t*>(reinterpret_cast<char*>(ws) + attn_ua_offset(plan))
                                      : nullptr;
  const int64_t nblk = plan.ua_blocks;
  int32_t* lpos = plan.ua_blocks > 0 ? reinterpret_cast<int32_t*>(reinterpret_cast<char*>(ws) + attn_ul_offset(plan))
                                      : nullptr;
  uint16_t* lmask = plan.ua_blocks > 0 ? reinterpret_cast<uint16_t*>(lpos + plan.ua_blocks * UA_UCAP) : nullptr;
  // what depends only on the index (block decisions, union lists, segment
  // bounds) is kept from the previous call on the same index when `reuse`
  if (!reuse) {
    if (nblk > 0) k_union_plan<<<dim3((unsigned)nblk), 256, 0, st>>>(idx, rows, Lq, kk, L, G, uflag, lpos, lmask);
    k_seg_bounds<<<dim3((unsigned)((rows + 3) / 4)), 256, 0, st>>>(idx, bnd, rows, kk, L, plan.seg_shift,
                                                                    plan.nseg, uflag, nblk);
  }
  if (nblk > 0) {
    // unions up to UA_SMALL positions, then the larger ones
    const dim3 ug((unsigned)(nblk * Hkv));
#define LCT_UA(GG, SM) \
  k_union_attn<GG, SM><<<ug, GG * 64, 0, st>>>(q, k, v, uflag, lpos, lmask, out, Lq, Hq, Hkv, L, sl2)
    switch (G) {
      case 4: LCT_UA(4, true); LCT_UA(4, false); break;
      case 8: LCT_UA(8, true); LCT_UA(8, false); break;
      case 16: LCT_UA(16, true); LCT_UA(16, false); break;
      default: return hipErrorInvalidValue;
    }
#undef LCT_UA
  }
  const int64_t wgs = (int64_t)plan.nseg * groups * Hkv;
  if (wgs >= ((int64_t)1 << 32)) return hipErrorInvalidValue;
#define LCT_ATT(GG)                                                                                \
  k_sparse_attn_seg<GG><<<dim3((unsigned)wgs), ATT_NW * 64, 0, st>>>(q, k, v, idx, bnd, out, part, rows, \
                                                                     groups, Lq, Hq, Hkv, L, kk, sl2,  \
                                                                     plan.nseg, uflag, nblk);          \
  k_seg_merge<GG><<<dim3((unsigned)rows), 256, 0, st>>>(part, bnd, out, Hq, Hkv, plan.nseg, uflag, nblk)
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

hipError_t launch_sparse_attn(const uint16_t* q, const uint16_t* k, const uint16_t* v,
                              const int32_t* idx, float* out, int B, int Lq, int Hq, int Hkv,
                              int64_t L, int kk, float scale, const AttnPlan& plan,
                              float* partials, hipStream_t st, bool reuse_index_work) {
  const int G = Hq / Hkv;
  const float sl2 = scale * LOG2E;
  if (plan.nseg > 0) return launch_sparse_attn_seg(q, k, v, idx, out, B, Lq, Hq, Hkv, L, kk, sl2, plan,
                                                   partials, st, reuse_index_work);
  const int64_t units = (int64_t)B * Lq * Hkv;
  const int64_t waves = units * plan.splits;
  const dim3 grid((unsigned)((waves + ATT_NW - 1) / ATT_NW));
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
