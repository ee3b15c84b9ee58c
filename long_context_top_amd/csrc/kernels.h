// Internal launch interface between the C-ABI layer and the gfx950 kernels.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace lct {

// ---------------------------------------------------------------- top-k ----
constexpr int TOPK_NB_LOG2 = 8;                 // bins of the multi-workgroup histogram
constexpr int TOPK_NB = 1 << TOPK_NB_LOG2;
constexpr int TOPK_CAP = 4096;                  // threshold-bin candidates resolved in LDS
constexpr int TOPK_K2_TILE = 256 * 16;          // keys per histogram workgroup
constexpr int TOPK_K3_THREADS = 512;
constexpr int TOPK_K3_TILE = TOPK_K3_THREADS * 8;   // positions per emit workgroup
constexpr int TOPK_MM_TILE = 256 * 16;          // keys per min/max workgroup
constexpr int TOPK_K4_TILE = 1024 * 32;         // positions per finalize workgroup
constexpr int TOPK_MULTI_MAX_ROWS = 64;
constexpr uint32_t TOPK_ALL = 0xFFFFFFFFu;       // "every valid position is chosen"

// Rows up to this length use the one-workgroup-per-row kernel's LDS bitmap.
constexpr int64_t TOPK_ROW_MAX_N = (int64_t)1 << 18;

struct TopkRowState {
  uint32_t lo, shift, tb, need;
  uint32_t cand_count, cand_fill, nvalid, kk;
  uint32_t pad[8];
};
static_assert(sizeof(TopkRowState) == 64, "row state is one 64-byte line");

// Workspace carve-up of the multi-workgroup select for `rows` rows of length n
// whose min/max partials come from `t1` producer tiles per row.
struct TopkMultiLayout {
  size_t state, mm, hist, cands, bitmap, tilecnt, total;
  int t1, t2, t3, t4;
  int64_t k2_tile;  // keys per histogram tile
  int64_t nwords;
};
TopkMultiLayout topk_multi_layout(int rows, int64_t n, int t1);

// Producer of the multi-workgroup select for existing score rows: per-tile
// (min, max) key partials [rows][t1] and a cleared candidate counter.  Row
// r's valid length is valid_len[r / vl_div] (null: n).
hipError_t launch_topk_minmax(const void* scores, int dtype, int rows, int64_t n, int64_t ld,
                              const int32_t* valid_len, int vl_div, char* ws,
                              const TopkMultiLayout& lay, hipStream_t s);
// The rest of the multi-workgroup select: histogram, emit, finalize (three
// kernels; kernel boundaries carry the hand-offs).
hipError_t launch_topk_select_multi(const void* scores, int dtype, int32_t* idx, int rows,
                                    int64_t n, int64_t ld, int k, const int32_t* valid_len,
                                    int vl_div, char* ws, const TopkMultiLayout& lay,
                                    hipStream_t s);
// One workgroup per row.  Row r's valid length is min(n, causal_pos0 + r + 1)
// when causal_pos0 >= 0, else valid_len[r / vl_div] (or n when valid_len is null).
hipError_t launch_topk_rows(const void* scores, int dtype, int32_t* idx, int rows, int64_t n,
                            int64_t ld, int k, const int32_t* valid_len, int vl_div,
                            int64_t causal_pos0, hipStream_t s);

// ------------------------------------------------------------- indexer ----
// Streaming decode scorer; optionally writes (min,max) partials + clears the
// row states of a following multi-workgroup select (mm/state may be null).
// One workgroup per tile of SCORE_TILE positions of a (batch, query chunk)
// row; the select reads `tiles` (min, max) partials per row.
constexpr int SCORE_TILE = 512;  // positions per workgroup (4 waves x 2 rounds x 64)
struct ScorePlan {
  int qc, nqc;  // query rows per workgroup, query chunks per batch entry
  int tiles;    // tiles (and partials) per row
};
ScorePlan score_plan(int B, int Lq, int64_t L, int HD);
hipError_t launch_idx_score_stream(const int8_t* q, const int8_t* k, int32_t* s, int B, int Lq,
                                   int64_t L, int HD, int64_t q_pos0, uint32_t* mm,
                                   TopkRowState* state, uint32_t* hist,
                                   const int32_t* valid_len, hipStream_t st);
// Causal/prefill scorer on int8 MFMA: rows [r0, r0+R) of q against all L keys.
hipError_t launch_idx_score_mfma(const int8_t* q, const int8_t* k, int32_t* s, int B, int Lq,
                                 int64_t L, int HD, int64_t q_pos0, hipStream_t st);

// -------------------------------------------------------------- gather ----
constexpr int MERGE_MAX_SPLITS = 64;  // split partials per unit the merge kernel combines
struct AttnPlan {
  int splits;       // waves per (b, row, kv head)
  int per_split;    // index entries per wave (a multiple of 32)
  size_t part_bytes;
  int nseg;         // > 0: segmented path with nseg position segments of 2^seg_shift
  int seg_shift;
  size_t bnd_bytes;  // segmented path: per-row segment bounds after the partials
  int64_t ua_blocks;  // segmented path: row blocks that may take the block-union path
                      // (an int32 flag each after the bounds, then each block's
                      // union list: UA_UCAP int32 positions, then UA_UCAP uint16
                      // row masks per block)
};
constexpr int UA_UCAP = 4096;  // largest union (positions) of a block on the block-union path
AttnPlan attn_plan(int B, int Lq, int Hq, int Hkv, int kk, int64_t L);
inline size_t attn_bnd_offset(const AttnPlan& p) { return (p.part_bytes + 255) / 256 * 256; }
inline size_t attn_ua_offset(const AttnPlan& p) { return (attn_bnd_offset(p) + p.bnd_bytes + 255) / 256 * 256; }
inline size_t attn_ul_offset(const AttnPlan& p) {
  return (attn_ua_offset(p) + (size_t)p.ua_blocks * sizeof(int32_t) + 255) / 256 * 256;
}
inline size_t attn_ws_bytes(const AttnPlan& p) {
  if (p.nseg == 0) return p.part_bytes;
  return p.ua_blocks > 0 ? attn_ul_offset(p) + (size_t)p.ua_blocks * UA_UCAP * (sizeof(int32_t) + sizeof(uint16_t))
                         : attn_bnd_offset(p) + p.bnd_bytes;
}
// With plan.splits > 1 the kernel writes (O, m, l) partials and a merge
// kernel combines them (log-sum-exp merge).
// reuse_index_work: the workspace already holds what the segmented path
// derives from this index (block-union decisions and lists, segment bounds),
// left by the previous call on the same index, shapes and workspace.
hipError_t launch_sparse_attn(const uint16_t* q, const uint16_t* k, const uint16_t* v,
                              const int32_t* idx, float* out, int B, int Lq, int Hq, int Hkv,
                              int64_t L, int kk, float scale, const AttnPlan& plan,
                              float* partials, hipStream_t st, bool reuse_index_work = false);
// Merge of split partials: part[unit][split][hs][rs] (O[D], m, l, pad) ->
// out[(unit * G + h) * D + d] for h < G.
hipError_t launch_split_merge(const float* part, float* out, int64_t units, int splits, int hs,
                              int G, int D, int rs, hipStream_t st);

// ----------------------------------------------------------------- GSA ----
hipError_t launch_gist_score(const uint16_t* q, const uint16_t* gk, float* s, int BH, int64_t Nc,
                             int D, hipStream_t st);
struct GsaPlan {
  int splits;
  size_t part_bytes;
};
GsaPlan gsa_plan(int BH, int kc, int tail_len);
// Hierarchical routing: one workgroup per (batch, head); limits on the
// meta-gists, the candidate chunks (km * group), km and kc.
constexpr int HG_NT = 256;
constexpr int HG_MAX_ITEMS = 4096;
constexpr int HG_MAX_KM = 64;
constexpr int HG_MAX_KC = 1024;
// GSA prefill under the gist mask: raw queries/outputs [BH, Nc*16, D], gist
// queries/outputs [BH, Nc, D], raw K/V [BH, raw_cap, D], gist K/V [BH, Nc, D].
hipError_t launch_gsa_prefill(const uint16_t* qr, const uint16_t* qg, const uint16_t* rk, const uint16_t* rv,
                              const uint16_t* gk, const uint16_t* gv, float* outr, float* outg, int BH,
                              int64_t Nc, int64_t raw_cap, float scale, hipStream_t st);
hipError_t launch_hgsa_route(const uint16_t* q, const uint16_t* mk, const uint16_t* gk, float* gscores,
                             int32_t* cidx, int BH, int64_t Nc, int Nm, int group, int km, int kc,
                             hipStream_t st);
hipError_t launch_gsa_attn(const uint16_t* q, const uint16_t* rk, const uint16_t* rv,
                           const uint16_t* gv, const float* gscores, const int32_t* cidx,
                           float* out, int BH, int64_t Nc, int64_t raw_cap, int kc, int tail_len,
                           float scale, const GsaPlan& plan, float* partials, hipStream_t st);

// ------------------------------------------------------------ prefill ----
// Fused causal prefill score + select (B = 1, Lq = L, HD = 256, L <= 2^16,
// k <= 2048): scores are filtered to per-row candidate lists (PF_CROW
// entries), an exact select runs on those, rows with few earlier positions
// take one plain block, and rows the lists cannot settle are listed on the
// device and taken by a fixed grid of whole-row selects (PF_FB_GRID
// workgroups), so nothing is read back to the host.  n_failed (device int32,
// may be null) receives the number of such rows.
constexpr int PF_CROW = 5120;
constexpr int PF_META = 4;  // words per row: candidates, overflow flag, threshold
constexpr int PF_FB_GRID = 256;
constexpr int64_t PF_MAX_L = (int64_t)1 << 16;
constexpr int PF_MAX_K = 2048;
struct PfLayout {
  size_t list, meta, fails, short_scores, fb_scores, total;
};
size_t pf_workspace_layout(int64_t L, int HD, int kk, PfLayout* lay);
hipError_t launch_pf_fused(const int8_t* q, const int8_t* k, int64_t L, int HD, int kk,
                           int32_t* idx, char* ws, hipStream_t st, int32_t* n_failed);

// --------------------------------------------------------------- misc ----
hipError_t launch_zero(void* p, size_t bytes, hipStream_t st);

}  // namespace lct
