/*
 * lct.h -- routed top-k sparse attention with a cross-layer shared index,
 * native to AMD Instinct MI355X (gfx950).
 *
 * The method, as described on the pages this library follows:
 *   1. a lightweight indexer scores every cached position for the current
 *      query ("长上下文：稀疏注意力 / DSA / IndexShare" tutorial, section
 *      "DSA 与 IndexShare"; CLSA explainer, section 2.3 "索引器");
 *   2. each query keeps its top-k positions (same sections);
 *   3. only the selected K/V rows are gathered and attended with softmax
 *      (CLSA explainer, section 1.1 formula and section 2.3 "选择器"; SSA
 *      article, section 6, decode kernel);
 *   4. one index set is reused by a group of layers (tutorial, IndexShare:
 *      every 4 layers; IndexCache article, sections 2 and 6: Full layers run
 *      the indexer into one temporary buffer that Shared layers read).
 *   The gist-chunk variant (SSA article sections 2-3; GSA summary page
 *   section 2.2) scores one gist per 16-token chunk, keeps the top chunks
 *   and unfolds their raw tokens together with their gists.
 *
 * Conventions for every entry point:
 *   - All tensor arguments are DEVICE pointers owned by the caller, dense
 *     row-major with the stated shape, 16-byte aligned.  The library never
 *     allocates, frees or retains them.
 *   - bf16 tensors are passed as uint16_t (bfloat16 bit patterns).
 *   - `stream` is a hipStream_t (NULL = the default stream).  Work is
 *     enqueued asynchronously; buffers must stay alive until it completes.
 *     No call synchronises the device or allocates memory.
 *   - Scratch memory is caller-provided (`ws`, `ws_bytes`), 256-byte
 *     aligned, sized by the matching *_workspace_bytes function (which may
 *     be 0, in which case `ws` may be NULL).  Its contents need no
 *     initialisation and are undefined afterwards.  Calls that share one
 *     workspace must not run concurrently.
 *   - No kernel of this library synchronises workgroups inside a kernel:
 *     every hand-off between workgroups happens at a kernel boundary on
 *     the caller's stream.
 *   - Every call validates its arguments on the host before enqueuing any
 *     work and returns LCT_OK or an error code; lct_last_error() returns a
 *     message for the last failing call on the calling thread.  No C++
 *     exception crosses this interface.
 *   - Outputs are written completely (index rows are padded with -1).
 */
#ifndef LCT_H
#define LCT_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* status codes */
#define LCT_OK 0
#define LCT_EINVAL 1        /* bad argument (null, shape, alignment, range) */
#define LCT_EUNSUPPORTED 2  /* valid but not implemented (e.g. head dim)    */
#define LCT_ENOWORKSPACE 3  /* ws_bytes smaller than required               */
#define LCT_ENODEV 4        /* no usable gfx950 device                      */
#define LCT_EHIP 5          /* a HIP runtime call failed                    */

/* score dtypes for lct_topk_select */
#define LCT_I32 0
#define LCT_F32 1

const char* lct_version(void);
const char* lct_last_error(void);

/*
 * Indexer scores (step 1).  Source: tutorial page, section "DSA 与
 * IndexShare" (the lightning indexer scores all history tokens).  Reading:
 * the score is the plain sum over indexer heads of per-head int8 dot
 * products, i.e. one dot product over the H_idx*d_idx features of a row.
 *
 *   q      int8  [B, Lq, HD]   indexer queries (HD = H_idx * d_idx)
 *   k      int8  [B, L, HD]    indexer key cache
 *   scores int32 [B, Lq, L]    out: scores[b,r,t] = sum_j q[b,r,j] * k[b,t,j]
 *   q_pos0 < 0: no mask (decode, every cached position is a candidate).
 *          >= 0: causal; query row r sits at position q_pos0 + r and the
 *          entries t > q_pos0 + r are undefined (not candidates).
 * Lq <= 16 runs a coalesced HBM streaming kernel; larger Lq (prefill) runs
 * an int8 MFMA kernel.  HD must be a power of two in [16, 512]
 * (LCT_EUNSUPPORTED otherwise; the MFMA kernel needs HD >= 64 and
 * L < 2^22, the streaming kernel L * HD < 2^31).
 */
int lct_idx_score_i8(const int8_t* q, const int8_t* k, int32_t* scores, int B, int Lq,
                     int64_t L, int HD, int64_t q_pos0, void* stream);

/*
 * Causal prefill index of one layer group (steps 1 and 2 together).
 * Source: tutorial page, sections "DSA 与 IndexShare" and "两个阶段各付一笔"
 * (in prefill every query scores all earlier positions and keeps its top k);
 * CLSA explainer section 2.3 (the index set is a small integer array).
 *   q    int8  [L, HD]     indexer queries; row i sits at position i
 *   k    int8  [L, HD]     indexer keys
 *   idx  int32 [L, topk]   out: row i holds the min(topk, i + 1) positions
 *                          t <= i with the largest q[i].k[t] (sum over HD of
 *                          int8 products, int32), equal scores to the lower
 *                          position, ascending, padded with -1.
 * HD = 256, L <= 65536, topk <= 2048: the scores are never stored; they are
 * filtered to per-row candidate lists on the fly and an exact select runs
 * on those; rows the lists cannot settle are listed on the device and get a
 * whole-row select from a fixed grid that reads their count on the device,
 * so the call is asynchronous like every other.  n_fallback (DEVICE int32,
 * may be NULL) receives the number of such rows when the stream reaches it.
 * Other shapes (HD a power of two in [64, 512], L <= 2^18) score blocks of
 * rows into the workspace and select per row; n_fallback then receives 0.
 * ws: at least lct_prefill_index_workspace_bytes(L, HD, topk) bytes, 256-byte
 * aligned, device memory owned by the caller.  q, k 16-byte aligned.
 * Errors: LCT_EINVAL (null / misaligned / bad sizes), LCT_EUNSUPPORTED
 * (shape), LCT_ENOWORKSPACE, LCT_EHIP.
 */
int lct_prefill_index_i8(const int8_t* q, const int8_t* k, int32_t* idx, int64_t L, int HD,
                         int topk, void* ws, size_t ws_bytes, int32_t* n_fallback, void* stream);
int lct_prefill_index_workspace_bytes(int64_t L, int HD, int topk, size_t* bytes);

/*
 * Gist scores (GSA step 1).  Source: SSA article section 3 / GSA summary
 * section 2.2 (the query is compared with every gist by a dot product).
 *   q      bf16 [BH, D], gk bf16 [BH, Nc, D], scores fp32 [BH, Nc] (unscaled).
 * Accumulation is fp32; it is exact when all partial sums are integers
 * below 2^24 in magnitude (integer-valued inputs).  D in {64, 128, 256}.
 */
int lct_gist_score_bf16(const uint16_t* q, const uint16_t* gk, float* scores, int BH,
                        int64_t Nc, int D, void* stream);

/*
 * Top-k position select (step 2).  Source: tutorial page, DSA section
 * (each query keeps its top-k); CLSA explainer section 2.3 (the index set
 * is a small integer array per query).
 *   scores   [rows, ld] of int32 (LCT_I32) or fp32 (LCT_F32); row r's
 *            candidates are positions [0, nv_r), nv_r = min(n, valid_len[r])
 *            (valid_len: device int32 [rows], or NULL for nv_r = n).
 *   idx      int32 [rows, k] out: the min(k, nv_r) positions with the largest
 *            scores; equal scores go to the lower position; listed in
 *            ascending order, padded with -1.
 * fp32 keys compare as numbers (-0.0 equals +0.0); NaN is not supported.
 * Few rows (rows <= 64, n large) use a multi-workgroup select; many rows use
 * one workgroup per row.  Requires 1 <= k, n < 2^31, ld >= n.
 */
int lct_topk_select(const void* scores, int dtype, int32_t* idx, int rows, int64_t n,
                    int64_t ld, int k, const int32_t* valid_len, void* ws, size_t ws_bytes,
                    void* stream);
int lct_topk_workspace_bytes(int rows, int64_t n, int k, size_t* bytes);

/*
 * Sparse attention over gathered rows (step 3).  Source: CLSA explainer
 * section 1.1 (softmax(QK^T/sqrt(d_k))V) evaluated over the selected keys
 * only (section 2.3 selector; tutorial DSA section); split decode with a
 * log-sum-exp merge of partial results (SSA article section 6).
 *   q    bf16 [B, Lq, Hq, D]   queries (post-projection)
 *   k, v bf16 [B, L, Hkv, D]   KV cache of one layer, token-major
 *   idx  int32 [B, Lq, kk]     positions per query row (any order); -1 = skip
 *   out  fp32 [B, Lq, Hq, D]   softmax(scale * q.K_sel^T) V_sel; query head h
 *                              reads KV head h / (Hq / Hkv).  A row with no
 *                              valid position gets zeros.
 * Positions must lie in [0, L) or be -1.  D = 128; Hq % Hkv == 0 and
 * Hq / Hkv in {1, 2, 4, 8, 16}.  fp32 online softmax; bf16 MFMA products.
 */
int lct_sparse_attn_gather(const uint16_t* q, const uint16_t* k, const uint16_t* v,
                           const int32_t* idx, float* out, int B, int Lq, int Hq, int Hkv,
                           int D, int64_t L, int kk, float scale, void* ws, size_t ws_bytes,
                           void* stream);
int lct_sparse_attn_workspace_bytes(int B, int Lq, int Hq, int Hkv, int D, int64_t L, int kk,
                                    size_t* bytes);

/*
 * Gist-chunk select-and-unfold attention (GSA step 3).  Source: SSA
 * article sections 2-3 and the ablation in section 8 (keep the selected
 * chunks' gists and raw tokens, drop unselected gists); GSA summary page
 * section 2.2.  One query per (batch, head) pair, MHA.
 *   q        bf16 [BH, D]
 *   rk, rv   bf16 [BH, raw_cap, D]  raw tokens; chunk c = positions
 *                                   [c*chunk, (c+1)*chunk); the unfinished
 *                                   chunk's tail is [Nc*chunk, Nc*chunk+tail_len)
 *   gv       bf16 [BH, Nc, D]       gist values
 *   gscores  fp32 [BH, Nc]          q . gist_key (unscaled), as produced by
 *                                   lct_gist_score_bf16; the gist logit is
 *                                   gscores * scale
 *   chunk_idx int32 [BH, kc]        chosen chunks (-1, or any id outside
 *                                   [0, Nc): skipped)
 *   out      fp32 [BH, D]
 * Requires chunk == 16, D == 128, 0 <= tail_len <= chunk,
 * raw_cap >= Nc*chunk + tail_len.
 */
int lct_gsa_attn(const uint16_t* q, const uint16_t* rk, const uint16_t* rv, const uint16_t* gv,
                 const float* gscores, const int32_t* chunk_idx, float* out, int BH, int D,
                 int64_t Nc, int64_t raw_cap, int chunk, int kc, int tail_len, float scale,
                 void* ws, size_t ws_bytes, void* stream);
int lct_gsa_attn_workspace_bytes(int BH, int D, int kc, int tail_len, size_t* bytes);

/*
 * Whole GSA decode step: gist scores, top-kc chunk select, unfold attention.
 *   gk bf16 [BH, Nc, D] gist keys; chunk_idx_out int32 [BH, kc] (may be NULL:
 *   then the workspace holds it); other arguments as above.
 */
int lct_gsa_decode(const uint16_t* q, const uint16_t* gk, const uint16_t* gv,
                   const uint16_t* rk, const uint16_t* rv, int32_t* chunk_idx_out, float* out,
                   int BH, int D, int64_t Nc, int64_t raw_cap, int chunk, int kc, int tail_len,
                   float scale, void* ws, size_t ws_bytes, void* stream);
int lct_gsa_decode_workspace_bytes(int BH, int D, int64_t Nc, int kc, size_t* bytes);

/*
 * GSA decode step with coarse-to-fine (hierarchical) routing.  Source: SSA
 * article section 5 (H-SSA: a meta-gist after every few gists summarises
 * them; the query picks the best meta-gists, then the best gists inside
 * their groups, then unfolds those chunks) and GSA summary page section 2.4
 * (gist-of-gist, coarse-to-fine selection, logarithmic routing cost).
 *   mk bf16 [BH, ceil(Nc/group), D]  meta-gist keys; meta-gist g covers
 *                                    gists [g*group, (g+1)*group) (the last
 *                                    group may be short)
 *   the km best meta-gists by q . mk (unscaled; ties to the lower group) are
 *   kept, then the kc best of their gists by q . gk (ties to the lower
 *   chunk); chunk_idx_out gets them ascending, -1 padded when the chosen
 *   groups hold fewer than kc chunks.  Meta-gists only route: the attention
 *   is lct_gsa_attn's over the chosen chunks' raw tokens and gists plus the
 *   tail.  Other arguments as lct_gsa_decode.  Requires 1 <= km <=
 *   ceil(Nc/group), ceil(Nc/group) <= 4096, km <= 64, km*group <= 4096,
 *   kc <= 1024 (LCT_EUNSUPPORTED otherwise).  Key rows read by the routing:
 *   ceil(Nc/group) + km*group per (batch, head) instead of Nc.
 */
int lct_hgsa_decode(const uint16_t* q, const uint16_t* mk, const uint16_t* gk, const uint16_t* gv,
                    const uint16_t* rk, const uint16_t* rv, int32_t* chunk_idx_out, float* out, int BH,
                    int D, int64_t Nc, int64_t raw_cap, int chunk, int group, int km, int kc,
                    int tail_len, float scale, void* ws, size_t ws_bytes, void* stream);
int lct_hgsa_decode_workspace_bytes(int BH, int D, int64_t Nc, int kc, int tail_len, size_t* bytes);

/*
 * GSA prefill: attention of every raw and gist token under the gist mask.
 * Source: SSA article section 4 (a segment's raw tokens see one another and
 * the gists of all earlier segments, never earlier segments' raw tokens) and
 * section 6 (global key columns moved in front: a dense block of gists plus
 * a diagonal band; softmax is unchanged by the key order).  Causal order is
 * the interleaved one (chunk c's 16 raw tokens, then its gist): raw token i
 * of chunk c attends to gists 0..c-1 and raw tokens 0..i of chunk c; gist c
 * to gists 0..c and the 16 raw tokens of chunk c.  No attention anchors.
 *   q_raw    bf16 [BH, Nc*chunk, D]   raw-token queries
 *   q_gist   bf16 [BH, Nc, D]         gist-token queries
 *   rk, rv   bf16 [BH, raw_cap, D]    raw keys/values (rows [0, Nc*chunk) used)
 *   gk, gv   bf16 [BH, Nc, D]         gist keys/values
 *   out_raw  fp32 [BH, Nc*chunk, D],  out_gist fp32 [BH, Nc, D]
 * Requires chunk == 16, D == 128; one (batch, head) array < 2 GiB.  No
 * workspace; fp32 online softmax, bf16 MFMA products.
 */
int lct_gsa_prefill(const uint16_t* q_raw, const uint16_t* q_gist, const uint16_t* rk, const uint16_t* rv,
                    const uint16_t* gk, const uint16_t* gv, float* out_raw, float* out_gist, int BH, int D,
                    int64_t Nc, int64_t raw_cap, int chunk, float scale, void* stream);

/*
 * Layer-group driver (step 4).  Sources: CLSA explainer section 2.3
 * workflow (indexer once, shared index to every layer's selector);
 * tutorial IndexShare (4 layers share one index); IndexCache article
 * sections 2 and 6 (the Full layer of a group runs its indexer into one
 * temporary index buffer, Shared layers read it, the next Full layer
 * overwrites it).
 *
 * Group g = layers [g*layers_per_group, (g+1)*layers_per_group), or, with
 * a layer_full pattern (IndexCache article section 3: the kept indexers
 * need not be evenly spaced), the run of layers from the g-th Full layer to
 * the next.  For each group: idx_g = topk(idx_score(qi[g], ki[g])), then
 * every layer of the group runs sparse attention with that same buffer.
 * With `causal` set the step is a causal prefill: Lq == L, query row r sits
 * at position r, may choose among positions 0..r and keeps min(topk, r+1) of
 * them; the L x L score matrix is never materialised.  What the attention of
 * many rows derives from the index alone (segment bounds, the block-union
 * decisions and union lists) is computed by the group's Full layer and kept
 * in the workspace for its Shared layers.
 */
typedef struct lct_group_desc {
  int B;                 /* batch                                          */
  int Lq;                /* query rows per batch entry (decode); == L causal */
  int64_t L;             /* cached positions                               */
  int HD;                /* indexer features per row (H_idx * d_idx)       */
  int Hq, Hkv, D;        /* attention heads and head dim                   */
  int topk;              /* k                                              */
  int n_layers;          /* multiple of layers_per_group without layer_full */
  int layers_per_group;  /* layers sharing one index set (4 in IndexShare) */
  int causal;            /* 0: decode, 1: causal prefill (B == 1)          */
  float scale;           /* softmax scale, usually 1/sqrt(D)               */
  const int32_t* valid_len;       /* device int32 [B] or NULL (decode only) */
  const int8_t* const* qi;        /* host array [n_groups] of device [B, Lq, HD] */
  const int8_t* const* ki;        /* host array [n_groups] of device [B, L, HD]  */
  const uint16_t* const* q;       /* host array [n_layers] of device bf16 [B, Lq, Hq, D] */
  const uint16_t* const* k;       /* host array [n_layers] of device bf16 [B, L, Hkv, D];
                                     entries may repeat: layers sharing one KV cache
                                     (YOCO / CLSA explainer section 2.1) pass the same
                                     pointer, and then the layers of a group gather the
                                     same rows, which the later layers find in cache   */
  const uint16_t* const* v;       /* host array [n_layers] of device bf16 [B, L, Hkv, D];
                                     may repeat like k                                  */
  float* const* out;              /* host array [n_layers] of device fp32 [B, Lq, Hq, D] */
  int32_t* const* idx_out;        /* NULL, or host array [n_groups] of device int32
                                     [B, Lq, topk] (NULL entries allowed): where each
                                     group's index set is kept; otherwise one workspace
                                     buffer is reused by every group                 */
  const int32_t** layer_idx_seen; /* NULL, or host array [n_layers]: filled with the
                                     device address of the index set each layer read */
  const uint8_t* layer_full;      /* NULL (uniform: every layers_per_group-th layer is
                                     Full), or host array [n_layers]: non-zero marks a
                                     Full layer, which runs the indexer; every other
                                     (Shared) layer reuses the index of the most recent
                                     Full layer.  layer_full[0] must be non-zero; the
                                     groups (qi, ki, idx_out entries) are then the Full
                                     layers in order and layers_per_group is ignored  */
} lct_group_desc;

int lct_group_run(const lct_group_desc* d, void* ws, size_t ws_bytes, void* stream);
int lct_group_workspace_bytes(const lct_group_desc* d, size_t* bytes);

/*
 * lct_group_run without a workspace argument and without any allocation, for
 * callers that cannot allocate device memory (code under HIP-graph capture,
 * tight serving loops, harnesses that forbid hipMalloc).  The scratch memory
 * is a fixed array of LCT_NOALLOC_SCRATCH_BYTES bytes inside the library, one
 * per GPU, placed when the library's code is loaded on that device and held
 * until the process ends; the call allocates and frees nothing.  Same
 * descriptor, semantics and outputs as lct_group_run.  A step whose workspace
 * (lct_group_workspace_bytes) exceeds LCT_NOALLOC_SCRATCH_BYTES is rejected
 * with LCT_ENOWORKSPACE before anything is enqueued (decode steps of the
 * 128K x 8 and 1M x 1 workloads need about 9 MiB and 5 MiB; a causal prefill
 * of thousands of rows does not fit).  Every call on one GPU shares that
 * GPU's array: calls that overlap on one GPU (two streams, two threads) race
 * and must be serialised by the caller.  The array needs no initialisation
 * (as for lct_group_run's workspace).
 */
#define LCT_NOALLOC_SCRATCH_BYTES ((size_t)32 << 20)
int lct_group_run_noalloc(const lct_group_desc* d, void* stream);

#ifdef __cplusplus
}
#endif
#endif /* LCT_H */
