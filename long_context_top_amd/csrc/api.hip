// C-ABI entry points of liblct: argument validation, workspace carve-up,
// kernel dispatch and the layer-group driver.  See include/lct.h for the
// contract of every function.

#include <atomic>
#include <cmath>
#include <cstdarg>
#include <cstdio>
#include <cstring>
#include <mutex>
#include <string>

#include "lct.h"
#include "kernels.h"

using namespace lct;

namespace {

thread_local std::string g_err;

int fail(int code, const char* fmt, ...) {
  char buf[512];
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(buf, sizeof(buf), fmt, ap);
  va_end(ap);
  g_err = buf;
  return code;
}

#define LCT_REQUIRE(cond, ...)                                   \
  do {                                                           \
    if (!(cond)) return fail(LCT_EINVAL, __VA_ARGS__);           \
  } while (0)

#define LCT_HIP(expr, what)                                                            \
  do {                                                                                 \
    hipError_t e_ = (expr);                                                            \
    if (e_ != hipSuccess) return fail(LCT_EHIP, "%s: %s", what, hipGetErrorString(e_)); \
  } while (0)

bool aligned(const void* p, size_t a) { return ((uintptr_t)p % a) == 0; }
bool pow2(int64_t x) { return x > 0 && (x & (x - 1)) == 0; }
size_t up256(size_t x) { return (x + 255) & ~size_t(255); }

// 1 = ok (gfx950), -1 = other device; cached per device ordinal.
std::atomic<int> g_dev_ok[64];

int check_device() {
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0)
    return fail(LCT_ENODEV, "no HIP device is available");
  if (dev < 64) {
    int c = g_dev_ok[dev].load(std::memory_order_relaxed);
    if (c == 1) return LCT_OK;
    if (c == -1) return fail(LCT_ENODEV, "device %d is not a gfx950 (MI355X) GPU", dev);
  }
  hipDeviceProp_t prop;
  if (hipGetDeviceProperties(&prop, dev) != hipSuccess)
    return fail(LCT_ENODEV, "cannot query device %d", dev);
  const bool ok = strncmp(prop.gcnArchName, "gfx950", 6) == 0;
  if (dev < 64) g_dev_ok[dev].store(ok ? 1 : -1, std::memory_order_relaxed);
  if (!ok) return fail(LCT_ENODEV, "device %d is %s, this library is built for gfx950", dev,
                       prop.gcnArchName);
  return LCT_OK;
}

hipStream_t as_stream(void* s) { return reinterpret_cast<hipStream_t>(s); }

// ------------------------------------------------------------ top-k plan ----
// Few long rows go to the multi-workgroup select (in chunks of at most
// TOPK_MULTI_MAX_ROWS rows); everything else to one workgroup per row.
bool topk_use_multi(int rows, int64_t n) {
  if (n > TOPK_ROW_MAX_N) return true;
  return rows <= TOPK_MULTI_MAX_ROWS && n >= 32768;
}

size_t topk_scratch_bytes(int rows, int64_t n) {
  if (!topk_use_multi(rows, n)) return 0;
  const int chunk = rows < TOPK_MULTI_MAX_ROWS ? rows : TOPK_MULTI_MAX_ROWS;
  const int t1 = (int)((n + TOPK_MM_TILE - 1) / TOPK_MM_TILE);
  return topk_multi_layout(chunk, n, t1).total;
}

int run_topk(const void* scores, int dtype, int32_t* idx, int rows, int64_t n, int64_t ld, int k,
             const int32_t* valid_len, int vl_div, char* scratch, hipStream_t st) {
  if (!topk_use_multi(rows, n)) {
    LCT_HIP(launch_topk_rows(scores, dtype, idx, rows, n, ld, k, valid_len, vl_div, -1, st),
            "topk_select (row kernel)");
    return LCT_OK;
  }
  const int t1 = (int)((n + TOPK_MM_TILE - 1) / TOPK_MM_TILE);
  for (int r0 = 0; r0 < rows; r0 += TOPK_MULTI_MAX_ROWS) {
    const int rc = rows - r0 < TOPK_MULTI_MAX_ROWS ? rows - r0 : TOPK_MULTI_MAX_ROWS;
    const TopkMultiLayout lay = topk_multi_layout(rc, n, t1);
    const char* sp = reinterpret_cast<const char*>(scores) + (size_t)r0 * ld * 4;
    // valid_len is indexed by (row / vl_div); offset it only when rows map 1:1
    const int32_t* vl = valid_len;
    if (vl && vl_div == 1) vl += r0;
    if (vl && vl_div != 1 && r0 != 0)
      return fail(LCT_EUNSUPPORTED, "valid_len with grouped rows needs <= %d rows",
                  TOPK_MULTI_MAX_ROWS);
    LCT_HIP(launch_topk_minmax(sp, dtype, rc, n, ld, vl, vl_div, scratch, lay, st), "topk minmax");
    LCT_HIP(launch_topk_select_multi(sp, dtype, idx + (size_t)r0 * k, rc, n, ld, k, vl, vl_div,
                                     scratch, lay, st),
            "topk select");
  }
  return LCT_OK;
}

// --------------------------------------------------------- attention plan ----
size_t attn_scratch_bytes(int B, int Lq, int Hq, int Hkv, int kk, int64_t L) {
  return attn_ws_bytes(attn_plan(B, Lq, Hq, Hkv, kk, L));
}

constexpr int64_t PREFILL_BLOCK_BYTES = (int64_t)512 << 20;  // score block of the causal path

// Causal prefill index of one group: the fused filter + select when the
// shape fits it, else blocks of plain scores + a row select.
struct PrefillPlan {
  bool fused;
  int64_t block_rows;  // plain path: query rows scored per block
  size_t bytes;        // workspace
};

PrefillPlan prefill_plan(int64_t L, int HD, int kk) {
  PrefillPlan p;
  p.fused = HD == 256 && L <= PF_MAX_L && kk <= PF_MAX_K;
  if (p.fused) {
    p.block_rows = 0;
    p.bytes = pf_workspace_layout(L, HD, kk, nullptr);
  } else {
    int64_t br = PREFILL_BLOCK_BYTES / (L * 4);
    br = br < 128 ? 128 : (br / 128) * 128;
    p.block_rows = br < L ? br : L;
    p.bytes = up256((size_t)p.block_rows * L * sizeof(int32_t));
  }
  return p;
}

int validate_prefill(int64_t L, int HD, int kk) {
  LCT_REQUIRE(L >= 1 && kk >= 1, "L and topk must be >= 1");
  if (!pow2(HD) || HD < 64 || HD > 512)
    return fail(LCT_EUNSUPPORTED, "causal prefill needs HD a power of two in [64, 512] (got %d)", HD);
  if (L > TOPK_ROW_MAX_N) return fail(LCT_EUNSUPPORTED, "causal prefill supports L <= %lld", (long long)TOPK_ROW_MAX_N);
  return LCT_OK;
}

int run_prefill(const int8_t* q, const int8_t* k, int32_t* idx, int64_t L, int HD, int kk,
                char* ws, int32_t* n_fallback, hipStream_t st) {
  const PrefillPlan p = prefill_plan(L, HD, kk);
  if (p.fused) {
    LCT_HIP(launch_pf_fused(q, k, L, HD, kk, idx, ws, st, n_fallback), "prefill index (fused)");
    return LCT_OK;
  }
  int32_t* scores = reinterpret_cast<int32_t*>(ws);
  for (int64_t r0 = 0; r0 < L; r0 += p.block_rows) {
    const int64_t nr = L - r0 < p.block_rows ? L - r0 : p.block_rows;
    LCT_HIP(launch_idx_score_mfma(q + r0 * HD, k, scores, 1, (int)nr, L, HD, r0, st),
            "prefill index: idx_score");
    LCT_HIP(launch_topk_rows(scores, LCT_I32, idx + r0 * kk, (int)nr, L, L, kk, nullptr, 1, r0, st),
            "prefill index: topk rows");
  }
  if (n_fallback) LCT_HIP(launch_zero(n_fallback, sizeof(int32_t), st), "prefill index: n_fallback");
  return LCT_OK;
}

}  // namespace

extern "C" {

const char* lct_version(void) { return "lct 0.1.0 (gfx950)"; }

const char* lct_last_error(void) { return g_err.c_str(); }

int lct_idx_score_i8(const int8_t* q, const int8_t* k, int32_t* scores, int B, int Lq,
                     int64_t L, int HD, int64_t q_pos0, void* stream) {
  LCT_REQUIRE(q && k && scores, "null tensor pointer");
  LCT_REQUIRE(aligned(q, 16) && aligned(k, 16) && aligned(scores, 16), "tensors must be 16-byte aligned");
  LCT_REQUIRE(B >= 1 && Lq >= 1 && L >= 1, "B, Lq and L must be >= 1 (got %d, %d, %lld)", B, Lq, (long long)L);
  LCT_REQUIRE(L < ((int64_t)1 << 31), "L must be < 2^31");
  if (!pow2(HD) || HD < 16 || HD > 512)
    return fail(LCT_EUNSUPPORTED, "HD must be a power of two in [16, 512] (got %d)", HD);
  const bool mfma = Lq > 16;
  if (!mfma && L * HD >= ((int64_t)1 << 31))
    return fail(LCT_EUNSUPPORTED, "one batch entry's key cache must be < 2 GiB (L*HD = %lld)", (long long)(L * HD));
  if (mfma && HD < 64) return fail(LCT_EUNSUPPORTED, "the MFMA scorer needs HD >= 64");
  if (mfma && L >= ((int64_t)1 << 22))
    return fail(LCT_EUNSUPPORTED, "the MFMA scorer needs L < 2^22 (128 score rows < 2 GiB)");
  int rc = check_device();
  if (rc) return rc;
  if (!mfma)
    LCT_HIP(launch_idx_score_stream(q, k, scores, B, Lq, L, HD, q_pos0, nullptr, nullptr, nullptr,
                                    nullptr, as_stream(stream)),
            "idx_score (stream)");
  else
    LCT_HIP(launch_idx_score_mfma(q, k, scores, B, Lq, L, HD, q_pos0, as_stream(stream)),
            "idx_score (mfma)");
  return LCT_OK;
}

int lct_prefill_index_workspace_bytes(int64_t L, int HD, int topk, size_t* bytes) {
  LCT_REQUIRE(bytes, "bytes is null");
  int rc = validate_prefill(L, HD, topk);
  if (rc) return rc;
  *bytes = prefill_plan(L, HD, topk).bytes;
  return LCT_OK;
}

int lct_prefill_index_i8(const int8_t* q, const int8_t* k, int32_t* idx, int64_t L, int HD,
                         int topk, void* ws, size_t ws_bytes, int32_t* n_fallback, void* stream) {
  LCT_REQUIRE(q && k && idx, "null tensor pointer");
  LCT_REQUIRE(aligned(q, 16) && aligned(k, 16) && aligned(idx, 4) && aligned(n_fallback, 4), "misaligned tensor");
  int rc = validate_prefill(L, HD, topk);
  if (rc) return rc;
  const size_t need = prefill_plan(L, HD, topk).bytes;
  LCT_REQUIRE(ws != nullptr && aligned(ws, 256), "workspace must be non-null and 256-byte aligned");
  if (ws_bytes < need) return fail(LCT_ENOWORKSPACE, "prefill index needs %zu workspace bytes, got %zu", need, ws_bytes);
  rc = check_device();
  if (rc) return rc;
  return run_prefill(q, k, idx, L, HD, topk, reinterpret_cast<char*>(ws), n_fallback, as_stream(stream));
}

int lct_gist_score_bf16(const uint16_t* q, const uint16_t* gk, float* scores, int BH, int64_t Nc,
                        int D, void* stream) {
  LCT_REQUIRE(q && gk && scores, "null tensor pointer");
  LCT_REQUIRE(aligned(q, 16) && aligned(gk, 16) && aligned(scores, 4), "misaligned tensor");
  LCT_REQUIRE(BH >= 1 && Nc >= 1 && Nc < ((int64_t)1 << 31), "bad BH / Nc");
  if (D != 64 && D != 128 && D != 256) return fail(LCT_EUNSUPPORTED, "D must be 64, 128 or 256");
  int rc = check_device();
  if (rc) return rc;
  LCT_HIP(launch_gist_score(q, gk, scores, BH, Nc, D, as_stream(stream)), "gist_score");
  return LCT_OK;
}

int lct_topk_workspace_bytes(int rows, int64_t n, int k, size_t* bytes) {
  LCT_REQUIRE(bytes, "bytes is null");
  LCT_REQUIRE(rows >= 1 && n >= 1 && n < ((int64_t)1 << 31) && k >= 1, "bad rows / n / k");
  *bytes = topk_scratch_bytes(rows, n);
  return LCT_OK;
}

int lct_topk_select(const void* scores, int dtype, int32_t* idx, int rows, int64_t n,
                    int64_t ld, int k, const int32_t* valid_len, void* ws, size_t ws_bytes,
                    void* stream) {
  LCT_REQUIRE(scores && idx, "null tensor pointer");
  LCT_REQUIRE(dtype == LCT_I32 || dtype == LCT_F32, "dtype must be LCT_I32 or LCT_F32");
  LCT_REQUIRE(aligned(scores, 4) && aligned(idx, 4) && aligned(valid_len, 4), "misaligned tensor");
  LCT_REQUIRE(rows >= 1 && n >= 1 && n < ((int64_t)1 << 31), "bad rows / n");
  LCT_REQUIRE(ld >= n, "ld must be >= n");
  LCT_REQUIRE(k >= 1, "k must be >= 1");
  const size_t need = topk_scratch_bytes(rows, n);
  if (topk_use_multi(rows, n)) {
    LCT_REQUIRE(ws != nullptr && aligned(ws, 256), "workspace must be non-null and 256-byte aligned");
    if (ws_bytes < need) return fail(LCT_ENOWORKSPACE, "topk needs %zu workspace bytes, got %zu", need, ws_bytes);
  }
  int rc = check_device();
  if (rc) return rc;
  return run_topk(scores, dtype, idx, rows, n, ld, k, valid_len, 1, reinterpret_cast<char*>(ws),
                  as_stream(stream));
}

int lct_sparse_attn_workspace_bytes(int B, int Lq, int Hq, int Hkv, int D, int64_t L, int kk,
                                    size_t* bytes) {
  LCT_REQUIRE(bytes, "bytes is null");
  LCT_REQUIRE(B >= 1 && Lq >= 1 && Hq >= 1 && Hkv >= 1 && D >= 1 && kk >= 1 && L >= 1, "bad shape");
  LCT_REQUIRE(Hq % Hkv == 0, "Hq must be a multiple of Hkv");
  *bytes = attn_scratch_bytes(B, Lq, Hq, Hkv, kk, L);
  return LCT_OK;
}

static int validate_attn_shape(int B, int Lq, int Hq, int Hkv, int D, int64_t L, int kk,
                               float scale) {
  LCT_REQUIRE(B >= 1 && Lq >= 1 && Hq >= 1 && Hkv >= 1 && kk >= 1 && L >= 1, "bad shape");
  LCT_REQUIRE(L < ((int64_t)1 << 31), "L must be < 2^31");
  LCT_REQUIRE(Hq % Hkv == 0, "Hq must be a multiple of Hkv");
  LCT_REQUIRE(std::isfinite(scale), "scale must be finite");
  if (D != 128) return fail(LCT_EUNSUPPORTED, "head dim %d (only 128 is built)", D);
  if (L * Hkv * D * 2 >= ((int64_t)1 << 31))
    return fail(LCT_EUNSUPPORTED, "one batch entry's K (or V) cache must be < 2 GiB");
  const int G = Hq / Hkv;
  if (G != 1 && G != 2 && G != 4 && G != 8 && G != 16)
    return fail(LCT_EUNSUPPORTED, "Hq/Hkv = %d (1, 2, 4, 8 or 16 supported)", G);
  return LCT_OK;
}

static int validate_attn_ptrs(const uint16_t* q, const uint16_t* k, const uint16_t* v,
                              const float* out) {
  LCT_REQUIRE(q && k && v && out, "null tensor pointer");
  LCT_REQUIRE(aligned(q, 16) && aligned(k, 16) && aligned(v, 16) && aligned(out, 16),
              "q, k, v, out must be 16-byte aligned");
  return LCT_OK;
}

static int validate_attn(const uint16_t* q, const uint16_t* k, const uint16_t* v,
                         const int32_t* idx, float* out, int B, int Lq, int Hq, int Hkv, int D,
                         int64_t L, int kk, float scale) {
  int rc = validate_attn_ptrs(q, k, v, out);
  if (rc) return rc;
  LCT_REQUIRE(idx && aligned(idx, 4), "idx must be non-null and 4-byte aligned");
  return validate_attn_shape(B, Lq, Hq, Hkv, D, L, kk, scale);
}

static int run_attn(const uint16_t* q, const uint16_t* k, const uint16_t* v, const int32_t* idx,
                    float* out, int B, int Lq, int Hq, int Hkv, int64_t L, int kk, float scale,
                    char* partials, hipStream_t st, bool reuse_index_work = false) {
  const AttnPlan plan = attn_plan(B, Lq, Hq, Hkv, kk, L);
  LCT_HIP(launch_sparse_attn(q, k, v, idx, out, B, Lq, Hq, Hkv, L, kk, scale, plan,
                             reinterpret_cast<float*>(partials), st, reuse_index_work),
          "sparse_attn_gather");
  return LCT_OK;
}

int lct_sparse_attn_gather(const uint16_t* q, const uint16_t* k, const uint16_t* v,
                           const int32_t* idx, float* out, int B, int Lq, int Hq, int Hkv,
                           int D, int64_t L, int kk, float scale, void* ws, size_t ws_bytes,
                           void* stream) {
  int rc = validate_attn(q, k, v, idx, out, B, Lq, Hq, Hkv, D, L, kk, scale);
  if (rc) return rc;
  const size_t need = attn_scratch_bytes(B, Lq, Hq, Hkv, kk, L);
  LCT_REQUIRE(need == 0 || (ws != nullptr && aligned(ws, 256)), "workspace must be non-null and 256-byte aligned");
  if (ws_bytes < need) return fail(LCT_ENOWORKSPACE, "attention needs %zu workspace bytes, got %zu", need, ws_bytes);
  rc = check_device();
  if (rc) return rc;
  return run_attn(q, k, v, idx, out, B, Lq, Hq, Hkv, L, kk, scale, reinterpret_cast<char*>(ws),
                  as_stream(stream));
}

static int validate_gsa(const uint16_t* q, const uint16_t* rk, const uint16_t* rv,
                        const uint16_t* gv, float* out, int BH, int D, int64_t Nc,
                        int64_t raw_cap, int chunk, int kc, int tail_len, float scale) {
  LCT_REQUIRE(q && rk && rv && gv && out, "null tensor pointer");
  LCT_REQUIRE(aligned(q, 16) && aligned(rk, 16) && aligned(rv, 16) && aligned(gv, 16) && aligned(out, 4),
              "misaligned tensor");
  LCT_REQUIRE(BH >= 1 && Nc >= 1 && kc >= 1, "bad BH / Nc / kc");
  LCT_REQUIRE(Nc < ((int64_t)1 << 27), "Nc too large");
  LCT_REQUIRE(tail_len >= 0 && tail_len <= chunk, "tail_len must be in [0, chunk]");
  LCT_REQUIRE(raw_cap >= Nc * chunk + tail_len, "raw_cap must hold Nc*chunk + tail_len rows");
  LCT_REQUIRE(std::isfinite(scale), "scale must be finite");
  if (chunk != 16) return fail(LCT_EUNSUPPORTED, "chunk %d (only 16 is built)", chunk);
  if (D != 128) return fail(LCT_EUNSUPPORTED, "head dim %d (only 128 is built)", D);
  return LCT_OK;
}

int lct_gsa_attn_workspace_bytes(int BH, int D, int kc, int tail_len, size_t* bytes) {
  LCT_REQUIRE(bytes, "bytes is null");
  LCT_REQUIRE(BH >= 1 && D >= 1 && kc >= 1 && tail_len >= 0, "bad shape");
  *bytes = gsa_plan(BH, kc, tail_len).part_bytes;
  return LCT_OK;
}

int lct_gsa_attn(const uint16_t* q, const uint16_t* rk, const uint16_t* rv, const uint16_t* gv,
                 const float* gscores, const int32_t* chunk_idx, float* out, int BH, int D,
                 int64_t Nc, int64_t raw_cap, int chunk, int kc, int tail_len, float scale,
                 void* ws, size_t ws_bytes, void* stream) {
  int rc = validate_gsa(q, rk, rv, gv, out, BH, D, Nc, raw_cap, chunk, kc, tail_len, scale);
  if (rc) return rc;
  LCT_REQUIRE(gscores && chunk_idx, "null gscores / chunk_idx");
  const GsaPlan plan = gsa_plan(BH, kc, tail_len);
  const size_t need = plan.part_bytes;
  LCT_REQUIRE(need == 0 || (ws != nullptr && aligned(ws, 256)), "workspace must be non-null and 256-byte aligned");
  if (ws_bytes < need) return fail(LCT_ENOWORKSPACE, "gsa_attn needs %zu workspace bytes, got %zu", need, ws_bytes);
  rc = check_device();
  if (rc) return rc;
  char* w = reinterpret_cast<char*>(ws);
  LCT_HIP(launch_gsa_attn(q, rk, rv, gv, gscores, chunk_idx, out, BH, Nc, raw_cap, kc, tail_len,
                          scale, plan, reinterpret_cast<float*>(w), as_stream(stream)),
          "gsa_attn");
  return LCT_OK;
}

namespace {
struct GsaLayout {
  size_t scores, cidx, topk, part, total;
};
GsaLayout gsa_layout(int BH, int64_t Nc, int kc, int tail_len) {
  GsaLayout l;
  size_t off = 0;
  l.scores = off;
  off += up256((size_t)BH * Nc * sizeof(float));
  l.cidx = off;
  off += up256((size_t)BH * kc * sizeof(int32_t));
  l.topk = off;
  off += up256(topk_scratch_bytes(BH, Nc));
  l.part = off;
  off += up256(gsa_plan(BH, kc, tail_len).part_bytes);
  l.total = off;
  return l;
}
}  // namespace

int lct_gsa_decode_workspace_bytes(int BH, int D, int64_t Nc, int kc, size_t* bytes) {
  LCT_REQUIRE(bytes, "bytes is null");
  LCT_REQUIRE(BH >= 1 && D >= 1 && Nc >= 1 && kc >= 1, "bad shape");
  *bytes = gsa_layout(BH, Nc, kc, 16).total;
  return LCT_OK;
}

int lct_gsa_decode(const uint16_t* q, const uint16_t* gk, const uint16_t* gv,
                   const uint16_t* rk, const uint16_t* rv, int32_t* chunk_idx_out, float* out,
                   int BH, int D, int64_t Nc, int64_t raw_cap, int chunk, int kc, int tail_len,
                   float scale, void* ws, size_t ws_bytes, void* stream) {
  int rc = validate_gsa(q, rk, rv, gv, out, BH, D, Nc, raw_cap, chunk, kc, tail_len, scale);
  if (rc) return rc;
  LCT_REQUIRE(gk && aligned(gk, 16), "gk must be non-null and 16-byte aligned");
  LCT_REQUIRE(aligned(chunk_idx_out, 4), "misaligned chunk_idx_out");
  LCT_REQUIRE(ws != nullptr && aligned(ws, 256), "workspace must be non-null and 256-byte aligned");
  const GsaLayout lay = gsa_layout(BH, Nc, kc, tail_len);
  if (ws_bytes < lay.total) return fail(LCT_ENOWORKSPACE, "gsa_decode needs %zu workspace bytes, got %zu", lay.total, ws_bytes);
  rc = check_device();
  if (rc) return rc;
  hipStream_t st = as_stream(stream);
  char* w = reinterpret_cast<char*>(ws);
  float* sc = reinterpret_cast<float*>(w + lay.scores);
  int32_t* cidx = chunk_idx_out ? chunk_idx_out : reinterpret_cast<int32_t*>(w + lay.cidx);
  LCT_HIP(launch_gist_score(q, gk, sc, BH, Nc, D, st), "gsa_decode: gist_score");
  rc = run_topk(sc, LCT_F32, cidx, BH, Nc, Nc, kc, nullptr, 1, w + lay.topk, st);
  if (rc) return rc;
  const GsaPlan plan = gsa_plan(BH, kc, tail_len);
  LCT_HIP(launch_gsa_attn(q, rk, rv, gv, sc, cidx, out, BH, Nc, raw_cap, kc, tail_len, scale,
                          plan, reinterpret_cast<float*>(w + lay.part), st),
          "gsa_decode: gsa_attn");
  return LCT_OK;
}

int lct_hgsa_decode_workspace_bytes(int BH, int D, int64_t Nc, int kc, int tail_len, size_t* bytes) {
  LCT_REQUIRE(bytes, "bytes is null");
  LCT_REQUIRE(BH >= 1 && D >= 1 && Nc >= 1 && kc >= 1 && tail_len >= 0, "bad shape");
  // gist scores (only the candidates' are written) + chunk ids + attention partials
  const GsaLayout l = gsa_layout(BH, Nc, kc, tail_len);
  *bytes = l.total - up256(topk_scratch_bytes(BH, Nc));
  return LCT_OK;
}

int lct_hgsa_decode(const uint16_t* q, const uint16_t* mk, const uint16_t* gk, const uint16_t* gv,
                    const uint16_t* rk, const uint16_t* rv, int32_t* chunk_idx_out, float* out, int BH,
                    int D, int64_t Nc, int64_t raw_cap, int chunk, int group, int km, int kc,
                    int tail_len, float scale, void* ws, size_t ws_bytes, void* stream) {
  int rc = validate_gsa(q, rk, rv, gv, out, BH, D, Nc, raw_cap, chunk, kc, tail_len, scale);
  if (rc) return rc;
  LCT_REQUIRE(gk && aligned(gk, 16) && mk && aligned(mk, 16), "gk and mk must be non-null and 16-byte aligned");
  LCT_REQUIRE(aligned(chunk_idx_out, 4), "misaligned chunk_idx_out");
  LCT_REQUIRE(group >= 1 && km >= 1, "group and km must be >= 1");
  const int64_t Nm = (Nc + group - 1) / group;
  LCT_REQUIRE(km <= Nm, "km must be <= the number of meta-gists (ceil(Nc / group))");
  if (Nm > HG_MAX_ITEMS || km > HG_MAX_KM || (int64_t)km * group > HG_MAX_ITEMS || kc > HG_MAX_KC)
    return fail(LCT_EUNSUPPORTED, "hgsa: needs ceil(Nc/group) <= %d, km <= %d, km*group <= %d, kc <= %d",
                HG_MAX_ITEMS, HG_MAX_KM, HG_MAX_ITEMS, HG_MAX_KC);
  LCT_REQUIRE(ws != nullptr && aligned(ws, 256), "workspace must be non-null and 256-byte aligned");
  size_t need = 0;
  lct_hgsa_decode_workspace_bytes(BH, D, Nc, kc, tail_len, &need);
  if (ws_bytes < need) return fail(LCT_ENOWORKSPACE, "hgsa_decode needs %zu workspace bytes, got %zu", need, ws_bytes);
  rc = check_device();
  if (rc) return rc;
  hipStream_t st = as_stream(stream);
  // layout: [gist scores][chunk ids][attention partials]
  char* w = reinterpret_cast<char*>(ws);
  float* sc = reinterpret_cast<float*>(w);
  const size_t cidx_off = up256((size_t)BH * Nc * sizeof(float));
  const size_t part_off = cidx_off + up256((size_t)BH * kc * sizeof(int32_t));
  int32_t* cidx = chunk_idx_out ? chunk_idx_out : reinterpret_cast<int32_t*>(w + cidx_off);
  LCT_HIP(launch_hgsa_route(q, mk, gk, sc, cidx, BH, Nc, (int)Nm, group, km, kc, st), "hgsa_decode: route");
  const GsaPlan plan = gsa_plan(BH, kc, tail_len);
  LCT_HIP(launch_gsa_attn(q, rk, rv, gv, sc, cidx, out, BH, Nc, raw_cap, kc, tail_len, scale, plan,
                          reinterpret_cast<float*>(w + part_off), st),
          "hgsa_decode: gsa_attn");
  return LCT_OK;
}

int lct_gsa_prefill(const uint16_t* q_raw, const uint16_t* q_gist, const uint16_t* rk, const uint16_t* rv,
                    const uint16_t* gk, const uint16_t* gv, float* out_raw, float* out_gist, int BH, int D,
                    int64_t Nc, int64_t raw_cap, int chunk, float scale, void* stream) {
  LCT_REQUIRE(q_raw && q_gist && rk && rv && gk && gv && out_raw && out_gist, "null tensor pointer");
  LCT_REQUIRE(aligned(q_raw, 16) && aligned(q_gist, 16) && aligned(rk, 16) && aligned(rv, 16) && aligned(gk, 16) &&
                  aligned(gv, 16) && aligned(out_raw, 16) && aligned(out_gist, 16),
              "misaligned tensor");
  LCT_REQUIRE(BH >= 1 && Nc >= 1, "bad BH / Nc");
  LCT_REQUIRE(raw_cap >= Nc * chunk, "raw_cap must hold Nc*chunk rows");
  LCT_REQUIRE(std::isfinite(scale), "scale must be finite");
  if (chunk != 16) return fail(LCT_EUNSUPPORTED, "chunk %d (only 16 is built)", chunk);
  if (D != 128) return fail(LCT_EUNSUPPORTED, "head dim %d (only 128 is built)", D);
  if (raw_cap * D * 2 >= ((int64_t)1 << 31) || Nc * D * 2 >= ((int64_t)1 << 31))
    return fail(LCT_EUNSUPPORTED, "one (batch, head) K or V array must be < 2 GiB");
  int rc = check_device();
  if (rc) return rc;
  LCT_HIP(launch_gsa_prefill(q_raw, q_gist, rk, rv, gk, gv, out_raw, out_gist, BH, Nc, raw_cap, scale,
                             as_stream(stream)),
          "gsa_prefill");
  return LCT_OK;
}

// ------------------------------------------------------------- driver ----
namespace {

struct GroupLayout {
  size_t scores, idx, topk, attn, total;
  int64_t block_rows;  // causal: query rows scored per block
  bool multi;          // decode: multi-workgroup select fused with the scorer
};

GroupLayout group_layout(const lct_group_desc* d) {
  GroupLayout l;
  size_t off = 0;
  const int64_t rows = (int64_t)d->B * d->Lq;
  if (!d->causal) {
    l.block_rows = rows;
    l.multi = topk_use_multi((int)rows, d->L);
  } else {
    l.block_rows = 0;
    l.multi = false;
  }
  l.scores = off;
  if (!d->causal) off += up256((size_t)l.block_rows * d->L * sizeof(int32_t));
  else off += prefill_plan(d->L, d->HD, d->topk).bytes;
  l.idx = off;
  off += up256((size_t)rows * d->topk * sizeof(int32_t));
  l.topk = off;
  if (l.multi) {
    const int t1 = score_plan(d->B, d->Lq, d->L, d->HD).tiles;
    off += up256(topk_multi_layout((int)rows, d->L, t1).total);
  }
  l.attn = off;
  off += up256(attn_scratch_bytes(d->B, d->Lq, d->Hq, d->Hkv, d->topk, d->L));
  l.total = off;
  return l;
}

// Full layer test and the number of groups (Full layers)
bool layer_is_full(const lct_group_desc* d, int l) {
  return d->layer_full ? d->layer_full[l] != 0 : l % d->layers_per_group == 0;
}

int group_count(const lct_group_desc* d) {
  int ng = 0;
  for (int l = 0; l < d->n_layers; ++l) ng += layer_is_full(d, l) ? 1 : 0;
  return ng;
}

int validate_group(const lct_group_desc* d) {
  LCT_REQUIRE(d != nullptr, "descriptor is null");
  LCT_REQUIRE(d->B >= 1 && d->Lq >= 1 && d->L >= 1 && d->topk >= 1, "bad B / Lq / L / topk");
  LCT_REQUIRE(d->L < ((int64_t)1 << 31), "L must be < 2^31");
  LCT_REQUIRE(d->n_layers >= 1, "n_layers must be >= 1");
  if (d->layer_full) {
    LCT_REQUIRE(d->layer_full[0] != 0, "layer_full[0] must mark a Full layer (no index to reuse yet)");
  } else {
    LCT_REQUIRE(d->layers_per_group >= 1 && d->n_layers % d->layers_per_group == 0,
                "n_layers must be a positive multiple of layers_per_group");
  }
  LCT_REQUIRE(d->qi && d->ki && d->q && d->k && d->v && d->out, "null pointer array");
  const int ng = group_count(d);
  for (int g = 0; g < ng; ++g) {
    LCT_REQUIRE(d->qi[g] && d->ki[g], "null indexer tensor for group %d", g);
    LCT_REQUIRE(aligned(d->qi[g], 16) && aligned(d->ki[g], 16), "misaligned indexer tensor (group %d)", g);
    if (d->idx_out && d->idx_out[g]) LCT_REQUIRE(aligned(d->idx_out[g], 4), "misaligned idx_out[%d]", g);
  }
  {
    int rc = validate_attn_shape(d->B, d->Lq, d->Hq, d->Hkv, d->D, d->L, d->topk, d->scale);
    if (rc) return rc;
  }
  for (int l = 0; l < d->n_layers; ++l) {
    int rc = validate_attn_ptrs(d->q[l], d->k[l], d->v[l], d->out[l]);
    if (rc) return fail(rc, "layer %d: %s", l, g_err.c_str());
  }
  LCT_REQUIRE(aligned(d->valid_len, 4), "misaligned valid_len");
  if (!pow2(d->HD) || d->HD < 16 || d->HD > 512)
    return fail(LCT_EUNSUPPORTED, "HD must be a power of two in [16, 512] (got %d)", d->HD);
  if (d->causal) {
    LCT_REQUIRE(d->B == 1 && d->Lq == d->L, "causal prefill needs B == 1 and Lq == L");
    LCT_REQUIRE(d->valid_len == nullptr, "valid_len is not used by the causal path");
    int rc = validate_prefill(d->L, d->HD, d->topk);
    if (rc) return rc;
  } else {
    LCT_REQUIRE(d->Lq <= 64, "decode takes at most 64 query rows per batch entry");
    if (d->L * d->HD >= ((int64_t)1 << 31))
      return fail(LCT_EUNSUPPORTED, "one batch entry's indexer keys must be < 2 GiB");
    const GroupLayout lay = group_layout(d);
    if (!lay.multi && d->L > TOPK_ROW_MAX_N)
      return fail(LCT_EUNSUPPORTED, "too many rows for L = %lld", (long long)d->L);
  }
  return LCT_OK;
}

}  // namespace

int lct_group_workspace_bytes(const lct_group_desc* d, size_t* bytes) {
  LCT_REQUIRE(bytes, "bytes is null");
  int rc = validate_group(d);
  if (rc) return rc;
  *bytes = group_layout(d).total;
  return LCT_OK;
}

int lct_group_run(const lct_group_desc* d, void* ws, size_t ws_bytes, void* stream) {
  int rc = validate_group(d);
  if (rc) return rc;
  LCT_REQUIRE(ws != nullptr && aligned(ws, 256), "workspace must be non-null and 256-byte aligned");
  const GroupLayout lay = group_layout(d);
  if (ws_bytes < lay.total) return fail(LCT_ENOWORKSPACE, "group_run needs %zu workspace bytes, got %zu", lay.total, ws_bytes);
  rc = check_device();
  if (rc) return rc;
  hipStream_t st = as_stream(stream);
  char* w = reinterpret_cast<char*>(ws);
  int32_t* scores = reinterpret_cast<int32_t*>(w + lay.scores);
  const int rows = d->B * d->Lq;
  int32_t* ib = nullptr;
  for (int l = 0, g = -1; l < d->n_layers; ++l) {
    if (layer_is_full(d, l)) {
      // a Full layer: indexer + select into its group's index buffer
      ++g;
      ib = (d->idx_out && d->idx_out[g]) ? d->idx_out[g] : reinterpret_cast<int32_t*>(w + lay.idx);
      if (!d->causal) {
        if (lay.multi) {
          const int t1 = score_plan(d->B, d->Lq, d->L, d->HD).tiles;
          const TopkMultiLayout tl = topk_multi_layout(rows, d->L, t1);
          char* tw = w + lay.topk;
          LCT_HIP(launch_idx_score_stream(d->qi[g], d->ki[g], scores, d->B, d->Lq, d->L, d->HD, -1,
                                          reinterpret_cast<uint32_t*>(tw + tl.mm),
                                          reinterpret_cast<TopkRowState*>(tw + tl.state),
                                          reinterpret_cast<uint32_t*>(tw + tl.hist), d->valid_len, st),
                  "group: idx_score");
          LCT_HIP(launch_topk_select_multi(scores, LCT_I32, ib, rows, d->L, d->L, d->topk,
                                           d->valid_len, d->Lq, tw, tl, st),
                  "group: topk select");
        } else {
          LCT_HIP(launch_idx_score_stream(d->qi[g], d->ki[g], scores, d->B, d->Lq, d->L, d->HD, -1,
                                          nullptr, nullptr, nullptr, nullptr, st),
                  "group: idx_score");
          LCT_HIP(launch_topk_rows(scores, LCT_I32, ib, rows, d->L, d->L, d->topk, d->valid_len, d->Lq, -1, st),
                  "group: topk rows");
        }
      } else {
        rc = run_prefill(d->qi[g], d->ki[g], ib, d->L, d->HD, d->topk, w + lay.scores, nullptr, st);
        if (rc) return rc;
      }
    }
    // the Full layer and the Shared layers after it read the same buffer;
    // a Shared layer also reuses what the attention derived from it in the
    // layer before (same index, shapes and workspace)
    if (d->layer_idx_seen) d->layer_idx_seen[l] = ib;
    rc = run_attn(d->q[l], d->k[l], d->v[l], ib, d->out[l], d->B, d->Lq, d->Hq, d->Hkv, d->L,
                  d->topk, d->scale, w + lay.attn, st, !layer_is_full(d, l));
    if (rc) return rc;
  }
  return LCT_OK;
}

}  // extern "C"

// ------------------------------------------------- no-allocation driver ----
// Scratch memory of lct_group_run_noalloc: one array per GPU, part of the code
// object (placed when the library's code is loaded on a device, never by a
// call) and held until the process ends.  Host code never uses the array's
// name as an address: the device address comes from hipGetSymbolAddress,
// once per device, with that device current.
static __device__ __align__(256) unsigned char scratch[LCT_NOALLOC_SCRATCH_BYTES];

namespace {
std::mutex g_scratch_mu;
void* g_scratch_ptr[64];

int scratch_address(void** out) {
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64)
    return fail(LCT_ENODEV, "no HIP device is available");
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (!g_scratch_ptr[dev]) {
    void* p = nullptr;
    const hipError_t e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess || !p) return fail(LCT_EHIP, "hipGetSymbolAddress(scratch): %s", hipGetErrorString(e));
    g_scratch_ptr[dev] = p;
  }
  *out = g_scratch_ptr[dev];
  return LCT_OK;
}
}  // namespace

extern "C" int lct_group_run_noalloc(const lct_group_desc* d, void* stream) {
  int rc = validate_group(d);
  if (rc) return rc;
  const size_t need = group_layout(d).total;
  if (need > LCT_NOALLOC_SCRATCH_BYTES)
    return fail(LCT_ENOWORKSPACE,
                "group_run_noalloc: this step needs %zu bytes of scratch, the built-in array holds %zu "
                "(use lct_group_run with a workspace)", need, (size_t)LCT_NOALLOC_SCRATCH_BYTES);
  rc = check_device();
  if (rc) return rc;
  void* ws = nullptr;
  rc = scratch_address(&ws);
  if (rc) return rc;
  return lct_group_run(d, ws, LCT_NOALLOC_SCRATCH_BYTES, stream);
}
