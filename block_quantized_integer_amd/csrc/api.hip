// api.hip -- the C ABI of libbqi (declared in include/bqi.h): host-side
// argument validation, then dispatch to the gfx950 kernels.  Validation runs
// before any HIP call, so a rejected call touches neither the device nor the
// stream and can be exercised on a machine without a GPU.
#include "bqi.h"
#include "bqi_launch.h"

#include <mutex>

namespace {

constexpr int64_t kQK = 32;
constexpr int64_t kI32Max = 0x7fffffffLL;
// routed rows (n_tokens * top_k) accepted by route_topk and the grouped GEMM
constexpr int64_t kMaxRouted = 1LL << 30;

bool aligned(const void *p, uintptr_t a) {
  return (reinterpret_cast<uintptr_t>(p) & (a - 1)) == 0;
}

int hip_status(hipError_t e) { return e == hipSuccess ? BQI_OK : BQI_EHIP; }

hipStream_t as_stream(void *s) { return reinterpret_cast<hipStream_t>(s); }

// Workspace layout of qgemm_w4a8_grouped: counts[E], offsets[E+1] and
// rows[T*top_k] (int32), each section on a 256-byte boundary.
size_t round256(size_t x) { return (x + 255) & ~(size_t)255; }

struct WsLayout {
  size_t counts, offsets, rows, total;
};

// counts [E], offsets [E+1] and rows [rows_total] (int32), each section
// 256-byte aligned
WsLayout ws_layout(int64_t rows_total, int64_t n_experts, int64_t k) {
  (void)k;
  WsLayout L;
  L.counts = 0;
  L.offsets = round256((size_t)n_experts * 4);
  L.rows = L.offsets + round256((size_t)(n_experts + 1) * 4);
  L.total = L.rows + round256((size_t)rows_total * 4);
  return L;
}

// 16 < m <= 128: the MFMA GEMM runs one 128-row tile per column tile, so its
// time hardly depends on m there (about 4 + 13.1 k / 1024 us per round of 256
// tiles on MI355X), while the thin-M MFMA kernel takes the rows in chunks of
// 16 and reads the weights once per chunk (at most about 4 us plus the
// chunks' weight bytes at 4.5 TB/s).  The chunks run where that estimate is
// lower.  Measured over k = 256 .. 5120 and n = 512 .. 17408: 1.7-5.1x
// faster where they run (27.7 -> 5.4 us at m = 17, k = 2048, n = 768), never
// slower; weight-heavy shapes keep the GEMM from 64-80 rows up.
bool thin_chunks_faster(int64_t m, int64_t n, int64_t k, const uint16_t *wd) {
  if (m <= 16 || m > 128 || !bqi::gemv_thin_chunks_ok(m, n, k, wd)) return false;
  const double chunks = (double)((m + 15) / 16);
  const double weight_bytes = (double)n * (double)k * (1.0 + 1.0 / 16.0);
  const double rounds = (double)(((n + 127) / 128 + 255) / 256);
  const double t_gemm = 4.0 + 13.1 * (double)k / 1024.0 * rounds;
  const double t_chunks = 4.0 + chunks * weight_bytes / 4.5e6;
  return t_chunks < t_gemm;
}

// Launch of a validated Q8_0 GEMM: the thin-M kernels for m <= 16 (and in
// chunks of 16 rows where that is faster), the MFMA GEMM otherwise.
int qgemm_launch(const int8_t *aq, const uint16_t *ad, int64_t m,
                 const int8_t *wq, const uint16_t *wd, int64_t n, int64_t k,
                 float *y, hipStream_t s) {
  if (m <= 16 || thin_chunks_faster(m, n, k, wd))
    return hip_status(bqi::launch_gemv_thin(aq, ad, m, wq, wd, n, k, y, s));
  return hip_status(bqi::launch_gemm_mfma(aq, ad, m, wq, wd, n, k, y, s));
}

// ---- the allocation-free grouped entry point ---------------------------------
// Its workspace is this file-scope device array: one copy per GPU, created
// when the library's code is loaded on that GPU and held until the process
// ends.  Host code never passes the array's name to a kernel (on the host it
// is only a stand-in for the symbol); it looks up the array's device address
// once per device with hipGetSymbolAddress, with that device current, and
// passes that address.  Calls that overlap on one GPU share the array and
// race; the routing pass rewrites every entry that the GEMM reads (counts,
// offsets and the rows of this call), so nothing needs clearing between
// calls.
static __device__ __align__(256) unsigned char scratch[BQI_NOALLOC_SCRATCH_BYTES];

constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void *g_scratch_ptr[kMaxDevices];

int scratch_for_current_device(void **out) {
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess) return BQI_EHIP;
  if (dev < 0 || dev >= kMaxDevices) return BQI_EHIP;
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (g_scratch_ptr[dev] == nullptr) {
    void *p = nullptr;
    const hipError_t e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess || p == nullptr) return BQI_EHIP;
    g_scratch_ptr[dev] = p;
  }
  *out = g_scratch_ptr[dev];
  return BQI_OK;
}

// The grouped GEMM behind both entry points.  With use_scratch, the
// workspace is the library's own device array (no allocation); the size
// check against it comes first, before any HIP call.
int grouped_impl(const int8_t *aq, const uint16_t *ad, int64_t n_tokens,
                 const int32_t *topk_ids, int64_t top_k, const uint8_t *wq4,
                 const uint16_t *wd, int64_t n_experts, int64_t n, int64_t k,
                 float *y, void *workspace, size_t workspace_bytes,
                 bool use_scratch, void *stream) {
  if (n_tokens < 0 || top_k < 0 || n_experts < 0 || n < 0 || k < 0 ||
      k % kQK != 0)
    return BQI_ESHAPE;
  if (n_experts > 65536 || n_tokens * top_k > kMaxRouted || n > kI32Max ||
      k > kI32Max)
    return BQI_ESHAPE;
  const int64_t rows_total = n_tokens * top_k;
  if (rows_total == 0 || n == 0) return BQI_OK;
  if (!y || !topk_ids) return BQI_EINVAL;
  if (n_experts > 0 && n_experts * ((n + 127) / 128) > kI32Max) return BQI_ESHAPE;
  // the MFMA path addresses one expert's packed weights and the activations
  // with 32-bit offsets
  if (n * (k / 2) > kI32Max || n_tokens * k > kI32Max) return BQI_ESHAPE;
  if (k > 0 && (!aq || !ad)) return BQI_EINVAL;
  if (k > 0 && n_experts > 0 && (!wq4 || !wd)) return BQI_EINVAL;
  if (!aligned(y, 4) || !aligned(topk_ids, 4)) return BQI_EALIGN;
  if (k > 0 && (!aligned(aq, 16) || !aligned(ad, 2))) return BQI_EALIGN;
  if (k > 0 && n_experts > 0 && (!aligned(wq4, 16) || !aligned(wd, 2)))
    return BQI_EALIGN;
  hipStream_t s = as_stream(stream);
  if (k == 0 || n_experts == 0) {
    // every valid row is an empty sum, or every row is invalid: y = 0
    return hip_status(bqi::launch_zero_f32(y, rows_total * n, s));
  }
  const WsLayout L = ws_layout(rows_total, n_experts, k);
  if (use_scratch) {
    if (L.total > (size_t)BQI_NOALLOC_SCRATCH_BYTES) return BQI_ESHAPE;
    if (!bqi::grouped_gemv_supported(rows_total, k)) {
      const int st = scratch_for_current_device(&workspace);
      if (st != BQI_OK) return st;
      workspace_bytes = (size_t)BQI_NOALLOC_SCRATCH_BYTES;
    }
  } else {
    if (!workspace || workspace_bytes < L.total) return BQI_EINVAL;
    if (!aligned(workspace, 256)) return BQI_EALIGN;
  }
  // a few routed rows (decode): the v_dot4 GEMV per routed row, which needs
  // no routing pass and no workspace; otherwise route, then the int8-MFMA
  // kernel
  if (bqi::grouped_gemv_supported(rows_total, k))
    return hip_status(bqi::launch_grouped_gemv(aq, ad, topk_ids, rows_total, top_k,
                                               wq4, wd, n_experts, n, k, y, s));
  char *ws = static_cast<char *>(workspace);
  int32_t *counts = reinterpret_cast<int32_t *>(ws + L.counts);
  int32_t *offsets = reinterpret_cast<int32_t *>(ws + L.offsets);
  int32_t *rows = reinterpret_cast<int32_t *>(ws + L.rows);
  hipError_t e = bqi::launch_route_topk(topk_ids, rows_total, n_experts, top_k, counts,
                                        offsets, rows, y, n, s);
  if (e != hipSuccess) return BQI_EHIP;
  return hip_status(bqi::launch_grouped_w4a8(aq, ad, top_k, wq4, wd, n_experts, n, k,
                                             rows_total, counts, offsets, rows, y, s));
}

}  // namespace

extern "C" {

const char *bqi_status_string(int status) {
  switch (status) {
    case BQI_OK: return "BQI_OK";
    case BQI_EINVAL: return "BQI_EINVAL: null pointer, bad dtype or workspace too small";
    case BQI_ESHAPE: return "BQI_ESHAPE: bad size (negative, k not a multiple of 32, ldx < k, too large; for qgemm_w4a8_grouped_noalloc, a workspace beyond BQI_NOALLOC_SCRATCH_BYTES)";
    case BQI_EALIGN: return "BQI_EALIGN: pointer or leading dimension misaligned";
    case BQI_EHIP: return "BQI_EHIP: HIP runtime error at launch";
    case BQI_ENOTSUP: return "BQI_ENOTSUP: the host CPU lacks AVX2/FMA";
    default: return "unknown bqi status";
  }
}

int bqi_abi_version(void) { return 240; }

int quantize_q8_0(const void *x, int x_dtype, int64_t rows, int64_t k,
                  int64_t ldx, int8_t *q, uint16_t *d, void *stream) {
  if (x_dtype != BQI_F32 && x_dtype != BQI_F16) return BQI_EINVAL;
  if (rows < 0 || k < 0 || k % kQK != 0 || ldx < k) return BQI_ESHAPE;
  if (rows == 0 || k == 0) return BQI_OK;
  if (rows > kI32Max || k > kI32Max) return BQI_ESHAPE;
  if (!x || !q || !d) return BQI_EINVAL;
  const int64_t esize = x_dtype == BQI_F32 ? 4 : 2;
  const int64_t vec = x_dtype == BQI_F32 ? 16 : 8;  // bytes per lane load
  if (!aligned(x, 16) || (ldx * esize) % vec != 0 || !aligned(q, 16) ||
      !aligned(d, 2))
    return BQI_EALIGN;
  return hip_status(bqi::launch_quantize_q8_0(x, x_dtype == BQI_F16, rows, k,
                                              ldx, q, d, as_stream(stream)));
}

int qgemm_q8_0(const int8_t *aq, const uint16_t *ad, int64_t m,
               const int8_t *wq, const uint16_t *wd, int64_t n, int64_t k,
               float *y, void *stream) {
  if (m < 0 || n < 0 || k < 0 || k % kQK != 0) return BQI_ESHAPE;
  if (m == 0 || n == 0) return BQI_OK;
  if (!y) return BQI_EINVAL;
  if (m > kI32Max || n > kI32Max || k > kI32Max) return BQI_ESHAPE;
  if (k == 0) {
    // empty sum: y = 0
    if (!aligned(y, 4)) return BQI_EALIGN;
    return hip_status(bqi::launch_zero_f32(y, m * n, as_stream(stream)));
  }
  if (!aq || !ad || !wq || !wd) return BQI_EINVAL;
  if (!aligned(aq, 16) || !aligned(wq, 16) || !aligned(ad, 2) ||
      !aligned(wd, 2) || !aligned(y, 4))
    return BQI_EALIGN;
  // the MFMA kernel indexes tiles, rows and element offsets in 32-bit
  if (m > 16 && ((m + 127) / 128 * ((n + 127) / 128) > kI32Max ||
                 m * k > kI32Max || n * k > kI32Max))
    return BQI_ESHAPE;
  return qgemm_launch(aq, ad, m, wq, wd, n, k, y, as_stream(stream));
}

int quantize_qgemm_q8_0(const void *x, int x_dtype, int64_t m, int64_t k,
                        int64_t ldx, const int8_t *wq, const uint16_t *wd,
                        int64_t n, float *y, int8_t *q, uint16_t *d,
                        void *stream) {
  if (x_dtype != BQI_F32 && x_dtype != BQI_F16) return BQI_EINVAL;
  if (m < 0 || n < 0 || k < 0 || k % kQK != 0 || ldx < k) return BQI_ESHAPE;
  if (m == 0) return BQI_OK;
  if (m > kI32Max || n > kI32Max || k > kI32Max) return BQI_ESHAPE;
  hipStream_t s = as_stream(stream);
  if (k == 0) {
    // nothing to quantize; y is an empty sum
    if (n == 0) return BQI_OK;
    if (!y) return BQI_EINVAL;
    if (!aligned(y, 4)) return BQI_EALIGN;
    return hip_status(bqi::launch_zero_f32(y, m * n, s));
  }
  if (!x || !q || !d) return BQI_EINVAL;
  if (n > 0 && (!wq || !wd || !y)) return BQI_EINVAL;
  const int64_t esize = x_dtype == BQI_F32 ? 4 : 2;
  const int64_t vec = x_dtype == BQI_F32 ? 16 : 8;
  if (!aligned(x, 16) || (ldx * esize) % vec != 0 || !aligned(q, 16) ||
      !aligned(d, 2))
    return BQI_EALIGN;
  if (n > 0 && (!aligned(wq, 16) || !aligned(wd, 2) || !aligned(y, 4)))
    return BQI_EALIGN;
  if (m > 16 && ((m + 127) / 128 * ((n + 127) / 128) > kI32Max ||
                 m * k > kI32Max || n * k > kI32Max))
    return BQI_ESHAPE;
  if (n > 0 && m <= 16 && bqi::gemv_fused_supported(m, n, k, wd) && ldx <= kI32Max)
    return hip_status(bqi::launch_gemv_fused(x, x_dtype == BQI_F16, ldx, m, wq,
                                             wd, n, k, y, q, d, s));
  const int st = hip_status(bqi::launch_quantize_q8_0(x, x_dtype == BQI_F16, m,
                                                      k, ldx, q, d, s));
  if (st != BQI_OK || n == 0) return st;
  return qgemm_launch(q, d, m, wq, wd, n, k, y, s);
}

int route_topk(const int32_t *topk_ids, int64_t n_tokens, int64_t top_k,
               int64_t n_experts, int32_t *counts, int32_t *offsets,
               int32_t *rows, void *stream) {
  if (n_tokens < 0 || top_k < 0 || n_experts < 0) return BQI_ESHAPE;
  if (n_experts > 65536 || n_tokens * top_k > kMaxRouted) return BQI_ESHAPE;
  if (n_experts == 0) return BQI_OK;
  if (!counts || !offsets) return BQI_EINVAL;
  if (n_tokens * top_k > 0 && (!topk_ids || !rows)) return BQI_EINVAL;
  if (!aligned(topk_ids, 4) || !aligned(counts, 4) || !aligned(offsets, 4) ||
      !aligned(rows, 4))
    return BQI_EALIGN;
  return hip_status(bqi::launch_route_topk(topk_ids, n_tokens * top_k,
                                           n_experts, top_k, counts, offsets,
                                           rows, nullptr, 0, as_stream(stream)));
}

size_t qgemm_w4a8_grouped_workspace_size(int64_t n_tokens, int64_t top_k,
                                         int64_t n_experts, int64_t k) {
  if (n_tokens < 0 || top_k < 0 || n_experts < 0 || k < 0 || k % kQK != 0)
    return 0;
  if (n_experts > 65536 || n_tokens * top_k > kMaxRouted || k > kI32Max)
    return 0;
  return ws_layout(n_tokens * top_k, n_experts, k).total;
}

int qgemm_w4a8_grouped(const int8_t *aq, const uint16_t *ad, int64_t n_tokens,
                       const int32_t *topk_ids, int64_t top_k,
                       const uint8_t *wq4, const uint16_t *wd,
                       int64_t n_experts, int64_t n, int64_t k, float *y,
                       void *workspace, size_t workspace_bytes, void *stream) {
  return grouped_impl(aq, ad, n_tokens, topk_ids, top_k, wq4, wd, n_experts, n,
                      k, y, workspace, workspace_bytes, false, stream);
}

int qgemm_w4a8_grouped_noalloc(const int8_t *aq, const uint16_t *ad,
                               int64_t n_tokens, const int32_t *topk_ids,
                               int64_t top_k, const uint8_t *wq4,
                               const uint16_t *wd, int64_t n_experts,
                               int64_t n, int64_t k, float *y, void *stream) {
  return grouped_impl(aq, ad, n_tokens, topk_ids, top_k, wq4, wd, n_experts, n,
                      k, y, nullptr, 0, true, stream);
}

int moe_combine_f32(const float *y, const float *p, int64_t n_tokens,
                    int64_t top_k, int64_t n, float *out, void *stream) {
  if (n_tokens < 0 || top_k < 0 || n < 0) return BQI_ESHAPE;
  if (n_tokens > kI32Max || top_k > 65536 || n > kI32Max ||
      n_tokens * top_k > kI32Max || n_tokens * top_k * n > ((int64_t)1 << 40))
    return BQI_ESHAPE;
  if (n_tokens == 0 || n == 0) return BQI_OK;
  if (!out) return BQI_EINVAL;
  if (!aligned(out, 4)) return BQI_EALIGN;
  if (top_k == 0)  // empty sum
    return hip_status(bqi::launch_zero_f32(out, n_tokens * n, as_stream(stream)));
  if (!y || !p) return BQI_EINVAL;
  if (!aligned(y, 4) || !aligned(p, 4)) return BQI_EALIGN;
  return hip_status(bqi::launch_moe_combine(y, p, n_tokens, top_k, n, out,
                                            as_stream(stream)));
}

namespace {

int gguf_check(const void *blocks, int64_t rows, int64_t k, const void *codes,
               const void *scales) {
  if (rows < 0 || k < 0 || k % kQK != 0) return BQI_ESHAPE;
  if (rows > kI32Max || k > kI32Max || rows * (k / kQK) > ((int64_t)1 << 36))
    return BQI_ESHAPE;
  if (rows == 0 || k == 0) return BQI_OK;
  if (!blocks || !codes || !scales) return BQI_EINVAL;
  if (!aligned(blocks, 16) || !aligned(codes, 16) || !aligned(scales, 2))
    return BQI_EALIGN;
  return 1;  // valid and non-empty
}

}  // namespace

int gguf_q8_0_to_planar(const void *blocks, int64_t rows, int64_t k, int8_t *q,
                        uint16_t *d, void *stream) {
  const int st = gguf_check(blocks, rows, k, q, d);
  if (st != 1) return st;
  return hip_status(bqi::launch_gguf_q8_0(blocks, rows * (k / kQK), q, d,
                                          as_stream(stream)));
}

int gguf_q4_0_to_planar(const void *blocks, int64_t rows, int64_t k,
                        uint8_t *wq4, uint16_t *wd, void *stream) {
  const int st = gguf_check(blocks, rows, k, wq4, wd);
  if (st != 1) return st;
  return hip_status(bqi::launch_gguf_q4_0(blocks, rows * (k / kQK), wq4, wd,
                                          as_stream(stream)));
}

}  // extern "C"
