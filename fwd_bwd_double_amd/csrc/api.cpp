// C ABI of libfbd.so (declared in include/fbd.h): argument validation, then
// the kernel launches.  Every check runs before anything is enqueued, so a
// call that returns an error has written nothing.  There is no fallback.
#include <hip/hip_runtime.h>

#include <climits>
#include <cmath>
#include <cstdint>
#include <mutex>
#include <vector>

#include "../../include/fbd.h"
#include "launch.hpp"

namespace {

thread_local int g_last_hip_error = 0;

struct Span {
  uintptr_t lo, hi;   // [lo, hi)
};

bool overlaps(const Span& a, const Span& b) { return a.lo < b.hi && b.lo < a.hi; }

size_t elem_size(attn_dtype dt) { return dt == ATTN_BF16 ? 2 : 4; }

// Shape checks shared by all entry points.  The kernels index one head's
// N x 64 matrix with 32-bit integers and launch ceil(N/128) * B * H
// workgroups on a 1-D grid.
attn_status check_shape(attn_dtype dt, int64_t B, int64_t H, int64_t N, int64_t d, float scale) {
  if (dt != ATTN_BF16 && dt != ATTN_F32) return ATTN_EUNSUPPORTED;
  if (B <= 0 || H <= 0 || N <= 0 || d <= 0) return ATTN_EINVAL;
  if (d != 64) return ATTN_EUNSUPPORTED;
  if (!std::isfinite(scale) || !(scale > 0.f)) return ATTN_EINVAL;
  if (N > (int64_t)INT_MAX / 64) return ATTN_EUNSUPPORTED;
  if (B > INT_MAX || H > INT_MAX) return ATTN_EUNSUPPORTED;
  const int64_t bh = B * H;
  if (bh > INT_MAX) return ATTN_EUNSUPPORTED;
  if (bh > (int64_t)INT_MAX / N) return ATTN_EUNSUPPORTED;     // B*H*N fits int
  const int64_t nblk = (N + 127) / 128;
  if (bh > (int64_t)INT_MAX / nblk) return ATTN_EUNSUPPORTED;  // grid size
  // tiles are fetched through buffer resources with 32-bit byte offsets that
  // may run one tile past the head's last row
  const int64_t head_bytes = N * 64 * (dt == ATTN_BF16 ? 2 : 4);
  if (head_bytes + (int64_t)(1 << 20) > (int64_t)UINT32_MAX) return ATTN_EUNSUPPORTED;
  return ATTN_OK;
}

// Key/value heads: 1 <= Hkv <= H and H a multiple of Hkv.
attn_status check_heads(int64_t H, int64_t Hkv) {
  if (Hkv <= 0 || Hkv > H || H % Hkv != 0) return ATTN_EINVAL;
  return ATTN_OK;
}

// Sliding window: 0 = none; w > 0 keeps keys i - w < j <= i and needs the
// causal mask.  The kernels take a window of 2^30 (beyond any N) for none.
constexpr int kNoWindow = 1 << 30;
attn_status check_window(int causal, int64_t window, int* win) {
  if (window < 0) return ATTN_EINVAL;
  if (window > 0 && !causal) return ATTN_EUNSUPPORTED;
  *win = (window == 0 || window >= kNoWindow) ? kNoWindow : (int)window;
  return ATTN_OK;
}

struct Arg {
  const void* p;
  size_t bytes;
};

// Document starts: an int32 (B, N) input, 4-byte aligned, causal only, and
// disjoint from every output.
attn_status check_docs(const int32_t* ds, int causal, int64_t B, int64_t N,
                       const std::vector<Arg>& outs) {
  if (!ds) return ATTN_OK;
  if (!causal) return ATTN_EUNSUPPORTED;
  if (reinterpret_cast<uintptr_t>(ds) % 4) return ATTN_EALIGN;
  const uintptr_t lo = reinterpret_cast<uintptr_t>(ds), hi = lo + (size_t)B * N * 4;
  for (const Arg& a : outs) {
    const uintptr_t olo = reinterpret_cast<uintptr_t>(a.p), ohi = olo + a.bytes;
    if (olo < hi && lo < ohi) return ATTN_EINVAL;
  }
  return ATTN_OK;
}

// Block-sparse mask: a (B, ceil(N/128), ceil(N/128)) byte input, disjoint
// from every output (any alignment; causal or not).
attn_status check_block_mask(const uint8_t* bm, int64_t B, int64_t N,
                             const std::vector<Arg>& outs) {
  if (!bm) return ATTN_OK;
  const int64_t nb = (N + 127) / 128;
  const uintptr_t lo = reinterpret_cast<uintptr_t>(bm), hi = lo + (size_t)(B * nb * nb);
  for (const Arg& a : outs) {
    const uintptr_t olo = reinterpret_cast<uintptr_t>(a.p), ohi = olo + a.bytes;
    if (olo < hi && lo < ohi) return ATTN_EINVAL;
  }
  return ATTN_OK;
}

// Null, alignment and overlap checks.  `ins` are read-only, `outs` written.
attn_status check_ptrs(const std::vector<Arg>& ins, const std::vector<Arg>& outs) {
  for (const Arg& a : ins) {
    if (!a.p) return ATTN_EINVAL;
    if (reinterpret_cast<uintptr_t>(a.p) % 16) return ATTN_EALIGN;
  }
  for (const Arg& a : outs) {
    if (!a.p) return ATTN_EINVAL;
    if (reinterpret_cast<uintptr_t>(a.p) % 16) return ATTN_EALIGN;
  }
  for (size_t i = 0; i < outs.size(); ++i) {
    const Span so{reinterpret_cast<uintptr_t>(outs[i].p),
                  reinterpret_cast<uintptr_t>(outs[i].p) + outs[i].bytes};
    for (const Arg& a : ins) {
      const Span si{reinterpret_cast<uintptr_t>(a.p), reinterpret_cast<uintptr_t>(a.p) + a.bytes};
      if (overlaps(so, si)) return ATTN_EINVAL;
    }
    for (size_t k = i + 1; k < outs.size(); ++k) {
      const Span sk{reinterpret_cast<uintptr_t>(outs[k].p),
                    reinterpret_cast<uintptr_t>(outs[k].p) + outs[k].bytes};
      if (overlaps(so, sk)) return ATTN_EINVAL;
    }
  }
  return ATTN_OK;
}

// Column-pass slices for grouped-query heads.  A column-pass workgroup owns
// a (key block, key head) pair and streams all grp query heads of the group;
// at few key heads that leaves too few, too long workgroups for 256 CUs (and
// the causal blocks' unequal lengths no longer even out).  The smallest
// divisor nsl of grp that gives at least 1536 workgroups (six per CU) splits
// each group into nsl slices of query heads (nsl = grp when none does); the
// slices write fp32 partial sums that one more kernel adds up.
int col_slices(int64_t B, int64_t H, int64_t Hkv, int64_t N) {
  const int64_t grp = H / Hkv;
  const int64_t wgs = (N + 127) / 128 * B * Hkv;
  for (int64_t s = 1; s < grp; ++s)
    if (grp % s == 0 && wgs * s >= 1536) return (int)s;
  return (int)grp;
}
// Bytes of the partial sums of nsl slices (two fp32 key-side tensors each),
// placed after the row states at a 256-byte boundary.
size_t part_bytes(int64_t B, int64_t Hkv, int64_t N, int nsl) {
  return nsl > 1 ? (size_t)2 * nsl * (size_t)B * Hkv * N * 64 * sizeof(float) : 0;
}
size_t round256(size_t x) { return (x + 255) & ~(size_t)255; }

attn_status finish(hipError_t e) {
  if (e != hipSuccess) {
    g_last_hip_error = (int)e;
    return ATTN_EHIP;
  }
  return ATTN_OK;
}

}  // namespace

extern "C" {

const char* attn_status_str(attn_status s) {
  switch (s) {
    case ATTN_OK: return "ok";
    case ATTN_EINVAL: return "invalid argument";
    case ATTN_EUNSUPPORTED: return "unsupported dtype or shape";
    case ATTN_EALIGN: return "pointer not 16-byte aligned";
    case ATTN_EWORKSPACE: return "workspace missing or too small";
    case ATTN_EHIP: return "HIP kernel launch failed";
  }
  return "unknown status";
}

int attn_last_hip_error(void) { return g_last_hip_error; }

size_t attn_bwd_workspace_bytes(int64_t B, int64_t H, int64_t N) {
  if (B <= 0 || H <= 0 || N <= 0) return 0;
  return (size_t)3 * (size_t)B * (size_t)H * (size_t)N * sizeof(float);
}

size_t attn_bob_workspace_bytes(int64_t B, int64_t H, int64_t N) {
  if (B <= 0 || H <= 0 || N <= 0) return 0;
  return (size_t)5 * (size_t)B * (size_t)H * (size_t)N * sizeof(float);
}

size_t attn_bwd_ex_workspace_bytes(int64_t B, int64_t H, int64_t Hkv, int64_t N) {
  if (B <= 0 || H <= 0 || N <= 0 || check_heads(H, Hkv) != ATTN_OK) return 0;
  const size_t base = attn_bwd_workspace_bytes(B, H, N);
  const int nsl = col_slices(B, H, Hkv, N);
  return nsl > 1 ? round256(base) + part_bytes(B, Hkv, N, nsl) : base;
}

size_t attn_bob_ex_workspace_bytes(int64_t B, int64_t H, int64_t Hkv, int64_t N) {
  if (B <= 0 || H <= 0 || N <= 0 || check_heads(H, Hkv) != ATTN_OK) return 0;
  const size_t base = attn_bob_workspace_bytes(B, H, N);
  const int nsl = col_slices(B, H, Hkv, N);
  return nsl > 1 ? round256(base) + part_bytes(B, Hkv, N, nsl) : base;
}

attn_status attn_fwd_ex(attn_dtype dt, int64_t B, int64_t H, int64_t Hkv, int64_t N, int64_t d,
                        const void* Q, const void* K, const void* V, int causal, int64_t window,
                        const int32_t* doc_start, const uint8_t* block_mask, float scale,
                        void* O, float* LSE, void* stream) {
  attn_status st = check_shape(dt, B, H, N, d, scale);
  if (st != ATTN_OK) return st;
  if ((st = check_heads(H, Hkv)) != ATTN_OK) return st;
  int win = 0;
  if ((st = check_window(causal, window, &win)) != ATTN_OK) return st;
  const size_t t = (size_t)B * H * N * d * elem_size(dt), s = (size_t)B * H * N * sizeof(float);
  const size_t tk = (size_t)B * Hkv * N * d * elem_size(dt);
  st = check_ptrs({{Q, t}, {K, tk}, {V, tk}}, {{O, t}, {LSE, s}});
  if (st != ATTN_OK) return st;
  if ((st = check_docs(doc_start, causal, B, N, {{O, t}, {LSE, s}})) != ATTN_OK) return st;
  if ((st = check_block_mask(block_mask, B, N, {{O, t}, {LSE, s}})) != ATTN_OK) return st;
  return finish(fbd::launch_fwd((int)dt, Q, K, V, O, LSE, (int)(B * H), (int)H, (int)(H / Hkv),
                                win, doc_start, block_mask, (int)N, causal ? 1 : 0, scale,
                                (hipStream_t)stream));
}

attn_status attn_fwd(attn_dtype dt, int64_t B, int64_t H, int64_t N, int64_t d, const void* Q,
                     const void* K, const void* V, int causal, float scale, void* O, float* LSE,
                     void* stream) {
  return attn_fwd_ex(dt, B, H, H, N, d, Q, K, V, causal, 0, nullptr, nullptr, scale, O, LSE,
                     stream);
}

static attn_status bwd_impl(int passes, attn_dtype dt, int64_t B, int64_t H, int64_t Hkv,
                            int64_t N, int64_t d, const void* Q, const void* K, const void* V,
                            const void* O, const float* LSE, const void* dO, int causal,
                            int64_t window, const int32_t* doc_start,
                            const uint8_t* block_mask, float scale, int gproj, void* dQ,
                            void* dK, void* dV, void* ws, size_t ws_bytes, void* stream) {
  if (passes < 1 || passes > 3) return ATTN_EINVAL;
  attn_status st = check_shape(dt, B, H, N, d, scale);
  if (st != ATTN_OK) return st;
  if ((st = check_heads(H, Hkv)) != ATTN_OK) return st;
  int win = 0;
  if ((st = check_window(causal, window, &win)) != ATTN_OK) return st;
  size_t need = attn_bwd_workspace_bytes(B, H, N);
  if (!ws || ws_bytes < need) return ATTN_EWORKSPACE;
  // split column pass when the workspace also holds the partial sums
  int nsl = col_slices(B, H, Hkv, N);
  const size_t poff = round256(need);
  if (nsl > 1 && ws_bytes >= poff + part_bytes(B, Hkv, N, nsl)) need = poff + part_bytes(B, Hkv, N, nsl);
  else nsl = 1;
  const size_t t = (size_t)B * H * N * d * elem_size(dt), s = (size_t)B * H * N * sizeof(float);
  const size_t tk = (size_t)B * Hkv * N * d * elem_size(dt);
  st = check_ptrs({{Q, t}, {K, tk}, {V, tk}, {O, t}, {LSE, s}, {dO, t}},
                  {{dQ, t}, {dK, tk}, {dV, tk}, {ws, need}});
  if (st != ATTN_OK) return st;
  st = check_docs(doc_start, causal, B, N, {{dQ, t}, {dK, tk}, {dV, tk}, {ws, need}});
  if (st != ATTN_OK) return st;
  st = check_block_mask(block_mask, B, N, {{dQ, t}, {dK, tk}, {dV, tk}, {ws, need}});
  if (st != ATTN_OK) return st;
  const size_t bhn = (size_t)B * H * N;
  float* Dws = static_cast<float*>(ws);
  float* Rws = Dws + bhn;
  float* Lws = Rws + bhn;
  return finish(fbd::launch_bwd((int)dt, Q, K, V, O, LSE, dO, dQ, dK, dV, Dws, Rws, Lws,
                                (int)(B * H), (int)H, (int)(H / Hkv), win, doc_start, block_mask,
                                (int)N, causal ? 1 : 0, scale, gproj ? 1 : 0, passes, nsl,
                                nsl > 1 ? (float*)((char*)ws + poff) : nullptr,
                                (hipStream_t)stream));
}

attn_status attn_bwd_passes(int passes, attn_dtype dt, int64_t B, int64_t H, int64_t N, int64_t d,
                            const void* Q, const void* K, const void* V, const void* O,
                            const float* LSE, const void* dO, int causal, float scale, int gproj,
                            void* dQ, void* dK, void* dV, void* ws, size_t ws_bytes,
                            void* stream) {
  return bwd_impl(passes, dt, B, H, H, N, d, Q, K, V, O, LSE, dO, causal, 0, nullptr, nullptr,
                  scale, gproj, dQ, dK, dV, ws, ws_bytes, stream);
}

attn_status attn_bwd_ex(attn_dtype dt, int64_t B, int64_t H, int64_t Hkv, int64_t N, int64_t d,
                        const void* Q, const void* K, const void* V, const void* O,
                        const float* LSE, const void* dO, int causal, int64_t window,
                        const int32_t* doc_start, const uint8_t* block_mask, float scale,
                        int gproj, void* dQ, void* dK, void* dV, void* ws, size_t ws_bytes,
                        void* stream) {
  return bwd_impl(3, dt, B, H, Hkv, N, d, Q, K, V, O, LSE, dO, causal, window, doc_start,
                  block_mask, scale, gproj, dQ, dK, dV, ws, ws_bytes, stream);
}

attn_status attn_bwd(attn_dtype dt, int64_t B, int64_t H, int64_t N, int64_t d, const void* Q,
                     const void* K, const void* V, const void* O, const float* LSE,
                     const void* dO, int causal, float scale, int gproj, void* dQ, void* dK,
                     void* dV, void* ws, size_t ws_bytes, void* stream) {
  return attn_bwd_passes(3, dt, B, H, N, d, Q, K, V, O, LSE, dO, causal, scale, gproj, dQ, dK,
                         dV, ws, ws_bytes, stream);
}

static attn_status bob_impl(int passes, attn_dtype dt, int64_t B, int64_t H, int64_t Hkv,
                            int64_t N, int64_t d, const void* Q, const void* K, const void* V,
                            const void* O, const float* LSE, const void* dO, const void* g_dQ,
                            const void* g_dK, const void* g_dV, int causal, int64_t window,
                            const int32_t* doc_start, const uint8_t* block_mask, float scale,
                            int gproj, void* g_Q, void* g_K, void* g_V, void* g_dO, void* ws,
                            size_t ws_bytes, void* stream) {
  if (passes < 1 || passes > 3) return ATTN_EINVAL;
  attn_status st = check_shape(dt, B, H, N, d, scale);
  if (st != ATTN_OK) return st;
  if ((st = check_heads(H, Hkv)) != ATTN_OK) return st;
  int win = 0;
  if ((st = check_window(causal, window, &win)) != ATTN_OK) return st;
  size_t need = attn_bob_workspace_bytes(B, H, N);
  if (!ws || ws_bytes < need) return ATTN_EWORKSPACE;
  // split column pass when the workspace also holds the partial sums
  int nsl = col_slices(B, H, Hkv, N);
  const size_t poff = round256(need);
  if (nsl > 1 && ws_bytes >= poff + part_bytes(B, Hkv, N, nsl)) need = poff + part_bytes(B, Hkv, N, nsl);
  else nsl = 1;
  const size_t t = (size_t)B * H * N * d * elem_size(dt), s = (size_t)B * H * N * sizeof(float);
  const size_t tk = (size_t)B * Hkv * N * d * elem_size(dt);
  st = check_ptrs({{Q, t}, {K, tk}, {V, tk}, {O, t}, {LSE, s}, {dO, t}, {g_dQ, t}, {g_dK, tk},
                   {g_dV, tk}},
                  {{g_Q, t}, {g_K, tk}, {g_V, tk}, {g_dO, t}, {ws, need}});
  if (st != ATTN_OK) return st;
  st = check_docs(doc_start, causal, B, N,
                  {{g_Q, t}, {g_K, tk}, {g_V, tk}, {g_dO, t}, {ws, need}});
  if (st != ATTN_OK) return st;
  st = check_block_mask(block_mask, B, N,
                        {{g_Q, t}, {g_K, tk}, {g_V, tk}, {g_dO, t}, {ws, need}});
  if (st != ATTN_OK) return st;
  const size_t bhn = (size_t)B * H * N;
  float* Dws = static_cast<float*>(ws);
  float* Aws = Dws + bhn;
  float* Bws = Aws + bhn;
  float* Lws = Bws + bhn;
  float* Kws = Lws + bhn;
  return finish(fbd::launch_bob((int)dt, Q, K, V, O, LSE, dO, g_dQ, g_dK, g_dV, g_Q, g_K, g_V,
                                g_dO, Dws, Aws, Bws, Lws, Kws, (int)(B * H), (int)H,
                                (int)(H / Hkv), win, doc_start, block_mask, (int)N,
                                causal ? 1 : 0, scale, passes, nsl,
                                nsl > 1 ? (float*)((char*)ws + poff) : nullptr, gproj ? 1 : 0,
                                (hipStream_t)stream));
}

attn_status attn_bob_passes(int passes, attn_dtype dt, int64_t B, int64_t H, int64_t N, int64_t d,
                            const void* Q, const void* K, const void* V, const void* O,
                            const float* LSE, const void* dO, const void* g_dQ, const void* g_dK,
                            const void* g_dV, int causal, float scale, void* g_Q, void* g_K,
                            void* g_V, void* g_dO, void* ws, size_t ws_bytes, void* stream) {
  return bob_impl(passes, dt, B, H, H, N, d, Q, K, V, O, LSE, dO, g_dQ, g_dK, g_dV, causal, 0,
                  nullptr, nullptr, scale, 0, g_Q, g_K, g_V, g_dO, ws, ws_bytes, stream);
}

attn_status attn_bob_ex(attn_dtype dt, int64_t B, int64_t H, int64_t Hkv, int64_t N, int64_t d,
                        const void* Q, const void* K, const void* V, const void* O,
                        const float* LSE, const void* dO, const void* g_dQ, const void* g_dK,
                        const void* g_dV, int causal, int64_t window,
                        const int32_t* doc_start, const uint8_t* block_mask, float scale,
                        int gproj, void* g_Q, void* g_K, void* g_V, void* g_dO, void* ws,
                        size_t ws_bytes, void* stream) {
  return bob_impl(3, dt, B, H, Hkv, N, d, Q, K, V, O, LSE, dO, g_dQ, g_dK, g_dV, causal, window,
                  doc_start, block_mask, scale, gproj, g_Q, g_K, g_V, g_dO, ws, ws_bytes, stream);
}

attn_status attn_bob(attn_dtype dt, int64_t B, int64_t H, int64_t N, int64_t d, const void* Q,
                     const void* K, const void* V, const void* O, const float* LSE,
                     const void* dO, const void* g_dQ, const void* g_dK, const void* g_dV,
                     int causal, float scale, void* g_Q, void* g_K, void* g_V, void* g_dO,
                     void* ws, size_t ws_bytes, void* stream) {
  return attn_bob_passes(3, dt, B, H, N, d, Q, K, V, O, LSE, dO, g_dQ, g_dK, g_dV, causal, scale,
                         g_Q, g_K, g_V, g_dO, ws, ws_bytes, stream);
}

// BoB's five row states and the backward's GProj row sums r
size_t attn_hvp_workspace_bytes(int64_t B, int64_t H, int64_t N) {
  if (B <= 0 || H <= 0 || N <= 0) return 0;
  return (size_t)6 * (size_t)B * (size_t)H * (size_t)N * sizeof(float);
}

size_t attn_hvp_ex_workspace_bytes(int64_t B, int64_t H, int64_t Hkv, int64_t N) {
  if (B <= 0 || H <= 0 || N <= 0 || check_heads(H, Hkv) != ATTN_OK) return 0;
  const size_t base = attn_hvp_workspace_bytes(B, H, N);
  const int nsl = col_slices(B, H, Hkv, N);
  return nsl > 1 ? round256(base) + part_bytes(B, Hkv, N, nsl) : base;
}

attn_status attn_hvp_ex(attn_dtype dt, int64_t B, int64_t H, int64_t Hkv, int64_t N, int64_t d,
                        const void* Q, const void* K, const void* V, const void* dO,
                        const void* v_Q, const void* v_K, const void* v_V, int causal,
                        int64_t window, const int32_t* doc_start, const uint8_t* block_mask,
                        float scale, int gproj, void* O, float* LSE, void* dQ, void* dK,
                        void* dV, void* Hv_Q, void* Hv_K, void* Hv_V, void* Hv_dO, void* ws,
                        size_t ws_bytes, void* stream) {
  attn_status st = check_shape(dt, B, H, N, d, scale);
  if (st != ATTN_OK) return st;
  if ((st = check_heads(H, Hkv)) != ATTN_OK) return st;
  int win = 0;
  if ((st = check_window(causal, window, &win)) != ATTN_OK) return st;
  const int ngrad = (dQ != nullptr) + (dK != nullptr) + (dV != nullptr);
  if (ngrad != 0 && ngrad != 3) return ATTN_EINVAL;
  // BoB's row states (D, alpha, beta, -LSE log2(e), -kappa) and the
  // backward's r fill the front of the workspace; the split column passes'
  // partial sums, when the workspace holds them, follow
  size_t need = attn_hvp_workspace_bytes(B, H, N);
  if (!ws || ws_bytes < need) return ATTN_EWORKSPACE;
  int nsl = col_slices(B, H, Hkv, N);
  const size_t poff = round256(need);
  if (nsl > 1 && ws_bytes >= poff + part_bytes(B, Hkv, N, nsl)) need = poff + part_bytes(B, Hkv, N, nsl);
  else nsl = 1;
  const size_t t = (size_t)B * H * N * d * elem_size(dt), s = (size_t)B * H * N * sizeof(float);
  const size_t tk = (size_t)B * Hkv * N * d * elem_size(dt);
  std::vector<Arg> outs = {{O, t}, {LSE, s}, {Hv_Q, t}, {Hv_K, tk}, {Hv_V, tk}, {Hv_dO, t},
                           {ws, need}};
  if (ngrad == 3) {
    outs.push_back({dQ, t});
    outs.push_back({dK, tk});
    outs.push_back({dV, tk});
  }
  st = check_ptrs({{Q, t}, {K, tk}, {V, tk}, {dO, t}, {v_Q, t}, {v_K, tk}, {v_V, tk}}, outs);
  if (st != ATTN_OK) return st;
  if ((st = check_docs(doc_start, causal, B, N, outs)) != ATTN_OK) return st;
  if ((st = check_block_mask(block_mask, B, N, outs)) != ATTN_OK) return st;
  const int bh = (int)(B * H), n = (int)N, c = causal ? 1 : 0, h = (int)H, grp = (int)(H / Hkv);
  const hipStream_t hs = (hipStream_t)stream;
  const size_t bhn = (size_t)B * H * N;
  float* w0 = static_cast<float*>(ws);
  float* part = nsl > 1 ? (float*)((char*)ws + poff) : nullptr;
  float *Dw = w0, *Aw = w0 + bhn, *Bw = w0 + 2 * bhn, *Lw = w0 + 3 * bhn, *Kw = w0 + 4 * bhn,
        *Rw = w0 + 5 * bhn;
  const int gp = gproj ? 1 : 0;
  hipError_t e = fbd::launch_fwd((int)dt, Q, K, V, O, LSE, bh, h, grp, win, doc_start,
                                 block_mask, n, c, scale, hs);
  if (ngrad == 3 && dt == ATTN_BF16) {
    // bf16 with the gradient: one row pass for both (its R(dS) K and R(P) K
    // products are the backward's dQ terms), then the two column passes
    if (e == hipSuccess)
      e = fbd::launch_bob_row_grad(Q, K, V, O, LSE, dO, v_Q, v_K, v_V, Hv_Q, Hv_dO, dQ, Dw, Aw,
                                   Bw, Lw, Kw, Rw, bh, h, grp, win, doc_start, block_mask, n, c,
                                   scale, gp, gp, hs);
    if (e == hipSuccess)
      e = fbd::launch_bwd((int)dt, Q, K, V, O, LSE, dO, dQ, dK, dV, Dw, Rw, Lw, bh, h, grp, win,
                          doc_start, block_mask, n, c, scale, gp, 2, nsl, part, hs);
    if (e == hipSuccess)
      e = fbd::launch_bob((int)dt, Q, K, V, O, LSE, dO, v_Q, v_K, v_V, Hv_Q, Hv_K, Hv_V, Hv_dO,
                          Dw, Aw, Bw, Lw, Kw, bh, h, grp, win, doc_start, block_mask, n, c, scale,
                          2, nsl, part, gp, hs);
    return finish(e);
  }
  if (e == hipSuccess && ngrad == 3)
    e = fbd::launch_bwd((int)dt, Q, K, V, O, LSE, dO, dQ, dK, dV, Dw, Rw, Lw, bh, h, grp, win,
                        doc_start, block_mask, n, c, scale, gp, 3, nsl, part, hs);
  if (e == hipSuccess)
    e = fbd::launch_bob((int)dt, Q, K, V, O, LSE, dO, v_Q, v_K, v_V, Hv_Q, Hv_K, Hv_V, Hv_dO, Dw,
                        Aw, Bw, Lw, Kw, bh, h, grp, win, doc_start, block_mask, n, c, scale, 3,
                        nsl, part, gp, hs);
  return finish(e);
}

attn_status attn_hvp(attn_dtype dt, int64_t B, int64_t H, int64_t N, int64_t d, const void* Q,
                     const void* K, const void* V, const void* dO, const void* v_Q,
                     const void* v_K, const void* v_V, int causal, float scale, int gproj,
                     void* O, float* LSE, void* dQ, void* dK, void* dV, void* Hv_Q, void* Hv_K,
                     void* Hv_V, void* Hv_dO, void* ws, size_t ws_bytes, void* stream) {
  return attn_hvp_ex(dt, B, H, H, N, d, Q, K, V, dO, v_Q, v_K, v_V, causal, 0, nullptr, nullptr,
                     scale, gproj, O, LSE, dQ, dK, dV, Hv_Q, Hv_K, Hv_V, Hv_dO, ws, ws_bytes,
                     stream);
}

}  // extern "C"

namespace {

struct F8Layout {
  size_t off[ATTN_FP8_NPARTS];
  size_t total;
};

F8Layout fp8_layout(int64_t B, int64_t H, int64_t Hkv, int64_t N) {
  const size_t nb = (size_t)(N + 63) / 64, np = nb * 64;
  const size_t bh = (size_t)B * H, bhk = (size_t)B * Hkv;
  const size_t bytes[ATTN_FP8_NPARTS] = {bh * N * 64, bhk * N * 64, bhk * 64 * np,
                                         bh * nb * 4, bhk * nb * 4, bhk * 64 * 4, bhk * 64 * 4};
  F8Layout L;
  size_t off = 0;
  for (int i = 0; i < ATTN_FP8_NPARTS; ++i) {
    L.off[i] = off;
    off = (off + bytes[i] + 255) & ~(size_t)255;
  }
  L.total = off;
  return L;
}

// Shape checks of the FP8 entry points (the V code rows take N rounded up to
// 64, still within 32-bit offsets).
attn_status fp8_shape(attn_dtype dt, int64_t B, int64_t H, int64_t Hkv, int64_t N, int64_t d,
                      float scale) {
  attn_status st = check_shape(dt, B, H, N, d, scale);
  if (st != ATTN_OK) return st;
  return check_heads(H, Hkv);
}

}  // namespace

extern "C" {

size_t attn_fp8_workspace_bytes(int64_t B, int64_t H, int64_t Hkv, int64_t N) {
  if (B <= 0 || H <= 0 || Hkv <= 0 || N <= 0) return 0;
  return fp8_layout(B, H, Hkv, N).total;
}

attn_status attn_fp8_workspace_layout(int64_t B, int64_t H, int64_t Hkv, int64_t N,
                                      size_t* offsets) {
  if (!offsets) return ATTN_EINVAL;
  if (fp8_shape(ATTN_BF16, B, H, Hkv, N, 64, 1.f) != ATTN_OK) return ATTN_EINVAL;
  const F8Layout L = fp8_layout(B, H, Hkv, N);
  for (int i = 0; i < ATTN_FP8_NPARTS; ++i) offsets[i] = L.off[i];
  return ATTN_OK;
}

attn_status attn_fp8_quantize(attn_dtype dt, int64_t B, int64_t H, int64_t Hkv, int64_t N,
                              int64_t d, const void* Q, const void* K, const void* V, int rotate,
                              uint64_t signs, void* ws, size_t ws_bytes, void* stream) {
  attn_status st = fp8_shape(dt, B, H, Hkv, N, d, 1.f);
  if (st != ATTN_OK) return st;
  const F8Layout L = fp8_layout(B, H, Hkv, N);
  if (!ws || ws_bytes < L.total) return ATTN_EWORKSPACE;
  const size_t t = (size_t)B * H * N * d * elem_size(dt);
  const size_t tk = (size_t)B * Hkv * N * d * elem_size(dt);
  st = check_ptrs({{Q, t}, {K, tk}, {V, tk}}, {{ws, L.total}});
  if (st != ATTN_OK) return st;
  char* w = static_cast<char*>(ws);
  return finish(fbd::launch_fp8_quantize(
      (int)dt, Q, K, V, (uint8_t*)(w + L.off[ATTN_FP8_Q]), (uint8_t*)(w + L.off[ATTN_FP8_K]),
      (uint8_t*)(w + L.off[ATTN_FP8_VT]), (int*)(w + L.off[ATTN_FP8_EQ]),
      (int*)(w + L.off[ATTN_FP8_EK]), (int*)(w + L.off[ATTN_FP8_EV]),
      (uint32_t*)(w + L.off[ATTN_FP8_VMAX]), (int)(B * H), (int)(B * Hkv), (int)N,
      rotate ? 1 : 0, signs, (hipStream_t)stream));
}

attn_status attn_fwd_fp8(attn_dtype dt, int64_t B, int64_t H, int64_t Hkv, int64_t N, int64_t d,
                         const void* ws, size_t ws_bytes, int causal, int64_t window,
                         const int32_t* doc_start, const uint8_t* block_mask, float scale,
                         void* O, float* LSE, void* stream) {
  attn_status st = fp8_shape(dt, B, H, Hkv, N, d, scale);
  if (st != ATTN_OK) return st;
  int win = 0;
  if ((st = check_window(causal, window, &win)) != ATTN_OK) return st;
  const F8Layout L = fp8_layout(B, H, Hkv, N);
  if (!ws || ws_bytes < L.total) return ATTN_EWORKSPACE;
  const size_t t = (size_t)B * H * N * d * elem_size(dt), s = (size_t)B * H * N * sizeof(float);
  st = check_ptrs({{ws, L.total}}, {{O, t}, {LSE, s}});
  if (st != ATTN_OK) return st;
  if ((st = check_docs(doc_start, causal, B, N, {{O, t}, {LSE, s}})) != ATTN_OK) return st;
  if ((st = check_block_mask(block_mask, B, N, {{O, t}, {LSE, s}})) != ATTN_OK) return st;
  const char* w = static_cast<const char*>(ws);
  return finish(fbd::launch_fwd_fp8(
      (int)dt, (const uint8_t*)(w + L.off[ATTN_FP8_Q]), (const uint8_t*)(w + L.off[ATTN_FP8_K]),
      (const uint8_t*)(w + L.off[ATTN_FP8_VT]), (const int*)(w + L.off[ATTN_FP8_EQ]),
      (const int*)(w + L.off[ATTN_FP8_EK]), (const int*)(w + L.off[ATTN_FP8_EV]), O, LSE,
      (int)(B * H), (int)H, (int)(H / Hkv), win, doc_start, block_mask, (int)N, causal ? 1 : 0,
      scale, (hipStream_t)stream));
}

}  // extern "C"

// ---------------------------------------------------------------------------
// Backward-over-backward without a caller workspace.  Its row states live in
// a file-scope device array, one copy per GPU the library runs on, held until
// the process ends.  Host code never passes the array's name to a kernel (in
// host code the name is a stand-in, not a device address): the device
// address comes from hipGetSymbolAddress, once per device, with that device
// current, and is kept per device.
static __device__ __align__(256) float scratch[ATTN_BOB_NOALLOC_MAX_ROWS * 5];

namespace {
constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
float* g_scratch[kMaxDevices] = {};

// Device address of `scratch` on the device `stream` belongs to (the current
// device for the null stream).
attn_status scratch_on(void* stream, float** out) {
  int dev = 0;
  hipError_t e = stream ? hipStreamGetDevice((hipStream_t)stream, &dev) : hipGetDevice(&dev);
  if (e != hipSuccess) return finish(e);
  if (dev < 0 || dev >= kMaxDevices) return ATTN_EINVAL;
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (!g_scratch[dev]) {
    int cur = 0;
    if ((e = hipGetDevice(&cur)) != hipSuccess) return finish(e);
    if (cur != dev && (e = hipSetDevice(dev)) != hipSuccess) return finish(e);
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    const hipError_t e2 = cur != dev ? hipSetDevice(cur) : hipSuccess;
    if (e != hipSuccess) return finish(e);
    if (e2 != hipSuccess) return finish(e2);
    if (!p) return ATTN_EHIP;
    g_scratch[dev] = static_cast<float*>(p);
  }
  *out = g_scratch[dev];
  return ATTN_OK;
}
}  // namespace

extern "C" attn_status attn_bob_noalloc(attn_dtype dt, int64_t B, int64_t H, int64_t N,
                                        int64_t d, const void* Q, const void* K, const void* V,
                                        const void* O, const float* LSE, const void* dO,
                                        const void* g_dQ, const void* g_dK, const void* g_dV,
                                        int causal, float scale, void* g_Q, void* g_K, void* g_V,
                                        void* g_dO, void* stream) {
  attn_status st = check_shape(dt, B, H, N, d, scale);
  if (st != ATTN_OK) return st;
  if ((uint64_t)B * (uint64_t)H * (uint64_t)N > (uint64_t)ATTN_BOB_NOALLOC_MAX_ROWS)
    return ATTN_EWORKSPACE;
  // the caller's pointers first, so argument errors are reported as such
  // before any device query
  const size_t t = (size_t)B * H * N * d * elem_size(dt), s = (size_t)B * H * N * sizeof(float);
  st = check_ptrs({{Q, t}, {K, t}, {V, t}, {O, t}, {LSE, s}, {dO, t}, {g_dQ, t}, {g_dK, t},
                   {g_dV, t}},
                  {{g_Q, t}, {g_K, t}, {g_V, t}, {g_dO, t}});
  if (st != ATTN_OK) return st;
  float* ws = nullptr;
  if ((st = scratch_on(stream, &ws)) != ATTN_OK) return st;
  // the multi-head workspace size: the unsplit column pass, as attn_bob with
  // attn_bob_workspace_bytes; every row state is written by the row pass
  // before the column pass reads it, so nothing needs clearing
  return bob_impl(3, dt, B, H, H, N, d, Q, K, V, O, LSE, dO, g_dQ, g_dK, g_dV, causal, 0,
                  nullptr, nullptr, scale, 0, g_Q, g_K, g_V, g_dO, ws,
                  attn_bob_workspace_bytes(B, H, N), stream);
}
