// C ABI of the shifted local-window attention library: argument validation, shift
// reduction, kernel selection. Every check runs before the first HIP call, so a bad
// argument never reaches the device. Declarations and contracts: include/basa.h.
#include <math.h>
#include <stdint.h>

#include <hip/hip_runtime_api.h>

#include "../../include/basa.h"
#include "attn_launch.hpp"
#include "index_map.hpp"

namespace {

constexpr int64_t kInt32Max = 0x7fffffff;
constexpr uint32_t kBf16HeadBytesMax = 0xffffff00u;

int reduce_mod(int s, int n) {
  const int r = s % n;  // in (-n, n)
  return r < 0 ? r + n : r;
}

bool aligned(const void* p, uintptr_t a) { return (reinterpret_cast<uintptr_t>(p) & (a - 1)) == 0; }

bool overlaps(const void* a, const void* b, int64_t bytes) {
  const uintptr_t x = reinterpret_cast<uintptr_t>(a), y = reinterpret_cast<uintptr_t>(b);
  return x < y + uint64_t(bytes) && y < x + uint64_t(bytes);
}

bool overlaps2(const void* a, int64_t abytes, const void* b, int64_t bbytes) {
  const uintptr_t x = reinterpret_cast<uintptr_t>(a), y = reinterpret_cast<uintptr_t>(b);
  return x < y + uint64_t(bbytes) && y < x + uint64_t(abytes);
}

int check_grid(int T, int H, int W, int wt, int wh, int ww) {
  if (T <= 0 || H <= 0 || W <= 0 || wt <= 0 || wh <= 0 || ww <= 0) return BASA_ERR_SHAPE;
  if (T % wt || H % wh || W % ww) return BASA_ERR_SHAPE;
  if (int64_t(T) * H * W > kInt32Max) return BASA_ERR_OVERFLOW;
  return BASA_OK;
}

// Memory (kmem, vmem, n_mem), lse and route are optional: n_mem = 0 with null kmem/vmem,
// null lse, null route.
int run_attention(const void* q, const void* k, const void* v, const int32_t* route, const void* kmem,
                  const void* vmem, int n_mem, void* out, float* lse, int B, int heads, int T, int H, int W, int wt,
                  int wh, int ww, int st, int sh, int sw, int head_dim, int dtype, hipStream_t stream,
                  bool no_alloc = false) {
  if (!q || !k || !v || !out) return BASA_ERR_NULL;
  if (n_mem < 0) return BASA_ERR_SHAPE;
  if (n_mem > 0 && (!kmem || !vmem)) return BASA_ERR_NULL;
  if (dtype != BASA_DTYPE_F32 && dtype != BASA_DTYPE_BF16) return BASA_ERR_UNSUPPORTED;
  if (head_dim != 64 && head_dim != 128) return BASA_ERR_UNSUPPORTED;
  if (B <= 0 || heads <= 0) return BASA_ERR_SHAPE;
  const int g = check_grid(T, H, W, wt, wh, ww);
  if (g != BASA_OK) return g;
  const int64_t N = int64_t(T) * H * W;
  const int64_t bh = int64_t(B) * heads;
  if (bh > kInt32Max || N * head_dim > kInt32Max) return BASA_ERR_OVERFLOW;
  // The bf16 kernel addresses one head through a buffer resource of 32-bit byte range and
  // reads rows past a window at byte offsets from 0xffffff00 up, which must lie outside the
  // head's range to read as zeros.
  if (dtype == BASA_DTYPE_BF16 && N * head_dim * 2 > int64_t(kBf16HeadBytesMax)) return BASA_ERR_OVERFLOW;
  if (int64_t(n_mem) * head_dim > kInt32Max) return BASA_ERR_OVERFLOW;
  if (dtype == BASA_DTYPE_BF16 && int64_t(n_mem) * head_dim * 2 > int64_t(kBf16HeadBytesMax)) return BASA_ERR_OVERFLOW;
  if (!aligned(q, 16) || !aligned(k, 16) || !aligned(v, 16) || !aligned(out, 16)) return BASA_ERR_ALIGN;
  if (n_mem > 0 && (!aligned(kmem, 16) || !aligned(vmem, 16))) return BASA_ERR_ALIGN;
  if (lse && !aligned(lse, 4)) return BASA_ERR_ALIGN;
  if (route && !aligned(route, 4)) return BASA_ERR_ALIGN;
  const int64_t elem = dtype == BASA_DTYPE_BF16 ? 2 : 4;
  const int64_t bytes = bh * N * head_dim * elem;
  const int64_t mem_bytes = bh * int64_t(n_mem) * head_dim * elem;
  if (overlaps(out, q, bytes) || overlaps(out, k, bytes) || overlaps(out, v, bytes)) return BASA_ERR_ALIAS;
  if (n_mem > 0 && (overlaps2(out, bytes, kmem, mem_bytes) || overlaps2(out, bytes, vmem, mem_bytes)))
    return BASA_ERR_ALIAS;
  if (lse) {
    const int64_t lse_bytes = bh * N * 4;
    if (overlaps2(lse, lse_bytes, q, bytes) || overlaps2(lse, lse_bytes, k, bytes) ||
        overlaps2(lse, lse_bytes, v, bytes) || overlaps2(lse, lse_bytes, out, bytes))
      return BASA_ERR_ALIAS;
    if (n_mem > 0 && (overlaps2(lse, lse_bytes, kmem, mem_bytes) || overlaps2(lse, lse_bytes, vmem, mem_bytes)))
      return BASA_ERR_ALIAS;
  }
  // route is an input the kernel reads at the start of every work item while other
  // workgroups already write out and lse
  if (route) {
    const int64_t route_bytes = bh * (N / (int64_t(wt) * wh * ww)) * 4;
    if (overlaps2(out, bytes, route, route_bytes)) return BASA_ERR_ALIAS;
    if (lse && overlaps2(lse, bh * N * 4, route, route_bytes)) return BASA_ERR_ALIAS;
  }

  basa::AttnParams p;
  p.map = basa::make_winmap(T, H, W, wt, wh, ww, reduce_mod(st, T), reduce_mod(sh, H), reduce_mod(sw, W));
  p.wtok = wt * wh * ww;
  p.n_win = int32_t(N / p.wtok);
  p.q_tiles = 0;
  p.kv_tiles = 0;
  p.heads_total = int32_t(bh);
  p.head_stride = N * head_dim;
  p.scale_log2 = float(1.4426950408889634 / sqrt(double(head_dim)));
  p.kmem = n_mem > 0 ? kmem : nullptr;
  p.vmem = n_mem > 0 ? vmem : nullptr;
  p.n_mem = n_mem;
  p.mem_tiles = 0;
  p.lse = lse;
  p.n_tokens = int32_t(N);
  p.route = route;
  const hipError_t e =
      basa::launch_window_attention(q, k, v, out, p, head_dim, dtype == BASA_DTYPE_BF16, no_alloc, stream);
  if (e == hipErrorInvalidConfiguration) return BASA_ERR_OVERFLOW;
  if (no_alloc && e == hipErrorOutOfMemory) return BASA_ERR_SCRATCH;
  return e == hipSuccess ? BASA_OK : BASA_ERR_HIP;
}

}  // namespace

extern "C" {

int basa_window_attn_fwd(const void* q, const void* k, const void* v, void* out, int B, int heads, int T, int H,
                         int W, int wt, int wh, int ww, int st, int sh, int sw, int head_dim, int dtype,
                         hipStream_t stream) {
  return run_attention(q, k, v, nullptr, nullptr, nullptr, 0, out, nullptr, B, heads, T, H, W, wt, wh, ww, st, sh,
                       sw, head_dim, dtype, stream);
}

int basa_window_attn_fwd_noalloc(const void* q, const void* k, const void* v, void* out, int B, int heads, int T,
                                 int H, int W, int wt, int wh, int ww, int st, int sh, int sw, int head_dim,
                                 int dtype, hipStream_t stream) {
  return run_attention(q, k, v, nullptr, nullptr, nullptr, 0, out, nullptr, B, heads, T, H, W, wt, wh, ww, st, sh,
                       sw, head_dim, dtype, stream, true);
}

int basa_full_attn_fwd(const void* q, const void* k, const void* v, void* out, int B, int heads, int N,
                       int head_dim, int dtype, hipStream_t stream) {
  return run_attention(q, k, v, nullptr, nullptr, nullptr, 0, out, nullptr, B, heads, 1, 1, N, 1, 1, N, 0, 0, 0,
                       head_dim, dtype, stream);
}

int basa_window_attn_mem_fwd(const void* q, const void* k, const void* v, const void* kmem, const void* vmem,
                             int n_mem, void* out, float* lse, int B, int heads, int T, int H, int W, int wt, int wh,
                             int ww, int st, int sh, int sw, int head_dim, int dtype, hipStream_t stream) {
  return run_attention(q, k, v, nullptr, kmem, vmem, n_mem, out, lse, B, heads, T, H, W, wt, wh, ww, st, sh, sw,
                       head_dim, dtype, stream);
}

int basa_window_attn_routed_fwd(const void* q, const void* k, const void* v, const int32_t* route, const void* kmem,
                                const void* vmem, int n_mem, void* out, float* lse, int B, int heads, int T, int H,
                                int W, int wt, int wh, int ww, int st, int sh, int sw, int head_dim, int dtype,
                                hipStream_t stream) {
  return run_attention(q, k, v, route, kmem, vmem, n_mem, out, lse, B, heads, T, H, W, wt, wh, ww, st, sh, sw,
                       head_dim, dtype, stream);
}

int basa_window_means(const void* q, const void* k, float* qbar, float* kbar, int B, int heads, int T, int H, int W,
                      int wt, int wh, int ww, int st, int sh, int sw, int head_dim, int dtype, hipStream_t stream) {
  if (!q || !k || !qbar || !kbar) return BASA_ERR_NULL;
  if (dtype != BASA_DTYPE_F32 && dtype != BASA_DTYPE_BF16) return BASA_ERR_UNSUPPORTED;
  if (head_dim != 64 && head_dim != 128) return BASA_ERR_UNSUPPORTED;
  if (B <= 0 || heads <= 0) return BASA_ERR_SHAPE;
  const int g = check_grid(T, H, W, wt, wh, ww);
  if (g != BASA_OK) return g;
  const int64_t N = int64_t(T) * H * W;
  const int64_t bh = int64_t(B) * heads;
  if (bh > kInt32Max || N * head_dim > kInt32Max) return BASA_ERR_OVERFLOW;
  if (!aligned(q, 16) || !aligned(k, 16) || !aligned(qbar, 16) || !aligned(kbar, 16)) return BASA_ERR_ALIGN;
  const int64_t wtok = int64_t(wt) * wh * ww;
  const int64_t n_win = N / wtok;
  const int64_t elem = dtype == BASA_DTYPE_BF16 ? 2 : 4;
  const int64_t in_bytes = bh * N * head_dim * elem, out_bytes = bh * n_win * head_dim * 4;
  if (overlaps2(qbar, out_bytes, q, in_bytes) || overlaps2(qbar, out_bytes, k, in_bytes) ||
      overlaps2(kbar, out_bytes, q, in_bytes) || overlaps2(kbar, out_bytes, k, in_bytes) ||
      overlaps2(qbar, out_bytes, kbar, out_bytes))
    return BASA_ERR_ALIAS;
  const basa::WinMap map =
      basa::make_winmap(T, H, W, wt, wh, ww, reduce_mod(st, T), reduce_mod(sh, H), reduce_mod(sw, W));
  const hipError_t e = basa::launch_window_means(q, k, qbar, kbar, map, int32_t(wtok), int32_t(n_win), int32_t(bh),
                                                 N * head_dim, head_dim, dtype == BASA_DTYPE_BF16, stream);
  if (e == hipErrorInvalidConfiguration) return BASA_ERR_OVERFLOW;
  return e == hipSuccess ? BASA_OK : BASA_ERR_HIP;
}

int basa_route_top1(const float* qbar, const float* kbar, int32_t* route, int B, int heads, int T, int H, int W,
                    int wt, int wh, int ww, int radius, int head_dim, hipStream_t stream) {
  if (!qbar || !kbar || !route) return BASA_ERR_NULL;
  if (head_dim != 64 && head_dim != 128) return BASA_ERR_UNSUPPORTED;
  if (B <= 0 || heads <= 0 || radius < 0) return BASA_ERR_SHAPE;
  const int g = check_grid(T, H, W, wt, wh, ww);
  if (g != BASA_OK) return g;
  const int64_t bh = int64_t(B) * heads;
  if (bh > kInt32Max) return BASA_ERR_OVERFLOW;
  if (!aligned(qbar, 4) || !aligned(kbar, 4) || !aligned(route, 4)) return BASA_ERR_ALIGN;
  const int64_t n_win = int64_t(T / wt) * (H / wh) * (W / ww);
  const int64_t desc_bytes = bh * n_win * head_dim * 4, route_bytes = bh * n_win * 4;
  if (overlaps2(route, route_bytes, qbar, desc_bytes) || overlaps2(route, route_bytes, kbar, desc_bytes))
    return BASA_ERR_ALIAS;
  const hipError_t e = basa::launch_route_top1(qbar, kbar, route, int32_t(bh), T / wt, H / wh, W / ww, radius,
                                               head_dim, stream);
  if (e == hipErrorInvalidConfiguration) return BASA_ERR_OVERFLOW;
  return e == hipSuccess ? BASA_OK : BASA_ERR_HIP;
}

int basa_pool_kv(const void* k, const void* v, void* kmem, void* vmem, int B, int heads, int T, int H, int W,
                 int ph, int pw, int head_dim, int dtype, hipStream_t stream) {
  if (!k || !v || !kmem || !vmem) return BASA_ERR_NULL;
  if (dtype != BASA_DTYPE_F32 && dtype != BASA_DTYPE_BF16) return BASA_ERR_UNSUPPORTED;
  if (head_dim != 64 && head_dim != 128) return BASA_ERR_UNSUPPORTED;
  if (B <= 0 || heads <= 0 || T <= 0 || H <= 0 || W <= 0 || ph <= 0 || pw <= 0) return BASA_ERR_SHAPE;
  const int64_t bh = int64_t(B) * heads;
  const int64_t N = int64_t(T) * H * W;
  if (bh > kInt32Max || N * head_dim > kInt32Max) return BASA_ERR_OVERFLOW;
  const int64_t G = int64_t(T) * ((H + ph - 1) / ph) * ((W + pw - 1) / pw);
  if (!aligned(k, 16) || !aligned(v, 16) || !aligned(kmem, 16) || !aligned(vmem, 16)) return BASA_ERR_ALIGN;
  const int64_t elem = dtype == BASA_DTYPE_BF16 ? 2 : 4;
  const int64_t in_bytes = bh * N * head_dim * elem, out_bytes = bh * G * head_dim * elem;
  if (overlaps2(kmem, out_bytes, k, in_bytes) || overlaps2(kmem, out_bytes, v, in_bytes) ||
      overlaps2(vmem, out_bytes, k, in_bytes) || overlaps2(vmem, out_bytes, v, in_bytes) ||
      overlaps2(kmem, out_bytes, vmem, out_bytes))
    return BASA_ERR_ALIAS;
  const hipError_t e = basa::launch_pool_kv(k, v, kmem, vmem, int32_t(bh), T, H, W, ph, pw, head_dim,
                                            dtype == BASA_DTYPE_BF16, stream);
  if (e == hipErrorInvalidConfiguration) return BASA_ERR_OVERFLOW;
  return e == hipSuccess ? BASA_OK : BASA_ERR_HIP;
}

int basa_window_perm(int T, int H, int W, int wt, int wh, int ww, int st, int sh, int sw, int32_t* perm,
                     hipStream_t stream) {
  if (!perm) return BASA_ERR_NULL;
  const int g = check_grid(T, H, W, wt, wh, ww);
  if (g != BASA_OK) return g;
  if (!aligned(perm, 4)) return BASA_ERR_ALIGN;
  const basa::WinMap map =
      basa::make_winmap(T, H, W, wt, wh, ww, reduce_mod(st, T), reduce_mod(sh, H), reduce_mod(sw, W));
  const int32_t total = T * H * W;
  const hipError_t e = basa::launch_window_perm(map, wt * wh * ww, total, perm, stream);
  return e == hipSuccess ? BASA_OK : BASA_ERR_HIP;
}

const char* basa_status_string(int status) {
  switch (status) {
    case BASA_OK: return "ok";
    case BASA_ERR_NULL: return "a required pointer is NULL";
    case BASA_ERR_SHAPE: return "non-positive size, or the window does not divide the grid";
    case BASA_ERR_UNSUPPORTED: return "unsupported dtype or head_dim (supported: f32/bf16 x 64/128)";
    case BASA_ERR_ALIAS: return "an output buffer overlaps an input or another output";
    case BASA_ERR_OVERFLOW: return "size exceeds the 32-bit per-head indexing";
    case BASA_ERR_HIP: return "HIP launch error";
    case BASA_ERR_ALIGN: return "tensor pointer is not 16-byte aligned (perm: 4-byte)";
    case BASA_ERR_SCRATCH: return "the call needs more than the static scratch buffer holds";
    default: return "unknown status";
  }
}

int basa_version(void) { return (1 << 16) | 4; }

// Interleaved shift schedule, BASA §3.1: per axis the offsets (i * delta) mod w with
// delta = max(1, floor(w / L)) are taken alternately from their first ceil(L/2) and the
// remaining entries; the step offset c is added modulo the window side.
int basa_shift_schedule(int L, int wh, int ww, int ch, int cw, int32_t* dh, int32_t* dw) {
  if (!dh || !dw) return BASA_ERR_NULL;
  if (L <= 0 || wh <= 0 || ww <= 0) return BASA_ERR_SHAPE;
  const int K = (L + 1) / 2;
  for (int l = 0; l < L; ++l) {
    // position l of the interleaving holds entry i of the offset sequence
    const int i = (l % 2 == 0) ? l / 2 : K + l / 2;
    const int sides[2] = {wh, ww};
    const int steps[2] = {ch, cw};
    int32_t* outs[2] = {dh, dw};
    for (int ax = 0; ax < 2; ++ax) {
      const int w = sides[ax];
      const int64_t delta = w / L > 1 ? w / L : 1;
      const int64_t a = (int64_t(i) * delta) % w;
      outs[ax][l] = int32_t(reduce_mod(int(a) + reduce_mod(steps[ax], w), w));
    }
  }
  return BASA_OK;
}

}  // extern "C"
