// Internal interface between the C ABI (basa_abi.cpp) and the HIP kernels.
#pragma once
#include <hip/hip_runtime_api.h>
#include <stdint.h>

#include "index_map.hpp"

namespace basa {

// MI355X: 8 XCDs; the dispatcher hands workgroup i to XCD i % 8.
constexpr uint32_t kNumXcd = 8;

struct AttnParams {
  WinMap map;
  int32_t wtok;         // tokens per window
  int32_t n_win;        // windows per (batch, head)
  int32_t q_tiles;      // filled by the launcher
  int32_t kv_tiles;     // filled by the launcher
  FastDiv f_kv_tiles;   // division by kv_tiles (stream kernel), filled by the launcher
  FastDiv f_q_tiles;    // division by q_tiles (work-item decode), filled by the launcher
  FastDiv f_n_win;      // division by n_win (work-item decode), filled by the launcher
  int32_t heads_total;  // B * heads
  int64_t head_stride;  // N * head_dim elements
  float scale_log2;     // log2(e) / sqrt(head_dim)
  // K/V-pooled global memory appended to every window's keys (n_mem = 0: none), laid out
  // [B*heads, n_mem, head_dim] like k and v; mem_tiles is filled by the launcher
  const void* kmem;
  const void* vmem;
  int32_t n_mem;
  int32_t mem_tiles;
  float* lse;           // optional [B*heads, N] natural-log log-sum-exp of each row's logits
  int32_t n_tokens;     // N
  // optional routed window per (batch*head, window) (§3.3): its tokens follow the window's
  // own in the key/value stream; -1 (or any value outside [0, n_win)) routes nothing
  const int32_t* route;
};

// no_alloc: the split work items of the bf16 per-item kernels use the library's static scratch
// array instead of a workspace allocated for the stream (hipErrorOutOfMemory when the split
// needs more than the array holds).
hipError_t launch_window_attention(const void* q, const void* k, const void* v, void* out, const AttnParams& p,
                                   int head_dim, bool bf16, bool no_alloc, hipStream_t stream);

hipError_t launch_window_perm(const WinMap& map, int32_t wtok, int32_t total, int32_t* perm, hipStream_t stream);

// Window descriptors (§3.3): qbar/kbar [BH, n_win, D] fp32 = means of q/k over each window.
hipError_t launch_window_means(const void* q, const void* k, float* qbar, float* kbar, const WinMap& map,
                               int32_t wtok, int32_t n_win, int32_t bh, int64_t head_stride, int head_dim, bool bf16,
                               hipStream_t stream);

// Top-1 routing (§3.3): route[bh, i] = argmax over windows j at Chebyshev distance 1..radius
// of qbar[bh,i] . kbar[bh,j] / sqrt(D) (lowest j on ties, -1 without candidates).
hipError_t launch_route_top1(const float* qbar, const float* kbar, int32_t* route, int32_t bh, int32_t nt,
                             int32_t nh, int32_t nw, int32_t radius, int head_dim, hipStream_t stream);

// Pooled memory: kmem/vmem [BH, T*gh*gw, D] = means of k/v over ph x pw regions per frame.
hipError_t launch_pool_kv(const void* k, const void* v, void* kmem, void* vmem, int32_t bh, int32_t T, int32_t H,
                          int32_t W, int32_t ph, int32_t pw, int head_dim, bool bf16, hipStream_t stream);

}  // namespace basa
