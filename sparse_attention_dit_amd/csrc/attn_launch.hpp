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
  int32_t heads_total;  // B * heads
  int64_t head_stride;  // N * head_dim elements
  float scale_log2;     // log2(e) / sqrt(head_dim)
};

hipError_t launch_window_attention(const void* q, const void* k, const void* v, void* out, const AttnParams& p,
                                   int head_dim, bool bf16, hipStream_t stream);

hipError_t launch_window_perm(const WinMap& map, int32_t wtok, int32_t total, int32_t* perm, hipStream_t stream);

}  // namespace basa
