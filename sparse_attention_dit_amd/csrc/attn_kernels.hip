// Shifted local-window attention kernels for gfx950 (MI355X).
//
// Operation: BASA paper (arXiv 2610.08772) §3.1 "Shifted Window Sparse Attention" --
// roll the token grid by -Delta, cut it into non-overlapping windows, run dense scaled
// dot-product softmax attention inside each window, roll the result back by +Delta.
// App. A.1 runs this as roll + reshape/permute copies + batched SDPA; here the roll, the
// partition and the inverse roll are folded into the kernel's row addressing: each
// workgroup reads its window's rows straight from their original positions and writes
// the outputs straight back to them, so there is no copy pass.
//
// bf16 kernel layout (one workgroup = one (batch*head, window, query tile)):
//   * S^T = K Q^T with v_mfma_f32_32x32x16_bf16 (A = K rows from LDS, B = Q rows kept
//     in registers). In the 32x32 accumulator lane l holds column l%32 and rows
//     8*(r/4) + 4*(l/32) + r%4, so every lane owns ONE query row: row max and row sum
//     are in-lane reductions plus one exchange between the two lane halves.
//   * The K rows of a 32-key block are fed in a bit-permuted order (bits 2 and 3 of the
//     row swapped) so that the accumulator registers 8c..8c+7 of lane half h hold the
//     probabilities of 8 consecutive keys 16c + 8h .. 16c + 8h + 7. Packed to bf16 they
//     are, unchanged, the B operand of O^T = V^T P^T.
//   * V is transposed into LDS (Vt[d][key]) so the A operand of O^T = V^T P^T is one
//     16-byte LDS read. The d rows of Vt are assigned so each lane's O^T registers are
//     head_dim/2 consecutive output elements of its query row.
//   * Online softmax in fp32 with exp2 and the 1/sqrt(d)*log2(e) scale folded into one
//     FMA; the running max is only raised (and O rescaled) when a row's max grows by
//     more than 2^8, which keeps the final O/l exact while skipping most rescales.
//   * Workgroups are renumbered so that all query tiles of one (head, window) land on
//     the same XCD (hardware dispatches workgroup i to XCD i % 8) and share its L2.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "attn_launch.hpp"
#include "index_map.hpp"

namespace basa {

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
typedef float f32x16_t __attribute__((ext_vector_type(16)));
typedef uint32_t u32x4_t __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2_t __attribute__((ext_vector_type(2)));

// Decode a workgroup into (batch*head, window, query tile), placing consecutive
// logical tiles on the same XCD.
struct TileId {
  int32_t bh, win, qtile;
};

__device__ __forceinline__ TileId decode_tile(const AttnParams& p) {
  const uint32_t bid = blockIdx.x;
  const uint32_t total = gridDim.x;
  const uint32_t xcd = bid % kNumXcd;
  const uint32_t idx = bid / kNumXcd;
  const uint32_t per = total / kNumXcd;
  const uint32_t rem = total % kNumXcd;
  const uint32_t logical = xcd < rem ? xcd * (per + 1) + idx : rem * (per + 1) + (xcd - rem) * per + idx;
  TileId t;
  t.qtile = int32_t(logical % uint32_t(p.q_tiles));
  const uint32_t rest = logical / uint32_t(p.q_tiles);
  t.win = int32_t(rest % uint32_t(p.n_win));
  t.bh = int32_t(rest / uint32_t(p.n_win));
  return t;
}

__device__ __forceinline__ float wave_half_max(float x) {
  // v_permlane32_swap: afterwards r[0] = x of lane l%32, r[1] = x of lane 32 + l%32.
  auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}

__device__ __forceinline__ float wave_half_sum(float x) {
  auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}

__device__ __forceinline__ uint32_t pack_bf16x2(float a, float b) {
  bf16x2_t r;
  r[0] = (__bf16)a;
  r[1] = (__bf16)b;
  return __builtin_bit_cast(uint32_t, r);
}

// Row of the 32-key block that feeds accumulator row m: bits 2 and 3 swapped.
__device__ __forceinline__ int key_perm(int m) {
  return (m & ~12) | ((m & 4) << 1) | ((m & 8) >> 1);
}

template <int D, int NW, int QB>
struct Bf16Cfg {
  static constexpr int BN = 64;                 // keys per K/V tile
  static constexpr int BM = NW * 32 * QB;       // query rows per workgroup
  static constexpr int NT = NW * 64;            // threads
  static constexpr int KS = D + 8;              // K row stride in LDS (elements)
  static constexpr int VS = BN + 8;             // Vt row stride in LDS (elements)
  static constexpr int VSKEW = 64;              // extra offset of Vt rows d >= D/2
  static constexpr int DK = D / 16;             // k-steps of S^T per key block
  static constexpr int DB = D / 32;             // 32-row d blocks of O^T
  static constexpr int KCH = D / 8;             // 16-byte chunks per row
  static constexpr int RK = BN * KCH / NT;      // K chunks per thread
  static constexpr int RV = BN * KCH / NT;      // V rows per thread (one 8-wide d chunk each)
  static constexpr int VKG = BN / RV;           // key groups of the V transpose
  static_assert(RK >= 1 && RV >= 1 && (RV & (RV - 1)) == 0 && RV <= 8, "tile/thread mismatch");
  static constexpr int KS_BYTES = BN * KS * 2;
  static constexpr int VT_BYTES = (D * VS + VSKEW) * 2;
};

__device__ __forceinline__ int vt_row_offset(int d, int D, int VS, int VSKEW) {
  return d * VS + (d >= D / 2 ? VSKEW : 0);
}

template <int D, int NW, int QB>
__global__ __launch_bounds__(NW * 64) void win_attn_bf16_kernel(const uint16_t* __restrict__ q,
                                                                 const uint16_t* __restrict__ k,
                                                                 const uint16_t* __restrict__ v,
                                                                 uint16_t* __restrict__ out,
                                                                 AttnParams p) {
  using C = Bf16Cfg<D, NW, QB>;
  constexpr int BN = C::BN, BM = C::BM, NT = C::NT, KS = C::KS, VS = C::VS, VSKEW = C::VSKEW;
  constexpr int DK = C::DK, DB = C::DB, KCH = C::KCH, RK = C::RK, RV = C::RV, VKG = C::VKG;

  __shared__ __attribute__((aligned(16))) uint16_t Ks[BN * KS];
  __shared__ __attribute__((aligned(16))) uint16_t Vt[D * VS + VSKEW];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int l32 = lane & 31;
  const int hh = lane >> 5;

  const TileId tile = decode_tile(p);
  const int64_t base = int64_t(tile.bh) * p.head_stride;
  const WinOrigin org = window_origin(p.map, uint32_t(tile.win));
  const uint16_t* qh = q + base;
  const uint16_t* kh = k + base;
  const uint16_t* vh = v + base;

  // ---- Q fragments (B operand of S^T): lane holds d = hh*D/2 + 8*kk .. +7 of its row.
  bf16x8_t qf[QB][DK];
#pragma unroll
  for (int qb = 0; qb < QB; ++qb) {
    const int row = tile.qtile * BM + (wave * QB + qb) * 32 + l32;
    if (row < p.wtok) {
      const int tok = token_of(p.map, org, uint32_t(row));
      const u32x4_t* src = reinterpret_cast<const u32x4_t*>(qh + int64_t(tok) * D + hh * (D / 2));
#pragma unroll
      for (int kk = 0; kk < DK; ++kk) qf[qb][kk] = __builtin_bit_cast(bf16x8_t, src[kk]);
    } else {
#pragma unroll
      for (int kk = 0; kk < DK; ++kk) qf[qb][kk] = __builtin_bit_cast(bf16x8_t, u32x4_t{0, 0, 0, 0});
    }
  }

  // ---- K/V tile staging: global -> registers (prefetch) -> LDS.
  const int k_col = tid % KCH;           // K: row-major chunks, 16 lanes per 256-byte row
  const int k_row0 = tid / KCH;
  constexpr int K_ROW_STEP = NT / KCH;
  const int v_kg = tid % VKG;            // V: RV consecutive keys x 8 d per thread
  const int v_dg = tid / VKG;
  u32x4_t kreg[RK];
  u32x4_t vreg[RV];

  auto load_tile = [&](int t) {
    const int local = t * BN + lane;  // lane j computes the token of tile row j
    const int my_tok = local < p.wtok ? token_of(p.map, org, uint32_t(local)) : -1;
#pragma unroll
    for (int i = 0; i < RK; ++i) {
      const int r = k_row0 + i * K_ROW_STEP;
      const int tok = __shfl(my_tok, r);
      kreg[i] = tok >= 0 ? *reinterpret_cast<const u32x4_t*>(kh + int64_t(tok) * D + k_col * 8)
                         : u32x4_t{0, 0, 0, 0};
    }
#pragma unroll
    for (int i = 0; i < RV; ++i) {
      const int r = v_kg * RV + i;
      const int tok = __shfl(my_tok, r);
      vreg[i] = tok >= 0 ? *reinterpret_cast<const u32x4_t*>(vh + int64_t(tok) * D + v_dg * 8)
                         : u32x4_t{0, 0, 0, 0};
    }
  };

  auto store_tile = [&]() {
#pragma unroll
    for (int i = 0; i < RK; ++i) {
      const int r = k_row0 + i * K_ROW_STEP;
      *reinterpret_cast<u32x4_t*>(&Ks[r * KS + k_col * 8]) = kreg[i];
    }
    // transpose RV rows x 8 d into 8 d-rows x RV keys
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      const int d = v_dg * 8 + e;
      uint16_t* dst = &Vt[vt_row_offset(d, D, VS, VSKEW) + v_kg * RV];
      const int w = e >> 1;
      const uint32_t sel = (e & 1) ? 0x07060302u : 0x05040100u;
      if constexpr (RV == 1) {
        dst[0] = uint16_t((e & 1) ? (vreg[0][w] >> 16) : (vreg[0][w] & 0xffffu));
      } else if constexpr (RV == 2) {
        *reinterpret_cast<uint32_t*>(dst) = __builtin_amdgcn_perm(vreg[1][w], vreg[0][w], sel);
      } else if constexpr (RV == 4) {
        u32x2_t x;
        x[0] = __builtin_amdgcn_perm(vreg[1][w], vreg[0][w], sel);
        x[1] = __builtin_amdgcn_perm(vreg[3][w], vreg[2][w], sel);
        *reinterpret_cast<u32x2_t*>(dst) = x;
      } else {
        u32x4_t x;
        x[0] = __builtin_amdgcn_perm(vreg[1][w], vreg[0][w], sel);
        x[1] = __builtin_amdgcn_perm(vreg[3][w], vreg[2][w], sel);
        x[2] = __builtin_amdgcn_perm(vreg[5][w], vreg[4][w], sel);
        x[3] = __builtin_amdgcn_perm(vreg[7][w], vreg[6][w], sel);
        *reinterpret_cast<u32x4_t*>(dst) = x;
      }
    }
  };

  // ---- per-lane constant LDS offsets
  const int k_frag_row = key_perm(l32);  // + 32*kb
  int v_frag_off[DB];
#pragma unroll
  for (int db = 0; db < DB; ++db) {
    const int m = l32;
    const int dphys = ((m >> 2) & 1) * (D / 2) + 16 * db + 4 * (m >> 3) + (m & 3);
    v_frag_off[db] = vt_row_offset(dphys, D, VS, VSKEW) + 8 * hh;
  }
  // key index (within a 64-key tile) of accumulator register r of key block kb
  auto acc_key = [&](int kb, int r) { return 32 * kb + key_perm(8 * (r >> 2) + 4 * hh + (r & 3)); };

  f32x16_t oacc[QB][DB];
#pragma unroll
  for (int qb = 0; qb < QB; ++qb)
#pragma unroll
    for (int db = 0; db < DB; ++db)
#pragma unroll
      for (int r = 0; r < 16; ++r) oacc[qb][db][r] = 0.0f;
  float m_run[QB], l_run[QB];
#pragma unroll
  for (int qb = 0; qb < QB; ++qb) {
    m_run[qb] = -__builtin_inff();
    l_run[qb] = 0.0f;
  }
  const float c = p.scale_log2;

  load_tile(0);
  for (int t = 0; t < p.kv_tiles; ++t) {
    __syncthreads();
    store_tile();
    __syncthreads();
    if (t + 1 < p.kv_tiles) load_tile(t + 1);

    // S^T = K Q^T for 64 keys (two 32-key blocks)
    f32x16_t sacc[QB][2];
#pragma unroll
    for (int qb = 0; qb < QB; ++qb)
#pragma unroll
      for (int kb = 0; kb < 2; ++kb)
#pragma unroll
        for (int r = 0; r < 16; ++r) sacc[qb][kb][r] = 0.0f;
#pragma unroll
    for (int kk = 0; kk < DK; ++kk) {
#pragma unroll
      for (int kb = 0; kb < 2; ++kb) {
        const bf16x8_t kf =
            *reinterpret_cast<const bf16x8_t*>(&Ks[(32 * kb + k_frag_row) * KS + hh * (D / 2) + kk * 8]);
#pragma unroll
        for (int qb = 0; qb < QB; ++qb)
          sacc[qb][kb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(kf, qf[qb][kk], sacc[qb][kb], 0, 0, 0);
      }
    }

    // ragged last tile: keys past the window get -inf
    if ((t + 1) * BN > p.wtok) {
      const int lim = p.wtok - t * BN;
#pragma unroll
      for (int kb = 0; kb < 2; ++kb)
#pragma unroll
        for (int r = 0; r < 16; ++r)
          if (acc_key(kb, r) >= lim)
#pragma unroll
            for (int qb = 0; qb < QB; ++qb) sacc[qb][kb][r] = -__builtin_inff();
    }

    // online softmax (fp32), P^T packed to bf16 as the B operand of O^T += V^T P^T
    bf16x8_t pf[QB][4];
#pragma unroll
    for (int qb = 0; qb < QB; ++qb) {
      float mx = sacc[qb][0][0];
#pragma unroll
      for (int kb = 0; kb < 2; ++kb)
#pragma unroll
        for (int r = 0; r < 16; ++r) mx = fmaxf(mx, sacc[qb][kb][r]);
      mx = wave_half_max(mx) * c;
      const bool need = mx > m_run[qb] + 8.0f;
      if (__builtin_amdgcn_ballot_w64(need) != 0) {
        const float m_new = need ? mx : m_run[qb];
        const float alpha = __builtin_amdgcn_exp2f(m_run[qb] - m_new);
        m_run[qb] = m_new;
        l_run[qb] *= alpha;
#pragma unroll
        for (int db = 0; db < DB; ++db)
#pragma unroll
          for (int r = 0; r < 16; ++r) oacc[qb][db][r] *= alpha;
      }
      const float neg_m = -m_run[qb];
      float lsum = 0.0f;
#pragma unroll
      for (int kb = 0; kb < 2; ++kb) {
#pragma unroll
        for (int ch = 0; ch < 2; ++ch) {
          u32x4_t packed;
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            const float p0 = __builtin_amdgcn_exp2f(__builtin_fmaf(sacc[qb][kb][8 * ch + 2 * e], c, neg_m));
            const float p1 = __builtin_amdgcn_exp2f(__builtin_fmaf(sacc[qb][kb][8 * ch + 2 * e + 1], c, neg_m));
            // The row sum adds the bf16-rounded p that the PV product uses. The packed word
            // goes through a scalar temporary: bit-casting the vector element directly
            // (packed[e]) makes hipcc 7.2 feed the same register to every v_dot2c.
            const uint32_t w = pack_bf16x2(p0, p1);
            lsum = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2_t, w),
                                                  __builtin_bit_cast(bf16x2_t, 0x3f803f80u), lsum, false);
            packed[e] = w;
          }
          pf[qb][kb * 2 + ch] = __builtin_bit_cast(bf16x8_t, packed);
        }
      }
      l_run[qb] += lsum;
    }

    // O^T += V^T P^T
#pragma unroll
    for (int kb = 0; kb < 2; ++kb) {
#pragma unroll
      for (int ch = 0; ch < 2; ++ch) {
#pragma unroll
        for (int db = 0; db < DB; ++db) {
          const bf16x8_t vf = *reinterpret_cast<const bf16x8_t*>(&Vt[v_frag_off[db] + 32 * kb + 16 * ch]);
#pragma unroll
          for (int qb = 0; qb < QB; ++qb)
            oacc[qb][db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(vf, pf[qb][kb * 2 + ch], oacc[qb][db], 0, 0, 0);
        }
      }
    }
  }

  // ---- normalise and store each row at its original (un-shifted) position
#pragma unroll
  for (int qb = 0; qb < QB; ++qb) {
    const float l = wave_half_sum(l_run[qb]);
    const float inv = 1.0f / l;
    const int row = tile.qtile * BM + (wave * QB + qb) * 32 + l32;
    if (row < p.wtok) {
      const int tok = token_of(p.map, org, uint32_t(row));
      u32x4_t* dst = reinterpret_cast<u32x4_t*>(out + base + int64_t(tok) * D + hh * (D / 2));
#pragma unroll
      for (int db = 0; db < DB; ++db) {
#pragma unroll
        for (int half = 0; half < 2; ++half) {
          u32x4_t w;
#pragma unroll
          for (int e = 0; e < 4; ++e)
            w[e] = pack_bf16x2(oacc[qb][db][8 * half + 2 * e] * inv, oacc[qb][db][8 * half + 2 * e + 1] * inv);
          dst[db * 2 + half] = w;
        }
      }
    }
  }
}

// ---------------------------------------------------------------------------------
// fp32 kernel: one wave per 64 query rows, one query row per lane, K/V tiles of 32 keys
// in LDS read as broadcasts. Plain fp32 FMA arithmetic throughout (no reduced-precision
// operands), online softmax with exp2. Used for fp32 inputs, where exactness to ~1e-6
// matters more than speed.
template <int D>
__global__ __launch_bounds__(64) void win_attn_f32_kernel(const float* __restrict__ q,
                                                          const float* __restrict__ k,
                                                          const float* __restrict__ v,
                                                          float* __restrict__ out, AttnParams p) {
  constexpr int BN = 32;
  constexpr int BM = 64;
  constexpr int CH = 8;  // keys per softmax chunk
  __shared__ __attribute__((aligned(16))) float Ks[BN * D];
  __shared__ __attribute__((aligned(16))) float Vs[BN * D];
  const int lane = threadIdx.x;
  const TileId tile = decode_tile(p);
  const int64_t base = int64_t(tile.bh) * p.head_stride;
  const WinOrigin org = window_origin(p.map, uint32_t(tile.win));
  const int row = tile.qtile * BM + lane;
  const bool valid = row < p.wtok;
  const int my_tok = valid ? token_of(p.map, org, uint32_t(row)) : 0;

  float qv[D];
  float o[D];
#pragma unroll
  for (int d = 0; d < D; ++d) {
    qv[d] = valid ? q[base + int64_t(my_tok) * D + d] : 0.0f;
    o[d] = 0.0f;
  }
  float m = -__builtin_inff(), l = 0.0f;
  const float c = p.scale_log2;

  for (int t = 0; t * BN < p.wtok; ++t) {
    __syncthreads();
    // 64 lanes load 32 rows: two lanes per row, each half of the row
    {
      const int r = lane >> 1;
      const int half = lane & 1;
      const int local = t * BN + r;
      float* kd = &Ks[r * D + half * (D / 2)];
      float* vd = &Vs[r * D + half * (D / 2)];
      if (local < p.wtok) {
        const int tok = token_of(p.map, org, uint32_t(local));
        const float* ks = k + base + int64_t(tok) * D + half * (D / 2);
        const float* vs = v + base + int64_t(tok) * D + half * (D / 2);
#pragma unroll
        for (int d = 0; d < D / 2; ++d) {
          kd[d] = ks[d];
          vd[d] = vs[d];
        }
      } else {
#pragma unroll
        for (int d = 0; d < D / 2; ++d) {
          kd[d] = 0.0f;
          vd[d] = 0.0f;
        }
      }
    }
    __syncthreads();
    const int nk = min(BN, p.wtok - t * BN);
    for (int j0 = 0; j0 < nk; j0 += CH) {
      float s[CH];
      float mx = -__builtin_inff();
#pragma unroll
      for (int j = 0; j < CH; ++j) {
        float acc = 0.0f;
#pragma unroll
        for (int d = 0; d < D; ++d) acc = __builtin_fmaf(qv[d], Ks[(j0 + j) * D + d], acc);
        s[j] = (j0 + j < nk) ? acc * c : -__builtin_inff();
        mx = fmaxf(mx, s[j]);
      }
      const float m_new = fmaxf(m, mx);
      const float alpha = __builtin_amdgcn_exp2f(m - m_new);
      l *= alpha;
#pragma unroll
      for (int d = 0; d < D; ++d) o[d] *= alpha;
#pragma unroll
      for (int j = 0; j < CH; ++j) {
        const float pj = __builtin_amdgcn_exp2f(s[j] - m_new);
        l += pj;
#pragma unroll
        for (int d = 0; d < D; ++d) o[d] = __builtin_fmaf(pj, Vs[(j0 + j) * D + d], o[d]);
      }
      m = m_new;
    }
  }
  if (valid) {
    const float inv = 1.0f / l;
#pragma unroll
    for (int d = 0; d < D; ++d) out[base + int64_t(my_tok) * D + d] = o[d] * inv;
  }
}

// ---------------------------------------------------------------------------------
__global__ void win_perm_kernel(WinMap map, int32_t wtok, int32_t total, int32_t* __restrict__ perm) {
  const int32_t idx = int32_t(blockIdx.x) * 256 + int32_t(threadIdx.x);
  if (idx >= total) return;
  const int32_t win = idx / wtok;
  const int32_t local = idx - win * wtok;
  perm[idx] = token_of(map, window_origin(map, uint32_t(win)), uint32_t(local));
}

// ---------------------------------------------------------------------------------
template <int D, int NW, int QB>
static hipError_t launch_bf16(const void* q, const void* k, const void* v, void* out, AttnParams p,
                              hipStream_t stream) {
  using C = Bf16Cfg<D, NW, QB>;
  p.q_tiles = (p.wtok + C::BM - 1) / C::BM;
  p.kv_tiles = (p.wtok + C::BN - 1) / C::BN;
  const uint64_t blocks = uint64_t(p.q_tiles) * uint64_t(p.n_win) * uint64_t(p.heads_total);
  if (blocks == 0 || blocks > 0x7fffffffu) return hipErrorInvalidConfiguration;
  hipLaunchKernelGGL((win_attn_bf16_kernel<D, NW, QB>), dim3(uint32_t(blocks)), dim3(C::NT), 0, stream,
                     static_cast<const uint16_t*>(q), static_cast<const uint16_t*>(k),
                     static_cast<const uint16_t*>(v), static_cast<uint16_t*>(out), p);
  return hipGetLastError();
}

template <int D>
static hipError_t launch_f32(const void* q, const void* k, const void* v, void* out, AttnParams p,
                             hipStream_t stream) {
  p.q_tiles = (p.wtok + 63) / 64;
  p.kv_tiles = (p.wtok + 31) / 32;
  const uint64_t blocks = uint64_t(p.q_tiles) * uint64_t(p.n_win) * uint64_t(p.heads_total);
  if (blocks == 0 || blocks > 0x7fffffffu) return hipErrorInvalidConfiguration;
  hipLaunchKernelGGL((win_attn_f32_kernel<D>), dim3(uint32_t(blocks)), dim3(64), 0, stream,
                     static_cast<const float*>(q), static_cast<const float*>(k), static_cast<const float*>(v),
                     static_cast<float*>(out), p);
  return hipGetLastError();
}

hipError_t launch_window_attention(const void* q, const void* k, const void* v, void* out, const AttnParams& p,
                                   int head_dim, bool bf16, hipStream_t stream) {
  if (bf16) {
    if (head_dim == 128) return launch_bf16<128, 4, 1>(q, k, v, out, p, stream);
    if (head_dim == 64) return launch_bf16<64, 4, 1>(q, k, v, out, p, stream);
  } else {
    if (head_dim == 128) return launch_f32<128>(q, k, v, out, p, stream);
    if (head_dim == 64) return launch_f32<64>(q, k, v, out, p, stream);
  }
  return hipErrorInvalidValue;
}

hipError_t launch_window_perm(const WinMap& map, int32_t wtok, int32_t total, int32_t* perm, hipStream_t stream) {
  const uint32_t blocks = uint32_t((total + 255) / 256);
  hipLaunchKernelGGL(win_perm_kernel, dim3(blocks), dim3(256), 0, stream, map, wtok, total, perm);
  return hipGetLastError();
}

}  // namespace basa
