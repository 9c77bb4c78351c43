// Shifted local-window attention kernels for gfx950 (MI355X).
//
// Operation: BASA paper (arXiv 2610.08772) §3.1 "Shifted Window Sparse Attention" --
// roll the token grid by -Delta, cut it into non-overlapping windows, run dense scaled
// dot-product softmax attention inside each window, roll the result back by +Delta.
// App. A.1 runs this as roll + reshape/permute copies + batched SDPA; here the roll, the
// partition and the inverse roll are folded into the kernel's row addressing: each
// workgroup reads its window's rows straight from their original positions and writes
// the outputs straight back to them, so there is no copy pass. Optionally (§3.2) every
// window's keys and values are followed by a shared set of pooled memory tokens, and the
// per-row log-sum-exp is written for merging with other attention results (App. A.1).
//
// bf16 kernel layout (one work item = one (batch*head, window, query tile); a persistent
// grid of one workgroup per CU walks the items):
//   * S^T = K Q^T with v_mfma_f32_32x32x16_bf16 (A = K rows from LDS, B = Q rows kept
//     in registers). In the 32x32 accumulator lane l holds column l%32 and rows
//     8*(r/4) + 4*(l/32) + r%4, so every lane owns ONE query row: row max and row sum
//     are in-lane reductions plus one exchange between the two lane halves.
//   * The K rows of a 32-key block are fed in a bit-permuted order (bits 2 and 3 of the
//     row swapped) so that the accumulator registers 8c..8c+7 of lane half h hold the
//     probabilities of 8 consecutive keys 16c + 8h .. 16c + 8h + 7. Packed to bf16 they
//     are, unchanged, the B operand of O^T = V^T P^T.
//   * V stays row-major in LDS; gfx950's transposing LDS read (ds_read_b64_tr_b16)
//     delivers the A operand of O^T = V^T P^T. The d rows are assigned so each lane's
//     O^T registers are head_dim/2 consecutive output elements of its query row.
//   * Online softmax in fp32 with exp2 and the 1/sqrt(d)*log2(e) scale folded into one
//     FMA; the running max is only raised (and O rescaled) when a row's max grows by
//     more than 2^8, which keeps the final O/l exact while skipping most rescales.
//   * Work items are renumbered so that all query tiles of one (head, window) land on
//     the same XCD (hardware dispatches workgroup i to XCD i % 8; the persistent grid is a
//     multiple of 8, so a workgroup's items stay on its XCD) and share its L2. Q loads and
//     output stores are non-temporal, so that L2 keeps the window's K/V for the other
//     query tiles.
#include <hip/hip_runtime.h>
#include <stdint.h>

#include <atomic>
#include <map>
#include <mutex>
#include <utility>

#include "attn_launch.hpp"
#include "index_map.hpp"

namespace basa {

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
typedef float f32x16_t __attribute__((ext_vector_type(16)));
typedef uint32_t u32x4_t __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2_t __attribute__((ext_vector_type(2)));

// Decode work item `bid` of `total` into (batch*head, window, query tile), placing
// consecutive logical tiles on the same XCD (item i runs on XCD i % 8: a workgroup's
// items are blockIdx.x + k * gridDim.x, with gridDim.x a multiple of 8 when it loops).
struct TileId {
  int32_t bh, win, qtile;
};

__device__ __forceinline__ TileId decode_tile(const AttnParams& p, uint32_t bid, uint32_t total) {
  const uint32_t xcd = bid % kNumXcd;
  const uint32_t idx = bid / kNumXcd;
  const uint32_t per = total / kNumXcd;
  const uint32_t rem = total % kNumXcd;
  const uint32_t logical = xcd < rem ? xcd * (per + 1) + idx : rem * (per + 1) + (xcd - rem) * per + idx;
  TileId t;
  const uint32_t rest = fdiv(logical, p.f_q_tiles);
  t.qtile = int32_t(logical - rest * uint32_t(p.q_tiles));
  const uint32_t bh = fdiv(rest, p.f_n_win);
  t.win = int32_t(rest - bh * uint32_t(p.n_win));
  t.bh = int32_t(bh);
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
__host__ __device__ constexpr int key_perm(int m) {
  return (m & ~12) | ((m & 4) << 1) | ((m & 8) >> 1);
}

// LDS tile layout (one K tile or one V tile of BN rows x D bf16).
// Rows are grouped RPG at a time (RPG * D * 2 = 1 KB, the bytes one wave-wide 16-byte
// load moves). Inside a group the 16-byte chunks are interleaved by row:
//   byte(row, chunk) = (row / RPG) * RG + slot(chunk) * RPG * 16 + (row % RPG) * 16
// with groups RG = 1 KB + RPG * 16 apart. One wave-wide direct global->LDS load fills one
// group (lane j -> slot j / RPG, row j % RPG: 16-byte pieces of RPG whole rows, so the
// global reads stay row-contiguous). gfx950's LDS has 64 four-byte banks and serves 256
// bytes per clock; the skew between groups keeps the 16-byte K operand reads (rows in
// key_perm order) conflict-free. For V, slot() moves chunks of the upper half of d: a
// transpose read of d block db has the two 16-lane groups of each half-wave read chunks
// 2db and 2db+1 and their upper-half partners, four rows each. For D = 128 the partners
// are swapped with the chunk two slots away, so the four chunks fall in four different
// 16-bank blocks (measured: 1.5x the transpose-read rate of swapping neighbours). For
// D = 64 chunk slots are 128 bytes apart and only two bank offsets exist; neighbours are
// swapped.
template <int D>
struct TileLayout {
  static constexpr int ROW_BYTES = D * 2;
  static constexpr int CPR = D / 8;                  // 16-byte chunks per row
  static constexpr int RPG = 1024 / ROW_BYTES;       // rows per group (4 for D=128, 8 for D=64)
  static constexpr int CS = RPG * 16;                // chunk-slot stride inside a group
  static constexpr int RG = 1024 + CS;               // group stride
  __host__ __device__ static constexpr int v_slot(int c) { return c >= CPR / 2 ? (c ^ (D == 128 ? 2 : 1)) : c; }
  // D = 64: in V, the upper-half chunks of row r of a group are stored at row position r ^ 4,
  // so a transpose read of rows 0-3 touches the lower half's bytes 0-63 and the upper half's
  // bytes 64-127 of their slots: with the neighbour swap, the four chunks of one half-wave's
  // read then cover the 64 banks once.
  static constexpr bool V_ROW_SWIZZLE = D == 64;
};

template <int D, int NW>
struct Bf16Cfg {
  using L = TileLayout<D>;
  static constexpr int BN = 64;                       // keys per K/V tile
  static constexpr int BM = NW * 32;                  // query rows per workgroup (32 per wave)
  static constexpr int NT = NW * 64;
  static constexpr int GROUPS = BN / L::RPG;          // row groups per tile
  static constexpr int TILE_BYTES = GROUPS * L::RG;   // one K or V tile in LDS
  static constexpr int STAGE_BYTES = 2 * TILE_BYTES;  // K tile then V tile
  static constexpr int STAGES = 2;
  static constexpr int LOADS = GROUPS / NW;           // wave-wide loads per tensor per wave
  static constexpr int DK = D / 16;                   // MFMA k-steps of S^T per key block
  static constexpr int DB = D / 32;                   // 32-row d blocks of O^T
  static_assert(LOADS >= 1 && LOADS * NW == GROUPS, "tile/wave mismatch");
  static constexpr int LDS_BYTES = STAGES * STAGE_BYTES;
};

typedef __bf16 bf16x4_t __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) bf16x4_t lds_bf16x4_t;
typedef __attribute__((address_space(3))) void lds_void_t;

__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc(const void* base, uint32_t bytes) {
  // raw buffer, 32-bit data format (gfx9 descriptor word 3); reads past `bytes` return 0
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, (int)bytes, 0x00020000);
}

// Device-only builtins are called through __device__ functions: called directly from a
// lambda inside a kernel template, the buffer-to-LDS builtin can make hipcc's host pass
// drop the kernel's launch stub without a diagnostic.
// cache-policy operand of the buffer intrinsics: NT (non-temporal, streaming) on gfx950
constexpr int kCachePolicyNT = 2;
template <int CPOL = 0>
__device__ __forceinline__ void dma16_to_lds(__amdgpu_buffer_rsrc_t rs, char* dst, uint32_t off) {
  __builtin_amdgcn_raw_ptr_buffer_load_lds(rs, (lds_void_t*)dst, 16, off, 0, 0, CPOL);
}
// Output rows are written once and not read again by this kernel: non-temporal stores
// (cache policy NT) keep them from displacing the window's K/V in L2, which the window's
// other query tiles still read.
__device__ __forceinline__ void buffer_store16(__amdgpu_buffer_rsrc_t rs, uint32_t off, u32x4_t x) {
  __builtin_amdgcn_raw_buffer_store_b128(x, rs, off, 0, kCachePolicyNT);
}

// Workgroup barrier that waits only for each wave's own LDS accesses (s_waitcnt lgkmcnt(0),
// gfx9 immediate 0xC07F), not for its outstanding global loads and stores as __syncthreads()
// does. The empty asm statements keep the compiler from moving memory accesses across it.
__device__ __forceinline__ void lds_barrier() {
  __builtin_amdgcn_s_waitcnt(0xC07F);
  asm volatile("" ::: "memory");
  __builtin_amdgcn_s_barrier();
  asm volatile("" ::: "memory");
}

// Per-lane view of the bf16 tile math: the lane's LDS read bases and the three products of a
// K/V step. A wave owns 32 query rows; lane (l32, hh) holds query row l32 of the wave and
// half hh of its head_dim.
template <int D, int NW>
struct Bf16Lane {
  using C = Bf16Cfg<D, NW>;
  using L = TileLayout<D>;
  static constexpr int BN = C::BN, DK = C::DK, DB = C::DB;
  static constexpr int RPG = L::RPG, CS = L::CS, RG = L::RG, CPR = L::CPR;
  static constexpr int QG = 32 / RPG;  // row groups of one wave's 32 query rows

  int l32, hh;
  int ld_slot, ld_row, v_ld_row;  // chunk slot and group row the lane moves in a wave-wide load
  uint32_t k_chunk_off, v_chunk_off;
  int q_rd, k_rd;
  int v_rd[DB], v_rd1[DB];

  __device__ __forceinline__ Bf16Lane(int lane, int wave) {
    l32 = lane & 31;
    hh = lane >> 5;
    // K/V/Q tile loads: lane j moves 16 bytes, chunk slot j / RPG of row (group*RPG + j % RPG)
    ld_slot = lane / RPG;
    ld_row = lane % RPG;
    k_chunk_off = uint32_t(ld_slot) * 16u;
    v_chunk_off = uint32_t(L::v_slot(ld_slot)) * 16u;
    // row of its group that the lane loads for V (differs from ld_row only for the upper-half
    // chunks of D = 64; see TileLayout)
    v_ld_row = (L::V_ROW_SWIZZLE && ld_slot >= CPR / 2) ? (ld_row ^ 4) : ld_row;
    // B operand of S^T: lane holds d = hh*D/2 + 8*kk .. +7 of query row wave*32 + l32
    const int qrow = wave * 32 + l32;
    q_rd = (qrow / RPG) * RG + (qrow % RPG) * 16 + hh * (CPR / 2) * CS;
    // K (A operand of S^T): row 32*kb + key_perm(l32), chunk hh*CPR/2 + kk
    const int krow = key_perm(l32);
    k_rd = (krow / RPG) * RG + (krow % RPG) * 16 + hh * (CPR / 2) * CS;
    // V^T (A operand of O^T) by transpose reads: in each 16-lane group lane i supplies the
    // address of 4 consecutive d of key row (i / 4) and receives one d of 4 keys. Lane
    // (g, i, hh) of block db reads d-chunk 2*db + g (lower half of d) for i%4 in {0, 2} and
    // CPR/2 + 2*db + g (upper half) for i%4 in {1, 3}; i%4 in {2, 3} take the chunk's upper
    // 8 bytes. Per d block: the slot of chunk v_chunk + 2*db, less the 2*db*CS added at each
    // read. v_rd1 is the base of the second read (rows +4): with the D = 64 row swizzle the
    // upper-half lanes find rows 0-3 at positions 4-7 and rows 4-7 at positions 0-3.
    const int vg = l32 >> 4;
    const int vi = lane & 15;
    const int v_chunk = ((vi & 1) ? CPR / 2 : 0) + vg;
    const bool v_swz = L::V_ROW_SWIZZLE && (vi & 1);
#pragma unroll
    for (int db = 0; db < DB; ++db) {
      v_rd[db] = ((8 * hh) / RPG) * RG + ((8 * hh) % RPG + (vi >> 2) + (v_swz ? 4 : 0)) * 16 +
                 (L::v_slot(v_chunk + 2 * db) - 2 * db) * CS + ((vi >> 1) & 1) * 8;
      v_rd1[db] = v_rd[db] - (v_swz ? 128 : 0);
    }
  }

  // Key of accumulator register r of block kb: 32kb + key_perm(8(r/4) + 4hh + r%4), which is
  // 8hh plus a compile-time constant (key_perm moves hh to bit 3).
  static constexpr int acc_key0(int kb, int r) { return 32 * kb + key_perm(8 * (r >> 2) + (r & 3)); }

  __device__ __forceinline__ void load_q(const char* qbuf, bf16x8_t* qf) const {
#pragma unroll
    for (int kk = 0; kk < DK; ++kk) qf[kk] = *reinterpret_cast<const bf16x8_t*>(qbuf + q_rd + kk * CS);
  }

  // S^T = K Q^T for one 64-key tile (two 32-key blocks) from the K tile at `ks`.
  __device__ __forceinline__ void s_products(const char* ks, const bf16x8_t* qf, f32x16_t* sacc) const {
#pragma unroll
    for (int kb = 0; kb < 2; ++kb)
#pragma unroll
      for (int r = 0; r < 16; ++r) sacc[kb][r] = 0.0f;
    bf16x8_t kf[DK][2];
#pragma unroll
    for (int kk = 0; kk < DK; ++kk)
#pragma unroll
      for (int kb = 0; kb < 2; ++kb)
        kf[kk][kb] = *reinterpret_cast<const bf16x8_t*>(ks + k_rd + kb * (32 / RPG) * RG + kk * CS);
    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
    for (int kk = 0; kk < DK; ++kk)
#pragma unroll
      for (int kb = 0; kb < 2; ++kb)
        sacc[kb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(kf[kk][kb], qf[kk], sacc[kb], 0, 0, 0);
  }

  // Online softmax (fp32, exp2 with the scale c = log2(e)/sqrt(d) folded into one FMA) of one
  // tile's scores; P^T packed to bf16 as the B operand of O^T += V^T P^T. Keys at index >= lim
  // within the tile (the ragged end of a key range) get -inf. The running max is raised, and O
  // and l rescaled, only when a row's max grows by more than 2^8.
  __device__ __forceinline__ void softmax(int lim, float c, f32x16_t* sacc, bf16x8_t* pf, float& m_run, float& l_run,
                                          f32x16_t* oacc) const {
    if (lim < BN) {
      const int lim_l = lim - 8 * hh;
#pragma unroll
      for (int kb = 0; kb < 2; ++kb)
#pragma unroll
        for (int r = 0; r < 16; ++r)
          if (acc_key0(kb, r) >= lim_l) sacc[kb][r] = -__builtin_inff();
    }
    float mx = sacc[0][0];
#pragma unroll
    for (int kb = 0; kb < 2; ++kb)
#pragma unroll
      for (int r = 0; r < 16; ++r) mx = fmaxf(mx, sacc[kb][r]);
    mx = wave_half_max(mx) * c;
    const bool need = mx > m_run + 8.0f;
    if (__builtin_amdgcn_ballot_w64(need) != 0) {
      const float m_new = need ? mx : m_run;
      const float alpha = __builtin_amdgcn_exp2f(m_run - m_new);
      m_run = m_new;
      l_run *= alpha;
#pragma unroll
      for (int db = 0; db < DB; ++db)
#pragma unroll
        for (int r = 0; r < 16; ++r) oacc[db][r] *= alpha;
    }
    const float neg_m = -m_run;
    float lsum = 0.0f;
#pragma unroll
    for (int kb = 0; kb < 2; ++kb) {
#pragma unroll
      for (int ch = 0; ch < 2; ++ch) {
        u32x4_t packed;
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const float p0 = __builtin_amdgcn_exp2f(__builtin_fmaf(sacc[kb][8 * ch + 2 * e], c, neg_m));
          const float p1 = __builtin_amdgcn_exp2f(__builtin_fmaf(sacc[kb][8 * ch + 2 * e + 1], c, neg_m));
          // The row sum adds the bf16-rounded p that the PV product uses. The packed word
          // goes through a scalar temporary: bit-casting the vector element directly
          // (packed[e]) makes hipcc 7.2 feed the same register to every v_dot2c.
          const uint32_t w = pack_bf16x2(p0, p1);
          lsum = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2_t, w),
                                                __builtin_bit_cast(bf16x2_t, 0x3f803f80u), lsum, false);
          packed[e] = w;
        }
        pf[kb * 2 + ch] = __builtin_bit_cast(bf16x8_t, packed);
      }
    }
    l_run += lsum;
  }

  // O^T += V^T P^T for one tile from the V tile at `vs`; the 16 keys of chunk (kb, ch) are
  // rows 32kb + 16ch + 8hh + 0..7
  __device__ __forceinline__ void pv_products(const char* vs, const bf16x8_t* pf, f32x16_t* oacc) const {
#pragma unroll
    for (int kb = 0; kb < 2; ++kb) {
#pragma unroll
      for (int ch = 0; ch < 2; ++ch) {
#pragma unroll
        for (int db = 0; db < DB; ++db) {
          const char* a0 = vs + v_rd[db] + ((32 * kb + 16 * ch) / RPG) * RG + 2 * db * CS;
          const char* a1 = vs + v_rd1[db] + ((32 * kb + 16 * ch + 4) / RPG) * RG + ((32 * kb + 16 * ch + 4) % RPG) * 16 -
                           ((32 * kb + 16 * ch) % RPG) * 16 + 2 * db * CS;
          const bf16x4_t lo = __builtin_amdgcn_ds_read_tr16_b64_v4bf16((lds_bf16x4_t*)a0);
          const bf16x4_t hi = __builtin_amdgcn_ds_read_tr16_b64_v4bf16((lds_bf16x4_t*)a1);
          const bf16x8_t vf = __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7);
          oacc[db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(vf, pf[kb * 2 + ch], oacc[db], 0, 0, 0);
        }
      }
    }
  }

  // Normalise the wave's 32 output rows by 1/l and store each at its original (un-shifted)
  // position. The packed rows go through the wave's part of `buf` (QG / PASSES row groups,
  // laid out like a K tile) in PASSES rounds of 32 / PASSES rows, so that each wave-wide store
  // writes RPG whole rows (16 lanes per 256-byte row) instead of 16 bytes of 64 different
  // rows. row_off[r] is the byte offset (in the resource `ors`) of the tile's query row r;
  // rows past the window hold an offset beyond the resource range and are dropped.
  template <int PASSES>
  __device__ __forceinline__ void store_rows(char* buf, const f32x16_t* oacc, float inv, const uint32_t* row_off,
                                             __amdgpu_buffer_rsrc_t ors, int wave) const {
    constexpr int RP = 32 / PASSES;  // rows per pass
    constexpr int GP = QG / PASSES;  // row groups per pass
#pragma unroll
    for (int pass = 0; pass < PASSES; ++pass) {
      const int lr = l32 - pass * RP;
      if (PASSES == 1 || (lr >= 0 && lr < RP)) {
        const int base = (wave * GP + lr / RPG) * RG + (lr % RPG) * 16 + hh * (CPR / 2) * CS;
#pragma unroll
        for (int db = 0; db < DB; ++db)
#pragma unroll
          for (int half = 0; half < 2; ++half) {
            u32x4_t w;
#pragma unroll
            for (int e = 0; e < 4; ++e)
              w[e] = pack_bf16x2(oacc[db][8 * half + 2 * e] * inv, oacc[db][8 * half + 2 * e + 1] * inv);
            // chunk hh*CPR/2 + 2*db + half of the row
            *reinterpret_cast<u32x4_t*>(buf + base + (2 * db + half) * CS) = w;
          }
      }
      // Lanes read what other lanes of the wave just wrote. The hardware keeps one wave's LDS
      // accesses in order; this compiler barrier stops the compiler from treating the reads as
      // private to each lane (it would otherwise reuse the previous pass's values in the lanes
      // that did not write in this pass).
      asm volatile("" ::: "memory");
      u32x4_t w[GP];
#pragma unroll
      for (int i = 0; i < GP; ++i)
        w[i] = *reinterpret_cast<const u32x4_t*>(buf + (wave * GP + i) * RG + ld_slot * CS + ld_row * 16);
#pragma unroll
      for (int i = 0; i < GP; ++i)
        buffer_store16(ors, row_off[wave * 32 + pass * RP + i * RPG + ld_row] + k_chunk_off, w[i]);
    }
  }
};

// One work item: query tile tile.qtile of window tile.win of head tile.bh. EXT enables the
// routed window and the pooled memory; without them the key/value stream is the window's
// own tiles and the kernel needs fewer scalar registers.
// The single argument of the bf16 kernels: the kernel's argument segment is this struct,
// so the loops can re-read the parameters from it by address.
struct Bf16KernelArgs {
  const uint16_t* q;
  const uint16_t* k;
  const uint16_t* v;
  uint16_t* out;
  AttnParams p;
  uint32_t total;       // work items
  // Per-item kernels: work units >= split_from are the halves of items split_from .. total-1
  // (split_from == total: none); part holds their partial results (SplitPart layout, pair
  // index item - split_from) and arrive one counter per split item, zero between launches.
  uint32_t split_from;
  void* part;
  uint32_t* arrive;
};

// The kernel's parameters, re-read from the argument segment through a pointer the compiler
// cannot see through: kept in scalar registers across the loops they would spill.
__device__ __forceinline__ const Bf16KernelArgs& kernel_args() {
  using ArgPtr = const __attribute__((address_space(4))) Bf16KernelArgs*;
  ArgPtr ap = (ArgPtr)__builtin_amdgcn_kernarg_segment_ptr();
  asm volatile("" : "+s"(ap));
  return *(const Bf16KernelArgs*)ap;
}

// Partial result of half an item (a split item, see win_attn_bf16_items): per wave and lane,
// DB*4 float4 chunks of the unnormalised O accumulators, then (m, l, 0, 0); chunk c of lane
// l at float4 index c*64 + l, so that each chunk is one contiguous wave-wide access.
template <int D, int NW>
struct SplitPart {
  static constexpr int CHUNKS = D / 32 * 4 + 1;
  static constexpr uint64_t HALF_BYTES = uint64_t(NW) * CHUNKS * 64 * 16;  // one half of one item
};

// LDS of one item of the per-item kernels, one set per <D, NW>, shared by the whole-item and
// the half-item code (function-local __shared__ arrays: declared in the item function, each
// instantiation would get its own). The two stages are separate objects: with the stage fixed
// at compile time in each half of the unrolled tile loop, the compiler can tell that the
// transpose reads of one stage do not alias the DMA into the other and does not make them
// wait for it.
template <int D, int NW>
struct ItemLds {
  using C = Bf16Cfg<D, NW>;
  static constexpr int QBUF_BYTES = NW * (32 / TileLayout<D>::RPG) * TileLayout<D>::RG;
  static constexpr int TAB_TILES = 16;  // ring of K/V row offsets, in tiles
  __device__ static __forceinline__ char* stage0() {
    __shared__ __attribute__((aligned(1024))) char b[C::STAGE_BYTES];
    return b;
  }
  __device__ static __forceinline__ char* stage1() {
    __shared__ __attribute__((aligned(1024))) char b[C::STAGE_BYTES];
    return b;
  }
  __device__ static __forceinline__ char* qbuf() {
    __shared__ __attribute__((aligned(1024))) char b[QBUF_BYTES];
    return b;
  }
  __device__ static __forceinline__ uint32_t* rowtab() {
    __shared__ uint32_t b[TAB_TILES * C::BN];
    return b;
  }
  __device__ static __forceinline__ uint32_t* qrowtab() {
    __shared__ uint32_t b[C::BM];
    return b;
  }
};

// HALF: the work item is one half of a split item (key tiles [0, Th) for half 0, [Th, Tn) for
// half 1, Th = ceil(Tn / 2)); the two halves are merged by whichever finishes second.
template <int D, int NW, bool EXT, bool HALF>
__device__ __forceinline__ void win_attn_bf16_item(const uint16_t* __restrict__ q, const uint16_t* __restrict__ k,
                                                   const uint16_t* __restrict__ v, uint16_t* __restrict__ out,
                                                   const AttnParams& p, uint32_t item, uint32_t total, int half) {
  using C = Bf16Cfg<D, NW>;
  using L = TileLayout<D>;
  using LN = Bf16Lane<D, NW>;
  constexpr int BN = C::BN, BM = C::BM, DK = C::DK, DB = C::DB;
  constexpr int RPG = L::RPG, RG = L::RG;
  constexpr int QG = LN::QG;

  using LDS = ItemLds<D, NW>;
  char* const stage0 = LDS::stage0();
  char* const stage1 = LDS::stage1();

  // threadIdx.x through an opaque move: in the item loop of the persistent kernel the
  // compiler would otherwise hoist the lane-derived values of the prologue and keep them
  // live across the tile loop (spills at D = 128).
  int tid;
  asm volatile("v_mov_b32 %0, %1" : "=v"(tid) : "v"(int(threadIdx.x)));
  const int lane = tid & 63;
  // The wave index is the same on every lane. Saying so keeps the LDS addresses derived from
  // it (the DMA destinations) in scalar registers: 10 fewer VGPRs at D = 128 and no
  // readfirstlane before each DMA.
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const LN ln(lane, wave);

  const TileId tile = decode_tile(p, item, total);
  const int64_t base = int64_t(tile.bh) * p.head_stride;
  const WinOrigin org = window_origin(p.map, uint32_t(tile.win));
  const uint32_t head_bytes = uint32_t(p.head_stride) * 2u;
  const __amdgpu_buffer_rsrc_t krs = make_rsrc(k + base, head_bytes);
  const __amdgpu_buffer_rsrc_t vrs = make_rsrc(v + base, head_bytes);
  // The key/value stream is the window's Tw tiles, then (§3.3) as many tiles of the routed
  // window, if any, then (§3.2) mem_tiles tiles of the pooled memory, a plain [n_mem, D]
  // block per head.
  int32_t routed = EXT && p.route != nullptr ? p.route[int64_t(tile.bh) * p.n_win + tile.win] : -1;
  if (routed < 0 || routed >= p.n_win) routed = -1;
  const WinOrigin org_r = window_origin(p.map, uint32_t(routed < 0 ? 0 : routed));
  const int Tw = p.kv_tiles;
  const int Tr = routed < 0 ? 0 : Tw;
  const int Tn = EXT ? Tw + Tr + p.mem_tiles : Tw;
  // key tiles [t0, t1) of the stream; the whole stream unless HALF
  const int Th = (Tn + 1) >> 1;
  const int t0 = HALF && half == 1 ? Th : 0;
  const int t1 = HALF && half == 0 ? Th : Tn;
  const int64_t mem_base = int64_t(tile.bh) * int64_t(p.n_mem) * D;
  const uint32_t mem_bytes = uint32_t(p.n_mem) * uint32_t(L::ROW_BYTES);
  const __amdgpu_buffer_rsrc_t kmrs = make_rsrc(static_cast<const uint16_t*>(p.kmem) + mem_base, mem_bytes);
  const __amdgpu_buffer_rsrc_t vmrs = make_rsrc(static_cast<const uint16_t*>(p.vmem) + mem_base, mem_bytes);

  // Byte offset of a window row in the head (rows past the window get an offset beyond the
  // buffer range, so they read as zeros).
  auto row_offset = [&](int local) __attribute__((always_inline)) -> uint32_t {
    return local < p.wtok ? uint32_t(token_of(p.map, org, uint32_t(local))) * uint32_t(L::ROW_BYTES) : 0xffffff00u;
  };
  // Byte offset of row r of key/value tile t (window tile, or memory tile past Tw).
  auto tile_row_offset = [&](int t, int r) __attribute__((always_inline)) -> uint32_t {
    if (!EXT || t < Tw) return row_offset(t * BN + r);
    if (t < Tw + Tr) {
      const int local = (t - Tw) * BN + r;
      return local < p.wtok ? uint32_t(token_of(p.map, org_r, uint32_t(local))) * uint32_t(L::ROW_BYTES)
                            : 0xffffff00u;
    }
    const int j = (t - Tw - Tr) * BN + r;
    return j < p.n_mem ? uint32_t(j) * uint32_t(L::ROW_BYTES) : 0xffffff00u;
  };
  // ---- K/V tile loads: wave `wave` fills row groups wave*LOADS .. +LOADS-1 of both tiles.
  // row_off: LOADS byte offsets of the lane's K rows, then LOADS of its V rows
  auto dma_tile = [&](const uint32_t* row_off, char* st, int t) __attribute__((always_inline)) {
    const bool mem = EXT && t >= Tw + Tr;
    const __amdgpu_buffer_rsrc_t ks = mem ? kmrs : krs;
    const __amdgpu_buffer_rsrc_t vs = mem ? vmrs : vrs;
#pragma unroll
    for (int i = 0; i < C::LOADS; ++i) {
      const int g = wave * C::LOADS + i;
      dma16_to_lds(ks, st + g * RG, row_off[i] + ln.k_chunk_off);
      dma16_to_lds(vs, st + C::TILE_BYTES + g * RG, row_off[C::LOADS + i] + ln.v_chunk_off);
    }
  };
  // The row offsets of the K/V tiles are computed cooperatively a few tiles ahead into a
  // ring of TAB_TILES tiles in LDS (one row per thread per refill), and each lane reads the
  // LOADS offsets it needs one step before it issues the DMA. The shift/partition index
  // arithmetic thus costs a few instructions per 8 tiles instead of several per row.
  constexpr int TAB_TILES = LDS::TAB_TILES;
  constexpr int REFILL = 8;  // tiles per refill
  uint32_t* const rowtab = LDS::rowtab();
  auto fill_tab = [&](int first, int ntiles) __attribute__((always_inline)) {
    for (int e = tid; e < ntiles * BN; e += C::NT) {
      const int t = first + e / BN;
      rowtab[(t % TAB_TILES) * BN + e % BN] = tile_row_offset(t, e % BN);
    }
  };
  auto read_offs = [&](int t, uint32_t* row_off) __attribute__((always_inline)) {
#pragma unroll
    for (int i = 0; i < C::LOADS; ++i) {
      row_off[i] = rowtab[(t % TAB_TILES) * BN + (wave * C::LOADS + i) * RPG + ln.ld_row];
      if constexpr (L::V_ROW_SWIZZLE)
        row_off[C::LOADS + i] = rowtab[(t % TAB_TILES) * BN + (wave * C::LOADS + i) * RPG + ln.v_ld_row];
      else
        row_off[C::LOADS + i] = row_off[i];
    }
  };

  {  // tile t0 straight from the index map, the table for tiles t0 .. t0 + TAB_TILES - 1
    uint32_t off0[2 * C::LOADS];
#pragma unroll
    for (int i = 0; i < C::LOADS; ++i) {
      off0[i] = tile_row_offset(t0, (wave * C::LOADS + i) * RPG + ln.ld_row);
      off0[C::LOADS + i] = tile_row_offset(t0, (wave * C::LOADS + i) * RPG + ln.v_ld_row);
    }
    dma_tile(off0, stage0, t0);
  }
  fill_tab(t0, min(TAB_TILES, t1 - t0));

  // ---- Q: each wave DMAs its own 32 rows into the Q buffer (laid out like a K tile, 4 whole
  // rows per wave-wide load), and after the prologue barrier reads its fragments from there.
  // Q is read once per workgroup: non-temporal loads keep it out of the way of the K/V in L2.
  // qrowtab keeps the byte offset of every query row for the output stores.
  static_assert(LDS::QBUF_BYTES == NW * QG * RG, "Q buffer size");
  char* const qbuf = LDS::qbuf();
  uint32_t* const qrowtab = LDS::qrowtab();
  {
    const __amdgpu_buffer_rsrc_t qrs = make_rsrc(q + base, head_bytes);
#pragma unroll
    for (int i = 0; i < QG; ++i) {
      const int g = wave * QG + i;
      dma16_to_lds<kCachePolicyNT>(qrs, qbuf + g * RG, row_offset(tile.qtile * BM + g * RPG + ln.ld_row) + ln.k_chunk_off);
    }
    if (tid < BM) qrowtab[tid] = row_offset(tile.qtile * BM + tid);
  }
  bf16x8_t qf[DK];
  f32x16_t oacc[DB];
#pragma unroll
  for (int db = 0; db < DB; ++db)
#pragma unroll
    for (int r = 0; r < 16; ++r) oacc[db][r] = 0.0f;
  float m_run = -__builtin_inff(), l_run = 0.0f;
  const float c = p.scale_log2;

  // One K/V tile: prefetch tile t+1 into `nxt`, compute tile t from `cur`. `next_off`
  // holds the row offsets of tile t+1 (read from the table during the previous step).
  uint32_t next_off[2 * C::LOADS];
  auto tile_step = [&](int t, const char* cur, char* nxt) {
    if (t + 1 < t1) dma_tile(next_off, nxt, t + 1);
    if (t + 2 < t1) read_offs(t + 2, next_off);
    // refill the ring slots of tiles t-8 .. t-1 (all issued) with tiles t+8 .. t+15, first
    // needed by the DMA of step t+7; the barrier ending this step publishes them
    if ((t - t0) % REFILL == 0 && t - t0 >= REFILL && t + REFILL < t1)
      fill_tab(t + REFILL, min(REFILL, t1 - t - REFILL));
    // ragged last tile of the window, the routed window or the memory
    const int lim = !EXT || t < Tw ? p.wtok - t * BN : t < Tw + Tr ? p.wtok - (t - Tw) * BN : p.n_mem - (t - Tw - Tr) * BN;
    f32x16_t sacc[2];
    bf16x8_t pf[4];
    ln.s_products(cur, qf, sacc);
    ln.softmax(lim, c, sacc, pf, m_run, l_run, oacc);
    ln.pv_products(cur + C::TILE_BYTES, pf, oacc);
    __syncthreads();  // next tile resident; everyone is done with this stage
  };

  __syncthreads();  // tile t0 and Q resident, row tables written
  ln.load_q(qbuf, qf);
  if (t0 + 1 < t1) read_offs(t0 + 1, next_off);
  for (int t = t0; t < t1; t += 2) {
    tile_step(t, stage0, stage1);
    if (t + 1 < t1) tile_step(t + 1, stage1, stage0);
  }

  if constexpr (HALF) {
    // Both halves write their partial (O, m, l); the one that arrives second at the item's
    // counter reads the other's and finishes the item. Every wave's stores are complete at
    // the barrier, and the counter's agent-scope release and acquire make them visible to
    // the other half on another XCD.
    typedef float f32x4_t __attribute__((ext_vector_type(4)));
    using SP = SplitPart<D, NW>;
    const Bf16KernelArgs& a = kernel_args();
    const uint32_t pair = item - a.split_from;
    f32x4_t* part = reinterpret_cast<f32x4_t*>(a.part);
    const uint64_t wave_chunks = uint64_t(SP::CHUNKS) * 64;
    f32x4_t* mine = part + ((uint64_t(pair) * 2 + uint64_t(half)) * NW + uint64_t(wave)) * wave_chunks + lane;
    const f32x4_t* other =
        part + ((uint64_t(pair) * 2 + uint64_t(half ^ 1)) * NW + uint64_t(wave)) * wave_chunks + lane;
#pragma unroll
    for (int db = 0; db < DB; ++db)
#pragma unroll
      for (int j = 0; j < 4; ++j)
        mine[(db * 4 + j) * 64] =
            f32x4_t{oacc[db][4 * j], oacc[db][4 * j + 1], oacc[db][4 * j + 2], oacc[db][4 * j + 3]};
    mine[DB * 4 * 64] = f32x4_t{m_run, l_run, 0.0f, 0.0f};
    __shared__ uint32_t first;
    __syncthreads();
    if (tid == 0)
      first = __hip_atomic_fetch_add(a.arrive + pair, 1u, __ATOMIC_ACQ_REL, __HIP_MEMORY_SCOPE_AGENT) == 0u;
    __syncthreads();
    if (first) return;
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "agent");
    // O = O0 2^(m0 - m) + O1 2^(m1 - m), l likewise, m = max(m0, m1), with half 0's terms
    // always first: the result does not depend on which half merges.
    const f32x4_t ml = other[DB * 4 * 64];
    const float m0 = half == 0 ? m_run : ml[0], m1 = half == 0 ? ml[0] : m_run;
    const float l0 = half == 0 ? l_run : ml[1], l1 = half == 0 ? ml[1] : l_run;
    const float mx = fmaxf(m0, m1);
    const float s0 = __builtin_amdgcn_exp2f(m0 - mx), s1 = __builtin_amdgcn_exp2f(m1 - mx);
    m_run = mx;
    l_run = l0 * s0 + l1 * s1;
#pragma unroll
    for (int db = 0; db < DB; ++db)
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const f32x4_t o = other[(db * 4 + j) * 64];
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const float own = oacc[db][4 * j + e];
          oacc[db][4 * j + e] = (half == 0 ? own : o[e]) * s0 + (half == 0 ? o[e] : own) * s1;
        }
      }
    // the counter starts the next launch at zero
    if (tid == 0) __hip_atomic_store(a.arrive + pair, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  }

  // ---- normalise and store each row at its original (un-shifted) position, staged through
  // this wave's part of the Q buffer
  const float l = wave_half_sum(l_run);
  ln.template store_rows<1>(qbuf, oacc, 1.0f / l, qrowtab, make_rsrc(out + base, head_bytes), wave);
  // log-sum-exp of the row's scaled logits, natural log: (m + log2 l) * ln 2
  if (p.lse != nullptr && ln.hh == 0 && tile.qtile * BM + wave * 32 + ln.l32 < p.wtok) {
    const uint32_t tok = qrowtab[wave * 32 + ln.l32] / uint32_t(L::ROW_BYTES);
    p.lse[int64_t(tile.bh) * p.n_tokens + tok] = (m_run + __builtin_amdgcn_logf(l)) * 0.69314718055994531f;
  }
}

// Per-item kernels: a persistent grid of (at most) one workgroup per CU walks the work units
// blockIdx.x, blockIdx.x + gridDim.x, ... This drops the CU's gap between workgroups, which
// is a visible share of a 16-tile item. When the last round would leave more than half of the
// grid idle, its items are split in two along the key stream (unit split_from + 2j + h is half
// h of item split_from + j), so that it takes about half an item instead of a whole one.
template <int D, int NW, bool EXT>
__device__ __forceinline__ void win_attn_bf16_items(const Bf16KernelArgs& a) {
  const uint32_t split_from = a.split_from;
  const uint32_t units = split_from + 2 * (a.total - split_from);
  for (uint32_t u = blockIdx.x; u < units; u += gridDim.x) {
    if (u < split_from) {
      win_attn_bf16_item<D, NW, EXT, false>(a.q, a.k, a.v, a.out, kernel_args().p, u, a.total, 0);
    } else {
      const uint32_t s = u - split_from;
      win_attn_bf16_item<D, NW, EXT, true>(a.q, a.k, a.v, a.out, kernel_args().p, split_from + (s >> 1), a.total,
                                           int(s & 1u));
    }
    __syncthreads();  // the next item's prologue rewrites LDS the epilogue may still read
  }
}

// Plain shifted-window attention (§3.1), one item at a time: windows of one or two key tiles
// or of more than 16, and tensors beyond the stream kernel's 32-bit offsets.
template <int D, int NW>
__global__ __launch_bounds__(NW * 64) __attribute__((amdgpu_waves_per_eu(2))) void win_attn_bf16_kernel(
    Bf16KernelArgs a) {
  win_attn_bf16_items<D, NW, false>(a);
}

// With a routed window (§3.3) and/or pooled memory (§3.2).
template <int D, int NW>
__global__ __launch_bounds__(NW * 64) __attribute__((amdgpu_waves_per_eu(2))) void win_attn_bf16_ext_kernel(
    Bf16KernelArgs a) {
  win_attn_bf16_items<D, NW, true>(a);
}

// Plain shifted-window attention (§3.1) as one continuous K/V tile stream per workgroup.
//
// The persistent workgroup walks items blockIdx.x, blockIdx.x + gridDim.x, ... as one
// sequence of K/V tiles (global tile g = item sequence number * Tn + tile), so that the work
// between two items is off the critical path:
//   * a ring of K/V row offsets holds two items: in the first step of an item every thread
//     writes its share of the next item's row offsets (and query-row offsets), decoding
//     that item once;
//   * the K/V DMA of the last step of an item fetches the next item's first tile;
//   * the next item's query-row offsets are computed in the first step of an item and its
//     Q rows DMA'd into the Q buffer in the second (the Q buffer is free once an item's Q
//     fragments are in registers);
//   * the output rows are staged through the stage the last tile was read from, in two
//     passes of 16 rows per wave (the other stage already holds the next item's first tile).
// Every tensor is addressed through one buffer resource over the whole tensor, with byte
// offsets bh * head_bytes + token * row_bytes: the launcher uses this kernel only when a
// tensor fits in 0xffffff00 bytes and every window has 3 to 16 K/V tiles (the ring holds
// two items, and the next item's offsets, written in an item's first step, are read from
// its second-to-last step on).
template <int D, int NW>
__global__ __launch_bounds__(NW * 64) __attribute__((amdgpu_waves_per_eu(2))) void win_attn_bf16_stream_kernel(
    Bf16KernelArgs a) {
  using C = Bf16Cfg<D, NW>;
  using L = TileLayout<D>;
  using LN = Bf16Lane<D, NW>;
  constexpr int BN = C::BN, BM = C::BM, DK = C::DK, DB = C::DB;
  constexpr int RPG = L::RPG, RG = L::RG;
  constexpr int QG = LN::QG;
  constexpr int TAB_TILES = 32;  // ring slots: two items of at most 16 tiles

  __shared__ __attribute__((aligned(1024))) char stage0[C::STAGE_BYTES];
  __shared__ __attribute__((aligned(1024))) char stage1[C::STAGE_BYTES];
  __shared__ __attribute__((aligned(1024))) char qbuf[NW * QG * RG];
  __shared__ uint32_t rowtab[TAB_TILES * BN];
  __shared__ uint32_t qrowtab[2][BM];
  static_assert(NW * (QG / 2) * RG <= C::STAGE_BYTES, "two-pass output staging must fit one stage");

  int tid;
  asm volatile("v_mov_b32 %0, %1" : "=v"(tid) : "v"(int(threadIdx.x)));
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const LN ln(lane, wave);

  const uint32_t total = a.total;
  const int Tn = a.p.kv_tiles;
  const int wtok = a.p.wtok;
  const float c = a.p.scale_log2;
  const uint32_t head_bytes = uint32_t(a.p.head_stride) * 2u;
  const uint32_t tensor_bytes = uint32_t(a.p.heads_total) * head_bytes;
  const __amdgpu_buffer_rsrc_t krs = make_rsrc(a.k, tensor_bytes);
  const __amdgpu_buffer_rsrc_t vrs = make_rsrc(a.v, tensor_bytes);
  // Q and out are touched a few times per item: their resources are built where used, from
  // the re-read arguments, so that they hold no scalar registers across the tile loop

  // this workgroup's items: blockIdx.x + j * gridDim.x, j < n_items; global tiles g < g_end
  const uint32_t n_items = (total - blockIdx.x + gridDim.x - 1) / gridDim.x;
  const int g_end = int(n_items) * Tn;
  uint32_t item = blockIdx.x;  // current item
  int g0 = 0;                  // global index of its first tile
  int qb = 0;                  // which qrowtab holds its query-row offsets
  // All row offsets of item `it`, whose tiles are global tiles gfirst .. gfirst + Tn - 1:
  // its key/value rows into their ring slots and its query rows into `qrow`, as byte offsets
  // in the whole tensor (rows past the window get an offset beyond the resource range: zero
  // reads, dropped writes). The item is decoded, and the parameters read, once for all.
  auto fill_item = [&](uint32_t it, int gfirst, uint32_t* qrow) __attribute__((always_inline)) {
    const AttnParams& p = kernel_args().p;
    const TileId tl = decode_tile(p, it, total);
    const WinOrigin o = window_origin(p.map, uint32_t(tl.win));
    const uint32_t hb = uint32_t(tl.bh) * head_bytes;
    auto row = [&](int local) __attribute__((always_inline)) -> uint32_t {
      return local < wtok ? hb + uint32_t(token_of(p.map, o, uint32_t(local))) * L::ROW_BYTES : 0xffffff00u;
    };
    for (int e = tid; e < Tn * BN; e += C::NT) rowtab[((gfirst + e / BN) % TAB_TILES) * BN + e % BN] = row(e);
    if (tid < BM) qrow[tid] = row(tl.qtile * BM + tid);
  };
  auto dma_tile = [&](const uint32_t* row_off, char* st) __attribute__((always_inline)) {
#pragma unroll
    for (int i = 0; i < C::LOADS; ++i) {
      const int g = wave * C::LOADS + i;
      dma16_to_lds(krs, st + g * RG, row_off[i] + ln.k_chunk_off);
      dma16_to_lds(vrs, st + C::TILE_BYTES + g * RG, row_off[C::LOADS + i] + ln.v_chunk_off);
    }
  };
  auto read_offs = [&](int g, uint32_t* row_off) __attribute__((always_inline)) {
#pragma unroll
    for (int i = 0; i < C::LOADS; ++i) {
      row_off[i] = rowtab[(g % TAB_TILES) * BN + (wave * C::LOADS + i) * RPG + ln.ld_row];
      if constexpr (L::V_ROW_SWIZZLE)
        row_off[C::LOADS + i] = rowtab[(g % TAB_TILES) * BN + (wave * C::LOADS + i) * RPG + ln.v_ld_row];
      else
        row_off[C::LOADS + i] = row_off[i];
    }
  };
  auto dma_q = [&](int grp, const uint32_t* qrow) __attribute__((always_inline)) {
    const int g = wave * QG + grp;
    dma16_to_lds<kCachePolicyNT>(make_rsrc(kernel_args().q, tensor_bytes), qbuf + g * RG,
                                 qrow[g * RPG + ln.ld_row] + ln.k_chunk_off);
  };

  // ---- prologue: the first item's key/value and query row offsets
  fill_item(item, 0, qrowtab[0]);
  __syncthreads();
  uint32_t next_off[2 * C::LOADS];
  read_offs(0, next_off);
  dma_tile(next_off, stage0);
#pragma unroll
  for (int i = 0; i < QG; ++i) dma_q(i, qrowtab[0]);
  if (1 < g_end) read_offs(1, next_off);
  __syncthreads();  // tile 0 and Q resident

  bf16x8_t qf[DK];
  ln.load_q(qbuf, qf);
  f32x16_t oacc[DB];
#pragma unroll
  for (int db = 0; db < DB; ++db)
#pragma unroll
    for (int r = 0; r < 16; ++r) oacc[db][r] = 0.0f;
  float m_run = -__builtin_inff(), l_run = 0.0f;

  // Work of the first two steps of an item that has a successor: out of line, so that the
  // common step runs straight through.
  auto rare_work = [&](int t) __attribute__((always_inline)) {
    if (t == 0) {
      // all row offsets of the next item, into the ring slots of its tiles (which held the
      // previous item's, all read by now) and into the other query-row table. The ring
      // holds two items, so these are first read in the step before the next item's first
      // DMA, at least one barrier later (an item has at least 3 tiles).
      fill_item(item + gridDim.x, g0 + Tn, qrowtab[qb ^ 1]);
    } else {
      // all of its Q rows in step 1 (measured 2-3 % faster on 4-tile items than spreading
      // them over the item's steps: one short branch instead of a per-step range); a rolled
      // loop keeps the DMA addresses out of the scalar registers held across the tile loop
#pragma unroll 1
      for (int i = 0; i < QG; ++i) dma_q(i, qrowtab[qb ^ 1]);
    }
  };

  // One step of the stream: compute global tile g from `cur`, prefetch tile g+1 into `nxt`.
  // Returns true when g was the last tile of the current item.
  auto step = [&](int g, const char* cur, char* nxt) __attribute__((always_inline)) -> bool {
    const int t = g - g0;
    if (__builtin_expect(g + 1 < g_end, 1)) dma_tile(next_off, nxt);
    if (__builtin_expect(g0 + Tn < g_end && t <= 1, 0)) rare_work(t);
    // Scalar loads the compiler issues above (parameters it re-reads instead of keeping them
    // in registers) return out of order with LDS reads; with one in flight, every wait for
    // the K fragments below would have to be a wait for all of them. Draining here lets the
    // S products start as soon as their first fragments arrive.
    __builtin_amdgcn_s_waitcnt(0xC07F);  // lgkmcnt(0)
    if (__builtin_expect(g + 2 < g_end, 1)) read_offs(g + 2, next_off);
    f32x16_t sacc[2];
    bf16x8_t pf[4];
    ln.s_products(cur, qf, sacc);
    ln.softmax(wtok - t * BN, c, sacc, pf, m_run, l_run, oacc);
    ln.pv_products(cur + C::TILE_BYTES, pf, oacc);
    __syncthreads();  // tile g+1 resident; everyone is done with this stage
    return __builtin_expect(t + 1 == Tn, 0);
  };
  // End of an item: normalise and store its rows through `cur` (free after the last step's
  // barrier), then start the next item. Returns false when there is none.
  auto finish_item = [&](char* cur) __attribute__((always_inline)) -> bool {
    ln.template store_rows<2>(cur, oacc, 1.0f / wave_half_sum(l_run), qrowtab[qb],
                              make_rsrc(kernel_args().out, tensor_bytes), wave);
#pragma unroll
    for (int db = 0; db < DB; ++db)
#pragma unroll
      for (int r = 0; r < 16; ++r) oacc[db][r] = 0.0f;
    m_run = -__builtin_inff();
    l_run = 0.0f;
    if (g0 >= g_end) return false;
    item += gridDim.x;
    qb ^= 1;
    // the staging reads of `cur` are done before the next step's DMA rewrites it; the next
    // item's Q has been in the Q buffer since the first steps of this item. The barrier does
    // not wait for the output stores.
    lds_barrier();
    ln.load_q(qbuf, qf);
    return true;
  };

  for (int g = 0;; g += 2) {
    if (step(g, stage0, stage1)) {
      g0 = g + 1;
      if (!finish_item(stage0)) break;
    }
    if (step(g + 1, stage1, stage0)) {
      g0 = g + 2;
      if (!finish_item(stage1)) break;
    }
  }
}

// ---------------------------------------------------------------------------------
// fp32 kernel: the bf16 kernel's dataflow on fp32 operands, with v_mfma_f32_32x32x2_f32
// (fp32 products, fp32 accumulation; no reduced-precision step anywhere).
//   * A workgroup of 4 waves takes 128 query rows of one (head, window); each wave owns 32
//     rows and keeps its rows' q in registers as the B operand of S^T = K Q^T. For MFMA step
//     s, lane half hh supplies d = hh*D/2 + s (the order of the d terms is free), so each
//     lane's K and Q reads are contiguous.
//   * S^T accumulator register r of lane (l32, hh) holds key 8*(r/4) + 4*hh + r%4 of query
//     row l32. After the softmax, register s is exactly the B operand P^T[key][query] of
//     step s of O^T = V^T P^T, with the A operand V[key][d] read from LDS for the same key.
//   * K/V tiles of 32 keys pass global -> registers -> LDS, double buffered: the loads of
//     tile t+1 are in flight while tile t is computed. Row strides are padded (K by 4
//     floats, V by 8) so that the 16-byte K reads of 32 rows and the 4-byte V reads of
//     two rows four apart are free of bank conflicts.
//   * Online softmax in fp32 with exp2, the same lazy max raise as the bf16 kernel.
template <int D>
struct F32Cfg {
  static constexpr int NW = 4;
  static constexpr int NT = NW * 64;
  static constexpr int BM = NW * 32;         // query rows per workgroup
  static constexpr int BN = 32;              // keys per K/V tile
  static constexpr int KS = D + 4;           // K row stride (floats)
  static constexpr int VS = D + 8;           // V row stride (floats)
  static constexpr int CPR = D / 4;          // 16-byte chunks per row
  static constexpr int CH = BN * CPR / NT;   // chunks per thread per tensor per tile
  static_assert(CH >= 1 && CH * NT == BN * CPR, "tile/thread mismatch");
};

template <int D>
__global__ __launch_bounds__(F32Cfg<D>::NT) __attribute__((amdgpu_waves_per_eu(2))) void win_attn_f32_kernel(const float* __restrict__ q,
                                                                     const float* __restrict__ k,
                                                                     const float* __restrict__ v,
                                                                     float* __restrict__ out, AttnParams p) {
  using C = F32Cfg<D>;
  constexpr int BN = C::BN, KS = C::KS, VS = C::VS, CPR = C::CPR, CH = C::CH, DB = D / 32;
  __shared__ __attribute__((aligned(16))) float Ks[2][BN * KS];
  __shared__ __attribute__((aligned(16))) float Vs[2][BN * VS];

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int l32 = lane & 31;
  const int hh = lane >> 5;

  const TileId tile = decode_tile(p, blockIdx.x, gridDim.x);
  const int64_t base = int64_t(tile.bh) * p.head_stride;
  const WinOrigin org = window_origin(p.map, uint32_t(tile.win));
  // key/value tiles: the window's, the routed window's if any (§3.3), then those of the
  // pooled memory (§3.2)
  int32_t routed = p.route != nullptr ? p.route[int64_t(tile.bh) * p.n_win + tile.win] : -1;
  if (routed < 0 || routed >= p.n_win) routed = -1;
  const WinOrigin org_r = window_origin(p.map, uint32_t(routed < 0 ? 0 : routed));
  const int Tw = (p.wtok + BN - 1) / BN;
  const int Tr = routed < 0 ? 0 : Tw;
  const int Tn = Tw + Tr + (p.n_mem + BN - 1) / BN;
  const float* kmem = static_cast<const float*>(p.kmem) + int64_t(tile.bh) * int64_t(p.n_mem) * D;
  const float* vmem = static_cast<const float*>(p.vmem) + int64_t(tile.bh) * int64_t(p.n_mem) * D;
  auto tile_rows = [&](int t) -> int {  // valid rows of key/value tile t
    if (t < Tw) return p.wtok - t * BN;
    if (t < Tw + Tr) return p.wtok - (t - Tw) * BN;
    return p.n_mem - (t - Tw - Tr) * BN;
  };

  // q row of this lane (B operand of S^T): d = hh*D/2 .. hh*D/2 + D/2 - 1
  const int qlocal = tile.qtile * C::BM + wave * 32 + l32;
  const bool qvalid = qlocal < p.wtok;
  const int qtok = qvalid ? token_of(p.map, org, uint32_t(qlocal)) : 0;
  float qf[D / 2];
  {
    const float4* src = reinterpret_cast<const float4*>(q + base + int64_t(qtok) * D + hh * (D / 2));
#pragma unroll
    for (int i = 0; i < D / 8; ++i) {
      const float4 x = qvalid ? src[i] : make_float4(0.0f, 0.0f, 0.0f, 0.0f);
      qf[4 * i + 0] = x.x;
      qf[4 * i + 1] = x.y;
      qf[4 * i + 2] = x.z;
      qf[4 * i + 3] = x.w;
    }
  }

  // Tile loads: thread tid moves chunks e = tid + j*NT (row e / CPR, chunk e % CPR) of K and V.
  float4 kreg[CH], vreg[CH];
  auto load_tile = [&](int t) __attribute__((always_inline)) {
    const int nrows = tile_rows(t);
    const bool mem = t >= Tw + Tr;
    const bool rt = !mem && t >= Tw;
#pragma unroll
    for (int j = 0; j < CH; ++j) {
      const int e = tid + j * C::NT;
      const int r = e / CPR;
      const int cc = e % CPR;
      kreg[j] = make_float4(0.0f, 0.0f, 0.0f, 0.0f);
      vreg[j] = kreg[j];
      if (r < nrows) {
        const float* ks;
        const float* vs;
        if (mem) {
          const int64_t off = int64_t((t - Tw - Tr) * BN + r) * D + cc * 4;
          ks = kmem + off;
          vs = vmem + off;
        } else {
          const int tok = rt ? token_of(p.map, org_r, uint32_t((t - Tw) * BN + r))
                             : token_of(p.map, org, uint32_t(t * BN + r));
          const int64_t off = base + int64_t(tok) * D + cc * 4;
          ks = k + off;
          vs = v + off;
        }
        kreg[j] = *reinterpret_cast<const float4*>(ks);
        vreg[j] = *reinterpret_cast<const float4*>(vs);
      }
    }
  };
  auto store_tile = [&](int b) __attribute__((always_inline)) {
#pragma unroll
    for (int j = 0; j < CH; ++j) {
      const int e = tid + j * C::NT;
      const int r = e / CPR;
      const int cc = e % CPR;
      *reinterpret_cast<float4*>(&Ks[b][r * KS + cc * 4]) = kreg[j];
      *reinterpret_cast<float4*>(&Vs[b][r * VS + cc * 4]) = vreg[j];
    }
  };

  f32x16_t oacc[DB];
#pragma unroll
  for (int db = 0; db < DB; ++db)
#pragma unroll
    for (int r = 0; r < 16; ++r) oacc[db][r] = 0.0f;
  float m_run = -__builtin_inff(), l_run = 0.0f;
  const float c = p.scale_log2;

  load_tile(0);
  store_tile(0);
  __syncthreads();
  for (int t = 0; t < Tn; ++t) {
    const int cur = t & 1;
    if (t + 1 < Tn) load_tile(t + 1);  // in flight during this tile's products

    // S^T = K Q^T: 32 keys x 32 query rows, D/2 steps of two d each
    f32x16_t sacc;
#pragma unroll
    for (int r = 0; r < 16; ++r) sacc[r] = 0.0f;
    const float* kr = &Ks[cur][l32 * KS + hh * (D / 2)];
#pragma unroll
    for (int s = 0; s < D / 2; s += 4) {
      const float4 kk = *reinterpret_cast<const float4*>(kr + s);
      sacc = __builtin_amdgcn_mfma_f32_32x32x2f32(kk.x, qf[s + 0], sacc, 0, 0, 0);
      sacc = __builtin_amdgcn_mfma_f32_32x32x2f32(kk.y, qf[s + 1], sacc, 0, 0, 0);
      sacc = __builtin_amdgcn_mfma_f32_32x32x2f32(kk.z, qf[s + 2], sacc, 0, 0, 0);
      sacc = __builtin_amdgcn_mfma_f32_32x32x2f32(kk.w, qf[s + 3], sacc, 0, 0, 0);
    }
    // keys past the end of a ragged tile get -inf
    const int nrows = tile_rows(t);
    if (nrows < BN) {
#pragma unroll
      for (int r = 0; r < 16; ++r)
        if (8 * (r >> 2) + 4 * hh + (r & 3) >= nrows) sacc[r] = -__builtin_inff();
    }

    // online softmax (the row's two lane halves agree on the running max)
    float mx = sacc[0];
#pragma unroll
    for (int r = 1; r < 16; ++r) mx = fmaxf(mx, sacc[r]);
    mx = wave_half_max(mx) * c;
    const bool need = mx > m_run + 8.0f;
    if (__builtin_amdgcn_ballot_w64(need) != 0) {
      const float m_new = need ? mx : m_run;
      const float alpha = __builtin_amdgcn_exp2f(m_run - m_new);
      m_run = m_new;
      l_run *= alpha;
#pragma unroll
      for (int db = 0; db < DB; ++db)
#pragma unroll
        for (int r = 0; r < 16; ++r) oacc[db][r] *= alpha;
    }
    const float neg_m = -m_run;
    float lsum = 0.0f;
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      sacc[r] = __builtin_amdgcn_exp2f(__builtin_fmaf(sacc[r], c, neg_m));
      lsum += sacc[r];
    }
    l_run += lsum;

    // O^T += V^T P^T: step s pairs key 8*(s/4) + 4*hh + s%4 of V with register s of P^T
    const float* vr = &Vs[cur][(4 * hh) * VS + l32];
#pragma unroll
    for (int s = 0; s < 16; ++s) {
      const int key_off = (8 * (s >> 2) + (s & 3)) * VS;
#pragma unroll
      for (int db = 0; db < DB; ++db)
        oacc[db] = __builtin_amdgcn_mfma_f32_32x32x2f32(vr[key_off + 32 * db], sacc[s], oacc[db], 0, 0, 0);
    }

    if (t + 1 < Tn) store_tile(cur ^ 1);  // everyone finished reading that buffer last step
    __syncthreads();
  }

  const float l = wave_half_sum(l_run);
  if (qvalid) {
    const float inv = 1.0f / l;
    float* orow = out + base + int64_t(qtok) * D;
#pragma unroll
    for (int db = 0; db < DB; ++db)
#pragma unroll
      for (int g = 0; g < 4; ++g)  // registers 4g..4g+3: d = 32db + 8g + 4hh + 0..3
        *reinterpret_cast<float4*>(orow + 32 * db + 8 * g + 4 * hh) =
            make_float4(oacc[db][4 * g] * inv, oacc[db][4 * g + 1] * inv, oacc[db][4 * g + 2] * inv,
                        oacc[db][4 * g + 3] * inv);
    if (p.lse != nullptr && hh == 0)
      p.lse[int64_t(tile.bh) * p.n_tokens + qtok] = (m_run + __builtin_amdgcn_logf(l)) * 0.69314718055994531f;
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
// Window descriptors (BASA §3.3): the mean of q (blockIdx.y = 0) or k (1) over each
// window's members, in fp32. One workgroup per (bh, window): 256 threads take CPR chunks
// of 256/CPR rows at a time (whole rows per group of CPR threads), then reduce the row
// groups through LDS.
template <int D, typename T>
__global__ __launch_bounds__(256) void window_mean_kernel(const T* __restrict__ q, const T* __restrict__ k,
                                                          float* __restrict__ qbar, float* __restrict__ kbar,
                                                          WinMap map, int32_t wtok, int32_t n_win,
                                                          int64_t head_stride) {
  constexpr int EPC = 16 / sizeof(T);
  constexpr int CPR = D / EPC;
  constexpr int RPP = 256 / CPR;  // rows per pass
  __shared__ float part[RPP][D];
  const T* src = blockIdx.y == 0 ? q : k;
  float* dst = blockIdx.y == 0 ? qbar : kbar;
  const int win = int(blockIdx.x % uint32_t(n_win));
  const int64_t bh = blockIdx.x / uint32_t(n_win);
  const WinOrigin org = window_origin(map, uint32_t(win));
  const int chunk = threadIdx.x % CPR;
  const int rsub = threadIdx.x / CPR;
  const T* head = src + bh * head_stride + chunk * EPC;
  float acc[EPC];
#pragma unroll
  for (int e = 0; e < EPC; ++e) acc[e] = 0.0f;
  for (int local = rsub; local < wtok; local += RPP) {
    const T* row = head + int64_t(token_of(map, org, uint32_t(local))) * D;
    if constexpr (sizeof(T) == 2) {
      const u32x4_t x = *reinterpret_cast<const u32x4_t*>(row);
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        acc[2 * e] += __uint_as_float(x[e] << 16);
        acc[2 * e + 1] += __uint_as_float(x[e] & 0xffff0000u);
      }
    } else {
      const float4 x = *reinterpret_cast<const float4*>(row);
      acc[0] += x.x;
      acc[1] += x.y;
      acc[2] += x.z;
      acc[3] += x.w;
    }
  }
#pragma unroll
  for (int e = 0; e < EPC; ++e) part[rsub][chunk * EPC + e] = acc[e];
  __syncthreads();
  if (threadIdx.x < D) {
    float sum = 0.0f;
    for (int r = 0; r < RPP; ++r) sum += part[r][threadIdx.x];
    dst[(bh * n_win + win) * D + threadIdx.x] = sum / float(wtok);
  }
}

// Top-1 routing over the radius neighbourhood of each window (BASA §3.3, App. A.2): one
// thread per (bh, window); candidates in ascending index order, strict comparison, so
// ties keep the lowest index.
template <int D>
__global__ __launch_bounds__(64) void route_top1_kernel(const float* __restrict__ qbar,
                                                        const float* __restrict__ kbar, int32_t* __restrict__ route,
                                                        int32_t bh_total, int32_t nt, int32_t nh, int32_t nw,
                                                        int32_t radius, float scale) {
  const int64_t idx = int64_t(blockIdx.x) * 64 + threadIdx.x;
  const int64_t n_win = int64_t(nt) * nh * nw;
  if (idx >= int64_t(bh_total) * n_win) return;
  const int64_t bh = idx / n_win;
  const int i = int(idx % n_win);
  const int ti = i / (nh * nw), hi = (i / nw) % nh, wi = i % nw;
  const float* qi = qbar + idx * D;
  int best = -1;
  float best_s = 0.0f;
  for (int tj = max(0, ti - radius); tj <= min(nt - 1, ti + radius); ++tj)
    for (int hj = max(0, hi - radius); hj <= min(nh - 1, hi + radius); ++hj)
      for (int wj = max(0, wi - radius); wj <= min(nw - 1, wi + radius); ++wj) {
        const int j = (tj * nh + hj) * nw + wj;
        if (j == i) continue;
        const float* kj = kbar + (bh * n_win + j) * D;
        float s = 0.0f;
        for (int d = 0; d < D; ++d) s = __builtin_fmaf(qi[d], kj[d], s);
        s *= scale;
        if (best < 0 || s > best_s) {
          best = j;
          best_s = s;
        }
      }
  route[idx] = best;
}

hipError_t launch_window_means(const void* q, const void* k, float* qbar, float* kbar, const WinMap& map,
                               int32_t wtok, int32_t n_win, int32_t bh, int64_t head_stride, int head_dim, bool bf16,
                               hipStream_t stream) {
  const uint64_t blocks = uint64_t(bh) * uint64_t(n_win);
  if (blocks == 0 || blocks > 0x7fffffffu) return hipErrorInvalidConfiguration;
  const dim3 grid(uint32_t(blocks), 2);
#define BASA_MEANS(DD, TT)                                                                                      \
  hipLaunchKernelGGL((window_mean_kernel<DD, TT>), grid, dim3(256), 0, stream, static_cast<const TT*>(q),      \
                     static_cast<const TT*>(k), qbar, kbar, map, wtok, n_win, head_stride)
  if (bf16 && head_dim == 128) BASA_MEANS(128, uint16_t);
  else if (bf16 && head_dim == 64) BASA_MEANS(64, uint16_t);
  else if (!bf16 && head_dim == 128) BASA_MEANS(128, float);
  else if (!bf16 && head_dim == 64) BASA_MEANS(64, float);
  else return hipErrorInvalidValue;
#undef BASA_MEANS
  return hipGetLastError();
}

hipError_t launch_route_top1(const float* qbar, const float* kbar, int32_t* route, int32_t bh, int32_t nt,
                             int32_t nh, int32_t nw, int32_t radius, int head_dim, hipStream_t stream) {
  const uint64_t threads = uint64_t(bh) * uint64_t(nt) * uint64_t(nh) * uint64_t(nw);
  const uint64_t blocks = (threads + 63) / 64;
  if (blocks == 0 || blocks > 0x7fffffffu) return hipErrorInvalidConfiguration;
  const float scale = float(1.0 / sqrt(double(head_dim)));
  if (head_dim == 128)
    hipLaunchKernelGGL(route_top1_kernel<128>, dim3(uint32_t(blocks)), dim3(64), 0, stream, qbar, kbar, route, bh,
                       nt, nh, nw, radius, scale);
  else if (head_dim == 64)
    hipLaunchKernelGGL(route_top1_kernel<64>, dim3(uint32_t(blocks)), dim3(64), 0, stream, qbar, kbar, route, bh,
                       nt, nh, nw, radius, scale);
  else
    return hipErrorInvalidValue;
  return hipGetLastError();
}

// ---------------------------------------------------------------------------------
// K/V pooling (BASA §3.2): one thread per (bh, frame, region, 16-byte chunk of the row).
// Consecutive threads take consecutive chunks of one region, so each token row of the
// region is read as whole coalesced rows; the mean is accumulated in fp32 and stored in
// the tensor's type (bf16: round to nearest even). blockIdx.y selects k (0) or v (1).
template <int D, typename T>
__global__ __launch_bounds__(256) void pool_kv_kernel(const T* __restrict__ k, const T* __restrict__ v,
                                                      T* __restrict__ kmem, T* __restrict__ vmem, int32_t bh_total,
                                                      int32_t nT, int32_t H, int32_t W, int32_t ph, int32_t pw,
                                                      int32_t gh, int32_t gw) {
  constexpr int EPC = 16 / sizeof(T);  // elements per 16-byte chunk
  constexpr int CPR = D / EPC;         // chunks per row
  const T* src = blockIdx.y == 0 ? k : v;
  T* dst = blockIdx.y == 0 ? kmem : vmem;
  const int64_t idx = int64_t(blockIdx.x) * 256 + threadIdx.x;
  const int64_t G = int64_t(gh) * gw;
  const int64_t total = int64_t(bh_total) * nT * G * CPR;
  if (idx >= total) return;
  const int chunk = int(idx % CPR);
  const int64_t region = idx / CPR;  // (bh, t, i, j) row-major
  const int j = int(region % gw);
  const int i = int((region / gw) % gh);
  const int64_t frame = region / G;  // bh * nT + t
  const int h0 = i * ph, w0 = j * pw;
  const int h1 = min(h0 + ph, H), w1 = min(w0 + pw, W);
  float acc[EPC];
#pragma unroll
  for (int e = 0; e < EPC; ++e) acc[e] = 0.0f;
  for (int h = h0; h < h1; ++h) {
    const T* row = src + ((frame * H + h) * W + w0) * D + chunk * EPC;
    for (int w = w0; w < w1; ++w, row += D) {
      if constexpr (sizeof(T) == 2) {
        const u32x4_t x = *reinterpret_cast<const u32x4_t*>(row);
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          acc[2 * e] += __uint_as_float(x[e] << 16);
          acc[2 * e + 1] += __uint_as_float(x[e] & 0xffff0000u);
        }
      } else {
        const float4 x = *reinterpret_cast<const float4*>(row);
        acc[0] += x.x;
        acc[1] += x.y;
        acc[2] += x.z;
        acc[3] += x.w;
      }
    }
  }
  const float inv = 1.0f / float((h1 - h0) * (w1 - w0));
  T* o = dst + region * D + chunk * EPC;
  if constexpr (sizeof(T) == 2) {
    u32x4_t y;
#pragma unroll
    for (int e = 0; e < 4; ++e) y[e] = pack_bf16x2(acc[2 * e] * inv, acc[2 * e + 1] * inv);
    *reinterpret_cast<u32x4_t*>(o) = y;
  } else {
    *reinterpret_cast<float4*>(o) = make_float4(acc[0] * inv, acc[1] * inv, acc[2] * inv, acc[3] * inv);
  }
}

hipError_t launch_pool_kv(const void* k, const void* v, void* kmem, void* vmem, int32_t bh, int32_t T, int32_t H,
                          int32_t W, int32_t ph, int32_t pw, int head_dim, bool bf16, hipStream_t stream) {
  const int32_t gh = (H + ph - 1) / ph, gw = (W + pw - 1) / pw;
  const int epc = bf16 ? 8 : 4;
  const uint64_t threads = uint64_t(bh) * uint64_t(T) * uint64_t(gh) * uint64_t(gw) * uint64_t(head_dim / epc);
  const uint64_t blocks = (threads + 255) / 256;
  if (blocks == 0 || blocks > 0x7fffffffu) return hipErrorInvalidConfiguration;
  const dim3 grid(uint32_t(blocks), 2);
#define BASA_POOL(DD, TT)                                                                                      \
  hipLaunchKernelGGL((pool_kv_kernel<DD, TT>), grid, dim3(256), 0, stream, static_cast<const TT*>(k),        \
                     static_cast<const TT*>(v), static_cast<TT*>(kmem), static_cast<TT*>(vmem), bh, T, H, W, ph, \
                     pw, gh, gw)
  if (bf16 && head_dim == 128) BASA_POOL(128, uint16_t);
  else if (bf16 && head_dim == 64) BASA_POOL(64, uint16_t);
  else if (!bf16 && head_dim == 128) BASA_POOL(128, float);
  else if (!bf16 && head_dim == 64) BASA_POOL(64, float);
  else return hipErrorInvalidValue;
#undef BASA_POOL
  return hipGetLastError();
}

// ---------------------------------------------------------------------------------
// Workgroups of the persistent bf16 kernel: one per CU of the current device (a workgroup
// takes most of a CU's LDS), rounded down to a multiple of the XCD count so that every
// workgroup's items stay on its XCD. Queried once per device.
static hipError_t persistent_slots(uint32_t* slots) {
  static std::atomic<uint32_t> cache[64];  // 0 = not read yet; concurrent first reads agree
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  const bool cached = dev >= 0 && dev < 64;
  if (cached) {
    const uint32_t n = cache[dev].load(std::memory_order_relaxed);
    if (n != 0) {
      *slots = n;
      return hipSuccess;
    }
  }
  int cus = 0;
  e = hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev);
  if (e != hipSuccess) return e;
  uint32_t n = uint32_t(cus) / kNumXcd * kNumXcd;
  if (n == 0) n = kNumXcd;
  if (cached) cache[dev].store(n, std::memory_order_relaxed);
  *slots = n;
  return hipSuccess;
}

// Workspace of split items for the per-item kernels: for each of at most slots/2 items, two
// SplitPart halves (sized for D = 128, which also holds D = 64), then one arrival counter per
// item. The counters are zeroed when the workspace is made and every launch leaves them at
// zero (the merging half resets its item's).
static constexpr uint64_t split_counter_offset(uint32_t slots) {
  return uint64_t(slots / 2) * 2 * SplitPart<128, 8>::HALF_BYTES;
}
static constexpr uint64_t split_workspace_bytes(uint32_t slots) {
  return split_counter_offset(slots) + uint64_t(slots / 2) * 4;
}

// The workspace of basa_window_attn_fwd_noalloc, for callers that cannot allocate: a static
// device array (one per device the library runs on, held until the process ends) in the
// split-workspace layout for grids of up to kScratchSlots workgroups, i.e. at most 128 split
// items: 35.7 MB. Every such call on a device uses the same array; calls that overlap on one
// device race. Host code uses the address from scratch_address(), never the array's name
// (which on the host is a stand-in, not a device address).
constexpr uint32_t kScratchSlots = 256;
static __device__ __attribute__((aligned(256))) char scratch[split_workspace_bytes(kScratchSlots)];

// Device address of `scratch` on the current device, looked up once per device.
static hipError_t scratch_address(void** addr) {
  static std::mutex mu;
  static void* known[64] = {};
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= 64) return hipErrorInvalidDevice;
  std::lock_guard<std::mutex> lock(mu);
  if (known[dev] == nullptr) {
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return e;
    known[dev] = p;
  }
  *addr = known[dev];
  return hipSuccess;
}

// Zero n counters (a kernel rather than a memset, so that a graph capturing the call replays
// it correctly).
__global__ __launch_bounds__(256) void clear_counters_kernel(uint32_t* c, uint32_t n) {
  const uint32_t i = blockIdx.x * 256u + threadIdx.x;
  if (i < n) c[i] = 0u;
}

// The library's own workspace, one per (device, stream), made on the first launch on that
// stream that splits items and kept until the process ends; at most kMaxWorkspaces per
// device. Launches on one stream run in order, so they can share it; launches on different
// streams never do. Returns null (no split) while the stream is being captured into a graph
// and has no workspace yet, when the device already has kMaxWorkspaces, or when the
// allocation fails.
constexpr int kMaxWorkspaces = 16;
static void* split_workspace(hipStream_t stream, uint32_t slots) {
  static std::mutex mu;
  static std::map<std::pair<int, hipStream_t>, void*> made;
  static std::map<int, int> per_device;
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess) return nullptr;
  std::lock_guard<std::mutex> lock(mu);
  const auto key = std::make_pair(dev, stream);
  const auto it = made.find(key);
  if (it != made.end()) return it->second;
  if (per_device[dev] >= kMaxWorkspaces) return nullptr;
  hipStreamCaptureStatus cap = hipStreamCaptureStatusNone;
  if (hipStreamIsCapturing(stream, &cap) != hipSuccess || cap != hipStreamCaptureStatusNone) return nullptr;
  void* ws = nullptr;
  if (hipMalloc(&ws, split_workspace_bytes(slots)) != hipSuccess) {
    (void)hipGetLastError();  // not an error of this launch: it runs unsplit
    return nullptr;
  }
  if (hipMemsetAsync(static_cast<char*>(ws) + split_counter_offset(slots), 0, uint64_t(slots / 2) * 4, stream) !=
      hipSuccess) {
    (void)hipGetLastError();
    (void)hipFree(ws);
    return nullptr;
  }
  made.emplace(key, ws);
  ++per_device[dev];
  return ws;
}

// no_alloc: split items keep their partial results in `scratch` instead of a workspace of the
// stream (hipErrorOutOfMemory if the split needs more than it holds).
template <int D, int NW>
static hipError_t launch_bf16(const void* q, const void* k, const void* v, void* out, AttnParams p,
                              bool no_alloc, hipStream_t stream) {
  using C = Bf16Cfg<D, NW>;
  p.q_tiles = (p.wtok + C::BM - 1) / C::BM;
  p.kv_tiles = (p.wtok + C::BN - 1) / C::BN;
  p.mem_tiles = (p.n_mem + C::BN - 1) / C::BN;
  const uint64_t blocks = uint64_t(p.q_tiles) * uint64_t(p.n_win) * uint64_t(p.heads_total);
  if (blocks == 0 || blocks > 0x7fffffffu) return hipErrorInvalidConfiguration;
  p.f_kv_tiles = make_fastdiv(uint32_t(p.kv_tiles));  // all three >= 1 here
  p.f_q_tiles = make_fastdiv(uint32_t(p.q_tiles));
  p.f_n_win = make_fastdiv(uint32_t(p.n_win));
  Bf16KernelArgs a;
  a.q = static_cast<const uint16_t*>(q);
  a.k = static_cast<const uint16_t*>(k);
  a.v = static_cast<const uint16_t*>(v);
  a.out = static_cast<uint16_t*>(out);
  a.p = p;
  a.total = uint32_t(blocks);
  a.split_from = a.total;
  a.part = nullptr;
  a.arrive = nullptr;
  uint32_t slots = 0;
  const hipError_t e = persistent_slots(&slots);
  if (e != hipSuccess) return e;
  // the static array's address on this device, taken on the first no_alloc call there
  void* scratch_ptr = nullptr;
  if (no_alloc) {
    const hipError_t es = scratch_address(&scratch_ptr);
    if (es != hipSuccess) return es;
  }
  const uint32_t grid = blocks < slots ? uint32_t(blocks) : slots;
  // The stream kernel takes the item transitions off the critical path (measured: FLUX-1024,
  // 4 tiles, 8 % faster than the per-item kernel; FLUX-2048 and FLUX-4096, 16 tiles, 2-4 %
  // faster). Its ring of row offsets holds two items of at most 16 tiles, the next item's
  // offsets are written in an item's first step and read from its second-to-last step on
  // (so at least 3 tiles), it addresses a whole tensor through one 32-bit buffer range
  // (rows past a window at offsets from 0xffffff00 up) and numbers a workgroup's tiles with
  // 32-bit integers.
  const uint64_t tensor_bytes = uint64_t(p.heads_total) * uint64_t(p.head_stride) * 2u;
  const uint64_t wg_tiles = (blocks + grid - 1) / grid * uint64_t(p.kv_tiles);
  const bool ext = p.route != nullptr || p.n_mem > 0 || p.lse != nullptr;
  const bool stream_kernel =
      !ext && p.kv_tiles >= 3 && p.kv_tiles <= 16 && tensor_bytes <= 0xffffff00u && wg_tiles < 0x7fffffffu;
  // Per-item kernels: split the items of a last round that would fill at most half the grid
  // (each half needs a key tile of its own). Measured on the 21x30x52 Wan grid (3168 items of
  // 43 tiles on 256 CUs, 96 in the last round): 2.5-4 % faster.
  const uint32_t tail = uint32_t(blocks % grid);
  if (!stream_kernel && blocks > grid && tail != 0 && tail <= grid / 2 && p.kv_tiles >= 2) {
    void* ws = nullptr;
    uint64_t counters = 0;
    if (no_alloc) {
      if (tail > kScratchSlots / 2) return hipErrorOutOfMemory;
      ws = scratch_ptr;
      counters = split_counter_offset(kScratchSlots);
      // the array keeps the last call's contents: the counters of this call start at zero
      hipLaunchKernelGGL(clear_counters_kernel, dim3((tail + 255) / 256), dim3(256), 0, stream,
                         reinterpret_cast<uint32_t*>(static_cast<char*>(ws) + counters), tail);
    } else {
      ws = split_workspace(stream, slots);
      counters = split_counter_offset(slots);
    }
    if (ws != nullptr) {
      a.split_from = uint32_t(blocks) - tail;
      a.part = ws;
      a.arrive = reinterpret_cast<uint32_t*>(static_cast<char*>(ws) + counters);
    }
  }
  if (ext)
    hipLaunchKernelGGL((win_attn_bf16_ext_kernel<D, NW>), dim3(grid), dim3(C::NT), 0, stream, a);
  else if (stream_kernel)
    hipLaunchKernelGGL((win_attn_bf16_stream_kernel<D, NW>), dim3(grid), dim3(C::NT), 0, stream, a);
  else
    hipLaunchKernelGGL((win_attn_bf16_kernel<D, NW>), dim3(grid), dim3(C::NT), 0, stream, a);
  return hipGetLastError();
}

template <int D>
static hipError_t launch_f32(const void* q, const void* k, const void* v, void* out, AttnParams p,
                             hipStream_t stream) {
  using C = F32Cfg<D>;
  p.q_tiles = (p.wtok + C::BM - 1) / C::BM;
  p.kv_tiles = (p.wtok + C::BN - 1) / C::BN;
  p.mem_tiles = (p.n_mem + C::BN - 1) / C::BN;
  const uint64_t blocks = uint64_t(p.q_tiles) * uint64_t(p.n_win) * uint64_t(p.heads_total);
  if (blocks == 0 || blocks > 0x7fffffffu) return hipErrorInvalidConfiguration;
  p.f_q_tiles = make_fastdiv(uint32_t(p.q_tiles));  // both >= 1 here
  p.f_n_win = make_fastdiv(uint32_t(p.n_win));
  hipLaunchKernelGGL((win_attn_f32_kernel<D>), dim3(uint32_t(blocks)), dim3(C::NT), 0, stream,
                     static_cast<const float*>(q), static_cast<const float*>(k), static_cast<const float*>(v),
                     static_cast<float*>(out), p);
  return hipGetLastError();
}

hipError_t launch_window_attention(const void* q, const void* k, const void* v, void* out, const AttnParams& p,
                                   int head_dim, bool bf16, bool no_alloc, hipStream_t stream) {
  if (bf16) {
    if (head_dim == 128) return launch_bf16<128, 8>(q, k, v, out, p, no_alloc, stream);
    if (head_dim == 64) return launch_bf16<64, 8>(q, k, v, out, p, no_alloc, stream);
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
