// Shifted-window index map: (window id, local slot) -> flat token of the original grid.
//
// BASA paper (arXiv 2610.08772), §3.1 "Shifted Window Sparse Attention": the token grid
// is rolled by -Delta and cut into non-overlapping windows; App. A.1 "Regular execution
// with standard attention backends": the cut is a plain reshape/permute of a grid that
// the window divides exactly. Rolling by -Delta puts original position (i + Delta) mod n
// at rolled position i, so along each axis window m, local slot l holds the original
// position (m*w + l + Delta) mod n. Windows and slots are numbered row-major over
// (t, h, w); tokens are flattened row-major over (t, h, w).
//
// This header is plain C++ (usable from a host-only compiler) and HIP device code.
#pragma once
#include <stdint.h>

#if defined(__HIPCC__)
#define BASA_HD __host__ __device__ __forceinline__
#else
#define BASA_HD inline
#endif

namespace basa {

// Unsigned division by a run-time invariant d >= 1 for numerators n < 2^31, by one
// 32x32->64 multiply and a shift (Granlund & Montgomery, "Division by Invariant Integers
// using Multiplication", PLDI 1994, Thm 4.2 with N = 31): with l = ceil(log2 d) and
// m = ceil(2^(31+l) / d), m*d lies in [2^(31+l), 2^(31+l) + 2^l], hence
// floor(n/d) = floor(n*m / 2^(31+l)) for all 0 <= n < 2^31. m < 2^32 for every d < 2^31.
struct FastDiv {
  uint32_t d;
  uint32_t m;
  uint32_t shift;  // 31 + l
};

inline FastDiv make_fastdiv(uint32_t d) {
  uint32_t l = 0;
  while ((uint64_t(1) << l) < d) ++l;
  const uint64_t two = uint64_t(1) << (31 + l);
  FastDiv f;
  f.d = d;
  f.m = uint32_t((two + d - 1) / d);
  f.shift = 31 + l;
  return f;
}

BASA_HD uint32_t fdiv(uint32_t n, const FastDiv& f) {
  return uint32_t((uint64_t(n) * f.m) >> f.shift);
}

// Geometry of one shifted partition. Shifts are already reduced into [0, n).
struct WinMap {
  int32_t T, H, W;     // token grid
  int32_t wt, wh, ww;  // window
  int32_t st, sh, sw;  // shift
  int32_t nh, nw;      // windows along h and w
  int32_t whw;         // wh * ww
  FastDiv f_whw;       // / (wh * ww)
  FastDiv f_ww;        // / ww
  FastDiv f_nhw;       // / (nh * nw)
  FastDiv f_nw;        // / nw
};

inline WinMap make_winmap(int T, int H, int W, int wt, int wh, int ww, int st, int sh, int sw) {
  WinMap m;
  m.T = T; m.H = H; m.W = W;
  m.wt = wt; m.wh = wh; m.ww = ww;
  m.st = st; m.sh = sh; m.sw = sw;
  m.nh = H / wh; m.nw = W / ww;
  m.whw = wh * ww;
  m.f_whw = make_fastdiv(uint32_t(wh * ww));
  m.f_ww = make_fastdiv(uint32_t(ww));
  m.f_nhw = make_fastdiv(uint32_t(m.nh * m.nw));
  m.f_nw = make_fastdiv(uint32_t(m.nw));
  return m;
}

// Grid position of local slot 0 of a window: (m_a * w_a + s_a) mod n_a per axis.
struct WinOrigin {
  int32_t t0, h0, w0;
};

BASA_HD WinOrigin window_origin(const WinMap& m, uint32_t win) {
  const uint32_t mt = fdiv(win, m.f_nhw);
  const uint32_t r = win - mt * uint32_t(m.nh * m.nw);
  const uint32_t mh = fdiv(r, m.f_nw);
  const uint32_t mw = r - mh * uint32_t(m.nw);
  WinOrigin o;
  o.t0 = int32_t(mt) * m.wt + m.st;
  if (o.t0 >= m.T) o.t0 -= m.T;
  o.h0 = int32_t(mh) * m.wh + m.sh;
  if (o.h0 >= m.H) o.h0 -= m.H;
  o.w0 = int32_t(mw) * m.ww + m.sw;
  if (o.w0 >= m.W) o.w0 -= m.W;
  return o;
}

// Flat original token of local slot `local` (< window tokens) of the window at `o`.
BASA_HD int32_t token_of(const WinMap& m, const WinOrigin& o, uint32_t local) {
  const uint32_t lt = fdiv(local, m.f_whw);
  const uint32_t r = local - lt * uint32_t(m.whw);
  const uint32_t lh = fdiv(r, m.f_ww);
  const uint32_t lw = r - lh * uint32_t(m.ww);
  int32_t pt = o.t0 + int32_t(lt);
  if (pt >= m.T) pt -= m.T;
  int32_t ph = o.h0 + int32_t(lh);
  if (ph >= m.H) ph -= m.H;
  int32_t pw = o.w0 + int32_t(lw);
  if (pw >= m.W) pw -= m.W;
  return (pt * m.H + ph) * m.W + pw;
}

}  // namespace basa
