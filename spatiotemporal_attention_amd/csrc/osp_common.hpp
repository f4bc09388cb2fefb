// osp_common.hpp -- index arithmetic shared by the host library and the
// gfx950 kernels: division by run-time constants, token -> (t, h, w)
// decode, Skiparse row -> token remap, RoPE angle.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#define OSP_HD __host__ __device__ __forceinline__

namespace osp {

// Division of unsigned 32-bit numerators by a run-time constant d >= 1,
// by multiply-high and shifts (Granlund & Montgomery, "Division by
// invariant integers using multiplication", PLDI 1994, section 4): with
// l = ceil(log2 d) and m = floor(2^32 (2^l - d) / d) + 1,
// n / d = (t + ((n - t) >> min(l,1))) >> max(l-1,0), t = mulhi(m, n).
struct FastDiv {
  uint32_t d, m, s1, s2;
};

inline FastDiv make_fastdiv(uint32_t d) {
  FastDiv f;
  f.d = d;
  uint32_t l = 0;
  while ((uint64_t(1) << l) < d) ++l;
  f.m = uint32_t(((uint64_t(1) << 32) * ((uint64_t(1) << l) - d)) / d + 1);
  f.s1 = l < 1 ? l : 1;
  f.s2 = l > 1 ? l - 1 : 0;
  return f;
}

OSP_HD uint32_t mulhi32(uint32_t a, uint32_t b) {
#if defined(__HIP_DEVICE_COMPILE__)
  return __umulhi(a, b);
#else
  return uint32_t((uint64_t(a) * uint64_t(b)) >> 32);
#endif
}

OSP_HD uint32_t fdiv(uint32_t n, const FastDiv& f) {
  uint32_t t = mulhi32(f.m, n);
  return (t + ((n - t) >> f.s1)) >> f.s2;
}

// Division by the subsequence count k, plus what the 2D modes need: the
// per-axis factor s (k = s*s), the rows of one subsequence per frame
// (H/s)*(W/s) and per lattice row W/s, and the grid's H and W.
struct SkipDiv : FastDiv {
  FastDiv axis, plane, row;
  uint32_t gh, gw;
};

inline SkipDiv make_skipdiv(uint32_t k, uint32_t s, uint32_t gh, uint32_t gw) {
  SkipDiv v;
  static_cast<FastDiv&>(v) = make_fastdiv(k);
  s = s ? s : 1;
  v.axis = make_fastdiv(s);
  v.plane = make_fastdiv((gh / s) * (gw / s) ? (gh / s) * (gw / s) : 1);
  v.row = make_fastdiv(gw / s ? gw / s : 1);
  v.gh = gh;
  v.gw = gw;
  return v;
}

// Token i of a subsequence-row r.  Skiparse regroups an N-token sequence
// into k subsequences of L = N/k rows (Open-Sora Plan section 2.2.2):
//   full:   i = r
//   single: row r of subsequence j holds token r*k + j        (i mod k = j)
//   group:  row r of subsequence j holds token
//           floor(r/k)*k*k + j*k + (r mod k)        (floor(i/k) mod k = j)
//   block:  row r of subsequence j holds token j*L + r   (floor(i/L) = j):
//           the spatial half of separated spatial / temporal attention
//           (CogVideoX section 2.2, Table 8) with k = frames, or window
//           attention with k = N / window
//   single2d, group2d: Skiparse-2D (named for OSP-Next on the Open-Sora Plan
//           blog page: a fixed rule along H and W).  Read as the single and
//           group rules applied to the h and w axes with s = sqrt(k), in
//           every frame: j = jh*s + jw, row r = (t*(H/s) + h')*(W/s) + w',
//           and h = skip(h', jh), w = skip(w', jw) with skip(x, c) = x*s + c
//           (single) or floor(x/s)*s*s + c*s + (x mod s) (group)
enum : int32_t { MODE_FULL = 0, MODE_SINGLE = 1, MODE_GROUP = 2, MODE_BLOCK = 3,
                 MODE_SINGLE2D = 4, MODE_GROUP2D = 5 };

OSP_HD uint32_t skip_axis(bool group, uint32_t x, uint32_t c, const FastDiv& s) {
  if (!group) return x * s.d + c;
  const uint32_t a = fdiv(x, s);
  return (a * s.d + c) * s.d + (x - a * s.d);
}

OSP_HD uint32_t skiparse_token(int32_t mode, uint32_t r, uint32_t j,
                               const SkipDiv& divk, uint32_t len) {
  if (mode == MODE_SINGLE) return r * divk.d + j;
  if (mode == MODE_GROUP) {
    uint32_t a = fdiv(r, divk);
    uint32_t c = r - a * divk.d;
    return (a * divk.d + j) * divk.d + c;
  }
  if (mode == MODE_BLOCK) return j * len + r;
  if (mode >= MODE_SINGLE2D) {
    const bool group = mode == MODE_GROUP2D;
    const uint32_t t = fdiv(r, divk.plane);
    const uint32_t rem = r - t * divk.plane.d;
    const uint32_t hh = fdiv(rem, divk.row);
    const uint32_t ww = rem - hh * divk.row.d;
    const uint32_t jh = fdiv(j, divk.axis);
    const uint32_t jw = j - jh * divk.axis.d;
    return (t * divk.gh + skip_axis(group, hh, jh, divk.axis)) * divk.gw +
           skip_axis(group, ww, jw, divk.axis);
  }
  return r;
}

// Latent coordinates of video token p (0-based after the text tokens),
// row-major over (t, h, w) with w fastest.
struct Coord3 {
  uint32_t t, h, w;
};

OSP_HD Coord3 decode_video(uint32_t p, const FastDiv& div_hw, const FastDiv& div_w) {
  Coord3 c;
  c.t = fdiv(p, div_hw);
  uint32_t rem = p - c.t * div_hw.d;
  c.h = fdiv(rem, div_w);
  c.w = rem - c.h * div_w.d;
  return c;
}

}  // namespace osp
