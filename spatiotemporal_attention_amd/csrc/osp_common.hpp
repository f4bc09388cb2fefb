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
enum : int32_t { MODE_FULL = 0, MODE_SINGLE = 1, MODE_GROUP = 2, MODE_BLOCK = 3 };

OSP_HD uint32_t skiparse_token(int32_t mode, uint32_t r, uint32_t j,
                               const FastDiv& divk, uint32_t len) {
  if (mode == MODE_SINGLE) return r * divk.d + j;
  if (mode == MODE_GROUP) {
    uint32_t a = fdiv(r, divk);
    uint32_t c = r - a * divk.d;
    return (a * divk.d + j) * divk.d + c;
  }
  if (mode == MODE_BLOCK) return j * len + r;
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
