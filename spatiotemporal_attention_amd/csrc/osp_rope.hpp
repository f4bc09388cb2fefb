// osp_rope.hpp -- 3D RoPE pieces shared by the standalone rope3d kernel and
// the attention loaders, so that both produce bit-identical rotated bf16.
//
// CogVideoX section 2.2 "3D-RoPE": 1D RoPE is applied separately to the
// t, h and w coordinate of a latent token, each on its own chunk of the
// channels, and the chunks are concatenated.  RoFormer (CogVideoX ref. [14]):
// pair (x_a, x_b) at position m turns by m * omega_r into
// (x_a cos - x_b sin, x_a sin + x_b cos).  Here the chunks are ordered
// [t | h | w], pairs are adjacent channels and omega_r = theta^(-2r/d_a)
// inside a chunk of d_a channels.
//
// (cos, sin) come from an LDS table with one block per axis: entry
// off_a + x * pairs_a + r holds the angle (x + pos0_a) * omega of pair r of
// axis a at latent coordinate x.  Every field below is a scalar so that no
// kernel argument is ever indexed dynamically (which would force it into
// private memory).
#pragma once

#include "osp_common.hpp"

namespace osp {

constexpr int kMaxPairs = 64;          // head_dim <= 128
constexpr int kMaxTableBytes = 24576;  // LDS cos/sin table cap (3072 entries)
constexpr int kMaxTableEntries = kMaxTableBytes / 8;

struct RopeGeom {
  int32_t n_text;
  int32_t np0, np1, np2;        // pairs per axis (t, h, w)
  int32_t pos0_t, pos0_h, pos0_w;
  int32_t off1, off2;           // first table entry of the h and w blocks (t block at 0)
  int32_t tab_entries;          // total entries; 0 => too big, compute on the fly
  int32_t aligned8;             // every axis chunk is a multiple of 8 channels
  FastDiv div_hw, div_w;
  float omega[kMaxPairs];       // rate of head-dim pair p (host double -> float)
};

// LDS-resident pieces: per-pair rates and the cos/sin table.
struct RopeLds {
  float omega[kMaxPairs];
  float2 tab[kMaxTableEntries];
};

typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));

__device__ __forceinline__ float bf16lo(uint32_t u) { return __uint_as_float(u << 16); }
__device__ __forceinline__ float bf16hi(uint32_t u) { return __uint_as_float(u & 0xffff0000u); }

__device__ __forceinline__ uint32_t pack_bf16(float a, float b) {
  bf16x2_t v = {(__bf16)a, (__bf16)b};   // v_cvt_pk_bf16_f32: round to nearest even
  return __builtin_bit_cast(uint32_t, v);
}

template <typename T>
__device__ __forceinline__ T sel3(int a, T x0, T x1, T x2) {
  return a == 0 ? x0 : (a == 1 ? x1 : x2);
}

// (cos, sin) of the angle pos * omega, in fp32.
__device__ __forceinline__ float2 rope_cs(int32_t pos, float omega) {
  float s, c;
  sincosf(float(pos) * omega, &s, &c);
  return make_float2(c, s);
}

// Rotate one packed bf16 pair by (c, s) and repack (RNE).
__device__ __forceinline__ uint32_t rotate_pair(uint32_t xy, float2 cs) {
  float x0 = bf16lo(xy), x1 = bf16hi(xy);
  float y0 = fmaf(x0, cs.x, -(x1 * cs.y));
  float y1 = fmaf(x0, cs.y, x1 * cs.x);
  return pack_bf16(y0, y1);
}

// Rotate one packed bf16 pair, multiply by `scale` in fp32, repack (one
// rounding).
__device__ __forceinline__ uint32_t rotate_pair_scaled(uint32_t xy, float2 cs, float scale) {
  float x0 = bf16lo(xy), x1 = bf16hi(xy);
  float y0 = fmaf(x0, cs.x, -(x1 * cs.y));
  float y1 = fmaf(x0, cs.y, x1 * cs.x);
  return pack_bf16(y0 * scale, y1 * scale);
}

// Axis of head-dim pair p, its index r inside the axis chunk.
__device__ __forceinline__ int pair_axis(const RopeGeom& g, int p, int* r) {
  const int a = (p < g.np0) ? 0 : (p < g.np0 + g.np1 ? 1 : 2);
  *r = p - sel3(a, 0, g.np0, g.np0 + g.np1);
  return a;
}

// Stage the rates in LDS (all threads), then -- after the caller's barrier
// -- fill the table with fill_rope_table.
template <int NT>
__device__ __forceinline__ void stage_rope_rates(const float (&omega)[kMaxPairs], RopeLds* s,
                                                 int tid) {
#pragma unroll
  for (int p = 0; p < kMaxPairs; ++p)
    if ((p % NT) == tid) s->omega[p] = omega[p];
}

__device__ __forceinline__ void fill_rope_table(const RopeGeom& g, RopeLds* s, int tid,
                                                int nthreads) {
  for (int e = tid; e < g.tab_entries; e += nthreads) {
    const int a = (e >= g.off2) ? 2 : (e >= g.off1 ? 1 : 0);
    const int np = sel3(a, g.np0, g.np1, g.np2);
    const int local = e - sel3(a, 0, g.off1, g.off2);
    const int x = local / np;
    const int r = local - x * np;
    const int p = r + sel3(a, 0, g.np0, g.np0 + g.np1);
    s->tab[e] = rope_cs(x + sel3(a, g.pos0_t, g.pos0_h, g.pos0_w), s->omega[p]);
  }
}

// The geometry without the rates (small enough for scalar registers).
__device__ __forceinline__ RopeGeom rope_scalars(const RopeGeom& g) {
  RopeGeom r;
  r.n_text = g.n_text;
  r.np0 = g.np0; r.np1 = g.np1; r.np2 = g.np2;
  r.pos0_t = g.pos0_t; r.pos0_h = g.pos0_h; r.pos0_w = g.pos0_w;
  r.off1 = g.off1; r.off2 = g.off2;
  r.tab_entries = g.tab_entries;
  r.aligned8 = g.aligned8;
  r.div_hw = g.div_hw; r.div_w = g.div_w;
  return r;
}

// (cos, sin) of pair p for a token at coordinates c (general path).
__device__ __forceinline__ float2 pair_cs(const RopeGeom& g, const RopeLds* s, int p,
                                          const Coord3& c) {
  int r;
  const int a = pair_axis(g, p, &r);
  const int x = int(sel3(a, c.t, c.h, c.w));
  if (g.tab_entries)
    return s->tab[sel3(a, 0, g.off1, g.off2) + x * sel3(a, g.np0, g.np1, g.np2) + r];
  return rope_cs(x + sel3(a, g.pos0_t, g.pos0_h, g.pos0_w), s->omega[p]);
}

// Rotate an 8-channel chunk (4 pairs starting at pair p0) of the token with
// coordinates c; the pairs may fall in different axis chunks.
__device__ __forceinline__ uint4 rotate_chunk(const RopeGeom& g, const RopeLds* s, int p0,
                                              const Coord3& c, uint4 x) {
  x.x = rotate_pair(x.x, pair_cs(g, s, p0 + 0, c));
  x.y = rotate_pair(x.y, pair_cs(g, s, p0 + 1, c));
  x.z = rotate_pair(x.z, pair_cs(g, s, p0 + 2, c));
  x.w = rotate_pair(x.w, pair_cs(g, s, p0 + 3, c));
  return x;
}

// rotate_chunk with the result multiplied by `scale` before rounding.
__device__ __forceinline__ uint4 rotate_chunk_scaled(const RopeGeom& g, const RopeLds* s, int p0,
                                                     const Coord3& c, uint4 x, float scale) {
  x.x = rotate_pair_scaled(x.x, pair_cs(g, s, p0 + 0, c), scale);
  x.y = rotate_pair_scaled(x.y, pair_cs(g, s, p0 + 1, c), scale);
  x.z = rotate_pair_scaled(x.z, pair_cs(g, s, p0 + 2, c), scale);
  x.w = rotate_pair_scaled(x.w, pair_cs(g, s, p0 + 3, c), scale);
  return x;
}

// Same as rotate_chunk, table only (requires tab_entries != 0).
__device__ __forceinline__ uint4 rotate_chunk_tab(const RopeGeom& g, const RopeLds* s, int p0,
                                                  const Coord3& c, uint4 x) {
  uint32_t* w = reinterpret_cast<uint32_t*>(&x);
#pragma unroll
  for (int t = 0; t < 4; ++t) {
    int r;
    const int a = pair_axis(g, p0 + t, &r);
    const int pos = int(sel3(a, c.t, c.h, c.w));
    w[t] = rotate_pair(w[t], s->tab[sel3(a, 0, g.off1, g.off2) + pos * sel3(a, g.np0, g.np1, g.np2) + r]);
  }
  return x;
}

// Fast path for a chunk whose 4 pairs lie in one axis (aligned8 and a table):
// the precomputed column (axis, first entry, row stride) of the chunk.
struct ChunkCol {
  int axis;
  int base;     // off_a + r of the first pair
  int stride;   // pairs of the axis
};

__device__ __forceinline__ ChunkCol chunk_col(const RopeGeom& g, int p0) {
  int r;
  ChunkCol k;
  k.axis = pair_axis(g, p0, &r);
  k.base = sel3(k.axis, 0, g.off1, g.off2) + r;
  k.stride = sel3(k.axis, g.np0, g.np1, g.np2);
  return k;
}

__device__ __forceinline__ uint4 rotate_chunk_col(const RopeLds* s, const ChunkCol& k,
                                                  const Coord3& c, uint4 x) {
  const int pos = int(sel3(k.axis, c.t, c.h, c.w));
  const float4* t = reinterpret_cast<const float4*>(s->tab + k.base + pos * k.stride);
  const float4 a = t[0], b = t[1];
  x.x = rotate_pair(x.x, make_float2(a.x, a.y));
  x.y = rotate_pair(x.y, make_float2(a.z, a.w));
  x.z = rotate_pair(x.z, make_float2(b.x, b.y));
  x.w = rotate_pair(x.w, make_float2(b.z, b.w));
  return x;
}

// rotate_chunk_col with the result multiplied by `scale` before rounding
// (the same table entries as rotate_chunk_scaled reads, so the same bits).
__device__ __forceinline__ uint4 rotate_chunk_col_scaled(const RopeLds* s, const ChunkCol& k,
                                                         const Coord3& c, uint4 x, float scale) {
  const int pos = int(sel3(k.axis, c.t, c.h, c.w));
  const float4* t = reinterpret_cast<const float4*>(s->tab + k.base + pos * k.stride);
  const float4 a = t[0], b = t[1];
  x.x = rotate_pair_scaled(x.x, make_float2(a.x, a.y), scale);
  x.y = rotate_pair_scaled(x.y, make_float2(a.z, a.w), scale);
  x.z = rotate_pair_scaled(x.z, make_float2(b.x, b.y), scale);
  x.w = rotate_pair_scaled(x.w, make_float2(b.z, b.w), scale);
  return x;
}

// Is token i a video token (text tokens come first and are not rotated).
__device__ __forceinline__ bool is_video(const RopeGeom& g, uint32_t i) {
  return int32_t(i) >= g.n_text;
}

// Latent coordinates of video token i.
__device__ __forceinline__ Coord3 video_coords(const RopeGeom& g, uint32_t i) {
  return decode_video(i - uint32_t(g.n_text), g.div_hw, g.div_w);
}

}  // namespace osp
