// osp_mfma.hpp -- vector types, LDS tile layout and lane helpers shared by
// the attention kernels (forward and backward) on gfx950.
//
// MFMA 32x32x16 bf16 operand layout used throughout: lane l of the A
// operand holds row l%32 and k = 8*(l/32) .. +7; lane l of the B operand
// holds column l%32 and the same k; the fp32 C block gives lane l column
// l%32 and rows 8*(e/4) + 4*(l/32) + (e%4), e = 0..15.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include <type_traits>

namespace osp {

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x2v_t __attribute__((ext_vector_type(2)));
typedef float f32x16_t __attribute__((ext_vector_type(16)));
typedef short i16x4_t __attribute__((ext_vector_type(4)));
typedef i16x4_t __attribute__((address_space(3))) * lds_i16x4_ptr;
typedef __attribute__((address_space(3))) void* lds_void_ptr;

constexpr int32_t kRecords = 0x40000000;   // buffer range of one LDS DMA tile (bytes)

// XOR swizzle of the 16-byte chunks of LDS row r: a permutation of the
// row's chunks.  It has period 16 in r, which keeps the operand addresses
// of different 16/32-row blocks a constant apart.
template <int D> __device__ __forceinline__ int chunk_swz(int r);
template <> __device__ __forceinline__ int chunk_swz<64>(int r) { return (5 * (r >> 1)) & 7; }
template <> __device__ __forceinline__ int chunk_swz<96>(int r) { return (r >> 2) & 3; }
template <> __device__ __forceinline__ int chunk_swz<128>(int r) { return (5 * r) & 15; }

template <bool B> using bool_c = std::integral_constant<bool, B>;
template <int I> using int_c = std::integral_constant<int, I>;

__device__ __forceinline__ uint4 ld16(const uint16_t* p) {
  return *reinterpret_cast<const uint4*>(p);
}

// max / sum over lanes l and l^32
__device__ __forceinline__ float max_pair32(float x) {
  auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
__device__ __forceinline__ float sum_pair32(float x) {
  auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}

// Per-lane byte offsets, inside an LDS tile of rows of D bf16 (chunks
// swizzled), of the two operand reads used on it.
//
// row_off[c]: the A (or B) operand of the 16-channel block c for row l%32
// of a 32-row block: one 16-byte chunk, 2c + l/32.
template <int D>
__device__ __forceinline__ void row_read_offsets(int lane, int (&off)[D / 16]) {
  constexpr int KCH = D / 8;
  const int l32 = lane & 31, g = lane >> 5;
  const int hsw = g ^ chunk_swz<D>(l32);
#pragma unroll
  for (int c = 0; c < D / 16; ++c) off[c] = (l32 * KCH + ((2 * c) ^ hsw)) * 16;
}

// tr_off[s][db]: the transposed A operand (rows = channels 32db .. +31,
// k = 16 rows of the tile) of a 16-row block, in the k order of a C block's
// rows: lane l gets rows 4*(l/32) + 0..3 (s = 0) and 8 + 4*(l/32) + 0..3
// (s = 1) of channel 32db + l%32.  Source lane (ta, te) of 16-lane group G
// points at row 4(G/2) + te + 8s, channels 32db + 16(G%2) + 4ta .. +3; the
// transposing read (ds_read_b64_tr_b16) hands each lane 4 rows of one
// channel.
template <int D>
__device__ __forceinline__ void tr_read_offsets(int lane, int (&off)[2][D / 32]) {
  constexpr int KCH = D / 8;
  const int G = lane >> 4, s16 = lane & 15;
  const int ta = s16 & 3, te = s16 >> 2;
#pragma unroll
  for (int s = 0; s < 2; ++s)
#pragma unroll
    for (int db = 0; db < D / 32; ++db) {
      const int row = 4 * (G >> 1) + te + 8 * s;
      const int chunk = 4 * db + 2 * (G & 1) + (ta >> 1);
      off[s][db] = (row * KCH + (chunk ^ chunk_swz<D>(row))) * 16 + 8 * (ta & 1);
    }
}

// The offsets above, held per lane.  At head_dim 96 the swizzle flips only
// the two low bits of a chunk index ((r >> 2) & 3), so the offsets of the
// 16-channel blocks c (rows) or 32-channel blocks db (transposed) differ by
// constants: row block c sits at one of two bases (c even or odd) plus
// 64 (c / 2) bytes, transposed block db at its base for s plus 64 db bytes.
// Two registers then hold what takes six, and the constants become the LDS
// reads' immediate offsets.
template <int D> struct RowOff {
  int v[D / 16];
  __device__ __forceinline__ explicit RowOff(int lane) { row_read_offsets<D>(lane, v); }
  __device__ __forceinline__ int operator()(int c) const { return v[c]; }
};
template <> struct RowOff<96> {
  int e[2];
  __device__ __forceinline__ explicit RowOff(int lane) {
    int v[6];
    row_read_offsets<96>(lane, v);
    e[0] = v[0];
    e[1] = v[1];
  }
  __device__ __forceinline__ int operator()(int c) const { return e[c & 1] + 64 * (c >> 1); }
};
template <int D> struct TrOff {
  int v[2][D / 32];
  __device__ __forceinline__ explicit TrOff(int lane) { tr_read_offsets<D>(lane, v); }
  __device__ __forceinline__ int operator()(int s, int db) const { return v[s][db]; }
};
template <> struct TrOff<96> {
  int e[2];
  __device__ __forceinline__ explicit TrOff(int lane) {
    int v[2][3];
    tr_read_offsets<96>(lane, v);
    e[0] = v[0][0];
    e[1] = v[1][0];
  }
  __device__ __forceinline__ int operator()(int s, int db) const { return e[s] + 64 * db; }
};

// The transposed A operand of block db, at offsets off(., db) from blk.
template <int D>
__device__ __forceinline__ bf16x8_t tr_read(const char* blk, const TrOff<D>& off, int db) {
  const i16x4_t lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4_ptr)(blk + off(0, db)));
  const i16x4_t hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4_ptr)(blk + off(1, db)));
  const uint2 l2 = __builtin_bit_cast(uint2, lo), h2 = __builtin_bit_cast(uint2, hi);
  return __builtin_bit_cast(bf16x8_t, make_uint4(l2.x, l2.y, h2.x, h2.y));
}

}  // namespace osp
