// attn3d_bwd.hip -- attention backward for gfx950 (MI355X): the gradients
// dQ, dK, dV of softmax(scale * q k^T) v over every token of a subsequence
// (full attention of CogVideoX section 2.2 "3D Full Attention"; Skiparse
// subsequences of Open-Sora Plan section 2.2.2; block attention), given the
// forward's output O and row log-sum-exp lse.  q and k are the rotated ones
// (the RoPE transpose is a separate pass, rope3d with the inverse flag).
//
// The derivative written out: with S = q k^T and P = exp(scale S - lse),
//   dV = P^T dO,   dP = dO V^T,   delta_i = sum_j P_ij dP_ij,
//   dS = P o (dP - delta),   dQ = scale dS K,   dK = scale dS^T Q.
// delta_i also equals sum_d O_id dO_id (O = P V), which is how it is formed:
// from O and dO, before the blocked passes (the FlashAttention-2 backward).
//
// Three kernels:
//  1. bwd_prep: per row, -delta and -lse / scale into the workspace.
//  2. bwd_dkdv: a workgroup of 8 waves owns 4*KB*32 keys of one (batch,
//     head, subsequence) and streams the subsequence's queries through LDS
//     in tiles of 64 rows (Q, dO and the two workspace rows).  The waves
//     work in pairs on the same keys: the P wave (K rows in registers)
//     forms S - lse/scale = Q K^T - lse/scale, the dS wave (V rows) forms
//     dP - delta = dO V^T - delta, with the rows of the Q / dO tile as A
//     operand and K / V as B and the row terms as the C init, so a lane
//     holds ONE key (column l%32) and 16 queries; P = exp2(scale log2(e)
//     (S - lse/scale)) goes from the P wave to the dS wave through LDS,
//     dS = P o (dP - delta); both are packed to bf16 as B operands in the C
//     row order, and dV^T += dO^T P (P wave), dK^T += Q^T dS (dS wave)
//     take their A operands transposed from the same LDS tiles
//     (ds_read_b64_tr_b16) in that row order.
//  3. bwd_dq: a workgroup owns NW*32 queries, 32 per wave, Q (times scale
//     log2(e), rounded to bf16 once, as the forward rounds its scaled Q)
//     and dO in registers, and streams the keys (K and V tiles): X^T =
//     K Q'^T - lse log2(e), dP^T - delta = V dO^T - delta (a lane holds ONE
//     query, so both row terms are one value per lane), P^T = exp2(X^T),
//     dS^T as above, dQ^T += K^T dS^T with K^T read transposed.
// dQ gets a pass of its own instead of atomic fp32 adds from the dK/dV
// pass: the score products are formed twice (7 MFMA products per 32x32
// block instead of 5), but no workspace for dQ and no atomics are needed.
//
// Tiles arrive by LDS DMA (buffer_load ... lds) into two slots per tensor,
// the next tile loading while the current one is used; rows past the end of
// the subsequence read as zeros (out of the buffer range), which makes
// their contributions exactly zero.
#include <atomic>

#include "osp_internal.hpp"
#include "osp_mfma.hpp"

namespace osp {

constexpr int kBwdRows = 64;         // rows of one streamed LDS tile
constexpr int kPrepThreads = 256;

// Geometry of the blocked kernels.  Both stream 64-row tiles through LDS,
// each loaded by 4 waves (in the dQ kernel waves 0-3 load K and 4-7 load V,
// or with 4 waves each loads both; in the dK/dV kernel the 4 waves of each
// role load their tensor).
template <int D> struct BwdCfg {
  static constexpr int KCH = D / 8;                       // 16-byte chunks per row
  static constexpr int TILE = kBwdRows * D;               // bf16 elements of a tile
  static constexpr int LW = 4;                            // waves loading one tensor
  static constexpr int DPW = kBwdRows * KCH / 64 / LW;    // DMA loads per wave and tensor
  static_assert((kBwdRows * KCH / 64) % LW == 0, "every loading wave has the same share");
  // dK/dV: 4 pairs of waves, each pair owning KB blocks of 32 keys
  static constexpr int KB = (D == 128) ? 1 : 2;
  static constexpr int KV_ROWS = 4 * KB * 32;
  // dQ: waves of 32 queries each; with 8, waves 0-3 load K and 4-7 load V,
  // with 4 every wave loads both
  static constexpr int NW_Q = (D == 128) ? 4 : 8;
  static constexpr int OCC_Q = (D == 128) ? 1 : 2;
  static constexpr int Q_ROWS = NW_Q * 32;
};

int bwd_kv_rows_per_block(int head_dim) {
  switch (head_dim) {
    case 64: return BwdCfg<64>::KV_ROWS;
    case 96: return BwdCfg<96>::KV_ROWS;
    default: return BwdCfg<128>::KV_ROWS;
  }
}
int bwd_q_rows_per_block(int head_dim) {
  switch (head_dim) {
    case 64: return BwdCfg<64>::Q_ROWS;
    case 96: return BwdCfg<96>::Q_ROWS;
    default: return BwdCfg<128>::Q_ROWS;
  }
}
int bwd_tile_rows(int) { return kBwdRows; }

// ---------------------------------------------------------------------------
// 1. -delta_i = -sum_d O_id dO_id and -lse_i / scale, per (b, h, token);
//    thread idx = (b*H + h)*N + n, the workspace layout.
template <int D>
__global__ __launch_bounds__(kPrepThreads) void bwd_prep_kernel(const BwdArgs a, uint32_t total,
                                                                 FastDiv div_n, FastDiv div_h) {
  const uint32_t idx = blockIdx.x * kPrepThreads + threadIdx.x;
  if (idx >= total) return;
  const uint32_t bh = fdiv(idx, div_n);
  const uint32_t n = idx - bh * div_n.d;
  const uint32_t b = fdiv(bh, div_h);
  const uint32_t h = bh - b * div_h.d;
  const int64_t off = int64_t(b) * a.sb + int64_t(n) * a.sn + int64_t(h) * a.sh;
  const uint16_t* po = a.o + off;
  const uint16_t* pd = a.dout + off;
  float acc[4] = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
  for (int c = 0; c < D / 8; ++c) {
    const uint4 x = ld16(po + 8 * c), y = ld16(pd + 8 * c);
    const uint32_t xs[4] = {x.x, x.y, x.z, x.w}, ys[4] = {y.x, y.y, y.z, y.w};
#pragma unroll
    for (int t = 0; t < 4; ++t) {
      acc[t] = fmaf(bf16lo(xs[t]), bf16lo(ys[t]), acc[t]);
      acc[t] = fmaf(bf16hi(xs[t]), bf16hi(ys[t]), acc[t]);
    }
  }
  const int64_t w = int64_t(bh) * a.ws_ld + n;
  a.neg_delta[w] = -((acc[0] + acc[1]) + (acc[2] + acc[3]));
  a.neg_lse_s[w] = -a.lse[int64_t(bh) * a.lse_ld + n] / a.scale;
}

// ---------------------------------------------------------------------------
// Shared pieces of the two blocked kernels.

// Which (b, h, subsequence j, row block) a workgroup takes: consecutive
// row blocks of one (b, h, j) share their streamed tiles and stay on one
// XCD (workgroups are dealt to the 8 XCDs round robin).  In a packed
// launch the workgroup first finds its segment (every index a constant, no
// dynamic indexing into the argument block); each segment starts at a
// multiple of 8 workgroups and is spread over the 8 XCDs on its own, and
// its padding workgroups are not live.
struct BwdBlock {
  uint32_t b, h, j, blk;
  int L;                        // rows of a subsequence
  int64_t tok0;                 // first token of the sequence
  bool live;
};
template <bool PACKED, bool KV>
__device__ __forceinline__ BwdBlock bwd_block(const BwdArgs& a) {
  const uint32_t x = blockIdx.x;
  BwdBlock r;
  uint32_t u, blocks;
  r.live = true;
  if constexpr (PACKED) {
    BwdPackSeg ps = a.pack[0];
#pragma unroll
    for (int sg = 1; sg < kMaxPackSegs; ++sg)
      if (sg < a.n_pack && x >= uint32_t(KV ? a.pack[sg].kv_tile0 : a.pack[sg].q_tile0))
        ps = a.pack[sg];
    const uint32_t tiles = uint32_t(KV ? ps.kv_tiles : ps.q_tiles);
    const uint32_t xs = x - uint32_t(KV ? ps.kv_tile0 : ps.q_tile0);
    u = (xs & 7u) * ((tiles + 7u) >> 3) + (xs >> 3);
    r.live = u < tiles;
    if (!r.live) u = 0;
    blocks = uint32_t(KV ? ps.kv_blocks : ps.q_blocks);
    r.L = ps.seq_len;
    r.tok0 = ps.start;
  } else {
    const uint32_t total = gridDim.x;
    const uint32_t t8 = total & ~7u;
    u = (x < t8) ? (x & 7u) * (t8 >> 3) + (x >> 3) : x;
    blocks = uint32_t(KV ? a.kv_blocks : a.q_blocks);
    r.L = a.seq_len;
    r.tok0 = 0;
  }
  r.blk = u % blocks;
  u /= blocks;
  r.j = u % uint32_t(a.groups);
  u /= uint32_t(a.groups);
  r.h = u % uint32_t(a.heads);
  r.b = u / uint32_t(a.heads);
  return r;
}

// LDS DMA of row tiles: loading wave w (of LW) issues the 64-lane loads
// w + LW*u, u < DPW, of each tile; position p = 64*(w + LW*u) + lane of the
// tile is row p / KCH, stored chunk p % KCH, which holds logical chunk
// (p % KCH) ^ chunk_swz(row).
template <int D>
struct TileDma {
  using C = BwdCfg<D>;
  int w, lane;
  int32_t off[C::DPW];   // byte offsets of the current tile, relative to its first token

  __device__ __forceinline__ void init(int w_, int lane_) {
    w = w_;
    lane = lane_;
  }
  // row and stored chunk of load u (formed again for each tile rather than
  // held: the dK/dV kernel is short of registers)
  __device__ __forceinline__ int row(int u) const { return (64 * (w + C::LW * u) + lane) / C::KCH; }
  __device__ __forceinline__ int col(int u) const {
    const int p = 64 * (w + C::LW * u) + lane;
    return (p % C::KCH) ^ chunk_swz<D>(p / C::KCH);
  }
  // offsets of tile t (rows 64t ..) of subsequence j; returns its first token
  __device__ __forceinline__ uint32_t at(int t, int mode, uint32_t j, const SkipDiv& divk, int L,
                                         int64_t sn) {
    const int r0 = t * kBwdRows;
    const uint32_t i0 = skiparse_token(mode, uint32_t(r0), j, divk, uint32_t(L));
#pragma unroll
    for (int u = 0; u < C::DPW; ++u) {
      const int r = r0 + row(u);
      const uint32_t i = skiparse_token(mode, uint32_t(min(r, L - 1)), j, divk, uint32_t(L));
      off[u] = (r < L) ? int32_t((int64_t(i - i0) * sn + 8 * col(u)) * 2) : kRecords;
    }
    return i0;
  }
  // the same from a row table: tab[r] = token of row r of subsequence 0,
  // cj = token(0, j) (the per-row remaps differ between subsequences by a
  // constant)
  __device__ __forceinline__ uint32_t at_tab(int t, const uint32_t* tab, uint32_t cj, int L,
                                             int64_t sn) {
    const int r0 = t * kBwdRows;
    const uint32_t base = tab[min(r0, L - 1)];
#pragma unroll
    for (int u = 0; u < C::DPW; ++u) {
      const int r = r0 + row(u);
      const uint32_t tok = tab[min(r, L - 1)];
      off[u] = (r < L) ? int32_t((int64_t(tok - base) * sn + 8 * col(u)) * 2) : kRecords;
    }
    return base + cj;
  }
};

// TAB instances (per-row remaps): the workgroup tabulates token(r, 0) for
// the L rows of a subsequence in dynamic LDS before its first load.
extern __shared__ __attribute__((aligned(16))) uint32_t bwd_row_tab[];
template <bool TAB>
__device__ __forceinline__ uint32_t build_row_tab(int mode, uint32_t j, const SkipDiv& divk, int L) {
  if constexpr (!TAB) return 0u;
  for (int r = threadIdx.x; r < L; r += blockDim.x)
    bwd_row_tab[r] = skiparse_token(mode, uint32_t(r), 0u, divk, uint32_t(L));
  __syncthreads();
  return skiparse_token(mode, 0u, j, divk, uint32_t(L));
}
// (The DMA instructions are issued from lambdas inside each kernel, with
// the offset copied to a local first: this compiler's host pass drops a
// kernel, without a diagnostic, whose buffer_load_lds builtin takes a
// struct member or sits in a shared function template.)

// Store a transposed fp32 accumulator (rows = channels 32db + 8*r4 + 4g
// + 0..3, column = this lane's token row) times `mul` as bf16 at p.
template <int D>
__device__ __forceinline__ void store_rows_t(uint16_t* p, const f32x16_t (&acc)[D / 32], float mul,
                                             int g) {
#pragma unroll
  for (int db = 0; db < D / 32; ++db)
#pragma unroll
    for (int r4 = 0; r4 < 4; ++r4) {
      const uint32_t w0 = pack_bf16(acc[db][4 * r4 + 0] * mul, acc[db][4 * r4 + 1] * mul);
      const uint32_t w1 = pack_bf16(acc[db][4 * r4 + 2] * mul, acc[db][4 * r4 + 3] * mul);
      *reinterpret_cast<uint2*>(p + 32 * db + 8 * r4 + 4 * g) = make_uint2(w0, w1);
    }
}

// Multiply an operand row by m in fp32 and round it to bf16 again (RNE).
template <int D>
__device__ __forceinline__ void scale_operand(bf16x8_t (&x)[D / 16], float m) {
#pragma unroll
  for (int c = 0; c < D / 16; ++c) {
    uint4 u = __builtin_bit_cast(uint4, x[c]);
    u.x = pack_bf16(bf16lo(u.x) * m, bf16hi(u.x) * m);
    u.y = pack_bf16(bf16lo(u.y) * m, bf16hi(u.y) * m);
    u.z = pack_bf16(bf16lo(u.z) * m, bf16hi(u.z) * m);
    u.w = pack_bf16(bf16lo(u.w) * m, bf16hi(u.w) * m);
    x[c] = __builtin_bit_cast(bf16x8_t, u);
  }
}

// Rows 16c + 8g .. +7 (channels) of this lane's token row, as B operands.
template <int D>
__device__ __forceinline__ void load_row_operand(const uint16_t* row, bool valid, int g,
                                                 bf16x8_t (&x)[D / 16]) {
#pragma unroll
  for (int c = 0; c < D / 16; ++c)
    x[c] = __builtin_bit_cast(bf16x8_t, valid ? ld16(row + 16 * c + 8 * g) : make_uint4(0, 0, 0, 0));
}

// ---------------------------------------------------------------------------
// 2. dK, dV.  8 waves in 4 pairs; pair p owns KB blocks of 32 keys.  In a
// pair, wave p (the P wave, K rows in registers) forms S - lse/scale and
// P, and accumulates dV^T; wave p + 4 (the dS wave, V rows in registers)
// forms dP - delta, takes P from the P wave through LDS, and accumulates
// dK^T.  Both waves of a pair sit on one SIMD, so each one's exp or
// multiply work overlaps the other's MFMAs, and each wave holds one K-or-V
// operand and one accumulator set instead of two.
//
// Per 32-query block qb of a tile, two phases split by a workgroup barrier:
//   1. both: X = A_rows . R + C0 (MFMA; A_rows = Q rows, R = K, C0 =
//      -lse/scale for the P wave; dO rows, V, -delta for the dS wave);
//      P wave: P = exp2(scale log2(e) X), written to the exchange buffer
//      (fp32) and packed to bf16;
//   2. P wave: dV^T += dO^T P; dS wave: dS = P o X, packed, and its
//      dK^T += Q^T dS in the next block's phase 1 (T^T read transposed).
// The exchange buffer alternates between two halves from block to block:
// a half is rewritten two blocks later, after the barrier that the reading
// wave reaches only once it has used it.  KB = 2 (64 keys per pair) halves
// the LDS reads and the barriers per product; at head_dim 96 it needs a
// few more than the 256 registers a wave gets at two waves per SIMD and
// spills some loop-invariant values, which still runs 10% faster than
// KB = 1 (forming them again in every phase instead costs more); head_dim
// 128 takes KB = 1.
// S2D: the Skiparse-2D remap is compiled in; without it the mode is known
// to be one of the four 1D ones, so their kernels carry none of its code.
// TAB: tile rows from the LDS row table (build_row_tab).
template <int D, bool PACKED, bool S2D, bool TAB>
__global__ __launch_bounds__(512, 2) void bwd_dkdv_kernel(const BwdArgs a) {
  using C = BwdCfg<D>;
  constexpr int KCH = C::KCH, KB = C::KB;
  constexpr int XB = 4 * KB * 4 * 64;          // float4 per exchange half
  // two slots per streamed tensor, separate arrays so that the compiler
  // sees that a DMA into one slot does not touch the other
  __shared__ __attribute__((aligned(1024))) uint16_t q_s0[C::TILE];
  __shared__ __attribute__((aligned(1024))) uint16_t q_s1[C::TILE];
  __shared__ __attribute__((aligned(1024))) uint16_t d_s0[C::TILE];
  __shared__ __attribute__((aligned(1024))) uint16_t d_s1[C::TILE];
  __shared__ __attribute__((aligned(256))) float l_s0[kBwdRows];
  __shared__ __attribute__((aligned(256))) float l_s1[kBwdRows];
  __shared__ __attribute__((aligned(256))) float e_s0[kBwdRows];
  __shared__ __attribute__((aligned(256))) float e_s1[kBwdRows];
  __shared__ __attribute__((aligned(1024))) float4 x_s0[XB];
  __shared__ __attribute__((aligned(1024))) float4 x_s1[XB];
  auto qslot = [&](auto sl) __attribute__((always_inline)) -> uint16_t* {
    if constexpr (decltype(sl)::value == 0) return q_s0; else return q_s1;
  };
  auto dslot = [&](auto sl) __attribute__((always_inline)) -> uint16_t* {
    if constexpr (decltype(sl)::value == 0) return d_s0; else return d_s1;
  };
  auto lslot = [&](auto sl) __attribute__((always_inline)) -> float* {
    if constexpr (decltype(sl)::value == 0) return l_s0; else return l_s1;
  };
  auto eslot = [&](auto sl) __attribute__((always_inline)) -> float* {
    if constexpr (decltype(sl)::value == 0) return e_s0; else return e_s1;
  };
  auto xslot = [&](auto h) __attribute__((always_inline)) -> float4* {
    if constexpr (decltype(h)::value == 0) return x_s0; else return x_s1;
  };

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const bool pw = wave < 4;          // P wave (else dS wave)
  const int pr = wave & 3;           // pair, and rank among the loading waves of a role
  const int g = lane >> 5;
  const int l32 = lane & 31;

  const BwdBlock wb = bwd_block<PACKED, true>(a);
  if (!wb.live) return;              // padding of a packed launch, before any barrier
  const int mode = S2D ? a.mode : (a.mode & 3);
  const SkipDiv divk = a.divk;
  const int L = wb.L;
  const int64_t sn = a.sn;
  const int64_t in_off = int64_t(wb.b) * a.sb + int64_t(wb.h) * a.sh + wb.tok0 * sn;
  const int64_t bhn = (int64_t(wb.b) * a.heads + wb.h) * a.ws_ld + wb.tok0;
  const float c2 = a.scale_log2;

  // ---- this lane's keys (one per key block): K rows (P wave) or V rows
  // (dS wave) as B operands
  // (the key rows and tokens are formed again for the store at the end
  // rather than held through the query loop)
  auto key_row = [&](int kb) __attribute__((always_inline)) {
    return int(wb.blk) * C::KV_ROWS + (pr * KB + kb) * 32 + l32;
  };
  bf16x8_t xreg[KB][D / 16];
  {
    const uint16_t* src = (pw ? a.k : a.v) + in_off;
#pragma unroll
    for (int kb = 0; kb < KB; ++kb) {
      const int r = key_row(kb);
      const uint32_t tok = skiparse_token(mode, uint32_t(r < L ? r : 0), wb.j, divk, uint32_t(L));
      load_row_operand<D>(src + int64_t(tok) * sn, r < L, g, xreg[kb]);
    }
  }

  f32x16_t acc[KB][D / 32];          // dV^T (P wave) or dK^T (dS wave)
#pragma unroll
  for (int kb = 0; kb < KB; ++kb)
#pragma unroll
    for (int db = 0; db < D / 32; ++db)
#pragma unroll
      for (int e = 0; e < 16; ++e) acc[kb][db][e] = 0.f;
  const RowOff<D> r_off(lane);
  const TrOff<D> t_off(lane);

  // ---- loads: the P waves load the Q tile and the -lse/scale row, the dS
  // waves the dO tile and the -delta row
  const uint32_t tab_cj = build_row_tab<TAB>(mode, wb.j, divk, L);
  TileDma<D> dma;
  dma.init(pr, lane);
  const uint16_t* tsrc = (pw ? a.q : a.dout) + in_off;
  const float* fsrc = (pw ? a.neg_lse_s : a.neg_delta) + bhn;
  auto load = [&](uint32_t i0, uint16_t* dst) __attribute__((always_inline)) {
    const __amdgpu_buffer_rsrc_t rs = __builtin_amdgcn_make_buffer_rsrc(
        const_cast<uint16_t*>(tsrc + int64_t(i0) * sn), (short)0, kRecords, 0x00020000);
#pragma unroll
    for (int u = 0; u < C::DPW; ++u) {
      const int32_t off = dma.off[u];
      __builtin_amdgcn_raw_ptr_buffer_load_lds(rs, (lds_void_ptr)(dst + 512 * (pr + C::LW * u)),
                                               16, off, 0, 0, 0);
    }
  };
  auto load_floats = [&](uint32_t i0, int t, float* dst) __attribute__((always_inline)) {
    const int r = t * kBwdRows + lane;
    const uint32_t i = TAB ? bwd_row_tab[min(r, L - 1)] + tab_cj
                           : skiparse_token(mode, uint32_t(min(r, L - 1)), wb.j, divk, uint32_t(L));
    const int32_t off = (r < L) ? int32_t((i - i0) * 4) : kRecords;
    const __amdgpu_buffer_rsrc_t rs = __builtin_amdgcn_make_buffer_rsrc(
        const_cast<float*>(fsrc + i0), (short)0, kRecords, 0x00020000);
    __builtin_amdgcn_raw_ptr_buffer_load_lds(rs, (lds_void_ptr)dst, 4, off, 0, 0, 0);
  };
  auto issue = [&](int t, auto sl) __attribute__((always_inline)) {
    const uint32_t i0 = TAB ? dma.at_tab(t, bwd_row_tab, tab_cj, L, sn)
                            : dma.at(t, mode, wb.j, divk, L, sn);
    if (pw) {
      load(i0, qslot(sl));
      if (pr == 0) load_floats(i0, t, lslot(sl));
    } else {
      load(i0, dslot(sl));
      if (pr == 0) load_floats(i0, t, eslot(sl));
    }
  };

  auto barrier = [&]() __attribute__((always_inline)) {
    __builtin_amdgcn_sched_barrier(0);
    asm volatile("s_barrier" ::: "memory");
    __builtin_amdgcn_sched_barrier(0);
  };

  // phase 1 of block qb for role R (true: P wave) from tile slot SL into
  // exchange half XH; x: the phase-1 products, bop: the phase-2 B operands
  // (P or dS)
  auto phase1 = [&](auto role, auto sl, auto xh, int qb, f32x16_t (&x)[KB], bf16x8_t (&bop)[KB][2])
      __attribute__((always_inline)) {
    constexpr bool R = decltype(role)::value;
    const char* rows = reinterpret_cast<const char*>(R ? qslot(sl) : dslot(sl)) + 32 * qb * KCH * 16;
    const float* c0 = (R ? lslot(sl) : eslot(sl)) + 32 * qb;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const float4 v = *reinterpret_cast<const float4*>(c0 + 8 * i + 4 * g);
#pragma unroll
      for (int kb = 0; kb < KB; ++kb) {
        x[kb][4 * i + 0] = v.x; x[kb][4 * i + 1] = v.y; x[kb][4 * i + 2] = v.z; x[kb][4 * i + 3] = v.w;
      }
    }
    __builtin_amdgcn_s_setprio(1);
#pragma unroll
    for (int c = 0; c < D / 16; ++c) {
      const bf16x8_t ra = *reinterpret_cast<const bf16x8_t*>(rows + r_off(c));
#pragma unroll
      for (int kb = 0; kb < KB; ++kb)
        x[kb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(ra, xreg[kb][c], x[kb], 0, 0, 0);
    }
    __builtin_amdgcn_s_setprio(0);
    if constexpr (R) {
      float4* xo = xslot(xh) + pr * KB * 4 * 64 + lane;
#pragma unroll
      for (int kb = 0; kb < KB; ++kb) {
#pragma unroll
        for (int e = 0; e < 16; ++e) x[kb][e] = __builtin_amdgcn_exp2f(x[kb][e] * c2);
#pragma unroll
        for (int i = 0; i < 4; ++i)
          xo[(kb * 4 + i) * 64] = make_float4(x[kb][4 * i], x[kb][4 * i + 1], x[kb][4 * i + 2],
                                              x[kb][4 * i + 3]);
#pragma unroll
        for (int hh = 0; hh < 2; ++hh) {
          uint32_t w[4];
#pragma unroll
          for (int t = 0; t < 4; ++t) w[t] = pack_bf16(x[kb][8 * hh + 2 * t], x[kb][8 * hh + 2 * t + 1]);
          bop[kb][hh] = __builtin_bit_cast(bf16x8_t, make_uint4(w[0], w[1], w[2], w[3]));
        }
      }
      // the stores must have landed before the barrier that publishes them
      __builtin_amdgcn_s_waitcnt(0xC07F);   // lgkmcnt(0)
    }
  };
  // dS wave, after the barrier of block qb: dS = P o (dP - delta) from the
  // exchange half XH, packed as the B operand of its dK product
  auto ds_make = [&](auto xh, f32x16_t (&x)[KB], bf16x8_t (&bop)[KB][2])
      __attribute__((always_inline)) {
    const float4* xi = xslot(xh) + pr * KB * 4 * 64 + lane;
#pragma unroll
    for (int kb = 0; kb < KB; ++kb) {
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const float4 p = xi[(kb * 4 + i) * 64];
        x[kb][4 * i + 0] *= p.x; x[kb][4 * i + 1] *= p.y;
        x[kb][4 * i + 2] *= p.z; x[kb][4 * i + 3] *= p.w;
      }
#pragma unroll
      for (int hh = 0; hh < 2; ++hh) {
        uint32_t w[4];
#pragma unroll
        for (int t = 0; t < 4; ++t) w[t] = pack_bf16(x[kb][8 * hh + 2 * t], x[kb][8 * hh + 2 * t + 1]);
        bop[kb][hh] = __builtin_bit_cast(bf16x8_t, make_uint4(w[0], w[1], w[2], w[3]));
      }
    }
  };
  // acc += T^T B for block qb of the tile in slot SL (T = dO for the P
  // wave, Q for the dS wave; T^T read transposed)
  auto mma_t = [&](auto role, auto sl, int qb, const bf16x8_t (&bop)[KB][2])
      __attribute__((always_inline)) {
    constexpr bool R = decltype(role)::value;
    const char* tsl = reinterpret_cast<const char*>(R ? dslot(sl) : qslot(sl)) + 32 * qb * KCH * 16;
    __builtin_amdgcn_s_setprio(1);
#pragma unroll
    for (int hh = 0; hh < 2; ++hh) {
      const char* blk = tsl + 16 * hh * KCH * 16;
#pragma unroll
      for (int db = 0; db < D / 32; ++db) {
        const bf16x8_t ta = tr_read<D>(blk, t_off, db);
#pragma unroll
        for (int kb = 0; kb < KB; ++kb)
          acc[kb][db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(ta, bop[kb][hh], acc[kb][db], 0, 0, 0);
      }
    }
    __builtin_amdgcn_s_setprio(0);
  };
  // end of a tile: this wave's DMA has landed, then every wave's has
  auto tile_end = [&]() __attribute__((always_inline)) {
    __builtin_amdgcn_s_waitcnt(0x0070);   // vmcnt(0) lgkmcnt(0)
    barrier();
  };
  // The whole query loop of one role; the two roles pass the same sequence
  // of barriers.  The dS wave runs its dK product one block late, in the
  // phase where the P wave exponentiates (and its dS arithmetic beside the
  // P wave's dV product), so that on each SIMD one wave's VALU work meets
  // the other's MFMAs.  The next tile's DMA is therefore issued only after
  // the first barrier of a tile, when the late dK product of the previous
  // tile has read its slot.
  auto run = [&](auto role) __attribute__((always_inline)) {
    constexpr bool R = decltype(role)::value;
    f32x16_t x[KB];
    bf16x8_t bop[KB][2];
    const int nqt = (L + kBwdRows - 1) / kBwdRows;
    auto tile = [&](auto sl, auto osl, int t) __attribute__((always_inline)) {
      // block 0
      if constexpr (!R) {
        if (t > 0) mma_t(role, osl, 1, bop);    // block 1 of the previous tile
      }
      phase1(role, sl, int_c<0>{}, 0, x, bop);
      barrier();
      if (t + 1 < nqt) issue(t + 1, osl);
      if constexpr (R) mma_t(role, sl, 0, bop);
      else ds_make(int_c<0>{}, x, bop);
      // block 1
      if constexpr (!R) mma_t(role, sl, 0, bop);
      phase1(role, sl, int_c<1>{}, 1, x, bop);
      barrier();
      if constexpr (R) mma_t(role, sl, 1, bop);
      else ds_make(int_c<1>{}, x, bop);
      tile_end();
    };
    issue(0, int_c<0>{});
    tile_end();
    for (int t = 0; t < nqt; t += 2) {
      tile(int_c<0>{}, int_c<1>{}, t);
      if (t + 1 >= nqt) break;
      tile(int_c<1>{}, int_c<0>{}, t + 1);
    }
    if constexpr (!R) {
      if ((nqt - 1) & 1) mma_t(role, int_c<1>{}, 1, bop);
      else mma_t(role, int_c<0>{}, 1, bop);
    }
  };
  if (pw) run(bool_c<true>{});
  else run(bool_c<false>{});

#pragma unroll
  for (int kb = 0; kb < KB; ++kb)
    if (key_row(kb) < L) {
      const uint32_t tok = skiparse_token(mode, uint32_t(key_row(kb)), wb.j, divk, uint32_t(L));
      const int64_t out = int64_t(wb.b) * a.osb + int64_t(wb.h) * a.osh +
                          (wb.tok0 + int64_t(tok)) * a.osn;
      if (pw) store_rows_t<D>(a.dv + out, acc[kb], 1.0f, g);
      else store_rows_t<D>(a.dk + out, acc[kb], a.scale, g);
    }
}

// ---------------------------------------------------------------------------
// 3. dQ.  Each wave owns 32 queries: Q (times scale log2(e)) and dO rows in
// registers, the row's -lse log2(e) and -delta from the workspace.  Per streamed tile of 64
// keys (K and V through LDS, double-buffered): S^T and dP^T - delta per
// 32-key block (C operand layout: keys are rows, the lane's query the
// column), P = exp2 of one fma, dS^T = P o (dP^T - delta) packed to bf16,
// and dQ^T += K^T dS^T with K^T read transposed.
template <int D, bool PACKED, bool S2D, bool TAB>
__global__ __launch_bounds__(BwdCfg<D>::NW_Q * 64, BwdCfg<D>::OCC_Q) void bwd_dq_kernel(const BwdArgs a) {
  using C = BwdCfg<D>;
  constexpr int NW = C::NW_Q;
  constexpr int KCH = C::KCH;
  __shared__ __attribute__((aligned(1024))) uint16_t k_s0[C::TILE];
  __shared__ __attribute__((aligned(1024))) uint16_t k_s1[C::TILE];
  __shared__ __attribute__((aligned(1024))) uint16_t v_s0[C::TILE];
  __shared__ __attribute__((aligned(1024))) uint16_t v_s1[C::TILE];
  auto kslot = [&](auto sl) __attribute__((always_inline)) -> uint16_t* {
    if constexpr (decltype(sl)::value == 0) return k_s0; else return k_s1;
  };
  auto vslot = [&](auto sl) __attribute__((always_inline)) -> uint16_t* {
    if constexpr (decltype(sl)::value == 0) return v_s0; else return v_s1;
  };

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int g = lane >> 5;
  const int l32 = lane & 31;

  const BwdBlock wb = bwd_block<PACKED, false>(a);
  if (!wb.live) return;              // padding of a packed launch, before any barrier
  const int mode = S2D ? a.mode : (a.mode & 3);
  const SkipDiv divk = a.divk;
  const int L = wb.L;
  const int64_t sn = a.sn;
  const int64_t in_off = int64_t(wb.b) * a.sb + int64_t(wb.h) * a.sh + wb.tok0 * sn;
  const int64_t bhn = (int64_t(wb.b) * a.heads + wb.h) * a.ws_ld + wb.tok0;
  const float c2 = a.scale_log2;

  // ---- this lane's query: Q and dO rows as B operands, its two workspace
  // values.  Q is multiplied by scale * log2(e) and rounded to bf16 once,
  // so that the score product started from -lse log2(e) is the exponent of
  // P in base 2 (Q enters no other product of this kernel).
  const int qr = int(wb.blk) * NW * 32 + wave * 32 + l32;
  const bool qvalid = qr < L;
  const uint32_t qi = skiparse_token(mode, uint32_t(qvalid ? qr : 0), wb.j, divk, uint32_t(L));
  bf16x8_t qreg[D / 16], oreg[D / 16];
  load_row_operand<D>(a.q + in_off + int64_t(qi) * sn, qvalid, g, qreg);
  scale_operand<D>(qreg, c2);
  load_row_operand<D>(a.dout + in_off + int64_t(qi) * sn, qvalid, g, oreg);
  const float nl2 = (qvalid ? a.neg_lse_s[bhn + qi] : 0.f) * c2;     // -lse log2(e)
  const float ne = qvalid ? a.neg_delta[bhn + qi] : 0.f;

  f32x16_t dq[D / 32];
#pragma unroll
  for (int db = 0; db < D / 32; ++db)
#pragma unroll
    for (int e = 0; e < 16; ++e) dq[db][e] = 0.f;
  const RowOff<D> r_off(lane);
  const TrOff<D> t_off(lane);

  static_assert(NW == C::LW || NW == 2 * C::LW, "one or two loading wave groups");
  const int lw = wave % C::LW;       // rank among the waves loading a tensor
  const uint32_t tab_cj = build_row_tab<TAB>(mode, wb.j, divk, L);
  TileDma<D> dma;
  dma.init(lw, lane);
  const uint16_t* kg = a.k + in_off;
  const uint16_t* vg = a.v + in_off;
  auto load = [&](const uint16_t* src, uint32_t i0, uint16_t* dst) __attribute__((always_inline)) {
    const __amdgpu_buffer_rsrc_t rs = __builtin_amdgcn_make_buffer_rsrc(
        const_cast<uint16_t*>(src + int64_t(i0) * sn), (short)0, kRecords, 0x00020000);
#pragma unroll
    for (int u = 0; u < C::DPW; ++u) {
      const int32_t off = dma.off[u];
      __builtin_amdgcn_raw_ptr_buffer_load_lds(rs, (lds_void_ptr)(dst + 512 * (lw + C::LW * u)),
                                               16, off, 0, 0, 0);
    }
  };
  auto issue = [&](int t, auto sl) __attribute__((always_inline)) {
    const uint32_t i0 = TAB ? dma.at_tab(t, bwd_row_tab, tab_cj, L, sn)
                            : dma.at(t, mode, wb.j, divk, L, sn);
    if constexpr (NW == C::LW) {
      load(kg, i0, kslot(sl));
      load(vg, i0, vslot(sl));
    } else if (wave < C::LW) {
      load(kg, i0, kslot(sl));
    } else {
      load(vg, i0, vslot(sl));
    }
  };

  // CLAMP (the last tile, when it holds keys past the end of the
  // subsequence): those keys have zero K and V rows, so they add dS * 0 to
  // dQ; P is clamped to [0, 1] (its true range), which keeps their
  // exp2(-lse log2(e)) finite without a branch per element.
  auto compute = [&](int t, auto sl, auto clamp) __attribute__((always_inline)) {
    constexpr bool CLAMP = decltype(clamp)::value;
    const char* ks = reinterpret_cast<const char*>(kslot(sl));
    const char* vs = reinterpret_cast<const char*>(vslot(sl));
#pragma unroll
    for (int kb = 0; kb < kBwdRows / 32; ++kb) {
      const char* kblk = ks + 32 * kb * KCH * 16;
      const char* vblk = vs + 32 * kb * KCH * 16;
      f32x16_t s, dp;
#pragma unroll
      for (int e = 0; e < 16; ++e) {
        s[e] = nl2;
        dp[e] = ne;
      }
      // At head_dim 128 (one wave per SIMD) nothing else hides the LDS
      // latency: the S and dP products keep three reads in flight.
      constexpr int PFD = 3;
      if constexpr (NW == C::LW) __builtin_amdgcn_sched_barrier(0);
#pragma unroll
      for (int c = 0; c < D / 16; ++c) {
        const bf16x8_t ka = *reinterpret_cast<const bf16x8_t*>(kblk + r_off(c));
        s = __builtin_amdgcn_mfma_f32_32x32x16_bf16(ka, qreg[c], s, 0, 0, 0);
        const bf16x8_t va = *reinterpret_cast<const bf16x8_t*>(vblk + r_off(c));
        dp = __builtin_amdgcn_mfma_f32_32x32x16_bf16(va, oreg[c], dp, 0, 0, 0);
      }
      if constexpr (NW == C::LW) {
        __builtin_amdgcn_sched_group_barrier(0x100, PFD, 0);      // LDS reads
#pragma unroll
        for (int c = 0; c < 2 * (D / 16) - PFD; ++c) {
          __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);      // one MFMA
          __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);      // one LDS read
        }
        __builtin_amdgcn_sched_group_barrier(0x008, PFD, 0);
        __builtin_amdgcn_sched_barrier(0);
      }
      bf16x8_t sb[2];
#pragma unroll
      for (int hh = 0; hh < 2; ++hh) {
        uint32_t sw[4];
#pragma unroll
        for (int tt = 0; tt < 4; ++tt) {
          const int e0 = 8 * hh + 2 * tt, e1 = e0 + 1;
          float p0 = __builtin_amdgcn_exp2f(s[e0]);
          float p1 = __builtin_amdgcn_exp2f(s[e1]);
          if constexpr (CLAMP) {
            p0 = __builtin_amdgcn_fmed3f(p0, 0.f, 1.f);
            p1 = __builtin_amdgcn_fmed3f(p1, 0.f, 1.f);
          }
          sw[tt] = pack_bf16(p0 * dp[e0], p1 * dp[e1]);
        }
        sb[hh] = __builtin_bit_cast(bf16x8_t, make_uint4(sw[0], sw[1], sw[2], sw[3]));
      }
#pragma unroll
      for (int hh = 0; hh < 2; ++hh) {
        const char* kh = kblk + 16 * hh * KCH * 16;
#pragma unroll
        for (int db = 0; db < D / 32; ++db)
          dq[db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(tr_read<D>(kh, t_off, db), sb[hh], dq[db], 0, 0, 0);
      }
    }
  };

  // Tiles alternate between the two slots; the loop runs the tiles that
  // hold no key past the end (tc of them), then the ragged last tile, if
  // any, runs once with the clamp.
  const int nkt = (L + kBwdRows - 1) / kBwdRows;
  const int tc = (L % kBwdRows) ? nkt - 1 : nkt;
  issue(0, int_c<0>{});
  __builtin_amdgcn_s_waitcnt(0x0070);
  __syncthreads();
  int t = 0;
  for (; t + 2 <= tc; t += 2) {
    if (t + 1 < nkt) issue(t + 1, int_c<1>{});
    compute(t, int_c<0>{}, bool_c<false>{});
    __builtin_amdgcn_s_waitcnt(0x0070);
    __syncthreads();
    if (t + 2 < nkt) issue(t + 2, int_c<0>{});
    compute(t + 1, int_c<1>{}, bool_c<false>{});
    __builtin_amdgcn_s_waitcnt(0x0070);
    __syncthreads();
  }
  // one or two tiles left: an odd tile count leaves one unclamped tile in
  // slot 0, and a ragged sequence one clamped tile after it
  if (t < tc) {
    if (t + 1 < nkt) issue(t + 1, int_c<1>{});
    compute(t, int_c<0>{}, bool_c<false>{});
    __builtin_amdgcn_s_waitcnt(0x0070);
    __syncthreads();
    ++t;
    if (t < nkt) compute(t, int_c<1>{}, bool_c<true>{});
  } else if (t < nkt) {
    compute(t, int_c<0>{}, bool_c<true>{});
  }

  if (qvalid) {
    const int64_t out = int64_t(wb.b) * a.osb + int64_t(wb.h) * a.osh + (wb.tok0 + int64_t(qi)) * a.osn;
    store_rows_t<D>(a.dq + out, dq, a.scale, g);
  }
}

// ---------------------------------------------------------------------------
template <int D>
static hipError_t launch_prep_d(const BwdArgs& a, hipStream_t s) {
  const uint64_t rows = uint64_t(a.batch) * uint64_t(a.heads) * uint64_t(a.n_tokens);
  const uint32_t prep_blocks = uint32_t((rows + kPrepThreads - 1) / kPrepThreads);
  hipLaunchKernelGGL((bwd_prep_kernel<D>), dim3(prep_blocks), dim3(kPrepThreads), 0, s, a,
                     uint32_t(rows), make_fastdiv(uint32_t(a.n_tokens)),
                     make_fastdiv(uint32_t(a.heads)));
  return hipGetLastError();
}

// LDS of a workgroup, static plus dynamic, in bytes; the static part of a
// kernel (-1 if the runtime cannot say)
constexpr int kBwdLdsBytes = 160 * 1024;
static int static_lds_bytes(const void* kernel) {
  hipFuncAttributes attr;
  return hipFuncGetAttributes(&attr, kernel) == hipSuccess ? int(attr.sharedSizeBytes) : -1;
}

template <int D>
static hipError_t launch_bwd_d(const BwdArgs& a, hipStream_t s) {
  using C = BwdCfg<D>;
  hipError_t e = launch_prep_d<D>(a, s);
  if (e != hipSuccess) return e;
  const uint32_t seqs = uint32_t(a.batch) * uint32_t(a.heads) * uint32_t(a.groups);
  const dim3 kv_grid(seqs * uint32_t(a.kv_blocks)), q_grid(seqs * uint32_t(a.q_blocks));
  // Skiparse-2D: rows from an LDS row table when it fits beside the
  // kernel's static LDS
  const size_t tab = size_t(a.seq_len) * 4;
  if (a.mode >= MODE_SINGLE2D) {
    auto kv = bwd_dkdv_kernel<D, false, true, true>;
    static std::atomic<int> kv_lds{-1};
    if (kv_lds.load() < 0) kv_lds.store(static_lds_bytes(reinterpret_cast<const void*>(kv)));
    if (kv_lds.load() >= 0 && kv_lds.load() + tab <= size_t(kBwdLdsBytes))
      hipLaunchKernelGGL(kv, kv_grid, dim3(512), tab, s, a);
    else
      hipLaunchKernelGGL((bwd_dkdv_kernel<D, false, true, false>), kv_grid, dim3(512), 0, s, a);
  } else {
    hipLaunchKernelGGL((bwd_dkdv_kernel<D, false, false, false>), kv_grid, dim3(512), 0, s, a);
  }
  e = hipGetLastError();
  if (e != hipSuccess) return e;
  if (a.mode >= MODE_SINGLE2D) {
    auto qk = bwd_dq_kernel<D, false, true, true>;
    static std::atomic<int> q_lds{-1};
    if (q_lds.load() < 0) q_lds.store(static_lds_bytes(reinterpret_cast<const void*>(qk)));
    if (q_lds.load() >= 0 && q_lds.load() + tab <= size_t(kBwdLdsBytes))
      hipLaunchKernelGGL(qk, q_grid, dim3(C::NW_Q * 64), tab, s, a);
    else
      hipLaunchKernelGGL((bwd_dq_kernel<D, false, true, false>), q_grid, dim3(C::NW_Q * 64), 0, s, a);
  } else {
    hipLaunchKernelGGL((bwd_dq_kernel<D, false, false, false>), q_grid, dim3(C::NW_Q * 64), 0, s, a);
  }
  return hipGetLastError();
}

template <int D>
static hipError_t launch_packed_d(const BwdArgs& pa, int kv_grid, int q_grid, hipStream_t s) {
  using C = BwdCfg<D>;
  // packed calls take the 1D modes only
  hipLaunchKernelGGL((bwd_dkdv_kernel<D, true, false, false>), dim3(kv_grid), dim3(512), 0, s, pa);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL((bwd_dq_kernel<D, true, false, false>), dim3(q_grid), dim3(C::NW_Q * 64), 0, s, pa);
  return hipGetLastError();
}

hipError_t launch_attn3d_bwd(const BwdArgs& a, int head_dim, hipStream_t s) {
  switch (head_dim) {
    case 64: return launch_bwd_d<64>(a, s);
    case 96: return launch_bwd_d<96>(a, s);
    case 128: return launch_bwd_d<128>(a, s);
  }
  return hipErrorInvalidValue;
}

hipError_t launch_attn3d_bwd_prep(const BwdArgs& a, int head_dim, hipStream_t s) {
  switch (head_dim) {
    case 64: return launch_prep_d<64>(a, s);
    case 96: return launch_prep_d<96>(a, s);
    case 128: return launch_prep_d<128>(a, s);
  }
  return hipErrorInvalidValue;
}

hipError_t launch_attn3d_bwd_packed(const BwdArgs& pa, int kv_grid, int q_grid, int head_dim,
                                    hipStream_t s) {
  switch (head_dim) {
    case 64: return launch_packed_d<64>(pa, kv_grid, q_grid, s);
    case 96: return launch_packed_d<96>(pa, kv_grid, q_grid, s);
    case 128: return launch_packed_d<128>(pa, kv_grid, q_grid, s);
  }
  return hipErrorInvalidValue;
}

}  // namespace osp
