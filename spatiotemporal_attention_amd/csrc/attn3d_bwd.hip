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
//  1. bwd_prep: per row, -delta and -lse * log2(e) into the workspace.
//  2. bwd_dkdv: a workgroup owns NW*32 keys of one (batch, head,
//     subsequence), 32 per wave, K and V in registers, and streams the
//     subsequence's queries through LDS in tiles of 64 rows (Q, dO and the
//     two workspace rows).  Per 32-query block:
//       S = Q K^T and dP - delta = dO V^T - delta, with the rows of the Q /
//       dO tile as A operand and K / V as B (the C init of the second
//       carries -delta): a lane holds ONE key (column l%32) and 16 queries;
//       P = exp2(scale log2(e) S - lse log2(e)), dS = P o (dP - delta), each
//       packed to bf16 as a B operand in the C row order;
//       dV^T += dO^T P and dK^T += Q^T dS, their A operands read transposed
//       from the same LDS tiles (ds_read_b64_tr_b16) in that row order.
//  3. bwd_dq: a workgroup owns NW*32 queries, 32 per wave, Q and dO in
//     registers, and streams the keys (K and V tiles): S^T = K Q^T,
//     dP^T - delta = V dO^T - delta (a lane holds ONE query), P^T and dS^T
//     as above, dQ^T += K^T dS^T with K^T read transposed.
// dQ gets a pass of its own instead of atomic fp32 adds from the dK/dV
// pass: the score products are formed twice (7 MFMA products per 32x32
// block instead of 5), but no workspace for dQ and no atomics are needed.
//
// Tiles arrive by LDS DMA (buffer_load ... lds) into two slots per tensor,
// the next tile loading while the current one is used; rows past the end of
// the subsequence read as zeros (out of the buffer range), which makes
// their contributions exactly zero.
#include "osp_internal.hpp"
#include "osp_mfma.hpp"

namespace osp {

constexpr float kLog2e = 1.4426950408889634f;
constexpr int kBwdRows = 64;         // rows of one streamed LDS tile
constexpr int kPrepThreads = 256;

// waves per workgroup of the two blocked kernels, and the waves per SIMD
// their register budget is sized for
template <int D> struct BwdCfg {
  static constexpr int NW = 4;
  static constexpr int OCC_KV = (D == 64) ? 2 : 1;
  static constexpr int OCC_Q = (D == 128) ? 1 : 2;
  static constexpr int KCH = D / 8;                       // 16-byte chunks per row
  static constexpr int TILE = kBwdRows * D;               // bf16 elements of a tile
  static constexpr int DPW = kBwdRows * KCH / 64 / NW;    // DMA loads per wave and tensor
  static_assert((kBwdRows * KCH / 64) % NW == 0, "every wave loads the same share");
};

static int bwd_waves(int head_dim) {
  switch (head_dim) {
    case 64: return BwdCfg<64>::NW;
    case 96: return BwdCfg<96>::NW;
    default: return BwdCfg<128>::NW;
  }
}
int bwd_kv_rows_per_block(int head_dim) { return bwd_waves(head_dim) * 32; }
int bwd_q_rows_per_block(int head_dim) { return bwd_waves(head_dim) * 32; }
int bwd_tile_rows(int) { return kBwdRows; }

// ---------------------------------------------------------------------------
// 1. -delta_i = -sum_d O_id dO_id and -lse_i log2(e), per (b, h, token);
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
  a.neg_delta[idx] = -((acc[0] + acc[1]) + (acc[2] + acc[3]));
  a.neg_lse2[idx] = -a.lse[idx] * kLog2e;
}

// ---------------------------------------------------------------------------
// Shared pieces of the two blocked kernels.

// Which (b, h, subsequence j, row block) a workgroup takes: consecutive
// row blocks of one (b, h, j) share their streamed tiles and stay on one
// XCD (workgroups are dealt to the 8 XCDs round robin).
struct BwdBlock {
  uint32_t b, h, j, blk;
};
__device__ __forceinline__ BwdBlock bwd_block(const BwdArgs& a, uint32_t blocks_per_seq) {
  const uint32_t total = gridDim.x;
  const uint32_t t8 = total & ~7u;
  const uint32_t x = blockIdx.x;
  uint32_t u = (x < t8) ? (x & 7u) * (t8 >> 3) + (x >> 3) : x;
  BwdBlock r;
  r.blk = u % blocks_per_seq;
  u /= blocks_per_seq;
  r.j = u % uint32_t(a.groups);
  u /= uint32_t(a.groups);
  r.h = u % uint32_t(a.heads);
  r.b = u / uint32_t(a.heads);
  return r;
}

// LDS DMA of row tiles: wave w issues the 64-lane loads w + NW*u, u < DPW,
// of each tile; position p = 64*(w + NW*u) + lane of the tile is row
// p / KCH, stored chunk p % KCH, which holds logical chunk
// (p % KCH) ^ chunk_swz(row).
template <int D>
struct TileDma {
  using C = BwdCfg<D>;
  int row[C::DPW], col[C::DPW];
  int32_t off[C::DPW];   // byte offsets of the current tile, relative to its first token

  __device__ __forceinline__ void init(int wave, int lane) {
#pragma unroll
    for (int u = 0; u < C::DPW; ++u) {
      const int p = 64 * (wave + C::NW * u) + lane;
      row[u] = p / C::KCH;
      col[u] = (p % C::KCH) ^ chunk_swz<D>(row[u]);
    }
  }
  // offsets of tile t (rows 64t ..) of subsequence j; returns its first token
  __device__ __forceinline__ uint32_t at(int t, int mode, uint32_t j, const FastDiv& divk, int L,
                                         int64_t sn) {
    const int r0 = t * kBwdRows;
    const uint32_t i0 = skiparse_token(mode, uint32_t(r0), j, divk, uint32_t(L));
#pragma unroll
    for (int u = 0; u < C::DPW; ++u) {
      const int r = r0 + row[u];
      const uint32_t i = skiparse_token(mode, uint32_t(min(r, L - 1)), j, divk, uint32_t(L));
      off[u] = (r < L) ? int32_t((int64_t(i - i0) * sn + 8 * col[u]) * 2) : kRecords;
    }
    return i0;
  }
};
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

// Rows 16c + 8g .. +7 (channels) of this lane's token row, as B operands.
template <int D>
__device__ __forceinline__ void load_row_operand(const uint16_t* row, bool valid, int g,
                                                 bf16x8_t (&x)[D / 16]) {
#pragma unroll
  for (int c = 0; c < D / 16; ++c)
    x[c] = __builtin_bit_cast(bf16x8_t, valid ? ld16(row + 16 * c + 8 * g) : make_uint4(0, 0, 0, 0));
}

// ---------------------------------------------------------------------------
// 2. dK, dV.
template <int D, int NW, int OCC>
__global__ __launch_bounds__(NW * 64, OCC) void bwd_dkdv_kernel(const BwdArgs a) {
  using C = BwdCfg<D>;
  constexpr int KCH = C::KCH;
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

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int g = lane >> 5;
  const int l32 = lane & 31;

  const BwdBlock wb = bwd_block(a, uint32_t(a.kv_blocks));
  const int mode = a.mode;
  const FastDiv divk = a.divk;
  const int L = a.seq_len;
  const int64_t sn = a.sn;
  const int64_t in_off = int64_t(wb.b) * a.sb + int64_t(wb.h) * a.sh;
  const int64_t bhn = (int64_t(wb.b) * a.heads + wb.h) * a.n_tokens;
  const float c2 = a.scale_log2;

  // ---- this lane's key: K and V rows as B operands
  const int kr = int(wb.blk) * NW * 32 + wave * 32 + l32;
  const bool kvalid = kr < L;
  const uint32_t ki = skiparse_token(mode, uint32_t(kvalid ? kr : 0), wb.j, divk, uint32_t(L));
  bf16x8_t kreg[D / 16], vreg[D / 16];
  load_row_operand<D>(a.k + in_off + int64_t(ki) * sn, kvalid, g, kreg);
  load_row_operand<D>(a.v + in_off + int64_t(ki) * sn, kvalid, g, vreg);

  f32x16_t dk[D / 32], dv[D / 32];
#pragma unroll
  for (int db = 0; db < D / 32; ++db)
#pragma unroll
    for (int e = 0; e < 16; ++e) {
      dk[db][e] = 0.f;
      dv[db][e] = 0.f;
    }
  int r_off[D / 16];
  row_read_offsets<D>(lane, r_off);
  int t_off[2][D / 32];
  tr_read_offsets<D>(lane, t_off);

  TileDma<D> dma;
  dma.init(wave, lane);
  const uint16_t* qg = a.q + in_off;
  const uint16_t* dg = a.dout + in_off;
  // the tile of src (this (b, h)'s base) whose first token is i0 into dst
  auto load = [&](const uint16_t* src, uint32_t i0, uint16_t* dst) __attribute__((always_inline)) {
    const __amdgpu_buffer_rsrc_t rs = __builtin_amdgcn_make_buffer_rsrc(
        const_cast<uint16_t*>(src + int64_t(i0) * sn), (short)0, kRecords, 0x00020000);
#pragma unroll
    for (int u = 0; u < C::DPW; ++u) {
      const int32_t off = dma.off[u];
      __builtin_amdgcn_raw_ptr_buffer_load_lds(rs, (lds_void_ptr)(dst + 512 * (wave + NW * u)),
                                               16, off, 0, 0, 0);
    }
  };
  // one fp32 per row of the tile (a workspace row), by one wave
  auto load_floats = [&](const float* src, uint32_t i0, int t, float* dst) __attribute__((always_inline)) {
    const int r = t * kBwdRows + lane;
    const uint32_t i = skiparse_token(mode, uint32_t(min(r, L - 1)), wb.j, divk, uint32_t(L));
    const int32_t off = (r < L) ? int32_t((i - i0) * 4) : kRecords;
    const __amdgpu_buffer_rsrc_t rs = __builtin_amdgcn_make_buffer_rsrc(
        const_cast<float*>(src + i0), (short)0, kRecords, 0x00020000);
    __builtin_amdgcn_raw_ptr_buffer_load_lds(rs, (lds_void_ptr)dst, 4, off, 0, 0, 0);
  };
  auto issue = [&](int t, auto sl) __attribute__((always_inline)) {
    const uint32_t i0 = dma.at(t, mode, wb.j, divk, L, sn);
    load(qg, i0, qslot(sl));
    load(dg, i0, dslot(sl));
    if (wave == 0) load_floats(a.neg_lse2 + bhn, i0, t, lslot(sl));
    if (wave == 1) load_floats(a.neg_delta + bhn, i0, t, eslot(sl));
  };

  auto compute = [&](auto sl) __attribute__((always_inline)) {
    const char* qs = reinterpret_cast<const char*>(qslot(sl));
    const char* ds = reinterpret_cast<const char*>(dslot(sl));
    const float* ls = lslot(sl);
    const float* es = eslot(sl);
#pragma unroll
    for (int qb = 0; qb < kBwdRows / 32; ++qb) {
      const char* qblk = qs + 32 * qb * KCH * 16;
      const char* dblk = ds + 32 * qb * KCH * 16;
      // C rows of this lane: queries 32qb + 8i + 4g + 0..3, i = 0..3
      f32x16_t s, dp;
      float nl[16];
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const float4 e4 = *reinterpret_cast<const float4*>(es + 32 * qb + 8 * i + 4 * g);
        const float4 l4 = *reinterpret_cast<const float4*>(ls + 32 * qb + 8 * i + 4 * g);
        dp[4 * i + 0] = e4.x; dp[4 * i + 1] = e4.y; dp[4 * i + 2] = e4.z; dp[4 * i + 3] = e4.w;
        nl[4 * i + 0] = l4.x; nl[4 * i + 1] = l4.y; nl[4 * i + 2] = l4.z; nl[4 * i + 3] = l4.w;
      }
#pragma unroll
      for (int e = 0; e < 16; ++e) s[e] = 0.f;
#pragma unroll
      for (int c = 0; c < D / 16; ++c) {
        const bf16x8_t qa = *reinterpret_cast<const bf16x8_t*>(qblk + r_off[c]);
        s = __builtin_amdgcn_mfma_f32_32x32x16_bf16(qa, kreg[c], s, 0, 0, 0);
        const bf16x8_t da = *reinterpret_cast<const bf16x8_t*>(dblk + r_off[c]);
        dp = __builtin_amdgcn_mfma_f32_32x32x16_bf16(da, vreg[c], dp, 0, 0, 0);
      }
      bf16x8_t pb[2], sb[2];
#pragma unroll
      for (int hh = 0; hh < 2; ++hh) {
        uint32_t pw[4], sw[4];
#pragma unroll
        for (int t = 0; t < 4; ++t) {
          const int e0 = 8 * hh + 2 * t, e1 = e0 + 1;
          const float p0 = __builtin_amdgcn_exp2f(fmaf(s[e0], c2, nl[e0]));
          const float p1 = __builtin_amdgcn_exp2f(fmaf(s[e1], c2, nl[e1]));
          pw[t] = pack_bf16(p0, p1);
          sw[t] = pack_bf16(p0 * dp[e0], p1 * dp[e1]);
        }
        pb[hh] = __builtin_bit_cast(bf16x8_t, make_uint4(pw[0], pw[1], pw[2], pw[3]));
        sb[hh] = __builtin_bit_cast(bf16x8_t, make_uint4(sw[0], sw[1], sw[2], sw[3]));
      }
#pragma unroll
      for (int hh = 0; hh < 2; ++hh) {
        const char* qh = qblk + 16 * hh * KCH * 16;
        const char* dh = dblk + 16 * hh * KCH * 16;
#pragma unroll
        for (int db = 0; db < D / 32; ++db) {
          dv[db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(tr_read<D>(dh, t_off, db), pb[hh], dv[db], 0, 0, 0);
          dk[db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(tr_read<D>(qh, t_off, db), sb[hh], dk[db], 0, 0, 0);
        }
      }
    }
  };

  const int nqt = (L + kBwdRows - 1) / kBwdRows;
  issue(0, int_c<0>{});
  __builtin_amdgcn_s_waitcnt(0x0070);   // vmcnt(0) lgkmcnt(0)
  __syncthreads();
  for (int t = 0; t < nqt; t += 2) {
    if (t + 1 < nqt) issue(t + 1, int_c<1>{});
    compute(int_c<0>{});
    __builtin_amdgcn_s_waitcnt(0x0070);
    __syncthreads();
    if (t + 1 >= nqt) break;
    if (t + 2 < nqt) issue(t + 2, int_c<0>{});
    compute(int_c<1>{});
    __builtin_amdgcn_s_waitcnt(0x0070);
    __syncthreads();
  }

  if (kvalid) {
    const int64_t out = int64_t(wb.b) * a.osb + int64_t(wb.h) * a.osh + int64_t(ki) * a.osn;
    store_rows_t<D>(a.dk + out, dk, a.scale, g);
    store_rows_t<D>(a.dv + out, dv, 1.0f, g);
  }
}

// ---------------------------------------------------------------------------
// 3. dQ.
template <int D, int NW, int OCC>
__global__ __launch_bounds__(NW * 64, OCC) void bwd_dq_kernel(const BwdArgs a) {
  using C = BwdCfg<D>;
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

  const BwdBlock wb = bwd_block(a, uint32_t(a.q_blocks));
  const int mode = a.mode;
  const FastDiv divk = a.divk;
  const int L = a.seq_len;
  const int64_t sn = a.sn;
  const int64_t in_off = int64_t(wb.b) * a.sb + int64_t(wb.h) * a.sh;
  const int64_t bhn = (int64_t(wb.b) * a.heads + wb.h) * a.n_tokens;
  const float c2 = a.scale_log2;

  // ---- this lane's query: Q and dO rows as B operands, its two workspace values
  const int qr = int(wb.blk) * NW * 32 + wave * 32 + l32;
  const bool qvalid = qr < L;
  const uint32_t qi = skiparse_token(mode, uint32_t(qvalid ? qr : 0), wb.j, divk, uint32_t(L));
  bf16x8_t qreg[D / 16], oreg[D / 16];
  load_row_operand<D>(a.q + in_off + int64_t(qi) * sn, qvalid, g, qreg);
  load_row_operand<D>(a.dout + in_off + int64_t(qi) * sn, qvalid, g, oreg);
  const float nl = qvalid ? a.neg_lse2[bhn + qi] : 0.f;
  const float ne = qvalid ? a.neg_delta[bhn + qi] : 0.f;

  f32x16_t dq[D / 32];
#pragma unroll
  for (int db = 0; db < D / 32; ++db)
#pragma unroll
    for (int e = 0; e < 16; ++e) dq[db][e] = 0.f;
  int r_off[D / 16];
  row_read_offsets<D>(lane, r_off);
  int t_off[2][D / 32];
  tr_read_offsets<D>(lane, t_off);

  TileDma<D> dma;
  dma.init(wave, lane);
  const uint16_t* kg = a.k + in_off;
  const uint16_t* vg = a.v + in_off;
  auto load = [&](const uint16_t* src, uint32_t i0, uint16_t* dst) __attribute__((always_inline)) {
    const __amdgpu_buffer_rsrc_t rs = __builtin_amdgcn_make_buffer_rsrc(
        const_cast<uint16_t*>(src + int64_t(i0) * sn), (short)0, kRecords, 0x00020000);
#pragma unroll
    for (int u = 0; u < C::DPW; ++u) {
      const int32_t off = dma.off[u];
      __builtin_amdgcn_raw_ptr_buffer_load_lds(rs, (lds_void_ptr)(dst + 512 * (wave + NW * u)),
                                               16, off, 0, 0, 0);
    }
  };
  auto issue = [&](int t, auto sl) __attribute__((always_inline)) {
    const uint32_t i0 = dma.at(t, mode, wb.j, divk, L, sn);
    load(kg, i0, kslot(sl));
    load(vg, i0, vslot(sl));
  };

  auto compute = [&](int t, auto sl) __attribute__((always_inline)) {
    const char* ks = reinterpret_cast<const char*>(kslot(sl));
    const char* vs = reinterpret_cast<const char*>(vslot(sl));
    // keys past the end of the subsequence get P = 0 (their K and V rows
    // are zero; the select keeps an overflowing exp2 out of dQ)
    const bool tail = (t + 1) * kBwdRows > L;
#pragma unroll
    for (int kb = 0; kb < kBwdRows / 32; ++kb) {
      const char* kblk = ks + 32 * kb * KCH * 16;
      const char* vblk = vs + 32 * kb * KCH * 16;
      f32x16_t s, dp;
#pragma unroll
      for (int e = 0; e < 16; ++e) {
        s[e] = 0.f;
        dp[e] = ne;
      }
#pragma unroll
      for (int c = 0; c < D / 16; ++c) {
        const bf16x8_t ka = *reinterpret_cast<const bf16x8_t*>(kblk + r_off[c]);
        s = __builtin_amdgcn_mfma_f32_32x32x16_bf16(ka, qreg[c], s, 0, 0, 0);
        const bf16x8_t va = *reinterpret_cast<const bf16x8_t*>(vblk + r_off[c]);
        dp = __builtin_amdgcn_mfma_f32_32x32x16_bf16(va, oreg[c], dp, 0, 0, 0);
      }
      bf16x8_t sb[2];
#pragma unroll
      for (int hh = 0; hh < 2; ++hh) {
        uint32_t sw[4];
#pragma unroll
        for (int tt = 0; tt < 4; ++tt) {
          const int e0 = 8 * hh + 2 * tt, e1 = e0 + 1;
          float p0 = __builtin_amdgcn_exp2f(fmaf(s[e0], c2, nl));
          float p1 = __builtin_amdgcn_exp2f(fmaf(s[e1], c2, nl));
          if (tail) {
            const int key0 = t * kBwdRows + 32 * kb + 8 * (e0 >> 2) + 4 * g + (e0 & 3);
            p0 = (key0 < L) ? p0 : 0.f;
            p1 = (key0 + 1 < L) ? p1 : 0.f;
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

  const int nkt = (L + kBwdRows - 1) / kBwdRows;
  issue(0, int_c<0>{});
  __builtin_amdgcn_s_waitcnt(0x0070);
  __syncthreads();
  for (int t = 0; t < nkt; t += 2) {
    if (t + 1 < nkt) issue(t + 1, int_c<1>{});
    compute(t, int_c<0>{});
    __builtin_amdgcn_s_waitcnt(0x0070);
    __syncthreads();
    if (t + 1 >= nkt) break;
    if (t + 2 < nkt) issue(t + 2, int_c<0>{});
    compute(t + 1, int_c<1>{});
    __builtin_amdgcn_s_waitcnt(0x0070);
    __syncthreads();
  }

  if (qvalid) {
    const int64_t out = int64_t(wb.b) * a.osb + int64_t(wb.h) * a.osh + int64_t(qi) * a.osn;
    store_rows_t<D>(a.dq + out, dq, a.scale, g);
  }
}

// ---------------------------------------------------------------------------
template <int D>
static hipError_t launch_bwd_d(const BwdArgs& a, hipStream_t s) {
  using C = BwdCfg<D>;
  const uint64_t rows = uint64_t(a.batch) * uint64_t(a.heads) * uint64_t(a.n_tokens);
  const uint32_t prep_blocks = uint32_t((rows + kPrepThreads - 1) / kPrepThreads);
  hipLaunchKernelGGL((bwd_prep_kernel<D>), dim3(prep_blocks), dim3(kPrepThreads), 0, s, a,
                     uint32_t(rows), make_fastdiv(uint32_t(a.n_tokens)),
                     make_fastdiv(uint32_t(a.heads)));
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  const uint32_t seqs = uint32_t(a.batch) * uint32_t(a.heads) * uint32_t(a.groups);
  hipLaunchKernelGGL((bwd_dkdv_kernel<D, C::NW, C::OCC_KV>), dim3(seqs * uint32_t(a.kv_blocks)),
                     dim3(C::NW * 64), 0, s, a);
  e = hipGetLastError();
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL((bwd_dq_kernel<D, C::NW, C::OCC_Q>), dim3(seqs * uint32_t(a.q_blocks)),
                     dim3(C::NW * 64), 0, s, a);
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

}  // namespace osp
