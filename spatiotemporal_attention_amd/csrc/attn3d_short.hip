// attn3d_short.hip -- attention forward for short subsequences (L <= 64
// rows) on gfx950: the temporal half of separated spatial / temporal
// attention (CogVideoX section 2.2 "3D Full Attention", Table 8: each
// (h, w) position's T tokens, Single Skip with k = H*W), small windows, and
// Skiparse at large k.
//
// Same result as attn3d_fwd_kernel (softmax(scale q k^T) v per subsequence,
// fused RoPE, the row -> token remap, same operand rounding) for a unit
// whose rows fit in two 32-row blocks.  The flash kernel gives every
// (batch, head, subsequence) unit a workgroup of 256 query rows and
// 64-key tiles, which a unit of 24 rows leaves almost empty; here one wave
// owns one unit, so the work is one or two 32x32 score blocks per wave and
// the kernel runs at the speed of its loads and stores.
//
// Per wave: K and Q rows straight into registers in the MFMA operand layout
// (K rotated when the loader rotates K; Q rotated and scaled by
// scale*log2(e) with one rounding), V rows -> LDS (swizzled, rows past L
// zero), S^T = K Q^T (keys past L masked to -inf), the exact row maximum
// and sum (every key is in the block, so no running rescale), P rounded to
// bf16, O^T = V^T P^T with V^T read transposed, O / l stored at the
// tokens' rows.  All global loads are issued before the workgroup builds
// its cos/sin table, so the table hides their latency.  The waves of a
// workgroup take consecutive heads of one (batch, subsequence), whose rows
// sit next to each other in memory.
#include "osp_internal.hpp"
#include "osp_mfma.hpp"

// K and Q loaded as whole-row chunks and moved to the operand layout
// through LDS (see the kernel); build-time switch per block count, for
// comparing with loads straight into the operand layout.
#ifndef OSP_SHORT_ROWS_LDS
#define OSP_SHORT_ROWS_LDS(NB) (true)
#endif

namespace osp {

template <bool R> struct ShortRope {
  RopeLds r;
  __device__ RopeLds* get() { return &r; }
};
template <> struct ShortRope<false> {
  uint32_t pad[4];
  __device__ RopeLds* get() { return nullptr; }
};

// NB = 32-row blocks per unit (1: L <= 32, 2: L <= 64); W waves (units) per
// workgroup
template <int NB> struct ShortCfg {
  static constexpr int W = (NB == 1) ? 8 : 4;
};

template <int D, int NB, bool ROPE_Q, bool ROPE_K>
__global__ __launch_bounds__(ShortCfg<NB>::W * 64) void attn3d_short_kernel(const AttnArgs a,
                                                                            uint32_t units) {
  constexpr int W = ShortCfg<NB>::W;
  constexpr int KCH = D / 8;
  constexpr int ROWS = 32 * NB;
  constexpr int TILE = ROWS * D;                 // bf16 elements of one wave's V tile
  constexpr int CPL = ROWS * KCH / 64;           // V chunks per lane
  __shared__ __attribute__((aligned(1024))) uint16_t v_s[W][TILE];
  __shared__ __attribute__((aligned(16))) ShortRope<ROPE_Q || ROPE_K> rsm;
  RopeLds* const rl = rsm.get();

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int g = lane >> 5;
  const int l32 = lane & 31;

  // unit u = ((b * groups + j) * heads + h): heads fastest
  const uint32_t u0 = blockIdx.x * W + uint32_t(wave);
  const bool live = u0 < units;
  const uint32_t u = live ? u0 : 0;
  const uint32_t h = u % uint32_t(a.heads);
  const uint32_t bj = u / uint32_t(a.heads);
  const uint32_t j = bj % uint32_t(a.groups);
  const uint32_t b = bj / uint32_t(a.groups);

  const int mode = a.mode;
  const SkipDiv divk = a.divk;
  const int L = live ? a.seq_len : 0;
  const int64_t sn = a.sn;
  const int64_t in_off = int64_t(b) * a.sb + int64_t(h) * a.sh;
  const float c2 = a.scale_log2;
  const RopeGeom rg = rope_scalars(a.rope);

  // ---- every global load first (their latency overlaps the table fill),
  // the RoPE rate first of all: loads complete in order, so waiting for it
  // does not wait for the rows behind it.  V, K and Q as chunks idx = lane
  // + 64 e of whole rows (or K and Q in the operand layouts of S^T = K Q^T,
  // rows 32 rb + l32 at channels 16 c + 8 g .. +7, where that path is built)
  static_assert(W * 64 >= kMaxPairs, "one rate per thread");
  float omega = 0.f;
  if constexpr (ROPE_Q || ROPE_K) {
    if (tid < kMaxPairs) omega = a.rope.omega[tid];
    __builtin_amdgcn_sched_barrier(0);
  }
  uint4 vraw[CPL];
#pragma unroll
  for (int e = 0; e < CPL; ++e) {
    const int idx = lane + 64 * e;
    const int row = idx / KCH, col = idx % KCH;
    const uint32_t i = skiparse_token(mode, uint32_t(row < L ? row : 0), j, divk, uint32_t(L ? L : 1));
    vraw[e] = row < L ? ld16(a.v + in_off + int64_t(i) * sn + 8 * col) : make_uint4(0, 0, 0, 0);
  }
  // (K and Q rows load as whole-row chunks too, like V, and reach the
  // operand layout through the wave's LDS tile below)
  uint32_t tok[NB];
  constexpr bool ROWS_LDS = OSP_SHORT_ROWS_LDS(NB);
  uint4 kraw[NB][ROWS_LDS ? 1 : D / 16], qraw[NB][ROWS_LDS ? 1 : D / 16];
  uint4 kc[ROWS_LDS ? CPL : 1], qc[ROWS_LDS ? CPL : 1];
  if constexpr (ROWS_LDS) {
#pragma unroll
    for (int e = 0; e < CPL; ++e) {
      const int idx = lane + 64 * e;
      const int row = idx / KCH, col = idx % KCH;
      const uint32_t i = skiparse_token(mode, uint32_t(row < L ? row : 0), j, divk, uint32_t(L ? L : 1));
      kc[e] = row < L ? ld16(a.k + in_off + int64_t(i) * sn + 8 * col) : make_uint4(0, 0, 0, 0);
      qc[e] = row < L ? ld16(a.q + in_off + int64_t(i) * sn + 8 * col) : make_uint4(0, 0, 0, 0);
    }
#pragma unroll
    for (int rb = 0; rb < NB; ++rb) {
      const int r = 32 * rb + l32;
      tok[rb] = skiparse_token(mode, uint32_t(r < L ? r : 0), j, divk, uint32_t(L ? L : 1));
    }
  } else {
#pragma unroll
    for (int rb = 0; rb < NB; ++rb) {
      const int r = 32 * rb + l32;
      const bool on = r < L;
      tok[rb] = skiparse_token(mode, uint32_t(on ? r : 0), j, divk, uint32_t(L ? L : 1));
      const int64_t off = in_off + int64_t(tok[rb]) * sn + 8 * g;
#pragma unroll
      for (int c = 0; c < D / 16; ++c) {
        kraw[rb][c] = on ? ld16(a.k + off + 16 * c) : make_uint4(0, 0, 0, 0);
        qraw[rb][c] = on ? ld16(a.q + off + 16 * c) : make_uint4(0, 0, 0, 0);
      }
    }
  }

  if constexpr (ROPE_Q || ROPE_K) {
    // workgroup barriers that wait for LDS stores only, not for the loads
    auto lds_barrier = [&]() __attribute__((always_inline)) {
      __builtin_amdgcn_s_waitcnt(0xC07F);   // lgkmcnt(0)
      __builtin_amdgcn_sched_barrier(0);
      asm volatile("s_barrier" ::: "memory");
      __builtin_amdgcn_sched_barrier(0);
    };
    if (tid < kMaxPairs) rl->omega[tid] = omega;
    lds_barrier();
    fill_rope_table(rg, rl, tid, W * 64);
    lds_barrier();
  }
  if (!live) return;               // whole wave; no workgroup barrier follows

  uint16_t* vs = v_s[wave];
  // whole-row chunks idx = lane + 64 e -> this wave's LDS tile (swizzled)
  auto put_rows = [&](const uint4 (&x)[CPL]) __attribute__((always_inline)) {
#pragma unroll
    for (int e = 0; e < CPL; ++e) {
      const int idx = lane + 64 * e;
      const int row = idx / KCH, col = idx % KCH;
      *reinterpret_cast<uint4*>(vs + 8 * (row * KCH + (col ^ chunk_swz<D>(row)))) = x[e];
    }
  };

  // K rotated as osp_rope3d rotates it (then bf16); Q rotated and scaled by
  // scale*log2(e) with one rounding
  bf16x8_t kreg[NB][D / 16], qreg[NB][D / 16];
  const bool fast_rope = rg.aligned8 && rg.tab_entries;
  if constexpr (ROWS_LDS) {
    // rotate each whole-row chunk (pairs 4 col .. 4 col + 3 of its row's
    // token), then through the LDS tile into the operand layout: K first,
    // then Q over it (the wave's LDS operations run in order), then V
#pragma unroll
    for (int e = 0; e < CPL; ++e) {
      const int idx = lane + 64 * e;
      const int row = idx / KCH, col = idx % KCH;
      if (row < L) {
        const uint32_t i = skiparse_token(mode, uint32_t(row), j, divk, uint32_t(L));
        const bool video = is_video(rg, i);
        const Coord3 cc = video_coords(rg, i);
        if (ROPE_K && video)
          kc[e] = fast_rope ? rotate_chunk_col(rl, chunk_col(rg, 4 * col), cc, kc[e])
                            : rotate_chunk_tab(rg, rl, 4 * col, cc, kc[e]);
        uint4 raw = qc[e];
        if (ROPE_Q && video) {
          raw = fast_rope ? rotate_chunk_col_scaled(rl, chunk_col(rg, 4 * col), cc, raw, c2)
                           : rotate_chunk_scaled(rg, rl, 4 * col, cc, raw, c2);
        } else {
          raw.x = pack_bf16(bf16lo(raw.x) * c2, bf16hi(raw.x) * c2);
          raw.y = pack_bf16(bf16lo(raw.y) * c2, bf16hi(raw.y) * c2);
          raw.z = pack_bf16(bf16lo(raw.z) * c2, bf16hi(raw.z) * c2);
          raw.w = pack_bf16(bf16lo(raw.w) * c2, bf16hi(raw.w) * c2);
        }
        qc[e] = raw;
      }
    }
    const RowOff<D> r_off(lane);
    const char* vsb = reinterpret_cast<const char*>(vs);
    auto get_rows = [&](bf16x8_t (&y)[NB][D / 16]) __attribute__((always_inline)) {
      __builtin_amdgcn_s_waitcnt(0xC07F);   // lgkmcnt(0): this wave's stores landed
      __builtin_amdgcn_wave_barrier();
#pragma unroll
      for (int rb = 0; rb < NB; ++rb)
#pragma unroll
        for (int c = 0; c < D / 16; ++c)
          y[rb][c] = *reinterpret_cast<const bf16x8_t*>(vsb + 32 * rb * KCH * 16 + r_off(c));
    };
    put_rows(kc);
    get_rows(kreg);
    __builtin_amdgcn_wave_barrier();
    put_rows(qc);
    get_rows(qreg);
    __builtin_amdgcn_wave_barrier();
    put_rows(vraw);
  } else {
  // V -> this wave's LDS tile (swizzled; rows past L are zero)
  put_rows(vraw);
#pragma unroll
  for (int rb = 0; rb < NB; ++rb) {
    const bool video = is_video(rg, tok[rb]);
    const Coord3 cc = video_coords(rg, tok[rb]);
#pragma unroll
    for (int c = 0; c < D / 16; ++c) {
      uint4 kv = kraw[rb][c];
      if (ROPE_K && video)
        kv = fast_rope ? rotate_chunk_col(rl, chunk_col(rg, 8 * c + 4 * g), cc, kv)
                       : rotate_chunk_tab(rg, rl, 8 * c + 4 * g, cc, kv);
      kreg[rb][c] = __builtin_bit_cast(bf16x8_t, kv);
      uint4 raw = qraw[rb][c];
      if (ROPE_Q && video) {
        raw = fast_rope ? rotate_chunk_col_scaled(rl, chunk_col(rg, 8 * c + 4 * g), cc, raw, c2)
                        : rotate_chunk_scaled(rg, rl, 8 * c + 4 * g, cc, raw, c2);
      } else {
        raw.x = pack_bf16(bf16lo(raw.x) * c2, bf16hi(raw.x) * c2);
        raw.y = pack_bf16(bf16lo(raw.y) * c2, bf16hi(raw.y) * c2);
        raw.z = pack_bf16(bf16lo(raw.z) * c2, bf16hi(raw.z) * c2);
        raw.w = pack_bf16(bf16lo(raw.w) * c2, bf16hi(raw.w) * c2);
      }
      qreg[rb][c] = __builtin_bit_cast(bf16x8_t, raw);
    }
  }
  }
  // the V tile is this wave's own: its stores land before its reads
  __builtin_amdgcn_s_waitcnt(0xC07F);   // lgkmcnt(0)
  __builtin_amdgcn_wave_barrier();

  const TrOff<D> v_off(lane);
  const char* vb_ = reinterpret_cast<const char*>(vs);

  uint16_t* og = a.o + int64_t(b) * a.osb + int64_t(h) * a.osh;
#pragma unroll
  for (int qb = 0; qb < NB; ++qb) {
    // S^T (log2 units) for every key block; keys past L start from -inf
    f32x16_t s[NB];
#pragma unroll
    for (int kb = 0; kb < NB; ++kb) {
#pragma unroll
      for (int e = 0; e < 16; ++e) {
        const int key = 32 * kb + 8 * (e >> 2) + 4 * g + (e & 3);
        s[kb][e] = key < L ? 0.f : -INFINITY;
      }
#pragma unroll
      for (int c = 0; c < D / 16; ++c)
        s[kb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(kreg[kb][c], qreg[qb][c], s[kb], 0, 0, 0);
    }
    // exact row maximum and sum over all keys (lanes l and l^32 share a query)
    float mx = -INFINITY;
#pragma unroll
    for (int kb = 0; kb < NB; ++kb)
#pragma unroll
      for (int e = 0; e < 16; ++e) mx = fmaxf(mx, s[kb][e]);
    const float m = max_pair32(mx);
    float acc[4] = {0.f, 0.f, 0.f, 0.f};
    bf16x8_t pb[NB][2];
#pragma unroll
    for (int kb = 0; kb < NB; ++kb)
#pragma unroll
      for (int hh = 0; hh < 2; ++hh) {
        uint32_t w[4];
#pragma unroll
        for (int t = 0; t < 4; ++t) {
          const float p0 = __builtin_amdgcn_exp2f(s[kb][8 * hh + 2 * t] - m);
          const float p1 = __builtin_amdgcn_exp2f(s[kb][8 * hh + 2 * t + 1] - m);
          w[t] = pack_bf16(p0, p1);
          acc[t] += p0 + p1;
        }
        pb[kb][hh] = __builtin_bit_cast(bf16x8_t, make_uint4(w[0], w[1], w[2], w[3]));
      }
    const float lt = sum_pair32((acc[0] + acc[1]) + (acc[2] + acc[3]));
    // O^T = V^T P^T
    f32x16_t o[D / 32];
#pragma unroll
    for (int db = 0; db < D / 32; ++db)
#pragma unroll
      for (int e = 0; e < 16; ++e) o[db][e] = 0.f;
#pragma unroll
    for (int kb = 0; kb < NB; ++kb)
#pragma unroll
      for (int hh = 0; hh < 2; ++hh) {
        const char* blk = vb_ + (32 * kb + 16 * hh) * KCH * 16;
#pragma unroll
        for (int db = 0; db < D / 32; ++db)
          o[db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(tr_read<D>(blk, v_off, db), pb[kb][hh],
                                                          o[db], 0, 0, 0);
      }
    const int r = 32 * qb + l32;
    if constexpr (NB == 1) {
      // One block: the wave's V tile is free once its MFMAs have read it.
      // O / l goes there row-major (bf16), then each row is stored as 16-byte
      // chunks by consecutive lanes (12 lanes per 192-byte row at D=96)
      // instead of 8-byte pieces of 32 rows per instruction.
      const float inv = 1.0f / lt;
      __builtin_amdgcn_wave_barrier();
#pragma unroll
      for (int db = 0; db < D / 32; ++db)
#pragma unroll
        for (int r4 = 0; r4 < 4; ++r4) {
          const uint32_t w0 = pack_bf16(o[db][4 * r4 + 0] * inv, o[db][4 * r4 + 1] * inv);
          const uint32_t w1 = pack_bf16(o[db][4 * r4 + 2] * inv, o[db][4 * r4 + 3] * inv);
          *reinterpret_cast<uint2*>(vs + l32 * D + 32 * db + 8 * r4 + 4 * g) = make_uint2(w0, w1);
        }
      __builtin_amdgcn_s_waitcnt(0xC07F);   // lgkmcnt(0): the wave's own stores landed
      __builtin_amdgcn_wave_barrier();
#pragma unroll
      for (int e = 0; e < CPL; ++e) {
        const int idx = lane + 64 * e;
        const int row = idx / KCH, col = idx % KCH;
        if (row < L) {
          const uint32_t i = skiparse_token(mode, uint32_t(row), j, divk, uint32_t(L));
          *reinterpret_cast<uint4*>(og + int64_t(i) * a.osn + 8 * col) =
              *reinterpret_cast<const uint4*>(vs + row * D + 8 * col);
        }
      }
      if (r < L && a.lse && g == 0) {
        const uint32_t i = skiparse_token(mode, uint32_t(r), j, divk, uint32_t(L));
        a.lse[(int64_t(b) * a.heads + h) * a.lse_ld + i] = (m + __log2f(lt)) * 0.69314718055994530942f;
      }
      continue;
    }
    // O / l at the query's token row
    if (r < L) {
      const float inv = 1.0f / lt;
      const uint32_t i = skiparse_token(mode, uint32_t(r), j, divk, uint32_t(L));
      uint16_t* p = og + int64_t(i) * a.osn;
#pragma unroll
      for (int db = 0; db < D / 32; ++db)
#pragma unroll
        for (int r4 = 0; r4 < 4; ++r4) {
          const uint32_t w0 = pack_bf16(o[db][4 * r4 + 0] * inv, o[db][4 * r4 + 1] * inv);
          const uint32_t w1 = pack_bf16(o[db][4 * r4 + 2] * inv, o[db][4 * r4 + 3] * inv);
          *reinterpret_cast<uint2*>(p + 32 * db + 8 * r4 + 4 * g) = make_uint2(w0, w1);
        }
      if (a.lse && g == 0)
        a.lse[(int64_t(b) * a.heads + h) * a.lse_ld + i] = (m + __log2f(lt)) * 0.69314718055994530942f;
    }
  }
}

template <int D, int NB>
static hipError_t launch_short_nb(const AttnArgs& a, int rope_q, int rope_k, hipStream_t s) {
  constexpr int W = ShortCfg<NB>::W;
  const uint32_t units = uint32_t(a.batch) * uint32_t(a.heads) * uint32_t(a.groups);
  dim3 grid((units + W - 1) / W), block(W * 64);
#define OSP_LAUNCH(RQ, RK) \
  hipLaunchKernelGGL((attn3d_short_kernel<D, NB, RQ, RK>), grid, block, 0, s, a, units)
  if (rope_q && rope_k) OSP_LAUNCH(true, true);
  else if (rope_q) OSP_LAUNCH(true, false);
  else if (rope_k) OSP_LAUNCH(false, true);
  else OSP_LAUNCH(false, false);
#undef OSP_LAUNCH
  return hipGetLastError();
}

template <int D>
static hipError_t launch_short_d(const AttnArgs& a, int rope_q, int rope_k, hipStream_t s) {
  return a.seq_len <= 32 ? launch_short_nb<D, 1>(a, rope_q, rope_k, s)
                         : launch_short_nb<D, 2>(a, rope_q, rope_k, s);
}

hipError_t launch_attn3d_short(const AttnArgs& a, int head_dim, int rope_q, int rope_k,
                               hipStream_t s) {
  switch (head_dim) {
    case 64: return launch_short_d<64>(a, rope_q, rope_k, s);
    case 96: return launch_short_d<96>(a, rope_q, rope_k, s);
    case 128: return launch_short_d<128>(a, rope_q, rope_k, s);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace osp
