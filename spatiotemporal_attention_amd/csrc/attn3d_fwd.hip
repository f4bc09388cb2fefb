// attn3d_fwd.hip -- flash-style attention forward for gfx950 (MI355X):
// 3D RoPE fused into the Q (and optionally K) loaders, Skiparse as a
// row -> token remap in the loaders and the store, bf16 MFMA 32x32x16 with
// fp32 accumulation, fp32 online softmax.
//
// What it computes: softmax(scale * q k^T) v over every token of a
// subsequence (CogVideoX section 2.2 "3D Full Attention"; Skiparse
// subsequences from Open-Sora Plan section 2.2.2).  The blocked order with a
// running maximum reaches the plain definition's result up to rounding (the
// FlashAttention argument cited in CogVideoX section 2.2).
//
// Work split.  One workgroup = 4 waves owns BM = 4*32*QB query rows of one
// (batch, head, subsequence); each wave owns QB blocks of 32 rows.  Keys and
// values stream through LDS in tiles of BN rows (row-major, padded rows).
//
// Per wave and key tile, S^T = K Q^T is formed with K as the A operand (LDS)
// and Q^T as the B operand (registers), so a lane holds the scores of ONE
// query (column = lane mod 32): row max and row sum are in-lane reductions
// plus one exchange with lane +-32 (v_permlane32_swap).  O^T = V^T P^T takes
// the probabilities straight from the score registers as the B operand; the
// V^T A operand is read from row-major V with ds_read_b64_tr_b16 (a
// transposing LDS read), in the key order that matches the score layout.
//
// Software pipeline (one wave per SIMD, so MFMA and VALU overlap inside the
// wave): iteration j issues the S products of tile j+1 interleaved with the
// exponentials of tile j, then the PV products of tile j interleaved with the
// row max of tile j+1.  K runs one tile ahead of V in double-buffered LDS.
//
// Softmax: logits in log2 units (scale * log2 e folded into one FMA before
// v_exp_f32).  A row's reference maximum m only rises when a tile's maximum
// exceeds it by more than kTau (= 8, a factor 256), so the O rescale is
// skipped for most tiles; probabilities stay <= 2^8 and O / l is unchanged
// in exact arithmetic.  Row sums add the bf16-rounded probabilities (the
// same values the PV product uses) with v_dot2c_f32_bf16.
#include <type_traits>

#include "osp_internal.hpp"

namespace osp {

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x2v_t __attribute__((ext_vector_type(2)));
typedef float f32x16_t __attribute__((ext_vector_type(16)));
typedef short i16x4_t __attribute__((ext_vector_type(4)));
typedef i16x4_t __attribute__((address_space(3))) * lds_i16x4_ptr;

constexpr float kTau = 8.0f;
constexpr float kLn2 = 0.69314718055994530942f;

template <int D, int QB, int BN>
struct AttnCfg {
  static constexpr int NW = 4;
  static constexpr int NT = NW * 64;
  static constexpr int BM = NW * 32 * QB;
  static constexpr int KP = D + 8;              // LDS row pitch (bf16): 16 * odd bytes
  static constexpr int TILE = BN * KP;          // elements of one K or V tile
  static constexpr int KCH = D / 8;             // 16-byte chunks per row
  static constexpr int CH = BN * KCH;           // chunks per tile
  static_assert(D % 32 == 0 && BN % 32 == 0, "tile shape");
  static_assert(CH % 128 == 0, "each half of the workgroup loads whole chunks");
  static_assert(((KP * 2 / 16) & 1) == 1, "row pitch must be 16 * odd bytes");
};

// LDS for the RoPE rates and cos/sin table, only when a loader rotates.
template <bool R> struct RopeSmem {
  RopeLds r;
  __device__ RopeLds* get() { return &r; }
};
template <> struct RopeSmem<false> {
  uint32_t pad[4];
  __device__ RopeLds* get() { return nullptr; }
};

template <bool B> using bool_c = std::integral_constant<bool, B>;

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

// ROPE_Q / ROPE_K: rotate Q / K in the loaders (false = already rotated).
template <int D, int QB, int BN, bool ROPE_Q, bool ROPE_K>
__global__ __launch_bounds__(256) void attn3d_fwd_kernel(const AttnArgs a) {
  using C = AttnCfg<D, QB, BN>;
  constexpr int NKB = BN / 32;        // 32-key blocks per tile
  __shared__ __attribute__((aligned(16))) uint16_t kbuf[2 * C::TILE];
  __shared__ __attribute__((aligned(16))) uint16_t vbuf[2 * C::TILE];
  __shared__ __attribute__((aligned(16))) RopeSmem<ROPE_Q || ROPE_K> rsm;
  RopeLds* const rl = rsm.get();

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = tid >> 6;
  const int g = lane >> 5;      // half of the wave
  const int l32 = lane & 31;

  // ---- which tile: consecutive tiles of one (b, h, j) stay on one XCD ----
  const uint32_t total = uint32_t(a.total_tiles);
  const uint32_t t8 = total & ~7u;
  const uint32_t x = blockIdx.x;
  uint32_t u = (x < t8) ? (x & 7u) * (t8 >> 3) + (x >> 3) : x;
  const uint32_t qt = u % uint32_t(a.q_tiles);
  u /= uint32_t(a.q_tiles);
  const uint32_t j = u % uint32_t(a.groups);
  u /= uint32_t(a.groups);
  const uint32_t h = u % uint32_t(a.heads);
  const uint32_t b = u / uint32_t(a.heads);

  // kernel arguments used below, as locals (keeps the argument block out of
  // private memory)
  const int mode = a.mode;
  const FastDiv divk = a.divk;
  const RopeGeom rg = rope_scalars(a.rope);
  const int64_t a_sn = a.sn;

  const int L = a.seq_len;
  const int nkt = (L + BN - 1) / BN;
  const int64_t in_off = int64_t(b) * a.sb + int64_t(h) * a.sh;
  const uint16_t* __restrict__ qg = a.q + in_off;
  const uint16_t* __restrict__ kg = a.k + in_off;
  const uint16_t* __restrict__ vg = a.v + in_off;
  const float c2 = a.scale_log2;

  if constexpr (ROPE_Q || ROPE_K) {
    stage_rope_rates<C::NT>(a.rope.omega, rl, tid);
    __syncthreads();
    fill_rope_table(rg, rl, tid, C::NT);
    __syncthreads();
  }
  const bool fast_rope = rg.aligned8 && rg.tab_entries;

  // ---- Q^T operand: lane holds query (block, l32), channels 16c + 8g .. +7
  bf16x8_t qreg[QB][D / 16];
#pragma unroll
  for (int qb = 0; qb < QB; ++qb) {
    const int r = int(qt) * C::BM + (wave * QB + qb) * 32 + l32;
    const bool valid = r < L;
    const uint32_t i = skiparse_token(mode, uint32_t(valid ? r : 0), j, divk);
    const uint16_t* p = qg + int64_t(i) * a_sn;
    const bool video = ROPE_Q && is_video(rg, i);
    const Coord3 cc = video_coords(rg, i);
#pragma unroll
    for (int c = 0; c < D / 16; ++c) {
      uint4 raw = valid ? ld16(p + 16 * c + 8 * g) : make_uint4(0, 0, 0, 0);
      if (ROPE_Q && video) raw = rotate_chunk(rg, rl, 8 * c + 4 * g, cc, raw);
      qreg[qb][c] = __builtin_bit_cast(bf16x8_t, raw);
    }
  }

  // ---- loaders.  Each tile's K and V are fetched by the two halves of
  // the workgroup (waves 0-1 and 2-3), which swap roles every tile so that
  // K rotation work alternates.  Tile kt's first row r0 = kt*BN maps to
  // token i0(kt); the remap is increasing in the row, and when BN is a
  // multiple of the group-skip ratio (or the mode is full / single skip),
  // row r0 + row maps to i0(kt) + drow(row): every thread's byte offsets
  // are fixed and only the tile base moves.  Loads go through a buffer descriptor whose range ends
  // at kRecords, so rows past the end of the subsequence (offset kRecords)
  // read as zeros without a branch.
  constexpr int LDPT = C::CH / 128;
  constexpr int32_t kRecords = 0x40000000;
  const int half = __builtin_amdgcn_readfirstlane(tid >> 7);
  const int rt = tid & 127;
  const int kmul = (mode == MODE_FULL) ? 1 : int(divk.d);
  const bool fixed_rows = (mode != MODE_GROUP) || (BN % kmul == 0);
  int ld_row[LDPT], ld_col[LDPT];
  uint32_t ld_drow[LDPT];
  int32_t ld_off[LDPT];
  ChunkCol ld_rc[LDPT];
#pragma unroll
  for (int e = 0; e < LDPT; ++e) {
    const int idx = rt + 128 * e;
    ld_row[e] = idx / C::KCH;
    ld_col[e] = idx % C::KCH;
    const uint32_t rw = uint32_t(ld_row[e]);
    ld_drow[e] = (mode == MODE_FULL) ? rw
               : (mode == MODE_SINGLE) ? rw * uint32_t(kmul)
               : (rw / uint32_t(kmul)) * uint32_t(kmul * kmul) + rw % uint32_t(kmul);
    ld_off[e] = int32_t((int64_t(ld_drow[e]) * a_sn + 8 * ld_col[e]) * 2);
    if constexpr (ROPE_K) ld_rc[e] = chunk_col(rg, 4 * ld_col[e]);
  }

  uint4 ld_reg[LDPT];
  // Issue this thread's loads: the half whose index equals the tile
  // parity fetches K of tile kt_k, the other half V of tile kt_v (-1: none).
  auto issue_loads = [&](int kt_k, int kt_v, int parity) __attribute__((always_inline)) {
    const bool do_k = half == parity;
    const int kt = do_k ? kt_k : kt_v;
    if (kt < 0) return;
    const uint32_t i0 = skiparse_token(mode, uint32_t(kt * BN), j, divk);
    const uint16_t* tb = (do_k ? kg : vg) + int64_t(i0) * a_sn;
    const __amdgpu_buffer_rsrc_t rs =
        __builtin_amdgcn_make_buffer_rsrc(const_cast<uint16_t*>(tb), (short)0, kRecords, 0x00020000);
    const int rem = L - kt * BN;
#pragma unroll
    for (int e = 0; e < LDPT; ++e) {
      int32_t off = ld_off[e];
      if (!fixed_rows) {
        const uint32_t r = uint32_t(min(kt * BN + ld_row[e], L - 1));
        off = int32_t((int64_t(skiparse_token(mode, r, j, divk) - i0) * a_sn + 8 * ld_col[e]) * 2);
      }
      off = (ld_row[e] < rem) ? off : kRecords;
      ld_reg[e] = __builtin_bit_cast(uint4, __builtin_amdgcn_raw_buffer_load_b128(rs, off, 0, 0));
    }
  };
  // Store the staged chunks into LDS (rotating K when fused).
  auto store_loads = [&](int kt_k, int kt_v, int parity) __attribute__((always_inline)) {
    const bool do_k = half == parity;
    const int kt = do_k ? kt_k : kt_v;
    if (kt < 0) return;
    uint16_t* dst = (do_k ? kbuf : vbuf) + (kt & 1) * C::TILE;
    const uint32_t i0 = skiparse_token(mode, uint32_t(kt * BN), j, divk);
#pragma unroll
    for (int e = 0; e < LDPT; ++e) {
      uint4 val = ld_reg[e];
      if constexpr (ROPE_K) {
        if (do_k) {
          const int r = kt * BN + ld_row[e];
          const uint32_t i = fixed_rows ? i0 + ld_drow[e]
                                        : skiparse_token(mode, uint32_t(min(r, L - 1)), j, divk);
          if (r < L && is_video(rg, i)) {
            const Coord3 cc = video_coords(rg, i);
            val = fast_rope ? rotate_chunk_col(rl, ld_rc[e], cc, val)
                            : rotate_chunk_tab(rg, rl, 4 * ld_col[e], cc, val);
          }
        }
      }
      *reinterpret_cast<uint4*>(dst + ld_row[e] * C::KP + 8 * ld_col[e]) = val;
    }
  };

  // ---- accumulators and softmax state
  f32x16_t o[QB][D / 32];
  float mref[QB], lsum[QB];
#pragma unroll
  for (int qb = 0; qb < QB; ++qb) {
    mref[qb] = -INFINITY;
    lsum[qb] = 0.f;
#pragma unroll
    for (int db = 0; db < D / 32; ++db)
#pragma unroll
      for (int e = 0; e < 16; ++e) o[qb][db][e] = 0.f;
  }

  // S^T of tile kt into s (LDS buffer kt & 1)
  auto qk = [&](int kt, f32x16_t (&s)[NKB][QB]) __attribute__((always_inline)) {
    const uint16_t* ks = kbuf + (kt & 1) * C::TILE;
#pragma unroll
    for (int kb = 0; kb < NKB; ++kb)
#pragma unroll
      for (int qb = 0; qb < QB; ++qb)
#pragma unroll
        for (int e = 0; e < 16; ++e) s[kb][qb][e] = 0.f;
#pragma unroll
    for (int c = 0; c < D / 16; ++c) {
#pragma unroll
      for (int kb = 0; kb < NKB; ++kb) {
        const bf16x8_t ka = *reinterpret_cast<const bf16x8_t*>(
            ks + (32 * kb + l32) * C::KP + 16 * c + 8 * g);
#pragma unroll
        for (int qb = 0; qb < QB; ++qb)
          s[kb][qb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(ka, qreg[qb][c], s[kb][qb], 0, 0, 0);
      }
    }
  };
  // keys past the end of the subsequence in tile kt -> -inf
  auto mask = [&](int kt, f32x16_t (&s)[NKB][QB]) __attribute__((always_inline)) {
#pragma unroll
    for (int kb = 0; kb < NKB; ++kb)
#pragma unroll
      for (int e = 0; e < 16; ++e) {
        const int key = kt * BN + 32 * kb + 8 * (e >> 2) + 4 * g + (e & 3);
        if (key >= L) {
#pragma unroll
          for (int qb = 0; qb < QB; ++qb) s[kb][qb][e] = -INFINITY;
        }
      }
  };
  // row max of a tile (scaled to log2 units), raise m where needed, rescale
  auto update_max = [&](f32x16_t (&s)[NKB][QB]) __attribute__((always_inline)) {
    float zmax[QB];
    bool need = false;
#pragma unroll
    for (int qb = 0; qb < QB; ++qb) {
      float mx = -INFINITY;
#pragma unroll
      for (int kb = 0; kb < NKB; ++kb)
#pragma unroll
        for (int e = 0; e < 16; ++e) mx = fmaxf(mx, s[kb][qb][e]);
      zmax[qb] = max_pair32(mx) * c2;
      need |= zmax[qb] > mref[qb] + kTau;
    }
    if (__ballot(need)) {
#pragma unroll
      for (int qb = 0; qb < QB; ++qb) {
        const float mnew = (zmax[qb] > mref[qb] + kTau) ? zmax[qb] : mref[qb];
        const float alpha = __builtin_amdgcn_exp2f(mref[qb] - mnew);
        mref[qb] = mnew;
        lsum[qb] *= alpha;
#pragma unroll
        for (int db = 0; db < D / 32; ++db)
#pragma unroll
          for (int e = 0; e < 16; ++e) o[qb][db][e] *= alpha;
      }
    }
  };
  // probabilities of a tile as bf16 B operands, row sums
  auto softmax = [&](f32x16_t (&s)[NKB][QB], bf16x8_t (&pb)[QB][NKB][2]) __attribute__((always_inline)) {
    const bf16x2v_t one = {(__bf16)1.0f, (__bf16)1.0f};
#pragma unroll
    for (int qb = 0; qb < QB; ++qb) {
      const float nm = -mref[qb];
      float acc = 0.f;
#pragma unroll
      for (int kb = 0; kb < NKB; ++kb)
#pragma unroll
        for (int hh = 0; hh < 2; ++hh) {
          uint32_t w[4];
#pragma unroll
          for (int t = 0; t < 4; ++t) {
            const float p0 = __builtin_amdgcn_exp2f(fmaf(s[kb][qb][8 * hh + 2 * t], c2, nm));
            const float p1 = __builtin_amdgcn_exp2f(fmaf(s[kb][qb][8 * hh + 2 * t + 1], c2, nm));
            w[t] = pack_bf16(p0, p1);
            acc = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2v_t, w[t]), one, acc,
                                                  false);
          }
          pb[qb][kb][hh] = __builtin_bit_cast(bf16x8_t, make_uint4(w[0], w[1], w[2], w[3]));
        }
      lsum[qb] += acc;
    }
  };
  // O^T += V^T P^T for tile kt (V LDS buffer kt & 1)
  auto pv = [&](int kt, bf16x8_t (&pb)[QB][NKB][2]) __attribute__((always_inline)) {
    const uint16_t* vs = vbuf + (kt & 1) * C::TILE;
    const int G = lane >> 4, s16 = lane & 15;
    const int ta = s16 & 3, te = s16 >> 2;
#pragma unroll
    for (int kb = 0; kb < NKB; ++kb)
#pragma unroll
      for (int hh = 0; hh < 2; ++hh) {
        bf16x8_t va[D / 32];
#pragma unroll
        for (int db = 0; db < D / 32; ++db) {
          // source lane (ta, te) of its 16-lane group points at key
          // 32kb + 16hh + 4g + te (+8), channels 32db + 16(G%2) + 4ta .. +3
          const uint16_t* src = vs + (32 * kb + 16 * hh + 4 * (G >> 1) + te) * C::KP +
                                32 * db + 16 * (G & 1) + 4 * ta;
          const i16x4_t lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4_ptr)(src));
          const i16x4_t hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4_ptr)(src + 8 * C::KP));
          const uint2 l2 = __builtin_bit_cast(uint2, lo), h2 = __builtin_bit_cast(uint2, hi);
          va[db] = __builtin_bit_cast(bf16x8_t, make_uint4(l2.x, l2.y, h2.x, h2.y));
        }
#pragma unroll
        for (int db = 0; db < D / 32; ++db)
#pragma unroll
          for (int qb = 0; qb < QB; ++qb)
            o[qb][db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(va[db], pb[qb][kb][hh], o[qb][db], 0, 0, 0);
      }
  };

  // ---- prologue: K0, V0 (and K1) into LDS, S of tile 0
  f32x16_t sA[NKB][QB], sB[NKB][QB];
  issue_loads(0, 0, 0);
  store_loads(0, 0, 0);
  if (nkt > 1) {
    issue_loads(1, -1, 0);
    store_loads(1, -1, 0);
  }
  __syncthreads();
  qk(0, sA);
  if (nkt == 1 && L % BN) mask(0, sA);
  update_max(sA);
  __syncthreads();   // K0's buffer is refilled with K2 in the first iteration

  // ---- main loop.  Iteration jt: S(jt+1) with exp(jt); PV(jt) with
  // max(jt+1); stores K(jt+2), V(jt+1).  The two score arrays alternate.
  auto step = [&](int jt, f32x16_t (&s_cur)[NKB][QB], f32x16_t (&s_nxt)[NKB][QB],
                  auto has_next, auto load_k2, auto mask_next) __attribute__((always_inline)) {
    constexpr bool HAS_NEXT = decltype(has_next)::value;
    constexpr bool LOAD_K2 = decltype(load_k2)::value;
    constexpr bool MASK_NEXT = decltype(mask_next)::value;
    const int parity = jt & 1;
    if constexpr (HAS_NEXT) issue_loads(LOAD_K2 ? jt + 2 : -1, jt + 1, parity);
    bf16x8_t pb[QB][NKB][2];
    if constexpr (HAS_NEXT) qk(jt + 1, s_nxt);
    softmax(s_cur, pb);
    if constexpr (MASK_NEXT) mask(jt + 1, s_nxt);
    pv(jt, pb);
    if constexpr (HAS_NEXT) {
      store_loads(LOAD_K2 ? jt + 2 : -1, jt + 1, parity);
      update_max(s_nxt);
      __syncthreads();
    }
  };
  // the last tiles, starting at tile jt whose scores are in s_cur
  auto tail = [&](int jt, f32x16_t (&s_cur)[NKB][QB], f32x16_t (&s_nxt)[NKB][QB]) __attribute__((always_inline)) {
    if (jt + 1 < nkt) {
      if (L % BN) step(jt, s_cur, s_nxt, bool_c<true>{}, bool_c<false>{}, bool_c<true>{});
      else step(jt, s_cur, s_nxt, bool_c<true>{}, bool_c<false>{}, bool_c<false>{});
      step(jt + 1, s_nxt, s_cur, bool_c<false>{}, bool_c<false>{}, bool_c<false>{});
    } else {
      step(jt, s_cur, s_nxt, bool_c<false>{}, bool_c<false>{}, bool_c<false>{});
    }
  };
  int jt = 0;
  for (; jt + 3 < nkt; jt += 2) {
    step(jt, sA, sB, bool_c<true>{}, bool_c<true>{}, bool_c<false>{});
    step(jt + 1, sB, sA, bool_c<true>{}, bool_c<true>{}, bool_c<false>{});
  }
  if (jt + 2 < nkt) {
    step(jt, sA, sB, bool_c<true>{}, bool_c<true>{}, bool_c<false>{});
    tail(jt + 1, sB, sA);
  } else {
    tail(jt, sA, sB);
  }

  // ---- epilogue: O = O^T / l, stored at the original token row ----
  uint16_t* og = a.o + int64_t(b) * a.osb + int64_t(h) * a.osh;
#pragma unroll
  for (int qb = 0; qb < QB; ++qb) {
    const float lt = sum_pair32(lsum[qb]);
    const float inv = 1.0f / lt;
    const int r = int(qt) * C::BM + (wave * QB + qb) * 32 + l32;
    if (r < L) {
      const uint32_t i = skiparse_token(mode, uint32_t(r), j, divk);
      uint16_t* p = og + int64_t(i) * a.osn;
#pragma unroll
      for (int db = 0; db < D / 32; ++db)
#pragma unroll
        for (int r4 = 0; r4 < 4; ++r4) {
          const uint32_t w0 = pack_bf16(o[qb][db][4 * r4 + 0] * inv, o[qb][db][4 * r4 + 1] * inv);
          const uint32_t w1 = pack_bf16(o[qb][db][4 * r4 + 2] * inv, o[qb][db][4 * r4 + 3] * inv);
          *reinterpret_cast<uint2*>(p + 32 * db + 8 * r4 + 4 * g) = make_uint2(w0, w1);
        }
      if (a.lse && g == 0)
        a.lse[(int64_t(b) * a.heads + h) * a.n_tokens + i] = (mref[qb] + __log2f(lt)) * kLn2;
    }
  }
}

// Tile shape per head_dim: 32-row query blocks per wave, keys per tile.
template <int D> struct TileCfg;
template <> struct TileCfg<64> { static constexpr int QB = 2, BN = 32; };
template <> struct TileCfg<96> { static constexpr int QB = 2, BN = 32; };
template <> struct TileCfg<128> { static constexpr int QB = 1, BN = 32; };

int attn_keys_per_tile(int head_dim) {
  switch (head_dim) {
    case 64: return TileCfg<64>::BN;
    case 96: return TileCfg<96>::BN;
    case 128: return TileCfg<128>::BN;
    default: return 0;
  }
}

int attn_rows_per_block(int head_dim) {
  switch (head_dim) {
    case 64: return AttnCfg<64, TileCfg<64>::QB, TileCfg<64>::BN>::BM;
    case 96: return AttnCfg<96, TileCfg<96>::QB, TileCfg<96>::BN>::BM;
    case 128: return AttnCfg<128, TileCfg<128>::QB, TileCfg<128>::BN>::BM;
    default: return 0;
  }
}

template <int D>
static hipError_t launch_d(const AttnArgs& a, int rope_q, int rope_k, hipStream_t s) {
  using T = TileCfg<D>;
  dim3 grid(a.total_tiles), block(256);
  if (rope_q && rope_k)
    hipLaunchKernelGGL((attn3d_fwd_kernel<D, T::QB, T::BN, true, true>), grid, block, 0, s, a);
  else if (rope_q)
    hipLaunchKernelGGL((attn3d_fwd_kernel<D, T::QB, T::BN, true, false>), grid, block, 0, s, a);
  else if (rope_k)
    hipLaunchKernelGGL((attn3d_fwd_kernel<D, T::QB, T::BN, false, true>), grid, block, 0, s, a);
  else
    hipLaunchKernelGGL((attn3d_fwd_kernel<D, T::QB, T::BN, false, false>), grid, block, 0, s, a);
  return hipGetLastError();
}

hipError_t launch_attn3d(AttnArgs& a, int head_dim, int rope_q, int rope_k, hipStream_t s) {
  switch (head_dim) {
    case 64: return launch_d<64>(a, rope_q, rope_k, s);
    case 96: return launch_d<96>(a, rope_q, rope_k, s);
    case 128: return launch_d<128>(a, rope_q, rope_k, s);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace osp
