// attn3d_fwd.hip -- flash-style attention forward for gfx950 (MI355X):
// 3D RoPE fused into the Q/K loaders, Skiparse as a row -> token remap in
// the loaders and the store, bf16 MFMA 32x32x16 with fp32 accumulation,
// fp32 online softmax.
//
// What it computes: softmax(scale * q k^T) v over every token of a
// subsequence (CogVideoX section 2.2 "3D Full Attention"; Skiparse
// subsequences from Open-Sora Plan section 2.2.2).  The blocked order with a
// running maximum reaches the same result as the plain definition up to
// rounding (the FlashAttention argument cited in CogVideoX section 2.2).
//
// Work split.  One workgroup = NW waves owns BM = NW*32*QB query rows of one
// (batch, head, subsequence); each wave owns QB blocks of 32 rows.  Keys
// and values stream through LDS in tiles of BN rows, double buffered.
//
// Per wave and key tile, S^T = K Q^T is formed with K as the A operand
// (read from LDS) and Q^T as the B operand (held in registers), so each lane
// ends up holding scores of ONE query (column = lane mod 32): the row max
// and row sum are in-lane reductions plus one exchange with lane +-32.
// O^T = V^T P^T then takes the probabilities straight from the score
// registers as the B operand; V is stored transposed in LDS so the A operand
// is two 8-byte reads per lane.  The k-index order inside each PV product
// is permuted identically on both operands to match the score layout.
//
// Softmax: logits are kept in log2 units (scale * log2 e folded into one
// FMA before v_exp_f32).  The reference maximum m of a row is only raised
// when a tile's maximum exceeds it by more than kTau (= 8, i.e. factor 256),
// so the O rescale is skipped for most tiles; probabilities stay <= 2^8 and
// the final O / l is unchanged in exact arithmetic.
#include "osp_internal.hpp"

namespace osp {

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef float f32x16_t __attribute__((ext_vector_type(16)));

constexpr float kTau = 8.0f;
constexpr float kLn2 = 0.69314718055994530942f;

template <int D, int NW, int QB, int BN>
struct AttnCfg {
  static constexpr int NT = NW * 64;
  static constexpr int BM = NW * 32 * QB;
  static constexpr int KSTR = D + 8;    // LDS row pitch of K (bf16): 16*odd bytes
  static constexpr int VSTR = BN + 4;   // LDS row pitch of V^T (bf16): 8*odd bytes
  static constexpr int K_ELEMS = BN * KSTR;
  static constexpr int V_ELEMS = D * VSTR;
  static constexpr int STAGE = K_ELEMS + V_ELEMS;
  static constexpr int KCH = D / 8;     // 16-byte chunks per row
  static constexpr int K_ITEMS = BN * KCH;
  static constexpr int K_PER_T = (K_ITEMS + NT - 1) / NT;
  static constexpr int V_ITEMS = (BN / 4) * KCH;
  static constexpr int V_PER_T = (V_ITEMS + NT - 1) / NT;
  static_assert(D % 32 == 0 && BN % 32 == 0, "tile shape");
  static_assert(((KSTR * 2 / 16) & 1) == 1, "K pitch must be 16 * odd bytes");
  static_assert(((VSTR * 2 / 8) & 1) == 1, "V^T pitch must be 8 * odd bytes");
};

// LDS for the RoPE rates and cos/sin table, only when the kernel rotates.
template <bool R> struct RopeSmem {
  RopeLds r;
  __device__ RopeLds* get() { return &r; }
};
template <> struct RopeSmem<false> {
  uint32_t pad[4];
  __device__ RopeLds* get() { return nullptr; }
};

__device__ __forceinline__ uint4 ld16(const uint16_t* p) {
  return *reinterpret_cast<const uint4*>(p);
}

__device__ __forceinline__ float xor32(float x) { return __shfl_xor(x, 32); }

template <int D, int NW, int QB, int BN, int ROPE>
__global__ __launch_bounds__(NW * 64) void attn3d_fwd_kernel(const AttnArgs a) {
  using C = AttnCfg<D, NW, QB, BN>;
  __shared__ __attribute__((aligned(16))) uint16_t smem[2 * C::STAGE];
  __shared__ __attribute__((aligned(16))) RopeSmem<ROPE != 0> rsm;
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

  const int L = a.seq_len;
  const int64_t in_off = int64_t(b) * a.sb + int64_t(h) * a.sh;
  const uint16_t* __restrict__ qg = a.q + in_off;
  const uint16_t* __restrict__ kg = a.k + in_off;
  const uint16_t* __restrict__ vg = a.v + in_off;

  if constexpr (ROPE != 0) {
    build_rope_lds(a.rope, rl, tid, C::NT);
    __syncthreads();
  }

  // ---- Q^T operand: lane holds query (block, l32), channels 16c + 8g .. +7
  bf16x8_t qreg[QB][D / 16];
#pragma unroll
  for (int qb = 0; qb < QB; ++qb) {
    const int r = int(qt) * C::BM + (wave * QB + qb) * 32 + l32;
    const bool valid = r < L;
    const uint32_t i = skiparse_token(a.mode, uint32_t(valid ? r : 0), j, a.divk);
    const uint16_t* p = qg + int64_t(i) * a.sn;
    Coord3 cc;
    const bool video = ROPE ? token_coords(a.rope, i, &cc) : false;
#pragma unroll
    for (int c = 0; c < D / 16; ++c) {
      uint4 raw = valid ? ld16(p + 16 * c + 8 * g) : make_uint4(0, 0, 0, 0);
      if (ROPE == 1 && video) raw = rotate_chunk_col(rl, chunk_col(a.rope, 8 * c + 4 * g), cc, raw);
      if (ROPE == 2 && video) raw = rotate_chunk(a.rope, rl, 8 * c + 4 * g, cc, raw);
      qreg[qb][c] = __builtin_bit_cast(bf16x8_t, raw);
    }
  }

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

  // ---- K/V tile loaders: global -> registers -> (rotate / transpose) -> LDS
  uint4 kreg[C::K_PER_T];
  Coord3 kcrd[C::K_PER_T];
  bool kvid[C::K_PER_T];
  uint4 vreg[C::V_PER_T][4];
  ChunkCol kcol[C::K_PER_T];     // fast RoPE path: table column of each K chunk
  if constexpr (ROPE == 1) {
#pragma unroll
    for (int e = 0; e < C::K_PER_T; ++e)
      kcol[e] = chunk_col(a.rope, 4 * ((tid + e * C::NT) % C::KCH));
  }

  auto load_tile = [&](int kt) {
#pragma unroll
    for (int e = 0; e < C::K_PER_T; ++e) {
      const int idx = tid + e * C::NT;
      const int row = idx / C::KCH, ch = idx % C::KCH;
      const int r = kt * BN + row;
      const bool valid = (idx < C::K_ITEMS) && (r < L);
      const uint32_t i = skiparse_token(a.mode, uint32_t(valid ? r : 0), j, a.divk);
      kreg[e] = valid ? ld16(kg + int64_t(i) * a.sn + 8 * ch) : make_uint4(0, 0, 0, 0);
      if (ROPE) kvid[e] = valid && token_coords(a.rope, i, &kcrd[e]);
    }
#pragma unroll
    for (int e = 0; e < C::V_PER_T; ++e) {
      const int idx = tid + e * C::NT;
      const int kq = idx % (BN / 4), ch = idx / (BN / 4);
#pragma unroll
      for (int t = 0; t < 4; ++t) {
        const int r = kt * BN + 4 * kq + t;
        const bool valid = (idx < C::V_ITEMS) && (r < L);
        const uint32_t i = skiparse_token(a.mode, uint32_t(valid ? r : 0), j, a.divk);
        vreg[e][t] = valid ? ld16(vg + int64_t(i) * a.sn + 8 * ch) : make_uint4(0, 0, 0, 0);
      }
    }
  };

  auto store_tile = [&](int buf) {
    uint16_t* ks = smem + buf * C::STAGE;
    uint16_t* vs = ks + C::K_ELEMS;
#pragma unroll
    for (int e = 0; e < C::K_PER_T; ++e) {
      const int idx = tid + e * C::NT;
      if (idx < C::K_ITEMS) {
        const int row = idx / C::KCH, ch = idx % C::KCH;
        uint4 val = kreg[e];
        if (ROPE == 1 && kvid[e]) val = rotate_chunk_col(rl, kcol[e], kcrd[e], val);
        if (ROPE == 2 && kvid[e]) val = rotate_chunk(a.rope, rl, 4 * ch, kcrd[e], val);
        *reinterpret_cast<uint4*>(ks + row * C::KSTR + 8 * ch) = val;
      }
    }
#pragma unroll
    for (int e = 0; e < C::V_PER_T; ++e) {
      const int idx = tid + e * C::NT;
      if (idx < C::V_ITEMS) {
        const int kq = idx % (BN / 4), ch = idx / (BN / 4);
        const uint32_t w0[4] = {vreg[e][0].x, vreg[e][0].y, vreg[e][0].z, vreg[e][0].w};
        const uint32_t w1[4] = {vreg[e][1].x, vreg[e][1].y, vreg[e][1].z, vreg[e][1].w};
        const uint32_t w2[4] = {vreg[e][2].x, vreg[e][2].y, vreg[e][2].z, vreg[e][2].w};
        const uint32_t w3[4] = {vreg[e][3].x, vreg[e][3].y, vreg[e][3].z, vreg[e][3].w};
#pragma unroll
        for (int dd = 0; dd < 8; ++dd) {
          const int wi = dd >> 1;
          uint32_t lo, hi;
          if (dd & 1) {
            lo = (w0[wi] >> 16) | (w1[wi] & 0xffff0000u);
            hi = (w2[wi] >> 16) | (w3[wi] & 0xffff0000u);
          } else {
            lo = (w0[wi] & 0xffffu) | (w1[wi] << 16);
            hi = (w2[wi] & 0xffffu) | (w3[wi] << 16);
          }
          *reinterpret_cast<uint2*>(vs + (8 * ch + dd) * C::VSTR + 4 * kq) = make_uint2(lo, hi);
        }
      }
    }
  };

  const int nkt = (L + BN - 1) / BN;
  load_tile(0);
  store_tile(0);
  __syncthreads();

  for (int kt = 0; kt < nkt; ++kt) {
    const int buf = kt & 1;
    if (kt + 1 < nkt) load_tile(kt + 1);

    const uint16_t* ks = smem + buf * C::STAGE;
    const uint16_t* vs = ks + C::K_ELEMS;

    // S^T = K Q^T : lane holds query l32, keys 32kb + 8(e/4) + 4g + e%4
    f32x16_t s[BN / 32][QB];
#pragma unroll
    for (int kb = 0; kb < BN / 32; ++kb)
#pragma unroll
      for (int qb = 0; qb < QB; ++qb)
#pragma unroll
        for (int e = 0; e < 16; ++e) s[kb][qb][e] = 0.f;
#pragma unroll
    for (int c = 0; c < D / 16; ++c) {
#pragma unroll
      for (int kb = 0; kb < BN / 32; ++kb) {
        const bf16x8_t ka = *reinterpret_cast<const bf16x8_t*>(
            ks + (32 * kb + l32) * C::KSTR + 16 * c + 8 * g);
#pragma unroll
        for (int qb = 0; qb < QB; ++qb)
          s[kb][qb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(ka, qreg[qb][c], s[kb][qb], 0, 0, 0);
      }
    }

    if ((kt + 1) * BN > L) {   // ragged last tile: drop keys past the end
#pragma unroll
      for (int kb = 0; kb < BN / 32; ++kb)
#pragma unroll
        for (int e = 0; e < 16; ++e) {
          const int key = kt * BN + 32 * kb + 8 * (e >> 2) + 4 * g + (e & 3);
          if (key >= L) {
#pragma unroll
            for (int qb = 0; qb < QB; ++qb) s[kb][qb][e] = -INFINITY;
          }
        }
    }

    // online softmax, one query per lane (pair of lanes l, l^32)
    float zmax[QB];
    bool need = false;
#pragma unroll
    for (int qb = 0; qb < QB; ++qb) {
      float mx = -INFINITY;
#pragma unroll
      for (int kb = 0; kb < BN / 32; ++kb)
#pragma unroll
        for (int e = 0; e < 16; ++e) mx = fmaxf(mx, s[kb][qb][e]);
      mx = fmaxf(mx, xor32(mx));
      zmax[qb] = mx * a.scale_log2;
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

    bf16x8_t pb[QB][BN / 32][2];
#pragma unroll
    for (int qb = 0; qb < QB; ++qb) {
      const float nm = -mref[qb];
      float acc = 0.f;
#pragma unroll
      for (int kb = 0; kb < BN / 32; ++kb) {
        float pv[16];
#pragma unroll
        for (int e = 0; e < 16; ++e) {
          pv[e] = __builtin_amdgcn_exp2f(fmaf(s[kb][qb][e], a.scale_log2, nm));
          acc += pv[e];
        }
#pragma unroll
        for (int hh = 0; hh < 2; ++hh) {
          uint4 w;
          w.x = pack_bf16(pv[8 * hh + 0], pv[8 * hh + 1]);
          w.y = pack_bf16(pv[8 * hh + 2], pv[8 * hh + 3]);
          w.z = pack_bf16(pv[8 * hh + 4], pv[8 * hh + 5]);
          w.w = pack_bf16(pv[8 * hh + 6], pv[8 * hh + 7]);
          pb[qb][kb][hh] = __builtin_bit_cast(bf16x8_t, w);
        }
      }
      lsum[qb] += acc;
    }

    // O^T += V^T P^T  (db innermost: 3*QB independent accumulators between
    // two products into the same one)
#pragma unroll
    for (int kb = 0; kb < BN / 32; ++kb) {
#pragma unroll
      for (int hh = 0; hh < 2; ++hh) {
        bf16x8_t va[D / 32];
#pragma unroll
        for (int db = 0; db < D / 32; ++db) {
          const uint16_t* vrow = vs + (32 * db + l32) * C::VSTR + 32 * kb + 16 * hh + 4 * g;
          const uint2 lo = *reinterpret_cast<const uint2*>(vrow);
          const uint2 hi = *reinterpret_cast<const uint2*>(vrow + 8);
          va[db] = __builtin_bit_cast(bf16x8_t, make_uint4(lo.x, lo.y, hi.x, hi.y));
        }
#pragma unroll
        for (int db = 0; db < D / 32; ++db)
#pragma unroll
          for (int qb = 0; qb < QB; ++qb)
            o[qb][db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(va[db], pb[qb][kb][hh], o[qb][db], 0, 0, 0);
      }
    }

    if (kt + 1 < nkt) store_tile(buf ^ 1);
    __syncthreads();
  }

  // ---- epilogue: O = O^T / l, stored at the original token row ----
  uint16_t* og = a.o + int64_t(b) * a.osb + int64_t(h) * a.osh;
#pragma unroll
  for (int qb = 0; qb < QB; ++qb) {
    const float lt = lsum[qb] + xor32(lsum[qb]);
    const float inv = 1.0f / lt;
    const int r = int(qt) * C::BM + (wave * QB + qb) * 32 + l32;
    if (r < L) {
      const uint32_t i = skiparse_token(a.mode, uint32_t(r), j, a.divk);
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

// Tile shape per head_dim: waves per workgroup, 32-row query blocks per
// wave, keys per tile.
template <int D> struct TileCfg;
template <> struct TileCfg<64> { static constexpr int NW = 4, QB = 2, BN = 64; };
template <> struct TileCfg<96> { static constexpr int NW = 4, QB = 2, BN = 64; };
template <> struct TileCfg<128> { static constexpr int NW = 4, QB = 1, BN = 64; };

int attn_rows_per_block(int head_dim) {
  switch (head_dim) {
    case 64: return TileCfg<64>::NW * 32 * TileCfg<64>::QB;
    case 96: return TileCfg<96>::NW * 32 * TileCfg<96>::QB;
    case 128: return TileCfg<128>::NW * 32 * TileCfg<128>::QB;
    default: return 0;
  }
}

template <int D>
static hipError_t launch_d(const AttnArgs& a, int rope_kind, hipStream_t s) {
  using T = TileCfg<D>;
  dim3 grid(a.total_tiles), block(T::NW * 64);
  if (rope_kind == 1)
    hipLaunchKernelGGL((attn3d_fwd_kernel<D, T::NW, T::QB, T::BN, 1>), grid, block, 0, s, a);
  else if (rope_kind == 2)
    hipLaunchKernelGGL((attn3d_fwd_kernel<D, T::NW, T::QB, T::BN, 2>), grid, block, 0, s, a);
  else
    hipLaunchKernelGGL((attn3d_fwd_kernel<D, T::NW, T::QB, T::BN, 0>), grid, block, 0, s, a);
  return hipGetLastError();
}

hipError_t launch_attn3d(AttnArgs& a, int head_dim, int rope_kind, hipStream_t s) {
  switch (head_dim) {
    case 64: return launch_d<64>(a, rope_kind, s);
    case 96: return launch_d<96>(a, rope_kind, s);
    case 128: return launch_d<128>(a, rope_kind, s);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace osp
