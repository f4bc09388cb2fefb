// attn3d_fwd.hip -- flash-style attention forward for gfx950 (MI355X):
// 3D RoPE fused into the Q (and optionally K) loaders, Skiparse and block
// attention as a row -> token remap in the loaders and the store, bf16 MFMA
// 32x32x16 with fp32 accumulation, fp32 online softmax.
//
// What it computes: softmax(scale * q k^T) v over every token of a
// subsequence (CogVideoX section 2.2 "3D Full Attention"; Skiparse
// subsequences from Open-Sora Plan section 2.2.2; blocks of adjacent tokens
// for separated spatial attention or window attention).  The blocked order
// with a running maximum reaches the plain definition's result up to
// rounding (the FlashAttention argument cited in CogVideoX section 2.2).
//
// Work split.  One workgroup = NW = 8 waves owns BM = 8*32*QB query rows of
// one (batch, head, subsequence); each wave owns QB blocks of 32 rows.  Keys
// and values stream through LDS in tiles of BN rows.
//
// LDS tiles are unpadded rows of D bf16; the 16-byte chunks of row r are
// XOR-swizzled (chunk_swz) so that the operand reads below hit distinct
// banks.  Tiles arrive by LDS DMA (buffer_load ... lds): each wave issues a
// few 64-lane loads that write 1 KiB of a tile directly, with no registers
// and no LDS store instructions; rows past the end of a subsequence are
// fetched out of the buffer range and land as zeros.  When K is rotated in
// the loader, K chunks go through registers instead.
//
// Per wave and key tile, S^T = K Q^T is formed with K as the A operand (LDS)
// and Q^T as the B operand (registers), so a lane holds the scores of ONE
// query (column = lane mod 32): row reductions are in-lane plus one
// exchange with lane +-32 (v_permlane32_swap).  O^T = V^T P^T takes the
// probabilities straight from the score registers as the B operand; the
// V^T A operand is read from row-major V with ds_read_b64_tr_b16 (a
// transposing LDS read), in the key order that matches the score layout.
//
// Schedule: the waves form two halves that alternate a matrix phase (MFMAs)
// and a softmax phase (VALU) one phase apart, with a workgroup barrier
// after every phase, so that each SIMD runs one wave's MFMAs beside the
// other wave's softmax (see the schedule section below).
//
// Softmax: Q is multiplied by scale * log2(e) once (then bf16 again), so
// scores come out in log2 units, and the first product of each score block
// starts from -m instead of 0: the MFMA delivers z - m and v_exp_f32 takes
// it as is (keys past the end start from -inf).  A row's reference maximum
// m is set by its first tile and afterwards only rises when a tile's scores
// exceed it by more than kTau (= 8, a factor 256), so the O rescale is
// skipped for most tiles; probabilities stay <= 2^8 and O / l is unchanged
// in exact arithmetic.  Row sums add the fp32 probabilities.
#include <type_traits>

#include "osp_internal.hpp"
#include "osp_mfma.hpp"

namespace osp {

constexpr float kTau = 8.0f;
constexpr float kSumTau = 256.0f;   // 2^kTau
constexpr float kLn2 = 0.69314718055994530942f;

template <int D, int QB, int BN, int NW>
struct AttnCfg {
  static constexpr int NT = NW * 64;
  static constexpr int BM = NW * 32 * QB;
  static constexpr int KCH = D / 8;               // 16-byte chunks per row
  static constexpr int CH = BN * KCH;             // chunks per tile
  static constexpr int TILE = BN * D;             // bf16 elements of one K or V tile
  static constexpr int LW = NW / 2;               // waves per half
  static constexpr int LT = LW * 64;
  static constexpr int DPT = CH / 64;             // 64-lane DMA loads per tile
  static constexpr int DPW = DPT / LW;            // per wave of a half, one tensor
  static constexpr int SPT = CH / LT;             // staged K chunks per leading thread
  static_assert(D % 32 == 0 && BN % 32 == 0 && CH % 64 == 0 && NW % 8 == 0, "tile shape");
  static_assert(DPT % LW == 0 && CH % LT == 0, "every wave of a half loads the same amount");
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


// ROPE_Q / ROPE_K: rotate Q / K in the loaders (false = already rotated).
// FIXED_ROWS: the row -> token offsets inside a key tile are the same for
// every tile (full, block, single skip, or group skip with BN a multiple of
// k).
// OCC: waves per SIMD the register budget is sized for.
// Scheduling groups of a matrix phase: NMK QK MFMAs (one LDS read each)
// then NMV PV MFMAs (two reads each), in the program order of their reads
// (the transposing V reads are not moved above other LDS reads).  The
// reads of the first L MFMAs come first; after MFMA i come the reads of
// MFMA i + L.
template <int NMK, int NMV> __device__ constexpr int m_reads(int m) {
  return m < NMK ? 1 : (m < NMK + NMV ? 2 : 0);
}
template <int NMK, int NMV, int L> __device__ constexpr int m_first_reads() {
  int r = 0;
  for (int m = 0; m < L; ++m) r += m_reads<NMK, NMV>(m);
  return r;
}
template <int NMK, int NMV, int L, int G, int I = 0>
__device__ __forceinline__ void m_phase_order() {
  if constexpr (I < NMK + NMV) {
    __builtin_amdgcn_sched_group_barrier(0x008, G, 0);        // the G MFMAs of one read
    constexpr int r = m_reads<NMK, NMV>(I + L);
    if constexpr (r > 0) __builtin_amdgcn_sched_group_barrier(0x100, r, 0);   // DS read
    m_phase_order<NMK, NMV, L, G, I + 1>();
  }
}

#ifndef OSP_M_LEAD
#define OSP_M_LEAD 4
#endif
#ifndef OSP_LEAD_EXPR
#define OSP_LEAD_EXPR (wave < NW / 2)
#define OSP_LEAD_RANK (wave % (NW / 2))
#endif

template <int D, int QB, int BN, int NW, int OCC, bool ROPE_Q, bool ROPE_K, bool FIXED_ROWS,
          bool PACKED>
__global__ __launch_bounds__(NW * 64, OCC) void attn3d_fwd_kernel(const AttnArgs a) {
  using C = AttnCfg<D, QB, BN, NW>;
  constexpr int NKB = BN / 32;        // 32-key blocks per tile
  // K and V tiles, three slots each (tile x in slot x % 3); separate arrays
  // so that the compiler can see that an LDS DMA into one slot does not
  // touch the slot being read
  __shared__ __attribute__((aligned(1024))) uint16_t k_s0[C::TILE];
  __shared__ __attribute__((aligned(1024))) uint16_t k_s1[C::TILE];
  __shared__ __attribute__((aligned(1024))) uint16_t k_s2[C::TILE];
  __shared__ __attribute__((aligned(1024))) uint16_t v_s0[C::TILE];
  __shared__ __attribute__((aligned(1024))) uint16_t v_s1[C::TILE];
  __shared__ __attribute__((aligned(1024))) uint16_t v_s2[C::TILE];
  auto kslot = [&](auto sl) __attribute__((always_inline)) -> uint16_t* {
    constexpr int S = decltype(sl)::value;
    if constexpr (S == 0) return k_s0; else if constexpr (S == 1) return k_s1; else return k_s2;
  };
  auto vslot = [&](auto sl) __attribute__((always_inline)) -> uint16_t* {
    constexpr int S = decltype(sl)::value;
    if constexpr (S == 0) return v_s0; else if constexpr (S == 1) return v_s1; else return v_s2;
  };
  __shared__ __attribute__((aligned(16))) RopeSmem<ROPE_Q || ROPE_K> rsm;
  RopeLds* const rl = rsm.get();

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const bool lead = OSP_LEAD_EXPR;   // leading half of the waves (they load)
  const int lw = OSP_LEAD_RANK;      // rank inside the half
  const int g = lane >> 5;      // half of the wave
  const int l32 = lane & 31;

  // ---- which tile: consecutive tiles of one (b, h, j) stay on one XCD ----
  // (workgroup x runs on XCD x mod 8; XCD c takes the c-th eighth of the tiles)
  const uint32_t total = uint32_t(a.total_tiles);
  const uint32_t t8 = total & ~7u;
  const uint32_t x = blockIdx.x;
  uint32_t u = (x < t8) ? (x & 7u) * (t8 >> 3) + (x >> 3) : x;

  // kernel arguments used below, as locals (keeps the argument block out of
  // private memory)
  RopeGeom rg = rope_scalars(a.rope);
  int32_t seq_len = a.seq_len, q_tiles = a.q_tiles;
  int64_t tok0 = 0;   // first token of the tile's sequence (packed launches)
  if constexpr (PACKED) {
    // the segment of workgroup x; every index is a constant (no dynamic
    // indexing into the argument block).  Each segment starts at a multiple
    // of 8 workgroups and is spread over the 8 XCDs on its own, as a whole
    // launch is above, so that segments of different cost do not load the
    // XCDs unevenly; its padding workgroups exit at once.
    PackSeg ps = a.pack[0];
#pragma unroll
    for (int sg = 1; sg < kMaxPackSegs; ++sg)
      if (sg < a.n_pack && x >= uint32_t(a.pack[sg].tile0)) ps = a.pack[sg];
    const uint32_t xs = x - uint32_t(ps.tile0);
    const uint32_t n8 = (uint32_t(ps.tiles) + 7u) >> 3;
    u = (xs & 7u) * n8 + (xs >> 3);
    if (u >= uint32_t(ps.tiles)) return;   // before any barrier
    seq_len = ps.seq_len;
    q_tiles = ps.q_tiles;
    tok0 = ps.start;
    rg.n_text = ps.n_text;
    rg.off1 = ps.off1;
    rg.off2 = ps.off2;
    rg.tab_entries = ps.tab_entries;
    rg.div_hw = ps.div_hw;
    rg.div_w = ps.div_w;
  }
  const uint32_t qt = u % uint32_t(q_tiles);
  u /= uint32_t(q_tiles);
  const uint32_t j = u % uint32_t(a.groups);
  u /= uint32_t(a.groups);
  const uint32_t h = u % uint32_t(a.heads);
  const uint32_t b = u / uint32_t(a.heads);

  // the fixed-row path serves only 1D modes, which the compiler then knows
  const int mode = FIXED_ROWS ? (a.mode & 3) : a.mode;
  const SkipDiv divk = a.divk;
  const int64_t a_sn = a.sn;

  const int L = seq_len;
  const int nkt = (L + BN - 1) / BN;
  const int64_t in_off = int64_t(b) * a.sb + int64_t(h) * a.sh + tok0 * a_sn;
  const uint16_t* __restrict__ qg = a.q + in_off;
  const uint16_t* __restrict__ kg = a.k + in_off;
  const uint16_t* __restrict__ vg = a.v + in_off;
  const float c2 = a.scale_log2;

  const bool fast_rope = rg.aligned8 && rg.tab_entries;

  // ---- Q^T operand: lane holds query (block, l32), channels 16c + 8g .. +7
  // (loaded in the prologue below)
  bf16x8_t qreg[QB][D / 16];

  // ---- loaders.  Tile kt's first row r0 = kt*BN maps to token i0(kt); the
  // remap is increasing in the row, and with FIXED_ROWS row r0 + row maps
  // to i0(kt) + drow(row), so per-lane byte offsets are fixed and only the
  // tile base moves.  K of tile kt goes to K slot kt&1, V to V slot kt&1.
  const int kmul = (mode == MODE_SINGLE || mode == MODE_GROUP) ? int(divk.d) : 1;
  auto drow_of = [&](int rw) __attribute__((always_inline)) -> uint32_t {
    const uint32_t r = uint32_t(rw);
    return (mode == MODE_FULL || mode == MODE_BLOCK) ? r
         : (mode == MODE_SINGLE) ? r * uint32_t(kmul)
         : (r / uint32_t(kmul)) * uint32_t(kmul * kmul) + r % uint32_t(kmul);
  };

  // DMA path: wave w of a half (rank lw) loads the blocks i = lw + LW*t,
  // t < DPW, of one tile (64 lanes x 16 bytes each).
  int32_t dm_off[C::DPW];
  int dm_row[C::DPW], dm_col[C::DPW];
#pragma unroll
  for (int t = 0; t < C::DPW; ++t) {
    const int p = 64 * (lw + C::LW * t) + lane;
    dm_row[t] = p / C::KCH;
    dm_col[t] = (p % C::KCH) ^ chunk_swz<D>(dm_row[t]);    // logical chunk
    dm_off[t] = int32_t((int64_t(drow_of(dm_row[t])) * a_sn + 8 * dm_col[t]) * 2);
  }
  // first token of tile kt: with FIXED_ROWS, i0(kt) = kt*BN*kmul + c_j
  const int64_t tile_c0 = (mode == MODE_SINGLE) ? int64_t(j)
                        : (mode == MODE_GROUP) ? int64_t(j) * kmul
                        : (mode == MODE_BLOCK) ? int64_t(j) * L : 0;
  auto tile_first = [&](int kt) __attribute__((always_inline)) -> uint32_t {
    if constexpr (FIXED_ROWS) return uint32_t(int64_t(kt) * BN * kmul + tile_c0);
    else return skiparse_token(mode, uint32_t(kt * BN), j, divk, uint32_t(L));
  };
  // Skiparse-2D rows: a tile's row dm_row[t] split once into (frames,
  // lattice rows, columns) of the (H/s) x (W/s) lattice, packed 10 bits
  // each (rows < 64), so that each tile's rows follow from its first row
  // by two carries instead of three divisions.
  const bool s2d = !FIXED_ROWS && mode >= MODE_SINGLE2D;
  const uint32_t lat_h = divk.gh / divk.axis.d;
  const uint32_t sn2 = uint32_t(a_sn) * 2u;
  uint32_t dm_lat[C::DPW];
#pragma unroll
  for (int t = 0; t < C::DPW; ++t) {
    const uint32_t d = uint32_t(dm_row[t]);
    const uint32_t dt = fdiv(d, divk.plane);
    const uint32_t rem = d - dt * divk.plane.d;
    const uint32_t dh = fdiv(rem, divk.row);
    dm_lat[t] = dt | (dh << 10) | ((rem - dh * divk.row.d) << 20);
  }
  // tile kt of the tensor at src into LDS tile dst (rows past the end read
  // as zeros: their offsets are out of the buffer's range)
  auto dma_tile = [&](const uint16_t* src, int kt, uint16_t* dst) __attribute__((always_inline)) {
    const uint32_t i0 = tile_first(kt);
    const __amdgpu_buffer_rsrc_t rs = __builtin_amdgcn_make_buffer_rsrc(
        const_cast<uint16_t*>(src + int64_t(i0) * a_sn), (short)0, kRecords, 0x00020000);
    // lattice position of the tile's first row, and the subsequence's (jh, jw)
    const uint32_t r0 = uint32_t(kt * BN);
    const uint32_t t0 = fdiv(r0, divk.plane);
    const uint32_t h0 = fdiv(r0 - t0 * divk.plane.d, divk.row);
    const uint32_t w0 = r0 - t0 * divk.plane.d - h0 * divk.row.d;
    const uint32_t jh = fdiv(j, divk.axis), jw = j - jh * divk.axis.d;
#pragma unroll
    for (int t = 0; t < C::DPW; ++t) {
      int32_t off = dm_off[t];
      if constexpr (!FIXED_ROWS) {
        if (s2d) {
          // rows past the end give some token here; their offset is replaced below
          uint32_t w = w0 + (dm_lat[t] >> 20);
          const uint32_t cw = w >= divk.row.d ? 1u : 0u;
          w -= cw * divk.row.d;
          uint32_t h = h0 + ((dm_lat[t] >> 10) & 1023u) + cw;
          const uint32_t ch = h >= lat_h ? 1u : 0u;
          h -= ch * lat_h;
          const uint32_t tt = t0 + (dm_lat[t] & 1023u) + ch;
          const bool grp = mode == MODE_GROUP2D;
          const uint32_t i = (tt * divk.gh + skip_axis(grp, h, jh, divk.axis)) * divk.gw +
                             skip_axis(grp, w, jw, divk.axis);
          off = int32_t((i - i0) * sn2 + 16u * uint32_t(dm_col[t]));
        } else {
          const uint32_t r = uint32_t(min(kt * BN + dm_row[t], L - 1));
          off = int32_t((int64_t(skiparse_token(mode, r, j, divk, uint32_t(L)) - i0) * a_sn + 8 * dm_col[t]) * 2);
        }
      }
      off = (dm_row[t] < L - kt * BN) ? off : kRecords;
      __builtin_amdgcn_raw_ptr_buffer_load_lds(rs, (lds_void_ptr)(dst + 512 * (lw + C::LW * t)), 16,
                                               off, 0, 0, 0);
    }
  };

  // Staged K path (K rotated in the loader): leading thread chunks
  // idx = lw*64 + lane + LT*e of the K tile.
  uint4 st_reg[ROPE_K ? C::SPT : 1];
  auto staged_issue = [&](int kt) __attribute__((always_inline)) {
#pragma unroll
    for (int e = 0; e < C::SPT; ++e) {
      const int idx = lw * 64 + lane + C::LT * e;
      const int row = idx / C::KCH, col = idx % C::KCH;
      const bool on = kt * BN + row < L;
      const uint32_t r = uint32_t(min(kt * BN + row, L - 1));
      const uint32_t i = skiparse_token(mode, r, j, divk, uint32_t(L));
      st_reg[e] = on ? ld16(kg + int64_t(i) * a_sn + 8 * col) : make_uint4(0, 0, 0, 0);
    }
  };
  auto staged_store = [&](int kt, uint16_t* dst) __attribute__((always_inline)) {
#pragma unroll
    for (int e = 0; e < C::SPT; ++e) {
      const int idx = lw * 64 + lane + C::LT * e;
      const int row = idx / C::KCH, col = idx % C::KCH;
      uint4 val = st_reg[e];
      const int r = kt * BN + row;
      const uint32_t i = skiparse_token(mode, uint32_t(min(r, L - 1)), j, divk, uint32_t(L));
      if (r < L && is_video(rg, i)) {
        const Coord3 cc = video_coords(rg, i);
        val = fast_rope ? rotate_chunk_col(rl, chunk_col(rg, 4 * col), cc, val)
                        : rotate_chunk_tab(rg, rl, 4 * col, cc, val);
      }
      *reinterpret_cast<uint4*>(dst + 8 * (row * C::KCH + (col ^ chunk_swz<D>(row)))) = val;
    }
  };

  // ---- accumulators and softmax state.  Scores are kept relative to the
  // row's reference maximum m (log2 units): the first product of each score
  // block starts from negm = -m instead of 0.
  f32x16_t o[QB][D / 32];
  f32x16_t negm[QB];
  float mref[QB], lsum[QB];
#pragma unroll
  for (int qb = 0; qb < QB; ++qb) {
    mref[qb] = 0.f;
    lsum[qb] = 0.f;
#pragma unroll
    for (int e = 0; e < 16; ++e) negm[qb][e] = 0.f;
#pragma unroll
    for (int db = 0; db < D / 32; ++db)
#pragma unroll
      for (int e = 0; e < 16; ++e) o[qb][db][e] = 0.f;
  }

  // per-lane LDS byte offsets of the operand reads (swizzle folded in)
  int k_off[D / 16];
  {
    const int hsw = g ^ chunk_swz<D>(l32);
#pragma unroll
    for (int c = 0; c < D / 16; ++c) k_off[c] = (l32 * C::KCH + ((2 * c) ^ hsw)) * 16;
  }
  int v_off[2][D / 32];
  {
    const int G = lane >> 4, s16 = lane & 15;
    const int ta = s16 & 3, te = s16 >> 2;
#pragma unroll
    for (int s = 0; s < 2; ++s)
#pragma unroll
      for (int db = 0; db < D / 32; ++db) {
        const int key = 4 * (G >> 1) + te + 8 * s;
        const int chunk = 4 * db + 2 * (G & 1) + (ta >> 1);
        v_off[s][db] = (key * C::KCH + (chunk ^ chunk_swz<D>(key))) * 16 + 8 * (ta & 1);
      }
  }

  // S^T - m of the K tile in slot SK into s; MASKED: keys of tile kt past
  // the end of the subsequence start from -inf instead
  auto qk = [&](auto slot, f32x16_t (&s)[NKB][QB], int kt, auto masked) __attribute__((always_inline)) {
    constexpr bool MASKED = decltype(masked)::value;
    const char* ks = reinterpret_cast<const char*>(kslot(slot));
#pragma unroll
    for (int kb = 0; kb < NKB; ++kb)
#pragma unroll
      for (int qb = 0; qb < QB; ++qb) {
        if constexpr (MASKED) {
#pragma unroll
          for (int e = 0; e < 16; ++e) {
            const int key = kt * BN + 32 * kb + 8 * (e >> 2) + 4 * g + (e & 3);
            s[kb][qb][e] = (key < L) ? negm[qb][e] : -INFINITY;
          }
        } else {
          s[kb][qb] = negm[qb];
        }
      }
#pragma unroll
    for (int c = 0; c < D / 16; ++c) {
#pragma unroll
      for (int kb = 0; kb < NKB; ++kb) {
        const bf16x8_t ka = *reinterpret_cast<const bf16x8_t*>(ks + 32 * kb * C::KCH * 16 + k_off[c]);
#pragma unroll
        for (int qb = 0; qb < QB; ++qb)
          s[kb][qb] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(ka, qreg[qb][c], s[kb][qb], 0, 0, 0);
      }
    }
  };
  // Probabilities of a tile as bf16 B operands, and their row sums ts.
  // The sums are plain fp32 adds in four independent partial sums:
  // dot-product instructions (v_dot2*) do not overlap with the other
  // wave's MFMAs the way ordinary VALU instructions do.
  auto probs = [&](const f32x16_t (&s)[NKB][QB], bf16x8_t (&pb)[QB][NKB][2], float (&ts)[QB])
      __attribute__((always_inline)) {
#pragma unroll
    for (int qb = 0; qb < QB; ++qb) {
      float acc[4];
#pragma unroll
      for (int kb = 0; kb < NKB; ++kb)
#pragma unroll
        for (int hh = 0; hh < 2; ++hh) {
          uint32_t w[4];
#pragma unroll
          for (int t = 0; t < 4; ++t) {
            const float p0 = __builtin_amdgcn_exp2f(s[kb][qb][8 * hh + 2 * t]);
            const float p1 = __builtin_amdgcn_exp2f(s[kb][qb][8 * hh + 2 * t + 1]);
            w[t] = pack_bf16(p0, p1);
            acc[t] = (kb == 0 && hh == 0) ? p0 + p1 : acc[t] + (p0 + p1);
          }
          pb[qb][kb][hh] = __builtin_bit_cast(bf16x8_t, make_uint4(w[0], w[1], w[2], w[3]));
        }
      ts[qb] = (acc[0] + acc[1]) + (acc[2] + acc[3]);
    }
  };
  // Softmax phase of a tile.  The probabilities are computed from the
  // scores as shifted by the current m.  m must be raised (and O, l
  // rescaled) only where a score exceeds kTau, and such a score alone
  // makes the lane's tile sum exceed 2^kTau; so the row maximum t is
  // reduced only in the branch taken when some lane's sum exceeds 2^kTau
  // (or on the row's first tile, which sets m to its maximum whatever its
  // sign).  There m is raised by t where t > kTau and the probabilities are
  // computed again from the newly shifted scores; the branch is rare after
  // the first tile, and any overflow of the first computation is discarded
  // with it.
  auto softmax_phase = [&](f32x16_t (&s)[NKB][QB], bf16x8_t (&pb)[QB][NKB][2], bool first)
      __attribute__((always_inline)) {
    float ts[QB];
    probs(s, pb, ts);
    // keep this computation ahead of the branch (the compiler would
    // otherwise sink it into the path that uses it, behind the max chain)
#pragma unroll
    for (int qb = 0; qb < QB; ++qb) {
      asm volatile("" : "+v"(ts[qb]));
#pragma unroll
      for (int kb = 0; kb < NKB; ++kb)
#pragma unroll
        for (int hh = 0; hh < 2; ++hh) {
          uint4 u = __builtin_bit_cast(uint4, pb[qb][kb][hh]);
          asm volatile("" : "+v"(u.x), "+v"(u.y), "+v"(u.z), "+v"(u.w));
          pb[qb][kb][hh] = __builtin_bit_cast(bf16x8_t, u);
        }
    }
    bool need = first;
#pragma unroll
    for (int qb = 0; qb < QB; ++qb) need |= !(ts[qb] <= kSumTau);
    if (__builtin_expect(__ballot(need) != 0, 0)) {
      asm volatile("" ::: "memory");
#pragma unroll
      for (int qb = 0; qb < QB; ++qb) {
        float mx = -INFINITY;
#pragma unroll
        for (int kb = 0; kb < NKB; ++kb)
#pragma unroll
          for (int e = 0; e < 16; ++e) mx = fmaxf(mx, s[kb][qb][e]);
        const float tmax = max_pair32(mx);
        const float dm = (first || tmax > kTau) ? tmax : 0.f;
        mref[qb] += dm;
        const float alpha = first ? 1.f : __builtin_amdgcn_exp2f(-dm);
        lsum[qb] *= alpha;
#pragma unroll
        for (int db = 0; db < D / 32; ++db)
#pragma unroll
          for (int e = 0; e < 16; ++e) o[qb][db][e] *= alpha;
#pragma unroll
        for (int kb = 0; kb < NKB; ++kb)
#pragma unroll
          for (int e = 0; e < 16; ++e) s[kb][qb][e] -= dm;
#pragma unroll
        for (int e = 0; e < 16; ++e) negm[qb][e] = -mref[qb];
      }
      probs(s, pb, ts);
    }
#pragma unroll
    for (int qb = 0; qb < QB; ++qb) lsum[qb] += ts[qb];
  };
  // O^T += V^T P^T for the V tile in slot SV; the V^T operand of keys
  // 32kb + 16hh .. +15 comes in the key order of the score rows.
  auto pv = [&](auto slot, bf16x8_t (&pb)[QB][NKB][2]) __attribute__((always_inline)) {
    const char* vs = reinterpret_cast<const char*>(vslot(slot));
#pragma unroll
    for (int kb = 0; kb < NKB; ++kb)
#pragma unroll
      for (int hh = 0; hh < 2; ++hh) {
        bf16x8_t va[D / 32];
        const char* blk = vs + (32 * kb + 16 * hh) * C::KCH * 16;
#pragma unroll
        for (int db = 0; db < D / 32; ++db) va[db] = tr_read<D>(blk, v_off, db);
#pragma unroll
        for (int db = 0; db < D / 32; ++db)
#pragma unroll
          for (int qb = 0; qb < QB; ++qb)
            o[qb][db] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(va[db], pb[qb][kb][hh], o[qb][db], 0, 0, 0);
      }
  };

  // Loads of one tile: the leading half loads K tiles, the trailing half V
  // tiles.  issue_tile starts them; finish_tile completes the staged
  // (rotating) K path.
  auto issue_tile = [&](int kt, auto slot) __attribute__((always_inline)) {
    if (lead) {
      if constexpr (ROPE_K) staged_issue(kt);
      else dma_tile(kg, kt, kslot(slot));
    } else {
      dma_tile(vg, kt, vslot(slot));
    }
  };
  auto finish_tile = [&](int kt, auto slot) __attribute__((always_inline)) {
    if constexpr (ROPE_K) {
      if (lead) staged_store(kt, kslot(slot));
    }
  };

  // ---- prologue, part 1.  Without K rotation in the loader the first two
  // K and V tiles are requested first, then the Q rows, so that all these
  // latencies overlap each other and the RoPE table.  The LDS barriers
  // here wait for LDS stores only, not for those loads.
  auto lds_barrier = [&]() __attribute__((always_inline)) {
    __builtin_amdgcn_s_waitcnt(0xC07F);   // lgkmcnt(0)
    __builtin_amdgcn_sched_barrier(0);
    asm volatile("s_barrier" ::: "memory");
    __builtin_amdgcn_sched_barrier(0);
  };
  // (the rate load is issued first: loads complete in order, so waiting
  // for it does not wait for the tiles or the Q rows behind it)
  static_assert(C::NT >= kMaxPairs, "one rate per thread");
  float omega = 0.f;
  if constexpr (ROPE_Q || ROPE_K) {
    if (tid < kMaxPairs) omega = a.rope.omega[tid];
    __builtin_amdgcn_sched_barrier(0);
  }
  if constexpr (!ROPE_K) {
    issue_tile(0, int_c<0>{});
    issue_tile(1, int_c<1>{});
  }
  // Q rows: every chunk is requested before any is used (a row past the end
  // reads the last row and is zeroed afterwards, so the loads need no
  // branch); the table is built while they are in flight.
  uint4 qraw[QB][D / 16];
#pragma unroll
  for (int qb = 0; qb < QB; ++qb) {
    const int r = int(qt) * C::BM + (wave * QB + qb) * 32 + l32;
    const uint32_t i = skiparse_token(mode, uint32_t(min(r, L - 1)), j, divk, uint32_t(L));
    const uint16_t* p = qg + int64_t(i) * a_sn;
#pragma unroll
    for (int c = 0; c < D / 16; ++c) qraw[qb][c] = ld16(p + 16 * c + 8 * g);
  }
  if constexpr (ROPE_Q || ROPE_K) {
    if (tid < kMaxPairs) rl->omega[tid] = omega;
    lds_barrier();
    fill_rope_table(rg, rl, tid, C::NT);
    lds_barrier();
  }
#pragma unroll
  for (int qb = 0; qb < QB; ++qb) {
    const int r = int(qt) * C::BM + (wave * QB + qb) * 32 + l32;
    const bool valid = r < L;
    const uint32_t i = skiparse_token(mode, uint32_t(valid ? r : 0), j, divk, uint32_t(L));
    const bool video = ROPE_Q && is_video(rg, i);
    const Coord3 cc = video_coords(rg, i);
#pragma unroll
    for (int c = 0; c < D / 16; ++c) {
      uint4 raw = valid ? qraw[qb][c] : make_uint4(0, 0, 0, 0);
      // times scale * log2(e) so that the score products come out in log2
      // units; a rotated row is rotated and scaled in fp32, rounded once
      if (ROPE_Q && video) {
        raw = fast_rope ? rotate_chunk_col_scaled(rl, chunk_col(rg, 8 * c + 4 * g), cc, raw, c2)
                        : rotate_chunk_scaled(rg, rl, 8 * c + 4 * g, cc, raw, c2);
      } else {
        raw.x = pack_bf16(bf16lo(raw.x) * c2, bf16hi(raw.x) * c2);
        raw.y = pack_bf16(bf16lo(raw.y) * c2, bf16hi(raw.y) * c2);
        raw.z = pack_bf16(bf16lo(raw.z) * c2, bf16hi(raw.z) * c2);
        raw.w = pack_bf16(bf16lo(raw.w) * c2, bf16hi(raw.w) * c2);
      }
      qreg[qb][c] = __builtin_bit_cast(bf16x8_t, raw);
    }
  }

  // ---- ping-pong schedule.  The waves form two halves, one wave of each
  // on every SIMD.  Per key tile t a wave runs a matrix phase M(t) (S(t) =
  // K(t) Q^T, then O += P(t-1) V(t-1)) and a softmax phase V(t) (max,
  // rescale, exp2, row sums of S(t) into P), each ended by a workgroup
  // barrier.  The trailing half passes one barrier first and so runs one
  // phase behind: on each SIMD one wave's MFMAs overlap the other wave's
  // softmax.
  //
  // Loads: tile x of K and V lives in slot x % 3.  In its softmax phase
  // for tile t each wave of the leading half issues its share of K(t+2),
  // each wave of the trailing half its share of V(t+2); the tiles they
  // replace, K(t-1) and V(t-1), were last read in earlier phases.  At the
  // end of that phase a wave waits for its loads of the previous iteration
  // only (K(t+1) or V(t+1)), at least one phase before their first
  // reader, so each load has two phases or more to arrive.  The tile count
  // is padded to a multiple of 3 with tiles past the end of the
  // subsequence (keys masked to -inf, loads out of range of the buffer,
  // which read as zeros), so that every slot index is a compile-time
  // constant.
  const bool ragged = (L % BN) != 0;
  const int nkt3 = (nkt + 2) / 3 * 3;
  f32x16_t s[NKB][QB];
  bf16x8_t pb[QB][NKB][2];

  auto barrier = [&]() __attribute__((always_inline)) {
    __builtin_amdgcn_sched_barrier(0);
    asm volatile("s_barrier" ::: "memory");
    __builtin_amdgcn_sched_barrier(0);
  };
  // Wait for all but this iteration's DPW loads (vmcnt(DPW)); the leading
  // half on the staged path has just stored its tile and waits for all
  // (vmcnt(0) lgkmcnt(0)).  The compiler tracks these waits, so it knows
  // which slots are complete.
  auto loads_done = [&]() __attribute__((always_inline)) {
    __builtin_amdgcn_sched_barrier(0);
    if (ROPE_K && lead) __builtin_amdgcn_s_waitcnt(0x0070);
    else __builtin_amdgcn_s_waitcnt((C::DPW & 15) | ((C::DPW >> 4) << 14) | 0x0F70);
  };
  // matrix phase of tile t: QK(t) from K slot P (QK) and PV(t-1) from V
  // slot (P + 2) % 3 (PV).  Instruction order inside it (one query block
  // per wave): the LDS reads run OSP_M_LEAD MFMAs ahead of the MFMAs that
  // use them.  With two blocks the compiler's own order was as fast.
  auto m_phase = [&](int t, auto slot, auto do_qk, auto do_pv, auto masked) __attribute__((always_inline)) {
    constexpr int P = decltype(slot)::value;
    constexpr bool QK = decltype(do_qk)::value, PV = decltype(do_pv)::value;
    __builtin_amdgcn_s_setprio(1);
    if constexpr (QK) qk(int_c<P>{}, s, t, masked);
    if constexpr (PV) pv(int_c<(P + 2) % 3>{}, pb);
    if constexpr (QB == 1) {
      constexpr int NMV = PV ? NKB * 2 * (D / 32) : 0, NMK = QK ? NKB * (D / 16) : 0;
      __builtin_amdgcn_sched_group_barrier(0x100, m_first_reads<NMK, NMV, OSP_M_LEAD>(), 0);
      m_phase_order<NMK, NMV, OSP_M_LEAD, QB>();
    }
    __builtin_amdgcn_s_setprio(0);
  };
  // tiles from tu on hold keys past the end (the last real tile when
  // ragged, and the padding); whole groups before tu run unmasked
  const int tu = nkt - (ragged ? 1 : 0);
  // one iteration (two phases) for tile t in slot P = t % 3; MASKED: mask
  // keys past the end (correct for any tile; used for the last groups)
  auto iter = [&](int t, auto slot, auto masked) __attribute__((always_inline)) {
    constexpr int P = decltype(slot)::value;
    m_phase(t, slot, bool_c<true>{}, bool_c<true>{}, masked);
    barrier();
    issue_tile(t + 2, int_c<(P + 2) % 3>{});
    softmax_phase(s, pb, t == 0);
    finish_tile(t + 2, int_c<(P + 2) % 3>{});
    loads_done();
    barrier();
  };

  // prologue, part 2: K(0), K(1), V(0), V(1) into slots 0 and 1 (with K
  // rotation in the loader: here); V slot 2 (read as "V(-1)" by the first
  // matrix phase, with P = 0) cleared
  for (int e = tid; e < C::TILE / 8; e += C::NT)
    reinterpret_cast<uint4*>(v_s2)[e] = make_uint4(0, 0, 0, 0);
#pragma unroll
  for (int qb = 0; qb < QB; ++qb)
#pragma unroll
    for (int kb = 0; kb < NKB; ++kb) {
      pb[qb][kb][0] = bf16x8_t{};
      pb[qb][kb][1] = bf16x8_t{};
    }
  if constexpr (ROPE_K) {
    issue_tile(0, int_c<0>{});
    finish_tile(0, int_c<0>{});
    issue_tile(1, int_c<1>{});
    finish_tile(1, int_c<1>{});
  }
  __syncthreads();
  if (!lead) barrier();
  int t = 0;
  for (; t + 3 <= tu; t += 3) {
    iter(t, int_c<0>{}, bool_c<false>{});
    iter(t + 1, int_c<1>{}, bool_c<false>{});
    iter(t + 2, int_c<2>{}, bool_c<false>{});
  }
  for (; t < nkt3; t += 3) {
    iter(t, int_c<0>{}, bool_c<true>{});
    iter(t + 1, int_c<1>{}, bool_c<true>{});
    iter(t + 2, int_c<2>{}, bool_c<true>{});
  }
  // the last matrix phase: PV of tile nkt3 - 1 (V slot 2)
  m_phase(nkt3, int_c<0>{}, bool_c<false>{}, bool_c<true>{}, bool_c<false>{});
  if (lead) barrier();   // the trailing half's last barrier
  // loads of the padding tiles past nkt3 may still be writing LDS: finish
  // them before the workgroup's LDS is released
  __builtin_amdgcn_s_waitcnt(0x0070);

  // ---- epilogue: O = O^T / l, stored at the original token row ----
  uint16_t* og = a.o + int64_t(b) * a.osb + int64_t(h) * a.osh + tok0 * a.osn;
  float* const lse_out = a.lse ? a.lse + tok0 : nullptr;
#pragma unroll
  for (int qb = 0; qb < QB; ++qb) {
    const float lt = sum_pair32(lsum[qb]);
    const float inv = 1.0f / lt;
    const int r = int(qt) * C::BM + (wave * QB + qb) * 32 + l32;
    if (r < L) {
      const uint32_t i = skiparse_token(mode, uint32_t(r), j, divk, uint32_t(L));
      uint16_t* p = og + int64_t(i) * a.osn;
#pragma unroll
      for (int db = 0; db < D / 32; ++db)
#pragma unroll
        for (int r4 = 0; r4 < 4; ++r4) {
          const uint32_t w0 = pack_bf16(o[qb][db][4 * r4 + 0] * inv, o[qb][db][4 * r4 + 1] * inv);
          const uint32_t w1 = pack_bf16(o[qb][db][4 * r4 + 2] * inv, o[qb][db][4 * r4 + 3] * inv);
          *reinterpret_cast<uint2*>(p + 32 * db + 8 * r4 + 4 * g) = make_uint2(w0, w1);
        }
      if (lse_out && g == 0)
        lse_out[(int64_t(b) * a.heads + h) * a.lse_ld + i] = (mref[qb] + __log2f(lt)) * kLn2;
    }
  }
}

// Tile shape per head_dim: 32-row query blocks per wave (QB), keys per
// tile (BN), waves per workgroup (NW), waves per SIMD (OCC).  Build-time
// overridable for tuning.
// D=64: two 32-row query blocks per wave over 32-key tiles; each K or V
// fragment read from LDS then feeds two MFMAs, and the matrix phase is as
// long as at D=128 with half the registers per block (7% faster on
// CogVideoX's 17,776 tokens than one block over 64-key tiles)
#ifndef OSP_D64_TILE
#define OSP_D64_TILE 2, 32, 8, 2
#endif
#ifndef OSP_D96_TILE
#define OSP_D96_TILE 1, 64, 8, 2
#endif
#ifndef OSP_D128_TILE
#define OSP_D128_TILE 1, 64, 8, 2
#endif
// D=128 with K rotated in the loader: 64-key tiles spill, 32 do not
#ifndef OSP_D128_ROPE_K_TILE
#define OSP_D128_ROPE_K_TILE 1, 32, 8, 2
#endif
template <int QB_, int BN_, int NW_, int OCC_> struct TileShape {
  static constexpr int QB = QB_, BN = BN_, NW = NW_, OCC = OCC_;
};
template <int D, bool RK> struct TileCfg;
template <bool RK> struct TileCfg<64, RK> : TileShape<OSP_D64_TILE> {};
template <bool RK> struct TileCfg<96, RK> : TileShape<OSP_D96_TILE> {};
template <> struct TileCfg<128, false> : TileShape<OSP_D128_TILE> {};
template <> struct TileCfg<128, true> : TileShape<OSP_D128_ROPE_K_TILE> {};

template <int D> constexpr int max_keys_per_tile() {
  return TileCfg<D, false>::BN > TileCfg<D, true>::BN ? TileCfg<D, false>::BN : TileCfg<D, true>::BN;
}
int attn_keys_per_tile(int head_dim) {
  switch (head_dim) {
    case 64: return max_keys_per_tile<64>();
    case 96: return max_keys_per_tile<96>();
    case 128: return max_keys_per_tile<128>();
    default: return 0;
  }
}

// (rows per workgroup are the same with and without K rotation)
int attn_rows_per_block(int head_dim) {
  switch (head_dim) {
    case 64: return TileCfg<64, false>::NW * 32 * TileCfg<64, false>::QB;
    case 96: return TileCfg<96, false>::NW * 32 * TileCfg<96, false>::QB;
    case 128: return TileCfg<128, false>::NW * 32 * TileCfg<128, false>::QB;
    default: return 0;
  }
}
static_assert(TileCfg<128, false>::NW * TileCfg<128, false>::QB ==
              TileCfg<128, true>::NW * TileCfg<128, true>::QB, "rows per workgroup");

template <int D, bool RQ, bool RK, bool PK>
static hipError_t launch_drk(const AttnArgs& a, hipStream_t s) {
  using T = TileCfg<D, RK>;
  dim3 grid(a.total_tiles), block(T::NW * 64);
  const bool fixed = a.mode <= MODE_BLOCK && (a.mode != MODE_GROUP || T::BN % int(a.divk.d) == 0);
  if (fixed)
    hipLaunchKernelGGL((attn3d_fwd_kernel<D, T::QB, T::BN, T::NW, T::OCC, RQ, RK, true, PK>),
                       grid, block, 0, s, a);
  else
    hipLaunchKernelGGL((attn3d_fwd_kernel<D, T::QB, T::BN, T::NW, T::OCC, RQ, RK, false, PK>),
                       grid, block, 0, s, a);
  return hipGetLastError();
}

template <int D, bool PK>
static hipError_t launch_d(const AttnArgs& a, int rope_q, int rope_k, hipStream_t s) {
  if (rope_q && rope_k) return launch_drk<D, true, true, PK>(a, s);
  if (rope_q) return launch_drk<D, true, false, PK>(a, s);
  if (rope_k) return launch_drk<D, false, true, PK>(a, s);
  return launch_drk<D, false, false, PK>(a, s);
}

hipError_t launch_attn3d(AttnArgs& a, int head_dim, int rope_q, int rope_k, hipStream_t s) {
  if (a.seq_len <= kShortRows) return launch_attn3d_short(a, head_dim, rope_q, rope_k, s);
  switch (head_dim) {
    case 64: return launch_d<64, false>(a, rope_q, rope_k, s);
    case 96: return launch_d<96, false>(a, rope_q, rope_k, s);
    case 128: return launch_d<128, false>(a, rope_q, rope_k, s);
    default: return hipErrorInvalidValue;
  }
}

hipError_t launch_attn3d_packed(const AttnArgs& a, int head_dim, int rope_q, int rope_k,
                                hipStream_t s) {
  switch (head_dim) {
    case 64: return launch_d<64, true>(a, rope_q, rope_k, s);
    case 96: return launch_d<96, true>(a, rope_q, rope_k, s);
    case 128: return launch_d<128, true>(a, rope_q, rope_k, s);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace osp
