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
#include <atomic>
#include <type_traits>
#include <utility>

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

// Calls f(int_c<0>), ..., f(int_c<N-1>) in order.
template <typename F, int... I>
__device__ __forceinline__ void for_slots(F&& f, std::integer_sequence<int, I...>) {
  (f(int_c<I>{}), ...);
}

// NS: LDS slots per K and V tile (3 to 6): tile x lives in slot x % NS and
// is requested NS - 1 tiles ahead of its use.
// TAB (per-row remap only): the remap of a subsequence differs from that of
// subsequence 0 by a constant, token(r, j) = token(r, 0) + token(0, j)
// (Group Skip: j*k; Skiparse-2D: jh*W + jw, times s for group), so the
// workgroup tabulates token(r, 0) for its L rows once, in dynamic LDS, and
// the loader looks rows up instead of dividing.
// PERSIST: the grid holds one workgroup per slot the chip can run at once,
// and each workgroup walks its XCD's list of query tiles (see "which tiles"
// below) instead of taking one: the RoPE and row tables are built once,
// and the first K/V tiles and the Q rows of the next query tile are
// requested while the current one finishes.
template <int D, int QB, int BN, int NW, int OCC, int NS, bool ROPE_Q, bool ROPE_K,
          bool FIXED_ROWS, bool PACKED, bool TAB, bool PERSIST>
__global__ __launch_bounds__(NW * 64, OCC) void attn3d_fwd_kernel(const AttnArgs a) {
  static_assert(!TAB || !FIXED_ROWS, "the row table serves the per-row remap");
  static_assert(!PERSIST || (!PACKED && !ROPE_K), "persistent launches: plain calls, K rotated before");
  extern __shared__ __attribute__((aligned(16))) uint32_t row_tab[];   // TAB: L entries
  using C = AttnCfg<D, QB, BN, NW>;
  constexpr int NKB = BN / 32;        // 32-key blocks per tile
  static_assert(NS >= 3 && NS <= 6, "three to six tile slots");
  // K and V tiles, NS slots each; separate arrays so that the compiler can
  // see that an LDS DMA into one slot does not touch the slot being read.
  // The last slot of K and of V share one array, which also holds the RoPE
  // cos/sin table while Q is rotated in the prologue (when K is not
  // rotated in the loader, the table is used nowhere else); it is at least
  // a RopeLds long.  A persistent workgroup rotates the Q rows of every
  // tile it takes, so there the table has an array of its own.
  constexpr bool kOwnTable = ROPE_K || (ROPE_Q && PERSIST);
  constexpr int kSL = (ROPE_Q && !kOwnTable && 2 * C::TILE * 2 < int(sizeof(RopeLds)))
                          ? int((sizeof(RopeLds) + 1) / 2) : 2 * C::TILE;
  // (slots 2 .. 4 that are not used, or are the last, take 8 elements)
  constexpr int kT2 = NS > 3 ? C::TILE : 8, kT3 = NS > 4 ? C::TILE : 8, kT4 = NS > 5 ? C::TILE : 8;
  __shared__ __attribute__((aligned(1024))) uint16_t k_s0[C::TILE];
  __shared__ __attribute__((aligned(1024))) uint16_t k_s1[C::TILE];
  __shared__ __attribute__((aligned(1024))) uint16_t k_s2[kT2];
  __shared__ __attribute__((aligned(1024))) uint16_t k_s3[kT3];
  __shared__ __attribute__((aligned(1024))) uint16_t k_s4[kT4];
  __shared__ __attribute__((aligned(1024))) uint16_t v_s0[C::TILE];
  __shared__ __attribute__((aligned(1024))) uint16_t v_s1[C::TILE];
  __shared__ __attribute__((aligned(1024))) uint16_t v_s2[kT2];
  __shared__ __attribute__((aligned(1024))) uint16_t v_s3[kT3];
  __shared__ __attribute__((aligned(1024))) uint16_t v_s4[kT4];
  __shared__ __attribute__((aligned(1024))) uint16_t kv_sl[kSL];
  auto kslot = [&](auto sl) __attribute__((always_inline)) -> uint16_t* {
    constexpr int S = decltype(sl)::value;
    if constexpr (S == NS - 1) return kv_sl;
    else if constexpr (S == 0) return k_s0; else if constexpr (S == 1) return k_s1;
    else if constexpr (S == 2) return k_s2; else if constexpr (S == 3) return k_s3;
    else return k_s4;
  };
  auto vslot = [&](auto sl) __attribute__((always_inline)) -> uint16_t* {
    constexpr int S = decltype(sl)::value;
    if constexpr (S == NS - 1) return kv_sl + C::TILE;
    else if constexpr (S == 0) return v_s0; else if constexpr (S == 1) return v_s1;
    else if constexpr (S == 2) return v_s2; else if constexpr (S == 3) return v_s3;
    else return v_s4;
  };
  // K rotated in the loader reads the table in every tile: its own array
  __shared__ __attribute__((aligned(16))) RopeSmem<kOwnTable> rsm;
  RopeLds* const rl = kOwnTable ? rsm.get() : ROPE_Q ? reinterpret_cast<RopeLds*>(kv_sl) : nullptr;

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const bool lead = OSP_LEAD_EXPR;   // leading half of the waves (they load)
  const int lw = OSP_LEAD_RANK;      // rank inside the half
  const int g = lane >> 5;      // half of the wave
  const int l32 = lane & 31;

  // ---- which tiles: consecutive tiles of one (b, h, j) stay on one XCD ----
  // Workgroup x runs on XCD x mod 8.  XCD c takes the c-th eighth of the
  // tiles (the last total mod 8 tiles go one to each of the first XCDs),
  // and its workgroups take that list in order: workgroup x the entry
  // x / 8, a persistent one every (grid / 8)-th entry from there.
  const uint32_t total = uint32_t(a.total_tiles);
  const uint32_t t8 = total & ~7u, q8 = t8 >> 3;
  const uint32_t x = blockIdx.x;
  const uint32_t xcd = x & 7u;
  uint32_t wn = x >> 3;
  if (PERSIST && wn >= q8 + (xcd < (total & 7u) ? 1u : 0u)) return;   // (not launched so)
  uint32_t u = wn < q8 ? xcd * q8 + wn : t8 + xcd;

  // The argument block, for values read once per tile.  A persistent
  // workgroup reads it through a pointer the compiler cannot see through,
  // so that such values are read again at each tile instead of being held
  // in registers through the tile loop.
  auto args = [&]() __attribute__((always_inline)) -> const AttnArgs* {
    auto p = (const __attribute__((address_space(4))) AttnArgs*)__builtin_amdgcn_kernarg_segment_ptr();
    if constexpr (PERSIST) asm volatile("" : "+s"(p));
    return (const AttnArgs*)p;
  };

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
  // (query tile, subsequence, head, batch) of tile w
  struct TileId {
    uint32_t qt, j, h, b;
  };
  auto decode = [&](uint32_t w) __attribute__((always_inline)) {
    const AttnArgs* A = args();
    const uint32_t nq = PACKED ? uint32_t(q_tiles) : uint32_t(A->q_tiles);
    TileId r;
    r.qt = w % nq;
    w /= nq;
    r.j = w % uint32_t(A->groups);
    w /= uint32_t(A->groups);
    r.h = w % uint32_t(A->heads);
    r.b = w / uint32_t(A->heads);
    return r;
  };
  uint32_t ucur = u;                   // the current tile
  const uint32_t jcur = decode(u).j;   // its subsequence (one-tile workgroups)

  // the fixed-row path serves only 1D modes, which the compiler then knows
  const int mode = FIXED_ROWS ? (a.mode & 3) : a.mode;
  const SkipDiv divk = a.divk;
  const int64_t a_sn = a.sn;

  const int L = seq_len;
  const int nkt = (L + BN - 1) / BN;
  // element offset of tile w's (batch, head) in q, k and v
  auto in_off = [&](uint32_t w) __attribute__((always_inline)) {
    const TileId t = decode(w);
    const AttnArgs* A = args();
    return int64_t(t.b) * A->sb + int64_t(t.h) * A->sh + tok0 * a_sn;
  };
  // K and V at the tile's (batch, head) (one-tile workgroups)
  const uint16_t* kg = a.k + in_off(ucur);
  const uint16_t* vg = a.v + in_off(ucur);
  // tiles of one query tile, padded to a multiple of the slot count (see
  // the schedule below)
  const bool ragged = (L % BN) != 0;
  const int nkt3 = (nkt + NS - 1) / NS * NS;

  const bool fast_rope = rg.aligned8 && rg.tab_entries;

  // ---- Q^T operand: lane holds query (block, l32), channels 16c + 8g .. +7
  // (loaded in the prologue below)
  bf16x8_t qreg[QB][D / 16];

  // ---- loaders.  Tile kt's first row r0 = kt*BN maps to token i0(kt); the
  // remap is increasing in the row, and with FIXED_ROWS row r0 + row maps
  // to i0(kt) + drow(row), so per-lane byte offsets are fixed and only the
  // tile base moves.  K of tile kt goes to K slot kt&1, V to V slot kt&1.
  const int kmul = (mode == MODE_SINGLE || mode == MODE_GROUP) ? int(divk.d) : 1;
  auto drow_of = [mode, kmul](int rw) __attribute__((always_inline)) -> uint32_t {
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
  // first token of tile kt of subsequence jj: with FIXED_ROWS, i0(kt) =
  // kt*BN*kmul + c_jj
  auto tile_first = [mode, kmul, L, divk](int kt, uint32_t jj) __attribute__((always_inline))
      -> uint32_t {
    if constexpr (FIXED_ROWS) {
      const int64_t c0 = (mode == MODE_SINGLE) ? int64_t(jj)
                       : (mode == MODE_GROUP) ? int64_t(jj) * kmul
                       : (mode == MODE_BLOCK) ? int64_t(jj) * L : 0;
      return uint32_t(int64_t(kt) * BN * kmul + c0);
    } else {
      return skiparse_token(mode, uint32_t(kt * BN), jj, divk, uint32_t(L));
    }
  };
  // Skiparse-2D rows: a tile's row dm_row[t] split once into (frames,
  // lattice rows, columns) of the (H/s) x (W/s) lattice, packed 10 bits
  // each (rows < 64), so that each tile's rows follow from its first row
  // by two carries instead of three divisions.
  const bool s2d = !FIXED_ROWS && !TAB && mode >= MODE_SINGLE2D;
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
  // TAB: token(0, jj), subsequence jj's offset from the table's tokens
  auto tab_cj = [&](uint32_t jj) __attribute__((always_inline)) {
    return TAB ? skiparse_token(mode, 0u, jj, divk, uint32_t(L)) : 0u;
  };
  // tile kt of the tensor at src into LDS tile dst (rows past the end read
  // as zeros: their offsets are out of the buffer's range).  USE_TAB: rows
  // from the row table (built in the prologue, after the first tiles are
  // requested)
  // The table entries of a tile (its first row, then this lane's rows) are
  // read one tile ahead: each half requests consecutive tiles, one per
  // iteration, so the entries of the next are read right after a tile is
  // requested and have arrived when it is its turn (fetch_kt: the next
  // request's tile, in its own subsequence).
  uint32_t tab_nx[C::DPW + 1];
  auto tab_fetch = [&](int kt) __attribute__((always_inline)) {
    const uint32_t r0 = uint32_t(kt * BN);
    tab_nx[0] = row_tab[min(r0, uint32_t(L - 1))];
#pragma unroll
    for (int t = 0; t < C::DPW; ++t)
      tab_nx[t + 1] = row_tab[min(r0 + uint32_t(dm_row[t]), uint32_t(L - 1))];
  };
  // The DMA descriptor's base address is the same in every lane.  Where the
  // compiler cannot prove it, it wraps each DMA in a loop over the distinct
  // values.  The persistent instances at head_dim 64 and 128 hold the
  // stream base in vector registers and got such loops in the key loop;
  // there the address is read from the first lane, which tells the
  // compiler.  Elsewhere that read moves the address arithmetic to vector
  // instructions and measured 1-2% slower (no such loop in their key
  // loops), so it is left out.
  auto wave_ptr = [](const uint16_t* p) __attribute__((always_inline)) {
    if constexpr (PERSIST && D != 96) {
      const uint64_t v = reinterpret_cast<uint64_t>(p);
      const uint32_t lo = __builtin_amdgcn_readfirstlane(uint32_t(v));
      const uint32_t hi = __builtin_amdgcn_readfirstlane(uint32_t(v >> 32));
      return reinterpret_cast<uint16_t*>((uint64_t(hi) << 32) | lo);
    } else {
      return const_cast<uint16_t*>(p);
    }
  };
  auto dma_tile_tab = [&](const uint16_t* src, int kt, uint16_t* dst, uint32_t cj, int fetch_kt)
      __attribute__((always_inline)) {
    const uint32_t base = tab_nx[0];
    const __amdgpu_buffer_rsrc_t rs = __builtin_amdgcn_make_buffer_rsrc(
        wave_ptr(src + int64_t(base + cj) * a_sn), (short)0, kRecords, 0x00020000);
#pragma unroll
    for (int t = 0; t < C::DPW; ++t) {
      int32_t off = int32_t((tab_nx[t + 1] - base) * sn2 + 16u * uint32_t(dm_col[t]));
      off = (dm_row[t] < L - kt * BN) ? off : kRecords;
      __builtin_amdgcn_raw_ptr_buffer_load_lds(rs, (lds_void_ptr)(dst + 512 * (lw + C::LW * t)), 16,
                                               off, 0, 0, 0);
    }
    tab_fetch(fetch_kt);
  };
  auto dma_tile = [&](const uint16_t* src, int kt, uint16_t* dst, uint32_t jj)
      __attribute__((always_inline)) {
    const uint32_t i0 = tile_first(kt, jj);
    const __amdgpu_buffer_rsrc_t rs = __builtin_amdgcn_make_buffer_rsrc(
        wave_ptr(src + int64_t(i0) * a_sn), (short)0, kRecords, 0x00020000);
    // lattice position of the tile's first row, and the subsequence's (jh, jw)
    const uint32_t r0 = uint32_t(kt * BN);
    const uint32_t t0 = fdiv(r0, divk.plane);
    const uint32_t h0 = fdiv(r0 - t0 * divk.plane.d, divk.row);
    const uint32_t w0 = r0 - t0 * divk.plane.d - h0 * divk.row.d;
    const uint32_t jh = fdiv(jj, divk.axis), jw = jj - jh * divk.axis.d;
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
          off = int32_t((int64_t(skiparse_token(mode, r, jj, divk, uint32_t(L)) - i0) * a_sn + 8 * dm_col[t]) * 2);
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
      const uint32_t i = skiparse_token(mode, r, jcur, divk, uint32_t(L));
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
      const uint32_t i = skiparse_token(mode, uint32_t(min(r, L - 1)), jcur, divk, uint32_t(L));
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
  auto init_acc = [&]() __attribute__((always_inline)) {
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
  };

  // per-lane LDS byte offsets of the operand reads (swizzle folded in)
  const RowOff<D> k_off(lane);
  const TrOff<D> v_off(lane);

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
        const bf16x8_t ka = *reinterpret_cast<const bf16x8_t*>(ks + 32 * kb * C::KCH * 16 + k_off(c));
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
  // (rotating) K path.  Requests kt >= nkt3 are the padding of the last
  // group; a persistent workgroup with a next tile requests that tile's
  // tiles 0, 1, ... there instead (into the same slots, nkt3 being a
  // multiple of NS).
  //
  // A persistent workgroup keeps, per wave, one base sb for the tensor the
  // wave loads (K in the leading half, V in the trailing half) with the
  // subsequence's offset folded in (c_j with fixed rows, token(0, j) with
  // the row table; both instances take subsequence 0's offsets from
  // there).  It moves to the next tile's at that tile's first request.
  // (The base is formed there rather than chosen between two variables:
  // a run-time choice between two variables these lambdas capture by
  // reference becomes a load at a computed offset into the capture block,
  // which the compiler then keeps in scratch memory, with everything it
  // points to.)
  const uint32_t cj_cur = tab_cj(jcur);
  auto stream_base = [&](uint32_t w) __attribute__((always_inline)) -> const uint16_t* {
    const AttnArgs* A = args();
    const uint32_t jj = decode(w).j;
    const int64_t c = FIXED_ROWS ? int64_t(tile_first(0, jj)) : int64_t(tab_cj(jj));
    return (lead ? A->k : A->v) + in_off(w) + c * a_sn;
  };
  bool has_next = false;
  uint32_t unxt = ucur;
  const uint16_t* sb = nullptr;
  if constexpr (PERSIST) sb = stream_base(ucur);
  // NEAR_END: kt may reach nkt3 (the loop's last two groups); earlier
  // groups request the current tile's tiles only
  auto issue_tile = [&](int kt, auto slot, auto near_end) __attribute__((always_inline)) {
    if constexpr (PERSIST && !decltype(near_end)::value) {
      if constexpr (TAB) {
        if (lead) dma_tile_tab(sb, kt, kslot(slot), 0u, kt + 1);
        else dma_tile_tab(sb, kt, vslot(slot), 0u, kt + 1);
      } else {
        if (lead) dma_tile(sb, kt, kslot(slot), 0u);
        else dma_tile(sb, kt, vslot(slot), 0u);
      }
    } else if constexpr (PERSIST) {
      const bool nx = has_next && kt >= nkt3;
      if (has_next && kt == nkt3) sb = stream_base(unxt);
      const int kk = nx ? kt - nkt3 : kt;
      const int fetch = (has_next && kt + 1 >= nkt3) ? kt + 1 - nkt3 : kt + 1;
      if constexpr (TAB) {
        if (lead) dma_tile_tab(sb, kk, kslot(slot), 0u, fetch);
        else dma_tile_tab(sb, kk, vslot(slot), 0u, fetch);
      } else {
        if (lead) dma_tile(sb, kk, kslot(slot), 0u);
        else dma_tile(sb, kk, vslot(slot), 0u);
      }
    } else if (lead) {
      if constexpr (ROPE_K) staged_issue(kt);
      else if constexpr (TAB) dma_tile_tab(kg, kt, kslot(slot), cj_cur, kt + 1);
      else dma_tile(kg, kt, kslot(slot), jcur);
    } else {
      if constexpr (TAB) dma_tile_tab(vg, kt, vslot(slot), cj_cur, kt + 1);
      else dma_tile(vg, kt, vslot(slot), jcur);
    }
  };
  // the first tile's first tiles, requested before the row table exists
  auto issue_tile_first = [&](int kt, auto slot) __attribute__((always_inline)) {
    if (lead) {
      if constexpr (ROPE_K) staged_issue(kt);
      else dma_tile(kg, kt, kslot(slot), jcur);
    } else {
      dma_tile(vg, kt, vslot(slot), jcur);
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
    for_slots([&](auto sl) __attribute__((always_inline)) {
      if constexpr (decltype(sl)::value < NS - 1) issue_tile_first(decltype(sl)::value, sl);
    }, std::make_integer_sequence<int, NS>{});
  }
  // Q rows: every chunk is requested before any is used (a row past the end
  // reads the last row and is zeroed afterwards, so the loads need no
  // branch); the tables are built while they are in flight.
  uint4 qraw[QB][D / 16];
  // Lane coordinates formed again where a persistent workgroup uses them
  // once per tile, so that the compiler does not hold what it derives from
  // them through the tile loop.
  auto lane_ids = [&](int& l, int& gg) __attribute__((always_inline)) {
    int x = lane;
    if constexpr (PERSIST) asm volatile("" : "+v"(x));
    l = x & 31;
    gg = x >> 5;
  };
  auto load_q = [&](uint32_t w) __attribute__((always_inline)) {
    const TileId tl = decode(w);
    const uint16_t* qsrc = args()->q + in_off(w);
    int lq, gq;
    lane_ids(lq, gq);
#pragma unroll
    for (int qb = 0; qb < QB; ++qb) {
      const int r = int(tl.qt) * C::BM + (wave * QB + qb) * 32 + lq;
      const uint32_t i = skiparse_token(mode, uint32_t(min(r, L - 1)), tl.j, divk, uint32_t(L));
      const uint16_t* p = qsrc + int64_t(i) * a_sn;
#pragma unroll
      for (int c = 0; c < D / 16; ++c) qraw[qb][c] = ld16(p + 16 * c + 8 * gq);
    }
  };
  load_q(ucur);
  // the row table, while the loads above are in flight (the barriers below
  // or the prologue's last one publish it)
  if constexpr (TAB) {
    for (int r = tid; r < L; r += C::NT)
      row_tab[r] = skiparse_token(mode, uint32_t(r), 0u, divk, uint32_t(L));
  }
  if constexpr (ROPE_Q || ROPE_K) {
    if (tid < kMaxPairs) rl->omega[tid] = omega;
    lds_barrier();
    fill_rope_table(rg, rl, tid, C::NT);
    lds_barrier();
  }
  // Q^T operand of the current tile from the rows in qraw
  auto rotate_q = [&]() __attribute__((always_inline)) {
    const TileId tc = decode(ucur);
    // (a persistent workgroup reads the geometry and the scale again here)
    const RopeGeom rq = PERSIST ? rope_scalars(args()->rope) : rg;
    const bool fast_rq = rq.aligned8 && rq.tab_entries;
    const float c2 = args()->scale_log2;
    int lq, gq;
    lane_ids(lq, gq);
#pragma unroll
    for (int qb = 0; qb < QB; ++qb) {
      const int r = int(tc.qt) * C::BM + (wave * QB + qb) * 32 + lq;
      const bool valid = r < L;
      const uint32_t i = skiparse_token(mode, uint32_t(valid ? r : 0), tc.j, divk, uint32_t(L));
      const bool video = ROPE_Q && is_video(rq, i);
      const Coord3 cc = video_coords(rq, i);
#pragma unroll
      for (int c = 0; c < D / 16; ++c) {
        uint4 raw = valid ? qraw[qb][c] : make_uint4(0, 0, 0, 0);
        // times scale * log2(e) so that the score products come out in log2
        // units; a rotated row is rotated and scaled in fp32, rounded once
        if (ROPE_Q && video) {
          raw = fast_rq ? rotate_chunk_col_scaled(rl, chunk_col(rq, 8 * c + 4 * gq), cc, raw, c2)
                        : rotate_chunk_scaled(rq, rl, 8 * c + 4 * gq, cc, raw, c2);
        } else {
          raw.x = pack_bf16(bf16lo(raw.x) * c2, bf16hi(raw.x) * c2);
          raw.y = pack_bf16(bf16lo(raw.y) * c2, bf16hi(raw.y) * c2);
          raw.z = pack_bf16(bf16lo(raw.z) * c2, bf16hi(raw.z) * c2);
          raw.w = pack_bf16(bf16lo(raw.w) * c2, bf16hi(raw.w) * c2);
        }
        qreg[qb][c] = __builtin_bit_cast(bf16x8_t, raw);
      }
    }
  };

  // ---- ping-pong schedule.  The waves form two halves, one wave of each
  // on every SIMD.  Per key tile t a wave runs a matrix phase M(t) (S(t) =
  // K(t) Q^T, then O += P(t-1) V(t-1)) and a softmax phase V(t) (max,
  // rescale, exp2, row sums of S(t) into P), each ended by a workgroup
  // barrier.  The trailing half passes one barrier first and so runs one
  // phase behind: on each SIMD one wave's MFMAs overlap the other wave's
  // softmax.
  //
  // Loads: tile x of K and V lives in slot x % NS.  In its softmax phase
  // for tile t each wave of the leading half issues its share of
  // K(t+NS-1), each wave of the trailing half its share of V(t+NS-1); the
  // tiles they replace, K(t-1) and V(t-1), were last read in earlier
  // phases.  At the end of that phase a wave waits for its loads of
  // K(t+1) or V(t+1) only (issued NS-2 iterations before), at least one
  // phase before their first reader, so each load has 2(NS-2) phases or
  // more to arrive.  The tile count is padded to a multiple of NS with
  // tiles past the end of the subsequence (keys masked to -inf, loads out
  // of range of the buffer, which read as zeros), so that every slot index
  // is a compile-time constant.
  f32x16_t s[NKB][QB];
  bf16x8_t pb[QB][NKB][2];

  auto barrier = [&]() __attribute__((always_inline)) {
    __builtin_amdgcn_sched_barrier(0);
    asm volatile("s_barrier" ::: "memory");
    __builtin_amdgcn_sched_barrier(0);
  };
  // Wait for all but the last NS-2 iterations' loads (vmcnt((NS-2)*DPW));
  // the leading half on the staged path has just stored its tile and waits
  // for all (vmcnt(0) lgkmcnt(0)).  The compiler tracks these waits, so it
  // knows which slots are complete.
  constexpr int kInFlight = (NS - 2) * C::DPW;
  static_assert(kInFlight < 64, "vmcnt field");
  auto loads_done = [&]() __attribute__((always_inline)) {
    __builtin_amdgcn_sched_barrier(0);
    if (ROPE_K && lead) __builtin_amdgcn_s_waitcnt(0x0070);
    else __builtin_amdgcn_s_waitcnt((kInFlight & 15) | ((kInFlight >> 4) << 14) | 0x0F70);
  };
  // matrix phase of tile t: QK(t) from K slot P (QK) and PV(t-1) from V
  // slot (P + NS - 1) % NS (PV).  Instruction order inside it (one query block
  // per wave): the LDS reads run OSP_M_LEAD MFMAs ahead of the MFMAs that
  // use them.  With two blocks the compiler's own order was as fast.
  auto m_phase = [&](int t, auto slot, auto do_qk, auto do_pv, auto masked) __attribute__((always_inline)) {
    constexpr int P = decltype(slot)::value;
    constexpr bool QK = decltype(do_qk)::value, PV = decltype(do_pv)::value;
    __builtin_amdgcn_s_setprio(1);
    if constexpr (QK) qk(int_c<P>{}, s, t, masked);
    if constexpr (PV) pv(int_c<(P + NS - 1) % NS>{}, pb);
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
  // one iteration (two phases) for tile t in slot P = t % NS; MASKED: mask
  // keys past the end (correct for any tile; used for the last groups)
  auto iter = [&](int t, auto slot, auto masked, auto near_end) __attribute__((always_inline)) {
    constexpr int P = decltype(slot)::value;
    m_phase(t, slot, bool_c<true>{}, bool_c<true>{}, masked);
    barrier();
    issue_tile(t + NS - 1, int_c<(P + NS - 1) % NS>{}, near_end);
    softmax_phase(s, pb, t == 0);
    finish_tile(t + NS - 1, int_c<(P + NS - 1) % NS>{});
    loads_done();
    barrier();
  };

  // an iteration of the last group for a tile t that may lie past the end:
  // as iter when t < nkt; for t == nkt only the PV product of tile t - 1;
  // beyond, no work.  The loads and barriers are those of iter.
  // (with K rotated in the loader, or two query blocks per wave and a
  // per-row remap, the padding runs as masked tiles: the branches would
  // push those variants' registers past the budget)
  constexpr bool kSkipPad = !ROPE_K && (FIXED_ROWS || QB == 1);
  auto iter_pad = [&](int t, auto slot) __attribute__((always_inline)) {
    constexpr int P = decltype(slot)::value;
    if (!kSkipPad || t < nkt) {
      iter(t, slot, bool_c<true>{}, bool_c<true>{});
    } else {
      if (t == nkt) m_phase(t, slot, bool_c<false>{}, bool_c<true>{}, bool_c<false>{});
      barrier();
      issue_tile(t + NS - 1, int_c<(P + NS - 1) % NS>{}, bool_c<true>{});
      finish_tile(t + NS - 1, int_c<(P + NS - 1) % NS>{});
      loads_done();
      barrier();
    }
  };

  // ---- the tiles of this workgroup: one, or (persistent) a list ----
  for (;;) {
    rotate_q();
    init_acc();
    if constexpr (PERSIST) {
      const AttnArgs* A = args();
      const uint32_t tot = uint32_t(A->total_tiles), tq8 = tot >> 3, xc = blockIdx.x & 7u;
      const uint32_t wnx = wn + (gridDim.x >> 3);
      has_next = wnx < tq8 + (xc < (tot & 7u) ? 1u : 0u);
      if (has_next) unxt = wnx < tq8 ? xc * tq8 + wnx : (tot & ~7u) + xc;
    }
    // prologue, part 2: K and V of tiles 0 .. NS-2 into their slots (with K
    // rotation in the loader: here); V slot NS-1 (read as "V(-1)" by the
    // first matrix phase, with P = 0) cleared, once every wave has finished
    // reading it: the RoPE table it holds in the prologue, or (persistent)
    // the previous tile's last V tile
    if constexpr ((ROPE_Q && !ROPE_K) || PERSIST) lds_barrier();
    for (int e = tid; e < C::TILE / 8; e += C::NT)
      reinterpret_cast<uint4*>(vslot(int_c<NS - 1>{}))[e] = make_uint4(0, 0, 0, 0);
#pragma unroll
    for (int qb = 0; qb < QB; ++qb)
#pragma unroll
      for (int kb = 0; kb < NKB; ++kb) {
        pb[qb][kb][0] = bf16x8_t{};
        pb[qb][kb][1] = bf16x8_t{};
      }
    if constexpr (ROPE_K) {
      for_slots([&](auto sl) __attribute__((always_inline)) {
        if constexpr (decltype(sl)::value < NS - 1) {
          issue_tile_first(decltype(sl)::value, sl);
          finish_tile(decltype(sl)::value, sl);
        }
      }, std::make_integer_sequence<int, NS>{});
    }
    __syncthreads();
    if constexpr (TAB) tab_fetch(NS - 1);    // the first tile the loop requests
    if (!lead) barrier();
    int t = 0;
    auto group = [&](auto near_end) __attribute__((always_inline)) {
      for_slots([&](auto sl) __attribute__((always_inline)) {
        iter(t + decltype(sl)::value, sl, bool_c<false>{}, near_end);
      }, std::make_integer_sequence<int, NS>{});
    };
    if constexpr (PERSIST) {
      // the groups whose requests stay below nkt3, then at most one more
      for (; t + 2 * NS <= tu; t += NS) group(bool_c<false>{});
      for (; t + NS <= tu; t += NS) group(bool_c<true>{});
    } else {
      for (; t + NS <= tu; t += NS) group(bool_c<true>{});
    }
    // the last group: tiles past nkt - 1 only pad the group to NS slots;
    // their matrix and softmax work is skipped (uniform branches), except
    // the PV product of the last real tile
    for (; t < nkt3; t += NS) {
      for_slots([&](auto sl) __attribute__((always_inline)) {
        if constexpr (decltype(sl)::value == 0) iter(t, sl, bool_c<true>{}, bool_c<true>{});
        else iter_pad(t + decltype(sl)::value, sl);
      }, std::make_integer_sequence<int, NS>{});
    }
    // the last matrix phase: PV of tile nkt3 - 1 (V slot NS-1), when it is real
    if (!kSkipPad || nkt3 == nkt)
      m_phase(nkt3, int_c<0>{}, bool_c<false>{}, bool_c<true>{}, bool_c<false>{});
    if (lead) barrier();   // the trailing half's last barrier
    if (PERSIST && has_next) {
      // the next tile's Q rows, in flight during this tile's stores (its
      // first K/V tiles were requested in the last group)
      load_q(unxt);
    } else {
      // loads of the padding tiles past nkt3 may still be writing LDS:
      // finish them before the workgroup's LDS is released
      __builtin_amdgcn_s_waitcnt(0x0070);
    }

    // ---- epilogue: O = O^T / l, stored at the original token row ----
    const TileId cur = decode(ucur);
    const AttnArgs* A = args();
    uint16_t* og = A->o + int64_t(cur.b) * A->osb + int64_t(cur.h) * A->osh + tok0 * A->osn;
    float* const lse_out = A->lse ? A->lse + tok0 : nullptr;
    int le, ge;
    lane_ids(le, ge);
#pragma unroll
    for (int qb = 0; qb < QB; ++qb) {
      const float lt = sum_pair32(lsum[qb]);
      const float inv = 1.0f / lt;
      const int r = int(cur.qt) * C::BM + (wave * QB + qb) * 32 + le;
      if (r < L) {
        const uint32_t i = skiparse_token(mode, uint32_t(r), cur.j, divk, uint32_t(L));
        uint16_t* p = og + int64_t(i) * A->osn;
#pragma unroll
        for (int db = 0; db < D / 32; ++db)
#pragma unroll
          for (int r4 = 0; r4 < 4; ++r4) {
            const uint32_t w0 = pack_bf16(o[qb][db][4 * r4 + 0] * inv, o[qb][db][4 * r4 + 1] * inv);
            const uint32_t w1 = pack_bf16(o[qb][db][4 * r4 + 2] * inv, o[qb][db][4 * r4 + 3] * inv);
            *reinterpret_cast<uint2*>(p + 32 * db + 8 * r4 + 4 * ge) = make_uint2(w0, w1);
          }
        if (lse_out && ge == 0)
          lse_out[(int64_t(cur.b) * A->heads + cur.h) * A->lse_ld + i] = (mref[qb] + __log2f(lt)) * kLn2;
      }
    }
    if (!PERSIST || !has_next) break;
    wn += gridDim.x >> 3;
    ucur = unxt;
  }
}

// Tile shape per head_dim: 32-row query blocks per wave (QB), keys per
// tile (BN), waves per workgroup (NW), waves per SIMD (OCC).  Build-time
// overridable for tuning.
// D=64: two 32-row query blocks per wave over 32-key tiles; each K or V
// fragment read from LDS then feeds two MFMAs, and the matrix phase is as
// long as at D=128 with half the registers per block (7% faster on
// CogVideoX's 17,776 tokens than one block over 64-key tiles)
// NS: tile slots of the fixed-row instances (see the kernel).  D=96 takes
// four (loads issued three tiles ahead): 0.5-1.5% faster than three on the
// 28,800-token workload, full and Skiparse k=4; five or six gain nothing
// more.  At D=64 and D=128 a fourth slot spills.  The per-row-remap
// instances keep three (a fourth spills at D=96 and ran 2.5% slower on
// Skiparse-2D), and so does K rotated in the loader, whose K tile goes
// through registers and is waited for at once.
#ifndef OSP_D64_TILE
#define OSP_D64_TILE 2, 32, 8, 2, 3
#endif
#ifndef OSP_D96_TILE
#define OSP_D96_TILE 1, 64, 8, 2, 4
#endif
#ifndef OSP_D128_TILE
#define OSP_D128_TILE 1, 64, 8, 2, 3
#endif
// D=128 with K rotated in the loader: 64-key tiles spill, 32 do not
#ifndef OSP_D128_ROPE_K_TILE
#define OSP_D128_ROPE_K_TILE 1, 32, 8, 2, 3
#endif
template <int QB_, int BN_, int NW_, int OCC_, int NS_> struct TileShape {
  static constexpr int QB = QB_, BN = BN_, NW = NW_, OCC = OCC_, NS = NS_;
};
template <typename T> struct RopeKShape : T {
  static constexpr int NS = 3;
};
template <int D, bool RK> struct TileCfg;
template <> struct TileCfg<64, false> : TileShape<OSP_D64_TILE> {};
template <> struct TileCfg<64, true> : RopeKShape<TileShape<OSP_D64_TILE>> {};
template <> struct TileCfg<96, false> : TileShape<OSP_D96_TILE> {};
template <> struct TileCfg<96, true> : RopeKShape<TileShape<OSP_D96_TILE>> {};
template <> struct TileCfg<128, false> : TileShape<OSP_D128_TILE> {};
template <> struct TileCfg<128, true> : RopeKShape<TileShape<OSP_D128_ROPE_K_TILE>> {};

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

#ifndef OSP_TAB_NS
#define OSP_TAB_NS 3
#endif
// LDS of a workgroup, static plus dynamic, in bytes
constexpr int kLdsBytes = 160 * 1024;

// Workgroups of `kern` the current device runs at once: CUs times the
// workgroups of `block` threads and `dyn` bytes of dynamic LDS that fit on
// one CU, rounded down to a multiple of 8 (the XCDs), so that every XCD
// holds as many; 0 when the runtime cannot tell.
static int persist_grid(const void* kern, int block, size_t dyn) {
  int dev = 0, cus = 0, per_cu = 0;
  if (hipGetDevice(&dev) != hipSuccess) return 0;
  if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess) return 0;
  if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, kern, block, dyn) != hipSuccess) return 0;
  return (cus * per_cu) & ~7;
}

// Static LDS of a kernel in bytes (-1 if the runtime cannot say), looked
// up once per kernel
template <typename K> static int static_lds_of(K kern) {
  static std::atomic<int> bytes{-2};
  if (bytes.load() == -2) {
    hipFuncAttributes attr;
    bytes.store(hipFuncGetAttributes(&attr, reinterpret_cast<const void*>(kern)) == hipSuccess
                    ? int(attr.sharedSizeBytes) : -1);
  }
  return bytes.load();
}

// One launch of `kern` over the tiles of `a`: persistent (PERSIST
// instances, when the tiles outnumber the workgroups the chip runs at once)
// or one workgroup per tile.
template <typename K>
static hipError_t launch_tiles(K kern, bool persist, const AttnArgs& a, dim3 block, size_t dyn,
                               hipStream_t s) {
  int grid = a.total_tiles;
  if (persist) {
    const int g = persist_grid(reinterpret_cast<const void*>(kern), int(block.x), dyn);
    if (g <= 0 || a.total_tiles <= g) return hipErrorNotSupported;   // caller takes the other
    grid = g;
  }
  hipLaunchKernelGGL(kern, dim3(grid), block, dyn, s, a);
  return hipGetLastError();
}

// Persistent launches are taken where they measured faster, with fixed
// rows (full, block, Single and Group Skip with k dividing the key tile):
// at head_dim 96, 2-4% on the 28,800-token workload's full and Skiparse
// k=4 attention and 8% on its spatial (1,200-token) attention; at head_dim
// 64, 2.4% on CogVideoX's 17,776 tokens.  At head_dim 128 it measured
// within the noise (+0.4%), and the row-table instance 1% slower than one
// workgroup per tile: those launches keep one workgroup per tile.
#ifndef OSP_PERSIST_ALL_D
#define OSP_PERSIST_ALL_D 0
#endif
template <int D> constexpr bool kPersistFixed = OSP_PERSIST_ALL_D || D == 96 || D == 64;
#ifndef OSP_PERSIST_TAB
#define OSP_PERSIST_TAB 0
#endif
template <int D> constexpr bool kPersistTab = OSP_PERSIST_TAB && D == 96;

template <int D, bool RQ, bool RK, bool PK>
static hipError_t launch_drk(const AttnArgs& a, bool persist, hipStream_t s) {
  using T = TileCfg<D, RK>;
  const dim3 block(T::NW * 64);
  const bool fixed = a.mode <= MODE_BLOCK && (a.mode != MODE_GROUP || T::BN % int(a.divk.d) == 0);
  if (fixed) {
    if constexpr (!RK && !PK && kPersistFixed<D>) {
      const hipError_t e = !persist ? hipErrorNotSupported : launch_tiles(
          attn3d_fwd_kernel<D, T::QB, T::BN, T::NW, T::OCC, T::NS, RQ, RK, true, PK, false, true>,
          true, a, block, 0, s);
      if (e != hipErrorNotSupported) return e;
    }
    return launch_tiles(
        attn3d_fwd_kernel<D, T::QB, T::BN, T::NW, T::OCC, T::NS, RQ, RK, true, PK, false, false>,
        false, a, block, 0, s);
  }
  // per-row remap: with Q rotated in the loader and K already rotated (the
  // fast path), rows come from an LDS row table when it fits beside the
  // kernel's static LDS
  if constexpr (RQ && !RK && !PK) {
    constexpr int NS = D == 96 ? OSP_TAB_NS : 3;
    const int64_t tab = int64_t(a.seq_len) * 4;
    if constexpr (kPersistTab<D>) {
      auto pkern = attn3d_fwd_kernel<D, T::QB, T::BN, T::NW, T::OCC, NS, RQ, RK, false, PK, true, true>;
      const int plds = static_lds_of(pkern);
      if (persist && plds >= 0 && plds + tab <= kLdsBytes) {
        const hipError_t e = launch_tiles(pkern, true, a, block, size_t(tab), s);
        if (e != hipErrorNotSupported) return e;
      }
    }
    auto kern = attn3d_fwd_kernel<D, T::QB, T::BN, T::NW, T::OCC, NS, RQ, RK, false, PK, true, false>;
    const int lds = static_lds_of(kern);
    if (lds < 0) return hipErrorInvalidDeviceFunction;
    if (lds + tab <= kLdsBytes) return launch_tiles(kern, false, a, block, size_t(tab), s);
  }
  return launch_tiles(
      attn3d_fwd_kernel<D, T::QB, T::BN, T::NW, T::OCC, 3, RQ, RK, false, PK, false, false>, false, a,
      block, 0, s);
}

template <int D, bool PK>
static hipError_t launch_d(const AttnArgs& a, int rope_q, int rope_k, bool persist,
                           hipStream_t s) {
  if (rope_q && rope_k) return launch_drk<D, true, true, PK>(a, persist, s);
  if (rope_q) return launch_drk<D, true, false, PK>(a, persist, s);
  if (rope_k) return launch_drk<D, false, true, PK>(a, persist, s);
  return launch_drk<D, false, false, PK>(a, persist, s);
}

hipError_t launch_attn3d(AttnArgs& a, int head_dim, int rope_q, int rope_k, int persist,
                         hipStream_t s) {
  if (a.seq_len <= kShortRows) return launch_attn3d_short(a, head_dim, rope_q, rope_k, s);
  switch (head_dim) {
    case 64: return launch_d<64, false>(a, rope_q, rope_k, persist != 0, s);
    case 96: return launch_d<96, false>(a, rope_q, rope_k, persist != 0, s);
    case 128: return launch_d<128, false>(a, rope_q, rope_k, persist != 0, s);
    default: return hipErrorInvalidValue;
  }
}

hipError_t launch_attn3d_packed(const AttnArgs& a, int head_dim, int rope_q, int rope_k,
                                hipStream_t s) {
  switch (head_dim) {
    case 64: return launch_d<64, true>(a, rope_q, rope_k, false, s);
    case 96: return launch_d<96, true>(a, rope_q, rope_k, false, s);
    case 128: return launch_d<128, true>(a, rope_q, rope_k, false, s);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace osp
