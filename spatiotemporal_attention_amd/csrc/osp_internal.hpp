// osp_internal.hpp -- kernel argument blocks and launchers behind the C ABI.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "osp_common.hpp"
#include "osp_rope.hpp"

namespace osp {

// Segments of a packed sequence served by one launch of the flash kernel.
constexpr int kMaxPackSegs = 16;
struct PackSeg {
  int32_t tile0;                // first workgroup of the segment (a multiple of 8)
  int32_t tiles;                // its tiles; tiles rounded up to 8 workgroups are launched
  int32_t start;                // first token of the segment in the packed sequence
  int32_t seq_len, q_tiles;     // subsequence length and query tiles of the segment
  int32_t n_text, off1, off2, tab_entries;   // the segment's RopeGeom fields
  FastDiv div_hw, div_w;
};

// One attention call, after validation.  Sequence of the call: N tokens,
// split into `groups` subsequences of seq_len rows (groups = 1 for full).
struct AttnArgs {
  const uint16_t* q;
  const uint16_t* k;
  const uint16_t* v;
  uint16_t* o;
  float* lse;                   // nullable, [B, H, lse_ld] (token i of (b, h) at (b*H + h)*lse_ld + i)
  int64_t lse_ld;               // n_tokens, or the packed sequence's length
  int64_t sb, sn, sh;           // q/k/v strides (elements)
  int64_t osb, osn, osh;        // o strides (elements)
  int32_t batch, heads, n_tokens, seq_len, groups, mode;
  int32_t q_tiles;              // ceil(seq_len / rows per workgroup)
  int32_t total_tiles;          // batch * heads * groups * q_tiles
  SkipDiv divk;                 // division by the Skiparse ratio (and the 2D lattice)
  float scale_log2;             // sm_scale * log2(e)
  RopeGeom rope;
  // packed launches only: n_pack segments (workgroups from pack[s].tile0
  // belong to segment s); the fields above that differ per segment are
  // taken from the table
  int32_t n_pack;
  PackSeg pack[kMaxPackSegs];
};

// Rows of queries handled by one workgroup of the attention kernel, and
// keys per LDS tile.
int attn_rows_per_block(int head_dim);
int attn_keys_per_tile(int head_dim);

// rope_q / rope_k: rotate Q / K in the loaders (0 = already rotated).
// Subsequences of at most kShortRows rows go to the one-wave-per-unit
// kernel (launch_attn3d_short), longer ones to the flash kernel.
constexpr int kShortRows = 64;
// persist: a call with more query tiles than the GPU holds workgroups at
// once may take a persistent launch (one workgroup per slot, each walking a
// list of tiles).
hipError_t launch_attn3d(AttnArgs& a, int head_dim, int rope_q, int rope_k, int persist,
                         hipStream_t s);
hipError_t launch_attn3d_short(const AttnArgs& a, int head_dim, int rope_q, int rope_k,
                               hipStream_t s);
// One flash-kernel launch over a.n_pack segments (each longer than kShortRows).
hipError_t launch_attn3d_packed(const AttnArgs& a, int head_dim, int rope_q, int rope_k,
                                hipStream_t s);

struct RopeArgs {
  const uint16_t* x;
  uint16_t* y;
  int64_t sb, sn, sh, osb, osn, osh;
  int32_t batch, n_tokens, heads, head_dim;
  int32_t inverse;              // rotate by the negative angle (the transpose)
  RopeGeom rope;
};

hipError_t launch_rope3d(const RopeArgs& a, hipStream_t s);

// One attention backward call, after validation.  q, k, v, o, dout are
// read with the input strides, dq, dk, dv written with the output strides.
// One segment of a packed backward launch: its dK/dV and dQ workgroups
// start at kv_tile0 / q_tile0 of their launches (multiples of 8) and
// number kv_tiles / q_tiles (B*H*groups*blocks, before padding).
struct BwdPackSeg {
  int32_t kv_tile0, kv_tiles, q_tile0, q_tiles;
  int32_t start;                // first token of the segment in the packed sequence
  int32_t seq_len, kv_blocks, q_blocks;
};

struct BwdArgs {
  const uint16_t* q;
  const uint16_t* k;
  const uint16_t* v;
  const uint16_t* o;
  const uint16_t* dout;
  const float* lse;             // [B, H, lse_ld], token n at lse[(b H + h) lse_ld + n], natural log
  int64_t lse_ld;
  float* neg_delta;             // workspace [B, H, N]: -sum_d o * dout
  float* neg_lse_s;             // workspace [B, H, N]: -lse / sm_scale
  uint16_t* dq;
  uint16_t* dk;
  uint16_t* dv;
  int64_t sb, sn, sh;
  int64_t osb, osn, osh;
  int32_t batch, heads, n_tokens, seq_len, groups, mode;
  int32_t kv_blocks;            // per (b, h, subsequence): key rows / rows per dK-dV workgroup
  int32_t q_blocks;             // per (b, h, subsequence): query rows / rows per dQ workgroup
  SkipDiv divk;
  float scale;                  // sm_scale
  float scale_log2;             // sm_scale * log2(e)
  int64_t ws_ld;                // token stride of a (b, h) row of the workspace arrays
  int32_t n_pack;               // packed launches: segments in pack[]
  BwdPackSeg pack[kMaxPackSegs];
};

// Rows handled by one workgroup of the dK/dV and of the dQ kernel, and the
// rows of one streamed LDS tile.
int bwd_kv_rows_per_block(int head_dim);
int bwd_q_rows_per_block(int head_dim);
int bwd_tile_rows(int head_dim);

hipError_t launch_attn3d_bwd(const BwdArgs& a, int head_dim, hipStream_t s);
// The packed backward: the workspace pass over every token (a as for a
// plain call over the packed length), then dK/dV and dQ launches whose
// workgroups find their segment in pa.pack (pa.n_pack <= kMaxPackSegs).
hipError_t launch_attn3d_bwd_prep(const BwdArgs& a, int head_dim, hipStream_t s);
hipError_t launch_attn3d_bwd_packed(const BwdArgs& pa, int kv_grid, int q_grid, int head_dim,
                                    hipStream_t s);

hipError_t launch_skiparse_index(int32_t mode, const SkipDiv& divk, int32_t n, int32_t* perm,
                                 int32_t* inv, hipStream_t s);

}  // namespace osp
