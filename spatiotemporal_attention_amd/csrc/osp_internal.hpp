// osp_internal.hpp -- kernel argument blocks and launchers behind the C ABI.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "osp_common.hpp"
#include "osp_rope.hpp"

namespace osp {

// One attention call, after validation.  Sequence of the call: N tokens,
// split into `groups` subsequences of seq_len rows (groups = 1 for full).
struct AttnArgs {
  const uint16_t* q;
  const uint16_t* k;
  const uint16_t* v;
  uint16_t* o;
  float* lse;                   // nullable, [B, H, N]
  int64_t sb, sn, sh;           // q/k/v strides (elements)
  int64_t osb, osn, osh;        // o strides (elements)
  int32_t batch, heads, n_tokens, seq_len, groups, mode;
  int32_t q_tiles;              // ceil(seq_len / rows per workgroup)
  int32_t total_tiles;          // batch * heads * groups * q_tiles
  FastDiv divk;                 // division by the Skiparse ratio
  float scale_log2;             // sm_scale * log2(e)
  RopeGeom rope;
};

// Rows of queries handled by one workgroup of the attention kernel, and
// keys per LDS tile.
int attn_rows_per_block(int head_dim);
int attn_keys_per_tile(int head_dim);

// rope_q / rope_k: rotate Q / K in the loaders (0 = already rotated).
hipError_t launch_attn3d(AttnArgs& a, int head_dim, int rope_q, int rope_k, hipStream_t s);

struct RopeArgs {
  const uint16_t* x;
  uint16_t* y;
  int64_t sb, sn, sh, osb, osn, osh;
  int32_t batch, n_tokens, heads, head_dim;
  RopeGeom rope;
};

hipError_t launch_rope3d(const RopeArgs& a, hipStream_t s);

hipError_t launch_skiparse_index(int32_t mode, int32_t k, int32_t n, int32_t* perm,
                                 int32_t* inv, hipStream_t s);

}  // namespace osp
