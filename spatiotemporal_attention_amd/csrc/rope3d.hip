// rope3d.hip -- standalone 3D RoPE over a [B, N, H, D] bf16 tensor
// (CogVideoX section 2.2 "3D-RoPE"; RoFormer rotation of channel pairs).
//
// Memory-bound elementwise pass: one 16-byte chunk (4 channel pairs) per
// thread and step, coalesced along (h, channel).  Each workgroup first fills
// an LDS table of (cos, sin) per (axis, coordinate, pair) -- the same values
// and the same rotation routine the attention loaders use, so a rope3d pass
// followed by unfused attention equals fused attention bit for bit.
#include "osp_internal.hpp"

namespace osp {

constexpr int kRopeThreads = 256;

// (x0, x1) -> (x0, -x1) for the 4 bf16 pairs of a chunk (sign bit only, exact)
__device__ __forceinline__ uint4 flip_pairs(uint4 v) {
  v.x ^= 0x80000000u; v.y ^= 0x80000000u; v.z ^= 0x80000000u; v.w ^= 0x80000000u;
  return v;
}

__global__ __launch_bounds__(kRopeThreads) void rope3d_kernel(const RopeArgs a,
                                                               uint32_t total,
                                                               FastDiv div_row_chunks,
                                                               FastDiv div_heads,
                                                               FastDiv div_tokens) {
  __shared__ __attribute__((aligned(16))) RopeLds rl;
  stage_rope_rates<kRopeThreads>(a.rope.omega, &rl, threadIdx.x);
  __syncthreads();
  fill_rope_table(a.rope, &rl, threadIdx.x, kRopeThreads);
  __syncthreads();
  const uint32_t kch = uint32_t(a.head_dim / 8);
  for (uint32_t idx = blockIdx.x * kRopeThreads + threadIdx.x; idx < total;
       idx += gridDim.x * kRopeThreads) {
    // idx -> (b, n, h, chunk), chunk fastest
    const uint32_t row = fdiv(idx, div_row_chunks);     // (b, n, h)
    const uint32_t ch = idx - row * kch;
    const uint32_t bn = fdiv(row, div_heads);
    const uint32_t h = row - bn * div_heads.d;
    const uint32_t b = fdiv(bn, div_tokens);
    const uint32_t n = bn - b * div_tokens.d;
    const uint16_t* src = a.x + int64_t(b) * a.sb + int64_t(n) * a.sn + int64_t(h) * a.sh + 8 * ch;
    uint16_t* dst = a.y + int64_t(b) * a.osb + int64_t(n) * a.osn + int64_t(h) * a.osh + 8 * ch;
    uint4 v = *reinterpret_cast<const uint4*>(src);
    if (is_video(a.rope, n)) {
      // the transpose of a rotation is the rotation by the negative angle:
      // negate the second channel of every pair before and after rotating
      if (a.inverse) v = flip_pairs(v);
      v = rotate_chunk(a.rope, &rl, 4 * int(ch), video_coords(a.rope, n), v);
      if (a.inverse) v = flip_pairs(v);
    }
    *reinterpret_cast<uint4*>(dst) = v;
  }
}

hipError_t launch_rope3d(const RopeArgs& a, hipStream_t s) {
  const uint64_t total64 = uint64_t(a.batch) * uint64_t(a.n_tokens) * uint64_t(a.heads) *
                           uint64_t(a.head_dim / 8);
  if (total64 == 0) return hipSuccess;
  if (total64 > 0xffffffffull - uint64_t(2048) * kRopeThreads) return hipErrorInvalidValue;
  const uint32_t total = uint32_t(total64);
  uint32_t blocks = uint32_t((total64 + kRopeThreads - 1) / kRopeThreads);
  if (blocks > 2048) blocks = 2048;   // grid-stride beyond 8 workgroups per CU
  hipLaunchKernelGGL(rope3d_kernel, dim3(blocks), dim3(kRopeThreads), 0, s, a, total,
                     make_fastdiv(uint32_t(a.head_dim / 8)), make_fastdiv(uint32_t(a.heads)),
                     make_fastdiv(uint32_t(a.n_tokens)));
  return hipGetLastError();
}

}  // namespace osp
