// skiparse_index.hip -- subsequence index maps on the device (Skiparse,
// Open-Sora Plan section 2.2.2, and block attention): perm[j*L + r] = token
// of row r of subsequence j, and its inverse.  Uses the same remap routine
// as the attention loaders.
#include "osp_internal.hpp"

namespace osp {

__global__ __launch_bounds__(256) void skiparse_index_kernel(int32_t mode, uint32_t n,
                                                             FastDiv div_len, SkipDiv divk,
                                                             int32_t* perm, int32_t* inv) {
  for (uint32_t pos = blockIdx.x * 256 + threadIdx.x; pos < n; pos += gridDim.x * 256) {
    const uint32_t j = fdiv(pos, div_len);
    const uint32_t r = pos - j * div_len.d;
    const uint32_t i = skiparse_token(mode, r, j, divk, div_len.d);
    if (perm) perm[pos] = int32_t(i);
    if (inv) inv[i] = int32_t(pos);
  }
}

hipError_t launch_skiparse_index(int32_t mode, const SkipDiv& divk, int32_t n, int32_t* perm,
                                 int32_t* inv, hipStream_t s) {
  if (n == 0) return hipSuccess;
  const uint32_t len = uint32_t(n) / divk.d;
  uint32_t blocks = (uint32_t(n) + 255) / 256;
  if (blocks > 4096) blocks = 4096;
  hipLaunchKernelGGL(skiparse_index_kernel, dim3(blocks), dim3(256), 0, s, mode, uint32_t(n),
                     make_fastdiv(len), divk, perm, inv);
  return hipGetLastError();
}

}  // namespace osp
