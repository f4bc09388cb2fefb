/*
 * osp.h -- C ABI of libosp: 3D-RoPE full and Skiparse attention (forward
 * and backward) for video diffusion transformers, on AMD Instinct MI355X
 * (gfx950).
 *
 * What is computed (sources are web pages; sections named per function):
 *   - A video clip's latent grid after a causal VAE and patchify
 *     ("Open Video Models", section "The Mathematics"; CogVideoX section 2.2
 *     "Patchify"; Open-Sora Plan section 2.2.1).
 *   - 3D RoPE on the query and key of every video token (CogVideoX section 2.2
 *     "3D-RoPE"; Open-Sora Plan section 2.2.1; RoFormer, CogVideoX ref. [14]).
 *   - Attention over the whole [text | video] sequence (CogVideoX section 2.2
 *     "3D Full Attention"), or within the k subsequences of a Skiparse step
 *     (Open-Sora Plan section 2.2.2 "Skiparse Attention").
 *
 * Conventions shared by every entry point:
 *   - Tensors are bfloat16, logically [B, N, H, D] (batch, token, head,
 *     channel), channel stride 1; batch/token/head strides are given in
 *     elements (0 selects the contiguous value).  Token order: n_text text
 *     tokens first, then the T x H' x W' video tokens unfolded row-major
 *     (t slowest, w fastest).
 *   - The head dimension is split into channel chunks [rope_t | rope_h |
 *     rope_w]; within a chunk of size d_a, channel pair (2r, 2r+1) is
 *     rotated by the angle pos_a * theta^(-2r/d_a), where pos_a is the
 *     token's integer latent coordinate on that axis plus pos_*0.  Text
 *     tokens are not rotated.
 *   - All memory is owned by the caller; device pointers must stay valid
 *     until the enqueued work has finished.  The library allocates no device
 *     memory and keeps no state besides a thread-local error string.
 *   - Device work is enqueued on the caller's hipStream_t (NULL = the null
 *     stream) and the call returns without waiting.
 *   - Every argument is checked on the host before anything is enqueued; on
 *     error nothing is written or enqueued, the call returns a status code
 *     and osp_last_error() describes the problem.  No call aborts, asserts or
 *     throws across this interface.
 */
#ifndef OSP_H
#define OSP_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define OSP_ABI_VERSION 1

typedef enum {
  OSP_OK = 0,
  OSP_ERR_NULL = 1,        /* a required pointer is NULL                     */
  OSP_ERR_SHAPE = 2,       /* sizes inconsistent or not divisible            */
  OSP_ERR_PARAM = 3,       /* a scalar parameter is out of range             */
  OSP_ERR_UNSUPPORTED = 4, /* valid, but not implemented (e.g. head_dim)     */
  OSP_ERR_DEVICE = 5       /* the HIP runtime reported an error at launch    */
} osp_status;

typedef enum {
  OSP_MODE_FULL = 0,             /* every token attends to every token       */
  OSP_MODE_SKIPARSE_SINGLE = 1,  /* subsequence j = tokens i with i mod k = j */
  OSP_MODE_SKIPARSE_GROUP = 2,   /* subsequence j = tokens i with
                                    floor(i/k) mod k = j (groups of k
                                    adjacent tokens, k-1 groups apart)       */
  OSP_MODE_BLOCK = 3,            /* subsequence j = tokens i with
                                    floor(i/(N/k)) = j (k runs of N/k
                                    adjacent tokens)                         */
  OSP_MODE_SKIPARSE2D_SINGLE = 4,/* Skiparse-2D, k = s*s: subsequence
                                    j = jh*s + jw = video tokens (t, h, w)
                                    with h mod s = jh and w mod s = jw       */
  OSP_MODE_SKIPARSE2D_GROUP = 5  /* Skiparse-2D, k = s*s: s x s patches of
                                    each frame, s-1 patches apart;
                                    subsequence j = jh*s + jw = tokens with
                                    floor(h/s) mod s = jh and
                                    floor(w/s) mod s = jw                    */
} osp_mode;

/* The two Skiparse-2D modes follow the Open-Sora Plan blog page, which
   names Skiparse-2D for OSP-Next as a fixed sparse rule along H and W that
   stays FlashAttention-compatible and gives no formula.  They are read as
   the single and group rules of Skiparse (Open-Sora Plan section 2.2.2)
   applied to the h and w axes with factor s = sqrt(k), in every frame:
   k subsequences of N/k tokens, rows in increasing token order.  They need
   n_text == 0, sparse_k a square, and grid_h, grid_w divisible by s
   (single) or s*s (group), else OSP_ERR_UNSUPPORTED, OSP_ERR_PARAM or
   OSP_ERR_SHAPE.  The packed entry points do not take them
   (OSP_ERR_UNSUPPORTED): the lattice depends on each segment's grid. */

/* flags of osp_attn3d_fwd */
#define OSP_FUSE_ROPE_Q 1  /* rotate Q inside the attention loader; without it
                              Q is taken as already rotated                  */
#define OSP_FUSE_ROPE_K 2  /* rotate K inside the attention loader; without it
                              K is taken as already rotated                  */
#define OSP_FUSE_ROPE 3    /* both                                           */
#define OSP_ONE_TILE_PER_WORKGROUP 4
                           /* launch one workgroup per query tile.  Without
                              it, a call at head_dim 64 or 96 whose rows map to
                              tokens with a fixed stride (full, BLOCK,
                              SKIPARSE_SINGLE, SKIPARSE_GROUP with 64 % k ==
                              0) and with more query tiles than the GPU holds
                              workgroups at once launches that many
                              workgroups, each taking its XCD's tiles in
                              turn (the RoPE table built once, the next
                              tile's first loads overlapping the current
                              tile's end).  Results are the same bits either
                              way; the flag is for comparison and for
                              callers sharing the GPU with concurrent
                              kernels.  Other calls, packed calls and
                              OSP_FUSE_ROPE_K always take one tile per
                              workgroup. */

/* Shape, layout and RoPE settings of one attention call. */
typedef struct {
  int32_t batch;                    /* B >= 1                                  */
  int32_t n_text;                   /* text tokens in front, >= 0              */
  int32_t grid_t, grid_h, grid_w;   /* latent video grid, each >= 1            */
  int32_t heads;                    /* H >= 1                                  */
  int32_t head_dim;                 /* D: 64, 96 or 128                        */
  int32_t rope_t, rope_h, rope_w;   /* channel chunk per axis: even, >= 0,
                                       sum == head_dim                         */
  int32_t pos_t0, pos_h0, pos_w0;   /* added to every latent coordinate       */
  float rope_theta;                 /* RoPE base, finite and > 0               */
  int64_t stride_b, stride_n, stride_h;    /* Q, K, V (and rope3d input)       */
  int64_t ostride_b, ostride_n, ostride_h; /* O (and rope3d output)            */
} osp_attn3d_desc;

/* One video of a packed sequence: n_text text tokens, then the
   grid_t x grid_h x grid_w video tokens. */
typedef struct {
  int32_t n_text;
  int32_t grid_t, grid_h, grid_w;
} osp_segment;

/* ABI version compiled into the library (OSP_ABI_VERSION). */
int32_t osp_abi_version(void);

/* Static text for a status code. */
const char* osp_status_string(osp_status s);

/* Text describing the last failure on the calling thread ("" if none).
   The pointer stays valid until the next libosp call on the same thread. */
const char* osp_last_error(void);

/* Latent token grid of a clip ("Open Video Models", "The Mathematics":
   T' = (T-1)/c_t + 1, H' = H/c_s, W' = W/c_s; then divided by the patch
   size p_t x p_s x p_s, CogVideoX section 2.2 "Patchify").  Host only.
   grid_out[3] receives (T'/p_t, H'/p_s, W'/p_s).  OSP_ERR_SHAPE if a size
   does not divide exactly, OSP_ERR_PARAM for non-positive arguments. */
osp_status osp_latent_grid(int32_t frames, int32_t height, int32_t width,
                           int32_t c_t, int32_t c_s, int32_t p_t, int32_t p_s,
                           int32_t* grid_out);

/* Host-only check of a call to osp_attn3d_fwd with these settings (no
   pointers involved): returns what osp_attn3d_fwd would return for valid,
   aligned pointers. */
osp_status osp_attn3d_check(const osp_attn3d_desc* desc, int32_t mode,
                            int32_t sparse_k, int32_t flags);

/* 3D RoPE (CogVideoX section 2.2 "3D-RoPE"): y = rotate(x) for every
   [b, n, h] row; text rows are copied unchanged.  x is read with the
   desc stride_*, y is written with ostride_*; y == x (same strides) works in
   place.  Rotation in fp32, result rounded to bf16 (round to nearest even).
   Pointers 16-byte aligned, strides multiples of 8. */
osp_status osp_rope3d(const osp_attn3d_desc* desc, const void* x, void* y,
                      void* stream);

/* Attention forward over a packed sequence: n_segments videos of different
   durations and resolutions, each [n_text text | grid video tokens], one
   after the other along N (CogVideoX section 3.1 "Multi-Resolution Frame
   Pack").  Each video attends only to its own tokens (block-diagonal
   attention) and its RoPE positions start from 0 on its own grid, so
   segment s gives exactly what osp_attn3d_fwd gives on its slice of the
   tensors with desc's grid and n_text set to the segment's.  mode,
   sparse_k, sm_scale and flags apply to every segment and are checked per
   segment (Skiparse and block need n_text == 0 and N_s divisible as in
   osp_attn3d_fwd).  desc supplies batch, heads, head_dim, the RoPE
   settings and the strides; its n_text and grid_* are ignored, and the
   contiguous default strides use the packed length N = sum of the
   segment lengths.  q, k, v, o: [B, N, H, D]; lse: NULL or [B, H, N] fp32
   contiguous over the packed N.  segments: host array, read during the
   call only.  Every segment is checked before anything is enqueued.
   Segments whose subsequences have at most 64 rows run one launch each;
   the others share flash launches of up to 16 segments, longest first. */
osp_status osp_attn3d_packed_fwd(const osp_attn3d_desc* desc,
                                 const osp_segment* segments,
                                 int32_t n_segments, int32_t mode,
                                 int32_t sparse_k, float sm_scale,
                                 int32_t flags, const void* q, const void* k,
                                 const void* v, void* o, float* lse,
                                 void* stream);

/* osp_rope3d over a packed sequence (segments as in osp_attn3d_packed_fwd):
   each segment's rows rotated on its own grid, from position 0.  One launch
   per segment; y == x works in place.  Rotating K this way and passing
   OSP_FUSE_ROPE_Q alone to osp_attn3d_packed_fwd gives the same result as
   OSP_FUSE_ROPE, usually faster. */
osp_status osp_rope3d_packed(const osp_attn3d_desc* desc,
                             const osp_segment* segments, int32_t n_segments,
                             const void* x, void* y, void* stream);

/* osp_rope3d_inv over a packed sequence: each segment's rows rotated back
   (by the negative angle) on its own grid.  It maps the gradients that
   osp_attn3d_packed_bwd returns for the rotated q and k to the tensors
   before osp_rope3d_packed.  One launch per segment; y == x works in
   place. */
osp_status osp_rope3d_packed_inv(const osp_attn3d_desc* desc,
                                 const osp_segment* segments,
                                 int32_t n_segments, const void* x, void* y,
                                 void* stream);

/* Transpose (= inverse) of osp_rope3d: y = rotate(x) by the negative
   angle for every video [b, n, h] row, text rows copied, same strides,
   layout and rounding as osp_rope3d.  It maps the gradient with respect to
   a rotated tensor to the gradient with respect to the tensor before the
   rotation (the rotation is orthogonal, so its Jacobian's transpose is the
   rotation by the negative angle; CogVideoX section 2.2 "3D-RoPE",
   RoFormer).  y == x works in place. */
osp_status osp_rope3d_inv(const osp_attn3d_desc* desc, const void* x, void* y,
                          void* stream);

/* Attention forward.
   mode: osp_mode.  sparse_k: the number k >= 1 of subsequences (ignored
   for FULL).  Skiparse (Open-Sora Plan section 2.2.2) needs N divisible by
   k (single) or by k*k (group).  BLOCK needs N divisible by k: with k = T
   it is the spatial half of separated spatial / temporal attention
   (CogVideoX section 2.2 "3D Full Attention", Table 8), each frame's H*W
   tokens attending among themselves, and with k = N / w it is window
   attention over windows of w tokens; the temporal half is SKIPARSE_SINGLE
   with k = H*W.  Modes other than FULL need n_text == 0 (else
   OSP_ERR_UNSUPPORTED); k == 1 equals full attention.  The k
   subsequences are attended independently and each output row is written
   back at its token's original position.
   sm_scale: logit scale; <= 0 selects 1/sqrt(head_dim).
   flags: OSP_FUSE_ROPE_Q / OSP_FUSE_ROPE_K rotate Q / K in the loaders; a
   tensor whose flag is clear must already be rotated.  K is rotated
   exactly as osp_rope3d would (then bf16), so results do not depend on
   OSP_FUSE_ROPE_K.  Q is multiplied by sm_scale * log2(e) in the loader
   and rounded to bf16: with OSP_FUSE_ROPE_Q the rotation and the scaling
   share that one rounding, without it the already rotated bf16 Q is
   rounded a second time.  OSP_FUSE_ROPE_K needs the per-axis cos/sin
   table in LDS: grid_t*rope_t + grid_h*rope_h + grid_w*rope_w <= 6144
   (else OSP_ERR_UNSUPPORTED; rotate K with osp_rope3d instead).  It is
   slower than rotating K once with osp_rope3d and passing OSP_FUSE_ROPE_Q
   alone, since every query tile rotates the same K again: use it where a
   rotated copy of K cannot be held.  OSP_ONE_TILE_PER_WORKGROUP: see its
   definition above.
   q, k, v: [B, N, H, D] bf16 read with stride_*; o: written with ostride_*,
   must not overlap q, k or v.  lse: NULL, or [B, H, N] fp32 contiguous,
   receives ln(sum_j exp(sm_scale * q_i . k_j)) over the row's subsequence,
   at the original token position.
   Arithmetic: bf16 MFMA products with fp32 accumulation, fp32 online
   softmax; probabilities rounded to bf16 for the second product; output
   rounded to bf16.  Pointers 16-byte aligned, strides multiples of 8. */
osp_status osp_attn3d_fwd(const osp_attn3d_desc* desc, int32_t mode,
                          int32_t sparse_k, float sm_scale, int32_t flags,
                          const void* q, const void* k, const void* v, void* o,
                          float* lse, void* stream);

/* Bytes of device workspace osp_attn3d_bwd needs for these settings:
   two fp32 [B, H, N] arrays, each rounded up to 256 bytes.  Host only. */
osp_status osp_attn3d_bwd_workspace(const osp_attn3d_desc* desc, int32_t mode,
                                    int32_t sparse_k, int64_t* bytes);

/* Attention backward: the gradients of the loss with respect to the
   (rotated) q and k and to v, given dout = dLoss/do of the forward
   o = softmax(sm_scale * q k^T) v, attended over the same subsequences
   (mode, sparse_k as in osp_attn3d_fwd; CogVideoX section 2.2 "3D Full
   Attention", Open-Sora Plan section 2.2.2).  With P = softmax rows:
   dv = P^T dout, dP = dout v^T, dS = P o (dP - rowsum(o o dout)),
   dq = sm_scale dS k, dk = sm_scale dS^T q.
   q and k must be the ROTATED tensors (osp_rope3d output, or what the
   forward rotated in its loaders); dq and dk are the gradients with
   respect to them: apply osp_rope3d_inv to get the gradients with respect
   to q and k before the rotation.  Text tokens (FULL only) work as in the
   forward.
   q, k, v, o, dout: [B, N, H, D] bf16 read with stride_*; o is the
   forward's output.  lse: [B, H, N] fp32 contiguous, the forward's row
   log-sum-exp (natural log).  dq, dk, dv: [B, N, H, D] bf16 written with
   ostride_*; they must not overlap any input or each other.
   workspace: device memory of at least osp_attn3d_bwd_workspace() bytes,
   256-byte aligned, owned by the caller, contents on entry ignored; it is
   in use until the enqueued work has finished.
   sm_scale: as in osp_attn3d_fwd (<= 0 selects 1/sqrt(head_dim)); it
   must be the forward's.
   Arithmetic: bf16 MFMA products with fp32 accumulation; probabilities
   exp2(sm_scale log2(e) s - lse log2(e)) in fp32, rounded to bf16 (as
   dS) for the products that take them; outputs rounded to bf16.
   Pointers 16-byte aligned, strides multiples of 8.  OSP_ERR_PARAM if
   workspace_bytes is too small. */
osp_status osp_attn3d_bwd(const osp_attn3d_desc* desc, int32_t mode,
                          int32_t sparse_k, float sm_scale, const void* q,
                          const void* k, const void* v, const void* o,
                          const float* lse, const void* dout, void* dq,
                          void* dk, void* dv, void* workspace,
                          int64_t workspace_bytes, void* stream);

/* osp_attn3d_bwd without a workspace argument, for callers that cannot
   allocate device memory (code under stream capture, serving loops,
   harnesses that forbid allocation).  It calls no allocator: the two fp32
   row arrays live in a 32 MiB device array inside the library, one per
   GPU, held until the process ends; its address is looked up once per
   device.  The call runs on the CURRENT HIP device (stream must belong to
   it).  Limit: 2 * roundup256(4 * B * H * N) <= 32 MiB, i.e. B*H*N up to
   4,194,304 rows (OSP_ERR_SHAPE beyond it, before anything is enqueued).
   Every call on one GPU shares that array, and nothing in it needs to start
   at zero (each call writes the rows it reads before reading them), so
   calls that overlap in time on one GPU (other streams, other threads)
   RACE: serialise them.  Arguments, results and other errors as
   osp_attn3d_bwd; the results are bit-identical to it. */
osp_status osp_attn3d_bwd_noalloc(const osp_attn3d_desc* desc, int32_t mode,
                                  int32_t sparse_k, float sm_scale,
                                  const void* q, const void* k, const void* v,
                                  const void* o, const float* lse,
                                  const void* dout, void* dq, void* dk, void* dv,
                                  void* stream);

/* Bytes of device workspace osp_attn3d_packed_bwd needs: two fp32
   [B, H, N] arrays over the packed N, each rounded up to 256 bytes.
   Checks every segment as osp_attn3d_packed_bwd does.  Host only. */
osp_status osp_attn3d_packed_bwd_workspace(const osp_attn3d_desc* desc,
                                           const osp_segment* segments,
                                           int32_t n_segments, int32_t mode,
                                           int32_t sparse_k, int64_t* bytes);

/* Attention backward over a packed sequence (CogVideoX section 3.1,
   "Multi-Resolution Frame Pack"; segments, desc and strides as in
   osp_attn3d_packed_fwd): for each segment s, exactly what osp_attn3d_bwd
   gives on its slice of the tensors with desc's grid and n_text set to the
   segment's.  q and k are the rotated tensors (osp_rope3d_packed output);
   dq and dk are gradients with respect to them (osp_rope3d_packed_inv maps
   them back).  lse: [B, H, N] fp32 contiguous over the packed N, from
   osp_attn3d_packed_fwd.  workspace: at least
   osp_attn3d_packed_bwd_workspace() bytes, 256-byte aligned, owned by the
   caller.  Every segment is checked before anything is enqueued; then one
   workspace pass runs over all tokens, and dK/dV and dQ launches of up to
   16 segments each, whose workgroups find their segment in a table.
   Other rules as in osp_attn3d_bwd. */
osp_status osp_attn3d_packed_bwd(const osp_attn3d_desc* desc,
                                 const osp_segment* segments,
                                 int32_t n_segments, int32_t mode,
                                 int32_t sparse_k, float sm_scale,
                                 const void* q, const void* k, const void* v,
                                 const void* o, const float* lse,
                                 const void* dout, void* dq, void* dk, void* dv,
                                 void* workspace, int64_t workspace_bytes,
                                 void* stream);

/* Index maps of the subsequences of an N-token sequence (Skiparse,
   Open-Sora Plan section 2.2.2; BLOCK as above).
   perm[j*L + r] = token at row r of subsequence j (L = N/k; rows in
   increasing token order); inv[token] = its regrouped position.  FULL,
   BLOCK and k == 1 give the identity.  Either of perm/inv may be NULL, not both.
   on_device == 0: perm/inv are host arrays, filled before returning
   (stream ignored).  on_device != 0: they are device arrays, filled by a
   kernel enqueued on stream.  OSP_ERR_SHAPE if N does not divide. */
osp_status osp_skiparse_index(int32_t mode, int32_t sparse_k, int64_t n_tokens,
                              int32_t* perm, int32_t* inv, int32_t on_device,
                              void* stream);
/* The Skiparse-2D modes depend on the latent grid, so osp_skiparse_index
   rejects them (OSP_ERR_PARAM).  osp_skiparse_index3d takes the grid
   (N = grid_t*grid_h*grid_w, no text tokens) and accepts every mode, with
   the same perm/inv, on_device and stream conventions and the same
   errors as the attention calls for that grid. */
osp_status osp_skiparse_index3d(int32_t mode, int32_t sparse_k, int32_t grid_t,
                                int32_t grid_h, int32_t grid_w, int32_t* perm,
                                int32_t* inv, int32_t on_device, void* stream);

#ifdef __cplusplus
}
#endif

#endif /* OSP_H */
