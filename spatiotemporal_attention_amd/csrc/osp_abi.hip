// osp_abi.hip -- the extern "C" entry points of libosp (declared in
// include/osp.h): argument checks, descriptor -> kernel arguments, launch.
#include <math.h>
#include <stdarg.h>
#include <stdio.h>

#include <algorithm>
#include <mutex>
#include <string>
#include <vector>

#include "../../include/osp.h"
#include "osp_internal.hpp"

namespace {

thread_local std::string g_last_error;

osp_status fail(osp_status s, const char* fmt, ...) {
  char buf[512];
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(buf, sizeof buf, fmt, ap);
  va_end(ap);
  g_last_error = buf;
  return s;
}

osp_status ok() {
  g_last_error.clear();
  return OSP_OK;
}

osp_status device_error(hipError_t e, const char* what) {
  return fail(OSP_ERR_DEVICE, "%s: %s", what, hipGetErrorString(e));
}

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

// Resolved geometry of a descriptor.
struct Shape {
  int64_t n_tokens;
  int64_t sb, sn, sh, osb, osn, osh;
};

// Checks shared by rope3d and attention.  attn: head_dim must be one the
// attention kernel is built for.
osp_status check_desc(const osp_attn3d_desc* d, bool attn, Shape* out) {
  if (!d) return fail(OSP_ERR_NULL, "desc is NULL");
  if (d->batch < 1 || d->heads < 1)
    return fail(OSP_ERR_PARAM, "batch (%d) and heads (%d) must be >= 1", d->batch, d->heads);
  if (d->grid_t < 1 || d->grid_h < 1 || d->grid_w < 1)
    return fail(OSP_ERR_PARAM, "grid %dx%dx%d: every extent must be >= 1", d->grid_t, d->grid_h,
                d->grid_w);
  if (d->n_text < 0) return fail(OSP_ERR_PARAM, "n_text (%d) must be >= 0", d->n_text);
  const int D = d->head_dim;
  if (attn) {
    if (D != 64 && D != 96 && D != 128)
      return fail(OSP_ERR_UNSUPPORTED, "head_dim %d: attention supports 64, 96 and 128", D);
  } else if (D < 8 || D > 128 || D % 8) {
    return fail(OSP_ERR_UNSUPPORTED, "head_dim %d: rope3d supports multiples of 8 up to 128", D);
  }
  const int32_t rs[3] = {d->rope_t, d->rope_h, d->rope_w};
  for (int a = 0; a < 3; ++a)
    if (rs[a] < 0 || rs[a] % 2)
      return fail(OSP_ERR_PARAM, "rope chunk %d (%d) must be even and >= 0", a, rs[a]);
  if (int64_t(rs[0]) + rs[1] + rs[2] != D)
    return fail(OSP_ERR_PARAM, "rope chunks %d+%d+%d must sum to head_dim %d", rs[0], rs[1],
                rs[2], D);
  if (!(d->rope_theta > 0.f) || !isfinite(d->rope_theta))
    return fail(OSP_ERR_PARAM, "rope_theta must be finite and > 0");
  const int64_t video = int64_t(d->grid_t) * d->grid_h * d->grid_w;
  const int64_t n = int64_t(d->n_text) + video;
  if (n > 0x7fffffffLL)
    return fail(OSP_ERR_SHAPE, "sequence of %lld tokens exceeds 2^31-1", (long long)n);
  if (int64_t(d->grid_h) * d->grid_w > 0x7fffffffLL)
    return fail(OSP_ERR_SHAPE, "grid_h*grid_w exceeds 2^31-1");
  const int64_t hd = int64_t(d->heads) * D;
  Shape s;
  s.n_tokens = n;
  s.sb = d->stride_b ? d->stride_b : n * hd;
  s.sn = d->stride_n ? d->stride_n : hd;
  s.sh = d->stride_h ? d->stride_h : D;
  s.osb = d->ostride_b ? d->ostride_b : n * hd;
  s.osn = d->ostride_n ? d->ostride_n : hd;
  s.osh = d->ostride_h ? d->ostride_h : D;
  const int64_t st[6] = {s.sb, s.sn, s.sh, s.osb, s.osn, s.osh};
  for (int i = 0; i < 6; ++i)
    if (st[i] < 0 || st[i] % 8)
      return fail(OSP_ERR_PARAM, "stride %lld must be >= 0 and a multiple of 8 elements",
                  (long long)st[i]);
  *out = s;
  return OSP_OK;
}

void fill_rope(const osp_attn3d_desc* d, osp::RopeGeom* g) {
  *g = osp::RopeGeom{};
  g->n_text = d->n_text;
  const int32_t rs[3] = {d->rope_t, d->rope_h, d->rope_w};
  const int32_t grid[3] = {d->grid_t, d->grid_h, d->grid_w};
  g->np0 = rs[0] / 2;
  g->np1 = rs[1] / 2;
  g->np2 = rs[2] / 2;
  g->pos0_t = d->pos_t0;
  g->pos0_h = d->pos_h0;
  g->pos0_w = d->pos_w0;
  const int64_t e0 = int64_t(grid[0]) * g->np0, e1 = int64_t(grid[1]) * g->np1,
                e2 = int64_t(grid[2]) * g->np2;
  const bool fits = (e0 + e1 + e2) <= osp::kMaxTableEntries;
  g->off1 = fits ? int32_t(e0) : 0;
  g->off2 = fits ? int32_t(e0 + e1) : 0;
  g->tab_entries = fits ? int32_t(e0 + e1 + e2) : 0;
  g->aligned8 = (rs[0] % 8 == 0 && rs[1] % 8 == 0 && rs[2] % 8 == 0) ? 1 : 0;
  int p = 0;
  for (int a = 0; a < 3; ++a)
    for (int r = 0; r < rs[a] / 2; ++r)   // omega_r = theta^(-2r/d_a), in double
      g->omega[p++] = float(pow(double(d->rope_theta), -2.0 * r / double(rs[a])));
  g->div_hw = osp::make_fastdiv(uint32_t(d->grid_h) * uint32_t(d->grid_w));
  g->div_w = osp::make_fastdiv(uint32_t(d->grid_w));
}

// Per-axis factor s of the Skiparse-2D modes (k = s*s), 0 if k is not a square.
int32_t skip2d_axis(int32_t k) {
  int32_t s = int32_t(sqrt(double(k)) + 0.5);
  return (s >= 1 && s * s == k) ? s : 0;
}

bool is_skip2d(int32_t mode) {
  return mode == OSP_MODE_SKIPARSE2D_SINGLE || mode == OSP_MODE_SKIPARSE2D_GROUP;
}

// Remap divisors of a checked (mode, k) on the grid of d.
osp::SkipDiv skip_div(const osp_attn3d_desc* d, int32_t mode, int32_t groups) {
  if (!is_skip2d(mode)) return osp::make_skipdiv(uint32_t(groups), 1, 1, 1);
  return osp::make_skipdiv(uint32_t(groups), uint32_t(skip2d_axis(groups)), uint32_t(d->grid_h),
                           uint32_t(d->grid_w));
}

osp_status check_mode(const osp_attn3d_desc* d, int64_t n, int32_t mode, int32_t k) {
  if (mode < OSP_MODE_FULL || mode > OSP_MODE_SKIPARSE2D_GROUP)
    return fail(OSP_ERR_PARAM, "unknown mode %d", mode);
  if (mode == OSP_MODE_FULL) return OSP_OK;
  if (k < 1) return fail(OSP_ERR_PARAM, "sparse_k (%d) must be >= 1", k);
  if (d && d->n_text != 0)
    return fail(OSP_ERR_UNSUPPORTED, "Skiparse and block attention take no text tokens (n_text = %d)",
                d->n_text);
  if (is_skip2d(mode)) {
    if (!d)
      return fail(OSP_ERR_PARAM, "Skiparse-2D index maps need the latent grid: use osp_skiparse_index3d");
    const int32_t s = skip2d_axis(k);
    if (!s) return fail(OSP_ERR_PARAM, "Skiparse-2D needs sparse_k = s*s (got %d)", k);
    const int32_t step = (mode == OSP_MODE_SKIPARSE2D_SINGLE) ? s : s * s;
    if (d->grid_h % step || d->grid_w % step)
      return fail(OSP_ERR_SHAPE, "Skiparse-2D %s with k=%d needs grid_h (%d) and grid_w (%d) divisible by %d",
                  mode == OSP_MODE_SKIPARSE2D_SINGLE ? "single" : "group", k, d->grid_h, d->grid_w,
                  step);
    return OSP_OK;
  }
  const int64_t div = (mode == OSP_MODE_SKIPARSE_GROUP) ? int64_t(k) * k : int64_t(k);
  if (n % div)
    return fail(OSP_ERR_SHAPE, "%s needs N (%lld) divisible by %lld",
                mode == OSP_MODE_SKIPARSE_SINGLE ? "single skip"
                : mode == OSP_MODE_SKIPARSE_GROUP ? "group skip" : "block attention",
                (long long)n, (long long)div);
  return OSP_OK;
}

// Tokens spanned by bn consecutive rows of a Skiparse-2D subsequence: at
// most bn/(W/s) + 2 lattice rows, each within s*s rows of the grid.
int64_t skip2d_span(const osp_attn3d_desc* d, int64_t k, int64_t bn) {
  const int64_t s = skip2d_axis(int32_t(k));
  return (bn / std::max<int64_t>(1, d->grid_w / s) + 2) * k * d->grid_w;
}

osp_status check_attn(const osp_attn3d_desc* d, int32_t mode, int32_t k, int32_t flags,
                      Shape* s) {
  osp_status st = check_desc(d, true, s);
  if (st) return st;
  if (flags & ~int32_t(OSP_FUSE_ROPE_Q | OSP_FUSE_ROPE_K | OSP_ONE_TILE_PER_WORKGROUP))
    return fail(OSP_ERR_PARAM, "unknown flags 0x%x", flags);
  st = check_mode(d, s->n_tokens, mode, k);
  if (st) return st;
  if (flags & OSP_FUSE_ROPE_K) {
    osp::RopeGeom g;
    fill_rope(d, &g);
    if (!g.tab_entries)
      return fail(OSP_ERR_UNSUPPORTED,
                  "K rotation in the loader needs the cos/sin table (grid_t*rope_t + grid_h*rope_h "
                  "+ grid_w*rope_w <= %d); rotate K with osp_rope3d first",
                  2 * osp::kMaxTableEntries);
  }
  const int64_t groups = (mode == OSP_MODE_FULL) ? 1 : k;
  const int64_t len = s->n_tokens / groups;
  const int64_t bm = osp::attn_rows_per_block(d->head_dim);
  const int64_t tiles = int64_t(d->batch) * d->heads * groups * ((len + bm - 1) / bm);
  if (tiles > 0x7fffffffLL) return fail(OSP_ERR_SHAPE, "too many tiles (%lld)", (long long)tiles);
  // the loaders address one key tile through 32-bit byte offsets below 2^30
  const int64_t bn = osp::attn_keys_per_tile(d->head_dim);
  // rows of one key tile span bn tokens (full, block), bn*k (single skip)
  // or up to (bn + k)*k (group skip)
  const int64_t rows = (mode == OSP_MODE_SKIPARSE_SINGLE) ? bn * groups
                     : (mode == OSP_MODE_SKIPARSE_GROUP) ? (bn + groups) * groups
                     : is_skip2d(mode) ? skip2d_span(d, groups, bn) : bn;
  const int64_t span = rows * s->sn * 2 + int64_t(d->head_dim) * 2;
  if (span >= (int64_t(1) << 30))
    return fail(OSP_ERR_UNSUPPORTED, "token stride %lld with k=%lld spans more than 1 GiB per key tile",
                (long long)s->sn, (long long)groups);
  return OSP_OK;
}

// Checks of an attention backward call (q and k taken as already rotated).
osp_status check_bwd(const osp_attn3d_desc* d, int32_t mode, int32_t k, Shape* s) {
  osp_status st = check_desc(d, true, s);
  if (st) return st;
  st = check_mode(d, s->n_tokens, mode, k);
  if (st) return st;
  const int64_t groups = (mode == OSP_MODE_FULL) ? 1 : k;
  const int64_t len = s->n_tokens / groups;
  const int64_t rows_total = int64_t(d->batch) * d->heads * s->n_tokens;
  if (rows_total > 0x7fffffffLL)
    return fail(OSP_ERR_SHAPE, "batch*heads*N = %lld exceeds 2^31-1", (long long)rows_total);
  const int64_t rb = std::min(osp::bwd_kv_rows_per_block(d->head_dim),
                              osp::bwd_q_rows_per_block(d->head_dim));
  const int64_t blocks = int64_t(d->batch) * d->heads * groups * ((len + rb - 1) / rb);
  if (blocks > 0x7fffffffLL)
    return fail(OSP_ERR_SHAPE, "too many workgroups (%lld)", (long long)blocks);
  // streamed tiles are addressed through 32-bit byte offsets below 2^30
  // from their first token
  const int64_t bn = osp::bwd_tile_rows(d->head_dim);
  const int64_t rows = (mode == OSP_MODE_SKIPARSE_SINGLE) ? bn * groups
                     : (mode == OSP_MODE_SKIPARSE_GROUP) ? (bn + groups) * groups
                     : is_skip2d(mode) ? skip2d_span(d, groups, bn) : bn;
  const int64_t span = rows * s->sn * 2 + int64_t(d->head_dim) * 2;
  if (span >= (int64_t(1) << 30))
    return fail(OSP_ERR_UNSUPPORTED, "token stride %lld with k=%lld spans more than 1 GiB per tile",
                (long long)s->sn, (long long)groups);
  return OSP_OK;
}

osp_status check_fwd_pointers(const void* q, const void* k, const void* v, const void* o,
                              const float* lse, float sm_scale) {
  if (!q || !k || !v || !o) return fail(OSP_ERR_NULL, "q, k, v and o must be non-NULL");
  if (!aligned16(q) || !aligned16(k) || !aligned16(v) || !aligned16(o))
    return fail(OSP_ERR_PARAM, "q, k, v and o must be 16-byte aligned");
  if (lse && (reinterpret_cast<uintptr_t>(lse) & 3u))
    return fail(OSP_ERR_PARAM, "lse must be 4-byte aligned");
  if (isnan(sm_scale) || isinf(sm_scale)) return fail(OSP_ERR_PARAM, "sm_scale must be finite");
  return OSP_OK;
}

// Kernel arguments of one checked forward call; lse_ld: the lse row length.
void fill_fwd_args(const osp_attn3d_desc* desc, const Shape& s, int32_t mode, int32_t sparse_k,
                   float sm_scale, const void* q, const void* k, const void* v, void* o,
                   float* lse, int64_t lse_ld, osp::AttnArgs* out) {
  const int D = desc->head_dim;
  const double scale = sm_scale > 0.f ? double(sm_scale) : 1.0 / sqrt(double(D));
  const int32_t groups = (mode == OSP_MODE_FULL) ? 1 : sparse_k;
  osp::AttnArgs& a = *out;
  a.q = static_cast<const uint16_t*>(q);
  a.k = static_cast<const uint16_t*>(k);
  a.v = static_cast<const uint16_t*>(v);
  a.o = static_cast<uint16_t*>(o);
  a.lse = lse;
  a.lse_ld = lse_ld;
  a.sb = s.sb; a.sn = s.sn; a.sh = s.sh;
  a.osb = s.osb; a.osn = s.osn; a.osh = s.osh;
  a.batch = desc->batch;
  a.heads = desc->heads;
  a.n_tokens = int32_t(s.n_tokens);
  a.groups = groups;
  a.seq_len = int32_t(s.n_tokens / groups);
  a.mode = mode;
  a.divk = skip_div(desc, mode, groups);
  a.scale_log2 = float(scale * 1.4426950408889634);
  const int bm = osp::attn_rows_per_block(D);
  a.q_tiles = (a.seq_len + bm - 1) / bm;
  a.total_tiles = a.batch * a.heads * groups * a.q_tiles;
  fill_rope(desc, &a.rope);
  a.n_pack = 0;
}

// Checks of a packed backward: every segment as a backward call of its
// own, then the packed length; *total = the packed N.
osp_status check_packed_bwd(const osp_attn3d_desc* desc, const osp_segment* segments,
                            int32_t n_segments, int32_t mode, int32_t sparse_k, int64_t* total) {
  if (!desc) return fail(OSP_ERR_NULL, "desc is NULL");
  if (!segments) return fail(OSP_ERR_NULL, "segments is NULL");
  if (n_segments < 1) return fail(OSP_ERR_PARAM, "n_segments (%d) must be >= 1", n_segments);
  if (is_skip2d(mode))
    return fail(OSP_ERR_UNSUPPORTED,
                "packed sequences take full, Skiparse or block attention (the Skiparse-2D lattice "
                "depends on each segment's grid)");
  int64_t n = 0, grid = 0;
  for (int32_t i = 0; i < n_segments; ++i) {
    osp_attn3d_desc d = *desc;
    d.n_text = segments[i].n_text;
    d.grid_t = segments[i].grid_t;
    d.grid_h = segments[i].grid_h;
    d.grid_w = segments[i].grid_w;
    Shape s;
    osp_status st = check_bwd(&d, mode, sparse_k, &s);
    if (st) {
      const std::string why = g_last_error;
      return fail(st, "segment %d: %s", i, why.c_str());
    }
    n += s.n_tokens;
    if (n > 0x7fffffffLL || int64_t(desc->batch) * desc->heads * n > 0x7fffffffLL)
      return fail(OSP_ERR_SHAPE, "packed batch*heads*N exceeds 2^31-1");
    // workgroups of one packed launch (at most every segment in it)
    const int64_t groups = (mode == OSP_MODE_FULL) ? 1 : sparse_k;
    const int64_t rb = std::min(osp::bwd_kv_rows_per_block(d.head_dim),
                                osp::bwd_q_rows_per_block(d.head_dim));
    grid += (int64_t(d.batch) * d.heads * groups * ((s.n_tokens / groups + rb - 1) / rb) + 7) / 8 * 8;
    if (grid > 0x7fffffffLL) return fail(OSP_ERR_SHAPE, "too many workgroups in the packed sequence");
  }
  *total = n;
  return OSP_OK;
}

// bytes of one of the two fp32 [B, H, N] workspace arrays, rounded up to 256
int64_t bwd_ws_half(int64_t batch, int64_t heads, int64_t n_tokens) {
  const int64_t b = batch * heads * n_tokens * 4;
  return (b + 255) / 256 * 256;
}

osp_status check_bwd_pointers(const void* q, const void* k, const void* v, const void* o,
                              const float* lse, const void* dout, void* dq, void* dk, void* dv,
                              void* workspace, float sm_scale) {
  if (!q || !k || !v || !o || !lse || !dout || !dq || !dk || !dv || !workspace)
    return fail(OSP_ERR_NULL, "q, k, v, o, lse, dout, dq, dk, dv and workspace must be non-NULL");
  const void* bf[] = {q, k, v, o, dout, dq, dk, dv};
  for (const void* p : bf)
    if (!aligned16(p)) return fail(OSP_ERR_PARAM, "bf16 tensors must be 16-byte aligned");
  if (reinterpret_cast<uintptr_t>(lse) & 3u) return fail(OSP_ERR_PARAM, "lse must be 4-byte aligned");
  if (reinterpret_cast<uintptr_t>(workspace) & 255u)
    return fail(OSP_ERR_PARAM, "workspace must be 256-byte aligned");
  if (isnan(sm_scale) || isinf(sm_scale)) return fail(OSP_ERR_PARAM, "sm_scale must be finite");
  return OSP_OK;
}

// The three backward launches for one (checked) sequence: tensors at the
// given bases with the strides of s, lse rows lse_ld apart, and the two
// workspace arrays of B*H*N_s floats each.  launch == false only fills
// *out with the arguments.
osp_status enqueue_bwd(const osp_attn3d_desc* desc, const Shape& s, int32_t mode,
                       int32_t sparse_k, float sm_scale, const void* q, const void* k,
                       const void* v, const void* o, const float* lse, int64_t lse_ld,
                       const void* dout, void* dq, void* dk, void* dv, float* ws_delta,
                       float* ws_lse, hipStream_t stream, bool launch = true,
                       osp::BwdArgs* out = nullptr) {
  const int D = desc->head_dim;
  const double scale = sm_scale > 0.f ? double(sm_scale) : 1.0 / sqrt(double(D));
  const int32_t groups = (mode == OSP_MODE_FULL) ? 1 : sparse_k;
  osp::BwdArgs a;
  a.q = static_cast<const uint16_t*>(q);
  a.k = static_cast<const uint16_t*>(k);
  a.v = static_cast<const uint16_t*>(v);
  a.o = static_cast<const uint16_t*>(o);
  a.dout = static_cast<const uint16_t*>(dout);
  a.lse = lse;
  a.lse_ld = lse_ld;
  a.neg_delta = ws_delta;
  a.neg_lse_s = ws_lse;
  a.dq = static_cast<uint16_t*>(dq);
  a.dk = static_cast<uint16_t*>(dk);
  a.dv = static_cast<uint16_t*>(dv);
  a.sb = s.sb; a.sn = s.sn; a.sh = s.sh;
  a.osb = s.osb; a.osn = s.osn; a.osh = s.osh;
  a.batch = desc->batch;
  a.heads = desc->heads;
  a.n_tokens = int32_t(s.n_tokens);
  a.groups = groups;
  a.seq_len = int32_t(s.n_tokens / groups);
  a.mode = mode;
  a.divk = skip_div(desc, mode, groups);
  a.scale = float(scale);
  a.scale_log2 = float(scale * 1.4426950408889634);
  const int kvr = osp::bwd_kv_rows_per_block(D), qr = osp::bwd_q_rows_per_block(D);
  a.kv_blocks = (a.seq_len + kvr - 1) / kvr;
  a.q_blocks = (a.seq_len + qr - 1) / qr;
  a.ws_ld = s.n_tokens;
  a.n_pack = 0;
  if (a.seq_len == 0 || !launch) {
    if (out) *out = a;
    return OSP_OK;
  }
  hipError_t e = osp::launch_attn3d_bwd(a, D, stream);
  if (e != hipSuccess) return device_error(e, "attn3d_bwd launch");
  return OSP_OK;
}

}  // namespace

// Device scratch of osp_attn3d_bwd_noalloc: the backward's two fp32 row
// arrays (-delta and -lse/scale, bwd_ws_half bytes each) for callers that
// cannot allocate.  Every GPU the library runs on holds one copy, at its own
// address, until the process ends.  In host code the name is only a handle:
// kernels get the device address that hipGetSymbolAddress returns for the
// current device (noalloc_scratch below).
constexpr int64_t kNoAllocScratchBytes = int64_t(32) << 20;
static __device__ __align__(256) unsigned char scratch[kNoAllocScratchBytes];

namespace {

constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch_ptr[kMaxDevices] = {};

// The device address of the current device's scratch, looked up once per
// device (with that device current) and kept.
osp_status noalloc_scratch(void** out) {
  int dev = -1;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return device_error(e, "hipGetDevice");
  if (dev < 0 || dev >= kMaxDevices)
    return fail(OSP_ERR_UNSUPPORTED, "device %d: at most %d devices", dev, kMaxDevices);
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (!g_scratch_ptr[dev]) {
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess || !p) return device_error(e, "hipGetSymbolAddress(scratch)");
    g_scratch_ptr[dev] = p;
  }
  *out = g_scratch_ptr[dev];
  return OSP_OK;
}

}  // namespace

extern "C" {

int32_t osp_abi_version(void) { return OSP_ABI_VERSION; }

const char* osp_status_string(osp_status s) {
  switch (s) {
    case OSP_OK: return "ok";
    case OSP_ERR_NULL: return "null pointer";
    case OSP_ERR_SHAPE: return "inconsistent or indivisible shape";
    case OSP_ERR_PARAM: return "parameter out of range";
    case OSP_ERR_UNSUPPORTED: return "unsupported configuration";
    case OSP_ERR_DEVICE: return "device error";
  }
  return "unknown status";
}

const char* osp_last_error(void) { return g_last_error.c_str(); }

osp_status osp_latent_grid(int32_t frames, int32_t height, int32_t width, int32_t c_t,
                           int32_t c_s, int32_t p_t, int32_t p_s, int32_t* grid_out) {
  if (!grid_out) return fail(OSP_ERR_NULL, "grid_out is NULL");
  if (frames < 1 || height < 1 || width < 1 || c_t < 1 || c_s < 1 || p_t < 1 || p_s < 1)
    return fail(OSP_ERR_PARAM, "sizes and factors must be >= 1");
  if ((frames - 1) % c_t || height % c_s || width % c_s)
    return fail(OSP_ERR_SHAPE, "clip %dx%dx%d not divisible by VAE factors %d/%d", frames,
                height, width, c_t, c_s);
  const int32_t t = (frames - 1) / c_t + 1, h = height / c_s, w = width / c_s;
  if (t % p_t || h % p_s || w % p_s)
    return fail(OSP_ERR_SHAPE, "latent %dx%dx%d not divisible by patch %dx%dx%d", t, h, w, p_t,
                p_s, p_s);
  grid_out[0] = t / p_t;
  grid_out[1] = h / p_s;
  grid_out[2] = w / p_s;
  return ok();
}

osp_status osp_attn3d_check(const osp_attn3d_desc* desc, int32_t mode, int32_t sparse_k,
                            int32_t flags) {
  Shape s;
  osp_status st = check_attn(desc, mode, sparse_k, flags, &s);
  return st ? st : ok();
}

static osp_status rope3d_call(const osp_attn3d_desc* desc, const void* x, void* y, void* stream,
                              int inverse) {
  Shape s;
  osp_status st = check_desc(desc, false, &s);
  if (st) return st;
  if (!x || !y) return fail(OSP_ERR_NULL, "x and y must be non-NULL");
  if (!aligned16(x) || !aligned16(y)) return fail(OSP_ERR_PARAM, "x and y must be 16-byte aligned");
  osp::RopeArgs a;
  a.x = static_cast<const uint16_t*>(x);
  a.y = static_cast<uint16_t*>(y);
  a.sb = s.sb; a.sn = s.sn; a.sh = s.sh;
  a.osb = s.osb; a.osn = s.osn; a.osh = s.osh;
  a.batch = desc->batch;
  a.n_tokens = int32_t(s.n_tokens);
  a.heads = desc->heads;
  a.head_dim = desc->head_dim;
  a.inverse = inverse;
  fill_rope(desc, &a.rope);
  const uint64_t total = uint64_t(a.batch) * uint64_t(a.n_tokens) * uint64_t(a.heads) *
                         uint64_t(a.head_dim / 8);
  if (total > 0xffffffffull - 2048ull * 256ull)
    return fail(OSP_ERR_SHAPE, "tensor too large for one rope3d call");
  hipError_t e = osp::launch_rope3d(a, static_cast<hipStream_t>(stream));
  if (e != hipSuccess) return device_error(e, "rope3d launch");
  return ok();
}

osp_status osp_rope3d(const osp_attn3d_desc* desc, const void* x, void* y, void* stream) {
  return rope3d_call(desc, x, y, stream, 0);
}

osp_status osp_rope3d_inv(const osp_attn3d_desc* desc, const void* x, void* y, void* stream) {
  return rope3d_call(desc, x, y, stream, 1);
}

static osp_status rope3d_packed_call(const osp_attn3d_desc* desc, const osp_segment* segments,
                                     int32_t n_segments, const void* x, void* y, void* stream,
                                     int32_t inverse) {
  if (!desc) return fail(OSP_ERR_NULL, "desc is NULL");
  if (!segments) return fail(OSP_ERR_NULL, "segments is NULL");
  if (n_segments < 1) return fail(OSP_ERR_PARAM, "n_segments (%d) must be >= 1", n_segments);
  int64_t total = 0;
  for (int32_t i = 0; i < n_segments; ++i) {
    osp_attn3d_desc d = *desc;
    d.n_text = segments[i].n_text;
    d.grid_t = segments[i].grid_t;
    d.grid_h = segments[i].grid_h;
    d.grid_w = segments[i].grid_w;
    Shape s;
    osp_status st = check_desc(&d, false, &s);
    if (st) {
      const std::string why = g_last_error;
      return fail(st, "segment %d: %s", i, why.c_str());
    }
    total += s.n_tokens;
    if (total > 0x7fffffffLL)
      return fail(OSP_ERR_SHAPE, "packed sequence of more than 2^31-1 tokens");
  }
  if (!x || !y) return fail(OSP_ERR_NULL, "x and y must be non-NULL");
  if (!aligned16(x) || !aligned16(y)) return fail(OSP_ERR_PARAM, "x and y must be 16-byte aligned");
  osp_attn3d_desc pd = *desc;
  pd.n_text = 0;
  pd.grid_t = 1;
  pd.grid_h = 1;
  pd.grid_w = int32_t(total);
  Shape ps;
  osp_status st = check_desc(&pd, false, &ps);
  if (st) return st;
  if (uint64_t(desc->batch) * uint64_t(total) * uint64_t(desc->heads) * uint64_t(desc->head_dim / 8) >
      0xffffffffull - 2048ull * 256ull)
    return fail(OSP_ERR_SHAPE, "tensor too large for one rope3d call");
  int64_t start = 0;
  for (int32_t i = 0; i < n_segments; ++i) {
    osp_attn3d_desc d = *desc;
    d.n_text = segments[i].n_text;
    d.grid_t = segments[i].grid_t;
    d.grid_h = segments[i].grid_h;
    d.grid_w = segments[i].grid_w;
    const int64_t n = int64_t(d.n_text) + int64_t(d.grid_t) * d.grid_h * d.grid_w;
    osp::RopeArgs a;
    a.x = static_cast<const uint16_t*>(x) + start * ps.sn;
    a.y = static_cast<uint16_t*>(y) + start * ps.osn;
    a.sb = ps.sb; a.sn = ps.sn; a.sh = ps.sh;
    a.osb = ps.osb; a.osn = ps.osn; a.osh = ps.osh;
    a.batch = desc->batch;
    a.n_tokens = int32_t(n);
    a.heads = desc->heads;
    a.head_dim = desc->head_dim;
    a.inverse = inverse;
    fill_rope(&d, &a.rope);
    hipError_t e = osp::launch_rope3d(a, static_cast<hipStream_t>(stream));
    if (e != hipSuccess) return device_error(e, "rope3d launch");
    start += n;
  }
  return ok();
}

osp_status osp_rope3d_packed(const osp_attn3d_desc* desc, const osp_segment* segments,
                             int32_t n_segments, const void* x, void* y, void* stream) {
  return rope3d_packed_call(desc, segments, n_segments, x, y, stream, 0);
}

osp_status osp_rope3d_packed_inv(const osp_attn3d_desc* desc, const osp_segment* segments,
                                 int32_t n_segments, const void* x, void* y, void* stream) {
  return rope3d_packed_call(desc, segments, n_segments, x, y, stream, 1);
}

osp_status osp_attn3d_fwd(const osp_attn3d_desc* desc, int32_t mode, int32_t sparse_k,
                          float sm_scale, int32_t flags, const void* q, const void* k,
                          const void* v, void* o, float* lse, void* stream) {
  Shape s;
  osp_status st = check_attn(desc, mode, sparse_k, flags, &s);
  if (st) return st;
  st = check_fwd_pointers(q, k, v, o, lse, sm_scale);
  if (st) return st;
  osp::AttnArgs a;
  fill_fwd_args(desc, s, mode, sparse_k, sm_scale, q, k, v, o, lse, s.n_tokens, &a);
  if (a.total_tiles == 0) return ok();
  hipError_t e = osp::launch_attn3d(a, desc->head_dim, (flags & OSP_FUSE_ROPE_Q) ? 1 : 0,
                                    (flags & OSP_FUSE_ROPE_K) ? 1 : 0,
                                    (flags & OSP_ONE_TILE_PER_WORKGROUP) ? 0 : 1,
                                    static_cast<hipStream_t>(stream));
  if (e != hipSuccess) return device_error(e, "attn3d_fwd launch");
  return ok();
}

osp_status osp_attn3d_packed_fwd(const osp_attn3d_desc* desc, const osp_segment* segments,
                                 int32_t n_segments, int32_t mode, int32_t sparse_k,
                                 float sm_scale, int32_t flags, const void* q, const void* k,
                                 const void* v, void* o, float* lse, void* stream) {
  if (!desc) return fail(OSP_ERR_NULL, "desc is NULL");
  if (!segments) return fail(OSP_ERR_NULL, "segments is NULL");
  if (n_segments < 1) return fail(OSP_ERR_PARAM, "n_segments (%d) must be >= 1", n_segments);
  if (is_skip2d(mode))
    return fail(OSP_ERR_UNSUPPORTED,
                "packed sequences take full, Skiparse or block attention (the Skiparse-2D lattice "
                "depends on each segment's grid)");
  // every segment is checked before anything is enqueued
  int64_t total = 0, tiles = 0;
  for (int32_t i = 0; i < n_segments; ++i) {
    osp_attn3d_desc d = *desc;
    d.n_text = segments[i].n_text;
    d.grid_t = segments[i].grid_t;
    d.grid_h = segments[i].grid_h;
    d.grid_w = segments[i].grid_w;
    Shape s;
    osp_status st = check_attn(&d, mode, sparse_k, flags, &s);
    if (st) {
      const std::string why = g_last_error;
      return fail(st, "segment %d: %s", i, why.c_str());
    }
    total += s.n_tokens;
    if (total > 0x7fffffffLL)
      return fail(OSP_ERR_SHAPE, "packed sequence of more than 2^31-1 tokens");
    const int64_t bm = osp::attn_rows_per_block(desc->head_dim);
    const int64_t groups = (mode == OSP_MODE_FULL) ? 1 : sparse_k;
    tiles += (int64_t(desc->batch) * desc->heads * groups * ((s.n_tokens / groups + bm - 1) / bm) +
              7) / 8 * 8;
    if (tiles > 0x7fffffffLL) return fail(OSP_ERR_SHAPE, "too many tiles in the packed sequence");
  }
  osp_status st = check_fwd_pointers(q, k, v, o, lse, sm_scale);
  if (st) return st;
  // the strides of the packed tensors: contiguous defaults use the total length
  osp_attn3d_desc pd = *desc;
  pd.n_text = 0;
  pd.grid_t = 1;
  pd.grid_h = 1;
  pd.grid_w = int32_t(total);
  Shape ps;
  st = check_desc(&pd, true, &ps);
  if (st) return st;
  // Segments whose subsequences are short go to the short-subsequence
  // kernel one launch each; the others share flash-kernel launches of up
  // to kMaxPackSegs segments, whose workgroups find their segment in a
  // table (so small segments do not leave the chip idle on their own),
  // longest first so that the shorter ones fill the tail.
  const int rq = (flags & OSP_FUSE_ROPE_Q) ? 1 : 0, rk = (flags & OSP_FUSE_ROPE_K) ? 1 : 0;
  const hipStream_t hs = static_cast<hipStream_t>(stream);
  const int32_t groups = (mode == OSP_MODE_FULL) ? 1 : sparse_k;
  struct Flash {
    osp::AttnArgs a;
    int64_t start;
  };
  std::vector<Flash> flash;
  int64_t start = 0;
  for (int32_t i = 0; i < n_segments; ++i) {
    osp_attn3d_desc d = *desc;
    d.n_text = segments[i].n_text;
    d.grid_t = segments[i].grid_t;
    d.grid_h = segments[i].grid_h;
    d.grid_w = segments[i].grid_w;
    Shape s;
    check_desc(&d, true, &s);
    s.sb = ps.sb; s.sn = ps.sn; s.sh = ps.sh;
    s.osb = ps.osb; s.osn = ps.osn; s.osh = ps.osh;
    const int64_t seg_start = start;
    start += s.n_tokens;
    if (s.n_tokens / groups <= osp::kShortRows) {
      osp::AttnArgs a;
      fill_fwd_args(&d, s, mode, sparse_k, sm_scale,
                    static_cast<const uint16_t*>(q) + seg_start * s.sn,
                    static_cast<const uint16_t*>(k) + seg_start * s.sn,
                    static_cast<const uint16_t*>(v) + seg_start * s.sn,
                    static_cast<uint16_t*>(o) + seg_start * s.osn,
                    lse ? lse + seg_start : nullptr, total, &a);
      hipError_t e = osp::launch_attn3d_short(a, desc->head_dim, rq, rk, hs);
      if (e != hipSuccess) return device_error(e, "attn3d_packed_fwd launch");
      continue;
    }
    Flash f;
    fill_fwd_args(&d, s, mode, sparse_k, sm_scale, q, k, v, o, lse, total, &f.a);
    f.start = seg_start;
    flash.push_back(f);
  }
  std::stable_sort(flash.begin(), flash.end(),
                   [](const Flash& x, const Flash& y) { return x.a.seq_len > y.a.seq_len; });
  for (size_t i0 = 0; i0 < flash.size(); i0 += osp::kMaxPackSegs) {
    osp::AttnArgs pa = flash[i0].a;
    pa.n_pack = 0;
    pa.total_tiles = 0;
    for (size_t i = i0; i < flash.size() && i < i0 + osp::kMaxPackSegs; ++i) {
      const osp::AttnArgs& a = flash[i].a;
      osp::PackSeg& sg = pa.pack[pa.n_pack++];
      sg.tile0 = pa.total_tiles;
      sg.tiles = a.total_tiles;
      sg.start = int32_t(flash[i].start);
      sg.seq_len = a.seq_len;
      sg.q_tiles = a.q_tiles;
      sg.n_text = a.rope.n_text;
      sg.off1 = a.rope.off1;
      sg.off2 = a.rope.off2;
      sg.tab_entries = a.rope.tab_entries;
      sg.div_hw = a.rope.div_hw;
      sg.div_w = a.rope.div_w;
      pa.total_tiles += (a.total_tiles + 7) / 8 * 8;
    }
    hipError_t e = osp::launch_attn3d_packed(pa, desc->head_dim, rq, rk, hs);
    if (e != hipSuccess) return device_error(e, "attn3d_packed_fwd launch");
  }
  return ok();
}

osp_status osp_attn3d_bwd_workspace(const osp_attn3d_desc* desc, int32_t mode, int32_t sparse_k,
                                    int64_t* bytes) {
  if (!bytes) return fail(OSP_ERR_NULL, "bytes is NULL");
  Shape s;
  osp_status st = check_bwd(desc, mode, sparse_k, &s);
  if (st) return st;
  *bytes = 2 * bwd_ws_half(desc->batch, desc->heads, s.n_tokens);
  return ok();
}

osp_status osp_attn3d_bwd(const osp_attn3d_desc* desc, int32_t mode, int32_t sparse_k,
                          float sm_scale, const void* q, const void* k, const void* v,
                          const void* o, const float* lse, const void* dout, void* dq, void* dk,
                          void* dv, void* workspace, int64_t workspace_bytes, void* stream) {
  Shape s;
  osp_status st = check_bwd(desc, mode, sparse_k, &s);
  if (st) return st;
  st = check_bwd_pointers(q, k, v, o, lse, dout, dq, dk, dv, workspace, sm_scale);
  if (st) return st;
  const int64_t half = bwd_ws_half(desc->batch, desc->heads, s.n_tokens);
  if (workspace_bytes < 2 * half)
    return fail(OSP_ERR_PARAM, "workspace of %lld bytes, %lld needed", (long long)workspace_bytes,
                (long long)(2 * half));
  float* ws = static_cast<float*>(workspace);
  return enqueue_bwd(desc, s, mode, sparse_k, sm_scale, q, k, v, o, lse, s.n_tokens, dout, dq, dk,
                     dv, ws, reinterpret_cast<float*>(static_cast<char*>(workspace) + half),
                     static_cast<hipStream_t>(stream));
}

osp_status osp_attn3d_bwd_noalloc(const osp_attn3d_desc* desc, int32_t mode, int32_t sparse_k,
                                  float sm_scale, const void* q, const void* k, const void* v,
                                  const void* o, const float* lse, const void* dout, void* dq,
                                  void* dk, void* dv, void* stream) {
  Shape s;
  osp_status st = check_bwd(desc, mode, sparse_k, &s);
  if (st) return st;
  // the pointer check wants a workspace: pass a stand-in aligned address
  // (the scratch itself is looked up below)
  st = check_bwd_pointers(q, k, v, o, lse, dout, dq, dk, dv,
                          reinterpret_cast<void*>(uintptr_t(256)), sm_scale);
  if (st) return st;
  const int64_t half = bwd_ws_half(desc->batch, desc->heads, s.n_tokens);
  if (2 * half > kNoAllocScratchBytes)
    return fail(OSP_ERR_SHAPE,
                "osp_attn3d_bwd_noalloc: batch*heads*N = %lld rows need %lld bytes of scratch, "
                "more than its %lld; use osp_attn3d_bwd with a workspace",
                (long long)(int64_t(desc->batch) * desc->heads * s.n_tokens),
                (long long)(2 * half), (long long)kNoAllocScratchBytes);
  void* ws = nullptr;
  st = noalloc_scratch(&ws);
  if (st) return st;
  return enqueue_bwd(desc, s, mode, sparse_k, sm_scale, q, k, v, o, lse, s.n_tokens, dout, dq, dk,
                     dv, static_cast<float*>(ws),
                     reinterpret_cast<float*>(static_cast<char*>(ws) + half),
                     static_cast<hipStream_t>(stream));
}

osp_status osp_attn3d_packed_bwd_workspace(const osp_attn3d_desc* desc,
                                           const osp_segment* segments, int32_t n_segments,
                                           int32_t mode, int32_t sparse_k, int64_t* bytes) {
  if (!bytes) return fail(OSP_ERR_NULL, "bytes is NULL");
  int64_t total = 0;
  osp_status st = check_packed_bwd(desc, segments, n_segments, mode, sparse_k, &total);
  if (st) return st;
  *bytes = 2 * bwd_ws_half(desc->batch, desc->heads, total);
  return ok();
}

osp_status osp_attn3d_packed_bwd(const osp_attn3d_desc* desc, const osp_segment* segments,
                                 int32_t n_segments, int32_t mode, int32_t sparse_k,
                                 float sm_scale, const void* q, const void* k, const void* v,
                                 const void* o, const float* lse, const void* dout, void* dq,
                                 void* dk, void* dv, void* workspace, int64_t workspace_bytes,
                                 void* stream) {
  int64_t total = 0;
  osp_status st = check_packed_bwd(desc, segments, n_segments, mode, sparse_k, &total);
  if (st) return st;
  st = check_bwd_pointers(q, k, v, o, lse, dout, dq, dk, dv, workspace, sm_scale);
  if (st) return st;
  const int64_t half = bwd_ws_half(desc->batch, desc->heads, total);
  if (workspace_bytes < 2 * half)
    return fail(OSP_ERR_PARAM, "workspace of %lld bytes, %lld needed", (long long)workspace_bytes,
                (long long)(2 * half));
  // strides of the packed tensors (contiguous defaults use the total length)
  osp_attn3d_desc pd = *desc;
  pd.n_text = 0;
  pd.grid_t = 1;
  pd.grid_h = 1;
  pd.grid_w = int32_t(total);
  Shape ps;
  st = check_desc(&pd, true, &ps);
  if (st) return st;
  // The workspace pass once over all tokens ([B, H, N] arrays over the
  // packed N), then dK/dV and dQ launches of up to kMaxPackSegs segments
  // each, whose workgroups look their segment up in a table, longest
  // segment first (so that the shorter ones fill the tail).
  const hipStream_t hs = static_cast<hipStream_t>(stream);
  float* ws_delta = static_cast<float*>(workspace);
  float* ws_lse = reinterpret_cast<float*>(static_cast<char*>(workspace) + half);
  osp::BwdArgs base;
  st = enqueue_bwd(&pd, ps, OSP_MODE_FULL, 1, sm_scale, q, k, v, o, lse, total, dout, dq, dk, dv,
                   ws_delta, ws_lse, hs, false, &base);
  if (st) return st;
  hipError_t e = osp::launch_attn3d_bwd_prep(base, desc->head_dim, hs);
  if (e != hipSuccess) return device_error(e, "attn3d_bwd prep launch");
  const int32_t groups = (mode == OSP_MODE_FULL) ? 1 : sparse_k;
  base.mode = mode;
  base.groups = groups;
  base.divk = skip_div(desc, mode, groups);
  const int kvr = osp::bwd_kv_rows_per_block(desc->head_dim);
  const int qr = osp::bwd_q_rows_per_block(desc->head_dim);
  std::vector<osp::BwdPackSeg> segs;
  int64_t start = 0;
  for (int32_t i = 0; i < n_segments; ++i) {
    const int64_t n = int64_t(segments[i].n_text) +
                      int64_t(segments[i].grid_t) * segments[i].grid_h * segments[i].grid_w;
    osp::BwdPackSeg g;
    g.start = int32_t(start);
    g.seq_len = int32_t(n / groups);
    g.kv_blocks = (g.seq_len + kvr - 1) / kvr;
    g.q_blocks = (g.seq_len + qr - 1) / qr;
    const int32_t seqs = desc->batch * desc->heads * groups;
    g.kv_tiles = seqs * g.kv_blocks;
    g.q_tiles = seqs * g.q_blocks;
    segs.push_back(g);
    start += n;
  }
  std::stable_sort(segs.begin(), segs.end(), [](const osp::BwdPackSeg& x,
                                                const osp::BwdPackSeg& y) {
    return x.seq_len > y.seq_len;
  });
  for (size_t i0 = 0; i0 < segs.size(); i0 += osp::kMaxPackSegs) {
    osp::BwdArgs pa = base;
    pa.n_pack = 0;
    int64_t kv_grid = 0, q_grid = 0;
    for (size_t i = i0; i < segs.size() && i < i0 + osp::kMaxPackSegs; ++i) {
      osp::BwdPackSeg g = segs[i];
      g.kv_tile0 = int32_t(kv_grid);
      g.q_tile0 = int32_t(q_grid);
      kv_grid += (int64_t(g.kv_tiles) + 7) / 8 * 8;
      q_grid += (int64_t(g.q_tiles) + 7) / 8 * 8;
      pa.pack[pa.n_pack++] = g;
    }
    e = osp::launch_attn3d_bwd_packed(pa, int(kv_grid), int(q_grid), desc->head_dim, hs);
    if (e != hipSuccess) return device_error(e, "attn3d_packed_bwd launch");
  }
  return ok();
}

static osp_status skiparse_index_impl(const osp_attn3d_desc* d, int32_t mode, int32_t sparse_k,
                                      int64_t n_tokens, int32_t* perm, int32_t* inv,
                                      int32_t on_device, void* stream) {
  if (!perm && !inv) return fail(OSP_ERR_NULL, "perm and inv are both NULL");
  if (n_tokens < 0 || n_tokens > 0x7fffffffLL)
    return fail(OSP_ERR_SHAPE, "n_tokens %lld out of range", (long long)n_tokens);
  osp_status st = check_mode(d, n_tokens, mode, sparse_k);
  if (st) return st;
  const int32_t n = int32_t(n_tokens);
  const int32_t k = (mode == OSP_MODE_FULL) ? 1 : sparse_k;
  const osp::SkipDiv divk = skip_div(d, mode, k);
  if (on_device) {
    hipError_t e = osp::launch_skiparse_index(mode, divk, n, perm, inv,
                                              static_cast<hipStream_t>(stream));
    if (e != hipSuccess) return device_error(e, "skiparse_index launch");
    return ok();
  }
  const uint32_t len = uint32_t(n / k);
  for (uint32_t j = 0; j < uint32_t(k); ++j)
    for (uint32_t r = 0; r < len; ++r) {
      const uint32_t pos = j * len + r;
      const uint32_t i = osp::skiparse_token(mode, r, j, divk, len);
      if (perm) perm[pos] = int32_t(i);
      if (inv) inv[i] = int32_t(pos);
    }
  return ok();
}

osp_status osp_skiparse_index(int32_t mode, int32_t sparse_k, int64_t n_tokens, int32_t* perm,
                              int32_t* inv, int32_t on_device, void* stream) {
  return skiparse_index_impl(nullptr, mode, sparse_k, n_tokens, perm, inv, on_device, stream);
}

osp_status osp_skiparse_index3d(int32_t mode, int32_t sparse_k, int32_t grid_t, int32_t grid_h,
                                int32_t grid_w, int32_t* perm, int32_t* inv, int32_t on_device,
                                void* stream) {
  if (grid_t < 1 || grid_h < 1 || grid_w < 1)
    return fail(OSP_ERR_SHAPE, "grid %d x %d x %d must be positive", grid_t, grid_h, grid_w);
  osp_attn3d_desc d{};
  d.grid_t = grid_t;
  d.grid_h = grid_h;
  d.grid_w = grid_w;
  return skiparse_index_impl(&d, mode, sparse_k, int64_t(grid_t) * grid_h * grid_w, perm, inv,
                             on_device, stream);
}

}  // extern "C"
