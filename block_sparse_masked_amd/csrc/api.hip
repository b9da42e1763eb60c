// C-ABI entry points of libbmattn: argument validation on the host, then the
// launches.  No allocation, no state between calls (the last-error text is
// thread-local), no exception crosses the boundary.
#include <hip/hip_runtime.h>

#include <cmath>
#include <cstdarg>
#include <cstdint>
#include <cstdio>
#include <string>

#include "../../include/bmattn.h"
#include "launch.h"

using namespace bmattn;

namespace {

thread_local std::string g_last_error;

int fail(int code, const char* fmt, ...) {
  char buf[512];
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(buf, sizeof(buf), fmt, ap);
  va_end(ap);
  g_last_error = buf;
  return code;
}

int hip_fail(hipError_t e, const char* what) {
  return fail(BMATTN_EHIP, "%s: %s", what, hipGetErrorString(e));
}

int64_t cdiv(int64_t a, int64_t b) { return (a + b - 1) / b; }

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

// Decode splits: consecutive entries of a row's kv-tile list per workgroup.
constexpr int32_t kDecodeSplitTiles = 8;

// The union of a COMPOSED description's term groups (4-bit nibbles).
int32_t term_union(int32_t groups) {
  return (groups | (groups >> 4) | (groups >> 8) | (groups >> 12)) & 15;
}

int check_desc(const bmattn_mask_desc* d) {
  if (d == nullptr) return fail(BMATTN_EINVAL, "mask description is NULL");
  if (d->kind < BMATTN_MASK_FULL || d->kind > BMATTN_MASK_COMPOSED)
    return fail(BMATTN_EINVAL, "unknown mask kind %d", d->kind);
  if (d->n_seqs < 1) return fail(BMATTN_EINVAL, "n_seqs must be >= 1 (got %d)", d->n_seqs);
  if (d->max_seqlen_q < 1 || d->max_seqlen_k < 1)
    return fail(BMATTN_EINVAL, "max_seqlen_q/k must be >= 1 (got %d, %d)", d->max_seqlen_q,
                d->max_seqlen_k);
  if (d->total_q < 0 || d->total_k < 0) return fail(BMATTN_EINVAL, "negative total_q/total_k");
  if (d->total_q > INT32_MAX || d->total_k > INT32_MAX)
    return fail(BMATTN_EINVAL, "total_q/total_k exceed int32 (cu_seqlens are int32)");
  if (d->cu_seqlens_q == nullptr || d->cu_seqlens_k == nullptr)
    return fail(BMATTN_EINVAL, "cu_seqlens_q/k must be non-NULL");
  if (d->kind == BMATTN_MASK_SHARED_PREFIX && (d->seg_q == nullptr || d->seg_k == nullptr))
    return fail(BMATTN_EINVAL, "SHARED_PREFIX needs seg_q and seg_k");
  if (d->kind == BMATTN_MASK_STRIP_THINKING &&
      (d->role_k == nullptr || d->turn_q == nullptr || d->turn_k == nullptr))
    return fail(BMATTN_EINVAL, "STRIP_THINKING needs role_k, turn_q and turn_k");
  if (d->kind == BMATTN_MASK_COMPOSED) {
    if (d->terms <= 0 || d->terms > 0xffff)
      return fail(BMATTN_EINVAL,
                  "COMPOSED needs terms: up to four groups of BMATTN_TERM_* bits, group g in bits "
                  "4g..4g+3, at least one non-empty (got %d)",
                  d->terms);
    const int32_t any = term_union(d->terms);
    if ((any & BMATTN_TERM_DOCUMENT) && (d->doc_q == nullptr || d->doc_k == nullptr))
      return fail(BMATTN_EINVAL, "the DOCUMENT term needs doc_q and doc_k");
    if ((any & BMATTN_TERM_SHARED_PREFIX) && (d->seg_q == nullptr || d->seg_k == nullptr))
      return fail(BMATTN_EINVAL, "the SHARED_PREFIX term needs seg_q and seg_k");
    if ((any & BMATTN_TERM_STRIP_THINKING) &&
        (d->role_k == nullptr || d->turn_q == nullptr || d->turn_k == nullptr))
      return fail(BMATTN_EINVAL, "the STRIP_THINKING term needs role_k, turn_q and turn_k");
  } else if (d->terms != 0) {
    return fail(BMATTN_EINVAL, "terms must be 0 unless the kind is COMPOSED (got %d)", d->terms);
  }
  return BMATTN_OK;
}

MaskDev to_dev(const bmattn_mask_desc* d) {
  MaskDev m{};
  m.kind = d->kind;
  m.n_seqs = d->n_seqs;
  m.think_role = d->think_role;
  switch (d->kind) {
    case BMATTN_MASK_FULL: m.groups = 0; break;
    case BMATTN_MASK_CAUSAL: m.groups = BMATTN_TERM_CAUSAL; break;
    case BMATTN_MASK_SHARED_PREFIX: m.groups = BMATTN_TERM_CAUSAL | BMATTN_TERM_SHARED_PREFIX; break;
    case BMATTN_MASK_STRIP_THINKING: m.groups = BMATTN_TERM_CAUSAL | BMATTN_TERM_STRIP_THINKING; break;
    default: m.groups = d->terms; break;
  }
  m.terms = term_union(m.groups);
  m.causal_all = m.groups != 0;
  for (int g = 0; g < 4; ++g) {
    const int32_t t = (m.groups >> (4 * g)) & 15;
    if (t != 0 && !(t & BMATTN_TERM_CAUSAL)) m.causal_all = 0;
  }
  m.total_q = d->total_q;
  m.total_k = d->total_k;
  m.cu_q = d->cu_seqlens_q;
  m.cu_k = d->cu_seqlens_k;
  m.seg_q = d->seg_q;
  m.seg_k = d->seg_k;
  m.role_k = d->role_k;
  m.turn_q = d->turn_q;
  m.turn_k = d->turn_k;
  m.doc_q = d->doc_q;
  m.doc_k = d->doc_k;
  return m;
}

int shape(const bmattn_mask_desc* d, int32_t bm, int32_t bn, int32_t* n_qt, int32_t* n_kt,
          int64_t* rows, int64_t* tiles) {
  if (bm < 1 || bm > 1024 || bn < 1 || bn > 1024)
    return fail(BMATTN_EUNSUPPORTED, "block_m/block_n must lie in [1, 1024] (got %d, %d)", bm, bn);
  const int64_t qt = cdiv(d->max_seqlen_q, bm), kt = cdiv(d->max_seqlen_k, bn);
  const int64_t r = qt * d->n_seqs;
  if (r > INT32_MAX || r * kt > ((int64_t)1 << 40))
    return fail(BMATTN_EINVAL, "block mask too large (%lld rows x %lld tiles)", (long long)r,
                (long long)kt);
  *n_qt = (int32_t)qt;
  *n_kt = (int32_t)kt;
  *rows = r;
  *tiles = r * kt;
  return BMATTN_OK;
}

int check_tiles(const bmattn_mask_desc* d, const bmattn_block_mask* t, bool need_write) {
  if (t == nullptr) return fail(BMATTN_EINVAL, "block mask is NULL");
  int32_t n_qt, n_kt;
  int64_t rows, tiles;
  int rc = shape(d, t->block_m, t->block_n, &n_qt, &n_kt, &rows, &tiles);
  if (rc) return rc;
  if (t->n_seqs != d->n_seqs || t->n_qt != n_qt || t->n_kt != n_kt)
    return fail(BMATTN_EINVAL,
                "block mask shape (n_seqs %d, n_qt %d, n_kt %d) does not match the description "
                "(n_seqs %d, n_qt %d, n_kt %d)",
                t->n_seqs, t->n_qt, t->n_kt, d->n_seqs, n_qt, n_kt);
  if (t->full_cnt == nullptr || t->part_cnt == nullptr || t->full_idx == nullptr ||
      t->part_idx == nullptr || t->row_order == nullptr || (need_write && t->tile_class == nullptr))
    return fail(BMATTN_EINVAL, "block mask array is NULL");
  return BMATTN_OK;
}

// A launch puts one workgroup on each (tile row or column, head); the grid
// must fit the 32-bit dispatch size.
int check_grid(int64_t units, int32_t heads, const char* what) {
  if (units * (int64_t)heads > (int64_t)INT32_MAX)
    return fail(BMATTN_EUNSUPPORTED, "%s grid of %lld tile rows x %d heads exceeds 2^31 - 1 workgroups",
                what, (long long)units, heads);
  return BMATTN_OK;
}

TilesDev tiles_dev(const bmattn_mask_desc* d, const bmattn_block_mask* t) {
  TilesDev x{};
  x.block_m = t->block_m;
  x.block_n = t->block_n;
  x.n_seqs = t->n_seqs;
  x.n_qt = t->n_qt;
  x.n_kt = t->n_kt;
  x.max_lq = d->max_seqlen_q;
  x.max_lk = d->max_seqlen_k;
  x.tile_class = t->tile_class;
  x.full_cnt = t->full_cnt;
  x.part_cnt = t->part_cnt;
  x.full_idx = t->full_idx;
  x.part_idx = t->part_idx;
  x.row_order = t->row_order;
  return x;
}

enum class Path { kPrefill, kDecode, kNone };

Path path_of(const bmattn_block_mask* t) {
  if (t->block_m == 128 && t->block_n == 64) return Path::kPrefill;
  if (t->block_m == 1 && t->block_n == 64) return Path::kDecode;
  return Path::kNone;
}

size_t decode_workspace(const bmattn_fwd_args* a, const bmattn_block_mask* t) {
  const int64_t rows = (int64_t)t->n_seqs * t->n_qt;
  const int64_t splits = cdiv(t->n_kt, kDecodeSplitTiles);
  return (size_t)(rows * splits * a->num_heads * (a->head_dim + 2)) * sizeof(float);
}

int check_fwd(const bmattn_fwd_args* a, const bmattn_mask_desc* d, const bmattn_block_mask* t) {
  if (a == nullptr) return fail(BMATTN_EINVAL, "forward arguments are NULL");
  int rc = check_desc(d);
  if (rc) return rc;
  rc = check_tiles(d, t, false);
  if (rc) return rc;
  if (a->dtype != BMATTN_F32 && a->dtype != BMATTN_BF16)
    return fail(BMATTN_EUNSUPPORTED, "dtype %d is not compiled (F32 = 0, BF16 = 1)", a->dtype);
  if (a->head_dim != 64 && a->head_dim != 128)
    return fail(BMATTN_EUNSUPPORTED, "head_dim %d is not compiled (64 or 128)", a->head_dim);
  if (a->num_heads < 1) return fail(BMATTN_EINVAL, "num_heads must be >= 1");
  if (path_of(t) == Path::kNone)
    return fail(BMATTN_EUNSUPPORTED,
                "tile shape %dx%d is not compiled for the forward (128x64 or 1x64)", t->block_m,
                t->block_n);
  if (a->q == nullptr || a->k == nullptr || a->v == nullptr || a->o == nullptr)
    return fail(BMATTN_EINVAL, "q, k, v and o must be non-NULL");
  const int64_t eb = a->dtype == BMATTN_BF16 ? 2 : 4;
  if (!aligned16(a->q) || !aligned16(a->k) || !aligned16(a->v) || !aligned16(a->o))
    return fail(BMATTN_EALIGN, "q, k, v and o must be 16-byte aligned");
  const int64_t strides[8] = {a->q_stride_tok, a->q_stride_head, a->k_stride_tok, a->k_stride_head,
                              a->v_stride_tok, a->v_stride_head, a->o_stride_tok, a->o_stride_head};
  for (int i = 0; i < 8; ++i) {
    if (strides[i] < 0) return fail(BMATTN_EINVAL, "negative stride");
    if ((strides[i] * eb) % 16 != 0)
      return fail(BMATTN_EALIGN, "token/head strides must be multiples of 16 bytes");
  }
  if (a->block_table != nullptr) {
    if (a->page_size < 1) return fail(BMATTN_EINVAL, "page_size must be >= 1");
    if (a->num_pages < 1) return fail(BMATTN_EINVAL, "num_pages must be >= 1");
    if (a->block_table_stride < cdiv(d->max_seqlen_k, a->page_size))
      return fail(BMATTN_EINVAL,
                  "block_table_stride %lld is smaller than ceil(max_seqlen_k / page_size) = %lld",
                  (long long)a->block_table_stride,
                  (long long)cdiv(d->max_seqlen_k, a->page_size));
  }
  if (a->lse != nullptr && a->lse_stride_head < d->total_q)
    return fail(BMATTN_EINVAL, "lse_stride_head must be >= total_q");
  if (!(std::isfinite(a->scale)) || a->scale < 0.f)
    return fail(BMATTN_EINVAL, "scale must be finite and >= 0 (0 selects 1/sqrt(head_dim))");
  return check_grid((int64_t)t->n_seqs * t->n_qt, a->num_heads, "forward");
}

int check_cols(const bmattn_block_mask* t, const bmattn_block_mask_cols* c) {
  if (c == nullptr) return fail(BMATTN_EINVAL, "column lists are NULL");
  if (c->block_m != t->block_m || c->block_n != t->block_n || c->n_seqs != t->n_seqs ||
      c->n_qt != t->n_qt || c->n_kt != t->n_kt)
    return fail(BMATTN_EINVAL,
                "column lists shape (%dx%d, n_seqs %d, n_qt %d, n_kt %d) does not match the block "
                "mask (%dx%d, n_seqs %d, n_qt %d, n_kt %d)",
                c->block_m, c->block_n, c->n_seqs, c->n_qt, c->n_kt, t->block_m, t->block_n,
                t->n_seqs, t->n_qt, t->n_kt);
  if (c->full_cnt == nullptr || c->part_cnt == nullptr || c->full_idx == nullptr ||
      c->part_idx == nullptr || c->col_order == nullptr)
    return fail(BMATTN_EINVAL, "column list array is NULL");
  return BMATTN_OK;
}

ColsDev cols_dev(const bmattn_block_mask_cols* c) {
  ColsDev x{};
  x.n_seqs = c->n_seqs;
  x.n_qt = c->n_qt;
  x.n_kt = c->n_kt;
  x.full_cnt = c->full_cnt;
  x.part_cnt = c->part_cnt;
  x.full_idx = c->full_idx;
  x.part_idx = c->part_idx;
  x.col_order = c->col_order;
  return x;
}

size_t bwd_workspace(const bmattn_bwd_args* a, const bmattn_mask_desc* d) {
  return (size_t)(2 * (int64_t)a->num_heads * d->total_q) * sizeof(float);
}

// dtype, head_dim and head count (all the workspace size depends on).
int check_bwd_shape(const bmattn_bwd_args* a, const bmattn_mask_desc* d) {
  if (a == nullptr) return fail(BMATTN_EINVAL, "backward arguments are NULL");
  int rc = check_desc(d);
  if (rc) return rc;
  if (a->dtype != BMATTN_BF16)
    return fail(BMATTN_EUNSUPPORTED, "the backward is compiled for BF16 only (got dtype %d)", a->dtype);
  if (a->head_dim != 64 && a->head_dim != 128)
    return fail(BMATTN_EUNSUPPORTED, "head_dim %d is not compiled (64 or 128)", a->head_dim);
  if (a->num_heads < 1) return fail(BMATTN_EINVAL, "num_heads must be >= 1");
  return BMATTN_OK;
}

int check_bwd(const bmattn_bwd_args* a, const bmattn_mask_desc* d) {
  int rc = check_bwd_shape(a, d);
  if (rc) return rc;
  const void* ptrs[9] = {a->q, a->k, a->v, a->o, a->dout, a->dq, a->dk, a->dv, a->lse};
  for (const void* x : ptrs)
    if (x == nullptr) return fail(BMATTN_EINVAL, "q, k, v, o, dout, lse, dq, dk and dv must be non-NULL");
  for (int i = 0; i < 8; ++i)
    if (!aligned16(ptrs[i])) return fail(BMATTN_EALIGN, "q, k, v, o, dout, dq, dk and dv must be 16-byte aligned");
  const int64_t strides[16] = {a->q_stride_tok,  a->q_stride_head,  a->k_stride_tok,  a->k_stride_head,
                               a->v_stride_tok,  a->v_stride_head,  a->o_stride_tok,  a->o_stride_head,
                               a->do_stride_tok, a->do_stride_head, a->dq_stride_tok, a->dq_stride_head,
                               a->dk_stride_tok, a->dk_stride_head, a->dv_stride_tok, a->dv_stride_head};
  for (int i = 0; i < 16; ++i) {
    if (strides[i] < 0) return fail(BMATTN_EINVAL, "negative stride");
    if ((strides[i] * 2) % 16 != 0)
      return fail(BMATTN_EALIGN, "token/head strides must be multiples of 16 bytes");
  }
  if (a->lse_stride_head < d->total_q) return fail(BMATTN_EINVAL, "lse_stride_head must be >= total_q");
  if (!(std::isfinite(a->scale)) || a->scale < 0.f)
    return fail(BMATTN_EINVAL, "scale must be finite and >= 0 (0 selects 1/sqrt(head_dim))");
  return BMATTN_OK;
}

}  // namespace

extern "C" {

int bmattn_abi_version(void) { return BMATTN_ABI_VERSION; }

const char* bmattn_last_error(void) { return g_last_error.c_str(); }

const char* bmattn_status_string(int status) {
  switch (status) {
    case BMATTN_OK: return "ok";
    case BMATTN_EINVAL: return "invalid argument";
    case BMATTN_EUNSUPPORTED: return "unsupported configuration";
    case BMATTN_EALIGN: return "misaligned pointer or stride";
    case BMATTN_EHIP: return "HIP runtime error";
    case BMATTN_EWORKSPACE: return "workspace missing or too small";
    default: return "unknown status";
  }
}

int bmattn_block_mask_shape(const bmattn_mask_desc* desc, int32_t block_m, int32_t block_n,
                            int32_t* n_qt, int32_t* n_kt, int64_t* rows, int64_t* tiles) {
  int rc = check_desc(desc);
  if (rc) return rc;
  if (!n_qt || !n_kt || !rows || !tiles) return fail(BMATTN_EINVAL, "output pointer is NULL");
  return shape(desc, block_m, block_n, n_qt, n_kt, rows, tiles);
}

int bmattn_build_block_mask(const bmattn_mask_desc* desc, const bmattn_block_mask* out,
                            void* stream) {
  int rc = check_desc(desc);
  if (rc) return rc;
  rc = check_tiles(desc, out, true);
  if (rc) return rc;
  hipError_t e = launch_build_block_mask(to_dev(desc), tiles_dev(desc, out),
                                         static_cast<hipStream_t>(stream));
  if (e != hipSuccess) return hip_fail(e, "bmattn_build_block_mask launch");
  return BMATTN_OK;
}

int bmattn_forward_workspace_size(const bmattn_fwd_args* args, const bmattn_mask_desc* desc,
                                  const bmattn_block_mask* tiles, size_t* bytes) {
  if (bytes == nullptr) return fail(BMATTN_EINVAL, "bytes is NULL");
  int rc = check_fwd(args, desc, tiles);
  if (rc) return rc;
  *bytes = path_of(tiles) == Path::kDecode ? decode_workspace(args, tiles) : 0;
  return BMATTN_OK;
}

}  // extern "C"

namespace {

// The forward of both entry points: `noalloc` takes the decode split
// workspace from the library's static scratch instead of args->workspace.
int forward_run(const bmattn_fwd_args* a, const bmattn_mask_desc* desc, const bmattn_block_mask* t,
                void* stream, bool noalloc) {
  int rc = check_fwd(a, desc, t);
  if (rc) return rc;
  const Path path = path_of(t);
  FwdDev p{};
  p.mask = to_dev(desc);
  p.block_m = t->block_m;
  p.block_n = t->block_n;
  p.n_qt = t->n_qt;
  p.n_kt = t->n_kt;
  p.max_lq = desc->max_seqlen_q;
  p.max_lk = desc->max_seqlen_k;
  p.full_cnt = t->full_cnt;
  p.part_cnt = t->part_cnt;
  p.full_idx = t->full_idx;
  p.part_idx = t->part_idx;
  p.row_order = t->row_order;
  p.num_heads = a->num_heads;
  p.head_dim = a->head_dim;
  p.q = a->q;
  p.k = a->k;
  p.v = a->v;
  p.o = a->o;
  p.lse = a->lse;
  p.q_st = a->q_stride_tok;
  p.q_sh = a->q_stride_head;
  p.k_st = a->k_stride_tok;
  p.k_sh = a->k_stride_head;
  p.v_st = a->v_stride_tok;
  p.v_sh = a->v_stride_head;
  p.o_st = a->o_stride_tok;
  p.o_sh = a->o_stride_head;
  p.lse_sh = a->lse_stride_head;
  p.block_table = a->block_table;
  p.bt_stride = a->block_table_stride;
  p.num_pages = a->num_pages;
  p.page_size = a->page_size;
  p.page_shift = page_shift_of(a->page_size);
  const float scale = a->scale > 0.f ? a->scale : 1.0f / std::sqrt((float)a->head_dim);
  p.scale_log2 = scale * 1.4426950408889634f;
  const bool paged = a->block_table != nullptr;
  hipStream_t st = static_cast<hipStream_t>(stream);
  hipError_t e;
  if (noalloc && a->workspace != nullptr)
    return fail(BMATTN_EINVAL, "bmattn_forward_noalloc takes no workspace (it uses the library's "
                               "static scratch): pass workspace = NULL");
  if (path == Path::kDecode) {
    const size_t need = decode_workspace(a, t);
    if (noalloc) {
      if (need > decode_scratch_bytes())
        return fail(BMATTN_EWORKSPACE,
                    "this decode needs %zu bytes of split workspace; the static scratch of "
                    "bmattn_forward_noalloc holds %zu (use bmattn_forward with a workspace)",
                    need, decode_scratch_bytes());
      if (st != nullptr) {
        int sdev = -1, cdev = -1;
        hipError_t e2 = hipStreamGetDevice(st, &sdev);
        if (e2 != hipSuccess) return hip_fail(e2, "hipStreamGetDevice");
        e2 = hipGetDevice(&cdev);
        if (e2 != hipSuccess) return hip_fail(e2, "hipGetDevice");
        if (sdev != cdev)
          return fail(BMATTN_EINVAL, "the stream's device (%d) is not the current device (%d)",
                      sdev, cdev);
      }
      void* ws = nullptr;
      hipError_t e2 = decode_scratch(&ws);
      if (e2 != hipSuccess) return hip_fail(e2, "static scratch address");
      p.ws = static_cast<float*>(ws);
    } else {
      if (a->workspace == nullptr || a->workspace_bytes < need)
        return fail(BMATTN_EWORKSPACE, "decode needs a workspace of %zu bytes (got %zu)", need,
                    a->workspace == nullptr ? (size_t)0 : a->workspace_bytes);
      if (!aligned16(a->workspace)) return fail(BMATTN_EALIGN, "workspace must be 16-byte aligned");
      p.ws = static_cast<float*>(a->workspace);
    }
    p.split_tiles = kDecodeSplitTiles;
    p.n_splits = (int32_t)cdiv(t->n_kt, kDecodeSplitTiles);
    e = launch_forward_decode(p, a->dtype, paged, st);
  } else {
    e = launch_forward_prefill(p, a->dtype, paged, st);
  }
  if (e != hipSuccess) return hip_fail(e, "bmattn_forward launch");
  return BMATTN_OK;
}

}  // namespace

extern "C" {

int bmattn_forward(const bmattn_fwd_args* a, const bmattn_mask_desc* desc,
                   const bmattn_block_mask* t, void* stream) {
  return forward_run(a, desc, t, stream, false);
}

int bmattn_forward_noalloc(const bmattn_fwd_args* a, const bmattn_mask_desc* desc,
                           const bmattn_block_mask* t, void* stream) {
  return forward_run(a, desc, t, stream, true);
}

int bmattn_transpose_block_mask(const bmattn_block_mask* tiles, const bmattn_block_mask_cols* out,
                                void* stream) {
  if (tiles == nullptr) return fail(BMATTN_EINVAL, "block mask is NULL");
  if (tiles->tile_class == nullptr) return fail(BMATTN_EINVAL, "tile_class is NULL");
  if (tiles->n_seqs < 1 || tiles->n_qt < 1 || tiles->n_kt < 1)
    return fail(BMATTN_EINVAL, "block mask shape must be positive");
  int rc = check_cols(tiles, out);
  if (rc) return rc;
  if (out->full_cnt == nullptr) return fail(BMATTN_EINVAL, "column list array is NULL");
  TilesDev t{};
  t.block_m = tiles->block_m;
  t.block_n = tiles->block_n;
  t.n_seqs = tiles->n_seqs;
  t.n_qt = tiles->n_qt;
  t.n_kt = tiles->n_kt;
  t.tile_class = tiles->tile_class;
  hipError_t e = launch_transpose_block_mask(t, cols_dev(out), static_cast<hipStream_t>(stream));
  if (e != hipSuccess) return hip_fail(e, "bmattn_transpose_block_mask launch");
  return BMATTN_OK;
}

int bmattn_backward_workspace_size(const bmattn_bwd_args* args, const bmattn_mask_desc* desc,
                                   size_t* bytes) {
  if (bytes == nullptr) return fail(BMATTN_EINVAL, "bytes is NULL");
  int rc = check_bwd_shape(args, desc);
  if (rc) return rc;
  *bytes = bwd_workspace(args, desc);
  return BMATTN_OK;
}

int bmattn_backward(const bmattn_bwd_args* a, const bmattn_mask_desc* desc,
                    const bmattn_block_mask* rows, const bmattn_block_mask_cols* cols,
                    void* stream) {
  int rc = check_bwd(a, desc);
  if (rc) return rc;
  rc = check_tiles(desc, rows, false);
  if (rc) return rc;
  if (rows->block_m != 128 || rows->block_n != 64)
    return fail(BMATTN_EUNSUPPORTED, "rows must be a 128x64 block mask (got %dx%d)", rows->block_m,
                rows->block_n);
  if (cols == nullptr) return fail(BMATTN_EINVAL, "column lists are NULL");
  if (cols->block_m != 64 || cols->block_n != 128)
    return fail(BMATTN_EUNSUPPORTED, "cols must come from a 64x128 block mask (got %dx%d)",
                cols->block_m, cols->block_n);
  int32_t cq, ck;
  int64_t crows, ctiles;
  rc = shape(desc, 64, 128, &cq, &ck, &crows, &ctiles);
  if (rc) return rc;
  if (cols->n_seqs != desc->n_seqs || cols->n_qt != cq || cols->n_kt != ck)
    return fail(BMATTN_EINVAL, "column lists shape does not match the description");
  if (cols->full_cnt == nullptr || cols->part_cnt == nullptr || cols->full_idx == nullptr ||
      cols->part_idx == nullptr || cols->col_order == nullptr)
    return fail(BMATTN_EINVAL, "column list array is NULL");
  rc = check_grid((int64_t)rows->n_seqs * rows->n_qt, a->num_heads, "backward dQ");
  if (rc) return rc;
  rc = check_grid((int64_t)cols->n_seqs * cols->n_kt, a->num_heads, "backward dK/dV");
  if (rc) return rc;
  const size_t need = bwd_workspace(a, desc);
  if (need > 0 && (a->workspace == nullptr || a->workspace_bytes < need))
    return fail(BMATTN_EWORKSPACE, "the backward needs a workspace of %zu bytes (got %zu)", need,
                a->workspace == nullptr ? (size_t)0 : a->workspace_bytes);
  if (need > 0 && !aligned16(a->workspace)) return fail(BMATTN_EALIGN, "workspace must be 16-byte aligned");
  BwdDev p{};
  p.mask = to_dev(desc);
  p.max_lq = desc->max_seqlen_q;
  p.max_lk = desc->max_seqlen_k;
  p.n_qt = rows->n_qt;
  p.n_kt = rows->n_kt;
  p.full_cnt = rows->full_cnt;
  p.part_cnt = rows->part_cnt;
  p.full_idx = rows->full_idx;
  p.part_idx = rows->part_idx;
  p.row_order = rows->row_order;
  p.c_n_qt = cols->n_qt;
  p.c_n_kt = cols->n_kt;
  p.c_full_cnt = cols->full_cnt;
  p.c_part_cnt = cols->part_cnt;
  p.c_full_idx = cols->full_idx;
  p.c_part_idx = cols->part_idx;
  p.col_order = cols->col_order;
  p.num_heads = a->num_heads;
  p.head_dim = a->head_dim;
  p.q = a->q;
  p.k = a->k;
  p.v = a->v;
  p.o = a->o;
  p.dout = a->dout;
  p.dq = a->dq;
  p.dk = a->dk;
  p.dv = a->dv;
  p.lse = a->lse;
  p.q_st = a->q_stride_tok;
  p.q_sh = a->q_stride_head;
  p.k_st = a->k_stride_tok;
  p.k_sh = a->k_stride_head;
  p.v_st = a->v_stride_tok;
  p.v_sh = a->v_stride_head;
  p.o_st = a->o_stride_tok;
  p.o_sh = a->o_stride_head;
  p.do_st = a->do_stride_tok;
  p.do_sh = a->do_stride_head;
  p.dq_st = a->dq_stride_tok;
  p.dq_sh = a->dq_stride_head;
  p.dk_st = a->dk_stride_tok;
  p.dk_sh = a->dk_stride_head;
  p.dv_st = a->dv_stride_tok;
  p.dv_sh = a->dv_stride_head;
  p.lse_sh = a->lse_stride_head;
  const float scale = a->scale > 0.f ? a->scale : 1.0f / std::sqrt((float)a->head_dim);
  p.scale = scale;
  p.scale_log2 = scale * 1.4426950408889634f;
  float* ws = static_cast<float*>(a->workspace);
  p.ws_di = ws;
  p.ws_l2 = ws == nullptr ? nullptr : ws + (int64_t)a->num_heads * desc->total_q;
  hipError_t e = launch_backward_bf16(p, static_cast<hipStream_t>(stream));
  if (e != hipSuccess) return hip_fail(e, "bmattn_backward launch");
  return BMATTN_OK;
}

int bmattn_paged_gather(const void* pool, int64_t pool_stride_tok, int64_t pool_stride_head,
                        int32_t elem_bytes, int32_t num_heads, int32_t head_dim,
                        int32_t page_size, int64_t num_pages, const int32_t* block_table,
                        int64_t block_table_stride, const bmattn_mask_desc* desc, void* out,
                        void* stream) {
  int rc = check_desc(desc);
  if (rc) return rc;
  if (pool == nullptr || out == nullptr || block_table == nullptr)
    return fail(BMATTN_EINVAL, "pool, block_table and out must be non-NULL");
  if (elem_bytes != 2 && elem_bytes != 4) return fail(BMATTN_EINVAL, "elem_bytes must be 2 or 4");
  if (num_heads < 1 || head_dim < 1) return fail(BMATTN_EINVAL, "num_heads/head_dim must be >= 1");
  if ((head_dim * elem_bytes) % 16 != 0 || (pool_stride_tok * elem_bytes) % 16 != 0 ||
      (pool_stride_head * elem_bytes) % 16 != 0 || !aligned16(pool) || !aligned16(out))
    return fail(BMATTN_EALIGN, "rows, strides and pointers must be 16-byte aligned");
  if (page_size < 1 || num_pages < 1) return fail(BMATTN_EINVAL, "page_size/num_pages must be >= 1");
  if (block_table_stride < cdiv(desc->max_seqlen_k, page_size))
    return fail(BMATTN_EINVAL, "block_table_stride smaller than ceil(max_seqlen_k / page_size)");
  hipError_t e = launch_paged_gather(to_dev(desc), desc->max_seqlen_k, pool, pool_stride_tok,
                                     pool_stride_head, elem_bytes, num_heads, head_dim, page_size,
                                     num_pages, block_table, block_table_stride, out,
                                     static_cast<hipStream_t>(stream));
  if (e != hipSuccess) return hip_fail(e, "bmattn_paged_gather launch");
  return BMATTN_OK;
}

int bmattn_debug_dense_mask(const bmattn_mask_desc* desc, const bmattn_block_mask* tiles,
                            int32_t seq, uint8_t* out, int64_t out_stride, void* stream) {
  int rc = check_desc(desc);
  if (rc) return rc;
  rc = check_tiles(desc, tiles, true);
  if (rc) return rc;
  if (seq < 0 || seq >= desc->n_seqs) return fail(BMATTN_EINVAL, "seq %d out of range", seq);
  if (out == nullptr) return fail(BMATTN_EINVAL, "out is NULL");
  if (out_stride < (int64_t)tiles->n_kt * tiles->block_n)
    return fail(BMATTN_EINVAL, "out_stride must be >= n_kt * block_n");
  hipError_t e = launch_debug_dense_mask(to_dev(desc), tiles_dev(desc, tiles), seq, out,
                                         out_stride, static_cast<hipStream_t>(stream));
  if (e != hipSuccess) return hip_fail(e, "bmattn_debug_dense_mask launch");
  return BMATTN_OK;
}

int bmattn_validate(const bmattn_mask_desc* desc, const int32_t* block_table,
                    int64_t block_table_stride, int32_t page_size, int64_t num_pages,
                    int32_t* flags, void* stream) {
  int rc = check_desc(desc);
  if (rc) return rc;
  if (flags == nullptr) return fail(BMATTN_EINVAL, "flags is NULL");
  if (block_table != nullptr && (page_size < 1 || num_pages < 1 || block_table_stride < 1))
    return fail(BMATTN_EINVAL, "page_size, num_pages and block_table_stride must be >= 1");
  hipError_t e = launch_validate(to_dev(desc), desc->max_seqlen_q, desc->max_seqlen_k, block_table,
                                 block_table_stride, page_size, num_pages, flags,
                                 static_cast<hipStream_t>(stream));
  if (e != hipSuccess) return hip_fail(e, "bmattn_validate launch");
  return BMATTN_OK;
}

int bmattn_duplicated_answer_ids(const bmattn_mask_desc* desc, const int32_t* role_q,
                                 int32_t loss_role, int32_t history_role, int32_t* role_k_out,
                                 int32_t* turn_q_out, int32_t* flags, void* stream) {
  int rc = check_desc(desc);
  if (rc) return rc;
  if (desc->kind != BMATTN_MASK_STRIP_THINKING)
    return fail(BMATTN_EINVAL, "duplicated answers need a STRIP_THINKING description");
  if (role_q == nullptr || role_k_out == nullptr || turn_q_out == nullptr)
    return fail(BMATTN_EINVAL, "role_q, role_k_out and turn_q_out must be non-NULL");
  if (loss_role == history_role || loss_role == desc->think_role ||
      history_role == desc->think_role)
    return fail(BMATTN_EINVAL, "think, loss and history roles must differ (%d, %d, %d)",
                desc->think_role, loss_role, history_role);
  hipError_t e = launch_duplicated_answer_ids(to_dev(desc), desc->max_seqlen_q, desc->max_seqlen_k,
                                              role_q, loss_role, history_role, role_k_out,
                                              turn_q_out, flags, static_cast<hipStream_t>(stream));
  if (e != hipSuccess) return hip_fail(e, "bmattn_duplicated_answer_ids launch");
  return BMATTN_OK;
}

}  // extern "C"
