// Device helpers shared by the bmattn kernels (gfx950, wave64).
//
// One definition of the element predicate, the per-sequence bounds and the
// paged address serves every kernel: the tile classifier, the forward
// kernels' partial tiles, the dense-mask export and the paged gather.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "../../include/bmattn.h"

namespace bmattn {

// Mask description as the kernels see it (kernel-argument friendly copy).
// Every kind is an OR of AND-groups of BMATTN_TERM_* bits, set by the host:
// `groups` holds up to four groups, group g in bits 4g .. 4g+3 (FULL: 0,
// which means every pair; CAUSAL: {causal}; SHARED_PREFIX / STRIP_THINKING:
// {causal, the id term}; COMPOSED: the description's terms).  `terms` is the
// union of the groups (which id arrays are read) and `causal_all` tells
// whether every group holds the causal term (then no pair above the
// diagonal is visible).
struct MaskDev {
  int32_t kind;
  int32_t n_seqs;
  int32_t think_role;
  int32_t terms;
  int32_t groups;
  int32_t causal_all;
  int64_t total_q, total_k;
  const int32_t* cu_q;
  const int32_t* cu_k;
  const int32_t* seg_q;
  const int32_t* seg_k;
  const int32_t* role_k;
  const int32_t* turn_q;
  const int32_t* turn_k;
  const int32_t* doc_q;
  const int32_t* doc_k;
};

// Bounds of one sequence, clamped so that every index derived from them lies
// inside [0, total) whatever the device arrays hold: a malformed cu_seqlens
// gives wrong values, never an out-of-range access.
struct SeqBounds {
  int64_t q0, k0;  // first packed query row / key row
  int32_t lq, lk;  // query and key counts (clamped to the tile grid)
};

__device__ __forceinline__ int64_t clamp64(int64_t x, int64_t lo, int64_t hi) {
  return x < lo ? lo : (x > hi ? hi : x);
}

__device__ __forceinline__ SeqBounds seq_bounds(const MaskDev& m, int s, int32_t max_lq,
                                                int32_t max_lk) {
  SeqBounds b;
  int64_t q0 = clamp64(m.cu_q[s], 0, m.total_q);
  int64_t q1 = clamp64(m.cu_q[s + 1], q0, m.total_q);
  int64_t k0 = clamp64(m.cu_k[s], 0, m.total_k);
  int64_t k1 = clamp64(m.cu_k[s + 1], k0, m.total_k);
  b.q0 = q0;
  b.k0 = k0;
  b.lq = (int32_t)((q1 - q0) < max_lq ? (q1 - q0) : max_lq);
  b.lk = (int32_t)((k1 - k0) < max_lk ? (k1 - k0) : max_lk);
  return b;
}

// Query-side ids of one query row (loaded once per row); the ids the
// kind's terms do not read stay 0.
struct QIds {
  int32_t seg, turn, doc;
};

__device__ __forceinline__ QIds load_qids(const MaskDev& m, const SeqBounds& b, int i) {
  QIds r{0, 0, 0};
  if (i < b.lq) {
    if (m.terms & BMATTN_TERM_SHARED_PREFIX) r.seg = m.seg_q[b.q0 + i];
    if (m.terms & BMATTN_TERM_STRIP_THINKING) r.turn = m.turn_q[b.q0 + i];
    if (m.terms & BMATTN_TERM_DOCUMENT) r.doc = m.doc_q[b.q0 + i];
  }
  return r;
}

// Key-side ids of one key.  Plain kinds: a = segment (shared-prefix) or
// role (strip-thinking), b = turn (strip-thinking).  COMPOSED: a = segment,
// b = role, c = turn, d = document.  Unread fields are 0.
struct KIds {
  int32_t a, b, c, d;
};

__device__ __forceinline__ KIds load_kids(const MaskDev& m, const SeqBounds& b, int j) {
  KIds r{0, 0, 0, 0};
  if (j < b.lk) {
    if (m.kind == BMATTN_MASK_SHARED_PREFIX) r.a = m.seg_k[b.k0 + j];
    if (m.kind == BMATTN_MASK_STRIP_THINKING) {
      r.a = m.role_k[b.k0 + j];
      r.b = m.turn_k[b.k0 + j];
    }
    if (m.kind == BMATTN_MASK_COMPOSED) {
      if (m.terms & BMATTN_TERM_SHARED_PREFIX) r.a = m.seg_k[b.k0 + j];
      if (m.terms & BMATTN_TERM_STRIP_THINKING) {
        r.b = m.role_k[b.k0 + j];
        r.c = m.turn_k[b.k0 + j];
      }
      if (m.terms & BMATTN_TERM_DOCUMENT) r.d = m.doc_k[b.k0 + j];
    }
  }
  return r;
}

// The id terms of a COMPOSED mask for one pair (no causal, no bounds):
// key ids in COMPOSED order (segment, role, turn, document).
__device__ __forceinline__ bool composed_ids_ok(int32_t terms, int32_t think_role, QIds q,
                                                int32_t kseg, int32_t krole, int32_t kturn,
                                                int32_t kdoc) {
  const bool doc = !(terms & BMATTN_TERM_DOCUMENT) | ((kdoc == q.doc) & (kdoc >= 0));
  const bool pre = !(terms & BMATTN_TERM_SHARED_PREFIX) | (kseg == 0) | (kseg == q.seg);
  const bool strip = !(terms & BMATTN_TERM_STRIP_THINKING) | !((krole == think_role) & (kturn < q.turn));
  return doc & pre & strip;
}

// One pair through an OR of AND-groups: visible when some non-empty group
// passes, its causal term on `causal_ok` (j <= p(i)) and its id terms on the
// ids.  groups == 0 (FULL) passes every pair.
__device__ __forceinline__ bool composed_ok(int32_t groups, int32_t think_role, bool causal_ok, QIds q,
                                            int32_t kseg, int32_t krole, int32_t kturn, int32_t kdoc) {
  if (groups == 0) return true;
  bool v = false;
  for (int32_t gs = groups; gs != 0; gs >>= 4) {  // wave-uniform: one pass per group
    const int32_t t = gs & 15;
    v |= (t != 0) & (!(t & BMATTN_TERM_CAUSAL) | causal_ok) &
         composed_ids_ok(t, think_role, q, kseg, krole, kturn, kdoc);
  }
  return v;
}

// Element predicate: is key j of the sequence visible to its query row i?
// Query row i sits at position lk - lq + i; the causal condition keeps the
// diagonal (j <= position).  Pairs outside the sequence are not visible.
// kid holds key j's ids (load_kids).  Branch-free, one instance per kind.
template <int KIND>
__device__ __forceinline__ bool visible_k(const MaskDev& m, const SeqBounds& b, int i, QIds qi,
                                          int j, KIds kid) {
  const bool in = (i < b.lq) & (j < b.lk);
  if constexpr (KIND == BMATTN_MASK_FULL) return in;
  const bool causal = in & (j <= b.lk - b.lq + i);
  if constexpr (KIND == BMATTN_MASK_CAUSAL) return causal;
  if constexpr (KIND == BMATTN_MASK_SHARED_PREFIX) return causal & ((kid.a == 0) | (kid.a == qi.seg));
  if constexpr (KIND == BMATTN_MASK_STRIP_THINKING)
    return causal & !((kid.a == m.think_role) & (kid.b < qi.turn));
  // COMPOSED
  return in & composed_ok(m.groups, m.think_role, j <= b.lk - b.lq + i, qi, kid.a, kid.b, kid.c, kid.d);
}

__device__ __forceinline__ bool visible_ids(const MaskDev& m, const SeqBounds& b, int i, QIds qi,
                                            int j, KIds kid) {
  switch (m.kind) {
    case BMATTN_MASK_FULL: return visible_k<BMATTN_MASK_FULL>(m, b, i, qi, j, kid);
    case BMATTN_MASK_CAUSAL: return visible_k<BMATTN_MASK_CAUSAL>(m, b, i, qi, j, kid);
    case BMATTN_MASK_SHARED_PREFIX: return visible_k<BMATTN_MASK_SHARED_PREFIX>(m, b, i, qi, j, kid);
    case BMATTN_MASK_STRIP_THINKING: return visible_k<BMATTN_MASK_STRIP_THINKING>(m, b, i, qi, j, kid);
    default: return visible_k<BMATTN_MASK_COMPOSED>(m, b, i, qi, j, kid);
  }
}

__device__ __forceinline__ bool visible(const MaskDev& m, const SeqBounds& b, int i, QIds qi,
                                        int j) {
  return visible_ids(m, b, i, qi, j, load_kids(m, b, j));
}

// Physical pool row of logical key j of sequence s in a paged K/V: page
// block_table[s][j / page_size], slot j % page_size.  Entries outside
// [0, num_pages) are clamped (bmattn_validate reports them).  page_shift is
// log2(page_size) when the page size is a power of two, else -1.
__device__ __forceinline__ int32_t page_of(int j, int32_t page_size, int32_t page_shift) {
  return page_shift >= 0 ? (j >> page_shift) : (j / page_size);
}

__device__ __forceinline__ int32_t page_entry(const int32_t* block_table, int64_t bt_stride, int s,
                                              int j, int32_t page_size, int32_t page_shift) {
  return block_table[(int64_t)s * bt_stride + page_of(j, page_size, page_shift)];
}

__device__ __forceinline__ int64_t row_in_page(int32_t entry, int j, int32_t page_size,
                                               int32_t page_shift, int64_t num_pages) {
  const int64_t pg = clamp64(entry, 0, num_pages - 1);
  const int32_t slot = page_shift >= 0 ? (j & (page_size - 1)) : (j % page_size);
  return pg * page_size + slot;
}

__device__ __forceinline__ int64_t paged_row(const int32_t* block_table, int64_t bt_stride, int s,
                                             int j, int32_t page_size, int32_t page_shift,
                                             int64_t num_pages) {
  return row_in_page(page_entry(block_table, bt_stride, s, j, page_size, page_shift), j, page_size,
                     page_shift, num_pages);
}

}  // namespace bmattn
