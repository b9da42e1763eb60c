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
struct MaskDev {
  int32_t kind;
  int32_t n_seqs;
  int32_t think_role;
  int32_t pad0;
  int64_t total_q, total_k;
  const int32_t* cu_q;
  const int32_t* cu_k;
  const int32_t* seg_q;
  const int32_t* seg_k;
  const int32_t* role_k;
  const int32_t* turn_q;
  const int32_t* turn_k;
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

// Query-side ids of one query row (loaded once per row).
struct QIds {
  int32_t seg, turn;
};

__device__ __forceinline__ QIds load_qids(const MaskDev& m, const SeqBounds& b, int i) {
  QIds r{0, 0};
  if (i < b.lq) {
    if (m.kind == BMATTN_MASK_SHARED_PREFIX) r.seg = m.seg_q[b.q0 + i];
    if (m.kind == BMATTN_MASK_STRIP_THINKING) r.turn = m.turn_q[b.q0 + i];
  }
  return r;
}

// Element predicate: is key j of the sequence visible to its query row i?
// Query row i sits at position lk - lq + i; the causal condition keeps the
// diagonal (j <= position).  Pairs outside the sequence are not visible.
__device__ __forceinline__ bool visible(const MaskDev& m, const SeqBounds& b, int i, QIds qi,
                                        int j) {
  if (i >= b.lq || j >= b.lk) return false;
  if (m.kind == BMATTN_MASK_FULL) return true;
  if (j > b.lk - b.lq + i) return false;
  if (m.kind == BMATTN_MASK_SHARED_PREFIX) {
    int32_t sk = m.seg_k[b.k0 + j];
    return sk == 0 || sk == qi.seg;
  }
  if (m.kind == BMATTN_MASK_STRIP_THINKING) {
    return !(m.role_k[b.k0 + j] == m.think_role && m.turn_k[b.k0 + j] < qi.turn);
  }
  return true;  // CAUSAL
}

// Physical pool row of logical key j of sequence s in a paged K/V.  Entries
// outside [0, num_pages) are clamped (bmattn_validate reports them).
__device__ __forceinline__ int64_t paged_row(const int32_t* block_table, int64_t bt_stride, int s,
                                             int j, int32_t page_size, int64_t num_pages) {
  int32_t pg = block_table[(int64_t)s * bt_stride + j / page_size];
  int64_t p = clamp64(pg, 0, num_pages - 1);
  return p * page_size + (j % page_size);
}

// Workgroups are dispatched round-robin over the 8 XCDs of the chip.  This
// maps the dispatch index to a logical index so that consecutive logical
// indices run on the same XCD (and share its L2), in dispatch order.
__device__ __forceinline__ uint32_t xcd_remap(uint32_t w, uint32_t n) {
  constexpr uint32_t kXcd = 8;
  uint32_t xcd = w % kXcd, local = w / kXcd;
  uint32_t per = n / kXcd, rem = n % kXcd;
  return xcd * per + (xcd < rem ? xcd : rem) + local;
}

}  // namespace bmattn
