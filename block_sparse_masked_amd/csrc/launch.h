// Internal host-side launchers (not part of the C ABI).  Each .hip file
// defines its kernels and the launcher that configures them; api.cpp
// validates arguments and calls these.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "device_common.h"

namespace bmattn {

struct TilesDev {
  int32_t block_m, block_n, n_seqs, n_qt, n_kt;
  int32_t max_lq, max_lk;
  uint8_t* tile_class;
  int32_t* full_cnt;
  int32_t* part_cnt;
  int32_t* full_idx;
  int32_t* part_idx;
  int32_t* row_order;
};

// Common forward parameters for the kernels.
struct FwdDev {
  MaskDev mask;
  // read-only view of the tiles
  int32_t block_m, block_n, n_qt, n_kt;
  int32_t max_lq, max_lk;
  const int32_t* full_cnt;
  const int32_t* part_cnt;
  const int32_t* full_idx;
  const int32_t* part_idx;
  const int32_t* row_order;
  int32_t num_heads, head_dim;
  const void* q;
  const void* k;
  const void* v;
  void* o;
  float* lse;
  int64_t q_st, q_sh, k_st, k_sh, v_st, v_sh, o_st, o_sh, lse_sh;
  const int32_t* block_table;
  int64_t bt_stride, num_pages;
  int32_t page_size;
  int32_t page_shift;  // log2(page_size) for a power of two, else -1
  float scale_log2;    // softmax scale times log2(e)
  // decode split-KV
  float* ws;             // [n_rows, splits, H, D + 2] partial results
  int32_t split_tiles;   // kv tiles per split
  int32_t n_splits;      // splits per row
};

// Column lists of a block mask (kv-tile major): for column s * n_kt + b the
// ascending FULL / PARTIAL query-tile indices of tiles (a, b) of sequence s.
struct ColsDev {
  int32_t n_seqs, n_qt, n_kt;
  int32_t* full_cnt;   // [n_seqs * n_kt]
  int32_t* part_cnt;
  int32_t* full_idx;   // [n_seqs * n_kt * n_qt]
  int32_t* part_idx;
  int32_t* col_order;  // [n_seqs * n_kt]
};

// Backward parameters: the forward's row lists (query tiles of 128, kv tiles
// of 64) for the dQ pass and the column lists of a 64 x 128 block mask for
// the dK / dV pass.
struct BwdDev {
  MaskDev mask;
  int32_t max_lq, max_lk;
  int32_t n_qt, n_kt;  // row tiling
  const int32_t* full_cnt;
  const int32_t* part_cnt;
  const int32_t* full_idx;
  const int32_t* part_idx;
  const int32_t* row_order;
  int32_t c_n_qt, c_n_kt;  // column tiling
  const int32_t* c_full_cnt;
  const int32_t* c_part_cnt;
  const int32_t* c_full_idx;
  const int32_t* c_part_idx;
  const int32_t* col_order;
  int32_t num_heads, head_dim;
  const void* q;
  const void* k;
  const void* v;
  const void* o;
  const void* dout;
  void* dq;
  void* dk;
  void* dv;
  const float* lse;
  int64_t q_st, q_sh, k_st, k_sh, v_st, v_sh, o_st, o_sh, do_st, do_sh;
  int64_t dq_st, dq_sh, dk_st, dk_sh, dv_st, dv_sh, lse_sh;
  float scale;       // softmax scale
  float scale_log2;  // scale * log2(e)
  float* ws_di;      // [H, total_q] rowsum(dO * O)
  float* ws_l2;      // [H, total_q] LSE * log2(e) (0 where LSE = -inf)
};

hipError_t launch_build_block_mask(const MaskDev& m, const TilesDev& t, hipStream_t st);
hipError_t launch_transpose_block_mask(const TilesDev& t, const ColsDev& c, hipStream_t st);
hipError_t launch_backward_bf16(const BwdDev& p, hipStream_t st);
hipError_t launch_debug_dense_mask(const MaskDev& m, const TilesDev& t, int seq, uint8_t* out,
                                   int64_t out_stride, hipStream_t st);
hipError_t launch_validate(const MaskDev& m, int32_t max_lq, int32_t max_lk,
                           const int32_t* block_table, int64_t bt_stride, int32_t page_size,
                           int64_t num_pages, int32_t* flags, hipStream_t st);
hipError_t launch_duplicated_answer_ids(const MaskDev& m, int32_t max_lq, int32_t max_lk,
                                        const int32_t* role_q, int32_t loss_role,
                                        int32_t history_role, int32_t* role_k_out,
                                        int32_t* turn_q_out, int32_t* flags, hipStream_t st);
hipError_t launch_paged_gather(const MaskDev& m, int32_t max_lk, const void* pool, int64_t st_tok,
                               int64_t st_head, int32_t elem_bytes, int32_t H, int32_t D,
                               int32_t page_size, int64_t num_pages, const int32_t* block_table,
                               int64_t bt_stride, void* out, hipStream_t st);

// log2 of a power-of-two page size, else -1.
inline int32_t page_shift_of(int32_t page_size) {
  if (page_size < 1 || (page_size & (page_size - 1)) != 0) return -1;
  int32_t s = 0;
  while ((1 << s) < page_size) ++s;
  return s;
}

// Forward kernels.  Return hipErrorInvalidValue for a combination that is
// not compiled (the caller checks support first).
hipError_t launch_forward_prefill(const FwdDev& p, int dtype, bool paged, hipStream_t st);
hipError_t launch_forward_prefill_bf16(const FwdDev& p, bool paged, hipStream_t st);
hipError_t launch_forward_decode(const FwdDev& p, int dtype, bool paged, hipStream_t st);

// The static split workspace of the entry point that allocates nothing: its
// size in bytes, and its device address on the calling thread's current
// device (looked up once per device).
size_t decode_scratch_bytes();
hipError_t decode_scratch(void** ptr);

}  // namespace bmattn
