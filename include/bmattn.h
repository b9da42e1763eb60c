/*
 * bmattn -- block-sparse masked attention (forward and backward) for AMD MI355X
 * (gfx950).
 *
 * C ABI.  Plain pointers and sizes only.  Every buffer is owned by the
 * caller; device buffers are plain HIP device allocations.  Every call is
 * asynchronous on the stream it is given (a hipStream_t passed as void*;
 * NULL means the default stream).  The library allocates no memory and keeps
 * no state between calls beyond its loaded code objects (and the static
 * device array of bmattn_forward_noalloc, below), so calls from different
 * host threads are safe when they touch disjoint output buffers.
 *
 * Error behaviour: every entry point returns a bmattn_status.  Arguments are
 * validated on the host before anything is launched; an invalid or
 * unsupported call launches nothing and returns an error code.  There is no
 * fallback: a configuration that is not compiled is an error, never a slower
 * path.  bmattn_last_error() returns a thread-local description of the last
 * failure on the calling thread.  No C++ exception crosses this boundary.
 *
 * Contents that live on the device (cu_seqlens, ids, block tables) cannot be
 * checked by the host before a launch; bmattn_validate() checks them on the
 * device.  The kernels keep every address inside the ranges the host-side
 * sizes describe (out-of-range block-table entries are clamped), so an
 * inconsistent device array yields wrong values, not a fault.
 *
 * Sources (the pages this library implements):
 *  [TFP9]  Triton from First Principles, Ch. 9 "Mask and Structure Kernels"
 *          (causal element mask, whole-tile skip on a scalar flag, ragged
 *          per-row bound).
 *  [TFP21] Triton from First Principles, Ch. 21 "Flash Attention, MoE, and
 *          Advanced Features" (online-softmax attention loop, causal tile
 *          skip, the tiled causal diagram).
 *  [XORL]  xorl issue "Block-mask attention: express shared-prefix and
 *          strip-thinking multi-turn training that cu_seqlens cannot"
 *          (mask specifications, block mask built once and reused,
 *          cu_seq_lens kwargs, fail-closed behaviour).
 *  [NS21]  nanoserve Day 21 "the Triton programming model, modeled on the
 *          CPU" (paged gather through a block table, masked ragged tail).
 */
#ifndef BMATTN_H
#define BMATTN_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define BMATTN_ABI_VERSION 2

/* ---- status codes ----------------------------------------------------- */
typedef enum {
  BMATTN_OK = 0,
  BMATTN_EINVAL = 1,       /* null pointer, inconsistent sizes, bad enum     */
  BMATTN_EUNSUPPORTED = 2, /* valid but not compiled (head_dim, tile shape,  */
                           /* dtype, mask kind for this entry point)         */
  BMATTN_EALIGN = 3,       /* base pointer or stride breaks 16-byte vectors  */
  BMATTN_EHIP = 4,         /* a HIP runtime call or launch failed            */
  BMATTN_EWORKSPACE = 5    /* workspace missing or too small                 */
} bmattn_status;

/* ---- mask kinds -----------------------------------------------------------
 * Query row i of a sequence with Lq queries and Lk keys sits at position
 * p(i) = Lk - Lq + i (so Lq == Lk is self-attention and one query is the last
 * position of its context, the decode case).  Key j is visible to row i when
 *   FULL            always                                  [TFP21 21.1]
 *   CAUSAL          j <= p(i)  (diagonal kept)              [TFP9 9.1; TFP21 21.2]
 *   SHARED_PREFIX   j <= p(i) and (seg_k[j] == 0 or seg_k[j] == seg_q[i])
 *                                                           [XORL "Mask specifications"]
 *   STRIP_THINKING  j <= p(i) and not (role_k[j] == think_role and
 *                                       turn_k[j] < turn_q[i])
 *                                                           [XORL "Mask specifications"]
 *   COMPOSED        an OR of up to four AND-groups of terms: desc->terms
 *                   holds group g in bits 4g .. 4g+3 (BMATTN_TERM_GROUP),
 *                   and key j is visible when it passes every term of at
 *                   least one non-empty group.  One group (terms <= 15) is
 *                   the plain AND.  The terms:
 *     BMATTN_TERM_CAUSAL          j <= p(i)
 *     BMATTN_TERM_DOCUMENT        doc_k[j] == doc_q[i] and doc_k[j] >= 0
 *                                 (a negative document id marks padding)
 *     BMATTN_TERM_SHARED_PREFIX   seg_k[j] == 0 or seg_k[j] == seg_q[i]
 *     BMATTN_TERM_STRIP_THINKING  not (role_k[j] == think_role and
 *                                      turn_k[j] < turn_q[i])
 *                                 [XORL "Proposed work" 3: composable causal,
 *                                  document, shared-prefix and strip-thinking
 *                                  pieces; "Current state in this tree":
 *                                  causal + document + padding in one mask]
 *                                 [reading: AND inside a group, OR across
 *                                  groups, e.g. a prefix-LM mask is
 *                                  {CAUSAL} OR {DOCUMENT} with the prefix
 *                                  in document 0 and the rest in -1]
 *   (CAUSAL is COMPOSED with {CAUSAL}, SHARED_PREFIX with {CAUSAL,
 *   SHARED_PREFIX}, STRIP_THINKING with {CAUSAL, STRIP_THINKING}.)
 * Packed documents are sequences of cu_seqlens with the CAUSAL kind: every
 * document gets its own causal square and nothing off it; the DOCUMENT term
 * expresses the same inside one sequence.
 */
typedef enum {
  BMATTN_MASK_FULL = 0,
  BMATTN_MASK_CAUSAL = 1,
  BMATTN_MASK_SHARED_PREFIX = 2,
  BMATTN_MASK_STRIP_THINKING = 3,
  BMATTN_MASK_COMPOSED = 4
} bmattn_mask_kind;

/* Terms of a COMPOSED mask (bits of one group in bmattn_mask_desc.terms). */
enum {
  BMATTN_TERM_CAUSAL = 1,
  BMATTN_TERM_DOCUMENT = 2,
  BMATTN_TERM_SHARED_PREFIX = 4,
  BMATTN_TERM_STRIP_THINKING = 8
};
/* Group g (0 .. 3) of a COMPOSED mask's terms word: the groups are ORed. */
#define BMATTN_TERM_GROUP(g, bits) ((int32_t)(bits) << (4 * (g)))

typedef enum { BMATTN_F32 = 0, BMATTN_BF16 = 1 } bmattn_dtype;

/* Tile classes written by bmattn_build_block_mask. */
enum { BMATTN_TILE_EMPTY = 0, BMATTN_TILE_PARTIAL = 1, BMATTN_TILE_FULL = 2 };

/* ---- mask description --------------------------------------------------
 * Host fields are sizes; pointer fields are device arrays of int32.
 * Sequence s owns query rows cu_seqlens_q[s] .. cu_seqlens_q[s+1]-1 of the
 * packed query axis and keys cu_seqlens_k[s] .. cu_seqlens_k[s+1]-1 of the
 * packed key axis (or, for a paged K/V, logical positions
 * 0 .. cu_seqlens_k[s+1]-cu_seqlens_k[s]-1).  This is the cu_seq_lens_q/k and
 * max_length_q/k convention of [XORL "Current state in this tree"].
 * Id arrays are indexed by packed query row (…_q) or packed key row (…_k);
 * for self-attention pass the same array for both sides.  Only the ids the
 * kind reads must be non-NULL (SHARED_PREFIX: seg_q, seg_k; STRIP_THINKING:
 * role_k, turn_q, turn_k; COMPOSED: those of any group's terms, DOCUMENT: doc_q,
 * doc_k).
 */
typedef struct {
  int32_t kind;           /* bmattn_mask_kind                                  */
  int32_t n_seqs;         /* >= 1                                              */
  int32_t max_seqlen_q;   /* >= every sequence's query count (>= 1)            */
  int32_t max_seqlen_k;   /* >= every sequence's key count (>= 1)              */
  int64_t total_q;        /* cu_seqlens_q[n_seqs]: rows of Q, O, ids_q         */
  int64_t total_k;        /* cu_seqlens_k[n_seqs]: rows of K, V, ids_k         */
  int32_t think_role;     /* role value of think tokens (STRIP_THINKING)       */
  int32_t terms;          /* COMPOSED: term groups (1..0xffff, see above); else 0 */
  const int32_t* cu_seqlens_q; /* [n_seqs + 1], non-decreasing, starts at 0   */
  const int32_t* cu_seqlens_k; /* [n_seqs + 1], non-decreasing, starts at 0   */
  const int32_t* seg_q;   /* [total_q] segment id of each query (0 = prefix)   */
  const int32_t* seg_k;   /* [total_k] segment id of each key                  */
  const int32_t* role_k;  /* [total_k] role of each key                        */
  const int32_t* turn_q;  /* [total_q] turn of each query                      */
  const int32_t* turn_k;  /* [total_k] turn of each key                        */
  const int32_t* doc_q;   /* [total_q] document of each query (< 0: padding)   */
  const int32_t* doc_k;   /* [total_k] document of each key (< 0: padding)     */
} bmattn_mask_desc;

/* ---- block mask ------------------------------------------------------------
 * Tile (a, b) of sequence s covers query rows a*block_m .. a*block_m+block_m-1
 * and keys b*block_n .. b*block_n+block_n-1 of s.  Pairs outside the
 * sequence count as not visible, so a tile is
 *   EMPTY   no visible pair             -> skipped, never loaded
 *   FULL    all block_m*block_n visible -> run with no mask and no bounds code
 *   PARTIAL otherwise                   -> the element predicate is applied
 * [TFP21 21.2 diagram; TFP9 9.2].  Row r = s * n_qt + a, n_qt =
 * ceil(max_seqlen_q / block_m); every row has n_kt = ceil(max_seqlen_k /
 * block_n) kv tiles.  full_idx/part_idx hold each row's FULL/PARTIAL kv-tile
 * indices in ascending order in slots 0 .. cnt-1 (the rest is -1).
 * row_order is a schedule: the rows sorted by descending listed-tile count,
 * ties by ascending row.  All arrays are caller-allocated device memory; the
 * block mask is built once and reused across calls [XORL "Proposed work" 3].
 */
typedef struct {
  int32_t block_m, block_n;
  int32_t n_seqs, n_qt, n_kt;
  int32_t reserved0;
  uint8_t* tile_class;   /* [n_seqs * n_qt * n_kt]                            */
  int32_t* full_cnt;     /* [n_seqs * n_qt]                                   */
  int32_t* part_cnt;     /* [n_seqs * n_qt]                                   */
  int32_t* full_idx;     /* [n_seqs * n_qt * n_kt]                            */
  int32_t* part_idx;     /* [n_seqs * n_qt * n_kt]                            */
  int32_t* row_order;    /* [n_seqs * n_qt]                                   */
} bmattn_block_mask;

/* Sizes of a block mask for a description and tile shape (host only, no
 * device access).  Writes n_qt, n_kt and the element counts of the row
 * arrays (rows = n_seqs * n_qt) and tile arrays (rows * n_kt).  1 <= block_m,
 * block_n <= 1024. */
int bmattn_block_mask_shape(const bmattn_mask_desc* desc, int32_t block_m, int32_t block_n,
                            int32_t* n_qt, int32_t* n_kt, int64_t* rows, int64_t* tiles);

/* Classifies every tile and writes the ascending kv-tile lists and the row
 * schedule into *out (whose pointers and block_m/block_n the caller has set;
 * the shape fields are checked against bmattn_block_mask_shape).  Any tile
 * shape in 1..1024 x 1..1024 is accepted.  The result is bit-exact: it
 * depends only on the description. */
int bmattn_build_block_mask(const bmattn_mask_desc* desc, const bmattn_block_mask* out,
                            void* stream);

/* ---- forward ---------------------------------------------------------------
 * O = softmax(Q K^T * scale + M) V with M = 0 on visible pairs and -inf on
 * the others, computed tile by tile with the online softmax: running max,
 * running sum and an accumulator rescaled by exp(m_old - m_new)
 * [TFP21 21.1].  Each query-tile row visits only its listed kv tiles: FULL
 * tiles first, then PARTIAL tiles with the element predicate [TFP21 21.2;
 * TFP9 9.2].  LSE = m + ln(l), the natural-log log-sum-exp of the row's
 * scaled, masked scores (-inf for a row with no visible key, whose O is 0).
 *
 * Layout: Q [total_q, H, D] and O [total_q, H, D]; K, V [total_k, H, D] when
 * contiguous, or page pools [num_pages, page_size, H, D] when block_table is
 * given: logical key j of sequence s then lives in physical page
 * block_table[s * block_table_stride + j / page_size], slot j % page_size
 * [NS21].  Strides are in elements; head_dim is contiguous.  Q, K, V and O
 * share the dtype.  LSE is fp32 [H, total_q] with stride lse_stride_head
 * (may be NULL).  Compiled: head_dim 64 or 128; dtype F32 or BF16.  Tile
 * shapes: block_m = 128 with block_n = 64 (any query count), or block_m = 1
 * with block_n = 64 (one query per sequence; needs a workspace, see
 * bmattn_forward_workspace_size).  Bit-reproducible run to run.
 */
typedef struct {
  int32_t dtype;          /* bmattn_dtype of Q, K, V, O                        */
  int32_t num_heads;      /* H (same for Q and K/V)                            */
  int32_t head_dim;       /* D                                                 */
  int32_t page_size;      /* paged K/V only (>= 1)                             */
  const void* q; int64_t q_stride_tok, q_stride_head;
  const void* k; int64_t k_stride_tok, k_stride_head; /* tok stride: per pool row */
  const void* v; int64_t v_stride_tok, v_stride_head;
  void* o;       int64_t o_stride_tok, o_stride_head;
  float* lse;    int64_t lse_stride_head;
  const int32_t* block_table;  /* NULL: contiguous K/V                         */
  int64_t block_table_stride;  /* entries per sequence row                     */
  int64_t num_pages;           /* pool pages (entries are clamped to range)    */
  float scale;                 /* 0 -> 1/sqrt(head_dim)                        */
  int32_t reserved0;
  void* workspace;             /* device scratch (see workspace_size)          */
  size_t workspace_bytes;
} bmattn_fwd_args;

/* Bytes of device workspace bmattn_forward needs for these arguments (0 when
 * none).  Host only. */
int bmattn_forward_workspace_size(const bmattn_fwd_args* args, const bmattn_mask_desc* desc,
                                  const bmattn_block_mask* tiles, size_t* bytes);

/* Runs the forward on `stream`.  `tiles` must have been built from `desc`
 * with one of the compiled tile shapes. */
int bmattn_forward(const bmattn_fwd_args* args, const bmattn_mask_desc* desc,
                   const bmattn_block_mask* tiles, void* stream);

/* ---- forward without any allocation -----------------------------------------
 * For callers that cannot allocate device memory at call time: code under
 * HIP graph capture, tight serving loops, harnesses that forbid hipMalloc.
 * The same computation and kernels as bmattn_forward (bit-identical
 * results), but the decode path's split workspace is a static device array
 * of the library, BMATTN_NOALLOC_MAX_WORKSPACE bytes per GPU, held from the
 * library's first use on that GPU until the process ends; the call itself
 * allocates and frees nothing.  args->workspace must be NULL.  A decode
 * whose workspace (bmattn_forward_workspace_size) exceeds the static size
 * returns BMATTN_EWORKSPACE before anything is launched.  The prefill path
 * needs no workspace and is unchanged.
 *
 * Every call on one GPU shares that GPU's array: calls that overlap in time
 * on one GPU (other streams, other threads) race on it and must be
 * serialised by the caller.  Nothing in it needs to start at zero (each
 * value the merge reads is written earlier in the same call).  The stream
 * must belong to the calling thread's current device. */
#define BMATTN_NOALLOC_MAX_WORKSPACE ((size_t)96 << 20)
int bmattn_forward_noalloc(const bmattn_fwd_args* args, const bmattn_mask_desc* desc,
                           const bmattn_block_mask* tiles, void* stream);

/* ---- column lists (kv-tile major) -------------------------------------------
 * The classes of a block mask read by kv-tile column: for column
 * c = s * n_kt + b, the ascending indices a of the FULL tiles (a, b) of
 * sequence s in full_idx[c * n_qt + 0 .. full_cnt[c] - 1], the PARTIAL ones
 * likewise (unused slots -1), and col_order: the columns by descending
 * listed-tile count, ties by ascending column.  This is the transposed
 * orientation a backward pass that owns one kv tile needs [XORL "Verified
 * FA4 gaps": the missing transposed backward metadata].  All arrays are
 * caller-allocated device memory. */
typedef struct {
  int32_t block_m, block_n;
  int32_t n_seqs, n_qt, n_kt;
  int32_t reserved0;
  int32_t* full_cnt;   /* [n_seqs * n_kt]                                     */
  int32_t* part_cnt;   /* [n_seqs * n_kt]                                     */
  int32_t* full_idx;   /* [n_seqs * n_kt * n_qt]                              */
  int32_t* part_idx;   /* [n_seqs * n_kt * n_qt]                              */
  int32_t* col_order;  /* [n_seqs * n_kt]                                     */
} bmattn_block_mask_cols;

/* Writes the column lists of a built block mask (reads tiles->tile_class
 * only).  out's block_m, block_n, n_seqs, n_qt and n_kt must equal tiles'.
 * Bit-exact. */
int bmattn_transpose_block_mask(const bmattn_block_mask* tiles, const bmattn_block_mask_cols* out,
                                void* stream);

/* ---- backward ----------------------------------------------------------------
 * Gradients of the forward above for an upstream gradient dO: with
 * P = exp(S * scale - LSE) recomputed from the forward's LSE,
 *   dV = P^T dO,  dP = dO V^T,  dS = P (dP - rowsum(dO * O)),
 *   dQ = scale dS K,  dK = scale dS^T Q
 * (the chain rule of [TFP21 21.1] with the mask of [TFP21 21.2; TFP9 9.2];
 * the pages print no backward formulas).  Only listed tiles are visited:
 * dK and dV by kv tile over the column lists of a block mask with tiles of
 * 64 x 128 (cols; see bmattn_transpose_block_mask), dQ by query tile over
 * the forward's block mask with tiles of 128 x 64 (rows).  No atomics: each
 * output element has one writer and a fixed summation order, so the result
 * is bit-reproducible run to run and does not depend on the other sequences
 * of the batch [XORL "Determinism" and "Batch / packing invariance"].
 *
 * Compiled: dtype BF16 (inputs and gradients), head_dim 64 or 128,
 * contiguous K/V (no block table).  Layouts as the forward: Q, O, dO, dQ
 * [total_q, H, D]; K, V, dK, dV [total_k, H, D], head_dim contiguous, token
 * and head strides in elements (multiples of 8); LSE fp32 [H, total_q] with
 * lse_stride_head, as the forward wrote it.  dQ, dK and dV are overwritten
 * (keys that no query sees get 0).  The workspace holds two fp32 arrays of
 * H * total_q (bmattn_backward_workspace_size).
 */
typedef struct {
  int32_t dtype;          /* bmattn_dtype; BF16 only                          */
  int32_t num_heads;
  int32_t head_dim;
  int32_t reserved0;
  const void* q;    int64_t q_stride_tok, q_stride_head;
  const void* k;    int64_t k_stride_tok, k_stride_head;
  const void* v;    int64_t v_stride_tok, v_stride_head;
  const void* o;    int64_t o_stride_tok, o_stride_head;
  const void* dout; int64_t do_stride_tok, do_stride_head;
  const float* lse; int64_t lse_stride_head;
  void* dq;         int64_t dq_stride_tok, dq_stride_head;
  void* dk;         int64_t dk_stride_tok, dk_stride_head;
  void* dv;         int64_t dv_stride_tok, dv_stride_head;
  float scale;            /* 0 -> 1/sqrt(head_dim); must match the forward's  */
  int32_t reserved1;
  void* workspace;        /* device scratch                                   */
  size_t workspace_bytes;
} bmattn_bwd_args;

/* Bytes of workspace bmattn_backward needs (host only; reads dtype,
 * num_heads and head_dim of args and the description's total_q). */
int bmattn_backward_workspace_size(const bmattn_bwd_args* args, const bmattn_mask_desc* desc,
                                   size_t* bytes);

/* rows: built from desc with block_m 128, block_n 64 (the forward's).  cols:
 * the column lists of a block mask built from desc with block_m 64,
 * block_n 128. */
int bmattn_backward(const bmattn_bwd_args* args, const bmattn_mask_desc* desc,
                    const bmattn_block_mask* rows, const bmattn_block_mask_cols* cols,
                    void* stream);

/* ---- test and support exports ---------------------------------------------
 * Gathers the paged history of every sequence into out [total_k, H, D]
 * (contiguous, the pool's dtype) through the forward's own paged addressing
 * [NS21].  pool: [num_pages, page_size, H, D] with the given element
 * strides; elem_bytes is 2 or 4. */
int bmattn_paged_gather(const void* pool, int64_t pool_stride_tok, int64_t pool_stride_head,
                        int32_t elem_bytes, int32_t num_heads, int32_t head_dim,
                        int32_t page_size, int64_t num_pages, const int32_t* block_table,
                        int64_t block_table_stride, const bmattn_mask_desc* desc, void* out,
                        void* stream);

/* Expands sequence `seq`'s tile classes into a dense uint8 mask
 * out [Lq_max_rows, Lk_max_cols] (row stride out_stride): FULL tiles -> 1,
 * EMPTY tiles -> 0, PARTIAL tiles -> the device element predicate the
 * forward uses.  Rows/columns past the sequence are written 0.
 * out_rows = n_qt * block_m and out_cols = n_kt * block_n of `tiles`. */
int bmattn_debug_dense_mask(const bmattn_mask_desc* desc, const bmattn_block_mask* tiles,
                            int32_t seq, uint8_t* out, int64_t out_stride, void* stream);

/* Checks the device-side arrays of a description (and optionally a block
 * table) on the device: cu_seqlens start at 0, never decrease, end at the
 * totals and respect the max lengths; block-table entries that a sequence
 * uses lie in [0, num_pages).  Writes one int32 flag word to *flags (device):
 * bit 0 cu_seqlens_q, bit 1 cu_seqlens_k, bit 2 lengths vs maxima, bit 3
 * block table.  0 means valid.  block_table may be NULL. */
int bmattn_validate(const bmattn_mask_desc* desc, const int32_t* block_table,
                    int64_t block_table_stride, int32_t page_size, int64_t num_pages,
                    int32_t* flags, void* stream);

/* ---- strip-thinking with duplicated answers ------------------------------
 * [XORL "The exactness question", option (b)].  The conversation is packed
 * with every answer span written twice: a loss copy, which sees its own
 * turn's thinking, and right after it a history copy, which sees its turn
 * with the thinking stripped; later turns see the history copy and neither
 * the thinking nor the loss copy.  With roles think_role (desc), loss_role
 * and history_role marking those tokens, this call writes ids under which
 * the STRIP_THINKING kind yields exactly that mask:
 *   role_k_out[j] = think_role       if role_k[j] == loss_role, else role_k[j]
 *   turn_q_out[i] = turn_q[i] + 1    if role_q[i] == history_role, else turn_q[i]
 * (a loss copy is hidden from later turns as thinking is; a history-copy
 * query hides its own turn's thinking and loss copy as if they were one turn
 * earlier).  Build and run the forward with a STRIP_THINKING description
 * whose role_k is role_k_out, turn_q is turn_q_out and turn_k is unchanged.
 *
 * desc: kind STRIP_THINKING holding the duplicated layout's ids (role_k,
 * turn_q, turn_k, think_role).  role_q: [total_q] role of each query.
 * Outputs: role_k_out [total_k], turn_q_out [total_q], device int32; they may
 * be the input arrays themselves (rewritten in place).  think_role,
 * loss_role and history_role must differ (else BMATTN_EINVAL).
 *
 * The relabelling is exact when, in every sequence, turns never decrease
 * along the keys, a turn's history-copy tokens come after all its other
 * tokens, a query carries the ids of the key at its position, and no
 * history copy has turn INT32_MAX.  flags (device int32, may be NULL): when
 * given, those conditions are checked on the device first and one word is
 * written: bit 0 a turn decreases, bit 1 a non-history token follows a
 * history copy of its turn, bit 2 a query's ids differ from its position's
 * key, bit 3 a history copy at turn INT32_MAX; 0 means exact. */
int bmattn_duplicated_answer_ids(const bmattn_mask_desc* desc, const int32_t* role_q,
                                 int32_t loss_role, int32_t history_role, int32_t* role_k_out,
                                 int32_t* turn_q_out, int32_t* flags, void* stream);

/* Status text; thread-local last error text; ABI version. */
const char* bmattn_status_string(int status);
const char* bmattn_last_error(void);
int bmattn_abi_version(void);

#ifdef __cplusplus
}
#endif
#endif /* BMATTN_H */
