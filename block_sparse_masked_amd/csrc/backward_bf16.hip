// Block-sparse masked attention backward for bf16 inputs (gfx950).
//
// Gradients of O = softmax(scale Q K^T + M) V, the forward of Triton from
// First Principles, Ch. 21, sections 21.1 and 21.2, differentiated: with the
// probabilities recomputed from the forward's log-sum-exp,
//   P = exp(scale S - LSE),  dV = P^T dO,  dP = dO V^T,
//   dS = P (dP - Di) with Di = rowsum(dO * O),
//   dQ = scale dS K,  dK = scale dS^T Q.
// (Di equals rowsum(P * dP), the softmax Jacobian's row term, because
// O = P V.)
//
// Three launches and no atomics, so every gradient is bit-reproducible and a
// sequence's gradients do not depend on the other sequences of the batch:
//  * bwd_prep_kernel: Di and LSE * log2(e) per (head, query) into the
//    workspace;
//  * bwd_dkdv_kernel: one workgroup per (128-key column of a sequence, head)
//    walks the query tiles of 64 rows that see the column -- the column
//    (kv-major) lists of a 64 x 128 block mask, the transposed metadata the
//    xorl issue finds missing for the backward (section "Verified FA4
//    gaps") -- FULL tiles first, then PARTIAL ones with the element
//    predicate;
//  * bwd_dq_kernel: one workgroup per (128-row query tile, head) walks the
//    row's kv tiles of 64 keys -- the forward's block mask -- so each dQ row
//    has one writer and a fixed summation order.
//
// Mapping onto CDNA4: both passes are the forward's dataflow with operands
// exchanged.  The pass's own side (Q and dO rows in the dQ pass, K and V
// rows in the dK / dV pass) stays in registers as the B operand of
// v_mfma_f32_32x32x16_bf16, one 32-row block per wave; the other side's
// tiles (64 rows) go from HBM straight into LDS (global_load_lds_dwordx4,
// XOR-swizzled 16-byte columns, double-buffered, one barrier per tile) and
// are read twice: row-major with rows permuted by swapping bits 2 and 3 (the
// A operand of the score products, so that each lane's 8 consecutive
// accumulator registers hold 8 consecutive rows) and transposed with
// ds_read_b64_tr_b16 (the A operand of the gradient products).  P and dS are
// rounded to bf16 in registers and used as B operands directly.
#include <hip/hip_runtime.h>

#include <algorithm>

#include "device_common.h"
#include "launch.h"

namespace bmattn {
namespace {

typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef short i16x4 __attribute__((ext_vector_type(4)));
typedef short i16x8 __attribute__((ext_vector_type(8)));
typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));

#define LDS_PTR(T, p) ((__attribute__((address_space(3))) T*)(p))

constexpr int kWaves = 4;
constexpr int kThreads = 64 * kWaves;
constexpr int kTR = 64;       // rows of a staged tile
constexpr int kRowTile = 128; // query rows of a dQ workgroup / keys of a dK dV workgroup
constexpr float kLog2e = 1.44269504088896340736f;

template <int D>
struct Lay {
  static constexpr int kRowB = D * 2;                    // bytes of one staged row
  static constexpr int kCh = kRowB / 16;                 // 16-byte columns per row
  static constexpr int kTileB = kTR * kRowB;             // bytes of one staged tile
  static constexpr int kT1 = kTileB;                     // second tile of a stage
  static constexpr int kF = 2 * kTileB;                  // five float / int arrays of kTR
  static constexpr int kStage = 2 * kTileB + 5 * kTR * 4;
  static constexpr int kCopies = kTileB / 1024 / kWaves; // 1 KiB copies per wave per tile
  static constexpr int kDT = D / 32;                     // 32-wide d blocks
  static_assert(kCopies >= 1 && kCopies * 1024 * kWaves == kTileB, "tile / copy mismatch");
};

// Physical 16-byte column of logical column c in tile row r is c ^ swz(r);
// the 16 rows of an operand read and the 4 rows x 64 bytes of a transposing
// read then fall on distinct banks.
template <int D>
__device__ __forceinline__ int swz(int r) {
  if constexpr (D == 128) return ((r & 3) << 2) | ((r >> 2) & 3);
  else return (((r >> 1) & 1) << 2) | ((r >> 2) & 3);
}

__device__ __forceinline__ f32x16 mfma(const bf16x8& a, const bf16x8& b, const f32x16& c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
}

__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }

// Row permutation of a 32-row A operand: swaps bits 2 and 3.
__device__ __forceinline__ int sigma(int i) {
  return (i & ~12) | ((i & 4) << 1) | ((i & 8) >> 1);
}

__device__ __forceinline__ uint32_t lds_addr(const void* p) {
  return static_cast<uint32_t>(reinterpret_cast<uintptr_t>(LDS_PTR(const char, p)));
}
// HBM -> LDS: lane i's 16 (or 4) bytes land at LDS byte lds + 16 i (4 i).
__device__ __forceinline__ void copy16(const void* src, uint32_t lds) {
  asm volatile("global_load_lds_dwordx4 %0, off" ::"v"(src), "{m0}"(lds) : "memory");
}
__device__ __forceinline__ void copy4(const void* src, uint32_t lds) {
  asm volatile("global_load_lds_dword %0, off" ::"v"(src), "{m0}"(lds) : "memory");
}

__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
  return __builtin_bit_cast(uint32_t, __builtin_convertvector((f32x2{lo, hi}), bf16x2));
}

__device__ __forceinline__ void end_of_tile() {
  __builtin_amdgcn_s_waitcnt(0);
  __syncthreads();
}

// Per-lane LDS byte offsets of the operand reads of a staged tile.
template <int D>
struct Addr {
  using L = Lay<D>;
  int a[D / 16];     // row-major A operand, 16-d step ks, rows sigma(lane % 32) of a 32-row block
  int t[L::kDT][2];  // transposing A operand of d block dt, rows +0..3 / +4..7 of a 16-row chunk
  __device__ __forceinline__ Addr(int lane) {
    const int l32 = lane & 31, g = lane >> 5;
    const int r = sigma(l32);
#pragma unroll
    for (int ks = 0; ks < D / 16; ++ks) a[ks] = r * L::kRowB + (((ks * 2 + g) ^ swz<D>(r)) << 4);
    const int j = lane & 15, b = lane >> 4;
#pragma unroll
    for (int dt = 0; dt < L::kDT; ++dt) {
#pragma unroll
      for (int hf = 0; hf < 2; ++hf) {
        const int row = 8 * (b >> 1) + 4 * hf + (j >> 2);
        const int dcol = dt * 32 + 16 * (b & 1) + 4 * (j & 3);
        t[dt][hf] = row * L::kRowB + (((dcol >> 3) ^ swz<D>(row)) << 4) + ((dcol * 2) & 15);
      }
    }
  }
};

// One staged tile of kTR rows by one wave: copy u of wave gw fills 16-byte
// slots [64 (gw * kCopies + u), +64); slot s holds row s / kCh at physical
// column s % kCh.  Row r of the tile is row row0 + r of the sequence,
// clamped to [0, nrows - 1] (rows past the end are hidden by the predicate
// and read finite values).  base points at row 0 of the sequence for this
// head; stride in bytes.
template <int D>
__device__ __forceinline__ void copy_tile(const char* base, int64_t stride, int row0, int nrows,
                                          int gw, int lane, char* dst) {
  using L = Lay<D>;
#pragma unroll
  for (int u = 0; u < L::kCopies; ++u) {
    const int slot = (gw * L::kCopies + u) * 64 + lane;
    const int r = slot / L::kCh, col = (slot % L::kCh) ^ swz<D>(r);
    const int j = max(min(row0 + r, nrows - 1), 0);
    copy16(base + j * stride + col * 16, lds_addr(dst + (gw * L::kCopies + u) * 1024));
  }
}

// kTR 32-bit values of one wave: lane i copies element row0 + i (clamped).
__device__ __forceinline__ void copy_words(const void* base, int row0, int nrows, int lane, char* dst) {
  const int j = max(min(row0 + lane, nrows - 1), 0);
  copy4(static_cast<const char*>(base) + 4 * (int64_t)j, lds_addr(dst));
}

// One 32-row score block of one wave against a staged tile: the sum over
// 16-d steps of A(rows sigma of the block) * B[ks].
template <int D>
__device__ __forceinline__ f32x16 score_block(const char* T, const bf16x8 (&b)[D / 16], const Addr<D>& ad) {
  f32x16 s = f32x16{};
#pragma unroll
  for (int ks = 0; ks < D / 16; ++ks) s = mfma(*reinterpret_cast<const bf16x8*>(T + ad.a[ks]), b[ks], s);
  return s;
}

// acc[dt] += T^T(rows of 16-row chunk c at `chunk`) * B, B holding 8 of the
// chunk's rows per lane (the layout the score blocks leave in registers
// 8 c .. 8 c + 7).
template <int D>
__device__ __forceinline__ void grad_product(const char* chunk, const bf16x8& b, f32x16 (&acc)[D / 32],
                                             const Addr<D>& ad) {
#pragma unroll
  for (int dt = 0; dt < D / 32; ++dt) {
    const i16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16(LDS_PTR(i16x4, chunk + ad.t[dt][0]));
    const i16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16(LDS_PTR(i16x4, chunk + ad.t[dt][1]));
    const i16x8 tv = __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7);
    acc[dt] = mfma(__builtin_bit_cast(bf16x8, tv), b, acc[dt]);
  }
}

// 8 floats -> 8 bf16 (one B operand).
__device__ __forceinline__ bf16x8 pack8(const float (&x)[8]) {
  return __builtin_bit_cast(bf16x8, make_uint4(pack_bf16x2(x[0], x[1]), pack_bf16x2(x[2], x[3]),
                                               pack_bf16x2(x[4], x[5]), pack_bf16x2(x[6], x[7])));
}

// The 32-row block of the pass's own side as B operands: lane l holds row
// (l % 32), d = 16 ks + 8 (l / 32) .. + 7 for every step ks; rows past the
// sequence are zero.
template <int D>
__device__ __forceinline__ void load_b_rows(const void* src, int64_t off_elems, bool valid, int g,
                                            bf16x8 (&b)[D / 16]) {
  const char* row = static_cast<const char*>(src) + off_elems * 2;
#pragma unroll
  for (int ks = 0; ks < D / 16; ++ks) {
    const uint4 x = valid ? *reinterpret_cast<const uint4*>(row + (ks * 16 + g * 8) * 2) : make_uint4(0, 0, 0, 0);
    b[ks] = __builtin_bit_cast(bf16x8, x);
  }
}

// Stores a 32-row block held transposed (lane = row, registers 4 i + j of
// d block dt = d dt*32 + 8 i + 4 g + j), scaled, as bf16.
template <int D>
__device__ __forceinline__ void store_rows(void* dst, int64_t off_elems, const f32x16 (&acc)[D / 32],
                                           float scale, int g) {
  char* row = static_cast<char*>(dst) + off_elems * 2;
#pragma unroll
  for (int dt = 0; dt < D / 32; ++dt) {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int d0 = dt * 32 + 8 * i + 4 * g;
      const float x0 = acc[dt][4 * i + 0] * scale, x1 = acc[dt][4 * i + 1] * scale;
      const float x2 = acc[dt][4 * i + 2] * scale, x3 = acc[dt][4 * i + 3] * scale;
      *reinterpret_cast<uint2*>(row + d0 * 2) = make_uint2(pack_bf16x2(x0, x1), pack_bf16x2(x2, x3));
    }
  }
}

// The element predicate through the mask's term groups (every kind is an
// OR of AND-groups: m.groups), wave-uniform: query row i with ids q, key j
// with segment, role, turn and document ids.  Same condition as visible_k().
__device__ __forceinline__ bool visible_rt(const MaskDev& m, const SeqBounds& b, int i, QIds q,
                                           int j, int32_t kseg, int32_t krole, int32_t kturn,
                                           int32_t kdoc) {
  const bool in = (i < b.lq) & (j < b.lk);
  return in & composed_ok(m.groups, m.think_role, j <= b.lk - b.lq + i, q, kseg, krole, kturn, kdoc);
}

// Key ids in term order (segment, role, turn, document) from load_kids().
__device__ __forceinline__ KIds term_kids(const MaskDev& m, KIds k) {
  if (m.kind == BMATTN_MASK_SHARED_PREFIX) return KIds{k.a, 0, 0, 0};
  if (m.kind == BMATTN_MASK_STRIP_THINKING) return KIds{0, k.a, k.b, 0};
  return k;
}

// The id arrays the terms read, by slot: keys 0 segment, 1 role, 2 turn,
// 3 document; queries 0 segment, 1 turn, 2 document (nullptr: not read).
__device__ __forceinline__ const int32_t* key_ids(const MaskDev& m, int slot) {
  switch (slot) {
    case 0: return (m.terms & BMATTN_TERM_SHARED_PREFIX) ? m.seg_k : nullptr;
    case 1: return (m.terms & BMATTN_TERM_STRIP_THINKING) ? m.role_k : nullptr;
    case 2: return (m.terms & BMATTN_TERM_STRIP_THINKING) ? m.turn_k : nullptr;
    default: return (m.terms & BMATTN_TERM_DOCUMENT) ? m.doc_k : nullptr;
  }
}
__device__ __forceinline__ const int32_t* query_ids(const MaskDev& m, int slot) {
  switch (slot) {
    case 0: return (m.terms & BMATTN_TERM_SHARED_PREFIX) ? m.seg_q : nullptr;
    case 1: return (m.terms & BMATTN_TERM_STRIP_THINKING) ? m.turn_q : nullptr;
    default: return (m.terms & BMATTN_TERM_DOCUMENT) ? m.doc_q : nullptr;
  }
}

// ---- Di and LSE * log2(e) ---------------------------------------------------
// One row (query, head) per group of D / 8 lanes, 8 bf16 per lane.
template <int D>
__global__ __launch_bounds__(kThreads) void bwd_prep_kernel(BwdDev p) {
  constexpr int kLanes = D / 8;
  const int64_t rows = p.mask.total_q * p.num_heads;
  const int64_t r = ((int64_t)blockIdx.x * kThreads + threadIdx.x) / kLanes;
  const int c = threadIdx.x % kLanes;
  const bool ok = r < rows;
  const int64_t i = ok ? r / p.num_heads : 0;
  const int h = ok ? (int)(r % p.num_heads) : 0;
  float acc = 0.f;
  if (ok) {
    const uint4 a = *reinterpret_cast<const uint4*>(static_cast<const char*>(p.dout) +
                                                     (i * p.do_st + h * p.do_sh + c * 8) * 2);
    const uint4 b = *reinterpret_cast<const uint4*>(static_cast<const char*>(p.o) +
                                                     (i * p.o_st + h * p.o_sh + c * 8) * 2);
    const uint32_t av[4] = {a.x, a.y, a.z, a.w}, bv[4] = {b.x, b.y, b.z, b.w};
#pragma unroll
    for (int e = 0; e < 4; ++e)
      acc = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2, av[e]),
                                            __builtin_bit_cast(bf16x2, bv[e]), acc, false);
  }
#pragma unroll
  for (int o = kLanes / 2; o > 0; o >>= 1) acc += __shfl_xor(acc, o);
  if (ok && c == 0) {
    p.ws_di[(int64_t)h * p.mask.total_q + i] = acc;
    const float l = p.lse[(int64_t)h * p.lse_sh + i];
    p.ws_l2[(int64_t)h * p.mask.total_q + i] = l == -INFINITY ? 0.f : l * kLog2e;
  }
}

// ---- dK, dV: one workgroup per (128-key column, head) -------------------------
// Wave w owns keys 32 w .. 32 w + 31 of the column; per query tile (64 rows)
// and per 32-query block it computes S = Q K^T and dP = dO V^T (lane = key,
// registers = 16 of the block's queries), P and dS, then dV^T += dO^T P and
// dK^T += Q^T dS.
template <int D>
__device__ __forceinline__ void dkdv_block(const char* stage, int qb, bool masked,
                                           const bf16x8 (&kf)[D / 16], const bf16x8 (&vf)[D / 16],
                                           f32x16 (&dk)[D / 32], f32x16 (&dv)[D / 32],
                                           const Addr<D>& ad, const BwdDev& p, const SeqBounds& sb,
                                           int q0, int kj, KIds kids, int g) {
  using L = Lay<D>;
  const char* Qs = stage;
  const char* Os = stage + L::kT1;
  const f32x16 s = score_block<D>(Qs + qb * 32 * L::kRowB, kf, ad);
  const f32x16 dp = score_block<D>(Os + qb * 32 * L::kRowB, vf, ad);
  // Registers 8 c + e hold query q0 + 32 qb + 16 c + 8 g + e.
  const float* l2 = reinterpret_cast<const float*>(stage + L::kF);
  const float* di = l2 + kTR;
  const int32_t* qid = reinterpret_cast<const int32_t*>(di + kTR);  // segment, turn, document
  const float sl2 = p.scale_log2;
  bf16x8 pb[2], db[2];
#pragma unroll
  for (int c = 0; c < 2; ++c) {
    const int r0 = qb * 32 + 16 * c + 8 * g;  // row of the tile
    const float4 la = *reinterpret_cast<const float4*>(l2 + r0);
    const float4 lb = *reinterpret_cast<const float4*>(l2 + r0 + 4);
    const float4 da = *reinterpret_cast<const float4*>(di + r0);
    const float4 dbv = *reinterpret_cast<const float4*>(di + r0 + 4);
    const float lv[8] = {la.x, la.y, la.z, la.w, lb.x, lb.y, lb.z, lb.w};
    const float dvv[8] = {da.x, da.y, da.z, da.w, dbv.x, dbv.y, dbv.z, dbv.w};
    float pv[8];
#pragma unroll
    for (int e = 0; e < 8; ++e) pv[e] = fast_exp2(fmaf(s[8 * c + e], sl2, -lv[e]));
    if (masked) {
      int v[3][8];
#pragma unroll
      for (int a = 0; a < 3; ++a) {
        const int4 ia = *reinterpret_cast<const int4*>(qid + a * kTR + r0);
        const int4 ib = *reinterpret_cast<const int4*>(qid + a * kTR + r0 + 4);
        v[a][0] = ia.x; v[a][1] = ia.y; v[a][2] = ia.z; v[a][3] = ia.w;
        v[a][4] = ib.x; v[a][5] = ib.y; v[a][6] = ib.z; v[a][7] = ib.w;
      }
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        const QIds q{v[0][e], v[1][e], v[2][e]};
        pv[e] = visible_rt(p.mask, sb, q0 + r0 + e, q, kj, kids.a, kids.b, kids.c, kids.d) ? pv[e] : 0.f;
      }
    }
    float dsv[8];
#pragma unroll
    for (int e = 0; e < 8; ++e) dsv[e] = pv[e] * (dp[8 * c + e] - dvv[e]);
    pb[c] = pack8(pv);
    db[c] = pack8(dsv);
  }
#pragma unroll
  for (int c = 0; c < 2; ++c) {
    grad_product<D>(Os + (qb * 32 + 16 * c) * L::kRowB, pb[c], dv, ad);
    grad_product<D>(Qs + (qb * 32 + 16 * c) * L::kRowB, db[c], dk, ad);
  }
}

// One workgroup per CU: the dK and dV accumulators (2 D / 16 registers per
// lane per 32 keys) and the resident K and V operands need the register file
// of a single wave per SIMD.
template <int D>
__global__ __launch_bounds__(kThreads, 1) void bwd_dkdv_kernel(BwdDev p) {
  using L = Lay<D>;
  __shared__ __attribute__((aligned(1024))) char smem[2 * L::kStage];
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int l32 = lane & 31, g = lane >> 5;

  const uint32_t w = blockIdx.x;
  const int h = (int)(w % (uint32_t)p.num_heads);
  const int col = p.col_order[w / (uint32_t)p.num_heads];
  const int s = col / p.c_n_kt, b = col % p.c_n_kt;
  const SeqBounds sb = seq_bounds(p.mask, s, p.max_lq, p.max_lk);
  if (b * kRowTile >= sb.lk) return;
  const int32_t* flist = p.c_full_idx + (int64_t)col * p.c_n_qt;
  const int32_t* plist = p.c_part_idx + (int64_t)col * p.c_n_qt;
  const int nfull = p.c_full_cnt[col];
  const int ntiles = nfull + p.c_part_cnt[col];

  const int kj = b * kRowTile + wave * 32 + l32;  // key of the lane inside the sequence
  const bool kvalid = kj < sb.lk;
  const KIds kids = term_kids(p.mask, load_kids(p.mask, sb, kj));
  bf16x8 kf[D / 16], vf[D / 16];
  load_b_rows<D>(p.k, (sb.k0 + (kvalid ? kj : 0)) * p.k_st + (int64_t)h * p.k_sh, kvalid, g, kf);
  load_b_rows<D>(p.v, (sb.k0 + (kvalid ? kj : 0)) * p.v_st + (int64_t)h * p.v_sh, kvalid, g, vf);
  f32x16 dk[L::kDT], dv[L::kDT];
#pragma unroll
  for (int dt = 0; dt < L::kDT; ++dt) {
    dk[dt] = f32x16{};
    dv[dt] = f32x16{};
  }
  const Addr<D> ad(lane);

  const char* qbase = static_cast<const char*>(p.q) + (sb.q0 * p.q_st + (int64_t)h * p.q_sh) * 2;
  const char* obase = static_cast<const char*>(p.dout) + (sb.q0 * p.do_st + (int64_t)h * p.do_sh) * 2;
  const float* l2base = p.ws_l2 + (int64_t)h * p.mask.total_q + sb.q0;
  const float* dibase = p.ws_di + (int64_t)h * p.mask.total_q + sb.q0;
  // Wave w stages query-id slot w (w < 3) of PARTIAL tiles.
  const int32_t* qidsrc = wave < 3 ? query_ids(p.mask, wave) : nullptr;
  const int32_t* qidbase = qidsrc != nullptr ? qidsrc + sb.q0 : nullptr;
  auto entry = [&](int t) -> int { return t < nfull ? flist[t] : plist[t - nfull]; };
  auto issue = [&](int t, char* stage) {
    const int a = entry(t);
    const int r0 = a * kTR;
    copy_tile<D>(qbase, p.q_st * 2, r0, sb.lq, wave, lane, stage);
    copy_tile<D>(obase, p.do_st * 2, r0, sb.lq, wave, lane, stage + L::kT1);
    if (wave == 0) copy_words(l2base, r0, sb.lq, lane, stage + L::kF);
    if (wave == 1) copy_words(dibase, r0, sb.lq, lane, stage + L::kF + kTR * 4);
    if (qidbase != nullptr && t >= nfull) copy_words(qidbase, r0, sb.lq, lane, stage + L::kF + (2 + wave) * kTR * 4);
  };
  if (ntiles > 0) issue(0, smem);
  end_of_tile();
  for (int t = 0; t < ntiles; ++t) {
    char* cur = smem + (t & 1) * L::kStage;
    if (t + 1 < ntiles) issue(t + 1, smem + ((t + 1) & 1) * L::kStage);
    const int q0 = entry(t) * kTR;
    const bool masked = t >= nfull;
#pragma unroll 1
    for (int qb = 0; qb < 2; ++qb)
      dkdv_block<D>(cur, qb, masked, kf, vf, dk, dv, ad, p, sb, q0, kj, kids, g);
    end_of_tile();
  }
  if (kvalid) {
    store_rows<D>(p.dk, (sb.k0 + kj) * p.dk_st + (int64_t)h * p.dk_sh, dk, p.scale, g);
    store_rows<D>(p.dv, (sb.k0 + kj) * p.dv_st + (int64_t)h * p.dv_sh, dv, 1.0f, g);
  }
}

// ---- dQ: one workgroup per (128-row query tile, head) ----------------------
// Wave w owns queries 32 w .. 32 w + 31 of the tile; per kv tile (64 keys)
// it computes S^T = K Q^T and dP^T = V dO^T (lane = query, registers = 32
// keys over two blocks), dS^T, then dQ^T += K^T dS^T.
template <int D>
__device__ __forceinline__ void dq_tile(const char* stage, bool masked, const bf16x8 (&qf)[D / 16],
                                        const bf16x8 (&of)[D / 16], f32x16 (&dq)[D / 32],
                                        const Addr<D>& ad, const BwdDev& p, const SeqBounds& sb,
                                        int k0, int qi, QIds qids, float l2, float di, int g) {
  using L = Lay<D>;
  const int32_t* kid = reinterpret_cast<const int32_t*>(stage + L::kF);  // segment, role, turn, document
  const float sl2 = p.scale_log2;
  // One 32-key block at a time: register r holds key k0 + 32 bl + 16 (r / 8)
  // + 8 g + r % 8.
#pragma unroll 1
  for (int bl = 0; bl < 2; ++bl) {
    const char* Ks = stage + bl * 32 * L::kRowB;
    const char* Vs = stage + L::kT1 + bl * 32 * L::kRowB;
    const f32x16 s = score_block<D>(Ks, qf, ad);
    const f32x16 dp = score_block<D>(Vs, of, ad);
    bf16x8 db[2];
#pragma unroll
    for (int c = 0; c < 2; ++c) {
      const int j0 = 32 * bl + 16 * c + 8 * g;  // key of register 8 c within the tile
      float pv[8];
#pragma unroll
      for (int e = 0; e < 8; ++e) pv[e] = fast_exp2(fmaf(s[8 * c + e], sl2, -l2));
      if (masked) {
        int v[4][8];
#pragma unroll
        for (int a = 0; a < 4; ++a) {
          const int4 x0 = *reinterpret_cast<const int4*>(kid + a * kTR + j0);
          const int4 x1 = *reinterpret_cast<const int4*>(kid + a * kTR + j0 + 4);
          v[a][0] = x0.x; v[a][1] = x0.y; v[a][2] = x0.z; v[a][3] = x0.w;
          v[a][4] = x1.x; v[a][5] = x1.y; v[a][6] = x1.z; v[a][7] = x1.w;
        }
#pragma unroll
        for (int e = 0; e < 8; ++e)
          pv[e] = visible_rt(p.mask, sb, qi, qids, k0 + j0 + e, v[0][e], v[1][e], v[2][e], v[3][e])
                      ? pv[e] : 0.f;
      }
      float dsv[8];
#pragma unroll
      for (int e = 0; e < 8; ++e) dsv[e] = pv[e] * (dp[8 * c + e] - di);
      db[c] = pack8(dsv);
    }
#pragma unroll
    for (int c = 0; c < 2; ++c) grad_product<D>(Ks + 16 * c * L::kRowB, db[c], dq, ad);
  }
}

template <int D>
__global__ __launch_bounds__(kThreads, 2) void bwd_dq_kernel(BwdDev p) {
  using L = Lay<D>;
  __shared__ __attribute__((aligned(1024))) char smem[2 * L::kStage];
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int l32 = lane & 31, g = lane >> 5;

  const uint32_t w = blockIdx.x;
  const int h = (int)(w % (uint32_t)p.num_heads);
  const int row = p.row_order[w / (uint32_t)p.num_heads];
  const int s = row / p.n_qt, a = row % p.n_qt;
  const SeqBounds sb = seq_bounds(p.mask, s, p.max_lq, p.max_lk);
  if (a * kRowTile >= sb.lq) return;
  const int32_t* flist = p.full_idx + (int64_t)row * p.n_kt;
  const int32_t* plist = p.part_idx + (int64_t)row * p.n_kt;
  const int nfull = p.full_cnt[row];
  const int ntiles = nfull + p.part_cnt[row];

  const int qi = a * kRowTile + wave * 32 + l32;
  const bool qvalid = qi < sb.lq;
  const QIds qids = load_qids(p.mask, sb, qi);
  bf16x8 qf[D / 16], of[D / 16];
  load_b_rows<D>(p.q, (sb.q0 + (qvalid ? qi : 0)) * p.q_st + (int64_t)h * p.q_sh, qvalid, g, qf);
  load_b_rows<D>(p.dout, (sb.q0 + (qvalid ? qi : 0)) * p.do_st + (int64_t)h * p.do_sh, qvalid, g, of);
  const int64_t wi = (int64_t)h * p.mask.total_q + sb.q0 + (qvalid ? qi : 0);
  const float l2 = qvalid ? p.ws_l2[wi] : 0.f;
  const float di = qvalid ? p.ws_di[wi] : 0.f;
  f32x16 dq[L::kDT];
#pragma unroll
  for (int dt = 0; dt < L::kDT; ++dt) dq[dt] = f32x16{};
  const Addr<D> ad(lane);

  const char* kbase = static_cast<const char*>(p.k) + (sb.k0 * p.k_st + (int64_t)h * p.k_sh) * 2;
  const char* vbase = static_cast<const char*>(p.v) + (sb.k0 * p.v_st + (int64_t)h * p.v_sh) * 2;
  // Wave w stages key-id slot w of PARTIAL tiles.
  const int32_t* kidsrc = key_ids(p.mask, wave);
  const int32_t* kidbase = kidsrc != nullptr ? kidsrc + sb.k0 : nullptr;
  auto entry = [&](int t) -> int { return t < nfull ? flist[t] : plist[t - nfull]; };
  auto issue = [&](int t, char* stage) {
    const int r0 = entry(t) * kTR;
    copy_tile<D>(kbase, p.k_st * 2, r0, sb.lk, wave, lane, stage);
    copy_tile<D>(vbase, p.v_st * 2, r0, sb.lk, wave, lane, stage + L::kT1);
    if (t >= nfull && kidbase != nullptr) copy_words(kidbase, r0, sb.lk, lane, stage + L::kF + wave * kTR * 4);
  };
  if (ntiles > 0) issue(0, smem);
  end_of_tile();
  for (int t = 0; t < ntiles; ++t) {
    char* cur = smem + (t & 1) * L::kStage;
    if (t + 1 < ntiles) issue(t + 1, smem + ((t + 1) & 1) * L::kStage);
    const int k0 = entry(t) * kTR;
    dq_tile<D>(cur, t >= nfull, qf, of, dq, ad, p, sb, k0, qi, qids, l2, di, g);
    end_of_tile();
  }
  if (qvalid) store_rows<D>(p.dq, (sb.q0 + qi) * p.dq_st + (int64_t)h * p.dq_sh, dq, p.scale, g);
}

template <int D>
hipError_t launch_d(const BwdDev& p, hipStream_t st) {
  static_assert(2 * 2 * Lay<D>::kStage <= 160 * 1024, "two workgroups' LDS stages exceed 160 KiB");
  const int64_t rows = p.mask.total_q * p.num_heads;
  const int64_t prep_grid = (rows * (D / 8) + kThreads - 1) / kThreads;
  const int64_t cols = (int64_t)p.mask.n_seqs * p.c_n_kt * p.num_heads;
  const int64_t qrows = (int64_t)p.mask.n_seqs * p.n_qt * p.num_heads;
  if (prep_grid > INT32_MAX || cols > INT32_MAX || qrows > INT32_MAX) return hipErrorInvalidValue;
  if (rows > 0) {
    hipLaunchKernelGGL((bwd_prep_kernel<D>), dim3((uint32_t)prep_grid), dim3(kThreads), 0, st, p);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  if (cols > 0) {
    hipLaunchKernelGGL((bwd_dkdv_kernel<D>), dim3((uint32_t)cols), dim3(kThreads), 0, st, p);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  if (qrows > 0) {
    hipLaunchKernelGGL((bwd_dq_kernel<D>), dim3((uint32_t)qrows), dim3(kThreads), 0, st, p);
    return hipGetLastError();
  }
  return hipSuccess;
}

}  // namespace

hipError_t launch_backward_bf16(const BwdDev& p, hipStream_t st) {
  if (p.head_dim == 128) return launch_d<128>(p, st);
  if (p.head_dim == 64) return launch_d<64>(p, st);
  return hipErrorInvalidValue;
}

}  // namespace bmattn
