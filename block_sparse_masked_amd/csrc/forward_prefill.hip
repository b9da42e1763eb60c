// Block-sparse masked attention forward, query tiles of 128 rows (gfx950).
//
// Algorithm: Triton from First Principles, Ch. 21, section 21.1 -- the
// online softmax over kv tiles with a running max m, a running sum l and an
// accumulator rescaled by alpha = exp(m_old - m_new); section 21.2 -- the
// element mask applied only where a tile straddles the mask boundary, and
// tiles beyond it skipped.  Here the skip comes from the kv-tile lists of the
// block mask: a workgroup walks its row's FULL tiles (no mask code) and then
// its PARTIAL tiles (element predicate); EMPTY tiles are never loaded.
//
// Mapping onto CDNA4 (not the pages' design):
//  * one workgroup = 4 waves = 128 query rows of one (sequence, head); each
//    wave owns 32 query rows for the whole kv loop;
//  * a wave computes S^T = K Q^T with v_mfma_f32_32x32x16_bf16 (A = K tile
//    rows from LDS, B = the wave's Q rows held in registers), so lane l holds
//    the scores of query (l % 32) against 16 keys per 32-key block.  The row
//    max and row sum are then lane-local plus one exchange with lane l ^ 32;
//  * the A operand rows are permuted (bits 2 and 3 of the row index
//    swapped) so that each lane's 8 consecutive accumulator registers hold 8
//    consecutive keys: the probabilities feed the P V product as the B
//    operand directly from registers, with V^T read from LDS;
//  * K and V^T tiles (BLOCK_N = 64 keys) are double-buffered in LDS and the
//    next tile's global loads are in flight while the current one is used;
//  * exponentials are base 2 with log2(e) folded into the softmax scale.
// The fp32 variant uses v_mfma_f32_32x32x2_f32 with the same accumulator
// layout.
#include <hip/hip_runtime.h>

#include "device_common.h"
#include "launch.h"

namespace bmattn {
namespace {

typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));

constexpr int kBM = 128;
constexpr int kBN = 64;
constexpr int kThreads = 256;
constexpr float kLn2 = 0.69314718055994530942f;
constexpr float kRescaleSlack = 8.0f;

template <typename T, int D>
struct Cfg {
  static constexpr int kElem = sizeof(T);
  static constexpr int kRowB = D * kElem;           // bytes of one K/V row
  static constexpr int kCh = kRowB / 16;             // 16-byte chunks per row
  static constexpr int kEpc = 16 / kElem;            // elements per chunk
  static constexpr int kKP = kRowB + 16;             // K row pitch in LDS (bytes)
  static constexpr int kVP = kBN * kElem + 16;       // V^T row pitch in LDS (bytes)
  static constexpr int kKBuf = kBN * kKP;
  static constexpr int kVBuf = D * kVP;
  static constexpr int kIdBuf = 4 * kBN * 4;              // key ids of a PARTIAL tile (KIds)
  static constexpr int kStage = kKBuf + kVBuf + kIdBuf;
  static constexpr int kKChunks = kBN * kCh / kThreads;  // K chunks per thread
  static constexpr int kKpt = kBN * kCh / kThreads;      // keys per thread (V staging)
  static constexpr int kDT = D / 32;                     // 32-wide output d tiles
  static_assert(kKChunks * kThreads == kBN * kCh, "tile / thread mismatch");
};

__device__ __forceinline__ f32x16 mfma(const bf16x8& a, const bf16x8& b, const f32x16& c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
}
__device__ __forceinline__ f32x16 mfma(float a, float b, const f32x16& c) {
  return __builtin_amdgcn_mfma_f32_32x32x2f32(a, b, c, 0, 0, 0);
}

__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }

// Row index permutation of the 32-row MFMA operand: swaps bits 2 and 3.
__device__ __forceinline__ int sigma(int i) {
  return (i & ~12) | ((i & 4) << 1) | ((i & 8) >> 1);
}

typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

// Dword i of a 16-byte chunk.
__device__ __forceinline__ uint32_t dword(const uint4& v, int i) {
  return __builtin_bit_cast(u32x4, v)[i];
}
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));

// Two floats -> two bf16 (round to nearest even) in one dword, lo first.
__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
  return __builtin_bit_cast(uint32_t, __builtin_convertvector((f32x2{lo, hi}), bf16x2));
}

template <typename T, int D, bool PAGED>
struct Prefill {
  using C = Cfg<T, D>;

  // Per-thread byte offsets of the first K row and first V row this thread
  // stages, relative to the first key of the tile (contiguous K/V); the other
  // rows follow at uniform strides.  Computed once per workgroup.
  struct Offsets {
    uint32_t k, v;
  };
  static __device__ __forceinline__ Offsets offsets(const FwdDev& p, int tid) {
    const int ch = tid % C::kCh, kg = tid / C::kCh;
    return Offsets{(uint32_t)((tid / C::kCh) * p.k_st * C::kElem + ch * 16),
                   (uint32_t)(kg * C::kKpt * p.v_st * C::kElem + ch * 16)};
  }

  // Global -> registers, K rows of one kv tile.  MASKED (PARTIAL) tiles leave
  // rows past the sequence zero and never read them.
  template <bool MASKED>
  static __device__ __forceinline__ void load_k(const FwdDev& p, const SeqBounds& sb, int s, int h,
                                                int kt, int tid, const Offsets& off,
                                                uint4 (&kr)[C::kKChunks]) {
    const int ch = tid % C::kCh;
    if constexpr (!PAGED) {
      const char* kb = static_cast<const char*>(p.k) +
                       ((sb.k0 + (int64_t)kt * kBN) * p.k_st + (int64_t)h * p.k_sh) * C::kElem;
#pragma unroll
      for (int u = 0; u < C::kKChunks; ++u) {
        const int j = kt * kBN + (tid + kThreads * u) / C::kCh;
        const uint32_t o = off.k + (uint32_t)(u * (kThreads / C::kCh) * p.k_st * C::kElem);
        kr[u] = (!MASKED || j < sb.lk) ? *reinterpret_cast<const uint4*>(kb + o)
                                       : make_uint4(0, 0, 0, 0);
      }
    } else {
      // Paged: all block-table entries first, then the loads.
      const char* kb = static_cast<const char*>(p.k) + (int64_t)h * p.k_sh * C::kElem;
      int32_t pe[C::kKChunks];
#pragma unroll
      for (int u = 0; u < C::kKChunks; ++u) {
        const int j = min(kt * kBN + (tid + kThreads * u) / C::kCh, sb.lk - 1);
        pe[u] = page_entry(p.block_table, p.bt_stride, s, j, p.page_size, p.page_shift);
      }
#pragma unroll
      for (int u = 0; u < C::kKChunks; ++u) {
        const int j = kt * kBN + (tid + kThreads * u) / C::kCh;
        const int64_t r = row_in_page(pe[u], j, p.page_size, p.page_shift, p.num_pages);
        kr[u] = (!MASKED || j < sb.lk)
                    ? *reinterpret_cast<const uint4*>(kb + r * p.k_st * C::kElem + ch * 16)
                    : make_uint4(0, 0, 0, 0);
      }
    }
  }

  // Global -> registers, V rows (and, for MASKED tiles, the key ids).
  template <bool MASKED>
  static __device__ __forceinline__ void load_v(const FwdDev& p, const SeqBounds& sb, int s, int h,
                                                int kt, int tid, const Offsets& off,
                                                uint4 (&vr)[C::kKpt], KIds& kid) {
    if (MASKED && tid < kBN) kid = load_kids(p.mask, sb, kt * kBN + tid);
    const int ch = tid % C::kCh, kg = tid / C::kCh;
    if constexpr (!PAGED) {
      const char* vb = static_cast<const char*>(p.v) +
                       ((sb.k0 + (int64_t)kt * kBN) * p.v_st + (int64_t)h * p.v_sh) * C::kElem;
#pragma unroll
      for (int u = 0; u < C::kKpt; ++u) {
        const int j = kt * kBN + kg * C::kKpt + u;
        const uint32_t o = off.v + (uint32_t)(u * p.v_st * C::kElem);
        vr[u] = (!MASKED || j < sb.lk) ? *reinterpret_cast<const uint4*>(vb + o)
                                       : make_uint4(0, 0, 0, 0);
      }
    } else {
      const char* vb = static_cast<const char*>(p.v) + (int64_t)h * p.v_sh * C::kElem;
      int32_t pe[C::kKpt];
#pragma unroll
      for (int u = 0; u < C::kKpt; ++u) {
        const int j = min(kt * kBN + kg * C::kKpt + u, sb.lk - 1);
        pe[u] = page_entry(p.block_table, p.bt_stride, s, j, p.page_size, p.page_shift);
      }
#pragma unroll
      for (int u = 0; u < C::kKpt; ++u) {
        const int j = kt * kBN + kg * C::kKpt + u;
        const int64_t r = row_in_page(pe[u], j, p.page_size, p.page_shift, p.num_pages);
        vr[u] = (!MASKED || j < sb.lk)
                    ? *reinterpret_cast<const uint4*>(vb + r * p.v_st * C::kElem + ch * 16)
                    : make_uint4(0, 0, 0, 0);
      }
    }
  }

  // Registers -> LDS, K row-major.
  static __device__ __forceinline__ void store_k(char* stage, int tid,
                                                 const uint4 (&kr)[C::kKChunks]) {
#pragma unroll
    for (int u = 0; u < C::kKChunks; ++u) {
      const int c = tid + kThreads * u;
      const int row = c / C::kCh, ch = c % C::kCh;
      *reinterpret_cast<uint4*>(stage + row * C::kKP + ch * 16) = kr[u];
    }
  }

  // Registers -> LDS, V transposed (V^T[d][key]) and the key ids.
  static __device__ __forceinline__ void store_v(char* stage, int tid, bool masked,
                                                 const uint4 (&vr)[C::kKpt], const KIds& kid) {
    if (masked && tid < kBN) {
      int32_t* ids = reinterpret_cast<int32_t*>(stage + C::kKBuf + C::kVBuf);
      ids[tid] = kid.a;
      ids[kBN + tid] = kid.b;
      ids[2 * kBN + tid] = kid.c;
      ids[3 * kBN + tid] = kid.d;
    }
    char* vt = stage + C::kKBuf;
    const int ch = tid % C::kCh, kg = tid / C::kCh;
    if constexpr (sizeof(T) == 2) {
      // Dword i of key u holds d = 2i (low half) and 2i+1 (high half); pack
      // the same d of consecutive keys into one dword with v_perm.
#pragma unroll
      for (int i = 0; i < C::kEpc / 2; ++i) {
        const uint32_t w0 = dword(vr[0], i), w1 = dword(vr[1], i);
        const uint32_t lo01 = __builtin_amdgcn_perm(w1, w0, 0x05040100u);
        const uint32_t hi01 = __builtin_amdgcn_perm(w1, w0, 0x07060302u);
        char* d0 = vt + (ch * C::kEpc + 2 * i) * C::kVP + kg * C::kKpt * 2;
        if constexpr (C::kKpt == 4) {
          const uint32_t w2 = dword(vr[2], i), w3 = dword(vr[3], i);
          const uint32_t lo23 = __builtin_amdgcn_perm(w3, w2, 0x05040100u);
          const uint32_t hi23 = __builtin_amdgcn_perm(w3, w2, 0x07060302u);
          *reinterpret_cast<uint2*>(d0) = make_uint2(lo01, lo23);
          *reinterpret_cast<uint2*>(d0 + C::kVP) = make_uint2(hi01, hi23);
        } else {
          *reinterpret_cast<uint32_t*>(d0) = lo01;
          *reinterpret_cast<uint32_t*>(d0 + C::kVP) = hi01;
        }
      }
    } else {
      static_assert(C::kKpt == 4 || C::kKpt == 8, "fp32 staging expects 4 or 8 keys per thread");
#pragma unroll
      for (int e = 0; e < C::kEpc; ++e) {
        const int d = ch * C::kEpc + e;
        char* dst = vt + d * C::kVP + kg * C::kKpt * 4;
#pragma unroll
        for (int u0 = 0; u0 < C::kKpt; u0 += 4) {
          *reinterpret_cast<uint4*>(dst + u0 * 4) =
              make_uint4(dword(vr[u0 + 0], e), dword(vr[u0 + 1], e), dword(vr[u0 + 2], e), dword(vr[u0 + 3], e));
        }
      }
    }
  }
};

// Q operand of one lane: bf16 -> 8 values per 16-wide k step; fp32 -> one
// value per 2-wide k step, lane group g taking d in [g*D/2, g*D/2 + D/2).
template <typename T, int D>
struct QFrag;
template <int D>
struct QFrag<__bf16, D> {
  bf16x8 v[D / 16];
};
template <int D>
struct QFrag<float, D> {
  float v[D / 2];
};

// Per-wave running state of the online softmax for its 32 query rows.
template <int D>
struct RowState {
  f32x16 acc[D / 32];  // O^T accumulator: lane holds query (l % 32), 16 d rows per tile
  float m, l;          // running max (base-2 scaled) and this lane's partial sum
};

// Phase 1 of a kv tile: S^T = K Q^T for the tile's two 32-key blocks.
template <typename T, int D>
__device__ __forceinline__ void s_product(const char* Ks, const QFrag<T, D>& qf, int g, int krow_a,
                                          f32x16& s0, f32x16& s1) {
  using C = Cfg<T, D>;
  s0 = f32x16{};
  s1 = f32x16{};
  if constexpr (sizeof(T) == 2) {
#pragma unroll
    for (int ks = 0; ks < D / 16; ++ks) {
      const bf16x8 k0 = *reinterpret_cast<const bf16x8*>(Ks + krow_a * C::kKP + (ks * 16 + g * 8) * 2);
      const bf16x8 k1 = *reinterpret_cast<const bf16x8*>(Ks + (32 + krow_a) * C::kKP + (ks * 16 + g * 8) * 2);
      s0 = mfma(k0, qf.v[ks], s0);
      s1 = mfma(k1, qf.v[ks], s1);
    }
  } else {
#pragma unroll
    for (int c = 0; c < D / 8; ++c) {
      const float4 k0 = *reinterpret_cast<const float4*>(Ks + krow_a * C::kKP + (g * (D / 2) + c * 4) * 4);
      const float4 k1 = *reinterpret_cast<const float4*>(Ks + (32 + krow_a) * C::kKP + (g * (D / 2) + c * 4) * 4);
      s0 = mfma(k0.x, qf.v[c * 4 + 0], s0);
      s1 = mfma(k1.x, qf.v[c * 4 + 0], s1);
      s0 = mfma(k0.y, qf.v[c * 4 + 1], s0);
      s1 = mfma(k1.y, qf.v[c * 4 + 1], s1);
      s0 = mfma(k0.z, qf.v[c * 4 + 2], s0);
      s1 = mfma(k1.z, qf.v[c * 4 + 2], s1);
      s0 = mfma(k0.w, qf.v[c * 4 + 3], s0);
      s1 = mfma(k1.w, qf.v[c * 4 + 3], s1);
    }
  }
}

// The element predicate on one tile's scores (lane layout of the S product):
// hidden pairs become -inf.  Key ids of the tile come from LDS.
template <typename T, int D, int KIND>
__device__ __forceinline__ void mask_scores(float (&x)[32], const char* Ks, const FwdDev& p,
                                            const SeqBounds& sb, int kt, int qi, QIds qids,
                                            int g) {
  using C = Cfg<T, D>;
  const int32_t* ids = reinterpret_cast<const int32_t*>(Ks + C::kKBuf + C::kVBuf);
#pragma unroll
  for (int b = 0; b < 2; ++b) {
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      const int jj = b * 32 + 16 * (r >> 3) + 8 * g + (r & 7);
      KIds kid{0, 0, 0, 0};
      if constexpr (KIND == BMATTN_MASK_SHARED_PREFIX || KIND == BMATTN_MASK_STRIP_THINKING)
        kid = KIds{ids[jj], ids[kBN + jj], 0, 0};
      if constexpr (KIND == BMATTN_MASK_COMPOSED)
        kid = KIds{ids[jj], ids[kBN + jj], ids[2 * kBN + jj], ids[3 * kBN + jj]};
      x[b * 16 + r] = visible_k<KIND>(p.mask, sb, qi, qids, kt * kBN + jj, kid) ? x[b * 16 + r]
                                                                               : -INFINITY;
    }
  }
}

// Phase 2: the element mask (PARTIAL tiles), the online-softmax update and
// the probabilities in x (overwritten in place).
// Register r of block b holds key kt*64 + b*32 + 16*(r/8) + 8*g + r%8.
// Scores stay unscaled until the exponent: max(s * c) = c * max(s) for the
// positive scale c, and exp2(s * c - m) is one fma and one exp.
template <typename T, int D, bool MASKED>
__device__ __forceinline__ void softmax_update(f32x16& s0, f32x16& s1, RowState<D>& st,
                                               const char* Ks, const FwdDev& p,
                                               const SeqBounds& sb, int kt, int qi, QIds qids,
                                               int g) {
  using C = Cfg<T, D>;
  if constexpr (MASKED) {
    // The predicate is applied on a plain array copy: conditional element
    // stores through a reference to the MFMA result vector were not kept by
    // the compiler.  One straight-line instance per mask kind.
    float x[32];
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      x[r] = s0[r];
      x[16 + r] = s1[r];
    }
    switch (p.mask.kind) {
      case BMATTN_MASK_FULL: mask_scores<T, D, BMATTN_MASK_FULL>(x, Ks, p, sb, kt, qi, qids, g); break;
      case BMATTN_MASK_CAUSAL: mask_scores<T, D, BMATTN_MASK_CAUSAL>(x, Ks, p, sb, kt, qi, qids, g); break;
      case BMATTN_MASK_SHARED_PREFIX:
        mask_scores<T, D, BMATTN_MASK_SHARED_PREFIX>(x, Ks, p, sb, kt, qi, qids, g);
        break;
      case BMATTN_MASK_STRIP_THINKING:
        mask_scores<T, D, BMATTN_MASK_STRIP_THINKING>(x, Ks, p, sb, kt, qi, qids, g);
        break;
      default: mask_scores<T, D, BMATTN_MASK_COMPOSED>(x, Ks, p, sb, kt, qi, qids, g); break;
    }
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      s0[r] = x[r];
      s1[r] = x[16 + r];
    }
  }
  const float sl2 = p.scale_log2;
  float mx = s0[0];
#pragma unroll
  for (int r = 1; r < 16; ++r) mx = fmaxf(mx, s0[r]);
#pragma unroll
  for (int r = 0; r < 16; ++r) mx = fmaxf(mx, s1[r]);
  mx = fmaxf(mx, __shfl_xor(mx, 32)) * sl2;
  // Lazy rescaling: the reference max st.m moves only when the tile's max
  // exceeds it by more than kRescaleSlack (log2 units), or when it is still
  // -inf.  exp2(s - m_ref) then stays below 2^kRescaleSlack, and O = acc / l
  // is the same quantity for any reference, so skipping the rescale of acc
  // changes only rounding.  The decision is per wave so acc is rescaled in a
  // wave-uniform branch.
  const bool grow = !(mx <= st.m + kRescaleSlack);
  float m_ref = st.m;
  if (__ballot(grow)) {
    const float m_new = fmaxf(st.m, mx);
    const float m_use = (m_new == -INFINITY) ? 0.f : m_new;
    const float alpha = fast_exp2(st.m - m_use);
    st.l *= alpha;
#pragma unroll
    for (int dt = 0; dt < C::kDT; ++dt) st.acc[dt] *= alpha;
    st.m = m_new;
    m_ref = m_use;
  }
  // A row with nothing visible so far keeps -inf; its exponents use 0 so that
  // masked scores give exp2(-inf) = 0, never -inf + inf.
  if constexpr (MASKED) m_ref = (m_ref == -INFINITY) ? 0.f : m_ref;
  float rs = 0.f;
#pragma unroll
  for (int r = 0; r < 16; ++r) {
    s0[r] = fast_exp2(fmaf(s0[r], sl2, -m_ref));
    rs += s0[r];
  }
#pragma unroll
  for (int r = 0; r < 16; ++r) {
    s1[r] = fast_exp2(fmaf(s1[r], sl2, -m_ref));
    rs += s1[r];
  }
  st.l += rs;
}

// Phase 3: acc^T += V^T P^T; p0/p1 hold the probabilities of the two
// 32-key blocks in the accumulator layout of the S product.
template <typename T, int D>
__device__ __forceinline__ void pv_product(const char* Ks, const f32x16& p0, const f32x16& p1,
                                           RowState<D>& st, int g, int l32) {
  using C = Cfg<T, D>;
  const char* Vt = Ks + C::kKBuf;
  if constexpr (sizeof(T) == 2) {
    bf16x8 pf[4];
#pragma unroll
    for (int k = 0; k < 4; ++k) {
      const f32x16& src = (k < 2) ? p0 : p1;
      const int r0 = (k & 1) * 8;
      uint4 u;
      u.x = pack_bf16x2(src[r0 + 0], src[r0 + 1]);
      u.y = pack_bf16x2(src[r0 + 2], src[r0 + 3]);
      u.z = pack_bf16x2(src[r0 + 4], src[r0 + 5]);
      u.w = pack_bf16x2(src[r0 + 6], src[r0 + 7]);
      pf[k] = __builtin_bit_cast(bf16x8, u);
    }
#pragma unroll
    for (int k = 0; k < 4; ++k) {
#pragma unroll
      for (int dt = 0; dt < C::kDT; ++dt) {
        const bf16x8 vf = *reinterpret_cast<const bf16x8*>(Vt + (dt * 32 + l32) * C::kVP + (k * 16 + g * 8) * 2);
        st.acc[dt] = mfma(vf, pf[k], st.acc[dt]);
      }
    }
  } else {
#pragma unroll
    for (int b = 0; b < 2; ++b) {
      const f32x16& src = b == 0 ? p0 : p1;
#pragma unroll
      for (int hh = 0; hh < 2; ++hh) {
#pragma unroll
        for (int dt = 0; dt < C::kDT; ++dt) {
          const char* vs = Vt + (dt * 32 + l32) * C::kVP + (b * 32 + 16 * hh + 8 * g) * 4;
          const float4 v0 = *reinterpret_cast<const float4*>(vs);
          const float4 v1 = *reinterpret_cast<const float4*>(vs + 16);
          const int r0 = hh * 8;
          st.acc[dt] = mfma(v0.x, src[r0 + 0], st.acc[dt]);
          st.acc[dt] = mfma(v0.y, src[r0 + 1], st.acc[dt]);
          st.acc[dt] = mfma(v0.z, src[r0 + 2], st.acc[dt]);
          st.acc[dt] = mfma(v0.w, src[r0 + 3], st.acc[dt]);
          st.acc[dt] = mfma(v1.x, src[r0 + 4], st.acc[dt]);
          st.acc[dt] = mfma(v1.y, src[r0 + 5], st.acc[dt]);
          st.acc[dt] = mfma(v1.z, src[r0 + 6], st.acc[dt]);
          st.acc[dt] = mfma(v1.w, src[r0 + 7], st.acc[dt]);
        }
      }
    }
  }
}

// One kv tile for one wave group: the S product, softmax and P V product of
// tile kt from LDS stage `cur`, with the group's next tile (ktn) staged into
// `nxt`.  K(next) is loaded before the S product and stored after the
// softmax; V(next) is loaded after the S product and stored after the P V
// product, so at most one operand's staging registers are live at a time.
template <typename T, int D, bool PAGED, bool MASKED>
__device__ __forceinline__ void kv_step(const char* cur, char* nxt, bool has_next, bool mnext,
                                        int ktn, int kt, const FwdDev& p, const SeqBounds& sb,
                                        int s, int h, int gtid,
                                        const typename Prefill<T, D, PAGED>::Offsets& off,
                                        uint4 (&kr)[Cfg<T, D>::kKChunks],
                                        uint4 (&vr)[Cfg<T, D>::kKpt], KIds& kid,
                                        const QFrag<T, D>& qf, RowState<D>& st, int qi, QIds qids,
                                        int g, int l32, int krow_a) {
  using P = Prefill<T, D, PAGED>;
  mnext = MASKED || mnext;  // PARTIAL tiles follow FULL ones in the lists
  if (has_next) {
    if (mnext) P::template load_k<true>(p, sb, s, h, ktn, gtid, off, kr);
    else P::template load_k<false>(p, sb, s, h, ktn, gtid, off, kr);
  }
  f32x16 s0, s1;
  s_product<T, D>(cur, qf, g, krow_a, s0, s1);
  if (has_next) {
    if (mnext) P::template load_v<true>(p, sb, s, h, ktn, gtid, off, vr, kid);
    else P::template load_v<false>(p, sb, s, h, ktn, gtid, off, vr, kid);
  }
  softmax_update<T, D, MASKED>(s0, s1, st, cur, p, sb, kt, qi, qids, g);
  if (has_next) P::store_k(nxt, gtid, kr);
  pv_product<T, D>(cur, s0, s1, st, g, l32);
  if (has_next) P::store_v(nxt, gtid, mnext, vr, kid);
}

// A workgroup owns 128 query rows of one (sequence, head) and walks the
// row's kv-tile list.  With KG = 2 it has two groups of four waves over the
// same query rows: group 0 takes list entries 0, 2, 4, ..., group 1 entries
// 1, 3, 5, ..., each with its own double-buffered LDS stages, which halves
// the serial chain of a long row.  At the end the two partial states
// (running max, sum and accumulator) are combined through LDS:
// m = max(m0, m1), l = l0 2^(m0-m) + l1 2^(m1-m), acc likewise.
template <typename T, int D, bool PAGED, int KG>
__global__ __launch_bounds__(kThreads * KG, 2) void prefill_kernel(FwdDev p) {
  using C = Cfg<T, D>;
  using P = Prefill<T, D, PAGED>;
  __shared__ __attribute__((aligned(16))) char smem[2 * KG * C::kStage];

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int grp = wave >> 2;             // kv group
  const int gw = wave & 3;               // wave inside the group
  const int gtid = tid & (kThreads - 1);  // thread inside the group
  const int l32 = lane & 31, g = lane >> 5;
  char* gsm = smem + grp * 2 * C::kStage;

  // Dispatch order: row rank major (longest rows first, over all heads),
  // head minor.  Workgroups go round-robin over the 8 XCDs, so head h always
  // runs on XCD (h mod 8) when the head count is a multiple of 8 and its K/V
  // stay in that XCD's L2.
  const uint32_t w = blockIdx.x;
  const int h = (int)(w % (uint32_t)p.num_heads);
  const int row = p.row_order[w / (uint32_t)p.num_heads];
  const int s = row / p.n_qt, a = row % p.n_qt;
  const SeqBounds sb = seq_bounds(p.mask, s, p.max_lq, p.max_lk);
  if (a * kBM >= sb.lq) return;
  const int nfull = p.full_cnt[row];
  const int ntiles = nfull + p.part_cnt[row];
  const int32_t* flist = p.full_idx + (int64_t)row * p.n_kt;
  const int32_t* plist = p.part_idx + (int64_t)row * p.n_kt;

  const int qi = a * kBM + gw * 32 + l32;  // query row inside the sequence
  const bool qvalid = qi < sb.lq;
  const QIds qids = load_qids(p.mask, sb, qi);

  // Q operand (B of S^T = K Q^T), resident for the whole kv loop.
  QFrag<T, D> qf;
  {
    const char* qrow = static_cast<const char*>(p.q) +
                       ((sb.q0 + (qvalid ? qi : 0)) * p.q_st + (int64_t)h * p.q_sh) * C::kElem;
    if constexpr (sizeof(T) == 2) {
#pragma unroll
      for (int ks = 0; ks < D / 16; ++ks) {
        uint4 x = qvalid ? *reinterpret_cast<const uint4*>(qrow + (ks * 16 + g * 8) * 2)
                         : make_uint4(0, 0, 0, 0);
        qf.v[ks] = __builtin_bit_cast(bf16x8, x);
      }
    } else {
#pragma unroll
      for (int c = 0; c < D / 8; ++c) {
        float4 x = qvalid ? *reinterpret_cast<const float4*>(qrow + (g * (D / 2) + c * 4) * 4)
                          : make_float4(0, 0, 0, 0);
        qf.v[c * 4 + 0] = x.x;
        qf.v[c * 4 + 1] = x.y;
        qf.v[c * 4 + 2] = x.z;
        qf.v[c * 4 + 3] = x.w;
      }
    }
  }

  RowState<D> st;
#pragma unroll
  for (int dt = 0; dt < C::kDT; ++dt) st.acc[dt] = f32x16{};
  st.m = -INFINITY;
  st.l = 0.f;
  const int krow_a = sigma(l32);

  uint4 kr[C::kKChunks];
  uint4 vr[C::kKpt];
  KIds kid{0, 0, 0, 0};
  const typename P::Offsets off = P::offsets(p, gtid);
  // The group's first tile is list entry grp.
  if (grp < ntiles) {
    if (grp < nfull) {
      P::template load_k<false>(p, sb, s, h, flist[grp], gtid, off, kr);
      P::template load_v<false>(p, sb, s, h, flist[grp], gtid, off, vr, kid);
    } else {
      P::template load_k<true>(p, sb, s, h, plist[grp - nfull], gtid, off, kr);
      P::template load_v<true>(p, sb, s, h, plist[grp - nfull], gtid, off, vr, kid);
    }
    P::store_k(gsm, gtid, kr);
    P::store_v(gsm, gtid, grp >= nfull, vr, kid);
  }
  // Drain every outstanding load (the Q operand included) before the loops so
  // that no wait for them is carried into a loop body.
  __builtin_amdgcn_s_waitcnt(0);
  __syncthreads();

  // Iteration i handles list entry t = i*KG + grp of each group; all groups
  // run the same number of iterations (one barrier each).
  const int niter = (ntiles + KG - 1) / KG;
  const int nfull_iter = nfull / KG;  // iterations whose tiles are FULL for every group
  int i = 0;
  for (; i < nfull_iter; ++i) {
    const int t = i * KG + grp, tn = t + KG;
    const bool has_next = tn < ntiles;
    const bool mnext = tn >= nfull;
    const int ktn = has_next ? (mnext ? plist[tn - nfull] : flist[tn]) : 0;
    kv_step<T, D, PAGED, false>(gsm + (i & 1) * C::kStage, gsm + ((i + 1) & 1) * C::kStage,
                                has_next, mnext, ktn, flist[t], p, sb, s, h, gtid, off, kr, vr, kid,
                                qf, st, qi, qids, g, l32, krow_a);
    __syncthreads();
  }
  for (; i < niter; ++i) {
    const int t = i * KG + grp, tn = t + KG;
    if (t < ntiles) {
      const bool has_next = tn < ntiles;
      const bool mnext = tn >= nfull;
      const int ktn = has_next ? (mnext ? plist[tn - nfull] : flist[tn]) : 0;
      const char* cur = gsm + (i & 1) * C::kStage;
      char* nxt = gsm + ((i + 1) & 1) * C::kStage;
      if (t < nfull) {
        kv_step<T, D, PAGED, false>(cur, nxt, has_next, mnext, ktn, flist[t], p, sb, s, h, gtid,
                                    off, kr, vr, kid, qf, st, qi, qids, g, l32, krow_a);
      } else {
        kv_step<T, D, PAGED, true>(cur, nxt, has_next, true, ktn, plist[t - nfull], p, sb, s, h,
                                   gtid, off, kr, vr, kid, qf, st, qi, qids, g, l32, krow_a);
      }
    }
    __syncthreads();
  }

  if constexpr (KG == 2) {
    // Group 1 hands its state to group 0 through LDS (lane-major, so the
    // same lane of the partner wave holds the same query and d rows).
    constexpr int kRegs = C::kDT * 16 + 2;
    float* xch = reinterpret_cast<float*>(smem) + gw * kRegs * 64;
    if (grp == 1) {
#pragma unroll
      for (int dt = 0; dt < C::kDT; ++dt) {
#pragma unroll
        for (int r = 0; r < 16; ++r) xch[(dt * 16 + r) * 64 + lane] = st.acc[dt][r];
      }
      xch[(kRegs - 2) * 64 + lane] = st.m;
      xch[(kRegs - 1) * 64 + lane] = st.l;
    }
    __syncthreads();
    if (grp == 1) return;
    const float m1 = xch[(kRegs - 2) * 64 + lane];
    const float l1 = xch[(kRegs - 1) * 64 + lane];
    const float m = fmaxf(st.m, m1);
    const float mu = (m == -INFINITY) ? 0.f : m;
    const float a0 = fast_exp2(st.m - mu), a1 = fast_exp2(m1 - mu);
    st.l = st.l * a0 + l1 * a1;
#pragma unroll
    for (int dt = 0; dt < C::kDT; ++dt) {
#pragma unroll
      for (int r = 0; r < 16; ++r) st.acc[dt][r] = st.acc[dt][r] * a0 + xch[(dt * 16 + r) * 64 + lane] * a1;
    }
    st.m = m;
  }

  // ---- epilogue: O = acc / l, LSE = m + ln(l) ------------------------------
  const float l_tot = st.l + __shfl_xor(st.l, 32);
  const float inv = l_tot > 0.f ? 1.f / l_tot : 0.f;
  if (qvalid) {
    char* orow = static_cast<char*>(p.o) + ((sb.q0 + qi) * p.o_st + (int64_t)h * p.o_sh) * C::kElem;
#pragma unroll
    for (int dt = 0; dt < C::kDT; ++dt) {
#pragma unroll
      for (int a4 = 0; a4 < 4; ++a4) {
        const int d0 = dt * 32 + 8 * a4 + 4 * g;
        const float o0 = st.acc[dt][a4 * 4 + 0] * inv, o1 = st.acc[dt][a4 * 4 + 1] * inv;
        const float o2 = st.acc[dt][a4 * 4 + 2] * inv, o3 = st.acc[dt][a4 * 4 + 3] * inv;
        if constexpr (sizeof(T) == 2) {
          *reinterpret_cast<uint2*>(orow + d0 * 2) = make_uint2(pack_bf16x2(o0, o1), pack_bf16x2(o2, o3));
        } else {
          *reinterpret_cast<float4*>(orow + d0 * 4) = make_float4(o0, o1, o2, o3);
        }
      }
    }
    if (g == 0 && p.lse != nullptr) {
      const float lse = l_tot > 0.f ? (st.m + __log2f(l_tot)) * kLn2 : -INFINITY;
      p.lse[(int64_t)h * p.lse_sh + sb.q0 + qi] = lse;
    }
  }
}

// Two kv groups where four LDS stages fit (every compiled type but fp32 with
// head_dim 128, whose stage is twice as large).
template <typename T, int D>
constexpr int kv_groups() {
  return 4 * Cfg<T, D>::kStage <= 160 * 1024 ? 2 : 1;
}

template <typename T, int D>
hipError_t launch_typed(const FwdDev& p, bool paged, hipStream_t st) {
  constexpr int KG = kv_groups<T, D>();
  const int64_t grid = (int64_t)p.mask.n_seqs * p.n_qt * p.num_heads;
  if (grid == 0) return hipSuccess;
  if (grid > INT32_MAX) return hipErrorInvalidValue;
  if (paged) {
    hipLaunchKernelGGL((prefill_kernel<T, D, true, KG>), dim3((uint32_t)grid), dim3(kThreads * KG), 0, st, p);
  } else {
    hipLaunchKernelGGL((prefill_kernel<T, D, false, KG>), dim3((uint32_t)grid), dim3(kThreads * KG), 0, st, p);
  }
  return hipGetLastError();
}

}  // namespace

hipError_t launch_forward_prefill(const FwdDev& p, int dtype, bool paged, hipStream_t st) {
  if (p.block_m != kBM || p.block_n != kBN) return hipErrorInvalidValue;
  if (dtype == BMATTN_BF16) return launch_forward_prefill_bf16(p, paged, st);
  if (dtype == BMATTN_F32 && p.head_dim == 128) return launch_typed<float, 128>(p, paged, st);
  if (dtype == BMATTN_F32 && p.head_dim == 64) return launch_typed<float, 64>(p, paged, st);
  return hipErrorInvalidValue;
}

}  // namespace bmattn
