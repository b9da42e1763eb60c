// Block-sparse masked attention forward for bf16 inputs, query tiles of 128
// rows (gfx950).
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
//  * a workgroup = 4 waves = the 128 query rows of one (sequence, head);
//    each wave owns 32 query rows for the whole kv loop.  Two workgroups
//    share a CU and run out of phase;
//  * K and V tiles (64 keys) go from HBM straight into LDS with
//    global_load_lds_dwordx4 (no registers, no VALU): one wave instruction
//    fills 1 KiB, each lane choosing which 16-byte piece of the tile lands in
//    its slot.  Rows stay row-major with the 16-byte columns XOR-swizzled per
//    row, so both operand reads below are free of bank conflicts;
//  * a wave computes S^T = K Q^T with v_mfma_f32_32x32x16_bf16 (A = K rows
//    read with ds_read_b128, rows permuted by swapping bits 2 and 3 so each
//    lane's 8 consecutive accumulator registers hold 8 consecutive keys; B =
//    the wave's Q rows in registers), so lane l holds the scores of query
//    (l % 32) and the row max / sum are lane-local plus one exchange with
//    lane l ^ 32;
//  * the probabilities feed acc^T += V^T P^T as the B operand straight from
//    registers; the V^T operand comes from the row-major V tile through
//    ds_read_b64_tr_b16, the gfx950 transposing LDS read: 16 lanes each read
//    4 consecutive bf16 of one key row, and lane i receives column i of the
//    resulting 4 x 16 block, i.e. 4 keys of one d;
//  * the next tile's copies are issued one per 16-d step of the current
//    tile's S product, between its MFMA pairs, and waited for only at the
//    end of the iteration: one barrier per tile.  The list entry two tiles
//    ahead is loaded early and read after that barrier, and so are the
//    first four K fragments of the next tile, so that their LDS latency
//    runs beside the P V MFMAs still in flight;
//  * exponentials are base 2 with log2(e) folded into the softmax scale, and
//    the reference max moves only when it would grow by more than 8.
#include <hip/hip_runtime.h>

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

constexpr int kBM = 128;           // query rows of a workgroup
constexpr int kBN = 64;            // keys of a kv tile
constexpr int kWaves = 4;          // waves of a workgroup, 32 query rows each
constexpr int kThreads = 64 * kWaves;
constexpr float kLn2 = 0.69314718055994530942f;
constexpr float kRescaleSlack = 8.0f;

template <int D>
struct Lay {
  static constexpr int kRowB = D * 2;                 // bytes of one K/V row
  static constexpr int kCh = kRowB / 16;               // 16-byte columns per row
  static constexpr int kTileB = kBN * kRowB;           // bytes of a K (or V) tile
  static constexpr int kV = kTileB;                    // V tile offset in a stage
  static constexpr int kIds = 2 * kTileB;              // key ids of a PARTIAL tile (4 arrays)
  static constexpr int kStage = 2 * kTileB + 4 * kBN * 4;
  static constexpr int kCopies = kTileB / 1024 / kWaves;  // 1 KiB copies per wave per tile
  static constexpr int kDT = D / 32;                   // 32-wide output d tiles
  static_assert(kCopies >= 1 && kCopies * 1024 * kWaves == kTileB, "tile / copy mismatch");
};

// Physical 16-byte column of logical column c in tile row r is c ^ swz(r).
// D 128 (16 columns): the four low row bits with their halves swapped; D 64
// (8 columns): row bits 1..3 rotated.  Either way the 16 rows read by 16
// lanes of a K fragment, and the 4 rows x 64 bytes read by 32 lanes of a
// transposing V read, cover 256 bytes of distinct banks.
template <int D>
__device__ __forceinline__ int swz(int r) {
  if constexpr (D == 128) return ((r & 3) << 2) | ((r >> 2) & 3);
  else return (((r >> 1) & 1) << 2) | ((r >> 2) & 3);
}

__device__ __forceinline__ f32x16 mfma(const bf16x8& a, const bf16x8& b, const f32x16& c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
}

__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }

// Row index permutation of the 32-row MFMA operand: swaps bits 2 and 3.
__device__ __forceinline__ int sigma(int i) {
  return (i & ~12) | ((i & 4) << 1) | ((i & 8) >> 1);
}

// HBM -> LDS copies (global_load_lds_dword[x4]): lane i's 4 or 16 bytes from
// `src` land at LDS byte lds + 4i or lds + 16i.  Written as inline assembly
// so that the compiler does not treat the pending copies as writes that
// every later LDS read might depend on (it would wait for them before the
// first read of the current stage); the copies are waited for explicitly at
// the end of each tile.
__device__ __forceinline__ uint32_t lds_addr(const void* p) {
  return static_cast<uint32_t>(reinterpret_cast<uintptr_t>(LDS_PTR(const char, p)));
}
__device__ __forceinline__ void copy16(const void* src, uint32_t lds) {
  asm volatile("global_load_lds_dwordx4 %0, off" ::"v"(src), "{m0}"(lds) : "memory");
}
__device__ __forceinline__ void copy16s(uint32_t off, const void* base, uint32_t lds) {
  asm volatile("global_load_lds_dwordx4 %0, %1" ::"v"(off), "s"(base), "{m0}"(lds) : "memory");
}
__device__ __forceinline__ void copy4(const void* src, uint32_t lds) {
  asm volatile("global_load_lds_dword %0, off" ::"v"(src), "{m0}"(lds) : "memory");
}

// Two floats -> two bf16 (round to nearest even) in one dword, lo first.
__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
  return __builtin_bit_cast(uint32_t, __builtin_convertvector((f32x2{lo, hi}), bf16x2));
}

// The key-id array that wave gw stages for a PARTIAL tile, or none:
// shared-prefix: the segment; strip-thinking: role, turn; composed: segment,
// role, turn, document (those its terms read), one wave each.
template <bool COMP>
__device__ __forceinline__ const int32_t* id_source(const MaskDev& m, int gw) {
  if constexpr (COMP) {
    if (gw == 0) return (m.terms & BMATTN_TERM_SHARED_PREFIX) ? m.seg_k : nullptr;
    if (gw == 1) return (m.terms & BMATTN_TERM_STRIP_THINKING) ? m.role_k : nullptr;
    if (gw == 2) return (m.terms & BMATTN_TERM_STRIP_THINKING) ? m.turn_k : nullptr;
    return (m.terms & BMATTN_TERM_DOCUMENT) ? m.doc_k : nullptr;
  } else {
    if (gw >= 2) return nullptr;
    if (m.kind == BMATTN_MASK_SHARED_PREFIX) return gw == 0 ? m.seg_k : nullptr;
    if (m.kind == BMATTN_MASK_STRIP_THINKING) return gw == 0 ? m.role_k : m.turn_k;
    return nullptr;
  }
}

// HBM -> LDS copies of one kv tile by one wave of the workgroup.  Copy u of wave
// gw fills 16-byte slots [64 (gw*kCopies + u), +64) of the tile; slot s holds
// row s / kCh, physical column s % kCh, i.e. logical column
// (s % kCh) ^ swz(row).  Rows past the sequence end read its last row: those
// keys are hidden by the predicate (they only occur in PARTIAL tiles), and
// the values read are finite.
template <int D, bool PAGED, bool COMP>
struct Copy {
  using L = Lay<D>;
  uint32_t koff[L::kCopies], voff[L::kCopies];
  bool short_ok;
  __device__ __forceinline__ Copy(const FwdDev& p, int gw, int lane) {
    short_ok = !PAGED && (int64_t)kBN * (p.k_st > p.v_st ? p.k_st : p.v_st) * 2 < (int64_t(1) << 31);
#pragma unroll
    for (int u = 0; u < L::kCopies; ++u) {
      const int slot = (gw * L::kCopies + u) * 64 + lane;
      const int r = slot / L::kCh, col = (slot % L::kCh) ^ swz<D>(r);
      koff[u] = short_ok ? (uint32_t)(r * p.k_st * 2 + col * 16) : 0u;
      voff[u] = short_ok ? (uint32_t)(r * p.v_st * 2 + col * 16) : 0u;
    }
  }
  __device__ __forceinline__ void general(const FwdDev& p, const SeqBounds& sb, int s, int h, int kt,
                                          int gw, int lane, char* stage) const {
    int j[L::kCopies], col[L::kCopies];
    int64_t row[L::kCopies];
#pragma unroll
    for (int u = 0; u < L::kCopies; ++u) {
      const int slot = (gw * L::kCopies + u) * 64 + lane;
      const int r = slot / L::kCh;
      col[u] = (slot % L::kCh) ^ swz<D>(r);
      j[u] = max(min(kt * kBN + r, sb.lk - 1), 0);
    }
    if constexpr (!PAGED) {
#pragma unroll
      for (int u = 0; u < L::kCopies; ++u) row[u] = sb.k0 + j[u];
    } else {
      int32_t pe[L::kCopies];
#pragma unroll
      for (int u = 0; u < L::kCopies; ++u)
        pe[u] = page_entry(p.block_table, p.bt_stride, s, j[u], p.page_size, p.page_shift);
#pragma unroll
      for (int u = 0; u < L::kCopies; ++u)
        row[u] = row_in_page(pe[u], j[u], p.page_size, p.page_shift, p.num_pages);
    }
#pragma unroll
    for (int u = 0; u < L::kCopies; ++u) {
      const char* ks = static_cast<const char*>(p.k) + (row[u] * p.k_st + (int64_t)h * p.k_sh) * 2 + col[u] * 16;
      copy16(ks, lds_addr(stage + (gw * L::kCopies + u) * 1024));
    }
#pragma unroll
    for (int u = 0; u < L::kCopies; ++u) {
      const char* vs = static_cast<const char*>(p.v) + (row[u] * p.v_st + (int64_t)h * p.v_sh) * 2 + col[u] * 16;
      copy16(vs, lds_addr(stage + L::kV + (gw * L::kCopies + u) * 1024));
    }
  }
  __device__ __forceinline__ bool whole(const SeqBounds& sb, int kt) const {
    return short_ok && (kt + 1) * kBN <= sb.lk;
  }
  __device__ __forceinline__ void ids(const FwdDev& p, const SeqBounds& sb, int kt, int gw, int lane,
                                      char* stage) const {
    const int32_t* src = id_source<COMP>(p.mask, gw);
    if (src != nullptr) {
      const int jj = max(min(kt * kBN + lane, sb.lk - 1), 0);
      copy4(src + sb.k0 + jj, lds_addr(stage + L::kIds + gw * kBN * 4));
    }
  }
  __device__ __forceinline__ void tile(const FwdDev& p, const SeqBounds& sb, int s, int h, int kt,
                                       bool masked, int gw, int lane, char* stage) const {
    if (short_ok && (kt + 1) * kBN <= sb.lk) {
      const char* kb = static_cast<const char*>(p.k) + ((sb.k0 + (int64_t)kt * kBN) * p.k_st + (int64_t)h * p.k_sh) * 2;
      const char* vb = static_cast<const char*>(p.v) + ((sb.k0 + (int64_t)kt * kBN) * p.v_st + (int64_t)h * p.v_sh) * 2;
#pragma unroll
      for (int u = 0; u < L::kCopies; ++u) copy16s(koff[u], kb, lds_addr(stage + (gw * L::kCopies + u) * 1024));
#pragma unroll
      for (int u = 0; u < L::kCopies; ++u) copy16s(voff[u], vb, lds_addr(stage + L::kV + (gw * L::kCopies + u) * 1024));
    } else {
      general(p, sb, s, h, kt, gw, lane, stage);
    }
    if (masked) ids(p, sb, kt, gw, lane, stage);
  }
};

// Running state of the online softmax for the wave's 32 rows.
template <int D>
struct RowState {
  f32x16 acc[D / 32];  // O^T accumulator: lane holds query (l % 32), 16 d rows per tile
  float m, l;          // reference max (base-2 scaled) and this lane's partial sum
};

// Per-lane LDS byte offsets of the operand reads, fixed for the kernel.
template <int D>
struct Addr {
  using L = Lay<D>;
  int k[D / 16];          // K fragment of step ks, 32-key block 0 (block 1: + 32 rows)
  int v[L::kDT][2];       // V^T transposing read of d tile dt, keys +0..3 / +4..7 (chunk 0)
  __device__ __forceinline__ Addr(int lane) {
    const int l32 = lane & 31, g = lane >> 5;
    const int r = sigma(l32);
#pragma unroll
    for (int ks = 0; ks < D / 16; ++ks) k[ks] = r * L::kRowB + (((ks * 2 + g) ^ swz<D>(r)) << 4);
    const int j = lane & 15, b = lane >> 4;
#pragma unroll
    for (int dt = 0; dt < L::kDT; ++dt) {
#pragma unroll
      for (int hf = 0; hf < 2; ++hf) {
        const int row = 8 * (b >> 1) + 4 * hf + (j >> 2);  // + 16 per key chunk
        const int dcol = dt * 32 + 16 * (b & 1) + 4 * (j & 3);
        v[dt][hf] = row * L::kRowB + (((dcol >> 3) ^ swz<D>(row)) << 4) + ((dcol * 2) & 15);
      }
    }
  }
};

// The wave's short-form copies of one whole kv tile: per-copy offsets,
// the tile's K and V bases, and the LDS addresses of the wave's slots.
template <int D>
struct TileCopies {
  uint32_t koff[Lay<D>::kCopies], voff[Lay<D>::kCopies];
  const char* kb;
  const char* vb;
  uint32_t klds, vlds;  // LDS byte addresses of the wave's first K / V slot
};
// S^T = K Q^T for the tile's two 32-key blocks, K fragments read a few
// steps ahead (the first steps' fragments come in `kp`, read by the caller).  With COPIES, the wave's copies of the next (whole) tile are
// issued one per 16-d step, after that step's two MFMAs: a copy that has to
// wait for the memory pipeline then waits beside running matrix work.
// The K fragments of a tile's first (up to four) 16-d steps, both 32-key
// blocks.
template <int D>
struct KPre {
  static constexpr int N = (D / 16) < 4 ? (D / 16) : 4;
  bf16x8 k0[N], k1[N];
};
template <int D>
__device__ __forceinline__ void k_prefetch(const char* Ks, const Addr<D>& ad, KPre<D>& kp) {
#pragma unroll
  for (int ks = 0; ks < KPre<D>::N; ++ks) {
    kp.k0[ks] = *reinterpret_cast<const bf16x8*>(Ks + ad.k[ks]);
    kp.k1[ks] = *reinterpret_cast<const bf16x8*>(Ks + ad.k[ks] + 32 * Lay<D>::kRowB);
  }
}
template <int D, bool COPIES>
__device__ __forceinline__ void s_product(const char* Ks, const bf16x8 (&q)[D / 16], const Addr<D>& ad,
                                          f32x16& s0, f32x16& s1, const TileCopies<D>& tc,
                                          const KPre<D>& kp) {
  using L = Lay<D>;
  constexpr int N = D / 16;
  constexpr int kAhead = KPre<D>::N;
  static_assert(2 * L::kCopies == N, "one copy per 16-d step");
  bf16x8 k0[N], k1[N];
  s0 = f32x16{};
  s1 = f32x16{};
#pragma unroll
  for (int ks = 0; ks < kAhead; ++ks) {
    k0[ks] = kp.k0[ks];
    k1[ks] = kp.k1[ks];
  }
#pragma unroll
  for (int ks = 0; ks < N; ++ks) {
    if (ks + kAhead < N) {
      k0[ks + kAhead] = *reinterpret_cast<const bf16x8*>(Ks + ad.k[ks + kAhead]);
      k1[ks + kAhead] = *reinterpret_cast<const bf16x8*>(Ks + ad.k[ks + kAhead] + 32 * L::kRowB);
    }
    s0 = mfma(k0[ks], q[ks], s0);
    s1 = mfma(k1[ks], q[ks], s1);
    if constexpr (COPIES) {
      if (ks < L::kCopies) copy16s(tc.koff[ks], tc.kb, tc.klds + ks * 1024);
      else copy16s(tc.voff[ks - L::kCopies], tc.vb, tc.vlds + (ks - L::kCopies) * 1024);
    }
  }
}

// The element predicate on one tile, as a bit mask over the lane's 32
// scores: bit 16 b + r is set when the key of register r of block b (key
// kt*64 + 16 c + 8 g + e with c = 2 b + r / 8 and e = r % 8) is visible to
// query qi.  The same predicate as visible_k(), evaluated per lane:
//  * bounds and causality: the key must not pass lim = min(lk - 1,
//    lk - lq + qi) (FULL: lk - 1).  Key offsets grow with the bit index, so
//    the visible bits are a prefix whose length follows from lim directly;
//  * shared-prefix and strip-thinking then AND in the key-id condition, the
//    ids read from the tile's id stage 8 keys at a time;
//  * COMPOSED: each term group ANDs its id terms with its own limit (causal
//    or bounds only), and the groups are ORed.
// The prefix of the bits whose keys lie at or before key lim.
__device__ __forceinline__ uint32_t prefix_bits(int lim, int kt, int g) {
  const int n = lim - kt * kBN - 8 * g + 1;  // keys 16 c + e < n
  const int count = n <= 0 ? 0 : min(32, 8 * (n >> 4) + min(n & 15, 8));
  return count >= 32 ? 0xffffffffu : ((1u << count) - 1u);
}
template <int D, int KIND>
__device__ __forceinline__ uint32_t visible_bits(const char* kstage, const FwdDev& p,
                                                 const SeqBounds& sb, int kt, int qi, QIds qids,
                                                 int g) {
  const bool causal = KIND != BMATTN_MASK_FULL && KIND != BMATTN_MASK_COMPOSED;
  const int lim = causal ? min(sb.lk - 1, sb.lk - sb.lq + qi) : sb.lk - 1;
  uint32_t bits = qi < sb.lq ? prefix_bits(lim, kt, g) : 0u;
  if constexpr (KIND == BMATTN_MASK_SHARED_PREFIX || KIND == BMATTN_MASK_STRIP_THINKING) {
    const int32_t* ida = reinterpret_cast<const int32_t*>(kstage + Lay<D>::kIds);
    const int32_t* idb = ida + kBN;
    uint32_t keep = 0;
#pragma unroll
    for (int c = 0; c < 4; ++c) {
      const int j0 = 16 * c + 8 * g;
      const int4 a0 = *reinterpret_cast<const int4*>(ida + j0);
      const int4 a1 = *reinterpret_cast<const int4*>(ida + j0 + 4);
      const int av[8] = {a0.x, a0.y, a0.z, a0.w, a1.x, a1.y, a1.z, a1.w};
      if constexpr (KIND == BMATTN_MASK_SHARED_PREFIX) {
#pragma unroll
        for (int e = 0; e < 8; ++e) keep |= (uint32_t)((av[e] == 0) | (av[e] == qids.seg)) << (8 * c + e);
      } else {
        const int4 b0 = *reinterpret_cast<const int4*>(idb + j0);
        const int4 b1 = *reinterpret_cast<const int4*>(idb + j0 + 4);
        const int bv[8] = {b0.x, b0.y, b0.z, b0.w, b1.x, b1.y, b1.z, b1.w};
#pragma unroll
        for (int e = 0; e < 8; ++e)
          keep |= (uint32_t)!((av[e] == p.mask.think_role) & (bv[e] < qids.turn)) << (8 * c + e);
      }
    }
    bits &= keep;
  }
  if constexpr (KIND == BMATTN_MASK_COMPOSED) {
    // The four staged arrays: segment, role, turn, document (an array the
    // terms do not read holds stale values that composed_ids_ok ignores).
    // `bits` holds the in-bounds keys; the causal prefix is cb.
    const uint32_t cb = qi < sb.lq ? prefix_bits(min(sb.lk - 1, sb.lk - sb.lq + qi), kt, g) : 0u;
    const int32_t* ida = reinterpret_cast<const int32_t*>(kstage + Lay<D>::kIds);
    uint32_t vis = 0;
#pragma unroll
    for (int c = 0; c < 4; ++c) {
      const int j0 = 16 * c + 8 * g;
      int v[4][8];
#pragma unroll
      for (int a = 0; a < 4; ++a) {
        const int4 x0 = *reinterpret_cast<const int4*>(ida + a * kBN + j0);
        const int4 x1 = *reinterpret_cast<const int4*>(ida + a * kBN + j0 + 4);
        v[a][0] = x0.x; v[a][1] = x0.y; v[a][2] = x0.z; v[a][3] = x0.w;
        v[a][4] = x1.x; v[a][5] = x1.y; v[a][6] = x1.z; v[a][7] = x1.w;
      }
      for (int32_t gs = p.mask.groups; gs != 0; gs >>= 4) {  // wave-uniform
        const int32_t t = gs & 15;
        if (t == 0) continue;
        uint32_t keep = 0;
#pragma unroll
        for (int e = 0; e < 8; ++e)
          keep |= (uint32_t)composed_ids_ok(t, p.mask.think_role, qids, v[0][e], v[1][e], v[2][e], v[3][e])
                  << (8 * c + e);
        vis |= keep & ((t & BMATTN_TERM_CAUSAL) ? cb : bits);
      }
    }
    bits = vis;
  }
  return bits;
}

// The element mask (PARTIAL tiles), the online-softmax update and the
// probabilities, written over the scores.
// Register r of block b holds key kt*64 + b*32 + 16*(r/8) + 8*g + r%8.
// Scores stay unscaled until the exponent: max(s * c) = c * max(s) for the
// positive scale c, and exp2(s * c - m) is one fma and one exp.
template <int D, bool MASKED, bool COMP>
__device__ __forceinline__ void softmax_update(f32x16& s0, f32x16& s1, bf16x8 (&pf)[4], RowState<D>& st,
                                               const char* stage, const FwdDev& p,
                                               const SeqBounds& sb, int kt, int qi, QIds qids,
                                               int g) {
  if constexpr (MASKED) {
    uint32_t vis;
    if constexpr (COMP) {
      vis = visible_bits<D, BMATTN_MASK_COMPOSED>(stage, p, sb, kt, qi, qids, g);
    } else switch (p.mask.kind) {
      case BMATTN_MASK_FULL: vis = visible_bits<D, BMATTN_MASK_FULL>(stage, p, sb, kt, qi, qids, g); break;
      case BMATTN_MASK_CAUSAL: vis = visible_bits<D, BMATTN_MASK_CAUSAL>(stage, p, sb, kt, qi, qids, g); break;
      case BMATTN_MASK_SHARED_PREFIX:
        vis = visible_bits<D, BMATTN_MASK_SHARED_PREFIX>(stage, p, sb, kt, qi, qids, g);
        break;
      default: vis = visible_bits<D, BMATTN_MASK_STRIP_THINKING>(stage, p, sb, kt, qi, qids, g); break;
    }
    // Every element is written, selected -- never a conditional store.
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      s0[r] = ((vis >> r) & 1u) ? s0[r] : -INFINITY;
      s1[r] = ((vis >> (16 + r)) & 1u) ? s1[r] : -INFINITY;
    }
  }
  const float sl2 = p.scale_log2;
  float mx = s0[0];
#pragma unroll
  for (int r = 1; r < 16; ++r) mx = fmaxf(mx, s0[r]);
#pragma unroll
  for (int r = 0; r < 16; ++r) mx = fmaxf(mx, s1[r]);
  {
    // The partner half-wave's max without an LDS round trip: swapping the
    // upper half of one copy with the lower half of another leaves
    // {mx(l), mx(l ^ 32)} in the two results, in some order, on every lane.
    const unsigned u = __float_as_uint(mx);
    const auto sw = __builtin_amdgcn_permlane32_swap(u, u, false, false);
    const unsigned lo = sw[0], hi = sw[1];  // elements copied out before any cast
    mx = fmaxf(__uint_as_float(lo), __uint_as_float(hi)) * sl2;
  }
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
    for (int dt = 0; dt < Lay<D>::kDT; ++dt) st.acc[dt] *= alpha;
    st.m = m_new;
    m_ref = m_use;
  }
  // A row with nothing visible so far keeps -inf; its exponents use 0 so that
  // masked scores give exp2(-inf) = 0, never -inf + inf.
  if constexpr (MASKED) m_ref = (m_ref == -INFINITY) ? 0.f : m_ref;
  const bf16x2 ones = {(__bf16)1.0f, (__bf16)1.0f};
  float rs[4] = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
  for (int k = 0; k < 4; ++k) {
    const f32x16& src = (k < 2) ? s0 : s1;
    const int r0 = (k & 1) * 8;
    uint32_t w[4];
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const float a = fast_exp2(fmaf(src[r0 + 2 * e], sl2, -m_ref));
      const float b = fast_exp2(fmaf(src[r0 + 2 * e + 1], sl2, -m_ref));
      w[e] = pack_bf16x2(a, b);
      rs[k] = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2, w[e]), ones, rs[k], false);
    }
    pf[k] = __builtin_bit_cast(bf16x8, make_uint4(w[0], w[1], w[2], w[3]));
  }
  st.l += (rs[0] + rs[1]) + (rs[2] + rs[3]);
}

// acc^T += V^T P^T.  P (B operand, 8 keys per lane) comes from the softmax
// registers; V^T (A operand: d = lane % 32, keys 8*(lane/32) + 0..7 of each
// 16-key chunk) from two transposing reads of the row-major V tile.
template <int D>
__device__ __forceinline__ void pv_product(const char* stage, const bf16x8 (&pf)[4], RowState<D>& st,
                                           const Addr<D>& ad) {
  using L = Lay<D>;
  const char* Vs = stage + L::kV;
#pragma unroll
  for (int k = 0; k < 4; ++k) {
#pragma unroll
    for (int dt = 0; dt < L::kDT; ++dt) {
      const char* base = Vs + k * 16 * L::kRowB;
      const i16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16(LDS_PTR(i16x4, base + ad.v[dt][0]));
      const i16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16(LDS_PTR(i16x4, base + ad.v[dt][1]));
      const i16x8 vv = __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7);
      st.acc[dt] = mfma(__builtin_bit_cast(bf16x8, vv), pf[k], st.acc[dt]);
    }
  }
}

// One kv tile for one wave: copies of the next tile into `nxt`,
// then the S product, softmax and P V product of tile kt from `cur` (`kp`:
// the first K fragments of `cur`, read by the caller).
template <int D, bool PAGED, bool MASKED, bool COMP>
__device__ __forceinline__ void kv_step(const char* cur, char* nxt, bool has_next, bool mnext,
                                        int ktn, int kt, const int32_t* ahead, int& kt_ahead,
                                        const FwdDev& p, const SeqBounds& sb,
                                        int s, int h, int gw, int lane, const bf16x8 (&q)[D / 16],
                                        const Addr<D>& ad, const Copy<D, PAGED, COMP>& cp,
                                        RowState<D>& st, int qi, QIds qids, int g,
                                        const KPre<D>& kp) {
  using L = Lay<D>;
  const bool whole = has_next && cp.whole(sb, ktn);
  if (has_next && !whole) cp.tile(p, sb, s, h, ktn, MASKED || mnext, gw, lane, nxt);
  if (whole && (MASKED || mnext)) cp.ids(p, sb, ktn, gw, lane, nxt);
  // The list entry two tiles ahead, loaded now and used after the next
  // barrier (whose wait covers it).
  kt_ahead = ahead != nullptr ? *ahead : 0;
  TileCopies<D> tc;
#pragma unroll
  for (int u = 0; u < L::kCopies; ++u) {
    tc.koff[u] = cp.koff[u];
    tc.voff[u] = cp.voff[u];
  }
  tc.kb = static_cast<const char*>(p.k) + ((sb.k0 + (int64_t)ktn * kBN) * p.k_st + (int64_t)h * p.k_sh) * 2;
  tc.vb = static_cast<const char*>(p.v) + ((sb.k0 + (int64_t)ktn * kBN) * p.v_st + (int64_t)h * p.v_sh) * 2;
  tc.klds = lds_addr(nxt + gw * L::kCopies * 1024);
  tc.vlds = lds_addr(nxt + L::kV + gw * L::kCopies * 1024);
  f32x16 s0, s1;
  if (whole) s_product<D, true>(cur, q, ad, s0, s1, tc, kp);
  else s_product<D, false>(cur, q, ad, s0, s1, tc, kp);
  bf16x8 pf[4];
  softmax_update<D, MASKED, COMP>(s0, s1, pf, st, cur, p, sb, kt, qi, qids, g);
  pv_product<D>(cur, pf, st, ad);
}

// A loaded value kept in its vector register until this point (after the
// end-of-tile wait), then taken as wave-uniform: its load is never waited
// for separately, which would also wait for the copies issued before it.
__device__ __forceinline__ int uniform_after_wait(int v) {
  asm volatile("" : "+v"(v));
  return __builtin_amdgcn_readfirstlane(v);
}

// Copies in flight are waited for by every wave, then the barrier makes all
// waves' copies visible and frees the stage that was just read.
__device__ __forceinline__ void end_of_tile() {
  __builtin_amdgcn_s_waitcnt(0);
  __syncthreads();
}

// A workgroup (four waves) owns 128 query rows of one (sequence, head) and
// walks the row's kv-tile list with a double-buffered LDS stage.  Two
// workgroups share a CU (66 KiB of LDS each) and synchronise independently,
// so one workgroup's softmax runs beside the other's matrix work.
// COMP: the COMPOSED kind (its predicate only); otherwise the four plain kinds.
template <int D, bool PAGED, bool COMP>
__global__ __launch_bounds__(kThreads, 2) void prefill_bf16_kernel(FwdDev p) {
  using L = Lay<D>;
  __shared__ __attribute__((aligned(1024))) char smem[2 * L::kStage];

  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int l32 = lane & 31, g = lane >> 5;

  // Dispatch order: row rank major (longest rows first, over all heads),
  // head minor.  Workgroups go round-robin over the 8 XCDs, so head h always
  // runs on XCD (h mod 8) when the head count is a multiple of 8 and its K/V
  // stay in that XCD's L2.
  const uint32_t w = blockIdx.x;
  const int h = (int)(w % (uint32_t)p.num_heads);
  const int row = p.row_order[w / (uint32_t)p.num_heads];
  const int s = row / p.n_qt, a = row % p.n_qt;
  // Everything that depends only on the row is loaded together with the
  // sequence bounds (one round trip): the tile counts and the candidates for
  // the first tile, FULL entry 0 or PARTIAL entry 0.  Indices are clamped to
  // the row.
  const int32_t* flist = p.full_idx + (int64_t)row * p.n_kt;
  const int32_t* plist = p.part_idx + (int64_t)row * p.n_kt;
  const int nfull = p.full_cnt[row];
  const int npart = p.part_cnt[row];
  const int f_first = flist[0];
  const int p_first = plist[0];
  const SeqBounds sb = seq_bounds(p.mask, s, p.max_lq, p.max_lk);
  if (a * kBM >= sb.lq) return;
  const int ntiles = nfull + npart;

  const int qi = a * kBM + wave * 32 + l32;  // query row inside the sequence
  const bool qvalid = qi < sb.lq;
  const QIds qids = load_qids(p.mask, sb, qi);

  // Q operand (B of S^T = K Q^T), resident for the whole kv loop.
  bf16x8 q[D / 16];
  {
    const char* qrow = static_cast<const char*>(p.q) +
                       ((sb.q0 + (qvalid ? qi : 0)) * p.q_st + (int64_t)h * p.q_sh) * 2;
#pragma unroll
    for (int ks = 0; ks < D / 16; ++ks) {
      uint4 x = qvalid ? *reinterpret_cast<const uint4*>(qrow + (ks * 16 + g * 8) * 2)
                       : make_uint4(0, 0, 0, 0);
      q[ks] = __builtin_bit_cast(bf16x8, x);
    }
  }

  RowState<D> st;
#pragma unroll
  for (int dt = 0; dt < L::kDT; ++dt) st.acc[dt] = f32x16{};
  st.m = -INFINITY;
  st.l = 0.f;
  const Addr<D> ad(lane);
  const Copy<D, PAGED, COMP> cp(p, wave, lane);

  // List entry t (FULL entries first, then PARTIAL ones), or none.
  auto entry_ptr = [&](int t) -> const int32_t* {
    return t < ntiles ? (t < nfull ? flist + t : plist + (t - nfull)) : nullptr;
  };
  // The first tile's copies, then the entry of the second tile behind them.
  int kt_cur = 0, kt_nxt = 0;
  if (ntiles > 0) {
    const bool m0 = nfull == 0;
    kt_cur = m0 ? p_first : f_first;
    cp.tile(p, sb, s, h, kt_cur, m0, wave, lane, smem);
    if (ntiles > 1) kt_nxt = *entry_ptr(1);
  }
  end_of_tile();
  // The first K fragments of the next tile are read right after each
  // barrier, ahead of the previous tile's remaining P V MFMAs.  (After the
  // last tile that read is of a stage no copy fills any more; the values
  // are never used.)
  KPre<D> kp;
  k_prefetch<D>(smem, ad, kp);

  // Iteration t handles list entry t: FULL tiles first (no mask code), then
  // the PARTIAL ones.  One barrier per tile.
  int t = 0;
  for (; t < nfull; ++t) {
    const bool has_next = t + 1 < ntiles;
    const bool mnext = t + 1 >= nfull;
    int kt_ahead;
    kv_step<D, PAGED, false, COMP>(smem + (t & 1) * L::kStage, smem + ((t + 1) & 1) * L::kStage, has_next,
                             mnext, kt_nxt, kt_cur, entry_ptr(t + 2), kt_ahead, p, sb, s, h, wave,
                             lane, q, ad, cp, st, qi, qids, g, kp);
    end_of_tile();
    k_prefetch<D>(smem + ((t + 1) & 1) * L::kStage, ad, kp);
    kt_cur = kt_nxt;
    kt_nxt = uniform_after_wait(kt_ahead);
  }
  for (; t < ntiles; ++t) {
    int kt_ahead;
    kv_step<D, PAGED, true, COMP>(smem + (t & 1) * L::kStage, smem + ((t + 1) & 1) * L::kStage,
                            t + 1 < ntiles, true, kt_nxt, kt_cur, entry_ptr(t + 2), kt_ahead, p, sb,
                            s, h, wave, lane, q, ad, cp, st, qi, qids, g, kp);
    end_of_tile();
    k_prefetch<D>(smem + ((t + 1) & 1) * L::kStage, ad, kp);
    kt_cur = kt_nxt;
    kt_nxt = uniform_after_wait(kt_ahead);
  }

  // ---- epilogue: O = acc / l, LSE = m + ln(l) ------------------------------
  const float l_tot = st.l + __shfl_xor(st.l, 32);
  const float inv = l_tot > 0.f ? 1.f / l_tot : 0.f;
  if (qvalid) {
    char* orow = static_cast<char*>(p.o) + ((sb.q0 + qi) * p.o_st + (int64_t)h * p.o_sh) * 2;
#pragma unroll
    for (int dt = 0; dt < L::kDT; ++dt) {
#pragma unroll
      for (int a4 = 0; a4 < 4; ++a4) {
        const int d0 = dt * 32 + 8 * a4 + 4 * g;
        const float o0 = st.acc[dt][a4 * 4 + 0] * inv, o1 = st.acc[dt][a4 * 4 + 1] * inv;
        const float o2 = st.acc[dt][a4 * 4 + 2] * inv, o3 = st.acc[dt][a4 * 4 + 3] * inv;
        *reinterpret_cast<uint2*>(orow + d0 * 2) = make_uint2(pack_bf16x2(o0, o1), pack_bf16x2(o2, o3));
      }
    }
    if (g == 0 && p.lse != nullptr) {
      const float lse = l_tot > 0.f ? (st.m + __log2f(l_tot)) * kLn2 : -INFINITY;
      p.lse[(int64_t)h * p.lse_sh + sb.q0 + qi] = lse;
    }
  }
}

template <int D>
hipError_t launch_d(const FwdDev& p, bool paged, hipStream_t st) {
  static_assert(2 * 2 * Lay<D>::kStage <= 160 * 1024, "two workgroups' LDS stages exceed 160 KiB");
  const int64_t grid64 = (int64_t)p.mask.n_seqs * p.n_qt * p.num_heads;
  if (grid64 == 0) return hipSuccess;
  if (grid64 > INT32_MAX) return hipErrorInvalidValue;
  const uint32_t grid = (uint32_t)grid64;
  const bool comp = p.mask.kind == BMATTN_MASK_COMPOSED;
  if (paged && comp) {
    hipLaunchKernelGGL((prefill_bf16_kernel<D, true, true>), dim3(grid), dim3(kThreads), 0, st, p);
  } else if (paged) {
    hipLaunchKernelGGL((prefill_bf16_kernel<D, true, false>), dim3(grid), dim3(kThreads), 0, st, p);
  } else if (comp) {
    hipLaunchKernelGGL((prefill_bf16_kernel<D, false, true>), dim3(grid), dim3(kThreads), 0, st, p);
  } else {
    hipLaunchKernelGGL((prefill_bf16_kernel<D, false, false>), dim3(grid), dim3(kThreads), 0, st, p);
  }
  return hipGetLastError();
}

}  // namespace

hipError_t launch_forward_prefill_bf16(const FwdDev& p, bool paged, hipStream_t st) {
  if (p.block_m != kBM || p.block_n != kBN) return hipErrorInvalidValue;
  if (p.head_dim == 128) return launch_d<128>(p, paged, st);
  if (p.head_dim == 64) return launch_d<64>(p, paged, st);
  return hipErrorInvalidValue;
}

}  // namespace bmattn
