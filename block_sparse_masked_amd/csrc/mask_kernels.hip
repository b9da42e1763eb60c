// Tile classification, kv-tile lists, row schedule, dense-mask export,
// device-side validation and the paged gather export.
//
// Tile classes follow the tiled causal diagram of Triton from First
// Principles, Ch. 21, section 21.2 (all-valid blocks, the diagonal block
// checked per pair, blocks skipped without a load) with pairs outside the
// sequence counted as not visible.  The lists let a forward workgroup skip
// every empty tile on a scalar read, as in Ch. 9, section 9.2.
#include <hip/hip_runtime.h>

#include <algorithm>

#include "device_common.h"
#include "launch.h"

namespace bmattn {

namespace {

constexpr int kThreads = 256;
constexpr int kMaxBlock = 1024;

// Key ids as the classifier keeps them, one int per key: the segment
// (shared-prefix), or the turn of a think key and INT32_MAX for any other
// key (strip-thinking: a key is hidden from query turn tq iff its value is
// below tq).
__device__ __forceinline__ int32_t staged_kid(const MaskDev& m, const SeqBounds& b, int j) {
  if (m.kind == BMATTN_MASK_SHARED_PREFIX) return m.seg_k[b.k0 + j];
  return m.role_k[b.k0 + j] == m.think_role ? m.turn_k[b.k0 + j] : INT32_MAX;
}

// Visible query rows of a tile for a key with staged id kv when every pair
// of the tile passes the causal condition and lies inside the sequence.  qid
// holds the row ids (segment or turn) of the tile's query rows, [qmin, qmax]
// their range.
__device__ __forceinline__ int key_visible_rows(const MaskDev& m, int32_t kv, const int32_t* qid,
                                                int nrows, int32_t qmin, int32_t qmax) {
  if (m.kind == BMATTN_MASK_SHARED_PREFIX) {
    if (kv == 0) return nrows;
    if (kv < qmin || kv > qmax) return 0;
    if (qmin == qmax) return nrows;
    int c = 0;
    for (int i = 0; i < nrows; ++i) c += (qid[i] == kv);
    return c;
  }
  // STRIP_THINKING: hidden when the key is think and from an earlier turn.
  if (kv >= qmax) return nrows;
  if (kv < qmin) return 0;
  int c = 0;
  for (int i = 0; i < nrows; ++i) c += (kv >= qid[i]);
  return c;
}

// kid[j - klo] is the staged id of key j of this tile (id-based kinds).
__device__ uint8_t classify_tile(const MaskDev& m, const SeqBounds& b, int qlo, int klo, int BM,
                                 int BN, const int32_t* qid, int32_t qmin, int32_t qmax,
                                 const int32_t* kid) {
  if (qlo >= b.lq || klo >= b.lk) return BMATTN_TILE_EMPTY;
  const int qhi = min(qlo + BM, b.lq);
  const int khi = min(klo + BN, b.lk);
  const bool inside = (qlo + BM <= b.lq) && (klo + BN <= b.lk);
  if (m.kind == BMATTN_MASK_FULL) return inside ? BMATTN_TILE_FULL : BMATTN_TILE_PARTIAL;
  const int64_t off = (int64_t)b.lk - b.lq;
  // Every key beyond the last query's position: nothing visible.
  if ((int64_t)klo > (int64_t)(qhi - 1) + off) return BMATTN_TILE_EMPTY;
  const bool causal_full = inside && ((int64_t)klo + BN - 1 <= (int64_t)qlo + off);
  if (m.kind == BMATTN_MASK_CAUSAL)
    return causal_full ? BMATTN_TILE_FULL : BMATTN_TILE_PARTIAL;
  if (causal_full) {
    // Only the id condition can hide pairs: count visible rows key by key.
    int64_t nvis = 0;
    bool hidden = false;
    if (qmin == qmax) {
      // One id for all the tile's query rows: a key is visible to all of
      // them or to none, so the class follows from "every key" / "any key".
      bool all = true, any = false;
      for (int j = klo; j < khi; ++j) {
        const int32_t kv = kid[j - klo];
        const bool ok = m.kind == BMATTN_MASK_SHARED_PREFIX ? (kv == 0 || kv == qmin) : kv >= qmin;
        all &= ok;
        any |= ok;
      }
      return all ? BMATTN_TILE_FULL : (any ? BMATTN_TILE_PARTIAL : BMATTN_TILE_EMPTY);
    }
    for (int j = klo; j < khi; ++j) {
      int c = key_visible_rows(m, kid[j - klo], qid, BM, qmin, qmax);
      nvis += c;
      hidden |= (c < BM);
      if (nvis > 0 && hidden) return BMATTN_TILE_PARTIAL;
    }
    if (nvis == 0) return BMATTN_TILE_EMPTY;
    return hidden ? BMATTN_TILE_PARTIAL : BMATTN_TILE_FULL;
  }
  // Diagonal or edge tile: enumerate the pairs (out-of-range pairs hidden).
  bool any_vis = false, any_hid = !inside;
  const int64_t off2 = (int64_t)b.lk - b.lq;
  auto vis = [&](int i, int j) -> bool {
    // the element predicate on staged ids (pairs here are in range)
    const int32_t kv = kid[j - klo], qv = qid[i - qlo];
    const bool causal = (int64_t)j <= off2 + i;
    return causal && (m.kind == BMATTN_MASK_SHARED_PREFIX ? (kv == 0 || kv == qv) : !(kv < qv));
  };
  // The four corners first: a visible and a hidden one settle the class.
  {
    const bool c0 = vis(qhi - 1, klo), c1 = vis(qlo, khi - 1), c2 = vis(qlo, klo), c3 = vis(qhi - 1, khi - 1);
    any_vis = c0 | c1 | c2 | c3;
    any_hid |= !(c0 & c1 & c2 & c3);
    if (any_vis && any_hid) return BMATTN_TILE_PARTIAL;
  }
  for (int j = klo; j < khi; ++j) {
    const int32_t kv = kid[j - klo];
    for (int i = qlo; i < qhi; ++i) {
      // the element predicate on staged ids (pairs here are in range)
      const int32_t qv = qid[i - qlo];
      const bool causal = (int64_t)j <= off2 + i;
      const bool v = causal && (m.kind == BMATTN_MASK_SHARED_PREFIX ? (kv == 0 || kv == qv) : !(kv < qv));
      any_vis |= v;
      any_hid |= !v;
      if (any_vis && any_hid) return BMATTN_TILE_PARTIAL;
    }
  }
  if (!any_vis) return BMATTN_TILE_EMPTY;
  return any_hid ? BMATTN_TILE_PARTIAL : BMATTN_TILE_FULL;
}

// COMPOSED masks of one term group (an AND).  The queries of a row tile
// fall into a few groups of equal ids (segment, turn, document); the
// kernel lists them (up to
// kMaxGroups, with the largest row of each) before classifying.  With the
// causal term, pair (i, j) is visible iff j <= i + off and the key's ids
// pass the group's id terms, so a tile is
//   EMPTY  iff for every key j and group g: the ids fail, or j > hi_g + off;
//   FULL   iff it lies inside the sequence, the causal term cuts none of its
//          pairs (klo + BN - 1 <= qlo + off) and every key passes every group;
// exactly the classes of the element predicate.  The staging pass stores,
// per key, the bit mask of the groups whose ids it passes (one byte), so a
// tile costs one byte per key.  Rows with more groups enumerate their pairs
// (key ids from LDS: four arrays of kw words, segment, role, turn, document).
constexpr int kMaxGroups = 8;

struct RowGroups {
  int n;                        // number of groups, -1 when over kMaxGroups
  QIds ids[kMaxGroups];
  int lo[kMaxGroups];           // smallest row (inside the sequence) of each group
  int hi[kMaxGroups];           // largest row (inside the sequence) of each group
};

// A COMPOSED tile of an OR of several term groups.  The staging pass stores
// two bytes per key: the query groups that some term group without the
// causal term lets see the key (okN), and those that some causal term group
// lets see it (okC).  Pair (i, j), row i in query group g, is then visible
// iff okN_g(j) or (okC_g(j) and j <= i + off), so for the rows of group g
// the key is visible to all of them iff okN_g or (okC_g and j <= lo_g + off)
// and to some of them iff okN_g or (okC_g and j <= hi_g + off): exact, two
// bytes per key.
__device__ uint8_t classify_tile_or(const MaskDev& m, const SeqBounds& b, int qlo, int klo, int BM,
                                    int BN, int n, const int* lo, const int* hi, const uint8_t* okb,
                                    int k0) {
  if (qlo >= b.lq || klo >= b.lk) return BMATTN_TILE_EMPTY;
  const int qhi = min(qlo + BM, b.lq);
  const int khi = min(klo + BN, b.lk);
  const bool inside = (qlo + BM <= b.lq) && (klo + BN <= b.lk);
  const int64_t off = (int64_t)b.lk - b.lq;
  if (m.causal_all && (int64_t)klo > (int64_t)(qhi - 1) + off) return BMATTN_TILE_EMPTY;
  const uint32_t every = (1u << n) - 1u;
  bool all = inside, any = false;
  for (int j = klo; j < khi; ++j) {
    // With every term group causal, a key past the last row's position is
    // hidden from the whole tile (and was not staged).
    if (m.causal_all && (int64_t)j > (int64_t)(qhi - 1) + off) {
      all = false;
      continue;
    }
    const uint32_t okn = okb[2 * (j - k0)], okc = okb[2 * (j - k0) + 1];
    uint32_t to_all = okn, to_some = okn;
    for (int g = 0; g < n; ++g) {
      if ((okc >> g) & 1u) {
        to_all |= (uint32_t)((int64_t)j <= (int64_t)lo[g] + off) << g;
        to_some |= (uint32_t)((int64_t)j <= (int64_t)hi[g] + off) << g;
      }
    }
    all &= to_all == every;
    any |= to_some != 0;
    if (any && !all) return BMATTN_TILE_PARTIAL;
  }
  if (!any) return BMATTN_TILE_EMPTY;
  return all ? BMATTN_TILE_FULL : BMATTN_TILE_PARTIAL;
}

__device__ uint8_t classify_tile_groups(const MaskDev& m, const SeqBounds& b, int qlo, int klo,
                                        int BM, int BN, int n, const int* hi,
                                        const uint8_t* okb, int k0) {
  if (qlo >= b.lq || klo >= b.lk) return BMATTN_TILE_EMPTY;
  const int qhi = min(qlo + BM, b.lq);
  const int khi = min(klo + BN, b.lk);
  const bool inside = (qlo + BM <= b.lq) && (klo + BN <= b.lk);
  const bool causal = m.causal_all != 0;
  const int64_t off = (int64_t)b.lk - b.lq;
  if (causal && (int64_t)klo > (int64_t)(qhi - 1) + off) return BMATTN_TILE_EMPTY;
  const bool causal_full = !causal || ((int64_t)klo + BN - 1 <= (int64_t)qlo + off);
  const uint32_t every = (1u << n) - 1u;
  bool all = inside && causal_full, any = false;
  for (int j = klo; j < khi; ++j) {
    const uint32_t ok = okb[j - k0];
    uint32_t reach = every;  // groups with a row that the causal term lets see key j
    if (causal) {
      reach = 0;
      for (int g = 0; g < n; ++g) reach |= (uint32_t)((int64_t)j <= (int64_t)hi[g] + off) << g;
    }
    all &= ok == every;
    any |= (ok & reach) != 0;
    if (any && !all) return BMATTN_TILE_PARTIAL;
  }
  if (!any) return BMATTN_TILE_EMPTY;
  return all ? BMATTN_TILE_FULL : BMATTN_TILE_PARTIAL;
}

// A COMPOSED tile from the AND / OR of its keys' group bytes, when every
// group's causal reach covers the whole tile and all its keys were staged
// (then a key's reachable groups are all groups); otherwise key by key.
__device__ uint8_t classify_tile_summary(const MaskDev& m, const SeqBounds& b, int qlo, int klo,
                                         int BM, int BN, int n, int hmin, uint32_t tand,
                                         uint32_t tor, int tcnt, const int* hi, const uint8_t* okb,
                                         int k0) {
  if (qlo >= b.lq || klo >= b.lk) return BMATTN_TILE_EMPTY;
  const int qhi = min(qlo + BM, b.lq);
  const int khi = min(klo + BN, b.lk);
  const bool causal = m.causal_all != 0;
  const int64_t off = (int64_t)b.lk - b.lq;
  if (causal && (int64_t)klo > (int64_t)(qhi - 1) + off) return BMATTN_TILE_EMPTY;
  if ((!causal || (int64_t)hmin + off >= (int64_t)khi - 1) && tcnt == khi - klo) {
    const bool inside = (qlo + BM <= b.lq) && (klo + BN <= b.lk);
    const bool causal_full = !causal || ((int64_t)klo + BN - 1 <= (int64_t)qlo + off);
    const uint32_t every = (1u << n) - 1u;
    if ((tor & every) == 0) return BMATTN_TILE_EMPTY;
    return (inside && causal_full && (tand & every) == every) ? BMATTN_TILE_FULL : BMATTN_TILE_PARTIAL;
  }
  return classify_tile_groups(m, b, qlo, klo, BM, BN, n, hi, okb, k0);
}

__device__ uint8_t classify_tile_enum(const MaskDev& m, const SeqBounds& b, int qlo, int klo,
                                      int BM, int BN, const int32_t* qs, const int32_t* qt,
                                      const int32_t* qd, const int32_t* kid, int kw, int k0) {
  if (qlo >= b.lq || klo >= b.lk) return BMATTN_TILE_EMPTY;
  const int qhi = min(qlo + BM, b.lq);
  const int khi = min(klo + BN, b.lk);
  const bool inside = (qlo + BM <= b.lq) && (klo + BN <= b.lk);
  const int64_t off = (int64_t)b.lk - b.lq;
  if (m.causal_all && (int64_t)klo > (int64_t)(qhi - 1) + off) return BMATTN_TILE_EMPTY;
  // A group that is the causal term alone shows every pair on or below the
  // diagonal: a tile inside the sequence and wholly below it is FULL.
  bool causal_alone = false;
  for (int32_t gs = m.groups; gs != 0; gs >>= 4) causal_alone |= (gs & 15) == BMATTN_TERM_CAUSAL;
  if (causal_alone && inside && (int64_t)klo + BN - 1 <= (int64_t)qlo + off) return BMATTN_TILE_FULL;
  bool any_vis = false, any_hid = !inside;
  for (int j = klo; j < khi; ++j) {
    const int u = j - k0;
    const int32_t a0 = kid[u], a1 = kid[kw + u], a2 = kid[2 * kw + u], a3 = kid[3 * kw + u];
    for (int i = qlo; i < qhi; ++i) {
      const QIds q{qs[i - qlo], qt[i - qlo], qd[i - qlo]};
      const bool v = composed_ok(m.groups, m.think_role, (int64_t)j <= off + i, q, a0, a1, a2, a3);
      any_vis |= v;
      any_hid |= !v;
      if (any_vis && any_hid) return BMATTN_TILE_PARTIAL;
    }
  }
  if (!any_vis) return BMATTN_TILE_EMPTY;
  return any_hid ? BMATTN_TILE_PARTIAL : BMATTN_TILE_FULL;
}

// One workgroup per query-tile row: classifies the row's kv tiles in chunks
// of 256 and appends FULL / PARTIAL indices in ascending order.
// Staged key ids per chunk: tiles of BN keys, each run padded to BN + 1
// words so that lanes scanning different tiles hit different LDS banks.
constexpr int kKidKeys = 16384;
constexpr int kStageBatch = 8;

__global__ __launch_bounds__(kThreads) void classify_kernel(MaskDev m, TilesDev t) {
  __shared__ int32_t qid[kMaxBlock];
  __shared__ int32_t qturn[kMaxBlock], qdoc[kMaxBlock];  // COMPOSED only
  __shared__ int32_t kid[kKidKeys + kThreads];
  __shared__ int32_t wave_tot[2][kThreads / 64];
  __shared__ int32_t red[2][kThreads / 64];
  const int row = blockIdx.x;
  const int s = row / t.n_qt, a = row % t.n_qt;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int BM = t.block_m, BN = t.block_n;
  const SeqBounds b = seq_bounds(m, s, t.max_lq, t.max_lk);
  const int qlo = a * BM;

  const bool composed = m.kind == BMATTN_MASK_COMPOSED;
  __shared__ RowGroups rg;
  // Row ids (segment for shared-prefix, turn for strip-thinking) and range.
  int32_t lmin = INT32_MAX, lmax = INT32_MIN;
  for (int i = tid; i < BM; i += kThreads) {
    QIds x = load_qids(m, b, qlo + i);
    int32_t v = (m.kind == BMATTN_MASK_SHARED_PREFIX || composed) ? x.seg : x.turn;
    qid[i] = v;
    if (composed) {
      qturn[i] = x.turn;
      qdoc[i] = x.doc;
    }
    if (qlo + i < b.lq) {
      lmin = min(lmin, v);
      lmax = max(lmax, v);
    }
  }
  for (int o = 32; o > 0; o >>= 1) {
    lmin = min(lmin, __shfl_xor(lmin, o));
    lmax = max(lmax, __shfl_xor(lmax, o));
  }
  if (lane == 0) {
    red[0][wave] = lmin;
    red[1][wave] = lmax;
  }
  __syncthreads();
  int32_t qmin = red[0][0], qmax = red[1][0];
  for (int w = 1; w < kThreads / 64; ++w) {
    qmin = min(qmin, red[0][w]);
    qmax = max(qmax, red[1][w]);
  }

  // COMPOSED: the groups of equal query ids.  Row i's leader is the first
  // row with its ids; leaders, in row order, number the groups (more than
  // kMaxGroups: none, enumerate), and each group's largest row is an LDS
  // maximum over its rows.
  if (composed) {
    __shared__ int32_t lead[kMaxBlock];
    __shared__ int32_t nlead;
    const int nrows = max(0, min(BM, b.lq - qlo));
    if (tid == 0) nlead = 0;
    for (int i = tid; i < nrows; i += kThreads) {
      int r = 0;
      while (!(qid[r] == qid[i] && qturn[r] == qturn[i] && qdoc[r] == qdoc[i])) ++r;
      lead[i] = r;
    }
    __syncthreads();
    // leaders in row order: chunked ballots over the rows
    for (int i0 = 0; i0 < nrows; i0 += kThreads) {
      const int i = i0 + tid;
      const bool isl = i < nrows && lead[i] == i;
      const uint64_t bm = __ballot(isl);
      const uint64_t lt = (lane == 0) ? 0ull : (~0ull >> (64 - lane));
      if (lane == 0) wave_tot[0][wave] = __popcll(bm);
      __syncthreads();
      int base = nlead;
      for (int w = 0; w < wave; ++w) base += wave_tot[0][w];
      if (isl) {
        const int g = base + __popcll(bm & lt);
        lead[i] = -1 - g;  // a leader holds its group number, encoded below 0
        if (g < kMaxGroups) {
          rg.ids[g] = QIds{qid[i], qturn[i], qdoc[i]};
          rg.lo[g] = qlo + i;  // rows of the sequence, as the tile bounds
          rg.hi[g] = qlo + i;
        }
      }
      __syncthreads();
      if (tid == 0) for (int w = 0; w < kThreads / 64; ++w) nlead += wave_tot[0][w];
      __syncthreads();
    }
    for (int i = tid; i < nrows; i += kThreads) {
      const int l = lead[i];
      const int g = l < 0 ? -1 - l : -1 - lead[l];
      if (g < kMaxGroups) atomicMax(&rg.hi[g], qlo + i);
    }
    if (tid == 0) rg.n = nlead <= kMaxGroups ? nlead : -1;
    __syncthreads();
  }

  const int64_t rowoff = (int64_t)row * t.n_kt;
  int full_base = 0, part_base = 0;
  // Chunks of tpc kv tiles, one per thread; for the id-based kinds the ids of
  // the chunk's keys are first staged in LDS with coalesced loads.
  const bool ids = m.kind == BMATTN_MASK_SHARED_PREFIX || m.kind == BMATTN_MASK_STRIP_THINKING;
  // COMPOSED stages one group byte per key (kKidKeys * 4 keys per chunk) or,
  // for rows with too many groups, four arrays of kw keys.
  const int kw = kKidKeys / 4;
  const bool groups = composed && rg.n >= 0;
  // An OR of several term groups stages two bytes per key (classify_tile_or).
  const bool multi = composed && (m.groups >> 4) != 0;
  const int ckeys = !composed ? kKidKeys : (groups ? (multi ? 2 : 4) * kKidKeys : kw);
  const int tpc = std::max(1, std::min(kThreads, ckeys / BN));
  uint8_t* okb = reinterpret_cast<uint8_t*>(kid);
  const int ng = composed ? rg.n : 0;
  // COMPOSED groups: per tile of the chunk, the AND and OR of its keys'
  // group bytes and the number of keys staged; the smallest group end row.
  __shared__ uint8_t tand[kThreads], tor[kThreads];
  __shared__ int16_t tcnt[kThreads];
  // (only for 64-key tiles: one wave's lanes then cover one tile)
  const bool summ = groups && BN == 64 && !multi;
  int hmin = INT32_MAX;
  for (int gi = 0; gi < ng; ++gi) hmin = min(hmin, rg.hi[gi]);
  // With the causal term no key past the row's last query position is
  // visible: those tiles classify as EMPTY without reading ids, so their
  // ids are not staged.
  int64_t kvis = b.lk;
  if (m.causal_all && qlo < b.lq)
    kvis = std::min<int64_t>(b.lk, (int64_t)std::min(qlo + BM, b.lq) + ((int64_t)b.lk - b.lq));
  for (int c0 = 0; c0 < t.n_kt; c0 += tpc) {
    const int bidx = c0 + tid;
    const int kid0 = c0 * BN;
    // Staging loops take kStageBatch keys per thread per pass, all loads of
    // a pass issued before their first use.
    if (ids) {
      const int kend = (int)std::max<int64_t>(0, std::min<int64_t>((int64_t)(c0 + tpc) * BN, kvis));
      for (int j0 = kid0 + tid; j0 < kend; j0 += kStageBatch * kThreads) {
        int32_t v[kStageBatch];
#pragma unroll
        for (int e = 0; e < kStageBatch; ++e) {
          const int j = j0 + e * kThreads;
          v[e] = j < kend ? staged_kid(m, b, j) : 0;
        }
#pragma unroll
        for (int e = 0; e < kStageBatch; ++e) {
          const int u = j0 + e * kThreads - kid0;
          if (j0 + e * kThreads < kend) kid[u + u / BN] = v[e];
        }
      }
      __syncthreads();
    }
    if (composed) {
      const int kend = (int)std::max<int64_t>(0, std::min<int64_t>((int64_t)(c0 + tpc) * BN, kvis));
      if (summ && tid < tpc) tcnt[tid] = 0;
      if (summ) __syncthreads();
      for (int j0 = kid0 + tid; j0 < kend; j0 += kStageBatch * kThreads) {
       KIds kb[kStageBatch];
#pragma unroll
       for (int e = 0; e < kStageBatch; ++e) {
         const int j = j0 + e * kThreads;
         kb[e] = j < kend ? load_kids(m, b, j) : KIds{0, 0, 0, 0};
       }
#pragma unroll
       for (int e = 0; e < kStageBatch; ++e) {
        const int j = j0 + e * kThreads;
        if (j >= kend) continue;
        const KIds k = kb[e];
        const int u = j - kid0;
        if (groups && multi) {
          uint32_t okn = 0, okc = 0;
          for (int32_t gs = m.groups; gs != 0; gs >>= 4) {
            const int32_t tg = gs & 15;
            if (tg == 0) continue;
            uint32_t ok = 0;
            for (int g = 0; g < ng; ++g)
              ok |= (uint32_t)composed_ids_ok(tg, m.think_role, rg.ids[g], k.a, k.b, k.c, k.d) << g;
            if (tg & BMATTN_TERM_CAUSAL) okc |= ok;
            else okn |= ok;
          }
          okb[2 * u] = (uint8_t)okn;
          okb[2 * u + 1] = (uint8_t)okc;
        } else if (groups) {
          uint32_t ok = 0;
          for (int g = 0; g < ng; ++g)
            ok |= (uint32_t)composed_ids_ok(m.terms, m.think_role, rg.ids[g], k.a, k.b, k.c, k.d) << g;
          okb[u] = (uint8_t)ok;
        } else {
          kid[u] = k.a;
          kid[kw + u] = k.b;
          kid[2 * kw + u] = k.c;
          kid[3 * kw + u] = k.d;
        }
       }
       if (summ) {
         // Lane l of a wave holds key (tile start + l) for each e: the
         // chunk and the passes are tile-aligned, so a wave's 64 lanes
         // cover one tile; keys past kend are left out of the ballots.
#pragma unroll
         for (int e = 0; e < kStageBatch; ++e) {
           const int j = j0 + e * kThreads;
           const bool valid = j < kend;
           const uint32_t ok = valid ? okb[j - kid0] : 0u;
           const uint64_t vm = __ballot(valid);
           if (vm == 0) continue;
           uint32_t an = 0xffu, orr = 0u;
#pragma unroll
           for (int g = 0; g < kMaxGroups; ++g) {
             const uint64_t bm = __ballot(valid && ((ok >> g) & 1u));
             orr |= (uint32_t)(bm != 0) << g;
             an &= ~((uint32_t)(bm != vm) << g);
           }
           if (lane == 0) {
             const int tl = (j - kid0) / BN;
             tand[tl] = (uint8_t)an;
             tor[tl] = (uint8_t)orr;
             tcnt[tl] = (int16_t)__popcll(vm);
           }
         }
       }
      }
      __syncthreads();
    }
    uint8_t cls = BMATTN_TILE_EMPTY;
    if (tid < tpc && bidx < t.n_kt) {
      cls = summ       ? classify_tile_summary(m, b, qlo, bidx * BN, BM, BN, ng, hmin, tand[tid], tor[tid],
                                               tcnt[tid], rg.hi, okb, kid0)
            : (groups && multi) ? classify_tile_or(m, b, qlo, bidx * BN, BM, BN, ng, rg.lo, rg.hi, okb, kid0)
            : groups   ? classify_tile_groups(m, b, qlo, bidx * BN, BM, BN, ng, rg.hi, okb, kid0)
            : composed ? classify_tile_enum(m, b, qlo, bidx * BN, BM, BN, qid, qturn, qdoc, kid, kw, kid0)
                       : classify_tile(m, b, qlo, bidx * BN, BM, BN, qid, qmin, qmax, kid + tid * (BN + 1));
      t.tile_class[rowoff + bidx] = cls;
    }
    const uint64_t fm = __ballot(cls == BMATTN_TILE_FULL);
    const uint64_t pm = __ballot(cls == BMATTN_TILE_PARTIAL);
    const uint64_t lt = (lane == 0) ? 0ull : (~0ull >> (64 - lane));
    const int frank = __popcll(fm & lt), prank = __popcll(pm & lt);
    if (lane == 0) {
      wave_tot[0][wave] = __popcll(fm);
      wave_tot[1][wave] = __popcll(pm);
    }
    __syncthreads();
    int fo = full_base, po = part_base, ft = 0, pt = 0;
    for (int w = 0; w < kThreads / 64; ++w) {
      if (w < wave) {
        fo += wave_tot[0][w];
        po += wave_tot[1][w];
      }
      ft += wave_tot[0][w];
      pt += wave_tot[1][w];
    }
    if (cls == BMATTN_TILE_FULL) t.full_idx[rowoff + fo + frank] = bidx;
    if (cls == BMATTN_TILE_PARTIAL) t.part_idx[rowoff + po + prank] = bidx;
    full_base += ft;
    part_base += pt;
    __syncthreads();
  }
  for (int i = full_base + tid; i < t.n_kt; i += kThreads) t.full_idx[rowoff + i] = -1;
  for (int i = part_base + tid; i < t.n_kt; i += kThreads) t.part_idx[rowoff + i] = -1;
  if (tid == 0) {
    t.full_cnt[row] = full_base;
    t.part_cnt[row] = part_base;
  }
}

// Rows sorted by descending listed-tile count (ties: ascending row), so the
// longest rows are dispatched first.  Rank of row r = number of rows that
// sort before it; the keys are distinct, so the ranks are a permutation.
__global__ __launch_bounds__(kThreads) void schedule_kernel(TilesDev t, int rows) {
  __shared__ int32_t wsh[kThreads];
  const int r = blockIdx.x * kThreads + threadIdx.x;
  const int my = r < rows ? t.full_cnt[r] + t.part_cnt[r] : 0;
  int rank = 0;
  for (int c0 = 0; c0 < rows; c0 += kThreads) {
    const int idx = c0 + threadIdx.x;
    wsh[threadIdx.x] = idx < rows ? t.full_cnt[idx] + t.part_cnt[idx] : -1;
    __syncthreads();
    const int lim = min(kThreads, rows - c0);
    for (int k = 0; k < lim; ++k) {
      const int w = wsh[k];
      rank += (w > my) || (w == my && c0 + k < r);
    }
    __syncthreads();
  }
  if (r < rows) t.row_order[rank] = r;
}

// The same ranking from histograms of the counts, when they fit kMaxBins
// bins: rank of row r with count k = (rows with a count above k) + (rows
// before r with count k).  Every workgroup counts all rows into `all` and the
// rows before its own chunk into `before` (LDS atomics on integers, so the
// counts do not depend on their order), turns `all` into suffix sums, and
// ranks ties inside its chunk from the chunk's counts in LDS: each thread
// reads rows / kThreads + kMaxBins / kThreads + kThreads values instead of
// all rows.
constexpr int kMaxBins = 4096;

__global__ __launch_bounds__(kThreads) void schedule_hist_kernel(TilesDev t, int rows, int nbins) {
  __shared__ int32_t all[kMaxBins], before[kMaxBins];
  __shared__ int32_t key_s[kThreads];
  __shared__ int32_t wave_sum[kThreads / 64];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int64_t c0 = (int64_t)blockIdx.x * kThreads;
  auto key = [&](int64_t r) { return min(max(t.full_cnt[r] + t.part_cnt[r], 0), nbins - 1); };
  for (int b = tid; b < nbins; b += kThreads) {
    all[b] = 0;
    before[b] = 0;
  }
  __syncthreads();
  for (int64_t r = tid; r < rows; r += kThreads) {
    const int k = key(r);
    atomicAdd(&all[k], 1);
    if (r < c0) atomicAdd(&before[k], 1);
  }
  key_s[tid] = c0 + tid < rows ? key(c0 + tid) : -1;
  __syncthreads();
  // all[k] <- rows with a count above k: thread tid owns bins
  // [16 tid, 16 tid + 16); its sum, an inclusive prefix over threads (wave
  // shuffles, then the wave totals), and a descending pass over its bins.
  constexpr int kPer = kMaxBins / kThreads;
  const int b0 = tid * kPer;
  int own = 0;
#pragma unroll
  for (int i = 0; i < kPer; ++i) own += (b0 + i < nbins) ? all[b0 + i] : 0;
  int incl = own;
  for (int o = 1; o < 64; o <<= 1) {
    const int v = __shfl_up(incl, o);
    if (lane >= o) incl += v;
  }
  if (lane == 63) wave_sum[wave] = incl;
  __syncthreads();
  int total = 0, lower = 0;
  for (int w = 0; w < kThreads / 64; ++w) {
    total += wave_sum[w];
    if (w < wave) lower += wave_sum[w];
  }
  int above = total - (lower + incl);  // rows in the bins of higher threads
#pragma unroll
  for (int i = kPer - 1; i >= 0; --i) {
    const int b = b0 + i;
    if (b < nbins) {
      const int c = all[b];
      all[b] = above;
      above += c;
    }
  }
  __syncthreads();
  const int64_t r = c0 + tid;
  if (r < rows) {
    const int k = key_s[tid];
    int rank = all[k] + before[k];
    for (int j = 0; j < tid; ++j) rank += key_s[j] == k;
    t.row_order[rank] = (int32_t)r;
  }
}

// Column lists: one workgroup per (sequence s, kv tile b) reads the classes
// of tiles (a, b) down the column and compacts the FULL and PARTIAL query
// tiles in ascending a with ballots, as the row lists are compacted.
__global__ __launch_bounds__(kThreads) void transpose_kernel(TilesDev t, ColsDev c) {
  __shared__ int32_t wave_tot[2][kThreads / 64];
  const int col = blockIdx.x;
  const int s = col / c.n_kt, b = col % c.n_kt;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int64_t coloff = (int64_t)col * c.n_qt;
  int full_base = 0, part_base = 0;
  for (int a0 = 0; a0 < c.n_qt; a0 += kThreads) {
    const int a = a0 + tid;
    const uint8_t cls =
        a < c.n_qt ? t.tile_class[((int64_t)s * c.n_qt + a) * c.n_kt + b] : (uint8_t)BMATTN_TILE_EMPTY;
    const uint64_t fm = __ballot(cls == BMATTN_TILE_FULL);
    const uint64_t pm = __ballot(cls == BMATTN_TILE_PARTIAL);
    const uint64_t lt = (lane == 0) ? 0ull : (~0ull >> (64 - lane));
    const int frank = __popcll(fm & lt), prank = __popcll(pm & lt);
    if (lane == 0) {
      wave_tot[0][wave] = __popcll(fm);
      wave_tot[1][wave] = __popcll(pm);
    }
    __syncthreads();
    int fo = full_base, po = part_base, ft = 0, pt = 0;
    for (int w = 0; w < kThreads / 64; ++w) {
      if (w < wave) {
        fo += wave_tot[0][w];
        po += wave_tot[1][w];
      }
      ft += wave_tot[0][w];
      pt += wave_tot[1][w];
    }
    if (cls == BMATTN_TILE_FULL) c.full_idx[coloff + fo + frank] = a;
    if (cls == BMATTN_TILE_PARTIAL) c.part_idx[coloff + po + prank] = a;
    full_base += ft;
    part_base += pt;
    __syncthreads();
  }
  for (int i = full_base + tid; i < c.n_qt; i += kThreads) c.full_idx[coloff + i] = -1;
  for (int i = part_base + tid; i < c.n_qt; i += kThreads) c.part_idx[coloff + i] = -1;
  if (tid == 0) {
    c.full_cnt[col] = full_base;
    c.part_cnt[col] = part_base;
  }
}

// Small FULL / CAUSAL problems in one workgroup.  Without ids, a row's
// classes follow from the sequence bounds in closed form: the non-empty kv
// tiles are j < ne, with ne = floor(kmax / BN) + 1 for the last visible key
// kmax = min(lk - 1, off + qhi - 1) (CAUSAL; FULL: lk - 1), and of those the
// FULL ones are the prefix j < nf, nf = floor((lim + 1) / BN) for
// lim = min(lk - 1, off + qlo) (CAUSAL; FULL: lk - 1) when the row's queries
// lie inside the sequence (else nf = 0); the rest are PARTIAL.  This is the
// tile classification of classify_tile() restricted to these two kinds.  So
// the workgroup counts every row, writes the classes and both lists in one
// flat coalesced pass, and ranks the rows with several threads per row.
// Same results as classify_kernel followed by the row ranking, in one
// launch.
constexpr int kSmallThreads = 1024;
constexpr int kSmallMaxRows = 1024;

__global__ __launch_bounds__(kSmallThreads) void classify_schedule_small_kernel(MaskDev m, TilesDev t,
                                                                               int rows) {
  __shared__ SeqBounds bounds[kSmallMaxRows];
  __shared__ int32_t nf_s[kSmallMaxRows], np_s[kSmallMaxRows], rank_s[kSmallMaxRows];
  const int tid = threadIdx.x;
  const int BM = t.block_m, BN = t.block_n, nkt = t.n_kt;
  const bool causal = m.kind == BMATTN_MASK_CAUSAL;
  // Sequence bounds (rows >= n_seqs, so the table fits).
  for (int s = tid; s < t.n_seqs; s += kSmallThreads) bounds[s] = seq_bounds(m, s, t.max_lq, t.max_lk);
  for (int r = tid; r < rows; r += kSmallThreads) rank_s[r] = 0;
  __syncthreads();
  // Per-row counts.
  for (int row = tid; row < rows; row += kSmallThreads) {
    const SeqBounds b = bounds[row / t.n_qt];
    const int64_t qlo = (int64_t)(row % t.n_qt) * BM;
    int nf = 0, ne = 0;
    if (qlo < b.lq && b.lk > 0) {
      const int64_t qhi = std::min<int64_t>(qlo + BM, b.lq);
      const int64_t off = (int64_t)b.lk - b.lq;
      const int64_t kmax = causal ? std::min<int64_t>(b.lk - 1, off + qhi - 1) : b.lk - 1;
      const int64_t lim = causal ? std::min<int64_t>(b.lk - 1, off + qlo) : b.lk - 1;
      ne = kmax >= 0 ? (int)(kmax / BN) + 1 : 0;
      nf = (qlo + BM <= b.lq && lim >= 0) ? (int)((lim + 1) / BN) : 0;
    }
    nf_s[row] = nf;
    np_s[row] = ne - nf;
    t.full_cnt[row] = nf;
    t.part_cnt[row] = ne - nf;
  }
  __syncthreads();
  // Classes and lists: FULL entries 0..nf-1, PARTIAL entries nf..ne-1, the
  // rest of each list -1.
  const int total = rows * nkt;
  for (int idx = tid; idx < total; idx += kSmallThreads) {
    const int row = idx / nkt, j = idx - row * nkt;
    const int nf = nf_s[row], np = np_s[row];
    t.tile_class[idx] = j < nf ? BMATTN_TILE_FULL : (j < nf + np ? BMATTN_TILE_PARTIAL : BMATTN_TILE_EMPTY);
    t.full_idx[idx] = j < nf ? j : -1;
    t.part_idx[idx] = j < np ? nf + j : -1;
  }
  // Rank of row r: rows with more listed tiles, or as many and a lower index;
  // P threads per row each count over a slice of the rows.
  const int P = rows < kSmallThreads ? kSmallThreads / rows : 1;
  const int chunk = (rows + P - 1) / P;
  for (int u = tid; u < rows * P; u += kSmallThreads) {
    const int r = u / P, k0 = (u % P) * chunk, k1 = std::min(rows, k0 + chunk);
    const int my = nf_s[r] + np_s[r];
    int c = 0;
    for (int k = k0; k < k1; ++k) {
      const int w = nf_s[k] + np_s[k];
      c += (w > my) || (w == my && k < r);
    }
    if (c) atomicAdd(&rank_s[r], c);
  }
  __syncthreads();
  for (int r = tid; r < rows; r += kSmallThreads) t.row_order[rank_s[r]] = r;
}

__global__ __launch_bounds__(kThreads) void dense_mask_kernel(MaskDev m, TilesDev t, int seq,
                                                              uint8_t* out, int64_t stride) {
  const int64_t rows_out = (int64_t)t.n_qt * t.block_m;
  const int64_t cols_out = (int64_t)t.n_kt * t.block_n;
  const int64_t idx = (int64_t)blockIdx.x * kThreads + threadIdx.x;
  if (idx >= rows_out * cols_out) return;
  const int i = (int)(idx / cols_out), j = (int)(idx % cols_out);
  const SeqBounds b = seq_bounds(m, seq, t.max_lq, t.max_lk);
  const int a = i / t.block_m, bb = j / t.block_n;
  const uint8_t cls = t.tile_class[((int64_t)seq * t.n_qt + a) * t.n_kt + bb];
  uint8_t v = 0;
  if (cls == BMATTN_TILE_FULL) {
    v = 1;
  } else if (cls == BMATTN_TILE_PARTIAL) {
    v = visible(m, b, i, load_qids(m, b, i), j) ? 1 : 0;
  }
  out[(int64_t)i * stride + j] = v;
}

__global__ __launch_bounds__(kThreads) void validate_kernel(MaskDev m, int32_t max_lq,
                                                            int32_t max_lk, const int32_t* bt,
                                                            int64_t bt_stride, int32_t page_size,
                                                            int64_t num_pages, int32_t* flags) {
  int f = 0;
  if (threadIdx.x == 0) {
    if (m.cu_q[0] != 0 || (int64_t)m.cu_q[m.n_seqs] != m.total_q) f |= 1;
    if (m.cu_k[0] != 0 || (int64_t)m.cu_k[m.n_seqs] != m.total_k) f |= 2;
  }
  for (int s = threadIdx.x; s < m.n_seqs; s += kThreads) {
    const int32_t lq = m.cu_q[s + 1] - m.cu_q[s];
    const int32_t lk = m.cu_k[s + 1] - m.cu_k[s];
    if (lq < 0) f |= 1;
    if (lk < 0) f |= 2;
    if (lq > max_lq || lk > max_lk) f |= 4;
    if (bt != nullptr && lk > 0) {
      const int64_t pages = ((int64_t)lk + page_size - 1) / page_size;
      if (pages > bt_stride) {
        f |= 8;
      } else {
        for (int64_t p = 0; p < pages; ++p) {
          const int32_t e = bt[(int64_t)s * bt_stride + p];
          if (e < 0 || e >= num_pages) f |= 8;
        }
      }
    }
  }
  // OR-reduce over the workgroup.
  __shared__ int32_t red[kThreads / 64];
  for (int o = 32; o > 0; o >>= 1) f |= __shfl_xor(f, o);
  if ((threadIdx.x & 63) == 0) red[threadIdx.x >> 6] = f;
  __syncthreads();
  if (threadIdx.x == 0) {
    int tot = 0;
    for (int w = 0; w < kThreads / 64; ++w) tot |= red[w];
    flags[0] = tot;
  }
}

// Strip-thinking with duplicated answers (xorl issue, "The exactness
// question", option (b)): checks, per sequence, the layout under which the
// relabelled ids are exact.  One workgroup; wave w takes sequences w, w + 16,
// ...; its lanes walk the sequence's keys (adjacent pairs) and queries.
constexpr int kDupCheckThreads = 1024;

__global__ __launch_bounds__(kDupCheckThreads) void duplicated_check_kernel(
    MaskDev m, int32_t max_lq, int32_t max_lk, const int32_t* role_q, int32_t history_role,
    int32_t* flags) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  constexpr int kWaves = kDupCheckThreads / 64;
  int f = 0;
  for (int s = wave; s < m.n_seqs; s += kWaves) {
    const SeqBounds b = seq_bounds(m, s, max_lq, max_lk);
    for (int j = lane; j + 1 < b.lk; j += 64) {
      const int64_t a = b.k0 + j;
      const int32_t t0 = m.turn_k[a], t1 = m.turn_k[a + 1];
      if (t1 < t0) f |= 1;
      else if (t1 == t0 && m.role_k[a] == history_role && m.role_k[a + 1] != history_role) f |= 2;
    }
    for (int i = lane; i < b.lq; i += 64) {
      const int64_t qi = b.q0 + i;
      const int64_t pos = (int64_t)b.lk - b.lq + i;  // the query's key position
      const int32_t r = role_q[qi], t = m.turn_q[qi];
      if (pos >= 0 && (r != m.role_k[b.k0 + pos] || t != m.turn_k[b.k0 + pos])) f |= 4;
      if (r == history_role && t == INT32_MAX) f |= 8;
    }
  }
  __shared__ int32_t red[kWaves];
  for (int o = 32; o > 0; o >>= 1) f |= __shfl_xor(f, o);
  if (lane == 0) red[wave] = f;
  __syncthreads();
  if (threadIdx.x == 0) {
    int tot = 0;
    for (int w = 0; w < kWaves; ++w) tot |= red[w];
    flags[0] = tot;
  }
}

// The relabelling itself, one id per thread: a loss-copy key takes the think
// role, a history-copy query's turn goes up by one (saturating; the check
// reports INT32_MAX).  In place is allowed: each element is read before it
// is written by the same thread.
__global__ __launch_bounds__(kThreads) void duplicated_ids_kernel(
    const int32_t* role_k, const int32_t* role_q, const int32_t* turn_q, int64_t total_k,
    int64_t total_q, int32_t think_role, int32_t loss_role, int32_t history_role,
    int32_t* role_k_out, int32_t* turn_q_out) {
  const int64_t n = total_k > total_q ? total_k : total_q;
  const int64_t stride = (int64_t)gridDim.x * kThreads;
  for (int64_t i = (int64_t)blockIdx.x * kThreads + threadIdx.x; i < n; i += stride) {
    if (i < total_k) {
      const int32_t r = role_k[i];
      role_k_out[i] = r == loss_role ? think_role : r;
    }
    if (i < total_q) {
      const int32_t t = turn_q[i];
      turn_q_out[i] = t + ((role_q[i] == history_role && t < INT32_MAX) ? 1 : 0);
    }
  }
}

__device__ __forceinline__ int32_t page_shift_of_dev(int32_t page_size) {
  return (page_size & (page_size - 1)) == 0 ? __builtin_ctz((uint32_t)page_size) : -1;
}

// Copies 16-byte chunks of every (key, head) row from the pool to the
// contiguous output through paged_row, the forward's own addressing.
__global__ __launch_bounds__(kThreads) void paged_gather_kernel(
    MaskDev m, int32_t max_lk, const char* pool, int64_t st_tok_b, int64_t st_head_b, int32_t H,
    int32_t row_bytes, int32_t page_size, int64_t num_pages, const int32_t* bt, int64_t bt_stride,
    char* out) {
  const int s = blockIdx.y;
  const int chunks = row_bytes / 16;
  const int64_t idx = (int64_t)blockIdx.x * kThreads + threadIdx.x;
  const int64_t per_tok = (int64_t)H * chunks;
  const int j = (int)(idx / per_tok);
  const int rem = (int)(idx % per_tok);
  const int h = rem / chunks, c = rem % chunks;
  const SeqBounds b = seq_bounds(m, s, 1 << 30, max_lk);
  if (j >= b.lk) return;  // the ragged tail is masked: no read, no write
  const int64_t prow = paged_row(bt, bt_stride, s, j, page_size, page_shift_of_dev(page_size),
                                 num_pages);
  const uint4 v = *reinterpret_cast<const uint4*>(pool + prow * st_tok_b + h * st_head_b + c * 16);
  *reinterpret_cast<uint4*>(out + ((b.k0 + j) * H + h) * (int64_t)row_bytes + c * 16) = v;
}

}  // namespace

// The row ranking: from count histograms when the counts (0 .. nbins - 1)
// fit kMaxBins bins, else by comparing every pair of rows.
hipError_t launch_schedule(const TilesDev& t, int rows, int nbins, hipStream_t st) {
  if (rows == 0) return hipSuccess;
  const dim3 grid((uint32_t)(((int64_t)rows + kThreads - 1) / kThreads));
  if (nbins <= kMaxBins) hipLaunchKernelGGL(schedule_hist_kernel, grid, dim3(kThreads), 0, st, t, rows, nbins);
  else hipLaunchKernelGGL(schedule_kernel, grid, dim3(kThreads), 0, st, t, rows);
  return hipGetLastError();
}

hipError_t launch_build_block_mask(const MaskDev& m, const TilesDev& t, hipStream_t st) {
  const int rows = t.n_seqs * t.n_qt;
  const bool small = (m.kind == BMATTN_MASK_FULL || m.kind == BMATTN_MASK_CAUSAL) &&
                     rows <= kSmallMaxRows && (int64_t)rows * t.n_kt <= 64 * 1024;
  if (small) {
    hipLaunchKernelGGL(classify_schedule_small_kernel, dim3(1), dim3(kSmallThreads), 0, st, m, t, rows);
    return hipGetLastError();
  }
  hipLaunchKernelGGL(classify_kernel, dim3(rows), dim3(kThreads), 0, st, m, t);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  return launch_schedule(t, rows, t.n_kt + 1, st);
}

hipError_t launch_transpose_block_mask(const TilesDev& t, const ColsDev& c, hipStream_t st) {
  const int cols = c.n_seqs * c.n_kt;
  if (cols == 0) return hipSuccess;
  hipLaunchKernelGGL(transpose_kernel, dim3(cols), dim3(kThreads), 0, st, t, c);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  // The schedule of the columns: the row ranking over the column counts.
  TilesDev v = t;
  v.full_cnt = c.full_cnt;
  v.part_cnt = c.part_cnt;
  v.row_order = c.col_order;
  return launch_schedule(v, cols, c.n_qt + 1, st);
}

hipError_t launch_debug_dense_mask(const MaskDev& m, const TilesDev& t, int seq, uint8_t* out,
                                   int64_t out_stride, hipStream_t st) {
  const int64_t n = (int64_t)t.n_qt * t.block_m * t.n_kt * t.block_n;
  const int64_t blocks = (n + kThreads - 1) / kThreads;
  hipLaunchKernelGGL(dense_mask_kernel, dim3((uint32_t)blocks), dim3(kThreads), 0, st, m, t, seq,
                     out, out_stride);
  return hipGetLastError();
}

hipError_t launch_validate(const MaskDev& m, int32_t max_lq, int32_t max_lk,
                           const int32_t* block_table, int64_t bt_stride, int32_t page_size,
                           int64_t num_pages, int32_t* flags, hipStream_t st) {
  hipLaunchKernelGGL(validate_kernel, dim3(1), dim3(kThreads), 0, st, m, max_lq, max_lk,
                     block_table, bt_stride, page_size, num_pages, flags);
  return hipGetLastError();
}

hipError_t launch_duplicated_answer_ids(const MaskDev& m, int32_t max_lq, int32_t max_lk,
                                        const int32_t* role_q, int32_t loss_role,
                                        int32_t history_role, int32_t* role_k_out,
                                        int32_t* turn_q_out, int32_t* flags, hipStream_t st) {
  if (flags != nullptr) {
    hipLaunchKernelGGL(duplicated_check_kernel, dim3(1), dim3(kDupCheckThreads), 0, st, m, max_lq,
                       max_lk, role_q, history_role, flags);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  const int64_t n = m.total_k > m.total_q ? m.total_k : m.total_q;
  if (n == 0) return hipSuccess;
  const int64_t blocks = std::min<int64_t>((n + kThreads - 1) / kThreads, 4096);
  hipLaunchKernelGGL(duplicated_ids_kernel, dim3((uint32_t)blocks), dim3(kThreads), 0, st, m.role_k,
                     role_q, m.turn_q, m.total_k, m.total_q, m.think_role, loss_role, history_role,
                     role_k_out, turn_q_out);
  return hipGetLastError();
}

hipError_t launch_paged_gather(const MaskDev& m, int32_t max_lk, const void* pool, int64_t st_tok,
                               int64_t st_head, int32_t elem_bytes, int32_t H, int32_t D,
                               int32_t page_size, int64_t num_pages, const int32_t* block_table,
                               int64_t bt_stride, void* out, hipStream_t st) {
  const int32_t row_bytes = D * elem_bytes;
  const int64_t n = (int64_t)max_lk * H * (row_bytes / 16);
  const int64_t blocks = (n + kThreads - 1) / kThreads;
  hipLaunchKernelGGL(paged_gather_kernel, dim3((uint32_t)blocks, m.n_seqs), dim3(kThreads), 0, st,
                     m, max_lk, static_cast<const char*>(pool), st_tok * elem_bytes,
                     st_head * elem_bytes, H, row_bytes, page_size, num_pages, block_table,
                     bt_stride, static_cast<char*>(out));
  return hipGetLastError();
}

}  // namespace bmattn
