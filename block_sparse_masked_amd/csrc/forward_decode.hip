// Masked attention forward for query tiles of one row (decode), gfx950.
//
// One query per tile row attends a context read tile by tile (BLOCK_N = 64
// keys), optionally through a paged block table -- nanoserve Day 21's
// planned paged-attention kernel: the gather of the block-table pages folded
// into the score and softmax loop so K/V stream block by block and the
// history is never assembled.  The softmax is Triton from First Principles,
// Ch. 21, section 21.1's online recurrence.
//
// At one query per row the work is a stream of K/V bytes with two flops per
// byte, so it runs on the vector ALUs, not on MFMA.  Mapping:
//  * a workgroup = 4 waves = 4 heads of one (row, split); a split is a run of
//    consecutive entries of the row's kv-tile list, so the grid has enough
//    workgroups for the whole chip even when contexts differ 64x;
//  * inside a wave, 16 lanes cover one 256-byte key row (16 bytes each) and
//    the wave covers 4 keys per load; the q.k partial dots are summed over
//    the 16 lanes with DPP row operations;
//  * each split writes its unnormalised accumulator, running max and sum to
//    the workspace; a second kernel merges the splits of a row in ascending
//    order (deterministic), O = sum_i 2^(m_i - M) acc_i / sum_i 2^(m_i - M) l_i.
#include <hip/hip_runtime.h>

#include <mutex>

#include "device_common.h"
#include "launch.h"

namespace bmattn {
namespace {

// The split workspace of bmattn_forward_noalloc: a file-scope device array
// that every call on a GPU shares (each GPU holds its own copy until the
// process ends).  Host code never passes `scratch` itself to a kernel (on
// the host it names a stand-in, not device memory): decode_scratch() looks
// up the array's device address once per device and hands that out.
constexpr size_t kScratchBytes = BMATTN_NOALLOC_MAX_WORKSPACE;
static __device__ __align__(256) char scratch[kScratchBytes];
constexpr int kMaxDevices = 64;

constexpr int kBN = 64;
constexpr int kThreads = 256;
constexpr int kHeadsPerWG = kThreads / 64;
constexpr float kLn2 = 0.69314718055994530942f;

__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }

// Sum over aligned groups of G lanes (G in {4, 8, 16, 32}); every lane of a
// group receives the group's sum.
template <int G>
__device__ __forceinline__ float group_sum(float x) {
  // quad_perm [1,0,3,2] and [2,3,0,1]
  x += __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, x), 0xB1, 0xF, 0xF, false));
  x += __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, x), 0x4E, 0xF, 0xF, false));
  if constexpr (G >= 8) {  // row_half_mirror: the other quad of the 8-lane half row
    x += __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, x), 0x141, 0xF, 0xF, false));
  }
  if constexpr (G >= 16) {  // row_mirror: the other half of the 16-lane row
    x += __builtin_bit_cast(float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, x), 0x140, 0xF, 0xF, false));
  }
  if constexpr (G >= 32) x += __shfl_xor(x, 16);
  return x;
}

template <typename T>
__device__ __forceinline__ void to_float(const uint4& u, float (&f)[16 / sizeof(T)]) {
  if constexpr (sizeof(T) == 2) {
    const uint32_t w[4] = {u.x, u.y, u.z, u.w};
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      f[2 * i] = __builtin_bit_cast(float, w[i] << 16);
      f[2 * i + 1] = __builtin_bit_cast(float, w[i] & 0xffff0000u);
    }
  } else {
    f[0] = __builtin_bit_cast(float, u.x);
    f[1] = __builtin_bit_cast(float, u.y);
    f[2] = __builtin_bit_cast(float, u.z);
    f[3] = __builtin_bit_cast(float, u.w);
  }
}

template <typename T, int D, bool PAGED>
__global__ __launch_bounds__(kThreads, 2) void decode_kernel(FwdDev p) {
  constexpr int kElem = sizeof(T);
  constexpr int kCh = D * kElem / 16;  // lanes per key row
  constexpr int kEpc = 16 / kElem;     // elements per lane
  constexpr int kTpi = 64 / kCh;       // keys per wave load
  constexpr int kSteps = kBN / kTpi;   // loads per tile and operand
  constexpr int kChunk = kSteps < 8 ? kSteps : 8;  // loads per operand in one chunk
  constexpr int kChunks = kSteps / kChunk;         // chunks per tile
  static_assert(kChunks * kChunk == kSteps, "chunking");

  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int c = lane % kCh, tg = lane / kCh;
  const int hg_count = (p.num_heads + kHeadsPerWG - 1) / kHeadsPerWG;
  const int hg = blockIdx.x % hg_count;
  const int rest = blockIdx.x / hg_count;
  const int sp = rest % p.n_splits;
  const int row = rest / p.n_splits;
  const int h = hg * kHeadsPerWG + wave;
  if (h >= p.num_heads) return;
  const int s = row / p.n_qt, a = row % p.n_qt;
  const SeqBounds sb = seq_bounds(p.mask, s, p.max_lq, p.max_lk);
  if (a >= sb.lq) return;
  const int nfull = p.full_cnt[row];
  const int ntot = nfull + p.part_cnt[row];
  const int e0 = sp * p.split_tiles;
  if (e0 >= ntot) return;
  const int e1 = min(ntot, e0 + p.split_tiles);
  const int32_t* flist = p.full_idx + (int64_t)row * p.n_kt;
  const int32_t* plist = p.part_idx + (int64_t)row * p.n_kt;
  const QIds qids = load_qids(p.mask, sb, a);

  float qv[kEpc];
  {
    const uint4 u = *reinterpret_cast<const uint4*>(
        static_cast<const char*>(p.q) + ((sb.q0 + a) * p.q_st + (int64_t)h * p.q_sh) * kElem + c * 16);
    to_float<T>(u, qv);
  }
  const char* kbase = static_cast<const char*>(p.k);
  const char* vbase = static_cast<const char*>(p.v);
  const int64_t k_off = (int64_t)h * p.k_sh * kElem + c * 16;
  const int64_t v_off = (int64_t)h * p.v_sh * kElem + c * 16;
  const int64_t k_rs = p.k_st * kElem, v_rs = p.v_st * kElem;

  // The split's kv tiles: lane i holds the tile of list entry e0 + i.
  const int my_e = e0 + lane;
  const int my_kt = my_e < e1 ? (my_e < nfull ? flist[my_e] : plist[my_e - nfull]) : 0;
  // Paged fast path: when a load's keys never straddle a page and the
  // split's pages fit in one register per lane, every block-table entry the
  // split needs is read once, up front; a load then picks its (wave-uniform)
  // page with a lane read instead of a dependent global load.
  const int ps = p.page_size;
  const int ppt = ps < kBN ? kBN / ps : 1;  // pages per tile
  const bool fast_pages = PAGED && ps % kTpi == 0 && (kBN % ps == 0 || ps % kBN == 0) &&
                          ppt * p.split_tiles <= 64;
  int32_t my_page = 0;
  if (fast_pages) {
    const int ti = lane / ppt, pi = lane % ppt;
    const int kt_i = __shfl(my_kt, ti);
    const int j = min(kt_i * kBN + pi * ps, sb.lk - 1);
    if (e0 + ti < e1) my_page = page_entry(p.block_table, p.bt_stride, s, j, ps, p.page_shift);
  }

  float acc[kEpc];
#pragma unroll
  for (int e = 0; e < kEpc; ++e) acc[e] = 0.f;
  float m_run = -INFINITY, l_run = 0.f;
  const float sl2 = p.scale_log2;

  // Pool row of the key that this lane's group reads at load step st of the
  // split's tile ti (-1: past the sequence, read as zero).
  auto key_row = [&](int ti, int st) -> int64_t {
    const int kt = __shfl(my_kt, ti);
    const int j = kt * kBN + st * kTpi + tg;
    if (j >= sb.lk) return -1;
    if constexpr (!PAGED) {
      return sb.k0 + j;
    } else {
      if (fast_pages) {
        const int slot = ps < kBN ? ti * ppt + (st * kTpi) / ps : ti;
        const int32_t pe = __builtin_amdgcn_readlane(my_page, slot);
        return row_in_page(pe, j, ps, p.page_shift, p.num_pages);
      }
      return paged_row(p.block_table, p.bt_stride, s, j, ps, p.page_shift, p.num_pages);
    }
  };

  // The split's loads stream in chunks of kChunk loads per operand: the next
  // chunk's K and V loads are issued before the current chunk is used, so
  // one chunk is always in flight.
  const int nt = e1 - e0;
  const int nchunks = nt * kChunks;
  uint4 kr[2][kChunk], vr[2][kChunk];
  auto issue = [&](int ci, uint4 (&kd)[kChunk], uint4 (&vd)[kChunk]) {
    const int ti = ci / kChunks, st0 = (ci % kChunks) * kChunk;
    int64_t rows[kChunk];
#pragma unroll
    for (int u = 0; u < kChunk; ++u) rows[u] = key_row(ti, st0 + u);
#pragma unroll
    for (int u = 0; u < kChunk; ++u)
      kd[u] = rows[u] >= 0 ? *reinterpret_cast<const uint4*>(kbase + rows[u] * k_rs + k_off) : make_uint4(0, 0, 0, 0);
#pragma unroll
    for (int u = 0; u < kChunk; ++u)
      vd[u] = rows[u] >= 0 ? *reinterpret_cast<const uint4*>(vbase + rows[u] * v_rs + v_off) : make_uint4(0, 0, 0, 0);
  };
  auto consume = [&](int ci, const uint4 (&kd)[kChunk], const uint4 (&vd)[kChunk]) {
    const int ti = ci / kChunks, st0 = (ci % kChunks) * kChunk;
    const bool masked = e0 + ti >= nfull;
    float sc[kChunk];
#pragma unroll
    for (int u = 0; u < kChunk; ++u) {
      float kf[kEpc];
      to_float<T>(kd[u], kf);
      float d = 0.f;
#pragma unroll
      for (int i = 0; i < kEpc; ++i) d = fmaf(qv[i], kf[i], d);
      sc[u] = group_sum<kCh>(d) * sl2;
    }
    if (masked) {
      const int kt = __shfl(my_kt, ti);
#pragma unroll
      for (int u = 0; u < kChunk; ++u) {
        const int j = kt * kBN + (st0 + u) * kTpi + tg;
        if (!visible(p.mask, sb, a, qids, j)) sc[u] = -INFINITY;
      }
    }
    float mx = sc[0];
#pragma unroll
    for (int u = 1; u < kChunk; ++u) mx = fmaxf(mx, sc[u]);
#pragma unroll
    for (int o = kCh; o < 64; o <<= 1) mx = fmaxf(mx, __shfl_xor(mx, o));
    const float m_new = fmaxf(m_run, mx);
    const float m_use = (m_new == -INFINITY) ? 0.f : m_new;
    const float alpha = fast_exp2(m_run - m_use);
    float rs = 0.f;
#pragma unroll
    for (int i = 0; i < kEpc; ++i) acc[i] *= alpha;
#pragma unroll
    for (int u = 0; u < kChunk; ++u) {
      const float pr = fast_exp2(sc[u] - m_use);
      rs += pr;
      float vf[kEpc];
      to_float<T>(vd[u], vf);
#pragma unroll
      for (int i = 0; i < kEpc; ++i) acc[i] = fmaf(pr, vf[i], acc[i]);
    }
    l_run = l_run * alpha + rs;
    m_run = m_new;
  };
  issue(0, kr[0], vr[0]);
  for (int ci = 0; ci < nchunks; ci += 2) {
    if (ci + 1 < nchunks) issue(ci + 1, kr[1], vr[1]);
    consume(ci, kr[0], vr[0]);
    if (ci + 1 < nchunks) {
      if (ci + 2 < nchunks) issue(ci + 2, kr[0], vr[0]);
      consume(ci + 1, kr[1], vr[1]);
    }
  }
  // Combine the key groups of the wave (they share m_run).
#pragma unroll
  for (int o = kCh; o < 64; o <<= 1) {
    l_run += __shfl_xor(l_run, o);
#pragma unroll
    for (int i = 0; i < kEpc; ++i) acc[i] += __shfl_xor(acc[i], o);
  }
  float* ws = p.ws + (((int64_t)row * p.n_splits + sp) * p.num_heads + h) * (D + 2);
  if (tg == 0) {
#pragma unroll
    for (int i = 0; i < kEpc; ++i) ws[c * kEpc + i] = acc[i];
    if (c == 0) {
      ws[D] = m_run;
      ws[D + 1] = l_run;
    }
  }
}

// Merges the splits of each (row, head): M = max_i m_i, f_i = 2^(m_i - M),
// O = sum_i f_i acc_i / sum_i f_i l_i, the sums taken in ascending split
// order (deterministic).  One wave per (row, head): lane i reads split i's
// (m, l), and the accumulator loads of all splits are issued 8 at a time.
template <typename T, int D>
__global__ __launch_bounds__(kThreads) void decode_merge_kernel(FwdDev p) {
  constexpr int kPer = (D + 63) / 64;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int64_t unit = (int64_t)blockIdx.x * kHeadsPerWG + wave;
  const int64_t n_rows = (int64_t)p.mask.n_seqs * p.n_qt;
  if (unit >= n_rows * p.num_heads) return;
  const int row = (int)(unit / p.num_heads), h = (int)(unit % p.num_heads);
  const int s = row / p.n_qt, a = row % p.n_qt;
  const SeqBounds sb = seq_bounds(p.mask, s, p.max_lq, p.max_lk);
  if (a >= sb.lq) return;
  const int ntot = p.full_cnt[row] + p.part_cnt[row];
  const int nsp = (ntot + p.split_tiles - 1) / p.split_tiles;
  const float* ws = p.ws + ((int64_t)row * p.n_splits * p.num_heads + h) * (D + 2);
  const int64_t sstride = (int64_t)p.num_heads * (D + 2);
  float M = -INFINITY, L = 0.f;
  float o[kPer];
#pragma unroll
  for (int k = 0; k < kPer; ++k) o[k] = 0.f;
  // Splits in batches of 64 (one per lane) for the weights.
  float Mb = -INFINITY;
  for (int b0 = 0; b0 < nsp; b0 += 64) {
    const int i = b0 + lane;
    const float mi = i < nsp ? ws[i * sstride + D] : -INFINITY;
    Mb = fmaxf(Mb, mi);
  }
#pragma unroll
  for (int o2 = 32; o2 > 0; o2 >>= 1) Mb = fmaxf(Mb, __shfl_xor(Mb, o2));
  M = Mb;
  const float Mu = (M == -INFINITY) ? 0.f : M;
  for (int b0 = 0; b0 < nsp; b0 += 64) {
    const int i = b0 + lane;
    const float f = i < nsp ? fast_exp2(ws[i * sstride + D] - Mu) : 0.f;
    const float fl = i < nsp ? f * ws[i * sstride + D + 1] : 0.f;
    // ascending-order sum of f_i l_i: prefix over lanes via readlane
    const int nb = min(64, nsp - b0);
    for (int j0 = 0; j0 < nb; j0 += 8) {
      float x[8][kPer];
#pragma unroll
      for (int u = 0; u < 8; ++u) {
#pragma unroll
        for (int k = 0; k < kPer; ++k) {
          const int d = lane + 64 * k;
          x[u][k] = (j0 + u < nb && d < D) ? ws[(b0 + j0 + u) * sstride + d] : 0.f;
        }
      }
#pragma unroll
      for (int u = 0; u < 8; ++u) {
        if (j0 + u < nb) {
          const float fu = __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, f), j0 + u));
          L += __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, fl), j0 + u));
#pragma unroll
          for (int k = 0; k < kPer; ++k) o[k] += fu * x[u][k];
        }
      }
    }
  }
  const float inv = L > 0.f ? 1.f / L : 0.f;
  char* orow = static_cast<char*>(p.o) + ((sb.q0 + a) * p.o_st + (int64_t)h * p.o_sh) * sizeof(T);
#pragma unroll
  for (int k = 0; k < kPer; ++k) {
    const int d = lane + 64 * k;
    if (d < D) reinterpret_cast<T*>(orow)[d] = static_cast<T>(o[k] * inv);
  }
  if (lane == 0 && p.lse != nullptr) {
    p.lse[(int64_t)h * p.lse_sh + sb.q0 + a] = L > 0.f ? (M + __log2f(L)) * kLn2 : -INFINITY;
  }
}

template <typename T, int D>
hipError_t launch_typed(const FwdDev& p, bool paged, hipStream_t st) {
  const int64_t n_rows = (int64_t)p.mask.n_seqs * p.n_qt;
  const int64_t hg = (p.num_heads + kHeadsPerWG - 1) / kHeadsPerWG;
  const int64_t grid = n_rows * p.n_splits * hg;
  if (grid == 0) return hipSuccess;
  if (grid > 0x7fffffff) return hipErrorInvalidValue;
  if (paged) {
    hipLaunchKernelGGL((decode_kernel<T, D, true>), dim3((uint32_t)grid), dim3(kThreads), 0, st, p);
  } else {
    hipLaunchKernelGGL((decode_kernel<T, D, false>), dim3((uint32_t)grid), dim3(kThreads), 0, st, p);
  }
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  const int64_t units = n_rows * p.num_heads;
  const int64_t mgrid = (units + kHeadsPerWG - 1) / kHeadsPerWG;
  hipLaunchKernelGGL((decode_merge_kernel<T, D>), dim3((uint32_t)mgrid), dim3(kThreads), 0, st, p);
  return hipGetLastError();
}

}  // namespace

size_t decode_scratch_bytes() { return kScratchBytes; }

hipError_t decode_scratch(void** ptr) {
  static std::mutex mu;
  static void* addr[kMaxDevices] = {};
  int dev = -1;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
  std::lock_guard<std::mutex> lock(mu);
  if (addr[dev] == nullptr) {
    void* a = nullptr;
    e = hipGetSymbolAddress(&a, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return e;
    addr[dev] = a;
  }
  *ptr = addr[dev];
  return hipSuccess;
}

hipError_t launch_forward_decode(const FwdDev& p, int dtype, bool paged, hipStream_t st) {
  if (p.block_m != 1 || p.block_n != kBN) return hipErrorInvalidValue;
  if (dtype == BMATTN_BF16 && p.head_dim == 128) return launch_typed<__bf16, 128>(p, paged, st);
  if (dtype == BMATTN_BF16 && p.head_dim == 64) return launch_typed<__bf16, 64>(p, paged, st);
  if (dtype == BMATTN_F32 && p.head_dim == 128) return launch_typed<float, 128>(p, paged, st);
  if (dtype == BMATTN_F32 && p.head_dim == 64) return launch_typed<float, 64>(p, paged, st);
  return hipErrorInvalidValue;
}

}  // namespace bmattn
