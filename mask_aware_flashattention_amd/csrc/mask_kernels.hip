// Integer kernels on the four boundary vectors: per-key-block min/max, tile classification with
// list compaction, and the clip-shift-max localisation.  All three are O(n) (classification is
// O(tiles)) scans bound by HBM bandwidth or launch latency; none touches the matrix cores.
//
// Sources: "FlashMask-3 sends each GPU its mask without sending any mask" (learnaivisually.com),
// tile-classification paragraph (per-key-block extremes of the vectors, three tile classes, a
// queue of the valid blocks) and clip-shift-max paragraph; "FlashMask-3: Efficient and
// Expressive Mask-Aware Distributed Attention", abstract (zero-communication localisation).
#include <limits.h>

#include "fm_common.hpp"
#include "launch.hpp"

namespace fm {

namespace {

constexpr int kWave = 64;
constexpr int kWavesPerBlock = 4;

__device__ inline int lane_id() { return threadIdx.x & (kWave - 1); }

template <typename F>
__device__ inline int32_t wave_reduce(int32_t x, F op) {
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) x = op(x, __shfl_xor(x, off));
  return x;
}

struct MinOp {
  __device__ int32_t operator()(int32_t a, int32_t b) const { return a < b ? a : b; }
};
struct MaxOp {
  __device__ int32_t operator()(int32_t a, int32_t b) const { return a > b ? a : b; }
};

// One wave per key block; lanes stride over the block's keys.  blockIdx.y is the mask set:
// vectors at offset set * vec_stride, output at mm + set * 8 * n_kb.
__global__ __launch_bounds__(256) void block_minmax_kernel(MaskVecs v, int64_t vec_stride,
                                                           int32_t nk, int32_t BN, int32_t n_kb,
                                                           int32_t* __restrict__ mm) {
  const int kb = blockIdx.x * kWavesPerBlock + (threadIdx.x >> 6);
  if (kb >= n_kb) return;
  const int64_t set = blockIdx.y;
  v.lts += set * vec_stride;
  v.lte += set * vec_stride;
  v.uts += set * vec_stride;
  v.ute += set * vec_stride;
  mm += set * 8 * n_kb;
  const int lane = lane_id();
  const int64_t j0 = (int64_t)kb * BN;
  const int64_t j1 = j0 + BN < nk ? j0 + BN : nk;
  int32_t lo[4] = {INT_MAX, INT_MAX, INT_MAX, INT_MAX};
  int32_t hi[4] = {INT_MIN, INT_MIN, INT_MIN, INT_MIN};
  for (int64_t j = j0 + lane; j < j1; j += kWave) {
    const int32_t x[4] = {v.lts[j], v.lte[j], v.uts[j], v.ute[j]};
#pragma unroll
    for (int t = 0; t < 4; ++t) {
      lo[t] = x[t] < lo[t] ? x[t] : lo[t];
      hi[t] = x[t] > hi[t] ? x[t] : hi[t];
    }
  }
#pragma unroll
  for (int t = 0; t < 4; ++t) {
    lo[t] = wave_reduce(lo[t], MinOp());
    hi[t] = wave_reduce(hi[t], MaxOp());
  }
  if (lane == 0) {
#pragma unroll
    for (int t = 0; t < 4; ++t) {
      mm[(2 * t) * n_kb + kb] = lo[t];
      mm[(2 * t + 1) * n_kb + kb] = hi[t];
    }
  }
}

// The same per key block min/max for blocks of BN = 4 * LPB keys (64 or 128, the attention
// kernels' key-block widths) with 16-byte aligned vectors: LPB lanes share a block, each loading
// four consecutive keys of every vector with one 16-byte load (whole 64-byte segments per group
// of four lanes), and the 8 results are reduced over those lanes.  A wave covers 64 / LPB blocks;
// keys past nk are read one by one, never as part of a 16-byte load.
template <int LPB>
__global__ __launch_bounds__(256) void block_minmax_vec_kernel(MaskVecs v, int64_t vec_stride,
                                                               int32_t nk, int32_t n_kb,
                                                               int32_t* __restrict__ mm) {
  constexpr int BN = 4 * LPB, BPW = kWave / LPB;
  const int64_t set = blockIdx.y;
  const int32_t* src[4] = {v.lts + set * vec_stride, v.lte + set * vec_stride,
                           v.uts + set * vec_stride, v.ute + set * vec_stride};
  mm += set * 8 * n_kb;
  const int lane = lane_id();
  const int li = lane % LPB;
  const int64_t kb = ((int64_t)blockIdx.x * kWavesPerBlock + (threadIdx.x >> 6)) * BPW + lane / LPB;
  int32_t lo[4] = {INT_MAX, INT_MAX, INT_MAX, INT_MAX};
  int32_t hi[4] = {INT_MIN, INT_MIN, INT_MIN, INT_MIN};
  if (kb < n_kb) {
    const int64_t j = kb * BN + 4 * li;
    if (j + 3 < nk) {
#pragma unroll
      for (int t = 0; t < 4; ++t) {
        const int4 x = *reinterpret_cast<const int4*>(src[t] + j);
        const int32_t a = x.x < x.y ? x.x : x.y, b = x.z < x.w ? x.z : x.w;
        const int32_t c = x.x > x.y ? x.x : x.y, d = x.z > x.w ? x.z : x.w;
        lo[t] = a < b ? a : b;
        hi[t] = c > d ? c : d;
      }
    } else {
      for (int64_t e = j; e < nk && e < j + 4; ++e)
#pragma unroll
        for (int t = 0; t < 4; ++t) {
          const int32_t x = src[t][e];
          lo[t] = x < lo[t] ? x : lo[t];
          hi[t] = x > hi[t] ? x : hi[t];
        }
    }
  }
#pragma unroll
  for (int off = LPB / 2; off >= 1; off >>= 1)
#pragma unroll
    for (int t = 0; t < 4; ++t) {
      const int32_t a = __shfl_xor(lo[t], off), b = __shfl_xor(hi[t], off);
      lo[t] = a < lo[t] ? a : lo[t];
      hi[t] = b > hi[t] ? b : hi[t];
    }
  if (li == 0 && kb < n_kb) {
#pragma unroll
    for (int t = 0; t < 4; ++t) {
      mm[(2 * t) * n_kb + kb] = lo[t];
      mm[(2 * t + 1) * n_kb + kb] = hi[t];
    }
  }
}

struct BlockBounds {
  int32_t lts_lo, lts_hi, lte_lo, lte_hi, uts_lo, uts_hi, ute_lo, ute_hi;
};

__device__ inline BlockBounds load_bounds(const int32_t* __restrict__ mm, int n_kb, int kb) {
  BlockBounds b;
  b.lts_lo = mm[0 * n_kb + kb];
  b.lts_hi = mm[1 * n_kb + kb];
  b.lte_lo = mm[2 * n_kb + kb];
  b.lte_hi = mm[3 * n_kb + kb];
  b.uts_lo = mm[4 * n_kb + kb];
  b.uts_hi = mm[5 * n_kb + kb];
  b.ute_lo = mm[6 * n_kb + kb];
  b.ute_hi = mm[7 * n_kb + kb];
  return b;
}

// 0 = fully masked, 1 = partly masked, 2 = unmasked, for query rows [r0, r1).
__device__ inline int tile_class(const BlockBounds& b, int32_t r0, int32_t r1) {
  const bool lt_full = b.lts_hi <= r0 && b.lte_lo >= r1;
  const bool ut_full = b.uts_hi <= r0 && b.ute_lo >= r1;
  const bool lt_none = b.lte_hi <= r0 || b.lts_lo >= r1;
  const bool ut_none = b.ute_hi <= r0 || b.uts_lo >= r1;
  return (lt_full || ut_full) ? 0 : ((lt_none && ut_none) ? 2 : 1);
}

__device__ inline int lanes_below(uint64_t mask) {
  return __builtin_amdgcn_mbcnt_hi((uint32_t)(mask >> 32),
                                   __builtin_amdgcn_mbcnt_lo((uint32_t)mask, 0u));
}

// Waves [0, row_waves) each own one query block and scan every key block (forward lists,
// class matrix); the following waves each own one key block and scan every query block
// (backward lists).  Compaction is a wave ballot + prefix count, so lists come out ascending.
// blockIdx.y is the mask set: every input and output is offset by its per-set size.
__global__ __launch_bounds__(256) void classify_kernel(const int32_t* __restrict__ mm, int32_t n_kb,
                                                       int32_t nq, int32_t BM, int32_t n_qb,
                                                       int32_t row_waves, int32_t col_waves,
                                                       uint8_t* __restrict__ cls,
                                                       int32_t* __restrict__ qcnt,
                                                       int32_t* __restrict__ qlist,
                                                       int32_t* __restrict__ kcnt,
                                                       int32_t* __restrict__ klist) {
  const int wid = blockIdx.x * kWavesPerBlock + (threadIdx.x >> 6);
  const int lane = lane_id();
  {
    const int64_t set = blockIdx.y;
    mm += set * 8 * n_kb;
    if (cls) cls += set * n_qb * n_kb;
    if (qcnt) qcnt += set * n_qb;
    if (qlist) qlist += set * n_qb * n_kb;
    if (kcnt) kcnt += set * n_kb;
    if (klist) klist += set * n_kb * n_qb;
  }
  if (wid < row_waves) {
    const int qb = wid;
    const int32_t r0 = qb * BM;
    const int32_t r1 = r0 + BM < nq ? r0 + BM : nq;
    int32_t cnt = 0;
    const int64_t row = (int64_t)qb * n_kb;
    for (int base = 0; base < n_kb; base += kWave) {
      const int kb = base + lane;
      int c = 0;
      if (kb < n_kb) {
        c = tile_class(load_bounds(mm, n_kb, kb), r0, r1);
        if (cls) cls[row + kb] = (uint8_t)c;
      }
      const bool valid = kb < n_kb && c != 0;
      const uint64_t ballot = __ballot(valid);
      if (valid && qlist) qlist[row + cnt + lanes_below(ballot)] = kb * 2 + (c == 1);
      cnt += __popcll(ballot);
    }
    if (lane == 0 && qcnt) qcnt[qb] = cnt;
  } else if (wid < row_waves + col_waves) {
    const int kb = wid - row_waves;
    const BlockBounds b = load_bounds(mm, n_kb, kb);
    int32_t cnt = 0;
    const int64_t row = (int64_t)kb * n_qb;
    for (int base = 0; base < n_qb; base += kWave) {
      const int qb = base + lane;
      int c = 0;
      if (qb < n_qb) {
        const int32_t r0 = qb * BM;
        const int32_t r1 = r0 + BM < nq ? r0 + BM : nq;
        c = tile_class(b, r0, r1);
      }
      const bool valid = qb < n_qb && c != 0;
      const uint64_t ballot = __ballot(valid);
      if (valid) klist[row + cnt + lanes_below(ballot)] = qb * 2 + (c == 1);
      cnt += __popcll(ballot);
    }
    if (lane == 0) kcnt[kb] = cnt;
  }
}

// local(x) = max(0, max_k(min(x, o_k + L_k) + P_k - o_k)).  Negative marks are raised to 0
// first: that leaves the result unchanged (no owned row lies below 0) and keeps every sum inside
// int32.
__device__ inline int32_t clip_shift_max(int32_t x, const ChunkTable& t) {
  x = x > 0 ? x : 0;
  int32_t best = 0;
  for (int k = 0; k < t.n_chunks; ++k) {
    const int32_t c = (x < t.end[k] ? x : t.end[k]) + t.shift[k];
    best = c > best ? c : best;
  }
  return best;
}

template <int VEC>
__global__ __launch_bounds__(256) void localize_kernel(MaskVecs in, int32_t n, ChunkTable table,
                                                       int32_t* __restrict__ o0,
                                                       int32_t* __restrict__ o1,
                                                       int32_t* __restrict__ o2,
                                                       int32_t* __restrict__ o3) {
  const int64_t stride = (int64_t)gridDim.x * blockDim.x;
  const int32_t* src[4] = {in.lts, in.lte, in.uts, in.ute};
  int32_t* dst[4] = {o0, o1, o2, o3};
  if constexpr (VEC == 4) {
    const int64_t nvec = n / 4;
    for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < nvec; i += stride) {
#pragma unroll
      for (int t = 0; t < 4; ++t) {
        int4 x = reinterpret_cast<const int4*>(src[t])[i];
        x.x = clip_shift_max(x.x, table);
        x.y = clip_shift_max(x.y, table);
        x.z = clip_shift_max(x.z, table);
        x.w = clip_shift_max(x.w, table);
        reinterpret_cast<int4*>(dst[t])[i] = x;
      }
    }
    // tail (n % 4 elements) handled by the first threads
    const int64_t i = nvec * 4 + (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
    if (i < n) {
#pragma unroll
      for (int t = 0; t < 4; ++t) dst[t][i] = clip_shift_max(src[t][i], table);
    }
  } else {
    for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < n; i += stride) {
#pragma unroll
      for (int t = 0; t < 4; ++t) dst[t][i] = clip_shift_max(src[t][i], table);
    }
  }
}

inline int grid_for(int64_t work, int threads, int cap) {
  int64_t g = (work + threads - 1) / threads;
  if (g < 1) g = 1;
  return (int)(g < cap ? g : cap);
}

// Work order of the attention kernels: blocks go into kOrderBuckets buckets by list length
// (bucket b holds counts c with floor(c * kOrderBuckets / (max + 1)) = b), the bucket of the
// longest lists first, so that long workgroups start early and short ones fill the tail of each
// compute unit's queue.  Inside a bucket the blocks keep descending index order, so workgroups
// that run at the same time stay close in the sequence and share K / V tiles in the L2 cache.
// One workgroup, deterministic: thread t owns a contiguous run of the descending index sequence
// and a scan over threads gives each of its blocks its slot.
constexpr int kOrderBuckets = 4;
constexpr int kOrderThreads = 1024;
// One workgroup per mask set (blockIdx.x): counts and order at offset set * n.
__global__ __launch_bounds__(kOrderThreads) void block_order_kernel(const int32_t* __restrict__ cnt,
                                                                    int32_t n,
                                                                    int32_t* __restrict__ order) {
  cnt += (int64_t)blockIdx.x * n;
  order += (int64_t)blockIdx.x * n;
  constexpr int kWaves = kOrderThreads / kWave;
  __shared__ int32_t wmax[kWaves];
  __shared__ int32_t slot[kOrderBuckets][kOrderThreads];  // per-thread counts, then first slots
  __shared__ int32_t total[kOrderBuckets];
  const int t = threadIdx.x, lane = t & (kWave - 1), wv = t >> 6;
  int32_t mx = 0;
  for (int i = t; i < n; i += kOrderThreads) mx = cnt[i] > mx ? cnt[i] : mx;
  mx = wave_reduce(mx, MaxOp());
  if (lane == 0) wmax[wv] = mx;
  __syncthreads();
  mx = 0;
  for (int k = 0; k < kWaves; ++k) mx = wmax[k] > mx ? wmax[k] : mx;
  const int64_t span = (int64_t)mx + 1;
  auto bucket_of = [&](int32_t c) { return (int)(((int64_t)(c > 0 ? c : 0) * kOrderBuckets) / span); };
  const int chunk = (n + kOrderThreads - 1) / kOrderThreads;
  const int p0 = t * chunk < n ? t * chunk : n;
  const int p1 = p0 + chunk < n ? p0 + chunk : n;
  int32_t mine[kOrderBuckets] = {};
  for (int p = p0; p < p1; ++p) {
    const int b = bucket_of(cnt[n - 1 - p]);
#pragma unroll
    for (int k = 0; k < kOrderBuckets; ++k) mine[k] += (b == k);
  }
#pragma unroll
  for (int k = 0; k < kOrderBuckets; ++k) slot[k][t] = mine[k];
  __syncthreads();
  // exclusive scan over threads, wave b for bucket b (kOrderThreads / kWave entries per lane)
  if (wv < kOrderBuckets) {
    constexpr int PER = kOrderThreads / kWave;
    int32_t* row = slot[wv];
    int32_t sum = 0;
    for (int k = 0; k < PER; ++k) sum += row[lane * PER + k];
    int32_t incl = sum;
#pragma unroll
    for (int off = 1; off < kWave; off <<= 1) {
      const int32_t y = __shfl_up(incl, off);
      if (lane >= off) incl += y;
    }
    int32_t run = incl - sum;
    for (int k = 0; k < PER; ++k) {
      const int32_t c = row[lane * PER + k];
      row[lane * PER + k] = run;
      run += c;
    }
    if (lane == kWave - 1) total[wv] = incl;
  }
  __syncthreads();
  int32_t pos[kOrderBuckets];
  int32_t base = 0;
#pragma unroll
  for (int k = kOrderBuckets - 1; k >= 0; --k) {
    pos[k] = base + slot[k][t];
    base += total[k];
  }
  for (int p = p0; p < p1; ++p) {
    const int i = n - 1 - p;
    const int b = bucket_of(cnt[i]);
    int32_t at = 0;
#pragma unroll
    for (int k = 0; k < kOrderBuckets; ++k) {
      if (b == k) at = pos[k]++;
    }
    order[at] = i;
  }
}

}  // namespace

hipError_t launch_block_minmax(MaskVecs v, int32_t nk, int32_t BN, int32_t* mm,
                               hipStream_t stream, int32_t sets, int64_t vec_stride) {
  const int32_t n_kb = (nk + BN - 1) / BN;
  const uintptr_t all = (uintptr_t)v.lts | (uintptr_t)v.lte | (uintptr_t)v.uts | (uintptr_t)v.ute;
  if ((BN == 64 || BN == 128) && (all & 15) == 0 && (sets == 1 || vec_stride % 4 == 0)) {
    const int bpw = kWave / (BN / 4);  // key blocks per wave
    const int64_t grid = ((int64_t)n_kb + bpw * kWavesPerBlock - 1) / (bpw * kWavesPerBlock);
    if (BN == 64)
      hipLaunchKernelGGL(block_minmax_vec_kernel<16>, dim3((unsigned)grid, sets), dim3(256), 0,
                         stream, v, vec_stride, nk, n_kb, mm);
    else
      hipLaunchKernelGGL(block_minmax_vec_kernel<32>, dim3((unsigned)grid, sets), dim3(256), 0,
                         stream, v, vec_stride, nk, n_kb, mm);
    return hipGetLastError();
  }
  const int grid = (n_kb + kWavesPerBlock - 1) / kWavesPerBlock;
  hipLaunchKernelGGL(block_minmax_kernel, dim3(grid, sets), dim3(256), 0, stream, v, vec_stride, nk,
                     BN, n_kb, mm);
  return hipGetLastError();
}

hipError_t launch_classify(const int32_t* mm, int32_t n_kb, int32_t nq, int32_t BM,
                           uint8_t* cls, int32_t* qcnt, int32_t* qlist, int32_t* kcnt,
                           int32_t* klist, hipStream_t stream, int32_t sets) {
  const int32_t n_qb = (nq + BM - 1) / BM;
  const int32_t row_waves = (cls || qcnt || qlist) ? n_qb : 0;
  const int32_t col_waves = (kcnt && klist) ? n_kb : 0;
  const int64_t waves = (int64_t)row_waves + col_waves;
  if (waves == 0) return hipSuccess;
  const int grid = (int)((waves + kWavesPerBlock - 1) / kWavesPerBlock);
  hipLaunchKernelGGL(classify_kernel, dim3(grid, sets), dim3(256), 0, stream, mm, n_kb, nq, BM,
                     n_qb, row_waves, col_waves, cls, qcnt, qlist, kcnt, klist);
  return hipGetLastError();
}

hipError_t launch_block_order(const int32_t* cnt, int32_t n, int32_t* order, hipStream_t stream,
                              int32_t sets) {
  if (n <= 0) return hipSuccess;
  hipLaunchKernelGGL(block_order_kernel, dim3(sets), dim3(kOrderThreads), 0, stream, cnt, n, order);
  return hipGetLastError();
}

hipError_t launch_localize(MaskVecs in, int32_t n, const ChunkTable& table, int32_t* lts,
                           int32_t* lte, int32_t* uts, int32_t* ute, hipStream_t stream) {
  const uintptr_t all = (uintptr_t)in.lts | (uintptr_t)in.lte | (uintptr_t)in.uts |
                        (uintptr_t)in.ute | (uintptr_t)lts | (uintptr_t)lte | (uintptr_t)uts |
                        (uintptr_t)ute;
  if ((all & 15) == 0) {
    const int grid = grid_for((n / 4) > 0 ? n / 4 : 1, 256, 4096);
    hipLaunchKernelGGL(localize_kernel<4>, dim3(grid), dim3(256), 0, stream, in, n, table, lts,
                       lte, uts, ute);
  } else {
    const int grid = grid_for(n, 256, 4096);
    hipLaunchKernelGGL(localize_kernel<1>, dim3(grid), dim3(256), 0, stream, in, n, table, lts,
                       lte, uts, ute);
  }
  return hipGetLastError();
}

}  // namespace fm
