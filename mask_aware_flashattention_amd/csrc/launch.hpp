// Internal launch wrappers (host side).  Each returns the hipError_t of its launch(es); the
// C ABI in api.cpp validates every argument before calling them.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace fm {

struct MaskVecs {
  const int32_t* lts;
  const int32_t* lte;
  const int32_t* uts;
  const int32_t* ute;
};

// Per key block of BN keys: min and max of each vector.  mm is int32[8][n_kb], rows
// (LTS min, LTS max, LTE min, LTE max, UTS min, UTS max, UTE min, UTE max).  With sets > 1 the
// vectors of set s start at s * vec_stride and its output at mm + s * 8 * n_kb.
hipError_t launch_block_minmax(MaskVecs v, int32_t nk, int32_t BN, int32_t* mm,
                               hipStream_t stream, int32_t sets = 1, int64_t vec_stride = 0);

// Tile classes and compacted lists from the block min/max (NULL outputs are skipped).  With
// sets > 1 every array is repeated per set ([sets][...] with the single-set sizes).
hipError_t launch_classify(const int32_t* mm, int32_t n_kb, int32_t nq, int32_t BM,
                           uint8_t* cls, int32_t* qcnt, int32_t* qlist, int32_t* kcnt,
                           int32_t* klist, hipStream_t stream, int32_t sets = 1);

// Block indices 0..n-1 in four buckets by cnt[i], the bucket of the largest counts first,
// descending index order inside a bucket (order must hold n entries; per set with sets > 1).
hipError_t launch_block_order(const int32_t* cnt, int32_t n, int32_t* order, hipStream_t stream,
                              int32_t sets = 1);

constexpr int kMaxChunks = 64;
struct ChunkTable {
  int32_t n_chunks;
  int32_t end[kMaxChunks];    // o_k + L_k
  int32_t shift[kMaxChunks];  // P_k - o_k
};

hipError_t launch_localize(MaskVecs in, int32_t n, const ChunkTable& table, int32_t* lts,
                           int32_t* lte, int32_t* uts, int32_t* ute, hipStream_t stream);

// Tensor layout and grouping shared by the attention kernels.  Element strides (batch, head,
// row) of the query-side tensors Q, O, dQ, dO and of the key-side tensors K, V, dK, dV; the d
// axis is contiguous.  Query head h reads key/value head h / G.  Mask vector set of (b, h):
// (mask_b > 1 ? b : 0) * mask_h + (mask_h > 1 ? h : 0); set s of each vector starts at
// s * mask_stride, and its lists / counts / order at s times their single-set size.  LSE, D and
// LSE * log2(e) stay contiguous [B][H][nq].
struct Layout {
  int32_t B, H, G;
  int64_t qs_b, qs_h, qs_r;
  int64_t ks_b, ks_h, ks_r;
  int32_t mask_b, mask_h;
  int64_t mask_stride;
};
__host__ __device__ inline int32_t mask_set(const Layout& L, int32_t b, int32_t h) {
  return (L.mask_b > 1 ? b : 0) * L.mask_h + (L.mask_h > 1 ? h : 0);
}
__host__ __device__ inline int32_t mask_sets(const Layout& L) { return L.mask_b * L.mask_h; }
// Contiguous [B][H][n][d] tensors, K/V with H heads, one mask set.
inline Layout contiguous_layout(int32_t B, int32_t H, int32_t nq, int32_t nk, int32_t d) {
  return Layout{B, H, 1, (int64_t)H * nq * d, (int64_t)nq * d, d, (int64_t)H * nk * d,
                (int64_t)nk * d, d, 1, 1, nk};
}

// Forward attention over precomputed lists.  dtype 0 = bf16 (d 128), 1 = fp32 (d 64).
struct FwdArgs {
  const void* q;
  const void* k;
  const void* v;
  MaskVecs mask;
  void* o;
  float* lse;
  const int32_t* qcnt;
  const int32_t* qlist;
  const int32_t* order;  // query blocks, longest list first
  int32_t list_stride;  // n_kb
  Layout L;
  int32_t nq, nk;
  float scale;
};
// ev_begin / ev_end (may be null) are recorded on the stream around the attention kernel.
hipError_t launch_attn_fwd(int dtype, const FwdArgs& a, hipStream_t stream, hipEvent_t ev_begin,
                           hipEvent_t ev_end);

// Backward, query-stationary part, run first: dQ over the forward's tile lists; it also writes,
// per row, -D (D_i = sum_d dO_id O_id) and LSE * log2(e) (+inf on fully masked rows) for the
// dK/dV kernel.
struct DqArgs {
  const void* q;
  const void* k;
  const void* v;
  const void* o;
  const void* dout;
  const float* lse;
  MaskVecs mask;
  void* dq;
  float* delta;  // float32 [B,H,nq]: -D
  float* lse2;   // float32 [B,H,nq]
  const int32_t* qcnt;
  const int32_t* qlist;
  const int32_t* order;  // query blocks, longest list first
  int32_t list_stride;  // n_kb at the forward tile shape
  Layout L;
  int32_t nq, nk;
  float scale;
};
// ev_begin (may be null) is recorded before the dQ kernel.
hipError_t launch_attn_dq(int dtype, const DqArgs& a, hipStream_t stream, hipEvent_t ev_begin);

// Backward, key-stationary part: dK, dV (needs delta and lse2 from launch_attn_dq on the same
// stream).
struct BwdArgs {
  const void* q;
  const void* k;
  const void* v;
  const void* dout;
  MaskVecs mask;
  void* dk;
  void* dv;
  const float* delta;  // -D per row
  const float* lse2;   // LSE * log2(e) per row
  const int32_t* kcnt;
  const int32_t* klist;
  const int32_t* order;  // key blocks, longest list first
  int32_t list_stride;  // n_qb at the backward tile shape
  int32_t list_bn;      // keys per key block of the lists: 64, or 128 for long query sequences
  Layout L;
  int32_t nq, nk;
  float scale;
};
// ev_end (may be null) is recorded after the dK/dV kernel.
hipError_t launch_attn_bwd(int dtype, const BwdArgs& a, hipStream_t stream, hipEvent_t ev_end);

// Tile shapes of the attention kernels (the shapes tiles are classified at).
struct TileShape {
  int32_t bm_fwd, bn_fwd, bm_bwd, bn_bwd;
};
TileShape tile_shape(int dtype);

}  // namespace fm
