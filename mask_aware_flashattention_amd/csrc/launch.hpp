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
// (LTS min, LTS max, LTE min, LTE max, UTS min, UTS max, UTE min, UTE max).
hipError_t launch_block_minmax(MaskVecs v, int32_t nk, int32_t BN, int32_t* mm,
                               hipStream_t stream);

// Tile classes and compacted lists from the block min/max (NULL outputs are skipped).
hipError_t launch_classify(const int32_t* mm, int32_t n_kb, int32_t nq, int32_t BM,
                           uint8_t* cls, int32_t* qcnt, int32_t* qlist, int32_t* kcnt,
                           int32_t* klist, hipStream_t stream);

// Block indices 0..n-1 in four buckets by cnt[i], the bucket of the largest counts first,
// descending index order inside a bucket (order must hold n entries).
hipError_t launch_block_order(const int32_t* cnt, int32_t n, int32_t* order, hipStream_t stream);

constexpr int kMaxChunks = 64;
struct ChunkTable {
  int32_t n_chunks;
  int32_t end[kMaxChunks];    // o_k + L_k
  int32_t shift[kMaxChunks];  // P_k - o_k
};

hipError_t launch_localize(MaskVecs in, int32_t n, const ChunkTable& table, int32_t* lts,
                           int32_t* lte, int32_t* uts, int32_t* ute, hipStream_t stream);

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
  int32_t B, H, nq, nk;
  float scale;
};
// ev_begin / ev_end (may be null) are recorded on the stream around the attention kernel.
hipError_t launch_attn_fwd(int dtype, const FwdArgs& a, hipStream_t stream, hipEvent_t ev_begin,
                           hipEvent_t ev_end);

// Backward, key-stationary part: D = rowsum(dO * O) and LSE * log2(e) (bwd_pre), then dK, dV.
struct BwdArgs {
  const void* q;
  const void* k;
  const void* v;
  const void* o;
  const void* dout;
  const float* lse;
  MaskVecs mask;
  void* dk;
  void* dv;
  float* delta;   // float32 [B,H,nq]
  float* lse2;    // float32 [B,H,nq]: LSE * log2(e), +inf on fully masked rows
  const int32_t* kcnt;
  const int32_t* klist;
  const int32_t* order;  // key blocks, longest list first
  int32_t list_stride;  // n_qb at the backward tile shape
  int32_t B, H, nq, nk;
  float scale;
};
// Runs bwd_pre and the dK/dV kernel; ev_begin (may be null) is recorded before the dK/dV kernel.
hipError_t launch_attn_bwd(int dtype, const BwdArgs& a, hipStream_t stream, hipEvent_t ev_begin);

// Backward, query-stationary part: dQ over the forward's tile lists (needs delta and lse2 from
// launch_attn_bwd on the same stream).
struct DqArgs {
  const void* q;
  const void* k;
  const void* v;
  const void* dout;
  MaskVecs mask;
  void* dq;
  const float* delta;
  const float* lse2;
  const int32_t* qcnt;
  const int32_t* qlist;
  const int32_t* order;  // query blocks, longest list first
  int32_t list_stride;  // n_kb at the forward tile shape
  int32_t B, H, nq, nk;
  float scale;
};
// ev_end (may be null) is recorded after the dQ kernel.
hipError_t launch_attn_dq(int dtype, const DqArgs& a, hipStream_t stream, hipEvent_t ev_end);

// Tile shapes of the attention kernels (the shapes tiles are classified at).
struct TileShape {
  int32_t bm_fwd, bn_fwd, bm_bwd, bn_bwd;
};
TileShape tile_shape(int dtype);

}  // namespace fm
