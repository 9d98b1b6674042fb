// C ABI of the mask-aware attention library: host-side argument checks (all before any device
// work), workspace layout, and the launch sequence of each call on the caller's stream.
#include <hip/hip_runtime.h>

#include <cmath>
#include <cstdint>
#include <cstring>

#include "../../include/flashmask.h"
#include "launch.hpp"

namespace {

constexpr size_t kAlign = 256;
constexpr int64_t kMaxListEntries = (int64_t(1) << 31) - 1;
// Per (batch, head) every slab the kernels address with 32-bit buffer offsets (Q, K, V, O, dO;
// 256 bytes per row) must stay below 4 GiB.
constexpr int32_t kMaxLen = int32_t(1) << 22;

inline size_t round_up(size_t x) { return (x + kAlign - 1) / kAlign * kAlign; }
inline int64_t ceil_div(int64_t a, int64_t b) { return (a + b - 1) / b; }
inline bool aligned(const void* p, uintptr_t a) { return (reinterpret_cast<uintptr_t>(p) % a) == 0; }

struct Geometry {
  int64_t n_qb, n_kb;
};

int32_t check_dtype(int32_t dtype, int32_t d) {
  if (dtype != FM_BF16 && dtype != FM_FP32) return FM_ERR_DTYPE;
  if ((dtype == FM_BF16 && d != 128) || (dtype == FM_FP32 && d != 64)) return FM_ERR_UNSUPPORTED;
  return FM_OK;
}

int32_t check_vectors(const int32_t* a, const int32_t* b, const int32_t* c, const int32_t* d) {
  if (!a || !b || !c || !d) return FM_ERR_NULL;
  if (!aligned(a, 4) || !aligned(b, 4) || !aligned(c, 4) || !aligned(d, 4)) return FM_ERR_ALIGN;
  return FM_OK;
}

int32_t check_scale(float scale) {
  return (std::isfinite(scale) && scale > 0.0f) ? FM_OK : FM_ERR_VALUE;
}

fm::TileShape tiles(int32_t dtype) { return fm::tile_shape(dtype); }

inline int64_t elem_size(int32_t dtype) { return dtype == FM_BF16 ? 2 : 4; }

// Contiguous layout of an fm_shape: [B][H][n][d] tensors, H key/value heads, one mask set.
fm_layout from_shape(const fm_shape* s) {
  fm_layout l;
  l.B = s->B;
  l.H = s->H;
  l.H_kv = s->H;
  l.nq = s->nq;
  l.nk = s->nk;
  l.d = s->d;
  l.dtype = s->dtype;
  l.mask_b = 1;
  l.mask_h = 1;
  l.q_stride[0] = int64_t(s->H) * s->nq * s->d;
  l.q_stride[1] = int64_t(s->nq) * s->d;
  l.q_stride[2] = s->d;
  l.kv_stride[0] = int64_t(s->H) * s->nk * s->d;
  l.kv_stride[1] = int64_t(s->nk) * s->d;
  l.kv_stride[2] = s->d;
  return l;
}

fm::Layout to_internal(const fm_layout* l) {
  return fm::Layout{l->B,           l->H,           l->H / l->H_kv,
                    l->q_stride[0], l->q_stride[1], l->q_stride[2],
                    l->kv_stride[0], l->kv_stride[1], l->kv_stride[2],
                    l->mask_b,      l->mask_h,      l->nk};
}

inline int32_t mask_sets(const fm_layout* l) { return l->mask_b * l->mask_h; }

// Rows of the largest tile any attention kernel reads at once (query blocks of the forward and
// dQ kernels, key blocks of the dK/dV kernel's 8-wave shape).
constexpr int64_t kPadRows = 128;

// True if the (batch, head, row) element offsets of a [B][H][n][d] view with these element
// strides (d contiguous) never coincide: sorted by stride, each axis of extent > 1 must step
// over everything the smaller axes span.  A zero stride on an axis of extent > 1 fails.
bool non_overlapping(int64_t B, int64_t H, int64_t n, int64_t d, const int64_t* stride) {
  struct Ax {
    int64_t extent, stride;
  } ax[3] = {{B, stride[0]}, {H, stride[1]}, {n, stride[2]}};
  // insertion sort by stride (three entries)
  for (int i = 1; i < 3; ++i)
    for (int j = i; j > 0 && ax[j].stride < ax[j - 1].stride; --j) {
      const Ax t = ax[j];
      ax[j] = ax[j - 1];
      ax[j - 1] = t;
    }
  int64_t span = d;  // elements spanned by the axes below (a row is d contiguous elements)
  for (int i = 0; i < 3; ++i) {
    if (ax[i].extent <= 1) continue;
    if (ax[i].stride < span) return false;
    span = (ax[i].extent - 1) * ax[i].stride + span;
  }
  return true;
}

// Layout checks shared by forward and backward (bwd: the dK/dV kernel also spans the query
// heads of a group); fills the tile geometry for (BM, BN).
int32_t check_layout(const fm_layout* l, int32_t BM, int32_t BN, bool bwd, Geometry* g) {
  if (!l) return FM_ERR_NULL;
  const int32_t st = check_dtype(l->dtype, l->d);
  if (st != FM_OK) return st;
  if (l->B < 1 || l->H < 1 || l->H_kv < 1 || l->nq < 1 || l->nk < 1) return FM_ERR_SHAPE;
  if (l->H % l->H_kv != 0) return FM_ERR_SHAPE;
  if (l->nq > kMaxLen || l->nk > kMaxLen) return FM_ERR_SHAPE;
  if ((l->mask_b != 1 && l->mask_b != l->B) || (l->mask_h != 1 && l->mask_h != l->H))
    return FM_ERR_SHAPE;
  const int64_t n_qb = ceil_div(l->nq, BM), n_kb = ceil_div(l->nk, BN);
  if (n_qb * n_kb > kMaxListEntries) return FM_ERR_SHAPE;
  const int64_t bh = int64_t(l->B) * l->H;
  if (bh * n_qb > 0x7fffffffLL || bh * n_kb > 0x7fffffffLL) return FM_ERR_SHAPE;
  const int64_t es = elem_size(l->dtype);
  for (int i = 0; i < 3; ++i) {
    if (l->q_stride[i] < 0 || l->kv_stride[i] < 0) return FM_ERR_SHAPE;
    if (l->q_stride[i] > (int64_t(1) << 40) || l->kv_stride[i] > (int64_t(1) << 40)) return FM_ERR_SHAPE;
  }
  if (l->q_stride[2] < l->d || l->kv_stride[2] < l->d) return FM_ERR_SHAPE;
  for (int i = 0; i < 3; ++i)
    if ((l->q_stride[i] * es) % 16 != 0 || (l->kv_stride[i] * es) % 16 != 0) return FM_ERR_ALIGN;
  // O and dQ are written through q_stride, dK and dV through kv_stride: distinct (batch, head,
  // row) must reach distinct memory.
  if (!non_overlapping(l->B, l->H, l->nq, l->d, l->q_stride) ||
      !non_overlapping(l->B, l->H_kv, l->nk, l->d, l->kv_stride))
    return FM_ERR_SHAPE;
  // Every buffer a kernel addresses with 32-bit offsets stays below 4 GiB, including the rows
  // past the end that the last (ragged) tile addresses: the kernels read whole tiles of up to
  // kPadRows rows and rely on such offsets landing past the buffer's end (where loads return
  // zeros), so they must not wrap around 2^32.
  const int64_t G = l->H / l->H_kv;
  const int64_t nq_pad = ceil_div(l->nq, kPadRows) * kPadRows;
  const int64_t nk_pad = ceil_div(l->nk, kPadRows) * kPadRows;
  int64_t q_span = ((nq_pad - 1) * l->q_stride[2] + l->d) * es;
  if (bwd) {
    if (G > 256) return FM_ERR_SHAPE;
    q_span += (G - 1) * l->q_stride[1] * es;
  }
  const int64_t k_span = ((nk_pad - 1) * l->kv_stride[2] + l->d) * es;
  if (q_span >= (int64_t(1) << 32) || k_span >= (int64_t(1) << 32)) return FM_ERR_SHAPE;
  if (g) *g = Geometry{n_qb, n_kb};
  return FM_OK;
}

// Forward workspace: key-block min/max, query-block lists and the longest-first block order.
struct FwdWs {
  size_t mm, qcnt, qlist, order, total;
};
FwdWs fwd_layout(const Geometry& g, int64_t sets = 1) {
  FwdWs w;
  w.mm = 0;
  w.qcnt = w.mm + round_up(sizeof(int32_t) * 8 * g.n_kb * sets);
  w.qlist = w.qcnt + round_up(sizeof(int32_t) * g.n_qb * sets);
  w.order = w.qlist + round_up(sizeof(int32_t) * g.n_qb * g.n_kb * sets);
  w.total = w.order + round_up(sizeof(int32_t) * g.n_qb * sets);
  return w;
}

// Backward workspace: key-block lists at the backward tile shape (dK/dV kernel), query-block
// lists at the forward tile shape (dQ kernel), both block orders, and the per-row D and
// LSE * log2(e).
struct BwdWs {
  size_t mm, kcnt, klist, mm_f, qcnt, qlist, korder, qorder, delta, lse2, total;
};
BwdWs bwd_layout(const fm_layout* s, const Geometry& g, const Geometry& gf) {
  BwdWs w;
  const size_t rows = size_t(s->B) * s->H * s->nq;
  const size_t sets = size_t(mask_sets(s));
  w.mm = 0;
  w.kcnt = w.mm + round_up(sizeof(int32_t) * 8 * g.n_kb * sets);
  w.klist = w.kcnt + round_up(sizeof(int32_t) * g.n_kb * sets);
  w.mm_f = w.klist + round_up(sizeof(int32_t) * g.n_qb * g.n_kb * sets);
  w.qcnt = w.mm_f + round_up(sizeof(int32_t) * 8 * gf.n_kb * sets);
  w.qlist = w.qcnt + round_up(sizeof(int32_t) * gf.n_qb * sets);
  w.korder = w.qlist + round_up(sizeof(int32_t) * gf.n_qb * gf.n_kb * sets);
  w.qorder = w.korder + round_up(sizeof(int32_t) * g.n_kb * sets);
  w.delta = w.qorder + round_up(sizeof(int32_t) * gf.n_qb * sets);
  w.lse2 = w.delta + round_up(sizeof(float) * rows);
  w.total = w.lse2 + round_up(sizeof(float) * rows);
  return w;
}

inline int32_t hip_status(hipError_t e) { return e == hipSuccess ? FM_OK : FM_ERR_HIP; }

// Optional timing events (flashmask_set_profile_events); null unless a benchmark sets them.
// Per calling thread, so calls made from other threads never record into them.
thread_local hipEvent_t g_fwd_begin = nullptr, g_fwd_end = nullptr, g_bwd_begin = nullptr,
                        g_bwd_end = nullptr;

}  // namespace

extern "C" {

const char* flashmask_strerror(int32_t status) {
  switch (status) {
    case FM_OK: return "ok";
    case FM_ERR_NULL: return "a required pointer is NULL";
    case FM_ERR_SHAPE: return "a size is out of range";
    case FM_ERR_DTYPE: return "unknown dtype";
    case FM_ERR_UNSUPPORTED: return "unsupported (dtype, head dim); built: (bf16, 128), (fp32, 64)";
    case FM_ERR_ALIGN: return "pointer misaligned (tensors need 16 bytes, vectors 4)";
    case FM_ERR_WORKSPACE: return "workspace missing or too small";
    case FM_ERR_CHUNKS: return "chunk table not sorted, disjoint, non-empty and in range (1..64 chunks)";
    case FM_ERR_HIP: return "HIP launch failed";
    case FM_ERR_VALUE: return "invalid scalar argument (scale must be finite and > 0)";
    case FM_ERR_SCRATCH: return "problem too large for the no-alloc call's fixed scratch array";
    default: return "unknown status";
  }
}

int32_t flashmask_tile_sizes(int32_t dtype, int32_t d, int32_t* BM_fwd, int32_t* BN_fwd,
                             int32_t* BM_bwd, int32_t* BN_bwd) {
  const int32_t st = check_dtype(dtype, d);
  if (st != FM_OK) return st;
  if (!BM_fwd || !BN_fwd || !BM_bwd || !BN_bwd) return FM_ERR_NULL;
  const fm::TileShape t = tiles(dtype);
  *BM_fwd = t.bm_fwd;
  *BN_fwd = t.bn_fwd;
  *BM_bwd = t.bm_bwd;
  *BN_bwd = t.bn_bwd;
  return FM_OK;
}

size_t flashmask_fwd_ex_workspace_bytes(const fm_layout* l) {
  if (!l || check_dtype(l->dtype, l->d) != FM_OK) return 0;
  const fm::TileShape t = tiles(l->dtype);
  Geometry g;
  if (check_layout(l, t.bm_fwd, t.bn_fwd, false, &g) != FM_OK) return 0;
  return fwd_layout(g, mask_sets(l)).total;
}

int32_t flashmask_fwd_ex(const fm_layout* l, const void* Q, const void* K, const void* V,
                         const int32_t* LTS, const int32_t* LTE, const int32_t* UTS,
                         const int32_t* UTE, float scale, void* O, float* LSE, void* ws,
                         size_t ws_bytes, void* stream) {
  if (!l) return FM_ERR_NULL;
  int32_t st = check_dtype(l->dtype, l->d);
  if (st != FM_OK) return st;
  const fm::TileShape t = tiles(l->dtype);
  Geometry g;
  if ((st = check_layout(l, t.bm_fwd, t.bn_fwd, false, &g)) != FM_OK) return st;
  if (!Q || !K || !V || !O || !LSE) return FM_ERR_NULL;
  if ((st = check_vectors(LTS, LTE, UTS, UTE)) != FM_OK) return st;
  if (!aligned(Q, 16) || !aligned(K, 16) || !aligned(V, 16) || !aligned(O, 16) || !aligned(LSE, 4))
    return FM_ERR_ALIGN;
  if ((st = check_scale(scale)) != FM_OK) return st;
  const int32_t sets = mask_sets(l);
  const FwdWs L = fwd_layout(g, sets);
  if (!ws || ws_bytes < L.total) return FM_ERR_WORKSPACE;
  if (!aligned(ws, 16)) return FM_ERR_ALIGN;

  hipStream_t hs = static_cast<hipStream_t>(stream);
  char* base = static_cast<char*>(ws);
  int32_t* mm = reinterpret_cast<int32_t*>(base + L.mm);
  int32_t* qcnt = reinterpret_cast<int32_t*>(base + L.qcnt);
  int32_t* qlist = reinterpret_cast<int32_t*>(base + L.qlist);
  int32_t* order = reinterpret_cast<int32_t*>(base + L.order);
  const fm::MaskVecs mv{LTS, LTE, UTS, UTE};

  hipError_t e = fm::launch_block_minmax(mv, l->nk, t.bn_fwd, mm, hs, sets, l->nk);
  if (e == hipSuccess)
    e = fm::launch_classify(mm, (int32_t)g.n_kb, l->nq, t.bm_fwd, nullptr, qcnt, qlist, nullptr,
                            nullptr, hs, sets);
  if (e == hipSuccess) e = fm::launch_block_order(qcnt, (int32_t)g.n_qb, order, hs, sets);
  if (e == hipSuccess) {
    fm::FwdArgs a{Q,     K,     V,     mv,   O,    LSE,  qcnt, qlist, order, (int32_t)g.n_kb,
                  to_internal(l), l->nq, l->nk, scale};
    e = fm::launch_attn_fwd(l->dtype, a, hs, g_fwd_begin, g_fwd_end);
  }
  return hip_status(e);
}

size_t flashmask_fwd_workspace_bytes(const fm_shape* s) {
  if (!s) return 0;
  const fm_layout l = from_shape(s);
  return flashmask_fwd_ex_workspace_bytes(&l);
}

int32_t flashmask_fwd(const fm_shape* s, const void* Q, const void* K, const void* V,
                      const int32_t* LTS, const int32_t* LTE, const int32_t* UTS,
                      const int32_t* UTE, float scale, void* O, float* LSE, void* ws,
                      size_t ws_bytes, void* stream) {
  if (!s) return FM_ERR_NULL;
  const fm_layout l = from_shape(s);
  return flashmask_fwd_ex(&l, Q, K, V, LTS, LTE, UTS, UTE, scale, O, LSE, ws, ws_bytes, stream);
}

// Geometry of the dK/dV kernel's column lists: key blocks of t.bn_bwd keys, or of twice that
// for long query sequences (the kernel shape that keeps Q/dO loads further ahead) and where the
// finer grid would exceed the list limits; *bn gets the width, which selects the kernel shape.
constexpr int32_t kLongQuery = 65536;
int32_t bwd_col_geometry(const fm_layout* l, const fm::TileShape& t, Geometry* g, int32_t* bn) {
  if (l && l->nq < kLongQuery) {
    *bn = t.bn_bwd;
    const int32_t st = check_layout(l, t.bm_bwd, t.bn_bwd, true, g);
    if (st != FM_ERR_SHAPE) return st;
  }
  *bn = 2 * t.bn_bwd;
  return check_layout(l, t.bm_bwd, 2 * t.bn_bwd, true, g);
}

size_t flashmask_bwd_ex_workspace_bytes(const fm_layout* l) {
  if (!l || check_dtype(l->dtype, l->d) != FM_OK) return 0;
  const fm::TileShape t = tiles(l->dtype);
  Geometry g, gf;
  int32_t bn_b;
  if (bwd_col_geometry(l, t, &g, &bn_b) != FM_OK) return 0;
  if (check_layout(l, t.bm_fwd, t.bn_fwd, true, &gf) != FM_OK) return 0;
  return bwd_layout(l, g, gf).total;
}

int32_t flashmask_bwd_ex(const fm_layout* l, const void* Q, const void* K, const void* V,
                         const void* O, const void* dO, const float* LSE, const int32_t* LTS,
                         const int32_t* LTE, const int32_t* UTS, const int32_t* UTE, float scale,
                         void* dQ, void* dK, void* dV, void* ws, size_t ws_bytes, void* stream) {
  if (!l) return FM_ERR_NULL;
  int32_t st = check_dtype(l->dtype, l->d);
  if (st != FM_OK) return st;
  const fm::TileShape t = tiles(l->dtype);
  Geometry g, gf;
  int32_t bn_b;
  if ((st = bwd_col_geometry(l, t, &g, &bn_b)) != FM_OK) return st;
  if ((st = check_layout(l, t.bm_fwd, t.bn_fwd, true, &gf)) != FM_OK) return st;
  if (!Q || !K || !V || !O || !dO || !LSE || !dQ || !dK || !dV) return FM_ERR_NULL;
  if ((st = check_vectors(LTS, LTE, UTS, UTE)) != FM_OK) return st;
  if (!aligned(Q, 16) || !aligned(K, 16) || !aligned(V, 16) || !aligned(O, 16) ||
      !aligned(dO, 16) || !aligned(dQ, 16) || !aligned(dK, 16) || !aligned(dV, 16) ||
      !aligned(LSE, 4))
    return FM_ERR_ALIGN;
  if ((st = check_scale(scale)) != FM_OK) return st;
  const int32_t sets = mask_sets(l);
  const BwdWs L = bwd_layout(l, g, gf);
  if (!ws || ws_bytes < L.total) return FM_ERR_WORKSPACE;
  if (!aligned(ws, 16)) return FM_ERR_ALIGN;

  hipStream_t hs = static_cast<hipStream_t>(stream);
  char* base = static_cast<char*>(ws);
  int32_t* mm = reinterpret_cast<int32_t*>(base + L.mm);
  int32_t* kcnt = reinterpret_cast<int32_t*>(base + L.kcnt);
  int32_t* klist = reinterpret_cast<int32_t*>(base + L.klist);
  int32_t* mm_f = reinterpret_cast<int32_t*>(base + L.mm_f);
  int32_t* qcnt = reinterpret_cast<int32_t*>(base + L.qcnt);
  int32_t* qlist = reinterpret_cast<int32_t*>(base + L.qlist);
  int32_t* korder = reinterpret_cast<int32_t*>(base + L.korder);
  int32_t* qorder = reinterpret_cast<int32_t*>(base + L.qorder);
  float* delta = reinterpret_cast<float*>(base + L.delta);
  float* lse2 = reinterpret_cast<float*>(base + L.lse2);
  const fm::MaskVecs mv{LTS, LTE, UTS, UTE};
  const fm::Layout lay = to_internal(l);

  hipError_t e = fm::launch_block_minmax(mv, l->nk, bn_b, mm, hs, sets, l->nk);
  if (e == hipSuccess)
    e = fm::launch_classify(mm, (int32_t)g.n_kb, l->nq, t.bm_bwd, nullptr, nullptr, nullptr, kcnt,
                            klist, hs, sets);
  if (e == hipSuccess) e = fm::launch_block_minmax(mv, l->nk, t.bn_fwd, mm_f, hs, sets, l->nk);
  if (e == hipSuccess)
    e = fm::launch_classify(mm_f, (int32_t)gf.n_kb, l->nq, t.bm_fwd, nullptr, qcnt, qlist, nullptr,
                            nullptr, hs, sets);
  if (e == hipSuccess) e = fm::launch_block_order(kcnt, (int32_t)g.n_kb, korder, hs, sets);
  if (e == hipSuccess) e = fm::launch_block_order(qcnt, (int32_t)gf.n_qb, qorder, hs, sets);
  if (e == hipSuccess) {
    fm::DqArgs a{Q,    K,     V,     O,     dO,   LSE,  mv,    dQ,   delta, lse2, qcnt, qlist,
                 qorder, (int32_t)gf.n_kb, lay, l->nq, l->nk, scale};
    e = fm::launch_attn_dq(l->dtype, a, hs, g_bwd_begin);
  }
  if (e == hipSuccess) {
    fm::BwdArgs a{Q,     K,    V,      dO,   mv,   dK, dV, delta, lse2, kcnt, klist,
                  korder, (int32_t)g.n_qb, bn_b, lay, l->nq, l->nk, scale};
    e = fm::launch_attn_bwd(l->dtype, a, hs, g_bwd_end);
  }
  return hip_status(e);
}

size_t flashmask_bwd_workspace_bytes(const fm_shape* s) {
  if (!s) return 0;
  const fm_layout l = from_shape(s);
  return flashmask_bwd_ex_workspace_bytes(&l);
}

int32_t flashmask_bwd(const fm_shape* s, const void* Q, const void* K, const void* V,
                      const void* O, const void* dO, const float* LSE, const int32_t* LTS,
                      const int32_t* LTE, const int32_t* UTS, const int32_t* UTE, float scale,
                      void* dQ, void* dK, void* dV, void* ws, size_t ws_bytes, void* stream) {
  if (!s) return FM_ERR_NULL;
  const fm_layout l = from_shape(s);
  return flashmask_bwd_ex(&l, Q, K, V, O, dO, LSE, LTS, LTE, UTS, UTE, scale, dQ, dK, dV, ws,
                          ws_bytes, stream);
}

int32_t flashmask_localize(const int32_t* LTS_g, const int32_t* LTE_g, const int32_t* UTS_g,
                           const int32_t* UTE_g, int32_t n, int32_t nq_global,
                           const int32_t* chunk_start, const int32_t* chunk_len,
                           int32_t n_chunks, int32_t* LTS_l, int32_t* LTE_l, int32_t* UTS_l,
                           int32_t* UTE_l, int32_t* n_local, void* stream) {
  if (!chunk_start || !chunk_len || !n_local) return FM_ERR_NULL;
  if (n < 0 || nq_global < 0) return FM_ERR_SHAPE;
  if (n_chunks < 1 || n_chunks > fm::kMaxChunks) return FM_ERR_CHUNKS;
  fm::ChunkTable table;
  std::memset(&table, 0, sizeof(table));
  table.n_chunks = n_chunks;
  int64_t prefix = 0, prev_end = 0;
  for (int k = 0; k < n_chunks; ++k) {
    const int64_t o = chunk_start[k], L = chunk_len[k];
    if (L < 1 || o < 0 || o + L > nq_global || o < prev_end) return FM_ERR_CHUNKS;
    table.end[k] = (int32_t)(o + L);
    table.shift[k] = (int32_t)(prefix - o);
    prefix += L;
    prev_end = o + L;
  }
  if (n > 0) {
    int32_t st = check_vectors(LTS_g, LTE_g, UTS_g, UTE_g);
    if (st != FM_OK) return st;
    if ((st = check_vectors(LTS_l, LTE_l, UTS_l, UTE_l)) != FM_OK) return st;
  }
  *n_local = (int32_t)prefix;
  if (n == 0) return FM_OK;
  const fm::MaskVecs in{LTS_g, LTE_g, UTS_g, UTE_g};
  return hip_status(fm::launch_localize(in, n, table, LTS_l, LTE_l, UTS_l, UTE_l,
                                        static_cast<hipStream_t>(stream)));
}

size_t flashmask_classify_workspace_bytes(int32_t nk, int32_t BN) {
  if (nk < 1 || BN < 1) return 0;
  return round_up(sizeof(int32_t) * 8 * (size_t)ceil_div(nk, BN));
}

int32_t flashmask_classify(const int32_t* LTS, const int32_t* LTE, const int32_t* UTS,
                           const int32_t* UTE, int32_t nq, int32_t nk, int32_t BM, int32_t BN,
                           uint8_t* cls, int32_t* qcnt, int32_t* qlist, int32_t* kcnt,
                           int32_t* klist, void* ws, size_t ws_bytes, void* stream) {
  int32_t st = check_vectors(LTS, LTE, UTS, UTE);
  if (st != FM_OK) return st;
  if (nq < 1 || nk < 1 || BM < 1 || BN < 1) return FM_ERR_SHAPE;
  const int64_t n_qb = ceil_div(nq, BM), n_kb = ceil_div(nk, BN);
  if (n_qb * n_kb > kMaxListEntries || n_qb > 0x7fffffffLL / 4 || n_kb > 0x7fffffffLL / 4)
    return FM_ERR_SHAPE;
  if ((kcnt == nullptr) != (klist == nullptr)) return FM_ERR_NULL;
  if ((qcnt && !aligned(qcnt, 4)) || (qlist && !aligned(qlist, 4)) || (kcnt && !aligned(kcnt, 4)) ||
      (klist && !aligned(klist, 4)))
    return FM_ERR_ALIGN;
  const size_t need = flashmask_classify_workspace_bytes(nk, BN);
  if (!ws || ws_bytes < need) return FM_ERR_WORKSPACE;
  if (!aligned(ws, 4)) return FM_ERR_ALIGN;
  hipStream_t hs = static_cast<hipStream_t>(stream);
  int32_t* mm = static_cast<int32_t*>(ws);
  const fm::MaskVecs mv{LTS, LTE, UTS, UTE};
  hipError_t e = fm::launch_block_minmax(mv, nk, BN, mm, hs);
  if (e == hipSuccess)
    e = fm::launch_classify(mm, (int32_t)n_kb, nq, BM, cls, qcnt, qlist, kcnt, klist, hs);
  return hip_status(e);
}

size_t flashmask_prune_workspace_bytes(int32_t nk, int32_t n_local, int32_t BM, int32_t chunk) {
  if (nk < 1 || n_local < 1 || BM < 1 || chunk < 1) return 0;
  const int64_t n_qb = ceil_div(n_local, BM), n_c = ceil_div(nk, chunk);
  if (n_qb * n_c > kMaxListEntries) return 0;
  return round_up(sizeof(int32_t) * 8 * (size_t)n_c) + round_up(sizeof(int32_t) * (size_t)(n_qb * n_c));
}

int32_t flashmask_prune_chunks(const int32_t* LTS, const int32_t* LTE, const int32_t* UTS,
                               const int32_t* UTE, int32_t nk, int32_t n_local, int32_t BM,
                               int32_t chunk, int32_t* live, void* ws, size_t ws_bytes,
                               void* stream) {
  int32_t st = check_vectors(LTS, LTE, UTS, UTE);
  if (st != FM_OK) return st;
  if (!live) return FM_ERR_NULL;
  if (nk < 1 || n_local < 1 || BM < 1 || chunk < 1) return FM_ERR_SHAPE;
  const int64_t n_qb = ceil_div(n_local, BM), n_c = ceil_div(nk, chunk);
  if (n_qb * n_c > kMaxListEntries || n_qb > 0x7fffffffLL / 4 || n_c > 0x7fffffffLL / 4)
    return FM_ERR_SHAPE;
  if (!aligned(live, 4)) return FM_ERR_ALIGN;
  const size_t need = flashmask_prune_workspace_bytes(nk, n_local, BM, chunk);
  if (!ws || ws_bytes < need) return FM_ERR_WORKSPACE;
  if (!aligned(ws, 4)) return FM_ERR_ALIGN;
  hipStream_t hs = static_cast<hipStream_t>(stream);
  int32_t* mm = static_cast<int32_t*>(ws);
  int32_t* klist = reinterpret_cast<int32_t*>(static_cast<char*>(ws) + round_up(sizeof(int32_t) * 8 * (size_t)n_c));
  const fm::MaskVecs mv{LTS, LTE, UTS, UTE};
  // The column-orientation count of the tile classification at (BM, chunk) is the answer.
  hipError_t e = fm::launch_block_minmax(mv, nk, chunk, mm, hs);
  if (e == hipSuccess)
    e = fm::launch_classify(mm, (int32_t)n_c, n_local, BM, nullptr, nullptr, nullptr, live, klist, hs);
  return hip_status(e);
}

int32_t flashmask_block_order(const int32_t* cnt, int32_t n, int32_t* order, void* stream) {
  if (!cnt || !order) return FM_ERR_NULL;
  if (n < 1) return FM_ERR_SHAPE;
  if (!aligned(cnt, 4) || !aligned(order, 4)) return FM_ERR_ALIGN;
  return hip_status(fm::launch_block_order(cnt, n, order, static_cast<hipStream_t>(stream)));
}

int32_t flashmask_set_profile_events(void* fwd_begin, void* fwd_end, void* bwd_begin,
                                     void* bwd_end) {
  g_fwd_begin = static_cast<hipEvent_t>(fwd_begin);
  g_fwd_end = static_cast<hipEvent_t>(fwd_end);
  g_bwd_begin = static_cast<hipEvent_t>(bwd_begin);
  g_bwd_end = static_cast<hipEvent_t>(bwd_end);
  return FM_OK;
}

}  // extern "C"
