/*
 * flashmask.h -- C ABI of the MI355X (gfx950) mask-aware attention library.
 *
 * The mask is the column-wise sparse mask of FlashMask: four int32 vectors LTS, LTE, UTS, UTE,
 * indexed by key column j and holding query-row numbers.  Row i is masked for key j iff
 * LTS[j] <= i < LTE[j] or UTS[j] <= i < UTE[j] (half-open stretches; a stretch whose start is
 * not below its end is empty).  Source: "FlashMask-3 sends each GPU its mask without sending
 * any mask" (learnaivisually.com), four-vector paragraph; "FlashMask-3: Efficient and
 * Expressive Mask-Aware Distributed Attention", abstract.
 *
 * Conventions shared by every entry point
 *   - Device pointers are plain device addresses (hipMalloc'd or torch-allocated memory on the
 *     current device).  Host pointers are marked "host".
 *   - Tensors are contiguous, row-major: Q, O, dQ, dO are [B][H][nq][d]; K, V, dK, dV are
 *     [B][H][nk][d]; LSE is float32 [B][H][nq].  The four vectors are int32[nk], shared by every
 *     batch and head; any int32 values are accepted.
 *   - Supported (dtype, d): (FM_BF16, 128) and (FM_FP32, 64).  bf16 tensors are read and written
 *     as bf16; accumulation is float32.
 *   - The caller owns every buffer, including the workspace sized by the *_workspace_bytes
 *     call.  The library allocates no device memory, keeps no state between calls and is
 *     reentrant; calls that share a workspace must not overlap in time.
 *   - Outputs are overwritten (never accumulated into).  Inputs are read only.
 *   - `stream` is a hipStream_t passed as void*; NULL is the default stream.  Every call is
 *     asynchronous on that stream.
 *   - Errors: every argument check runs on the host before any device work, and a failed check
 *     returns its code without touching the device.  FM_ERR_HIP reports a failed kernel launch.
 *     Nothing is printed and nothing aborts.
 */
#ifndef FLASHMASK_H
#define FLASHMASK_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  FM_OK = 0,
  FM_ERR_NULL = 1,        /* a required pointer is NULL                                      */
  FM_ERR_SHAPE = 2,       /* a size is out of range (B, H, nq, nk < 1, nq or nk > 2^22, a tile
                             grid of 2^31 tiles or more, ...) */
  FM_ERR_DTYPE = 3,       /* unknown dtype code                                               */
  FM_ERR_UNSUPPORTED = 4, /* (dtype, d) pair not built                                        */
  FM_ERR_ALIGN = 5,       /* tensor pointer not 16-byte aligned, or vector not 4-byte aligned */
  FM_ERR_WORKSPACE = 6,   /* workspace smaller than the *_workspace_bytes value, or NULL      */
  FM_ERR_CHUNKS = 7,      /* chunk table not sorted / disjoint / non-empty / inside range     */
  FM_ERR_HIP = 8,         /* a HIP launch failed                                              */
  FM_ERR_VALUE = 9,       /* a scalar argument is invalid (scale not finite and positive)    */
  FM_ERR_SCRATCH = 10     /* the problem needs more workspace than a no-alloc call's fixed
                             scratch array holds                                             */
} fm_status;

typedef enum { FM_BF16 = 0, FM_FP32 = 1 } fm_dtype;

typedef struct {
  int32_t B, H, nq, nk, d;
  int32_t dtype; /* fm_dtype */
} fm_shape;

/* Human-readable name of a status code (static string, never NULL). */
const char* flashmask_strerror(int32_t status);

/*
 * Tile shape used by the attention kernels for (dtype, d): the forward runs BM_fwd query rows
 * against BN_fwd key columns per tile, the backward BM_bwd x BN_bwd.  These are the tile shapes
 * at which tiles are classified (see flashmask_classify); for nq >= 65536, or where the
 * backward's BM_bwd x BN_bwd grid would hold 2^31 tiles or more, its key blocks are 2 * BN_bwd
 * wide instead (another shape of the dK/dV kernel).  Returns FM_ERR_DTYPE / FM_ERR_UNSUPPORTED /
 * FM_ERR_NULL, or FM_OK.
 */
int32_t flashmask_tile_sizes(int32_t dtype, int32_t d, int32_t* BM_fwd, int32_t* BN_fwd,
                             int32_t* BM_bwd, int32_t* BN_bwd);

/*
 * Forward attention.  "FlashMask-3: Efficient and Expressive Mask-Aware Distributed
 * Attention", abstract (mask-aware kernel); "FlashMask-3 sends each GPU its mask ...",
 * tile-classification paragraph (fully masked tiles never loaded, the row test only in partly
 * masked tiles).
 *
 * For every batch b, head h and query row i:
 *   S_ij = scale * Q_i . K_j over unmasked j;  LSE_i = ln sum_j exp(S_ij);
 *   O_i = sum_j exp(S_ij - LSE_i) V_j.
 * A row with every key masked gets O_i = 0 and LSE_i = -inf.
 * scale: finite and > 0 (else FM_ERR_VALUE).
 * Q [B,H,nq,d], K/V [B,H,nk,d] in `dtype`; O [B,H,nq,d] in `dtype`; LSE float32 [B,H,nq].
 * Sizes: 1 <= nq, nk <= 2^22, and the tile grid ceil(nq/BM) x ceil(nk/BN) at both tile shapes
 * (flashmask_tile_sizes) below 2^31 tiles, so nq = nk = 2^22 - 128 is the longest square case.
 * ws: device workspace of at least flashmask_fwd_workspace_bytes(shape) bytes (256-byte
 * aligned), clobbered by the call; it holds a dense [n_qb][n_kb] list array (8.6 GB at the
 * longest case, 8 MiB at nq = nk = 131072).
 */
size_t flashmask_fwd_workspace_bytes(const fm_shape* shape);
int32_t flashmask_fwd(const fm_shape* shape, const void* Q, const void* K, const void* V,
                      const int32_t* LTS, const int32_t* LTE, const int32_t* UTS,
                      const int32_t* UTE, float scale, void* O, float* LSE, void* ws,
                      size_t ws_bytes, void* stream);

/*
 * Backward attention: the exact gradient of L = sum(O * dO) with P recomputed from the saved
 * LSE.  The pages report forward and backward speed ("FlashMask-3 ..." zicq.com summary,
 * end-to-end paragraph) without describing the backward; this is the standard recompute form:
 *   P = exp(S - LSE) (0 where masked), dP = dO V^T, D_i = sum_d dO_id O_id,
 *   dS = P * (dP - D), dV = P^T dO, dK = scale dS^T Q, dQ = scale dS K.
 * O and LSE are the forward's outputs.  Rows with LSE = -inf contribute nothing; their dQ is 0.
 * dQ [B,H,nq,d], dK/dV [B,H,nk,d] in `dtype`, overwritten.  dK and dV come from a kernel that
 * holds a key block and walks its query blocks, dQ from one that holds a query block and walks
 * its key blocks (both skip fully masked tiles); no atomics are used and all three results are
 * deterministic.
 * ws: device workspace of at least flashmask_bwd_workspace_bytes(shape) bytes (256-byte
 * aligned slabs: tile lists at both tile shapes, and float32 D and LSE*log2(e) per row).
 */
size_t flashmask_bwd_workspace_bytes(const fm_shape* shape);
int32_t flashmask_bwd(const fm_shape* shape, const void* Q, const void* K, const void* V,
                      const void* O, const void* dO, const float* LSE, const int32_t* LTS,
                      const int32_t* LTE, const int32_t* UTS, const int32_t* UTE, float scale,
                      void* dQ, void* dK, void* dV, void* ws, size_t ws_bytes, void* stream);

/*
 * Interface variants of the two attention calls: strided tensors, grouped key/value heads and
 * per-batch or per-head mask vectors.  The pages do not describe these; they are the usual
 * interface of attention libraries and change no arithmetic: every output equals what the
 * calls above return on the same per-(batch, head) data.
 *
 * fm_layout:
 *   B, H, nq, nk, d, dtype  as in fm_shape; H_kv key/value heads (1 <= H_kv, H % H_kv == 0):
 *                           query head h reads key/value head h / (H / H_kv).
 *   q_stride[3]             element strides (batch, head, row) of Q, O, dQ and dO; the d axis is
 *                           contiguous.  Contiguous [B][H][nq][d] is {H*nq*d, nq*d, d}.
 *   kv_stride[3]            the same for K, V, dK and dV ([B][H_kv][nk][d] when contiguous).
 *   mask_b, mask_h          the four vectors hold mask_b * mask_h sets of nk int32 each
 *                           (set s at offset s*nk); batch b, head h uses set
 *                           (mask_b > 1 ? b : 0) * mask_h + (mask_h > 1 ? h : 0).
 *                           mask_b is 1 or B, mask_h is 1 or H.
 * Requirements (FM_ERR_SHAPE unless noted): strides >= 0, row strides >= d, every row
 * start 16-byte aligned (stride * element size a multiple of 16, FM_ERR_ALIGN); no two
 * (batch, head, row) positions of one layout share memory (sorted by stride, every axis with
 * more than one entry steps over the span of the smaller axes, so a zero batch or head stride
 * is rejected when B or H is above 1: outputs are written through these strides); per batch
 * and head the rows, counted up to the next multiple of 128 (the kernels address whole tiles),
 * span less than 4 GiB: (ceil(nq/128)*128 - 1)*q_stride[2] + d elements (and for the backward
 * also (H/H_kv - 1)*q_stride[1] more, with H/H_kv <= 256), (ceil(nk/128)*128 - 1)*kv_stride[2]
 * + d elements.  Distinct tensors must not overlap each other (not checked).  LSE stays
 * contiguous float32 [B][H][nq].  In the backward dK and dV of a key/value head sum the
 * gradients of its H/H_kv query heads, still without atomics and deterministic.
 * Workspaces grow with the number of mask sets (lists per set).
 */
typedef struct {
  int32_t B, H, H_kv, nq, nk, d;
  int32_t dtype; /* fm_dtype */
  int32_t mask_b, mask_h;
  int64_t q_stride[3];
  int64_t kv_stride[3];
} fm_layout;

size_t flashmask_fwd_ex_workspace_bytes(const fm_layout* layout);
int32_t flashmask_fwd_ex(const fm_layout* layout, const void* Q, const void* K, const void* V,
                         const int32_t* LTS, const int32_t* LTE, const int32_t* UTS,
                         const int32_t* UTE, float scale, void* O, float* LSE, void* ws,
                         size_t ws_bytes, void* stream);
size_t flashmask_bwd_ex_workspace_bytes(const fm_layout* layout);
int32_t flashmask_bwd_ex(const fm_layout* layout, const void* Q, const void* K, const void* V,
                         const void* O, const void* dO, const float* LSE, const int32_t* LTS,
                         const int32_t* LTE, const int32_t* UTS, const int32_t* UTE, float scale,
                         void* dQ, void* dK, void* dV, void* ws, size_t ws_bytes, void* stream);

/*
 * Rank-local vectors by clip-shift-max.  "FlashMask-3: Efficient and Expressive Mask-Aware
 * Distributed Attention", abstract (zero-communication mask localisation); "FlashMask-3 sends
 * each GPU its mask ...", clip-shift-max paragraph (with Theorem 1).
 *
 * The rank owns query-row chunks [chunk_start[k], chunk_start[k] + chunk_len[k]) for
 * k < n_chunks (host arrays; ascending, disjoint, non-empty, inside [0, nq_global];
 * 1 <= n_chunks <= 64), numbered locally by concatenation.  For every entry x of each global
 * vector (int32[n], device):
 *   local(x) = max(0, max_k( min(x, o_k + L_k) - o_k + P_k )),  P_k = L_0 + ... + L_{k-1},
 * i.e. the number of owned rows below x.  Keys are not renumbered.  Outputs are int32[n]
 * (device) with values in [0, n_local]; *n_local (host) receives sum_k L_k.  Input and output
 * vectors may not overlap.
 */
int32_t flashmask_localize(const int32_t* LTS_g, const int32_t* LTE_g, const int32_t* UTS_g,
                           const int32_t* UTE_g, int32_t n, int32_t nq_global,
                           const int32_t* chunk_start, const int32_t* chunk_len,
                           int32_t n_chunks, int32_t* LTS_l, int32_t* LTE_l, int32_t* UTS_l,
                           int32_t* UTE_l, int32_t* n_local, void* stream);

/*
 * Tile classification and list compaction at an arbitrary tile shape (BM query rows x BN key
 * columns, both >= 1), the same kernels the attention calls run internally.  "FlashMask-3
 * sends each GPU its mask ...", tile-classification paragraph.
 *
 * With r0 = qb*BM, r1 = min(r0 + BM, nq) and the per-key-block minimum (lo) and maximum (hi) of
 * each vector over keys [kb*BN, min((kb+1)*BN, nk)):
 *   full(S,E) = hi(S) <= r0 && lo(E) >= r1;   none(S,E) = hi(E) <= r0 || lo(S) >= r1
 *   cls = 0 if full(LT) || full(UT);  2 if none(LT) && none(UT);  1 otherwise.
 * Outputs (device; any may be NULL to skip it):
 *   cls   uint8 [n_qb][n_kb]
 *   qcnt  int32 [n_qb],  qlist int32 [n_qb][n_kb]: tiles of class != 0 in ascending kb,
 *         entry = kb*2 + (cls == 1); entries past qcnt[qb] are unspecified.
 *   kcnt  int32 [n_kb],  klist int32 [n_kb][n_qb]: the same per key block over qb.
 * n_qb = ceil(nq/BM), n_kb = ceil(nk/BN); n_qb * n_kb must be below 2^31.
 * ws: at least flashmask_classify_workspace_bytes(nk, BN) bytes.
 */
size_t flashmask_classify_workspace_bytes(int32_t nk, int32_t BN);
int32_t flashmask_classify(const int32_t* LTS, const int32_t* LTE, const int32_t* UTS,
                           const int32_t* UTE, int32_t nq, int32_t nk, int32_t BM, int32_t BN,
                           uint8_t* cls, int32_t* qcnt, int32_t* qlist, int32_t* kcnt,
                           int32_t* klist, void* ws, size_t ws_bytes, void* stream);

/*
 * Key/value chunk prune list for a context-parallel rank: the decision half of mask-driven
 * communication pruning.  "FlashMask-3 sends each GPU its mask ..." (learnaivisually.com),
 * across-ranks paragraph: the forward all-gather skips key-value chunks that are fully masked;
 * "FlashMask-3: Efficient and Expressive Mask-Aware Distributed Attention", abstract.
 * Inputs: the rank's localised vectors (flashmask_localize; device int32 [nk], values in local
 * row numbering, indexed by global key), n_local local rows, query blocks of BM local rows and
 * key chunks of `chunk` keys (the unit the all-gather moves).
 * Output live (device int32 [ceil(nk/chunk)], overwritten): for chunk c, the number of BM-row
 * blocks whose tile in column c is not fully masked under the min/max classification rule of
 * flashmask_classify; 0 means the rank never needs chunk c.  With BM equal to the rank's chunk
 * length each query block is one contiguous run of global rows and the rule is exact for the
 * causal, document and sliding-window families.
 * ws: at least flashmask_prune_workspace_bytes(nk, n_local, BM, chunk) device bytes, 4-byte
 * aligned (block min/max and the column lists).  Deterministic.  Errors: FM_ERR_NULL,
 * FM_ERR_SHAPE (a size < 1, or too many tiles), FM_ERR_ALIGN, FM_ERR_WORKSPACE, FM_ERR_HIP.
 */
size_t flashmask_prune_workspace_bytes(int32_t nk, int32_t n_local, int32_t BM, int32_t chunk);
int32_t flashmask_prune_chunks(const int32_t* LTS, const int32_t* LTE, const int32_t* UTS,
                               const int32_t* UTE, int32_t nk, int32_t n_local, int32_t BM,
                               int32_t chunk, int32_t* live, void* ws, size_t ws_bytes,
                               void* stream);

/*
 * Work order of the attention kernels (a scheduling aid; exposed for testing).  Writes to
 * order[0..n) a permutation of 0..n-1: blocks i go into four buckets by
 * floor(max(cnt[i], 0) * 4 / (max_k cnt[k] + 1)), the bucket of the largest counts first, and
 * inside a bucket in descending i.  The forward and both backward kernels take their blocks in
 * this order (cnt = their list lengths): long blocks start early, and blocks that run together
 * stay close in the sequence, so they share K / V tiles in cache.  The order changes no result.
 * "FlashMask-3 ..." (zicq.com summary) names load balance across ranks as a goal; this is its
 * counterpart inside one GPU.
 * cnt, order: device int32 [n], 4-byte aligned.  Errors: FM_ERR_NULL, FM_ERR_SHAPE (n < 1),
 * FM_ERR_ALIGN, FM_ERR_HIP.
 */
int32_t flashmask_block_order(const int32_t* cnt, int32_t n, int32_t* order, void* stream);

/*
 * Forward attention that allocates nothing and takes no workspace, for callers that cannot
 * allocate device memory (code under HIP graph capture, tight serving loops, harnesses that
 * forbid hipMalloc).  Same arguments, kernels and results as flashmask_fwd without ws/ws_bytes:
 * the workspace is a fixed device array inside the library of
 * flashmask_fwd_noalloc_max_workspace_bytes() = 16 MiB per GPU (held until the process ends;
 * its device address is looked up once per device, on the first call made with that device
 * current).  A problem whose flashmask_fwd_workspace_bytes exceeds it returns FM_ERR_SCRATCH
 * before any device work (one mask set at nq = nk = 131072 needs 8.1 MiB).  Every call on a GPU
 * shares that GPU's array: calls that overlap in time on one GPU (other streams, other
 * threads) race and must not be made.  No hipMalloc, hipFree or allocating library routine is
 * called.
 */
size_t flashmask_fwd_noalloc_max_workspace_bytes(void);
int32_t flashmask_fwd_noalloc(const fm_shape* shape, const void* Q, const void* K, const void* V,
                              const int32_t* LTS, const int32_t* LTE, const int32_t* UTS,
                              const int32_t* UTE, float scale, void* O, float* LSE, void* stream);

/*
 * Diagnostic hook for timing the attention kernels alone (a benchmark aid; not needed to use the
 * library).  After this call, flashmask_fwd records fwd_begin / fwd_end and flashmask_bwd
 * records bwd_begin / bwd_end (hipEvent_t passed as void*, created by the caller) on the call's
 * stream immediately before and after its attention kernels (for the backward: before the dQ
 * kernel and after the dK/dV kernel, which runs second).  NULL disables a pair.  The events
 * are kept per calling thread (thread-local): they apply only to later calls from the same
 * thread, so other threads' calls never record into them.  This is the library's only state.
 */
int32_t flashmask_set_profile_events(void* fwd_begin, void* fwd_end, void* bwd_begin,
                                     void* bwd_end);

#ifdef __cplusplus
}
#endif

#endif /* FLASHMASK_H */
