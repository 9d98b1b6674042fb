// Mask-aware attention backward for gfx950: the dK / dV kernel.
//
// The pages report the backward's speed ("FlashMask-3 ..." zicq.com summary, end-to-end
// paragraph) but do not describe it; this is the standard recompute-from-LSE backward restricted
// to the tiles the classification lists (fully masked tiles skipped, the row test only in
// partly masked tiles, as the forward; "FlashMask-3 sends each GPU its mask ...",
// tile-classification paragraph).
//
//   K5 dK / dV:  one workgroup of 4 waves per block of BN = 64 keys (two workgroups per CU;
//                queries of 65536 rows or more use 8 waves per 128 keys, one workgroup per CU):
//                key groups of 32 keys, and per key group a pair of waves that split the work:
//                  the P wave keeps K rows in registers, computes S = Q K^T, P = exp2(S*scale*
//                  log2e - LSE*log2e) (0 where masked) and accumulates dV^T += dO^T P;
//                  the dS wave keeps V rows, computes dP = dO V^T, takes P from the P wave
//                  through LDS, forms dS = P (dP - D) and accumulates dK^T += Q^T dS.
//                Each wave then needs under 256 registers, so two run on every SIMD and one's
//                elementwise work overlaps the other's matrix products (in the 4-wave shape the
//                two waves of a SIMD belong to the two workgroups on the CU, and which SIMD gets
//                which wave varies between workgroups, so their roles mix; in the 8-wave shape
//                waves w and w + 4, the P and dS waves of key group w, share a SIMD).  The
//                workgroup walks the query blocks (BM = 64 rows) of its list in 32-row units;
//                Q and dO rows are A operands read from LDS in a permuted row order so the
//                accumulators double as operands, Q^T and dO^T come from the gfx950 LDS
//                transpose read.
//                Q/dO tiles go from HBM straight into two LDS buffers (three in the 8-wave
//                shape), each requested while the one before it (the two before it) compute;
//                one workgroup barrier per unit (P handed over) also publishes the next tile,
//                and these barriers wait only for LDS traffic, not for loads in flight.
//   dQ comes from the query-stationary kernel in attn_bwd_dq.hip, so no float32 atomics are
//   needed and every gradient is deterministic.
#include <math.h>

#include <type_traits>

#include "fm_common.hpp"
#include "launch.hpp"

namespace fm {

FM_STAMP_ARRAY(g_stamps_dkdv, flashmask_debug_stamps_dkdv)

namespace {

// Two shapes of the kernel (NG key groups of 32 keys, a P wave and a dS wave each; NBUF tile
// buffers):
//   NG = 2, NBUF = 2: 4 waves per 64-key block, two workgroups per CU, which run independently of
//     each other, and finer column lists (64-key blocks skip more fully masked tiles);
//   NG = 4, NBUF = 3: 8 waves per 128-key block, one workgroup per CU, each tile requested two
//     tiles ahead: better where Q and dO no longer stay in the caches (long sequences), since
//     each workgroup of the first shape loads the same Q/dO tiles for half as many keys.
template <typename T, int D, int NG_, int NBUF_>
struct BwdTile {
  static constexpr int NG = NG_, NBUF = NBUF_;
  static constexpr int BN = 32 * NG, BM = 64, NT = 128 * NG;
  static constexpr int BPW = 16 / NG, SPW = 4 / NG;  // per wave and tile: 1-KiB blocks, row slots
  static constexpr int LPT = BPW + SPW;             // loads per wave and tile
  static constexpr int KPL = Elem<T>::KPL, KSTEP = 2 * KPL;
  static constexpr int CH = 16 / (int)sizeof(T);
  static constexpr int CPR = D / CH;  // 16-byte chunks per Q / dO / K row
  static constexpr int ROW_BYTES = D * (int)sizeof(T);
  static constexpr int NDB = D / 32;
  static constexpr int QK_STEPS = D / KSTEP;
  static constexpr int US = 32 / KSTEP;  // k-steps over a unit's 32 queries
  static constexpr int TILE_BYTES = BM * ROW_BYTES;
  // Q | dO | rows: LSE2 and D of the tile's rows in 8 slots of 64 floats, wave w filling slots
  // SPW*w .. SPW*w + SPW - 1 (16 rows in a slot's first 16 floats; LSE2 in slots 0-3, D in 4-7)
  static constexpr int ROWS_BYTES = 8 * 64 * (int)sizeof(float);
  static constexpr int BUF_BYTES = 2 * TILE_BYTES + ROWS_BYTES;
  // one unit's P as operand fragments (US per lane), 4 groups
  static constexpr int XCH_BYTES = NG * US * 64 * KPL * (int)sizeof(T);
  static_assert(CPR == 16, "tile loads assume 256-byte rows");
  static_assert(TILE_BYTES == 16 * 1024, "16 blocks of 1 KiB per tile");
};

struct MaskRegs {
  int32_t lts, lte, uts, ute;
};

// GQ: more than one query head per key/value head (a.L.G > 1); the G = 1 instantiation walks a
// single list and needs no guard for rows past nq.
template <typename T, int D, bool GQ, int NG, int NBUF>
__global__ __launch_bounds__(128 * NG, sizeof(T) == 2 ? 4 / NG : 1) void attn_bwd_kernel(BwdArgs a) {
  using C = BwdTile<T, D, NG, NBUF>;
  using E = Elem<T>;
  using frag = typename E::frag;
  constexpr int KPL = C::KPL, KSTEP = C::KSTEP, US = C::US;

  // NBUF tile buffers, Q|dO|LSE2|D each, as separate arrays: the compiler then sees that the
  // loads straight into one buffer never alias reads of another and adds no waits for them.
  // (Two workgroups of the 4-wave shape, 76 KiB each, fit in a CU's LDS.)
  __shared__ __attribute__((aligned(16))) unsigned char lds0[C::BUF_BYTES];
  __shared__ __attribute__((aligned(16))) unsigned char lds1[C::BUF_BYTES];
  __shared__ __attribute__((aligned(16))) unsigned char lds2[NBUF > 2 ? C::BUF_BYTES : 16];
  __shared__ __attribute__((aligned(16))) unsigned char xch[2 * C::XCH_BYTES];  // P of two units
  auto bufp = [&](auto bc) -> unsigned char* {
    constexpr int bi = decltype(bc)::value;
    if constexpr (bi == 0)
      return lds0;
    else if constexpr (bi == 1)
      return lds1;
    else
      return lds2;
  };
  using I0 = std::integral_constant<int, 0>;
  using I1 = std::integral_constant<int, 1>;
  using I2 = std::integral_constant<int, 2>;

  WgStamps stamps;  // workgroup timeline (debug build only)
  const int tid = threadIdx.x;
  const int lane = tid & 63, g = lane >> 5, l32 = lane & 31;
  const int wv = __builtin_amdgcn_readfirstlane(tid >> 6);  // wave index (uniform)
  const int kg = wv % C::NG;                                 // key group
  const bool dsw = wv >= C::NG;                              // the dS wave of the pair

  // The workgroup owns key block kb (BN keys) of key/value head hk of batch b; with G query heads
  // per key/value head it walks the tile lists of all G heads in turn, accumulating into the
  // same dK and dV registers (no atomics).
  const int n_kb = (a.nk + C::BN - 1) / C::BN;
  const int work = xcd_contiguous_index(blockIdx.x, gridDim.x);
  // (every index here is the same for the whole workgroup; readfirstlane keeps it in scalar
  // registers, and with it every pointer and buffer descriptor derived from it)
  const int G = GQ ? a.L.G : 1;
  const int Hk = a.L.H / G;
  const int bhk = __builtin_amdgcn_readfirstlane(work / n_kb);
  const int b = __builtin_amdgcn_readfirstlane(bhk / Hk);
  const int hk = bhk - b * Hk, h0 = hk * G;
  const int kb = __builtin_amdgcn_readfirstlane(a.order[(size_t)mask_set(a.L, b, h0) * n_kb + work % n_kb]);
  const int key = kb * C::BN + kg * 32 + l32;  // this lane's key (a column of S)
  const bool key_ok = key < a.nk;
  const int64_t kbase = b * a.L.ks_b + hk * a.L.ks_h;
  int total = 0;
  for (int gi = 0; gi < G; ++gi) total += a.kcnt[(size_t)mask_set(a.L, b, h0 + gi) * n_kb + kb];
  if (total == 0) {
    // No listed tile: every query row is masked for these keys, so dK = dV = 0.  Each lane
    // clears half of its key's row (128 bytes) in the tensor of its wave's role.
    if (key_ok) {
      T* row = static_cast<T*>(dsw ? a.dk : a.dv) + kbase + (size_t)key * a.L.ks_r;
      uint4* p = reinterpret_cast<uint4*>(row + g * (D / 2));
#pragma unroll
      for (int i = 0; i < 8; ++i) p[i] = make_uint4(0u, 0u, 0u, 0u);
    }
    stamps.store(FM_STAMP_BUF(g_stamps_dkdv), 0);
    return;
  }

  const T* __restrict__ Kp = static_cast<const T*>(a.k) + kbase;
  const T* __restrict__ Vp = static_cast<const T*>(a.v) + kbase;
  const uint32_t qrs = (uint32_t)a.L.qs_r * sizeof(T);  // row strides in bytes
  const uint32_t krs = (uint32_t)a.L.ks_r * sizeof(T);
  const buf_rsrc kvbuf = make_buf(dsw ? Vp : Kp, (uint32_t)(a.nk - 1) * krs + C::ROW_BYTES);

  // K (P wave) or V (dS wave) rows of this lane's key as B operands (k-step s: d = s*KSTEP +
  // g*KPL + 0..KPL); keys past nk read as zeros.
  frag bop[C::QK_STEPS];
#pragma unroll
  for (int s = 0; s < C::QK_STEPS; ++s) {
    const uint32_t off = (uint32_t)key * krs + (uint32_t)(s * KSTEP + g * KPL) * sizeof(T);
    if constexpr (KPL == 8)
      bop[s] = __builtin_bit_cast(frag, buf_load16(kvbuf, off, 0));
    else
      bop[s] = __builtin_bit_cast(frag, buf_load4(kvbuf, off, 0));
  }
  const bool ragged_block = (kb == n_kb - 1) && (a.nk % C::BN) != 0;

  // ---- per-lane LDS byte offsets, constant for the whole kernel ------------------------------
  // Transpose-read lane geometry: lane i of 16-lane block b addresses row k0 + 8*(b/2) + i/4,
  // column m0 + 16*(b%2) + 4*(i%4), and receives rows k0 + 8*(l/32) + 0..3 of column m0 + l%32.
  // The swizzle depends only on row & 15, so an offset computed for a row below 16 stays valid
  // when a multiple of 16 rows is added as a constant.
  const int tb = lane >> 4, ti = lane & 15;
  const int tr_row = 8 * (tb >> 1) + (ti >> 2);
  const int tr_col = 16 * (tb & 1) + 4 * (ti & 3);
  int off_s[C::QK_STEPS];  // row operand (query row source row, k-step s) of a unit
  int off_tq[C::NDB][2];   // transposed operand rows (tr_row, tr_row + 4), columns 32*db
  {
    const int srow = row_source<KPL>(l32);
#pragma unroll
    for (int st = 0; st < C::QK_STEPS; ++st)
      off_s[st] = tile_off<T, 0>(srow, st * KSTEP + g * KPL, C::ROW_BYTES);
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      const int r = KPL == 8 ? tr_row + 4 * h : g;
      const int cc = KPL == 8 ? tr_col : l32;
#pragma unroll
      for (int db = 0; db < C::NDB; ++db) off_tq[db][h] = tile_off<T, 0>(r, 32 * db + cc, C::ROW_BYTES);
    }
  }
  // The P wave reads Q rows and dO^T, the dS wave dO rows and Q^T.
  const int row_region = dsw ? C::TILE_BYTES : 0;
  const int tr_region = dsw ? 0 : C::TILE_BYTES;

  auto tr_operand = [&](const unsigned char* tile, const int* off, int k0_bytes) -> frag {
    if constexpr (KPL == 8) {
      const s16x4 lo = lds_read_tr16(tile + off[0] + k0_bytes);
      const s16x4 hi = lds_read_tr16(tile + off[1] + k0_bytes);
      return __builtin_bit_cast(frag, __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7));
    } else {
      return *reinterpret_cast<const T*>(tile + off[0] + k0_bytes);
    }
  };

  f32x16 acc[C::NDB];  // dV^T (P wave) or dK^T (dS wave): row d, column this lane's key
#pragma unroll
  for (int db = 0; db < C::NDB; ++db) acc[db] = f32x16{};

  const float cexp = a.scale * kLog2e;

  // The tiles of the G query heads of the group form one flat sequence: the list of head h0,
  // then of h0 + 1, and so on (total tiles in all).  Q, dO and the LSE2 / D rows of all G heads
  // lie in one buffer each, and a tile's head becomes part of its scalar offset.
  const int64_t qbase = b * a.L.qs_b + h0 * a.L.qs_h;
  const size_t rbase = ((size_t)b * a.L.H + h0) * a.nq;
  const uint32_t qhs = (uint32_t)a.L.qs_h * sizeof(T);  // bytes from one head to the next
  const uint32_t q_span = (uint32_t)(G - 1) * qhs + (uint32_t)(a.nq - 1) * qrs + C::ROW_BYTES;
  const buf_rsrc qbuf = make_buf(static_cast<const T*>(a.q) + qbase, q_span);
  const buf_rsrc dobuf = make_buf(static_cast<const T*>(a.dout) + qbase, q_span);
  const buf_rsrc lbuf = make_buf(a.lse2 + rbase, (uint32_t)G * a.nq * sizeof(float));
  const buf_rsrc dlbuf = make_buf(a.delta + rbase, (uint32_t)G * a.nq * sizeof(float));
  // Position in the flat sequence: head gi of the group, index i in its list of c entries.
  struct Cursor {
    int gi, i, c;
    const int32_t* l;
  };
  // Move u to the first head at or after u.gi whose list is not empty (u.gi = G past the end).
  auto head_list = [&](Cursor& u) {
    for (; u.gi < G; ++u.gi) {
      const int set = mask_set(a.L, b, h0 + u.gi);
      u.c = __builtin_amdgcn_readfirstlane(a.kcnt[(size_t)set * n_kb + kb]);
      u.l = a.klist + ((size_t)set * n_kb + kb) * a.list_stride;
      if (u.c > 0) return;
    }
  };
  auto advance = [&](Cursor& u) {
    if (++u.i == u.c && GQ) {
      u.i = 0;
      ++u.gi;
      if (u.gi < G) head_list(u);
    }
  };
  auto entry_of = [&](const Cursor& u) { return load_uniform(u.l, u.i); };
  // This lane's key's mask values for the tile's head; reloaded only when the head's mask set
  // changes (never with one set per batch).
  MaskRegs mk = {0, 0, 0, 0};  // past the last key every row is masked
  int mk_set = -1;
  auto load_mask = [&](int gi) {
    const int set = mask_set(a.L, b, h0 + gi);
    if (set == mk_set) return;
    mk_set = set;
    if (key_ok) {
      const int64_t o = set * a.L.mask_stride + key;
      mk = {a.mask.lts[o], a.mask.lte[o], a.mask.uts[o], a.mask.ute[o]};
    }
  };
  Cursor first{0, 0, 0, nullptr};
  head_list(first);
  load_mask(first.gi);
  // The K/V rows and the mask values are waited for before the walk, together with the first
  // tile's loads (issued below, so that the two requests overlap): the main loop keeps tile loads
  // in flight, and a wait the compiler would place there for a register loaded now would also
  // wait for those.

  // A tile's 64 rows of Q, then of dO, are 32 blocks of 1 KiB; wave w moves blocks
  // BPW*w .. BPW*w + BPW - 1 (the P waves Q, the dS waves dO), lane l the 16-byte slot l of a
  // block: row 4j + l/16 of its tensor, physical chunk l%16, which holds logical chunk
  // (l%16) ^ swz_row(row).  Rows past nq read as zeros.  Each wave also fills SPW row slots, 16
  // LSE2 (slots 0-3) or D (slots 4-7) values each, in lanes 0-15 (lanes 16-63 read out of range
  // and write zeros into the rest of the slot).  The loads go straight into LDS (no registers, no
  // LDS writes by the waves).
  // The buffers span all G heads, so rows past nq of one head are another head's rows: their
  // offsets are moved to the buffer's end, where loads return zeros (dO = 0 and D = 0 make such a
  // row contribute nothing).
  auto load_tile = [&](int gi, int entry, auto bc) {
    unsigned char* t = bufp(bc);
    const int q0 = (entry >> 1) * C::BM;
    const uint32_t tile_base = (uint32_t)gi * qhs + (uint32_t)q0 * qrs;
    const buf_rsrc src = wv < C::NG ? qbuf : dobuf;
#pragma unroll
    for (int i = 0; i < C::BPW; ++i) {
      const int row = 4 * ((C::BPW * wv + i) & 15) + (lane >> 4);
      const uint32_t voff = !GQ || q0 + row < a.nq
                                ? (uint32_t)row * qrs + (uint32_t)(((lane & 15) ^ swz_row<T>(row)) * 16)
                                : q_span - tile_base;
      buf_load_lds<16>(src, t + (C::BPW * wv + i) * 1024, voff, tile_base);
    }
#pragma unroll
    for (int i = 0; i < C::SPW; ++i) {
      const int slot = C::SPW * wv + i;
      const int r = 16 * (slot & 3) + lane;  // tile row of this lane (lanes below 16)
      const uint32_t roff = ((uint32_t)gi * a.nq + (uint32_t)q0) * sizeof(float);
      const uint32_t r_span = (uint32_t)G * a.nq * sizeof(float);
      const uint32_t loff = lane < 16 && (!GQ || q0 + r < a.nq) ? (uint32_t)r * sizeof(float) : r_span - roff;
      buf_load_lds<4>(slot < 4 ? lbuf : dlbuf, t + 2 * C::TILE_BYTES + slot * 64 * sizeof(float), loff, roff);
    }
  };
  // Every tile step issues exactly one tile's five loads (near the end of the walk a real tile is
  // loaded again into a buffer nothing reads any more), so one wait without a branch, vmcnt(5),
  // leaves only the newest tile's loads in flight; a wait under a branch would make the
  // compiler's own wait tracking assume the no-wait path and add vmcnt(0) before later reads.

  // Row mask of this lane's key over a tile's BM query rows starting at q0 (bit i = row q0 + i
  // masked), pre-shifted by g*KPL so that bit h*32 + perm_index(r, 0) belongs to register r of
  // unit h in this lane group.
  auto tile_row_mask = [&](int32_t q0) -> uint64_t {
    auto bits = [&](int32_t s0, int32_t e0) -> uint64_t {
      const int32_t lo = s0 <= q0 ? 0 : (s0 >= q0 + 64 ? 64 : s0 - q0);
      const int32_t hi = e0 <= q0 ? 0 : (e0 >= q0 + 64 ? 64 : e0 - q0);
      if (hi <= lo) return 0ull;
      const uint64_t upto_hi = hi >= 64 ? ~0ull : ((1ull << hi) - 1ull);
      return upto_hi & ~((1ull << lo) - 1ull);  // lo < 64 here
    };
    const uint64_t m = key_ok ? (bits(mk.lts, mk.lte) | bits(mk.uts, mk.ute)) : ~0ull;
    return m >> (g * KPL);
  };

  // ---- one 32-query unit ----------------------------------------------------------------------
  // P of unit parity h in LDS as the P wave's operand fragments (bf16 in the bf16 kernel, so
  // the hand-over moves half the bytes of float32): [h][group][k-step u][lane], each lane's
  // fragment contiguous.
  // Row operands (Q for the P wave, dO for the dS wave) of unit h of the tile at qt.
  auto read_ops = [&](const unsigned char* qt, int h, frag* op) {
#pragma unroll
    for (int st = 0; st < C::QK_STEPS; ++st)
      op[st] = *reinterpret_cast<const frag*>(qt + row_region + off_s[st] + h * 32 * C::ROW_BYTES);
  };
  // Rows of a unit's LSE2 (P wave) or D (dS wave) for the 16 queries this lane holds: runs of
  // KPL consecutive rows h*32 + (r/KPL)*2*KPL + g*KPL + 0..KPL-1.
  auto read_rows = [&](const unsigned char* qt, int h, float* rv) {
    // row q of the tile is float (q / 16) * 64 + q % 16 of the LSE2 or D half of the slots
    const float* rows = reinterpret_cast<const float*>(qt + 2 * C::TILE_BYTES) + (dsw ? 4 * 64 : 0);
    if constexpr (KPL == 8) {
#pragma unroll
      for (int j = 0; j < 2; ++j) {
        const float4 x0 = *reinterpret_cast<const float4*>(rows + (2 * h + j) * 64 + 8 * g);
        const float4 x1 = *reinterpret_cast<const float4*>(rows + (2 * h + j) * 64 + 8 * g + 4);
        rv[8 * j + 0] = x0.x; rv[8 * j + 1] = x0.y; rv[8 * j + 2] = x0.z; rv[8 * j + 3] = x0.w;
        rv[8 * j + 4] = x1.x; rv[8 * j + 5] = x1.y; rv[8 * j + 6] = x1.z; rv[8 * j + 7] = x1.w;
      }
    } else {
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int q = h * 32 + perm_index<KPL>(r, g);
        rv[r] = rows[(q >> 4) * 64 + (q & 15)];
      }
    }
  };
  // operand fragments of P or dS: k-step u covers queries h*32 + u*KSTEP + g*KPL + e =
  // registers u*KPL + e
  auto to_frags = [&](const float* pv, frag* fr) {
#pragma unroll
    for (int u = 0; u < US; ++u) {
      if constexpr (KPL == 1) {
        fr[u] = pv[u];
      } else {
#pragma unroll
        for (int e = 0; e < KPL; ++e) fr[u][e] = E::from_float(pv[u * KPL + e]);
      }
    }
  };
  auto xfrag = [&](int h, int u) -> frag* {
    return reinterpret_cast<frag*>(xch) + ((h * C::NG + kg) * US + u) * 64 + lane;
  };
  // dS = P (dP - D) of a unit, from its P fragments in exchange slot h; dp holds dP - D.
  auto ds_frags = [&](int h, const f32x16& dp, frag* fr) {
    float pv[16];
#pragma unroll
    for (int u = 0; u < US; ++u) {
      const frag f = *xfrag(h, u);
      if constexpr (KPL == 1) {
        pv[u] = f * dp[u];
      } else {
#pragma unroll
        for (int e = 0; e < KPL; ++e) pv[u * KPL + e] = (float)f[e] * dp[u * KPL + e];
      }
    }
    to_frags(pv, fr);
  };
  // dV^T += dO^T P or dK^T += Q^T dS over the 32 queries of unit h of the tile at qt.
  auto accumulate = [&](const unsigned char* qt, int h, const frag* fr) {
#pragma unroll
    for (int u = 0; u < US; ++u)
#pragma unroll
      for (int db = 0; db < C::NDB; ++db)
        acc[db] = E::mfma(tr_operand(qt + tr_region, off_tq[db], (h * 32 + u * KSTEP) * C::ROW_BYTES),
                          fr[u], acc[db]);
  };

  // One step per 32-query unit, one workgroup barrier per step (publish).  The dS wave runs one
  // unit behind the P wave, so that between two barriers both waves of a pair have their matrix
  // products and their vector work to interleave (neither waits for the other's products):
  //   P wave,  unit (qt, h):  S = Q K^T; P = exp2(S*scale*log2e - LSE2), 0 where masked; P to
  //                           exchange slot h; barrier; dV^T += dO^T P.
  //   dS wave:                the pending unit (qp, 1-h), whose P was published at the previous
  //                           barrier: dS = P (dP - D), dK^T += Q^T dS; then dP = dO V^T of unit
  //                           (qt, h), kept for the next step; barrier.
  // op holds the unit's row operands (read one unit ahead); after the barrier the next unit's
  // are read into it (from qn, half hn) when next is set.
  auto step = [&](auto role, const unsigned char* qt, auto hc, bool test, uint64_t mrow,
                  auto&& publish, frag* op, f32x16& dp_prev, bool next, const unsigned char* qn,
                  int hn, const unsigned char* qp, bool pending) {
    constexpr int h = decltype(hc)::value;
    constexpr bool DS = decltype(role)::value;
    if constexpr (!DS) {
      // S = Q K^T: register r of group g is query h*32 + perm_index(r, g) of the tile; the
      // column is this lane's key.
      f32x16 sacc = {};
#pragma unroll
      for (int st = 0; st < C::QK_STEPS; ++st) sacc = E::mfma(op[st], bop[st], sacc);
      float rv[16], pv[16];
      read_rows(qt, h, rv);
#pragma unroll
      for (int r = 0; r < 16; ++r) pv[r] = fast_exp2(fmaf(sacc[r], cexp, -rv[r]));
      if (test) {
        const uint32_t mw = (uint32_t)(mrow >> (32 * h));
#pragma unroll
        for (int r = 0; r < 16; ++r) pv[r] = select_bit(mw, perm_index<KPL>(r, 0), pv[r], 0u);
      }
      frag fr[US];
      to_frags(pv, fr);
#pragma unroll
      for (int u = 0; u < US; ++u) *xfrag(h, u) = fr[u];
      publish();  // workgroup barrier: P of this unit (and possibly the next tile) visible
      if (next) read_ops(qn, hn, op);
      accumulate(qt, h, fr);
    } else {
      if (pending) {
        // dS = P (dP - D) of the pending unit (the other half: slot 1 - h); dp_prev already
        // holds dP - D
        frag fr[US];
        ds_frags(1 - h, dp_prev, fr);
        accumulate(qp, 1 - h, fr);
      }
      // dP - D = dO V^T - D of this unit: the products accumulate onto the rows' -D values
      // (the dQ kernel stores -D), which saves the subtraction per element
      float rv[16];
      read_rows(qt, h, rv);
      f32x16 pacc;
#pragma unroll
      for (int r = 0; r < 16; ++r) pacc[r] = rv[r];
#pragma unroll
      for (int st = 0; st < C::QK_STEPS; ++st) pacc = E::mfma(op[st], bop[st], pacc);
      dp_prev = pacc;
      publish();
      if (next) read_ops(qn, hn, op);
    }
  };

  // ---- the walk over the key block's query tiles ---------------------------------------------
  // Tile t sits in buffer t % NBUF.  Right after the barrier of tile t's first unit, the loads
  // of tile t+NBUF-1 into the buffer tile t-1 used are issued (after that barrier no wave reads
  // tile t-1: the dS wave finished its lagging unit of tile t-1 before it); before the barrier of
  // tile t's second unit each wave waits until only the loads of tiles after t+1 are in flight,
  // and that barrier publishes tile t+1.  A load so has 2*NBUF - 3 units to land (with two
  // buffers the other workgroup on the CU covers the wait).  With three buffers every tile step
  // issues exactly one tile's LPT loads (near the end a real tile is loaded again into a buffer
  // nothing reads), so the wait needs no branch; a wait under a branch would make the compiler's
  // own tracking assume the no-wait path and add vmcnt(0) before later reads.
  // The walk is written out once per role (same barriers in the same order), so that neither
  // role's loop carries the other's registers.
  using H0 = std::integral_constant<int, 0>;
  using H1 = std::integral_constant<int, 1>;
  {
    load_tile(first.gi, entry_of(first), I0{});
    if constexpr (NBUF == 3) {
      Cursor second = first;
      if (total > 1) advance(second);
      load_tile(second.gi, entry_of(second), I1{});  // tile 1, or tile 0 again (never read)
      wait_vmem_n<C::LPT>();  // the rows, the mask values and tile 0 have landed
    } else {
      wait_vmem();
    }
    lds_barrier();
    stamps.first_tile();
  }
  f32x16 dp_prev = {};  // dS wave: dP of the pending unit
  auto walk = [&](auto role) {
    Cursor cur = first;    // the tile being walked
    Cursor ahead = first;  // the tile NBUF-1 ahead, loaded during this one
    advance(ahead);
    if (NBUF == 3 && total > 1) advance(ahead);
    int entry = entry_of(cur);
    frag op[C::QK_STEPS];
    read_ops(bufp(I0{}), 0, op);
    // tile t in buffer bc = t % NBUF (a compile-time constant, so LDS offsets fold into the
    // instructions); tile t+1 is in buffer (bc+1) % NBUF, tile t-1 was in (bc+NBUF-1) % NBUF
    auto tile = [&](const int t, auto bc) {
      constexpr int bi = decltype(bc)::value;
      using BNext = std::integral_constant<int, (bi + 1) % NBUF>;
      using BPrev = std::integral_constant<int, (bi + NBUF - 1) % NBUF>;
      const bool test = (entry & 1) || ragged_block;
      uint64_t mrow = 0ull;  // the row test belongs to the P wave only
      if constexpr (!decltype(role)::value) {
        if (test) {
          load_mask(cur.gi);
          mrow = tile_row_mask((entry >> 1) * C::BM);
        }
      }
      const unsigned char* qt = bufp(bc);
      const bool more = t + 1 < total;
      const bool more_a = t + NBUF - 1 < total;  // the tile NBUF-1 ahead exists
      step(role, qt, H0{}, test, mrow, [&] {
        lds_barrier();
        if constexpr (NBUF == 3) {
          load_tile(more_a ? ahead.gi : cur.gi, more_a ? entry_of(ahead) : entry, BPrev{});
          if (more_a) advance(ahead);
        } else if (more_a) {
          load_tile(ahead.gi, entry_of(ahead), BPrev{});
          advance(ahead);
        }
      }, op, dp_prev, true, qt, 1, bufp(BPrev{}), t > 0);
      step(role, qt, H1{}, test, mrow, [&] {
        // this wave's part of tile t+1 has landed ...
        if constexpr (NBUF == 3)
          wait_vmem_n<C::LPT>();
        else
          wait_vmem();
        lds_barrier();  // ... and everyone's
      }, op, dp_prev, more, bufp(BNext{}), 0, qt, true);
      if (more) {
        advance(cur);
        entry = entry_of(cur);
      }
    };
    int t = 0;
    if constexpr (NBUF == 3) {
      for (; t + 2 < total; t += 3) {
        tile(t, I0{});
        tile(t + 1, I1{});
        tile(t + 2, I2{});
      }
      if (t < total) tile(t, I0{});
      if (t + 1 < total) tile(t + 1, I1{});
    } else {
      for (; t + 1 < total; t += 2) {
        tile(t, I0{});
        tile(t + 1, I1{});
      }
      if (t < total) tile(t, I0{});
    }
  };
  if (dsw)
    walk(std::true_type{});
  else
    walk(std::false_type{});
  stamps.walk_done();
  // The last two tile steps loaded a tile again into a free buffer; those loads must land before
  // the workgroup ends and its LDS is handed to another.
  wait_vmem();
  // the dS wave's last pending unit: the second half of the last tile
  if (dsw) {
    const int lb = (total - 1) % NBUF;
    const unsigned char* ql = lb == 0 ? lds0 : (lb == 1 ? lds1 : lds2);
    frag fr[US];
    ds_frags(1, dp_prev, fr);
    accumulate(ql, 1, fr);
  }

  if (key_ok) {
    T* dst = static_cast<T*>(dsw ? a.dk : a.dv) + kbase + (size_t)key * a.L.ks_r;
    const float sc = dsw ? a.scale : 1.0f;
#pragma unroll
    for (int db = 0; db < C::NDB; ++db)
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int d0 = db * 32 + 8 * i + 4 * g;
        if constexpr (sizeof(T) == 2) {
          uint2 out;
          out.x = pack_bf16x2(acc[db][4 * i + 0] * sc, acc[db][4 * i + 1] * sc);
          out.y = pack_bf16x2(acc[db][4 * i + 2] * sc, acc[db][4 * i + 3] * sc);
          *reinterpret_cast<uint2*>(dst + d0) = out;
        } else {
          *reinterpret_cast<float4*>(dst + d0) =
              make_float4(acc[db][4 * i + 0] * sc, acc[db][4 * i + 1] * sc, acc[db][4 * i + 2] * sc,
                          acc[db][4 * i + 3] * sc);
        }
      }
  }
  stamps.store(FM_STAMP_BUF(g_stamps_dkdv), total);
}

template <typename T, int D, int NG, int NBUF>
hipError_t run_shape(const BwdArgs& a, hipStream_t stream, hipEvent_t ev_end) {
  using C = BwdTile<T, D, NG, NBUF>;
  auto kernel = a.L.G > 1 ? &attn_bwd_kernel<T, D, true, NG, NBUF> : &attn_bwd_kernel<T, D, false, NG, NBUF>;
  const int64_t n_kb = (a.nk + C::BN - 1) / C::BN;
  const int64_t grid = n_kb * a.L.B * (a.L.H / a.L.G);
  hipLaunchKernelGGL(kernel, dim3((unsigned)grid), dim3(C::NT), 0, stream, a);
  hipError_t err = hipGetLastError();
  if (ev_end) (void)hipEventRecord(ev_end, stream);
  return err;
}

// The shape follows the width of the column lists' key blocks.
template <typename T, int D>
hipError_t run_bwd(const BwdArgs& a, hipStream_t stream, hipEvent_t ev_end) {
  if (a.list_bn == BwdTile<T, D, 2, 2>::BN) return run_shape<T, D, 2, 2>(a, stream, ev_end);
  if (a.list_bn == BwdTile<T, D, 4, 3>::BN) return run_shape<T, D, 4, 3>(a, stream, ev_end);
  return hipErrorInvalidValue;
}

}  // namespace

hipError_t launch_attn_bwd(int dtype, const BwdArgs& a, hipStream_t stream, hipEvent_t ev_end) {
  return dtype == 0 ? run_bwd<bf16, 128>(a, stream, ev_end) : run_bwd<float, 64>(a, stream, ev_end);
}

}  // namespace fm
