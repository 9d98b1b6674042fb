// Mask-aware attention backward for gfx950.
//
// The pages report the backward's speed ("FlashMask-3 ..." zicq.com summary, end-to-end
// paragraph) but do not describe it; this is the standard recompute-from-LSE backward restricted
// to the tiles the classification lists (fully masked tiles skipped, the row test only in
// partly masked tiles, as the forward; "FlashMask-3 sends each GPU its mask ...",
// tile-classification paragraph).
//
//   K4 bwd_pre:  D_i = sum_d dO_id O_id and LSE_i * log2(e) per query row.
//   K5 bwd_dkdv: one workgroup per key block of BN = 128 keys (4 waves x 32 keys).  K and V rows
//                of the wave's keys stay in registers (B operands of S = Q K^T and dP = dO V^T)
//                and dK^T, dV^T accumulate in registers.  The workgroup walks the query blocks
//                (BM = 64 rows) of its list.  Per tile: S, dP on 32x32 MFMAs with the query rows
//                loaded in a permuted order so the accumulators double as operands;
//                P = exp2(S*scale*log2e - LSE*log2e) (0 in masked entries); dS = P (dP - D);
//                dV^T += dO^T P and dK^T += Q^T dS with the transposed operands read from the
//                row-major Q / dO tiles by the gfx950 LDS transpose read.  Q / dO tiles go
//                straight from HBM into LDS, double-buffered, one workgroup barrier per tile.
//   dQ comes from the query-stationary kernel in attn_bwd_dq.hip, so no float32 atomics are
//   needed and every gradient is deterministic.
#include <math.h>

#include <type_traits>

#include "fm_common.hpp"
#include "launch.hpp"

namespace fm {

namespace {

template <typename T, int D>
struct BwdTile {
  static constexpr int BN = 128, BM = 64, NT = 256;
  static constexpr int KPL = Elem<T>::KPL, KSTEP = 2 * KPL;
  static constexpr int CH = 16 / (int)sizeof(T);
  static constexpr int CPR = D / CH;               // 16-byte chunks per Q / dO / K row
  static constexpr int ROW_BYTES = D * (int)sizeof(T);
  static constexpr int NDB = D / 32;
  static constexpr int QK_STEPS = D / KSTEP;
  static constexpr int TILE_BYTES = BM * ROW_BYTES;
  static_assert(CPR == 16, "tile loads assume 256-byte rows");
  static_assert(BM * ROW_BYTES == 16 * 1024, "16 blocks of 1 KiB per tile");
};

struct MaskRegs {
  int32_t lts, lte, uts, ute;
};

template <typename T, int D>
__global__ __launch_bounds__(256, 1) void attn_bwd_kernel(BwdArgs a) {
  using C = BwdTile<T, D>;
  using E = Elem<T>;
  using frag = typename E::frag;
  constexpr int KPL = C::KPL, KSTEP = C::KSTEP;

  // LDS: three tile buffers [Q | dO | LSE2 | D].
  constexpr int BUF_BYTES = 2 * C::TILE_BYTES + 2 * C::BM * (int)sizeof(float);
  extern __shared__ __attribute__((aligned(16))) unsigned char smem[];
  auto bufp = [&](int b) -> unsigned char* { return smem + b * BUF_BYTES; };
  auto rowsp = [&](int b) -> float* { return reinterpret_cast<float*>(smem + b * BUF_BYTES + 2 * C::TILE_BYTES); };

  const int tid = threadIdx.x;
  const int lane = tid & 63, g = lane >> 5, l32 = lane & 31;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);  // wave index (uniform)

  const int n_kb = (a.nk + C::BN - 1) / C::BN;
  const int work = xcd_contiguous_index(blockIdx.x, gridDim.x);
  const int bh = work / n_kb;
  const int kb = a.order[work % n_kb];
  const int key = kb * C::BN + w * 32 + l32;  // this lane's key (a column of S)
  const bool key_ok = key < a.nk;

  const T* __restrict__ Qp = static_cast<const T*>(a.q) + (size_t)bh * a.nq * D;
  const T* __restrict__ dOp = static_cast<const T*>(a.dout) + (size_t)bh * a.nq * D;
  const T* __restrict__ Kp = static_cast<const T*>(a.k) + (size_t)bh * a.nk * D;
  const T* __restrict__ Vp = static_cast<const T*>(a.v) + (size_t)bh * a.nk * D;
  const float* __restrict__ lse2 = a.lse2 + (size_t)bh * a.nq;
  const float* __restrict__ dlt = a.delta + (size_t)bh * a.nq;
  const buf_rsrc qbuf = make_buf(Qp, (uint32_t)a.nq * C::ROW_BYTES);
  const buf_rsrc dobuf = make_buf(dOp, (uint32_t)a.nq * C::ROW_BYTES);
  const buf_rsrc kbuf = make_buf(Kp, (uint32_t)a.nk * C::ROW_BYTES);
  const buf_rsrc vbuf = make_buf(Vp, (uint32_t)a.nk * C::ROW_BYTES);
  const buf_rsrc lbuf = make_buf(lse2, (uint32_t)a.nq * sizeof(float));
  const buf_rsrc dlbuf = make_buf(dlt, (uint32_t)a.nq * sizeof(float));

  // K and V rows of this lane's key as B operands (k-step s: d = s*KSTEP + g*KPL + 0..KPL).
  frag kf[C::QK_STEPS], vf[C::QK_STEPS];
#pragma unroll
  for (int s = 0; s < C::QK_STEPS; ++s) {
    const uint32_t off = (uint32_t)key * C::ROW_BYTES + (uint32_t)(s * KSTEP + g * KPL) * sizeof(T);
    if constexpr (KPL == 8) {
      kf[s] = __builtin_bit_cast(frag, buf_load16(kbuf, off, 0));
      vf[s] = __builtin_bit_cast(frag, buf_load16(vbuf, off, 0));
    } else {
      kf[s] = __builtin_bit_cast(frag, buf_load4(kbuf, off, 0));
      vf[s] = __builtin_bit_cast(frag, buf_load4(vbuf, off, 0));
    }
  }
  MaskRegs mk = {0, 0, 0, 0};  // this lane's key; past the last key every row is masked
  if (key_ok) mk = {a.mask.lts[key], a.mask.lte[key], a.mask.uts[key], a.mask.ute[key]};
  // Wait for these loads here: the main loop keeps tile loads in flight, and a wait the compiler
  // would place there for a register loaded now would also wait for those.
  wait_vmem();
  const bool ragged_block = (kb == n_kb - 1) && (a.nk % C::BN) != 0;

  // ---- per-lane LDS byte offsets, constant for the whole kernel ------------------------------
  // Transpose-read lane geometry: lane i of 16-lane block b addresses row k0 + 8*(b/2) + i/4,
  // column m0 + 16*(b%2) + 4*(i%4), and receives rows k0 + 8*(l/32) + 0..3 of column m0 + l%32.
  // The swizzle depends only on row & 15, so an offset computed for a row below 16 stays valid when a multiple of 16 rows is added as a constant;
  // every LDS access below is then one of these registers plus an immediate.
  const int tb = lane >> 4, ti = lane & 15;
  const int tr_row = 8 * (tb >> 1) + (ti >> 2);
  const int tr_col = 16 * (tb & 1) + 4 * (ti & 3);
  constexpr int US = 32 / KSTEP;  // k-steps in a 32-query half

  int off_s[C::QK_STEPS];  // S / dP operand (query row source row, k-step s) of a half
  int off_tq[C::NDB][2];   // Q^T / dO^T operand rows (tr_row, tr_row + 4), columns 32*db
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

  // Operand of a contraction over the rows of a row-major tile (k = tile row): rows
  // k0 + g*KPL + 0..KPL-1 of this lane's column; `off` = {row tr_row, row tr_row + 4} offsets.
  auto tr_operand = [&](const unsigned char* tile, const int* off, int k0_bytes) -> frag {
    if constexpr (KPL == 8) {
      const s16x4 lo = lds_read_tr16(tile + off[0] + k0_bytes);
      const s16x4 hi = lds_read_tr16(tile + off[1] + k0_bytes);
      return __builtin_bit_cast(frag, __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7));
    } else {
      return *reinterpret_cast<const T*>(tile + off[0] + k0_bytes);
    }
  };

  f32x16 dv_acc[C::NDB], dk_acc[C::NDB];
#pragma unroll
  for (int db = 0; db < C::NDB; ++db) {
    dv_acc[db] = f32x16{};
    dk_acc[db] = f32x16{};
  }

  const int cnt = a.kcnt[kb];
  const int32_t* __restrict__ lst = a.klist + (size_t)kb * a.list_stride;
  const float cexp = a.scale * kLog2e;

  // A tile's 64 rows of Q (then dO) are 16 blocks of 1 KiB; wave w moves blocks 4w..4w+3, lane l
  // the 16-byte slot l of a block, i.e. row 4j + l/16, physical chunk l%16, which holds logical
  // chunk (l%16) ^ swz_row(row).  Rows past nq read as zeros.  Waves 0 and 1 also move the tile's
  // LSE2 and D rows.  The loads go to registers first (load_tile) and are written to LDS one
  // tile later (commit_tile), so no LDS read ever waits on a load in flight.
  uint4 stq[4], std_[4];
  float strow = 0.0f;
  auto load_tile = [&](int entry) {
    const uint32_t tile_base = (uint32_t)(entry >> 1) * C::BM * C::ROW_BYTES;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int row = 4 * (4 * w + i) + (lane >> 4);
      const uint32_t voff = (uint32_t)row * C::ROW_BYTES + (uint32_t)(((lane & 15) ^ swz_row<T>(row)) * 16);
      stq[i] = buf_load16(qbuf, voff, tile_base);
      std_[i] = buf_load16(dobuf, voff, tile_base);
    }
    if (w < 2) {
      const uint32_t roff = (uint32_t)(entry >> 1) * C::BM * sizeof(float);
      strow = __builtin_bit_cast(float, buf_load4(w == 0 ? lbuf : dlbuf, (uint32_t)lane * sizeof(float), roff));
    }
  };
  auto commit_tile = [&](int b) {
    unsigned char* qt = bufp(b);
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int j = 4 * w + i;
      *reinterpret_cast<uint4*>(qt + j * 1024 + lane * 16) = stq[i];
      *reinterpret_cast<uint4*>(qt + C::TILE_BYTES + j * 1024 + lane * 16) = std_[i];
    }
    if (w < 2) rowsp(b)[w * C::BM + lane] = strow;
  };

  // Row mask of this lane's key over a tile's BM query rows starting at q0 (bit i = row q0 + i
  // masked), pre-shifted by g*KPL so that bit qr*32 + perm_index(r, 0) belongs to register r of
  // row block qr in this lane group.
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

  // ---- one 32-query half ("unit") of a tile, in three steps ---------------------------------
  // S = Q K^T and dP = dO V^T for the tile's rows h*32..h*32+31: register r of group g is query
  // h*32 + perm_index(r, g); the column is this lane's key.
  auto sdp = [&](const unsigned char* qt, auto hc, f32x16& sacc, f32x16& pacc) {
    constexpr int h = decltype(hc)::value;
    sacc = f32x16{};
    pacc = f32x16{};
#pragma unroll
    for (int st = 0; st < C::QK_STEPS; ++st) {
      const int off = off_s[st] + h * 32 * C::ROW_BYTES;
      const frag qa = *reinterpret_cast<const frag*>(qt + off);
      const frag da = *reinterpret_cast<const frag*>(qt + C::TILE_BYTES + off);
      sacc = E::mfma(qa, kf[st], sacc);
      pacc = E::mfma(da, vf[st], pacc);
    }
  };

  // P = exp2(S*scale*log2e - LSE2) (0 where masked: bit h*32 + perm_index(r, 0) of mrow) and
  // dS = P (dP - D), rounded into operand fragments: k-step u covers queries
  // h*32 + u*KSTEP + g*KPL + e = registers u*KPL + e.
  struct Rows {
    float lse[16], dlt[16];  // LSE2 and D of the 16 queries this lane holds
  };
  auto load_rows = [&](const float* lse_t, auto hc, Rows& rw) {
    constexpr int h = decltype(hc)::value;
    const float* dlt_t = lse_t + C::BM;
    if constexpr (KPL == 8) {
#pragma unroll
      for (int j = 0; j < 2; ++j) {
        const int q = h * 32 + 16 * j + 8 * g;
        const float4 l0 = *reinterpret_cast<const float4*>(lse_t + q);
        const float4 l1 = *reinterpret_cast<const float4*>(lse_t + q + 4);
        const float4 d0 = *reinterpret_cast<const float4*>(dlt_t + q);
        const float4 d1 = *reinterpret_cast<const float4*>(dlt_t + q + 4);
        const float lv[8] = {l0.x, l0.y, l0.z, l0.w, l1.x, l1.y, l1.z, l1.w};
        const float dv[8] = {d0.x, d0.y, d0.z, d0.w, d1.x, d1.y, d1.z, d1.w};
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          rw.lse[8 * j + e] = lv[e];
          rw.dlt[8 * j + e] = dv[e];
        }
      }
    } else {
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        rw.lse[r] = lse_t[h * 32 + perm_index<KPL>(r, g)];
        rw.dlt[r] = dlt_t[h * 32 + perm_index<KPL>(r, g)];
      }
    }
  };
  // One 32-query unit with a fixed issue order (a wave per SIMD issues in order): the next
  // unit's S / dP products are interleaved with this unit's elementwise work
  //   P = exp2(S*scale*log2e - LSE2) (0 where masked), dS = P (dP - D),
  // then dV^T += dO^T P and dK^T += Q^T dS run with their transpose reads.  sched_barrier fences
  // pin the order; operand reads run a few products ahead of their use.
  constexpr int AH = 4;  // operand reads of the S / dP products issued ahead of their use
  // The first AH operand reads of a unit's S / dP products can be issued by the unit before it
  // (pre: they are already in opio; pfn: issue the following unit's into opio, from tile q2,
  // half h2, at the end of this unit).
  auto unit = [&](const unsigned char* qt, auto hc, auto maskedc, bool test, uint64_t mrow,
                  const Rows& rw, const f32x16& sc, const f32x16& pc, const unsigned char* qn,
                  auto hnc, auto nextc, const float* lse_n, Rows& rw_n, f32x16& sn, f32x16& pn,
                  frag* opio, auto prec, auto pfnc, const unsigned char* q2, auto h2c,
                  auto barc, auto&& bar) {
    constexpr int h = decltype(hc)::value, hn = decltype(hnc)::value, h2 = decltype(h2c)::value;
    constexpr bool MASKED = decltype(maskedc)::value;
    constexpr bool NEXT = decltype(nextc)::value;
    constexpr bool PRE = decltype(prec)::value, PFN = decltype(pfnc)::value;
    constexpr bool BAR = decltype(barc)::value;  // run bar() before the read-ahead at the end
    constexpr int NS = 2 * C::QK_STEPS;  // S / dP products of a unit
    constexpr int NDV = 2 * US * C::NDB, AT = 3;  // dV / dK products of a unit, read-ahead
    // Registers 0..7 feed the first half of the dV / dK products, 8..15 the second half: the
    // elementwise work of registers 0..RA-1 runs beside the S / dP products, the rest beside the
    // first half of the dV / dK products.
    constexpr int RA = 10;
    if constexpr (NEXT) load_rows(lse_n, hnc, rw_n);
    auto sread = [&](int i) -> frag {
      return *reinterpret_cast<const frag*>(qn + ((i & 1) ? C::TILE_BYTES : 0) + off_s[i >> 1] +
                                            hn * 32 * C::ROW_BYTES);
    };
    // dV / dK product j: k-step u = j / (2 NDB), d block (j % (2 NDB)) / 2, dV (even j) or dK
    auto tread = [&](int j) -> frag {
      const int u = j / (2 * C::NDB), db = (j % (2 * C::NDB)) >> 1;
      return tr_operand((j & 1) ? qt : qt + C::TILE_BYTES, off_tq[db], (h * 32 + u * KSTEP) * C::ROW_BYTES);
    };
    frag op[NS], top[NDV];
    if constexpr (NEXT) {
      sn = f32x16{};
      pn = f32x16{};
#pragma unroll
      for (int i = 0; i < AH; ++i) op[i] = PRE ? opio[i] : sread(i);
    }
    // P = exp2(S*scale*log2e - LSE2) and dS = P (dP - D) for register r.
    float pv[16], dsv[16];
    auto elem = [&](int r) {
      pv[r] = fast_exp2(fmaf(sc[r], cexp, -rw.lse[r]));
      dsv[r] = pv[r] * (pc[r] - rw.dlt[r]);
    };
    // In partly masked tiles P and dS are zeroed where masked (bit perm_index(r, 0) of this
    // unit's mask word) before they are rounded into operands; other tiles skip this.
    const uint32_t mw = (uint32_t)(mrow >> (32 * h));
    auto apply_mask = [&](int r0, int r1) {
      if constexpr (MASKED) {
        if (test) {  // uniform across the wave
#pragma unroll
          for (int r = r0; r < r1; ++r) {
            const bool m = (mw >> perm_index<KPL>(r, 0)) & 1u;
            pv[r] = m ? 0.0f : pv[r];
            dsv[r] = m ? 0.0f : dsv[r];
          }
        }
      }
    };
    // operand fragments: k-step u covers queries h*32 + u*KSTEP + g*KPL + e = registers u*KPL + e
    frag pf[US], sf[US];
    auto frags = [&](int u) {
      if constexpr (KPL == 1) {
        pf[u] = pv[u];
        sf[u] = dsv[u];
      } else {
#pragma unroll
        for (int e = 0; e < KPL; ++e) {
          pf[u][e] = E::from_float(pv[u * KPL + e]);
          sf[u][e] = E::from_float(dsv[u * KPL + e]);
        }
      }
    };
    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
    for (int i = 0; i < NS; ++i) {
      if constexpr (NEXT) {
        if (i & 1)
          pn = E::mfma(op[i], vf[i >> 1], pn);
        else
          sn = E::mfma(op[i], kf[i >> 1], sn);
        if (i + AH < NS) op[i + AH] = sread(i + AH);
      }
#pragma unroll
      for (int r = i * RA / NS; r < (i + 1) * RA / NS; ++r) elem(r);
      if (i + AT >= NS) top[i + AT - NS] = tread(i + AT - NS);
      __builtin_amdgcn_sched_barrier(0);
    }
    apply_mask(0, 8);
#pragma unroll
    for (int u = 0; u < US / 2; ++u) frags(u);
    __builtin_amdgcn_sched_barrier(0);
    constexpr int HALF = NDV / 2;
#pragma unroll
    for (int j = 0; j < NDV; ++j) {
      const int u = j / (2 * C::NDB), db = (j % (2 * C::NDB)) >> 1;
      if (j & 1)
        dk_acc[db] = E::mfma(top[j], sf[u], dk_acc[db]);
      else
        dv_acc[db] = E::mfma(top[j], pf[u], dv_acc[db]);
      if (j + AT < NDV) top[j + AT] = tread(j + AT);
      if constexpr (BAR) {
        if (j == NDV - AH - 1) bar();
      }
      if constexpr (PFN) {
        if (j >= NDV - AH) {
          const int i = j - (NDV - AH);
          opio[i] = *reinterpret_cast<const frag*>(q2 + ((i & 1) ? C::TILE_BYTES : 0) + off_s[i >> 1] +
                                                   h2 * 32 * C::ROW_BYTES);
        }
      }
      if (j < HALF) {
#pragma unroll
        for (int r = RA + j * (16 - RA) / HALF; r < RA + (j + 1) * (16 - RA) / HALF; ++r) elem(r);
        if (j == HALF - 1) {
          apply_mask(8, 16);
#pragma unroll
          for (int u = US / 2; u < US; ++u) frags(u);
        }
      }
      __builtin_amdgcn_sched_barrier(0);
    }
  };

  // ---- software pipeline over units -----------------------------------------------------------
  // Tile t sits in buffer t % 3.  While the elementwise step of one unit runs, the S / dP
  // products of the next unit (the second half of the tile, or the first half of the next tile)
  // are already issued.  Tile t+1 is waited for, with one workgroup barrier, before the second
  // unit of tile t; that barrier also frees the buffer of tile t-1, which then receives tile t+2.
  using H0 = std::integral_constant<int, 0>;
  using H1 = std::integral_constant<int, 1>;
  f32x16 sn, pn;  // S / dP of the next unit
  Rows rw, rw_n;  // LSE2 / D of the current and the next unit
  frag opio[AH];  // operands read ahead for the next unit's S / dP products
  int entry = 0, cur = 0;
  if (cnt > 0) {
    entry = __builtin_amdgcn_readfirstlane(lst[0]);
    load_tile(entry);
    wait_vmem();
    commit_tile(0);
    __syncthreads();
    if (cnt > 1) load_tile(__builtin_amdgcn_readfirstlane(lst[1]));
    load_rows(rowsp(0), H0{}, rw);
    sdp(bufp(0), H0{}, sn, pn);
#pragma unroll
    for (int i = 0; i < AH; ++i)
      opio[i] = *reinterpret_cast<const frag*>(bufp(0) + ((i & 1) ? C::TILE_BYTES : 0) + off_s[i >> 1] +
                                               32 * C::ROW_BYTES);
  }
  // Tile t sits in buffer t % 3.
  auto tile_step = [&](const int t, auto has_next_c, auto maskedc) {
    constexpr bool HAS_NEXT = decltype(has_next_c)::value;
    const bool test = (entry & 1) || ragged_block;
    const uint64_t mrow = decltype(maskedc)::value && test ? tile_row_mask((entry >> 1) * C::BM) : 0ull;
    const unsigned char* qt = bufp(cur);
    const float* lse_t = rowsp(cur);
    const int nxt = cur == 2 ? 0 : cur + 1;
    // first half, with the second half's S / dP
    f32x16 sc = sn, pc = pn;
    auto none = [] {};
    unit(qt, H0{}, maskedc, test, mrow, rw, sc, pc, qt, H1{}, std::true_type{}, lse_t, rw_n, sn, pn,
         opio, std::true_type{}, std::false_type{}, qt, H0{}, std::false_type{}, none);
    rw = rw_n;
    sc = sn;
    pc = pn;
    if constexpr (HAS_NEXT) {
      // second half, with the next tile's first half
      entry = __builtin_amdgcn_readfirstlane(lst[t + 1]);
      wait_vmem();        // tile t+1 is in this wave's registers
      commit_tile(nxt);   // its buffer last held tile t-2
      __syncthreads();    // tile t+1 complete in LDS
      if (t + 2 < cnt) load_tile(__builtin_amdgcn_readfirstlane(lst[t + 2]));
      unit(qt, H1{}, maskedc, test, mrow, rw, sc, pc, bufp(nxt), H0{}, std::true_type{},
           rowsp(nxt), rw_n, sn, pn, opio, std::false_type{}, std::true_type{}, bufp(nxt), H1{},
           std::false_type{}, none);
      rw = rw_n;
    } else {
      unit(qt, H1{}, maskedc, test, mrow, rw, sc, pc, qt, H0{}, std::false_type{}, lse_t, rw_n, sn,
           pn, opio, std::false_type{}, std::false_type{}, qt, H0{}, std::false_type{}, none);
    }
    cur = nxt;
  };
  // Every tile takes the row test (an unmasked tile's mask word is zero): one code path keeps
  // the loop free of branches the accumulators would have to merge across.
  auto step = [&](const int t, auto has_next_c) { tile_step(t, has_next_c, std::true_type{}); };
  for (int t = 0; t + 1 < cnt; ++t) step(t, std::true_type{});
  if (cnt > 0) step(cnt - 1, std::false_type{});

  if (key_ok) {
    T* dkr = static_cast<T*>(a.dk) + ((size_t)bh * a.nk + key) * D;
    T* dvr = static_cast<T*>(a.dv) + ((size_t)bh * a.nk + key) * D;
#pragma unroll
    for (int db = 0; db < C::NDB; ++db)
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int d0 = db * 32 + 8 * i + 4 * g;
        if constexpr (sizeof(T) == 2) {
          uint2 ok, ov;
          ok.x = pack_bf16x2(dk_acc[db][4 * i + 0] * a.scale, dk_acc[db][4 * i + 1] * a.scale);
          ok.y = pack_bf16x2(dk_acc[db][4 * i + 2] * a.scale, dk_acc[db][4 * i + 3] * a.scale);
          ov.x = pack_bf16x2(dv_acc[db][4 * i + 0], dv_acc[db][4 * i + 1]);
          ov.y = pack_bf16x2(dv_acc[db][4 * i + 2], dv_acc[db][4 * i + 3]);
          *reinterpret_cast<uint2*>(dkr + d0) = ok;
          *reinterpret_cast<uint2*>(dvr + d0) = ov;
        } else {
          *reinterpret_cast<float4*>(dkr + d0) =
              make_float4(dk_acc[db][4 * i + 0] * a.scale, dk_acc[db][4 * i + 1] * a.scale,
                          dk_acc[db][4 * i + 2] * a.scale, dk_acc[db][4 * i + 3] * a.scale);
          *reinterpret_cast<float4*>(dvr + d0) =
              make_float4(dv_acc[db][4 * i + 0], dv_acc[db][4 * i + 1], dv_acc[db][4 * i + 2],
                          dv_acc[db][4 * i + 3]);
        }
      }
  }
}

// D_i = sum_d dO_id O_id (float32) and LSE_i * log2(e) (+inf for fully masked rows).  16 threads
// per row, one 16-byte chunk of O and dO each.
template <typename T, int D>
__global__ __launch_bounds__(256) void bwd_pre_kernel(const T* __restrict__ o,
                                                      const T* __restrict__ dout,
                                                      const float* __restrict__ lse,
                                                      float* __restrict__ delta,
                                                      float* __restrict__ lse2, int64_t rows) {
  constexpr int CH = 16 / (int)sizeof(T);
  static_assert(D / CH == 16, "16 chunks per row");
  const int64_t row = (int64_t)blockIdx.x * 16 + (threadIdx.x >> 4);
  const int c = threadIdx.x & 15;
  if (row >= rows) return;
  const uint4 xo = *reinterpret_cast<const uint4*>(o + row * D + c * CH);
  const uint4 xd = *reinterpret_cast<const uint4*>(dout + row * D + c * CH);
  const T* eo = reinterpret_cast<const T*>(&xo);
  const T* ed = reinterpret_cast<const T*>(&xd);
  float acc = 0.0f;
#pragma unroll
  for (int e = 0; e < CH; ++e) acc = fmaf((float)eo[e], (float)ed[e], acc);
#pragma unroll
  for (int off = 8; off >= 1; off >>= 1) acc += __shfl_xor(acc, off);
  if (c == 0) {
    delta[row] = acc;
    // LSE in log2 units; a fully masked row (LSE = -inf) gets +inf so that exp2(s - lse2) = 0
    const float x = lse[row];
    lse2[row] = x == -INFINITY ? INFINITY : x * kLog2e;
  }
}

template <typename T, int D>
hipError_t run_bwd(const BwdArgs& a, hipStream_t stream, hipEvent_t ev_begin) {
  const int64_t rows = (int64_t)a.B * a.H * a.nq;
  const int pre_grid = (int)((rows + 15) / 16);
  hipLaunchKernelGGL((bwd_pre_kernel<T, D>), dim3(pre_grid), dim3(256), 0, stream,
                     static_cast<const T*>(a.o), static_cast<const T*>(a.dout), a.lse, a.delta,
                     a.lse2, rows);
  hipError_t err = hipGetLastError();
  if (err != hipSuccess) return err;

  using C = BwdTile<T, D>;
  const size_t smem = 3 * (2 * C::TILE_BYTES + 2 * C::BM * sizeof(float));
  // The main kernel uses more than 64 KiB of LDS; allow it on the current device.
  err = hipFuncSetAttribute(reinterpret_cast<const void*>(&attn_bwd_kernel<T, D>),
                            hipFuncAttributeMaxDynamicSharedMemorySize, (int)smem);
  if (err != hipSuccess) return err;
  const int64_t n_kb = (a.nk + C::BN - 1) / C::BN;
  const int64_t grid = n_kb * a.B * a.H;
  if (ev_begin) (void)hipEventRecord(ev_begin, stream);
  hipLaunchKernelGGL((attn_bwd_kernel<T, D>), dim3((unsigned)grid), dim3(256), smem, stream, a);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_attn_bwd(int dtype, const BwdArgs& a, hipStream_t stream, hipEvent_t ev_begin) {
  return dtype == 0 ? run_bwd<bf16, 128>(a, stream, ev_begin) : run_bwd<float, 64>(a, stream, ev_begin);
}

}  // namespace fm
