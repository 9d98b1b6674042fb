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
  static constexpr int NQB = BM / 32;
  static constexpr int NDB = D / 32;
  static constexpr int QK_STEPS = D / KSTEP;
  static constexpr int PQ_STEPS = BM / KSTEP;  // k-steps over a tile's queries
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

  // LDS: two (Q, dO) tile buffers and two (LSE, D) rows.
  extern __shared__ __attribute__((aligned(16))) unsigned char smem[];
  unsigned char* qdo_lds = smem;                                         // [2][Q | dO]
  float* rows_lds = reinterpret_cast<float*>(smem + 4 * C::TILE_BYTES);  // [2][LSE2 | D]

  const int tid = threadIdx.x;
  const int lane = tid & 63, g = lane >> 5, l32 = lane & 31;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);  // wave index (uniform)

  const int n_kb = (a.nk + C::BN - 1) / C::BN;
  const int work = xcd_contiguous_index(blockIdx.x, gridDim.x);
  const int bh = work / n_kb;
  const int kb = n_kb - 1 - (work % n_kb);
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

  // Stage tile `entry` into buffer `buf` with loads straight into LDS: the tile's 64 rows of Q
  // (then dO) are 16 blocks of 1 KiB; wave w fills blocks 4w..4w+3, lane l the 16-byte slot l
  // of a block, i.e. row 4j + l/16, physical chunk l%16, which holds logical chunk
  // (l%16) ^ swz_row(row).  Rows past nq read as zeros.  Waves 0 and 1 also copy the tile's
  // LSE2 and D rows.
  auto issue_tile = [&](int entry, auto bufc) {
    constexpr int buf = decltype(bufc)::value;
    unsigned char* qt = qdo_lds + buf * 2 * C::TILE_BYTES;
    const uint32_t tile_base = (uint32_t)(entry >> 1) * C::BM * C::ROW_BYTES;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int j = 4 * w + i;
      const int row = 4 * j + (lane >> 4);
      const uint32_t voff = (uint32_t)row * C::ROW_BYTES + (uint32_t)(((lane & 15) ^ swz_row<T>(row)) * 16);
      buf_load_lds<16>(qbuf, qt + j * 1024, voff, tile_base);
      buf_load_lds<16>(dobuf, qt + C::TILE_BYTES + j * 1024, voff, tile_base);
    }
    if (w < 2) {
      const uint32_t roff = (uint32_t)(entry >> 1) * C::BM * sizeof(float);
      buf_load_lds<4>(w == 0 ? lbuf : dlbuf, rows_lds + buf * 2 * C::BM + w * C::BM,
                      (uint32_t)lane * sizeof(float), roff);
    }
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

  // List entries are read into scalar registers: the buffer loads take the tile offset as a
  // scalar operand.
  int entry = cnt > 0 ? __builtin_amdgcn_readfirstlane(lst[0]) : 0;

  auto body = [&](const int it, auto bufc) {
    constexpr int buf = decltype(bufc)::value;
    const int qb = entry >> 1;
    const bool test = (entry & 1) || ragged_block;
    const int next = it + 1 < cnt ? __builtin_amdgcn_readfirstlane(lst[it + 1]) : 0;
    wait_vmem();      // this wave's loads of tile `it` have landed in LDS
    __syncthreads();  // ... everyone's; buffer buf ^ 1 is free again
    if (it + 1 < cnt) issue_tile(next, std::integral_constant<int, buf ^ 1>{});

    const unsigned char* qt = qdo_lds + buf * 2 * C::TILE_BYTES;
    const unsigned char* dt = qt + C::TILE_BYTES;
    const float* lse_t = rows_lds + buf * 2 * C::BM;
    const float* dlt_t = lse_t + C::BM;
    const uint64_t mrow = test ? tile_row_mask(qb * C::BM) : 0ull;

    // The tile is processed as NQB row blocks of 32 queries, one after the other, so only one
    // block's S, dP, P and dS are live at a time.
#pragma unroll
    for (int qr = 0; qr < C::NQB; ++qr) {
      // S = Q K^T and dP = dO V^T for rows qr*32..: register r of group g is tile query
      // qr*32 + perm_index(r, g); the column is this lane's key.
      f32x16 sacc = {}, pacc = {};
      if constexpr (KPL == 8) __builtin_amdgcn_sched_barrier(0);
#pragma unroll
      for (int st = 0; st < C::QK_STEPS; ++st) {
        const int off = off_s[st] + qr * 32 * C::ROW_BYTES;
        const frag qa = *reinterpret_cast<const frag*>(qt + off);
        const frag da = *reinterpret_cast<const frag*>(dt + off);
        sacc = E::mfma(qa, kf[st], sacc);
        pacc = E::mfma(da, vf[st], pacc);
      }
      if constexpr (KPL == 8) {
        // operand reads one k-step ahead of their MFMAs
        __builtin_amdgcn_sched_group_barrier(0x100, 2, 1);
#pragma unroll
        for (int st = 0; st < C::QK_STEPS; ++st) {
          __builtin_amdgcn_sched_group_barrier(0x008, 2, 1);
          if (st + 1 < C::QK_STEPS) __builtin_amdgcn_sched_group_barrier(0x100, 2, 1);
        }
        __builtin_amdgcn_sched_barrier(0);
      }

      // LSE (log2 units) and D of the 16 queries this lane holds: runs of KPL consecutive rows
      // qr*32 + (r/KPL)*2*KPL + g*KPL + 0..KPL-1.
      float lsev[16], dltv[16];
      if constexpr (KPL == 8) {
#pragma unroll
        for (int j = 0; j < 2; ++j) {
          const int q = qr * 32 + 16 * j + 8 * g;
          const float4 l0 = *reinterpret_cast<const float4*>(lse_t + q);
          const float4 l1 = *reinterpret_cast<const float4*>(lse_t + q + 4);
          const float4 d0 = *reinterpret_cast<const float4*>(dlt_t + q);
          const float4 d1 = *reinterpret_cast<const float4*>(dlt_t + q + 4);
          const float lv[8] = {l0.x, l0.y, l0.z, l0.w, l1.x, l1.y, l1.z, l1.w};
          const float dv[8] = {d0.x, d0.y, d0.z, d0.w, d1.x, d1.y, d1.z, d1.w};
#pragma unroll
          for (int e = 0; e < 8; ++e) {
            lsev[8 * j + e] = lv[e];
            dltv[8 * j + e] = dv[e];
          }
        }
      } else {
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          lsev[r] = lse_t[qr * 32 + perm_index<KPL>(r, g)];
          dltv[r] = dlt_t[qr * 32 + perm_index<KPL>(r, g)];
        }
      }

      // P and dS (overwriting sacc and pacc); the masked variant is a separate code path so
      // unmasked tiles pay nothing for the test.
      auto elementwise = [&](auto masked_c) {
        constexpr bool MASKED = decltype(masked_c)::value;
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          float p = fast_exp2(fmaf(sacc[r], cexp, -lsev[r]));
          if constexpr (MASKED) {
            const int bit = qr * 32 + perm_index<KPL>(r, 0);
            p = ((mrow >> bit) & 1ull) ? 0.0f : p;
          }
          sacc[r] = p;
          pacc[r] = p * (pacc[r] - dltv[r]);
        }
      };
      if (test)
        elementwise(std::true_type{});
      else
        elementwise(std::false_type{});

      // Operand fragments of P and dS: k-step u covers tile queries
      // qr*32 + u*KSTEP + g*KPL + e = registers u*KPL + e.
#pragma unroll
      for (int u = 0; u < US; ++u) {
        frag pf, sf;
        if constexpr (KPL == 1) {
          pf = sacc[u];
          sf = pacc[u];
        } else {
#pragma unroll
          for (int e = 0; e < KPL; ++e) {
            pf[e] = E::from_float(sacc[u * KPL + e]);
            sf[e] = E::from_float(pacc[u * KPL + e]);
          }
        }
        const int q0 = qr * 32 + u * KSTEP;
        // dV^T += dO^T P and dK^T += Q^T dS: A = rows d of the transposed tiles (contraction
        // over the tile's queries q0..q0+KSTEP), read with the transpose read.
#pragma unroll
        for (int db = 0; db < C::NDB; ++db) {
          dv_acc[db] = E::mfma(tr_operand(dt, off_tq[db], q0 * C::ROW_BYTES), pf, dv_acc[db]);
          dk_acc[db] = E::mfma(tr_operand(qt, off_tq[db], q0 * C::ROW_BYTES), sf, dk_acc[db]);
        }
      }
      if constexpr (KPL == 8) {
        // transpose reads (4 per d block) one d block ahead of their two MFMAs
        __builtin_amdgcn_sched_group_barrier(0x100, 4, 2);
#pragma unroll
        for (int i = 0; i < US * C::NDB; ++i) {
          __builtin_amdgcn_sched_group_barrier(0x008, 2, 2);
          if (i + 1 < US * C::NDB) __builtin_amdgcn_sched_group_barrier(0x100, 4, 2);
        }
      }
    }

    entry = next;
  };

  if (cnt > 0) issue_tile(entry, std::integral_constant<int, 0>{});
  // Unrolled by two so each buffer index is a compile-time constant; an odd last tile runs after
  // the loop, so the loop body has no conditional path the accumulators must merge across.
  int it = 0;
  for (; it + 1 < cnt; it += 2) {
    body(it, std::integral_constant<int, 0>{});
    body(it + 1, std::integral_constant<int, 1>{});
  }
  if (it < cnt) body(it, std::integral_constant<int, 0>{});

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
size_t bwd_smem_bytes() {
  using C = BwdTile<T, D>;
  return 4 * C::TILE_BYTES + sizeof(float) * 4 * C::BM;
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

  const size_t smem = bwd_smem_bytes<T, D>();
  // The main kernel uses more than 64 KiB of LDS; allow it on the current device.
  err = hipFuncSetAttribute(reinterpret_cast<const void*>(&attn_bwd_kernel<T, D>),
                            hipFuncAttributeMaxDynamicSharedMemorySize, (int)smem);
  if (err != hipSuccess) return err;
  const int64_t n_kb = (a.nk + BwdTile<T, D>::BN - 1) / BwdTile<T, D>::BN;
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
