// Mask-aware attention backward for gfx950.
//
// The pages report the backward's speed ("FlashMask-3 ..." zicq.com summary, end-to-end
// paragraph) but do not describe it; this is the standard recompute-from-LSE backward restricted
// to the tiles the classification lists (fully masked tiles skipped, the row test only in
// partly masked tiles, as the forward; "FlashMask-3 sends each GPU its mask ...",
// tile-classification paragraph).
//
//   K4 bwd_pre:  D_i = sum_d dO_id O_id, and the float32 dQ accumulator cleared.
//   K5 bwd_main: one workgroup per key block of BN = 128 keys (4 waves x 32 keys).  K and V rows
//                of the wave's keys stay in registers (B operands of S = Q K^T and dP = dO V^T),
//                dK^T and dV^T accumulate in registers, and so does the slice of K each wave
//                needs for its share of dQ.  The workgroup walks the query blocks (BM = 64
//                rows) of its list.  Per tile:
//                  S, dP on 32x32 MFMAs with the query rows loaded in a permuted order so the
//                  accumulators double as operands; P = exp2(S*scale*log2e - LSE*log2e) (0 in
//                  masked entries); dS = P (dP - D); dV^T += dO^T P and dK^T += Q^T dS with the
//                  transposed operands read from the row-major Q / dO tiles by the gfx950 LDS
//                  transpose read; dS goes to LDS key-major (16-byte stores) and the next
//                  iteration reads it back transposed for dQ += dS K, added to the float32
//                  accumulator with atomics.
//                Q / dO tiles are double-buffered and the dQ product of tile i runs after the
//                barrier of tile i+1, so each tile costs one workgroup barrier.
//   K6 dq_convert: dQ = scale * accumulator, rounded to the output dtype.
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
  static constexpr int DS_ROW_BYTES = BM * (int)sizeof(T);  // dS^T rows: one key, BM queries
  static constexpr int NQB = BM / 32;
  static constexpr int NDB = D / 32;
  static constexpr int QK_STEPS = D / KSTEP;
  static constexpr int PQ_STEPS = BM / KSTEP;  // k-steps over a tile's queries
  static constexpr int DQ_STEPS = BN / KSTEP;  // k-steps over the block's keys
  static constexpr int NOB = NQB * NDB / 4;    // 32x32 dQ output blocks per wave
  static constexpr int TILE_BYTES = BM * ROW_BYTES;
  static constexpr int DS_BYTES = BN * DS_ROW_BYTES;
  // bf16 keeps the block's K rows resident in LDS for the dQ product; fp32 (whose tiles are
  // twice as large) keeps each wave's slice in registers instead.
  static constexpr bool K_IN_LDS = sizeof(T) == 2;
  static constexpr int K_BYTES = K_IN_LDS ? BN * ROW_BYTES : 0;
  static_assert(CPR == 16, "thread mapping assumes 256-byte rows");
  static_assert(BM == 4 * (NT / CPR), "staging: 4 rows per thread");
  static_assert(NOB >= 1 && NQB % NOB == 0 || NOB % NQB == 0, "dQ split");
};

// XOR swizzles of 16-byte chunks (bf16 only; fp32 tiles are left plain).  For 256-byte rows
// (Q, dO, K tiles): chunk c of row r sits at c ^ swz_row(r), a bijection on 16 consecutive rows
// (conflict-free row reads of 16 rows at one chunk) whose bits 2..3 differ across 4 consecutive
// rows (conflict-free transpose reads: 4 rows x 4 chunks per 32 lanes).  For the 128-byte dS^T
// rows the same two properties hold with swz_ds over 8 chunks and the 64-bank pairs of rows.
template <typename T>
__device__ __host__ constexpr int swz_row(int r) {
  return sizeof(T) == 2 ? (((r & 3) << 2) | ((r >> 2) & 3)) : 0;
}
template <typename T>
__device__ __host__ constexpr int swz_ds(int k) {
  return sizeof(T) == 2 ? ((((k >> 1) & 1) << 2) | ((k >> 2) & 3)) : 0;
}

// Byte offset of element (row, col) in a tile of `row_bytes`-byte rows with swizzle kind SK
// (0 = swz_row, 1 = swz_ds).
template <typename T, int SK>
__device__ inline int tile_off(int row, int col, int row_bytes) {
  constexpr int CH = 16 / (int)sizeof(T);
  const int sw = SK == 0 ? swz_row<T>(row) : swz_ds<T>(row);
  return row * row_bytes + (((col / CH) ^ sw) * 16) + (col % CH) * (int)sizeof(T);
}

struct MaskRegs {
  int32_t lts, lte, uts, ute;
};

template <typename T, int D>
__global__ __launch_bounds__(256, 1) void attn_bwd_kernel(BwdArgs a) {
  using C = BwdTile<T, D>;
  using E = Elem<T>;
  using frag = typename E::frag;
  constexpr int KPL = C::KPL, KSTEP = C::KSTEP, CH = C::CH;
  using SwzRow = std::integral_constant<int, 0>;
  using SwzDs = std::integral_constant<int, 1>;

  // LDS: two (Q, dO) tile buffers, two dS^T buffers, the block's K rows, two (LSE, D) rows.
  extern __shared__ __attribute__((aligned(16))) unsigned char smem[];
  unsigned char* qdo_lds = smem;                                         // [2][Q | dO]
  unsigned char* ds_lds = smem + 4 * C::TILE_BYTES;                      // [2][BN][BM]
  unsigned char* k_lds = ds_lds + 2 * C::DS_BYTES;                       // [BN][D]
  float* rows_lds = reinterpret_cast<float*>(k_lds + C::K_BYTES);       // [2][LSE2 | D]

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
  float* __restrict__ dqa = a.dq_acc + (size_t)bh * a.nq * D;
  // dQ accumulator rows past nq fall outside this buffer, so their atomics are dropped.
  const buf_rsrc dqbuf = make_buf(dqa, (uint32_t)a.nq * D * (uint32_t)sizeof(float));
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

  // staging map: chunk c of a 256-byte row; rows 4*rq + i
  const int c = tid % C::CPR;
  const int rq = tid / C::CPR;

  // ---- per-lane LDS byte offsets, constant for the whole kernel ------------------------------
  // Transpose-read lane geometry: lane i of 16-lane block b addresses row k0 + 8*(b/2) + i/4,
  // column m0 + 16*(b%2) + 4*(i%4), and receives rows k0 + 8*(l/32) + 0..3 of column m0 + l%32.
  // The swizzles depend only on row & 15 (swz_row) or row bits 1..3 (swz_ds), so an offset
  // computed for a row below 16 stays valid when a multiple of 16 rows is added as a constant;
  // every LDS access below is then one of these registers plus an immediate.
  const int tb = lane >> 4, ti = lane & 15;
  const int tr_row = 8 * (tb >> 1) + (ti >> 2);
  const int tr_col = 16 * (tb & 1) + 4 * (ti & 3);
  const int wave_db = (w * C::NOB) / C::NQB;  // the d block this wave produces in dQ
  const int krow = w * 32 + l32;              // this lane's key row of dS^T
  constexpr int US = 32 / KSTEP;              // k-steps in a 32-query half

  int off_s[C::QK_STEPS];  // S / dP operand (query row source row, k-step s) of a half
  int off_tq[C::NDB][2];   // Q^T / dO^T operand rows (tr_row, tr_row + 4), columns 32*db
  int off_dsr[C::NQB][2];  // dS^T operand rows (tr_row, tr_row + 4), columns 32*qr
  int off_k[2];            // K operand rows (tr_row, tr_row + 4), columns 32*wave_db
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
#pragma unroll
      for (int qr = 0; qr < C::NQB; ++qr) off_dsr[qr][h] = tile_off<T, 1>(r, 32 * qr + cc, C::DS_ROW_BYTES);
      off_k[h] = tile_off<T, 0>(r, 32 * wave_db + cc, C::ROW_BYTES);
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

  // The block's K rows are the B operand of dQ += dS K (k = the block's keys, n = d): read by
  // transpose reads from LDS (bf16), or read once into registers through the first (Q, dO)
  // buffer (fp32).
  unsigned char* kstage = C::K_IN_LDS ? k_lds : qdo_lds;
#pragma unroll
  for (int i = 0; i < C::BN / 16; ++i) {
    const int row = rq + 16 * i;
    const uint4 x = buf_load16(kbuf, (uint32_t)(kb * C::BN + row) * C::ROW_BYTES + c * 16, 0);
    *reinterpret_cast<uint4*>(kstage + tile_off<T, 0>(row, c * CH, C::ROW_BYTES)) = x;
  }
  frag kq[C::K_IN_LDS ? 1 : C::DQ_STEPS];
  if constexpr (!C::K_IN_LDS) {
    __syncthreads();
#pragma unroll
    for (int t = 0; t < C::DQ_STEPS; ++t) kq[t] = tr_operand(kstage, off_k, t * KSTEP * C::ROW_BYTES);
    __syncthreads();
  }

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

  // dQ[q][d] += sum_keys dS[q][key] K[key][d] for the tile held in dS^T buffer `buf`; wave w
  // owns d columns [32*wave_db, +32) and NOB query row blocks of them.
  auto dq_product = [&](auto bufc, int qb) {
    constexpr int buf = decltype(bufc)::value;
    const unsigned char* dst = ds_lds + buf * C::DS_BYTES;
    // acc register r: query qr*32 + acc_row(r, g) = (qr*32 + 8*(r/4) + r%4) + 4*g,
    // d = 32*wave_db + l32: the first part is uniform (scalar offset), the rest per lane.
    const uint32_t lane_off = (uint32_t)((4 * g * D + wave_db * 32 + l32) * sizeof(float));
#pragma unroll
    for (int ob = 0; ob < C::NOB; ++ob) {
      const int qr = (w * C::NOB + ob) % C::NQB;
      f32x16 acc = {};
#pragma unroll
      for (int t = 0; t < C::DQ_STEPS; ++t) {
        frag kb_op;
        if constexpr (C::K_IN_LDS)
          kb_op = tr_operand(k_lds, off_k, t * KSTEP * C::ROW_BYTES);
        else
          kb_op = kq[t];
        acc = E::mfma(tr_operand(dst, off_dsr[qr], t * KSTEP * C::DS_ROW_BYTES), kb_op, acc);
      }
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const uint32_t row = (uint32_t)(qb * C::BM + qr * 32 + 8 * (r / 4) + (r % 4));
        __builtin_amdgcn_raw_ptr_buffer_atomic_fadd_f32(acc[r], dqbuf, (int)lane_off,
                                                        (int)(row * D * sizeof(float)), 0);
      }
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
  int prev_qb = 0;

  auto body = [&](const int it, auto bufc) {
    constexpr int buf = decltype(bufc)::value;
    const int qb = entry >> 1;
    const bool test = (entry & 1) || ragged_block;
    const int next = it + 1 < cnt ? __builtin_amdgcn_readfirstlane(lst[it + 1]) : 0;
    wait_vmem();      // this wave's loads of tile `it` have landed in LDS
    __syncthreads();  // ... everyone's; dS^T of tile it-1 complete in buf ^ 1
    if (it + 1 < cnt) issue_tile(next, std::integral_constant<int, buf ^ 1>{});
    if (it > 0) dq_product(std::integral_constant<int, buf ^ 1>{}, prev_qb);

    const unsigned char* qt = qdo_lds + buf * 2 * C::TILE_BYTES;
    const unsigned char* dt = qt + C::TILE_BYTES;
    const float* lse_t = rows_lds + buf * 2 * C::BM;
    const float* dlt_t = lse_t + C::BM;
    unsigned char* dsw = ds_lds + buf * C::DS_BYTES;
    const uint64_t mrow = test ? tile_row_mask(qb * C::BM) : 0ull;

    // The tile is processed as NQB row blocks of 32 queries, one after the other, so only one
    // block's S, dP, P and dS are live at a time.
#pragma unroll
    for (int qr = 0; qr < C::NQB; ++qr) {
      // S = Q K^T and dP = dO V^T for rows qr*32..: register r of group g is tile query
      // qr*32 + perm_index(r, g); the column is this lane's key.
      f32x16 sacc = {}, pacc = {};
#pragma unroll
      for (int st = 0; st < C::QK_STEPS; ++st) {
        const int off = off_s[st] + qr * 32 * C::ROW_BYTES;
        const frag qa = *reinterpret_cast<const frag*>(qt + off);
        const frag da = *reinterpret_cast<const frag*>(dt + off);
        sacc = E::mfma(qa, kf[st], sacc);
        pacc = E::mfma(da, vf[st], pacc);
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
        // dS^T -> LDS (key-major): this lane's key row, queries q0 + g*KPL + 0..KPL.
        *reinterpret_cast<frag*>(dsw + tile_off<T, 1>(krow, q0 + g * KPL, C::DS_ROW_BYTES)) = sf;
        // dV^T += dO^T P and dK^T += Q^T dS: A = rows d of the transposed tiles (contraction
        // over the tile's queries q0..q0+KSTEP), read with the transpose read.
#pragma unroll
        for (int db = 0; db < C::NDB; ++db) {
          dv_acc[db] = E::mfma(tr_operand(dt, off_tq[db], q0 * C::ROW_BYTES), pf, dv_acc[db]);
          dk_acc[db] = E::mfma(tr_operand(qt, off_tq[db], q0 * C::ROW_BYTES), sf, dk_acc[db]);
        }
      }
    }

    prev_qb = qb;
    entry = next;
  };

  if (cnt > 0) issue_tile(entry, std::integral_constant<int, 0>{});
  // Unrolled by two so each buffer index is a compile-time constant.
  for (int it = 0; it < cnt; it += 2) {
    body(it, std::integral_constant<int, 0>{});
    if (it + 1 < cnt) body(it + 1, std::integral_constant<int, 1>{});
  }
  if (cnt > 0) {
    __syncthreads();
    if ((cnt - 1) & 1)
      dq_product(std::integral_constant<int, 1>{}, prev_qb);
    else
      dq_product(std::integral_constant<int, 0>{}, prev_qb);
  }

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

// D_i = sum_d dO_id O_id (float32), LSE_i * log2(e) (+inf for fully masked rows) and the dQ
// accumulator row cleared.  16 threads per row, one 16-byte chunk of O and dO each.
template <typename T, int D>
__global__ __launch_bounds__(256) void bwd_pre_kernel(const T* __restrict__ o,
                                                      const T* __restrict__ dout,
                                                      const float* __restrict__ lse,
                                                      float* __restrict__ delta,
                                                      float* __restrict__ lse2,
                                                      float* __restrict__ dq_acc, int64_t rows) {
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
  float4* z = reinterpret_cast<float4*>(dq_acc + row * D);
  constexpr int per = D / 4 / 16;  // float4 stores per thread
#pragma unroll
  for (int i = 0; i < per; ++i) z[c * per + i] = make_float4(0.f, 0.f, 0.f, 0.f);
}

template <typename T>
__global__ __launch_bounds__(256) void dq_convert_kernel(const float* __restrict__ acc,
                                                         T* __restrict__ dq, float scale,
                                                         int64_t n4) {
  const int64_t stride = (int64_t)gridDim.x * blockDim.x;
  for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < n4; i += stride) {
    const float4 x = reinterpret_cast<const float4*>(acc)[i];
    if constexpr (sizeof(T) == 2) {
      uint2 out;
      out.x = pack_bf16x2(x.x * scale, x.y * scale);
      out.y = pack_bf16x2(x.z * scale, x.w * scale);
      reinterpret_cast<uint2*>(dq)[i] = out;
    } else {
      reinterpret_cast<float4*>(dq)[i] = make_float4(x.x * scale, x.y * scale, x.z * scale, x.w * scale);
    }
  }
}

template <typename T, int D>
size_t bwd_smem_bytes() {
  using C = BwdTile<T, D>;
  return 4 * C::TILE_BYTES + 2 * C::DS_BYTES + C::K_BYTES + sizeof(float) * 4 * C::BM;
}

template <typename T, int D>
hipError_t run_bwd(const BwdArgs& a, hipStream_t stream, hipEvent_t ev_begin, hipEvent_t ev_end) {
  const int64_t rows = (int64_t)a.B * a.H * a.nq;
  const int pre_grid = (int)((rows + 15) / 16);
  hipLaunchKernelGGL((bwd_pre_kernel<T, D>), dim3(pre_grid), dim3(256), 0, stream,
                     static_cast<const T*>(a.o), static_cast<const T*>(a.dout), a.lse, a.delta,
                     a.lse2, a.dq_acc, rows);
  hipError_t err = hipGetLastError();
  if (err != hipSuccess) return err;

  const size_t smem = bwd_smem_bytes<T, D>();
  // The main kernel uses more than 64 KiB of LDS; allow it on the current device.
  err = hipFuncSetAttribute(reinterpret_cast<const void*>(&attn_bwd_kernel<T, D>),
                            hipFuncAttributeMaxDynamicSharedMemorySize, (int)smem);
  if (err != hipSuccess) return err;
  const int64_t n_kb = (a.nk + 127) / 128;
  const int64_t grid = n_kb * a.B * a.H;
  if (ev_begin) (void)hipEventRecord(ev_begin, stream);
  hipLaunchKernelGGL((attn_bwd_kernel<T, D>), dim3((unsigned)grid), dim3(256), smem, stream, a);
  err = hipGetLastError();
  if (ev_end) (void)hipEventRecord(ev_end, stream);
  if (err != hipSuccess) return err;

  const int64_t n4 = rows * D / 4;
  int cgrid = (int)((n4 + 255) / 256);
  if (cgrid > 8192) cgrid = 8192;
  hipLaunchKernelGGL((dq_convert_kernel<T>), dim3(cgrid), dim3(256), 0, stream, a.dq_acc,
                     static_cast<T*>(a.dq), a.scale, n4);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_attn_bwd(int dtype, const BwdArgs& a, hipStream_t stream, hipEvent_t ev_begin,
                           hipEvent_t ev_end) {
  return dtype == 0 ? run_bwd<bf16, 128>(a, stream, ev_begin, ev_end)
                    : run_bwd<float, 64>(a, stream, ev_begin, ev_end);
}

}  // namespace fm
