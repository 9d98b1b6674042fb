// Mask-aware attention forward for gfx950: online-softmax attention that walks only the tiles
// a query block's list names (fully masked tiles are never loaded) and applies the row-interval
// test only in tiles listed as partly masked.
//
// Sources: "FlashMask-3 sends each GPU its mask without sending any mask" (learnaivisually.com),
// tile-classification paragraph; "FlashMask-3: Efficient and Expressive Mask-Aware Distributed
// Attention", abstract (mask-aware kernel in the FlashAttention line).  The Hopper design on the
// pages (warp-specialised TMA/WGMMA pipeline) is not used; this is a CDNA4 layout:
//
//   * one workgroup = 4 waves = one query block of BM = 128 rows against key tiles of BN = 64;
//     each wave owns 32 query rows, held in registers as the B operand of the score product;
//   * the score tile is computed transposed, S^T = K Q^T, on 32x32 MFMAs, with the K rows loaded
//     in a permuted order so that the probabilities P^T come out of the accumulator already laid
//     out as the B operand of O^T += V^T P^T: no shuffle and no LDS round trip for P;
//   * each lane owns one query row (a column of S^T), so the row max and row sum need a single
//     exchange with the lane 32 apart, and the O^T rescale is a per-lane scalar; the running
//     max is only moved when a row's max grows by more than 2^8, so rescales are rare;
//   * K (row-padded) and V (row-major, 16-byte chunks XOR-swizzled by row) are staged in LDS;
//     the V^T operand is read with the gfx950 LDS transpose read, so V is never transposed in
//     memory; the next tile's global loads are in flight while the current tile computes;
//   * in partly masked tiles each wave first turns the four vectors of the tile's keys into one
//     32-bit word per key (bit t = query row t of the wave is masked), so the per-score test is a
//     bit extract.
#include <math.h>

#include "fm_common.hpp"
#include "launch.hpp"

namespace fm {

namespace {

template <typename T, int D>
struct FwdTile {
  static constexpr int BM = 128, BN = 64, NT = 256;
  static constexpr int KPL = Elem<T>::KPL, KSTEP = 2 * KPL;
  static constexpr int CH = 16 / (int)sizeof(T);  // elements per 16-byte chunk
  static constexpr int CPR = D / CH;              // 16-byte chunks per K/V row
  static constexpr int K_LD = D + CH;             // padded K row (elements)
  static constexpr int NRB = BN / 32;             // 32-key row blocks of S^T
  static constexpr int NDB = D / 32;              // 32-wide d blocks of O^T
  static constexpr int QK_STEPS = D / KSTEP;
  static constexpr int PV_STEPS = BN / KSTEP;
  static constexpr int ROW_BYTES = D * (int)sizeof(T);
  static_assert(CPR == 16, "thread mapping assumes 256-byte rows");
  static_assert(BN == 4 * (NT / CPR), "staging: 4 rows per thread");
};

// 16-byte chunk c of V row `key` lives at chunk c ^ vswz(key): consecutive keys land in
// different bank groups, which keeps the transpose reads (4 keys x 4 chunks per 32 lanes)
// conflict-free on the 64-bank LDS.
template <typename T>
__device__ __host__ constexpr int vswz(int key) {
  return sizeof(T) == 2 ? 4 * (key & 3) : 0;
}

constexpr float kRescaleThreshold = 8.0f;  // log2 units

template <typename T, int D>
__global__ __launch_bounds__(256, 2) void attn_fwd_kernel(FwdArgs a) {
  using C = FwdTile<T, D>;
  using E = Elem<T>;
  using frag = typename E::frag;
  constexpr int KPL = C::KPL, KSTEP = C::KSTEP, CH = C::CH;

  __shared__ __attribute__((aligned(16))) T k_lds[C::BN * C::K_LD];
  __shared__ __attribute__((aligned(16))) T v_lds[C::BN * D];
  __shared__ __attribute__((aligned(16))) uint32_t mw_lds[4][C::BN];  // per wave, per key

  const int tid = threadIdx.x;
  const int lane = tid & 63, w = tid >> 6, g = lane >> 5, l32 = lane & 31;

  const int n_qb = (a.nq + C::BM - 1) / C::BM;
  const int work = xcd_contiguous_index(blockIdx.x, gridDim.x);
  const int bh = work / n_qb;
  // Query blocks in the order of a.order (longest lists first, neighbours kept together).
  const int qb = a.order[work % n_qb];

  const T* __restrict__ Qp = static_cast<const T*>(a.q) + (size_t)bh * a.nq * D;
  const T* __restrict__ Kp = static_cast<const T*>(a.k) + (size_t)bh * a.nk * D;
  const T* __restrict__ Vp = static_cast<const T*>(a.v) + (size_t)bh * a.nk * D;
  const buf_rsrc qbuf = make_buf(Qp, (uint32_t)a.nq * C::ROW_BYTES);
  const buf_rsrc kbuf = make_buf(Kp, (uint32_t)a.nk * C::ROW_BYTES);
  const buf_rsrc vbuf = make_buf(Vp, (uint32_t)a.nk * C::ROW_BYTES);

  const int q0w = qb * C::BM + w * 32;  // first query row of this wave
  const int q_row = q0w + l32;          // this lane's query row
  const bool row_ok = q_row < a.nq;
  const int cnt = a.qcnt[qb];
  if (cnt == 0) {
    // No listed tile: the block's rows are fully masked: O = 0, LSE = -inf (each lane clears
    // half of its row, 128 bytes).
    if (row_ok) {
      uint4* p = reinterpret_cast<uint4*>(static_cast<T*>(a.o) + ((size_t)bh * a.nq + q_row) * D + g * (D / 2));
#pragma unroll
      for (int i = 0; i < 8; ++i) p[i] = make_uint4(0u, 0u, 0u, 0u);
      if (g == 0) a.lse[(size_t)bh * a.nq + q_row] = -INFINITY;
    }
    return;
  }

  // Q^T as the B operand of S^T = K Q^T: k-step s holds Q[q_row][s*KSTEP + g*KPL + 0..KPL).
  frag qf[C::QK_STEPS];
#pragma unroll
  for (int s = 0; s < C::QK_STEPS; ++s) {
    const uint32_t off = (uint32_t)q_row * C::ROW_BYTES + (uint32_t)(s * KSTEP + g * KPL) * sizeof(T);
    if constexpr (KPL == 8) {
      qf[s] = __builtin_bit_cast(frag, buf_load16(qbuf, off, 0));
    } else {
      qf[s] = __builtin_bit_cast(frag, buf_load4(qbuf, off, 0));
    }
  }

  const int32_t* __restrict__ lst = a.qlist + (size_t)qb * a.list_stride;
  const int last_kb = (a.nk - 1) / C::BN;
  const bool ragged = (a.nk % C::BN) != 0;

  // staging map: chunk c of a 256-byte row; K rows r0 + 16*i, V rows r0 + 16*i
  const int c = tid % C::CPR;
  const int r0 = tid / C::CPR;
  const uint32_t lane_off = (uint32_t)r0 * C::ROW_BYTES + (uint32_t)c * 16;
  const int mkey = tid & 63;  // mask word: key mkey of the tile, for wave w's 32 rows
  uint4 kreg[4], vreg[4];
  uint32_t mword = 0;

  auto load_tile = [&](int entry) {
    const int kb = entry >> 1;
    const uint32_t tile_off = (uint32_t)kb * C::BN * C::ROW_BYTES;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      kreg[i] = buf_load16(kbuf, lane_off + i * 16 * C::ROW_BYTES, tile_off);
      vreg[i] = buf_load16(vbuf, lane_off + i * 16 * C::ROW_BYTES, tile_off);
    }
    const bool test = (entry & 1) || (kb == last_kb && ragged);
    if (test) {
      const int j = kb * C::BN + mkey;
      if (j < a.nk) {
        // rows [q0w, q0w + 32) of this wave inside [s, e): bits [lo, hi)
        auto bits = [&](int32_t s, int32_t e) -> uint32_t {
          const int32_t lo = s <= q0w ? 0 : (s >= q0w + 32 ? 32 : s - q0w);
          const int32_t hi = e <= q0w ? 0 : (e >= q0w + 32 ? 32 : e - q0w);
          if (hi <= lo) return 0u;
          const uint32_t upto_hi = hi >= 32 ? 0xffffffffu : ((1u << hi) - 1u);
          const uint32_t upto_lo = (1u << lo) - 1u;  // lo < 32 here
          return upto_hi & ~upto_lo;
        };
        mword = bits(a.mask.lts[j], a.mask.lte[j]) | bits(a.mask.uts[j], a.mask.ute[j]);
      } else {
        mword = 0xffffffffu;  // past the last key: masked for every row
      }
    }
  };

  auto store_tile = [&](bool test) {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int row = r0 + 16 * i;
      *reinterpret_cast<uint4*>(&k_lds[row * C::K_LD + c * CH]) = kreg[i];
      *reinterpret_cast<uint4*>(&v_lds[row * D + (c ^ vswz<T>(row)) * CH]) = vreg[i];
    }
    if (test) mw_lds[w][mkey] = mword;
  };

  f32x16 oacc[C::NDB];
#pragma unroll
  for (int db = 0; db < C::NDB; ++db)
#pragma unroll
    for (int r = 0; r < 16; ++r) oacc[db][r] = 0.0f;
  float m_run = -INFINITY;  // reference max (scale*log2(e) units) for this lane's row
  float l_run = 0.0f;       // this lane's share of the running sum (its 32 keys of each tile)
  const float cexp = a.scale * kLog2e;

  // transpose-read address of the V^T operand (bf16): lane i of 16-lane block b reads
  // V[k0 + i/4][m0 + 4*(i%4)] with m0 = 16*(b%2) + 32*db, k0 = t*KSTEP + 8*(b/2) (+4).
  const int tb = lane >> 4, ti = lane & 15;
  const int tr_krow = 8 * (tb >> 1) + (ti >> 2);  // + t*KSTEP (+4)
  const int tr_col = 16 * (tb & 1) + 4 * (ti & 3);  // + 32*db (elements)

  // List entries are read into scalar registers (the buffer loads take the tile offset as a
  // scalar operand).
  if (cnt > 0) load_tile(__builtin_amdgcn_readfirstlane(lst[0]));

  for (int it = 0; it < cnt; ++it) {
    const int entry = __builtin_amdgcn_readfirstlane(lst[it]);
    const int kb = entry >> 1;
    const bool test = (entry & 1) || (kb == last_kb && ragged);
    __syncthreads();  // every wave is done reading the previous tile
    store_tile(test);
    __syncthreads();
    if (it + 1 < cnt) load_tile(__builtin_amdgcn_readfirstlane(lst[it + 1]));

    // S^T = K Q^T: accumulator register r of group g in row block rb is key
    // rb*32 + perm_index(r, g) of the tile, column = this lane's query.
    f32x16 sacc[C::NRB];
#pragma unroll
    for (int rb = 0; rb < C::NRB; ++rb) {
      const T* kp = &k_lds[(rb * 32 + row_source<KPL>(l32)) * C::K_LD + g * KPL];
      sacc[rb] = E::mfma(E::load_frag(kp), qf[0], f32x16{});
#pragma unroll
      for (int s = 1; s < C::QK_STEPS; ++s)
        sacc[rb] = E::mfma(E::load_frag(kp + s * KSTEP), qf[s], sacc[rb]);
    }

    if (test) {
      // keys rb*32 + (r/KPL)*2*KPL + g*KPL + r%KPL: runs of KPL consecutive keys
#pragma unroll
      for (int rb = 0; rb < C::NRB; ++rb)
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const uint32_t word = mw_lds[w][rb * 32 + perm_index<KPL>(r, g)];
          sacc[rb][r] = ((word >> l32) & 1u) ? -INFINITY : sacc[rb][r];
        }
    }

    float mx = -INFINITY;
#pragma unroll
    for (int rb = 0; rb < C::NRB; ++rb)
#pragma unroll
      for (int r = 0; r < 16; ++r) mx = fmaxf(mx, sacc[rb][r]);
    mx = fmaxf(mx, wave_xor32(mx)) * cexp;
    // Move the reference max only when it grows by more than the threshold: probabilities
    // then stay below 2^threshold and the O rescale (a pass over 64 registers) is rare.
    const bool grow = mx > m_run + kRescaleThreshold;
    if (__ballot(grow)) {
      const float m_new = grow ? mx : m_run;
      const float alpha = grow ? fast_exp2(m_run - mx) : 1.0f;  // 0 when m_run = -inf
      l_run *= alpha;
#pragma unroll
      for (int db = 0; db < C::NDB; ++db)
#pragma unroll
        for (int r = 0; r < 16; ++r) oacc[db][r] *= alpha;
      m_run = m_new;
    }
    const float m_use = m_run == -INFINITY ? 0.0f : m_run;

    // P^T (exp2 of the scaled scores) as operand fragments; the row sum stays in fp32 (a sum of
    // bf16-rounded values would cost up to 2^-9 relative on short rows, too much for the LSE).
    frag pf[C::PV_STEPS];
#pragma unroll
    for (int t = 0; t < C::PV_STEPS; ++t) {
#pragma unroll
      for (int e = 0; e < KPL; ++e) {
        const int rb = (t * KPL) / 16, r = (t * KPL) % 16 + e;
        const float p = fast_exp2(fmaf(sacc[rb][r], cexp, -m_use));
        l_run += p;
        if constexpr (KPL == 1) {
          pf[t] = p;
        } else {
          pf[t][e] = E::from_float(p);
        }
      }
    }

    // O^T += V^T P^T.  k-step t covers tile keys t*KSTEP + g*KPL + e.
#pragma unroll
    for (int t = 0; t < C::PV_STEPS; ++t) {
#pragma unroll
      for (int db = 0; db < C::NDB; ++db) {
        frag vf;
        if constexpr (KPL == 8) {
          const int k0 = t * KSTEP + tr_krow;
          const int col = 32 * db + tr_col;
          const int ch = col / 8, half = (col % 8) / 4;
          const T* p0 = &v_lds[k0 * D + ((ch ^ vswz<T>(k0)) * CH) + half * 4];
          const T* p1 = &v_lds[(k0 + 4) * D + ((ch ^ vswz<T>(k0 + 4)) * CH) + half * 4];
          const s16x4 lo = lds_read_tr16(p0), hi = lds_read_tr16(p1);
          vf = __builtin_bit_cast(frag, __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7));
        } else {
          vf = v_lds[(t * KSTEP + g) * D + 32 * db + l32];
        }
        oacc[db] = E::mfma(vf, pf[t], oacc[db]);
      }
    }
  }

  const float l = l_run + wave_xor32(l_run);
  if (row_ok) {
    const float inv = l > 0.0f ? 1.0f / l : 0.0f;
    if (g == 0)
      a.lse[(size_t)bh * a.nq + q_row] = l > 0.0f ? (m_run + log2f(l)) * kLn2 : -INFINITY;
    T* orow = static_cast<T*>(a.o) + ((size_t)bh * a.nq + q_row) * D;
#pragma unroll
    for (int db = 0; db < C::NDB; ++db)
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int d0 = db * 32 + 8 * i + 4 * g;
        if constexpr (sizeof(T) == 2) {
          uint2 out;
          out.x = pack_bf16x2(oacc[db][4 * i + 0] * inv, oacc[db][4 * i + 1] * inv);
          out.y = pack_bf16x2(oacc[db][4 * i + 2] * inv, oacc[db][4 * i + 3] * inv);
          *reinterpret_cast<uint2*>(orow + d0) = out;
        } else {
          float4 out = make_float4(oacc[db][4 * i + 0] * inv, oacc[db][4 * i + 1] * inv,
                                   oacc[db][4 * i + 2] * inv, oacc[db][4 * i + 3] * inv);
          *reinterpret_cast<float4*>(orow + d0) = out;
        }
      }
  }
}

}  // namespace

TileShape tile_shape(int dtype) {
  (void)dtype;
  return TileShape{FwdTile<bf16, 128>::BM, FwdTile<bf16, 128>::BN, 64, 128};
}

hipError_t launch_attn_fwd(int dtype, const FwdArgs& a, hipStream_t stream, hipEvent_t ev_begin,
                           hipEvent_t ev_end) {
  const int64_t n_qb = (a.nq + 127) / 128;
  const int64_t grid = n_qb * a.B * a.H;
  if (ev_begin) (void)hipEventRecord(ev_begin, stream);
  if (dtype == 0)
    hipLaunchKernelGGL((attn_fwd_kernel<bf16, 128>), dim3((unsigned)grid), dim3(256), 0, stream, a);
  else
    hipLaunchKernelGGL((attn_fwd_kernel<float, 64>), dim3((unsigned)grid), dim3(256), 0, stream, a);
  const hipError_t err = hipGetLastError();
  if (ev_end) (void)hipEventRecord(ev_end, stream);
  return err;
}

}  // namespace fm
