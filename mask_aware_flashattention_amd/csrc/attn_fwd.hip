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
//     exchange with the lane 32 apart, and the O^T rescale is a per-lane scalar;
//   * K and V^T tiles are staged in LDS with padded rows; the next tile's global loads are in
//     flight in registers while the current tile computes.
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
  static constexpr int CPR = D / CH;              // chunks per K/V row
  static constexpr int K_LD = D + CH;             // padded K row (elements)
  static constexpr int VT_LD = BN + CH;           // padded V^T row (elements)
  static constexpr int NRB = BN / 32;             // 32-key row blocks of S^T
  static constexpr int NDB = D / 32;              // 32-wide d blocks of O^T
  static constexpr int QK_STEPS = D / KSTEP;
  static constexpr int PV_STEPS = BN / KSTEP;
  static_assert(CPR == 16, "thread mapping assumes 256-byte rows");
  static_assert(BN == 4 * (NT / CPR), "V staging: 4 keys per thread");
};

struct MaskEntry {
  int32_t s1;
  uint32_t len1;
  int32_t s2;
  uint32_t len2;
};

template <typename T, int D>
__global__ __launch_bounds__(256, 2) void attn_fwd_kernel(FwdArgs a) {
  using C = FwdTile<T, D>;
  using E = Elem<T>;
  using frag = typename E::frag;
  constexpr int KPL = C::KPL, KSTEP = C::KSTEP, CH = C::CH;

  __shared__ __attribute__((aligned(16))) T k_lds[C::BN * C::K_LD];
  __shared__ __attribute__((aligned(16))) T vt_lds[D * C::VT_LD];
  __shared__ __attribute__((aligned(16))) MaskEntry msk_lds[C::BN];

  const int tid = threadIdx.x;
  const int lane = tid & 63, w = tid >> 6, g = lane >> 5, l32 = lane & 31;

  const int n_qb = (a.nq + C::BM - 1) / C::BM;
  const int bh = blockIdx.x / n_qb;
  // Query blocks are visited last-first: under causal-like masks the later blocks have the
  // longest lists, so the longest work is dispatched first.
  const int qb = n_qb - 1 - (int)(blockIdx.x % n_qb);

  const T* __restrict__ Qp = static_cast<const T*>(a.q) + (size_t)bh * a.nq * D;
  const T* __restrict__ Kp = static_cast<const T*>(a.k) + (size_t)bh * a.nk * D;
  const T* __restrict__ Vp = static_cast<const T*>(a.v) + (size_t)bh * a.nk * D;

  const int q_row = qb * C::BM + w * 32 + l32;  // this lane's query row
  const bool row_ok = q_row < a.nq;

  // Q^T as the B operand of S^T = K Q^T: k-step s holds Q[q_row][s*KSTEP + g*KPL + 0..KPL).
  frag qf[C::QK_STEPS];
#pragma unroll
  for (int s = 0; s < C::QK_STEPS; ++s)
    qf[s] = row_ok ? E::load_frag(Qp + (size_t)q_row * D + s * KSTEP + g * KPL) : E::zero_frag();

  const int cnt = a.qcnt[qb];
  const int32_t* __restrict__ lst = a.qlist + (size_t)qb * a.list_stride;
  const int last_kb = (a.nk - 1) / C::BN;
  const bool ragged = (a.nk % C::BN) != 0;

  // staging map: chunk c of a 256-byte row; K rows r0 + 16*i; V keys 4*kq + i
  const int c = tid % C::CPR;
  const int r0 = tid / C::CPR;
  uint4 kreg[4], vreg[4];
  MaskEntry mreg = {0, 0u, 0, 0u};

  auto load_tile = [&](int entry) {
    const int kb = entry >> 1;
    const int key0 = kb * C::BN;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int kr = key0 + r0 + 16 * i;
      kreg[i] = kr < a.nk ? *reinterpret_cast<const uint4*>(Kp + (size_t)kr * D + c * CH)
                          : make_uint4(0, 0, 0, 0);
      const int vr = key0 + 4 * r0 + i;
      vreg[i] = vr < a.nk ? *reinterpret_cast<const uint4*>(Vp + (size_t)vr * D + c * CH)
                          : make_uint4(0, 0, 0, 0);
    }
    const bool test = (entry & 1) || (kb == last_kb && ragged);
    if (test && tid < C::BN) {
      const int j = key0 + tid;
      if (j < a.nk) {
        const int32_t lts = a.mask.lts[j], lte = a.mask.lte[j];
        const int32_t uts = a.mask.uts[j], ute = a.mask.ute[j];
        mreg = {lts, stretch_len(lts, lte), uts, stretch_len(uts, ute)};
      } else {
        mreg = {INT32_MIN, 0xffffffffu, 0, 0u};  // past the last key: masked for every row
      }
    }
  };

  auto store_tile = [&](bool test) {
#pragma unroll
    for (int i = 0; i < 4; ++i)
      *reinterpret_cast<uint4*>(&k_lds[(r0 + 16 * i) * C::K_LD + c * CH]) = kreg[i];
    if constexpr (sizeof(T) == 2) {
      // vreg[i] = V[4*r0 + i][8c .. 8c+8); write V^T[8c + e][4*r0 .. 4*r0+4)
      const uint32_t* v0 = reinterpret_cast<const uint32_t*>(&vreg[0]);
      const uint32_t* v1 = reinterpret_cast<const uint32_t*>(&vreg[1]);
      const uint32_t* v2 = reinterpret_cast<const uint32_t*>(&vreg[2]);
      const uint32_t* v3 = reinterpret_cast<const uint32_t*>(&vreg[3]);
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        const int wd = e >> 1;
        uint2 out;
        if ((e & 1) == 0) {
          out.x = (v0[wd] & 0xffffu) | (v1[wd] << 16);
          out.y = (v2[wd] & 0xffffu) | (v3[wd] << 16);
        } else {
          out.x = (v0[wd] >> 16) | (v1[wd] & 0xffff0000u);
          out.y = (v2[wd] >> 16) | (v3[wd] & 0xffff0000u);
        }
        *reinterpret_cast<uint2*>(&vt_lds[(8 * c + e) * C::VT_LD + 4 * r0]) = out;
      }
    } else {
      // vreg[i] = V[4*r0 + i][4c .. 4c+4) (fp32); write V^T[4c + e][4*r0 .. 4*r0+4)
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        uint4 out;
        out.x = reinterpret_cast<const uint32_t*>(&vreg[0])[e];
        out.y = reinterpret_cast<const uint32_t*>(&vreg[1])[e];
        out.z = reinterpret_cast<const uint32_t*>(&vreg[2])[e];
        out.w = reinterpret_cast<const uint32_t*>(&vreg[3])[e];
        *reinterpret_cast<uint4*>(&vt_lds[(4 * c + e) * C::VT_LD + 4 * r0]) = out;
      }
    }
    if (test && tid < C::BN) msk_lds[tid] = mreg;
  };

  f32x16 oacc[C::NDB];
#pragma unroll
  for (int db = 0; db < C::NDB; ++db)
#pragma unroll
    for (int r = 0; r < 16; ++r) oacc[db][r] = 0.0f;
  float m_run = -INFINITY;  // running max of scale*log2(e)*S for this lane's row
  float l_run = 0.0f;       // this lane's share of the running sum (its 32 keys of each tile)
  const float cexp = a.scale * kLog2e;

  if (cnt > 0) load_tile(lst[0]);

  for (int it = 0; it < cnt; ++it) {
    const int entry = lst[it];
    const int kb = entry >> 1;
    const bool test = (entry & 1) || (kb == last_kb && ragged);
    __syncthreads();  // every wave is done reading the previous tile
    store_tile(test);
    __syncthreads();
    if (it + 1 < cnt) load_tile(lst[it + 1]);  // in flight during this tile's compute

    // S^T = K Q^T: accumulator register r of group g in row block rb is key
    // rb*32 + perm_index(r, g) of the tile, column = this lane's query.
    f32x16 sacc[C::NRB];
#pragma unroll
    for (int rb = 0; rb < C::NRB; ++rb) {
#pragma unroll
      for (int r = 0; r < 16; ++r) sacc[rb][r] = 0.0f;
      const T* kp = &k_lds[(rb * 32 + row_source<KPL>(l32)) * C::K_LD + g * KPL];
#pragma unroll
      for (int s = 0; s < C::QK_STEPS; ++s)
        sacc[rb] = E::mfma(E::load_frag(kp + s * KSTEP), qf[s], sacc[rb]);
    }

    if (test) {
#pragma unroll
      for (int rb = 0; rb < C::NRB; ++rb)
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const MaskEntry me = msk_lds[rb * 32 + perm_index<KPL>(r, g)];
          if (in_stretch(q_row, me.s1, me.len1) || in_stretch(q_row, me.s2, me.len2))
            sacc[rb][r] = -INFINITY;
        }
    }

    float mx = -INFINITY;
#pragma unroll
    for (int rb = 0; rb < C::NRB; ++rb)
#pragma unroll
      for (int r = 0; r < 16; ++r) mx = fmaxf(mx, sacc[rb][r]);
    mx = fmaxf(mx, wave_xor32(mx));
    const float m_new = fmaxf(m_run, mx * cexp);
    const float m_use = m_new == -INFINITY ? 0.0f : m_new;
    const float alpha = fast_exp2(m_run - m_use);
    float psum = 0.0f;
#pragma unroll
    for (int rb = 0; rb < C::NRB; ++rb)
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const float p = fast_exp2(fmaf(sacc[rb][r], cexp, -m_use));
        sacc[rb][r] = p;
        psum += p;
      }
    l_run = l_run * alpha + psum;
    m_run = m_new;
    if (__ballot(alpha != 1.0f)) {
#pragma unroll
      for (int db = 0; db < C::NDB; ++db)
#pragma unroll
        for (int r = 0; r < 16; ++r) oacc[db][r] *= alpha;
    }

    // O^T += V^T P^T.  k-step t covers tile keys t*KSTEP + g*KPL + e, which are accumulator
    // registers (t*KPL)%16 + e of row block (t*KPL)/16.
#pragma unroll
    for (int t = 0; t < C::PV_STEPS; ++t) {
      frag pf;
      if constexpr (KPL == 1) {
        pf = sacc[t / 16][t % 16];
      } else {
#pragma unroll
        for (int e = 0; e < KPL; ++e) pf[e] = E::from_float(sacc[(t * KPL) / 16][(t * KPL) % 16 + e]);
      }
#pragma unroll
      for (int db = 0; db < C::NDB; ++db) {
        const T* vp = &vt_lds[(db * 32 + l32) * C::VT_LD + t * KSTEP + g * KPL];
        oacc[db] = E::mfma(E::load_frag(vp), pf, oacc[db]);
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
