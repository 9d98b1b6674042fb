// Mask-aware attention backward for gfx950.
//
// The pages report the backward's speed ("FlashMask-3 ..." zicq.com summary, end-to-end
// paragraph) but do not describe it; this is the standard recompute-from-LSE backward restricted
// to the tiles the classification lists (fully masked tiles skipped, the row test only in
// partly masked tiles, as the forward; "FlashMask-3 sends each GPU its mask ...",
// tile-classification paragraph).
//
//   K4 bwd_pre:  D_i = sum_d dO_id O_id, and the float32 dQ accumulator cleared.
//   K5 bwd_main: one workgroup per key block of BN = 128 keys (4 waves x 32 keys); K and V rows
//                stay in registers, dK^T and dV^T accumulate in registers; the workgroup walks
//                the query blocks (BM = 64 rows) of its list.  Per tile:
//                  S = Q K^T and dP = dO V^T (query rows loaded in a permuted order so the
//                  accumulators double as operands), P = exp2(S*scale*log2e - LSE*log2e),
//                  dS = P (dP - D); dV^T += dO^T P; dK^T += Q^T dS; then dS goes through LDS
//                  (keys contiguous) and dQ += dS K is added to the float32 accumulator with
//                  atomics.
//   K6 dq_convert: dQ = scale * accumulator, rounded to the output dtype.
#include <math.h>

#include "fm_common.hpp"
#include "launch.hpp"

namespace fm {

namespace {

template <typename T, int D>
struct BwdTile {
  static constexpr int BN = 128, BM = 64, NT = 256;
  static constexpr int KPL = Elem<T>::KPL, KSTEP = 2 * KPL;
  static constexpr int CH = 16 / (int)sizeof(T);
  static constexpr int CPR = D / CH;
  static constexpr int Q_LD = D + CH;    // Q, dO row-major [BM][Q_LD]
  static constexpr int QT_LD = BM + CH;  // Q^T, dO^T [D][QT_LD]
  static constexpr int DS_LD = BN + CH;  // dS [BM][DS_LD], keys contiguous
  static constexpr int KT_LD = BN + CH;  // K^T [D][KT_LD]
  static constexpr int NQB = BM / 32;
  static constexpr int NDB = D / 32;
  static constexpr int QK_STEPS = D / KSTEP;
  static constexpr int PQ_STEPS = BM / KSTEP;  // k-steps over a tile's queries
  static constexpr int DQ_STEPS = BN / KSTEP;  // k-steps over the block's keys
  static constexpr int NOB = NQB * NDB / 4;    // dQ output blocks per wave
  static_assert(CPR == 16, "thread mapping assumes 256-byte rows");
  static_assert(BM == 4 * (NT / CPR), "staging: 4 rows per thread");
  static_assert(NOB >= 1, "dQ split");
};

struct MaskRegs {
  int32_t s1;
  uint32_t len1;
  int32_t s2;
  uint32_t len2;
};

template <typename T, int D>
__global__ __launch_bounds__(256, 1) void attn_bwd_kernel(BwdArgs a) {
  using C = BwdTile<T, D>;
  using E = Elem<T>;
  using frag = typename E::frag;
  constexpr int KPL = C::KPL, KSTEP = C::KSTEP, CH = C::CH;

  extern __shared__ __attribute__((aligned(16))) unsigned char smem[];
  T* q_lds = reinterpret_cast<T*>(smem);
  T* do_lds = q_lds + C::BM * C::Q_LD;
  T* qt_lds = do_lds + C::BM * C::Q_LD;
  T* dot_lds = qt_lds + D * C::QT_LD;
  T* ds_lds = dot_lds + D * C::QT_LD;
  T* kt_lds = ds_lds + C::BM * C::DS_LD;
  float* lse_lds = reinterpret_cast<float*>(kt_lds + D * C::KT_LD);
  float* dlt_lds = lse_lds + C::BM;

  const int tid = threadIdx.x;
  const int lane = tid & 63, w = tid >> 6, g = lane >> 5, l32 = lane & 31;

  const int n_kb = (a.nk + C::BN - 1) / C::BN;
  const int bh = blockIdx.x / n_kb;
  const int kb = n_kb - 1 - (int)(blockIdx.x % n_kb);
  const int key = kb * C::BN + w * 32 + l32;  // this lane's key (a column of S)
  const bool key_ok = key < a.nk;

  const T* __restrict__ Qp = static_cast<const T*>(a.q) + (size_t)bh * a.nq * D;
  const T* __restrict__ dOp = static_cast<const T*>(a.dout) + (size_t)bh * a.nq * D;
  const T* __restrict__ Kp = static_cast<const T*>(a.k) + (size_t)bh * a.nk * D;
  const T* __restrict__ Vp = static_cast<const T*>(a.v) + (size_t)bh * a.nk * D;
  const float* __restrict__ lse = a.lse + (size_t)bh * a.nq;
  const float* __restrict__ dlt = a.delta + (size_t)bh * a.nq;
  float* __restrict__ dqa = a.dq_acc + (size_t)bh * a.nq * D;

  // K and V rows of this lane's key as B operands (k-step s: d = s*KSTEP + g*KPL + 0..KPL).
  frag kf[C::QK_STEPS], vf[C::QK_STEPS];
#pragma unroll
  for (int s = 0; s < C::QK_STEPS; ++s) {
    kf[s] = key_ok ? E::load_frag(Kp + (size_t)key * D + s * KSTEP + g * KPL) : E::zero_frag();
    vf[s] = key_ok ? E::load_frag(Vp + (size_t)key * D + s * KSTEP + g * KPL) : E::zero_frag();
  }
  MaskRegs mk;
  if (key_ok) {
    const int32_t lts = a.mask.lts[key], lte = a.mask.lte[key];
    const int32_t uts = a.mask.uts[key], ute = a.mask.ute[key];
    mk = {lts, stretch_len(lts, lte), uts, stretch_len(uts, ute)};
  } else {
    mk = {INT32_MIN, 0xffffffffu, 0, 0u};
  }
  const bool ragged_block = (kb == n_kb - 1) && (a.nk % C::BN) != 0;

  const int c = tid % C::CPR;
  const int rq = tid / C::CPR;  // staging: rows 4*rq + i

  // K^T of the whole key block into LDS once (operand of dQ += dS K).
  for (int i = 0; i < C::BN / 16; ++i) {
    // thread covers key kb*BN + 16*i + rq ... one 16-byte chunk each
    const int kl = 16 * i + rq;
    const int kr = kb * C::BN + kl;
    uint4 x = kr < a.nk ? *reinterpret_cast<const uint4*>(Kp + (size_t)kr * D + c * CH)
                        : make_uint4(0, 0, 0, 0);
    const T* xe = reinterpret_cast<const T*>(&x);
#pragma unroll
    for (int e = 0; e < CH; ++e) kt_lds[(c * CH + e) * C::KT_LD + kl] = xe[e];
  }

  f32x16 dv_acc[C::NDB], dk_acc[C::NDB];
#pragma unroll
  for (int db = 0; db < C::NDB; ++db)
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      dv_acc[db][r] = 0.0f;
      dk_acc[db][r] = 0.0f;
    }

  const int cnt = a.kcnt[kb];
  const int32_t* __restrict__ lst = a.klist + (size_t)kb * a.list_stride;
  const float cexp = a.scale * kLog2e;

  uint4 qreg[4], doreg[4];
  float lse_r = INFINITY, dlt_r = 0.0f;
  auto load_tile = [&](int entry) {
    const int qb = entry >> 1;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int r = qb * C::BM + 4 * rq + i;
      const bool ok = r < a.nq;
      qreg[i] = ok ? *reinterpret_cast<const uint4*>(Qp + (size_t)r * D + c * CH) : make_uint4(0, 0, 0, 0);
      doreg[i] = ok ? *reinterpret_cast<const uint4*>(dOp + (size_t)r * D + c * CH) : make_uint4(0, 0, 0, 0);
    }
    if (tid < C::BM) {
      const int r = qb * C::BM + tid;
      if (r < a.nq) {
        const float x = lse[r];
        // a fully masked row (LSE = -inf) must give P = 0: exp2(s - inf) = 0
        lse_r = x == -INFINITY ? INFINITY : x * kLog2e;
        dlt_r = dlt[r];
      } else {
        lse_r = INFINITY;
        dlt_r = 0.0f;
      }
    }
  };

  auto store_rows = [&](T* rm, T* tr, const uint4* regs) {
#pragma unroll
    for (int i = 0; i < 4; ++i)
      *reinterpret_cast<uint4*>(&rm[(4 * rq + i) * C::Q_LD + c * CH]) = regs[i];
    if constexpr (sizeof(T) == 2) {
      const uint32_t* v0 = reinterpret_cast<const uint32_t*>(&regs[0]);
      const uint32_t* v1 = reinterpret_cast<const uint32_t*>(&regs[1]);
      const uint32_t* v2 = reinterpret_cast<const uint32_t*>(&regs[2]);
      const uint32_t* v3 = reinterpret_cast<const uint32_t*>(&regs[3]);
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
        *reinterpret_cast<uint2*>(&tr[(8 * c + e) * C::QT_LD + 4 * rq]) = out;
      }
    } else {
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        uint4 out;
        out.x = reinterpret_cast<const uint32_t*>(&regs[0])[e];
        out.y = reinterpret_cast<const uint32_t*>(&regs[1])[e];
        out.z = reinterpret_cast<const uint32_t*>(&regs[2])[e];
        out.w = reinterpret_cast<const uint32_t*>(&regs[3])[e];
        *reinterpret_cast<uint4*>(&tr[(4 * c + e) * C::QT_LD + 4 * rq]) = out;
      }
    }
  };

  if (cnt > 0) load_tile(lst[0]);

  for (int it = 0; it < cnt; ++it) {
    const int entry = lst[it];
    const int qb = entry >> 1;
    const bool test = (entry & 1) || ragged_block;
    __syncthreads();  // previous tile fully consumed (including dS and the dQ product)
    store_rows(q_lds, qt_lds, qreg);
    store_rows(do_lds, dot_lds, doreg);
    if (tid < C::BM) {
      lse_lds[tid] = lse_r;
      dlt_lds[tid] = dlt_r;
    }
    __syncthreads();
    if (it + 1 < cnt) load_tile(lst[it + 1]);

    // S = Q K^T and dP = dO V^T.  Register r of group g in query row block qr is tile query
    // qr*32 + perm_index(r, g); the column is this lane's key.
    f32x16 sacc[C::NQB], pacc[C::NQB];
#pragma unroll
    for (int qr = 0; qr < C::NQB; ++qr) {
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        sacc[qr][r] = 0.0f;
        pacc[qr][r] = 0.0f;
      }
      const int row = qr * 32 + row_source<KPL>(l32);
      const T* qp = &q_lds[row * C::Q_LD + g * KPL];
      const T* dp = &do_lds[row * C::Q_LD + g * KPL];
#pragma unroll
      for (int s = 0; s < C::QK_STEPS; ++s) {
        sacc[qr] = E::mfma(E::load_frag(qp + s * KSTEP), kf[s], sacc[qr]);
        pacc[qr] = E::mfma(E::load_frag(dp + s * KSTEP), vf[s], pacc[qr]);
      }
    }

    // P and dS (overwriting sacc and pacc)
#pragma unroll
    for (int qr = 0; qr < C::NQB; ++qr)
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int ql = qr * 32 + perm_index<KPL>(r, g);
        float p = fast_exp2(fmaf(sacc[qr][r], cexp, -lse_lds[ql]));
        if (test) {
          const int32_t q = qb * C::BM + ql;
          if (in_stretch(q, mk.s1, mk.len1) || in_stretch(q, mk.s2, mk.len2)) p = 0.0f;
        }
        sacc[qr][r] = p;
        pacc[qr][r] = p * (pacc[qr][r] - dlt_lds[ql]);
      }

    // dV^T += dO^T P and dK^T += Q^T dS.  k-step t covers tile queries t*KSTEP + g*KPL + e,
    // registers (t*KPL)%16 + e of query row block (t*KPL)/16.
#pragma unroll
    for (int t = 0; t < C::PQ_STEPS; ++t) {
      frag pf, sf;
      if constexpr (KPL == 1) {
        pf = sacc[t / 16][t % 16];
        sf = pacc[t / 16][t % 16];
      } else {
#pragma unroll
        for (int e = 0; e < KPL; ++e) {
          pf[e] = E::from_float(sacc[(t * KPL) / 16][(t * KPL) % 16 + e]);
          sf[e] = E::from_float(pacc[(t * KPL) / 16][(t * KPL) % 16 + e]);
        }
      }
#pragma unroll
      for (int db = 0; db < C::NDB; ++db) {
        const int off = (db * 32 + l32) * C::QT_LD + t * KSTEP + g * KPL;
        dv_acc[db] = E::mfma(E::load_frag(&dot_lds[off]), pf, dv_acc[db]);
        dk_acc[db] = E::mfma(E::load_frag(&qt_lds[off]), sf, dk_acc[db]);
      }
    }

    // dS -> LDS as [query][key] (keys contiguous) for the dQ product.
#pragma unroll
    for (int qr = 0; qr < C::NQB; ++qr)
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int ql = qr * 32 + perm_index<KPL>(r, g);
        ds_lds[ql * C::DS_LD + w * 32 + l32] = E::from_float(pacc[qr][r]);
      }
    __syncthreads();

    // dQ[q][d] += sum_keys dS[q][key] K[key][d]; wave w owns NOB 32x32 output blocks.
#pragma unroll
    for (int ob = 0; ob < C::NOB; ++ob) {
      const int blk = w * C::NOB + ob;
      const int qr = blk % C::NQB, db = blk / C::NQB;
      f32x16 acc;
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[r] = 0.0f;
      const T* ap = &ds_lds[(qr * 32 + l32) * C::DS_LD + g * KPL];
      const T* bp = &kt_lds[(db * 32 + l32) * C::KT_LD + g * KPL];
#pragma unroll
      for (int t = 0; t < C::DQ_STEPS; ++t)
        acc = E::mfma(E::load_frag(ap + t * KSTEP), E::load_frag(bp + t * KSTEP), acc);
      // acc register r: query qr*32 + acc_row(r, g), d = db*32 + l32
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int q = qb * C::BM + qr * 32 + acc_row(r, g);
        if (q < a.nq) unsafeAtomicAdd(&dqa[(size_t)q * D + db * 32 + l32], acc[r]);
      }
    }
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

// D_i = sum_d dO_id O_id (float32) and the dQ accumulator row cleared.  16 threads per row,
// one 16-byte chunk of O and dO each.
template <typename T, int D>
__global__ __launch_bounds__(256) void bwd_pre_kernel(const T* __restrict__ o,
                                                      const T* __restrict__ dout,
                                                      float* __restrict__ delta,
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
  if (c == 0) delta[row] = acc;
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
  return sizeof(T) * (2 * C::BM * C::Q_LD + 2 * D * C::QT_LD + C::BM * C::DS_LD + D * C::KT_LD) +
         sizeof(float) * 2 * C::BM;
}

template <typename T, int D>
hipError_t run_bwd(const BwdArgs& a, hipStream_t stream, hipEvent_t ev_begin, hipEvent_t ev_end) {
  const int64_t rows = (int64_t)a.B * a.H * a.nq;
  const int pre_grid = (int)((rows + 15) / 16);
  hipLaunchKernelGGL((bwd_pre_kernel<T, D>), dim3(pre_grid), dim3(256), 0, stream,
                     static_cast<const T*>(a.o), static_cast<const T*>(a.dout), a.delta, a.dq_acc,
                     rows);
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
