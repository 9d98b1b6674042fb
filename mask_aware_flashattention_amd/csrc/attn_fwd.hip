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
//   * K and V tiles go from HBM straight into LDS (buffer loads into LDS, 16-byte chunks
//     XOR-swizzled by row), double-buffered with one barrier per tile; the next tile's loads are
//     in flight while the current tile computes; the V^T operand is read with the gfx950 LDS
//     transpose read, so V is never transposed in memory;
//   * the row max and the row sum are exchanged between the two lanes of a row with
//     v_permlane32_swap (registers only);
//   * in partly masked tiles each wave first turns the four vectors of the tile's keys into one
//     32-bit word per key (bit t = query row t of the wave is masked), so the per-score test is a
//     bit extract.
#include <math.h>

#include "fm_common.hpp"
#include "launch.hpp"

namespace fm {

FM_STAMP_ARRAY(g_stamps_fwd, flashmask_debug_stamps_fwd)

namespace {

template <typename T, int D>
struct FwdTile {
  static constexpr int BM = 128, BN = 64, NT = 256;
  static constexpr int KPL = Elem<T>::KPL, KSTEP = 2 * KPL;
  static constexpr int ROW_BYTES = D * (int)sizeof(T);
  static constexpr int NRB = BN / 32;             // 32-key row blocks of S^T
  static constexpr int NDB = D / 32;              // 32-wide d blocks of O^T
  static constexpr int QK_STEPS = D / KSTEP;      // k-steps of the score product
  static constexpr int PV_STEPS = BN / KSTEP;     // k-steps of the P V product
  static constexpr int TILE_BYTES = BN * ROW_BYTES;
  static constexpr int MW_BYTES = 4 * BN * 4;     // per wave, per key: one 32-bit row mask
  static_assert(ROW_BYTES == 256, "256-byte rows");
  static_assert(TILE_BYTES == 16 * 1024, "16 blocks of 1 KiB per tile");
};

constexpr float kRescaleThreshold = 8.0f;  // log2 units

template <typename T, int D>
__global__ __launch_bounds__(256, 2) void attn_fwd_kernel(FwdArgs a) {
  using C = FwdTile<T, D>;
  using E = Elem<T>;
  using frag = typename E::frag;
  constexpr int KPL = C::KPL, KSTEP = C::KSTEP;

  // LDS: two tile buffers [K | V] and two arrays of mask words.  They are separate arrays so
  // that the compiler can tell that loads into one buffer never overlap reads of the other or
  // the mask words, and adds no wait on the loads in flight before those accesses.
  __shared__ __attribute__((aligned(16))) unsigned char lds0[2 * C::TILE_BYTES];
  __shared__ __attribute__((aligned(16))) unsigned char lds1[2 * C::TILE_BYTES];
  __shared__ uint32_t mw0[C::MW_BYTES / 4];
  __shared__ uint32_t mw1[C::MW_BYTES / 4];
  auto bufp = [&](auto bc) -> unsigned char* {
    if constexpr (decltype(bc)::value == 0)
      return lds0;
    else
      return lds1;
  };
  auto mwp = [&](auto bc) -> uint32_t* {
    if constexpr (decltype(bc)::value == 0)
      return mw0;
    else
      return mw1;
  };

  WgStamps stamps;  // workgroup timeline (debug build only)
  const int tid = threadIdx.x;
  const int lane = tid & 63, g = lane >> 5, l32 = lane & 31;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);

  const int n_qb = (a.nq + C::BM - 1) / C::BM;
  const int work = xcd_contiguous_index(blockIdx.x, gridDim.x);
  // (readfirstlane keeps these workgroup-wide indices, and every pointer and buffer descriptor
  // derived from them, in scalar registers)
  const int bh = __builtin_amdgcn_readfirstlane(work / n_qb);
  const int b = __builtin_amdgcn_readfirstlane(bh / a.L.H), head = bh - b * a.L.H;
  const int set = mask_set(a.L, b, head);
  // Query blocks in the order of a.order (longest lists first, neighbours kept together).
  const int qb = a.order[(size_t)set * n_qb + work % n_qb];

  const T* __restrict__ Qp = static_cast<const T*>(a.q) + b * a.L.qs_b + head * a.L.qs_h;
  const T* __restrict__ Kp = static_cast<const T*>(a.k) + b * a.L.ks_b + (head / a.L.G) * a.L.ks_h;
  const T* __restrict__ Vp = static_cast<const T*>(a.v) + b * a.L.ks_b + (head / a.L.G) * a.L.ks_h;
  const uint32_t qrs = (uint32_t)a.L.qs_r * sizeof(T);  // row strides in bytes
  const uint32_t krs = (uint32_t)a.L.ks_r * sizeof(T);
  const buf_rsrc qbuf = make_buf(Qp, (uint32_t)(a.nq - 1) * qrs + C::ROW_BYTES);
  const buf_rsrc kbuf = make_buf(Kp, (uint32_t)(a.nk - 1) * krs + C::ROW_BYTES);
  const buf_rsrc vbuf = make_buf(Vp, (uint32_t)(a.nk - 1) * krs + C::ROW_BYTES);
  const MaskVecs mask{a.mask.lts + set * a.L.mask_stride, a.mask.lte + set * a.L.mask_stride,
                      a.mask.uts + set * a.L.mask_stride, a.mask.ute + set * a.L.mask_stride};
  T* const Op = static_cast<T*>(a.o) + b * a.L.qs_b + head * a.L.qs_h;
  float* const lse_row = a.lse + (size_t)bh * a.nq;

  const int q0w = qb * C::BM + w * 32;  // first query row of this wave
  const int q_row = q0w + l32;          // this lane's query row
  const bool row_ok = q_row < a.nq;
  const int cnt = a.qcnt[(size_t)set * n_qb + qb];
  if (cnt == 0) {
    // No listed tile: the block's rows are fully masked: O = 0, LSE = -inf (each lane clears
    // half of its row, 128 bytes).
    if (row_ok) {
      uint4* p = reinterpret_cast<uint4*>(Op + (size_t)q_row * a.L.qs_r + g * (D / 2));
#pragma unroll
      for (int i = 0; i < 8; ++i) p[i] = make_uint4(0u, 0u, 0u, 0u);
      if (g == 0) lse_row[q_row] = -INFINITY;
    }
    stamps.store(FM_STAMP_BUF(g_stamps_fwd), 0);
    return;
  }

  // Q^T as the B operand of S^T = K Q^T: k-step s holds Q[q_row][s*KSTEP + g*KPL + 0..KPL);
  // rows past nq read as zeros.
  frag qf[C::QK_STEPS];
#pragma unroll
  for (int s = 0; s < C::QK_STEPS; ++s) {
    const uint32_t off = (uint32_t)q_row * qrs + (uint32_t)(s * KSTEP + g * KPL) * sizeof(T);
    if constexpr (KPL == 8) {
      qf[s] = __builtin_bit_cast(frag, buf_load16(qbuf, off, 0));
    } else {
      qf[s] = __builtin_bit_cast(frag, buf_load4(qbuf, off, 0));
    }
  }

  const int32_t* __restrict__ lst = a.qlist + ((size_t)set * n_qb + qb) * a.list_stride;
  const int last_kb = (a.nk - 1) / C::BN;
  const bool ragged = (a.nk % C::BN) != 0;
  const float cexp = a.scale * kLog2e;

  // Per-lane LDS byte offsets; the swizzle depends on row & 15 only, so row blocks of 16 keys
  // share them.  K operand of S^T: the permuted row source of lane l32, k-step s.  V^T operand:
  // transpose-read rows (tr_row, tr_row + 4) and columns 32*db + tr_col of a 16-key step (fp32:
  // row g, column 32*db + l32 of a 2-key step).
  int off_k[C::QK_STEPS];
  int off_v[C::NDB][2];
  {
    const int srow = row_source<KPL>(l32);
#pragma unroll
    for (int s = 0; s < C::QK_STEPS; ++s)
      off_k[s] = tile_off<T, 0>(srow, s * KSTEP + g * KPL, C::ROW_BYTES);
    const int tb = lane >> 4, ti = lane & 15;
    const int tr_row = 8 * (tb >> 1) + (ti >> 2);
    const int tr_col = 16 * (tb & 1) + 4 * (ti & 3);
#pragma unroll
    for (int h = 0; h < 2; ++h)
#pragma unroll
      for (int db = 0; db < C::NDB; ++db)
        off_v[db][h] = KPL == 8 ? tile_off<T, 0>(tr_row + 4 * h, 32 * db + tr_col, C::ROW_BYTES)
                                : tile_off<T, 0>(g, 32 * db + l32, C::ROW_BYTES);
  }

  // Stage key tile `entry` into buffer `bufc`: K then V, 16 blocks of 1 KiB each, wave w fills
  // blocks 4w..4w+3 (lane l: row 4j + l/16, physical chunk l%16 = logical chunk
  // (l%16) ^ swz_row(row)); keys past nk read as zeros.  Part i is one K and one V block; the
  // parts are spread over the score products, because eight waves issuing their loads at once
  // stall in order on the full memory queue before any of them reaches its products.
  auto stage_part = [&](int entry, auto bufc, int i) {
    unsigned char* kt = bufp(bufc);
    const uint32_t tile_base = (uint32_t)(entry >> 1) * C::BN * krs;
    const int j = 4 * w + i;
    const int row = 4 * j + (lane >> 4);
    const uint32_t voff = (uint32_t)row * krs + (uint32_t)(((lane & 15) ^ swz_row<T>(row)) * 16);
    buf_load_lds<16>(kbuf, kt + j * 1024, voff, tile_base);
    buf_load_lds<16>(vbuf, kt + C::TILE_BYTES + j * 1024, voff, tile_base);
  };
  // Row mask of a partly masked tile: lane l loads the four vectors at key l of the tile early
  // and writes the word for this wave's 32 rows (bit t = row q0w + t masked) late, so the wait
  // for the vectors does not hold up the products in between.
  struct MaskKey {
    int32_t s0, e0, s1, e1;
    bool live;
  };
  auto mask_load = [&](int entry) {
    MaskKey m{0, 0, 0, 0, false};
    const int jk = (entry >> 1) * C::BN + lane;
    m.live = jk < a.nk;  // keys past nk are masked for every row
    if (m.live) {
      m.s0 = mask.lts[jk];
      m.e0 = mask.lte[jk];
      m.s1 = mask.uts[jk];
      m.e1 = mask.ute[jk];
    }
    return m;
  };
  auto mask_store = [&](const MaskKey& m, auto bufc) {
    // rows [q0w, q0w + 32) inside [s, e): bits [lo, hi)
    auto bits = [&](int32_t s, int32_t e) -> uint32_t {
      const int32_t lo = s <= q0w ? 0 : (s >= q0w + 32 ? 32 : s - q0w);
      const int32_t hi = e <= q0w ? 0 : (e >= q0w + 32 ? 32 : e - q0w);
      if (hi <= lo) return 0u;
      const uint32_t upto_hi = hi >= 32 ? 0xffffffffu : ((1u << hi) - 1u);
      return upto_hi & ~((1u << lo) - 1u);  // lo < 32 here
    };
    mwp(bufc)[w * C::BN + lane] = m.live ? (bits(m.s0, m.e0) | bits(m.s1, m.e1)) : 0xffffffffu;
  };
  auto is_test = [&](int entry) { return (entry & 1) || ((entry >> 1) == last_kb && ragged); };

  f32x16 oacc[C::NDB];
#pragma unroll
  for (int db = 0; db < C::NDB; ++db) oacc[db] = f32x16{};
  float m_run = -INFINITY;  // reference max (scale*log2(e) units) for this lane's row
  float l_run = 0.0f;       // this lane's share of the running sum (its 32 keys of each tile)

  // List entries are read one tile ahead of their use (scalar loads: their latency then hides
  // behind a tile instead of stalling the wave, and behind a barrier that waits for them anyway).
  int entry = load_uniform(lst, 0);
  int pre = load_uniform(lst, cnt > 1 ? 1 : 0);  // entry of the tile after `entry`

  auto body = [&](const int it, auto bufc) {
    constexpr int buf = decltype(bufc)::value;
    const auto other = std::integral_constant<int, buf ^ 1>{};
    const bool test = is_test(entry);
    // The last tile stages its own rows again into the free buffer, which is never read: the
    // staging then needs no branch inside the products.
    const bool has_next = it + 1 < cnt;
    const int next = has_next ? pre : entry;
    pre = load_uniform(lst, it + 2 < cnt ? it + 2 : cnt - 1);
    const bool next_test = has_next && is_test(next);
    wait_vmem();      // this wave's loads of tile `it` have landed in LDS
    __syncthreads();  // ... everyone's, and the mask words; the other buffer is free
    if (it == 0) stamps.first_tile();
    MaskKey mk{0, 0, 0, 0, false};
    if (next_test) mk = mask_load(next);

    const unsigned char* kt = bufp(bufc);
    const unsigned char* vt = kt + C::TILE_BYTES;

    // S^T = K Q^T: register r of group g in row block rb is tile key rb*32 + perm_index(r, g);
    // the column is this lane's query.  The two row blocks' products alternate (independent
    // accumulators), and the K reads run six products ahead of their use.
    f32x16 sacc[C::NRB];
#pragma unroll
    for (int rb = 0; rb < C::NRB; ++rb) sacc[rb] = f32x16{};
#pragma unroll
    for (int st = 0; st < C::QK_STEPS; ++st)
#pragma unroll
      for (int rb = 0; rb < C::NRB; ++rb) {
        sacc[rb] = E::mfma(*reinterpret_cast<const frag*>(kt + off_k[st] + rb * 32 * C::ROW_BYTES),
                           qf[st], sacc[rb]);
        constexpr int every = C::QK_STEPS * C::NRB / 4;
        if ((st * C::NRB + rb) % every == every - 1) stage_part(next, other, (st * C::NRB + rb) / every);
      }
    if constexpr (KPL == 8) sched_mfma_reads_ahead<C::QK_STEPS * C::NRB, 1, 6>();

    if (test) {
      const uint32_t* mw = mwp(bufc) + w * C::BN;
#pragma unroll
      for (int rb = 0; rb < C::NRB; ++rb)
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          const uint32_t word = mw[rb * 32 + perm_index<KPL>(r, g)];
          sacc[rb][r] = select_bit(word, l32, sacc[rb][r], kNegInfBits);
        }
    }

    float mx = -INFINITY;
#pragma unroll
    for (int rb = 0; rb < C::NRB; ++rb)
#pragma unroll
      for (int r = 0; r < 16; ++r) mx = fmaxf(mx, sacc[rb][r]);
    mx = pair_max32(mx) * cexp;
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

    // P^T (exp2 of the scaled scores) as operand fragments: k-step t covers tile keys
    // t*KSTEP + g*KPL + e = registers (t*KPL)%16 + e of row block (t*KPL)/16.  The row sum stays
    // in fp32 (a sum of bf16-rounded values would cost up to 2^-9 relative on short rows, too
    // much for the LSE).
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

    // O^T += V^T P^T (contraction over the tile's keys; V^T read with the transpose read).
#pragma unroll
    for (int t = 0; t < C::PV_STEPS; ++t) {
      const int k0_bytes = t * KSTEP * C::ROW_BYTES;
#pragma unroll
      for (int db = 0; db < C::NDB; ++db) {
        frag vf;
        if constexpr (KPL == 8) {
          const s16x4 lo = lds_read_tr16(vt + off_v[db][0] + k0_bytes);
          const s16x4 hi = lds_read_tr16(vt + off_v[db][1] + k0_bytes);
          vf = __builtin_bit_cast(frag, __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7));
        } else {
          vf = *reinterpret_cast<const T*>(vt + off_v[db][0] + k0_bytes);
        }
        oacc[db] = E::mfma(vf, pf[t], oacc[db]);
      }
    }
    if constexpr (KPL == 8) sched_mfma_reads_ahead<C::PV_STEPS * C::NDB, 2, 3>();  // V^T 3 ahead
    if (next_test) mask_store(mk, other);
    entry = next;
  };

  {
    const auto first = std::integral_constant<int, 0>{};
#pragma unroll
    for (int i = 0; i < 4; ++i) stage_part(entry, first, i);
    if (is_test(entry)) mask_store(mask_load(entry), first);
  }
  // Unrolled by two so each buffer index is a compile-time constant; an odd last tile runs after
  // the loop, so the loop body has no conditional path the accumulators must merge across.
  int it = 0;
  for (; it + 1 < cnt; it += 2) {
    body(it, std::integral_constant<int, 0>{});
    body(it + 1, std::integral_constant<int, 1>{});
  }
  if (it < cnt) body(it, std::integral_constant<int, 0>{});
  stamps.walk_done();
  wait_vmem();  // the last tile's extra loads land before the workgroup's LDS is released

  const float l = pair_sum32(l_run);
  if (row_ok) {
    const float inv = l > 0.0f ? 1.0f / l : 0.0f;
    if (g == 0) lse_row[q_row] = l > 0.0f ? (m_run + log2f(l)) * kLn2 : -INFINITY;
    T* orow = Op + (size_t)q_row * a.L.qs_r;
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
  stamps.store(FM_STAMP_BUF(g_stamps_fwd), cnt);
}

}  // namespace

TileShape tile_shape(int dtype) {
  (void)dtype;
  return TileShape{FwdTile<bf16, 128>::BM, FwdTile<bf16, 128>::BN, 64, 64};
}

hipError_t launch_attn_fwd(int dtype, const FwdArgs& a, hipStream_t stream, hipEvent_t ev_begin,
                           hipEvent_t ev_end) {
  const int64_t n_qb = (a.nq + 127) / 128;
  const int64_t grid = n_qb * a.L.B * a.L.H;
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
