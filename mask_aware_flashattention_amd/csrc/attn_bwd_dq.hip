// dQ of the mask-aware attention backward, query-stationary, without atomics.
//
// The pages report the backward's speed ("FlashMask-3 ..." zicq.com summary, end-to-end
// paragraph) but do not describe it.  This kernel computes dQ = scale * dS K for one query
// block per workgroup, walking the same list of key tiles the forward walks (fully masked tiles
// skipped, the row test only in partly masked tiles; "FlashMask-3 sends each GPU its mask ...",
// tile-classification paragraph), recomputing P from the saved LSE and dP from dO and V.
// dK and dV come from the key-stationary kernel in attn_bwd.hip, launched after this one;
// splitting the two products this way needs no float32 atomics and gives a deterministic dQ.
// Before its tile loop each workgroup reads its rows of O once and writes, per row,
// -D = -sum_d dO_id O_id and LSE * log2(e) for the dK / dV kernel (no separate pass).
//
// Layout (the forward's, with dP added): one workgroup = 4 waves = 128 query rows against key
// tiles of 64; each wave holds its 32 rows of Q and dO in registers as the B operands of
// S^T = K Q^T and dP^T = V dO^T (K, V rows loaded in a permuted order so the accumulators are
// already laid out as operands), forms dS^T = P^T * (dP^T - D) in registers, and accumulates
// dQ^T += K^T dS^T with the K^T operand read by the gfx950 LDS transpose read.  K and V tiles go
// straight from HBM into LDS (XOR-swizzled, double-buffered, one barrier per tile).
#include <math.h>

#include "fm_common.hpp"
#include "launch.hpp"

namespace fm {

FM_STAMP_ARRAY(g_stamps_dq, flashmask_debug_stamps_dq)

namespace {

template <typename T, int D>
struct DqTile {
  static constexpr int BM = 128, BN = 64, NT = 256;
  static constexpr int KPL = Elem<T>::KPL, KSTEP = 2 * KPL;
  static constexpr int CH = 16 / (int)sizeof(T);
  static constexpr int CPR = D / CH;
  static constexpr int ROW_BYTES = D * (int)sizeof(T);
  static constexpr int NRB = BN / 32;  // 32-key row blocks of S^T
  static constexpr int NDB = D / 32;   // 32-wide d blocks of dQ^T
  static constexpr int QK_STEPS = D / KSTEP;
  static constexpr int KV_STEPS = BN / KSTEP;  // k-steps over a tile's keys
  static constexpr int TILE_BYTES = BN * ROW_BYTES;
  static constexpr int MW_BYTES = 4 * BN * 4;  // per wave, per key: one 32-bit row mask
  static_assert(CPR == 16, "256-byte rows");
  static_assert(BN * ROW_BYTES == 16 * 1024, "16 blocks of 1 KiB per tile");
};

template <typename T, int D>
__global__ __launch_bounds__(256, 2) void attn_dq_kernel(DqArgs a) {
  using C = DqTile<T, D>;
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
  const int qb = a.order[(size_t)set * n_qb + work % n_qb];

  const int64_t qbase = b * a.L.qs_b + head * a.L.qs_h;
  const int64_t kbase = b * a.L.ks_b + (head / a.L.G) * a.L.ks_h;
  const T* __restrict__ Qp = static_cast<const T*>(a.q) + qbase;
  const T* __restrict__ dOp = static_cast<const T*>(a.dout) + qbase;
  const T* __restrict__ Kp = static_cast<const T*>(a.k) + kbase;
  const T* __restrict__ Vp = static_cast<const T*>(a.v) + kbase;
  const uint32_t qrs = (uint32_t)a.L.qs_r * sizeof(T);  // row strides in bytes
  const uint32_t krs = (uint32_t)a.L.ks_r * sizeof(T);
  const buf_rsrc qbuf = make_buf(Qp, (uint32_t)(a.nq - 1) * qrs + C::ROW_BYTES);
  const buf_rsrc dobuf = make_buf(dOp, (uint32_t)(a.nq - 1) * qrs + C::ROW_BYTES);
  const buf_rsrc kbuf = make_buf(Kp, (uint32_t)(a.nk - 1) * krs + C::ROW_BYTES);
  const buf_rsrc vbuf = make_buf(Vp, (uint32_t)(a.nk - 1) * krs + C::ROW_BYTES);
  const MaskVecs mask{a.mask.lts + set * a.L.mask_stride, a.mask.lte + set * a.L.mask_stride,
                      a.mask.uts + set * a.L.mask_stride, a.mask.ute + set * a.L.mask_stride};
  T* const dQp = static_cast<T*>(a.dq) + qbase;

  const int q0w = qb * C::BM + w * 32;  // first query row of this wave
  const int q_row = q0w + l32;          // this lane's query row
  const bool row_ok = q_row < a.nq;
  const int cnt = a.qcnt[(size_t)set * n_qb + qb];
  // Per row, for this kernel and the dK/dV kernel that runs after it: LSE * log2(e) (+inf on a
  // fully masked row, so that exp2(s - lse2) = 0) and -D, D = sum_d dO_id O_id.
  const size_t row_idx = (size_t)bh * a.nq + q_row;
  const float lse_row = row_ok ? a.lse[row_idx] : -INFINITY;
  const float lse2 = lse_row == -INFINITY ? INFINITY : lse_row * kLog2e;
  if (cnt == 0) {
    // No listed tile: the block's rows are fully masked, so dQ = 0 (each lane clears half of
    // its row, 128 bytes) and the rows' D is never used.
    if (row_ok) {
      uint4* p = reinterpret_cast<uint4*>(dQp + (size_t)q_row * a.L.qs_r + g * (D / 2));
#pragma unroll
      for (int i = 0; i < 8; ++i) p[i] = make_uint4(0u, 0u, 0u, 0u);
      if (g == 0) {
        a.delta[row_idx] = 0.0f;
        a.lse2[row_idx] = lse2;
      }
    }
    stamps.store(FM_STAMP_BUF(g_stamps_dq), 0);
    return;
  }

  // Q and dO rows of this lane's query as B operands (k-step s: d = s*KSTEP + g*KPL + 0..KPL);
  // rows past nq read as zeros.
  frag qf[C::QK_STEPS], dof[C::QK_STEPS];
#pragma unroll
  for (int s = 0; s < C::QK_STEPS; ++s) {
    const uint32_t off = (uint32_t)q_row * qrs + (uint32_t)(s * KSTEP + g * KPL) * sizeof(T);
    if constexpr (KPL == 8) {
      qf[s] = __builtin_bit_cast(frag, buf_load16(qbuf, off, 0));
      dof[s] = __builtin_bit_cast(frag, buf_load16(dobuf, off, 0));
    } else {
      qf[s] = __builtin_bit_cast(frag, buf_load4(qbuf, off, 0));
      dof[s] = __builtin_bit_cast(frag, buf_load4(dobuf, off, 0));
    }
  }
  float ndlt = 0.0f;  // -D of this lane's row, formed once the first tile is on its way

  const int32_t* __restrict__ lst = a.qlist + ((size_t)set * n_qb + qb) * a.list_stride;
  const int last_kb = (a.nk - 1) / C::BN;
  const bool ragged = (a.nk % C::BN) != 0;
  const float cexp = a.scale * kLog2e;

  // per-lane LDS byte offsets (see attn_bwd.hip: swizzles depend on row & 15 only)
  const int tb = lane >> 4, ti = lane & 15;
  const int tr_row = 8 * (tb >> 1) + (ti >> 2);
  const int tr_col = 16 * (tb & 1) + 4 * (ti & 3);
  int off_s[C::QK_STEPS];  // K / V row operand (permuted row source, k-step s) of a 32-key block
  int off_tk[C::NDB][2];   // K^T operand rows (tr_row, tr_row + 4), columns 32*db
  {
    const int srow = row_source<KPL>(l32);
#pragma unroll
    for (int st = 0; st < C::QK_STEPS; ++st)
      off_s[st] = tile_off<T, 0>(srow, st * KSTEP + g * KPL, C::ROW_BYTES);
#pragma unroll
    for (int h = 0; h < 2; ++h)
#pragma unroll
      for (int db = 0; db < C::NDB; ++db)
        off_tk[db][h] = KPL == 8 ? tile_off<T, 0>(tr_row + 4 * h, 32 * db + tr_col, C::ROW_BYTES)
                                 : tile_off<T, 0>(g, 32 * db + l32, C::ROW_BYTES);
  }
  auto tr_operand = [&](const unsigned char* tile, const int* off, int k0_bytes) -> frag {
    if constexpr (KPL == 8) {
      const s16x4 lo = lds_read_tr16(tile + off[0] + k0_bytes);
      const s16x4 hi = lds_read_tr16(tile + off[1] + k0_bytes);
      return __builtin_bit_cast(frag, __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7));
    } else {
      return *reinterpret_cast<const T*>(tile + off[0] + k0_bytes);
    }
  };

  // Stage key tile `entry` into buffer `bufc`: K then V, 16 blocks of 1 KiB each, wave w fills
  // blocks 4w..4w+3 (lane l: row 4j + l/16, physical chunk l%16 = logical chunk
  // (l%16) ^ swz_row(row)); keys past nk read as zeros.
  auto issue_tile = [&](int entry, auto bufc) {
    const int kb = entry >> 1;
    unsigned char* kt = bufp(bufc);
    const uint32_t tile_base = (uint32_t)kb * C::BN * krs;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int j = 4 * w + i;
      const int row = 4 * j + (lane >> 4);
      const uint32_t voff = (uint32_t)row * krs + (uint32_t)(((lane & 15) ^ swz_row<T>(row)) * 16);
      buf_load_lds<16>(kbuf, kt + j * 1024, voff, tile_base);
      buf_load_lds<16>(vbuf, kt + C::TILE_BYTES + j * 1024, voff, tile_base);
    }
  };
  // Row mask of a partly masked tile: lane l loads the four vectors at key l of the tile before
  // the tile's loads are issued and writes the word for this wave's 32 rows (bit t = row q0w + t
  // masked) at the end of the iteration, so neither the tile loads nor the products wait for the
  // vectors.
  struct MaskKey {
    int32_t s0, e0, s1, e1;
    bool live;
  };
  auto is_test = [&](int entry) { return (entry & 1) || ((entry >> 1) == last_kb && ragged); };
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
    auto bits = [&](int32_t s0, int32_t e0) -> uint32_t {
      const int32_t lo = s0 <= q0w ? 0 : (s0 >= q0w + 32 ? 32 : s0 - q0w);
      const int32_t hi = e0 <= q0w ? 0 : (e0 >= q0w + 32 ? 32 : e0 - q0w);
      if (hi <= lo) return 0u;
      const uint32_t upto_hi = hi >= 32 ? 0xffffffffu : ((1u << hi) - 1u);
      return upto_hi & ~((1u << lo) - 1u);  // lo < 32 here
    };
    mwp(bufc)[w * C::BN + lane] = m.live ? (bits(m.s0, m.e0) | bits(m.s1, m.e1)) : 0xffffffffu;
  };

  f32x16 dq_acc[C::NDB];
#pragma unroll
  for (int db = 0; db < C::NDB; ++db) dq_acc[db] = f32x16{};

  // List entries are read one tile ahead of their use (scalar loads: their latency then hides
  // behind a tile instead of stalling the wave).  cnt > 0 here.
  int entry = load_uniform(lst, 0);
  int pre = load_uniform(lst, cnt > 1 ? 1 : 0);  // entry of the tile after `entry`

  auto body = [&](const int it, auto bufc) {
    constexpr int buf = decltype(bufc)::value;
    const bool test = is_test(entry);
    const bool has_next = it + 1 < cnt;
    const int next = has_next ? pre : 0;
    pre = load_uniform(lst, it + 2 < cnt ? it + 2 : cnt - 1);
    const bool next_test = has_next && is_test(next);
    const auto other = std::integral_constant<int, buf ^ 1>{};
    wait_vmem();      // this wave's loads of tile `it` have landed in LDS
    __syncthreads();  // ... everyone's, and the mask words
    if (it == 0) stamps.first_tile();
    MaskKey mk{0, 0, 0, 0, false};
    if (next_test) mk = mask_load(next);
    // The last tile stages its own rows again into the free buffer, which is never read: the
    // load count is then the same on every path and the compiler's waits stay exact.
    issue_tile(has_next ? next : entry, other);

    const unsigned char* kt = bufp(bufc);
    const unsigned char* vt = kt + C::TILE_BYTES;

    // S^T = K Q^T and dP^T = V dO^T: register r of group g in row block rb is tile key
    // rb*32 + perm_index(r, g); the column is this lane's query.
    f32x16 sacc[C::NRB], pacc[C::NRB];
#pragma unroll
    for (int rb = 0; rb < C::NRB; ++rb) {
      sacc[rb] = f32x16{};
      pacc[rb] = f32x16{};
    }
    // four independent accumulators in turn; the K / V reads run six products ahead
#pragma unroll
    for (int st = 0; st < C::QK_STEPS; ++st)
#pragma unroll
      for (int rb = 0; rb < C::NRB; ++rb) {
        const int off = off_s[st] + rb * 32 * C::ROW_BYTES;
        const frag ka = *reinterpret_cast<const frag*>(kt + off);
        const frag va = *reinterpret_cast<const frag*>(vt + off);
        sacc[rb] = E::mfma(ka, qf[st], sacc[rb]);
        pacc[rb] = E::mfma(va, dof[st], pacc[rb]);
      }
    if constexpr (KPL == 8) sched_mfma_reads_ahead<2 * C::NRB * C::QK_STEPS, 1, 6>();

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

    // dS^T = P^T (dP^T - D) as operand fragments: k-step t covers tile keys
    // t*KSTEP + g*KPL + e = registers (t*KPL)%16 + e of row block (t*KPL)/16.
    frag sf[C::KV_STEPS];
#pragma unroll
    for (int t = 0; t < C::KV_STEPS; ++t) {
#pragma unroll
      for (int e = 0; e < KPL; ++e) {
        const int rb = (t * KPL) / 16, r = (t * KPL) % 16 + e;
        const float p = fast_exp2(fmaf(sacc[rb][r], cexp, -lse2));
        const float ds = p * (pacc[rb][r] + ndlt);
        if constexpr (KPL == 1)
          sf[t] = ds;
        else
          sf[t][e] = E::from_float(ds);
      }
    }

    // dQ^T += K^T dS^T (contraction over the tile's keys; K^T read with the transpose read)
#pragma unroll
    for (int t = 0; t < C::KV_STEPS; ++t)
#pragma unroll
      for (int db = 0; db < C::NDB; ++db)
        dq_acc[db] = E::mfma(tr_operand(kt, off_tk[db], t * KSTEP * C::ROW_BYTES), sf[t], dq_acc[db]);
    if constexpr (KPL == 8) sched_mfma_reads_ahead<C::KV_STEPS * C::NDB, 2, 3>();  // K^T 3 ahead

    if (next_test) mask_store(mk, other);
    entry = next;
  };

  {
    const auto first = std::integral_constant<int, 0>{};
    issue_tile(entry, first);
    if (is_test(entry)) mask_store(mask_load(entry), first);
  }
  // D of this row from its O and dO (lanes l and l ^ 32 hold the two halves of the row), read
  // after the first tile's loads are issued so that the two requests overlap.
  {
    const T* __restrict__ Op = static_cast<const T*>(a.o) + qbase;
    const buf_rsrc obuf = make_buf(Op, (uint32_t)(a.nq - 1) * qrs + C::ROW_BYTES);
    float part = 0.0f;
#pragma unroll
    for (int s = 0; s < C::QK_STEPS; ++s) {
      const uint32_t off = (uint32_t)q_row * qrs + (uint32_t)(s * KSTEP + g * KPL) * sizeof(T);
      if constexpr (KPL == 8) {
        const frag of = __builtin_bit_cast(frag, buf_load16(obuf, off, 0));
#pragma unroll
        for (int e = 0; e < KPL; ++e) part = fmaf((float)dof[s][e], (float)of[e], part);
      } else {
        const float of = __builtin_bit_cast(float, buf_load4(obuf, off, 0));
        part = fmaf(dof[s], of, part);
      }
    }
    ndlt = -pair_sum32(part);
    if (row_ok && g == 0) {
      a.delta[row_idx] = ndlt;
      a.lse2[row_idx] = lse2;
    }
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

  if (row_ok) {
    T* orow = dQp + (size_t)q_row * a.L.qs_r;
#pragma unroll
    for (int db = 0; db < C::NDB; ++db)
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int d0 = db * 32 + 8 * i + 4 * g;
        const float s = a.scale;
        if constexpr (sizeof(T) == 2) {
          uint2 out;
          out.x = pack_bf16x2(dq_acc[db][4 * i + 0] * s, dq_acc[db][4 * i + 1] * s);
          out.y = pack_bf16x2(dq_acc[db][4 * i + 2] * s, dq_acc[db][4 * i + 3] * s);
          *reinterpret_cast<uint2*>(orow + d0) = out;
        } else {
          *reinterpret_cast<float4*>(orow + d0) =
              make_float4(dq_acc[db][4 * i + 0] * s, dq_acc[db][4 * i + 1] * s,
                          dq_acc[db][4 * i + 2] * s, dq_acc[db][4 * i + 3] * s);
        }
      }
  }
  stamps.store(FM_STAMP_BUF(g_stamps_dq), cnt);
}

template <typename T, int D>
hipError_t run_dq(const DqArgs& a, hipStream_t stream, hipEvent_t ev_begin) {
  using C = DqTile<T, D>;
  const int64_t n_qb = (a.nq + C::BM - 1) / C::BM;
  const int64_t grid = n_qb * a.L.B * a.L.H;
  if (ev_begin) (void)hipEventRecord(ev_begin, stream);
  hipLaunchKernelGGL((attn_dq_kernel<T, D>), dim3((unsigned)grid), dim3(256), 0, stream, a);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_attn_dq(int dtype, const DqArgs& a, hipStream_t stream, hipEvent_t ev_begin) {
  // The lists were built at the forward's tile shape; this kernel walks them at the same shape.
  const TileShape t = tile_shape(dtype);
  if (t.bm_fwd != DqTile<bf16, 128>::BM || t.bn_fwd != DqTile<bf16, 128>::BN) return hipErrorInvalidValue;
  return dtype == 0 ? run_dq<bf16, 128>(a, stream, ev_begin) : run_dq<float, 64>(a, stream, ev_begin);
}

}  // namespace fm
