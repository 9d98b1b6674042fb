// Device-side helpers shared by the gfx950 kernels: vector types, MFMA wrappers and the
// element traits that let one attention kernel body serve bf16 (d = 128) and fp32 (d = 64).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace fm {

typedef __bf16 bf16;
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;

// Element traits.  One MFMA k-step covers KSTEP = 2*KPL elements of the contraction: lanes
// 0..31 hold KPL consecutive elements and lanes 32..63 the next KPL, for both the A and the B
// operand (v_mfma_f32_32x32x16_bf16: KPL = 8; v_mfma_f32_32x32x2_f32: KPL = 1).  The 32x32
// fp32 accumulator holds, in lane l and register r, row 8*(r/4) + 4*(l/32) + r%4, column l%32.
template <typename T> struct Elem;

template <> struct Elem<bf16> {
  static constexpr int KPL = 8;
  typedef bf16x8 frag;  // one lane's share of an operand for one k-step
  __device__ static inline f32x16 mfma(const frag& a, const frag& b, const f32x16& c) {
    return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
  }
  __device__ static inline frag load_frag(const bf16* p) {
    return *reinterpret_cast<const frag*>(p);
  }
  __device__ static inline frag zero_frag() {
    frag z;
#pragma unroll
    for (int i = 0; i < 8; ++i) z[i] = (bf16)0.0f;
    return z;
  }
  __device__ static inline bf16 from_float(float x) { return (bf16)x; }
};

template <> struct Elem<float> {
  static constexpr int KPL = 1;
  typedef float frag;
  __device__ static inline f32x16 mfma(const frag& a, const frag& b, const f32x16& c) {
    return __builtin_amdgcn_mfma_f32_32x32x2f32(a, b, c, 0, 0, 0);
  }
  __device__ static inline frag load_frag(const float* p) { return *p; }
  __device__ static inline frag zero_frag() { return 0.0f; }
  __device__ static inline float from_float(float x) { return x; }
};

// Accumulator register r of lane group g (= lane/32) sits at row acc_row(r, g) of the 32x32
// result tile.
__device__ __host__ constexpr int acc_row(int r, int g) { return 8 * (r / 4) + 4 * g + (r % 4); }

// Permuted row order used for the operand that becomes the accumulator's row index (keys in the
// forward S^T, queries in the backward S).  Loading MFMA row acc_row(r, g) from original index
// perm_index(r, g) makes accumulator register r of group g hold index
//   (r / KPL) * 2*KPL + g*KPL + r % KPL,
// so that the KPL registers r = s*KPL .. s*KPL + KPL-1 of group g are exactly the KPL
// consecutive indices that k-step s of the next product needs in that lane group.  The result
// (P, or dS) can then be fed to the next MFMA as an operand straight from registers.
template <int KPL>
__device__ __host__ constexpr int perm_index(int r, int g) {
  return (r / KPL) * 2 * KPL + g * KPL + (r % KPL);
}

// Inverse of the above for a row index m in [0, 32): the original index loaded into MFMA row m.
template <int KPL>
__device__ __host__ constexpr int row_source(int m) {
  // m = 8*(r/4) + 4*g + r%4  ->  r = 4*(m/8) + m%4, g = (m/4)%2
  return perm_index<KPL>(4 * (m / 8) + (m % 4), (m / 4) % 2);
}

// The two 32-lane halves of x, each across the whole wave: lo[l] = x[l % 32] and
// hi[l] = x[l % 32 + 32].  v_permlane32_swap exchanges lanes 32..63 of its first operand with
// lanes 0..31 of its second, in registers (no LDS round trip); the s_nop pairs cover the
// wait states around a cross-lane VALU operation.
__device__ inline void wave_halves(float x, float& lo, float& hi) {
  float a = x, b = x;
  asm("s_nop 1\n\tv_permlane32_swap_b32 %0, %1\n\ts_nop 1" : "+v"(a), "+v"(b));
  lo = a;
  hi = b;
}
// max / sum of x over lanes l and l ^ 32, the same value in both lanes.
__device__ inline float pair_max32(float x) {
  float lo, hi;
  wave_halves(x, lo, hi);
  return fmaxf(lo, hi);
}
__device__ inline float pair_sum32(float x) {
  float lo, hi;
  wave_halves(x, lo, hi);
  return lo + hi;
}

// Empty asm that takes a value in vector registers: the value must be computed before this
// point, so code placement passes cannot move its computation into later blocks.
template <typename X>
__device__ inline void pin_value(X& x) {
  static_assert(sizeof(X) % 4 == 0 && sizeof(X) <= 16, "1 to 4 registers");
  if constexpr (sizeof(X) == 16) {
    u32x4 u = __builtin_bit_cast(u32x4, x);
    asm volatile("" : "+v"(u));
    x = __builtin_bit_cast(X, u);
  } else if constexpr (sizeof(X) == 8) {
    u32x2 u = __builtin_bit_cast(u32x2, x);
    asm volatile("" : "+v"(u));
    x = __builtin_bit_cast(X, u);
  } else {
    uint32_t u = __builtin_bit_cast(uint32_t, x);
    asm volatile("" : "+v"(u));
    x = __builtin_bit_cast(X, u);
  }
}

// x where bit `pos` of `word` is clear, else the float whose bits are `to`: the sign-extended
// bit is an all-ones / all-zeros select mask for v_bitop3 (two VALU operations in all).
__device__ inline float select_bit(uint32_t word, uint32_t pos, float x, uint32_t to) {
  const uint32_t sel = (uint32_t)__builtin_amdgcn_sbfe((int)word, pos, 1);
  return __builtin_bit_cast(float, __builtin_amdgcn_bitop3_b32(sel, to, __builtin_bit_cast(uint32_t, x), 0xCA));
}
constexpr uint32_t kNegInfBits = 0xff800000u;

__device__ inline float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }

// Round float to bf16 (round to nearest even) and pack two into a 32-bit word.
__device__ inline uint32_t pack_bf16x2(float lo, float hi) {
  bf16 a = (bf16)lo, b = (bf16)hi;
  uint16_t ua = __builtin_bit_cast(uint16_t, a), ub = __builtin_bit_cast(uint16_t, b);
  return (uint32_t)ua | ((uint32_t)ub << 16);
}

// Masked-stretch test: q in [s, s + len) with len = max(e - s, 0) computed in 32-bit unsigned
// arithmetic.  Exact for every int32 s, e and every q >= 0.
__device__ inline bool in_stretch(int32_t q, int32_t s, uint32_t len) {
  return (uint32_t)q - (uint32_t)s < len;
}
__host__ __device__ inline uint32_t stretch_len(int32_t s, int32_t e) {
  return e > s ? (uint32_t)e - (uint32_t)s : 0u;
}

// ---- swizzled LDS tiles ------------------------------------------------------------------------
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

// ---- XCD-aware work order ---------------------------------------------------------------------
// Workgroups are dispatched round-robin over the 8 XCDs (workgroup i to XCD i % 8), each with
// its own L2.  This maps the dispatch index to a work index so that every XCD walks one
// contiguous range of the work list: neighbouring work items (query or key blocks of the same
// head, which read the same K/V or Q/dO rows) then share an L2.
constexpr int kNumXcd = 8;
__device__ inline int xcd_contiguous_index(int bid, int nwg) {
  const int xcd = bid % kNumXcd, slot = bid / kNumXcd;
  const int q = nwg / kNumXcd, r = nwg % kNumXcd;
  return xcd < r ? xcd * (q + 1) + slot : r * (q + 1) + (xcd - r) * q + slot;
}

// ---- workgroup timeline (debug build only) -----------------------------------------------------
// Built with FM_WG_STAMPS (libflashmask_stamps.so), each attention workgroup records, through
// thread 0, the real-time counter (s_memrealtime, 100 MHz) at its start, after its first tile's
// barrier and after its tile walk, then at its end: slot blockIdx.x of a per-kernel device array
// of kStampSlots * 8 words gets {start, first tile, walk done, end, HW_ID | XCC_ID << 32, tiles}.
// In the default build every member is empty and the compiler removes the calls.
constexpr int kStampSlots = 1 << 16;
struct WgStamps {
#ifdef FM_WG_STAMPS
  unsigned long long t0, t1 = 0, t2 = 0;
  __device__ WgStamps() : t0(__builtin_amdgcn_s_memrealtime()) {}
  __device__ void first_tile() { t1 = __builtin_amdgcn_s_memrealtime(); }
  __device__ void walk_done() { t2 = __builtin_amdgcn_s_memrealtime(); }
  __device__ void store(unsigned long long* buf, int tiles) const {
    if (threadIdx.x == 0 && blockIdx.x < (unsigned)kStampSlots) {
      const unsigned long long t3 = __builtin_amdgcn_s_memrealtime();
      const unsigned hw = __builtin_amdgcn_s_getreg(4 | (31 << 11));    // HW_ID
      const unsigned xcc = __builtin_amdgcn_s_getreg(20 | (31 << 11));  // XCC_ID
      unsigned long long* p = buf + (size_t)blockIdx.x * 8;
      p[0] = t0;
      p[1] = t1;
      p[2] = t2;
      p[3] = t3;
      p[4] = hw | ((unsigned long long)xcc << 32);
      p[5] = (unsigned long long)tiles;
    }
  }
#else
  __device__ void first_tile() {}
  __device__ void walk_done() {}
  __device__ void store(unsigned long long*, int) const {}
#endif
};
// The per-kernel array behind WgStamps::store and the host call that copies it out (debug build
// only; declared in include/flashmask_debug.h).
#ifdef FM_WG_STAMPS
#define FM_STAMP_ARRAY(name, getter)                                                           \
  __device__ unsigned long long name[kStampSlots * 8];                                         \
  }                                                                                            \
  extern "C" int getter(void* host, size_t bytes) {                                            \
    if (!host || bytes > sizeof(unsigned long long) * fm::kStampSlots * 8) return -1;          \
    return hipMemcpyFromSymbol(host, HIP_SYMBOL(fm::name), bytes, 0, hipMemcpyDeviceToHost) == \
                   hipSuccess                                                                  \
               ? 0                                                                             \
               : -1;                                                                           \
  }                                                                                            \
  namespace fm {
#define FM_STAMP_BUF(name) name
#else
#define FM_STAMP_ARRAY(name, getter)
#define FM_STAMP_BUF(name) nullptr
#endif

// ---- raw buffer loads: out-of-range offsets return zeros, so tails need no branches ----------
typedef __amdgpu_buffer_rsrc_t buf_rsrc;

// Raw (unstructured) buffer over [base, base + bytes): dword 3 is the gfx9-family value for a
// plain 32-bit-data raw buffer.
__device__ inline buf_rsrc make_buf(const void* base, uint32_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, bytes, 0x00020000);
}
__device__ inline uint4 buf_load16(buf_rsrc r, uint32_t voff, uint32_t soff) {
  return __builtin_bit_cast(uint4, __builtin_amdgcn_raw_buffer_load_b128(r, voff, soff, 0));
}
__device__ inline uint32_t buf_load4(buf_rsrc r, uint32_t voff, uint32_t soff) {
  return __builtin_amdgcn_raw_buffer_load_b32(r, voff, soff, 0);
}

// Buffer load straight into LDS (no registers): lane l's `bytes` (4 or 16) land at
// lds_base + l * bytes, where lds_base must be the same for the whole wave; lanes whose offset
// is out of range write zeros.
template <int BYTES>
__device__ inline void buf_load_lds(buf_rsrc r, void* lds_base, uint32_t voff, uint32_t soff) {
  typedef __attribute__((address_space(3))) void lds_void;
  if constexpr (BYTES == 16) {
    __builtin_amdgcn_raw_ptr_buffer_load_lds(r, (lds_void*)(lds_base), 16, voff, soff, 0, 0);
  } else {
    static_assert(BYTES == 4, "4 or 16 bytes per lane");
    __builtin_amdgcn_raw_ptr_buffer_load_lds(r, (lds_void*)(lds_base), 4, voff, soff, 0, 0);
  }
}
// Wait until this wave's outstanding vector-memory operations (including loads into LDS) are
// complete: s_waitcnt vmcnt(0), other counters left alone.
__device__ inline void wait_vmem() { __builtin_amdgcn_s_waitcnt(0x0f70); }
// Read a value that is the same for the whole wave and constant while the kernel runs (written
// by an earlier launch) through the scalar path: s_load, counted by lgkmcnt, so the read never
// has to wait for vector loads in flight (a vector load would need s_waitcnt vmcnt(0)).
__device__ inline int32_t load_uniform(const int32_t* p, int i) {
  typedef const __attribute__((address_space(4))) int32_t const_i32;
  return ((const_i32*)p)[i];
}
// Workgroup barrier for data exchanged through LDS only: waits for this wave's LDS (and scalar)
// operations, lgkmcnt(0), but not for its vector-memory loads; __syncthreads() also waits
// vmcnt(0), which would stall on loads still in flight for a later tile.  Loads straight into
// LDS are covered by the caller's own vmcnt wait.  The empty asm statements keep the compiler
// from moving memory accesses across the barrier.
__device__ inline void lds_barrier() {
  asm volatile("" ::: "memory");
  __builtin_amdgcn_s_waitcnt(0xc07f);
  __builtin_amdgcn_s_barrier();
  asm volatile("" ::: "memory");
}
// s_waitcnt vmcnt(N): wait until at most N of this wave's vector-memory operations are in
// flight (they complete in issue order).
template <int N>
__device__ inline void wait_vmem_n() {
  static_assert(N >= 0 && N < 16, "vmcnt immediate");
  __builtin_amdgcn_s_waitcnt(0x0f70 | N);
}

// ---- LDS transpose read (gfx950 ds_read_b64_tr_b16) ------------------------------------------
// Within each block of 16 lanes, lane i receives element i%4 of the four 16-bit elements that
// lane 4*j + i/4 addressed, for j = 0..3.  So if lane i addresses X[k0 + i/4][m0 + 4*(i%4)] of a
// row-major (k-major) matrix X, it receives X[k0 + j][m0 + i], j = 0..3: four consecutive k of
// column m0 + i, which is the operand layout MFMA wants for a contraction over k.
typedef short s16x4 __attribute__((ext_vector_type(4)));
__device__ inline s16x4 lds_read_tr16(const void* p) {
  typedef __attribute__((address_space(3))) s16x4 lds_s16x4;
  return __builtin_amdgcn_ds_read_tr16_b64_v4i16(
      (lds_s16x4*)((__attribute__((address_space(3))) char*)(p)));
}

// ---- scheduling hint for a run of MFMAs fed from LDS -----------------------------------------
// Placed right after a block of N MFMAs whose A operands are LDS reads (R read instructions per
// MFMA), it asks the compiler's scheduler to issue the reads of the first AHEAD MFMAs up front and
// then alternate one MFMA with the reads of the MFMA AHEAD places later, so each MFMA finds its
// operand about AHEAD MFMAs after requesting it.  (Without it the compiler keeps one or two reads
// in flight where registers are scarce and waits for each operand just before its MFMA.)  Only
// the order of instructions changes: the waits the compiler inserts stay exact.
template <int N, int R, int AHEAD>
__device__ inline void sched_mfma_reads_ahead() {
  static_assert(AHEAD > 0 && AHEAD <= N, "lead within the run");
  constexpr int kMfma = 0x008, kDsRead = 0x100;  // instruction classes of the scheduler hint
  __builtin_amdgcn_sched_group_barrier(kDsRead, R * AHEAD, 0);
#pragma unroll
  for (int i = 0; i < N - AHEAD; ++i) {
    __builtin_amdgcn_sched_group_barrier(kMfma, 1, 0);
    __builtin_amdgcn_sched_group_barrier(kDsRead, R, 0);
  }
  __builtin_amdgcn_sched_group_barrier(kMfma, AHEAD, 0);
}

}  // namespace fm
