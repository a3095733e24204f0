// Device-side building blocks shared by the gfx950 attention kernels.
//
// Layout facts used throughout (checked on the device with an in-bounds
// probe of each instruction):
//
// * v_mfma_f32_32x32x16_bf16  A[m][k]: lane l holds m = l%32, k = 8(l/32)+e
//   (e = 0..7); B[k][n]: n = l%32, k = 8(l/32)+e; C[m][n]: lane l, register
//   r holds m = 8(r/4) + 4(l/32) + r%4, n = l%32.
// * v_mfma_f32_32x32x2_f32    A: m = l%32, k = l/32; B: k = l/32, n = l%32;
//   C as above.
// * ds_read_b64_tr_b16: in each 16-lane group the 16 lane addresses name a
//   16 x 4 block M[r][c] of 16-bit elements (row r = the lane, 4 contiguous
//   elements); lane i receives M[4t + i/4][i%4] for t = 0..3.  Giving lane i
//   the address of X[k0 + i/4][n0 + 4(i%4)] of a row-major tile X therefore
//   hands lane i the column slice X[k0 .. k0+3][n0 + i]: four consecutive
//   contraction indices of one output column, which is what an MFMA operand
//   needs when the contraction runs down the rows of X.
// * Workgroups are dispatched round-robin over the 8 XCDs (XCC id =
//   blockIdx.x % 8).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include <type_traits>

namespace eta {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef short i16x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

typedef __attribute__((address_space(3))) i16x4 lds_i16x4;

constexpr int kWave = 64;
constexpr int kXcds = 8;
constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;

enum : int { kMaskNone = 0, kMaskCausal = 1, kMaskBitmask = 2 };
enum : uint8_t { kTileEmpty = 0, kTilePartial = 1, kTileFull = 2 };

// ---------------------------------------------------------------------------
// Scalars
// ---------------------------------------------------------------------------

__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }
__device__ __forceinline__ float fast_log2(float x) { return __builtin_amdgcn_logf(x); }

typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef float f32x2 __attribute__((ext_vector_type(2)));

// Two fp32 -> packed bf16 (lo in bits 0..15), round to nearest even: one
// v_cvt_pk_bf16_f32 on gfx950.
__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
  bf16x2 y = __builtin_convertvector(f32x2{lo, hi}, bf16x2);
  return *reinterpret_cast<uint32_t*>(&y);
}
__device__ __forceinline__ float bf16_bits_to_f32(uint32_t b) { return __uint_as_float(b << 16); }
__device__ __forceinline__ bf16x2 ones_bf16x2() {
  const uint32_t u = 0x3F803F80u;  // (1.0, 1.0)
  return *reinterpret_cast<const bf16x2*>(&u);
}

// Max over the two 32-lane halves holding the same column (lane l and l^32).
__device__ __forceinline__ float max_halves(float x) {
  auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
__device__ __forceinline__ float sum_halves(float x) {
  auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}

// ---------------------------------------------------------------------------
// MFMA wrappers
// ---------------------------------------------------------------------------

__device__ __forceinline__ f32x16 mfma_bf16(const bf16x8& a, const bf16x8& b, const f32x16& c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
}
__device__ __forceinline__ f32x16 mfma_f32(float a, float b, const f32x16& c) {
  return __builtin_amdgcn_mfma_f32_32x32x2f32(a, b, c, 0, 0, 0);
}

// ---------------------------------------------------------------------------
// LDS operand fetches
// ---------------------------------------------------------------------------

// Row operand: lane reads 8 contiguous bf16 at byte offset `off` of LDS.
__device__ __forceinline__ bf16x8 lds_read_b128(const char* lds_base, uint32_t off) {
  return *reinterpret_cast<const bf16x8*>(lds_base + off);
}

// Column operand, transposed read: returns X[k0..k0+3][col] where the lane's
// address (computed by tr_addr) names X[k0 + i/4][n0 + 4(i%4)].
__device__ __forceinline__ i16x4 lds_read_tr(const char* lds_base, uint32_t off) {
  const __attribute__((address_space(3))) char* p =
      (const __attribute__((address_space(3))) char*)(lds_base) + off;
  return __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4*)p);
}

// Byte offset for a transposed read of the 4 x 16 block of a row-major bf16
// tile with `stride` bytes per row, rows k0..k0+3, columns n0..n0+15.
__device__ __forceinline__ uint32_t tr_addr(int lane, int k0, int n0, int stride) {
  int i = lane & 15;
  return (uint32_t)((k0 + (i >> 2)) * stride + (n0 + 4 * (i & 3)) * 2);
}

typedef short i16x8 __attribute__((ext_vector_type(8)));
__device__ __forceinline__ bf16x8 join_tr(i16x4 lo, i16x4 hi) {
  return __builtin_bit_cast(bf16x8, __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7));
}

// Raw buffer resource over [base, base + bytes): loads at offsets >= bytes
// return zero (gfx9 descriptor word 3 = 0x00020000, 32-bit data format).
// Buffer resource over [base, base + bytes).  The host bounds every valid
// access of one (batch, head) slice below 2^31 - 1 bytes, but a size taken as
// whole rows times the row stride can pass 2^31 (the last row's padding);
// the size is formed in 64 bits by the callers and clamped here, so it never
// wraps to a small or negative count that would cut off valid rows.
__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc(const void* base, int64_t bytes) {
  const int nb = bytes < 0 ? 0 : (bytes > 0x7FFFFFFF ? 0x7FFFFFFF : (int)bytes);
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, nb, 0x00020000);
}

// The same for `rows` rows of `row_bytes` each, in 32-bit scalar arithmetic:
// max_rows = 0x7FFFFFFF / row_bytes, computed once by the caller.
__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc_rows(const void* base, int rows, int row_bytes,
                                                                 int max_rows) {
  const int nb = rows <= 0 ? 0 : (rows >= max_rows ? 0x7FFFFFFF : rows * row_bytes);
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, nb, 0x00020000);
}

// Swizzled LDS tile layout.  A tile row holds CPR 16-byte chunks.  LDS has
// 64 four-byte banks, so a wave's 16-lane b128 row reads (16 rows, one chunk
// each) and 32-lane transposed b64 reads (4 rows x an aligned quad of chunks)
// are conflict-free when the chunk index is XORed with a row-dependent value
// whose low 2 bits spread the 16 rows of a b128 read and whose bits 2..3
// separate the 4 rows of a transposed read:
//   256-byte rows (CPR % 16 == 0): c ^ (4 (r % 4) + (r / 4) % 4)
//   128-byte rows (CPR == 8, two rows per bank line): c ^ (4 ((r / 2) % 2) + (r / 4) % 4)
// Other widths are padded by one chunk instead.
template <int CPR>
struct Swz {
  static constexpr bool kSwizzle = (CPR % 16 == 0) || CPR == 8;
  static constexpr int kStride = kSwizzle ? CPR * 16 : CPR * 16 + 16;  // bytes per row
  static __device__ __forceinline__ int chunk(int r, int c) {
    if constexpr (CPR % 16 == 0) return c ^ (4 * (r & 3) + ((r >> 2) & 3));
    else if constexpr (CPR == 8) return c ^ (4 * ((r >> 1) & 1) + ((r >> 2) & 3));
    else return c;
  }
  // Byte offset of chunk c of row r.
  static __device__ __forceinline__ uint32_t off(int r, int c) {
    return (uint32_t)(r * kStride + chunk(r, c) * 16);
  }
  // Byte offset of 4-byte element e (fp32 tiles) or the pair holding bf16 2e.
  static __device__ __forceinline__ uint32_t off_dword(int r, int e) { return off(r, e >> 2) + (e & 3) * 4; }
  // Lane address of a transposed read of bf16 rows k0..k0+3 (k0 % 4 == 0),
  // columns n0..n0+15 (n0 % 8 == 0): lane i of its 16-lane group reads the
  // 8 bytes at row k0 + i/4, column n0 + 4 (i % 4).
  static __device__ __forceinline__ uint32_t tr(int lane, int k0, int n0) {
    const int i = lane & 15;
    return off(k0 + (i >> 2), (n0 >> 3) + ((i & 3) >> 1)) + 8 * (i & 1);
  }
  // Direct-to-LDS fills (swizzled widths only) write 1 KB windows lane by
  // lane: lane l of window `win` fills physical chunk l % CPR of row
  // win * (64 / CPR) + l / CPR, which holds logical chunk chunk(row, l % CPR)
  // (the XOR is its own inverse).  Returns the source byte offset of that
  // chunk in a row-major tile with `row_bytes` bytes per row.
  static __device__ __forceinline__ int dma_src(int win, int lane, int row_bytes) {
    static_assert(kSwizzle && 1024 % kStride == 0, "direct fills need unpadded rows");
    const int r = win * (64 / CPR) + lane / CPR;
    return r * row_bytes + chunk(r, lane % CPR) * 16;
  }
};

// Padded LDS tile layout for direct fills: rows of RB data bytes at a stride
// of RB + PAD bytes (RB a multiple of 16).  With PAD = 16 a wave's b128 row
// reads (16 rows, one chunk each) spread over all 64 banks for RB = 128 or
// 256; with PAD = 64 the four rows of a transposed b64 read land on
// disjoint 64-byte bank spans for RB = 256 (PAD = 64 for RB = 128 as well).
// Every read address is a per-lane base plus a compile-time offset.
constexpr int kPastEnd = (int)0x80000000u;  // source offset past any buffer: reads zero
template <int RB, int PAD>
struct PadTile {
  static constexpr int kStride = RB + PAD;
  // Source offset, in a row-major tile of `row_bytes` bytes per row, of the
  // 16 bytes a direct fill writes at byte `o` of the LDS tile; padding slots
  // read zeros.
  static __device__ __forceinline__ int fill_src(int o, int row_bytes) {
    const int r = o / kStride, c = o % kStride;
    return c < RB ? r * row_bytes + c : kPastEnd;
  }
};

// Direct global -> LDS copy: the lanes' 16-byte chunks, read at their own
// byte offsets `voff` of buffer `r`, land lane-contiguously at lds[16 lane]
// (1 KB per wave).  Completion is tracked by vmcnt: wait_vm() before the
// barrier that publishes the data.
__device__ __forceinline__ void dma16(__amdgpu_buffer_rsrc_t r, char* lds, int voff) {
  __builtin_amdgcn_raw_ptr_buffer_load_lds(r, (__attribute__((address_space(3))) void*)lds, 16, voff, 0, 0, 0);
}
__device__ __forceinline__ void wait_vm() { asm volatile("s_waitcnt vmcnt(0)" ::: "memory"); }

typedef int i32x4 __attribute__((ext_vector_type(4)));


// Buffer descriptor words (raw 32-bit format): loads at byte offsets >=
// `bytes` return zero.
__device__ __forceinline__ i32x4 rsrc_words(const void* base, int64_t bytes) {
  const uint64_t a = reinterpret_cast<uint64_t>(base);
  const int nb = bytes < 0 ? 0 : (bytes > 0x7FFFFFFF ? 0x7FFFFFFF : (int)bytes);
  return i32x4{(int)(uint32_t)a, (int)((a >> 32) & 0xFFFFu), nb, 0x00020000};
}

__device__ __forceinline__ uint32_t lds_address(const void* p) {
  return (uint32_t)(uintptr_t)(const __attribute__((address_space(3))) void*)p;
}

// Direct HBM -> LDS copies: lane l's 16 (4) bytes, read at byte offset
// `voff` of the buffer, land at LDS byte address lds + 16 l (lds + 4 l).  The
// compiler does not see these as LDS writes, so it inserts no waits for them;
// completion is awaited explicitly (wait_vm_n) before the barrier that
// publishes the data.
__device__ __forceinline__ void fill16(i32x4 r, uint32_t lds, int voff) {
  asm volatile("s_mov_b32 m0, %0\n\ts_nop 0\n\tbuffer_load_dwordx4 %1, %2, 0 offen lds"
               :
               : "s"(lds), "v"(voff), "s"(r)
               : "memory", "m0");
}
__device__ __forceinline__ void fill4(i32x4 r, uint32_t lds, int voff) {
  asm volatile("s_mov_b32 m0, %0\n\ts_nop 0\n\tbuffer_load_dword %1, %2, 0 offen lds"
               :
               : "s"(lds), "v"(voff), "s"(r)
               : "memory", "m0");
}
// Copies that share one M0 value: set_m0 writes the LDS base, fill16_off
// copies with an immediate offset of k KB (k = 0..3), which the hardware adds
// to both the source offset and the LDS address (M0 + k KB + 16 lane), so
// four consecutive 1 KB windows need one M0 write.  Nothing else in the
// kernels that use them writes M0 (checked in the assembly by the tests).
__device__ __forceinline__ void set_m0(uint32_t v) {
  asm volatile("s_mov_b32 m0, %0\n\ts_nop 0" : : "s"(v) : "memory", "m0");
}
__device__ __forceinline__ void fill16_off(i32x4 r, int voff, int k) {
  switch (k) {
    case 0: asm volatile("buffer_load_dwordx4 %0, %1, 0 offen lds" : : "v"(voff), "s"(r) : "memory"); break;
    case 1: asm volatile("buffer_load_dwordx4 %0, %1, 0 offen offset:1024 lds" : : "v"(voff), "s"(r) : "memory"); break;
    case 2: asm volatile("buffer_load_dwordx4 %0, %1, 0 offen offset:2048 lds" : : "v"(voff), "s"(r) : "memory"); break;
    default: asm volatile("buffer_load_dwordx4 %0, %1, 0 offen offset:3072 lds" : : "v"(voff), "s"(r) : "memory"); break;
  }
}
template <int N>
__device__ __forceinline__ void wait_vm_n() {
  asm volatile("s_waitcnt vmcnt(%0)" : : "n"(N) : "memory");
}

// 32x32x16 bf16 MFMAs with explicit operand register classes (inline
// assembly), for kernels that keep some accumulators in VGPRs and others in
// AGPRs: mfma_vz / mfma_vc / mfma_vacc accumulate in VGPRs with the B
// operand in AGPRs (start from zero / from c / in place), mfma_aacc
// accumulates in AGPRs with both operands in VGPRs.  The compiler's hazard
// tracking does not see inside these statements: a caller reads a VGPR
// result with a vector instruction only after at least 19 wait states (for
// instance nops_after_mfma), writes an A / B operand with a vector
// instruction at least 2 wait states before the MFMA, and reads AGPR
// results only after nops_after_mfma.
__device__ __forceinline__ void mfma_vz(f32x16& d, const bf16x8& a, const bf16x8& b) {
  asm volatile("v_mfma_f32_32x32x16_bf16 %0, %1, %2, 0" : "=&v"(d) : "v"(a), "a"(b));
}
// mfma_vc may receive c in registers the compiler copied (from AGPRs) just
// before the statement: the statement itself waits for such a copy.  Its
// callers keep c live well past the product, so nothing overwrites c while
// the MFMA still reads it; the wait-state test of the compiled kernels checks
// this (a write of a separate accumulator input within 18 wait states) for
// every instance.
__device__ __forceinline__ void mfma_vc(f32x16& d, const bf16x8& a, const bf16x8& b, const f32x16& c) {
  asm volatile("s_nop 4\n\tv_mfma_f32_32x32x16_bf16 %0, %1, %2, %3"
               : "=&v"(d)
               : "v"(a), "a"(b), "v"(c));
}
__device__ __forceinline__ void mfma_vacc(f32x16& d, const bf16x8& a, const bf16x8& b) {
  asm volatile("v_mfma_f32_32x32x16_bf16 %0, %1, %2, %0" : "+v"(d) : "v"(a), "a"(b));
}
__device__ __forceinline__ void mfma_aacc(f32x16& d, const bf16x8& a, const bf16x8& b) {
  asm volatile("v_mfma_f32_32x32x16_bf16 %0, %1, %2, %0" : "+a"(d) : "v"(a), "v"(b));
}
// mfma_aacc behind 5 wait states (kGuard): for template instances whose
// register allocation carries an accumulator through VGPRs and writes it
// back to its AGPRs just before the product.
template <bool kGuard>
__device__ __forceinline__ void mfma_aacc_g(f32x16& d, const bf16x8& a, const bf16x8& b) {
  if constexpr (kGuard) asm volatile("s_nop 4\n\tv_mfma_f32_32x32x16_bf16 %0, %1, %2, %0" : "+a"(d) : "v"(a), "v"(b));
  else mfma_aacc(d, a, b);
}
__device__ __forceinline__ void nops_after_mfma() { asm volatile("s_nop 7\n\ts_nop 7\n\ts_nop 3" ::: "memory"); }
// After nops_after_mfma: tie the MFMA results to it, so that no read of them
// is scheduled above the nops (the nops have no data dependence of their
// own).  Volatile statements keep their relative order.
template <typename T>
__device__ __forceinline__ void tie_v(T& x) {
  asm volatile("" : "+v"(x));
}
template <typename T>
__device__ __forceinline__ void tie_a(T& x) {
  asm volatile("" : "+a"(x));
}
template <typename... T>
__device__ __forceinline__ void after_nops_v(T&... x) {
  (tie_v(x), ...);
}
template <typename... T>
__device__ __forceinline__ void after_nops_a(T&... x) {
  (tie_a(x), ...);
}

// Instruction classes for __builtin_amdgcn_sched_group_barrier.
enum : int { kSchedValu = 0x002, kSchedMfma = 0x008, kSchedDsRead = 0x100, kSchedDsWrite = 0x200 };

// Pack 8 fp32 accumulator values (registers r0..r0+7 of a 32x32 C block)
// as a bf16x8 MFMA operand, RNE.
__device__ __forceinline__ bf16x8 pack8(const f32x16& c, int r0) {
  u32x4 u;
  u[0] = pack_bf16x2(c[r0 + 0], c[r0 + 1]);
  u[1] = pack_bf16x2(c[r0 + 2], c[r0 + 3]);
  u[2] = pack_bf16x2(c[r0 + 4], c[r0 + 5]);
  u[3] = pack_bf16x2(c[r0 + 6], c[r0 + 7]);
  return *reinterpret_cast<bf16x8*>(&u);
}

// ---------------------------------------------------------------------------
// Launch mapping
// ---------------------------------------------------------------------------

// Map the hardware block index to a logical work index so that each XCD
// receives one contiguous range of logical indices, dispatched in order.
// The grid is padded to a multiple of 8; returns -1 for padding blocks.
__device__ __forceinline__ int64_t xcd_logical(int64_t bid, int64_t grid_pad, int64_t total) {
  int64_t per = grid_pad / kXcds;
  int64_t l = (bid % kXcds) * per + bid / kXcds;
  return l < total ? l : -1;
}

// Dropout keep decisions, regenerated wherever they are needed (the reverse
// pass replays the forward's mask without storing it).  Generator:
// Philox4x32-10 (Salmon, Moraes, Dror and Shaw, "Parallel random numbers: as
// easy as 1, 2, 3", SC 2011), counter (j / 4, i / 4, unit, 0), key
// (seed_lo, seed_hi).  Its four words cover the 4 x 4 block of pairs with
// i / 4, j / 4: pair (i, j) takes byte j % 4 (least significant first) of
// word i % 4 as its 8-bit draw and is kept iff draw >= p8.
// Round r (0..9) of Philox4x32-10 on the counter (c0..c3), key (k0, k1):
// the round key is the key plus r times the Weyl increments.
__device__ __forceinline__ void philox_round(uint32_t& c0, uint32_t& c1, uint32_t& c2, uint32_t& c3, uint32_t k0,
                                             uint32_t k1, int r) {
  // Each 64-bit product is one v_mad_u64_u32 (about 1.5x the round rate of
  // separate high and low multiplies), each three-way XOR one v_bitop3_b32
  // (truth table 0x96).
  const uint64_t m0 = (uint64_t)0xD2511F53u * c0, m1 = (uint64_t)0xCD9E8D57u * c2;
  const uint32_t n0 = __builtin_amdgcn_bitop3_b32((uint32_t)(m1 >> 32), c1, k0 + (uint32_t)r * 0x9E3779B9u, 0x96);
  const uint32_t n2 = __builtin_amdgcn_bitop3_b32((uint32_t)(m0 >> 32), c3, k1 + (uint32_t)r * 0xBB67AE85u, 0x96);
  c0 = n0;
  c1 = (uint32_t)m1;
  c2 = n2;
  c3 = (uint32_t)m0;
}
__device__ __forceinline__ void philox4x32_10(uint32_t& c0, uint32_t& c1, uint32_t& c2, uint32_t& c3,
                                              uint32_t k0, uint32_t k1) {
#pragma unroll
  for (int r = 0; r < 10; ++r) philox_round(c0, c1, c2, c3, k0, k1, r);
}
// Keep flags of the four bytes of one output word of a call, all at once.
// With q = 256 - p8 (p8 in [1, 255]), byte x >= p8 iff x + q carries out of
// 8 bits, and that carry is the majority of bit 7 of x, bit 7 of q and the
// carry out of the low 7 bits, which one add forms for all four bytes
// (their low 7-bit sums stay below 256).  keep_flags sets bit 8 b + 7 iff
// byte b is kept; its other bits are unspecified.
struct KeepConsts {
  uint32_t lo;  // the low 7 bits of q in every byte
  uint32_t hi;  // bit 7 of q in every byte
};
__device__ __forceinline__ KeepConsts keep_consts(uint32_t p8) {
  const uint32_t q = 256u - p8;
  return KeepConsts{(q & 0x7Fu) * 0x01010101u, (q & 0x80u) ? 0x80808080u : 0u};
}
__device__ __forceinline__ uint32_t keep_flags(uint32_t w, KeepConsts k) {
  const uint32_t s = (w & 0x7F7F7F7Fu) + k.lo;
  return __builtin_amdgcn_bitop3_b32(w, s, k.hi, 0xE8);  // bitwise majority
}
// Adds word r's flags f to the packed keep bits m of a call: bit
// 8 (j % 4) + 4 + i % 4 is set iff pair (i, j) is kept (word r = i % 4).
__device__ __forceinline__ uint32_t pack_keep(uint32_t m, uint32_t f, int r) {
  return m | ((f >> (3 - r)) & (0x10101010u << r));
}

// Keep bits of the pairs (i, j0 + e), e = 0..3, for j0 % 4 == 0: bit e set
// iff the pair is kept.
__device__ __forceinline__ uint32_t keep4_row(uint32_t seed_lo, uint32_t seed_hi, uint32_t p8, uint32_t unit,
                                              uint32_t i, uint32_t j0) {
  uint32_t c0 = j0 >> 2, c1 = i >> 2, c2 = unit, c3 = 0;
  philox4x32_10(c0, c1, c2, c3, seed_lo, seed_hi);
  const uint32_t w = (i & 2) ? ((i & 1) ? c3 : c2) : ((i & 1) ? c1 : c0);
  uint32_t bits = 0;
#pragma unroll
  for (int e = 0; e < 4; ++e) bits |= (((w >> (8 * e)) & 0xFFu) >= p8 ? 1u : 0u) << e;
  return bits;
}

// Keep bits of the pairs (i0 + e, j), e = 0..3, for i0 % 4 == 0.
__device__ __forceinline__ uint32_t keep4_col(uint32_t seed_lo, uint32_t seed_hi, uint32_t p8, uint32_t unit,
                                              uint32_t i0, uint32_t j) {
  uint32_t c0 = j >> 2, c1 = i0 >> 2, c2 = unit, c3 = 0;
  philox4x32_10(c0, c1, c2, c3, seed_lo, seed_hi);
  const uint32_t sh = 8 * (j & 3);
  return (((c0 >> sh) & 0xFFu) >= p8 ? 1u : 0u) | (((c1 >> sh) & 0xFFu) >= p8 ? 2u : 0u) |
         (((c2 >> sh) & 0xFFu) >= p8 ? 4u : 0u) | (((c3 >> sh) & 0xFFu) >= p8 ? 8u : 0u);
}

// The four lanes of a quad share the 4 x 4 blocks of pairs they draw from:
// in the forward-shaped layouts the quad holds rows 4a..4a+3 of the same
// keys, in the key-tile-outer layout keys 4a..4a+3 of the same rows.  So
// each lane computes one of the quad's four Philox calls (its group
// g = lane % 4) and packs its 16 keep bits; quad_bcast<g> then hands every
// lane the mask of group g.  keep_mask16 packs bit 4r + b (by_key = false:
// one nibble per row r, bits over the 4 keys b) or 4b + r (by_key = true:
// one nibble per key b, bits over the 4 rows r) for row r = word, key b =
// byte of the call.
__device__ __forceinline__ uint32_t keep_mask16(uint32_t seed_lo, uint32_t seed_hi, uint32_t p8, uint32_t jblk,
                                                uint32_t iblk, uint32_t unit, bool by_key) {
  uint32_t c0 = jblk, c1 = iblk, c2 = unit, c3 = 0;
  philox4x32_10(c0, c1, c2, c3, seed_lo, seed_hi);
  const uint32_t w[4] = {c0, c1, c2, c3};
  uint32_t m = 0;
#pragma unroll
  for (int r = 0; r < 4; ++r)
#pragma unroll
    for (int b = 0; b < 4; ++b) m |= (((w[r] >> (8 * b)) & 0xFFu) >= p8 ? 1u : 0u) << (by_key ? 4 * b + r : 4 * r + b);
  return m;
}

// Value of lane G of this lane's quad (DPP quad permutation, all lanes from lane G).
template <int G>
__device__ __forceinline__ uint32_t quad_bcast(uint32_t x) {
  return (uint32_t)__builtin_amdgcn_mov_dpp((int)x, G | (G << 2) | (G << 4) | (G << 6), 0xF, 0xF, false);
}

// Debug tile counter: a 64-bit atomic add, by the workgroup's first lane, of
// tiles the workgroup computed (ntiles is workgroup-uniform); nothing while
// the counter pointer is null.
__device__ __forceinline__ void count_tiles(unsigned long long* counter, int ntiles) {
  if (counter != nullptr && threadIdx.x == 0 && ntiles > 0) atomicAdd(counter, (unsigned long long)ntiles);
}

// Classification of a tile from its corners for none/causal masks: the same
// rule the skip logic and the partial-tile masking follow.  nq query rows,
// nk key rows; causal: key j allowed for query i iff j <= i + coff.
__device__ __forceinline__ uint8_t classify_analytic(int mask_mode, int64_t q0, int bq, int64_t k0,
                                                     int bk, int64_t nq, int64_t nk, int64_t coff) {
  const int64_t q_hi = (q0 + bq < nq ? q0 + bq : nq) - 1;
  const int64_t k_hi = k0 + bk - 1;
  if (mask_mode == kMaskCausal) {
    if (k0 > q_hi + coff) return kTileEmpty;
    if (k_hi <= q0 + coff && k_hi < nk) return kTileFull;
    return kTilePartial;
  }
  return (k_hi < nk) ? kTileFull : kTilePartial;
}

}  // namespace eta
