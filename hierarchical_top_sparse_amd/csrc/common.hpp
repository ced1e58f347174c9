// Shared device helpers for the gfx950 LLSA kernels: vector types, Morton addressing,
// MFMA wrappers, LDS transpose reads and wave-level reductions.
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>
#include <type_traits>

namespace llsa {

typedef __bf16 bf16;
typedef __attribute__((__vector_size__(8 * sizeof(__bf16)))) __bf16 bf16x8;
typedef __attribute__((__vector_size__(4 * sizeof(__bf16)))) __bf16 bf16x4;
typedef __attribute__((__vector_size__(4 * sizeof(float)))) float f32x4;
typedef __attribute__((__vector_size__(4 * sizeof(short)))) short i16x4;
typedef __attribute__((__vector_size__(4 * sizeof(int)))) int i32x4;

constexpr int kDim = 64;        // head_dim
constexpr int kBlock = 16;      // B: a 4x4 pixel tile
constexpr int kBlockShift = 4;  // log2(B)
constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;

// ------------------------------------------------------------------ token addressing
// Geometry of the pixel grid: log2 of height/width.  In raster layout a token at Morton
// position m lives at row y*W + x; in Morton layout at row m.
struct Grid {
  int hbits;   // log2(height)
  int wbits;   // log2(width)
  int raster;  // 1: tensors are raster-ordered
};

__device__ __forceinline__ uint32_t compact_even_bits(uint32_t v) {
  v &= 0x55555555u;
  v = (v | (v >> 1)) & 0x33333333u;
  v = (v | (v >> 2)) & 0x0f0f0f0fu;
  v = (v | (v >> 4)) & 0x00ff00ffu;
  v = (v | (v >> 8)) & 0x0000ffffu;
  return v;
}

// Morton position -> raster index.  Low 2r bits interleave x (even) and y (odd), r = min side
// bits; the remaining high bits extend the longer side.
__device__ __forceinline__ int morton_to_raster(int m, int hbits, int wbits) {
  const int r = hbits < wbits ? hbits : wbits;
  const uint32_t um = (uint32_t)m;
  const uint32_t low = um & ((1u << (2 * r)) - 1u);
  const uint32_t high = um >> (2 * r);
  uint32_t x = compact_even_bits(low);
  uint32_t y = compact_even_bits(low >> 1);
  if (wbits > hbits) x |= high << r;
  else y |= high << r;
  return (int)((y << wbits) | x);
}

__device__ __forceinline__ int token_row(int m, const Grid& g) {
  return g.raster ? morton_to_raster(m, g.hbits, g.wbits) : m;
}

// Row of the first token of level-1 block j (its 4x4 tile's top-left pixel in raster layout).
__device__ __forceinline__ int block_corner(int j, const Grid& g) {
  return g.raster ? morton_to_raster(j << 4, g.hbits, g.wbits) : (j << 4);
}

// Row offset of token t (0..15) of a level-1 block from the block's first row: in raster
// layout the tile's pixel (x, y) = (bits 0,2 ; bits 1,3) of t; both sides are >= 4 pixels.
__device__ __forceinline__ int tile_offset(int t, const Grid& g) {
  if (!g.raster) return t;
  const int tx = (t & 1) | ((t >> 1) & 2);
  const int ty = ((t >> 1) & 1) | ((t >> 2) & 2);
  return (ty << g.wbits) + tx;
}

// ------------------------------------------------------------------ buffer loads
// Raw buffer resources over one head's tensor: 32-bit byte offsets, and any access past
// `bytes` returns zeros (used for masked rows: offset kNoRow).
typedef __amdgpu_buffer_rsrc_t rsrc_t;
constexpr uint32_t kNoRow = 0x80000000u;
__device__ __forceinline__ rsrc_t make_rsrc(const void* base, uint32_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc((void*)base, (short)0, (int)bytes, 0x00020000);
}
__device__ __forceinline__ bf16x8 buf_load8(rsrc_t r, uint32_t off) {
  const i32x4 v = __builtin_amdgcn_raw_buffer_load_b128(r, off, 0, 0);
  return *(const bf16x8*)&v;
}
__device__ __forceinline__ f32x4 buf_load4f(rsrc_t r, uint32_t off) {
  const i32x4 v = __builtin_amdgcn_raw_buffer_load_b128(r, off, 0, 0);
  return *(const f32x4*)&v;
}
__device__ __forceinline__ int uniform(int v) { return __builtin_amdgcn_readfirstlane(v); }
// A wave-uniform pointer moved to scalar registers (buffer descriptors must be scalar; a
// descriptor the compiler cannot prove uniform costs a readfirstlane loop per load).
__device__ __forceinline__ const void* uniform_ptr(const void* p) {
  const uint64_t v = (uint64_t)p;
  const uint32_t lo = __builtin_amdgcn_readfirstlane((uint32_t)v);
  const uint32_t hi = __builtin_amdgcn_readfirstlane((uint32_t)(v >> 32));
  return (const void*)(((uint64_t)hi << 32) | lo);
}
__device__ __forceinline__ rsrc_t make_rsrc_uniform(const void* base, uint32_t bytes) {
  return make_rsrc(uniform_ptr(base), (uint32_t)__builtin_amdgcn_readfirstlane(bytes));
}

// 2^x on the hardware exp unit (v_exp_f32), no denormal fix-up: arguments here are <= 0 and
// results below 2^-126 only ever multiply probabilities that are negligible anyway.
__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }

// ------------------------------------------------------------------ conversions
// Floats go to bf16 (round to nearest even) two at a time: one v_cvt_pk_bf16_f32 per pair,
// already packed the way the MFMA operands hold them (element 2i in the low half).
typedef __attribute__((__vector_size__(2 * sizeof(float)))) float f32x2;
typedef __attribute__((__vector_size__(2 * sizeof(__bf16)))) __bf16 bf16x2;
typedef __attribute__((__vector_size__(2 * sizeof(uint32_t)))) uint32_t u32x2;
typedef __attribute__((__vector_size__(4 * sizeof(uint32_t)))) uint32_t u32x4;

__device__ __forceinline__ uint32_t pack2_bf16(float a, float b) {
  return __builtin_bit_cast(uint32_t, __builtin_convertvector((f32x2){a, b}, bf16x2));
}
// a = hi.x + lo.x, b = hi.y + lo.y with hi = bf16(a, b) and lo = bf16 of the remainders: the
// pair carries ~16 mantissa bits.  The bf16 halves of hi are widened back by a shift / mask.
__device__ __forceinline__ void split2_bf16(float a, float b, uint32_t& hi, uint32_t& lo) {
  hi = pack2_bf16(a, b);
  lo = pack2_bf16(a - __builtin_bit_cast(float, hi << 16),
                  b - __builtin_bit_cast(float, hi & 0xffff0000u));
}
__device__ __forceinline__ bf16x4 pack4_bf16(float a, float b, float c, float d) {
  return __builtin_bit_cast(bf16x4, (u32x2){pack2_bf16(a, b), pack2_bf16(c, d)});
}
__device__ __forceinline__ bf16x4 pack4_bf16(f32x4 a) { return pack4_bf16(a[0], a[1], a[2], a[3]); }
// x[0..3] = hi + lo elementwise
__device__ __forceinline__ void split4_bf16(float x0, float x1, float x2, float x3, bf16x4& hi,
                                            bf16x4& lo) {
  uint32_t h0, l0, h1, l1;
  split2_bf16(x0, x1, h0, l0);
  split2_bf16(x2, x3, h1, l1);
  hi = __builtin_bit_cast(bf16x4, (u32x2){h0, h1});
  lo = __builtin_bit_cast(bf16x4, (u32x2){l0, l1});
}
// (a, b) = hi + lo elementwise, a in elements 0..3, b in 4..7
__device__ __forceinline__ void split8_bf16(f32x4 a, f32x4 b, bf16x8& hi, bf16x8& lo) {
  uint32_t h[4], l[4];
  split2_bf16(a[0], a[1], h[0], l[0]);
  split2_bf16(a[2], a[3], h[1], l[1]);
  split2_bf16(b[0], b[1], h[2], l[2]);
  split2_bf16(b[2], b[3], h[3], l[3]);
  hi = __builtin_bit_cast(bf16x8, (u32x4){h[0], h[1], h[2], h[3]});
  lo = __builtin_bit_cast(bf16x8, (u32x4){l[0], l[1], l[2], l[3]});
}
__device__ __forceinline__ bf16x8 cvt8_bf16(f32x4 a, f32x4 b) {
  return __builtin_bit_cast(bf16x8, (u32x4){pack2_bf16(a[0], a[1]), pack2_bf16(a[2], a[3]),
                                            pack2_bf16(b[0], b[1]), pack2_bf16(b[2], b[3])});
}
__device__ __forceinline__ bf16x8 cvt8_bf16(const float* f) {
  return cvt8_bf16(f32x4{f[0], f[1], f[2], f[3]}, f32x4{f[4], f[5], f[6], f[7]});
}

// ------------------------------------------------------------------ MFMA
// v_mfma_f32_16x16x32_bf16: lane l holds A[l%16][8*(l/16) .. +7], B[8*(l/16) .. +7][l%16];
// the result C[4*(l/16) + i][l%16], i = 0..3.
__device__ __forceinline__ f32x4 mfma_bf16_k32(bf16x8 a, bf16x8 b, f32x4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}
// v_mfma_f32_16x16x16_bf16: lane l holds A[l%16][4*(l/16) .. +3], B[4*(l/16) .. +3][l%16].
// On gfx950 it takes as many cycles as the 16x16x32 form (measured: ~18 cycles per SIMD for
// either), so it runs at half the rate per flop.
__device__ __forceinline__ f32x4 mfma_bf16_k16(bf16x4 a, bf16x4 b, f32x4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(*(i16x4*)&a, *(i16x4*)&b, c, 0, 0, 0);
}
__device__ __forceinline__ bf16x8 cat8(bf16x4 x, bf16x4 y) {
  return __builtin_shufflevector(x, y, 0, 1, 2, 3, 4, 5, 6, 7);
}
// Two 16x16x16 products in one 16x16x32: a0 b0 + a1 b1, with each operand pair laid out as
// the 16x16x16 form holds it.  Lane l's k slots 8(l/16) .. +3 take the first pair's k values
// 4(l/16) .. +3 and slots +4 .. +7 the second's, so the sum over the 32 slots is the sum of
// both products (hi + lo parts of one operand: a0 = a1 or b0 = b1).
__device__ __forceinline__ f32x4 mfma_bf16_k16x2(bf16x4 a0, bf16x4 b0, bf16x4 a1, bf16x4 b1,
                                                 f32x4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(cat8(a0, a1), cat8(b0, b1), c, 0, 0, 0);
}
// v_mfma_f32_16x16x4_f32: lane l holds A[l%16][l/16], B[l/16][l%16].
__device__ __forceinline__ f32x4 mfma_f32_k4(float a, float b, f32x4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x4f32(a, b, c, 0, 0, 0);
}

// ------------------------------------------------------------------ LDS transpose read
// ds_read_b64_tr_b16: within each 16-lane group, lane 4r+c supplies the address of row r,
// columns 4c..4c+3 of a 4x16 block of 16-bit values; lane n of the group receives column n
// (rows 0..3).  So reading rows k0..k0+3 of a row-major [k][n] LDS matrix this way gives
// each lane the MFMA operand slice B[k0 .. k0+3][n].
typedef __attribute__((address_space(3))) i16x4 lds_i16x4;
typedef __attribute__((address_space(3))) void lds_void;
__device__ __forceinline__ bf16x4 lds_read_tr16(const bf16* lds_ptr) {
  i16x4 r = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4*)(lds_ptr));
  return *(bf16x4*)&r;
}

// Orders this wave's LDS accesses: writes before it are visible to reads after it, and reads
// before it complete before later writes.  The LDS executes one wave's requests in issue order,
// so only compiler reordering has to be stopped: a compiler memory barrier does that without a
// memory fence (a fence would also wait for every vector load in flight, including the
// prefetches that load into LDS).
__device__ __forceinline__ void wave_lds_sync() {
  __builtin_amdgcn_wave_barrier();
  asm volatile("" ::: "memory");
}

// ------------------------------------------------------------------ XCD-aware numbering
// The dispatcher sends workgroup i to XCD i % 8.  Renumbering gives XCD x the contiguous range
// [x*q + min(x, r), ...) of logical workgroups (q = n / 8, r = n % 8), so spatially adjacent
// work shares one L2.
__device__ __forceinline__ int xcd_block(int bid, int nblocks) {
  const int x = bid & 7, k = bid >> 3;
  const int q = nblocks >> 3, r = nblocks & 7;
  return x * q + (x < r ? x : r) + k;
}

// ------------------------------------------------------------------ cross-lane
// Reduce over the four 16-lane rows of the wave (lanes n, n+16, n+32, n+48) on the VALU:
// v_permlane16_swap exchanges rows 0<->1 and 2<->3 between its two operands, and
// v_permlane32_swap the two 32-lane halves, so with both operands holding v the two results
// of each swap are v and its partner row's v (the order does not matter for max and sum).
__device__ __forceinline__ float bits_f(unsigned u) { return __builtin_bit_cast(float, u); }
__device__ __forceinline__ unsigned f_bits(float f) { return __builtin_bit_cast(unsigned, f); }
__device__ __forceinline__ float group4_max(float v) {
  const auto r = __builtin_amdgcn_permlane16_swap(f_bits(v), f_bits(v), false, false);
  const float m = fmaxf(bits_f(r[0]), bits_f(r[1]));
  const auto s = __builtin_amdgcn_permlane32_swap(f_bits(m), f_bits(m), false, false);
  return fmaxf(bits_f(s[0]), bits_f(s[1]));
}
__device__ __forceinline__ float group4_sum(float v) {
  const auto r = __builtin_amdgcn_permlane16_swap(f_bits(v), f_bits(v), false, false);
  const float m = bits_f(r[0]) + bits_f(r[1]);
  const auto s = __builtin_amdgcn_permlane32_swap(f_bits(m), f_bits(m), false, false);
  return bits_f(s[0]) + bits_f(s[1]);
}

}  // namespace llsa
