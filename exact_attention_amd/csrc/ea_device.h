// Device primitives for the gfx950 attention kernels: MFMA wrappers, the two
// exp2 implementations, LDS swizzle, transposed LDS reads and lane exchanges.
//
// Lane layouts used throughout (wave64, verified on the device):
//   v_mfma_f32_32x32x16_bf16  A[m][k]: lane l holds row m = l%32,
//       k = 8*(l/32) + 0..7;  B[k][n]: column n = l%32, k = 8*(l/32) + 0..7;
//       C[m][n] element i of lane l: m = 8*(i/4) + 4*(l/32) + i%4, n = l%32.
//   v_mfma_f32_16x16x32_bf16  A: row l%16, k = 8*(l/16) + 0..7; B alike;
//       C element i of lane l: m = 4*(l/16) + i, n = l%16.
//   ds_read_b64_tr_b16: within each group of 16 lanes, result lane n, element
//       j is element n%4 of the four 16-bit values addressed by lane 4*j + n/4.
//   v_mfma_scale_f32_32x32x64_f8f6f4 (fp8 A/B): lane l holds row/column l%32
//       and k = 16*(l/32) + 0..15 (bytes 0..15) and 32 + 16*(l/32) + 0..15
//       (bytes 16..31); the e8m0 scale of (row m, k-block b of 32) comes from
//       lane m + 32*b.
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace ea {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef short i16x4 __attribute__((ext_vector_type(4)));
typedef int i32x4 __attribute__((ext_vector_type(4)));
typedef int i32x2 __attribute__((ext_vector_type(2)));
typedef int i32x8 __attribute__((ext_vector_type(8)));

#define EA_LDS __attribute__((address_space(3)))

constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;
constexpr float kNegInf = -__builtin_inff();

__device__ __forceinline__ f32x16 mfma32x32x16(bf16x8 a, bf16x8 b, f32x16 c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
}
__device__ __forceinline__ f32x4 mfma16x16x32(bf16x8 a, bf16x8 b, f32x4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}

// ---------------------------------------------------------------------------
// exp2
// ---------------------------------------------------------------------------
// Hardware: v_exp_f32 (returns 0 for -inf).
__device__ __forceinline__ float exp2_hw(float x) { return __builtin_amdgcn_exp2f(x); }

// FMA-pipe exp2 following the range-reduction + cubic scheme of
// "FlashAttention-4: algorithm-pipeline co-design for Blackwell" (hybrid
// exponent section) and "FlashAttention4 close reading" (section 3.1.3):
// clamp x at -127 (below it the result is 0), split x = n + f with n = floor(x), f in [0,1), evaluate a
// cubic for 2^f by Horner (3 FMAs) and put n into the exponent field
// (v_ldexp_f32). On gfx950 the round-down split is one v_floor_f32 and a
// subtraction instead of the magic-bias add.
// Coefficients: degree-3 fit with p0 = 1 minimising the maximum relative error
// on [0,1) (linear-programming minimax on a 20001-point grid); max relative
// error 8.57e-5, mean 5.44e-5 when evaluated in fp32.
constexpr float kExp2P1 = 0.6951173f;
constexpr float kExp2P2 = 0.22764353f;
constexpr float kExp2P3 = 0.07706803f;

__device__ __forceinline__ float exp2_poly(float x) {
  // n = floor(x) is an exact integer; f = x - n lies in [0, 1] (it rounds up to
  // exactly 1.0 for x just below an integer, which the cubic still handles:
  // p(1) ~ 2). v_fract_f32 is not used: it clamps its result below 1.0, so
  // x - fract(x) is then not an integer for tiny negative x. Inputs below
  // -127 (masked scores are -inf) give exactly 0, as an underflow would.
  const float xc = __builtin_fmaxf(x, -127.0f);
  const float n = __builtin_floorf(xc);
  const float f = xc - n;
  const float p = __builtin_fmaf(__builtin_fmaf(__builtin_fmaf(kExp2P3, f, kExp2P2), f, kExp2P1), f, 1.0f);
  const float r = __builtin_amdgcn_ldexpf(p, (int)n);
  return x < -127.0f ? 0.0f : r;
}

// ---------------------------------------------------------------------------
// lane exchange: value of the partner lane l ^ 32 (v_permlane32_swap, no LDS)
// ---------------------------------------------------------------------------
__device__ __forceinline__ float max_with_partner32(float x) {
  auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return __builtin_fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
__device__ __forceinline__ float sum_with_partner32(float x) {
  auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}

// ---------------------------------------------------------------------------
// bf16 packing
// ---------------------------------------------------------------------------
__device__ __forceinline__ uint32_t pack_bf16x2(float a, float b) {
  bf16x2 v;
  v[0] = (__bf16)a;
  v[1] = (__bf16)b;
  return __builtin_bit_cast(uint32_t, v);
}

// One 32-wide d tile of a transposed output accumulator (a lane holds row c
// = lane mod 32 and d chunks 8 g + 4 hh .. + 3, g = 0..3, hh = lane div 32),
// scaled by f and rounded to bf16, as 16-byte row pieces: lanes c and c + 32
// trade one chunk of each pair (g = 2 j, 2 j + 1) across the lane halves, so
// out[j] holds d 16 j + 8 hh .. + 7 of row c. Writing 16 bytes per lane halves
// the store instructions of the 8-byte chunks. Every lane of the wave must
// call it (the partners of a row hold the same row).
__device__ __forceinline__ void pack_rows16(const f32x16& acc, float f, uint4 (&out)[2]) {
#pragma unroll
  for (int j = 0; j < 2; ++j) {
    const int ga = 2 * j, gb = 2 * j + 1;
    const uint32_t a0 = pack_bf16x2(acc[4 * ga] * f, acc[4 * ga + 1] * f);
    const uint32_t a1 = pack_bf16x2(acc[4 * ga + 2] * f, acc[4 * ga + 3] * f);
    const uint32_t b0 = pack_bf16x2(acc[4 * gb] * f, acc[4 * gb + 1] * f);
    const uint32_t b1 = pack_bf16x2(acc[4 * gb + 2] * f, acc[4 * gb + 3] * f);
    // lanes 32..63 of the first operand trade with lanes 0..31 of the second:
    // lane c keeps its chunk 2 j and takes its partner's, lane c + 32 takes
    // lane c's chunk 2 j + 1 and keeps its own
    const auto s0 = __builtin_amdgcn_permlane32_swap(a0, b0, false, false);
    const auto s1 = __builtin_amdgcn_permlane32_swap(a1, b1, false, false);
    out[j] = uint4{s0[0], s1[0], s0[1], s1[1]};
  }
}

// Sum of the two bf16 halves of a packed word, accumulated in fp32
// (v_dot2c_f32_bf16 with (1,1)).
__device__ __forceinline__ float add_bf16x2(uint32_t packed, float acc) {
  bf16x2 ones;
  ones[0] = (__bf16)1.0f;
  ones[1] = (__bf16)1.0f;
  return __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2, packed), ones, acc, false);
}

// ---------------------------------------------------------------------------
// LDS tiles: rows of D bf16, stored in 16-byte chunks permuted per row:
// chunk position = chunk ^ swz(row). For D = 128 (16 chunks per row)
// swz(row) = ((row & 3) << 2) | ((row >> 2) & 3), which is a bijection on
// row % 16, so
//  (a) 16 consecutive rows read at one chunk (MFMA A/B operand reads) hit 16
//      distinct 16-byte bank groups, and
//  (b) 4 consecutive rows x 4 consecutive chunks (32 lanes of a transposed
//      read) also hit 16 distinct bank groups: the row picks bits 2-3 of the
//      position, the chunk bits 0-1.
// swz depends on row % 16 only, so moving 16 rows (or 32) is a constant
// address offset. D = 64 rows have 8 chunks: swz(row) = ((row & 3) << 1) |
// ((row >> 2) & 1). D = 192 rows (384 bytes, 24 chunks) span one and a half
// 256-byte bank lines, so a row's parity already picks the bank half of a
// chunk; swz(row) = (row >> 1) & 7 permutes the chunk within its aligned
// group of 8 (it stays inside the row) and gives the 8 rows of each parity
// distinct bank groups: 16 consecutive rows at one chunk hit all 16 groups.
// ---------------------------------------------------------------------------
template <int D>
__device__ __forceinline__ int swz(int row) {
  if constexpr (D == 192) return (row >> 1) & 7;
  if constexpr (D >= 128) return ((row & 3) << 2) | ((row >> 2) & 3);
  return ((row & 3) << 1) | ((row >> 2) & 1);
}
// element offset (in bf16 units) of (row, col) in a swizzled tile
template <int D>
__device__ __forceinline__ int tile_off(int row, int col) {
  return row * D + (((col >> 3) ^ swz<D>(row)) << 3) + (col & 7);
}

// Packed (varlen) forwards walk sequences in a virtual order: the actual
// sequence of virtual index sv, or -1 when the order holds an index outside
// [0, nseq) (such an entry then contributes no rows).
__device__ __forceinline__ int varlen_seq(const int* order, int nseq, int sv) {
  if (order == nullptr) return sv;
  const int s = order[sv];
  return (s >= 0 && s < nseq) ? s : -1;
}

// Workgroup-uniform integer pinned to a scalar register (the compiler cannot
// always prove uniformity through divisions done on the vector unit).
__device__ __forceinline__ int uniform(int x) { return __builtin_amdgcn_readfirstlane(x); }
// Workgroup-uniform pointer pinned to scalar registers (both 32-bit halves).
template <typename T>
__device__ __forceinline__ T* uniform_ptr(T* p) {
  const uint64_t v = (uint64_t)p;
  const uint32_t lo = (uint32_t)__builtin_amdgcn_readfirstlane((int)(uint32_t)v);
  const uint32_t hi = (uint32_t)__builtin_amdgcn_readfirstlane((int)(uint32_t)(v >> 32));
  return (T*)(((uint64_t)hi << 32) | lo);
}

// Buffer resource over [base, base + nbytes) (raw, stride 0): loads at offsets
// >= nbytes return zeros. The range check covers the VGPR offset only.
__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc(const void* base, uint32_t nbytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, (int)nbytes, 0x00020000);
}
__device__ __forceinline__ i32x4 buffer_load16(__amdgpu_buffer_rsrc_t r, uint32_t voff) {
  return __builtin_amdgcn_raw_buffer_load_b128(r, (int)voff, 0, 0);
}
// LDS DMA: 16 bytes per lane from the buffer at voff into LDS; lane s lands at
// lds + 16 s (lds must be wave-uniform). Out-of-range lanes write zeros.
__device__ __forceinline__ void buffer_load16_lds(__amdgpu_buffer_rsrc_t r, EA_LDS void* lds, uint32_t voff) {
  __builtin_amdgcn_raw_ptr_buffer_load_lds(r, lds, 16, (int)voff, 0, 0, 0);
}

__device__ __forceinline__ i16x4 ds_read_tr16(const EA_LDS uint16_t* p) {
  return __builtin_amdgcn_ds_read_tr16_b64_v4i16((EA_LDS i16x4*)p);
}

template <typename T>
__device__ __forceinline__ T lds_load(const EA_LDS void* p) {
  return *(const EA_LDS T*)p;
}
template <typename T>
__device__ __forceinline__ void lds_store(EA_LDS void* p, T v) {
  *(EA_LDS T*)p = v;
}

}  // namespace ea
