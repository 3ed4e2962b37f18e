// Device-side building blocks for the gfx950 attention kernels.
//
// Matrix-core fragment layouts used throughout (CDNA3/CDNA4 MFMA, wave64):
//   v_mfma_f32_32x32x16_bf16  D[32x32] += A[32x16] * B[16x32]
//     A: lane l holds row (l % 32), k = 8*(l/32) + t for its 8 elements t
//     B: lane l holds col (l % 32), k = 8*(l/32) + t
//     D: lane l holds col (l % 32), rows 8*(r/4) + 4*(l/32) + (r%4), r = 0..15
// Because k is summed over, any consistent relabelling of k between A and B
// leaves the product unchanged; the kernels exploit that freely.
//
// ds_read_b64_tr_b16 (gfx950): within each group of 16 lanes, lane i receives
// element t (t = 0..3) from the 8 bytes addressed by lane (4t + i/4) of the
// group, at position (i % 4).  Pointing lane j of a group at row (r0 + j/4),
// column (c0 + 4*(j%4)) of a row-major bf16 tile therefore hands lane i the
// four values tile[r0 + t][c0 + i]: a transposed 4 x 16 block.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace fa {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef short i16x4 __attribute__((ext_vector_type(4)));
typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));

constexpr float kLn2 = 0.693147180559945309f;
constexpr float kLog2e = 1.442695040888963407f;
constexpr float kNegInf = -__builtin_inff();
// Lazy-rescale slack of the online softmax, in base-2 exponent units: the
// reference max is only raised when a new score exceeds it by more than this,
// so unnormalised probabilities stay <= 2^8.
constexpr float kRescaleSlack = 8.0f;

__device__ __forceinline__ f32x16 mfma32x32x16(bf16x8 a, bf16x8 b, f32x16 c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
}

// 2^x on the transcendental unit; 2^-inf = 0.
__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }

// Round two floats to bf16 (round-to-nearest-even) and pack them.
__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
  f32x2 v = {lo, hi};
  bf16x2 p = __builtin_convertvector(v, bf16x2);
  return __builtin_bit_cast(uint32_t, p);
}

__device__ __forceinline__ bf16x8 pack_bf16x8(const float* x) {
  uint4 u;
  u.x = pack_bf16x2(x[0], x[1]);
  u.y = pack_bf16x2(x[2], x[3]);
  u.z = pack_bf16x2(x[4], x[5]);
  u.w = pack_bf16x2(x[6], x[7]);
  return __builtin_bit_cast(bf16x8, u);
}

// Round eight floats to bf16 and add the ROUNDED values to `sum` (one
// v_dot2_f32_bf16 against (1, 1) per pair).  Summing exactly the weights the
// P.V product uses makes O a properly normalised average of V rows even
// though P is rounded: the rounding of a dominant weight cancels in O / l.
__device__ __forceinline__ bf16x8 pack_bf16x8_sum(const float* x, float& sum) {
  const bf16x8 p = pack_bf16x8(x);
  const uint4 u = __builtin_bit_cast(uint4, p);
  const bf16x2 ones = __builtin_bit_cast(bf16x2, 0x3f803f80u);
  sum = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2, u.x), ones, sum, false);
  sum = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2, u.y), ones, sum, false);
  sum = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2, u.z), ones, sum, false);
  sum = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2, u.w), ones, sum, false);
  return p;
}

// One row of a transposed 32 x 32 accumulator tile (lane pair l, l+32: the
// pair's row; register r: column 8*(r/4) + 4*(l/32) + r%4), scaled by `mul`,
// stored as 32 bf16 with 16-byte stores.  Each lane holds four-column groups;
// one v_permlane32_swap per packed register hands a lane's second group to
// its partner and takes the partner's first, so lane l (l < 32) stores columns
// 16k .. 16k+7 and lane l+32 columns 16k+8 .. 16k+15 of each 16-column half k.
// Both lanes of a pair must execute it.
__device__ __forceinline__ void store_row_bf16x32(uint16_t* dst, const f32x16& acc, float mul, int hi) {
#pragma unroll
  for (int k = 0; k < 2; ++k) {
    const uint32_t x0 = pack_bf16x2(acc[8 * k] * mul, acc[8 * k + 1] * mul);
    const uint32_t x1 = pack_bf16x2(acc[8 * k + 2] * mul, acc[8 * k + 3] * mul);
    const uint32_t y0 = pack_bf16x2(acc[8 * k + 4] * mul, acc[8 * k + 5] * mul);
    const uint32_t y1 = pack_bf16x2(acc[8 * k + 6] * mul, acc[8 * k + 7] * mul);
    // lanes < 32 keep x and receive the partner's x; lanes >= 32 keep y and
    // receive the partner's y
    const auto r0 = __builtin_amdgcn_permlane32_swap(x0, y0, false, false);
    const auto r1 = __builtin_amdgcn_permlane32_swap(x1, y1, false, false);
    uint4 w;
    w.x = (uint32_t)r0[0];
    w.y = (uint32_t)r1[0];
    w.z = (uint32_t)r0[1];
    w.w = (uint32_t)r1[1];
    *(uint4*)(dst + 16 * k + 8 * hi) = w;
  }
}

// Transposed 4 x 16 read of a row-major bf16 tile in LDS (see header note).
__device__ __forceinline__ i16x4 lds_read_tr16(const uint16_t* p) {
  typedef __attribute__((address_space(3))) i16x4 lds_i16x4;
  return __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_i16x4*)(p));
}

__device__ __forceinline__ bf16x8 join_bf16x8(i16x4 lo, i16x4 hi) {
  typedef short i16x8 __attribute__((ext_vector_type(8)));
  i16x8 v = {lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
  return __builtin_bit_cast(bf16x8, v);
}

// Asynchronous 16-byte-per-lane copy global -> LDS (global_load_lds_dwordx4):
// lane i's 16 bytes land at lds_base + 16*i, lds_base being wave-uniform.
// Completion is tracked by vmcnt; a __syncthreads() (which waits for vmcnt(0))
// makes the data visible to the whole work-group.
__device__ __forceinline__ void load_lds_16B(const void* gptr, void* lds_base) {
  typedef __attribute__((address_space(1))) void glob_void;
  typedef __attribute__((address_space(3))) void lds_void;
  __builtin_amdgcn_global_load_lds((glob_void*)gptr, (lds_void*)lds_base, 16, 0, 0);
}

// The same copy issued from inline assembly, so the compiler does not track
// it as an LDS write: callers order it themselves with s_waitcnt vmcnt and
// barriers.  gbase and lds_base must be wave-uniform; lane i copies the 16
// bytes at gbase + voff_bytes into LDS at lds_base + 16*i.  m0 is saved and
// restored around the copy.  No VGPR is written, so nothing is left in flight
// towards a register.
__device__ __forceinline__ void copy16_to_lds(const void* gbase, int voff_bytes, const void* lds_base) {
  const uint32_t la = (uint32_t)(uintptr_t)(__attribute__((address_space(3))) const void*)lds_base;
  uint32_t saved;
  asm volatile(
      "s_mov_b32 %0, m0\n\t"
      "s_mov_b32 m0, %3\n\t"
      "s_nop 0\n\t"
      "global_load_lds_dwordx4 %1, %2\n\t"
      "s_mov_b32 m0, %0"
      : "=&s"(saved)
      : "v"(voff_bytes), "s"(gbase), "s"(la)
      : "memory");
}

// Two such copies under one m0 setting.  Copy 0: lane i reads the 16 bytes
// at gbase + voff0 and writes them to lds_base + 16*i.  Copy 1: it reads
// gbase + voff1 + 1024 and writes lds_base + 1024 + 16*i (the instruction
// offset applies to both the global and the LDS address).  Offsets are
// unsigned: callers pass a gbase 1 KiB below their data so that both offsets
// stay non-negative.
__device__ __forceinline__ void copy16x2_to_lds(const void* gbase, int voff0, int voff1, const void* lds_base) {
  const uint32_t la = (uint32_t)(uintptr_t)(__attribute__((address_space(3))) const void*)lds_base;
  uint32_t saved;
  asm volatile(
      "s_mov_b32 %0, m0\n\t"
      "s_mov_b32 m0, %4\n\t"
      "s_nop 0\n\t"
      "global_load_lds_dwordx4 %1, %3\n\t"
      "global_load_lds_dwordx4 %2, %3 offset:1024\n\t"
      "s_mov_b32 m0, %0"
      : "=&s"(saved)
      : "v"(voff0), "v"(voff1), "s"(gbase), "s"(la)
      : "memory");
}

// XOR swizzle of the 16-byte chunks of a bf16 K/V tile row in LDS: chunk c of
// row r lives at position c ^ swz<D>(r).  Chosen so that both the K reads of
// the S^T product (16 lanes, 16 consecutive rows, one chunk) and the
// transposed V reads (4 consecutive rows x 4 consecutive chunks per half
// wave) touch every one of the 64 LDS banks exactly once.
template <int D>
__device__ __forceinline__ int swz(int r) {
  if constexpr (D == 128) return 4 * (r & 3) + ((r >> 2) & 3);
  else return 4 * ((r >> 1) & 1) + ((r >> 2) & 3);
}

// Swizzle for d = 128 V tiles that are only read transposed: each half wave
// reads 4 consecutive rows (starting at a multiple of 4) x 4 consecutive
// chunks, so XOR-ing the chunk with 4*(r % 4) already spreads them over all 64
// banks, and rows 8 apart share one swizzle (their offset is an immediate).
__device__ __forceinline__ int swz_v128(int r) { return 4 * (r & 3); }

// (batch, query head) of slot j of a query-tile slot's B*Hq work-groups.
// Work-groups are dispatched to the 8 XCDs round-robin (XCD = block index mod
// 8, and B*Hq is then a multiple of 8), each XCD with its own L2.  The g
// query heads of a KV head read the same K/V tiles: when the (batch, KV head)
// groups divide evenly over the XCDs, slot j = 8c + x goes to group
// x + 8*(c / g), head c % g of it, so a group's heads all run on XCD x and
// its K/V is fetched into one L2 instead of g.  Otherwise heads stay in order.
__device__ __forceinline__ int xcd_grouped_head(int j, int B, int Hq, int Hkv) {
  const int g = Hq / Hkv;
  if (g == 1 || (B * Hkv) % 8 != 0) return j;
  const int x = j & 7, c = j >> 3;
  const int group = x + 8 * (c / g);
  const int b = group / Hkv, hk = group - b * Hkv;
  return b * Hq + hk * g + (c - (c / g) * g);
}

__device__ __forceinline__ float wave_xor32(float x) { return __shfl_xor(x, 32, 64); }

// max / sum of x over the lane pair (l, l ^ 32) with one v_permlane32_swap:
// after the swap the two returned registers hold x and the partner's x (in
// some order) in every lane.
__device__ __forceinline__ float pair_max32(float x) {
  const unsigned u = __builtin_bit_cast(unsigned, x);
  const auto r = __builtin_amdgcn_permlane32_swap(u, u, false, false);
  return fmaxf(__builtin_bit_cast(float, (unsigned)r[0]), __builtin_bit_cast(float, (unsigned)r[1]));
}
__device__ __forceinline__ float pair_sum32(float x) {
  const unsigned u = __builtin_bit_cast(unsigned, x);
  const auto r = __builtin_amdgcn_permlane32_swap(u, u, false, false);
  return __builtin_bit_cast(float, (unsigned)r[0]) + __builtin_bit_cast(float, (unsigned)r[1]);
}

// Packed variable-length sequences: sequence b owns rows cu[b] .. cu[b+1]-1
// of a [.., total, d] tensor.  Returns (first row, row count), with the
// offsets clamped to [0, total] and a decreasing pair read as empty, so that
// no row outside the tensor is ever addressed.
__device__ __forceinline__ int2 packed_rows(const int32_t* cu, int b, int total) {
  int s = cu[b], e = cu[b + 1];
  s = s < 0 ? 0 : (s > total ? total : s);
  e = e < s ? s : (e > total ? total : e);
  return make_int2(s, e - s);
}

__device__ __forceinline__ int clamp_len(const int32_t* lens, int b, int nk) {
  if (lens == nullptr) return nk;
  int L = lens[b];
  return L < 0 ? 0 : (L > nk ? nk : L);
}

}  // namespace fa
