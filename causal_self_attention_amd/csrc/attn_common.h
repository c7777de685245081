// Device-side building blocks shared by the gfx950 attention kernels:
// vector types, the MFMA wrappers for bf16 and fp16 operands and their
// register layout, conversions, and the launch-side helpers the host code
// needs.
//
// MFMA v_mfma_f32_32x32x16_bf16 / _f16 (CDNA4), one wave of 64 lanes, lane
// l, h = l / 32:
//   A (32 x 16, row-major M x K): lane l holds row l % 32, k = 8h .. 8h+7.
//   B (16 x 32, K x N):           lane l holds col l % 32, k = 8h .. 8h+7.
//   C (32 x 32, fp32, 16 regs):   lane l holds col l % 32; register v holds
//                                 row 8 * (v / 4) + 4h + (v % 4).
// These layouts were confirmed on the device with an in-bounds probe (every
// element of a known product in the expected lane and register), and every
// parity test of the kernels depends on them.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace gpt_attn {

// Race check for the LDS pipelines: built with GPT_ATTN_EXTRA_BARRIERS, every
// point marked with extra_barrier() (each reached by every wave of the
// workgroup) becomes a full workgroup barrier, so every LDS stage completes
// before the next begins; a race in the release schedule would make that
// build's results differ from the release build's.
__device__ __forceinline__ void extra_barrier() {
#ifdef GPT_ATTN_EXTRA_BARRIERS
  __syncthreads();
#endif
}

typedef __bf16 bf16;
typedef __bf16 bf16x8 __attribute__((__vector_size__(8 * sizeof(__bf16))));
typedef __bf16 bf16x4 __attribute__((__vector_size__(4 * sizeof(__bf16))));
typedef __bf16 bf16x2 __attribute__((__vector_size__(2 * sizeof(__bf16))));
typedef float f32x16 __attribute__((__vector_size__(16 * sizeof(float))));
typedef float f32x4 __attribute__((__vector_size__(4 * sizeof(float))));
typedef _Float16 f16;
typedef _Float16 f16x8 __attribute__((__vector_size__(8 * sizeof(_Float16))));
typedef _Float16 f16x4 __attribute__((__vector_size__(4 * sizeof(_Float16))));
typedef _Float16 f16x2 __attribute__((__vector_size__(2 * sizeof(_Float16))));
typedef int i32x4 __attribute__((__vector_size__(4 * sizeof(int))));
typedef int i32x2 __attribute__((__vector_size__(2 * sizeof(int))));

constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.69314718055994531f;
constexpr int kHeadDim = 64;

__device__ __forceinline__ f32x16 mfma32x32x16(bf16x8 a, bf16x8 b, f32x16 c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
}

// Same shapes and lane layout with fp16 operands (11-bit significands): used
// where one operand is a probability or a score gradient that must be rounded
// for the matrix core. The other operand is a bf16 input converted exactly.
__device__ __forceinline__ f32x16 mfma32x32x16_f16(f16x8 a, f16x8 b, f32x16 c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_f16(a, b, c, 0, 0, 0);
}

__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }
__device__ __forceinline__ float fast_log2(float x) { return __builtin_amdgcn_logf(x); }

__device__ __forceinline__ bf16x8 zero_bf16x8() {
  i32x4 z = {0, 0, 0, 0};
  return __builtin_bit_cast(bf16x8, z);
}

// 16-byte global load of 8 bf16, or zeros when !valid.
__device__ __forceinline__ bf16x8 load_bf16x8(const bf16* p, bool valid) {
  if (!valid) return zero_bf16x8();
  return *reinterpret_cast<const bf16x8*>(p);
}

// Pack eight fp32 values into eight bf16 (round to nearest even).
__device__ __forceinline__ bf16x8 pack_bf16x8(float a0, float a1, float a2, float a3,
                                              float a4, float a5, float a6, float a7) {
  bf16x8 r = {(bf16)a0, (bf16)a1, (bf16)a2, (bf16)a3, (bf16)a4, (bf16)a5, (bf16)a6, (bf16)a7};
  return r;
}

// Pack eight fp32 values into eight fp16 (round to nearest even).
__device__ __forceinline__ f16x8 pack_f16x8(float a0, float a1, float a2, float a3, float a4,
                                            float a5, float a6, float a7) {
  f16x8 r = {(f16)a0, (f16)a1, (f16)a2, (f16)a3, (f16)a4, (f16)a5, (f16)a6, (f16)a7};
  return r;
}

// bf16 -> fp16. Exact for finite |x| in [2^-14, 65504] (bf16 carries 8
// significant bits, fp16 11); smaller magnitudes become fp16 subnormals
// (absolute error below 2^-25) and larger ones overflow to infinity.
__device__ __forceinline__ f16 bf16_to_f16(bf16 x) { return (f16)(float)x; }

// Eight consecutive accumulator registers c[base .. base+7] as bf16.
__device__ __forceinline__ bf16x8 acc_to_bf16x8(const f32x16& c, int base) {
  return pack_bf16x8(c[base + 0], c[base + 1], c[base + 2], c[base + 3], c[base + 4],
                     c[base + 5], c[base + 6], c[base + 7]);
}

// Bit 2 <-> bit 3 swap of a row index inside a 32-row MFMA block. Loading the
// A operand's row l%32 from source row perm32(l%32) makes accumulator
// register v = 8c + t of lane half h hold source row 16c + 8h + t: eight
// consecutive rows per half, exactly the k order the next MFMA's B operand
// wants, so P / dS never need a lane shuffle.
__device__ __forceinline__ int perm32(int r) {
  return (r & ~12) | ((r & 4) << 1) | ((r & 8) >> 1);
}

__device__ __forceinline__ float wave_xor32(float x) { return __shfl_xor(x, 32, 64); }

// Sum of the eight fp16 values of v added to acc (two-element dot products
// with (1, 1), fp32 accumulation).
__device__ __forceinline__ float sum_f16x8(f16x8 v, float acc) {
  const f16x2 one = {(f16)1.0f, (f16)1.0f};
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const f16x2 pair = {v[2 * i], v[2 * i + 1]};
    acc = __builtin_amdgcn_fdot2(pair, one, acc, false);
  }
  return acc;
}

// True when pred holds on any lane of the wave (wave-uniform result).
__device__ __forceinline__ bool wave_any(bool pred) { return __any(pred); }

// Kinds of 32-key x 32-query block, decided once per block (wave-uniform):
// every key <= every query (no mask), the aligned diagonal block (key0 ==
// q0, mask is a fixed triangle), no visible pair at all, or a block at the
// end of the sequence (general mask).
enum BlockKind { kFull = 0, kDiag = 1, kEmpty = 2, kGeneral = 3 };

__device__ __forceinline__ int block_kind(int key0, int q0, int T) {
  if (key0 > q0 + 31 || key0 >= T || q0 >= T) return kEmpty;
  const bool in_range = key0 + 32 <= T && q0 + 32 <= T;
  if (in_range && key0 + 31 <= q0) return kFull;
  if (in_range && key0 == q0) return kDiag;
  return kGeneral;
}

// Eight bf16 -> eight fp16 (see bf16_to_f16).
__device__ __forceinline__ f16x8 bf16x8_to_f16x8(bf16x8 x) {
  return pack_f16x8((float)x[0], (float)x[1], (float)x[2], (float)x[3], (float)x[4],
                    (float)x[5], (float)x[6], (float)x[7]);
}

__device__ __forceinline__ f16x8 zero_f16x8() {
  i32x4 z = {0, 0, 0, 0};
  return __builtin_bit_cast(f16x8, z);
}

// x, through an empty volatile asm statement: a value the compiler cannot
// compute ahead of the branch it sits in. Work that only a rare branch needs
// starts from such a value, so the compiler neither does it on every pass
// nor hoists its invariant parts into registers kept live for the whole
// loop.
__device__ __forceinline__ float opaque_f32(float x) {
  asm volatile("" : "+v"(x));
  return x;
}
// The same for a wave-uniform value, kept in a scalar register.
__device__ __forceinline__ uint32_t opaque_u32_uniform(uint32_t x) {
  asm volatile("" : "+s"(x));
  return x;
}

// The float value of a bf16 bit pattern (the pattern in the low 16 bits).
__device__ __forceinline__ float bf16_bits_to_float(uint32_t b) { return __uint_as_float(b << 16); }

// Block exponents. The fp16 matrix-core operands carry a power-of-two scale
// per operand block: x_s = x * 2^e is formed exactly (ldexp) before the
// rounding to fp16, and every product of scaled operands is unscaled exactly
// at the end, so fp16's narrow exponent range (normal 2^-14 .. 65504) costs
// nothing while the block's largest magnitude sits near the top of it. A
// scale that only moves the exponent commutes with every rounding in
// between, so outputs are equivariant under power-of-two scaling of the
// inputs.
//
// block_exp(m, target): the e with m * 2^e in [2^target, 2^(target+1)) for
// finite m > 0, or 0 when m is 0 or not finite (a non-finite input gives
// non-finite outputs whatever the scale). m = f * 2^k with f in [0.5, 1)
// gives e = target + 1 - k.
__device__ __forceinline__ int block_exp(float m, int target) {
  if (!(m > 0.f) || !(m <= 3.402823466e38f)) return 0;
  return target + 1 - __builtin_amdgcn_frexp_expf(m);
}

// Eight 16-bit values times 2^e, rounded to fp16: exact when the scaled
// value is an fp16 normal number, as it is for every bf16 value of a block
// down to 2^(-14-target) times the block's largest magnitude.
template <typename V>
__device__ __forceinline__ f16x8 cvt_f16_scaled(V x, int e) {
  return pack_f16x8(ldexpf((float)x[0], e), ldexpf((float)x[1], e), ldexpf((float)x[2], e),
                    ldexpf((float)x[3], e), ldexpf((float)x[4], e), ldexpf((float)x[5], e),
                    ldexpf((float)x[6], e), ldexpf((float)x[7], e));
}

// Largest magnitude of eight 16-bit values folded into mx.
template <typename V>
__device__ __forceinline__ void fold_absmax(V x, float& mx) {
#pragma unroll
  for (int i = 0; i < 8; ++i) mx = fmaxf(mx, fabsf((float)x[i]));
}

// Maximum of a wave-uniform reduction over all 64 lanes.
__device__ __forceinline__ float wave_max(float x) {
#pragma unroll
  for (int m = 1; m < 64; m <<= 1) x = fmaxf(x, __shfl_xor(x, m, 64));
  return x;
}

// The two 16-bit input types of the MFMA kernels. vec is eight elements (one
// 16-byte load); mfma is the 32x32x16 product of two such operands with fp32
// accumulation; to_f16 converts for the products that run in fp16 (exact for
// bf16 in fp16's normal range, the identity for fp16); round rounds an fp32
// value to the type (nearest even).
template <typename T>
struct In16;

template <>
struct In16<bf16> {
  typedef bf16x8 vec;
  typedef bf16x4 vec4;
  __device__ static __forceinline__ f32x16 mfma(vec a, vec b, f32x16 c) {
    return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
  }
  __device__ static __forceinline__ f16x8 to_f16(vec x) { return bf16x8_to_f16x8(x); }
  __device__ static __forceinline__ vec zero() { return zero_bf16x8(); }
  __device__ static __forceinline__ bf16 round(float x) { return (bf16)x; }
};

template <>
struct In16<f16> {
  typedef f16x8 vec;
  typedef f16x4 vec4;
  __device__ static __forceinline__ f32x16 mfma(vec a, vec b, f32x16 c) {
    return __builtin_amdgcn_mfma_f32_32x32x16_f16(a, b, c, 0, 0, 0);
  }
  __device__ static __forceinline__ f16x8 to_f16(vec x) { return x; }
  __device__ static __forceinline__ vec zero() { return zero_f16x8(); }
  __device__ static __forceinline__ f16 round(float x) { return (f16)x; }
};

// ds_read_b64_tr_b16 (CDNA4): each lane supplies the LDS address of four
// consecutive 16-bit elements; inside every group of 16 lanes the 16 x 4
// block is transposed, so that lane i of the group receives element i of the
// four rows that lanes 4e..4e+3 (e = 0..3) addressed. (Characterised on the
// device with an in-bounds probe.)
__device__ __forceinline__ f16x4 lds_read_tr16(const f16* p) {
#if __HIP_DEVICE_COMPILE__
  typedef __fp16 half4 __attribute__((__vector_size__(4 * sizeof(__fp16))));
  typedef _Float16 __attribute__((address_space(3))) lds_f16;
  typedef half4 __attribute__((address_space(3))) lds_half4;
  return __builtin_bit_cast(f16x4,
                            __builtin_amdgcn_ds_read_tr16_b64_v4f16((lds_half4*)((lds_f16*)p)));
#else
  (void)p;
  f16x4 z = {};
  return z;
#endif
}

// MFMA 32x32x16 operand whose k index runs down the rows of an LDS tile
// stored [k][n] (n contiguous, row stride ld elements, rows 8-byte aligned):
// lane l receives tile[k0 + 8h + t][n0 + l % 32], t = 0..7, h = l / 32 --
// i.e. the A operand of a product whose M index is the tile's column, or the
// B operand whose N index is. Two transposing reads of four rows each.
__device__ __forceinline__ f16x8 lds_operand_tr(const f16* tile, int ld, int k0, int n0,
                                                int lane) {
  const int g = lane >> 4, i = lane & 15;
  const int row = k0 + 8 * (g >> 1) + (i >> 2);
  const int col = n0 + 16 * (g & 1) + 4 * (i & 3);
  const f16x4 lo = lds_read_tr16(tile + row * ld + col);
  const f16x4 hi = lds_read_tr16(tile + (row + 4) * ld + col);
  f16x8 r = {lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
  return r;
}

}  // namespace gpt_attn
