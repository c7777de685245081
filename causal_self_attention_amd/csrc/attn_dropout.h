// Attention dropout on the device: the keep decision for (head, query, key)
// from the counter-based generator Philox4x32-10 (Salmon, Moraes, Dror and
// Shaw, "Parallel random numbers: as easy as 1, 2, 3", SC'11, section 4).
//
// nanoGPT hands its dropout rate to the fused attention call in training
// (page "nanoGPT: a real GPT in two 300-line files", section 2 "How the code
// works"): each attention weight is zeroed with probability p after the
// softmax and the survivors are scaled by 1/(1-p). The kernels never store a
// mask: forward and backward both regenerate it from
//   key     = (seed low word, seed high word)
//   counter = (key index / 8, query index, flat head b*H + h, offset)
// One Philox block (four 32-bit words) covers 8 consecutive keys of one
// query: key j takes the 16-bit field j % 2 of word (j % 8) / 2, and is kept
// iff that field is >= thr = round(p * 65536). Kept weights are scaled by
// 65536 / (65536 - thr).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace gpt_attn {

struct Dropout {
  uint32_t thr;     // 0 disables dropout
  float scale;      // 65536 / (65536 - thr)
  uint32_t key0, key1, offset;
};

// Philox4x32-10 on counter (x0..x3) under key (k0, k1). Per round: the
// products M0*x0 and M1*x2 (64-bit), then the words become
// (hi(M1 x2) ^ x1 ^ k0, lo(M1 x2), hi(M0 x0) ^ x3 ^ k1, lo(M0 x0)), and the
// key advances by the Weyl increments. Each product is written as one
// 32 x 32 -> 64-bit multiply, which gfx950 does in one v_mad_u64_u32
// (measured 1.46x the throughput of separate low and high multiplies).
__device__ __forceinline__ void philox4x32_10(uint32_t x0, uint32_t x1, uint32_t x2, uint32_t x3,
                                              uint32_t k0, uint32_t k1, uint32_t (&out)[4]) {
  constexpr uint32_t kMul0 = 0xD2511F53u, kMul1 = 0xCD9E8D57u;
  constexpr uint32_t kWeyl0 = 0x9E3779B9u, kWeyl1 = 0xBB67AE85u;
#pragma unroll
  for (int r = 0; r < 10; ++r) {
    const uint64_t p0 = (uint64_t)kMul0 * (uint64_t)x0;
    const uint64_t p1 = (uint64_t)kMul1 * (uint64_t)x2;
    const uint32_t hi0 = (uint32_t)(p0 >> 32), lo0 = (uint32_t)p0;
    const uint32_t hi1 = (uint32_t)(p1 >> 32), lo1 = (uint32_t)p1;
    x0 = hi1 ^ x1 ^ k0;
    x1 = lo1;
    x2 = hi0 ^ x3 ^ k1;
    x3 = lo0;
    k0 += kWeyl0;
    k1 += kWeyl1;
  }
  out[0] = x0;
  out[1] = x1;
  out[2] = x2;
  out[3] = x3;
}

// Keep masks of keys 8*group .. 8*group+7 for one query: word w holds keys
// 8*group + 2w (low half) and 8*group + 2w + 1 (high half), each half 0xFFFF
// when kept and 0 when dropped, ready to AND with packed 16-bit weights.
__device__ __forceinline__ void keep_mask8(const Dropout& d, uint32_t head, uint32_t query,
                                           uint32_t group, uint32_t (&m)[4]) {
  uint32_t r[4];
  // The key words are wave-uniform. Hiding them from loop-invariant code
  // motion keeps the ten round keys from being hoisted into twenty scalar
  // registers that stay live across a whole kernel; they are recomputed on
  // the scalar unit instead.
  uint32_t k0 = d.key0, k1 = d.key1;
  asm volatile("" : "+s"(k0), "+s"(k1));
  philox4x32_10(group, query, head, d.offset, k0, k1, r);
#pragma unroll
  for (int w = 0; w < 4; ++w) {
    const uint32_t lo = (r[w] & 0xFFFFu) >= d.thr ? 0x0000FFFFu : 0u;
    const uint32_t hi = (r[w] >> 16) >= d.thr ? 0xFFFF0000u : 0u;
    m[w] = lo | hi;
  }
}

}  // namespace gpt_attn
