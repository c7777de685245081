// Internal launch interface between the C-ABI layer and the kernel files.
// Every function enqueues on `stream` and returns hipGetLastError().
#pragma once

#include <hip/hip_runtime.h>

#include "attn_dropout.h"

namespace gpt_attn {

// Work-item placement shared by the tiled kernels. Workgroups are handed to
// the 8 XCDs round-robin (workgroup id modulo 8). Each XCD is given a
// contiguous range of heads so the K/V (or Q/dO) tiles one head's workgroups
// re-read stay in that XCD's L2; inside the XCD, tiles with the most work are
// handed out first. The grid is 8 * ceil(heads/8) * tiles; slots beyond an
// XCD's share exit at once.
struct TileMap {
  int head;
  int tile;
  bool valid;
};

__device__ __forceinline__ TileMap map_tile_xcd(int bid, int n_heads, int n_tiles,
                                                bool descending) {
  const int xcd = bid & 7;
  const int slot = bid >> 3;
  const int base = n_heads >> 3, extra = n_heads & 7;
  const int nh = base + (xcd < extra ? 1 : 0);
  const int h0 = xcd * base + (xcd < extra ? xcd : extra);
  TileMap m;
  m.valid = slot < nh * n_tiles;
  if (!m.valid) {
    m.head = 0;
    m.tile = 0;
    return m;
  }
  const int t = slot / nh;
  m.head = h0 + (slot - t * nh);
  m.tile = descending ? n_tiles - 1 - t : t;
  return m;
}

inline unsigned tiled_grid(int n_heads, int n_tiles) {
  return 8u * (unsigned)((n_heads + 7) / 8) * (unsigned)n_tiles;
}

// Element strides of one [B, H, T, D] operand whose last (D) dimension is
// contiguous: element (b, h, t, d) lives at b*b_ + h*h_ + t*t_ + d.
struct Layout {
  long long b, h, t;
};

// Offset in elements of head hd = b*H + h.
__host__ __device__ __forceinline__ long long head_base(const Layout& L, int hd, int H) {
  return (long long)(hd / H) * L.b + (long long)(hd % H) * L.h;
}

// Kernel arguments, passed by value. q, k, v, o, o_lo, dout are the input
// dtype; lse, delta, dq, dk, dv fp32. lse and delta are contiguous [B, H, T].
struct FwdArgs {
  const void* q;
  const void* k;
  const void* v;
  void* o;
  void* o_lo;  // may be null (16-bit inputs only)
  float* lse;
  Layout lq, lk, lv, lo, llo;
  int n_heads, H, T;
  Dropout drop;  // drop.thr == 0: no dropout
};

struct BwdArgs {
  const void* q;
  const void* k;
  const void* v;
  const void* o;
  const void* o_lo;  // may be null (16-bit inputs only)
  const void* dout;
  const float* lse;
  float* delta;
  float* stats;  // per (head, kStatRows-row chunk): see bwd_workspace_bytes
  float* dq;
  float* dk;
  float* dv;
  Layout lq, lk, lv, lo, llo, ldo, ldq, ldk, ldv;
  int n_heads, H, T;
  Dropout drop;  // drop.thr == 0: no dropout
};

// Backward workspace: delta [n_heads * T] fp32, then, from the next 16-byte
// boundary, eight floats per (head, chunk of kStatRows rows): the largest
// |Q|, |dO| and |delta| of the chunk's rows and a zero (written by the
// preprocess), then the largest |K| and |V| of the chunk's rows and two
// zeros (written by the D = 128 dK/dV kernel, whose workgroup covers one
// chunk of keys, for the dQ kernel after it). The 16-bit backward kernels
// set their block exponents from them.
constexpr int kStatRows = 128;
constexpr int kStatFloats = 8;

// The 16-bit backward at D = 32 and 64 accumulates dQ with atomic adds into
// the dQ the preprocess zero-filled (one main kernel, 256 keys per
// workgroup); at D = 128 it runs the split dK/dV and dQ kernels, which write
// dQ once, and the preprocess leaves dQ alone.
__host__ __device__ inline bool bwd_dq_atomic(int D) { return D <= 64; }

inline long long bwd_stat_chunks(int T) { return ((long long)T + kStatRows - 1) / kStatRows; }

inline long long bwd_stats_offset_bytes(long long rows) { return (rows * 4 + 15) / 16 * 16; }

inline long long bwd_workspace_bytes(long long n_heads, int T) {
  return bwd_stats_offset_bytes(n_heads * T) + 4 * kStatFloats * n_heads * bwd_stat_chunks(T);
}

// One query per head against a key/value cache. q and o are [B, H, D]
// (lq.t, lo.t unused), k and v [B, H, L, D]; lengths [B] (device, int32) or
// null for L everywhere, clamped to [0, L]. part is the workspace:
// [n_heads, ceil(L / decode_chunk), kDecPart] fp32 partial (O, max, sum).
struct DecArgs {
  const void* q;
  const void* k;
  const void* v;
  const int* lengths;
  void* o;
  float* lse;
  float* part;
  Layout lq, lk, lv, lo;
  int n_heads, H, L;
};

// One chunk's partial: D (<= 128) unnormalized outputs, then max and sum.
constexpr int kDecPart = 132;
constexpr int kDecMax = 128, kDecSum = 129;

// Cache rows per split workgroup: about 2048 workgroups in total, a multiple
// of 128 keys (one step of the split kernel), between 128 and 1024.
__host__ __device__ inline int decode_chunk(int n_heads, int L) {
  const long long per = ((long long)n_heads * L + 2047) / 2048;
  const long long c = (per + 127) / 128 * 128;
  return (int)(c < 128 ? 128 : (c > 1024 ? 1024 : c));
}

// dtype_code: 0 fp32, 1 bf16, 2 fp16 (the C ABI's codes); D is 32, 64 or 128.
hipError_t launch_decode(const DecArgs& a, int dtype_code, int D, hipStream_t stream);

// Keep mask [n_heads, T, T] (uint8, 1 = kept; 0 above the diagonal).
hipError_t launch_dropout_mask(const Dropout& d, int n_heads, int T, uint8_t* mask,
                               hipStream_t stream);

// 16-bit inputs (bf16, or fp16 when fp16 is set) on the matrix cores, and
// fp32 inputs on the vector ALUs; D is 32, 64 or 128.
hipError_t launch_fwd_16(const FwdArgs& a, bool fp16, int D, hipStream_t stream);
hipError_t launch_bwd_prep_16(const BwdArgs& a, bool fp16, int D, hipStream_t stream);
hipError_t launch_bwd_main_16(const BwdArgs& a, bool fp16, int D, hipStream_t stream);
hipError_t launch_fwd_f32(const FwdArgs& a, int D, hipStream_t stream);
hipError_t launch_bwd_prep_f32(const BwdArgs& a, int D, hipStream_t stream);
hipError_t launch_bwd_main_f32(const BwdArgs& a, int D, hipStream_t stream);

}  // namespace gpt_attn
