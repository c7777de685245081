// Causal attention forward and backward in fp32, head dim D in {32, 64, 128}, for
// gfx950.
//
// The fp32 path serves the small fp32 workload (the Shakespeare-char "baby
// GPT" layer: 6 heads, block size 256) where the tolerance is 1e-5 max-abs,
// so every product and sum stays in fp32 on the vector ALUs and exp/log are
// the accurate device-library functions. Same definition as the bf16 path
// (page "nanoGPT: a real GPT in two 300-line files", section 2 "How the code
// works": q @ k^T / sqrt(head size), future at -inf, softmax, @ v; the
// gradient autograd forms for it, section 1 "Summary").
//
// Layout of the work: 16 lanes per row (a query, or a key for dK/dV), each
// holding D/16 consecutive dims of that row's vectors, so a wave carries four
// rows; a dot product is the lanes' partial sums added across the 16 lanes
// with four DPP steps, which leave the same sum in every lane. Keys (or
// queries) are read straight from global memory: the four rows of a wave
// read the same key at the same time, so each load is one coalesced 256-byte
// row shared by the wave. Forward: a wave per four queries, online softmax
// (running max and sum) over batches of 8 or 4 keys. Backward: delta =
// rowsum(dO * O) first; then dK, dV with a wave per four keys looping over
// the queries at and after them, and dQ with a wave per four queries looping
// over the keys up to them. Nothing is accumulated with atomics, so every
// output is bitwise reproducible. Operands are addressed through per-tensor
// element strides (D contiguous), like the bf16 path.
// Attention dropout regenerates the same Philox keep mask as the bf16 path
// (one block per query and 8 keys) wherever a (query, key) weight is used.
#include "attn_common.h"
#include "attn_launch.h"

namespace gpt_attn {
namespace {

// Keep bit of key 8*group + t from keep_mask8's words.
__device__ __forceinline__ bool kept_bit(const uint32_t (&m)[4], int t) {
  return (m[t >> 1] >> (16 * (t & 1))) & 1u;
}

__device__ __forceinline__ const float* fptr(const void* base, const Layout& L, int hd, int H) {
  return static_cast<const float*>(base) + head_base(L, hd, H);
}
__device__ __forceinline__ float* fptr_w(void* base, const Layout& L, int hd, int H) {
  return static_cast<float*>(base) + head_base(L, hd, H);
}

// Sum over the 16 lanes of a row of x (DPP: swap neighbours, swap pairs,
// mirror within 8 lanes, mirror within 16). Every step adds two values that
// partner lanes hold in opposite order, so all 16 lanes end with the same sum.
template <int kCtrl>
__device__ __forceinline__ float dpp_get(float x) {
  return __builtin_bit_cast(
      float, __builtin_amdgcn_update_dpp(0, __builtin_bit_cast(int, x), kCtrl, 0xF, 0xF, false));
}
__device__ __forceinline__ float sum16(float x) {
  x += dpp_get<0xB1>(x);   // quad_perm [1,0,3,2]
  x += dpp_get<0x4E>(x);   // quad_perm [2,3,0,1]
  x += dpp_get<0x141>(x);  // row_half_mirror
  x += dpp_get<0x140>(x);  // row_mirror
  return x;
}

typedef float f32x2 __attribute__((ext_vector_type(2)));

// kE consecutive floats at p (8-byte aligned for kE = 2, 16-byte otherwise).
template <int kE>
__device__ __forceinline__ void load_part(const float* p, float (&x)[kE]) {
  if constexpr (kE == 2) {
    const f32x2 v = *reinterpret_cast<const f32x2*>(p);
    x[0] = v[0];
    x[1] = v[1];
  } else {
#pragma unroll
    for (int c = 0; c < kE / 4; ++c) {
      const f32x4 v = *reinterpret_cast<const f32x4*>(p + 4 * c);
#pragma unroll
      for (int t = 0; t < 4; ++t) x[4 * c + t] = v[t];
    }
  }
}

template <int kE>
__device__ __forceinline__ float dot_part(const float (&x)[kE], const float (&y)[kE]) {
  float d = 0.f;
#pragma unroll
  for (int e = 0; e < kE; ++e) d = fmaf(x[e], y[e], d);
  return d;
}

// A workgroup of kW waves per four rows: every wave holds the same four rows
// and takes every kW-th batch of the loop, and the waves' partial results
// meet in LDS at the end (in a fixed order, so the outputs stay
// reproducible). kU rows of the loop per batch; the next batch's loads are
// issued before the current batch is used. Two shapes: 4 waves of 8-row
// batches, and for sequences of kLongT and more at D <= 64, 12 waves of
// 4-row batches, which shortens each wave's chain of dependent loads
// (measured at T = 256, D = 64: 4.2 against 3.4 TFLOP/s per step; at T = 64
// the 4-wave shape is 10% faster, and at D = 128 three waves per SIMD
// would spill).
constexpr int kLongT = 192;
// A batch of kU keys (kU divides 8, batches start at multiples of kU) lies
// inside one Philox block of 8 keys: the dropout bits of key j0 + t are bits
// (j0 mod 8) + t of the block that keep_mask8 returns for j0 / 8.

// One workgroup per four queries (16 lanes each, kE = D/16 dims per lane).
// Each wave runs the online softmax over its share of the key batches; the
// partial (max, sum, output) triples are merged with the log-sum-exp rule.
template <int kD, int kW, int kU>
__global__ __launch_bounds__(64 * kW) void attn_fwd_f32_kernel(const FwdArgs a, int n_tiles,
                                                               float scale) {
  constexpr int kE = kD / 16;
  static_assert(8 % kU == 0, "a batch of keys lies in one dropout block");
  __shared__ float s_part[kW][64][kE + 2];
  const int T = a.T;
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6, g = lane & 15;
  const int head = blockIdx.x / n_tiles;
  const int q0 = (blockIdx.x % n_tiles) * 4;
  const int i = q0 + (lane >> 4);
  const int ie = min(i, T - 1);  // rows past T run as row T - 1 and store nothing
  const float* qh = fptr(a.q, a.lq, head, a.H);
  const float* kh = fptr(a.k, a.lk, head, a.H) + g * kE;
  const float* vh = fptr(a.v, a.lv, head, a.H) + g * kE;
  const int ldk = (int)a.lk.t, ldv = (int)a.lv.t;
  const bool drop = a.drop.thr != 0;

  float qr[kE], acc[kE];
  load_part<kE>(qh + ie * a.lq.t + g * kE, qr);
#pragma unroll
  for (int e = 0; e < kE; ++e) acc[e] = 0.f;
  float m = -INFINITY, l = 0.f;
  const int kend = min(q0 + 3, T - 1) + 1;  // keys 0 .. the block's last query
  float kb[2][kU][kE], vb[2][kU][kE];
  auto load_block = [&](int j0, int b) {
#pragma unroll
    for (int t = 0; t < kU; ++t) {
      const int j = min(j0 + t, T - 1);
      load_part<kE>(kh + j * ldk, kb[b][t]);
      load_part<kE>(vh + j * ldv, vb[b][t]);
    }
  };
  auto use_block = [&](int j0, int b) {
    float sc[kU];
    float mx = m;
#pragma unroll
    for (int t = 0; t < kU; ++t) {
      const float d = sum16(dot_part<kE>(qr, kb[b][t]));
      sc[t] = j0 + t <= ie ? d * scale : -INFINITY;
      mx = fmaxf(mx, sc[t]);
    }
    if (mx == -INFINITY) return;  // nothing visible yet in this wave's share
    const float alpha = expf(m - mx);
    l *= alpha;
#pragma unroll
    for (int e = 0; e < kE; ++e) acc[e] *= alpha;
    uint32_t km[4] = {0xFFFFFFFFu, 0xFFFFFFFFu, 0xFFFFFFFFu, 0xFFFFFFFFu};
    if (drop) keep_mask8(a.drop, head, ie, (uint32_t)j0 >> 3, km);
#pragma unroll
    for (int t = 0; t < kU; ++t) {
      const float p = expf(sc[t] - mx);
      l += p;
      const float pd = kept_bit(km, (j0 & 7) + t) ? p : 0.f;
#pragma unroll
      for (int e = 0; e < kE; ++e) acc[e] = fmaf(pd, vb[b][t][e], acc[e]);
    }
    m = mx;
  };
  // Wave w takes key batches w, w + kW, ...
  // (Two register buffers with fixed indices: a loop-carried buffer index
  // would put the arrays in scratch memory.)
  const int step = kW * kU;
  int j0 = w * kU;
  if (j0 < kend) load_block(j0, 0);
  for (; j0 < kend; j0 += 2 * step) {
    if (j0 + step < kend) load_block(j0 + step, 1);
    use_block(j0, 0);
    if (j0 + step >= kend) break;
    if (j0 + 2 * step < kend) load_block(j0 + 2 * step, 0);
    use_block(j0 + step, 1);
  }
  s_part[w][lane][0] = m;
  s_part[w][lane][1] = l;
#pragma unroll
  for (int e = 0; e < kE; ++e) s_part[w][lane][2 + e] = acc[e];
  __syncthreads();
  if (w != 0 || i >= T) return;
  // Wave 0 merges the partials in wave order. Wave 0's share holds key 0,
  // which every row sees, so the merged max is finite.
  float M = -INFINITY;
#pragma unroll
  for (int v = 0; v < kW; ++v) M = fmaxf(M, s_part[v][lane][0]);
  float L = 0.f, o[kE];
#pragma unroll
  for (int e = 0; e < kE; ++e) o[e] = 0.f;
#pragma unroll
  for (int v = 0; v < kW; ++v) {
    const float mv = s_part[v][lane][0];
    const float f = mv == -INFINITY ? 0.f : expf(mv - M);
    L = fmaf(s_part[v][lane][1], f, L);
#pragma unroll
    for (int e = 0; e < kE; ++e) o[e] = fmaf(s_part[v][lane][2 + e], f, o[e]);
  }
  const float inv = (drop ? a.drop.scale : 1.f) / L;
  float* orow = fptr_w(a.o, a.lo, head, a.H) + i * a.lo.t + g * kE;
#pragma unroll
  for (int e = 0; e < kE; ++e) orow[e] = o[e] * inv;
  if (g == 0) a.lse[(size_t)head * T + i] = M + logf(L);
}

// Eight threads per (head, row); row r of [B*H, T] is head r / T, position r % T.
template <int kD>
__global__ __launch_bounds__(256) void attn_bwd_prep_f32_kernel(const BwdArgs a, int rows) {
  constexpr int kTPR = kD / 8;  // threads per row, 8 elements each
  const long long gid = (long long)blockIdx.x * 256 + threadIdx.x;
  const int row = (int)(gid / kTPR);
  const int part = (int)(gid % kTPR);
  float acc = 0.f;
  if (row < rows) {
    const int hd = row / a.T, t = row - hd * a.T;
    const float* o = fptr(a.o, a.lo, hd, a.H) + t * a.lo.t + part * 8;
    const float* dout = fptr(a.dout, a.ldo, hd, a.H) + t * a.ldo.t + part * 8;
#pragma unroll
    for (int e = 0; e < 8; ++e) acc = fmaf(o[e], dout[e], acc);
  }
#pragma unroll
  for (int m = 1; m < kTPR; m <<= 1) acc += __shfl_xor(acc, m, 64);
  if (row < rows && part == 0) a.delta[row] = acc;
}

// dK, dV: one workgroup per four keys (16 lanes each, kE = D/16 dims of
// K_j, V_j, dK_j, dV_j per lane); its waves share the queries at and after
// the first key.
template <int kD, int kW, int kU>
__global__ __launch_bounds__(64 * kW) void attn_bwd_dkdv_f32_kernel(const BwdArgs a,
                                                                    int n_tiles, float scale) {
  constexpr int kE = kD / 16;
  __shared__ float s_part[kW][64][2 * kE];
  const int T = a.T;
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6, g = lane & 15;
  const int head = blockIdx.x / n_tiles;
  const int k0 = (blockIdx.x % n_tiles) * 4;
  const int j = k0 + (lane >> 4);
  const float* qh = fptr(a.q, a.lq, head, a.H) + g * kE;
  const float* doh = fptr(a.dout, a.ldo, head, a.H) + g * kE;
  const int ldq = (int)a.lq.t, lddo = (int)a.ldo.t;
  const size_t roff = (size_t)head * T;
  const bool drop = a.drop.thr != 0;
  const float zs = drop ? a.drop.scale : 1.f;

  float kr[kE], vr[kE], dka[kE], dva[kE];
  const int jr = min(j, T - 1);
  load_part<kE>(fptr(a.k, a.lk, head, a.H) + jr * a.lk.t + g * kE, kr);
  load_part<kE>(fptr(a.v, a.lv, head, a.H) + jr * a.lv.t + g * kE, vr);
#pragma unroll
  for (int e = 0; e < kE; ++e) {
    dka[e] = 0.f;
    dva[e] = 0.f;
  }
  // The block's four keys lie in one 8-key group (k0 is a multiple of 4), so
  // one keep-mask block per query serves every lane.
  float qb[2][kU][kE], db[2][kU][kE], lb[2][kU], eb[2][kU];
  auto load_batch = [&](int i0, int b) {
#pragma unroll
    for (int u = 0; u < kU; ++u) {
      const int i = min(i0 + u, T - 1);
      load_part<kE>(qh + i * ldq, qb[b][u]);
      load_part<kE>(doh + i * lddo, db[b][u]);
      lb[b][u] = a.lse[roff + i];
      eb[b][u] = a.delta[roff + i];
    }
  };
  auto use_batch = [&](int i0, int b) {
#pragma unroll
    for (int u = 0; u < kU; ++u) {
      const int i = i0 + u;
      const float s = sum16(dot_part<kE>(qb[b][u], kr));
      const float dp = sum16(dot_part<kE>(db[b][u], vr));
      float ds = 0.f, pd = 0.f;
      if (j <= i && i < T && j < T) {
        bool kept = true;
        if (drop) {
          uint32_t km[4];
          keep_mask8(a.drop, head, i, (uint32_t)j >> 3, km);
          kept = kept_bit(km, j & 7);
        }
        const float p = expf(s * scale - lb[b][u]);
        ds = p * ((kept ? dp * zs : 0.f) - eb[b][u]);
        pd = kept ? p : 0.f;
      }
#pragma unroll
      for (int e = 0; e < kE; ++e) {
        dva[e] = fmaf(pd, db[b][u][e], dva[e]);
        dka[e] = fmaf(ds, qb[b][u][e], dka[e]);
      }
    }
  };
  // Wave w takes query batches k0 + w kU, k0 + (w + kW) kU, ...
  const int step = kW * kU;
  int i0 = k0 + w * kU;
  if (i0 < T) load_batch(i0, 0);
  for (; i0 < T; i0 += 2 * step) {
    if (i0 + step < T) load_batch(i0 + step, 1);
    use_batch(i0, 0);
    if (i0 + step >= T) break;
    if (i0 + 2 * step < T) load_batch(i0 + 2 * step, 0);
    use_batch(i0 + step, 1);
  }
#pragma unroll
  for (int e = 0; e < kE; ++e) {
    s_part[w][lane][e] = dka[e];
    s_part[w][lane][kE + e] = dva[e];
  }
  __syncthreads();
  if (w != 0 || j >= T) return;
  float* dkr = fptr_w(a.dk, a.ldk, head, a.H) + j * a.ldk.t + g * kE;
  float* dvr = fptr_w(a.dv, a.ldv, head, a.H) + j * a.ldv.t + g * kE;
#pragma unroll
  for (int e = 0; e < kE; ++e) {
    float sk = 0.f, sv = 0.f;
#pragma unroll
    for (int v = 0; v < kW; ++v) {
      sk += s_part[v][lane][e];
      sv += s_part[v][lane][kE + e];
    }
    dkr[e] = sk * scale;
    dvr[e] = sv * zs;
  }
}

// dQ: one workgroup per four queries (16 lanes each, kE dims of Q_i, dO_i,
// dQ_i per lane); its waves share the keys up to the last query.
template <int kD, int kW, int kU>
__global__ __launch_bounds__(64 * kW) void attn_bwd_dq_f32_kernel(const BwdArgs a, int n_tiles,
                                                                  float scale) {
  constexpr int kE = kD / 16;
  static_assert(8 % kU == 0, "a batch of keys lies in one dropout block");
  __shared__ float s_part[kW][64][kE];
  const int T = a.T;
  const int lane = threadIdx.x & 63, w = threadIdx.x >> 6, g = lane & 15;
  const int head = blockIdx.x / n_tiles;
  const int q0 = (blockIdx.x % n_tiles) * 4;
  const int i = q0 + (lane >> 4);
  const int ie = min(i, T - 1);
  const float* kh = fptr(a.k, a.lk, head, a.H) + g * kE;
  const float* vh = fptr(a.v, a.lv, head, a.H) + g * kE;
  const int ldk = (int)a.lk.t, ldv = (int)a.lv.t;
  const size_t roff = (size_t)head * T;
  const bool drop = a.drop.thr != 0;
  const float zs = drop ? a.drop.scale : 1.f;

  float qr[kE], dor[kE], dqa[kE];
  load_part<kE>(fptr(a.q, a.lq, head, a.H) + ie * a.lq.t + g * kE, qr);
  load_part<kE>(fptr(a.dout, a.ldo, head, a.H) + ie * a.ldo.t + g * kE, dor);
#pragma unroll
  for (int e = 0; e < kE; ++e) dqa[e] = 0.f;
  const float lse_i = a.lse[roff + ie];
  const float del_i = a.delta[roff + ie];
  const int kend = min(q0 + 3, T - 1) + 1;
  // Key batches of kU keys (inside one keep-mask block).
  float kb[2][kU][kE], vb[2][kU][kE];
  auto load_batch = [&](int j0, int b) {
#pragma unroll
    for (int u = 0; u < kU; ++u) {
      const int jj = min(j0 + u, T - 1);
      load_part<kE>(kh + jj * ldk, kb[b][u]);
      load_part<kE>(vh + jj * ldv, vb[b][u]);
    }
  };
  auto use_batch = [&](int j0, int b) {
    uint32_t km[4] = {0xFFFFFFFFu, 0xFFFFFFFFu, 0xFFFFFFFFu, 0xFFFFFFFFu};
    if (drop) keep_mask8(a.drop, head, ie, (uint32_t)j0 >> 3, km);
#pragma unroll
    for (int u = 0; u < kU; ++u) {
      const int jj = j0 + u;
      const float s = sum16(dot_part<kE>(qr, kb[b][u]));
      const float dp = sum16(dot_part<kE>(dor, vb[b][u]));
      float ds = 0.f;
      if (jj <= ie) {
        const float p = expf(s * scale - lse_i);
        ds = p * ((kept_bit(km, (j0 & 7) + u) ? dp * zs : 0.f) - del_i);
      }
#pragma unroll
      for (int e = 0; e < kE; ++e) dqa[e] = fmaf(ds, kb[b][u][e], dqa[e]);
    }
  };
  // Wave w takes key batches w kU, (w + kW) kU, ...
  const int step = kW * kU;
  int j0 = w * kU;
  if (j0 < kend) load_batch(j0, 0);
  for (; j0 < kend; j0 += 2 * step) {
    if (j0 + step < kend) load_batch(j0 + step, 1);
    use_batch(j0, 0);
    if (j0 + step >= kend) break;
    if (j0 + 2 * step < kend) load_batch(j0 + 2 * step, 0);
    use_batch(j0 + step, 1);
  }
#pragma unroll
  for (int e = 0; e < kE; ++e) s_part[w][lane][e] = dqa[e];
  __syncthreads();
  if (w != 0 || i >= T) return;
  float* dqr = fptr_w(a.dq, a.ldq, head, a.H) + i * a.ldq.t + g * kE;
#pragma unroll
  for (int e = 0; e < kE; ++e) {
    float sq = 0.f;
#pragma unroll
    for (int v = 0; v < kW; ++v) sq += s_part[v][lane][e];
    dqr[e] = sq * scale;
  }
}

// Keep mask [n_heads, T, T]: one thread per (head, query, 8-key group).
__global__ __launch_bounds__(256) void dropout_mask_kernel(const Dropout d, int T, int n_groups,
                                                           long long n_items, uint8_t* mask) {
  const long long gid = (long long)blockIdx.x * 256 + threadIdx.x;
  if (gid >= n_items) return;
  const int g = (int)(gid % n_groups);
  const long long row = gid / n_groups;  // head * T + query
  const int i = (int)(row % T);
  const int head = (int)(row / T);
  uint32_t km[4];
  keep_mask8(d, (uint32_t)head, (uint32_t)i, (uint32_t)g, km);
  uint8_t* out = mask + row * T;
#pragma unroll
  for (int t = 0; t < 8; ++t) {
    const int j = 8 * g + t;
    if (j < T) out[j] = (j <= i && kept_bit(km, t)) ? 1 : 0;
  }
}

}  // namespace

hipError_t launch_dropout_mask(const Dropout& d, int n_heads, int T, uint8_t* mask,
                               hipStream_t stream) {
  const int n_groups = (T + 7) / 8;
  const long long n_items = (long long)n_heads * T * n_groups;
  hipLaunchKernelGGL(dropout_mask_kernel, dim3((unsigned)((n_items + 255) / 256)), dim3(256), 0,
                     stream, d, T, n_groups, n_items, mask);
  return hipGetLastError();
}

namespace {

template <int D, int kW, int kU>
hipError_t fwd_f32_shape(const FwdArgs& a, hipStream_t stream) {
  const int n_tiles = (a.T + 3) / 4;
  hipLaunchKernelGGL((attn_fwd_f32_kernel<D, kW, kU>), dim3((unsigned)a.n_heads * n_tiles),
                     dim3(64 * kW), 0, stream, a, n_tiles, 1.f / __builtin_sqrtf((float)D));
  return hipGetLastError();
}

template <int D>
hipError_t fwd_f32(const FwdArgs& a, hipStream_t stream) {
  if constexpr (D <= 64) {
    if (a.T >= kLongT) return fwd_f32_shape<D, 12, 4>(a, stream);
  }
  return fwd_f32_shape<D, 4, 8>(a, stream);
}

template <int D>
hipError_t prep_f32(const BwdArgs& a, hipStream_t stream) {
  const int rows = a.n_heads * a.T;
  hipLaunchKernelGGL(attn_bwd_prep_f32_kernel<D>,
                     dim3((unsigned)(((long long)rows * (D / 8) + 255) / 256)), dim3(256), 0,
                     stream, a, rows);
  return hipGetLastError();
}

template <int D, int kW, int kU>
hipError_t main_f32_shape(const BwdArgs& a, hipStream_t stream) {
  const int n_tiles = (a.T + 3) / 4;
  const dim3 grid((unsigned)a.n_heads * n_tiles);
  const float scale = 1.f / __builtin_sqrtf((float)D);
  hipLaunchKernelGGL((attn_bwd_dkdv_f32_kernel<D, kW, kU>), grid, dim3(64 * kW), 0, stream, a,
                     n_tiles, scale);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL((attn_bwd_dq_f32_kernel<D, kW, kU>), grid, dim3(64 * kW), 0, stream, a,
                     n_tiles, scale);
  return hipGetLastError();
}

template <int D>
hipError_t main_f32(const BwdArgs& a, hipStream_t stream) {
  if constexpr (D <= 64) {
    if (a.T >= kLongT) return main_f32_shape<D, 12, 4>(a, stream);
  }
  return main_f32_shape<D, 4, 8>(a, stream);
}

}  // namespace

hipError_t launch_fwd_f32(const FwdArgs& a, int D, hipStream_t stream) {
  return D == 32   ? fwd_f32<32>(a, stream)
         : D == 64 ? fwd_f32<64>(a, stream)
                   : fwd_f32<128>(a, stream);
}

hipError_t launch_bwd_prep_f32(const BwdArgs& a, int D, hipStream_t stream) {
  return D == 32   ? prep_f32<32>(a, stream)
         : D == 64 ? prep_f32<64>(a, stream)
                   : prep_f32<128>(a, stream);
}

hipError_t launch_bwd_main_f32(const BwdArgs& a, int D, hipStream_t stream) {
  return D == 32   ? main_f32<32>(a, stream)
         : D == 64 ? main_f32<64>(a, stream)
                   : main_f32<128>(a, stream);
}

}  // namespace gpt_attn
