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
// Forward: one thread per query row; K/V tiles of 64 rows are staged in LDS
// and read by broadcast; the softmax is the online (running max / sum) form
// over tiles, so no T x T matrix exists. Backward: delta = rowsum(dO * O)
// first; then dK, dV with two threads per key (32 dims each) looping over
// the query tiles at and after the key, and dQ with two threads per query
// looping over the key tiles up to the query. Nothing is accumulated with
// atomics, so every output is bitwise reproducible. Operands are addressed
// through per-tensor element strides (D contiguous), like the bf16 path.
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

template <int kD>
__global__ __launch_bounds__(64) void attn_fwd_f32_kernel(const FwdArgs a, int n_tiles,
                                                          float scale) {
  __shared__ float Ks[64 * kD];
  __shared__ float Vs[64 * kD];
  const int T = a.T;
  const int tid = threadIdx.x;
  const int head = blockIdx.x / n_tiles;
  const int q0 = (blockIdx.x % n_tiles) * 64;
  const int i = q0 + tid;
  const float* qh = fptr(a.q, a.lq, head, a.H);
  const float* kh = fptr(a.k, a.lk, head, a.H);
  const float* vh = fptr(a.v, a.lv, head, a.H);
  const long long ldq = a.lq.t, ldk = a.lk.t, ldv = a.lv.t;
  const bool drop = a.drop.thr != 0;

  float qr[kD], acc[kD];
#pragma unroll
  for (int d = 0; d < kD; ++d) {
    qr[d] = i < T ? qh[i * ldq + d] : 0.f;
    acc[d] = 0.f;
  }
  float m = -INFINITY, l = 0.f;
  const int kv_end = min(T, q0 + 64);
  for (int k0 = 0; k0 < kv_end; k0 += 64) {
    __syncthreads();
    for (int e = tid; e < 64 * kD; e += 64) {
      const int r = e / kD, d = e % kD;
      const bool ok = k0 + r < T;
      Ks[e] = ok ? kh[(k0 + r) * ldk + d] : 0.f;
      Vs[e] = ok ? vh[(k0 + r) * ldv + d] : 0.f;
    }
    __syncthreads();
    float sc[64];
    float mx = -INFINITY;
#pragma unroll
    for (int j = 0; j < 64; ++j) {
      float dot = 0.f;
#pragma unroll
      for (int d = 0; d < kD; ++d) dot = fmaf(qr[d], Ks[j * kD + d], dot);
      const int key = k0 + j;
      sc[j] = (key <= i && key < T) ? dot * scale : -INFINITY;
      mx = fmaxf(mx, sc[j]);
    }
    const float m_new = fmaxf(m, mx);
    const float alpha = expf(m - m_new);
    l *= alpha;
#pragma unroll
    for (int d = 0; d < kD; ++d) acc[d] *= alpha;
    uint32_t km[4] = {0xFFFFFFFFu, 0xFFFFFFFFu, 0xFFFFFFFFu, 0xFFFFFFFFu};
#pragma unroll
    for (int j = 0; j < 64; ++j) {
      if (drop && (j & 7) == 0) keep_mask8(a.drop, head, i, (uint32_t)(k0 + j) >> 3, km);
      const float p = expf(sc[j] - m_new);
      l += p;
      const float pd = kept_bit(km, j & 7) ? p : 0.f;
#pragma unroll
      for (int d = 0; d < kD; ++d) acc[d] = fmaf(pd, Vs[j * kD + d], acc[d]);
    }
    m = m_new;
  }
  if (i < T) {
    const float inv = (drop ? a.drop.scale : 1.f) / l;
    float* orow = fptr_w(a.o, a.lo, head, a.H) + i * a.lo.t;
#pragma unroll
    for (int d = 0; d < kD; ++d) orow[d] = acc[d] * inv;
    a.lse[(size_t)head * T + i] = m + logf(l);
  }
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

// dK, dV: thread pair (key j, half) holds D/2 dims of K_j, V_j, dK_j, dV_j.
template <int kD>
__global__ __launch_bounds__(64) void attn_bwd_dkdv_f32_kernel(const BwdArgs a, int n_tiles,
                                                               float scale) {
  constexpr int kH = kD / 2;
  __shared__ float Qs[32 * kD];
  __shared__ float dOs[32 * kD];
  __shared__ float lses[32];
  __shared__ float dels[32];
  const int T = a.T;
  const int tid = threadIdx.x;
  const int head = blockIdx.x / n_tiles;
  const int k0 = (blockIdx.x % n_tiles) * 32;
  const int j = k0 + (tid >> 1);
  const int half = tid & 1;
  const float* qh = fptr(a.q, a.lq, head, a.H);
  const float* kh = fptr(a.k, a.lk, head, a.H);
  const float* vh = fptr(a.v, a.lv, head, a.H);
  const float* doh = fptr(a.dout, a.ldo, head, a.H);
  const size_t roff = (size_t)head * T;
  const bool drop = a.drop.thr != 0;
  const float zs = drop ? a.drop.scale : 1.f;

  float kr[kH], vr[kH], dka[kH], dva[kH];
#pragma unroll
  for (int d = 0; d < kH; ++d) {
    kr[d] = j < T ? kh[j * a.lk.t + half * kH + d] : 0.f;
    vr[d] = j < T ? vh[j * a.lv.t + half * kH + d] : 0.f;
    dka[d] = 0.f;
    dva[d] = 0.f;
  }
  for (int qs = k0; qs < T; qs += 32) {
    __syncthreads();
    for (int e = tid; e < 32 * kD; e += 64) {
      const int r = e / kD, d = e % kD;
      const bool ok = qs + r < T;
      Qs[e] = ok ? qh[(qs + r) * a.lq.t + d] : 0.f;
      dOs[e] = ok ? doh[(qs + r) * a.ldo.t + d] : 0.f;
    }
    if (tid < 32) {
      const bool ok = qs + tid < T;
      lses[tid] = ok ? a.lse[roff + qs + tid] : 0.f;
      dels[tid] = ok ? a.delta[roff + qs + tid] : 0.f;
    }
    __syncthreads();
    for (int ii = 0; ii < 32; ++ii) {
      const int i = qs + ii;
      float s = 0.f, dp = 0.f;
#pragma unroll
      for (int d = 0; d < kH; ++d) {
        s = fmaf(Qs[ii * kD + half * kH + d], kr[d], s);
        dp = fmaf(dOs[ii * kD + half * kH + d], vr[d], dp);
      }
      s += __shfl_xor(s, 1, 64);
      dp += __shfl_xor(dp, 1, 64);
      if (i < T && j < T && j <= i) {
        bool kept = true;
        if (drop) {
          uint32_t km[4];
          keep_mask8(a.drop, head, i, (uint32_t)j >> 3, km);
          kept = kept_bit(km, j & 7);
        }
        const float p = expf(s * scale - lses[ii]);
        const float ds = p * ((kept ? dp * zs : 0.f) - dels[ii]);
        const float pd = kept ? p : 0.f;
#pragma unroll
        for (int d = 0; d < kH; ++d) {
          dva[d] = fmaf(pd, dOs[ii * kD + half * kH + d], dva[d]);
          dka[d] = fmaf(ds, Qs[ii * kD + half * kH + d], dka[d]);
        }
      }
    }
  }
  if (j < T) {
    float* dkr = fptr_w(a.dk, a.ldk, head, a.H) + j * a.ldk.t + half * kH;
    float* dvr = fptr_w(a.dv, a.ldv, head, a.H) + j * a.ldv.t + half * kH;
#pragma unroll
    for (int d = 0; d < kH; ++d) {
      dkr[d] = dka[d] * scale;
      dvr[d] = dva[d] * zs;
    }
  }
}

// dQ: thread pair (query i, half) holds D/2 dims of Q_i, dO_i, dQ_i.
template <int kD>
__global__ __launch_bounds__(64) void attn_bwd_dq_f32_kernel(const BwdArgs a, int n_tiles,
                                                             float scale) {
  constexpr int kH = kD / 2;
  __shared__ float Ks[32 * kD];
  __shared__ float Vs[32 * kD];
  const int T = a.T;
  const int tid = threadIdx.x;
  const int head = blockIdx.x / n_tiles;
  const int q0 = (blockIdx.x % n_tiles) * 32;
  const int i = q0 + (tid >> 1);
  const int half = tid & 1;
  const float* qh = fptr(a.q, a.lq, head, a.H);
  const float* kh = fptr(a.k, a.lk, head, a.H);
  const float* vh = fptr(a.v, a.lv, head, a.H);
  const float* doh = fptr(a.dout, a.ldo, head, a.H);
  const size_t roff = (size_t)head * T;

  float qr[kH], dor[kH], dqa[kH];
#pragma unroll
  for (int d = 0; d < kH; ++d) {
    qr[d] = i < T ? qh[i * a.lq.t + half * kH + d] : 0.f;
    dor[d] = i < T ? doh[i * a.ldo.t + half * kH + d] : 0.f;
    dqa[d] = 0.f;
  }
  const bool drop = a.drop.thr != 0;
  const float zs = drop ? a.drop.scale : 1.f;
  const float lse_i = i < T ? a.lse[roff + i] : 0.f;
  const float del_i = i < T ? a.delta[roff + i] : 0.f;
  const int kv_end = min(T, q0 + 32);
  for (int k0 = 0; k0 < kv_end; k0 += 32) {
    __syncthreads();
    for (int e = tid; e < 32 * kD; e += 64) {
      const int r = e / kD, d = e % kD;
      const bool ok = k0 + r < T;
      Ks[e] = ok ? kh[(k0 + r) * a.lk.t + d] : 0.f;
      Vs[e] = ok ? vh[(k0 + r) * a.lv.t + d] : 0.f;
    }
    __syncthreads();
    uint32_t km[4] = {0xFFFFFFFFu, 0xFFFFFFFFu, 0xFFFFFFFFu, 0xFFFFFFFFu};
    for (int jj = 0; jj < 32; ++jj) {
      const int j = k0 + jj;
      if (drop && (jj & 7) == 0) keep_mask8(a.drop, head, i, (uint32_t)j >> 3, km);
      float s = 0.f, dp = 0.f;
#pragma unroll
      for (int d = 0; d < kH; ++d) {
        s = fmaf(qr[d], Ks[jj * kD + half * kH + d], s);
        dp = fmaf(dor[d], Vs[jj * kD + half * kH + d], dp);
      }
      s += __shfl_xor(s, 1, 64);
      dp += __shfl_xor(dp, 1, 64);
      if (i < T && j < T && j <= i) {
        const float p = expf(s * scale - lse_i);
        const float ds = p * ((kept_bit(km, jj & 7) ? dp * zs : 0.f) - del_i);
#pragma unroll
        for (int d = 0; d < kH; ++d) dqa[d] = fmaf(ds, Ks[jj * kD + half * kH + d], dqa[d]);
      }
    }
  }
  if (i < T) {
    float* dqr = fptr_w(a.dq, a.ldq, head, a.H) + i * a.ldq.t + half * kH;
#pragma unroll
    for (int d = 0; d < kH; ++d) dqr[d] = dqa[d] * scale;
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

template <int D>
hipError_t fwd_f32(const FwdArgs& a, hipStream_t stream) {
  const int n_tiles = (a.T + 63) / 64;
  hipLaunchKernelGGL(attn_fwd_f32_kernel<D>, dim3((unsigned)a.n_heads * n_tiles), dim3(64), 0,
                     stream, a, n_tiles, 1.f / __builtin_sqrtf((float)D));
  return hipGetLastError();
}

template <int D>
hipError_t prep_f32(const BwdArgs& a, hipStream_t stream) {
  const int rows = a.n_heads * a.T;
  hipLaunchKernelGGL(attn_bwd_prep_f32_kernel<D>,
                     dim3((unsigned)(((long long)rows * (D / 8) + 255) / 256)), dim3(256), 0,
                     stream, a, rows);
  return hipGetLastError();
}

template <int D>
hipError_t main_f32(const BwdArgs& a, hipStream_t stream) {
  const int n_tiles = (a.T + 31) / 32;
  const dim3 grid((unsigned)a.n_heads * n_tiles);
  const float scale = 1.f / __builtin_sqrtf((float)D);
  hipLaunchKernelGGL(attn_bwd_dkdv_f32_kernel<D>, grid, dim3(64), 0, stream, a, n_tiles, scale);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(attn_bwd_dq_f32_kernel<D>, grid, dim3(64), 0, stream, a, n_tiles, scale);
  return hipGetLastError();
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
