// Causal attention forward and backward in fp32, head dim 64, for gfx950.
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
// atomics, so every output is bitwise reproducible.
#include "attn_common.h"
#include "attn_launch.h"

namespace gpt_attn {
namespace {

constexpr int kD = kHeadDim;

__global__ __launch_bounds__(64) void attn_fwd_f32_kernel(
    const float* __restrict__ q, const float* __restrict__ k, const float* __restrict__ v,
    float* __restrict__ o, float* __restrict__ lse, int T, int n_tiles, float scale) {
  __shared__ float Ks[64 * kD];
  __shared__ float Vs[64 * kD];
  const int tid = threadIdx.x;
  const int head = blockIdx.x / n_tiles;
  const int q0 = (blockIdx.x % n_tiles) * 64;
  const int i = q0 + tid;
  const size_t hoff = (size_t)head * T * kD;

  float qr[kD], acc[kD];
#pragma unroll
  for (int d = 0; d < kD; ++d) {
    qr[d] = i < T ? q[hoff + (size_t)i * kD + d] : 0.f;
    acc[d] = 0.f;
  }
  float m = -INFINITY, l = 0.f;
  const int kv_end = min(T, q0 + 64);
  for (int k0 = 0; k0 < kv_end; k0 += 64) {
    __syncthreads();
    for (int e = tid; e < 64 * kD; e += 64) {
      const int r = e / kD;
      const bool ok = k0 + r < T;
      Ks[e] = ok ? k[hoff + (size_t)k0 * kD + e] : 0.f;
      Vs[e] = ok ? v[hoff + (size_t)k0 * kD + e] : 0.f;
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
#pragma unroll
    for (int j = 0; j < 64; ++j) {
      const float p = expf(sc[j] - m_new);
      l += p;
#pragma unroll
      for (int d = 0; d < kD; ++d) acc[d] = fmaf(p, Vs[j * kD + d], acc[d]);
    }
    m = m_new;
  }
  if (i < T) {
    const float inv = 1.f / l;
#pragma unroll
    for (int d = 0; d < kD; ++d) o[hoff + (size_t)i * kD + d] = acc[d] * inv;
    lse[(size_t)head * T + i] = m + logf(l);
  }
}

__global__ __launch_bounds__(256) void attn_bwd_prep_f32_kernel(
    const float* __restrict__ o, const float* __restrict__ dout, float* __restrict__ delta,
    long long rows) {
  const long long gid = (long long)blockIdx.x * 256 + threadIdx.x;
  const long long row = gid >> 3;
  const int part = (int)(gid & 7);
  float acc = 0.f;
  if (row < rows) {
#pragma unroll
    for (int t = 0; t < 8; ++t) {
      const long long e = row * kD + part * 8 + t;
      acc = fmaf(o[e], dout[e], acc);
    }
  }
  acc += __shfl_xor(acc, 1, 64);
  acc += __shfl_xor(acc, 2, 64);
  acc += __shfl_xor(acc, 4, 64);
  if (row < rows && part == 0) delta[row] = acc;
}

// dK, dV: thread pair (key j, half) holds 32 dims of K_j, V_j, dK_j, dV_j.
__global__ __launch_bounds__(64) void attn_bwd_dkdv_f32_kernel(
    const float* __restrict__ q, const float* __restrict__ k, const float* __restrict__ v,
    const float* __restrict__ dout, const float* __restrict__ lse,
    const float* __restrict__ delta, float* __restrict__ dk, float* __restrict__ dv, int T,
    int n_tiles, float scale) {
  __shared__ float Qs[32 * kD];
  __shared__ float dOs[32 * kD];
  __shared__ float lses[32];
  __shared__ float dels[32];
  const int tid = threadIdx.x;
  const int head = blockIdx.x / n_tiles;
  const int k0 = (blockIdx.x % n_tiles) * 32;
  const int j = k0 + (tid >> 1);
  const int half = tid & 1;
  const size_t hoff = (size_t)head * T * kD;
  const size_t roff = (size_t)head * T;

  float kr[32], vr[32], dka[32], dva[32];
#pragma unroll
  for (int d = 0; d < 32; ++d) {
    const size_t e = hoff + (size_t)j * kD + half * 32 + d;
    kr[d] = j < T ? k[e] : 0.f;
    vr[d] = j < T ? v[e] : 0.f;
    dka[d] = 0.f;
    dva[d] = 0.f;
  }
  for (int qs = k0; qs < T; qs += 32) {
    __syncthreads();
    for (int e = tid; e < 32 * kD; e += 64) {
      const int r = e / kD;
      const bool ok = qs + r < T;
      Qs[e] = ok ? q[hoff + (size_t)qs * kD + e] : 0.f;
      dOs[e] = ok ? dout[hoff + (size_t)qs * kD + e] : 0.f;
    }
    if (tid < 32) {
      const bool ok = qs + tid < T;
      lses[tid] = ok ? lse[roff + qs + tid] : 0.f;
      dels[tid] = ok ? delta[roff + qs + tid] : 0.f;
    }
    __syncthreads();
    for (int ii = 0; ii < 32; ++ii) {
      const int i = qs + ii;
      float s = 0.f, dp = 0.f;
#pragma unroll
      for (int d = 0; d < 32; ++d) {
        s = fmaf(Qs[ii * kD + half * 32 + d], kr[d], s);
        dp = fmaf(dOs[ii * kD + half * 32 + d], vr[d], dp);
      }
      s += __shfl_xor(s, 1, 64);
      dp += __shfl_xor(dp, 1, 64);
      if (i < T && j < T && j <= i) {
        const float p = expf(s * scale - lses[ii]);
        const float ds = p * (dp - dels[ii]);
#pragma unroll
        for (int d = 0; d < 32; ++d) {
          dva[d] = fmaf(p, dOs[ii * kD + half * 32 + d], dva[d]);
          dka[d] = fmaf(ds, Qs[ii * kD + half * 32 + d], dka[d]);
        }
      }
    }
  }
  if (j < T) {
#pragma unroll
    for (int d = 0; d < 32; ++d) {
      const size_t e = hoff + (size_t)j * kD + half * 32 + d;
      dk[e] = dka[d] * scale;
      dv[e] = dva[d];
    }
  }
}

// dQ: thread pair (query i, half) holds 32 dims of Q_i, dO_i, dQ_i.
__global__ __launch_bounds__(64) void attn_bwd_dq_f32_kernel(
    const float* __restrict__ q, const float* __restrict__ k, const float* __restrict__ v,
    const float* __restrict__ dout, const float* __restrict__ lse,
    const float* __restrict__ delta, float* __restrict__ dq, int T, int n_tiles, float scale) {
  __shared__ float Ks[32 * kD];
  __shared__ float Vs[32 * kD];
  const int tid = threadIdx.x;
  const int head = blockIdx.x / n_tiles;
  const int q0 = (blockIdx.x % n_tiles) * 32;
  const int i = q0 + (tid >> 1);
  const int half = tid & 1;
  const size_t hoff = (size_t)head * T * kD;
  const size_t roff = (size_t)head * T;

  float qr[32], dor[32], dqa[32];
#pragma unroll
  for (int d = 0; d < 32; ++d) {
    const size_t e = hoff + (size_t)i * kD + half * 32 + d;
    qr[d] = i < T ? q[e] : 0.f;
    dor[d] = i < T ? dout[e] : 0.f;
    dqa[d] = 0.f;
  }
  const float lse_i = i < T ? lse[roff + i] : 0.f;
  const float del_i = i < T ? delta[roff + i] : 0.f;
  const int kv_end = min(T, q0 + 32);
  for (int k0 = 0; k0 < kv_end; k0 += 32) {
    __syncthreads();
    for (int e = tid; e < 32 * kD; e += 64) {
      const int r = e / kD;
      const bool ok = k0 + r < T;
      Ks[e] = ok ? k[hoff + (size_t)k0 * kD + e] : 0.f;
      Vs[e] = ok ? v[hoff + (size_t)k0 * kD + e] : 0.f;
    }
    __syncthreads();
    for (int jj = 0; jj < 32; ++jj) {
      const int j = k0 + jj;
      float s = 0.f, dp = 0.f;
#pragma unroll
      for (int d = 0; d < 32; ++d) {
        s = fmaf(qr[d], Ks[jj * kD + half * 32 + d], s);
        dp = fmaf(dor[d], Vs[jj * kD + half * 32 + d], dp);
      }
      s += __shfl_xor(s, 1, 64);
      dp += __shfl_xor(dp, 1, 64);
      if (i < T && j < T && j <= i) {
        const float p = expf(s * scale - lse_i);
        const float ds = p * (dp - del_i);
#pragma unroll
        for (int d = 0; d < 32; ++d) dqa[d] = fmaf(ds, Ks[jj * kD + half * 32 + d], dqa[d]);
      }
    }
  }
  if (i < T) {
#pragma unroll
    for (int d = 0; d < 32; ++d) dq[hoff + (size_t)i * kD + half * 32 + d] = dqa[d] * scale;
  }
}

}  // namespace

hipError_t launch_fwd_f32(const float* q, const float* k, const float* v, float* o, float* lse,
                          int n_heads, int T, hipStream_t stream) {
  const int n_tiles = (T + 63) / 64;
  hipLaunchKernelGGL(attn_fwd_f32_kernel, dim3((unsigned)n_heads * n_tiles), dim3(64), 0, stream,
                     q, k, v, o, lse, T, n_tiles, 0.125f);
  return hipGetLastError();
}

hipError_t launch_bwd_prep_f32(const float* o, const float* dout, float* delta, int n_heads,
                               int T, hipStream_t stream) {
  const long long rows = (long long)n_heads * T;
  hipLaunchKernelGGL(attn_bwd_prep_f32_kernel, dim3((unsigned)((rows * 8 + 255) / 256)),
                     dim3(256), 0, stream, o, dout, delta, rows);
  return hipGetLastError();
}

hipError_t launch_bwd_main_f32(const float* q, const float* k, const float* v,
                               const float* dout, const float* lse, const float* delta,
                               float* dq, float* dk, float* dv, int n_heads, int T,
                               hipStream_t stream) {
  const int n_tiles = (T + 31) / 32;
  const dim3 grid((unsigned)n_heads * n_tiles);
  hipLaunchKernelGGL(attn_bwd_dkdv_f32_kernel, grid, dim3(64), 0, stream, q, k, v, dout, lse,
                     delta, dk, dv, T, n_tiles, 0.125f);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(attn_bwd_dq_f32_kernel, grid, dim3(64), 0, stream, q, k, v, dout, lse, delta,
                     dq, T, n_tiles, 0.125f);
  return hipGetLastError();
}

}  // namespace gpt_attn
