// One query per (sequence, head) against a key/value cache, for gfx950:
// bf16, fp16 or fp32 inputs, head dim D in {32, 64, 128}.
//
// Sampling feeds the sequence back one position at a time (generate(), page
// "nanoGPT: a real GPT in two 300-line files", section 2 "How the code
// works"); the newest query attends to every cached key up to and including
// its own position, which is the last row of the causal forward:
//   O = softmax(q K^T / sqrt(D)) V over the first n cache rows, LSE = ln sum.
// With one query there is no matrix product to feed the matrix cores: the
// work is two passes over the cache (K, V: 256 bytes per key in bf16) at four
// FLOPs per byte, so it is bound by HBM bandwidth, and the kernels are shaped
// for coalesced streaming and enough bytes in flight, not for MFMA.
//
// Split kernel: the cache rows of a head are cut into chunks; a workgroup
// of 256 threads owns one (head, chunk). D/8 lanes share a key: each loads
// 8 elements of the key's K and V rows (a whole row per D/8 lanes, so every
// load of a wave covers whole rows), forms its partial dot product with its
// 8 elements of q and completes it with lane exchanges. The 256/(D/8) key
// groups of the workgroup each run an online softmax (base 2, fp32) over
// every group-count-th key of the chunk, 4 keys per step with all loads
// issued first;
// the group states meet in LDS and the chunk's unnormalized O with its
// running max and sum goes to the workspace. Merge kernel: one wave per head
// combines the chunks with the log-sum-exp rule and writes O and LSE.
#include "attn_common.h"
#include "attn_launch.h"

namespace gpt_attn {
namespace {

constexpr int kThreads = 256;
constexpr int kUnroll = 4;             // keys per group per step

// Raw 8-element row pieces: loaded first, converted when used. The loads are
// nontemporal: every cache row is read once per call, and streaming it past
// the caches measured 11-15% faster per call (the cache not left in the
// Infinity Cache by the call before).
template <typename TIn>
struct Raw8;
template <>
struct Raw8<bf16> {
  bf16x8 x;
  __device__ __forceinline__ void load(const bf16* p) {
    x = __builtin_nontemporal_load(reinterpret_cast<const bf16x8*>(p));
  }
  __device__ __forceinline__ float operator[](int t) const { return (float)x[t]; }
};
template <>
struct Raw8<f16> {
  f16x8 x;
  __device__ __forceinline__ void load(const f16* p) {
    x = __builtin_nontemporal_load(reinterpret_cast<const f16x8*>(p));
  }
  __device__ __forceinline__ float operator[](int t) const { return (float)x[t]; }
};
template <>
struct Raw8<float> {
  f32x4 a, b;
  __device__ __forceinline__ void load(const float* p) {
    a = __builtin_nontemporal_load(reinterpret_cast<const f32x4*>(p));
    b = __builtin_nontemporal_load(reinterpret_cast<const f32x4*>(p) + 1);
  }
  __device__ __forceinline__ float operator[](int t) const { return t < 4 ? a[t] : b[t - 4]; }
};

__device__ __forceinline__ int cache_length(const DecArgs& a, int head) {
  const int n = a.lengths ? a.lengths[head / a.H] : a.L;
  return min(max(n, 0), a.L);
}

template <typename TIn, int D>
__global__ __launch_bounds__(kThreads) void attn_decode_split_kernel(const DecArgs a, int chunk,
                                                                     int n_chunks,
                                                                     float scale_log2) {
  constexpr int kLanes = D / 8;                 // lanes per key
  constexpr int kGroups = kThreads / kLanes;    // keys in flight per step per workgroup
  __shared__ float s_m[kGroups], s_l[kGroups];
  __shared__ __attribute__((aligned(16))) float s_acc[kGroups][D + 4];

  const int head = blockIdx.x / n_chunks;  // flat b*H + h
  const int c = blockIdx.x - head * n_chunks;
  const int n = cache_length(a, head);
  const int kb = c * chunk, ke = min(n, kb + chunk);
  float* part = a.part + ((size_t)head * n_chunks + c) * kDecPart;
  const int tid = threadIdx.x;
  if (kb >= ke) {  // nothing cached here: an empty partial (workgroup-uniform)
    if (tid < D) part[tid] = 0.f;
    if (tid == kDecMax) part[kDecMax] = -INFINITY;
    if (tid == kDecSum) part[kDecSum] = 0.f;
    return;
  }
  const int sub = tid % kLanes, grp = tid / kLanes;
  const TIn* qh = static_cast<const TIn*>(a.q) + head_base(a.lq, head, a.H);
  const TIn* kh = static_cast<const TIn*>(a.k) + head_base(a.lk, head, a.H) + sub * 8;
  const TIn* vh = static_cast<const TIn*>(a.v) + head_base(a.lv, head, a.H) + sub * 8;
  const int ldk = (int)a.lk.t, ldv = (int)a.lv.t;

  float qv[8];
  {
    Raw8<TIn> r;
    r.load(qh + sub * 8);
#pragma unroll
    for (int t = 0; t < 8; ++t) qv[t] = r[t] * scale_log2;
  }
  float m = -INFINITY, l = 0.f, acc[8];
#pragma unroll
  for (int t = 0; t < 8; ++t) acc[t] = 0.f;

  for (int key0 = kb + grp; key0 < ke; key0 += kGroups * kUnroll) {
    Raw8<TIn> kr[kUnroll], vr[kUnroll];
#pragma unroll
    for (int u = 0; u < kUnroll; ++u) {
      const int key = key0 + u * kGroups;
      const int row = key < ke ? key : key0;  // a valid row; its score is masked below
      kr[u].load(kh + row * ldk);
      vr[u].load(vh + row * ldv);
    }
    float s[kUnroll];
    float mx = m;
#pragma unroll
    for (int u = 0; u < kUnroll; ++u) {
      float d = 0.f;
#pragma unroll
      for (int t = 0; t < 8; ++t) d = fmaf(qv[t], kr[u][t], d);
#pragma unroll
      for (int msk = 1; msk < kLanes; msk <<= 1) d += __shfl_xor(d, msk, 64);
      s[u] = key0 + u * kGroups < ke ? d : -INFINITY;
      mx = fmaxf(mx, s[u]);
    }
    // key0 < ke, so s[0] and hence mx are finite.
    const float alpha = fast_exp2(m - mx);
    l *= alpha;
#pragma unroll
    for (int t = 0; t < 8; ++t) acc[t] *= alpha;
#pragma unroll
    for (int u = 0; u < kUnroll; ++u) {
      const float p = fast_exp2(s[u] - mx);
      l += p;
#pragma unroll
      for (int t = 0; t < 8; ++t) acc[t] = fmaf(p, vr[u][t], acc[t]);
    }
    m = mx;
  }

  if (sub == 0) {
    s_m[grp] = m;
    s_l[grp] = l;
  }
#pragma unroll
  for (int t = 0; t < 8; ++t) s_acc[grp][sub * 8 + t] = acc[t];
  __syncthreads();
  if (tid < D) {
    // Groups that saw no key hold m = -inf and contribute exp2(-inf) = 0.
    float M = s_m[0];
    for (int g = 1; g < kGroups; ++g) M = fmaxf(M, s_m[g]);
    float L = 0.f, O = 0.f;
    for (int g = 0; g < kGroups; ++g) {
      const float w = fast_exp2(s_m[g] - M);
      L = fmaf(s_l[g], w, L);
      O = fmaf(s_acc[g][tid], w, O);
    }
    part[tid] = O;
    if (tid == 0) {
      part[kDecMax] = M;
      part[kDecSum] = L;
    }
  }
}

template <typename TOut>
__device__ __forceinline__ void store_out(TOut* p, float x);
template <>
__device__ __forceinline__ void store_out<bf16>(bf16* p, float x) {
  *p = (bf16)x;
}
template <>
__device__ __forceinline__ void store_out<f16>(f16* p, float x) {
  *p = (f16)x;
}
template <>
__device__ __forceinline__ void store_out<float>(float* p, float x) {
  *p = x;
}

template <typename TOut, int D>
__global__ __launch_bounds__(D) void attn_decode_merge_kernel(const DecArgs a, int chunk,
                                                              int n_chunks) {
  const int head = blockIdx.x;
  const int d = threadIdx.x;
  const int n = cache_length(a, head);
  TOut* oh = static_cast<TOut*>(a.o) + head_base(a.lo, head, a.H);
  if (n == 0) {
    store_out<TOut>(oh + d, 0.f);
    if (d == 0) a.lse[head] = -INFINITY;
    return;
  }
  const int nc = (n + chunk - 1) / chunk;
  const float* part = a.part + (size_t)head * n_chunks * kDecPart;
  // One pass with a running max (the online rule the split kernel uses),
  // kMergeUnroll chunks at a time with every load issued before any is used,
  // so the chunks cost one memory round trip per group rather than two each.
  // Chunk 0 always holds keys (n > 0), so M is finite after the first group.
  constexpr int kMergeUnroll = 4;
  float M = -INFINITY, L = 0.f, O = 0.f;
  for (int c0 = 0; c0 < nc; c0 += kMergeUnroll) {
    float mc[kMergeUnroll], lc[kMergeUnroll], oc[kMergeUnroll];
#pragma unroll
    for (int u = 0; u < kMergeUnroll; ++u) {
      const int c = min(c0 + u, nc - 1);  // a valid chunk; repeats are dropped below
      mc[u] = part[c * kDecPart + kDecMax];
      lc[u] = part[c * kDecPart + kDecSum];
      oc[u] = part[c * kDecPart + d];
    }
    float mx = M;
#pragma unroll
    for (int u = 0; u < kMergeUnroll; ++u)
      if (c0 + u < nc) mx = fmaxf(mx, mc[u]);
    const float alpha = fast_exp2(M - mx);  // M = -inf on the first group: 0
    L *= alpha;
    O *= alpha;
#pragma unroll
    for (int u = 0; u < kMergeUnroll; ++u) {
      if (c0 + u < nc) {
        const float w = fast_exp2(mc[u] - mx);
        L = fmaf(lc[u], w, L);
        O = fmaf(oc[u], w, O);
      }
    }
    M = mx;
  }
  store_out<TOut>(oh + d, O / L);
  if (d == 0) a.lse[head] = (M + fast_log2(L)) * kLn2;
}

template <typename T, int D>
hipError_t launch_decode(const DecArgs& a, hipStream_t stream) {
  const int chunk = decode_chunk(a.n_heads, a.L);
  const int n_chunks = (a.L + chunk - 1) / chunk;
  const float scale_log2 = kLog2e / __builtin_sqrtf((float)D);  // 1/sqrt(D) * log2(e)
  if (n_chunks > 0) {  // L = 0: every length is 0 and the merge writes O = 0
    hipLaunchKernelGGL((attn_decode_split_kernel<T, D>), dim3((unsigned)(a.n_heads * n_chunks)),
                       dim3(kThreads), 0, stream, a, chunk, n_chunks, scale_log2);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  hipLaunchKernelGGL((attn_decode_merge_kernel<T, D>), dim3((unsigned)a.n_heads), dim3(D), 0,
                     stream, a, chunk, n_chunks);
  return hipGetLastError();
}

template <typename T>
hipError_t launch_decode_d(const DecArgs& a, int D, hipStream_t stream) {
  return D == 32   ? launch_decode<T, 32>(a, stream)
         : D == 64 ? launch_decode<T, 64>(a, stream)
                   : launch_decode<T, 128>(a, stream);
}

}  // namespace

hipError_t launch_decode(const DecArgs& a, int dtype_code, int D, hipStream_t stream) {
  if (dtype_code == 1) return launch_decode_d<bf16>(a, D, stream);
  if (dtype_code == 2) return launch_decode_d<f16>(a, D, stream);
  return launch_decode_d<float>(a, D, stream);
}

}  // namespace gpt_attn
