// Causal attention forward, bf16 inputs, fp32 accumulation, head dim 64, for
// gfx950 (CDNA4).
//
// Computes O = softmax(Q K^T / sqrt(64) with the future masked) V and the
// natural-log LSE of every row without storing the T x T matrix (the fused
// path nanoGPT calls through scaled_dot_product_attention(..., is_causal=True),
// page "nanoGPT: a real GPT in two 300-line files", section 2 "How the code
// works"; the causal rule is that page's section 8 "Self-check").
//
// Work split. A workgroup of 4 waves owns 128 consecutive queries of one
// head; wave w owns 32 of them. Key/value tiles of 64 keys are staged in LDS
// and shared by the 4 waves; tiles wholly in a query block's future are never
// loaded, and a wave skips the 32-key halves that lie wholly in its own
// future. Per tile each wave computes the transposed scores S^T = K Q^T with
// bf16 MFMA (so a lane owns one query column and a row max is mostly
// lane-local), folds them into a running max / sum in fp32 (online softmax,
// exp2 with the 1/sqrt(64) * log2(e) factor folded into one FMA), and
// accumulates O^T += V^T P^T with an fp16 MFMA: P is rounded to fp16 (11
// significant bits) rather than bf16, and the bf16 V converts to fp16
// exactly, which keeps O accurate enough for the backward's
// delta = rowsum(dO * O). K rows are loaded in the perm32 order so the
// accumulator registers already hold P in the MFMA B-operand order. V is
// staged transposed so its A operand is one 16-byte LDS read.
//
// Outputs: O rounded to bf16, optionally the bf16 rounding of what that
// dropped (o_lo = bf16(O - o)), and LSE in fp32.
#include "attn_common.h"
#include "attn_launch.h"

namespace gpt_attn {
namespace {

constexpr int kBM = 128;     // queries per workgroup
constexpr int kBN = 64;      // keys per staged tile
constexpr int kThreads = 256;
constexpr int kRow = 72;     // padded LDS row, bf16 elements (64 + 8)

__global__ __launch_bounds__(kThreads, 2) void attn_fwd_bf16_kernel(
    const bf16* __restrict__ q, const bf16* __restrict__ k, const bf16* __restrict__ v,
    bf16* __restrict__ o, bf16* __restrict__ o_lo, float* __restrict__ lse, int n_heads, int T,
    int n_qtiles, float scale_log2) {
  __shared__ __attribute__((aligned(16))) bf16 Ks[kBN * kRow];       // [key][d]
  __shared__ __attribute__((aligned(16))) f16 Vt[kHeadDim * kRow];   // [d][key], fp16

  const TileMap tm = map_tile_xcd(blockIdx.x, n_heads, n_qtiles, true);
  if (!tm.valid) return;

  const int tid = threadIdx.x;
  const int lane = tid & 63, wave = tid >> 6;
  const int hf = lane >> 5, l32 = lane & 31;

  const size_t hoff = (size_t)tm.head * (size_t)T * kHeadDim;
  const bf16* qh = q + hoff;
  const bf16* kh = k + hoff;
  const bf16* vh = v + hoff;

  const int q0 = tm.tile * kBM;
  const int qw0 = q0 + wave * 32;
  const int my_q = qw0 + l32;  // the query column this lane owns

  // Q^T as the B operand: lane holds d = 16*kk + 8*hf .. +7 of its query.
  bf16x8 qf[4];
#pragma unroll
  for (int kk = 0; kk < 4; ++kk)
    qf[kk] = load_bf16x8(qh + (size_t)my_q * kHeadDim + kk * 16 + 8 * hf, my_q < T);

  f32x16 oacc[2];
#pragma unroll
  for (int db = 0; db < 2; ++db)
#pragma unroll
    for (int r = 0; r < 16; ++r) oacc[db][r] = 0.f;
  float m_run = -INFINITY;  // running max, in scaled log2 units
  float l_run = 0.f;        // this lane's partial row sum

  const int kv_end = min(T, q0 + kBM);
  const int n_kt = (kv_end + kBN - 1) / kBN;

  for (int kt = 0; kt < n_kt; ++kt) {
    const int k0 = kt * kBN;
    __syncthreads();
    // Stage K rows [k0, k0+64) row-major.
#pragma unroll
    for (int p = 0; p < 2; ++p) {
      const int c = tid + kThreads * p;
      const int row = c >> 3, col = (c & 7) * 8;
      const int key = k0 + row;
      *reinterpret_cast<bf16x8*>(&Ks[row * kRow + col]) =
          load_bf16x8(kh + (size_t)key * kHeadDim + col, key < T);
    }
    // Stage V transposed: this thread takes rows j, j+1 and 8 dims.
    {
      const int j = 2 * (tid & 31), d0 = (tid >> 5) * 8;
      const bf16x8 v0 = load_bf16x8(vh + (size_t)(k0 + j) * kHeadDim + d0, k0 + j < T);
      const bf16x8 v1 = load_bf16x8(vh + (size_t)(k0 + j + 1) * kHeadDim + d0, k0 + j + 1 < T);
#pragma unroll
      for (int t = 0; t < 8; ++t) {
        f16x2 pr = {bf16_to_f16(v0[t]), bf16_to_f16(v1[t])};
        *reinterpret_cast<f16x2*>(&Vt[(d0 + t) * kRow + j]) = pr;
      }
    }
    __syncthreads();

    f32x16 s[2];
    bool act[2];
#pragma unroll
    for (int kb = 0; kb < 2; ++kb) {
      const int kbs = k0 + kb * 32;
      act[kb] = (kbs <= qw0 + 31) && (kbs < T);
#pragma unroll
      for (int r = 0; r < 16; ++r) s[kb][r] = 0.f;
      if (act[kb]) {
        const bf16* arow = &Ks[(kb * 32 + perm32(l32)) * kRow + 8 * hf];
#pragma unroll
        for (int kk = 0; kk < 4; ++kk)
          s[kb] = mfma32x32x16(*reinterpret_cast<const bf16x8*>(arow + kk * 16), qf[kk], s[kb]);
      }
    }

    // Mask and row max. Register v = 8c + t of half hf holds key
    // kbs + 16c + 8hf + t (perm32 order).
    float mx = -INFINITY;
#pragma unroll
    for (int kb = 0; kb < 2; ++kb) {
      if (!act[kb]) continue;
      const int kbs = k0 + kb * 32;
      const bool need_mask = (kbs + 31 > qw0) || (kbs + 32 > T);
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        const int key = kbs + 16 * (r >> 3) + 8 * hf + (r & 7);
        if (need_mask && (key > my_q || key >= T)) s[kb][r] = -INFINITY;
        mx = fmaxf(mx, s[kb][r]);
      }
    }
    mx = fmaxf(mx, wave_xor32(mx));
    const float m_new = fmaxf(m_run, mx * scale_log2);
    const float alpha = fast_exp2(m_run - m_new);
    m_run = m_new;
    l_run *= alpha;
#pragma unroll
    for (int db = 0; db < 2; ++db)
#pragma unroll
      for (int r = 0; r < 16; ++r) oacc[db][r] *= alpha;

#pragma unroll
    for (int kb = 0; kb < 2; ++kb) {
      if (!act[kb]) continue;
#pragma unroll
      for (int c = 0; c < 2; ++c) {
        float p[8];
#pragma unroll
        for (int t = 0; t < 8; ++t) {
          p[t] = fast_exp2(fmaf(s[kb][8 * c + t], scale_log2, -m_new));
          l_run += p[t];
        }
        const f16x8 pb = pack_f16x8(p[0], p[1], p[2], p[3], p[4], p[5], p[6], p[7]);
        const int ks = 2 * kb + c;  // 16-key step inside the tile
#pragma unroll
        for (int db = 0; db < 2; ++db) {
          const f16x8 a =
              *reinterpret_cast<const f16x8*>(&Vt[(db * 32 + l32) * kRow + ks * 16 + 8 * hf]);
          oacc[db] = mfma32x32x16_f16(a, pb, oacc[db]);
        }
      }
    }
  }

  // Epilogue: O = O_acc / l, LSE = (m + log2 l) * ln 2.
  const float l_tot = l_run + wave_xor32(l_run);
  const float inv = 1.f / l_tot;
  if (my_q < T) {
    bf16* orow = o + hoff + (size_t)my_q * kHeadDim;
    bf16* lrow = o_lo ? o_lo + hoff + (size_t)my_q * kHeadDim : nullptr;
#pragma unroll
    for (int db = 0; db < 2; ++db)
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        float x[4];
        bf16x4 hi, lo;
#pragma unroll
        for (int t = 0; t < 4; ++t) {
          x[t] = oacc[db][4 * g + t] * inv;
          hi[t] = (bf16)x[t];
          lo[t] = (bf16)(x[t] - (float)hi[t]);
        }
        *reinterpret_cast<bf16x4*>(orow + db * 32 + 8 * g + 4 * hf) = hi;
        if (lrow) *reinterpret_cast<bf16x4*>(lrow + db * 32 + 8 * g + 4 * hf) = lo;
      }
    if (hf == 0) lse[(size_t)tm.head * T + my_q] = (m_run + fast_log2(l_tot)) * kLn2;
  }
}

}  // namespace

hipError_t launch_fwd_bf16(const void* q, const void* k, const void* v, void* o, void* o_lo,
                           float* lse, int n_heads, int T, hipStream_t stream) {
  const int n_qtiles = (T + kBM - 1) / kBM;
  const float scale_log2 = 0.125f * kLog2e;  // 1/sqrt(64) * log2(e)
  hipLaunchKernelGGL(attn_fwd_bf16_kernel, dim3(tiled_grid(n_heads, n_qtiles)), dim3(kThreads),
                     0, stream, static_cast<const bf16*>(q), static_cast<const bf16*>(k),
                     static_cast<const bf16*>(v), static_cast<bf16*>(o), static_cast<bf16*>(o_lo),
                     lse, n_heads, T, n_qtiles, scale_log2);
  return hipGetLastError();
}

}  // namespace gpt_attn
