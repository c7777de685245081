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
// staged row-major and read transposed (ds_read_b64_tr_b16). The next K/V
// tile's global loads are issued before the current tile is computed and
// land in a second LDS buffer.
//
// Outputs: O rounded to bf16, optionally the bf16 rounding of what that
// dropped (o_lo = bf16(O - o)), and LSE in fp32.
//
// Attention dropout (a separate instantiation): the row sum keeps every
// weight (the softmax comes first), the fp16 weights entering P V are ANDed
// with the regenerated keep mask (one Philox block per lane per 8 keys, in
// exactly the lane's register order), and the survivor scale is folded into
// the final 1/l.
#include "attn_common.h"
#include "attn_launch.h"

namespace gpt_attn {
namespace {

constexpr int kBM = 128;     // queries per workgroup
constexpr int kBN = 64;      // keys per staged tile
constexpr int kThreads = 256;
constexpr int kRow = 72;     // padded LDS row, bf16 elements (64 + 8)
constexpr float kMaxSlack = 8.f;  // lazy-rescale threshold, log2 units

// K/V tile loads are issued one tile ahead: fwd_load_tile only issues raw
// 16-byte loads (rows clamped to T-1 so every address is valid);
// fwd_store_tile zeroes rows past T and writes K (bf16) and V (fp16,
// converted) row-major into an LDS buffer. Thread c moves chunk c and c+256
// of each 64 x 64 tile: row c/8, dims (c%8)*8.
struct KVRegs {
  bf16x8 k[2], v[2];
};

__device__ __forceinline__ void fwd_load_tile(const bf16* kh, int ldk, const bf16* vh, int ldv,
                                              int k0, int T, int tid, KVRegs& r) {
#pragma unroll
  for (int p = 0; p < 2; ++p) {
    const int c = tid + kThreads * p;
    const int row = min(k0 + (c >> 3), T - 1), col = (c & 7) * 8;
    r.k[p] = *reinterpret_cast<const bf16x8*>(kh + row * ldk + col);
    r.v[p] = *reinterpret_cast<const bf16x8*>(vh + row * ldv + col);
  }
}

__device__ __forceinline__ void fwd_store_tile(bf16* Ks, f16* Vs, const KVRegs& r, int k0, int T,
                                               int tid) {
#pragma unroll
  for (int p = 0; p < 2; ++p) {
    const int c = tid + kThreads * p;
    const int row = c >> 3, col = (c & 7) * 8;
    const bool ok = k0 + row < T;
    *reinterpret_cast<bf16x8*>(&Ks[row * kRow + col]) = ok ? r.k[p] : zero_bf16x8();
    *reinterpret_cast<f16x8*>(&Vs[row * kRow + col]) =
        ok ? bf16x8_to_f16x8(r.v[p]) : zero_f16x8();
  }
}

// Per-wave state of the online softmax.
struct FwdState {
  f32x16 oacc[2];  // O^T accumulators: lane = query, registers = dims
  float m_run;     // reference max, scaled log2 units (lazily updated)
  float l_run;     // this lane's partial row sum
};

// One 64-key tile for one wave. MASKED = false: every key of the tile
// precedes every query of the wave and lies below T (no compares at all).
// MASKED = true: keys after the lane's query or at/after T get -inf through
// branch-free selects against one per-lane limit.
template <bool MASKED, bool DROP>
__device__ __forceinline__ void fwd_tile(const bf16* cK, const f16* cV, const bf16x8 (&qf)[4],
                                         int k0, int my_q, int T, int l32, int hf, int lane,
                                         float scale_log2, const Dropout& drop, int head,
                                         FwdState& st) {
  // Scores S^T = K Q^T for the two 32-key halves; register v = 8c + t of half
  // hf holds key k0 + 32kb + 16c + 8hf + t (perm32 order) for query my_q.
  f32x16 s[2];
#pragma unroll
  for (int kb = 0; kb < 2; ++kb) {
    const bf16* arow = &cK[(kb * 32 + perm32(l32)) * kRow + 8 * hf];
    s[kb] = mfma32x32x16(*reinterpret_cast<const bf16x8*>(arow), qf[0], f32x16{});
#pragma unroll
    for (int kk = 1; kk < 4; ++kk)
      s[kb] = mfma32x32x16(*reinterpret_cast<const bf16x8*>(arow + kk * 16), qf[kk], s[kb]);
  }
  if (MASKED) {
    // Visible iff k0 + 32kb + 16c + 8hf + t <= min(my_q, T - 1).
    const int lim = min(my_q, T - 1) - k0 - 8 * hf;
#pragma unroll
    for (int kb = 0; kb < 2; ++kb)
#pragma unroll
      for (int r = 0; r < 16; ++r)
        s[kb][r] = (32 * kb + 16 * (r >> 3) + (r & 7) > lim) ? -INFINITY : s[kb][r];
  }

  // Lazy running max: the reference m_run moves only when some row's max
  // rises by more than kMaxSlack (log2 units); otherwise the exponentials
  // below may reach 2^kMaxSlack, which the fp32 sums and fp16 P hold exactly
  // as well, and the final division by l removes the reference. Most tiles
  // skip the rescale of O and l (wave-uniform branch).
  float mx = fmaxf(s[0][0], s[0][1]);
#pragma unroll
  for (int kb = 0; kb < 2; ++kb)
#pragma unroll
    for (int r = (kb == 0 ? 2 : 0); r < 16; ++r) mx = fmaxf(mx, s[kb][r]);
  mx = fmaxf(mx, wave_xor32(mx)) * scale_log2;
  if (wave_any(mx > st.m_run + kMaxSlack)) {
    const float m_new = fmaxf(st.m_run, mx);
    const float alpha = fast_exp2(st.m_run - m_new);
    st.m_run = m_new;
    st.l_run *= alpha;
#pragma unroll
    for (int db = 0; db < 2; ++db)
#pragma unroll
      for (int r = 0; r < 16; ++r) st.oacc[db][r] *= alpha;
  }

#pragma unroll
  for (int kb = 0; kb < 2; ++kb) {
#pragma unroll
    for (int c = 0; c < 2; ++c) {
      float p[8];
#pragma unroll
      for (int t = 0; t < 8; ++t) p[t] = fast_exp2(fmaf(s[kb][8 * c + t], scale_log2, -st.m_run));
      const f16x8 pb = pack_f16x8(p[0], p[1], p[2], p[3], p[4], p[5], p[6], p[7]);
      // The row sum uses the fp16 weights the MFMA multiplies by.
      st.l_run = sum_f16x8(pb, st.l_run);
      f16x8 pw = pb;
      if (DROP) {
        // Keys k0 + 32kb + 16c + 8hf .. +7 of query my_q: one Philox block.
        uint32_t m[4];
        keep_mask8(drop, (uint32_t)head, (uint32_t)my_q, (uint32_t)((k0 + 32 * kb + 16 * c) >> 3) + hf,
                   m);
        i32x4 bits = __builtin_bit_cast(i32x4, pb);
#pragma unroll
        for (int w = 0; w < 4; ++w) bits[w] &= (int)m[w];
        pw = __builtin_bit_cast(f16x8, bits);
      }
      const int ks = 2 * kb + c;  // 16-key step inside the tile
      // O^T += V^T P^T: the A operand (lane: dim, 8 consecutive keys) is a
      // transposing read of the row-major V tile.
#pragma unroll
      for (int db = 0; db < 2; ++db)
        st.oacc[db] = mfma32x32x16_f16(lds_operand_tr(cV, kRow, ks * 16, db * 32, lane), pw,
                                       st.oacc[db]);
    }
  }
}

// Row strides inside one head are 32-bit (the host checks T * stride < 2^31);
// head offsets are 64-bit.
template <bool DROP>
__global__ __launch_bounds__(kThreads, 2) void attn_fwd_bf16_kernel(const FwdArgs a, int n_qtiles,
                                                                    float scale_log2) {
  // LDS: two K/V tile buffers (K bf16, V fp16, both [key][d]). Buffer 1 also
  // holds the 128 x 64 Q tile during the prologue: Q fragments are read from
  // LDS so no global load inside the tile loop's dependence chain targets
  // them, and buffer 1 is first written after every wave has read them.
  __shared__ __attribute__((aligned(16))) bf16 lds_raw[2 * 2 * kBN * kRow];
  auto Kbuf = [&](int b) { return lds_raw + 2 * b * kBN * kRow; };
  auto Vbuf = [&](int b) { return reinterpret_cast<f16*>(lds_raw + (2 * b + 1) * kBN * kRow); };
  bf16* Qs = Kbuf(1);  // [query][d], 128 rows: spans K and V of buffer 1
  static_assert(kBM * kRow <= 2 * kBN * kRow, "Q tile must fit in buffer 1");

  const int T = a.T;
  const TileMap tm = map_tile_xcd(blockIdx.x, a.n_heads, n_qtiles, true);
  if (!tm.valid) return;

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int hf = lane >> 5, l32 = lane & 31;

  const bf16* __restrict__ qh = static_cast<const bf16*>(a.q) + head_base(a.lq, tm.head, a.H);
  const bf16* __restrict__ kh = static_cast<const bf16*>(a.k) + head_base(a.lk, tm.head, a.H);
  const bf16* __restrict__ vh = static_cast<const bf16*>(a.v) + head_base(a.lv, tm.head, a.H);
  const int ldq = (int)a.lq.t, ldk = (int)a.lk.t, ldv = (int)a.lv.t;

  const int q0 = tm.tile * kBM;
  const int qw0 = q0 + wave * 32;
  const int my_q = qw0 + l32;  // the query column this lane owns

  KVRegs nxt;
  fwd_load_tile(kh, ldk, vh, ldv, 0, T, tid, nxt);
  {
    bf16x8 xq[4];
#pragma unroll
    for (int p = 0; p < 4; ++p) {
      const int c = tid + kThreads * p;  // 0..1023: query c/8, dims (c%8)*8
      const int row = min(q0 + (c >> 3), T - 1);
      xq[p] = *reinterpret_cast<const bf16x8*>(qh + row * ldq + (c & 7) * 8);
    }
#pragma unroll
    for (int p = 0; p < 4; ++p) {
      const int c = tid + kThreads * p;
      const int row = c >> 3, col = (c & 7) * 8;
      *reinterpret_cast<bf16x8*>(&Qs[row * kRow + col]) =
          q0 + row < T ? xq[p] : zero_bf16x8();
    }
  }

  FwdState st;
#pragma unroll
  for (int db = 0; db < 2; ++db)
#pragma unroll
    for (int r = 0; r < 16; ++r) st.oacc[db][r] = 0.f;
  st.m_run = -INFINITY;
  st.l_run = 0.f;

  const int kv_end = min(T, q0 + kBM);
  const int n_kt = (kv_end + kBN - 1) / kBN;
  // Tiles [0, n_full) need no mask for any wave of the workgroup: all their
  // keys precede query q0 (and hence every query here) and lie below T.
  const int n_full = min(q0, T) / kBN;

  fwd_store_tile(Kbuf(0), Vbuf(0), nxt, 0, T, tid);
  __syncthreads();
  // Q^T as the B operand: lane holds d = 16*kk + 8*hf .. +7 of its query.
  bf16x8 qf[4];
#pragma unroll
  for (int kk = 0; kk < 4; ++kk)
    qf[kk] = *reinterpret_cast<const bf16x8*>(&Qs[(wave * 32 + l32) * kRow + kk * 16 + 8 * hf]);
  __syncthreads();  // every wave holds its Q fragments: buffer 1 is free

  int buf = 0;
  int kt = 0;
  for (; kt < n_full; ++kt, buf ^= 1) {
    const int k0 = kt * kBN;
    const bool has_next = kt + 1 < n_kt;
    if (has_next) fwd_load_tile(kh, ldk, vh, ldv, k0 + kBN, T, tid, nxt);
    fwd_tile<false, DROP>(Kbuf(buf), Vbuf(buf), qf, k0, my_q, T, l32, hf, lane, scale_log2,
                          a.drop, tm.head, st);
    if (has_next) fwd_store_tile(Kbuf(buf ^ 1), Vbuf(buf ^ 1), nxt, k0 + kBN, T, tid);
    __syncthreads();
  }
  for (; kt < n_kt; ++kt, buf ^= 1) {
    const int k0 = kt * kBN;
    const bool has_next = kt + 1 < n_kt;
    if (has_next) fwd_load_tile(kh, ldk, vh, ldv, k0 + kBN, T, tid, nxt);
    fwd_tile<true, DROP>(Kbuf(buf), Vbuf(buf), qf, k0, my_q, T, l32, hf, lane, scale_log2,
                         a.drop, tm.head, st);
    if (has_next) fwd_store_tile(Kbuf(buf ^ 1), Vbuf(buf ^ 1), nxt, k0 + kBN, T, tid);
    __syncthreads();
  }

  // Epilogue: O = O_acc / l, LSE = (m + log2 l) * ln 2.
  const float l_tot = st.l_run + wave_xor32(st.l_run);
  const float inv = (DROP ? a.drop.scale : 1.f) / l_tot;
  if (my_q < T) {
    bf16* orow = static_cast<bf16*>(a.o) + head_base(a.lo, tm.head, a.H) + my_q * (int)a.lo.t;
    bf16* lrow = a.o_lo ? static_cast<bf16*>(a.o_lo) + head_base(a.llo, tm.head, a.H) +
                              my_q * (int)a.llo.t
                        : nullptr;
#pragma unroll
    for (int db = 0; db < 2; ++db)
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        float x[4];
        bf16x4 hi, lo;
#pragma unroll
        for (int t = 0; t < 4; ++t) {
          x[t] = st.oacc[db][4 * g + t] * inv;
          hi[t] = (bf16)x[t];
          lo[t] = (bf16)(x[t] - (float)hi[t]);
        }
        *reinterpret_cast<bf16x4*>(orow + db * 32 + 8 * g + 4 * hf) = hi;
        if (lrow) *reinterpret_cast<bf16x4*>(lrow + db * 32 + 8 * g + 4 * hf) = lo;
      }
    if (hf == 0) a.lse[(size_t)tm.head * T + my_q] = (st.m_run + fast_log2(l_tot)) * kLn2;
  }
}

}  // namespace

hipError_t launch_fwd_bf16(const FwdArgs& a, hipStream_t stream) {
  const int n_qtiles = (a.T + kBM - 1) / kBM;
  const float scale_log2 = 0.125f * kLog2e;  // 1/sqrt(64) * log2(e)
  const dim3 grid(tiled_grid(a.n_heads, n_qtiles));
  if (a.drop.thr != 0)
    hipLaunchKernelGGL(attn_fwd_bf16_kernel<true>, grid, dim3(kThreads), 0, stream, a, n_qtiles,
                       scale_log2);
  else
    hipLaunchKernelGGL(attn_fwd_bf16_kernel<false>, grid, dim3(kThreads), 0, stream, a, n_qtiles,
                       scale_log2);
  return hipGetLastError();
}

}  // namespace gpt_attn
