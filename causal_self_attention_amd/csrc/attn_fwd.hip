// Causal attention forward, bf16 or fp16 inputs, fp32 accumulation, head dim
// D in {32, 64, 128}, for gfx950 (CDNA4).
//
// Computes O = softmax(Q K^T / sqrt(D) with the future masked) V and the
// natural-log LSE of every row without storing the T x T matrix (the fused
// path nanoGPT calls through scaled_dot_product_attention(..., is_causal=True),
// page "nanoGPT: a real GPT in two 300-line files", section 2 "How the code
// works"; the causal rule is that page's section 8 "Self-check").
//
// Work split. A workgroup of 4 waves owns 128 consecutive queries of one
// head; wave w owns 32 of them. Key/value tiles of 64 keys are staged in LDS
// and shared by the 4 waves; tiles wholly in a query block's future are never
// loaded. Per tile each wave computes the transposed scores S^T = K Q^T with
// an MFMA of the input type (so a lane owns one query column and a row max is
// mostly lane-local), folds them into a running max / sum in fp32 (online
// softmax, exp2 with the 1/sqrt(D) * log2(e) factor folded into one FMA), and
// accumulates O^T += V^T P^T with an fp16 MFMA: P is rounded to fp16 (11
// significant bits) rather than bf16, and a bf16 V converts to fp16
// exactly, which keeps O accurate enough for the backward's
// delta = rowsum(dO * O). K rows are loaded in the perm32 order so the
// accumulator registers already hold P in the MFMA B-operand order. V is
// staged row-major and read transposed (ds_read_b64_tr_b16). The next K/V
// tile's global loads are issued before the current tile is computed and
// land in a second LDS buffer.
//
// Outputs: O rounded to the input type, optionally the rounding of what that
// dropped (o_lo = round(O - o)), and LSE in fp32.
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
constexpr float kPMax = 32768.f;  // largest group sum of P taken without a rescale

// Padded LDS row of a D-wide 16-bit tile (D + 8 elements).
template <int D>
constexpr int row_of() {
  return D + 8;
}

// bf16 V can leave fp16's range; fp16 V cannot.
template <typename TIn>
constexpr bool kScaleV = !__is_same(TIn, f16);

// K/V tile loads are issued one tile ahead: fwd_load_tile only issues raw
// 16-byte loads (rows clamped to T-1 so every address is valid);
// fwd_store_tile zeroes rows past T and writes K (input type) and V (fp16,
// converted) row-major into an LDS buffer. Thread c moves chunks
// c, c+256, ... of each 64 x D tile: row c/(D/8), dims (c%(D/8))*8.
template <typename TIn, int D>
struct KVRegs {
  static constexpr int kN = kBN * D / 8 / kThreads;  // 16-byte chunks per thread
  typename In16<TIn>::vec k[kN], v[kN];
};

// A thread's chunk offsets in bytes from its tile's first K and V rows:
// fixed for the whole loop, so a tile that lies below T is loaded from a
// workgroup-uniform row pointer plus these (no per-tile address arithmetic
// on the vector unit). Below 2^32: the host checks T * stride < 2^31.
template <int D>
struct KVOffsets {
  static constexpr int kN = kBN * D / 8 / kThreads;
  static constexpr int kRowsPerPass = kThreads / (D / 8);  // rows between chunks p and p + 1
  uint32_t k, v;  // chunk 0; chunk p lies p * kRowsPerPass rows further
};

template <typename TIn, int D>
__device__ __forceinline__ KVOffsets<D> fwd_tile_offsets(int ldk, int ldv, int tid) {
  constexpr int kC = D / 8;
  const uint32_t row = (uint32_t)(tid / kC), col = (uint32_t)(tid % kC) * 8u;
  return {(row * (uint32_t)ldk + col) * (uint32_t)sizeof(TIn),
          (row * (uint32_t)ldv + col) * (uint32_t)sizeof(TIn)};
}

template <typename TIn, int D>
__device__ __forceinline__ void fwd_load_tile(const TIn* kh, int ldk, const TIn* vh, int ldv,
                                              int k0, int T, int tid, const KVOffsets<D>& off,
                                              KVRegs<TIn, D>& r) {
  typedef typename In16<TIn>::vec vec;
  constexpr int kC = D / 8;  // chunks per row
  const char* kb = reinterpret_cast<const char*>(kh + (size_t)k0 * (uint32_t)ldk);
  const char* vb = reinterpret_cast<const char*>(vh + (size_t)k0 * (uint32_t)ldv);
  uint32_t ok[KVOffsets<D>::kN], ov[KVOffsets<D>::kN];
#pragma unroll
  for (int p = 0; p < KVOffsets<D>::kN; ++p) {
    constexpr uint32_t kStep = KVOffsets<D>::kRowsPerPass * (uint32_t)sizeof(TIn);
    ok[p] = off.k + (uint32_t)p * kStep * (uint32_t)ldk;
    ov[p] = off.v + (uint32_t)p * kStep * (uint32_t)ldv;
  }
  if (k0 + kBN > T) {
    // The sequence's last tile: rows past T - 1 read row T - 1 instead.
#pragma unroll
    for (int p = 0; p < KVOffsets<D>::kN; ++p) {
      const int c = tid + kThreads * p;
      const uint32_t row = (uint32_t)min(c / kC, T - 1 - k0), col = (uint32_t)(c % kC) * 8u;
      ok[p] = (row * (uint32_t)ldk + col) * (uint32_t)sizeof(TIn);
      ov[p] = (row * (uint32_t)ldv + col) * (uint32_t)sizeof(TIn);
    }
  }
#pragma unroll
  for (int p = 0; p < KVRegs<TIn, D>::kN; ++p) {
    r.k[p] = *reinterpret_cast<const vec*>(kb + ok[p]);
    r.v[p] = *reinterpret_cast<const vec*>(vb + ov[p]);
  }
}

// For bf16, V is scaled by 2^vexp on its way to fp16 (see attn_fwd_kernel).
// MASK: zero the rows at or past T (only a sequence's last tile has any).
template <typename TIn, int D, bool MASK>
__device__ __forceinline__ void fwd_store_tile(TIn* Ks, f16* Vs, const KVRegs<TIn, D>& r, int k0,
                                               int T, int tid, int vexp) {
  typedef typename In16<TIn>::vec vec;
  constexpr int kC = D / 8, kRow = row_of<D>();
#pragma unroll
  for (int p = 0; p < KVRegs<TIn, D>::kN; ++p) {
    const int c = tid + kThreads * p;
    const int row = c / kC, col = (c % kC) * 8;
    const bool ok = !MASK || k0 + row < T;
    *reinterpret_cast<vec*>(&Ks[row * kRow + col]) = ok ? r.k[p] : In16<TIn>::zero();
    const f16x8 vs = (!kScaleV<TIn> || vexp == 0) ? In16<TIn>::to_f16(r.v[p])
                                                  : cvt_f16_scaled(r.v[p], vexp);
    *reinterpret_cast<f16x8*>(&Vs[row * kRow + col]) = ok ? vs : zero_f16x8();
  }
}

// Stage tile k0 into (Ks, Vs), with the row mask only where it can matter.
template <typename TIn, int D>
__device__ __forceinline__ void fwd_stage(TIn* Ks, f16* Vs, const KVRegs<TIn, D>& r, int k0, int T,
                                          int tid, int vexp) {
  if (k0 + kBN <= T)
    fwd_store_tile<TIn, D, false>(Ks, Vs, r, k0, T, tid, vexp);
  else
    fwd_store_tile<TIn, D, true>(Ks, Vs, r, k0, T, tid, vexp);
}

// Largest |V| among the thread's chunks of a loaded bf16 tile, as the bit
// pattern of a bf16 magnitude (sign cleared). Such patterns order like the
// magnitudes they encode, so two 16-bit lanes at a time go through one
// packed integer max.
template <typename TIn, int D>
__device__ __forceinline__ uint32_t tile_vmax_bits(const KVRegs<TIn, D>& r) {
  typedef unsigned short u16x2 __attribute__((ext_vector_type(2)));
  u16x2 m = {0, 0};
#pragma unroll
  for (int p = 0; p < KVRegs<TIn, D>::kN; ++p) {
    const i32x4 w = __builtin_bit_cast(i32x4, r.v[p]);
#pragma unroll
    for (int i = 0; i < 4; ++i)
      m = __builtin_elementwise_max(m, __builtin_bit_cast(u16x2, (uint32_t)w[i] & 0x7fff7fffu));
  }
  return m.x > m.y ? m.x : m.y;
}

// Per-wave state of the online softmax.
template <int D>
struct FwdState {
  f32x16 oacc[D / 32];  // O^T accumulators: lane = query, registers = dims
  float m_run;          // reference max, scaled log2 units (lazily updated)
  float l_run;          // this lane's partial row sum
};

// The weights of one group of 8 scores (registers base .. base + 7 of s)
// against the running reference, P = exp2(S * scale_log2 - m_run), packed to
// fp16, and their sum, which is added to l. The reference lags the row
// maximum: any P up to fp16's range is as good as P <= 1 (O and l carry the
// same reference, which the final division removes), so the reference moves
// only when a group's sum is not at most kPMax, i.e. some P of it could
// leave fp16's range (or the reference is still -infinity). Then the wave
// takes the exact maximum of the scores mx() covers (lanes l and l + 32
// hold two halves of one query's keys and exchange theirs), rescales O and
// l by 2^(m_run - m_new) and recomputes the group. Groups already taken
// this tile were consistent with the old reference and are rescaled with
// the rest. The group sum uses the fp16 values the P V product multiplies.
template <int D, typename MaxFn>
__device__ __forceinline__ f16x8 fwd_group(const f32x16& s, int base, float scale_log2,
                                           MaxFn mx, FwdState<D>& st) {
  float p[8];
#pragma unroll
  for (int t = 0; t < 8; ++t) p[t] = fast_exp2(fmaf(s[base + t], scale_log2, -st.m_run));
  f16x8 pb = pack_f16x8(p[0], p[1], p[2], p[3], p[4], p[5], p[6], p[7]);
  float gs = sum_f16x8(pb, 0.f);
  if (wave_any(!(gs <= kPMax))) {
    float m = mx();
    m = fmaxf(m, wave_xor32(m));
    const float m_new = fmaxf(st.m_run, m);
    const float alpha = fast_exp2(st.m_run - m_new);
    st.m_run = m_new;
    st.l_run *= alpha;
#pragma unroll
    for (int db = 0; db < D / 32; ++db)
#pragma unroll
      for (int r = 0; r < 16; ++r) st.oacc[db][r] *= alpha;
#pragma unroll
    for (int t = 0; t < 8; ++t) p[t] = fast_exp2(fmaf(s[base + t], scale_log2, -st.m_run));
    pb = pack_f16x8(p[0], p[1], p[2], p[3], p[4], p[5], p[6], p[7]);
    gs = sum_f16x8(pb, 0.f);
  }
  st.l_run += gs;
  return pb;
}

// One 64-key tile for one wave, off the diagonal: every key of the tile
// precedes every query of the wave and lies below T (no compares at all).
template <typename TIn, int D, bool DROP>
__device__ __forceinline__ void fwd_tile(const TIn* cK, const f16* cV,
                                         const typename In16<TIn>::vec (&qf)[D / 16], int k0,
                                         int my_q, int T, int l32, int hf, int lane,
                                         float scale_log2, const Dropout& drop, int head,
                                         FwdState<D>& st) {
  typedef typename In16<TIn>::vec vec;
  constexpr int kRow = row_of<D>();
  // Scores S^T = K Q^T for the two 32-key halves; register v = 8c + t of half
  // hf holds key k0 + 32kb + 16c + 8hf + t (perm32 order) for query my_q.
  f32x16 s[2];
#pragma unroll
  for (int kb = 0; kb < 2; ++kb) {
    const TIn* arow = &cK[(kb * 32 + perm32(l32)) * kRow + 8 * hf];
    s[kb] = In16<TIn>::mfma(*reinterpret_cast<const vec*>(arow), qf[0], f32x16{});
#pragma unroll
    for (int kk = 1; kk < D / 16; ++kk)
      s[kb] = In16<TIn>::mfma(*reinterpret_cast<const vec*>(arow + kk * 16), qf[kk], s[kb]);
  }

  // The lane's maximum over the tile, scaled log2 units (rescales only:
  // opaque_f32 keeps the compiler from computing it on every tile).
  auto tile_max = [&]() {
    float mx = opaque_f32(-INFINITY);
#pragma unroll
    for (int kb = 0; kb < 2; ++kb)
#pragma unroll
      for (int r = 0; r < 16; ++r) mx = fmaxf(mx, s[kb][r]);
    return mx * scale_log2;
  };
#pragma unroll
  for (int kb = 0; kb < 2; ++kb) {
#pragma unroll
    for (int c = 0; c < 2; ++c) {
      const f16x8 pb = fwd_group<D>(s[kb], 8 * c, scale_log2, tile_max, st);
      f16x8 pw = pb;
      if (DROP) {
        // Keys k0 + 32kb + 16c + 8hf .. +7 of query my_q: one Philox block.
        uint32_t m[4];
        keep_mask8(drop, (uint32_t)head, (uint32_t)my_q,
                   (uint32_t)((k0 + 32 * kb + 16 * c) >> 3) + hf, m);
        i32x4 bits = __builtin_bit_cast(i32x4, pb);
#pragma unroll
        for (int w = 0; w < 4; ++w) bits[w] &= (int)m[w];
        pw = __builtin_bit_cast(f16x8, bits);
      }
      const int ks = 2 * kb + c;  // 16-key step inside the tile
      // O^T += V^T P^T: the A operand (lane: dim, 8 consecutive keys) is a
      // transposing read of the row-major V tile.
#pragma unroll
      for (int db = 0; db < D / 32; ++db)
        st.oacc[db] = mfma32x32x16_f16(lds_operand_tr(cV, kRow, ks * 16, db * 32, lane), pw,
                                       st.oacc[db]);
    }
  }
}

// One 32-key half (keys k0 + 32kb ..) for one wave on the diagonal tiles,
// with its own running-max update. KIND is the half's block kind against the
// wave's 32 queries (wave-uniform; kEmpty halves are never called): kFull
// has no mask, kDiag the fixed triangle key offset <= query offset, kGeneral
// the per-lane limit min(query, T - 1).
template <typename TIn, int D, int KIND, bool DROP>
__device__ __forceinline__ void fwd_half(const TIn* cK, const f16* cV,
                                         const typename In16<TIn>::vec (&qf)[D / 16], int kb,
                                         int k0, int my_q, int T, int l32, int hf, int lane,
                                         float scale_log2, const Dropout& drop, int head,
                                         FwdState<D>& st) {
  typedef typename In16<TIn>::vec vec;
  constexpr int kRow = row_of<D>();
  // Register v = 8c + t of half hf holds key k0 + 32kb + 16c + 8hf + t.
  const TIn* arow = &cK[(kb * 32 + perm32(l32)) * kRow + 8 * hf];
  f32x16 s = In16<TIn>::mfma(*reinterpret_cast<const vec*>(arow), qf[0], f32x16{});
#pragma unroll
  for (int kk = 1; kk < D / 16; ++kk)
    s = In16<TIn>::mfma(*reinterpret_cast<const vec*>(arow + kk * 16), qf[kk], s);
  if (KIND == kDiag) {
    // Key offset 16c + 8hf + t against query offset l32.
#pragma unroll
    for (int r = 0; r < 16; ++r) s[r] = (16 * (r >> 3) + (r & 7) > l32 - 8 * hf) ? -INFINITY : s[r];
  } else if (KIND == kGeneral) {
    const int lim = min(my_q, T - 1) - (k0 + 32 * kb) - 8 * hf;
#pragma unroll
    for (int r = 0; r < 16; ++r) s[r] = (16 * (r >> 3) + (r & 7) > lim) ? -INFINITY : s[r];
  }
  // The lane's maximum over the half, scaled log2 units (rescales only).
  auto half_max = [&]() {
    float mx = opaque_f32(-INFINITY);
#pragma unroll
    for (int r = 0; r < 16; ++r) mx = fmaxf(mx, s[r]);
    return mx * scale_log2;
  };
#pragma unroll
  for (int c = 0; c < 2; ++c) {
    const f16x8 pb = fwd_group<D>(s, 8 * c, scale_log2, half_max, st);
    f16x8 pw = pb;
    if (DROP) {
      uint32_t m[4];
      keep_mask8(drop, (uint32_t)head, (uint32_t)my_q,
                 (uint32_t)((k0 + 32 * kb + 16 * c) >> 3) + hf, m);
      i32x4 bits = __builtin_bit_cast(i32x4, pb);
#pragma unroll
      for (int w = 0; w < 4; ++w) bits[w] &= (int)m[w];
      pw = __builtin_bit_cast(f16x8, bits);
    }
    const int ks = 2 * kb + c;
#pragma unroll
    for (int db = 0; db < D / 32; ++db)
      st.oacc[db] = mfma32x32x16_f16(lds_operand_tr(cV, kRow, ks * 16, db * 32, lane), pw,
                                     st.oacc[db]);
  }
}

// V's block exponent for bf16 inputs. P V runs on fp16 operands; V is
// staged as V * 2^vexp. The first K/V tile fixes vexp: 0 when its largest
// |V| lies in [2^-4, 2^8) (every bf16 value of such a tile converts exactly,
// bar fp16 subnormals, whose absolute error stays below 2^-21 of that
// largest |V|), otherwise the exponent that puts it in [2^8, 2^9). A later
// tile holding a |V| at or above vthr = 2^(15 - vexp) (or any nonzero V
// when every V so far was zero) would leave fp16's range: the staging
// threads flag it per wave, and after the barrier the workgroup lowers vexp
// to fit the tile, rescales O's accumulators to match, and stages the
// tile's V again. O is unscaled by 2^-vexp at the end.
struct VScale {
  int vexp;
  uint32_t thr;  // bf16 magnitude pattern of the smallest |V| that needs a smaller vexp
  bool set;      // some V so far was nonzero
};

// The bf16 pattern of 2^(15 - vexp): the top half of the float (an exact
// power of two, a subnormal, or infinity when no bf16 value can reach it).
__device__ __forceinline__ uint32_t vscale_thr(int vexp) {
  return __float_as_uint(ldexpf(1.f, 15 - vexp)) >> 16;
}

__device__ __forceinline__ VScale vscale_first(float m0) {
  VScale v;
  v.set = m0 > 0.f;
  v.vexp = (m0 >= 0.0625f && m0 < 256.f) ? 0 : block_exp(m0, 8);
  v.thr = !v.set ? 1u : (m0 <= 3.402823466e38f ? vscale_thr(v.vexp) : 0x7f80u);
  return v;
}

// After the barrier that follows the staging of a tile into (Kb, Vb), when
// some wave flagged the tile: move V's exponent down so that the tile fits,
// rescale the O accumulators, and stage the tile again.
template <typename TIn, int D>
__device__ __forceinline__ void fwd_rescale_v(float* s_red, const KVRegs<TIn, D>& r, TIn* Kb,
                                           f16* Vb, int k0, int T, int tid, int lane, int wave,
                                           VScale& vs, FwdState<D>& st) {
  const float m = wave_max(bf16_bits_to_float(tile_vmax_bits<TIn, D>(r)));
  if (lane == 0) s_red[wave] = m;
  __syncthreads();
  const float mt = fmaxf(fmaxf(s_red[0], s_red[1]), fmaxf(s_red[2], s_red[3]));
  const int e_fit = block_exp(mt, 8);
  const int e = vs.set ? min(vs.vexp, e_fit) : e_fit;
#pragma unroll
  for (int db = 0; db < D / 32; ++db)
#pragma unroll
    for (int i = 0; i < 16; ++i) st.oacc[db][i] = ldexpf(st.oacc[db][i], e - vs.vexp);
  vs.vexp = __builtin_amdgcn_readfirstlane(e);
  vs.set = true;
  vs.thr = mt <= 3.402823466e38f ? vscale_thr(e) : 0x7f80u;
  fwd_stage<TIn, D>(Kb, Vb, r, k0, T, tid, vs.vexp);
  __syncthreads();
}

// Row strides inside one head are 32-bit (the host checks T * stride < 2^31);
// head offsets are 64-bit.
template <typename TIn, int D, bool DROP>
__global__ __launch_bounds__(kThreads, 2) void attn_fwd_kernel(const FwdArgs a, int n_qtiles,
                                                               float scale_log2) {
  typedef typename In16<TIn>::vec vec;
  constexpr int kRow = row_of<D>();
  // LDS: two K/V tile buffers (K input type, V fp16, both [key][d]). Buffer 1
  // also holds the 128 x D Q tile during the prologue: Q fragments are read
  // from LDS so no global load inside the tile loop's dependence chain
  // targets them, and buffer 1 is first written after every wave has read
  // them.
  __shared__ __attribute__((aligned(16))) TIn lds_raw[2 * 2 * kBN * kRow];
  auto Kbuf = [&](int b) { return lds_raw + 2 * b * kBN * kRow; };
  auto Vbuf = [&](int b) { return reinterpret_cast<f16*>(lds_raw + (2 * b + 1) * kBN * kRow); };
  TIn* Qs = Kbuf(1);  // [query][d], 128 rows: spans K and V of buffer 1
  static_assert(kBM * kRow <= 2 * kBN * kRow, "Q tile must fit in buffer 1");

  const int T = a.T;
  const TileMap tm = map_tile_xcd(blockIdx.x, a.n_heads, n_qtiles, true);
  if (!tm.valid) return;

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int hf = lane >> 5, l32 = lane & 31;

  const TIn* __restrict__ qh = static_cast<const TIn*>(a.q) + head_base(a.lq, tm.head, a.H);
  const TIn* __restrict__ kh = static_cast<const TIn*>(a.k) + head_base(a.lk, tm.head, a.H);
  const TIn* __restrict__ vh = static_cast<const TIn*>(a.v) + head_base(a.lv, tm.head, a.H);
  const int ldq = (int)a.lq.t, ldk = (int)a.lk.t, ldv = (int)a.lv.t;

  const int q0 = tm.tile * kBM;
  const int qw0 = q0 + wave * 32;
  const int my_q = qw0 + l32;  // the query column this lane owns

  const KVOffsets<D> kvoff = fwd_tile_offsets<TIn, D>(ldk, ldv, tid);
  KVRegs<TIn, D> nxt;
  fwd_load_tile<TIn, D>(kh, ldk, vh, ldv, 0, T, tid, kvoff, nxt);
  {
    constexpr int kC = D / 8, kNQ = kBM * D / 8 / kThreads;
    vec xq[kNQ];
#pragma unroll
    for (int p = 0; p < kNQ; ++p) {
      const int c = tid + kThreads * p;  // query c/kC, dims (c%kC)*8
      const int row = min(q0 + c / kC, T - 1);
      xq[p] = *reinterpret_cast<const vec*>(qh + row * ldq + (c % kC) * 8);
    }
#pragma unroll
    for (int p = 0; p < kNQ; ++p) {
      const int c = tid + kThreads * p;
      const int row = c / kC, col = (c % kC) * 8;
      *reinterpret_cast<vec*>(&Qs[row * kRow + col]) = q0 + row < T ? xq[p] : In16<TIn>::zero();
    }
  }

  __shared__ float s_vred[4];   // per wave: largest |V| of a tile
  // Per tile parity and wave: the tile holds a |V| too large for V's exponent.
  __shared__ __attribute__((aligned(16))) int s_vflag[2][4];
  if (kScaleV<TIn>) {
    const float m = wave_max(bf16_bits_to_float(tile_vmax_bits<TIn, D>(nxt)));
    if (lane == 0) s_vred[wave] = m;
  }
  __syncthreads();  // Q staged, tile 0's largest |V| known
  VScale vs = {0, 0x7f80u, true};
  if (kScaleV<TIn>)
    vs = vscale_first(fmaxf(fmaxf(s_vred[0], s_vred[1]), fmaxf(s_vred[2], s_vred[3])));

  FwdState<D> st;
#pragma unroll
  for (int db = 0; db < D / 32; ++db)
#pragma unroll
    for (int r = 0; r < 16; ++r) st.oacc[db][r] = 0.f;
  st.m_run = -INFINITY;
  st.l_run = 0.f;

  const int kv_end = min(T, q0 + kBM);
  const int n_kt = (kv_end + kBN - 1) / kBN;
  // Tiles [0, n_full) need no mask for any wave of the workgroup: all their
  // keys precede query q0 (and hence every query here) and lie below T.
  const int n_full = min(q0, T) / kBN;

  fwd_stage<TIn, D>(Kbuf(0), Vbuf(0), nxt, 0, T, tid, vs.vexp);
  // Q^T as the B operand: lane holds d = 16*kk + 8*hf .. +7 of its query.
  vec qf[D / 16];
#pragma unroll
  for (int kk = 0; kk < D / 16; ++kk)
    qf[kk] = *reinterpret_cast<const vec*>(&Qs[(wave * 32 + l32) * kRow + kk * 16 + 8 * hf]);
  __syncthreads();  // tile 0 staged; every wave holds its Q fragments: buffer 1 is free

  int buf = 0;
  int kt = 0;
  for (; kt < n_full; ++kt, buf ^= 1) {
    const int k0 = kt * kBN;
    const bool has_next = kt + 1 < n_kt;
    if (has_next) fwd_load_tile<TIn, D>(kh, ldk, vh, ldv, k0 + kBN, T, tid, kvoff, nxt);
    if constexpr (D >= 128) {
      // Half by half: one half's scores at a time keep the register count
      // within two waves per SIMD at this head size.
#pragma unroll
      for (int kb = 0; kb < 2; ++kb)
        fwd_half<TIn, D, kFull, DROP>(Kbuf(buf), Vbuf(buf), qf, kb, k0, my_q, T, l32, hf, lane,
                                      scale_log2, a.drop, tm.head, st);
    } else {
      fwd_tile<TIn, D, DROP>(Kbuf(buf), Vbuf(buf), qf, k0, my_q, T, l32, hf, lane, scale_log2,
                             a.drop, tm.head, st);
    }
    extra_barrier();
    if (has_next) {
      fwd_stage<TIn, D>(Kbuf(buf ^ 1), Vbuf(buf ^ 1), nxt, k0 + kBN, T, tid, vs.vexp);
      if (kScaleV<TIn>) {
        const bool big = wave_any(tile_vmax_bits<TIn, D>(nxt) >= vs.thr);
        if (lane == 0) s_vflag[kt & 1][wave] = big;
      }
    }
    __syncthreads();
    if (kScaleV<TIn> && has_next) {
      const i32x4 f = *reinterpret_cast<const i32x4*>(s_vflag[kt & 1]);
      if (f[0] | f[1] | f[2] | f[3])
        fwd_rescale_v<TIn, D>(s_vred, nxt, Kbuf(buf ^ 1), Vbuf(buf ^ 1), k0 + kBN, T, tid, lane,
                              wave, vs, st);
    }
  }
  for (; kt < n_kt; ++kt, buf ^= 1) {
    const int k0 = kt * kBN;
    const bool has_next = kt + 1 < n_kt;
    if (has_next) fwd_load_tile<TIn, D>(kh, ldk, vh, ldv, k0 + kBN, T, tid, kvoff, nxt);
    // Diagonal and boundary tiles, half by half: halves wholly in this wave's
    // future are skipped, the diagonal half gets the fixed triangle.
#pragma unroll
    for (int kb = 0; kb < 2; ++kb) {
      const int kind = block_kind(k0 + 32 * kb, qw0, T);
      if (kind == kFull)
        fwd_half<TIn, D, kFull, DROP>(Kbuf(buf), Vbuf(buf), qf, kb, k0, my_q, T, l32, hf, lane,
                                      scale_log2, a.drop, tm.head, st);
      else if (kind == kDiag)
        fwd_half<TIn, D, kDiag, DROP>(Kbuf(buf), Vbuf(buf), qf, kb, k0, my_q, T, l32, hf, lane,
                                      scale_log2, a.drop, tm.head, st);
      else if (kind == kGeneral)
        fwd_half<TIn, D, kGeneral, DROP>(Kbuf(buf), Vbuf(buf), qf, kb, k0, my_q, T, l32, hf,
                                         lane, scale_log2, a.drop, tm.head, st);
    }
    extra_barrier();
    if (has_next) {
      fwd_stage<TIn, D>(Kbuf(buf ^ 1), Vbuf(buf ^ 1), nxt, k0 + kBN, T, tid, vs.vexp);
      if (kScaleV<TIn>) {
        const bool big = wave_any(tile_vmax_bits<TIn, D>(nxt) >= vs.thr);
        if (lane == 0) s_vflag[kt & 1][wave] = big;
      }
    }
    __syncthreads();
    if (kScaleV<TIn> && has_next) {
      const i32x4 f = *reinterpret_cast<const i32x4*>(s_vflag[kt & 1]);
      if (f[0] | f[1] | f[2] | f[3])
        fwd_rescale_v<TIn, D>(s_vred, nxt, Kbuf(buf ^ 1), Vbuf(buf ^ 1), k0 + kBN, T, tid, lane,
                              wave, vs, st);
    }
  }

  // Epilogue: O = O_acc / l, LSE = (m + log2 l) * ln 2. The wave's O rows
  // (and o_lo rows) go through LDS, which every wave finished reading at the
  // loop's last barrier, so that global stores write whole rows: D/8 lanes
  // per row, 16 bytes each.
  const float l_tot = st.l_run + wave_xor32(st.l_run);
  const float inv = ldexpf((DROP ? a.drop.scale : 1.f) / l_tot, -vs.vexp);
  {
    typedef typename In16<TIn>::vec4 vec4;
    TIn* so = lds_raw + (wave * 32) * kRow;        // O rows [query][d]
    TIn* sl = lds_raw + (kBM + wave * 32) * kRow;  // o_lo rows
    const bool want_lo = a.o_lo != nullptr;  // uniform: the low part only when asked for
#pragma unroll
    for (int db = 0; db < D / 32; ++db)
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        vec4 hi;
        float x[4];
#pragma unroll
        for (int t = 0; t < 4; ++t) {
          x[t] = st.oacc[db][4 * g + t] * inv;
          hi[t] = In16<TIn>::round(x[t]);
        }
        *reinterpret_cast<vec4*>(&so[l32 * kRow + db * 32 + 8 * g + 4 * hf]) = hi;
        if (want_lo) {
          vec4 lo;
#pragma unroll
          for (int t = 0; t < 4; ++t) lo[t] = In16<TIn>::round(x[t] - (float)hi[t]);
          *reinterpret_cast<vec4*>(&sl[l32 * kRow + db * 32 + 8 * g + 4 * hf]) = lo;
        }
      }
    __builtin_amdgcn_wave_barrier();
    extra_barrier();
    TIn* ob = static_cast<TIn*>(a.o) + head_base(a.lo, tm.head, a.H);
    TIn* lb = a.o_lo ? static_cast<TIn*>(a.o_lo) + head_base(a.llo, tm.head, a.H) : nullptr;
    constexpr int kC = D / 8;  // 16-byte chunks per row
#pragma unroll
    for (int i = 0; i < 32 * kC / 64; ++i) {
      const int c = i * 64 + lane;
      const int row = c / kC, col = (c % kC) * 8;
      const int qrow = qw0 + row;
      if (qrow < T) {  // nontemporal: O is read again only by the backward
        __builtin_nontemporal_store(*reinterpret_cast<const vec*>(&so[row * kRow + col]),
                                    reinterpret_cast<vec*>(ob + qrow * (int)a.lo.t + col));
        if (lb)
          __builtin_nontemporal_store(*reinterpret_cast<const vec*>(&sl[row * kRow + col]),
                                      reinterpret_cast<vec*>(lb + qrow * (int)a.llo.t + col));
      }
    }
  }
  if (my_q < T && hf == 0) a.lse[(size_t)tm.head * T + my_q] = (st.m_run + fast_log2(l_tot)) * kLn2;
}

template <typename TIn, int D>
hipError_t launch_fwd(const FwdArgs& a, hipStream_t stream) {
  const int n_qtiles = (a.T + kBM - 1) / kBM;
  const float scale_log2 = kLog2e / __builtin_sqrtf((float)D);  // 1/sqrt(D) * log2(e)
  const dim3 grid(tiled_grid(a.n_heads, n_qtiles));
  if (a.drop.thr != 0)
    hipLaunchKernelGGL((attn_fwd_kernel<TIn, D, true>), grid, dim3(kThreads), 0, stream, a,
                       n_qtiles, scale_log2);
  else
    hipLaunchKernelGGL((attn_fwd_kernel<TIn, D, false>), grid, dim3(kThreads), 0, stream, a,
                       n_qtiles, scale_log2);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_fwd_16(const FwdArgs& a, bool fp16, int D, hipStream_t stream) {
  if (fp16)
    return D == 32 ? launch_fwd<f16, 32>(a, stream)
           : D == 64 ? launch_fwd<f16, 64>(a, stream)
                     : launch_fwd<f16, 128>(a, stream);
  return D == 32 ? launch_fwd<bf16, 32>(a, stream)
         : D == 64 ? launch_fwd<bf16, 64>(a, stream)
                   : launch_fwd<bf16, 128>(a, stream);
}

}  // namespace gpt_attn
