// Causal attention backward, bf16 or fp16 inputs, fp32 accumulation and fp32
// gradients, head dim D in {32, 64, 128}, for gfx950 (CDNA4).
//
// The gradient of sum(dO * O) for O = softmax(Q K^T / sqrt(D), causal) V:
// what autograd forms for nanoGPT's loss.backward() through the fused
// attention call (page "nanoGPT: a real GPT in two 300-line files", sections
// 1 "Summary" and 2 "How the code works"). With s = 1/sqrt(D):
//   delta_i = sum_d dO_id O_id
//   P_ij    = exp(s Q_i.K_j - LSE_i)        (recomputed; j <= i)
//   dV_j    = sum_i P_ij dO_i
//   dP_ij   = dO_i . V_j
//   dS_ij   = P_ij (dP_ij - delta_i)
//   dK_j    = s sum_i dS_ij Q_i,   dQ_i = s sum_j dS_ij K_j
//
// Kernel 1 (prep) forms delta from the stored O (plus its low part o_lo
// when the forward kept it, which restores fp32 accuracy) and, at D = 32 and
// 64, zeroes dQ.
// Kernel 2 (main): a workgroup of 8 waves owns 256 consecutive keys of one
// head (32 per wave), stages their K in LDS, and keeps their V fragments and
// dK, dV accumulators in registers. It walks the 64-query tiles from its
// diagonal to the end of the sequence; each tile of Q and dO is staged once
// in LDS as row-major fp16
// (waves 4..7 prefetch the next tile a step ahead into a second buffer), and
// the transposed operands (Q^T, dO^T for dK^T += Q^T dS and dV^T += dO^T P)
// come from transposing LDS reads. Per tile each wave recomputes P from the
// saved LSE, forms dS and writes its dS^T rows to LDS (without dropout the
// dP accumulators start from -delta, so the MFMA chain yields dP - delta
// directly); then dQ = dS K over
// the 256 keys is formed as 2 * D/32 blocks of 32x32 and added into the fp32
// dQ with atomic adds (which the memory side performs; 256 keys per
// workgroup keep their number at T/256 per dQ element). Waves 0..3 alone
// issue the atomics, so a loader's wait for its prefetched tile never waits
// on atomics too.
//
// Who forms dQ depends on the shape. D = 64: each of waves 0..3 forms one
// whole 32x32 block over all 256 keys while the loaders go on to the next
// tile's S, P and dS; dS is double-buffered, so one barrier per step suffices
// and the two waves that share a SIMD (w and w + 4) are out of phase, one on
// the matrix cores while the other is on the vector unit. D = 32 (two
// blocks): every wave forms one block over a part of the keys, the parts
// meet in LDS after a second barrier, and waves 0..3 add the sums.
//
// Precision: every product runs on fp16 MFMA with fp32 accumulation. Q, K,
// V and dO are converted to fp16 when staged (exact for bf16 in fp16's
// normal range; nothing to do for fp16 inputs), so S = Q K^T and dP = dO V^T
// multiply the inputs exactly; P and dS are rounded to fp16 (11 significant
// bits) for dV += P^T dO, dK += dS^T Q and dQ += dS K.
//
// Attention dropout (a separate instantiation) regenerates the forward's
// keep mask M: per 32x32 block each lane draws the Philox blocks of one query
// and 16 keys, writes the 0 / 0xFFFF masks to a 32 x 32 LDS tile, and reads
// them back transposed (ds_read_b64_tr_b16) into its own register order (its
// key, 8 consecutive queries). The tile is the window of the wave's own dS
// rows that the block's dS overwrites afterwards, so it needs no LDS of its
// own. With z the survivor scale: dV accumulates
// (M P)^T dO and is scaled by z at the end, and dS = P (z M dP - delta);
// delta = rowsum(dO * O) holds with dropout too (O is the dropped output).
#include "attn_common.h"
#include "attn_launch.h"

namespace gpt_attn {
namespace {

constexpr int kBK = 256;      // keys per workgroup (8 waves x 32)
constexpr int kBQ = 64;       // queries per step
constexpr int kThreads = 512;
constexpr int kLoaders = 256; // threads of waves 4..7: they alone load Q/dO tiles
constexpr int kRowS = 72;     // row of the dS^T tile: 64 queries + 8 (144 bytes)

// Padded LDS row of a D-wide 16-bit tile (D + 8 elements).
template <int D>
constexpr int row_of() {
  return D + 8;
}

// One workgroup per (head, chunk of kStatRows rows): D/8 threads per row,
// 8 elements each, kStatRows * D / 2048 rows per thread. Every thread issues
// all of its loads (q, o, o_lo, dout of each of its rows) before using any,
// which keeps more bytes in flight per thread than one row would; rows past T
// are clamped for the loads (they repeat row T - 1, which lies in the same
// chunk) and skipped for the stores. Besides delta and the dQ zeros, the
// workgroup records the largest |Q|, |dO| and |delta| of its chunk, from which
// the main kernel sets its block exponents.
template <typename TIn, int D>
__global__ __launch_bounds__(256) void attn_bwd_prep_kernel(const BwdArgs a, int n_chunks) {
  typedef typename In16<TIn>::vec vec;
  constexpr int kTPR = D / 8, kRPP = 256 / kTPR;  // threads per row, rows per pass
  constexpr int kPass = kStatRows / kRPP;          // rows per thread
  const int head = blockIdx.x / n_chunks, chunk = blockIdx.x - head * n_chunks;
  const int T = a.T;
  const int part = threadIdx.x % kTPR;
  const int r0 = chunk * kStatRows + threadIdx.x / kTPR;
  const TIn* qh = static_cast<const TIn*>(a.q) + head_base(a.lq, head, a.H) + part * 8;
  const TIn* oh = static_cast<const TIn*>(a.o) + head_base(a.lo, head, a.H) + part * 8;
  const TIn* doh = static_cast<const TIn*>(a.dout) + head_base(a.ldo, head, a.H) + part * 8;
  const TIn* loh =
      a.o_lo ? static_cast<const TIn*>(a.o_lo) + head_base(a.llo, head, a.H) + part * 8 : nullptr;
  vec xq[kPass], x[kPass], y[kPass], c[kPass];
#pragma unroll
  for (int i = 0; i < kPass; ++i) {
    const int t = min(r0 + i * kRPP, T - 1);
    xq[i] = *reinterpret_cast<const vec*>(qh + t * a.lq.t);
    // Nontemporal loads: o, o_lo and dout rows are read once here. (They
    // measured 2% faster over a whole step, the main kernel's time included,
    // with the step's data not already in the Infinity Cache.)
    x[i] = __builtin_nontemporal_load(reinterpret_cast<const vec*>(oh + t * a.lo.t));
    y[i] = __builtin_nontemporal_load(reinterpret_cast<const vec*>(doh + t * a.ldo.t));
    if (loh) c[i] = __builtin_nontemporal_load(reinterpret_cast<const vec*>(loh + t * a.llo.t));
  }
  float mq = 0.f, mdo = 0.f, mdel = 0.f;
#pragma unroll
  for (int i = 0; i < kPass; ++i) {
    const int t = r0 + i * kRPP;
    float acc = 0.f;
    if (loh) {
#pragma unroll
      for (int e = 0; e < 8; ++e) acc = fmaf((float)x[i][e] + (float)c[i][e], (float)y[i][e], acc);
    } else {
#pragma unroll
      for (int e = 0; e < 8; ++e) acc = fmaf((float)x[i][e], (float)y[i][e], acc);
    }
#pragma unroll
    for (int m = 1; m < kTPR; m <<= 1) acc += __shfl_xor(acc, m, 64);
    fold_absmax(xq[i], mq);
    fold_absmax(y[i], mdo);
    mdel = fmaxf(mdel, fabsf(acc));
    if (t < T) {
      if (a.dq) {  // null when the main phase writes dQ without atomics
        const f32x4 z = {0.f, 0.f, 0.f, 0.f};
        f32x4* dst = reinterpret_cast<f32x4*>(a.dq + head_base(a.ldq, head, a.H) + t * a.ldq.t +
                                              part * 8);
        dst[0] = z;
        dst[1] = z;
      }
      if (part == 0) a.delta[(size_t)head * T + t] = acc;
    }
  }
  __shared__ float red[4][3];
  mq = wave_max(mq);
  mdo = wave_max(mdo);
  mdel = wave_max(mdel);
  const int wave = threadIdx.x >> 6;
  if ((threadIdx.x & 63) == 0) {
    red[wave][0] = mq;
    red[wave][1] = mdo;
    red[wave][2] = mdel;
  }
  __syncthreads();
  if (threadIdx.x == 0) {
    f32x4 st = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int w = 0; w < 4; ++w)
#pragma unroll
      for (int j = 0; j < 3; ++j) st[j] = fmaxf(st[j], red[w][j]);
    reinterpret_cast<f32x4*>(a.stats)[((size_t)head * n_chunks + chunk) * (kStatFloats / 4)] = st;
  }
}

// dO's block exponent: the largest e with |dS * 2^(e + ev)| < 2^14, from
// |dS| <= z |dP| + |delta| <= z D max|dO| max|V| + max|delta| (z: the dropout
// survivor scale, 1 without dropout; V staged as V * 2^ev), so every rounded
// dS fits fp16 with a factor of two to spare. 0 when both maxima are 0 or
// not finite.
__device__ __forceinline__ int dout_exp(float mdo, float mdel, float mv, int ev, float zs, int D) {
  constexpr int kNone = -(1 << 20);
  int t1 = kNone, t2 = kNone;
  if (mdo > 0.f && mdo <= 3.402823466e38f) {
    const int ka = __builtin_amdgcn_frexp_expf(mdo);  // mdo < 2^ka
    const float x = zs * (float)D * ldexpf(mv, ev) * ldexpf(mdo, -ka);
    t1 = ka + (x > 0.f ? __builtin_amdgcn_frexp_expf(x) : 0);  // z D max|dO| max|V_s| < 2^t1
  }
  if (mdel > 0.f && mdel <= 3.402823466e38f)
    t2 = __builtin_amdgcn_frexp_expf(mdel) + ev;  // max|delta| 2^ev < 2^t2
  return (t1 != kNone || t2 != kNone) ? 13 - max(t1, t2) : 0;
}

// Loading a 64-query tile is split in two so the global loads can be issued
// a whole step ahead: bwd_load_tile only issues raw loads (rows clamped to
// T-1, so every address is valid, and nothing is computed from the results);
// bwd_store_tile, a step later, zeroes rows past T, scales Q by 2^eq and dO
// by 2^edo while converting them to fp16, stores -delta * 2^(edo + ev) (the
// scale of dP), and writes the LDS buffers. Only the 256 threads of waves 4..7 take part (tid
// below is their index 0..255): each moves D/32 16-byte chunks of Q and of
// dO (row c/(D/8), dims (c%(D/8))*8 for c = tid, tid+256, ...), and those
// with tid < 64 also move the LSE and delta of row tid.
template <typename TIn, int D>
struct TileRegs {
  static constexpr int kN = kBQ * D / 8 / kLoaders;
  typename In16<TIn>::vec q[kN], d[kN];
  float lse, del;
};

template <typename TIn, int D>
__device__ __forceinline__ void bwd_load_tile(const TIn* qh, int ldq, const TIn* doh, int lddo,
                                              const float* lse, const float* delta, int qs, int T,
                                              int tid, TileRegs<TIn, D>& r) {
  typedef typename In16<TIn>::vec vec;
  constexpr int kC = D / 8;
#pragma unroll
  for (int p = 0; p < TileRegs<TIn, D>::kN; ++p) {
    const int c = tid + kLoaders * p;
    const int row = min(qs + c / kC, T - 1), col = (c % kC) * 8;
    r.q[p] = *reinterpret_cast<const vec*>(qh + row * ldq + col);
    r.d[p] = *reinterpret_cast<const vec*>(doh + row * lddo + col);
  }
  const int row = min(qs + (tid & (kBQ - 1)), T - 1);
  r.lse = lse[row];
  r.del = delta[row];
}

template <typename TIn, int D>
__device__ __forceinline__ void bwd_store_tile(f16* sQ, f16* sdO, float* sL, float* sD,
                                               const TileRegs<TIn, D>& r, int qs, int T,
                                               int tid, int eq, int edo, int eds) {
  constexpr int kC = D / 8, kRowQ = row_of<D>();
#pragma unroll
  for (int p = 0; p < TileRegs<TIn, D>::kN; ++p) {
    const int c = tid + kLoaders * p;
    const int row = c / kC, col = (c % kC) * 8;
    const bool ok = qs + row < T;
    *reinterpret_cast<f16x8*>(&sQ[row * kRowQ + col]) =
        ok ? cvt_f16_scaled(r.q[p], eq) : zero_f16x8();
    *reinterpret_cast<f16x8*>(&sdO[row * kRowQ + col]) =
        ok ? cvt_f16_scaled(r.d[p], edo) : zero_f16x8();
  }
  if (tid < kBQ) {
    const bool ok = qs + tid < T;
    sL[tid] = ok ? r.lse * kLog2e : 0.f;
    sD[tid] = ok ? ldexpf(-r.del, eds) : 0.f;
  }
}

// P = exp2(S s log2(e) - LSE log2(e)) and dS = P (dP - delta) for the 16
// (query, key) pairs of one lane in one 32x32 block, as fp16. Register
// 8c + t of half hf is query q0 + 16c + 8hf + t; the lane's key is key0 + l32.
// cD holds -delta. Without dropout the dP accumulator already holds
// dP - delta (its MFMA chain started from -delta); with dropout it holds dP.
template <int KIND, bool DROP>
__device__ __forceinline__ void bwd_p_ds(const f32x16& s, const f32x16& dp, const float* cL,
                                         const float* cD, int qoff0, int q0, int key0, int T,
                                         int l32, int hf, float scale_log2, const f16x8 (&mk)[2],
                                         float zscale, f16x8 (&pf)[2], f16x8 (&dsf)[2]) {
  const int key = key0 + l32;
#pragma unroll
  for (int c = 0; c < 2; ++c) {
    const int qoff = qoff0 + 16 * c + 8 * hf;
    const f32x4 L0 = *reinterpret_cast<const f32x4*>(&cL[qoff]);
    const f32x4 L1 = *reinterpret_cast<const f32x4*>(&cL[qoff + 4]);
    f32x4 E0 = {}, E1 = {};
    if (DROP) {
      E0 = *reinterpret_cast<const f32x4*>(&cD[qoff]);
      E1 = *reinterpret_cast<const f32x4*>(&cD[qoff + 4]);
    }
    float p[8], ds[8];
#pragma unroll
    for (int t = 0; t < 8; ++t) {
      const float lse2 = t < 4 ? L0[t] : L1[t - 4];
      float pv = fast_exp2(fmaf(s[8 * c + t], scale_log2, -lse2));
      if (KIND == kDiag) {
        // key0 == q0: visible iff l32 <= 16c + 8hf + t.
        pv = (l32 - 8 * hf > 16 * c + t) ? 0.f : pv;
      } else if (KIND == kGeneral) {
        const int qi = q0 + 16 * c + 8 * hf + t;
        pv = (key > qi || key >= T || qi >= T) ? 0.f : pv;
      }
      p[t] = pv;
      if (DROP) {
        const uint32_t w = (uint32_t)__builtin_bit_cast(i32x4, mk[c])[t >> 1];
        const bool kept = (w >> (16 * (t & 1))) & 1u;
        const float ndel = t < 4 ? E0[t] : E1[t - 4];
        ds[t] = pv * ((kept ? dp[8 * c + t] * zscale : 0.f) + ndel);
      } else {
        ds[t] = pv * dp[8 * c + t];
      }
    }
    pf[c] = pack_f16x8(p[0], p[1], p[2], p[3], p[4], p[5], p[6], p[7]);
    if (DROP) {  // dV takes the dropped weights M P
      i32x4 bits = __builtin_bit_cast(i32x4, pf[c]);
      const i32x4 mbits = __builtin_bit_cast(i32x4, mk[c]);
#pragma unroll
      for (int w = 0; w < 4; ++w) bits[w] &= mbits[w];
      pf[c] = __builtin_bit_cast(f16x8, bits);
    }
    dsf[c] = pack_f16x8(ds[0], ds[1], ds[2], ds[3], ds[4], ds[5], ds[6], ds[7]);
  }
}

// rows[kw0 + k][d] = mul * acc * 2^e for the wave's 32 keys k, through the wave's
// LDS staging area (pitch D + 4 floats): register r of block db of lane
// (l32, hf) is key l32, dim 32db + 8(r/4) + 4hf + r%4. Rows at or past T are
// skipped. Wave-local: LDS runs one wave's operations in order.
template <int D>
__device__ __forceinline__ void store_rows(float* stage, const f32x16 (&acc)[D / 32], float mul,
                                           int e, float* rows, int ld, int kw0, int T, int l32,
                                           int hf, int lane) {
  constexpr int kEp = D + 4, kLpr = D / 4, kRpi = 64 / kLpr;
#pragma unroll
  for (int db = 0; db < D / 32; ++db)
#pragma unroll
    for (int g = 0; g < 4; ++g) {
      const f32x4 x = {ldexpf(acc[db][4 * g] * mul, e), ldexpf(acc[db][4 * g + 1] * mul, e),
                       ldexpf(acc[db][4 * g + 2] * mul, e), ldexpf(acc[db][4 * g + 3] * mul, e)};
      *reinterpret_cast<f32x4*>(&stage[l32 * kEp + db * 32 + 8 * g + 4 * hf]) = x;
    }
  __builtin_amdgcn_wave_barrier();
  extra_barrier();
#pragma unroll
  for (int j = 0; j < 32 / kRpi; ++j) {
    const int row = j * kRpi + lane / kLpr, col = (lane % kLpr) * 4;
    if (kw0 + row < T)  // nontemporal: nothing here reads dK, dV again
      __builtin_nontemporal_store(*reinterpret_cast<const f32x4*>(&stage[row * kEp + col]),
                                  reinterpret_cast<f32x4*>(rows + (kw0 + row) * ld + col));
  }
  __builtin_amdgcn_wave_barrier();
  extra_barrier();
}

// dQ[queries qb0.., dims 32db..] += scale * acc * 2^e for one 32x32 block,
// with atomic adds; register r of lane (l32, hf) is query 8(r/4) + 4hf + r%4, dim
// l32. Rows at or past T are skipped.
__device__ __forceinline__ void add_dq_block(const BwdArgs& a, int head, int qb0, int db, int l32,
                                             int hf, int T, float scale, int e,
                                             const f32x16& acc) {
  // Register r holds row 8(r/4) + 4hf + r%4 of the block, column l32: a
  // workgroup-uniform row offset per register plus one per-lane byte offset
  // (4hf rows and l32 columns). Written as one per-lane pointer per
  // register, the compiler had computed all sixteen 64-bit pointers once and
  // kept them live across the caller's loop (32 vector registers); here the
  // row offsets are scalar and formed on every call (opaque_u32_uniform
  // keeps them from being hoisted).
  const uint32_t lddq = opaque_u32_uniform((uint32_t)a.ldq.t);
  const uint32_t voff = (4u * (uint32_t)hf * lddq + (uint32_t)l32) * (uint32_t)sizeof(float);
  float* blk = a.dq + head_base(a.ldq, head, a.H) + (size_t)(uint32_t)qb0 * lddq + db * 32;
  auto add = [&](int r) {
    float* row = blk + (size_t)(8 * (r >> 2) + (r & 3)) * lddq;
    atomicAdd(reinterpret_cast<float*>(reinterpret_cast<char*>(row) + voff),
              ldexpf(acc[r] * scale, e));
  };
  if (qb0 + 32 <= T) {
#pragma unroll
    for (int r = 0; r < 16; ++r) add(r);
  } else {
#pragma unroll
    for (int r = 0; r < 16; ++r)
      if (qb0 + 8 * (r >> 2) + (r & 3) + 4 * hf < T) add(r);
  }
}

// Row strides inside one head are 32-bit (the host checks T * stride < 2^31);
// head offsets are 64-bit.
template <typename TIn, int D, bool DROP>
__global__ __launch_bounds__(kThreads, 1) void attn_bwd_main_kernel(const BwdArgs a, int n_ktiles,
                                                                    float scale,
                                                                    float scale_log2) {
  typedef typename In16<TIn>::vec vec;
  constexpr int kRowQ = row_of<D>();
  constexpr int kDB = D / 32;          // 32-wide dimension blocks
  constexpr int kBlk = 2 * kDB;        // 32x32 blocks of a tile's dQ
  constexpr int kParts = 8 / kBlk;     // key parts per block (one wave each)
  constexpr int kSteps = kBK / 16 / kParts;  // 16-key MFMA steps per part
  // Waves 0..3 form whole dQ blocks (see the top of the file) when there is
  // one block per wave (D = 64).
  constexpr bool kSplit = kBlk == 4;
  constexpr int kNdS = kSplit ? 2 : 1;
  // All tiles fp16, row-major; transposed operands come from lds_operand_tr.
  __shared__ __attribute__((aligned(16))) f16 sK[kBK * kRowQ];          // [key][d]
  __shared__ __attribute__((aligned(16))) f16 sQ[2][kBQ * kRowQ];       // [q][d]
  __shared__ __attribute__((aligned(16))) f16 sdO[2][kBQ * kRowQ];      // [q][d]
  __shared__ __attribute__((aligned(16))) f16 sdS_buf[kNdS][kBK * kRowS];  // [key][q]
  __shared__ __attribute__((aligned(16))) float sPart[kSplit ? 1 : (kParts - 1) * kBlk][16][64];
  __shared__ __attribute__((aligned(16))) float sL[2][kBQ];             // LSE * log2(e)
  __shared__ __attribute__((aligned(16))) float sD[2][kBQ];             // -delta
  __shared__ float sRed[8][2];  // per wave: largest |K|, |V| of its keys

  const int T = a.T;
  const TileMap tm = map_tile_xcd(blockIdx.x, a.n_heads, n_ktiles, false);
  if (!tm.valid) return;

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int hf = lane >> 5, l32 = lane & 31;
  // Waves 4..7 load the query tiles; the waves of key part 0 (0 .. kBlk-1)
  // issue the dQ atomics. No wave does both, so a wait for a prefetched tile
  // never waits on atomics too.
  const bool loader = wave >= 4;
  const int ltid = tid - kLoaders;

  const size_t roff = (size_t)tm.head * (size_t)T;
  const TIn* __restrict__ qh = static_cast<const TIn*>(a.q) + head_base(a.lq, tm.head, a.H);
  const TIn* __restrict__ kh = static_cast<const TIn*>(a.k) + head_base(a.lk, tm.head, a.H);
  const TIn* __restrict__ vh = static_cast<const TIn*>(a.v) + head_base(a.lv, tm.head, a.H);
  const TIn* __restrict__ doh = static_cast<const TIn*>(a.dout) + head_base(a.ldo, tm.head, a.H);
  const int ldq = (int)a.lq.t, ldk = (int)a.lk.t, ldv = (int)a.lv.t, lddo = (int)a.ldo.t;
  const float* lseh = a.lse + roff;
  const float* delh = a.delta + roff;

  const int k0 = tm.tile * kBK;
  const int kw0 = k0 + wave * 32;
  const int my_key = kw0 + l32;  // the key column this lane owns

  // V of this wave's 32 keys as fp16 B operands (lane: its key, 8 dims).
  // All 256 keys of K, row-major fp16, for the dQ product. Every load of the
  // prologue is issued before any result is used (rows clamped to T - 1, so
  // every address is valid; rows past T are zeroed when converted), so their
  // latencies overlap.
  constexpr int kKP = kBK * D / 8 / kThreads;  // K chunks per thread
  vec kraw[kKP], vraw[D / 16];
  const int vrow = min(my_key, T - 1);
#pragma unroll
  for (int kk = 0; kk < D / 16; ++kk)
    vraw[kk] = *reinterpret_cast<const vec*>(vh + vrow * ldv + kk * 16 + 8 * hf);
#pragma unroll
  for (int p = 0; p < kKP; ++p) {
    constexpr int kC = D / 8;
    const int c = tid + kThreads * p;  // key c/kC, 8 dims at (c%kC)*8
    kraw[p] = *reinterpret_cast<const vec*>(kh + min(k0 + c / kC, T - 1) * ldk + (c % kC) * 8);
  }
  TileRegs<TIn, D> nxt;
  if (loader) bwd_load_tile<TIn, D>(qh, ldq, doh, lddo, lseh, delh, k0, T, ltid, nxt);

  // Block exponents (see block_exp). K and V: this workgroup's 256 keys,
  // reduced here; Q, dO and delta: every row the workgroup visits, from the
  // preprocess pass's per-chunk maxima (chunks from k0 on; k0 is a multiple
  // of kStatRows). Rows past T repeat row T - 1, one of this workgroup's.
  float mk = 0.f, mv = 0.f, mq = 0.f, mdo = 0.f, mdel = 0.f;
#pragma unroll
  for (int kk = 0; kk < D / 16; ++kk) fold_absmax(vraw[kk], mv);
#pragma unroll
  for (int p = 0; p < kKP; ++p) fold_absmax(kraw[p], mk);
  {
    const int n_chunks = (T + kStatRows - 1) / kStatRows;
    const f32x4* st =
        reinterpret_cast<const f32x4*>(a.stats) + (size_t)tm.head * n_chunks * (kStatFloats / 4);
    for (int c = k0 / kStatRows + lane; c < n_chunks; c += 64) {
      const f32x4 x = st[c * (kStatFloats / 4)];
      mq = fmaxf(mq, x[0]);
      mdo = fmaxf(mdo, x[1]);
      mdel = fmaxf(mdel, x[2]);
    }
  }
  mk = wave_max(mk);
  mv = wave_max(mv);
  mq = wave_max(mq);
  mdo = wave_max(mdo);
  mdel = wave_max(mdel);
  if (lane == 0) {
    sRed[wave][0] = mk;
    sRed[wave][1] = mv;
  }
  __syncthreads();
#pragma unroll
  for (int w = 0; w < 8; ++w) {
    mk = fmaxf(mk, sRed[w][0]);
    mv = fmaxf(mv, sRed[w][1]);
  }
  // Q and K to [2^13, 2^14) (only their fp16 range matters); V to [1, 2);
  // dO from the dS bound (dout_exp).
  const float zs = DROP ? a.drop.scale : 1.f;
  const int ek = __builtin_amdgcn_readfirstlane(block_exp(mk, 13));
  const int ev = __builtin_amdgcn_readfirstlane(block_exp(mv, 0));
  const int eq = __builtin_amdgcn_readfirstlane(block_exp(mq, 13));
  const int edo = __builtin_amdgcn_readfirstlane(dout_exp(mdo, mdel, mv, ev, zs, D));

  f16x8 vf[D / 16];
#pragma unroll
  for (int kk = 0; kk < D / 16; ++kk)
    vf[kk] = my_key < T ? cvt_f16_scaled(vraw[kk], ev) : zero_f16x8();
#pragma unroll
  for (int p = 0; p < kKP; ++p) {
    constexpr int kC = D / 8;
    const int c = tid + kThreads * p;
    const int row = c / kC, col = (c % kC) * 8;
    *reinterpret_cast<f16x8*>(&sK[row * kRowQ + col]) =
        k0 + row < T ? cvt_f16_scaled(kraw[p], ek) : zero_f16x8();
  }

  f32x16 dvacc[kDB], dkacc[kDB];
#pragma unroll
  for (int db = 0; db < kDB; ++db)
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      dvacc[db][r] = 0.f;
      dkacc[db][r] = 0.f;
    }

  if (loader) bwd_store_tile<TIn, D>(sQ[0], sdO[0], sL[0], sD[0], nxt, k0, T, ltid, eq, edo,
                                     edo + ev);
  __syncthreads();

  // With the operands scaled, S carries 2^(eq + ek), so the exponent's
  // scale shrinks by that; dV carries 2^edo, dK 2^(edo + ev + eq) and each
  // dQ block 2^(edo + ev + ek), removed when they are written.
  const float sl2 = ldexpf(scale_log2, -(eq + ek));
  const int e_dv = -edo, e_dk = -(edo + ev + eq), e_dq = -(edo + ev + ek);

  // The K operands of S = Q K^T (this wave's 32 keys), held in registers.
  f16x8 kreg[D / 16];
#pragma unroll
  for (int kk = 0; kk < D / 16; ++kk)
    kreg[kk] = *reinterpret_cast<const f16x8*>(&sK[(wave * 32 + l32) * kRowQ + kk * 16 + 8 * hf]);
  int buf = 0;
  for (int qs = k0; qs < T; qs += kBQ, buf ^= 1) {
    extra_barrier();
    // Prefetch the next tile into registers while this one is computed.
    const bool has_next = qs + kBQ < T;
    if (loader && has_next)
      bwd_load_tile<TIn, D>(qh, ldq, doh, lddo, lseh, delh, qs + kBQ, T, ltid, nxt);

    f16* sdS = sdS_buf[kSplit ? buf : 0];
    const f16* cQ = sQ[buf];
    const f16* cdO = sdO[buf];
    const float* cL = sL[buf];
    const float* cD = sD[buf];

#pragma unroll
    for (int mb = 0; mb < 2; ++mb) {
      const int qb0 = qs + mb * 32;
      const int kind = block_kind(kw0, qb0, T);
      f16x8 pf[2], dsf[2];
      if (kind == kEmpty) {
        pf[0] = pf[1] = dsf[0] = dsf[1] = zero_f16x8();
      } else {
        f16x8 mk[2];
        if (DROP) {
          // Lane L draws query qb0 + L/2, keys kw0 + 16 (L%2) .. +15 (two
          // Philox blocks) into row L/2 of the wave's tile [query][key]. The
          // tile lives in the 32 x 32 window of this wave's dS rows that the
          // block's dS overwrites below, after the tile has been read back.
          uint16_t* tile = reinterpret_cast<uint16_t*>(sdS + (wave * 32) * kRowS + mb * 32);
          uint32_t m0[4], m1[4];
          const uint32_t grp = (uint32_t)(kw0 >> 3) + 2u * (uint32_t)(lane & 1);
          keep_mask8(a.drop, (uint32_t)tm.head, (uint32_t)(qb0 + (lane >> 1)), grp, m0);
          keep_mask8(a.drop, (uint32_t)tm.head, (uint32_t)(qb0 + (lane >> 1)), grp + 1, m1);
          i32x4* dst = reinterpret_cast<i32x4*>(tile + (lane >> 1) * kRowS + 16 * (lane & 1));
          dst[0] = i32x4{(int)m0[0], (int)m0[1], (int)m0[2], (int)m0[3]};
          dst[1] = i32x4{(int)m1[0], (int)m1[1], (int)m1[2], (int)m1[3]};
          __builtin_amdgcn_wave_barrier();
        }
        // Without dropout the dP chain starts from -delta (register 8c + t of
        // half hf is query qb0 + 16c + 8hf + t), so it ends at dP - delta.
        f32x16 s, dp;
#pragma unroll
        for (int r = 0; r < 16; ++r) s[r] = 0.f;
        if (DROP) {
#pragma unroll
          for (int r = 0; r < 16; ++r) dp[r] = 0.f;
        } else {
#pragma unroll
          for (int c = 0; c < 2; ++c)
#pragma unroll
            for (int h = 0; h < 2; ++h) {
              const f32x4 nd =
                  *reinterpret_cast<const f32x4*>(&cD[mb * 32 + 16 * c + 8 * hf + 4 * h]);
#pragma unroll
              for (int t = 0; t < 4; ++t) dp[8 * c + 4 * h + t] = nd[t];
            }
        }
        const int arow = (mb * 32 + perm32(l32)) * kRowQ + 8 * hf;
#pragma unroll
        for (int kk = 0; kk < D / 16; ++kk) {
          s = mfma32x32x16_f16(*reinterpret_cast<const f16x8*>(&cQ[arow + kk * 16]), kreg[kk], s);
          dp = mfma32x32x16_f16(*reinterpret_cast<const f16x8*>(&cdO[arow + kk * 16]), vf[kk],
                                dp);
        }
        if (DROP) {
          // Lane (key l32, half hf): queries 16c + 8hf .. +7 of its key.
          const f16* tile = sdS + (wave * 32) * kRowS + mb * 32;
#pragma unroll
          for (int c = 0; c < 2; ++c) mk[c] = lds_operand_tr(tile, kRowS, 16 * c, 0, lane);
          __builtin_amdgcn_wave_barrier();
        } else {
          mk[0] = mk[1] = zero_f16x8();
        }
        if (kind == kFull)
          bwd_p_ds<kFull, DROP>(s, dp, cL, cD, mb * 32, qb0, kw0, T, l32, hf, sl2, mk, zs,
                                pf, dsf);
        else if (kind == kDiag)
          bwd_p_ds<kDiag, DROP>(s, dp, cL, cD, mb * 32, qb0, kw0, T, l32, hf, sl2, mk, zs,
                                pf, dsf);
        else
          bwd_p_ds<kGeneral, DROP>(s, dp, cL, cD, mb * 32, qb0, kw0, T, l32, hf, sl2, mk,
                                   zs, pf, dsf);
      }
#pragma unroll
      for (int c = 0; c < 2; ++c) {
        // dS^T row of this lane's key: 8 consecutive queries, one 16-byte write.
        *reinterpret_cast<f16x8*>(&sdS[(wave * 32 + l32) * kRowS + mb * 32 + 16 * c + 8 * hf]) =
            dsf[c];
        // dV^T += dO^T P and dK^T += Q^T dS over these 16 queries.
        const int ks = 2 * mb + c;
#pragma unroll
        for (int db = 0; db < kDB; ++db) {
          dvacc[db] = mfma32x32x16_f16(lds_operand_tr(cdO, kRowQ, ks * 16, db * 32, lane), pf[c],
                                       dvacc[db]);
          dkacc[db] = mfma32x32x16_f16(lds_operand_tr(cQ, kRowQ, ks * 16, db * 32, lane), dsf[c],
                                       dkacc[db]);
        }
      }
    }
    // Stage the prefetched tile into the other buffer, last read in the
    // previous step before its first barrier.
    extra_barrier();
    if (loader && has_next)
      bwd_store_tile<TIn, D>(sQ[buf ^ 1], sdO[buf ^ 1], sL[buf ^ 1], sD[buf ^ 1], nxt, qs + kBQ,
                             T, ltid, eq, edo, edo + ev);
    __syncthreads();

    // dQ of the 64-query tile = dS K over the 256 keys, as kBlk 32x32 blocks
    // (queries 32qb.., dims 32db..). Every wave wrote its dS rows (zeros where
    // nothing is visible).
    if (kSplit) {
      // Wave w < 4 forms block w over all keys and adds it into dQ; the
      // loaders go straight on to the next tile. This step's dS buffer is
      // rewritten two steps on, after the next barrier, which waves 0..3
      // reach only after these reads.
      if (!loader) {
        const int qb = wave / kDB, db = wave % kDB;
        const int qb0 = qs + qb * 32;
        if (qb0 < T) {
          f32x16 acc;
#pragma unroll
          for (int r = 0; r < 16; ++r) acc[r] = 0.f;
#pragma unroll
          for (int ks = 0; ks < kBK / 16; ++ks)
            acc = mfma32x32x16_f16(lds_operand_tr(sdS, kRowS, ks * 16, qb * 32, lane),
                                   lds_operand_tr(sK, kRowQ, ks * 16, db * 32, lane), acc);
          add_dq_block(a, tm.head, qb0, db, l32, hf, T, scale, e_dq, acc);
        }
      }
      continue;
    }
    // Wave w takes block w % kBlk over key part w / kBlk (kSteps steps of 16
    // keys); the other parts pass their sums to part 0 through LDS, whose
    // waves add the total into dQ.
    const int blk = wave % kBlk, kpart = wave / kBlk;
    const int qb = blk / kDB, db = blk % kDB;
    const int qb0 = qs + qb * 32;
    f32x16 acc;
#pragma unroll
    for (int r = 0; r < 16; ++r) acc[r] = 0.f;
    if (qb0 < T) {
#pragma unroll
      for (int j = 0; j < kSteps; ++j) {
        const int ks = kSteps * kpart + j;
        acc = mfma32x32x16_f16(lds_operand_tr(sdS, kRowS, ks * 16, qb * 32, lane),
                               lds_operand_tr(sK, kRowQ, ks * 16, db * 32, lane), acc);
      }
      if (kpart > 0) {
#pragma unroll
        for (int r = 0; r < 16; ++r) sPart[(kpart - 1) * kBlk + blk][r][lane] = acc[r];
      }
    }
    __syncthreads();
    if (kpart == 0 && qb0 < T) {
#pragma unroll
      for (int p = 0; p < kParts - 1; ++p)
#pragma unroll
        for (int r = 0; r < 16; ++r) acc[r] += sPart[p * kBlk + blk][r][lane];
      add_dq_block(a, tm.head, qb0, db, l32, hf, T, scale, e_dq, acc);
    }
    // The next step's dS and partial-sum writes come after its first
    // barrier, which every wave reaches only after the reads above.
  }

  // ---- epilogue: dV = z * dV_acc * 2^e_dv, dK = s * dK_acc * 2^e_dk, written
  // as whole rows.
  // Each wave stages its 32 key rows in LDS (waves 0..3 in the K tile's
  // space, waves 4..7 in the first dS buffer), then each store covers
  // 64 / (D/4) complete rows, D/4 lanes of 16 bytes per row. The barrier
  // ends the last step's reads of both areas.
  __syncthreads();
  constexpr int kEp = D + 4;  // staging row pitch, floats
  static_assert(sizeof(sK) >= 4 * 32 * kEp * sizeof(float), "staging must fit in sK");
  static_assert(sizeof(sdS_buf[0]) >= 4 * 32 * kEp * sizeof(float), "staging must fit in dS");
  float* stage =
      reinterpret_cast<float*>(wave < 4 ? static_cast<void*>(sK) : static_cast<void*>(sdS_buf[0])) +
      (wave & 3) * 32 * kEp;
  store_rows<D>(stage, dvacc, zs, e_dv, a.dv + head_base(a.ldv, tm.head, a.H), (int)a.ldv.t, kw0,
                T, l32, hf, lane);
  store_rows<D>(stage, dkacc, scale, e_dk, a.dk + head_base(a.ldk, tm.head, a.H), (int)a.ldk.t,
                kw0, T, l32, hf, lane);
}

// ---------------------------------------------------------------------------
// The split backward: attn_bwd_dkdv_kernel (the main kernel's step without
// dQ, 128 keys per workgroup) and attn_bwd_dq_kernel (dQ = dS K with S and dP
// recomputed, one workgroup per 128 queries, like the forward); dQ is written
// once instead of accumulated with atomics. The products and their block
// exponents are those of the main kernel. It serves head dimension 128,
// where a wave that owns 32 keys would hold 128 registers of dK and dV
// accumulators and 64 of K and V operands, more than two waves per SIMD can
// hold next to the main kernel's dQ work. (At D = 32 and 64 the main kernel
// is faster at every sequence length measured, 64 to 2048: the split pair
// computes S and dP twice.)

constexpr int kSplitWaves = 4;                   // waves per workgroup in both kernels
constexpr int kSplitThreads = 64 * kSplitWaves;  // threads
constexpr int kSplitKeys = 32 * kSplitWaves;     // keys per dK/dV workgroup (one statistics chunk)
constexpr int kSplitQueries = 32 * kSplitWaves;  // queries per dQ workgroup (one statistics chunk)
static_assert(kSplitKeys == kStatRows && kSplitQueries == kStatRows, "one chunk per workgroup");
static_assert(kSplitThreads == kLoaders, "every thread of the dK/dV kernel loads query tiles");

// dK and dV for one workgroup of 128 keys: waves 0..3 own 32 keys each, as
// the main kernel's waves do; all 256 threads load the next query tile a step
// ahead. Also records the largest |K| and |V| of its keys (one statistics
// chunk) for the dQ kernel.
template <typename TIn, int D, bool DROP>
__global__ __launch_bounds__(kSplitThreads, 1) void attn_bwd_dkdv_kernel(const BwdArgs a,
                                                                        int n_ktiles, float scale,
                                                                        float scale_log2) {
  typedef typename In16<TIn>::vec vec;
  constexpr int kRowQ = row_of<D>();
  constexpr int kDB = D / 32;
  __shared__ __attribute__((aligned(16))) f16 sQ[2][kBQ * kRowQ];   // [q][d]
  __shared__ __attribute__((aligned(16))) f16 sdO[2][kBQ * kRowQ];  // [q][d]
  __shared__ __attribute__((aligned(16))) float sL[2][kBQ];         // LSE * log2(e)
  __shared__ __attribute__((aligned(16))) float sD[2][kBQ];         // -delta
  // Dropout: each wave's 32 x 32 keep-mask tile [query][key].
  __shared__ __attribute__((aligned(16))) f16 sM[DROP ? kSplitWaves : 1][32 * kRowS];
  __shared__ float sRed[kSplitWaves][2];

  const int T = a.T;
  const TileMap tm = map_tile_xcd(blockIdx.x, a.n_heads, n_ktiles, false);
  if (!tm.valid) return;
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int hf = lane >> 5, l32 = lane & 31;

  const size_t roff = (size_t)tm.head * (size_t)T;
  const TIn* __restrict__ qh = static_cast<const TIn*>(a.q) + head_base(a.lq, tm.head, a.H);
  const TIn* __restrict__ kh = static_cast<const TIn*>(a.k) + head_base(a.lk, tm.head, a.H);
  const TIn* __restrict__ vh = static_cast<const TIn*>(a.v) + head_base(a.lv, tm.head, a.H);
  const TIn* __restrict__ doh = static_cast<const TIn*>(a.dout) + head_base(a.ldo, tm.head, a.H);
  const int ldq = (int)a.lq.t, ldk = (int)a.lk.t, ldv = (int)a.lv.t, lddo = (int)a.ldo.t;
  const float* lseh = a.lse + roff;
  const float* delh = a.delta + roff;

  const int k0 = tm.tile * kSplitKeys;
  const int kw0 = k0 + wave * 32;
  const int my_key = kw0 + l32;

  // K and V of this lane's key as the B operands of S and dP (8 dims per
  // 16-dim step, half hf); the first query tile; all issued before use.
  vec kraw[D / 16], vraw[D / 16];
  const int krow = min(my_key, T - 1);
#pragma unroll
  for (int kk = 0; kk < D / 16; ++kk) {
    kraw[kk] = *reinterpret_cast<const vec*>(kh + krow * ldk + kk * 16 + 8 * hf);
    vraw[kk] = *reinterpret_cast<const vec*>(vh + krow * ldv + kk * 16 + 8 * hf);
  }
  TileRegs<TIn, D> nxt;
  bwd_load_tile<TIn, D>(qh, ldq, doh, lddo, lseh, delh, k0, T, tid, nxt);

  const int n_chunks = (T + kStatRows - 1) / kStatRows;
  float mk = 0.f, mv = 0.f, mq = 0.f, mdo = 0.f, mdel = 0.f;
#pragma unroll
  for (int kk = 0; kk < D / 16; ++kk) {
    fold_absmax(kraw[kk], mk);
    fold_absmax(vraw[kk], mv);
  }
  {
    const f32x4* st =
        reinterpret_cast<const f32x4*>(a.stats) + (size_t)tm.head * n_chunks * (kStatFloats / 4);
    for (int c = k0 / kStatRows + lane; c < n_chunks; c += 64) {
      const f32x4 x = st[c * (kStatFloats / 4)];
      mq = fmaxf(mq, x[0]);
      mdo = fmaxf(mdo, x[1]);
      mdel = fmaxf(mdel, x[2]);
    }
  }
  mk = wave_max(mk);
  mv = wave_max(mv);
  mq = wave_max(mq);
  mdo = wave_max(mdo);
  mdel = wave_max(mdel);
  if (lane == 0) {
    sRed[wave][0] = mk;
    sRed[wave][1] = mv;
  }
  __syncthreads();
#pragma unroll
  for (int w = 0; w < kSplitWaves; ++w) {
    mk = fmaxf(mk, sRed[w][0]);
    mv = fmaxf(mv, sRed[w][1]);
  }
  if (tid == 0) {
    const f32x4 kv = {mk, mv, 0.f, 0.f};
    reinterpret_cast<f32x4*>(a.stats)[((size_t)tm.head * n_chunks + k0 / kStatRows) *
                                          (kStatFloats / 4) + 1] = kv;
  }
  const float zs = DROP ? a.drop.scale : 1.f;
  const int ek = __builtin_amdgcn_readfirstlane(block_exp(mk, 13));
  const int ev = __builtin_amdgcn_readfirstlane(block_exp(mv, 0));
  const int eq = __builtin_amdgcn_readfirstlane(block_exp(mq, 13));
  const int edo = __builtin_amdgcn_readfirstlane(dout_exp(mdo, mdel, mv, ev, zs, D));

  f16x8 kreg[D / 16], vf[D / 16];
#pragma unroll
  for (int kk = 0; kk < D / 16; ++kk) {
    kreg[kk] = my_key < T ? cvt_f16_scaled(kraw[kk], ek) : zero_f16x8();
    vf[kk] = my_key < T ? cvt_f16_scaled(vraw[kk], ev) : zero_f16x8();
  }
  f32x16 dvacc[kDB], dkacc[kDB];
#pragma unroll
  for (int db = 0; db < kDB; ++db)
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      dvacc[db][r] = 0.f;
      dkacc[db][r] = 0.f;
    }
  bwd_store_tile<TIn, D>(sQ[0], sdO[0], sL[0], sD[0], nxt, k0, T, tid, eq, edo, edo + ev);
  __syncthreads();

  const float sl2 = ldexpf(scale_log2, -(eq + ek));
  int buf = 0;
  for (int qs = k0; qs < T; qs += kBQ, buf ^= 1) {
    extra_barrier();
    const bool has_next = qs + kBQ < T;
    if (has_next) bwd_load_tile<TIn, D>(qh, ldq, doh, lddo, lseh, delh, qs + kBQ, T, tid, nxt);
    const f16* cQ = sQ[buf];
    const f16* cdO = sdO[buf];
    const float* cL = sL[buf];
    const float* cD = sD[buf];
#pragma unroll
    for (int mb = 0; mb < 2; ++mb) {
      const int qb0 = qs + mb * 32;
      const int kind = block_kind(kw0, qb0, T);
      if (kind == kEmpty) continue;
      f16x8 mk2[2];
      if (DROP) {
        // Lane L draws query qb0 + L/2, keys kw0 + 16 (L%2) .. +15 into row
        // L/2 of the wave's mask tile, read back in the lane = key order.
        uint16_t* tile = reinterpret_cast<uint16_t*>(sM[DROP ? wave : 0]);
        uint32_t m0[4], m1[4];
        const uint32_t grp = (uint32_t)(kw0 >> 3) + 2u * (uint32_t)(lane & 1);
        keep_mask8(a.drop, (uint32_t)tm.head, (uint32_t)(qb0 + (lane >> 1)), grp, m0);
        keep_mask8(a.drop, (uint32_t)tm.head, (uint32_t)(qb0 + (lane >> 1)), grp + 1, m1);
        i32x4* dst = reinterpret_cast<i32x4*>(tile + (lane >> 1) * kRowS + 16 * (lane & 1));
        dst[0] = i32x4{(int)m0[0], (int)m0[1], (int)m0[2], (int)m0[3]};
        dst[1] = i32x4{(int)m1[0], (int)m1[1], (int)m1[2], (int)m1[3]};
        __builtin_amdgcn_wave_barrier();
      }
      f32x16 s, dp;
#pragma unroll
      for (int r = 0; r < 16; ++r) s[r] = 0.f;
      if (DROP) {
#pragma unroll
        for (int r = 0; r < 16; ++r) dp[r] = 0.f;
      } else {
#pragma unroll
        for (int c = 0; c < 2; ++c)
#pragma unroll
          for (int h = 0; h < 2; ++h) {
            const f32x4 nd =
                *reinterpret_cast<const f32x4*>(&cD[mb * 32 + 16 * c + 8 * hf + 4 * h]);
#pragma unroll
            for (int t = 0; t < 4; ++t) dp[8 * c + 4 * h + t] = nd[t];
          }
      }
      const int arow = (mb * 32 + perm32(l32)) * kRowQ + 8 * hf;
#pragma unroll
      for (int kk = 0; kk < D / 16; ++kk) {
        s = mfma32x32x16_f16(*reinterpret_cast<const f16x8*>(&cQ[arow + kk * 16]), kreg[kk], s);
        dp = mfma32x32x16_f16(*reinterpret_cast<const f16x8*>(&cdO[arow + kk * 16]), vf[kk], dp);
      }
      if (DROP) {
        const f16* tile = sM[DROP ? wave : 0];
#pragma unroll
        for (int c = 0; c < 2; ++c) mk2[c] = lds_operand_tr(tile, kRowS, 16 * c, 0, lane);
        __builtin_amdgcn_wave_barrier();
      } else {
        mk2[0] = mk2[1] = zero_f16x8();
      }
      f16x8 pf[2], dsf[2];
      if (kind == kFull)
        bwd_p_ds<kFull, DROP>(s, dp, cL, cD, mb * 32, qb0, kw0, T, l32, hf, sl2, mk2, zs, pf, dsf);
      else if (kind == kDiag)
        bwd_p_ds<kDiag, DROP>(s, dp, cL, cD, mb * 32, qb0, kw0, T, l32, hf, sl2, mk2, zs, pf, dsf);
      else
        bwd_p_ds<kGeneral, DROP>(s, dp, cL, cD, mb * 32, qb0, kw0, T, l32, hf, sl2, mk2, zs, pf,
                                 dsf);
#pragma unroll
      for (int c = 0; c < 2; ++c) {
        const int ks = 2 * mb + c;
#pragma unroll
        for (int db = 0; db < kDB; ++db) {
          dvacc[db] = mfma32x32x16_f16(lds_operand_tr(cdO, kRowQ, ks * 16, db * 32, lane), pf[c],
                                       dvacc[db]);
          dkacc[db] = mfma32x32x16_f16(lds_operand_tr(cQ, kRowQ, ks * 16, db * 32, lane), dsf[c],
                                       dkacc[db]);
        }
      }
    }
    // Stage the prefetched tile into the other buffer, last read in the
    // previous step before its barrier.
    extra_barrier();
    if (has_next)
      bwd_store_tile<TIn, D>(sQ[buf ^ 1], sdO[buf ^ 1], sL[buf ^ 1], sD[buf ^ 1], nxt, qs + kBQ,
                             T, tid, eq, edo, edo + ev);
    __syncthreads();
  }

  // dV = z dV_acc 2^-edo and dK = s dK_acc 2^-(edo + ev + eq), whole rows
  // through LDS (each wave's 32 rows: waves 0, 1 in the Q buffers, waves 2, 3
  // in the dO buffers, free after the loop's last barrier).
  constexpr int kEp = D + 4;
  static_assert(sizeof(sQ) >= 2 * 32 * kEp * sizeof(float), "staging fits");
  static_assert(sizeof(sdO) >= 2 * 32 * kEp * sizeof(float), "staging fits");
  float* stage =
      reinterpret_cast<float*>(wave < 2 ? &sQ[0][0] : &sdO[0][0]) + (wave & 1) * 32 * kEp;
  store_rows<D>(stage, dvacc, zs, -edo, a.dv + head_base(a.ldv, tm.head, a.H), (int)a.ldv.t, kw0,
                T, l32, hf, lane);
  store_rows<D>(stage, dkacc, scale, -(edo + ev + eq), a.dk + head_base(a.ldk, tm.head, a.H),
                (int)a.ldk.t, kw0, T, l32, hf, lane);
}

// K and V tiles of the dQ kernel: 64 keys, staged into LDS as fp16 scaled by
// 2^ek and 2^ev, loaded a tile ahead as raw 16-byte chunks (rows clamped to
// T - 1; rows past T are zeroed when staged).
template <typename TIn, int D>
struct KVTile {
  static constexpr int kN = 64 * D / 8 / kSplitThreads;
  typename In16<TIn>::vec k[kN], v[kN];
};

template <typename TIn, int D>
__device__ __forceinline__ void dq_load_kv(const TIn* kh, int ldk, const TIn* vh, int ldv, int k0,
                                           int T, int tid, KVTile<TIn, D>& r) {
  typedef typename In16<TIn>::vec vec;
  constexpr int kC = D / 8;
#pragma unroll
  for (int p = 0; p < KVTile<TIn, D>::kN; ++p) {
    const int c = tid + kSplitThreads * p;
    const int row = min(k0 + c / kC, T - 1), col = (c % kC) * 8;
    r.k[p] = *reinterpret_cast<const vec*>(kh + row * ldk + col);
    r.v[p] = *reinterpret_cast<const vec*>(vh + row * ldv + col);
  }
}

template <typename TIn, int D>
__device__ __forceinline__ void dq_store_kv(f16* Ks, f16* Vs, const KVTile<TIn, D>& r, int k0,
                                            int T, int tid, int ek, int ev) {
  constexpr int kC = D / 8, kRow = row_of<D>();
#pragma unroll
  for (int p = 0; p < KVTile<TIn, D>::kN; ++p) {
    const int c = tid + kSplitThreads * p;
    const int row = c / kC, col = (c % kC) * 8;
    const bool ok = k0 + row < T;
    *reinterpret_cast<f16x8*>(&Ks[row * kRow + col]) =
        ok ? cvt_f16_scaled(r.k[p], ek) : zero_f16x8();
    *reinterpret_cast<f16x8*>(&Vs[row * kRow + col]) =
        ok ? cvt_f16_scaled(r.v[p], ev) : zero_f16x8();
  }
}

// One 32-key half (keys key0 ..) of a tile for one wave of the dQ kernel.
// S^T = K Q^T and dP^T = V dO^T (lane = query, registers = keys in the
// perm32 order), P = exp2(S s log2 e - LSE log2 e), dS = P (dP - delta), and
// dQ^T += K^T dS^T with dS^T straight from the registers as the B operand.
// KIND as in the forward: kFull unmasked, kDiag the fixed triangle, kGeneral
// the limit min(query, T - 1).
template <int D, int KIND, bool DROP>
__device__ __forceinline__ void dq_half(const f16* Ks, const f16* Vs, const f16x8 (&qf)[D / 16],
                                        const f16x8 (&dof)[D / 16], int kb, int k0, int my_q,
                                        int T, int l32, int hf, int lane, float sl2, float lse2,
                                        float ndel, float zs, const Dropout& drop, int head,
                                        f32x16 (&acc)[D / 32]) {
  constexpr int kRow = row_of<D>();
  const int arow = (kb * 32 + perm32(l32)) * kRow + 8 * hf;
  f32x16 s, dp;
#pragma unroll
  for (int r = 0; r < 16; ++r) {
    s[r] = 0.f;
    dp[r] = DROP ? 0.f : ndel;  // without dropout the chain ends at dP - delta
  }
#pragma unroll
  for (int kk = 0; kk < D / 16; ++kk) {
    s = mfma32x32x16_f16(*reinterpret_cast<const f16x8*>(&Ks[arow + kk * 16]), qf[kk], s);
    dp = mfma32x32x16_f16(*reinterpret_cast<const f16x8*>(&Vs[arow + kk * 16]), dof[kk], dp);
  }
  // Register 8c + t of half hf holds key k0 + 32kb + 16c + 8hf + t.
  const int lim = min(my_q, T - 1) - (k0 + 32 * kb) - 8 * hf;
#pragma unroll
  for (int c = 0; c < 2; ++c) {
    uint32_t m[4] = {0xffffffffu, 0xffffffffu, 0xffffffffu, 0xffffffffu};
    if (DROP)
      keep_mask8(drop, (uint32_t)head, (uint32_t)my_q,
                 (uint32_t)((k0 + 32 * kb + 16 * c) >> 3) + hf, m);
    float ds[8];
#pragma unroll
    for (int t = 0; t < 8; ++t) {
      const int r = 8 * c + t;
      float p = fast_exp2(fmaf(s[r], sl2, -lse2));
      if (KIND == kDiag) p = (16 * c + t > l32 - 8 * hf) ? 0.f : p;
      if (KIND == kGeneral) p = (16 * c + t > lim) ? 0.f : p;
      if (DROP) {
        const bool kept = (m[t >> 1] >> (16 * (t & 1))) & 1u;
        ds[t] = p * ((kept ? dp[r] * zs : 0.f) + ndel);
      } else {
        ds[t] = p * dp[r];
      }
    }
    const f16x8 dsf = pack_f16x8(ds[0], ds[1], ds[2], ds[3], ds[4], ds[5], ds[6], ds[7]);
    const int ks = 2 * kb + c;  // 16-key step inside the tile
#pragma unroll
    for (int db = 0; db < D / 32; ++db)
      acc[db] = mfma32x32x16_f16(lds_operand_tr(Ks, kRow, ks * 16, db * 32, lane), dsf, acc[db]);
  }
}

// dQ for one workgroup of 128 queries (4 waves x 32, one statistics chunk):
// the forward's loop over 64-key tiles up to the diagonal, with P taken
// exactly from the saved LSE. One wave per SIMD: the dQ accumulators and the
// Q and dO operands (128 registers) next to the tile's products exceed what
// two waves per SIMD can hold. Exponents: Q, dO and delta from this chunk's
// statistics, K and V from the chunks of every key visited (written by the
// dK/dV kernel), dO's from the dS bound.
template <typename TIn, int D, bool DROP>
__global__ __launch_bounds__(kSplitThreads, 1) void attn_bwd_dq_kernel(const BwdArgs a,
                                                                      int n_qtiles, float scale,
                                                                      float scale_log2) {
  typedef typename In16<TIn>::vec vec;
  constexpr int kRow = row_of<D>();
  constexpr int kBN = 64;
  // Two K/V buffers, fp16 [key][d]. In the prologue the Q rows (buffer 0)
  // and dO rows (buffer 1), 128 x D each, pass through them.
  __shared__ __attribute__((aligned(16))) f16 lds[2][2 * kBN * kRow];
  static_assert(kSplitQueries * kRow <= 2 * kBN * kRow, "Q / dO rows fit one buffer");

  const int T = a.T;
  const TileMap tm = map_tile_xcd(blockIdx.x, a.n_heads, n_qtiles, true);
  if (!tm.valid) return;
  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int hf = lane >> 5, l32 = lane & 31;

  const size_t roff = (size_t)tm.head * (size_t)T;
  const TIn* __restrict__ qh = static_cast<const TIn*>(a.q) + head_base(a.lq, tm.head, a.H);
  const TIn* __restrict__ kh = static_cast<const TIn*>(a.k) + head_base(a.lk, tm.head, a.H);
  const TIn* __restrict__ vh = static_cast<const TIn*>(a.v) + head_base(a.lv, tm.head, a.H);
  const TIn* __restrict__ doh = static_cast<const TIn*>(a.dout) + head_base(a.ldo, tm.head, a.H);
  const int ldq = (int)a.lq.t, ldk = (int)a.lk.t, ldv = (int)a.lv.t, lddo = (int)a.ldo.t;

  const int q0 = tm.tile * kSplitQueries;
  const int qw0 = q0 + wave * 32;
  const int my_q = qw0 + l32;

  // Issue the first K/V tile and this workgroup's Q and dO rows.
  KVTile<TIn, D> nxt;
  dq_load_kv<TIn, D>(kh, ldk, vh, ldv, 0, T, tid, nxt);
  constexpr int kC = D / 8, kNQ = kSplitQueries * D / 8 / kSplitThreads;
  vec xq[kNQ], xd[kNQ];
#pragma unroll
  for (int p = 0; p < kNQ; ++p) {
    const int c = tid + kSplitThreads * p;
    const int row = min(q0 + c / kC, T - 1);
    xq[p] = *reinterpret_cast<const vec*>(qh + row * ldq + (c % kC) * 8);
    xd[p] = *reinterpret_cast<const vec*>(doh + row * lddo + (c % kC) * 8);
  }
  const float lse2 = my_q < T ? a.lse[roff + my_q] * kLog2e : 0.f;
  const float del = my_q < T ? a.delta[roff + my_q] : 0.f;

  // Exponents.
  const int n_chunks = (T + kStatRows - 1) / kStatRows;
  const f32x4* st =
      reinterpret_cast<const f32x4*>(a.stats) + (size_t)tm.head * n_chunks * (kStatFloats / 4);
  const f32x4 own = st[(q0 / kStatRows) * (kStatFloats / 4)];
  float mk = 0.f, mv = 0.f;
  for (int c = lane; c <= q0 / kStatRows; c += 64) {
    const f32x4 x = st[c * (kStatFloats / 4) + 1];
    mk = fmaxf(mk, x[0]);
    mv = fmaxf(mv, x[1]);
  }
  mk = wave_max(mk);
  mv = wave_max(mv);
  const float zs = DROP ? a.drop.scale : 1.f;
  const int ek = __builtin_amdgcn_readfirstlane(block_exp(mk, 13));
  const int ev = __builtin_amdgcn_readfirstlane(block_exp(mv, 0));
  const int eq = __builtin_amdgcn_readfirstlane(block_exp(own[0], 13));
  const int edo = __builtin_amdgcn_readfirstlane(dout_exp(own[1], own[2], mv, ev, zs, D));
  const float sl2 = ldexpf(scale_log2, -(eq + ek));
  const float ndel = -ldexpf(del, edo + ev);

  // Q and dO rows into LDS (fp16, scaled), then each wave's fragments: lane
  // holds dims 16kk + 8hf .. +7 of its query (the B operands of S^T, dP^T).
  f16* Qs = lds[0];
  f16* dOs = lds[1];
#pragma unroll
  for (int p = 0; p < kNQ; ++p) {
    const int c = tid + kSplitThreads * p;
    const int row = c / kC, col = (c % kC) * 8;
    const bool ok = q0 + row < T;
    *reinterpret_cast<f16x8*>(&Qs[row * kRow + col]) =
        ok ? cvt_f16_scaled(xq[p], eq) : zero_f16x8();
    *reinterpret_cast<f16x8*>(&dOs[row * kRow + col]) =
        ok ? cvt_f16_scaled(xd[p], edo) : zero_f16x8();
  }
  __syncthreads();
  f16x8 qf[D / 16], dof[D / 16];
#pragma unroll
  for (int kk = 0; kk < D / 16; ++kk) {
    qf[kk] = *reinterpret_cast<const f16x8*>(&Qs[(wave * 32 + l32) * kRow + kk * 16 + 8 * hf]);
    dof[kk] = *reinterpret_cast<const f16x8*>(&dOs[(wave * 32 + l32) * kRow + kk * 16 + 8 * hf]);
  }
  __syncthreads();  // every wave holds its fragments: both buffers are free

  f32x16 acc[D / 32];
#pragma unroll
  for (int db = 0; db < D / 32; ++db)
#pragma unroll
    for (int r = 0; r < 16; ++r) acc[db][r] = 0.f;

  auto Kb = [&](int b) { return lds[b]; };
  auto Vb = [&](int b) { return lds[b] + kBN * kRow; };
  dq_store_kv<TIn, D>(Kb(0), Vb(0), nxt, 0, T, tid, ek, ev);
  __syncthreads();

  const int kv_end = min(T, q0 + kSplitQueries);
  const int n_kt = (kv_end + kBN - 1) / kBN;
  int buf = 0;
  for (int kt = 0; kt < n_kt; ++kt, buf ^= 1) {
    const int k0 = kt * kBN;
    const bool has_next = kt + 1 < n_kt;
    if (has_next) dq_load_kv<TIn, D>(kh, ldk, vh, ldv, k0 + kBN, T, tid, nxt);
#pragma unroll
    for (int kb = 0; kb < 2; ++kb) {
      const int kind = block_kind(k0 + 32 * kb, qw0, T);
      if (kind == kFull)
        dq_half<D, kFull, DROP>(Kb(buf), Vb(buf), qf, dof, kb, k0, my_q, T, l32, hf, lane, sl2,
                                lse2, ndel, zs, a.drop, tm.head, acc);
      else if (kind == kDiag)
        dq_half<D, kDiag, DROP>(Kb(buf), Vb(buf), qf, dof, kb, k0, my_q, T, l32, hf, lane, sl2,
                                lse2, ndel, zs, a.drop, tm.head, acc);
      else if (kind == kGeneral)
        dq_half<D, kGeneral, DROP>(Kb(buf), Vb(buf), qf, dof, kb, k0, my_q, T, l32, hf, lane,
                                   sl2, lse2, ndel, zs, a.drop, tm.head, acc);
    }
    extra_barrier();
    if (has_next) dq_store_kv<TIn, D>(Kb(buf ^ 1), Vb(buf ^ 1), nxt, k0 + kBN, T, tid, ek, ev);
    __syncthreads();
  }

  // dQ = s dQ_acc 2^-(edo + ev + ek), whole rows through LDS (both K/V
  // buffers are free after the loop's last barrier).
  constexpr int kEp = D + 4;
  static_assert(sizeof(lds) >= kSplitWaves * 32 * kEp * sizeof(float), "staging fits");
  float* stage = reinterpret_cast<float*>(&lds[0][0]) + wave * 32 * kEp;
  store_rows<D>(stage, acc, scale, -(edo + ev + ek), a.dq + head_base(a.ldq, tm.head, a.H),
                (int)a.ldq.t, qw0, T, l32, hf, lane);
}

template <typename TIn, int D>
hipError_t launch_prep(const BwdArgs& a_in, hipStream_t stream) {
  BwdArgs a = a_in;
  if (!bwd_dq_atomic(D)) a.dq = nullptr;  // dQ is written, not accumulated
  const int n_chunks = (int)bwd_stat_chunks(a.T);
  const unsigned blocks = (unsigned)a.n_heads * (unsigned)n_chunks;
  hipLaunchKernelGGL((attn_bwd_prep_kernel<TIn, D>), dim3(blocks), dim3(256), 0, stream, a,
                     n_chunks);
  return hipGetLastError();
}

template <typename TIn, int D>
hipError_t launch_split(const BwdArgs& a, hipStream_t stream) {
  const int n_tiles = (a.T + kStatRows - 1) / kStatRows;
  const float scale = 1.f / __builtin_sqrtf((float)D);
  const dim3 grid(tiled_grid(a.n_heads, n_tiles));
  if (a.drop.thr != 0)
    hipLaunchKernelGGL((attn_bwd_dkdv_kernel<TIn, D, true>), grid, dim3(kSplitThreads), 0, stream,
                       a, n_tiles, scale, scale * kLog2e);
  else
    hipLaunchKernelGGL((attn_bwd_dkdv_kernel<TIn, D, false>), grid, dim3(kSplitThreads), 0,
                       stream, a, n_tiles, scale, scale * kLog2e);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  if (a.drop.thr != 0)
    hipLaunchKernelGGL((attn_bwd_dq_kernel<TIn, D, true>), grid, dim3(kSplitThreads), 0, stream,
                       a, n_tiles, scale, scale * kLog2e);
  else
    hipLaunchKernelGGL((attn_bwd_dq_kernel<TIn, D, false>), grid, dim3(kSplitThreads), 0, stream,
                       a, n_tiles, scale, scale * kLog2e);
  return hipGetLastError();
}

template <typename TIn, int D>
hipError_t launch_main(const BwdArgs& a, hipStream_t stream) {
  if constexpr (D >= 128) {
    return launch_split<TIn, D>(a, stream);
  } else {
    const int n_ktiles = (a.T + kBK - 1) / kBK;
    const float scale = 1.f / __builtin_sqrtf((float)D);
    const dim3 grid(tiled_grid(a.n_heads, n_ktiles));
    if (a.drop.thr != 0)
      hipLaunchKernelGGL((attn_bwd_main_kernel<TIn, D, true>), grid, dim3(kThreads), 0, stream,
                         a, n_ktiles, scale, scale * kLog2e);
    else
      hipLaunchKernelGGL((attn_bwd_main_kernel<TIn, D, false>), grid, dim3(kThreads), 0, stream,
                         a, n_ktiles, scale, scale * kLog2e);
    return hipGetLastError();
  }
}

}  // namespace

template <typename TIn>
hipError_t launch_prep_d(const BwdArgs& a, int D, hipStream_t stream) {
  return D == 32   ? launch_prep<TIn, 32>(a, stream)
         : D == 64 ? launch_prep<TIn, 64>(a, stream)
                   : launch_prep<TIn, 128>(a, stream);
}

template <typename TIn>
hipError_t launch_main_d(const BwdArgs& a, int D, hipStream_t stream) {
  return D == 32   ? launch_main<TIn, 32>(a, stream)
         : D == 64 ? launch_main<TIn, 64>(a, stream)
                   : launch_main<TIn, 128>(a, stream);
}

hipError_t launch_bwd_prep_16(const BwdArgs& a, bool fp16, int D, hipStream_t stream) {
  return fp16 ? launch_prep_d<f16>(a, D, stream) : launch_prep_d<bf16>(a, D, stream);
}

hipError_t launch_bwd_main_16(const BwdArgs& a, bool fp16, int D, hipStream_t stream) {
  return fp16 ? launch_main_d<f16>(a, D, stream) : launch_main_d<bf16>(a, D, stream);
}

}  // namespace gpt_attn
