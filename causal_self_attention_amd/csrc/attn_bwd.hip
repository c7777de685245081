// Causal attention backward, bf16 or fp16 inputs, fp32 accumulation and fp32
// gradients, head dim D in {32, 64}, for gfx950 (CDNA4).
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
// when the forward kept it, which restores fp32 accuracy) and zeroes dQ.
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

// D/8 threads per (head, row), 8 elements each: row r of the flattened
// [B*H, T] index space is head r / T, position r % T. Each thread takes
// kPrepRows rows (a block covers kPrepRows consecutive runs of 256/(D/8)
// rows) and issues all of their loads before using any, which keeps more
// bytes in flight per thread than one row would; rows past the end are
// clamped for the loads and skipped for the stores.
constexpr int kPrepRows = 4;

template <typename TIn, int D>
__global__ __launch_bounds__(256) void attn_bwd_prep_kernel(const BwdArgs a, int rows) {
  typedef typename In16<TIn>::vec vec;
  constexpr int kTPR = D / 8, kRPB = 256 / kTPR;  // threads per row, rows per pass
  const int part = threadIdx.x % kTPR;
  const long long row0 = (long long)blockIdx.x * (kRPB * kPrepRows) + threadIdx.x / kTPR;
  vec x[kPrepRows], y[kPrepRows], c[kPrepRows];
  int hd[kPrepRows], t[kPrepRows];
#pragma unroll
  for (int i = 0; i < kPrepRows; ++i) {
    const int row = (int)min(row0 + (long long)i * kRPB, (long long)rows - 1);  // rows < 2^31
    hd[i] = row / a.T;
    t[i] = row - hd[i] * a.T;
    // Nontemporal loads: each row is read once here. (They measured 2%
    // faster over a whole step, the main kernel's time included, with the
    // step's data not already in the Infinity Cache.)
    x[i] = __builtin_nontemporal_load(reinterpret_cast<const vec*>(
        static_cast<const TIn*>(a.o) + head_base(a.lo, hd[i], a.H) + t[i] * a.lo.t + part * 8));
    y[i] = __builtin_nontemporal_load(reinterpret_cast<const vec*>(
        static_cast<const TIn*>(a.dout) + head_base(a.ldo, hd[i], a.H) + t[i] * a.ldo.t +
        part * 8));
    if (a.o_lo)
      c[i] = __builtin_nontemporal_load(reinterpret_cast<const vec*>(
          static_cast<const TIn*>(a.o_lo) + head_base(a.llo, hd[i], a.H) + t[i] * a.llo.t +
          part * 8));
  }
#pragma unroll
  for (int i = 0; i < kPrepRows; ++i) {
    const long long row = row0 + (long long)i * kRPB;
    float acc = 0.f;
    if (a.o_lo) {
#pragma unroll
      for (int e = 0; e < 8; ++e) acc = fmaf((float)x[i][e] + (float)c[i][e], (float)y[i][e], acc);
    } else {
#pragma unroll
      for (int e = 0; e < 8; ++e) acc = fmaf((float)x[i][e], (float)y[i][e], acc);
    }
#pragma unroll
    for (int m = 1; m < kTPR; m <<= 1) acc += __shfl_xor(acc, m, 64);
    if (row < rows) {
      const f32x4 z = {0.f, 0.f, 0.f, 0.f};
      f32x4* dst = reinterpret_cast<f32x4*>(a.dq + head_base(a.ldq, hd[i], a.H) + t[i] * a.ldq.t +
                                            part * 8);
      dst[0] = z;
      dst[1] = z;
      if (part == 0) a.delta[row] = acc;
    }
  }
}

// Loading a 64-query tile is split in two so the global loads can be issued
// a whole step ahead: bwd_load_tile only issues raw loads (rows clamped to
// T-1, so every address is valid, and nothing is computed from the results);
// bwd_store_tile, a step later, zeroes rows past T, converts to fp16 and
// writes the LDS buffers. Only the 256 threads of waves 4..7 take part (tid
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
                                               int tid) {
  constexpr int kC = D / 8, kRowQ = row_of<D>();
#pragma unroll
  for (int p = 0; p < TileRegs<TIn, D>::kN; ++p) {
    const int c = tid + kLoaders * p;
    const int row = c / kC, col = (c % kC) * 8;
    const bool ok = qs + row < T;
    *reinterpret_cast<f16x8*>(&sQ[row * kRowQ + col]) =
        ok ? In16<TIn>::to_f16(r.q[p]) : zero_f16x8();
    *reinterpret_cast<f16x8*>(&sdO[row * kRowQ + col]) =
        ok ? In16<TIn>::to_f16(r.d[p]) : zero_f16x8();
  }
  if (tid < kBQ) {
    const bool ok = qs + tid < T;
    sL[tid] = ok ? r.lse * kLog2e : 0.f;
    sD[tid] = ok ? -r.del : 0.f;
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

// rows[kw0 + k][d] = mul * acc for the wave's 32 keys k, through the wave's
// LDS staging area (pitch D + 4 floats): register r of block db of lane
// (l32, hf) is key l32, dim 32db + 8(r/4) + 4hf + r%4. Rows at or past T are
// skipped. Wave-local: LDS runs one wave's operations in order.
template <int D>
__device__ __forceinline__ void store_rows(float* stage, const f32x16 (&acc)[D / 32], float mul,
                                           float* rows, int ld, int kw0, int T, int l32, int hf,
                                           int lane) {
  constexpr int kEp = D + 4, kLpr = D / 4, kRpi = 64 / kLpr;
#pragma unroll
  for (int db = 0; db < D / 32; ++db)
#pragma unroll
    for (int g = 0; g < 4; ++g) {
      const f32x4 x = {acc[db][4 * g] * mul, acc[db][4 * g + 1] * mul, acc[db][4 * g + 2] * mul,
                       acc[db][4 * g + 3] * mul};
      *reinterpret_cast<f32x4*>(&stage[l32 * kEp + db * 32 + 8 * g + 4 * hf]) = x;
    }
  __builtin_amdgcn_wave_barrier();
#pragma unroll
  for (int j = 0; j < 32 / kRpi; ++j) {
    const int row = j * kRpi + lane / kLpr, col = (lane % kLpr) * 4;
    if (kw0 + row < T)  // nontemporal: nothing here reads dK, dV again
      __builtin_nontemporal_store(*reinterpret_cast<const f32x4*>(&stage[row * kEp + col]),
                                  reinterpret_cast<f32x4*>(rows + (kw0 + row) * ld + col));
  }
  __builtin_amdgcn_wave_barrier();
}

// dQ[queries qb0.., dims 32db..] += scale * acc for one 32x32 block, with
// atomic adds; register r of lane (l32, hf) is query 8(r/4) + 4hf + r%4, dim
// l32. Rows at or past T are skipped.
__device__ __forceinline__ void add_dq_block(const BwdArgs& a, int head, int qb0, int db, int l32,
                                             int hf, int T, float scale, const f32x16& acc) {
  const int lddq = (int)a.ldq.t;
  float* dqh = a.dq + head_base(a.ldq, head, a.H) + qb0 * lddq + db * 32 + l32;
  if (qb0 + 32 <= T) {
#pragma unroll
    for (int r = 0; r < 16; ++r)
      atomicAdd(dqh + (8 * (r >> 2) + 4 * hf + (r & 3)) * lddq, acc[r] * scale);
  } else {
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      const int qr = 8 * (r >> 2) + 4 * hf + (r & 3);
      if (qb0 + qr < T) atomicAdd(dqh + qr * lddq, acc[r] * scale);
    }
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
  f16x8 vf[D / 16];
#pragma unroll
  for (int kk = 0; kk < D / 16; ++kk)
    vf[kk] = my_key < T ? In16<TIn>::to_f16(vraw[kk]) : zero_f16x8();
#pragma unroll
  for (int p = 0; p < kKP; ++p) {
    constexpr int kC = D / 8;
    const int c = tid + kThreads * p;
    const int row = c / kC, col = (c % kC) * 8;
    *reinterpret_cast<f16x8*>(&sK[row * kRowQ + col]) =
        k0 + row < T ? In16<TIn>::to_f16(kraw[p]) : zero_f16x8();
  }

  f32x16 dvacc[kDB], dkacc[kDB];
#pragma unroll
  for (int db = 0; db < kDB; ++db)
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      dvacc[db][r] = 0.f;
      dkacc[db][r] = 0.f;
    }

  if (loader) bwd_store_tile<TIn, D>(sQ[0], sdO[0], sL[0], sD[0], nxt, k0, T, ltid);
  __syncthreads();

  // The K operands of S = Q K^T (this wave's 32 keys): held in registers
  // without dropout; the dropout build, short of registers, reads them from
  // the staged K tile when used.
  f16x8 kreg[D / 16];
#pragma unroll
  for (int kk = 0; kk < D / 16; ++kk)
    kreg[kk] = DROP ? zero_f16x8()
                    : *reinterpret_cast<const f16x8*>(
                          &sK[(wave * 32 + l32) * kRowQ + kk * 16 + 8 * hf]);
  int buf = 0;
  for (int qs = k0; qs < T; qs += kBQ, buf ^= 1) {
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
          const f16x8 kfr = DROP ? *reinterpret_cast<const f16x8*>(
                                        &sK[(wave * 32 + l32) * kRowQ + kk * 16 + 8 * hf])
                                  : kreg[kk];
          s = mfma32x32x16_f16(*reinterpret_cast<const f16x8*>(&cQ[arow + kk * 16]), kfr, s);
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
        const float zs = DROP ? a.drop.scale : 1.f;
        if (kind == kFull)
          bwd_p_ds<kFull, DROP>(s, dp, cL, cD, mb * 32, qb0, kw0, T, l32, hf, scale_log2, mk, zs,
                                pf, dsf);
        else if (kind == kDiag)
          bwd_p_ds<kDiag, DROP>(s, dp, cL, cD, mb * 32, qb0, kw0, T, l32, hf, scale_log2, mk, zs,
                                pf, dsf);
        else
          bwd_p_ds<kGeneral, DROP>(s, dp, cL, cD, mb * 32, qb0, kw0, T, l32, hf, scale_log2, mk,
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
    if (loader && has_next)
      bwd_store_tile<TIn, D>(sQ[buf ^ 1], sdO[buf ^ 1], sL[buf ^ 1], sD[buf ^ 1], nxt, qs + kBQ,
                             T, ltid);
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
          add_dq_block(a, tm.head, qb0, db, l32, hf, T, scale, acc);
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
      add_dq_block(a, tm.head, qb0, db, l32, hf, T, scale, acc);
    }
    // The next step's dS and partial-sum writes come after its first
    // barrier, which every wave reaches only after the reads above.
  }

  // ---- epilogue: dV = z * dV_acc, dK = s * dK_acc, written as whole rows.
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
  store_rows<D>(stage, dvacc, DROP ? a.drop.scale : 1.f, a.dv + head_base(a.ldv, tm.head, a.H),
                (int)a.ldv.t, kw0, T, l32, hf, lane);
  store_rows<D>(stage, dkacc, scale, a.dk + head_base(a.ldk, tm.head, a.H), (int)a.ldk.t, kw0, T,
                l32, hf, lane);
}

template <typename TIn, int D>
hipError_t launch_prep(const BwdArgs& a, hipStream_t stream) {
  const int rows = a.n_heads * a.T;
  constexpr int kRowsPerBlock = 256 / (D / 8) * kPrepRows;
  const unsigned blocks = (unsigned)(((long long)rows + kRowsPerBlock - 1) / kRowsPerBlock);
  hipLaunchKernelGGL((attn_bwd_prep_kernel<TIn, D>), dim3(blocks), dim3(256), 0, stream, a, rows);
  return hipGetLastError();
}

template <typename TIn, int D>
hipError_t launch_main(const BwdArgs& a, hipStream_t stream) {
  const int n_ktiles = (a.T + kBK - 1) / kBK;
  const float scale = 1.f / __builtin_sqrtf((float)D);
  const dim3 grid(tiled_grid(a.n_heads, n_ktiles));
  if (a.drop.thr != 0)
    hipLaunchKernelGGL((attn_bwd_main_kernel<TIn, D, true>), grid, dim3(kThreads), 0, stream, a,
                       n_ktiles, scale, scale * kLog2e);
  else
    hipLaunchKernelGGL((attn_bwd_main_kernel<TIn, D, false>), grid, dim3(kThreads), 0, stream, a,
                       n_ktiles, scale, scale * kLog2e);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_bwd_prep_16(const BwdArgs& a, bool fp16, int D, hipStream_t stream) {
  if (fp16) return D == 32 ? launch_prep<f16, 32>(a, stream) : launch_prep<f16, 64>(a, stream);
  return D == 32 ? launch_prep<bf16, 32>(a, stream) : launch_prep<bf16, 64>(a, stream);
}

hipError_t launch_bwd_main_16(const BwdArgs& a, bool fp16, int D, hipStream_t stream) {
  if (fp16) return D == 32 ? launch_main<f16, 32>(a, stream) : launch_main<f16, 64>(a, stream);
  return D == 32 ? launch_main<bf16, 32>(a, stream) : launch_main<bf16, 64>(a, stream);
}

}  // namespace gpt_attn
