// Causal attention backward, bf16 inputs, fp32 accumulation and fp32
// gradients, head dim 64, for gfx950 (CDNA4).
//
// The gradient of sum(dO * O) for O = softmax(Q K^T / sqrt(64), causal) V:
// what autograd forms for nanoGPT's loss.backward() through the fused
// attention call (page "nanoGPT: a real GPT in two 300-line files", sections
// 1 "Summary" and 2 "How the code works"). With s = 1/sqrt(64):
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
// head (32 per wave) and keeps their K, V fragments and dK, dV accumulators
// in registers. It walks the 64-query tiles from its diagonal to the end of
// the sequence; each tile of Q and dO is staged once in LDS as row-major fp16
// (waves 4..7 prefetch the next tile a step ahead into a second buffer), and
// the transposed operands (Q^T, dO^T for dK^T += Q^T dS and dV^T += dO^T P)
// come from transposing LDS reads. Per tile each wave recomputes P from the
// saved LSE, forms dS and writes its dS^T rows to LDS; then dQ = dS K over
// the 256 keys is formed as four 32x32 blocks, each split into two key
// halves whose sums meet in LDS, and waves 0..3 add the result into the fp32
// dQ with atomic adds (which the memory side performs; 256 keys per
// workgroup keep their number at T/256 per dQ element).
//
// Precision: S = Q K^T and dP = dO V^T multiply bf16 inputs exactly. The
// three products with a rounded operand (dV += P^T dO, dK += dS^T Q,
// dQ += dS K) use fp16 MFMA: P and dS are rounded to fp16 (11 significant
// bits) and the bf16 Q, K, dO tiles convert to fp16 exactly.
//
// Attention dropout (a separate instantiation) regenerates the forward's
// keep mask M: per 32x32 block each lane draws the Philox blocks of one query
// and 16 keys, writes the 0 / 0xFFFF masks to a per-wave LDS tile, and reads
// them back transposed (ds_read_b64_tr_b16) into its own register order (its
// key, 8 consecutive queries). With z the survivor scale: dV accumulates
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
constexpr int kRowQ = 72;     // padded row of a 64-wide 16-bit LDS tile (144 bytes)
constexpr int kRowM = 40;     // row of a wave's 32 x 32 keep-mask tile (80 bytes)

// Eight threads per (head, row): row r of the flattened [B*H, T] index space
// is head r / T, position r % T.
__global__ __launch_bounds__(256) void attn_bwd_prep_bf16_kernel(const BwdArgs a, int rows) {
  const long long gid = (long long)blockIdx.x * 256 + threadIdx.x;
  const int row = (int)(gid >> 3);  // rows < 2^31
  const int part = (int)(gid & 7);
  float acc = 0.f;
  if (row < rows) {
    const int hd = row / a.T, t = row - hd * a.T;
    const bf16* o = static_cast<const bf16*>(a.o) + head_base(a.lo, hd, a.H) + t * a.lo.t;
    const bf16* dout = static_cast<const bf16*>(a.dout) + head_base(a.ldo, hd, a.H) + t * a.ldo.t;
    const bf16x8 x = *reinterpret_cast<const bf16x8*>(o + part * 8);
    const bf16x8 y = *reinterpret_cast<const bf16x8*>(dout + part * 8);
    if (a.o_lo) {
      const bf16* o_lo =
          static_cast<const bf16*>(a.o_lo) + head_base(a.llo, hd, a.H) + t * a.llo.t;
      const bf16x8 c = *reinterpret_cast<const bf16x8*>(o_lo + part * 8);
#pragma unroll
      for (int i = 0; i < 8; ++i) acc = fmaf((float)x[i] + (float)c[i], (float)y[i], acc);
    } else {
#pragma unroll
      for (int i = 0; i < 8; ++i) acc = fmaf((float)x[i], (float)y[i], acc);
    }
    const f32x4 z = {0.f, 0.f, 0.f, 0.f};
    f32x4* dst = reinterpret_cast<f32x4*>(a.dq + head_base(a.ldq, hd, a.H) + t * a.ldq.t +
                                          part * 8);
    dst[0] = z;
    dst[1] = z;
  }
  acc += __shfl_xor(acc, 1, 64);
  acc += __shfl_xor(acc, 2, 64);
  acc += __shfl_xor(acc, 4, 64);
  if (row < rows && part == 0) a.delta[row] = acc;
}

// Loading a 64-query tile is split in two so the global loads can be issued
// a whole step ahead: bwd_load_tile only issues raw loads (rows clamped to
// T-1, so every address is valid, and nothing is computed from the results);
// bwd_store_tile, a step later, zeroes rows past T, converts to fp16 and
// writes the LDS buffers. Only the 256 threads of waves 4..7 take part (tid
// below is their index 0..255): each moves two 16-byte chunks of Q and of dO
// (row c/8, dims (c%8)*8 for c = tid, tid+256), and those with tid < 64 also
// move the LSE and delta of row tid.
struct TileRegs {
  bf16x8 q[2], d[2];
  float lse, del;
};

__device__ __forceinline__ void bwd_load_tile(const bf16* qh, int ldq, const bf16* doh, int lddo,
                                              const float* lse, const float* delta, int qs, int T,
                                              int tid, TileRegs& r) {
#pragma unroll
  for (int p = 0; p < 2; ++p) {
    const int c = tid + kLoaders * p;
    const int row = min(qs + (c >> 3), T - 1), col = (c & 7) * 8;
    r.q[p] = *reinterpret_cast<const bf16x8*>(qh + row * ldq + col);
    r.d[p] = *reinterpret_cast<const bf16x8*>(doh + row * lddo + col);
  }
  const int row = min(qs + (tid & (kBQ - 1)), T - 1);
  r.lse = lse[row];
  r.del = delta[row];
}

__device__ __forceinline__ void bwd_store_tile(f16* sQ, f16* sdO, float* sL, float* sD,
                                               const TileRegs& r, int qs, int T, int tid) {
#pragma unroll
  for (int p = 0; p < 2; ++p) {
    const int c = tid + kLoaders * p;
    const int row = c >> 3, col = (c & 7) * 8;
    const bool ok = qs + row < T;
    *reinterpret_cast<f16x8*>(&sQ[row * kRowQ + col]) =
        ok ? bf16x8_to_f16x8(r.q[p]) : zero_f16x8();
    *reinterpret_cast<f16x8*>(&sdO[row * kRowQ + col]) =
        ok ? bf16x8_to_f16x8(r.d[p]) : zero_f16x8();
  }
  if (tid < kBQ) {
    const bool ok = qs + tid < T;
    sL[tid] = ok ? r.lse * kLog2e : 0.f;
    sD[tid] = ok ? r.del : 0.f;
  }
}

// P = exp2(S log2(e)/8 - LSE log2(e)) and dS = P (dP - delta) for the 16
// (query, key) pairs of one lane in one 32x32 block, as fp16. Register
// 8c + t of half hf is query q0 + 16c + 8hf + t; the lane's key is key0 + l32.
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
    const f32x4 E0 = *reinterpret_cast<const f32x4*>(&cD[qoff]);
    const f32x4 E1 = *reinterpret_cast<const f32x4*>(&cD[qoff + 4]);
    float p[8], ds[8];
#pragma unroll
    for (int t = 0; t < 8; ++t) {
      const float lse2 = t < 4 ? L0[t] : L1[t - 4];
      const float del = t < 4 ? E0[t] : E1[t - 4];
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
        ds[t] = pv * ((kept ? dp[8 * c + t] * zscale : 0.f) - del);
      } else {
        ds[t] = pv * (dp[8 * c + t] - del);
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

// Row strides inside one head are 32-bit (the host checks T * stride < 2^31);
// head offsets are 64-bit.
template <bool DROP>
__global__ __launch_bounds__(kThreads, 1) void attn_bwd_main_bf16_kernel(const BwdArgs a,
                                                                         int n_ktiles, float scale,
                                                                         float scale_log2) {
  // All tiles fp16, row-major; transposed operands come from lds_operand_tr.
  __shared__ __attribute__((aligned(16))) f16 sK[kBK * kRowQ];          // [key][d]
  __shared__ __attribute__((aligned(16))) f16 sQ[2][kBQ * kRowQ];       // [q][d]
  __shared__ __attribute__((aligned(16))) f16 sdO[2][kBQ * kRowQ];      // [q][d]
  __shared__ __attribute__((aligned(16))) f16 sdS[kBK * kRowQ];         // [key][q]
  __shared__ __attribute__((aligned(16))) float sPart[4][16][64];       // dQ half sums
  __shared__ __attribute__((aligned(16))) float sL[2][kBQ];             // LSE * log2(e)
  __shared__ __attribute__((aligned(16))) float sD[2][kBQ];             // delta
  __shared__ __attribute__((aligned(16))) uint16_t sMask[DROP ? 8 : 1][DROP ? 32 * kRowM : 8];

  const int T = a.T;
  const TileMap tm = map_tile_xcd(blockIdx.x, a.n_heads, n_ktiles, false);
  if (!tm.valid) return;

  const int tid = threadIdx.x;
  const int lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int hf = lane >> 5, l32 = lane & 31;
  // Waves 4..7 load the query tiles; waves 0..3 issue the dQ atomics. No wave
  // does both, so a wait for a prefetched tile never waits on atomics too.
  const bool loader = wave >= 4;
  const int ltid = tid - kLoaders;

  const size_t roff = (size_t)tm.head * (size_t)T;
  const bf16* __restrict__ qh = static_cast<const bf16*>(a.q) + head_base(a.lq, tm.head, a.H);
  const bf16* __restrict__ kh = static_cast<const bf16*>(a.k) + head_base(a.lk, tm.head, a.H);
  const bf16* __restrict__ vh = static_cast<const bf16*>(a.v) + head_base(a.lv, tm.head, a.H);
  const bf16* __restrict__ doh =
      static_cast<const bf16*>(a.dout) + head_base(a.ldo, tm.head, a.H);
  const int ldq = (int)a.lq.t, ldk = (int)a.lk.t, ldv = (int)a.lv.t, lddo = (int)a.ldo.t;
  const float* lseh = a.lse + roff;
  const float* delh = a.delta + roff;

  const int k0 = tm.tile * kBK;
  const int kw0 = k0 + wave * 32;
  const int my_key = kw0 + l32;  // the key column this lane owns

  // K and V of this wave's 32 keys as fp16 B operands (lane: its key, 8 dims).
  f16x8 kf[4], vf[4];
#pragma unroll
  for (int kk = 0; kk < 4; ++kk) {
    kf[kk] = bf16x8_to_f16x8(
        load_bf16x8(kh + my_key * ldk + kk * 16 + 8 * hf, my_key < T));
    vf[kk] = bf16x8_to_f16x8(
        load_bf16x8(vh + my_key * ldv + kk * 16 + 8 * hf, my_key < T));
  }
  // All 256 keys of K, row-major fp16, for the dQ product.
#pragma unroll
  for (int p = 0; p < 4; ++p) {
    const int c = tid + kThreads * p;  // 0..2047: key c/8, 8 dims at (c%8)*8
    const int row = c >> 3, col = (c & 7) * 8;
    *reinterpret_cast<f16x8*>(&sK[row * kRowQ + col]) = bf16x8_to_f16x8(
        load_bf16x8(kh + (k0 + row) * ldk + col, k0 + row < T));
  }

  f32x16 dvacc[2], dkacc[2];
#pragma unroll
  for (int db = 0; db < 2; ++db)
#pragma unroll
    for (int r = 0; r < 16; ++r) {
      dvacc[db][r] = 0.f;
      dkacc[db][r] = 0.f;
    }

  TileRegs nxt;
  if (loader) {
    bwd_load_tile(qh, ldq, doh, lddo, lseh, delh, k0, T, ltid, nxt);
    bwd_store_tile(sQ[0], sdO[0], sL[0], sD[0], nxt, k0, T, ltid);
  }
  __syncthreads();

  int buf = 0;
  for (int qs = k0; qs < T; qs += kBQ, buf ^= 1) {
    // Prefetch the next tile into registers while this one is computed.
    const bool has_next = qs + kBQ < T;
    if (loader && has_next) bwd_load_tile(qh, ldq, doh, lddo, lseh, delh, qs + kBQ, T, ltid, nxt);

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
          // Philox blocks) into row L/2 of the wave's tile [query][key].
          uint16_t* tile = sMask[wave];
          uint32_t m0[4], m1[4];
          const uint32_t grp = (uint32_t)(kw0 >> 3) + 2u * (uint32_t)(lane & 1);
          keep_mask8(a.drop, (uint32_t)tm.head, (uint32_t)(qb0 + (lane >> 1)), grp, m0);
          keep_mask8(a.drop, (uint32_t)tm.head, (uint32_t)(qb0 + (lane >> 1)), grp + 1, m1);
          i32x4* dst = reinterpret_cast<i32x4*>(tile + (lane >> 1) * kRowM + 16 * (lane & 1));
          dst[0] = i32x4{(int)m0[0], (int)m0[1], (int)m0[2], (int)m0[3]};
          dst[1] = i32x4{(int)m1[0], (int)m1[1], (int)m1[2], (int)m1[3]};
          __builtin_amdgcn_wave_barrier();
        }
        f32x16 s, dp;
#pragma unroll
        for (int r = 0; r < 16; ++r) {
          s[r] = 0.f;
          dp[r] = 0.f;
        }
        const int arow = (mb * 32 + perm32(l32)) * kRowQ + 8 * hf;
#pragma unroll
        for (int kk = 0; kk < 4; ++kk) {
          s = mfma32x32x16_f16(*reinterpret_cast<const f16x8*>(&cQ[arow + kk * 16]), kf[kk], s);
          dp = mfma32x32x16_f16(*reinterpret_cast<const f16x8*>(&cdO[arow + kk * 16]), vf[kk],
                                dp);
        }
        if (DROP) {
          // Lane (key l32, half hf): queries 16c + 8hf .. +7 of its key.
          const f16* tile = reinterpret_cast<const f16*>(sMask[wave]);
#pragma unroll
          for (int c = 0; c < 2; ++c) mk[c] = lds_operand_tr(tile, kRowM, 16 * c, 0, lane);
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
        *reinterpret_cast<f16x8*>(&sdS[(wave * 32 + l32) * kRowQ + mb * 32 + 16 * c + 8 * hf]) =
            dsf[c];
        // dV^T += dO^T P and dK^T += Q^T dS over these 16 queries.
        const int ks = 2 * mb + c;
#pragma unroll
        for (int db = 0; db < 2; ++db) {
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
      bwd_store_tile(sQ[buf ^ 1], sdO[buf ^ 1], sL[buf ^ 1], sD[buf ^ 1], nxt, qs + kBQ, T, ltid);
    __syncthreads();

    // dQ of the 64-query tile = dS K over the 256 keys, as four 32x32 blocks
    // (queries 32qb.., dims 32db..). Wave w takes block w % 4 over key half
    // w / 4 (8 steps of 16 keys); waves 4..7 pass their half sums to waves
    // 0..3 through LDS, which add them into dQ with atomics. Every wave wrote
    // its dS rows (zeros where nothing is visible).
    const int blk = wave & 3, khalf = wave >> 2;
    const int qb = blk >> 1, db = blk & 1;
    const int qb0 = qs + qb * 32;
    f32x16 acc;
#pragma unroll
    for (int r = 0; r < 16; ++r) acc[r] = 0.f;
    if (qb0 < T) {
#pragma unroll
      for (int j = 0; j < 8; ++j) {
        const int ks = 8 * khalf + j;
        acc = mfma32x32x16_f16(lds_operand_tr(sdS, kRowQ, ks * 16, qb * 32, lane),
                               lds_operand_tr(sK, kRowQ, ks * 16, db * 32, lane), acc);
      }
      if (khalf == 1) {
#pragma unroll
        for (int r = 0; r < 16; ++r) sPart[blk][r][lane] = acc[r];
      }
    }
    __syncthreads();
    if (khalf == 0 && qb0 < T) {
#pragma unroll
      for (int r = 0; r < 16; ++r) acc[r] += sPart[blk][r][lane];
      const int lddq = (int)a.ldq.t;
      float* dqh = a.dq + head_base(a.ldq, tm.head, a.H) + qb0 * lddq + db * 32 + l32;
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
    // The next step's dS and half-sum writes come after its first barrier,
    // which every wave reaches only after the reads above.
  }

  // ---- epilogue: dV, dK = s * acc (lane: its key; 4 consecutive dims per store)
  if (my_key < T) {
    float* dvr = a.dv + head_base(a.ldv, tm.head, a.H) + my_key * a.ldv.t;
    float* dkr = a.dk + head_base(a.ldk, tm.head, a.H) + my_key * a.ldk.t;
#pragma unroll
    for (int db2 = 0; db2 < 2; ++db2)
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        const int d = db2 * 32 + 8 * g + 4 * hf;
        const float zs = DROP ? a.drop.scale : 1.f;
        f32x4 x = {dvacc[db2][4 * g] * zs, dvacc[db2][4 * g + 1] * zs, dvacc[db2][4 * g + 2] * zs,
                   dvacc[db2][4 * g + 3] * zs};
        f32x4 y = {dkacc[db2][4 * g] * scale, dkacc[db2][4 * g + 1] * scale,
                   dkacc[db2][4 * g + 2] * scale, dkacc[db2][4 * g + 3] * scale};
        *reinterpret_cast<f32x4*>(dvr + d) = x;
        *reinterpret_cast<f32x4*>(dkr + d) = y;
      }
  }
}

}  // namespace

hipError_t launch_bwd_prep_bf16(const BwdArgs& a, hipStream_t stream) {
  const int rows = a.n_heads * a.T;
  const unsigned prep_blocks = (unsigned)(((long long)rows * 8 + 255) / 256);
  hipLaunchKernelGGL(attn_bwd_prep_bf16_kernel, dim3(prep_blocks), dim3(256), 0, stream, a, rows);
  return hipGetLastError();
}

hipError_t launch_bwd_main_bf16(const BwdArgs& a, hipStream_t stream) {
  const int n_ktiles = (a.T + kBK - 1) / kBK;
  const float scale = 0.125f;  // 1/sqrt(64)
  const dim3 grid(tiled_grid(a.n_heads, n_ktiles));
  if (a.drop.thr != 0)
    hipLaunchKernelGGL(attn_bwd_main_bf16_kernel<true>, grid, dim3(kThreads), 0, stream, a,
                       n_ktiles, scale, scale * kLog2e);
  else
    hipLaunchKernelGGL(attn_bwd_main_bf16_kernel<false>, grid, dim3(kThreads), 0, stream, a,
                       n_ktiles, scale, scale * kLog2e);
  return hipGetLastError();
}

}  // namespace gpt_attn
