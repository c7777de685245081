/*
 * gpt_attn.h - C ABI of the fused causal self-attention library for AMD
 * Instinct MI355X (gfx950).
 *
 * The operation is the causal multi-head attention at the core of nanoGPT's
 * CausalSelfAttention: PyTorch's fused scaled_dot_product_attention called
 * with is_causal=True, no mask tensor and the default scale (page "nanoGPT: a
 * real GPT in two 300-line files", section 2 "How the code works"), whose
 * written-out equivalent is softmax(Q K^T / sqrt(head size) with the future
 * set to -inf) V. A position attends to itself and earlier positions only
 * (same page, section 8 "Self-check"). The backward is the gradient that
 * autograd computes for it (section 1 "Summary"). The kernels never store the
 * T x T score matrix, which is what the fused kernels are credited with (page
 * "The 300-Line LLM Engine: Inside nanoGPT", section "Flat Architecture and
 * Flash Attention").
 *
 * Conventions shared by every entry point
 *   - Layout: q, k, v, o, dout, dq, dk, dv (and o_lo of the strided calls)
 *     are logically [B, H, T, D].
 *     The plain entry points take them contiguous row-major; the *_strided
 *     ones take a gpt_attn_layout per operand (below), so that q, k, v can be
 *     read straight out of a projection's [B, T, 3C] output and o written
 *     into a [B, T, C] buffer. Per-row statistics (lse, and the delta vector
 *     in the workspace) are always contiguous [B, H, T] fp32.
 *   - Scale: always 1/sqrt(D). Causal masking is always on: key j is visible
 *     to query i iff j <= i. There is no mask or scale argument; attention
 *     dropout is an optional gpt_attn_dropout on the strided calls.
 *   - Pointers are DEVICE pointers (hipMalloc or torch CUDA tensors) and must
 *     be 16-byte aligned. The caller owns every buffer; the library allocates
 *     nothing and keeps no state between calls. Outputs must not alias
 *     inputs or each other.
 *   - stream is a hipStream_t (NULL = the default stream). Calls only enqueue
 *     work and return; results are visible after the caller synchronizes.
 *   - Sizes: B, H, T >= 0; a call with B*H*T == 0 does nothing and returns
 *     GPT_ATTN_OK (pointers are not inspected). D must be 32, 64 or 128
 *     (64 and 32 are the head sizes of the pages' models: 768/12 = 64 for
 *     GPT-2, 128/4 = 32 for the small Shakespeare-char run on a laptop, page
 *     "nanoGPT: a real GPT in two 300-line files", section 3 "Run it,
 *     tested"; 128 is the common head size of larger models). B*H*T must be
 *     below 2^31 and B*H*T*D below 2^40.
 *   - Errors: argument errors are returned before any device work is
 *     enqueued and leave every buffer untouched. GPT_ATTN_E_HIP means the
 *     HIP runtime rejected a launch (hipGetLastError); a fault inside a
 *     kernel surfaces at the caller's next synchronization. No C++
 *     exception crosses this interface.
 *   - Thread safety: calls are reentrant. Concurrent calls on different
 *     streams need distinct output and workspace buffers.
 */
#ifndef GPT_ATTN_H
#define GPT_ATTN_H

#include <stddef.h>

#ifdef __cplusplus
extern "C" {
#endif

#define GPT_ATTN_ABI_VERSION 7

/* Status codes returned by every int-returning entry point. */
enum gpt_attn_status {
  GPT_ATTN_OK = 0,
  GPT_ATTN_E_INVAL = 1,       /* null pointer, negative or overflowing size, bad dtype code,
                                 o_lo given with GPT_ATTN_F32, bad dropout probability */
  GPT_ATTN_E_UNSUPPORTED = 2, /* a head dimension D with no kernel (D not 32, 64 or 128) */
  GPT_ATTN_E_ALIGN = 3,       /* a pointer that is not 16-byte aligned */
  GPT_ATTN_E_WORKSPACE = 4,   /* workspace NULL or smaller than the *_workspace_bytes size */
  GPT_ATTN_E_HIP = 5,         /* the HIP runtime reported an error when launching */
  GPT_ATTN_E_LAYOUT = 6,      /* a gpt_attn_layout breaking the rules below */
  GPT_ATTN_E_TOO_LARGE = 7    /* gpt_attn_bwd_noalloc: workspace beyond its static scratch */
};

/*
 * Element strides of one logically [B, H, T, D] operand whose D elements are
 * contiguous: element (b, h, t, d) is at base[b*batch + h*head + t*row + d].
 * A NULL layout pointer means contiguous [B, H, T, D] (row = D, head = T*D,
 * batch = H*T*D).
 *
 * The causal self-attention layer projects every token to q, k and v with
 * one linear layer and splits the result into heads (page "nanoGPT: a real
 * GPT in two 300-line files", section 2 "How the code works"). With that
 * layer's output qkv of shape [B, T, 3C], C = H*D, the head views are
 *   q: base = qkv,      batch = 3*T*C, head = D, row = 3*C
 *   k: base = qkv + C,  same strides;  v: base = qkv + 2*C, same strides
 * and the merged output y of shape [B, T, C] is batch = T*C, head = D, row = C.
 *
 * Rules (GPT_ATTN_E_LAYOUT otherwise):
 *   - strides are >= 0; those of dimensions with extent > 1 are multiples
 *     of 16 bytes (8 bf16 or 4 fp32 elements), so every row starts 16-byte
 *     aligned given an aligned base pointer;
 *   - (T-1)*row + D fits in a signed 32-bit integer (offsets inside one
 *     head are 32-bit in the kernels), and the whole operand spans below
 *     2^48 elements;
 *   - an output (o, o_lo, dq, dk, dv) does not overlap itself: sorted by
 *     stride (D counting as stride 1, extent D), every stride exceeds the
 *     largest offset the smaller ones reach.
 * Inputs may overlap each other (q, k, v in one buffer). Outputs must not
 * overlap inputs or each other; this is not checked.
 */
typedef struct gpt_attn_layout {
  long long batch;
  long long head;
  long long row;
} gpt_attn_layout;

/*
 * Attention dropout. In training nanoGPT passes its dropout rate to the
 * fused attention call (page "nanoGPT: a real GPT in two 300-line files",
 * section 2 "How the code works"): each attention weight P_ij is zeroed with
 * probability p after the softmax and the survivors are scaled by 1/(1-p),
 * O = (z M o P) V with keep mask M. The mask is never stored: the forward,
 * the backward and gpt_attn_dropout_mask all derive it from the
 * counter-based generator Philox4x32-10 (Salmon et al., "Parallel random
 * numbers: as easy as 1, 2, 3", SC'11) with
 *   key     = (seed & 0xFFFFFFFF, seed >> 32)
 *   counter = (j / 8, i, b*H + h, offset)        for query i, key j
 *   u_ij    = 16-bit field (j % 2) of output word (j % 8) / 2
 *   M_ij    = [u_ij >= thr],  thr = round(p * 65536),  z = 65536 / (65536 - thr)
 * so the drop probability is p rounded to a multiple of 2^-16. A backward
 * must get the same descriptor as its forward. LSE is unaffected by dropout.
 * p must satisfy 0 <= p < 1 with thr < 65536 (GPT_ATTN_E_INVAL otherwise);
 * p = 0 (or a NULL descriptor) means no dropout.
 */
typedef struct gpt_attn_dropout {
  double p;
  unsigned long long seed;
  unsigned int offset;
} gpt_attn_dropout;

/* Element type of q, k, v, o and dout (and of the decode caches). lse, dq,
 * dk, dv are always fp32. The pages' GPU training runs in automatic mixed
 * precision, BF16 or FP16 (page "nanoGPT: Minimal, Readable, and Fast
 * PyTorch Framework for Training Medium GPTs", feature list). */
enum gpt_attn_dtype {
  GPT_ATTN_F32 = 0,  /* IEEE binary32 inputs, fp32 arithmetic throughout */
  GPT_ATTN_BF16 = 1, /* bfloat16 inputs; matrix products accumulate in fp32 */
  GPT_ATTN_F16 = 2   /* IEEE binary16 inputs; matrix products accumulate in fp32 */
};

/*
 * Precision of the 16-bit dtypes. Matrix products run on the gfx950 matrix
 * cores with fp32 accumulation; the softmax statistics, delta and all
 * sums are fp32. Q K^T of the forward multiplies the inputs in their own
 * type. Every other product (P V of the forward, all five of the backward)
 * takes fp16 operands, because the rounded operand (the probabilities P,
 * the score gradient dS) keeps 11 significant bits in fp16 against bf16's
 * 8. fp16's exponent range (normal 2^-14 .. 65504) is not a limit: each
 * operand block is scaled by an exact power of two before the rounding to
 * fp16 and unscaled after the product, the exponent chosen from the block's
 * largest magnitude -- per workgroup for K and V, from the maxima the
 * backward's first phase records for Q, dO and delta, and for the forward's
 * V from the first key tile of each query block, lowered when a later tile
 * would not fit. Power-of-two scaling of an input therefore scales the
 * outputs it enters exactly, over bf16's whole range, as long as no fp32
 * intermediate (the scores Q K^T / sqrt(D), the accumulated sums)
 * overflows or falls below fp32's normal range. Non-finite inputs give
 * non-finite outputs.
 */

/*
 * Forward: O = softmax(Q K^T / sqrt(D), causal) V and the log-sum-exp of
 * each row, LSE_i = ln sum_{j<=i} exp(Q_i . K_j / sqrt(D)) (natural log of
 * the scaled scores).
 *
 *   q, k, v  in   [B,H,T,D] of dtype
 *   o        out  [B,H,T,D] of dtype (16-bit output is rounded to nearest even)
 *   lse      out  [B,H,T] fp32; the backward needs it
 *
 * o, lse are bitwise reproducible run to run.
 */
int gpt_attn_fwd(int dtype, int B, int H, int T, int D, const void* q, const void* k,
                 const void* v, void* o, float* lse, void* stream);

/*
 * Bytes of device workspace the backward needs for this shape, for every
 * dtype: the fp32 vector delta_i = sum_d dO_id O_id, [B,H,T], followed (from
 * the next 16-byte boundary) by 32 bytes per (head, 128-row chunk) of
 * per-chunk maxima the main phase reads. Returns 0 for an invalid or empty
 * shape.
 */
size_t gpt_attn_bwd_workspace_bytes(int B, int H, int T, int D);

/*
 * Backward: the gradient of sum(dout * O) with respect to Q, K and V,
 * computed without the T x T matrix: P is recomputed from q, k and lse, and
 * delta = rowsum(dout * O) is formed first by a separate pass.
 *
 *   q, k, v      in   [B,H,T,D] of dtype (the forward's inputs)
 *   o            in   [B,H,T,D] of dtype (the forward's output)
 *   dout         in   [B,H,T,D] of dtype (upstream gradient dL/dO)
 *   lse          in   [B,H,T] fp32 (the forward's output)
 *   dq, dk, dv   out  [B,H,T,D] fp32, fully overwritten
 *   workspace    scratch of at least gpt_attn_bwd_workspace_bytes(...)
 *                bytes, device memory owned by the caller; contents on entry
 *                are ignored and on return are unspecified.
 *
 * delta is formed from o as stored. For the 16-bit dtypes that is O rounded
 * to the dtype, and the rounding enters dq and dk through delta: with sharp
 * softmax rows (scores of standard deviation 4, keys concentrated on one
 * value row) dq then misses the 2e-2 max-abs bar of bf16 parity. The strided
 * calls below take the forward's optional o_lo, the part of the fp32 O that
 * the rounding dropped, and remove that error.
 *
 * dk, dv are bitwise reproducible run to run. dq is accumulated with fp32
 * atomic adds for the 16-bit dtypes at D = 32 and 64, so its low bits may
 * vary between runs; at D = 128 (two kernels: dk and dv, then dq, each
 * written once) and for fp32 it is reproducible too.
 */
int gpt_attn_bwd(int dtype, int B, int H, int T, int D, const void* q, const void* k,
                 const void* v, const void* o, const void* dout, const float* lse, float* dq,
                 float* dk, float* dv, void* workspace, size_t workspace_bytes, void* stream);

/*
 * The two phases of gpt_attn_bwd as separate calls, for callers that
 * schedule or time them apart. gpt_attn_bwd(...) is exactly
 * gpt_attn_bwd_prep(...) followed by gpt_attn_bwd_main(...) on one stream.
 *
 * gpt_attn_bwd_prep: the preprocess pass. Writes delta_i = sum_d dout_id O_id
 *   into the workspace; for the 16-bit dtypes it also records the largest
 *   |q|, |dout| and |delta| of every 128-row chunk of each head, from which
 *   the main phase sets its operand scales, and at D = 32 and 64 zero-fills
 *   dq, which the main phase accumulates into (q and dq may be NULL for
 *   GPT_ATTN_F32 and are not touched; dq is not touched at D = 128).
 * gpt_attn_bwd_main: everything else. Reads the workspace, which must hold
 *   the prep phase's result for the same q, o and dout (and, for the 16-bit
 *   dtypes at D = 32 and 64, dq must still hold the prep phase's zeros).
 *   Writes dq, dk, dv (and, at D = 128, per-chunk maxima of |k| and |v| into
 *   the workspace). Arguments mean what they mean for gpt_attn_bwd.
 */
int gpt_attn_bwd_prep(int dtype, int B, int H, int T, int D, const void* q, const void* o,
                      const void* dout, float* dq, void* workspace, size_t workspace_bytes,
                      void* stream);
int gpt_attn_bwd_main(int dtype, int B, int H, int T, int D, const void* q, const void* k,
                      const void* v, const void* dout, const float* lse, float* dq, float* dk,
                      float* dv, const void* workspace, size_t workspace_bytes, void* stream);

/*
 * gpt_attn_bwd for callers that cannot allocate device memory: code under
 * HIP graph capture, tight serving loops, harnesses that forbid allocation.
 * Arguments, outputs and errors are gpt_attn_bwd's without the workspace:
 * the library keeps the backward's workspace in a static device array of
 * GPT_ATTN_NOALLOC_SCRATCH_BYTES (8 MiB) per GPU it runs on, held until the
 * process ends. Shapes whose gpt_attn_bwd_workspace_bytes exceeds that
 * (B*H*T beyond about two million rows) return GPT_ATTN_E_TOO_LARGE before
 * any device work. The call allocates nothing; its first call on a device
 * looks up that device's copy of the array (hipGetSymbolAddress) and keeps
 * it. Every call on one GPU shares that GPU's copy, so calls that overlap in
 * time on one GPU (different streams, or host threads) race: serialize
 * them. Nothing in the array needs to start at zero: each call overwrites
 * what it reads.
 */
#define GPT_ATTN_NOALLOC_SCRATCH_BYTES (8u << 20)
int gpt_attn_bwd_noalloc(int dtype, int B, int H, int T, int D, const void* q, const void* k,
                         const void* v, const void* o, const void* dout, const float* lse,
                         float* dq, float* dk, float* dv, void* stream);

/*
 * Strided forms of the four calls above: each operand pointer is followed by
 * its layout (NULL = contiguous [B,H,T,D]). Operand meanings, dtypes,
 * workspace and errors are those of the plain entry points, which are these
 * calls with every layout NULL, no o_lo and no dropout. lse and the
 * workspace stay contiguous. gpt_attn_bwd_main_strided expects dq in the
 * layout the preceding gpt_attn_bwd_prep_strided zero-filled.
 *
 * o_lo (16-bit dtypes only; must be NULL for GPT_ATTN_F32; NULL skips it):
 *   the forward writes into it, in the dtype, round(O - o), the part of the
 *   fp32 result that rounding o to the dtype dropped; the backward and its
 *   prep phase, given it, form delta from o + o_lo, an O accurate to about
 *   twice the dtype's precision. It costs one more [B,H,T,D] tensor written
 *   by the forward and read by the prep phase, and keeps dq within the bf16
 *   bar when softmax rows are sharp (see gpt_attn_bwd).
 * dropout: NULL, or the descriptor above; the forward, gpt_attn_bwd_strided
 *   and gpt_attn_bwd_main_strided take it (the prep phase does not depend on
 *   it: delta = rowsum(dout * O) holds for the dropped output O too).
 */
int gpt_attn_fwd_strided(int dtype, int B, int H, int T, int D, const void* q,
                         const gpt_attn_layout* lq, const void* k, const gpt_attn_layout* lk,
                         const void* v, const gpt_attn_layout* lv, void* o,
                         const gpt_attn_layout* lo, void* o_lo, const gpt_attn_layout* llo,
                         float* lse, const gpt_attn_dropout* dropout, void* stream);
int gpt_attn_bwd_strided(int dtype, int B, int H, int T, int D, const void* q,
                         const gpt_attn_layout* lq, const void* k, const gpt_attn_layout* lk,
                         const void* v, const gpt_attn_layout* lv, const void* o,
                         const gpt_attn_layout* lo, const void* o_lo, const gpt_attn_layout* llo,
                         const void* dout, const gpt_attn_layout* ldo, const float* lse,
                         float* dq, const gpt_attn_layout* ldq, float* dk,
                         const gpt_attn_layout* ldk, float* dv, const gpt_attn_layout* ldv,
                         void* workspace, size_t workspace_bytes,
                         const gpt_attn_dropout* dropout, void* stream);
int gpt_attn_bwd_prep_strided(int dtype, int B, int H, int T, int D, const void* q,
                              const gpt_attn_layout* lq, const void* o, const gpt_attn_layout* lo,
                              const void* o_lo, const gpt_attn_layout* llo, const void* dout,
                              const gpt_attn_layout* ldo, float* dq, const gpt_attn_layout* ldq,
                              void* workspace, size_t workspace_bytes, void* stream);
int gpt_attn_bwd_main_strided(int dtype, int B, int H, int T, int D, const void* q,
                              const gpt_attn_layout* lq, const void* k, const gpt_attn_layout* lk,
                              const void* v, const gpt_attn_layout* lv, const void* dout,
                              const gpt_attn_layout* ldo, const float* lse, float* dq,
                              const gpt_attn_layout* ldq, float* dk, const gpt_attn_layout* ldk,
                              float* dv, const gpt_attn_layout* ldv, const void* workspace,
                              size_t workspace_bytes, const gpt_attn_dropout* dropout,
                              void* stream);

/*
 * The keep mask the kernels derive for a dropout descriptor, written out:
 * mask [B,H,T,T] uint8 (device memory, contiguous), 1 where key j is visible
 * to query i (j <= i) and kept, 0 elsewhere. For inspection and testing; the
 * attention calls never read or write it. GPT_ATTN_E_INVAL for a NULL
 * descriptor, a bad p, negative sizes, B*H*T >= 2^31 or B*H*T*T >= 2^40, or
 * a NULL mask with a non-empty shape.
 */
int gpt_attn_dropout_mask(int B, int H, int T, const gpt_attn_dropout* dropout,
                          unsigned char* mask, void* stream);

/*
 * One query per (sequence, head) against a key/value cache: what sampling
 * needs, since generate() feeds the sequence back one position at a time
 * (page "nanoGPT: a real GPT in two 300-line files", section 2 "How the code
 * works") and the newest query sees every earlier position and its own. With
 * n = lengths[b] cached rows for sequence b this is the last row of the
 * causal forward at T = n:
 *   O   = softmax(q K[0:n]^T / sqrt(D)) V[0:n],   LSE = ln sum_j exp(q.K_j / sqrt(D))
 *
 *   q          in   [B,H,D] of dtype (lq: batch and head strides; row unused)
 *   k_cache,
 *   v_cache    in   [B,H,L,D] of dtype (lk, lv: any gpt_attn_layout); rows at
 *                   and beyond lengths[b] are never read
 *   lengths    in   OPTIONAL device int32 [B]: cached rows per sequence,
 *                   clamped to [0, L]; NULL means L for every sequence. A
 *                   length of 0 gives O = 0 and LSE = -inf.
 *   o          out  [B,H,D] of dtype (lo: batch and head strides)
 *   lse        out  [B,H] fp32, contiguous
 *   workspace  scratch of gpt_attn_decode_workspace_bytes(...) bytes (the
 *              per-chunk partial results), owned by the caller
 *
 * Layout rules, alignment, errors and streams as for the other calls; the
 * shape rules apply to [B,H,L,D] (L may be 0). Arithmetic in fp32 for both
 * dtypes (bf16 inputs are widened exactly).
 */
size_t gpt_attn_decode_workspace_bytes(int dtype, int B, int H, int L, int D);
int gpt_attn_decode(int dtype, int B, int H, int L, int D, const void* q,
                    const gpt_attn_layout* lq, const void* k_cache, const gpt_attn_layout* lk,
                    const void* v_cache, const gpt_attn_layout* lv, const int* lengths, void* o,
                    const gpt_attn_layout* lo, float* lse, void* workspace,
                    size_t workspace_bytes, void* stream);

/* Static, NUL-terminated description of a status code. Never NULL. */
const char* gpt_attn_status_string(int status);

/* GPT_ATTN_ABI_VERSION of the built library. */
int gpt_attn_abi_version(void);

#ifdef __cplusplus
}
#endif

#endif /* GPT_ATTN_H */
