// The C ABI declared in include/gpt_attn.h: argument validation, dispatch
// by dtype, and launch-error reporting. Validation completes before any HIP
// call, so a rejected call touches neither the device nor the HIP runtime.
#include <math.h>
#include <stdint.h>

#include <mutex>

#include "attn_launch.h"
#include "gpt_attn.h"

// Backing store of gpt_attn_bwd_noalloc: the backward's workspace (delta and
// the per-chunk maxima), one copy per GPU that the library runs on, held
// until the process ends. In host code this name is only a handle for
// hipGetSymbolAddress; the device address comes from scratch_address().
static __device__ __align__(256) unsigned char scratch[GPT_ATTN_NOALLOC_SCRATCH_BYTES];

namespace {

using gpt_attn::Layout;

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

struct Shape {
  int dtype, B, H, T, D;
  long long rows;  // B*H*T
  long long esize; // bytes per element of q, k, v, o, dout
};

// Shape and dtype checks shared by every entry point.
int check_shape(int dtype, int B, int H, int T, int D, Shape* s) {
  if (dtype != GPT_ATTN_F32 && dtype != GPT_ATTN_BF16 && dtype != GPT_ATTN_F16)
    return GPT_ATTN_E_INVAL;
  if (B < 0 || H < 0 || T < 0 || D <= 0) return GPT_ATTN_E_INVAL;
  if (D != 32 && D != 64 && D != 128) return GPT_ATTN_E_UNSUPPORTED;
  const long long heads = (long long)B * (long long)H;
  const long long r = heads * (long long)T;
  if (r >= (1LL << 31)) return GPT_ATTN_E_INVAL;
  if (r * (long long)D >= (1LL << 40)) return GPT_ATTN_E_INVAL;
  if (r > 0) {
    // Every launch grid must fit the 32-bit workgroup index: the tiled grids
    // pad the head count to a multiple of 8 and use at least 32-row tiles.
    const long long tiles = ((long long)T + 31) / 32;
    if (8LL * ((heads + 7) / 8) * tiles >= (1LL << 31)) return GPT_ATTN_E_INVAL;
  }
  s->dtype = dtype;
  s->B = B;
  s->H = H;
  s->T = T;
  s->D = D;
  s->rows = r;
  s->esize = dtype == GPT_ATTN_F32 ? 4 : 2;
  return GPT_ATTN_OK;
}

// The layout a descriptor names, or the contiguous [B, H, T, D] one for NULL.
Layout resolve(const gpt_attn_layout* l, const Shape& s) {
  if (!l) {
    const long long row = s.D, head = row * s.T, batch = head * s.H;
    return Layout{batch, head, row};
  }
  return Layout{l->batch, l->head, l->row};
}

// Checks one operand's layout (see the header for the rules). esize is the
// operand's element size in bytes; output operands must not overlap
// themselves.
int check_layout(const Layout& L, const Shape& s, long long esize, bool output) {
  const long long st[3] = {L.b, L.h, L.t};
  const long long ext[3] = {s.B, s.H, s.T};
  const long long unit = 16 / esize;  // elements per 16 bytes
  __int128 span = s.D;                // elements from the first to past the last
  for (int i = 0; i < 3; ++i) {
    if (st[i] < 0) return GPT_ATTN_E_LAYOUT;
    if (ext[i] > 1) {
      if (st[i] % unit != 0) return GPT_ATTN_E_LAYOUT;
      span += (__int128)st[i] * (ext[i] - 1);
    }
  }
  if (span >= ((__int128)1 << 48)) return GPT_ATTN_E_LAYOUT;
  // The kernels address rows inside one head with 32-bit offsets.
  if ((long long)(s.T - 1) * L.t + s.D > INT32_MAX) return GPT_ATTN_E_LAYOUT;
  if (output) {
    // Sufficient condition for distinct addresses: with the dimensions of
    // extent > 1 sorted by stride (D first: stride 1, extent D), each stride
    // exceeds the largest offset the smaller ones reach.
    long long ds[4] = {1, 0, 0, 0}, de[4] = {s.D, 0, 0, 0};
    int n = 1;
    for (int i = 0; i < 3; ++i)
      if (ext[i] > 1) {
        ds[n] = st[i];
        de[n] = ext[i];
        ++n;
      }
    for (int i = 1; i < n; ++i)
      for (int j = i; j > 0 && ds[j] < ds[j - 1]; --j) {
        const long long a = ds[j], b = de[j];
        ds[j] = ds[j - 1];
        de[j] = de[j - 1];
        ds[j - 1] = a;
        de[j - 1] = b;
      }
    __int128 reach = 0;
    for (int i = 0; i < n; ++i) {
      if ((__int128)ds[i] <= reach) return GPT_ATTN_E_LAYOUT;
      reach += (__int128)ds[i] * (de[i] - 1);
    }
  }
  return GPT_ATTN_OK;
}

int launch_status(hipError_t e) { return e == hipSuccess ? GPT_ATTN_OK : GPT_ATTN_E_HIP; }

// Dropout descriptor -> kernel parameters (thr = 0 when d is NULL or p = 0).
int resolve_dropout(const gpt_attn_dropout* d, gpt_attn::Dropout* out) {
  *out = gpt_attn::Dropout{0u, 1.f, 0u, 0u, 0u};
  if (!d) return GPT_ATTN_OK;
  if (!(d->p >= 0.0 && d->p < 1.0)) return GPT_ATTN_E_INVAL;
  const double thr = floor(d->p * 65536.0 + 0.5);
  if (thr >= 65536.0) return GPT_ATTN_E_INVAL;
  out->thr = (uint32_t)thr;
  out->scale = (float)(65536.0 / (65536.0 - thr));
  out->key0 = (uint32_t)(d->seed & 0xFFFFFFFFull);
  out->key1 = (uint32_t)(d->seed >> 32);
  out->offset = d->offset;
  return GPT_ATTN_OK;
}

#define GA_TRY(expr)                       \
  do {                                     \
    const int st_ = (expr);                \
    if (st_ != GPT_ATTN_OK) return st_;    \
  } while (0)

int check_workspace(const void* workspace, size_t bytes, const Shape& s) {
  if (!workspace || bytes < (size_t)gpt_attn::bwd_workspace_bytes((long long)s.B * s.H, s.T))
    return GPT_ATTN_E_WORKSPACE;
  if (!aligned16(workspace)) return GPT_ATTN_E_ALIGN;
  return GPT_ATTN_OK;
}

// Validated arguments of the backward phases. which: 1 = prep, 2 = main,
// 3 = both.
int bwd_args(const Shape& s, int which, const void* q, const gpt_attn_layout* lq, const void* k,
             const gpt_attn_layout* lk, const void* v, const gpt_attn_layout* lv, const void* o,
             const gpt_attn_layout* lo, const void* o_lo, const gpt_attn_layout* llo,
             const void* dout, const gpt_attn_layout* ldo, const float* lse, float* dq,
             const gpt_attn_layout* ldq, float* dk, const gpt_attn_layout* ldk, float* dv,
             const gpt_attn_layout* ldv, const void* workspace, size_t workspace_bytes,
             const gpt_attn_dropout* dropout, gpt_attn::BwdArgs* a) {
  const bool prep = which & 1, main = which & 2;
  const bool half = s.dtype != GPT_ATTN_F32;  // 16-bit inputs: dQ by atomics, o_lo allowed
  if (!dout) return GPT_ATTN_E_INVAL;
  if (prep && (!o || (half && (!dq || !q)))) return GPT_ATTN_E_INVAL;
  if (main && (!q || !k || !v || !lse || !dq || !dk || !dv)) return GPT_ATTN_E_INVAL;
  if (o_lo && !half) return GPT_ATTN_E_INVAL;
  if (!aligned16(q) || !aligned16(k) || !aligned16(v) || !aligned16(o) || !aligned16(o_lo) ||
      !aligned16(dout) || !aligned16(lse) || !aligned16(dq) || !aligned16(dk) || !aligned16(dv))
    return GPT_ATTN_E_ALIGN;
  a->q = q;
  a->k = k;
  a->v = v;
  a->o = o;
  a->o_lo = prep ? o_lo : nullptr;
  a->dout = dout;
  a->lse = lse;
  a->delta = static_cast<float*>(const_cast<void*>(workspace));
  a->stats = reinterpret_cast<float*>(static_cast<char*>(const_cast<void*>(workspace)) +
                                      gpt_attn::bwd_stats_offset_bytes(s.rows));
  a->dq = dq;
  a->dk = dk;
  a->dv = dv;
  a->lq = resolve(lq, s);
  a->lk = resolve(lk, s);
  a->lv = resolve(lv, s);
  a->lo = resolve(lo, s);
  a->llo = resolve(llo, s);
  a->ldo = resolve(ldo, s);
  a->ldq = resolve(ldq, s);
  a->ldk = resolve(ldk, s);
  a->ldv = resolve(ldv, s);
  GA_TRY(check_layout(a->ldo, s, s.esize, false));
  if (prep) {
    if (half) GA_TRY(check_layout(a->lq, s, s.esize, false));
    GA_TRY(check_layout(a->lo, s, s.esize, false));
    if (o_lo) GA_TRY(check_layout(a->llo, s, 2, false));
  }
  if (prep || main) {
    if (dq) GA_TRY(check_layout(a->ldq, s, 4, true));
  }
  if (main) {
    GA_TRY(check_layout(a->lq, s, s.esize, false));
    GA_TRY(check_layout(a->lk, s, s.esize, false));
    GA_TRY(check_layout(a->lv, s, s.esize, false));
    GA_TRY(check_layout(a->ldk, s, 4, true));
    GA_TRY(check_layout(a->ldv, s, 4, true));
  }
  GA_TRY(resolve_dropout(main ? dropout : nullptr, &a->drop));
  GA_TRY(check_workspace(workspace, workspace_bytes, s));
  a->n_heads = s.B * s.H;
  a->H = s.H;
  a->T = s.T;
  return GPT_ATTN_OK;
}

int run_prep(const Shape& s, const gpt_attn::BwdArgs& a, hipStream_t st) {
  return launch_status(s.dtype == GPT_ATTN_F32
                           ? gpt_attn::launch_bwd_prep_f32(a, s.D, st)
                           : gpt_attn::launch_bwd_prep_16(a, s.dtype == GPT_ATTN_F16, s.D, st));
}

// Device address of `scratch` on the device that runs `stream` (the current
// device for the null stream), looked up once per device with that device
// current and kept.
constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch_ptr[kMaxDevices];

int scratch_address(hipStream_t stream, void** out) {
  int cur = 0, dev = 0;
  if (hipGetDevice(&cur) != hipSuccess) return GPT_ATTN_E_HIP;
  dev = cur;
  if (stream && hipStreamGetDevice(stream, &dev) != hipSuccess) return GPT_ATTN_E_HIP;
  if (dev < 0 || dev >= kMaxDevices) return GPT_ATTN_E_HIP;
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (!g_scratch_ptr[dev]) {
    if (dev != cur && hipSetDevice(dev) != hipSuccess) return GPT_ATTN_E_HIP;
    void* p = nullptr;
    const hipError_t e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (dev != cur && hipSetDevice(cur) != hipSuccess) return GPT_ATTN_E_HIP;
    if (e != hipSuccess || !p) return GPT_ATTN_E_HIP;
    g_scratch_ptr[dev] = p;
  }
  *out = g_scratch_ptr[dev];
  return GPT_ATTN_OK;
}

int run_main(const Shape& s, const gpt_attn::BwdArgs& a, hipStream_t st) {
  return launch_status(s.dtype == GPT_ATTN_F32
                           ? gpt_attn::launch_bwd_main_f32(a, s.D, st)
                           : gpt_attn::launch_bwd_main_16(a, s.dtype == GPT_ATTN_F16, s.D, st));
}

}  // namespace

extern "C" {

int gpt_attn_abi_version(void) { return GPT_ATTN_ABI_VERSION; }

const char* gpt_attn_status_string(int status) {
  switch (status) {
    case GPT_ATTN_OK:
      return "ok";
    case GPT_ATTN_E_INVAL:
      return "invalid argument (null pointer, negative or overflowing size, bad dtype, or bad "
             "dropout probability)";
    case GPT_ATTN_E_UNSUPPORTED:
      return "unsupported head dimension (kernels exist for D = 32, 64 and 128)";
    case GPT_ATTN_E_ALIGN:
      return "pointer not 16-byte aligned";
    case GPT_ATTN_E_WORKSPACE:
      return "workspace missing or smaller than the size its *_workspace_bytes call gives";
    case GPT_ATTN_E_HIP:
      return "HIP runtime error at kernel launch";
    case GPT_ATTN_E_LAYOUT:
      return "bad layout (negative or misaligned stride, overlapping output, or offsets "
             "beyond the supported range)";
    case GPT_ATTN_E_TOO_LARGE:
      return "shape needs more backward workspace than the allocation-free entry point's "
             "static scratch holds (GPT_ATTN_NOALLOC_SCRATCH_BYTES)";
    default:
      return "unknown status";
  }
}

int gpt_attn_fwd_strided(int dtype, int B, int H, int T, int D, const void* q,
                         const gpt_attn_layout* lq, const void* k, const gpt_attn_layout* lk,
                         const void* v, const gpt_attn_layout* lv, void* o,
                         const gpt_attn_layout* lo, void* o_lo, const gpt_attn_layout* llo,
                         float* lse, const gpt_attn_dropout* dropout, void* stream) {
  Shape s;
  GA_TRY(check_shape(dtype, B, H, T, D, &s));
  if (s.rows == 0) return GPT_ATTN_OK;
  if (!q || !k || !v || !o || !lse) return GPT_ATTN_E_INVAL;
  if (o_lo && dtype == GPT_ATTN_F32) return GPT_ATTN_E_INVAL;
  if (!aligned16(q) || !aligned16(k) || !aligned16(v) || !aligned16(o) || !aligned16(lse) ||
      !aligned16(o_lo))
    return GPT_ATTN_E_ALIGN;
  gpt_attn::FwdArgs a;
  a.q = q;
  a.k = k;
  a.v = v;
  a.o = o;
  a.o_lo = o_lo;
  a.lse = lse;
  a.lq = resolve(lq, s);
  a.lk = resolve(lk, s);
  a.lv = resolve(lv, s);
  a.lo = resolve(lo, s);
  a.llo = resolve(llo, s);
  GA_TRY(check_layout(a.lq, s, s.esize, false));
  GA_TRY(check_layout(a.lk, s, s.esize, false));
  GA_TRY(check_layout(a.lv, s, s.esize, false));
  GA_TRY(check_layout(a.lo, s, s.esize, true));
  if (o_lo) GA_TRY(check_layout(a.llo, s, 2, true));
  GA_TRY(resolve_dropout(dropout, &a.drop));
  a.n_heads = B * H;
  a.H = H;
  a.T = T;
  hipStream_t st = static_cast<hipStream_t>(stream);
  return launch_status(dtype == GPT_ATTN_F32
                           ? gpt_attn::launch_fwd_f32(a, D, st)
                           : gpt_attn::launch_fwd_16(a, dtype == GPT_ATTN_F16, D, st));
}

int gpt_attn_fwd(int dtype, int B, int H, int T, int D, const void* q, const void* k,
                 const void* v, void* o, float* lse, void* stream) {
  return gpt_attn_fwd_strided(dtype, B, H, T, D, q, nullptr, k, nullptr, v, nullptr, o, nullptr,
                              nullptr, nullptr, lse, nullptr, stream);
}

size_t gpt_attn_bwd_workspace_bytes(int B, int H, int T, int D) {
  Shape s;
  if (check_shape(GPT_ATTN_BF16, B, H, T, D, &s) != GPT_ATTN_OK || s.rows == 0) return 0;
  return (size_t)gpt_attn::bwd_workspace_bytes((long long)B * H, T);
}

int gpt_attn_bwd_prep_strided(int dtype, int B, int H, int T, int D, const void* q,
                              const gpt_attn_layout* lq, const void* o, const gpt_attn_layout* lo,
                              const void* o_lo, const gpt_attn_layout* llo, const void* dout,
                              const gpt_attn_layout* ldo, float* dq, const gpt_attn_layout* ldq,
                              void* workspace, size_t workspace_bytes, void* stream) {
  Shape s;
  GA_TRY(check_shape(dtype, B, H, T, D, &s));
  if (s.rows == 0) return GPT_ATTN_OK;
  gpt_attn::BwdArgs a;
  GA_TRY(bwd_args(s, 1, q, lq, nullptr, nullptr, nullptr, nullptr, o, lo, o_lo, llo, dout, ldo,
                  nullptr, dq, ldq, nullptr, nullptr, nullptr, nullptr, workspace,
                  workspace_bytes, nullptr, &a));
  return run_prep(s, a, static_cast<hipStream_t>(stream));
}

int gpt_attn_bwd_main_strided(int dtype, int B, int H, int T, int D, const void* q,
                              const gpt_attn_layout* lq, const void* k, const gpt_attn_layout* lk,
                              const void* v, const gpt_attn_layout* lv, const void* dout,
                              const gpt_attn_layout* ldo, const float* lse, float* dq,
                              const gpt_attn_layout* ldq, float* dk, const gpt_attn_layout* ldk,
                              float* dv, const gpt_attn_layout* ldv, const void* workspace,
                              size_t workspace_bytes, const gpt_attn_dropout* dropout,
                              void* stream) {
  Shape s;
  GA_TRY(check_shape(dtype, B, H, T, D, &s));
  if (s.rows == 0) return GPT_ATTN_OK;
  gpt_attn::BwdArgs a;
  GA_TRY(bwd_args(s, 2, q, lq, k, lk, v, lv, nullptr, nullptr, nullptr, nullptr, dout, ldo, lse,
                  dq, ldq, dk, ldk, dv, ldv, workspace, workspace_bytes, dropout, &a));
  return run_main(s, a, static_cast<hipStream_t>(stream));
}

int gpt_attn_bwd_strided(int dtype, int B, int H, int T, int D, const void* q,
                         const gpt_attn_layout* lq, const void* k, const gpt_attn_layout* lk,
                         const void* v, const gpt_attn_layout* lv, const void* o,
                         const gpt_attn_layout* lo, const void* o_lo, const gpt_attn_layout* llo,
                         const void* dout, const gpt_attn_layout* ldo, const float* lse,
                         float* dq, const gpt_attn_layout* ldq, float* dk,
                         const gpt_attn_layout* ldk, float* dv, const gpt_attn_layout* ldv,
                         void* workspace, size_t workspace_bytes,
                         const gpt_attn_dropout* dropout, void* stream) {
  Shape s;
  GA_TRY(check_shape(dtype, B, H, T, D, &s));
  if (s.rows == 0) return GPT_ATTN_OK;
  // Validate everything both phases need before enqueuing either.
  gpt_attn::BwdArgs a;
  GA_TRY(bwd_args(s, 3, q, lq, k, lk, v, lv, o, lo, o_lo, llo, dout, ldo, lse, dq, ldq, dk, ldk,
                  dv, ldv, workspace, workspace_bytes, dropout, &a));
  hipStream_t st = static_cast<hipStream_t>(stream);
  GA_TRY(run_prep(s, a, st));
  return run_main(s, a, st);
}

int gpt_attn_bwd_prep(int dtype, int B, int H, int T, int D, const void* q, const void* o,
                      const void* dout, float* dq, void* workspace, size_t workspace_bytes,
                      void* stream) {
  return gpt_attn_bwd_prep_strided(dtype, B, H, T, D, q, nullptr, o, nullptr, nullptr, nullptr,
                                   dout, nullptr, dq, nullptr, workspace, workspace_bytes, stream);
}

int gpt_attn_bwd_main(int dtype, int B, int H, int T, int D, const void* q, const void* k,
                      const void* v, const void* dout, const float* lse, float* dq, float* dk,
                      float* dv, const void* workspace, size_t workspace_bytes, void* stream) {
  return gpt_attn_bwd_main_strided(dtype, B, H, T, D, q, nullptr, k, nullptr, v, nullptr, dout,
                                   nullptr, lse, dq, nullptr, dk, nullptr, dv, nullptr, workspace,
                                   workspace_bytes, nullptr, stream);
}

int gpt_attn_bwd(int dtype, int B, int H, int T, int D, const void* q, const void* k,
                 const void* v, const void* o, const void* dout, const float* lse, float* dq,
                 float* dk, float* dv, void* workspace, size_t workspace_bytes, void* stream) {
  return gpt_attn_bwd_strided(dtype, B, H, T, D, q, nullptr, k, nullptr, v, nullptr, o, nullptr,
                              nullptr, nullptr, dout, nullptr, lse, dq, nullptr, dk, nullptr, dv,
                              nullptr, workspace, workspace_bytes, nullptr, stream);
}

int gpt_attn_bwd_noalloc(int dtype, int B, int H, int T, int D, const void* q, const void* k,
                         const void* v, const void* o, const void* dout, const float* lse,
                         float* dq, float* dk, float* dv, void* stream) {
  Shape s;
  GA_TRY(check_shape(dtype, B, H, T, D, &s));
  if (s.rows == 0) return GPT_ATTN_OK;
  const size_t need = (size_t)gpt_attn::bwd_workspace_bytes((long long)B * H, T);
  if (need > (size_t)GPT_ATTN_NOALLOC_SCRATCH_BYTES) return GPT_ATTN_E_TOO_LARGE;
  // Every argument check of the workspace form runs before the first HIP
  // call (a valid stand-in workspace address and size pass its checks).
  gpt_attn::BwdArgs a;
  GA_TRY(bwd_args(s, 3, q, nullptr, k, nullptr, v, nullptr, o, nullptr, nullptr, nullptr, dout,
                  nullptr, lse, dq, nullptr, dk, nullptr, dv, nullptr,
                  reinterpret_cast<void*>((uintptr_t)256), need, nullptr, &a));
  hipStream_t st = static_cast<hipStream_t>(stream);
  void* ws = nullptr;
  GA_TRY(scratch_address(st, &ws));
  return gpt_attn_bwd(dtype, B, H, T, D, q, k, v, o, dout, lse, dq, dk, dv, ws, need, stream);
}

size_t gpt_attn_decode_workspace_bytes(int dtype, int B, int H, int L, int D) {
  Shape s;
  if (check_shape(dtype, B, H, L, D, &s) != GPT_ATTN_OK) return 0;
  const long long heads = (long long)B * H;
  if (heads == 0 || L == 0) return 0;
  const long long chunks = ((long long)L + 127) / 128;  // the smallest chunk is 128 keys
  return (size_t)(heads * chunks * gpt_attn::kDecPart * (long long)sizeof(float));
}

int gpt_attn_decode(int dtype, int B, int H, int L, int D, const void* q,
                    const gpt_attn_layout* lq, const void* k_cache, const gpt_attn_layout* lk,
                    const void* v_cache, const gpt_attn_layout* lv, const int* lengths, void* o,
                    const gpt_attn_layout* lo, float* lse, void* workspace,
                    size_t workspace_bytes, void* stream) {
  Shape s;  // the caches: [B, H, L, D]
  GA_TRY(check_shape(dtype, B, H, L, D, &s));
  Shape s1;  // one query per head: [B, H, 1, D]
  GA_TRY(check_shape(dtype, B, H, 1, D, &s1));
  const long long heads = (long long)B * H;
  if (heads == 0) return GPT_ATTN_OK;
  if (!q || !o || !lse || (L > 0 && (!k_cache || !v_cache))) return GPT_ATTN_E_INVAL;
  if (!aligned16(q) || !aligned16(k_cache) || !aligned16(v_cache) || !aligned16(o) ||
      !aligned16(lse) || !aligned16(lengths))
    return GPT_ATTN_E_ALIGN;
  gpt_attn::DecArgs a;
  a.q = q;
  a.k = k_cache;
  a.v = v_cache;
  a.lengths = lengths;
  a.o = o;
  a.lse = lse;
  a.part = static_cast<float*>(workspace);
  a.lq = resolve(lq, s1);
  a.lo = resolve(lo, s1);
  a.lk = resolve(lk, s);
  a.lv = resolve(lv, s);
  GA_TRY(check_layout(a.lq, s1, s1.esize, false));
  GA_TRY(check_layout(a.lo, s1, s1.esize, true));
  if (L > 0) {
    GA_TRY(check_layout(a.lk, s, s.esize, false));
    GA_TRY(check_layout(a.lv, s, s.esize, false));
  }
  const size_t need = gpt_attn_decode_workspace_bytes(dtype, B, H, L, D);
  if (need > 0 && (!workspace || workspace_bytes < need)) return GPT_ATTN_E_WORKSPACE;
  if (!aligned16(workspace)) return GPT_ATTN_E_ALIGN;
  a.n_heads = (int)heads;
  a.H = H;
  a.L = L;
  return launch_status(gpt_attn::launch_decode(a, dtype, D, static_cast<hipStream_t>(stream)));
}

int gpt_attn_dropout_mask(int B, int H, int T, const gpt_attn_dropout* dropout,
                          unsigned char* mask, void* stream) {
  if (B < 0 || H < 0 || T < 0 || !dropout) return GPT_ATTN_E_INVAL;
  const long long heads = (long long)B * H;
  const long long bytes = heads * (long long)T * (long long)T;
  if (heads * (long long)T >= (1LL << 31) || bytes >= (1LL << 40)) return GPT_ATTN_E_INVAL;
  gpt_attn::Dropout d;
  GA_TRY(resolve_dropout(dropout, &d));
  if (bytes == 0) return GPT_ATTN_OK;
  if (!mask) return GPT_ATTN_E_INVAL;
  return launch_status(
      gpt_attn::launch_dropout_mask(d, (int)heads, T, mask, static_cast<hipStream_t>(stream)));
}

}  // extern "C"
