// The C ABI declared in include/gpt_attn.h: argument validation, dispatch
// by dtype, and launch-error reporting. Validation completes before any HIP
// call, so a rejected call touches neither the device nor the HIP runtime.
#include <stdint.h>

#include "attn_launch.h"
#include "gpt_attn.h"

namespace {


bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

// Shape and dtype checks shared by every entry point. On success *rows is
// B*H*T (possibly 0 for an empty call).
int check_shape(int dtype, int B, int H, int T, int D, long long* rows) {
  if (dtype != GPT_ATTN_F32 && dtype != GPT_ATTN_BF16) return GPT_ATTN_E_INVAL;
  if (B < 0 || H < 0 || T < 0 || D <= 0) return GPT_ATTN_E_INVAL;
  if (D != 64) return GPT_ATTN_E_UNSUPPORTED;
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
  *rows = r;
  return GPT_ATTN_OK;
}

int launch_status(hipError_t e) { return e == hipSuccess ? GPT_ATTN_OK : GPT_ATTN_E_HIP; }

}  // namespace

extern "C" {

int gpt_attn_abi_version(void) { return GPT_ATTN_ABI_VERSION; }

const char* gpt_attn_status_string(int status) {
  switch (status) {
    case GPT_ATTN_OK:
      return "ok";
    case GPT_ATTN_E_INVAL:
      return "invalid argument (null pointer, negative or overflowing size, or bad dtype)";
    case GPT_ATTN_E_UNSUPPORTED:
      return "unsupported head dimension (only D = 64 has kernels)";
    case GPT_ATTN_E_ALIGN:
      return "pointer not 16-byte aligned";
    case GPT_ATTN_E_WORKSPACE:
      return "workspace missing or smaller than gpt_attn_bwd_workspace_bytes";
    case GPT_ATTN_E_HIP:
      return "HIP runtime error at kernel launch";
    default:
      return "unknown status";
  }
}

int gpt_attn_fwd(int dtype, int B, int H, int T, int D, const void* q, const void* k,
                 const void* v, void* o, void* o_lo, float* lse, void* stream) {
  long long rows = 0;
  const int st = check_shape(dtype, B, H, T, D, &rows);
  if (st != GPT_ATTN_OK) return st;
  if (rows == 0) return GPT_ATTN_OK;
  if (!q || !k || !v || !o || !lse) return GPT_ATTN_E_INVAL;
  if (o_lo && dtype != GPT_ATTN_BF16) return GPT_ATTN_E_INVAL;
  if (!aligned16(q) || !aligned16(k) || !aligned16(v) || !aligned16(o) || !aligned16(lse) ||
      !aligned16(o_lo))
    return GPT_ATTN_E_ALIGN;
  const int heads = B * H;
  hipStream_t s = static_cast<hipStream_t>(stream);
  if (dtype == GPT_ATTN_BF16)
    return launch_status(gpt_attn::launch_fwd_bf16(q, k, v, o, o_lo, lse, heads, T, s));
  return launch_status(gpt_attn::launch_fwd_f32(static_cast<const float*>(q),
                                                static_cast<const float*>(k),
                                                static_cast<const float*>(v),
                                                static_cast<float*>(o), lse, heads, T, s));
}

size_t gpt_attn_bwd_workspace_bytes(int dtype, int B, int H, int T, int D) {
  long long rows = 0;
  if (check_shape(dtype, B, H, T, D, &rows) != GPT_ATTN_OK) return 0;
  return (size_t)rows * sizeof(float);
}

int gpt_attn_bwd_prep(int dtype, int B, int H, int T, int D, const void* o, const void* o_lo,
                      const void* dout, float* dq, void* workspace, size_t workspace_bytes,
                      void* stream) {
  long long rows = 0;
  const int st = check_shape(dtype, B, H, T, D, &rows);
  if (st != GPT_ATTN_OK) return st;
  if (rows == 0) return GPT_ATTN_OK;
  if (!o || !dout || (dtype == GPT_ATTN_BF16 && !dq)) return GPT_ATTN_E_INVAL;
  if (o_lo && dtype != GPT_ATTN_BF16) return GPT_ATTN_E_INVAL;
  if (!aligned16(o) || !aligned16(o_lo) || !aligned16(dout) || !aligned16(dq))
    return GPT_ATTN_E_ALIGN;
  if (!workspace || workspace_bytes < (size_t)rows * sizeof(float)) return GPT_ATTN_E_WORKSPACE;
  if (!aligned16(workspace)) return GPT_ATTN_E_ALIGN;
  float* delta = static_cast<float*>(workspace);
  hipStream_t s = static_cast<hipStream_t>(stream);
  const int heads = B * H;
  if (dtype == GPT_ATTN_BF16)
    return launch_status(gpt_attn::launch_bwd_prep_bf16(o, o_lo, dout, dq, delta, heads, T, s));
  return launch_status(gpt_attn::launch_bwd_prep_f32(static_cast<const float*>(o),
                                                     static_cast<const float*>(dout), delta,
                                                     heads, T, s));
}

int gpt_attn_bwd_main(int dtype, int B, int H, int T, int D, const void* q, const void* k,
                      const void* v, const void* dout, const float* lse, float* dq, float* dk,
                      float* dv, const void* workspace, size_t workspace_bytes, void* stream) {
  long long rows = 0;
  const int st = check_shape(dtype, B, H, T, D, &rows);
  if (st != GPT_ATTN_OK) return st;
  if (rows == 0) return GPT_ATTN_OK;
  if (!q || !k || !v || !dout || !lse || !dq || !dk || !dv) return GPT_ATTN_E_INVAL;
  if (!aligned16(q) || !aligned16(k) || !aligned16(v) || !aligned16(dout) || !aligned16(lse) ||
      !aligned16(dq) || !aligned16(dk) || !aligned16(dv))
    return GPT_ATTN_E_ALIGN;
  if (!workspace || workspace_bytes < (size_t)rows * sizeof(float)) return GPT_ATTN_E_WORKSPACE;
  if (!aligned16(workspace)) return GPT_ATTN_E_ALIGN;
  const float* delta = static_cast<const float*>(workspace);
  hipStream_t s = static_cast<hipStream_t>(stream);
  const int heads = B * H;
  if (dtype == GPT_ATTN_BF16)
    return launch_status(
        gpt_attn::launch_bwd_main_bf16(q, k, v, dout, lse, delta, dq, dk, dv, heads, T, s));
  return launch_status(gpt_attn::launch_bwd_main_f32(
      static_cast<const float*>(q), static_cast<const float*>(k), static_cast<const float*>(v),
      static_cast<const float*>(dout), lse, delta, dq, dk, dv, heads, T, s));
}

int gpt_attn_bwd(int dtype, int B, int H, int T, int D, const void* q, const void* k,
                 const void* v, const void* o, const void* o_lo, const void* dout,
                 const float* lse, float* dq, float* dk, float* dv, void* workspace,
                 size_t workspace_bytes, void* stream) {
  long long rows = 0;
  const int st = check_shape(dtype, B, H, T, D, &rows);
  if (st != GPT_ATTN_OK) return st;
  if (rows == 0) return GPT_ATTN_OK;
  // Validate everything both phases need before enqueuing either.
  if (!q || !k || !v || !o || !dout || !lse || !dq || !dk || !dv) return GPT_ATTN_E_INVAL;
  if (o_lo && dtype != GPT_ATTN_BF16) return GPT_ATTN_E_INVAL;
  if (!aligned16(q) || !aligned16(k) || !aligned16(v) || !aligned16(o) || !aligned16(dout) ||
      !aligned16(lse) || !aligned16(dq) || !aligned16(dk) || !aligned16(dv) || !aligned16(o_lo))
    return GPT_ATTN_E_ALIGN;
  if (!workspace || workspace_bytes < (size_t)rows * sizeof(float)) return GPT_ATTN_E_WORKSPACE;
  if (!aligned16(workspace)) return GPT_ATTN_E_ALIGN;
  const int r = gpt_attn_bwd_prep(dtype, B, H, T, D, o, o_lo, dout, dq, workspace,
                                  workspace_bytes, stream);
  if (r != GPT_ATTN_OK) return r;
  return gpt_attn_bwd_main(dtype, B, H, T, D, q, k, v, dout, lse, dq, dk, dv, workspace,
                           workspace_bytes, stream);
}

}  // extern "C"
