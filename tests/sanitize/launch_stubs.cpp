// Stand-ins for the kernel launch layer (attn_launch.h) for a host-only build
// of the C ABI: each records what it was asked to launch and returns
// hipSuccess, so the validation and argument marshalling of every entry
// point run under the address and undefined-behaviour sanitizers without a
// GPU.
#include "launch_record.h"

namespace gpt_attn {

Record g_record;

static hipError_t note(const char* which, int D, bool fp16) {
  g_record.calls.push_back(which);
  g_record.D = D;
  g_record.fp16 = fp16;
  return hipSuccess;
}

hipError_t launch_fwd_16(const FwdArgs& a, bool fp16, int D, hipStream_t) {
  g_record.fwd = a;
  return note("fwd_16", D, fp16);
}
hipError_t launch_fwd_f32(const FwdArgs& a, int D, hipStream_t) {
  g_record.fwd = a;
  return note("fwd_f32", D, false);
}
hipError_t launch_bwd_prep_16(const BwdArgs& a, bool fp16, int D, hipStream_t) {
  g_record.bwd = a;
  return note("prep_16", D, fp16);
}
hipError_t launch_bwd_main_16(const BwdArgs& a, bool fp16, int D, hipStream_t) {
  g_record.bwd = a;
  return note("main_16", D, fp16);
}
hipError_t launch_bwd_prep_f32(const BwdArgs& a, int D, hipStream_t) {
  g_record.bwd = a;
  return note("prep_f32", D, false);
}
hipError_t launch_bwd_main_f32(const BwdArgs& a, int D, hipStream_t) {
  g_record.bwd = a;
  return note("main_f32", D, false);
}
hipError_t launch_decode(const DecArgs& a, int dtype_code, int D, hipStream_t) {
  g_record.dec = a;
  return note("decode", D, dtype_code == 2);
}
hipError_t launch_dropout_mask(const Dropout& d, int n_heads, int T, uint8_t*, hipStream_t) {
  g_record.drop = d;
  g_record.n_heads = n_heads;
  g_record.T = T;
  return note("dropout_mask", 0, false);
}

}  // namespace gpt_attn
