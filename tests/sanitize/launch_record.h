// What the stand-in launch layer (launch_stubs.cpp) recorded.
#pragma once
#include <string>
#include <vector>

#include "attn_launch.h"

namespace gpt_attn {
struct Record {
  std::vector<std::string> calls;
  FwdArgs fwd;
  BwdArgs bwd;
  DecArgs dec;
  Dropout drop;
  int D = 0, n_heads = 0, T = 0;
  bool fp16 = false;
};
extern Record g_record;
}  // namespace gpt_attn
