// Drives the C ABI (include/gpt_attn.h) in a host-only build, linked with the
// stand-in launch layer of launch_stubs.cpp, for the run under
// -fsanitize=address,undefined in the CPU test suite. Pointers are fake,
// 16-byte aligned addresses that are never dereferenced: every call either
// stops at validation or reaches the stand-in launcher, whose record of the
// launch arguments is checked (head counts, layouts, the workspace split
// into delta and per-chunk maxima, the dropout parameters). Exit status 0
// when every check holds.
#include <stdint.h>
#include <stdio.h>

#include <string>
#include <vector>

#include "gpt_attn.h"
#include "launch_record.h"

using gpt_attn::g_record;

static int failures = 0;
#define CHECK(cond)                                              \
  do {                                                           \
    if (!(cond)) {                                               \
      fprintf(stderr, "FAIL line %d: %s\n", __LINE__, #cond);    \
      ++failures;                                                \
    }                                                            \
  } while (0)

static void* P(uintptr_t off = 0) { return reinterpret_cast<void*>(0x100000 + off); }
static float* F(uintptr_t off = 0) { return static_cast<float*>(P(off)); }

static std::vector<std::string> calls() {
  std::vector<std::string> c = g_record.calls;
  g_record.calls.clear();
  return c;
}

int main() {
  // ---- forward ----------------------------------------------------------
  CHECK(gpt_attn_fwd(GPT_ATTN_BF16, 2, 3, 100, 64, P(), P(), P(), P(), F(), nullptr) ==
        GPT_ATTN_OK);
  CHECK(calls() == std::vector<std::string>{"fwd_16"});
  CHECK(g_record.fwd.n_heads == 6 && g_record.fwd.H == 3 && g_record.fwd.T == 100);
  CHECK(g_record.fwd.lq.t == 64 && g_record.fwd.lq.h == 6400 && g_record.fwd.lq.b == 19200);
  CHECK(g_record.fwd.o_lo == nullptr && g_record.fwd.drop.thr == 0);
  CHECK(gpt_attn_fwd(GPT_ATTN_F16, 1, 1, 5, 32, P(), P(), P(), P(), F(), nullptr) == 0);
  CHECK(calls() == std::vector<std::string>{"fwd_16"} && g_record.fp16 && g_record.D == 32);
  CHECK(gpt_attn_fwd(GPT_ATTN_F32, 1, 1, 5, 64, P(), P(), P(), P(), F(), nullptr) == 0);
  CHECK(calls() == std::vector<std::string>{"fwd_f32"});
  // Bad arguments stop before any launch.
  CHECK(gpt_attn_fwd(3, 1, 1, 5, 64, P(), P(), P(), P(), F(), nullptr) == GPT_ATTN_E_INVAL);
  CHECK(gpt_attn_fwd(GPT_ATTN_BF16, 1, 1, 5, 256, P(), P(), P(), P(), F(), nullptr) ==
        GPT_ATTN_E_UNSUPPORTED);
  CHECK(gpt_attn_fwd(GPT_ATTN_BF16, 1, 1, 5, 64, P(8), P(), P(), P(), F(), nullptr) ==
        GPT_ATTN_E_ALIGN);
  CHECK(gpt_attn_fwd(GPT_ATTN_BF16, 1 << 16, 1 << 15, 1, 64, P(), P(), P(), P(), F(),
                     nullptr) == GPT_ATTN_E_INVAL);
  CHECK(gpt_attn_fwd(GPT_ATTN_BF16, 0, 3, 5, 64, nullptr, nullptr, nullptr, nullptr, nullptr,
                     nullptr) == GPT_ATTN_OK);
  CHECK(calls().empty());

  // ---- backward: workspace = delta, then per-chunk maxima -----------------
  const int B = 2, H = 3, T = 300;
  const size_t ws_bytes = gpt_attn_bwd_workspace_bytes(B, H, T, 64);
  const size_t rows = (size_t)B * H * T;
  const size_t stats_off = (rows * 4 + 15) / 16 * 16;
  CHECK(ws_bytes == stats_off + 32 * (size_t)B * H * ((T + 127) / 128));
  CHECK(gpt_attn_bwd(GPT_ATTN_BF16, B, H, T, 64, P(), P(), P(), P(), P(), F(), F(), F(), F(),
                     P(0x10000), ws_bytes, nullptr) == 0);
  CHECK((calls() == std::vector<std::string>{"prep_16", "main_16"}));
  CHECK(g_record.bwd.delta == F(0x10000));
  CHECK(reinterpret_cast<uintptr_t>(g_record.bwd.stats) == 0x110000 + stats_off);
  CHECK(g_record.bwd.o_lo == nullptr && g_record.bwd.n_heads == 6 && g_record.bwd.T == 300);
  CHECK(gpt_attn_bwd(GPT_ATTN_BF16, B, H, T, 64, P(), P(), P(), P(), P(), F(), F(), F(), F(),
                     P(0x10000), ws_bytes - 1, nullptr) == GPT_ATTN_E_WORKSPACE);
  CHECK(gpt_attn_bwd(GPT_ATTN_BF16, B, H, T, 64, P(), P(), P(), P(), P(), F(), F(), F(), F(),
                     P(0x10004), ws_bytes, nullptr) == GPT_ATTN_E_ALIGN);
  CHECK(gpt_attn_bwd(GPT_ATTN_F32, 1, 6, 256, 64, P(), P(), P(), P(), P(), F(), F(), F(), F(),
                     P(), gpt_attn_bwd_workspace_bytes(1, 6, 256, 64), nullptr) == 0);
  CHECK((calls() == std::vector<std::string>{"prep_f32", "main_f32"}));
  // The 16-bit prep phase needs q (its maxima); fp32 does not.
  CHECK(gpt_attn_bwd_prep(GPT_ATTN_BF16, 1, 1, 8, 64, nullptr, P(), P(), F(), P(), 1 << 20,
                          nullptr) == GPT_ATTN_E_INVAL);
  CHECK(gpt_attn_bwd_prep(GPT_ATTN_F32, 1, 1, 8, 64, nullptr, P(), P(), nullptr, P(), 1 << 20,
                          nullptr) == GPT_ATTN_OK);
  CHECK(calls() == std::vector<std::string>{"prep_f32"});
  CHECK(gpt_attn_bwd_workspace_bytes(-1, 1, 8, 64) == 0);
  CHECK(gpt_attn_bwd_workspace_bytes(1, 1, 8, 96) == 0);

  // ---- strided calls: the fused [B, T, 3C] projection layout, o_lo, dropout
  const int C = H * 64;
  gpt_attn_layout lqkv = {3LL * T * C, 64, 3 * C}, lout = {1LL * T * C, 64, C};
  gpt_attn_dropout drop = {0.2, 0x123456789ABCDEFull, 7u};
  CHECK(gpt_attn_fwd_strided(GPT_ATTN_BF16, B, H, T, 64, P(), &lqkv, P(128), &lqkv, P(256),
                             &lqkv, P(), &lout, P(), &lout, F(), &drop, nullptr) == 0);
  CHECK(calls() == std::vector<std::string>{"fwd_16"});
  CHECK(g_record.fwd.lq.t == 3 * C && g_record.fwd.lq.h == 64 && g_record.fwd.lo.t == C);
  CHECK(g_record.fwd.drop.thr == 13107 && g_record.fwd.drop.key0 == 0x89ABCDEFu &&
        g_record.fwd.drop.key1 == 0x01234567u && g_record.fwd.drop.offset == 7u);
  CHECK(g_record.fwd.o_lo == P());
  gpt_attn_layout overlap = {1LL * T * C, 0, C};  // heads of an output share rows
  CHECK(gpt_attn_fwd_strided(GPT_ATTN_BF16, B, H, T, 64, P(), &lqkv, P(), &lqkv, P(), &lqkv,
                             P(), &overlap, nullptr, nullptr, F(), nullptr, nullptr) ==
        GPT_ATTN_E_LAYOUT);
  gpt_attn_dropout bad = {1.0, 1, 0};
  CHECK(gpt_attn_fwd_strided(GPT_ATTN_BF16, B, H, T, 64, P(), nullptr, P(), nullptr, P(),
                             nullptr, P(), nullptr, nullptr, nullptr, F(), &bad, nullptr) ==
        GPT_ATTN_E_INVAL);
  CHECK(calls().empty());

  // ---- decode, dropout mask, no-alloc ---------------------------------------
  const size_t dws = gpt_attn_decode_workspace_bytes(GPT_ATTN_BF16, 2, 3, 100, 64);
  CHECK(gpt_attn_decode(GPT_ATTN_BF16, 2, 3, 100, 64, P(), nullptr, P(), nullptr, P(), nullptr,
                        nullptr, P(), nullptr, F(), P(), dws, nullptr) == 0);
  CHECK(calls() == std::vector<std::string>{"decode"} && g_record.dec.L == 100);
  CHECK(gpt_attn_dropout_mask(1, 2, 9, &drop, static_cast<unsigned char*>(P()), nullptr) == 0);
  CHECK(calls() == std::vector<std::string>{"dropout_mask"} && g_record.n_heads == 2 &&
        g_record.T == 9);
  CHECK(gpt_attn_bwd_noalloc(GPT_ATTN_BF16, 64, 64, 1024, 64, P(), P(), P(), P(), P(), F(), F(),
                             F(), F(), nullptr) == GPT_ATTN_E_TOO_LARGE);
  CHECK(gpt_attn_bwd_noalloc(GPT_ATTN_BF16, 1, 1, 8, 64, nullptr, P(), P(), P(), P(), F(), F(),
                             F(), F(), nullptr) == GPT_ATTN_E_INVAL);
  CHECK(calls().empty());
  for (int st = 0; st <= 8; ++st) CHECK(gpt_attn_status_string(st) != nullptr);
  CHECK(gpt_attn_abi_version() == GPT_ATTN_ABI_VERSION);

  if (failures) {
    fprintf(stderr, "%d check(s) failed\n", failures);
    return 1;
  }
  printf("ABI self-check ok\n");
  return 0;
}
