// Host-side validation paths of the C ABI, for a build of the library whose
// host code carries AddressSanitizer and UndefinedBehaviorSanitizer.
//
// Every call below is rejected (or is an n == 0 no-op) before the library
// touches a device, so the program needs no GPU.  Pointers are fake, aligned,
// non-null addresses that are never dereferenced.  Sizes include extremes
// (2^62 heads, 2^24 + 1 rows) so that any unchecked multiplication in the
// workspace arithmetic would show up as signed overflow.
#include <cstdint>
#include <cstdio>
#include <cstring>
#include <initializer_list>

#include "larard.h"

namespace {

int g_fail = 0;

void expect(const char* what, int got, int want) {
  if (got != want) {
    std::printf("FAIL %s: status %d, expected %d (%s)\n", what, got, want, larard_last_error());
    ++g_fail;
  }
}

void* fake(uintptr_t off = 0) { return reinterpret_cast<void*>(uintptr_t(1) << 20 | off); }
float* ffake(uintptr_t off = 0) { return static_cast<float*>(fake(off)); }

}  // namespace

int main() {
  const int64_t big = int64_t(1) << 62;
  const larard_dtype bf = LARARD_BF16, f32 = LARARD_FP32;

  // workspace sizing
  if (larard_workspace_bytes(bf, 1, 32, 16384) == 0) { std::printf("FAIL workspace size\n"); ++g_fail; }
  if (larard_workspace_bytes(bf, big, big, 1) != 0) { std::printf("FAIL huge B*H accepted\n"); ++g_fail; }
  if (larard_workspace_bytes(bf, 1, 1, (int64_t(1) << 24) + 1) != 0) { std::printf("FAIL huge n accepted\n"); ++g_fail; }
  if (larard_workspace_bytes(f32, 0, 1, 4) != 0) { std::printf("FAIL B=0 accepted\n"); ++g_fail; }
  // head groups of the whole-path calls (overflow-prone products of sizes)
  if (larard_loss_head_group(bf, 1, 32, 16384, 128, 0) != 32) { std::printf("FAIL head group 16K\n"); ++g_fail; }
  if (larard_loss_head_group(bf, 1, 32, 32768, 128, 1) != 8) { std::printf("FAIL head group cross\n"); ++g_fail; }
  if (larard_loss_head_group(bf, big, big, 64, 128, 0) != 0) { std::printf("FAIL huge head group accepted\n"); ++g_fail; }
  if (larard_loss_head_group(bf, 1, 1, int64_t(1) << 24, 128, 1) != 1) { std::printf("FAIL head group max n\n"); ++g_fail; }
  if (larard_loss_head_group(bf, 1, 4, -1, 128, 0) != 0) { std::printf("FAIL negative n accepted\n"); ++g_fail; }
  if (larard_loss_sweep_group(bf, 1, 32, 16384, 128, 0) != 16) { std::printf("FAIL sweep group 16K\n"); ++g_fail; }
  if (larard_loss_sweep_group(bf, big, big, 64, 128, 0) != 0) { std::printf("FAIL huge sweep group accepted\n"); ++g_fail; }
  size_t off[4];
  expect("layout null", larard_workspace_layout(bf, 1, 1, 4, nullptr), LARARD_E_INVALID);
  expect("layout", larard_workspace_layout(bf, 2, 8, 8192, off), LARARD_OK);
  expect("layout dtype", larard_workspace_layout(static_cast<larard_dtype>(9), 2, 8, 8192, off),
         LARARD_E_UNSUPPORTED);

  // phase 1
  expect("lse null x", larard_lse_fwd(nullptr, fake(), bf, 1, 1, 64, 128, 0.1f, 1, fake(), fake(), nullptr),
         LARARD_E_INVALID);
  expect("lse misaligned", larard_lse_fwd(fake(8), fake(), bf, 1, 1, 64, 128, 0.1f, 1, fake(), fake(), nullptr),
         LARARD_E_INVALID);
  expect("lse d", larard_lse_fwd(fake(), fake(), bf, 1, 1, 64, 96, 0.1f, 1, fake(), fake(), nullptr),
         LARARD_E_UNSUPPORTED);
  expect("lse huge", larard_lse_fwd(fake(), fake(), bf, big, big, 64, 128, 0.1f, 1, fake(), fake(), nullptr),
         LARARD_E_INVALID);
  expect("lse grid", larard_lse_fwd(fake(), fake(), f32, 1, 1 << 13, 1 << 24, 128, 0.1f, 1, fake(), fake(), nullptr),
         LARARD_E_INVALID);
  expect("lse scale", larard_lse_fwd(fake(), fake(), bf, 1, 1, 64, 128, -1.f, 1, fake(), fake(), nullptr),
         LARARD_E_INVALID);
  expect("lse n=0", larard_lse_fwd(nullptr, nullptr, bf, 1, 1, 0, 128, 0.1f, 1, nullptr, nullptr, nullptr),
         LARARD_OK);
  expect("kl_fwd row_kl", larard_kl_fwd(fake(), fake(), bf, 1, 2, 64, 128, 0.1f, 1, fake(), fake(), nullptr, nullptr),
         LARARD_E_INVALID);

  // phase 2
  for (int mode : {0, 1, 2, 3, 4, -7}) {
    const int want = (mode == 0 || mode == 1 || mode == 3) ? LARARD_OK
                     : mode == 2                           ? LARARD_E_UNSUPPORTED
                                                           : LARARD_E_INVALID;
    expect("kl_bwd mode", larard_kl_bwd(nullptr, nullptr, bf, 1, 1, 0, 64, 0.1f, 1, nullptr, nullptr, 1.f, nullptr,
                                        nullptr, mode, nullptr), want);
  }
  expect("kl_bwd dx align", larard_kl_bwd(fake(), fake(), bf, 1, 2, 64, 64, 0.1f, 1, fake(), fake(), 1.f, ffake(),
                                          ffake(4), 0, nullptr), LARARD_E_INVALID);
  expect("rows null row_kl", larard_kl_bwd_rows(fake(), fake(), bf, 1, 2, 64, 64, 0.1f, 1, fake(), fake(), 1.f,
                                                nullptr, nullptr, nullptr), LARARD_E_INVALID);
  expect("cols null dx", larard_kl_bwd_cols(fake(), fake(), bf, 1, 2, 64, 64, 0.1f, 1, fake(), fake(), 1.f, nullptr,
                                            nullptr), LARARD_E_INVALID);
  expect("reduce sizes", larard_reduce_loss(ffake(), big, big, 4, 1.f, static_cast<double*>(fake()), ffake(), nullptr),
         LARARD_E_INVALID);

  // whole path
  const size_t need = larard_workspace_bytes(bf, 1, 2, 64);
  expect("loss small ws", larard_loss(fake(), fake(), bf, 1, 2, 64, 128, 0.1f, 1, 1.f, fake(), need - 1, ffake(),
                                      ffake(), 0, nullptr), LARARD_E_WORKSPACE);
  expect("loss ws align", larard_loss(fake(), fake(), bf, 1, 2, 64, 128, 0.1f, 1, 1.f, fake(16), need, ffake(),
                                      ffake(), 0, nullptr), LARARD_E_WORKSPACE);
  expect("loss atomic", larard_loss(fake(), fake(), bf, 1, 2, 64, 128, 0.1f, 1, 1.f, fake(), need, ffake(), ffake(),
                                    LARARD_DX_ATOMIC, nullptr), LARARD_E_UNSUPPORTED);
  expect("noalloc limit", larard_loss_noalloc(fake(), fake(), bf, 1, 64, 65536, 64, 0.1f, 1, 1.f, ffake(), ffake(), 0,
                                              nullptr), LARARD_E_WORKSPACE);
  expect("noalloc loss null", larard_loss_noalloc(fake(), fake(), bf, 1, 2, 64, 64, 0.1f, 1, 1.f, nullptr, ffake(), 0,
                                                  nullptr), LARARD_E_INVALID);

  // cross relation
  expect("xy null y", larard_xy_lse_fwd(fake(), fake(), nullptr, fake(), bf, 1, 2, 64, 128, 0.1f, 1, fake(), fake(),
                                        nullptr), LARARD_E_INVALID);
  expect("xy dy align", larard_xy_kl_bwd(fake(), fake(), fake(), fake(), bf, 1, 2, 64, 128, 0.1f, 1, fake(), fake(),
                                         1.f, ffake(), ffake(), ffake(4), nullptr), LARARD_E_INVALID);
  expect("xy loss ws", larard_xy_loss(fake(), fake(), fake(), fake(), bf, 1, 2, 64, 128, 0.1f, 1, 1.f, nullptr, 0,
                                      ffake(), ffake(), ffake(), nullptr), LARARD_E_WORKSPACE);

  // several maps
  larard_map maps[3] = {{fake(), fake(), 32, 1.f, ffake()}, {fake(), fake(), 8, 1.f, ffake()},
                        {fake(), fake(), 8, 1.f, nullptr}};
  expect("multi all-or-none", larard_multi_loss(maps, 3, bf, 2, 64, 128, 0.1f, 1, 1.f, fake(), size_t(1) << 30,
                                                 ffake(), nullptr), LARARD_E_INVALID);
  maps[2].dx_s = ffake();
  maps[1].H = big;
  if (larard_multi_workspace_bytes(bf, 2, 64, maps, 3) != 0) { std::printf("FAIL huge map heads accepted\n"); ++g_fail; }
  expect("multi huge heads", larard_multi_loss(maps, 3, bf, 2, 64, 128, 0.1f, 1, 1.f, fake(), size_t(1) << 30,
                                               ffake(), nullptr), LARARD_E_INVALID);
  expect("multi count", larard_multi_loss(maps, 9, bf, 2, 64, 128, 0.1f, 1, 1.f, fake(), size_t(1) << 30, ffake(),
                                          nullptr), LARARD_E_INVALID);

  // projection backward
  if (larard_proj_bwd_workspace_bytes(big, big, 4096, 32, 128) != 0) { std::printf("FAIL huge proj accepted\n"); ++g_fail; }
  expect("proj dm", larard_proj_bwd(fake(), ffake(), 1, 100, 200, 2, 128, ffake(), ffake(), fake(), size_t(1) << 30,
                                    ffake(), nullptr), LARARD_E_UNSUPPORTED);
  expect("proj tables", larard_proj_bwd(fake(), ffake(), 1, 100, 256, 2, 128, ffake(), nullptr, fake(),
                                        size_t(1) << 30, ffake(), nullptr), LARARD_E_INVALID);

  // strings
  for (int s = 0; s <= 5; ++s)
    if (larard_status_str(static_cast<larard_status>(s)) == nullptr) { std::printf("FAIL status string\n"); ++g_fail; }
  if (std::strstr(larard_version(), "gfx950") == nullptr) { std::printf("FAIL version\n"); ++g_fail; }

  std::printf("%s: %d failure(s)\n", g_fail ? "FAILED" : "OK", g_fail);
  return g_fail ? 1 : 0;
}
