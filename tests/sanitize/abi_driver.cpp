// Sanitizer driver for the C-ABI validation of libmamba_scan (test
// infrastructure): built with AddressSanitizer and UndefinedBehaviorSanitizer
// on the host side of the library, it calls every entry point with arguments
// that validation must refuse (NULL, misaligned, overlapping, out-of-range
// and extreme dims, including values whose products overflow 32 bits) and
// checks the status. Calls that pass validation reach the device check; they
// are made only when no GPU is visible (then they must fail with
// MAMBA_ERR_DEVICE), so no fake address is ever handed to a kernel.
#include <hip/hip_runtime.h>
#include <stdint.h>
#include <stdio.h>
#include <string.h>

#include <climits>
#include <initializer_list>

#include "mamba2_ssd.h"
#include "mamba_scan.h"
#include "mamba_scan_testing.h"

namespace {

int fails = 0;
void expect(int got, int want, const char* what) {
  if (got != want) {
    fprintf(stderr, "%s: status %d (%s), expected %d\n", what, got, mamba_scan_last_error(), want);
    ++fails;
  }
}

// Fake device addresses, far apart and never dereferenced.
char* const P = reinterpret_cast<char*>(uintptr_t{0x7F0000000000});
void* at(uintptr_t off) { return P + off; }
float* fat(uintptr_t off) { return reinterpret_cast<float*>(P + off); }

struct Fwd {
  int32_t b = 2, L = 8, d = 64, n = 16, k = 4, io = 0;
  void *x = at(0), *dt = at(0x10000000), *z = at(0x20000000), *B = at(0x30000000), *C = at(0x40000000);
  float *w = fat(0x50000000), *cb = fat(0x60000000), *db = fat(0x70000000), *D = fat(0x80000000), *A = fat(0x90000000);
  float *cs = nullptr, *ss = nullptr;
  void* y = at(0xA0000000);
  float *cso = fat(0xB0000000), *sso = fat(0xC0000000);
  int call() const {
    return mamba_scan_fwd(b, L, d, n, k, io, x, dt, z, B, C, w, cb, db, D, A, cs, ss, y, cso, sso, nullptr, 0,
                          nullptr);
  }
  int noalloc() const {
    return mamba_scan_fwd_noalloc(b, L, d, n, k, io, x, dt, z, B, C, w, cb, db, D, A, cs, ss, y, cso, sso, nullptr);
  }
  int seq(const int32_t* s) const {
    return mamba_scan_fwd_seq(b, L, d, n, k, io, x, dt, z, B, C, s, w, cb, db, D, A, cs, ss, y, cso, sso, nullptr, 0,
                              nullptr);
  }
  int testing(int kind) const {
    return mamba_scan_testing_fwd(kind, 0, b, L, d, n, k, io, x, dt, z, B, C, nullptr, w, cb, db, D, A, cs, ss, y, cso,
                                  sso, nullptr, nullptr, 0, nullptr);
  }
  int step() const {
    return mamba_scan_step(b, d, n, k, io, x, dt, z, B, C, w, cb, db, D, A, fat(0xD0000000), fat(0xE0000000), y, cso,
                           sso, nullptr);
  }
  int bwd() const {
    return mamba_scan_bwd(b, L, d, n, k, io, x, dt, z, B, C, w, cb, db, D, A, cs, ss, at(0xD0000000), at(0xE0000000),
                          at(0xF0000000), at(0x100000000), fat(0x110000000), fat(0x120000000), fat(0x130000000),
                          fat(0x140000000), fat(0x150000000), fat(0x160000000), fat(0x170000000), nullptr, 0, nullptr);
  }
};

}  // namespace

int main() {
  int devices = 0;
  if (hipGetDeviceCount(&devices) != hipSuccess) devices = 0;
  (void)hipGetLastError();

  // status strings and the error text of a fresh thread
  for (int s = -3; s < 12; ++s) (void)strlen(mamba_scan_status_str(s));
  (void)strlen(mamba_scan_last_error());
  (void)mamba_scan_call_count();

  // workspace queries at extreme and invalid dims: 0 and no overflow
  const int32_t vals[] = {INT32_MIN, -1, 0, 1, 7, 16, 64, 1 << 16, (1 << 24) + 1, 1 << 30, INT32_MAX};
  for (int32_t b : vals)
    for (int32_t L : vals)
      for (int32_t d : vals)
        for (int32_t n : {8, 16, 12}) {
          (void)mamba_scan_fwd_workspace_bytes(b, L, d, n, 1);
          (void)mamba_scan_testing_fwd_workspace_bytes(1, b, L, d, n, 0);
          (void)mamba_scan_bwd_workspace_bytes(b, L, d, n, 1);
          (void)mamba_scan_bwd_ckpt_workspace_bytes(b, L, d, n, 1);
          (void)mamba_scan_ckpt_bytes(b, L, d, n);
          (void)mamba2_ssd_fwd_workspace_bytes(b, L, d, 64, n == 8 ? 64 : 128, 1, 1);
        }

  Fwd f;
  // refused before any HIP call
  for (auto over : {0, 1, 2, 3, 4, 5, 6, 7, 8, 9, 10, 11}) {
    Fwd g = f;
    int want = MAMBA_ERR_SHAPE;
    switch (over) {
      case 0: g.b = 0; break;
      case 1: g.L = INT32_MAX; g.b = INT32_MAX; break;                    // product past 2^31
      case 2: g.d = (1 << 24) + 1; g.b = 1; g.L = 16; break;              // prefill d_inner cap
      case 3: g.k = 3; break;
      case 4: g.n = 12; break;
      case 5: g.io = 9; want = MAMBA_ERR_DTYPE; break;
      case 6: g.x = nullptr; want = MAMBA_ERR_NULL; break;
      case 7: g.io = 1; g.z = static_cast<char*>(g.z) + 1; want = MAMBA_ERR_ALIGN; break;
      case 8: g.y = g.x; want = MAMBA_ERR_ALIAS; break;
      case 9: g.cso = g.w; want = MAMBA_ERR_ALIAS; break;
      case 10: g.ss = fat(0xF0000000); g.sso = fat(0xF0000004); want = MAMBA_ERR_ALIAS; break;
      default: g.b = INT32_MIN; break;
    }
    expect(g.call(), want, "fwd");
    expect(g.noalloc(), want, "fwd_noalloc");
    expect(g.testing(-1), want, "testing_fwd");
  }
  expect(f.seq(nullptr), MAMBA_ERR_NULL, "fwd_seq without ids");
  expect(f.testing(7), MAMBA_ERR_SHAPE, "testing_fwd unknown kind");
  {
    Fwd g = f;
    g.io = 1;
    expect(mamba_scan_fwd(1, 4096, 100, 16, 4, 1, g.x, g.dt, g.z, g.B, g.C, g.w, g.cb, g.db, g.D, g.A, nullptr,
                          nullptr, g.y, g.cso, g.sso, nullptr, 0, nullptr),
           MAMBA_ERR_WORKSPACE, "fwd without its workspace");
  }
  {
    Fwd g = f;
    g.d = INT32_MAX;
    expect(g.step(), MAMBA_ERR_SHAPE, "step huge");
    g = f;
    g.x = nullptr;
    expect(g.step(), MAMBA_ERR_NULL, "step null");
    g = f;
    g.n = 8;
    expect(g.bwd(), MAMBA_ERR_SHAPE, "bwd d_state 8");
    g = f;
    expect(g.bwd(), MAMBA_ERR_WORKSPACE, "bwd without workspace");
  }
  // SSD
  expect(mamba2_ssd_fwd(1, 16, 4, 32, 128, 1, 1, at(0), at(0x10000000), at(0x20000000), at(0x30000000),
                        fat(0x40000000), fat(0x50000000), fat(0x60000000), nullptr, at(0x70000000), nullptr, nullptr,
                        0, nullptr),
         MAMBA_ERR_SHAPE, "ssd headdim 32");
  expect(mamba2_ssd_fwd(INT32_MAX, INT32_MAX, 4, 64, 128, 1, 1, at(0), at(0x10000000), at(0x20000000),
                        at(0x30000000), fat(0x40000000), fat(0x50000000), fat(0x60000000), nullptr, at(0x70000000),
                        nullptr, nullptr, 0, nullptr),
         MAMBA_ERR_SHAPE, "ssd huge");
  expect(mamba2_ssd_step(2, 4, 64, 128, 3, 1, at(0), at(0x10000000), at(0x20000000), at(0x30000000),
                         fat(0x40000000), fat(0x50000000), fat(0x60000000), fat(0x70000000), at(0x80000000),
                         fat(0x90000000), nullptr),
         MAMBA_ERR_SHAPE, "ssd step groups");

  // valid arguments reach the device check; only without a GPU (never a
  // fake address on a real device)
  if (devices == 0) {
    expect(f.call(), MAMBA_ERR_DEVICE, "fwd without a device");
    expect(f.noalloc(), MAMBA_ERR_DEVICE, "fwd_noalloc without a device");
    expect(f.step(), MAMBA_ERR_DEVICE, "step without a device");
  }
  if (fails) return 1;
  printf("abi driver ok\n");
  return 0;
}
