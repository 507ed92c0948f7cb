// Host-only driver of the C-ABI layer (csrc/mla_api.cpp) for a build with
// AddressSanitizer and UndefinedBehaviorSanitizer (g++, no device code).  The
// kernel launchers are stubs that report failure: every case here must be
// decided on the host before any launch.  Prints one line per case and exits
// non-zero on the first unexpected status.
#include <cstdint>
#include <cstdio>
#include <cstring>
#include <vector>

#include "mla_decode.h"
#include "../../mla_paged_kv_metadata_amd/csrc/mla_kernels.h"

namespace mla {
hipError_t launch_metadata(const int32_t *, int, int, int, int32_t *, int32_t *, hipStream_t) {
  return hipErrorNotSupported;
}
hipError_t launch_decode(const DecodeArgs &, hipStream_t) { return hipErrorNotSupported; }
hipError_t launch_combine(const DecodeArgs &, hipStream_t) { return hipErrorNotSupported; }
hipError_t noalloc_scratch(void **) { return hipErrorNotSupported; }
hipError_t launch_lds_dma_read(const void *, size_t, hipStream_t) { return hipErrorNotSupported; }
}  // namespace mla

namespace {
int g_fail = 0;
void expect(const char *name, int got, int want) {
  const char *txt = mla_status_str(got);
  std::printf("%-44s status %d (%s)\n", name, got, txt ? txt : "(null)");
  if (got != want) {
    std::printf("  expected %d\n", want);
    g_fail = 1;
  }
}

struct Args {
  uintptr_t q = 1, kv = 1, bt = 1, sl = 1, md = 1, ns = 1, ws = 1, out = 1, lse = 1;
  int batch = 2, s_q = 1, hq = 16, d = 576, dt = 0, nb = 8, page = 64, hk = 1, maxb = 5, dv = 512, causal = 0,
      parts = 4;
  float scale = 1.0f / 24, vs = 1.0f;
  size_t wsb = (size_t)1 << 30;
};
int decode(const Args &a) {
  return mla_decode_fwd((const void *)a.q, a.batch, a.s_q, a.hq, a.d, (const void *)a.kv, a.dt, a.nb, a.page, a.hk,
                        (const int32_t *)a.bt, a.maxb, (const int32_t *)a.sl, a.dv, a.scale, a.vs, a.causal,
                        (const int32_t *)a.md, a.parts, (const int32_t *)a.ns, (void *)a.ws, a.wsb, (void *)a.out,
                        (float *)a.lse, nullptr);
}
int noalloc(const Args &a) {
  return mla_decode_fwd_noalloc((const void *)a.q, a.batch, a.s_q, a.hq, a.d, (const void *)a.kv, a.dt, a.nb,
                                a.page, a.hk, (const int32_t *)a.bt, a.maxb, (const int32_t *)a.sl, a.dv, a.scale,
                                a.vs, a.causal, (const int32_t *)a.md, a.parts, (const int32_t *)a.ns,
                                (void *)a.out, (float *)a.lse, nullptr);
}
}  // namespace

int main() {
  for (int s = -1; s < 8; ++s) expect("status string", mla_status_str(s) ? 0 : 1, 0);
  int np = 0;
  expect("num_parts NULL", mla_num_parts(2, 16, 1, nullptr), MLA_ERR_INVALID_ARG);
  expect("num_parts batch 0", mla_num_parts(0, 16, 1, &np), MLA_ERR_INVALID_ARG);
  expect("num_parts rows > max", mla_num_parts(2, MLA_MAX_ROWS + 1, 1, &np), MLA_ERR_UNSUPPORTED);
  size_t bytes = 0;
  expect("workspace_bytes ok", mla_workspace_bytes(64, 1, 128, 1, 512, 256, &bytes), MLA_OK);
  expect("workspace_bytes NULL", mla_workspace_bytes(64, 1, 128, 1, 512, 256, nullptr), MLA_ERR_INVALID_ARG);
  expect("workspace_bytes heads", mla_workspace_bytes(2, 1, 6, 4, 512, 8, &bytes), MLA_ERR_INVALID_ARG);
  std::vector<int32_t> dummy(64, 0);
  expect("metadata NULL seqlens",
         mla_get_metadata(nullptr, 2, 16, 1, dummy.data(), 4, dummy.data(), nullptr), MLA_ERR_INVALID_ARG);
  expect("metadata parts 0", mla_get_metadata_ex(dummy.data(), 2, 16, 1, 0, 4, dummy.data(), dummy.data(), nullptr),
         MLA_ERR_INVALID_ARG);
  expect("metadata fixed cost 0",
         mla_get_metadata_ex(dummy.data(), 2, 16, 1, 4, 0, dummy.data(), dummy.data(), nullptr), MLA_ERR_INVALID_ARG);
  struct Case {
    const char *name;
    void (*edit)(Args &);
    int want;
  } cases[] = {
      {"q NULL", [](Args &a) { a.q = 0; }, MLA_ERR_INVALID_ARG},
      {"out NULL", [](Args &a) { a.out = 0; }, MLA_ERR_INVALID_ARG},
      {"batch 0", [](Args &a) { a.batch = 0; }, MLA_ERR_INVALID_ARG},
      {"heads not divisible", [](Args &a) { a.hq = 6; a.hk = 4; }, MLA_ERR_INVALID_ARG},
      {"causal 2", [](Args &a) { a.causal = 2; }, MLA_ERR_INVALID_ARG},
      {"scale NaN", [](Args &a) { a.scale = __builtin_nanf(""); }, MLA_ERR_INVALID_ARG},
      {"scale inf", [](Args &a) { a.scale = __builtin_inff(); }, MLA_ERR_INVALID_ARG},
      {"scale negative", [](Args &a) { a.scale = -0.5f; }, MLA_ERR_UNSUPPORTED},
      {"head_dim 192", [](Args &a) { a.d = 192; }, MLA_ERR_UNSUPPORTED},
      {"head_dim_v 128", [](Args &a) { a.dv = 128; }, MLA_ERR_UNSUPPORTED},
      {"page 24", [](Args &a) { a.page = 24; }, MLA_ERR_UNSUPPORTED},
      {"page 0", [](Args &a) { a.page = 0; }, MLA_ERR_INVALID_ARG},
      {"kv dtype 7", [](Args &a) { a.dt = 7; }, MLA_ERR_UNSUPPORTED},
      {"rows > max", [](Args &a) { a.s_q = 9; a.hq = 128; }, MLA_ERR_UNSUPPORTED},
      {"batch > max", [](Args &a) { a.batch = MLA_MAX_BATCH + 1; }, MLA_ERR_UNSUPPORTED},
      {"workspace small", [](Args &a) { a.wsb = 16; }, MLA_ERR_WORKSPACE_TOO_SMALL},
      {"workspace NULL", [](Args &a) { a.ws = 0; }, MLA_ERR_WORKSPACE_TOO_SMALL},
      {"rows past 2^31", [](Args &a) { a.batch = 8192; a.s_q = 8; a.hq = 32768; a.hk = 256; },
       MLA_ERR_UNSUPPORTED},
  };
  for (const Case &c : cases) {
    Args a;
    c.edit(a);
    expect(c.name, decode(a), c.want);
  }
  Args big;
  big.batch = 4096;
  big.s_q = 8;
  big.hq = 128;
  big.parts = 256;
  expect("noalloc oversized", noalloc(big), MLA_ERR_WORKSPACE_TOO_SMALL);
  Args zero;
  zero.batch = 0;
  expect("noalloc batch 0", noalloc(zero), MLA_ERR_INVALID_ARG);
  // A valid request reaches the device gate: with no GPU it is NO_DEVICE; on
  // a GPU host the stub launcher makes it MLA_ERR_HIP.  Either way no
  // sanitizer report may appear.
  Args ok;
  const int rc = decode(ok);
  std::printf("%-44s status %d (%s)\n", "valid request (device gate)", rc, mla_status_str(rc));
  if (rc != MLA_ERR_NO_DEVICE && rc != MLA_ERR_HIP && rc != MLA_ERR_UNSUPPORTED) g_fail = 1;
  std::printf(g_fail ? "FAILED\n" : "ALL OK\n");
  return g_fail;
}
