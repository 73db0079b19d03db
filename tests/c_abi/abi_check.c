/*
 * A plain C99 caller of the library's C ABI: compiles against the public
 * headers (add_rmsnorm.h, log1p_f32.h) with no C++ and no HIP headers, links libaddrmsnorm.so, and exercises what
 * needs no GPU (host-side validation, zero-size calls, identity and status
 * queries).  Prints "ok" and returns 0 when every check holds, else names
 * the first failing check and returns 1.
 */
#include <stdint.h>
#include <stdio.h>
#include <string.h>

#include "add_rmsnorm.h"
#include "log1p_f32.h"

#define CHECK(cond)                                       \
  do {                                                    \
    if (!(cond)) {                                        \
      printf("failed: %s (line %d)\n", #cond, __LINE__);  \
      return 1;                                           \
    }                                                     \
  } while (0)

int main(void) {
  /* fake, 16-byte aligned device addresses: only validation ever sees them */
  uint16_t* const out = (uint16_t*)(uintptr_t)0x100000;
  uint16_t* const ro = (uint16_t*)(uintptr_t)0x2100000;
  const uint16_t* const x = (const uint16_t*)(uintptr_t)0x4100000;
  const uint16_t* const r = (const uint16_t*)(uintptr_t)0x6100000;
  const uint16_t* const w = (const uint16_t*)(uintptr_t)0x8100000;
  const char* info = add_rmsnorm_build_info();
  struct add_rmsnorm_launch_cfg cfg = {ADD_RMSNORM_PATH_PACKED, 0, 0, 3};
  int s;

  CHECK(add_rmsnorm_abi_version() == ADD_RMSNORM_ABI_VERSION);
  CHECK(info != NULL && strstr(info, "arch=gfx950") != NULL);
  for (s = ADD_RMSNORM_EHIP; s <= ADD_RMSNORM_OK; ++s)
    CHECK(add_rmsnorm_strerror(s) != NULL && add_rmsnorm_strerror(s)[0] != '\0');

  /* zero rows: nothing checked beyond the scalars, nothing enqueued */
  CHECK(add_rmsnorm_fwd(NULL, NULL, NULL, NULL, NULL, 0, 4096, 1e-6f, NULL) == ADD_RMSNORM_OK);
  CHECK(rmsnorm_fwd(NULL, NULL, NULL, 0, 128, 1e-6f, NULL) == ADD_RMSNORM_OK);
  CHECK(qk_rmsnorm_fwd(NULL, NULL, NULL, NULL, NULL, NULL, 0, 32, 8, 128, 4096, 1024, 4096, 1024,
                       1e-6f, NULL) == ADD_RMSNORM_OK);
  CHECK(log1p_f32(NULL, NULL, 0, NULL) == 0);

  /* host-side errors */
  CHECK(add_rmsnorm_fwd(out, ro, x, r, w, 4, 0, 1e-6f, NULL) == ADD_RMSNORM_EINVAL);
  CHECK(add_rmsnorm_fwd(out, ro, x, r, w, 4, 64, -1.0f, NULL) == ADD_RMSNORM_EINVAL);
  CHECK(add_rmsnorm_fwd(out, ro, x, r, w, 4, 40000, 1e-6f, NULL) == ADD_RMSNORM_ERANGE);
  CHECK(add_rmsnorm_fwd(out, (uint16_t*)x + 8, x, r, w, 4, 64, 1e-6f, NULL) ==
        ADD_RMSNORM_EALIAS); /* residual_out partly over x */
  CHECK(add_rmsnorm_fwd_cfg(out, ro, x, r, w, 4, 64, 1e-6f, &cfg, NULL) == ADD_RMSNORM_EINVAL);
  CHECK(qk_rmsnorm_fwd(out, ro, x, r, w, w, 4, 32, 8, 12, 384, 96, 384, 96, 1e-6f, NULL) ==
        ADD_RMSNORM_EALIGN);
  CHECK(qk_rmsnorm_fwd(out, ro, x, r, w, w, 4, 32, 8, 520, 32 * 520, 8 * 520, 32 * 520,
                       8 * 520, 1e-6f, NULL) == ADD_RMSNORM_ERANGE);
  CHECK(add_rmsnorm_quant_fwd((int8_t*)out, (float*)ro, (uint16_t*)r + 0x800000, x, r, w, 4, 12,
                              1e-6f, NULL) == ADD_RMSNORM_EALIGN);
  printf("ok\n");
  return 0;
}
