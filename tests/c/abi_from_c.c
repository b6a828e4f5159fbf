/* The C ABI used from plain C (no Python, no HIP headers): the header compiles as C11, the
 * program links against libulysses.so, and the host-side checks answer without a GPU. */
#include <stdio.h>
#include <string.h>

#include "ulysses.h"

static int fails = 0;
#define EXPECT(cond)                                              \
  do {                                                            \
    if (!(cond)) {                                                \
      fprintf(stderr, "%s:%d: %s\n", __FILE__, __LINE__, #cond); \
      ++fails;                                                    \
    }                                                             \
  } while (0)

int main(void) {
  /* a fake, 16-byte aligned device address: only host-side checks run on it */
  void* fake = (void*)(uintptr_t)0x100000;
  const void* shards[2] = {fake, fake};
  void* out_shards[2] = {fake, fake};
  EXPECT(uly_abi_version() >= 1);
  EXPECT(strcmp(uly_status_string(ULY_OK), "ULY_OK") == 0);
  EXPECT(strcmp(uly_status_string(ULY_ERR_SHAPE), "ULY_ERR_SHAPE") == 0);
  /* null pointers, bad shapes, unsupported head dims: rejected before any launch */
  EXPECT(attn_fwd(NULL, fake, fake, fake, NULL, (float*)fake, 16, 4, 2, 128, ULY_BF16, 0.1f, 1, NULL, 0, NULL, 0, NULL) ==
         ULY_ERR_NULL);
  EXPECT(attn_fwd(fake, fake, fake, fake, NULL, (float*)fake, 16, 3, 2, 128, ULY_BF16, 0.1f, 1, NULL, 0, NULL, 0, NULL) ==
         ULY_ERR_SHAPE);
  EXPECT(attn_fwd(fake, fake, fake, fake, NULL, (float*)fake, 16, 4, 2, 96, ULY_BF16, 0.1f, 1, NULL, 0, NULL, 0, NULL) ==
         ULY_ERR_UNSUPPORTED);
  EXPECT(ulysses_pack(shards, 2, 2, 4, 4, 64, ULY_BF16, fake, NULL) == ULY_ERR_SHAPE);
  EXPECT(ulysses_unpack(fake, 2, 0, 4, ULY_MAX_HEADS + 2, 64, ULY_BF16, out_shards, NULL) == ULY_ERR_SHAPE);
  /* a workspace query needs no device */
  EXPECT(attn_bwd_workspace_bytes(65536, 8, 2, 128) >= (size_t)65536 * 8 * sizeof(float));
  EXPECT(attn_fwd_workspace_bytes(65536, 8, 128) == 0);
  EXPECT(attn_fwd_workspace_bytes(8192, 8, 128) > 0);
  if (fails == 0) printf("c abi ok\n");
  return fails != 0;
}
