/* A plain C99 consumer of the C ABI: it includes include/qil.h as C, links
 * against libqil.so and calls entry points whose argument checks fail before
 * any HIP call, so it runs on a host without a GPU.  Built and run by
 * tests/test_c_consumer.py; exit status 0 when every call returns the
 * documented code. */
#include <stdio.h>
#include <string.h>

#include "qil.h"

static int failures = 0;

static void expect(const char* what, int got, int want) {
  if (got != want) {
    printf("FAIL %s: returned %d, expected %d (%s)\n", what, got, want, qil_last_error());
    ++failures;
  } else {
    printf("ok   %s\n", what);
  }
}

int main(void) {
  void* fake = (void*)(uintptr_t)0x100000; /* 16-byte aligned, never dereferenced */
  const char* v = qil_version();
  if (v == NULL || strncmp(v, "qil ", 4) != 0) {
    printf("FAIL qil_version: %s\n", v ? v : "(null)");
    ++failures;
  }
  /* kv_write: a negative token count, then an empty call (a no-op) */
  expect("kv_write num_tokens=-1",
         qil_kv_write(fake, fake, 1024, 1024, fake, fake, fake, -1, 8, 128, 16, 10, QIL_BF16, NULL, NULL),
         QIL_EINVAL);
  expect("kv_write num_tokens=0",
         qil_kv_write(fake, fake, 1024, 1024, fake, fake, fake, 0, 8, 128, 16, 10, QIL_BF16, NULL, NULL),
         QIL_OK);
  /* decode: head_dim 64 is not supported; a page size of 48 neither */
  expect("paged_decode head_dim=64",
         qil_paged_decode(fake, fake, fake, fake, fake, 128, fake, 2, 16, 8, 64, 16, 8192, 2048,
                          0.088f, QIL_BF16, 0, NULL, 0, NULL),
         QIL_EUNSUPPORTED);
  expect("paged_decode page_size=48",
         qil_paged_decode(fake, fake, fake, fake, fake, 128, fake, 2, 16, 8, 128, 48, 8192, 2048,
                          0.088f, QIL_BF16, 0, NULL, 0, NULL),
         QIL_EUNSUPPORTED);
  /* prefill: 12 query heads over 8 KV heads is not a whole group */
  expect("paged_prefill Hq=12 Hkv=8",
         qil_paged_prefill(fake, fake, fake, fake, fake, 200, fake, fake, 8, 8000, 2048, 2560, 12, 8,
                           128, 16, 900, 0.088f, QIL_BF16, 0, NULL, 0, NULL),
         QIL_EINVAL);
  if (strlen(qil_last_error()) == 0) {
    printf("FAIL qil_last_error is empty after an error\n");
    ++failures;
  }
  return failures == 0 ? 0 : 1;
}
