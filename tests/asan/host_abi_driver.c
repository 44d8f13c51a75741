/*
 * Host-side driver of the C ABI for a sanitizer build of the library's host
 * layer (AddressSanitizer + UndefinedBehaviorSanitizer on the host code only).
 *
 * Every call here stops in host validation or in a failing HIP call (the
 * build machine has no GPU): pointers are fake and never dereferenced, so the
 * run exercises argument checking, size arithmetic, status strings and the
 * HIP-error paths under the sanitizers.  Prints "ALL OK" and exits 0 when
 * every status matches the header's documentation.
 */
#include <stdint.h>
#include <stdio.h>
#include <string.h>

#include "mla_decode.h"

static int failures = 0;

#define EXPECT(cond, what)                                   \
  do {                                                       \
    if (!(cond)) {                                           \
      ++failures;                                            \
      fprintf(stderr, "FAIL line %d: %s\n", __LINE__, what); \
    }                                                        \
  } while (0)

#define P(v) ((void*)(uintptr_t)(v))

struct fwd_args {
  uintptr_t q, kc, bt, sl, tm, so, ws, out, lse;
  int64_t nblk;
  int bt_stride, batch, s_q, h_q, h_kv, causal, parts;
  float scale;
  size_t ws_bytes;
};

static struct fwd_args fwd_ok(void) {
  struct fwd_args a = {16, 16, 16, 16, 16, 16, 256, 16, 16, 8, 2, 2, 1, 16, 1, 0, 4, 0.04f,
                       (size_t)1 << 30};
  return a;
}

static int call_fwd(const struct fwd_args* a, int fp8) {
  if (fp8)
    return mla_decode_fwd_fp8(P(a->q), P(a->kc), a->nblk, (const int32_t*)P(a->bt), a->bt_stride,
                              (const int32_t*)P(a->sl), a->batch, a->s_q, a->h_q, a->h_kv,
                              a->scale, a->causal, (const int32_t*)P(a->tm),
                              (const int32_t*)P(a->so), a->parts, P(a->ws), a->ws_bytes,
                              P(a->out), (float*)P(a->lse), NULL);
  return mla_decode_fwd(P(a->q), P(a->kc), a->nblk, (const int32_t*)P(a->bt), a->bt_stride,
                        (const int32_t*)P(a->sl), a->batch, a->s_q, a->h_q, a->h_kv, a->scale,
                        a->causal, (const int32_t*)P(a->tm), (const int32_t*)P(a->so), a->parts,
                        P(a->ws), a->ws_bytes, P(a->out), (float*)P(a->lse), NULL);
}

static void fwd_rejects(int fp8) {
  struct fwd_args a;
  const float nan = __builtin_nanf(""), inf = __builtin_inff();
#define CASE(field, value, expect)                              \
  a = fwd_ok();                                                 \
  a.field = value;                                              \
  EXPECT(call_fwd(&a, fp8) == (expect), #field " = " #value);
  CASE(q, 0, MLA_ERR_INVALID_ARG)
  CASE(kc, 0, MLA_ERR_INVALID_ARG)
  CASE(bt, 0, MLA_ERR_INVALID_ARG)
  CASE(sl, 0, MLA_ERR_INVALID_ARG)
  CASE(tm, 0, MLA_ERR_INVALID_ARG)
  CASE(so, 0, MLA_ERR_INVALID_ARG)
  CASE(out, 0, MLA_ERR_INVALID_ARG)
  CASE(lse, 0, MLA_ERR_INVALID_ARG)
  CASE(q, 8, MLA_ERR_INVALID_ARG)
  CASE(kc, 4, MLA_ERR_INVALID_ARG)
  CASE(out, 8, MLA_ERR_INVALID_ARG)
  CASE(lse, 2, MLA_ERR_INVALID_ARG)
  CASE(ws, 128, MLA_ERR_INVALID_ARG)
  CASE(ws, 0, MLA_ERR_INVALID_ARG)
  CASE(batch, 0, MLA_ERR_INVALID_ARG)
  CASE(s_q, 129, MLA_ERR_INVALID_ARG)
  CASE(s_q, 0, MLA_ERR_INVALID_ARG)
  CASE(h_kv, 2, MLA_ERR_INVALID_ARG)
  CASE(h_q, 48, MLA_ERR_UNSUPPORTED)
  CASE(h_q, 8, MLA_ERR_UNSUPPORTED)
  CASE(parts, 0, MLA_ERR_INVALID_ARG)
  CASE(nblk, 0, MLA_ERR_INVALID_ARG)
  CASE(bt_stride, 0, MLA_ERR_INVALID_ARG)
  CASE(scale, nan, MLA_ERR_INVALID_ARG)
  CASE(scale, inf, MLA_ERR_INVALID_ARG)
  CASE(causal, 2, MLA_ERR_INVALID_ARG)
  CASE(ws_bytes, 1024, MLA_ERR_WORKSPACE)
#undef CASE
  /* valid arguments: no device here, so the launch fails with a HIP error */
  a = fwd_ok();
  const int st = call_fwd(&a, fp8);
  EXPECT(st == MLA_ERR_HIP, "valid arguments without a device give MLA_ERR_HIP");
  EXPECT(strlen(mla_last_hip_error()) > 0, "the HIP error text is kept");
}

int main(void) {
  int parts = 0;
  size_t bytes = 0;
  EXPECT(mla_decode_num_parts(64, 1, 16, 1, 256, &parts) == MLA_OK && parts == 256, "num_parts 64x16");
  EXPECT(mla_decode_num_parts(2, 129, 16, 1, 256, &parts) == MLA_ERR_INVALID_ARG, "num_parts s_q 129");
  EXPECT(mla_decode_num_parts(2, 1, 48, 1, 256, &parts) == MLA_ERR_UNSUPPORTED, "num_parts h_q 48");
  EXPECT(mla_decode_num_parts(2, 1, 16, 1, 0, &parts) == MLA_ERR_INVALID_ARG, "num_parts 0 CUs");
  EXPECT(mla_decode_num_parts(2, 1, 16, 1, 256, NULL) == MLA_ERR_INVALID_ARG, "num_parts NULL out");
  EXPECT(mla_decode_workspace_bytes(4, 1, 16, 1, &bytes) == MLA_OK && bytes == 0, "workspace 1 part");
  EXPECT(mla_decode_workspace_bytes(4, 1, 16, 256, &bytes) == MLA_OK &&
             bytes >= (size_t)2 * 255 * 16 * (512 * 2 + 4) && bytes % 256 == 0,
         "workspace 256 parts");
  EXPECT(mla_decode_workspace_bytes(4, 1, 16, (1 << 16) + 1, &bytes) == MLA_ERR_INVALID_ARG,
         "workspace beyond the part cap");
  EXPECT(mla_decode_workspace_bytes(4, 1, 16, 4, NULL) == MLA_ERR_INVALID_ARG, "workspace NULL out");

  fwd_rejects(0);
  fwd_rejects(1);

  EXPECT(mla_decode_metadata((const int32_t*)P(16), 2, 1, 16, 1, 32, 4, (int32_t*)P(16),
                             (int32_t*)P(16), NULL) == MLA_ERR_INVALID_ARG, "metadata block size");
  EXPECT(mla_decode_metadata(NULL, 2, 1, 16, 1, 64, 4, (int32_t*)P(16), (int32_t*)P(16), NULL) ==
             MLA_ERR_INVALID_ARG, "metadata NULL seqlens");
  EXPECT(mla_decode_metadata((const int32_t*)P(18), 2, 1, 16, 1, 64, 4, (int32_t*)P(16),
                             (int32_t*)P(16), NULL) == MLA_ERR_INVALID_ARG, "metadata misaligned");
  EXPECT(mla_decode_combine((const int32_t*)P(16), 2, 1, 16, (const int32_t*)P(16), 4, P(256), 10,
                            P(16), (float*)P(16), NULL) == MLA_ERR_WORKSPACE, "combine workspace");
  EXPECT(mla_kv_append(NULL, P(16), 8, (const int32_t*)P(16), 2, (const int32_t*)P(16), 2, 1, NULL) ==
             MLA_ERR_INVALID_ARG, "append NULL rows");
  EXPECT(mla_kv_append_fp8(P(16), P(8), 8, (const int32_t*)P(16), 2, (const int32_t*)P(16), 2, 1,
                           NULL) == MLA_ERR_INVALID_ARG, "append fp8 misaligned");

  EXPECT(mla_decode_sparse_workspace_bytes(2, 1, 64, 48, 4, &bytes) == MLA_ERR_INVALID_ARG,
         "sparse topk not a multiple of 32");
  EXPECT(mla_decode_sparse_workspace_bytes(2, 1, 64, 128, 4, &bytes) == MLA_OK && bytes > 0,
         "sparse workspace");
  EXPECT(mla_decode_sparse_fwd(P(16), P(16), 8, (const int32_t*)P(16), 2, (const int32_t*)P(16), 2,
                               1, 64, 1, 0.04f, 0, (const int32_t*)P(16), 40,
                               (const int32_t*)P(16), (const int32_t*)P(16), 4, P(256),
                               (size_t)1 << 30, P(16), (float*)P(16), NULL, NULL, NULL) ==
             MLA_ERR_INVALID_ARG, "sparse fwd topk 40");

  EXPECT(mla_decode_fwd_noalloc(P(16), P(16), 8, (const int32_t*)P(16), 2, (const int32_t*)P(16),
                                MLA_NOALLOC_MAX_BATCH + 1, 1, 16, 1, 0.04f, 0, P(16),
                                (float*)P(16), NULL) == MLA_ERR_INVALID_ARG, "noalloc batch cap");

  EXPECT(mla_device_num_cus(0, NULL) == MLA_ERR_INVALID_ARG, "num_cus NULL out");
  for (int st = 0; st >= -4; --st)
    EXPECT(strncmp(mla_status_string(st), "MLA_", 4) == 0, "status string");
  EXPECT(strcmp(mla_status_string(12345), "unknown status") == 0, "unknown status string");

  if (failures) {
    fprintf(stderr, "%d failure(s)\n", failures);
    return 1;
  }
  printf("ALL OK\n");
  return 0;
}
