/* A plain C caller of the library: include/fbd.h compiles as ISO C99 and
 * every entry point used here links against libfbd.so.  Only calls that the
 * host-side argument checks reject are made (nothing is enqueued), so this
 * runs without a GPU.  Exit status 0 when every check holds; otherwise it
 * prints the first failed check and exits with 1. */
#include <stdint.h>
#include <stdio.h>
#include <string.h>

#include "fbd.h"

static int failures = 0;

static void expect(int cond, const char* what) {
  if (!cond && failures++ == 0) fprintf(stderr, "check_abi: failed: %s\n", what);
}

int main(void) {
  /* distinct, 256-byte aligned stand-ins for device pointers: the argument
   * checks look at their values only */
  char* base = (char*)(uintptr_t)0x100000000ull;
  void* Q = base + (1u << 24);
  void* K = base + (2u << 24);
  void* V = base + (3u << 24);
  void* O = base + (4u << 24);
  float* LSE = (float*)(base + (5u << 24));
  void* dO = base + (6u << 24);
  void* out[4] = {base + (7u << 24), base + (8u << 24), base + (9u << 24), base + (10u << 24)};
  void* ws = base + (11u << 24);

  /* workspace sizes: fp32 row arrays of B*H*N rows (3 for the backward, 5 for
   * backward-over-backward, 6 for the Hessian-vector product), 0 for sizes <= 0 */
  expect(attn_bwd_workspace_bytes(2, 3, 5) == 3u * 2 * 3 * 5 * 4, "bwd workspace size");
  expect(attn_bob_workspace_bytes(2, 3, 5) == 5u * 2 * 3 * 5 * 4, "bob workspace size");
  expect(attn_hvp_workspace_bytes(2, 3, 5) == 6u * 2 * 3 * 5 * 4, "hvp workspace size");
  expect(attn_bwd_workspace_bytes(0, 3, 5) == 0, "empty workspace size");

  /* the forward's checks, in the order the header lists them */
  expect(attn_fwd(ATTN_BF16, 1, 2, 8, 64, NULL, K, V, 1, 0.125f, O, LSE, NULL) == ATTN_EINVAL,
         "null Q");
  expect(attn_fwd(ATTN_BF16, 1, 2, 0, 64, Q, K, V, 1, 0.125f, O, LSE, NULL) == ATTN_EINVAL,
         "N = 0");
  expect(attn_fwd(ATTN_BF16, 1, 2, 8, 32, Q, K, V, 1, 0.125f, O, LSE, NULL) ==
             ATTN_EUNSUPPORTED,
         "d = 32");
  expect(attn_fwd((attn_dtype)7, 1, 2, 8, 64, Q, K, V, 1, 0.125f, O, LSE, NULL) ==
             ATTN_EUNSUPPORTED,
         "unknown dtype");
  expect(attn_fwd(ATTN_BF16, 1, 2, 8, 64, Q, K, V, 1, -1.0f, O, LSE, NULL) == ATTN_EINVAL,
         "negative scale");
  expect(attn_fwd(ATTN_BF16, 1, 2, 8, 64, (char*)Q + 8, K, V, 1, 0.125f, O, LSE, NULL) ==
             ATTN_EALIGN,
         "misaligned Q");
  expect(attn_fwd(ATTN_BF16, 1, 2, 8, 64, Q, K, V, 1, 0.125f, Q, LSE, NULL) == ATTN_EINVAL,
         "O overlapping Q");

  /* the backward and backward-over-backward: a short workspace */
  expect(attn_bwd(ATTN_BF16, 1, 2, 8, 64, Q, K, V, O, LSE, dO, 1, 0.125f, 1, out[0], out[1],
                  out[2], ws, attn_bwd_workspace_bytes(1, 2, 8) - 4, NULL) == ATTN_EWORKSPACE,
         "short backward workspace");
  expect(attn_bob(ATTN_BF16, 1, 2, 8, 64, Q, K, V, O, LSE, dO, out[0], out[1], out[2], 1,
                  0.125f, out[3], base + (12u << 24), base + (13u << 24), base + (14u << 24),
                  ws, attn_bob_workspace_bytes(1, 2, 8) - 4, NULL) == ATTN_EWORKSPACE,
         "short bob workspace");
  expect(attn_bob(ATTN_BF16, 1, 2, 8, 64, Q, K, V, O, LSE, dO, out[0], out[1], out[2], 1,
                  0.125f, out[3], base + (12u << 24), base + (13u << 24), base + (14u << 24),
                  NULL, attn_bob_workspace_bytes(1, 2, 8), NULL) == ATTN_EWORKSPACE,
         "null bob workspace");

  /* every status has a message */
  for (int s = ATTN_OK; s <= ATTN_EHIP; ++s) {
    const char* m = attn_status_str((attn_status)s);
    expect(m != NULL && strlen(m) > 0, "status message");
  }
  if (failures == 0) printf("check_abi: ok\n");
  return failures == 0 ? 0 : 1;
}
