/* Plain C99 client of the RACE attention C ABI: includes only the public
 * header, links the built library, and exercises the host-side contract
 * (size queries, argument checks, status strings) without touching a GPU.
 * Every call below must fail its host checks before anything is enqueued.
 * Prints "ok" and exits 0 on success. */
#include <stdint.h>
#include <stdio.h>
#include <string.h>

#include "race_attn.h"

static int failures = 0;

#define EXPECT(cond, what)                                                      \
  do {                                                                          \
    if (!(cond)) {                                                              \
      fprintf(stderr, "FAILED: %s (line %d)\n", what, __LINE__);                \
      ++failures;                                                               \
    }                                                                           \
  } while (0)

int main(void) {
  race_shape s;
  memset(&s, 0, sizeof s);
  s.B = 1; s.H = 4; s.N = 4096; s.d = 128; s.dtype = RACE_BF16; s.w_per_head = 0;

  /* non-causal state: B*H x LRP x (d + 1) float32 with LRP = 32 at P = 4, L = 2 */
  EXPECT(race_attn_state_bytes(&s, 4, 2, 0) == (size_t)4 * 32 * 129 * 4, "state bytes");
  const size_t wf = race_attn_workspace_bytes(&s, 4, 2, 0, 0);
  const size_t wb = race_attn_workspace_bytes(&s, 4, 2, 0, 1);
  const size_t ww = race_attn_workspace_bytes(&s, 4, 2, 0, 2);
  EXPECT(wf > 0 && wb > 0 && ww > wb, "workspace bytes (fwd, bwd, bwd with dW)");
  EXPECT(race_attn_workspace_bytes(&s, 4, 2, 0, 3) == 0, "workspace phase out of range");
  EXPECT(race_attn_state_bytes(&s, 0, 2, 0) == 0, "P = 0 rejected by the size query");
  EXPECT(race_attn_state_bytes(NULL, 4, 2, 0) == 0, "NULL shape rejected by the size query");

  /* argument checks: nothing below reaches the GPU */
  uintptr_t base = (uintptr_t)1 << 20;   /* aligned, never dereferenced */
  const void* Q = (const void*)(base);
  const void* K = (const void*)(base + ((uintptr_t)1 << 24));
  const void* V = (const void*)(base + ((uintptr_t)2 << 24));
  const float* W = (const float*)(base + ((uintptr_t)3 << 24));
  void* O = (void*)(base + ((uintptr_t)4 << 24));
  void* ws = (void*)(base + ((uintptr_t)5 << 24));

  EXPECT(race_attn_fwd(Q, K, V, W, 1.0f, 4, 2, 0, O, NULL, NULL, 0, ws, wf, NULL) == RACE_ERR_INVALID_ARG,
         "NULL shape");
  EXPECT(race_attn_fwd(NULL, K, V, W, 1.0f, 4, 2, 0, O, &s, NULL, 0, ws, wf, NULL) == RACE_ERR_INVALID_ARG,
         "NULL Q");
  EXPECT(race_attn_fwd(Q, K, V, W, 1.0f, 9, 2, 0, O, &s, NULL, 0, ws, wf, NULL) == RACE_ERR_INVALID_ARG, "P = 9");
  EXPECT(race_attn_fwd(Q, K, V, W, 1.0f, 4, 2, 0, (void*)Q, &s, NULL, 0, ws, wf, NULL) == RACE_ERR_INVALID_ARG,
         "O overlaps Q");
  EXPECT(race_attn_fwd(Q, K, V, W, 1.0f, 4, 2, 0, O, &s, NULL, 0, ws, 16, NULL) == RACE_ERR_WORKSPACE,
         "workspace too small");
  EXPECT(strlen(race_last_error()) > 0, "last error message set");
  s.d = 100;
  EXPECT(race_attn_fwd(Q, K, V, W, 1.0f, 4, 2, 0, O, &s, NULL, 0, ws, wf, NULL) == RACE_ERR_UNSUPPORTED,
         "d = 100 (not a multiple of 8) unsupported");
  s.d = 136;
  EXPECT(race_attn_fwd(Q, K, V, W, 1.0f, 4, 2, 0, O, &s, NULL, 0, ws, wf, NULL) == RACE_ERR_UNSUPPORTED,
         "d = 136 (above 128) unsupported");
  s.d = 96;
  EXPECT(race_attn_workspace_bytes(&s, 4, 2, 0, RACE_WS_FWD) > wf, "d = 96 runs on padded rows");
  s.d = 128;
  s.w_per_head = 2;
  EXPECT(race_attn_fwd(Q, K, V, W, 1.0f, 4, 2, 0, O, &s, NULL, 0, ws, wf, NULL) == RACE_ERR_INVALID_ARG,
         "w_per_head = 2");
  s.w_per_head = 0;

  void* dQ = (void*)(base + ((uintptr_t)6 << 24));
  void* dK = (void*)(base + ((uintptr_t)7 << 24));
  void* dV = (void*)(base + ((uintptr_t)8 << 24));
  const void* dO = (const void*)(base + ((uintptr_t)9 << 24));
  const void* st = (const void*)(base + ((uintptr_t)10 << 24));
  float* dW = (float*)(base + ((uintptr_t)11 << 24));
  void* wsb = (void*)(base + ((uintptr_t)12 << 24));
  /* without a state the backward rebuilds it in a larger workspace */
  const size_t wns = race_attn_workspace_bytes(&s, 4, 2, 0, RACE_WS_BWD | RACE_WS_NO_STATE);
  EXPECT(wns > wb, "workspace of the backward without a state");
  EXPECT(race_attn_workspace_bytes(&s, 4, 2, 0, RACE_WS_NO_STATE) == 0, "no-state flag needs a backward phase");
  EXPECT(race_attn_bwd(Q, K, V, W, 1.0f, 4, 2, 0, NULL, dO, dQ, dK, dV, NULL, NULL, &s, NULL, 0, wsb, wb, NULL) ==
             RACE_ERR_WORKSPACE,
         "backward without state needs the larger workspace");
  EXPECT(race_attn_bwd(Q, K, V, W, 1.0f, 4, 2, 0, NULL, dO, dQ, dK, dV, NULL, NULL, &s, dQ, 1 << 30, wsb, wb,
                       NULL) == RACE_ERR_INVALID_ARG,
         "state overlaps dQ");
  EXPECT(race_attn_bwd(Q, K, V, W, 1.0f, 4, 2, 0, NULL, dO, dQ, dK, dV, NULL, NULL, &s, wsb, 1 << 20, wsb, wb,
                       NULL) == RACE_ERR_INVALID_ARG,
         "state overlaps the workspace");
  EXPECT(race_attn_bwd(Q, K, V, W, 1.0f, 4, 2, 0, NULL, dO, dQ, dK, dV, NULL, dW, &s, st, 1 << 30, wsb, wb, NULL) ==
             RACE_ERR_WORKSPACE,
         "dW needs the larger workspace");
  EXPECT(race_attn_bwd(Q, K, V, W, 1.0f, 4, 2, 0, NULL, dO, dQ, dK, dV, NULL, (float*)W, &s, st, 1 << 30, wsb, ww,
                       NULL) == RACE_ERR_INVALID_ARG,
         "dW overlaps W");

  /* allocation-free forward: argument checks run before any device call */
  EXPECT(race_attn_fwd_noalloc_scratch_bytes() == (size_t)64 << 20, "allocation-free scratch size");
  EXPECT(race_attn_fwd_noalloc(NULL, K, V, W, 1.0f, 4, 2, 0, O, &s, NULL, 0, NULL) == RACE_ERR_INVALID_ARG,
         "allocation-free forward: NULL Q");
  EXPECT(race_attn_fwd_noalloc(Q, K, V, W, 1.0f, 9, 2, 0, O, &s, NULL, 0, NULL) == RACE_ERR_INVALID_ARG,
         "allocation-free forward: P = 9");

  EXPECT(race_attn_decode_state_bytes(&s, 4, 2) == (size_t)4 * 32 * 129 * 4, "decode state bytes");
  EXPECT(strcmp(race_status_string(RACE_OK), "RACE_OK") == 0, "status string");
  EXPECT(strcmp(race_status_string(RACE_ERR_WORKSPACE), "RACE_ERR_WORKSPACE") == 0, "status string");

  if (failures) return 1;
  printf("ok\n");
  return 0;
}
