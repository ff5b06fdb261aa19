/*
 * race_attn.h -- C ABI of the MI355X (gfx950) RACE attention library.
 *
 * RACE attention ("RACE Attention" slides on arXiv 2510.04008v5, frames
 * "Soft corner assignments make hashing differentiable", "Each bucket stores
 * mass and a weighted value sum", "Normalize after combining the tables" and
 * "Causality is a prefix update of the same statistics"; reading notes
 * sections 2.4-2.6) computes, per batch row b and head h, with L tables of
 * P Gaussian hyperplanes each (R = 2^P corners v_r in {+1,-1}^P):
 *
 *   u^(l)(x)   = tanh(W^(l) x)                                   (P values)
 *   phi^(l)(x) = softmax_r(beta * u^(l)(x) . v_r)                (R values)
 *   mass^(l)   = sum_j phi^(l)(K_j),  content^(l) = sum_j phi^(l)(K_j) V_j^T
 *   O_i        = sum_l phi^(l)(Q_i) content^(l) / sum_l phi^(l)(Q_i) mass^(l)
 *
 * The causal variant replaces the sums over all j by inclusive prefix sums
 * over j <= i (the current key is added before the query reads).
 * Corner order: v_{r,t} = +1 exactly when bit t of r is set.
 *
 * Conventions shared by every entry point
 *  - Q, K, V, O, dO, dQ, dK, dV are device pointers to contiguous
 *    [B][H][N][d] arrays of the I/O dtype (RACE_F32 or RACE_BF16), 16-byte
 *    aligned.  Outputs must not overlap inputs.
 *  - W is a device pointer to float32 [L][P][d] (table l, hyperplane t,
 *    column c at (l*P + t)*d + c), shared by every batch row and head; with
 *    shape->w_per_head = 1 it is [H][L][P][d], one set of tables per head
 *    (head h of every batch row uses the tables at h*L*P*d).
 *  - beta is a host float; any finite value is accepted.
 *  - stream is a hipStream_t (NULL = the default stream).  Every call only
 *    enqueues work on it and returns; device-side faults surface at the
 *    caller's next synchronisation.
 *  - The caller owns and allocates every buffer; the library never
 *    allocates device memory in these calls.
 *  - Argument checks run on the host before anything is enqueued.  On any
 *    error nothing is enqueued and no output is written.
 *  - Supported: P in [1, 8]; L >= 1 with L * 2^max(P,3) <= 256;
 *    N >= 1; B*H >= 1; d a multiple of 8 up to 128, for the (dtype, P, L,
 *    causal) combinations with a compiled kernel set (bf16 at d = 128: every
 *    P in [1, 8] in both variants; dW is not compiled at P = 7).  The kernels are
 *    compiled for head dims D = 64 and 128; a smaller d runs on the next
 *    one up with its token rows padded by zero columns in the workspace
 *    (zero columns add nothing to a projection and give zero output
 *    columns, so the results are the layer at d; the padding costs one more
 *    pass over each token tensor).  Other valid shapes return
 *    RACE_ERR_UNSUPPORTED.
 */
#ifndef RACE_ATTN_H
#define RACE_ATTN_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

struct ihipStream_t;
typedef struct ihipStream_t* race_stream_t;   /* same type as hipStream_t */

typedef enum {
  RACE_OK = 0,
  RACE_ERR_INVALID_ARG = 1,   /* null pointer, bad size, non-finite beta, ... */
  RACE_ERR_UNSUPPORTED = 2,   /* valid arguments, no compiled kernel for them */
  RACE_ERR_WORKSPACE = 3,     /* state or workspace smaller than required     */
  RACE_ERR_HIP = 4            /* a HIP runtime call failed; see race_last_error */
} race_status;

typedef enum { RACE_F32 = 0, RACE_BF16 = 1 } race_dtype;

typedef struct {
  int64_t B, H, N, d;
  int32_t dtype;              /* race_dtype */
  int32_t w_per_head;         /* 0: W is [L][P][d] for every head; 1: [H][L][P][d] */
} race_shape;

/* Bytes of the state buffer the forward pass fills and the backward pass
 * reads.  Non-causal: the bucket bank, content[B*H][LRP][D] float32
 * followed by mass[B*H][LRP] float32, where LRP = L * 2^max(P,3) rounded up
 * to the compiled bank size (rows past L*2^max(P,3) are zero; for P < 3 each
 * table is widened with zero hyperplanes, which leaves O unchanged) and D is
 * the kernels' head dim (columns past d are zero).  Causal: the
 * inclusive bucket bank at each segment end, plus one float32 per token.
 * Returns 0 for invalid arguments. */
size_t race_attn_state_bytes(const race_shape* shape, int P, int L, int causal);

/* Workspace phases for race_attn_workspace_bytes: the forward, the
 * backward, the backward with the table gradient dW; RACE_WS_NO_STATE is
 * OR-ed into a backward phase when race_attn_bwd will get no state (it then
 * rebuilds the state inside the workspace). */
enum {
  RACE_WS_FWD = 0,
  RACE_WS_BWD = 1,
  RACE_WS_BWD_DW = 2,
  RACE_WS_NO_STATE = 4
};

/* Bytes of scratch workspace for the phase is_bwd: RACE_WS_FWD (0),
 * RACE_WS_BWD (1) or RACE_WS_BWD_DW (2: adds float32 dL/dPre of every token
 * of both sides, 2 * B*H*N * (LRP / 2^max(P,3)) * max(P,3) floats, and one
 * partial per workgroup), optionally with RACE_WS_NO_STATE (adds room for
 * the rebuilt state: the bank, or for the causal layer the segment banks
 * and Den).  Returns 0 for invalid arguments. */
size_t race_attn_workspace_bytes(const race_shape* shape, int P, int L, int causal, int is_bwd);

/* Forward pass: O = RACE(Q, K, V; W, beta, P, L, causal).
 * state (may be NULL when state_bytes is 0) receives the statistics the
 * backward pass needs; workspace must hold race_attn_workspace_bytes(...,
 * RACE_WS_FWD).  state and O must not overlap each other or the workspace. */
race_status race_attn_fwd(const void* Q, const void* K, const void* V, const float* W,
                          float beta, int P, int L, int causal, void* O,
                          const race_shape* shape, void* state, size_t state_bytes,
                          void* workspace, size_t workspace_bytes, race_stream_t stream);

/* Allocation-free forward, for callers that cannot allocate device memory
 * (code under HIP graph capture, tight serving loops, harnesses that forbid
 * hipMalloc).  Same arguments and results as race_attn_fwd without the
 * workspace: its scratch is a device array inside the library, one copy per
 * GPU, of race_attn_fwd_noalloc_scratch_bytes() bytes (64 MiB), held until
 * the process ends.  A call needs the partial banks (non-causal) or
 * segment sums (causal) in it, plus room for the state when state is NULL;
 * a call needing more returns RACE_ERR_WORKSPACE and enqueues nothing.
 * The call allocates nothing; the first call on a device looks up that
 * device's scratch address.  Every call on a GPU shares its scratch, so
 * calls that overlap in time on one GPU (other streams, other threads)
 * race: serialise them. */
size_t race_attn_fwd_noalloc_scratch_bytes(void);
race_status race_attn_fwd_noalloc(const void* Q, const void* K, const void* V, const float* W,
                                  float beta, int P, int L, int causal, void* O,
                                  const race_shape* shape, void* state, size_t state_bytes,
                                  race_stream_t stream);

/* Backward pass: the exact gradients dQ, dK, dV of sum(O * dO) with W
 * held fixed (softmax, tanh and projection backward on both sides), and,
 * when dbeta (a device pointer to one float, 4-byte aligned) is not NULL,
 * dL/dbeta: beta multiplies the corner logits u . v_r (slides, frame "Soft
 * corner assignments make hashing differentiable"), one beta for every
 * batch row and head, so dbeta sums over both sides, every head, table and
 * token; it is summed in a fixed order (same bits on every run).
 * state is the one written by race_attn_fwd on the same inputs, or NULL:
 * the backward then rebuilds it from K, V (non-causal: one more read of K
 * and V; causal: the segment sums and a forward walk over Q, K, V that
 * writes Den but no O) in the workspace, which must then be sized with
 * RACE_WS_NO_STATE.  A given state must not overlap an output, the
 * workspace, dbeta or dW.  O is
 * the forward output or NULL: the non-causal backward never reads it; the
 * causal backward takes h = -(dO . O) / Den from it elementwise when given,
 * and rebuilds Den O with one more walk over Q, K, V when it is NULL.
 * When dW (a device pointer, 4-byte aligned, W's layout: [L][P][d] or
 * [H][L][P][d]) is not NULL it receives dL/dW: the pre-activations of a
 * row x are W^(l) x (same frame), so each table's gradient is the sum over
 * the query and key rows of dL/dPre^(l) x^T, over every batch row and head
 * that uses the table; summed in a fixed order (same bits on every run).
 * workspace must hold race_attn_workspace_bytes(..., RACE_WS_BWD), or
 * (..., RACE_WS_BWD_DW) when dW is requested, with RACE_WS_NO_STATE OR-ed in
 * when state is NULL; dW and dbeta must not overlap W, the workspace or any
 * other buffer. */
race_status race_attn_bwd(const void* Q, const void* K, const void* V, const float* W,
                          float beta, int P, int L, int causal, const void* O,
                          const void* dO, void* dQ, void* dK, void* dV, float* dbeta,
                          float* dW, const race_shape* shape, const void* state, size_t state_bytes,
                          void* workspace, size_t workspace_bytes, race_stream_t stream);

/* Recurrent decode (slides, frame "Causality is a prefix update of the same
 * statistics"): the causal layer as a fixed-size state per (batch, head),
 * the bucket bank after the tokens seen so far: float32 content
 * [B*H][LRP][D] followed by mass [B*H][LRP] (LRP = L * 2^max(P,3) padded to
 * the compiled size, D the kernels' head dim; the same layout as the
 * non-causal forward's state).  The decode kernel reads and writes rows of
 * the caller's d directly; the prefill pads K and V in its workspace when d
 * is below D.
 * shape->N is the number of tokens of the call; the state size does not
 * depend on it. */
size_t race_attn_decode_state_bytes(const race_shape* shape, int P, int L);

/* Workspace of race_attn_decode_prefill for a prompt of shape->N tokens. */
size_t race_attn_decode_prefill_workspace_bytes(const race_shape* shape, int P, int L);

/* The state after the prompt K, V [B][H][N][d]: the bank of all N tokens
 * (overwrites state).  Deterministic fixed-order sums. */
race_status race_attn_decode_prefill(const void* K, const void* V, const float* W, float beta,
                                     int P, int L, const race_shape* shape, void* state,
                                     size_t state_bytes, void* workspace, size_t workspace_bytes,
                                     race_stream_t stream);

/* Decode N new tokens Q, K, V [B][H][N][d] in order, updating state in
 * place: for each token the key and value enter the bank first, then
 * O_t = sum_l phi(Q_t) content / sum_l phi(Q_t) mass (the token attends to
 * itself and to every earlier token).  A zeroed state is the empty prefix.
 * Soft assignments are computed in float32 without rounding; O has the I/O
 * dtype.  Tokens are taken one after another inside one workgroup per
 * (batch, head): meant for a few tokens per call. */
race_status race_attn_decode(const void* Q, const void* K, const void* V, const float* W,
                             float beta, int P, int L, void* O, const race_shape* shape,
                             void* state, size_t state_bytes, race_stream_t stream);

/* Test export: the soft assignments phi^(l)(X) as float32 [B*H][N][L][2^P]
 * (slides frame "Soft corner assignments make hashing differentiable").
 * X has the I/O dtype; no workspace. */
race_status race_softbucket_debug(const void* X, const float* W, float beta, int P, int L,
                                  const race_shape* shape, float* phi_out,
                                  race_stream_t stream);

/* Test export of the bucket banks (slides frame "Each bucket stores mass and
 * a weighted value sum"; the causal banks follow frame "Causality is a
 * prefix update of the same statistics").  The number of banks per (batch,
 * head): 1 for the non-causal layer, one per sequence segment for the causal
 * one; *seg_tokens (if not NULL) receives the segment length (segment s
 * holds tokens [s * seg_tokens, min(N, (s + 1) * seg_tokens))).  Returns 0
 * for invalid or unsupported arguments. */
int race_bucket_stats_segments(const race_shape* shape, int P, int L, int causal, int64_t* seg_tokens);

/* Copies banks that race_attn_fwd left in state and race_attn_bwd left in
 * its workspace (the same shape, P, L and causal; a workspace sized for the
 * backward, used by no call since) into float32 arrays with S banks per
 * (batch, head) (S from race_bucket_stats_segments), tables l < L and
 * corners r < 2^P in the corner order above:
 *   content  [B*H][S][L][2^P][d]   mass  [B*H][S][L][2^P]
 *   dcontent [B*H][S][L][2^P][d]   dmass [B*H][S][L][2^P]
 * Non-causal: content / mass over all keys, content = sum_j phi(K_j) V_j^T;
 * dcontent = sum_t phi(Q_t) g_t^T and dmass = sum_t phi(Q_t) h_t over all
 * queries, with g_t = dO_t / Den_t and h_t = -(dO_t . O_t) / Den_t.  Causal:
 * bank s holds the keys before segment s (content, mass) and the queries
 * after segment s (dcontent, dmass).  Any output may be NULL; state may be
 * NULL when content and mass are, bwd_workspace when dcontent and dmass
 * are.  Device pointers; outputs 4-byte aligned, overlapping nothing else. */
race_status race_bucket_stats_debug(const race_shape* shape, int P, int L, int causal,
                                    const void* state, size_t state_bytes,
                                    const void* bwd_workspace, size_t bwd_workspace_bytes,
                                    float* content, float* mass, float* dcontent, float* dmass,
                                    race_stream_t stream);

/* Kernel timing for profiling tools.  While enabled, every kernel that the
 * calls above launch is bracketed by two HIP events recorded on the same
 * stream.  race_profile_report waits for the recorded events and writes one
 * line per kernel name, "name<TAB>launches<TAB>total_ms", NUL-terminated,
 * into buf (truncated to len bytes); it returns the bytes needed.
 * race_profile_reset forgets the records.  Events are created by the HIP
 * runtime on first use and reused; no device memory is allocated. */
race_status race_profile_enable(int on);
void race_profile_reset(void);
size_t race_profile_report(char* buf, size_t len);

/* Human-readable name of a status code (static storage). */
const char* race_status_string(race_status status);

/* Message of the last error raised on the calling thread ("" if none). */
const char* race_last_error(void);

#ifdef __cplusplus
}
#endif

#endif /* RACE_ATTN_H */
