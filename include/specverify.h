/*
 * specverify.h -- C ABI of the batched speculative-decoding verify library
 * (libspecverify.so, HIP kernels for MI355X / gfx950).
 *
 * The verify step it implements:
 *   - one target forward scores k+1 rows per request, and the verify looks at
 *     all of them in one batched call ("Adding Speculative Decoding",
 *     section "Verification and sampling", item 1; requests may carry
 *     different k, packed varlen here through cu_seqlens);
 *   - greedy requests accept drafts while each equals the argmax of its row and
 *     commit the argmax at the first mismatch (same page, "The existing base"
 *     and "Verification and sampling" item 2);
 *   - sampled requests accept draft x_i while u_i < min(1, p(x_i)/q(x_i)),
 *     stop at the first rejection and resample there from
 *     max(0, p - q) / sum max(0, p - q), or draw a bonus token from the last
 *     target row when every draft is accepted ("Speculative Decoding: Draft
 *     Model Sampling, Rejection Sampling & On-Device Acceleration", Key
 *     Topic 2 and Section 2; "Speculative Decoding in Custom LLM Servicing:
 *     Implementing Draft Models in Rust", sections "The Memory Bandwidth Wall
 *     and Speculative Math" and "The Verification Algorithm");
 *   - every row is processed with its own request's temperature, top-k,
 *     top-p and greedy flag ("FreeToken PR #836", section "Design").
 *   - only the accepted count and the committed tokens leave the device (the
 *     Rust page, "Production Pitfalls" item 1): the library never
 *     synchronises with the host.
 *
 * Conventions shared by every entry point
 * ---------------------------------------
 * Pointers: every array argument is a DEVICE pointer owned by the caller.
 *   The library never allocates, frees or synchronises; all work is enqueued
 *   on `stream` (a hipStream_t passed as void*; NULL = the null stream).
 *   Outputs must not alias inputs.  The library keeps no global state.
 * Return value: SV_OK, or an SV_ERR_* code detected on the host, in which
 *   case NOTHING was enqueued.  SV_ERR_LAUNCH reports a failed kernel launch.
 * Packing (varlen): request b has k_b = cu[b+1] - cu[b] - 1 drafts.
 *   - target rows   cu[b] .. cu[b] + k_b          (row j scores position j)
 *   - draft rows and draft tokens  cu[b]-b .. cu[b]-b+k_b-1
 *   - uniforms u[cu[b] + i]: i < k_b acceptance draws, i = k_b the final draw
 *   total_rows = cu[batch]; cu must be non-decreasing with cu[0] = 0 and every
 *   k_b >= 0.  A request whose first target row cu[b] is below an earlier
 *   request's, or whose first draft row cu[b]-b is below an earlier request's
 *   cu[e]-e, is reported BAD_K (after a request with no rows, or offsets that go
 *   back, the next draft rows would reach into an earlier request's), so neither
 *   the target rows nor the draft rows of the requests that are verified overlap.
 * Layouts: logit / probability buffers are row-major [rows, ld] with ld >= vocab
 *   elements; only the first `vocab` entries of a row are read.  Rows whose
 *   address is 16-byte aligned take 128-bit loads, others a scalar path.
 * Values: -inf in a logit row masks that token.  NaN or +inf in a needed logit
 *   row, or a NaN/inf/negative needed probability, is a data fault.
 * Per-request status (status[b]) is written on the device; first match wins:
 *   SV_ROW_BAD_K     offsets out of range, k_b < 0, k_b > max_k, cu[b] below
 *                    an earlier offset, or cu[b]-b below an earlier cu[e]-e
 *   SV_ROW_BAD_PARAM unknown draft kind, a kind that needs draft rows with a
 *                    NULL draft buffer, or temperature +inf
 *   SV_ROW_BAD_TOKEN a draft id outside [0, vocab)
 *   SV_ROW_NONFINITE a data fault in a needed row (see Values)
 *   SV_ROW_EMPTY     a needed logit row with no finite value
 *   SV_ROW_INTERNAL  see the enum below
 *   A request with a non-OK status gets accepted[b] = -1, out_tokens -1 and
 *   NaN probabilities; BAD_K requests leave out_tokens/probabilities untouched;
 *   for SV_ROW_INTERNAL only status and accepted are defined.
 *   Each output word of a request has one writer.
 * Workspace: device memory of at least spec_verify_workspace_bytes(); it must
 *   be zero-filled before its first use (spec_verify_workspace_init does it on
 *   a stream).  It is viewed as 64-bit words whose top bit marks a value in
 *   flight between workgroups; every call that reports no SV_ROW_INTERNAL
 *   leaves that bit clear in every word, so the same workspace serves the next
 *   call whatever its sizes.  A wait that runs out marks the workspace as
 *   poisoned: from then on every call on it reports SV_ROW_INTERNAL for each
 *   valid request until spec_verify_workspace_init clears it.  Two calls that
 *   may run concurrently must not share a workspace.
 * Determinism: identical inputs give bitwise identical outputs, and request
 *   b's results do not depend on the other requests of the batch.
 */
#ifndef SPECVERIFY_H
#define SPECVERIFY_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define SPECVERIFY_ABI_VERSION 1

/* host-detected errors (return values) */
enum {
  SV_OK = 0,
  SV_ERR_NULL = 1,      /* a required pointer is NULL */
  SV_ERR_SHAPE = 2,     /* batch < 1 or > 1024, total_rows < batch, max_k outside
                           [0,63], vocab < 1 or > 4194304, ld < vocab,
                           (2*max_k+1) * ceil(vocab/8192) > 6144, or the grid
                           would be too large */
  SV_ERR_DTYPE = 3,     /* unknown dtype code */
  SV_ERR_WORKSPACE = 4, /* workspace_bytes smaller than required */
  SV_ERR_LAUNCH = 5,    /* the HIP runtime refused a launch */
  SV_ERR_SCRATCH = 6    /* spec_verify_sampled_noalloc: the call needs more than its
                           static scratch array holds (8 MiB) */
};

/* element types of logit / probability buffers */
enum { SV_F32 = 0, SV_BF16 = 1 };

/* draft kinds (per request) */
enum {
  SV_DRAFT_ONEHOT = 0, /* argmax / n-gram drafts: q = e_x, no draft row is read */
  SV_DRAFT_LOGITS = 1, /* draft logits: the request's temperature and filters apply */
  SV_DRAFT_PROBS = 2,  /* cached draft probabilities: used as supplied */
  SV_DRAFT_MATCH = 3   /* argmax drafts verified the way the PR page "FreeToken PR #836"
                          (section "Design", rejection row) does it: every row j is
                          sampled with its own uniform u[cu[b]+j] (inverse CDF, as the
                          final draw below), drafts are accepted while each equals its
                          row's sample, and the sample of the first other row (or of
                          row k_b) is committed; no draft row is read.  Same law as
                          SV_DRAFT_ONEHOT, different map from uniforms to tokens. */
};

/* per-request device status */
enum {
  SV_ROW_OK = 0,
  SV_ROW_NONFINITE = 1,
  SV_ROW_EMPTY = 2,
  SV_ROW_BAD_K = 3,
  SV_ROW_BAD_TOKEN = 4,
  SV_ROW_BAD_PARAM = 5,
  SV_ROW_INTERNAL = 6   /* a wait between workgroups ran out (another kernel kept the
                           GPU's compute units busy for a long time), or the workspace
                           was poisoned by such a call: accepted is -1, the request's
                           other outputs are undefined, and the workspace must be
                           re-initialised (spec_verify_workspace_init) */
};

/* ABI version of the loaded library (SPECVERIFY_ABI_VERSION). */
int spec_verify_abi_version(void);

/* Static string for an SV_ERR_* return code or an SV_ROW_* status
 * (status codes are looked up as 100 + code).  Never NULL. */
const char* spec_verify_status_string(int code);

/* Bytes of workspace a call with these sizes needs (0 on invalid sizes). */
size_t spec_verify_workspace_bytes(int batch, int total_rows, int vocab, int max_k);

/* Zero-fills `workspace_bytes` bytes of the workspace on `stream` with a small
 * fill kernel (safe inside stream capture).  Returns SV_OK, SV_ERR_NULL or
 * SV_ERR_LAUNCH. */
int spec_verify_workspace_init(void* workspace, size_t workspace_bytes, void* stream);

/*
 * Greedy verify (catalog page "Adding Speculative Decoding", "The existing
 * base"): per request, g_j = lowest index of the maximum raw value of target
 * row j (-0 equals +0); a = first i < k_b with draft[i] != g_i, else k_b.
 *   target_logits  [total_rows, ld_target] of target_dtype (SV_F32 / SV_BF16)
 *   cu_seqlens     int32 [batch + 1]
 *   draft_tokens   int32 [total_rows - batch]   (may be NULL iff total_rows == batch)
 *   accepted       int32 [batch]        out: a_b, or -1 on a non-OK status
 *   out_tokens     int32 [total_rows]   out: cu[b]..cu[b]+a_b-1 = the drafts,
 *                                       cu[b]+a_b = g_{a_b}, the rest of the
 *                                       request's slots -1
 *   status         int32 [batch]        out: SV_ROW_*
 */
int spec_verify_greedy(const void* target_logits, int target_dtype, int64_t ld_target,
                       const int32_t* cu_seqlens, const int32_t* draft_tokens,
                       int batch, int total_rows, int max_k, int vocab,
                       int32_t* accepted, int32_t* out_tokens, int32_t* status,
                       void* workspace, size_t workspace_bytes, void* stream);

/*
 * Sampled verify by lossless rejection sampling (pages cited above), with
 * greedy requests (temperature not a normal positive float) mixed in.
 *   target_logits  [total_rows, ld_target] of target_dtype
 *   draft          [total_rows - batch, ld_draft] of draft_dtype, or NULL if
 *                  no request uses SV_DRAFT_LOGITS / SV_DRAFT_PROBS.  LOGITS
 *                  rows are read in full; PROBS rows are gathered at the draft
 *                  ids and read in full only at a rejection position.
 *   draft_kind     int32 [batch]  SV_DRAFT_*
 *   cu_seqlens     int32 [batch + 1]
 *   draft_tokens   int32 [total_rows - batch]
 *   uniforms       float [total_rows]  values in [0, 1); u[cu[b]+i] is the
 *                  acceptance draw of draft i, u[cu[b]+k_b] the final draw.
 *                  Each draw maps to its outcome by: accept iff
 *                  u * q(x) < p(x); final token = min{t : C_t > u * W} with C
 *                  the running sum of the final weights in token order.
 *   temperature    float [batch]; a request is greedy unless T >= FLT_MIN
 *   top_k          int32 [batch] or NULL; k <= 0 or k >= vocab: off.  Keeps
 *                  every token whose value is >= the k-th largest.
 *   top_p          float [batch] or NULL; p outside (0, 1): off.  Keeps the
 *                  shortest run of whole tie groups, by descending value, whose
 *                  probability after temperature and top-k reaches p.
 *   accepted, out_tokens, status: as in spec_verify_greedy (out_tokens at
 *                  cu[b]+a_b holds the residual or bonus token)
 *   p_at_draft, q_at_draft  float [total_rows - batch] or NULL: p_i(x_i) and
 *                  q_i(x_i) after temperature and filters (greedy requests:
 *                  p = 1 if x_i is the argmax else 0, q = 1).
 */
int spec_verify_sampled(const void* target_logits, int target_dtype, int64_t ld_target,
                        const void* draft, int draft_dtype, int64_t ld_draft,
                        const int32_t* draft_kind, const int32_t* cu_seqlens,
                        const int32_t* draft_tokens, const float* uniforms,
                        const float* temperature, const int32_t* top_k, const float* top_p,
                        int batch, int total_rows, int max_k, int vocab,
                        int32_t* accepted, int32_t* out_tokens,
                        float* p_at_draft, float* q_at_draft, int32_t* status,
                        void* workspace, size_t workspace_bytes, void* stream);

/*
 * spec_verify_sampled with presence and frequency penalties applied per verify
 * row, the drafts before a row counted as already generated ("FreeToken PR
 * #836", section "Design", the bullet on argmax drafts).  Row j of request b
 * counts c(t) = h_b(t) + #{i < j : x_i = t}; every token with c(t) > 0 gets
 *   l'(t) = l(t) - (frequency[b] * c(t) + presence[b])
 * evaluated in fp64 and rounded to fp32, then to target_dtype (nearest, ties
 * to even), before temperature, top-k and top-p.  Penalties apply to the
 * target rows of every request, greedy ones included; draft rows are used as
 * supplied.  A request with both penalties 0 is verified exactly as by
 * spec_verify_sampled; a non-finite penalty makes it SV_ROW_BAD_PARAM.
 *   presence, frequency  float [batch], device.
 *   hist_offsets   int32 [batch + 1] or NULL (no history); request b's
 *                  generated-token counts are entries
 *                  [hist_offsets[b], hist_offsets[b+1]) of
 *   hist_tokens, hist_counts  int32 [hist_nnz]: token ids (unique within a
 *                  request) and counts.  Entries with a token outside
 *                  [0, vocab) or a negative count are ignored; offsets out of
 *                  order or outside [0, hist_nnz] give the request no history.
 *   penalized_target  device buffer of total_rows * ld_target elements of
 *                  target_dtype, written by the call (the penalized rows of
 *                  the requests with a nonzero penalty; other rows are left
 *                  as they were) and read by it; it must not alias the inputs.
 *   Other arguments, layouts and outputs: as spec_verify_sampled.  Returns as
 *   spec_verify_sampled, and SV_ERR_NULL for a NULL presence, frequency or
 *   penalized_target (or history arrays with hist_nnz > 0), SV_ERR_SHAPE for
 *   hist_nnz outside [0, 2^31).
 */
int spec_verify_sampled_penalized(const void* target_logits, int target_dtype, int64_t ld_target,
                                  const void* draft, int draft_dtype, int64_t ld_draft,
                                  const int32_t* draft_kind, const int32_t* cu_seqlens,
                                  const int32_t* draft_tokens, const float* uniforms,
                                  const float* temperature, const int32_t* top_k,
                                  const float* top_p, const float* presence,
                                  const float* frequency, const int32_t* hist_offsets,
                                  const int32_t* hist_tokens, const int32_t* hist_counts,
                                  int64_t hist_nnz, void* penalized_target, int batch,
                                  int total_rows, int max_k, int vocab, int32_t* accepted,
                                  int32_t* out_tokens, float* p_at_draft, float* q_at_draft,
                                  int32_t* status, void* workspace, size_t workspace_bytes,
                                  void* stream);

/*
 * Drain of a verified batch ("FreeToken PR #836", section "Design", drain row:
 * commit n = accepted + 1 tokens and give back the unused slots; "Adding
 * Speculative Decoding", "The four high-risk coupling points" item 1: accept
 * all / some / none).  Run after a verify on the same stream, on its outputs.
 * Per request b with k_b = cu[b+1] - cu[b] - 1 and a_b = accepted[b]:
 *   n_b          = a_b + 1 if status[b] == SV_ROW_OK and 0 <= a_b <= k_b, else 0
 *   rollback[b]  = k_b + 1 - n_b: verify slots (KV positions) to give back, or 0
 *                  for SV_ROW_BAD_K or rows outside [0, total_rows)
 *   commit_offsets[b] = n_0 + ... + n_{b-1}; commit_offsets[batch] = total
 *   committed[commit_offsets[b] + i] = out_tokens[cu[b] + i] for i < n_b
 *   cu_seqlens int32 [batch + 1], accepted / status int32 [batch],
 *   out_tokens int32 [total_rows] (device, read);
 *   committed int32 [total_rows], commit_offsets int32 [batch + 1],
 *   rollback int32 [batch] (device, written; committed only up to the total,
 *   never past total_rows).
 *   Returns SV_OK, SV_ERR_NULL, SV_ERR_SHAPE (batch outside [1, 1024] or
 *   total_rows < batch) or SV_ERR_LAUNCH.  Outputs must not alias inputs.
 */
int spec_verify_drain(const int32_t* cu_seqlens, const int32_t* accepted, const int32_t* status,
                      const int32_t* out_tokens, int batch, int total_rows, int32_t* committed,
                      int32_t* commit_offsets, int32_t* rollback, void* stream);

/*
 * Acceptance accounting of one verify step and the next lookahead.
 * counters (int64 [4], device, accumulated in place) += over the requests with
 * status OK and 0 <= a_b <= k_b: tokens generated (a_b + 1), tokens drafted
 * (k_b), tokens accepted (a_b), requests (1) -- the three counters of the
 * metrics in "Speculative Decoding in Custom LLM Servicing: Implementing Draft
 * Models in Rust", "Production Pitfalls & Mitigation Strategies", plus the
 * request count: acceptance rate = accepted / drafted, mean tokens per step =
 * generated / requests ("Adding Speculative Decoding", Acceptance bars item 2).
 * Per request, float32 throughout and in this order (no contraction):
 *   r = a_b / k_b; ema_out[b] = ema_in[b] + beta * (r - ema_in[b])
 *   (requests with k_b = 0 or not counted keep ema_in[b]);
 *   k_next[b] = k_low if ema_out[b] < threshold else k_high
 * -- the adaptive lookahead of the same Rust page section, item 3 (e.g. K from
 * 5 to 2 below 40 %; k_low = 0 switches speculation off).  ema_out may equal
 * ema_in.  Returns SV_OK, SV_ERR_NULL, SV_ERR_SHAPE (batch outside [1, 1024],
 * beta outside [0, 1], NaN threshold, k_low or k_high outside [0, 63]) or
 * SV_ERR_LAUNCH.
 */
int spec_verify_accounting(const int32_t* cu_seqlens, const int32_t* accepted,
                           const int32_t* status, int batch, const float* ema_in, float* ema_out,
                           float beta, float threshold, int k_low, int k_high, int32_t* k_next,
                           int64_t* counters, void* stream);

/*
 * spec_verify_sampled without a workspace argument, for callers that cannot
 * allocate device memory (code under HIP graph capture, tight serving loops,
 * harnesses that forbid hipMalloc).  It calls no hipMalloc, hipFree or other
 * allocating routine: its scratch is one static device array of 8 MiB per GPU
 * (held until the process ends; its address is looked up once per device).
 * Each call zero-fills the bytes it uses with a small kernel on `stream`, then
 * runs the same kernels as spec_verify_sampled, with the same results.
 *   Arguments, layouts and outputs: as spec_verify_sampled.
 *   Returns SV_ERR_SCRATCH (nothing enqueued) when
 *   spec_verify_workspace_bytes(batch, total_rows, vocab, max_k) > 8 MiB
 *   (B=512, k=5, V=152064 needs 3.1 MB), and SV_ERR_LAUNCH when the array's
 *   address cannot be found on the current device.
 *   Every call on one GPU uses that GPU's one array: two calls that may
 *   overlap on the same GPU (concurrent streams, threads) race and must not
 *   be issued.
 */
int spec_verify_sampled_noalloc(const void* target_logits, int target_dtype, int64_t ld_target,
                                const void* draft, int draft_dtype, int64_t ld_draft,
                                const int32_t* draft_kind, const int32_t* cu_seqlens,
                                const int32_t* draft_tokens, const float* uniforms,
                                const float* temperature, const int32_t* top_k,
                                const float* top_p, int batch, int total_rows, int max_k,
                                int vocab, int32_t* accepted, int32_t* out_tokens,
                                float* p_at_draft, float* q_at_draft, int32_t* status,
                                void* stream);

#ifdef __cplusplus
}
#endif

#endif /* SPECVERIFY_H */
