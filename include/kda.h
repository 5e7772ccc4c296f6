/*
 * kda.h — C ABI of the MI355X (gfx950) Kimi Delta Attention forward pass.
 *
 * The operation (one independent recurrence per sequence n and head h):
 *
 *   S_t = (Diag(alpha_t) - beta_t k_t (k_t ⊙ alpha_t)^T) S_{t-1} + beta_t k_t v_t^T,
 *   alpha_t = exp(g_t)   (a per-channel decay vector),
 *   o_t     = scale * S_t^T q_t   (readout after the update at t),
 *
 * with S a d x d (d_k x d_v) state, d = 128 (the published kernel's only
 * size) or d = 64 / 256
 *   [core.today "Kimi Linear 특집", ch.4 혁신 1 (channel-wise gate) and 혁신 2
 *    (state-update equation); ch.2 (linear-attention readout Q(K^T V));
 *    ch.8 (fixed 128 x 128 state)].
 * It is evaluated chunk by chunk (64 tokens) with the WY/UT form of the
 * diagonal-plus-low-rank transition [core.today ch.4 혁신 2, chunkwise remark;
 * hnts03 "논문 리뷰: Kimi Delta Attention", section "Kimi Delta Attention"].
 *
 * Argument conventions follow the kernel API the pages describe
 * [trend.ondo.sh "MoonshotAI/FlashKDA", section "커널 API와 제약 조건"]:
 * K = V = 128 (the forward and decode calls also take K = V = 64 or 256, see
 * below; the backward takes 128 only); variable-length packing through cu_seqlens requires
 * B = 1; the initial and final states are each bf16, fp32 or absent, and
 * must have the same dtype when both are given.
 *
 * Sequence splitting: when there are fewer (sequence, head) recurrences than
 * the device has compute units to keep busy, kda_fwd cuts long sequences into
 * segments that run in parallel.  The recurrence is affine in the state, so a
 * segment's end state is A S_start + B with A the product of its transition
 * matrices [core.today ch.4 혁신 2, state-update equation]: each later segment
 * runs once from a zero state (B, and outputs without the start state's share)
 * and once from the identity with zero values (A, and the map from the start
 * state to the outputs); a scan over the segments gives every start state and
 * a fix-up pass adds its share to the outputs.  kda_plan reports whether a
 * call may split.  KDA_SEQSPLIT=0 in the environment turns splitting off;
 * KDA_SEG_MIN=<chunks> sets the shortest sequence that may be split (default 8).
 *
 * Ownership: every pointer is caller-owned memory; the library never retains
 * or frees it.  A call that may split sequences takes a workspace (size from
 * kda_plan) that the library owns.  It keeps one workspace per stream (per
 * stream and thread for hipStreamPerThread), at most four of up to 2 GiB in
 * total per device, and reuses it for later calls on that stream, which orders
 * them; a call enqueues no synchronisation of its own.  A kept workspace that
 * must grow is reallocated after its stream has drained (a host wait); when a
 * new stream's workspace does not fit, every kept workspace of the device is
 * freed after the device has drained.  A workspace larger than 2 GiB comes
 * from a stream-ordered pool for that call alone.  kda_release_workspaces()
 * frees the kept workspaces of the current device.  A stream handle that is
 * destroyed and created again names a new stream: synchronise a stream before
 * destroying it while calls on it may still run.  kda_fwd_noalloc uses a
 * static scratch instead and allocates nothing.
 * Asynchrony: kda_fwd enqueues work on `stream` (a hipStream_t, or NULL for
 * the null stream) and returns; results are valid after the caller
 * synchronises that stream.  A call waits for the device on the host only when
 * a kept workspace is reallocated.  Calls are thread-safe: the kept workspaces
 * of a device are taken under a lock held while a call enqueues its work, and
 * the pool and kda_bwd's side stream are created under a lock; otherwise there
 * is no global mutable state except the thread-local error text.
 * Errors: invalid arguments are rejected before any launch with a negative
 * status and no output touched; kda_last_error() then holds a description.
 * There is no fallback path.
 */
#ifndef KDA_H_
#define KDA_H_

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define KDA_HEAD_DIM 128
#define KDA_CHUNK 64

typedef enum {
  KDA_BF16 = 0, /* bfloat16, round-to-nearest-even on store */
  KDA_FP32 = 1  /* IEEE float32 */
} kda_dtype;

typedef enum {
  KDA_OK = 0,
  KDA_ERR_NULL = -1,         /* a required pointer is NULL */
  KDA_ERR_HEAD_DIM = -2,     /* K, V not a supported head dimension (see each call) */
  KDA_ERR_VARLEN_BATCH = -3, /* cu_seqlens given with B != 1 */
  KDA_ERR_STATE_DTYPE = -4,  /* both states given with different dtypes */
  KDA_ERR_DTYPE = -5,        /* a dtype argument is not a kda_dtype */
  KDA_ERR_SHAPE = -6,        /* B, H, num_seqs <= 0, T < 0, or sizes overflow */
  KDA_ERR_ALIGN = -7,        /* a pointer is not aligned as required below */
  KDA_ERR_HIP = -8,          /* the HIP runtime reported an error (see kda_last_error) */
  KDA_ERR_WORKSPACE = -9     /* kda_fwd_noalloc: the call needs more workspace than its
                                static scratch holds */
} kda_status;

/*
 * kda_fwd — chunkwise KDA forward pass (prefill).
 *
 *  q, k, v    device, bf16, [B, T, H, d] contiguous (channel fastest), 16-byte
 *             aligned.  The kernel does not normalise q or k.
 *  g          device, fp32, [B, T, H, d], 16-byte aligned: the log-decay,
 *             alpha = exp(g) taken as given (g <= 0 expected).  Range limit of
 *             the chunked evaluation: within each 16-token block aligned to the
 *             start of a 64-token chunk, the per-channel sum of -g must stay
 *             below 80 (g >= -5 everywhere is sufficient); beyond that the
 *             intra-chunk exponent factors overflow fp32, and the outputs from
 *             the first such chunk on and the sequence's final state come out
 *             non-finite (inf or NaN).
 *  beta       device, fp32, [B, T, H], 4-byte aligned: write strength, as given.
 *  scale      multiplies every output (callers usually pass 1/sqrt(d)).
 *  initial_state / initial_dtype
 *             device, [N, H, d, d] (d_k-major: element (i, j) at i*d + j),
 *             16-byte aligned, or NULL for a zero initial state.
 *  final_state / final_dtype
 *             device, [N, H, d, d], 16-byte aligned, or NULL when not
 *             wanted.  It may alias initial_state (each state is read in full
 *             before it is overwritten).
 *  cu_seqlens device, int32, [num_seqs + 1], or NULL.  When given: B must be 1,
 *             cu_seqlens[0] = 0, non-decreasing, cu_seqlens[num_seqs] <= T;
 *             sequence n is rows [cu_seqlens[n], cu_seqlens[n+1]) and N =
 *             num_seqs.  The library never reads it on the host; it is not
 *             validated beyond the pointer.  Zero-length sequences are allowed
 *             (their final state equals their initial state).
 *             When NULL: every batch row is one sequence of T tokens, N = B,
 *             and num_seqs is ignored.
 *  B, T, H    batch rows, tokens per row (packed total when varlen), heads.
 *  K, V       head dimensions d = K = V: 128, 64 or 256.
 *  out        device, bf16, [B, T, H, d], 16-byte aligned; rows outside every
 *             sequence (varlen with cu_seqlens[num_seqs] < T) are not written.
 *  stream     hipStream_t to launch on (NULL = null stream).
 *
 * d = 64 runs on the d = 128 kernels with the key channels past 64 read as
 * zero, one 64-column value slice per (sequence, head, segment): the same plan,
 * sequence splitting and workspace as d = 128 (kda_plan), with value_splits
 * always 1.  d = 256 runs as two
 * launches: every (chunk, head) first writes a record of its chunk-local
 * operands (gated keys and queries, the transposed state-update operand,
 * (I + A)^-1 diag(beta), the masked Q K^T and the chunk decay) into a workspace
 * of kda_dim_workspace_bytes() bytes taken like kda_fwd's workspace (see
 * Ownership), then one workgroup per (sequence, head, value slice) walks the
 * chunks in order.  d = 256 never splits sequences.  The 16-token range limit
 * on g above applies at both sizes.
 */
kda_status kda_fwd(const void* q, const void* k, const void* v, const float* g, const float* beta,
                   float scale, const void* initial_state, int initial_dtype, void* final_state,
                   int final_dtype, const int32_t* cu_seqlens, int32_t num_seqs, int32_t B,
                   int64_t T, int32_t H, int32_t K, int32_t V, void* out, void* stream);

/*
 * kda_fwd_noalloc — kda_fwd for callers that cannot allocate device memory
 * (code under HIP graph capture, tight serving loops, harnesses that forbid
 * hipMalloc).  Same arguments, layouts, results and status codes as kda_fwd;
 * it calls no hipMalloc, hipFree or allocating library routine.  Its workspace
 * is a static device array of KDA_NOALLOC_SCRATCH_BYTES bytes, one per GPU,
 * held from the first call on that GPU until the process ends:
 *   d = 128: the plan for splitting long sequences into segments is sized to
 *            the scratch (segment state slots and the 64 x 128 output blocks
 *            of the later segments' chunks); sequences are split only as far
 *            as those fit, so every size runs, very long ones in fewer and
 *            longer segments than kda_fwd would use;
 *   d = 64:  as d = 128;
 *   d = 256: the per-chunk records must fit (slots x H x record bytes, see
 *            kda_dim_workspace_bytes); larger calls return KDA_ERR_WORKSPACE
 *            before any launch.
 * Every call on a GPU shares that GPU's scratch: calls that overlap on one GPU
 * (concurrent streams, threads) race and must be serialised by the caller.
 * Nothing in the scratch needs clearing between calls: each call writes every
 * entry it reads.
 */
#define KDA_NOALLOC_SCRATCH_BYTES (256u << 20)
kda_status kda_fwd_noalloc(const void* q, const void* k, const void* v, const float* g,
                           const float* beta, float scale, const void* initial_state,
                           int initial_dtype, void* final_state, int final_dtype,
                           const int32_t* cu_seqlens, int32_t num_seqs, int32_t B, int64_t T,
                           int32_t H, int32_t K, int32_t V, void* out, void* stream);

/*
 * kda_fwd_check — the host-side validation kda_fwd performs, without any
 * launch or device access (pointers are only tested for NULL and alignment).
 * Same arguments and status codes as kda_fwd.
 */
kda_status kda_fwd_check(const void* q, const void* k, const void* v, const float* g,
                         const float* beta, float scale, const void* initial_state,
                         int initial_dtype, const void* final_state, int final_dtype,
                         const int32_t* cu_seqlens, int32_t num_seqs, int32_t B, int64_t T,
                         int32_t H, int32_t K, int32_t V, const void* out);

/* Static description of a status code (never NULL). */
const char* kda_status_string(int status);

/* Detail of the last failure on the calling thread ("" if none). */
const char* kda_last_error(void);

/*
 * kda_plan — the launch plan kda_fwd uses for N independent sequences
 * (num_seqs, or B without cu_seqlens), T tokens (per row; the packed total
 * when varlen != 0) and H heads on a device with cu_count compute units
 * (cu_count <= 0: query the current HIP device):
 *   workgroups       workgroups of the main kernel (some exit at once when
 *                    fewer sequences are split than the bound allows);
 *   value_splits     value-column slices per (sequence, head), 1 or 2;
 *   workspace_bytes  device workspace a call takes (see Ownership);
 *                    0 when no sequence can be split (the call then launches
 *                    the main kernel only).
 * The environment variable KDA_VSPLIT (1 or 2) overrides the slice count
 * (2 also turns sequence splitting off).  At head dimension 64 kda_fwd uses
 * the same plan with one value slice (value_splits 1, KDA_VSPLIT ignored) and
 * the same workspace.  Host only; returns KDA_ERR_SHAPE for
 * N <= 0, H <= 0 or T < 0, KDA_ERR_NULL for NULL outputs, KDA_ERR_HIP if the
 * device query fails.
 */
kda_status kda_plan(int32_t n_sequences, int64_t T, int32_t H, int32_t varlen, int32_t cu_count,
                    int32_t* workgroups, int32_t* value_splits, int64_t* workspace_bytes);

/*
 * kda_decode — one recurrent step per sequence (decoding), the state updated in
 * place [core.today "Kimi Linear 특집", ch.4 혁신 2, state-update equation; the
 * decoding-speed comparison there rests on the state's fixed 128 x 128 size].
 * For each sequence n < N and head h, with S the state of slot s(n):
 *   S <- Diag(exp(g)) S;  e = v - S^T k;  S <- S + beta k e^T;  o = scale S^T q
 * -- the same step kda_fwd takes per token, so a prefill's final state can be
 * continued here.
 *
 *  q, k, v       device, bf16, [N, H, d] (one token per sequence), 16-byte aligned;
 *                d = K = V is 128, 64 or 256.
 *  g             device, fp32, [N, H, d], 16-byte aligned (log-decay).
 *  beta          device, fp32, [N, H], 4-byte aligned.
 *  state         device, [slots, H, d, d] (d_k-major), bf16 or fp32 per
 *                state_dtype, 16-byte aligned; read and overwritten in place
 *                (bf16 states are rounded to nearest even on store).
 *  state_indices device, int32, [N], or NULL: the slot s(n) of each sequence
 *                (NULL: s(n) = n).  A negative entry skips the sequence: neither
 *                its state nor its output row is touched.  Distinct sequences must
 *                name distinct slots (not checked).
 *  out           device, bf16, [N, H, d], 16-byte aligned.
 *  stream        hipStream_t (NULL = null stream); asynchronous like kda_fwd.
 * Memory: no workspace; each (sequence, head) reads and writes its state once.
 * Errors: as kda_fwd (KDA_ERR_HEAD_DIM, KDA_ERR_SHAPE for N < 0 or H <= 0,
 * KDA_ERR_DTYPE, KDA_ERR_NULL, KDA_ERR_ALIGN, KDA_ERR_HIP); N = 0 is a no-op.
 */
kda_status kda_decode(const void* q, const void* k, const void* v, const float* g,
                      const float* beta, float scale, void* state, int state_dtype,
                      const int32_t* state_indices, int32_t N, int32_t H, int32_t K, int32_t V,
                      void* out, void* stream);

/* kda_decode_check — kda_decode's host-side validation, with no launch. */
kda_status kda_decode_check(const void* q, const void* k, const void* v, const float* g,
                            const float* beta, float scale, const void* state, int state_dtype,
                            const int32_t* state_indices, int32_t N, int32_t H, int32_t K,
                            int32_t V, const void* out);

/*
 * kda_gdn_fwd — the scalar-gate special case (Gated DeltaNet): one decay per
 * token and head instead of one per key channel [core.today "Kimi Linear 특집",
 * ch.4 혁신 1: GDN forgets the whole state with a single scalar, KDA with a
 * per-channel vector; hnts03 "논문 리뷰: Kimi Delta Attention", section "Kimi
 * Delta Attention"].  Per token:
 *   S_t = exp(g_t) (I - beta_t k_t k_t^T) S_{t-1} + beta_t k_t v_t^T,   o_t = scale S_t^T q_t
 * which is kda_fwd's update with Diag(alpha_t) = exp(g_t) I.
 *  g          device, fp32, [B, T, H] (one value per token and head), 4-byte
 *             aligned; range limit as kda_fwd's with the same g on every channel.
 * Every other argument, the layouts, the workspace, asynchrony and the status
 * codes are those of kda_fwd (the same kernels run; only the gate load differs,
 * and it reads 4 bytes per token and head instead of 4d).
 */
kda_status kda_gdn_fwd(const void* q, const void* k, const void* v, const float* g,
                       const float* beta, float scale, const void* initial_state,
                       int initial_dtype, void* final_state, int final_dtype,
                       const int32_t* cu_seqlens, int32_t num_seqs, int32_t B, int64_t T,
                       int32_t H, int32_t K, int32_t V, void* out, void* stream);

/* kda_gdn_fwd_check — kda_gdn_fwd's host-side validation, with no launch. */
kda_status kda_gdn_fwd_check(const void* q, const void* k, const void* v, const float* g,
                             const float* beta, float scale, const void* initial_state,
                             int initial_dtype, const void* final_state, int final_dtype,
                             const int32_t* cu_seqlens, int32_t num_seqs, int32_t B, int64_t T,
                             int32_t H, int32_t K, int32_t V, const void* out);

/*
 * kda_gdn_decode — kda_decode with the scalar gate: g is fp32 [N, H], 4-byte
 * aligned, and S <- exp(g) S is the decay.  Arguments, in-place state update,
 * slot indices and errors as kda_decode.
 */
kda_status kda_gdn_decode(const void* q, const void* k, const void* v, const float* g,
                          const float* beta, float scale, void* state, int state_dtype,
                          const int32_t* state_indices, int32_t N, int32_t H, int32_t K, int32_t V,
                          void* out, void* stream);

/* kda_gdn_decode_check — kda_gdn_decode's host-side validation, with no launch. */
kda_status kda_gdn_decode_check(const void* q, const void* k, const void* v, const float* g,
                                const float* beta, float scale, const void* state, int state_dtype,
                                const int32_t* state_indices, int32_t N, int32_t H, int32_t K,
                                int32_t V, const void* out);

/*
 * kda_bwd — gradients of kda_fwd (training backward pass).  Given dL/do and
 * optionally dL/dS_final, returns dL/dq, dL/dk, dL/dv, dL/dg, dL/dbeta and
 * optionally dL/dS_initial, all fp32.  It differentiates the recurrence of
 * kda_fwd [core.today "Kimi Linear 특집", ch.4 혁신 2, state-update equation and
 * its chunkwise form; ch.2 readout]: a forward pass stores every chunk's start
 * state, chunk-local gradient products follow, and one serial pass per
 * (sequence, head) carries the state gradient from the last chunk to the first.
 *
 *  q, k, v, g, beta, scale, initial_state / initial_dtype, cu_seqlens, num_seqs,
 *  B, T, H, K, V    as kda_fwd.
 *  d_out            device, bf16, [B, T, H, 128], 16-byte aligned: dL/do.
 *  d_final_state / d_final_dtype
 *                   device, [N, H, 128, 128] bf16 or fp32, 16-byte aligned, or NULL
 *                   (zero).
 *  dq, dk, dg       device, fp32, [B, T, H, 128], 16-byte aligned (outputs).
 *  dv               device, fp32, [B, T, H, 128], 16-byte aligned (output).
 *  dbeta            device, fp32, [B, T, H], 4-byte aligned (output).
 *  d_initial_state  device, fp32, [N, H, 128, 128], 16-byte aligned, or NULL when
 *                   not wanted (output).
 * Rows outside every sequence (varlen) get zero gradients.  Range limit: the
 * same as kda_fwd's (within each 16-token block aligned to the start of a
 * 64-token chunk, the per-channel sum of -g below 80; g >= -5 everywhere is
 * sufficient): every product that pairs exp(G_r) with exp(-G_i) inside a chunk
 * is evaluated with the same 16-row block references as the forward pass.
 * Memory: a workspace of kda_bwd_workspace_bytes(N, rows, H) bytes (rows = T with
 * cu_seqlens, else B*T), taken like kda_fwd's workspace (see Ownership).
 * Asynchrony and errors as kda_fwd.
 */
kda_status kda_bwd(const void* q, const void* k, const void* v, const float* g, const float* beta,
                   float scale, const void* initial_state, int initial_dtype, const void* d_out,
                   const void* d_final_state, int d_final_dtype, const int32_t* cu_seqlens,
                   int32_t num_seqs, int32_t B, int64_t T, int32_t H, int32_t K, int32_t V,
                   float* dq, float* dk, float* dv, float* dg, float* dbeta,
                   float* d_initial_state, void* stream);

/* kda_bwd_check — kda_bwd's host-side validation, with no launch. */
kda_status kda_bwd_check(const void* q, const void* k, const void* v, const float* g,
                         const float* beta, float scale, const void* initial_state,
                         int initial_dtype, const void* d_out, const void* d_final_state,
                         int d_final_dtype, const int32_t* cu_seqlens, int32_t num_seqs,
                         int32_t B, int64_t T, int32_t H, int32_t K, int32_t V, const float* dq,
                         const float* dk, const float* dv, const float* dg, const float* dbeta,
                         const float* d_initial_state);

/* Per-chunk record bytes kda_fwd / kda_gdn_fwd take at head dimension d = 256
 * for N sequences over `rows` packed rows (T with cu_seqlens, else B*T) of H
 * heads: one record per (chunk slot, head), N + ceil(rows / 64) + 1 slots.
 * 0 for d = 64, which takes kda_plan's workspace instead (-1 for N <= 0,
 * rows < 0, H <= 0 or another d).  Host only. */
int64_t kda_dim_workspace_bytes(int32_t n_sequences, int64_t rows, int32_t H, int32_t D);

/* kda_release_workspaces — frees the workspaces the library keeps between calls
 * on the current device, after the device has drained (a host wait); later
 * calls allocate again.  It takes the lock the calls take, so it may run
 * beside calls on other threads.  Returns KDA_ERR_HIP on a runtime error. */
kda_status kda_release_workspaces(void);

/* Workspace bytes kda_bwd takes for N sequences over `rows` packed rows of H
 * heads (-1 for N <= 0, rows < 0 or H <= 0).  Host only.  With
 * s = N + ceil(rows / 64) + 1 chunk slots, it is (each term rounded up to 256 B)
 *   g * H * 722,180 bytes of per-chunk fp32 tiles for one group of g slots
 *     (operands and products), g = min(s, floor(8 GiB / (H * 722,180)));
 *   s * H * 65,536 bytes of fp32 state checkpoints (every chunk's start state);
 *   2 * H * 65,536 bytes of state-gradient carries when g < s;
 *   rows * H * 256 bytes for the forward pass's outputs.
 * Inputs longer than one group go through in groups of g slots, the last group
 * first, so the size grows by about 1.25 KB per token and head beyond 8 GiB (T = 8K
 * at H = 32: one group, 3.3 GB; T = 1M at H = 32: 45 groups, 52 GB).  The environment
 * variable KDA_BWD_GROUP_SLOTS, read at each call, sets g instead (g >= 1; the
 * results do not depend on it).  A call that cannot get the workspace returns
 * KDA_ERR_HIP. */
int64_t kda_bwd_workspace_bytes(int32_t n_sequences, int64_t rows, int32_t H);

#ifdef __cplusplus
}
#endif

#endif /* KDA_H_ */
