/*
 * streamkl.h — C ABI of the fused attention KL-divergence library for AMD
 * Instinct MI355X (gfx950).
 *
 * The operation (StreamKL, arXiv 2606.20005; technical summary pages
 * "StreamKL" on gist.science, ja/fr/ko):
 *
 *   S_t = scale_t * Q_t K_t^T            t = 1 (teacher), 2 (student)
 *   P_t = row-wise softmax of S_t over the visible keys
 *   KL[i] = sum_j P1[i,j] (log P1[i,j] - log P2[i,j])   = KL(P1 || P2)
 *
 * computed in one streaming pass over key tiles without materialising the
 * N_Q x N_K distributions (Problem statement; Method 1, online formulation
 * L = acc/l1 + LSE2 - LSE1 with LSE_t = m_t + log l_t).  Only KL, LSE1 and
 * LSE2 are kept for the backward, which regenerates P_t = exp(S_t - LSE_t)
 * tile by tile (Method 2, recomputation strategy).
 *
 * Conventions shared by every entry point
 * ---------------------------------------
 * - Tensor pointers are DEVICE pointers (HIP device memory of the current
 *   device), 16-byte aligned.  Descriptor pointers (streamkl_shape,
 *   streamkl_launch) are HOST pointers, read during the call only.
 * - Q_t is [B, H, n_q, d_t] and K_t is [B, H, n_k, d_t] (or [B, kv_heads_t,
 *   n_k, d_t] with grouped key heads, see streamkl_shape), row-major and
 *   contiguous, all four in the dtype of shape->dtype (fp32 or bf16).
 *   Supported head dims: d_t in {64, 128}; d1 and d2 may differ.
 * - Per-row vectors (kl, lse1, lse2, d_kl) are fp32 [B, H, n_q].
 * - causal != 0 applies a bottom-right aligned mask: key j is visible to
 *   query i iff j <= i + (n_k - n_q); this requires n_q <= n_k.  Key tiles
 *   past the boundary are skipped (Method 1).
 * - scale_t must be a finite number; scale_t <= 0 selects 1/sqrt(d_t)
 *   (NaN or an infinite scale returns STREAMKL_ERR_INVALID).
 * - LSE values are natural logarithms.
 * - `stream` is a hipStream_t (NULL = the null stream).  Every call only
 *   enqueues work: no host synchronisation, no device allocation, no
 *   device memory freed.  The caller owns every buffer, including the
 *   workspace.
 * - Every argument is validated on the host before anything is enqueued;
 *   a call that returns an error has enqueued nothing and written nothing.
 *   Errors are reported only through the return value.  If a HIP launch
 *   fails the call returns STREAMKL_ERR_HIP and streamkl_last_hip_error()
 *   gives the hipError_t value (per calling thread).
 */
#ifndef STREAMKL_H_
#define STREAMKL_H_

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  STREAMKL_OK = 0,
  STREAMKL_ERR_INVALID = 1,     /* null pointer, bad size, misaligned pointer, bad enum */
  STREAMKL_ERR_UNSUPPORTED = 2, /* head dim outside {64,128}, device not gfx950 */
  STREAMKL_ERR_WORKSPACE = 3,   /* split-K requested but workspace missing or too small */
  STREAMKL_ERR_HIP = 4          /* a HIP runtime call failed */
} streamkl_status;

typedef enum { STREAMKL_F32 = 0, STREAMKL_BF16 = 1 } streamkl_dtype;

typedef enum {
  STREAMKL_BWD_AUTO = 0,     /* choose by the cost model of streamkl_bwd_plan */
  STREAMKL_BWD_FUSED = 1,    /* one kernel visits each key tile once, dQ by fp32 atomics; bf16 with
                                n_q <= 32: one workgroup keeps every query row, sums dQ over its key
                                tiles and adds it once (the auto choice for those shapes) */
  STREAMKL_BWD_SEPARATE = 2, /* a key-outer dK kernel, then a query-outer dQ kernel */
  STREAMKL_BWD_DK_ONLY = 3,  /* only the key-outer dK kernel; dQ is not touched (may be NULL) */
  STREAMKL_BWD_DQ_ONLY = 4   /* only the query-outer dQ kernel; dK is not touched (may be NULL) */
} streamkl_bwd_mode;

/* Problem shape (host struct). */
typedef struct {
  int64_t B, H, n_q, n_k;
  int32_t d1, d2;   /* head dims of model 1 (teacher) and model 2 (student) */
  int32_t dtype;    /* streamkl_dtype */
  /* Key heads of model 1 and model 2 (grouped-query attention): K_t is
   * [B, kv_heads_t, n_k, d_t] and query head h reads key head
   * h / (H / kv_heads_t).  0 means H (every query head has its own keys).
   * kv_heads_t must divide H.  dK_t is then [B, kv_heads_t, n_k, d_t], the
   * sum over the query heads that share each key head. */
  int32_t kv_heads1, kv_heads2;
  /* Ragged batches (HOST arrays of B lengths, or NULL for all n_q / n_k):
   * batch element b uses its first q_len[b] query rows and k_len[b] key rows
   * of the padded tensors (n_q, n_k rows per head in memory), with
   * 0 <= q_len[b] <= n_q, 0 <= k_len[b] <= n_k, k_len[b] >= 1 when
   * q_len[b] >= 1, and q_len[b] <= k_len[b] under a causal mask (aligned
   * bottom-right within the element).  Outputs of padded rows (KL, LSE, dQ,
   * dK) are 0.  Read during the call only.  Elements that run the same
   * kernel share a launch (up to 64 per launch); a grouped element computes
   * what a call on its trimmed tensors with the same split count computes. */
  const int64_t* q_len;
  const int64_t* k_len;
  /* Packed batches (HOST arrays of B + 1 row offsets, or NULL; set both or
   * neither, and then leave q_len and k_len NULL): the sequences lie one
   * after another in every head, with no padding.  Batch element b owns
   * query rows [q_off[b], q_off[b+1]) and key rows [k_off[b], k_off[b+1])
   * of every head.  The tensors have no batch dimension: Q_t [H, n_q, d_t],
   * K_t [kv_heads_t, n_k, d_t], KL, LSE1, LSE2, weights and d_kl [H, n_q],
   * dQ_s [H, n_q, d_s], dK_s [kv_heads_s, n_k, d_s], where n_q = q_off[B]
   * and n_k = k_off[B] are the total rows.  Offsets start at 0 and never
   * decrease, and each element's lengths follow the rules of ragged batches
   * above, and the batch holds at least one query and one key row.  The
   * same per-sequence kernels serve both layouts; a packed batch has no
   * padded rows to clear.  Read during the call only. */
  const int64_t* q_off;
  const int64_t* k_off;
} streamkl_shape;

/* Launch options (host struct; a NULL pointer means all defaults). */
typedef struct {
  int32_t num_splits;      /* forward: 0 = auto, 1 = no key split, k = k key splits */
  int32_t bwd_mode;        /* streamkl_bwd_mode */
  void* workspace;         /* device memory for split-K partial states, may be NULL */
  size_t workspace_bytes;
} streamkl_launch;

/* Returned by the workspace queries below for invalid arguments. */
#define STREAMKL_INVALID_BYTES ((size_t)-1)

/*
 * Bytes of workspace the forward needs for this shape and launch options
 * (0 when no key split is used).  With num_splits = 0 (auto) this is the
 * size for the split count the library would choose.  Returns
 * STREAMKL_INVALID_BYTES for invalid arguments.  Split-K: the technical
 * summary, Method 3 (GPU kernel optimisations), partitions the key
 * dimension across thread blocks for small N_Q; each split leaves five fp32
 * partial scalars per row, so the workspace is 20 * B * H * n_q * splits
 * bytes.  Ragged batches: the largest of what any launch needs, launches
 * reusing it one after another; the split decode-shaped elements (bf16,
 * at most 32 query rows) of one grouped launch hold their partials side by
 * side.  A smaller workspace that still holds each element's own partials
 * runs those elements one after another instead.
 */
size_t streamkl_fwd_workspace_bytes(const streamkl_shape* shape, int causal,
                                    const streamkl_launch* launch);

/*
 * Bytes of workspace streamkl_fwd_loss needs: the split partials above
 * (rounded up to 256 bytes), then one fp64 partial sum per workgroup that
 * finalizes query rows (for the fused loss).  STREAMKL_INVALID_BYTES for
 * invalid arguments.
 */
size_t streamkl_fwd_loss_workspace_bytes(const streamkl_shape* shape, int causal,
                                         const streamkl_launch* launch);

/*
 * Bytes of workspace the backward needs: 0 for every valid shape, setting
 * and mode (Method 2, recomputation strategy: the backward regenerates P_t
 * from the stored LSE tile by tile and keeps everything else in registers
 * and LDS; the fused mode accumulates dQ in the caller's output).
 * STREAMKL_INVALID_BYTES for an invalid shape, setting (not 1 or 2) or
 * launch option.  Callers may size a backward workspace generically with it.
 */
size_t streamkl_bwd_workspace_bytes(const streamkl_shape* shape, int causal, int setting,
                                    const streamkl_launch* launch);

/* The key-split count the forward will use (>= 1), or 0 for invalid input. */
int streamkl_fwd_plan(const streamkl_shape* shape, int causal, const streamkl_launch* launch);

/*
 * Forward: KL[i], LSE1[i], LSE2[i] for every query row (Method 1).
 * Inputs Q1, K1, Q2, K2 (device, read only).  Outputs out_kl, out_lse1,
 * out_lse2 (device, fp32 [B,H,n_q], fully overwritten).  A split-K launch
 * (launch->num_splits > 1, or auto with a workspace given) writes partial
 * states to launch->workspace and merges them in a second kernel on the
 * same stream; if the needed workspace is not given, auto mode falls back
 * to one split and an explicit split count returns STREAMKL_ERR_WORKSPACE.
 */
streamkl_status streamkl_fwd(const void* Q1, const void* K1, const void* Q2, const void* K2,
                             int causal, float scale1, float scale2,
                             float* out_kl, float* out_lse1, float* out_lse2,
                             const streamkl_shape* shape, const streamkl_launch* launch,
                             void* stream);

/*
 * Forward with the distillation loss fused into its epilogue (the pages
 * name attention distillation as what the KL serves: technical summary,
 * Significance; the preprint's abstract).  Everything streamkl_fwd does,
 * plus, when out_loss is not NULL, *out_loss = sum_i w_i KL_i over every
 * query row (weights: device fp32 [B,H,n_q], or NULL for the mean KL over
 * the rows; ragged batches count only each element's rows, and a batch of
 * empty elements has the loss 0 and needs no workspace).  Each
 * workgroup that finalizes rows writes the sum of its rows' w_i KL_i to the
 * workspace and one small kernel adds those partials in a fixed order, so
 * the loss is bitwise repeatable and no second pass reads the KL.  The
 * loss's gradient with respect to KL_i is w_i (or 1 / rows): the d_kl that
 * streamkl_bwd takes.  out_loss: device, one fp32, 4-byte aligned.
 * The workspace (launch->workspace, 16-byte aligned) must hold
 * streamkl_fwd_loss_workspace_bytes; with num_splits = 0 a smaller one
 * that still holds the loss partials of an unsplit forward falls back to
 * one split, otherwise the call returns STREAMKL_ERR_WORKSPACE.  With
 * out_loss NULL the call is streamkl_fwd.
 */
streamkl_status streamkl_fwd_loss(const void* Q1, const void* K1, const void* Q2, const void* K2,
                                  int causal, float scale1, float scale2, const float* weights,
                                  float* out_kl, float* out_lse1, float* out_lse2, float* out_loss,
                                  const streamkl_shape* shape, const streamkl_launch* launch,
                                  void* stream);

/*
 * streamkl_fwd_loss for callers that cannot allocate device memory (code
 * under HIP graph capture, tight serving loops, harnesses that forbid
 * hipMalloc): the split-K partial states and the fused-loss partial sums go
 * to a scratch array inside the library instead of a caller workspace.  The
 * array holds STREAMKL_NOALLOC_SCRATCH_BYTES (4 MiB) on every device the
 * library runs on, from the library's first use on that device (when its
 * code is loaded there) until the process ends; the call allocates and
 * frees nothing.  Arguments, outputs and
 * semantics are those of streamkl_fwd_loss (out_loss may be NULL: the plain
 * forward), except that launch->workspace and launch->workspace_bytes are
 * ignored.  If the partials the plan needs do not fit in the scratch, an
 * automatic split count falls back to fewer partials (one split) and
 * otherwise the call returns STREAMKL_ERR_WORKSPACE having written nothing
 * (e.g. an explicit split count whose 20 * B * H * n_q * splits bytes exceed
 * it).  Every call on one device shares its scratch: calls that overlap in
 * time on one device (other streams, other threads) race and give undefined
 * results; calls ordered on one stream are safe.  Nothing in the scratch
 * needs clearing: every partial is written before it is read.
 */
#define STREAMKL_NOALLOC_SCRATCH_BYTES ((size_t)4 << 20)
streamkl_status streamkl_fwd_loss_noalloc(const void* Q1, const void* K1, const void* Q2, const void* K2,
                                          int causal, float scale1, float scale2, const float* weights,
                                          float* out_kl, float* out_lse1, float* out_lse2, float* out_loss,
                                          const streamkl_shape* shape, const streamkl_launch* launch,
                                          void* stream);

/* The backward mode streamkl_bwd will use (1 fused, 2 separate, or the
 * requested 3/4), 0 if invalid.  For a ragged batch, padded or packed, it is
 * the mode of the padded batch of the longest query and key lengths: the
 * plan streamkl_bwd_joint takes for the whole batch (in the automatic mode,
 * streamkl_bwd plans each element, or each group of elements, on its own). */
int streamkl_bwd_plan(const streamkl_shape* shape, int causal, int setting,
                      const streamkl_launch* launch);

/*
 * Backward (Method 2): gradients of sum_i d_kl[i] * KL[i].
 *  setting 1: P1 held fixed, gradients to the student:  dQ = dQ2, dK = dK2
 *             (dS2 = g (P2 - P1)), shapes [B,H,n_q,d2] and [B,H,n_k,d2];
 *  setting 2: P2 held fixed, gradients to the teacher:  dQ = dQ1, dK = dK1
 *             (dS1 = g P1 ((S1 - LSE1) - (S2 - LSE2) - KL), the log-ratio
 *             formed from logits and the stored LSE, Method 3), shapes with d1.
 * kl, lse1, lse2: the forward's outputs for the same inputs (device, fp32).
 *   setting 1 does not read kl (it may be NULL).
 * d_kl: upstream gradient per row (device, fp32 [B,H,n_q]).
 * dQ, dK: device fp32 outputs, fully overwritten (the fused mode clears dQ
 *   itself before accumulating into it with atomics, on the same stream).
 *   With bwd_mode DK_ONLY (DQ_ONLY) only dK (dQ) is computed and the other
 *   pointer may be NULL; these serve callers that train only keys or only
 *   queries, and per-kernel timing.
 * No workspace is needed (streamkl_bwd_workspace_bytes returns 0).
 */
streamkl_status streamkl_bwd(int setting,
                             const void* Q1, const void* K1, const void* Q2, const void* K2,
                             int causal, float scale1, float scale2,
                             const float* kl, const float* lse1, const float* lse2,
                             const float* d_kl, float* dQ, float* dK,
                             const streamkl_shape* shape, const streamkl_launch* launch,
                             void* stream);

/*
 * Joint backward: the gradients of sum_i d_kl[i] * KL[i] with respect to
 * both models at once (when teacher and student are both trained), equal to
 * setting 2 (dQ1 [B,H,n_q,d1], dK1 [B,H,n_k,d1]) and setting 1 (dQ2, dK2,
 * with d2) of streamkl_bwd.  Both settings need S1, S2 and P1 per tile
 * (Method 2): the key-outer kernel recomputes them once per tile pair and
 * forms dS1 and dS2 from them, accumulating dK1 and dK2 together
 * (2(d1+d2) + 2(d1+d2) matrix FLOPs per visible pair instead of twice
 * 2(d1+d2) + 2 d_s); dQ1 and dQ2 come from the query-outer kernel of each
 * setting.  bf16 in the separate mode only; fp32 inputs, and shapes whose
 * plan is the fused mode (few query rows), run the two settings one after the
 * other.  kl is required.  dQ1, dQ2 must be 16-byte aligned.
 * launch->bwd_mode DK_ONLY (DQ_ONLY) computes dK1 and dK2 (dQ1 and dQ2) only.
 * Every argument is checked before anything is enqueued; all four outputs are
 * fully overwritten.
 */
streamkl_status streamkl_bwd_joint(const void* Q1, const void* K1, const void* Q2, const void* K2,
                                   int causal, float scale1, float scale2,
                                   const float* kl, const float* lse1, const float* lse2,
                                   const float* d_kl, float* dQ1, float* dK1, float* dQ2, float* dK2,
                                   const streamkl_shape* shape, const streamkl_launch* launch,
                                   void* stream);

/*
 * Distillation loss from the forward's per-row KL: *out = sum_i w_i KL_i
 * over rows = B*H*n_q rows, or the mean KL when weights is NULL (device
 * pointers: kl and weights fp32 [rows], out one fp32).  Deterministic: one
 * workgroup sums in a fixed order, in fp64.  Its gradient with respect to
 * KL_i is w_i (or 1/rows), the d_kl that streamkl_bwd takes.  The loss is
 * the quantity the pages distil with; the fused kernels above keep it per
 * row so callers can weight, mask or reduce it as they need.
 */
streamkl_status streamkl_kl_loss(const float* kl, const float* weights, int64_t rows, float* out,
                                 void* stream);

/* Static text for a status code. */
const char* streamkl_status_string(int status);

/* hipError_t of the last STREAMKL_ERR_HIP returned on this thread (0 if none). */
int streamkl_last_hip_error(void);

/* Library version, for the Python binding's load check (3: streamkl_shape
 * carries kv_heads1, kv_heads2 and the ragged-batch lengths; 4: the fused
 * loss, the backward workspace query, STREAMKL_INVALID_BYTES; 5:
 * streamkl_shape carries the packed-batch offsets q_off, k_off). */
int streamkl_version(void);

#ifdef __cplusplus
}
#endif

#endif /* STREAMKL_H_ */
