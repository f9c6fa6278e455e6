/*
 * sla.h -- C ABI of the MI355X (gfx950) Sparse-Linear Attention library.
 *
 * The operation is the one described by "SLA: Beyond Sparsity in Diffusion
 * Transformers via Fine-Tunable Sparse-Linear Attention" (English abstract and
 * the method section of the paper card): for every query block the key blocks
 * are classified as critical, marginal or negligible; critical blocks get exact
 * O(N^2) softmax attention, marginal blocks O(N) linear attention, negligible
 * blocks are skipped, and the two results are fused into one output; forward
 * and backward are both provided.  The classifier ranks key blocks on a
 * compressed (block mean-pooled) score map, the selection family described in
 * the abstract of "Trainable Log-linear Sparse Attention for Efficient
 * Diffusion Transformers".
 *
 * Concretely, per (batch b, head h), with blocks of 64 tokens, T = N / 64,
 * L = valid_len, scale s, phi(x) = elu(x) + 1:
 *
 *   qbar_i, kbar_j   mean of the valid rows of Q / K block i / j
 *   S_ij             s * qbar_i . kbar_j                       (fp32)
 *   mask[i, j]       per row i, under the order (S_ij descending, j ascending):
 *                    first k_c -> +1 critical, last k_n -> -1 negligible,
 *                    the rest -> 0 marginal
 *   O_s[r]           softmax attention of row r over the valid tokens of the
 *                    critical blocks of its query block (0 when there are none)
 *   h_j, z_j         sum over valid t in block j of phi(k_t) v_t^T and phi(k_t)
 *   H_i, Z_i         sums of h_j, z_j over the marginal blocks of row i
 *   Y[r]             (phi(q_r) H_i) / (phi(q_r) . Z_i)   (0 if the denominator is 0)
 *   O[r]             O_s[r] + Y[r] W^T       (W: d x d, nn.Linear layout, no bias)
 *   rows r >= L      output zero and receive zero gradients
 *
 * with k_c = ceil(frac_critical * T - 1e-6) and k_n = floor(frac_negligible *
 * T + 1e-6) (computed in double from the float fractions).  The backward holds
 * the mask fixed (no gradient through the classifier).
 *
 * Variant (linear_mode = SLA_LINEAR_GLOBAL), after "SALAD: Achieve
 * High-Sparsity Attention via Efficient Linear Attention Tuning for Video
 * Diffusion Transformer" (method: parallel architecture; static-dynamic
 * scaling): the linear branch runs beside the sparse one over every key block,
 * H_i = sum_j h_j and Z_i = sum_j z_j for all i, and its projected output is
 * scaled by a gate g in [0, 1]: O[r] = O_s[r] + g Y[r] W^T.  The mask still
 * selects the critical blocks of the sparse branch.
 *
 * Two-level selection (select_group = G >= 1), after the abstract of
 * "Trainable Log-linear Sparse Attention for Efficient Diffusion Transformers"
 * (top-k chosen level by level, each level looking only at what the coarser
 * level kept): key blocks are grouped G at a time (Tg = ceil(T / G) groups,
 * the last possibly shorter); a group's coarse key kgbar_g is the mean of its
 * valid rows, and per row i, under the order (C_ig descending, g ascending)
 * with C_ig = s * qbar_i . kgbar_g (fp32):
 *   the first select_keep groups are kept, the last n_g = floor(k_n / G)
 *   groups are negligible (every block in them -> -1), and among the blocks of
 *   the kept groups, under the order (S_ij descending, j ascending), the first
 *   k_c -> +1 critical (also inside a negligible group); the rest -> 0.
 * Only the kept groups' fine scores are computed, so the selection costs
 * T * (Tg + select_keep * G) scores instead of T * T.  G = 1 with
 * select_keep = T is the flat rule above.
 *
 * Conventions for every entry point below:
 *  - Tensors are contiguous, row-major.  Q, K, V, O, dO are bf16 [B, H, N, d]
 *    ("BHND"); W is bf16 [d, d]; dQ, dK, dV, dW are fp32.  Device pointers must
 *    be 16-byte aligned.
 *  - The caller owns every buffer.  The library allocates no device memory,
 *    copies nothing between host and device and never synchronises the stream.
 *    Scratch memory is the caller's ``workspace`` (size from
 *    sla_workspace_size); state handed from forward to backward is the
 *    caller's ``saved`` buffer (size from sla_saved_size).
 *  - SLA_OK means "all work enqueued on ``stream``" (a hipStream_t; NULL is the
 *    default stream).  Arguments are validated on the host before anything is
 *    enqueued; on an error nothing is enqueued and no output is touched, and
 *    sla_last_error() returns a thread-local description.  A failed launch
 *    returns SLA_ERR_DEVICE; device faults surface at the caller's next
 *    synchronisation.
 *  - Outputs are overwritten, never accumulated; inputs are never written.
 *  - Calls are reentrant: no mutable global state apart from the static
 *    scratch of sla_forward_static (below).  Two calls that share a
 *    workspace or saved buffer must be ordered on one stream.
 */
#ifndef SLA_H_
#define SLA_H_

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum sla_status {
  SLA_OK = 0,
  SLA_ERR_INVALID_ARGUMENT = 1, /* bad shape, fraction, pointer or alignment */
  SLA_ERR_UNSUPPORTED = 2,      /* valid but not implemented (e.g. head_dim 96) */
  SLA_ERR_WORKSPACE = 3,        /* workspace smaller than sla_workspace_size() */
  SLA_ERR_DEVICE = 4            /* a HIP launch or runtime call failed */
} sla_status;

/* mask_mode */
enum {
  SLA_MASK_COMPUTE = 0, /* forward classifies and writes ``mask`` */
  SLA_MASK_GIVEN = 1    /* forward reads a caller-supplied ``mask`` (fixed mask) */
};

/* linear_mode */
enum {
  SLA_LINEAR_MARGINAL = 0, /* the method: linear branch over the marginal blocks of each row */
  SLA_LINEAR_GLOBAL = 1    /* variant: linear branch over every key block, output gated */
};

/* Number of timed stages in stage_events (see sla_config). */
#define SLA_NUM_STAGES 8
enum {
  SLA_STAGE_KV_STATE = 0,   /* forward: per-key-block states and pooled K   */
  SLA_STAGE_POOL_Q = 1,     /* forward: pooled Q                            */
  SLA_STAGE_CLASSIFY = 2,   /* forward: compressed scores + classification  */
  SLA_STAGE_AGGREGATE = 3,  /* forward: marginal sums H_i, Z_i (or totals)  */
  SLA_STAGE_ATTENTION = 4,  /* forward: fused sparse + linear + projection  */
  SLA_STAGE_BWD_PRE = 5,    /* backward: mask lists, D, dN, dW partials,
                                dH / dZ and their transposed sums        */
  SLA_STAGE_BWD_KV = 6,     /* backward: dK and dV (sparse + linear)        */
  SLA_STAGE_BWD_Q = 7       /* backward: dQ (sparse + linear), dW reduction */
};

typedef struct sla_config {
  int32_t batch;           /* B >= 1 */
  int32_t heads;           /* H >= 1 */
  int32_t seq_len;         /* N: a positive multiple of 64 */
  int32_t head_dim;        /* d: 64 or 128 */
  int32_t valid_len;       /* L: 0 means N; otherwise N - 64 < L <= N */
  int32_t block;           /* 64 (the only supported block size) */
  float frac_critical;     /* in [0, 1] */
  float frac_negligible;   /* in [0, 1]; k_c + k_n <= T */
  float softmax_scale;     /* <= 0 means 1 / sqrt(d) */
  int32_t mask_mode;       /* SLA_MASK_COMPUTE or SLA_MASK_GIVEN (forward only) */
  /* Optional per-stage timing: NULL, or an array of 2 * SLA_NUM_STAGES
     hipEvent_t created by the caller with timing enabled.  When set, the
     library records event [2 s] before and [2 s + 1] after stage s on
     ``stream`` (stages a call does not run are left unrecorded). */
  void* stage_events;
  int32_t linear_mode;     /* SLA_LINEAR_MARGINAL (0) or SLA_LINEAR_GLOBAL */
  float linear_gate;       /* SLA_LINEAR_GLOBAL only: g in [0, 1]; ignored otherwise */
  int32_t select_group;    /* 0: flat selection; G >= 1: two-level selection with groups of
                              G key blocks (SLA_MASK_COMPUTE only) */
  int32_t select_keep;     /* two-level only: groups kept per query block, in [1, Tg]; the
                              kept groups must hold k_c blocks even when the shorter last
                              group is among them */
} sla_config;

/* k_c, k_n, k_m (= T - k_c - k_n) for the configuration.  Host only. */
sla_status sla_block_counts(const sla_config* cfg, int32_t* k_c, int32_t* k_n, int32_t* k_m);

/* Bytes of scratch needed by sla_forward, sla_backward and sla_pool_scores
   for this configuration (one size serves all three); 0 if cfg is invalid. */
size_t sla_workspace_size(const sla_config* cfg);

/* Bytes of the forward-to-backward state written by sla_forward; 0 if invalid.
   Layout (each region 256-byte aligned, offsets from sla_saved_offsets):
     lse  fp32 [B,H,N]     log-sum-exp of the critical logits (-inf if none)
     den  fp32 [B,H,N]     linear denominator phi(q) . Z_i
     y    bf16 [B,H,N,d]   normalised linear output Y (before W)
     hst  bf16 [B,H,T,d,d] H_i stored transposed: element (c, a) at c*d + a
     zst  fp32 [B,H,T,2,d] Z_i as two fp32 parts whose sum is Z_i
   (SLA_LINEAR_GLOBAL: H and Z are the same for every i and only i = 0 is
   written).                                                                 */
size_t sla_saved_size(const sla_config* cfg);
sla_status sla_saved_offsets(const sla_config* cfg, size_t* lse, size_t* den, size_t* y,
                             size_t* hst, size_t* zst);

/*
 * Forward.  q, k, v: bf16 [B,H,N,d]; w: bf16 [d,d]; o: bf16 [B,H,N,d] (out).
 * mask: int8 [B,H,T,T]; written when mask_mode is SLA_MASK_COMPUTE, read when
 * SLA_MASK_GIVEN (values must be -1, 0 or +1; a given mask need not have the
 * k_c / k_n row counts).  saved: sla_saved_size() bytes (out), needed by
 * sla_backward.  With frac_critical = 1 and frac_negligible = 0 the call is
 * plain dense softmax attention (linear branch empty).
 */
sla_status sla_forward(const sla_config* cfg, const void* q, const void* k, const void* v,
                       const void* w, void* o, int8_t* mask, void* saved, void* workspace,
                       size_t workspace_bytes, void* stream);

/*
 * Backward of sum(dO * O) with the mask held fixed.  q, k, v, w, o, d_o as in
 * the forward (o is the forward's output, d_o bf16 [B,H,N,d]); mask and saved
 * exactly as the forward wrote or read them for the same inputs.  dq, dk, dv:
 * fp32 [B,H,N,d] (out); dw: fp32 [d,d] (out), summed over batch, heads and
 * valid rows.  Deterministic: no atomics in any reduction.
 */
sla_status sla_backward(const sla_config* cfg, const void* q, const void* k, const void* v,
                        const void* w, const void* o, const void* d_o, const int8_t* mask,
                        const void* saved, float* dq, float* dk, float* dv, float* dw,
                        void* workspace, size_t workspace_bytes, void* stream);

/*
 * Allocation-free forward, for callers that cannot allocate device memory or
 * hand the library a workspace: code under HIP graph capture, tight serving
 * loops (a denoising loop that calls the layer every step), harnesses that
 * forbid hipMalloc.  Same arguments and results as sla_forward without the
 * workspace: the scratch is a fixed device array of SLA_STATIC_SCRATCH_BYTES
 * inside the library, one per GPU, which each GPU the library runs on holds
 * until the process ends.  The call allocates nothing and uses the array of
 * the current device (``stream`` must belong to it).  The B*H (batch, head)
 * problems run in passes of as many problems as the array holds, so outputs
 * are bit-identical to sla_forward's; a configuration whose single (batch,
 * head) problem needs more scratch than the array returns SLA_ERR_WORKSPACE
 * before anything is enqueued (at d = 128 above T = 1440, i.e. N = 92160; every
 * supported size fits at d = 64).
 * cfg->stage_events is ignored.  Every call on one GPU shares that GPU's
 * array, whose contents persist between calls: two calls that can overlap on
 * one GPU (different streams, or threads without ordering) race on it and
 * must be serialised by the caller.
 */
#define SLA_STATIC_SCRATCH_BYTES (64ull << 20)
sla_status sla_forward_static(const sla_config* cfg, const void* q, const void* k,
                              const void* v, const void* w, void* o, int8_t* mask, void* saved,
                              void* stream);

/* The compressed score map alone: scores fp32 [B,H,T,T] (out), bit-identical
   to the map sla_forward classifies in SLA_MASK_COMPUTE mode. */
sla_status sla_pool_scores(const sla_config* cfg, const void* q, const void* k, float* scores,
                           void* workspace, size_t workspace_bytes, void* stream);

/* Classification alone: scores fp32 [B,H,T,T] (in, finite) -> mask int8
   [B,H,T,T] (out), by the rule above.  Uses cfg's sizes and fractions only. */
sla_status sla_classify(const sla_config* cfg, const float* scores, int8_t* mask, void* stream);

/* Two-level selection (cfg->select_group >= 1): the coarse score map alone,
   coarse fp32 [B,H,T,Tg] (out), bit-identical to the map the forward ranks. */
sla_status sla_coarse_scores(const sla_config* cfg, const void* q, const void* k, float* coarse,
                             void* workspace, size_t workspace_bytes, void* stream);

/* Two-level classification alone (cfg->select_group >= 1): coarse fp32
   [B,H,T,Tg] and scores fp32 [B,H,T,T] (in, finite; only the entries of kept
   groups are read) -> mask int8 [B,H,T,T] (out), by the two-level rule.  With
   the maps of sla_coarse_scores and sla_pool_scores it reproduces the mask of
   sla_forward exactly. */
sla_status sla_classify_hier(const sla_config* cfg, const float* coarse, const float* scores,
                             int8_t* mask, void* stream);

/* Static description of a status code. */
const char* sla_status_string(sla_status status);

/* Thread-local description of the last failure in this thread ("" if none). */
const char* sla_last_error(void);

#ifdef __cplusplus
}
#endif

#endif /* SLA_H_ */
