/*
 * libctopk -- certified Top-k attention truncation on AMD Instinct MI355X (gfx950).
 *
 * What the library computes, per query head h (definitions from the Abstract
 * of "A Mathematical Theory of Top-k Sparse Attention via Total Variation
 * Distance", arXiv 2512.07647):
 *
 *   s_i    = scale_h * <q_h, k_i>                 for every key i in [0, n)
 *   P      = softmax(s)                            the attention distribution
 *   order  = keys by score descending, index ascending among equal scores
 *   T_k    = softmax mass of the keys after the first k of that order
 *            (= TV(P, P_hat_k), the total-variation distance between P and its
 *            Top-k truncation)
 *   k_eps  = min { k in 1..n : T_k <= eps }        smallest certified head
 *   tau    = T_{k_eps}
 *   out_h  = sum_{i in H} P_i v_i / sum_{i in H} P_i   (H = first k_eps keys),
 *            the renormalised head-only output Attn_k(q, K, V).
 *
 * Conventions shared by every entry point:
 *   - Every array pointer is a DEVICE pointer owned by the caller.  The library
 *     never frees, retains or reads them after the enqueued work completes.
 *   - All arrays are dense and row-major.  q is [n_q_heads, d]; K and V are
 *     [n_kv_heads, n, d]; query head h reads KV head h / (n_q_heads / n_kv_heads)
 *     (grouped-query attention; batch is folded into the head dimensions).
 *   - Calls are asynchronous: work is enqueued on `stream` (NULL = the default
 *     stream) and the call returns.  No device-to-host copy, no host sync,
 *     with one exception: a call made without a caller workspace (other than
 *     ctopk_certify_noalloc) uses the library's cached per-device workspace,
 *     and when it needs more scratch than that holds it first waits for the
 *     whole device (hipDeviceSynchronize), frees it and allocates a larger one
 *     (hipMalloc); later calls with the same or smaller sizes never do.  Pass
 *     a workspace, or use ctopk_certify_noalloc, to avoid it.
 *   - Argument errors are detected on the host before anything is enqueued and
 *     return a negative ctopk_status; ctopk_last_error_string() describes the
 *     last error of the calling thread.  A failed kernel launch returns
 *     CTOPK_ERR_HIP.  Faults inside kernels surface at the caller's next sync.
 *   - No C++ exception crosses this interface.
 *   - Inputs must be finite.  NaN or infinite scores give unspecified results.
 *   - Inputs and outputs must not alias.
 */
#ifndef CTOPK_H
#define CTOPK_H

#include <stddef.h>
#include <stdint.h>

#if defined(__GNUC__)
#define CTOPK_API __attribute__((visibility("default")))
#else
#define CTOPK_API
#endif

#ifdef __cplusplus
extern "C" {
#endif

/* Same type as HIP's hipStream_t (a pointer to the runtime's stream object). */
typedef struct ihipStream_t* ctopk_stream_t;

typedef enum {
  CTOPK_OK = 0,
  CTOPK_ERR_NULL = -1,        /* a required pointer is NULL                      */
  CTOPK_ERR_SHAPE = -2,       /* n, d, head counts or their ratio are invalid    */
  CTOPK_ERR_EPS = -3,         /* eps is not a finite number in (0, 1)           */
  CTOPK_ERR_ALIGN = -4,       /* an input/output pointer is not 16-byte aligned  */
  CTOPK_ERR_UNSUPPORTED = -5, /* valid request the library does not handle       */
  CTOPK_ERR_WORKSPACE = -6,   /* caller workspace too small                      */
  CTOPK_ERR_HIP = -7          /* a HIP runtime call or kernel launch failed      */
} ctopk_status;

typedef enum { CTOPK_F32 = 0, CTOPK_BF16 = 1 } ctopk_dtype;

/*
 * ctopk_certify -- the decode call.
 *
 * q [n_q_heads, d], K [n_kv_heads, n, d], V [n_kv_heads, n, d]: bfloat16.
 * scale_h = float(1/sqrt(d)) for every head.  d must be 64 or 128;
 * 1 <= n <= 2^31 - 1; n_q_heads must be a multiple of n_kv_heads.
 * Outputs: out [n_q_heads, d] float32, k_eps [n_q_heads] int32,
 * tau [n_q_heads] float64.
 * Scratch memory comes from a per-device workspace that the library allocates
 * on first use and grows as needed (hipMalloc); it is shared by all calls on a
 * device, so concurrent calls on different streams of one device race.  Use
 * ctopk_certify_ex with a caller workspace for concurrent streams.
 */
CTOPK_API int ctopk_certify(const void* q, const void* K, const void* V, int64_t n, int32_t d,
                  int32_t n_q_heads, int32_t n_kv_heads, double eps, ctopk_stream_t stream,
                  float* out, int32_t* k_eps, double* tau);

/*
 * ctopk_certify_noalloc -- ctopk_certify for callers that cannot allocate
 * device memory: code under HIP graph capture, tight serving loops, and
 * harnesses that forbid hipMalloc.  Same arguments, outputs and kernels as
 * ctopk_certify; the scratch memory is instead one fixed device array of
 * CTOPK_NOALLOC_SCRATCH_BYTES bytes owned by the library (one per GPU, held
 * until the process ends; its address is looked up once per device on the
 * first call there).  The call makes no hipMalloc or hipFree and calls no
 * allocating library routine.  Returns CTOPK_ERR_WORKSPACE, before anything
 * is enqueued, when ctopk_workspace_bytes(n, d, n_q_heads, n_kv_heads,
 * CTOPK_BF16) exceeds that size, and the other statuses as ctopk_certify.
 * Every call on a GPU uses that GPU's one array, so calls that overlap on a
 * GPU (on different streams, or from several host threads) race; calls
 * ordered on one stream do not.  Nothing in the array needs to start at zero.
 */
#define CTOPK_NOALLOC_SCRATCH_BYTES (32u * 1024u * 1024u)
CTOPK_API int ctopk_certify_noalloc(const void* q, const void* K, const void* V, int64_t n,
                                    int32_t d, int32_t n_q_heads, int32_t n_kv_heads, double eps,
                                    ctopk_stream_t stream, float* out, int32_t* k_eps,
                                    double* tau);

/* Full-form arguments of ctopk_certify_ex. */
typedef struct ctopk_args {
  const void* q;            /* [n_q_heads, d], dtype                                   */
  const void* K;            /* [n_kv_heads, n, d], dtype                               */
  const void* V;            /* [n_kv_heads, n, d], dtype                               */
  int32_t dtype;            /* ctopk_dtype of q, K and V                               */
  int64_t n;                /* keys per head, 1 .. 2^31 - 1                            */
  int32_t d;                /* head dimension, 64 or 128                               */
  int32_t n_q_heads;        /* query heads (query rows)                                */
  int32_t n_kv_heads;       /* KV heads; divides n_q_heads                             */
  double eps;               /* TV budget, finite, 0 < eps < 1                          */
  const float* head_scale;  /* [n_q_heads] score scale per query head; NULL: 1/sqrt(d) */
  void* workspace;          /* caller scratch (device), or NULL for the cached one     */
  size_t workspace_bytes;   /* size of `workspace`; >= ctopk_workspace_bytes(...)      */
  float* out;               /* [n_q_heads, d] float32                                  */
  int32_t* k_eps;           /* [n_q_heads]                                             */
  double* tau;              /* [n_q_heads]                                             */
  uint32_t* sel_mask;       /* optional [n_q_heads, ceil(n/32)]: bit (i%32) of word
                               i/32 is set iff key i is in the head set; NULL: skip   */
  float* scores;            /* optional [n_q_heads, n] float32 scores as computed;
                               NULL: kept in the workspace                            */
  double* lse;              /* optional [n_q_heads] log-sum-exp of the scores; NULL    */
  /* Output-level certificate (head-tail factorisation in the Abstract): when
     either pointer, or out_var below, is non-NULL the value pass also
     accumulates the tail.                                                     */
  double* out_err;          /* optional [n_q_heads] ||Attn - Attn_k||_2 = tau *
                               ||mu_tail - mu_head||_2 (fp64); NULL: skip          */
  float* out_dense;         /* optional [n_q_heads, d] untruncated softmax output
                               Attn (fp32); NULL: skip                              */
  uint32_t flags;           /* CTOPK_FLAG_* bits; 0 for the exact certificate        */
  double* out_var;          /* optional [n_q_heads] Var_P(V) = sum_i P_i ||v_i - Attn||^2
                               (fp64; accumulated with the tail like out_err): the
                               Abstract refines the output error by it, and with
                               the factorisation above the law of total variance
                               gives ||Attn - Attn_k||_2 <= sqrt(tau Var_P(V) /
                               (1 - tau)); NULL: skip                                */
} ctopk_args;

/*
 * CTOPK_FLAG_BOUND -- certify with the blockwise deterministic bound instead
 * of the exact minimal k (the Abstract's "blockwise variants" of the bounds
 * that control TV from the ordered logits; its formula is not printed, this
 * is the library's reading).  With the keys in consecutive blocks B of 64
 * (maxima M_B, m the row maximum), the softmax mass of the keys scoring below
 * t is at most U(t) = sum_{M_B < t} |B| e^{M_B - m} + sum_{M_B >= t} (|B| - 1)
 * e^{t - m}; the call keeps every key scoring at or above an fp32 t with
 * U(t) <= eps * Z, the largest such t that a search of up to six rounds of 64
 * candidates finds (on the shapes tested, the largest to fp32 resolution).
 * Outputs then mean: k_eps = number of keys kept (at least the minimal k),
 * tau = U(t) / Z with the block masses rounded up (an upper bound on the
 * truncation's TV, <= eps), out = the renormalised output over the kept keys,
 * sel_mask = the kept keys.  Any shape the general path takes, with
 * n <= 262144 (the encoder-shaped fused path is not used); the score scan also
 * records each block's softmax mass, from which Z follows, and no key-by-key
 * select runs.
 */
#define CTOPK_FLAG_BOUND 1u

/*
 * ctopk_certify_ex -- full form of ctopk_certify: fp32 or bf16 inputs, per-head
 * scale, caller-owned workspace, optional selection mask, scores and lse.
 * bf16 inputs with d 64 or 128, n <= 512 and n_q_heads/n_kv_heads >= 64 (all
 * queries of a head against few keys, as in an encoder) run on a fused path
 * whose QK^T and head-only output use MFMA; it needs no workspace.  Other rows
 * of at most 1024 keys run on one fused kernel per call (scores, select and
 * head-only output by one workgroup per query row; no workspace either).
 * Calls that ask for out_err, out_dense or out_var take the general path.  Results
 * follow the same definitions on every path.
 */
CTOPK_API int ctopk_certify_ex(const ctopk_args* a, ctopk_stream_t stream);

/*
 * Execution plans of ctopk_certify_ex, named by the kernels each launches (in
 * launch order):
 *   CTOPK_PLAN_ENCODER: one fused kernel (MFMA scores, select, MFMA head-only
 *     output);
 *   CTOPK_PLAN_DECODE: score scan; level-0 histogram (only for rows of more
 *     than 32768 keys); select; value stream over the head; combine;
 *   CTOPK_PLAN_DECODE_OVERLAP: score scan; one launch in which the select runs
 *     beside the value stream: each stream workgroup guesses every head's cut
 *     from a sample of the scores, sums w v over the keys above its guess while
 *     the select runs, lists the keys the cut may still move (from the
 *     level-0 bin of the cut, which the select publishes first), then waits
 *     for the select's exact cut and head mass, corrects its sums by the
 *     listed keys the cut decides against the guess, and adds its chunk's
 *     share of out with device-scope float atomics.  On this plan out is
 *     therefore reproducible run to run only to fp32 rounding of those
 *     per-chunk terms.  On every plan k_eps and sel_mask repeat run to run
 *     except where a prefix mass lies within fp64 rounding of eps * Z (the
 *     select's fp64 histograms are summed by LDS atomics in varying order),
 *     and tau to fp64 rounding.  Taken for decode
 *     rows of 16385..32768 keys when at least half of the compute units (128)
 *     remain beside one workgroup per query row and the stream's chunks hold
 *     at most 2048 keys, and never for calls that ask for out_err,
 *     out_dense or out_var;
 *   CTOPK_PLAN_DECODE_BOUND (calls with CTOPK_FLAG_BOUND): score scan with
 *     per-block masses; the blockwise bound (one workgroup per row, in place
 *     of the select); value stream over the kept keys; combine;
 *   CTOPK_PLAN_DECODE_FUSED: rows of at most 1024 keys that the encoder path
 *     does not take, without out_err, out_dense or out_var: one kernel, one
 *     workgroup per query row, one key per thread: the scores (the same arithmetic as
 *     the score scan, so the same values), the select as a mass-weighted
 *     radix descent over 8-bit digits of the 64-bit key order, and the
 *     head-only output from the head keys' value rows.
 */
typedef enum {
  CTOPK_PLAN_ENCODER = 1,
  CTOPK_PLAN_DECODE = 2,
  CTOPK_PLAN_DECODE_OVERLAP = 3,
  CTOPK_PLAN_DECODE_BOUND = 4,
  CTOPK_PLAN_DECODE_FUSED = 5
} ctopk_plan_id;

/*
 * ctopk_plan -- the plan ctopk_certify_ex takes for these arguments: a
 * ctopk_plan_id, or (negative) the status ctopk_validate returns for them.
 * Host only, like ctopk_validate: no HIP call, no device memory touched.
 */
CTOPK_API int ctopk_plan(const ctopk_args* a);

/* Device scratch bytes ctopk_certify_ex needs for these sizes (0 on bad sizes);
 * enough for every call with these sizes, whichever path it takes. */
CTOPK_API size_t ctopk_workspace_bytes(int64_t n, int32_t d, int32_t n_q_heads, int32_t n_kv_heads,
                             int32_t dtype);

/*
 * ctopk_certify_logits -- selection and head-only output on given logits.
 *
 * logits [rows, n] float32 are the scores themselves (no scale is applied).
 * V [n_v, n, dv] (v_dtype) holds the value rows; logits row r reads V head
 * r / (rows / n_v), so n_v must divide rows.  dv must be 64 or 128.
 * Outputs as for ctopk_certify_ex: out [rows, dv] float32, k_eps [rows],
 * tau [rows] float64, optional sel_mask [rows, ceil(n/32)] and lse [rows].
 * workspace may be NULL (cached per-device workspace) or caller memory of at
 * least ctopk_logits_workspace_bytes(...) bytes.
 */
CTOPK_API int ctopk_certify_logits(const float* logits, const void* V, int32_t v_dtype, int64_t n,
                         int32_t dv, int32_t rows, int32_t n_v, double eps, void* workspace,
                         size_t workspace_bytes, ctopk_stream_t stream, float* out,
                         int32_t* k_eps, double* tau, uint32_t* sel_mask, double* lse);

/* Device scratch bytes ctopk_certify_logits needs (0 on bad sizes). */
CTOPK_API size_t ctopk_logits_workspace_bytes(int64_t n, int32_t dv, int32_t rows, int32_t n_v);

/*
 * ctopk_validate -- the host-side argument checks of ctopk_certify_ex, alone.
 * Makes no HIP call and touches no device memory (pointers are only tested for
 * NULL and alignment), so it runs without a GPU.  Returns CTOPK_OK or the
 * status ctopk_certify_ex would return for these arguments.
 */
CTOPK_API int ctopk_validate(const ctopk_args* a);

/*
 * 4-bit key copy and exact candidate generation.  The Abstract of
 * "Certified Sparse Attention via Perturbed Retrieval" (arXiv 2610.24991)
 * describes one pass over all keys in a 4-bit form, with a deterministic
 * bound on each score's error and one pass per grouped-query group, that
 * yields the exact candidate set; it gives no formula, so the copy and the
 * bound below are this library's reading.
 *
 * ctopk_quantize_k4 -- builds the copy of K [n_kv_heads, n, d] (dtype bf16 or
 * fp32, d 64 or 128, 16-byte aligned): per key a = amax / 7 (fp32, rounded to
 * nearest), codes c_j = clamp(rint(k_j / a), -7, 7) computed in fp32, packed
 * as two's-complement nibbles with element 2j in the low half of byte j
 * (K4 [n_kv_heads, n, d/2], 4-byte aligned), kscale [n_kv_heads, n] = a, and
 * kres [n_kv_heads, n] >= ||k - a c||_2 (rounded up).  A zero key gets a = 0
 * and codes 0.  Enqueued on `stream`; the caller owns every buffer and may
 * keep the copy for any later ctopk_candidates_k4 call on the same K.
 * n_kv_heads * n must be at most 2^34.  Returns CTOPK_ERR_NULL / _SHAPE /
 * _UNSUPPORTED / _ALIGN on bad arguments.
 */
CTOPK_API int ctopk_quantize_k4(const void* K, int32_t dtype, int64_t n, int32_t d,
                                int32_t n_kv_heads, uint8_t* K4, float* kscale, float* kres,
                                ctopk_stream_t stream);

/*
 * ctopk_candidates_k4 -- for per-head thresholds T_h, the exact candidate set
 * { i : s_hi >= T_h }, with s_hi = scale_h * <q_h, k_i> in the library's fp32
 * arithmetic (the scores ctopk_certify_ex returns): the 4-bit scan bounds every
 * score within R = |scale_h| ||q_h||_2 kres_i (plus the rounding of the fp32
 * dot products) of scale_h * kscale_i * <q_h, codes_i>, settles every key whose
 * interval lies wholly on one side of T_h, and reads the full-width row only
 * of keys whose interval straddles T_h for some head of its group.
 *
 * Inputs: q [n_q_heads, d] and K (as for ctopk_certify_ex, same dtype), the
 * copy from ctopk_quantize_k4, head_scale [n_q_heads] fp32 (NULL: 1/sqrt(d)),
 * threshold [n_q_heads] fp32.  Outputs: sel_mask [n_q_heads, ceil(n/32)] bit
 * words (bit i%32 of word i/32: key i is a candidate), count [n_q_heads] int32
 * (candidates per head), and optionally rescored [n_kv_heads] int32 (full-width
 * rows read per KV head, counted once per block of up to 8 query heads) and
 * bounds [n_q_heads, n] float2 (each score interval (lo, hi)).  workspace:
 * NULL (the cached per-device buffer ctopk_certify uses, with the same caveat:
 * calls on different streams of one device race) or 256-byte aligned with at
 * least ctopk_k4_workspace_bytes(...) bytes.
 */
typedef struct {
  const void* q;
  const void* K;
  int32_t dtype;
  int64_t n;
  int32_t d;
  int32_t n_q_heads;
  int32_t n_kv_heads;
  const float* head_scale;
  const uint8_t* K4;
  const float* kscale;
  const float* kres;
  const float* threshold;
  void* workspace;
  size_t workspace_bytes;
  uint32_t* sel_mask;
  int32_t* count;
  int32_t* rescored;
  float* bounds;
} ctopk_k4_args;

CTOPK_API int ctopk_candidates_k4(const ctopk_k4_args* a, ctopk_stream_t stream);

/* Host-side checks of ctopk_candidates_k4 alone (no HIP call). */
CTOPK_API int ctopk_validate_k4(const ctopk_k4_args* a);

/* Device scratch bytes ctopk_candidates_k4 needs (0 on bad sizes). */
CTOPK_API size_t ctopk_k4_workspace_bytes(int64_t n, int32_t n_q_heads, int32_t n_kv_heads);

/*
 * ctopk_record_kernel_events -- instrumentation for benchmarks and profilers.
 *
 * Arms the calling thread so that its NEXT ctopk_certify, ctopk_certify_ex,
 * ctopk_certify_noalloc, ctopk_certify_logits or ctopk_candidates_k4 call
 * attaches the event pair (events[2i],
 * events[2i+1]) -- hipEvent_t handles created by the caller -- to the i-th
 * kernel it launches: the events take that kernel's start and end times on
 * the call's stream (hipExtLaunchKernel), so hipEventElapsedTime on a pair is
 * the kernel's own duration.  Kernels in launch order are those of the call's
 * plan (ctopk_plan); the decode plans take the score scan's pair, then the
 * level-0 histogram's (when the plan launches none, its pair is recorded back
 * to back on the stream and measures only the stream's own gap between the
 * two records, not a kernel), then one pair per remaining kernel (select,
 * value stream and combine in the decode and bound plans; the one launch of
 * select and stream in the overlapped plan).  Logits
 * path: select, value stream, output combine.  Candidates: 4-bit scan, then
 * rescoring with the counts.  Kernels past count/2 pairs run
 * without events; pairs left over are
 * dropped when the call returns.  count must be even and at most 16 (0
 * disarms); returns CTOPK_ERR_SHAPE otherwise, CTOPK_ERR_NULL for a NULL
 * array or handle.
 */
CTOPK_API int ctopk_record_kernel_events(void* const* events, int32_t count);

/* Text of the last error on the calling thread ("" after success). */
CTOPK_API const char* ctopk_last_error_string(void);

/* Library version string, e.g. "libctopk 0.1 gfx950". */
CTOPK_API const char* ctopk_version(void);

#ifdef __cplusplus
}
#endif

#endif /* CTOPK_H */
