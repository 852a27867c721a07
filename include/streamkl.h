/*
 * streamkl.h — C ABI of the fused attention-KL primitive for AMD MI355X (gfx950).
 *
 * What is computed.  The StreamKL abstract ("StreamKL: Fast and Memory-Efficient
 * KL Divergence for Boosting Attention Distillation", arXiv 2026; its sentences
 * are cited as S1..S8 in reading order) defines the quantity as the KL
 * divergence that attention distillation minimises between two attention
 * distributions (S1), and asks that neither N_Q x N_K distribution be formed
 * (S2, S3).  For every batch b, head h and query row i:
 *
 *   a_ij = scale_t * <q_t[i], k_t[j]>        b_ij = scale_s * <q_s[i], k_s[j]>
 *   A_i  = { j < Nk : !causal || j <= i + Nk - Nq }   (bottom-right causal alignment)
 *   P_t  = softmax_{A_i}(a_i.)               P_s  = softmax_{A_i}(b_i.)
 *   KL_i = sum_{j in A_i} P_t,ij * (log P_t,ij - log P_s,ij)     (teacher || student)
 *   LSE_t,i = log sum_{A_i} exp(a_ij)        LSE_s,i = log sum_{A_i} exp(b_ij)
 *
 * The forward is one streaming pass over key tiles (S4); the backward recomputes
 * both probability tiles from the saved log-sum-exps (S5) and returns the
 * gradients of L = sum_i g_i KL_i:
 *
 *   dS_s = g_i (P_s - P_t)                   dQ_s = scale_s dS_s K_s     dK_s = scale_s dS_s^T Q_s
 *   dS_t = g_i P_t ((a - b) - (KL_i + LSE_t,i - LSE_s,i))
 *                                            dQ_t = scale_t dS_t K_t     dK_t = scale_t dS_t^T Q_t
 *
 * Conventions shared by every entry point.
 *  - Every data pointer is a DEVICE pointer owned by the caller.  The library
 *    allocates no memory and frees nothing: the only HBM it touches beyond the
 *    inputs is the outputs the caller passes (S8: no O(Nq*Nk) buffer), plus, for
 *    grouped key heads and small causal forwards only, an optional caller workspace
 *    (see streamkl_workspace_floats) or, for streamkl_bwd_noalloc, a fixed scratch array
 *    the library holds on each GPU.  Its only other state, per device: a second HIP
 *    stream (default priority) and two events, made by the first streamkl_bwd or
 *    streamkl_js_bwd call that runs kernels side by side and kept until the process
 *    ends.
 *  - Work is enqueued on `hip_stream` (a hipStream_t; NULL = the null stream) and
 *    is asynchronous: the call returns after launch.  Kernel faults surface at the
 *    caller's next synchronisation, as for any HIP launch.
 *  - Inputs are read only.  Outputs are overwritten in full (never accumulated
 *    into), so they need no zeroing.  Outputs must not alias inputs.
 *  - Return value: STREAMKL_OK or an error code; nothing is launched when an
 *    argument check fails.  Nothing is printed and nothing is thrown.
 *  - Thread-safe (the side stream and its events are used under a lock;
 *    streamkl_bwd_noalloc's calls on one GPU share that GPU's scratch).  Results are
 *    bitwise deterministic (no atomics; fixed reduction order) and do not depend on
 *    which stream a kernel ran on.
 */
#ifndef STREAMKL_H
#define STREAMKL_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define STREAMKL_VERSION 10700 /* 1.7.0: split key halves for small causal forwards; 1.6.1: paired causal blocks on the two streams; 1.6.0: small backward problems on two streams; 1.5.0: allocation-free backward; 1.4.0: workspace for grouped keys;
                                  1.3.0: Jensen-Shannon; 1.2.0: packed batches; 1.1.0: key heads */

typedef enum {
  STREAMKL_FP32 = 0, /* inputs float32; products on fp32 MFMA                */
  STREAMKL_BF16 = 1  /* inputs bfloat16; logit products on bf16 MFMA; the backward's gradient
                        products on fp16 MFMA (dS rounded once, 2^-11 relative; the bf16 operand
                        converted exactly) or, for values outside that range, bf16 hi + lo parts
                        of dS; fp32 accumulation throughout */
} streamkl_dtype_t;

typedef enum {
  STREAMKL_OK = 0,
  STREAMKL_ERR_INVALID = 1,     /* bad argument: NULL pointer, negative size, Nk == 0 with rows to
                                   compute, causal with Nq > Nk, non-positive or non-finite scale,
                                   d stride != 1, a key-head count that does not divide H, only one
                                   pointer of a gradient pair given, or no gradient asked for; packed
                                   batch: one cu_seqlens pointer NULL, or a max_seqlen below 0 or
                                   above the packed row count                                      */
  STREAMKL_ERR_UNSUPPORTED = 2, /* valid but not built: d_t or d_s not in {64, 128}, misaligned base
                                   pointer or stride (16-byte alignment needed; 4 bytes for the
                                   cu_seqlens arrays), dtype unknown, or
                                   one (b, h) slice spanning 2 GiB or more ((N + 512) * n-stride
                                   * element size must stay below 2^31 bytes)                     */
  STREAMKL_ERR_LAUNCH = 3,      /* the HIP launch itself failed (hipGetLastError after launch)     */
  STREAMKL_ERR_SCRATCH = 4      /* streamkl_bwd_noalloc: the problem needs more scratch than the
                                   library's static array holds (STREAMKL_NOALLOC_SCRATCH_FLOATS)   */
} streamkl_status_t;

/* Problem description.  Q tensors are [B, H, Nq, d], K tensors [B, Hk, Nk, d] with
 * Hk = Hk_t or Hk_s key heads for that side, each dividing H: query head h reads
 * key head h / (H / Hk) (grouped-query attention; Hk = H is one key head per query
 * head, Hk = 1 one shared head).  The d axis is contiguous; stride_*[0..2] are the
 * element strides of the b, head and n axes (any order of axes in memory is
 * allowed as long as d is unit-stride).  All four inputs share `dtype`.  Row
 * statistics and gradients are dense and contiguous: kl, lse_t, lse_s, g are
 * float32 [B, H, Nq]; dq_s [B, H, Nq, d_s], dk_s [B, Hk_s, Nk, d_s], dq_t
 * [B, H, Nq, d_t], dk_t [B, Hk_t, Nk, d_t], all float32; a key head's gradient
 * sums over the query heads that read it.
 *
 * Packed variable-length batch (cu_seqlens_q, cu_seqlens_k non-NULL).  The inputs
 * hold Nq query rows and Nk key rows along their n axis (the b stride is unused),
 * cut into B segments: segment b is query rows cu_seqlens_q[b] .. cu_seqlens_q[b+1]-1
 * and key rows cu_seqlens_k[b] .. cu_seqlens_k[b+1]-1, and is its own problem (its
 * keys only, causal alignment within it).  Both arrays are DEVICE int32 [B + 1],
 * non-decreasing, from >= 0 up to <= Nq (resp. Nk); max_seqlen_q / max_seqlen_k must
 * be >= every segment's length (they size the grid).  The kernels clamp every offset
 * into [0, Nq] (resp. [0, Nk]) and each segment's end to at least its start, so values
 * outside these rules cannot make them touch memory outside the caller's buffers; the
 * rows of such segments get unspecified outputs (the Python binding checks the rules on
 * a read-back of both arrays and raises).  A segment with queries needs keys (and, causal, at least as many keys as
 * queries); otherwise its rows' outputs are unspecified (no other row is
 * affected).  Statistics and gradients take the layout of a one-entry batch:
 * kl, lse_t, lse_s, g float32 [H, Nq]; dq [H, Nq, d]; dk [Hk, Nk, d].              */
typedef struct {
  int64_t B, H, Nq, Nk;   /* B, H, Nq >= 0 (any zero = nothing to do, returns OK); Nk >= 1 when
                             there are rows; causal needs Nq <= Nk                              */
  int32_t d_t, d_s;       /* head dims of teacher and student: each 64 or 128                    */
  float scale_t, scale_s; /* softmax scales (finite, > 0), usually 1/sqrt(d_t), 1/sqrt(d_s)      */
  int32_t causal;         /* 0: every key; 1: key j allowed for row i iff j <= i + Nk - Nq      */
  int32_t dtype;          /* streamkl_dtype_t                                                    */
  int64_t stride_qt[3], stride_kt[3], stride_qs[3], stride_ks[3]; /* (b, h, n) strides, elements */
  int64_t Hk_t, Hk_s;     /* key heads of teacher and student: each divides H; 0 means H          */
  const int32_t* cu_seqlens_q; /* packed batch: segment row offsets, DEVICE int32 [B + 1]; NULL =  */
  const int32_t* cu_seqlens_k; /* dense batch.  Both NULL or both non-NULL.                        */
  int64_t max_seqlen_q, max_seqlen_k; /* packed batch: longest segment (ignored when dense)         */
  float* workspace;            /* optional DEVICE scratch (16-byte aligned), NULL = none: see below */
  int64_t workspace_floats;    /* its size in floats                                               */
} streamkl_problem_t;

/* Workspace (grouped key heads; small causal forwards).  Without one, a key-owner launch whose gradient side has
 * G > 1 query heads per key head makes G passes per workgroup, and when the key heads are few the
 * grid cannot fill the chip.  With a workspace the size of an ungrouped dK (B H Nk d floats), the
 * ungrouped kernel runs over every query head, each writing its contribution to its own slice, and
 * the G slices of each key head are summed in head order into dk; with a smaller workspace each
 * group's passes are split over as many workgroups as it holds partial dK, summed in a fixed order.
 * Results are bitwise repeatable for a given workspace size (not bitwise equal across sizes).
 * streamkl_fwd of a small causal problem (dense bf16 batch, Nk >= Nq, at least two query blocks of
 * 128 rows and at most twice the device's compute units in such blocks) given a workspace of at
 * least 1280 B H ceil(ceil(Nq / 128) / 2) floats splits the key tiles of the later half of each
 * head's query blocks over two workgroups and merges their row states (5 floats a row) in a fixed
 * order with a second kernel: repeatable bits, within float rounding of the unsplit forward.
 * streamkl_workspace_floats(p) is the size of the best arrangement for p, for both directions (0
 * when neither uses one).  The workspace is used in stream order: overlapping calls need their own. */
int64_t streamkl_workspace_floats(const streamkl_problem_t* p);

/* Forward (S4): KL_i, LSE_t,i, LSE_s,i for every row, float32 [B, H, Nq] each.
 * One pass over the keys; per row only five running floats are kept (a small
 * causal problem given a workspace: see the workspace note above).               */
int streamkl_fwd(const streamkl_problem_t* p,
                 const void* q_t, const void* k_t, const void* q_s, const void* k_s,
                 float* kl, float* lse_t, float* lse_s,
                 void* hip_stream);

/* Backward (S5): gradients of sum_i g_i KL_i.  Needs the forward's lse_t, lse_s
 * (and kl when teacher gradients are asked for; may be NULL otherwise) and the
 * per-row weights g.  Outputs come in pairs, each pair both NULL (not computed)
 * or both non-NULL (written): dq_s, dk_s the student gradients, dq_t, dk_t the
 * teacher gradients.  One pointer of a pair NULL, or both pairs NULL, =
 * STREAMKL_ERR_INVALID.  Launches the key-owner kernel of each pair asked for
 * (student first) on hip_stream, then the query-owner kernels.  When both grids
 * are small (each at most twice the device's compute units in workgroups, where
 * causal blocks of unequal length leave units idle) and both stream at least 1024
 * rows (the longest query and key segments) the query-owner kernels go to
 * the device's side stream instead and run beside the key-owner ones: the side
 * stream first waits for everything issued to hip_stream before the call, and
 * hip_stream then waits for the side stream's kernels (event record and wait, so
 * a HIP graph capture of hip_stream takes both); for a causal dense batch each
 * workgroup of these kernels then runs a long owned block and a short one, half
 * as many workgroups per kernel (same results bit for bit).  Calls that overlap in time share
 * the side stream in the order they reach it; a capture of hip_stream should not
 * overlap another thread's uncaptured calls on the same device.  Should recording
 * or waiting on the join event fail, the call returns STREAMKL_ERR_LAUNCH and the
 * caller must synchronise the device before using the outputs.                   */
int streamkl_bwd(const streamkl_problem_t* p,
                 const void* q_t, const void* k_t, const void* q_s, const void* k_s,
                 const float* lse_t, const float* lse_s, const float* kl, const float* g,
                 float* dq_s, float* dk_s, float* dq_t, float* dk_t,
                 void* hip_stream);

/* The two halves of streamkl_bwd for the student side, each one kernel launch,
 * for callers (and profilers) that schedule them separately: the query-owner
 * kernel writes dq_s, the key-owner kernel writes dk_s.  Same arguments and
 * rules as streamkl_bwd.                                                          */
int streamkl_bwd_dq(const streamkl_problem_t* p,
                    const void* q_t, const void* k_t, const void* q_s, const void* k_s,
                    const float* lse_t, const float* lse_s, const float* g,
                    float* dq_s, void* hip_stream);
int streamkl_bwd_dk(const streamkl_problem_t* p,
                    const void* q_t, const void* k_t, const void* q_s, const void* k_s,
                    const float* lse_t, const float* lse_s, const float* g,
                    float* dk_s, void* hip_stream);

/* Jensen-Shannon divergence of the same two rows (the pages name only KL, S1; this
 * is its symmetric, bounded relative):
 *   M = (P_t + P_s) / 2,   JS_i = KL(P_t || M)_i / 2 + KL(P_s || M)_i / 2   (natural log, 0 <= JS <= ln 2)
 * streamkl_js_fwd: writes js = JS_i, lse_t, lse_s (as streamkl_fwd) and js_t =
 * KL(P_t || M)_i, all float32 in the layout of kl.  Two launches on hip_stream: the
 * KL forward (its KL goes to js first), then a second pass over the keys.        */
int streamkl_js_fwd(const streamkl_problem_t* p,
                    const void* q_t, const void* k_t, const void* q_s, const void* k_s,
                    float* js, float* lse_t, float* lse_s, float* js_t,
                    void* hip_stream);

/* Gradients of sum_i g_i JS_i.  Needs streamkl_js_fwd's lse_t, lse_s, js and js_t;
 * the gradient pairs follow the rules of streamkl_bwd:
 *   dS_t = g_i P_t (log(P_t/M) - KL(P_t || M)_i) / 2,   dS_s = g_i P_s (log(P_s/M) - KL(P_s || M)_i) / 2,
 * then dQ, dK as for the KL backward, with the kernels on the streams streamkl_bwd
 * uses.                                                                           */
int streamkl_js_bwd(const streamkl_problem_t* p,
                    const void* q_t, const void* k_t, const void* q_s, const void* k_s,
                    const float* lse_t, const float* lse_s, const float* js, const float* js_t,
                    const float* g, float* dq_s, float* dk_s, float* dq_t, float* dk_t,
                    void* hip_stream);

/* Allocation-free backward, for callers that cannot allocate device memory (code under HIP graph
 * capture, tight serving loops, harnesses that forbid hipMalloc).  Same arguments, outputs and rules
 * as streamkl_bwd, and the same bits as streamkl_bwd given a workspace of streamkl_workspace_floats(p)
 * floats (all kernels on hip_stream: this entry point creates no side stream), except that
 * p->workspace must be NULL (else STREAMKL_ERR_INVALID): the only scratch the
 * kernels use (grouped key heads' per-query-head dK before the group sum) is instead a fixed array
 * of STREAMKL_NOALLOC_SCRATCH_FLOATS floats that the library keeps on every GPU it runs on, held until
 * the process ends.  Its device address is resolved on the first call on each device (the current
 * device; hip_stream must belong to it).  A problem whose streamkl_workspace_floats(p) exceeds the
 * array is rejected with STREAMKL_ERR_SCRATCH before anything is launched.  Nothing is allocated or
 * freed (no hipMalloc, no hipFree, no allocating library call).  Every call on one GPU shares that
 * GPU's array: calls that overlap on one GPU (on different streams, or from different threads
 * without ordering) race and give undefined results; calls in stream order are safe.  The array
 * keeps the last call's contents; no call relies on them (every element a call reads it has
 * written first).  Problems without grouped key heads use no scratch.                           */
#define STREAMKL_NOALLOC_SCRATCH_FLOATS ((int64_t)16 << 20) /* 64 MiB per GPU */
int streamkl_bwd_noalloc(const streamkl_problem_t* p,
                         const void* q_t, const void* k_t, const void* q_s, const void* k_s,
                         const float* lse_t, const float* lse_s, const float* kl, const float* g,
                         float* dq_s, float* dk_s, float* dq_t, float* dk_t,
                         void* hip_stream);

/* Human-readable name of a status code (static storage; never NULL).            */
const char* streamkl_status_string(int status);

/* STREAMKL_VERSION of the built library.                                         */
int streamkl_version(void);

#ifdef __cplusplus
}
#endif
#endif /* STREAMKL_H */
