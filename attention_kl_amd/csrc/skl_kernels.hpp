// Kernel argument blocks and launchers of the attention-KL kernels (host + device).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace skl {

struct FwdArgs {
  const void* qt;
  const void* kt;
  const void* qs;
  const void* ks;
  float* kl;     // KL forward: KL_i.  JS pass: JS_i
  float* lse_t;  // KL forward: written.  JS pass: read
  float* lse_s;
  float* js_t;   // JS pass: KL(P_t || M)_i
  int64_t sqt[3], skt[3], sqs[3], sks[3];  // (b, h, n) element strides; K strides per key head
  int32_t B, H, Nq, Nk;
  int32_t gt, gs;   // query heads per key head (teacher, student): query head h reads key head h / g
  // Packed variable-length batch (cu_q non-NULL): batch entry b is the segment of query rows
  // cu_q[b] .. cu_q[b+1]-1 and key rows cu_k[b] .. cu_k[b+1]-1 of one packed axis of Nq / Nk rows;
  // mq, mk bound the segment lengths (the grid).  Dense batch: cu_q = cu_k = NULL, mq = Nq, mk = Nk.
  const int32_t* cu_q;
  const int32_t* cu_k;
  int32_t mq, mk;
  float c_t, c_s;   // scale * log2(e): logits enter exp2 in these units
  float ratio;      // scale_s / scale_t
  float scale_t;
  // KL forward with equal scales (bf16): the logit difference may come from a second MFMA chain
  // (skl_fwd_impl.hpp, ref_update_eq).  The Jensen-Shannon forward's first pass leaves it off, so that
  // identical rows keep bitwise-equal statistics there.
  int32_t eq_ok;
  // Small grids (set by the launcher): the two workgroups that share a CU pair a long query block with
  // a short one (see fwd_kernel); otherwise an XCD's share goes out head by head.
  int32_t fold;
  // Small causal grids given a workspace (set by the launcher): the key tiles of query blocks qsplit ..
  // nqb-1 are split in two halves, each run by a workgroup of its own that stores its row states (five
  // floats a row) in part; fwd_merge_kernel then merges the two halves in a fixed order and closes
  // those rows.  part = NULL: no split.  cpx: compute units per XCD (the workgroup order, see fwd_kernel).
  float* part;
  int32_t qsplit;
  int32_t cpx;
};

struct BwdArgs {
  const void* qt;
  const void* kt;
  const void* qs;
  const void* ks;
  const float* lse_t;
  const float* lse_s;
  const float* kl;  // KL: read only for teacher gradients.  JS: js_t, the teacher half KL(P_t || M)
  const float* js;  // JS: JS_i
  const float* g;
  float* dq;  // query-owner kernel output [B,H,Nq,d_side]
  float* dk;  // key-owner kernel output   [B,Hk_side,Nk,d_side]
  int64_t sqt[3], skt[3], sqs[3], sks[3];
  int32_t B, H, Nq, Nk;
  int32_t gt, gs;  // query heads per key head (teacher, student)
  const int32_t* cu_q;  // packed variable-length batch, as in FwdArgs
  const int32_t* cu_k;
  int32_t mq, mk;
  // Grouped key heads, key owner: the passes over a group's query heads may be split over nsplit
  // workgroups, each writing its partial dK to part (split) of ws (ws_part floats apart); the parts
  // are then summed in a fixed order.  nsplit is set by the launcher (split_count).
  float* ws;
  int64_t ws_floats;
  int64_t ws_part;
  int32_t nsplit;
  // Small grids (set by the launcher): inside each XCD's share of whole heads, workgroups go out in order
  // of stream length across those heads instead of head by head (see bwd_kernel).
  int32_t len_major;
  // Causal dense problems whose two kernels run side by side (set by the launcher): each workgroup
  // takes a long owned block and then a short one (see bwd_kernel), half the workgroups of one kernel.
  int32_t pair;
  float c_t, c_s;            // scale * log2(e)
  float scale_t, scale_s;
};
// Owned rows per backward workgroup: 8 waves of 32 (bf16) or 4 (fp32).
constexpr int kBwdRowsBf16 = 256, kBwdRowsF32 = 128;

// Rows of batch entry b.  Dense: all Nq query and Nk key rows, at batch index b of the strides.
// Packed: the segment's rows, which start at row q0 / k0 of the packed axis (batch index 0).  The
// row statistics and gradients of entry b start at ((bs * H + h) * Nq + q0) (keys: with Nk, k0).
struct Segment {
  int q0, k0, nq, nk, bs;
};
// Packed offsets are clamped into the packed axis (start in [0, N], end in [start, N]), so offsets
// that break the rules (decreasing, negative, past N) give meaningless rows for that segment but
// never an access outside the caller's buffers.
template <class A>
__device__ __forceinline__ Segment segment_of(const A& a, int b) {
  if (a.cu_q != nullptr) {
    const int q0 = min(max(__builtin_amdgcn_readfirstlane(a.cu_q[b]), 0), a.Nq);
    const int q1 = min(max(__builtin_amdgcn_readfirstlane(a.cu_q[b + 1]), q0), a.Nq);
    const int k0 = min(max(__builtin_amdgcn_readfirstlane(a.cu_k[b]), 0), a.Nk);
    const int k1 = min(max(__builtin_amdgcn_readfirstlane(a.cu_k[b + 1]), k0), a.Nk);
    return Segment{q0, k0, q1 - q0, k1 - k0, 0};
  }
  return Segment{0, 0, a.Nq, a.Nk, b};
}

// Grouped key heads, key owner, in order of preference by the caller's workspace:
//   ws holds an ungrouped dK (B H Nk d floats): the ungrouped kernel runs over every query head,
//     writing each head's contribution to its own slice, and the slices of a group are summed;
//   ws holds S >= 2 partial dK: each group's passes are split over S workgroups, parts summed;
//   no workspace: one workgroup makes all passes of its group.
// Split of a grouped key-owner launch: enough workgroups to fill the chip (about 1024) where the
// grid of owned key blocks is smaller, at most one split per query head of a group, and as many as
// the workspace holds.  `part` = floats of one partial dK of that side (the dK output's size).
constexpr int64_t kSplitTargetBlocks = 1024;
inline int64_t split_wanted(int64_t group, int64_t blocks) {
  if (group <= 1 || blocks <= 0) return 1;
  const int64_t want = (kSplitTargetBlocks + blocks - 1) / blocks;
  return want < group ? want : group;
}
inline int split_count(int64_t group, int64_t blocks, int64_t part, const float* ws, int64_t ws_floats) {
  int64_t n = split_wanted(group, blocks);
  if (ws == nullptr || part <= 0) return 1;
  if (n * part > ws_floats) n = ws_floats / part;
  return n < 2 ? 1 : (int)n;
}

// Scratch of the allocation-free backward (skl_scratch.hip): kScratchFloats floats per GPU, resolved
// for the current device by scratch_address (hipGetSymbolAddress on the first call per device).
constexpr int64_t kScratchFloats = (int64_t)16 << 20;  // 64 MiB
hipError_t scratch_address(float** out);

// dtype: 0 fp32, 1 bf16.  d_t, d_s in {64, 128}.  Return hipErrorInvalidValue for
// combinations that are not built (the C ABI rejects them before calling).
hipError_t launch_fwd(const FwdArgs& a, int dtype, int d_t, int d_s, bool causal, hipStream_t s);
hipError_t launch_bwd_dq(const BwdArgs& a, int dtype, int d_t, int d_s, bool causal, bool teacher, hipStream_t s);
hipError_t launch_bwd_dk(const BwdArgs& a, int dtype, int d_t, int d_s, bool causal, bool teacher, hipStream_t s);
// Jensen-Shannon: the forward's second pass (kl receives JS, js_t the teacher half; lse_t, lse_s are
// read) and the backward kernels of sum_i g_i JS_i (kl = js_t, js = JS).
hipError_t launch_js_fwd(const FwdArgs& a, int dtype, int d_t, int d_s, bool causal, hipStream_t s);
// dst[i] = parts[i] + parts[n + i] + ... (nsplit parts, in that order); n a multiple of 4.
hipError_t launch_sum_parts(float* dst, const float* parts, int nsplit, int64_t n, hipStream_t s);
// dst row r = src rows r G .. r G + G - 1 summed in that order (rows of `inner` floats, a multiple of 4).
hipError_t launch_group_sum(float* dst, const float* src, int64_t rows, int groups, int64_t inner, hipStream_t s);
hipError_t launch_js_bwd_dq(const BwdArgs& a, int dtype, int d_t, int d_s, bool causal, bool teacher, hipStream_t s);
hipError_t launch_js_bwd_dk(const BwdArgs& a, int dtype, int d_t, int d_s, bool causal, bool teacher, hipStream_t s);

}  // namespace skl
