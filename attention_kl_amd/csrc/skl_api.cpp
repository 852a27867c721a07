// C ABI of the attention-KL library: argument checks, kernel selection, launch.
// Declarations and the contract of every entry point are in include/streamkl.h.
#include "streamkl.h"

#include <hip/hip_runtime.h>

#include <algorithm>
#include <cmath>
#include <cstdint>
#include <type_traits>

#include "skl_kernels.hpp"

namespace {

constexpr int64_t kMaxDim = 0x7fffffff;

int elt_size(int32_t dtype) { return dtype == STREAMKL_BF16 ? 2 : (dtype == STREAMKL_FP32 ? 4 : 0); }

bool aligned(const void* p, uintptr_t a) { return (reinterpret_cast<uintptr_t>(p) % a) == 0; }

// Shape, dtype and scale checks common to all entry points.  Sets *empty when there is
// nothing to compute (B, H or Nq is zero).
int check_problem(const streamkl_problem_t* p, bool* empty) {
  if (!p) return STREAMKL_ERR_INVALID;
  if (p->B < 0 || p->H < 0 || p->Nq < 0 || p->Nk < 0) return STREAMKL_ERR_INVALID;
  if (p->causal != 0 && p->causal != 1) return STREAMKL_ERR_INVALID;
  if (!(std::isfinite(p->scale_t) && p->scale_t > 0.f && std::isfinite(p->scale_s) && p->scale_s > 0.f))
    return STREAMKL_ERR_INVALID;
  if (elt_size(p->dtype) == 0) return STREAMKL_ERR_UNSUPPORTED;
  if ((p->d_t != 64 && p->d_t != 128) || (p->d_s != 64 && p->d_s != 128)) return STREAMKL_ERR_UNSUPPORTED;
  // packed variable-length batch: the segment bounds live in device memory; what the host can check
  // is the pair of pointers and that the longest segment fits the packed axes
  const bool packed = p->cu_seqlens_q != nullptr || p->cu_seqlens_k != nullptr;
  if (packed) {
    if (!p->cu_seqlens_q || !p->cu_seqlens_k) return STREAMKL_ERR_INVALID;
    if (p->max_seqlen_q < 0 || p->max_seqlen_k < 0 || p->max_seqlen_q > p->Nq || p->max_seqlen_k > p->Nk)
      return STREAMKL_ERR_INVALID;
    if (!aligned(p->cu_seqlens_q, 4) || !aligned(p->cu_seqlens_k, 4)) return STREAMKL_ERR_UNSUPPORTED;
  }
  if (p->workspace != nullptr) {
    if (p->workspace_floats < 0) return STREAMKL_ERR_INVALID;
    if (!aligned(p->workspace, 16)) return STREAMKL_ERR_UNSUPPORTED;
  }
  *empty = (p->B == 0 || p->H == 0 || p->Nq == 0 || (packed && p->max_seqlen_q == 0));
  if (*empty) return STREAMKL_OK;
  if (p->Nk == 0) return STREAMKL_ERR_INVALID;  // softmax over no keys
  if (!packed && p->causal && p->Nq > p->Nk) return STREAMKL_ERR_INVALID;
  if (p->Nq > kMaxDim || p->Nk > kMaxDim || p->B > kMaxDim || p->H > kMaxDim || p->B * p->H > kMaxDim)
    return STREAMKL_ERR_UNSUPPORTED;
  for (const int64_t hk : {p->Hk_t, p->Hk_s})  // key heads per side: 0 (= H) or a divisor of H
    if (hk < 0 || hk > p->H || (hk > 0 && p->H % hk != 0)) return STREAMKL_ERR_INVALID;
  const int64_t* strides[4] = {p->stride_qt, p->stride_kt, p->stride_qs, p->stride_ks};
  const int64_t rows[4] = {p->Nq, p->Nk, p->Nq, p->Nk};
  const int es = elt_size(p->dtype);
  for (int t = 0; t < 4; ++t) {
    const int64_t* s = strides[t];
    for (int i = 0; i < 3; ++i) {
      if (s[i] < 0) return STREAMKL_ERR_INVALID;
      if ((s[i] * es) % 16 != 0) return STREAMKL_ERR_UNSUPPORTED;
    }
    // tiles are read through 32-bit buffer offsets within one (b, h) slice
    if ((rows[t] + 512) * s[2] * es > kMaxDim) return STREAMKL_ERR_UNSUPPORTED;
  }
  return STREAMKL_OK;
}

int check_inputs(const void* qt, const void* kt, const void* qs, const void* ks) {
  if (!qt || !kt || !qs || !ks) return STREAMKL_ERR_INVALID;
  if (!aligned(qt, 16) || !aligned(kt, 16) || !aligned(qs, 16) || !aligned(ks, 16)) return STREAMKL_ERR_UNSUPPORTED;
  return STREAMKL_OK;
}

int check_f32(const float* x) {
  if (!x) return STREAMKL_ERR_INVALID;
  if (!aligned(x, 4)) return STREAMKL_ERR_UNSUPPORTED;
  return STREAMKL_OK;
}

template <typename A>
void fill_common(A& a, const streamkl_problem_t* p, const void* qt, const void* kt, const void* qs, const void* ks) {
  a.qt = qt;
  a.kt = kt;
  a.qs = qs;
  a.ks = ks;
  for (int i = 0; i < 3; ++i) {
    a.sqt[i] = p->stride_qt[i];
    a.skt[i] = p->stride_kt[i];
    a.sqs[i] = p->stride_qs[i];
    a.sks[i] = p->stride_ks[i];
  }
  a.B = (int32_t)p->B;
  a.H = (int32_t)p->H;
  a.gt = (int32_t)(p->Hk_t > 0 ? p->H / p->Hk_t : 1);
  a.gs = (int32_t)(p->Hk_s > 0 ? p->H / p->Hk_s : 1);
  a.Nq = (int32_t)p->Nq;
  a.Nk = (int32_t)p->Nk;
  const bool packed = p->cu_seqlens_q != nullptr;
  a.cu_q = p->cu_seqlens_q;
  a.cu_k = p->cu_seqlens_k;
  a.mq = (int32_t)(packed ? p->max_seqlen_q : p->Nq);
  a.mk = (int32_t)(packed ? p->max_seqlen_k : p->Nk);
  a.c_t = p->scale_t * 1.4426950408889634f;
  a.c_s = p->scale_s * 1.4426950408889634f;
  if constexpr (std::is_same<A, skl::BwdArgs>::value) {
    a.ws = p->workspace;
    a.ws_floats = p->workspace != nullptr ? p->workspace_floats : 0;
  }
}

int to_status(hipError_t e) { return e == hipSuccess ? STREAMKL_OK : STREAMKL_ERR_LAUNCH; }

// Shared checks of the backward entry points.
int check_bwd(const streamkl_problem_t* p, const void* qt, const void* kt, const void* qs, const void* ks,
              const float* lse_t, const float* lse_s, const float* g, bool* empty) {
  int st = check_problem(p, empty);
  if (st != STREAMKL_OK || *empty) return st;
  if ((st = check_inputs(qt, kt, qs, ks)) != STREAMKL_OK) return st;
  if ((st = check_f32(lse_t)) != STREAMKL_OK) return st;
  if ((st = check_f32(lse_s)) != STREAMKL_OK) return st;
  return check_f32(g);
}

skl::BwdArgs bwd_args(const streamkl_problem_t* p, const void* qt, const void* kt, const void* qs, const void* ks,
                      const float* lse_t, const float* lse_s, const float* kl, const float* g) {
  skl::BwdArgs a{};
  fill_common(a, p, qt, kt, qs, ks);
  a.lse_t = lse_t;
  a.lse_s = lse_s;
  a.kl = kl;
  a.g = g;
  a.scale_t = p->scale_t;
  a.scale_s = p->scale_s;
  return a;
}

}  // namespace

extern "C" {

int streamkl_fwd(const streamkl_problem_t* p, const void* q_t, const void* k_t, const void* q_s, const void* k_s,
                 float* kl, float* lse_t, float* lse_s, void* hip_stream) {
  bool empty = false;
  int st = check_problem(p, &empty);
  if (st != STREAMKL_OK || empty) return st;
  if ((st = check_inputs(q_t, k_t, q_s, k_s)) != STREAMKL_OK) return st;
  if ((st = check_f32(kl)) != STREAMKL_OK || (st = check_f32(lse_t)) != STREAMKL_OK ||
      (st = check_f32(lse_s)) != STREAMKL_OK)
    return st;
  skl::FwdArgs a{};
  fill_common(a, p, q_t, k_t, q_s, k_s);
  a.kl = kl;
  a.lse_t = lse_t;
  a.lse_s = lse_s;
  a.ratio = p->scale_s / p->scale_t;
  a.scale_t = p->scale_t;
  return to_status(skl::launch_fwd(a, p->dtype, p->d_t, p->d_s, p->causal != 0, (hipStream_t)hip_stream));
}

int streamkl_bwd_dq(const streamkl_problem_t* p, const void* q_t, const void* k_t, const void* q_s, const void* k_s,
                    const float* lse_t, const float* lse_s, const float* g, float* dq_s, void* hip_stream) {
  bool empty = false;
  int st = check_bwd(p, q_t, k_t, q_s, k_s, lse_t, lse_s, g, &empty);
  if (st != STREAMKL_OK || empty) return st;
  if ((st = check_f32(dq_s)) != STREAMKL_OK) return st;
  skl::BwdArgs a = bwd_args(p, q_t, k_t, q_s, k_s, lse_t, lse_s, nullptr, g);
  a.dq = dq_s;
  return to_status(skl::launch_bwd_dq(a, p->dtype, p->d_t, p->d_s, p->causal != 0, false, (hipStream_t)hip_stream));
}

int streamkl_bwd_dk(const streamkl_problem_t* p, const void* q_t, const void* k_t, const void* q_s, const void* k_s,
                    const float* lse_t, const float* lse_s, const float* g, float* dk_s, void* hip_stream) {
  bool empty = false;
  int st = check_bwd(p, q_t, k_t, q_s, k_s, lse_t, lse_s, g, &empty);
  if (st != STREAMKL_OK || empty) return st;
  if ((st = check_f32(dk_s)) != STREAMKL_OK) return st;
  skl::BwdArgs a = bwd_args(p, q_t, k_t, q_s, k_s, lse_t, lse_s, nullptr, g);
  a.dk = dk_s;
  return to_status(skl::launch_bwd_dk(a, p->dtype, p->d_t, p->d_s, p->causal != 0, false, (hipStream_t)hip_stream));
}

int streamkl_bwd(const streamkl_problem_t* p, const void* q_t, const void* k_t, const void* q_s, const void* k_s,
                 const float* lse_t, const float* lse_s, const float* kl, const float* g, float* dq_s, float* dk_s,
                 float* dq_t, float* dk_t, void* hip_stream) {
  bool empty = false;
  int st = check_bwd(p, q_t, k_t, q_s, k_s, lse_t, lse_s, g, &empty);
  if (st != STREAMKL_OK) return st;
  if ((dq_t == nullptr) != (dk_t == nullptr) || (dq_s == nullptr) != (dk_s == nullptr)) return STREAMKL_ERR_INVALID;
  if (empty) return STREAMKL_OK;
  const bool teacher = dq_t != nullptr, student = dq_s != nullptr;
  if (!teacher && !student) return STREAMKL_ERR_INVALID;  // no gradient asked for
  if (student && ((st = check_f32(dq_s)) != STREAMKL_OK || (st = check_f32(dk_s)) != STREAMKL_OK)) return st;
  if (teacher) {
    if ((st = check_f32(dq_t)) != STREAMKL_OK || (st = check_f32(dk_t)) != STREAMKL_OK ||
        (st = check_f32(kl)) != STREAMKL_OK)
      return st;
  }
  const hipStream_t s = (hipStream_t)hip_stream;
  const bool causal = p->causal != 0;
  skl::BwdArgs a = bwd_args(p, q_t, k_t, q_s, k_s, lse_t, lse_s, kl, g);
  if (student) {
    a.dq = dq_s;
    a.dk = dk_s;
    if ((st = to_status(skl::launch_bwd_dk(a, p->dtype, p->d_t, p->d_s, causal, false, s))) != STREAMKL_OK) return st;
    if ((st = to_status(skl::launch_bwd_dq(a, p->dtype, p->d_t, p->d_s, causal, false, s))) != STREAMKL_OK) return st;
  }
  if (teacher) {
    a.dq = dq_t;
    a.dk = dk_t;
    if ((st = to_status(skl::launch_bwd_dk(a, p->dtype, p->d_t, p->d_s, causal, true, s))) != STREAMKL_OK) return st;
    if ((st = to_status(skl::launch_bwd_dq(a, p->dtype, p->d_t, p->d_s, causal, true, s))) != STREAMKL_OK) return st;
  }
  return STREAMKL_OK;
}

int streamkl_js_fwd(const streamkl_problem_t* p, const void* q_t, const void* k_t, const void* q_s, const void* k_s,
                    float* js, float* lse_t, float* lse_s, float* js_t, void* hip_stream) {
  bool empty = false;
  int st = check_problem(p, &empty);
  if (st != STREAMKL_OK || empty) return st;
  if ((st = check_inputs(q_t, k_t, q_s, k_s)) != STREAMKL_OK) return st;
  if ((st = check_f32(js)) != STREAMKL_OK || (st = check_f32(lse_t)) != STREAMKL_OK ||
      (st = check_f32(lse_s)) != STREAMKL_OK || (st = check_f32(js_t)) != STREAMKL_OK)
    return st;
  skl::FwdArgs a{};
  fill_common(a, p, q_t, k_t, q_s, k_s);
  a.kl = js;  // the KL forward's per-row KL lands here first, then the JS pass overwrites it
  a.lse_t = lse_t;
  a.lse_s = lse_s;
  a.js_t = js_t;
  a.ratio = p->scale_s / p->scale_t;
  a.scale_t = p->scale_t;
  const hipStream_t s = (hipStream_t)hip_stream;
  if ((st = to_status(skl::launch_fwd(a, p->dtype, p->d_t, p->d_s, p->causal != 0, s))) != STREAMKL_OK) return st;
  return to_status(skl::launch_js_fwd(a, p->dtype, p->d_t, p->d_s, p->causal != 0, s));
}

int streamkl_js_bwd(const streamkl_problem_t* p, const void* q_t, const void* k_t, const void* q_s, const void* k_s,
                    const float* lse_t, const float* lse_s, const float* js, const float* js_t, const float* g,
                    float* dq_s, float* dk_s, float* dq_t, float* dk_t, void* hip_stream) {
  bool empty = false;
  int st = check_bwd(p, q_t, k_t, q_s, k_s, lse_t, lse_s, g, &empty);
  if (st != STREAMKL_OK) return st;
  if ((dq_t == nullptr) != (dk_t == nullptr) || (dq_s == nullptr) != (dk_s == nullptr)) return STREAMKL_ERR_INVALID;
  if (empty) return STREAMKL_OK;
  const bool teacher = dq_t != nullptr, student = dq_s != nullptr;
  if (!teacher && !student) return STREAMKL_ERR_INVALID;  // no gradient asked for
  if ((st = check_f32(js)) != STREAMKL_OK || (st = check_f32(js_t)) != STREAMKL_OK) return st;
  if (student && ((st = check_f32(dq_s)) != STREAMKL_OK || (st = check_f32(dk_s)) != STREAMKL_OK)) return st;
  if (teacher && ((st = check_f32(dq_t)) != STREAMKL_OK || (st = check_f32(dk_t)) != STREAMKL_OK)) return st;
  const hipStream_t s = (hipStream_t)hip_stream;
  const bool causal = p->causal != 0;
  skl::BwdArgs a = bwd_args(p, q_t, k_t, q_s, k_s, lse_t, lse_s, js_t, g);
  a.js = js;
  if (student) {
    a.dq = dq_s;
    a.dk = dk_s;
    if ((st = to_status(skl::launch_js_bwd_dk(a, p->dtype, p->d_t, p->d_s, causal, false, s))) != STREAMKL_OK) return st;
    if ((st = to_status(skl::launch_js_bwd_dq(a, p->dtype, p->d_t, p->d_s, causal, false, s))) != STREAMKL_OK) return st;
  }
  if (teacher) {
    a.dq = dq_t;
    a.dk = dk_t;
    if ((st = to_status(skl::launch_js_bwd_dk(a, p->dtype, p->d_t, p->d_s, causal, true, s))) != STREAMKL_OK) return st;
    if ((st = to_status(skl::launch_js_bwd_dq(a, p->dtype, p->d_t, p->d_s, causal, true, s))) != STREAMKL_OK) return st;
  }
  return STREAMKL_OK;
}

const char* streamkl_status_string(int status) {
  switch (status) {
    case STREAMKL_OK:
      return "STREAMKL_OK";
    case STREAMKL_ERR_INVALID:
      return "STREAMKL_ERR_INVALID: invalid argument";
    case STREAMKL_ERR_UNSUPPORTED:
      return "STREAMKL_ERR_UNSUPPORTED: head dim, dtype or alignment not supported";
    case STREAMKL_ERR_LAUNCH:
      return "STREAMKL_ERR_LAUNCH: HIP kernel launch failed";
    default:
      return "STREAMKL: unknown status";
  }
}

int streamkl_version(void) { return STREAMKL_VERSION; }

int64_t streamkl_workspace_floats(const streamkl_problem_t* p) {
  bool empty = false;
  if (check_problem(p, &empty) != STREAMKL_OK || empty) return 0;
  // For each grouped side, the ungrouped dK (B H Nk d floats) the backward launcher can use to run
  // the ungrouped kernel over every query head; where the group-sum grid cannot hold the key heads,
  // the parts of the split the launcher would make (owned keys per workgroup: 256 bf16, 128 fp32).
  const bool packed = p->cu_seqlens_q != nullptr;
  const int64_t bw = p->dtype == STREAMKL_BF16 ? 256 : 128;
  const int64_t nob = ((packed ? p->max_seqlen_k : p->Nk) + bw - 1) / bw, nb = packed ? 1 : p->B;
  int64_t best = 0;
  const int64_t hk[2] = {p->Hk_t > 0 ? p->Hk_t : p->H, p->Hk_s > 0 ? p->Hk_s : p->H};
  const int64_t dd[2] = {p->d_t, p->d_s};
  for (int side = 0; side < 2; ++side) {
    const int64_t g = p->H / hk[side];
    if (g <= 1) continue;
    const int64_t n = nb * hk[side] <= 65535 ? g : skl::split_wanted(g, nob * p->B * hk[side]);
    if (n > 1) best = std::max(best, n * nb * hk[side] * p->Nk * dd[side]);
  }
  return best;
}

}  // extern "C"
