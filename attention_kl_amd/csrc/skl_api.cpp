// C ABI of the attention-KL library: argument checks, kernel selection, launch.
// Declarations and the contract of every entry point are in include/streamkl.h.
#include "streamkl.h"

#include <hip/hip_runtime.h>

#include <algorithm>
#include <cmath>
#include <cstdint>
#include <mutex>
#include <type_traits>

#include "skl_kernels.hpp"

static_assert(skl::kScratchFloats == STREAMKL_NOALLOC_SCRATCH_FLOATS, "scratch size of the header");

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

// Per device: the compute-unit count, and a second stream with two events on which a backward call
// runs its query-owner kernels beside its key-owner kernels (made at the first call that can use
// them, kept until the process ends; default priority).
struct DeviceSide {
  int ncu = 0;
  bool ready = false;
  hipStream_t side = nullptr;
  hipEvent_t fork = nullptr, join = nullptr;
};
constexpr int kMaxDevices = 64;
std::mutex g_side_mu;
DeviceSide g_side[kMaxDevices];

// The current device's entry (caller holds g_side_mu), or null.  Failed HIP calls here are cleared
// from the runtime's last-error state, so they never surface as the error of a later launch.
DeviceSide* device_side(bool need_stream) {
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) {
    (void)hipGetLastError();
    return nullptr;
  }
  DeviceSide& d = g_side[dev];
  if (d.ncu == 0 && hipDeviceGetAttribute(&d.ncu, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess) {
    d.ncu = 0;
    (void)hipGetLastError();
  }
  if (need_stream && !d.ready) {
    d.ready = hipStreamCreateWithFlags(&d.side, hipStreamNonBlocking) == hipSuccess &&
              hipEventCreateWithFlags(&d.fork, hipEventDisableTiming) == hipSuccess &&
              hipEventCreateWithFlags(&d.join, hipEventDisableTiming) == hipSuccess;
    if (!d.ready) {  // tried again at the next call
      (void)hipGetLastError();
      if (d.join) (void)hipEventDestroy(d.join);
      if (d.fork) (void)hipEventDestroy(d.fork);
      if (d.side) (void)hipStreamDestroy(d.side);
      d.side = nullptr, d.fork = nullptr, d.join = nullptr;
      (void)hipGetLastError();
    }
  }
  return &d;
}

// Workgroups of the query-owner (own_q) or key-owner backward kernel, counted over all query heads.
int64_t bwd_blocks(const streamkl_problem_t* p, const skl::BwdArgs& a, bool own_q) {
  const int bw = p->dtype == STREAMKL_BF16 ? skl::kBwdRowsBf16 : skl::kBwdRowsF32;
  return (int64_t)(((own_q ? a.mq : a.mk) + bw - 1) / bw) * a.B * a.H;
}

// A backward grid is small when it fills the device at most twice over (one backward workgroup per
// compute unit at a time): its causal blocks then go out longest first across heads (len_major), and
// a call with both kernels runs them side by side (when both stream enough rows to pay the two
// streams' handoff, about 15 us on MI355X), so that units freed by one kernel's short blocks take
// the other's long ones.
constexpr int kSideMinRows = 1024;
bool small_grid(int64_t nblk) {
  std::lock_guard<std::mutex> lk(g_side_mu);
  const DeviceSide* d = device_side(false);
  return d != nullptr && d->ncu > 0 && nblk <= 2 * (int64_t)d->ncu;
}

// Small forward grids (at most twice the device's compute units in workgroups of 128 query rows, so two
// workgroups to a CU): the two that share a CU pair a long causal query block with a short one.
int fwd_fold(const skl::FwdArgs& a) {
  return small_grid((int64_t)((a.mq + 127) / 128) * a.B * a.H) ? 1 : 0;
}

// Compute units per XCD of the current device (0 if unknown).
int device_cpx() {
  std::lock_guard<std::mutex> lk(g_side_mu);
  const DeviceSide* d = device_side(false);
  return d != nullptr && d->ncu > 0 ? d->ncu / 8 : 0;
}

// Small causal forward grids (dense bf16, Nk >= Nq, at least two query blocks of 128 rows, at most twice
// the device's compute units in workgroups, so a third of each CU's workgroup slots idle): given a
// workspace of this many floats, the key tiles of the later half of each head's query blocks are
// split over two workgroups, whose row states (5 floats a row) a second kernel merges.  0: no split.
int64_t fwd_split_floats(const streamkl_problem_t* p) {
  if (!p->causal || p->cu_seqlens_q != nullptr || p->dtype != STREAMKL_BF16 || p->Nk < p->Nq) return 0;
  const int64_t nqb = (p->Nq + 127) / 128;
  if (nqb < 2 || !small_grid(nqb * p->B * p->H)) return 0;
  return p->B * p->H * (nqb - nqb / 2) * 2 * 5 * 128;
}

skl::BwdArgs bwd_args(const streamkl_problem_t* p, const void* qt, const void* kt, const void* qs, const void* ks,
                      const float* lse_t, const float* lse_s, const float* kl, const float* g, bool own_q) {
  skl::BwdArgs a{};
  fill_common(a, p, qt, kt, qs, ks);
  a.lse_t = lse_t;
  a.lse_s = lse_s;
  a.kl = kl;
  a.g = g;
  a.scale_t = p->scale_t;
  a.scale_s = p->scale_s;
  a.len_major = small_grid(bwd_blocks(p, a, own_q)) ? 1 : 0;
  return a;
}

// Run on_main(s), then on_side(x), where x is the device's side stream if `fork` (both after all work
// issued to s so far, and s then waits for x), else s itself.  Returns the first failure.
template <class M, class S>
int fork_join(hipStream_t s, bool fork, M&& on_main, S&& on_side) {
  if (fork) {
    std::lock_guard<std::mutex> lk(g_side_mu);  // one caller at a time records and waits on the events
    DeviceSide* d = device_side(true);
    if (d != nullptr && d->ready && hipEventRecord(d->fork, s) == hipSuccess &&
        hipStreamWaitEvent(d->side, d->fork, 0) == hipSuccess) {
      const int st1 = on_main(s);
      const int st2 = on_side(d->side);
      // s waits for the side stream whatever happened above
      const bool joined = hipEventRecord(d->join, d->side) == hipSuccess && hipStreamWaitEvent(s, d->join, 0) == hipSuccess;
      if (st1 != STREAMKL_OK) return st1;
      if (st2 != STREAMKL_OK) return st2;
      return joined ? STREAMKL_OK : STREAMKL_ERR_LAUNCH;
    }
    (void)hipGetLastError();
  }
  const int st = on_main(s);
  return st != STREAMKL_OK ? st : on_side(s);
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
  a.eq_ok = 1;
  a.fold = fwd_fold(a);
  const int64_t need = fwd_split_floats(p);
  if (need > 0 && p->workspace != nullptr && p->workspace_floats >= need) {
    a.part = p->workspace;
    a.qsplit = (int32_t)((p->Nq + 127) / 128 / 2);
    a.cpx = device_cpx();
  }
  return to_status(skl::launch_fwd(a, p->dtype, p->d_t, p->d_s, p->causal != 0, (hipStream_t)hip_stream));
}

int streamkl_bwd_dq(const streamkl_problem_t* p, const void* q_t, const void* k_t, const void* q_s, const void* k_s,
                    const float* lse_t, const float* lse_s, const float* g, float* dq_s, void* hip_stream) {
  bool empty = false;
  int st = check_bwd(p, q_t, k_t, q_s, k_s, lse_t, lse_s, g, &empty);
  if (st != STREAMKL_OK || empty) return st;
  if ((st = check_f32(dq_s)) != STREAMKL_OK) return st;
  skl::BwdArgs a = bwd_args(p, q_t, k_t, q_s, k_s, lse_t, lse_s, nullptr, g, true);
  a.dq = dq_s;
  return to_status(skl::launch_bwd_dq(a, p->dtype, p->d_t, p->d_s, p->causal != 0, false, (hipStream_t)hip_stream));
}

int streamkl_bwd_dk(const streamkl_problem_t* p, const void* q_t, const void* k_t, const void* q_s, const void* k_s,
                    const float* lse_t, const float* lse_s, const float* g, float* dk_s, void* hip_stream) {
  bool empty = false;
  int st = check_bwd(p, q_t, k_t, q_s, k_s, lse_t, lse_s, g, &empty);
  if (st != STREAMKL_OK || empty) return st;
  if ((st = check_f32(dk_s)) != STREAMKL_OK) return st;
  skl::BwdArgs a = bwd_args(p, q_t, k_t, q_s, k_s, lse_t, lse_s, nullptr, g, false);
  a.dk = dk_s;
  return to_status(skl::launch_bwd_dk(a, p->dtype, p->d_t, p->d_s, p->causal != 0, false, (hipStream_t)hip_stream));
}

}  // extern "C"

namespace {

// streamkl_bwd; side: the query-owner kernels of a small problem may run on the device's side stream
int bwd_impl(const streamkl_problem_t* p, const void* q_t, const void* k_t, const void* q_s, const void* k_s,
             const float* lse_t, const float* lse_s, const float* kl, const float* g, float* dq_s, float* dk_s,
             float* dq_t, float* dk_t, void* hip_stream, bool side) {
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
  skl::BwdArgs ak = bwd_args(p, q_t, k_t, q_s, k_s, lse_t, lse_s, kl, g, false);  // key owners
  skl::BwdArgs aq = bwd_args(p, q_t, k_t, q_s, k_s, lse_t, lse_s, kl, g, true);   // query owners
  ak.dq = aq.dq = nullptr;
  // key-owner kernels on s, query-owner kernels beside them when both grids are small and both streams long
  const bool fork = side && ak.len_major && aq.len_major && std::min(ak.mq, ak.mk) >= kSideMinRows;
  ak.pair = aq.pair = fork ? 1 : 0;  // causal blocks in long + short pairs: half of each grid, side by side
  return fork_join(
      s, fork,
      [&](hipStream_t x) {
        int r = STREAMKL_OK;
        if (student) {
          ak.dk = dk_s;
          r = to_status(skl::launch_bwd_dk(ak, p->dtype, p->d_t, p->d_s, causal, false, x));
        }
        if (r == STREAMKL_OK && teacher) {
          ak.dk = dk_t;
          r = to_status(skl::launch_bwd_dk(ak, p->dtype, p->d_t, p->d_s, causal, true, x));
        }
        return r;
      },
      [&](hipStream_t x) {
        int r = STREAMKL_OK;
        if (student) {
          aq.dq = dq_s;
          r = to_status(skl::launch_bwd_dq(aq, p->dtype, p->d_t, p->d_s, causal, false, x));
        }
        if (r == STREAMKL_OK && teacher) {
          aq.dq = dq_t;
          r = to_status(skl::launch_bwd_dq(aq, p->dtype, p->d_t, p->d_s, causal, true, x));
        }
        return r;
      });
}

}  // namespace

extern "C" {

int streamkl_bwd(const streamkl_problem_t* p, const void* q_t, const void* k_t, const void* q_s, const void* k_s,
                 const float* lse_t, const float* lse_s, const float* kl, const float* g, float* dq_s, float* dk_s,
                 float* dq_t, float* dk_t, void* hip_stream) {
  return bwd_impl(p, q_t, k_t, q_s, k_s, lse_t, lse_s, kl, g, dq_s, dk_s, dq_t, dk_t, hip_stream, true);
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
  a.fold = fwd_fold(a);
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
  skl::BwdArgs ak = bwd_args(p, q_t, k_t, q_s, k_s, lse_t, lse_s, js_t, g, false);  // key owners
  skl::BwdArgs aq = bwd_args(p, q_t, k_t, q_s, k_s, lse_t, lse_s, js_t, g, true);   // query owners
  ak.js = aq.js = js;
  ak.dq = aq.dq = nullptr;
  const bool fork = ak.len_major && aq.len_major && std::min(ak.mq, ak.mk) >= kSideMinRows;
  ak.pair = aq.pair = fork ? 1 : 0;
  return fork_join(
      s, fork,
      [&](hipStream_t x) {
        int r = STREAMKL_OK;
        if (student) {
          ak.dk = dk_s;
          r = to_status(skl::launch_js_bwd_dk(ak, p->dtype, p->d_t, p->d_s, causal, false, x));
        }
        if (r == STREAMKL_OK && teacher) {
          ak.dk = dk_t;
          r = to_status(skl::launch_js_bwd_dk(ak, p->dtype, p->d_t, p->d_s, causal, true, x));
        }
        return r;
      },
      [&](hipStream_t x) {
        int r = STREAMKL_OK;
        if (student) {
          aq.dq = dq_s;
          r = to_status(skl::launch_js_bwd_dq(aq, p->dtype, p->d_t, p->d_s, causal, false, x));
        }
        if (r == STREAMKL_OK && teacher) {
          aq.dq = dq_t;
          r = to_status(skl::launch_js_bwd_dq(aq, p->dtype, p->d_t, p->d_s, causal, true, x));
        }
        return r;
      });
}

int streamkl_bwd_noalloc(const streamkl_problem_t* p, const void* q_t, const void* k_t, const void* q_s,
                         const void* k_s, const float* lse_t, const float* lse_s, const float* kl, const float* g,
                         float* dq_s, float* dk_s, float* dq_t, float* dk_t, void* hip_stream) {
  if (p != nullptr && p->workspace != nullptr) return STREAMKL_ERR_INVALID;  // the scratch takes its place
  bool empty = false;
  int st = check_problem(p, &empty);
  if (st != STREAMKL_OK) return st;
  streamkl_problem_t q = *p;
  q.workspace_floats = 0;
  // the arrangement streamkl_bwd takes with a caller workspace of the size streamkl_workspace_floats
  // reports, so both entry points give the same bits
  const int64_t need = streamkl_workspace_floats(p);
  if (need > skl::kScratchFloats) return STREAMKL_ERR_SCRATCH;
  if (need > 0 && !empty) {
    float* ptr = nullptr;
    if (skl::scratch_address(&ptr) != hipSuccess) return STREAMKL_ERR_LAUNCH;
    q.workspace = ptr;  // the device copy's address, never the host-side symbol
    q.workspace_floats = need;
  }
  // no side stream: creating one may allocate, and the kernels' results do not depend on it
  return bwd_impl(&q, q_t, k_t, q_s, k_s, lse_t, lse_s, kl, g, dq_s, dk_s, dq_t, dk_t, hip_stream, false);
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
    case STREAMKL_ERR_SCRATCH:
      return "STREAMKL_ERR_SCRATCH: the problem needs more scratch than the library's static array holds "
             "(pass a workspace to streamkl_bwd instead)";
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
  return std::max(best, fwd_split_floats(p));  // the forward's split of small causal grids
}

}  // extern "C"
