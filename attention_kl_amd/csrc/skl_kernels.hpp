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
  float* kl;
  float* lse_t;
  float* lse_s;
  int64_t sqt[3], skt[3], sqs[3], sks[3];  // (b, h, n) element strides; K strides per key head
  int32_t B, H, Nq, Nk;
  int32_t gt, gs;   // query heads per key head (teacher, student): query head h reads key head h / g
  float c_t, c_s;   // scale * log2(e): logits enter exp2 in these units
  float ratio;      // scale_s / scale_t
  float scale_t;
};

struct BwdArgs {
  const void* qt;
  const void* kt;
  const void* qs;
  const void* ks;
  const float* lse_t;
  const float* lse_s;
  const float* kl;  // read only for teacher gradients
  const float* g;
  float* dq;  // query-owner kernel output [B,H,Nq,d_side]
  float* dk;  // key-owner kernel output   [B,Hk_side,Nk,d_side]
  int64_t sqt[3], skt[3], sqs[3], sks[3];
  int32_t B, H, Nq, Nk;
  int32_t gt, gs;  // query heads per key head (teacher, student)
  float c_t, c_s;            // scale * log2(e)
  float scale_t, scale_s;
};

// dtype: 0 fp32, 1 bf16.  d_t, d_s in {64, 128}.  Return hipErrorInvalidValue for
// combinations that are not built (the C ABI rejects them before calling).
hipError_t launch_fwd(const FwdArgs& a, int dtype, int d_t, int d_s, bool causal, hipStream_t s);
hipError_t launch_bwd_dq(const BwdArgs& a, int dtype, int d_t, int d_s, bool causal, bool teacher, hipStream_t s);
hipError_t launch_bwd_dk(const BwdArgs& a, int dtype, int d_t, int d_s, bool causal, bool teacher, hipStream_t s);

}  // namespace skl
