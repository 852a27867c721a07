// Recompute backward of the attention KL divergence on gfx950.
//
// StreamKL abstract (arXiv 2026), S5: the backward recomputes the attention
// probabilities tile by tile instead of storing any N_Q x N_K intermediate.
// From the forward's per-row log-sum-exps, each logit tile gives
//   P_t = exp(a - LSE_t),  P_s = exp(b - LSE_s)
// and the gradients of L = sum_i g_i KL_i (calculus of the KL definition):
//   student  dS = g_i (P_s - P_t)
//   teacher  dS = g_i P_t ((a - b) - (KL_i + LSE_t,i - LSE_s,i))
//   dQ = scale dS K,   dK = scale dS^T Q     (K, Q of the same side)
//
// Two kernels, each owning its output rows so there are no atomics and no
// workspace: the query-owner kernel keeps 128 query rows in registers and
// streams key tiles (dQ), the key-owner kernel keeps 128 keys in registers and
// streams query tiles (dK).  Each recomputes both logit tiles.
//
// bf16: dS is fed to the MFMA as hi + lo bf16 parts (two products), so its
// rounding contributes about 2^-16 relative instead of bf16's 2^-9.
#include "skl_device.hpp"
#include "skl_kernels.hpp"

namespace skl {

// a * sa - b * sb with both products rounded before the subtraction (no FMA contraction), so the
// result is exactly 0 when (a, sa) == (b, sb): identical teacher and student give zero gradients.
__device__ __forceinline__ float scaled_diff(float a, float sa, float b, float sb) {
#pragma clang fp contract(off)
  return a * sa - b * sb;
}

template <typename T>
struct BwdTile {
  static constexpr int BW = 128;                       // owned rows per workgroup (4 waves x 32)
  static constexpr int BS = sizeof(T) == 2 ? 64 : 32;  // streamed rows per LDS tile
};

// Accumulate one 32x32 dS tile (register layout: lane = owned row, 16 streamed rows per
// lane at acc_row(i, hf)) against the streamed operand X, held transposed in LDS
// ([feature][streamed row], pitch PX bytes): out[db] += dS . X[:, 32db .. 32db+31].
template <typename T, int DX, int PX>
__device__ __forceinline__ void grad_product(f32x16* out, const float* ds, const char* xT, int sub, int hf, int r32) {
  if constexpr (sizeof(T) == 2) {
#pragma unroll
    for (int c = 0; c < 2; ++c) {
      u32x4 hi, lo;
      split_bf16x8(ds + 8 * c, hi, lo);
#pragma unroll
      for (int db = 0; db < DX / 32; ++db) {
        const char* col = xT + (db * 32 + r32) * PX + (sub * 32 + 16 * c + 4 * hf) * 2;
        const u32x2 p0 = lds_read8(col), p1 = lds_read8(col + 16);
        const u32x4 bop = {p0[0], p0[1], p1[0], p1[1]};
        mma_chunk<__bf16>(out[db], hi, bop);
        mma_chunk<__bf16>(out[db], lo, bop);
      }
    }
  } else {
#pragma unroll
    for (int g4 = 0; g4 < 4; ++g4) {
#pragma unroll
      for (int db = 0; db < DX / 32; ++db) {
        const u32x4 bop = lds_read16(xT + (db * 32 + r32) * PX + (sub * 32 + 8 * g4 + 4 * hf) * 4);
        const uint32_t bv[4] = {bop[0], bop[1], bop[2], bop[3]};
#pragma unroll
        for (int e = 0; e < 4; ++e)
          out[db] = __builtin_amdgcn_mfma_f32_32x32x2f32(ds[4 * g4 + e], __uint_as_float(bv[e]), out[db], 0, 0, 0);
      }
    }
  }
}

// ----------------------------------------------------------------------------------------------
// Query-owner kernel: dQ of one side for 128 query rows.
template <typename T, int DT, int DS, bool CAUSAL, bool TEACHER>
__global__ __launch_bounds__(256) void bwd_dq_kernel(const BwdArgs a) {
  constexpr int BW = BwdTile<T>::BW, BK = BwdTile<T>::BS, NT = 256;
  constexpr int DX = TEACHER ? DT : DS;
  constexpr int PT = DT * (int)sizeof(T) + 16, PS = DS * (int)sizeof(T) + 16;
  constexpr int PX = BK * (int)sizeof(T) + 16;  // pitch of the transposed tile
  __shared__ __attribute__((aligned(16))) char lds[BK * (PT + PS) + DX * PX];
  char* lds_kt = lds;
  char* lds_ks = lds + BK * PT;
  char* lds_xT = lds + BK * (PT + PS);

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6, hf = lane >> 5, r32 = lane & 31;
  const int nbh = a.B * a.H;
  const int nqb = (a.Nq + BW - 1) / BW;
  const int bh = blockIdx.x % nbh;
  const int qi = blockIdx.x / nbh;
  const int qb = CAUSAL ? (nqb - 1 - qi) : qi;
  const int b = bh / a.H, h = bh % a.H;
  const int off = a.Nk - a.Nq;

  const T* qt = reinterpret_cast<const T*>(a.qt) + b * a.sqt[0] + h * a.sqt[1];
  const T* kt = reinterpret_cast<const T*>(a.kt) + b * a.skt[0] + h * a.skt[1];
  const T* qs = reinterpret_cast<const T*>(a.qs) + b * a.sqs[0] + h * a.sqs[1];
  const T* ks = reinterpret_cast<const T*>(a.ks) + b * a.sks[0] + h * a.sks[1];

  const int q0w = qb * BW + wave * 32;
  const int qrow = q0w + r32;
  const bool qvalid = qrow < a.Nq;
  u32x4 qt_r[DT * sizeof(T) / 32], qs_r[DS * sizeof(T) / 32];
  load_row_regs<T, DT>(qt_r, qt + (int64_t)qrow * a.sqt[2], qvalid, hf);
  load_row_regs<T, DS>(qs_r, qs + (int64_t)qrow * a.sqs[2], qvalid, hf);

  const int64_t ro = (int64_t)bh * a.Nq + qrow;
  const float lse2_t = qvalid ? a.lse_t[ro] * kLog2e : 0.f;
  const float lse2_s = qvalid ? a.lse_s[ro] * kLog2e : 0.f;
  const float gq = qvalid ? a.g[ro] : 0.f;
  float cq = 0.f;  // teacher: KL_i + LSE_t,i - LSE_s,i = sum_j P_t (a - b)
  if constexpr (TEACHER) cq = qvalid ? a.kl[ro] + a.lse_t[ro] - a.lse_s[ro] : 0.f;

  f32x16 dacc[DX / 32];
#pragma unroll
  for (int db = 0; db < DX / 32; ++db) dacc[db] = f32x16{};

  const int q_last = min(a.Nq, (qb + 1) * BW) - 1;
  const int kend = CAUSAL ? min(a.Nk, q_last + off + 1) : a.Nk;
  const int ntiles = (kend + BK - 1) / BK;

  for (int t = 0; t < ntiles; ++t) {
    const int k0 = t * BK;
    __syncthreads();
    if constexpr (TEACHER) {
      stage_tile<T, DT, BK, NT, PX>(lds_kt, PT, lds_xT, kt + (int64_t)k0 * a.skt[2], a.skt[2], a.Nk - k0, tid);
      stage_tile<T, DS, BK, NT, 0>(lds_ks, PS, nullptr, ks + (int64_t)k0 * a.sks[2], a.sks[2], a.Nk - k0, tid);
    } else {
      stage_tile<T, DT, BK, NT, 0>(lds_kt, PT, nullptr, kt + (int64_t)k0 * a.skt[2], a.skt[2], a.Nk - k0, tid);
      stage_tile<T, DS, BK, NT, PX>(lds_ks, PS, lds_xT, ks + (int64_t)k0 * a.sks[2], a.sks[2], a.Nk - k0, tid);
    }
    __syncthreads();
#pragma unroll
    for (int sub = 0; sub < BK / 32; ++sub) {
      const int kb = k0 + sub * 32;
      if (kb >= a.Nk) break;
      if (CAUSAL && kb > q0w + 31 + off) break;
      f32x16 st = {}, ss = {};
      tile_dot_lds_a<T, DT>(st, lds_kt + (sub * 32 + r32) * PT, hf, qt_r);
      tile_dot_lds_a<T, DS>(ss, lds_ks + (sub * 32 + r32) * PS, hf, qs_r);
      const bool need_mask = (kb + 31 >= a.Nk) || (CAUSAL && kb + 31 > q0w + off);
      float ds[16];
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        const float pt = fast_exp2(fmaf(st[i], a.c_t, -lse2_t));
        if constexpr (TEACHER) {
          ds[i] = gq * pt * (scaled_diff(st[i], a.scale_t, ss[i], a.scale_s) - cq);
        } else {
          const float ps = fast_exp2(fmaf(ss[i], a.c_s, -lse2_s));
          ds[i] = gq * (ps - pt);
        }
        if (need_mask) {
          const int key = kb + acc_row(i, hf);
          const bool ok = key < a.Nk && (!CAUSAL || key <= qrow + off);
          ds[i] = ok ? ds[i] : 0.f;
        }
      }
      grad_product<T, DX, PX>(dacc, ds, lds_xT, sub, hf, r32);
    }
  }

  const float scale = TEACHER ? a.scale_t : a.scale_s;
  float* out = a.dq + (int64_t)bh * a.Nq * DX;
#pragma unroll
  for (int db = 0; db < DX / 32; ++db) {
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      const int q = q0w + acc_row(i, hf);
      if (q < a.Nq) out[(int64_t)q * DX + db * 32 + r32] = scale * dacc[db][i];
    }
  }
}

// ----------------------------------------------------------------------------------------------
// Key-owner kernel: dK of one side for 128 keys.
template <typename T, int DT, int DS, bool CAUSAL, bool TEACHER>
__global__ __launch_bounds__(256) void bwd_dk_kernel(const BwdArgs a) {
  constexpr int BW = BwdTile<T>::BW, BQ = BwdTile<T>::BS, NT = 256;
  constexpr int DX = TEACHER ? DT : DS;
  constexpr int PT = DT * (int)sizeof(T) + 16, PS = DS * (int)sizeof(T) + 16;
  constexpr int PX = BQ * (int)sizeof(T) + 16;
  __shared__ __attribute__((aligned(16))) char lds[BQ * (PT + PS) + DX * PX + 4 * BQ * 4];
  char* lds_qt = lds;
  char* lds_qs = lds + BQ * PT;
  char* lds_xT = lds + BQ * (PT + PS);
  float* st_lse_t = reinterpret_cast<float*>(lds + BQ * (PT + PS) + DX * PX);  // log2 units
  float* st_lse_s = st_lse_t + BQ;
  float* st_g = st_lse_s + BQ;
  float* st_c = st_g + BQ;

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6, hf = lane >> 5, r32 = lane & 31;
  const int nbh = a.B * a.H;
  const int bh = blockIdx.x % nbh;
  const int kb_i = blockIdx.x / nbh;  // causal: low key blocks see the most queries; they go first
  const int b = bh / a.H, h = bh % a.H;
  const int off = a.Nk - a.Nq;

  const T* qt = reinterpret_cast<const T*>(a.qt) + b * a.sqt[0] + h * a.sqt[1];
  const T* kt = reinterpret_cast<const T*>(a.kt) + b * a.skt[0] + h * a.skt[1];
  const T* qs = reinterpret_cast<const T*>(a.qs) + b * a.sqs[0] + h * a.sqs[1];
  const T* ks = reinterpret_cast<const T*>(a.ks) + b * a.sks[0] + h * a.sks[1];

  const int k0wg = kb_i * BW;
  const int k0w = k0wg + wave * 32;
  const int krow = k0w + r32;
  u32x4 kt_r[DT * sizeof(T) / 32], ks_r[DS * sizeof(T) / 32];
  load_row_regs<T, DT>(kt_r, kt + (int64_t)krow * a.skt[2], krow < a.Nk, hf);
  load_row_regs<T, DS>(ks_r, ks + (int64_t)krow * a.sks[2], krow < a.Nk, hf);

  f32x16 dacc[DX / 32];
#pragma unroll
  for (int db = 0; db < DX / 32; ++db) dacc[db] = f32x16{};

  // first query that may attend to this block's first key
  const int qmin = CAUSAL ? max(0, k0wg - off) : 0;
  const int tfirst = qmin / BQ;
  const int ntiles = (a.Nq + BQ - 1) / BQ;
  const float* lse_t_bh = a.lse_t + (int64_t)bh * a.Nq;
  const float* lse_s_bh = a.lse_s + (int64_t)bh * a.Nq;
  const float* g_bh = a.g + (int64_t)bh * a.Nq;
  const float* kl_bh = TEACHER ? a.kl + (int64_t)bh * a.Nq : nullptr;

  for (int t = tfirst; t < ntiles; ++t) {
    const int q0 = t * BQ;
    __syncthreads();
    if constexpr (TEACHER) {
      stage_tile<T, DT, BQ, NT, PX>(lds_qt, PT, lds_xT, qt + (int64_t)q0 * a.sqt[2], a.sqt[2], a.Nq - q0, tid);
      stage_tile<T, DS, BQ, NT, 0>(lds_qs, PS, nullptr, qs + (int64_t)q0 * a.sqs[2], a.sqs[2], a.Nq - q0, tid);
    } else {
      stage_tile<T, DT, BQ, NT, 0>(lds_qt, PT, nullptr, qt + (int64_t)q0 * a.sqt[2], a.sqt[2], a.Nq - q0, tid);
      stage_tile<T, DS, BQ, NT, PX>(lds_qs, PS, lds_xT, qs + (int64_t)q0 * a.sqs[2], a.sqs[2], a.Nq - q0, tid);
    }
    if (tid < BQ) {
      const int q = q0 + tid;
      const bool v = q < a.Nq;
      st_lse_t[tid] = v ? lse_t_bh[q] * kLog2e : 0.f;
      st_lse_s[tid] = v ? lse_s_bh[q] * kLog2e : 0.f;
      st_g[tid] = v ? g_bh[q] : 0.f;
      if constexpr (TEACHER) st_c[tid] = v ? kl_bh[q] + lse_t_bh[q] - lse_s_bh[q] : 0.f;
    }
    __syncthreads();
#pragma unroll
    for (int sub = 0; sub < BQ / 32; ++sub) {
      const int qb = q0 + sub * 32;
      if (qb >= a.Nq) break;
      if (CAUSAL && k0w > qb + 31 + off) continue;  // every key of this wave is past these rows' reach
      f32x16 st = {}, ss = {};
      // S = Q K^T: rows = the tile's queries (LDS), columns = this wave's keys (registers)
      tile_dot_lds_a<T, DT>(st, lds_qt + (sub * 32 + r32) * PT, hf, kt_r);
      tile_dot_lds_a<T, DS>(ss, lds_qs + (sub * 32 + r32) * PS, hf, ks_r);
      const bool need_mask = (qb + 31 >= a.Nq) || (CAUSAL && k0w + 31 > qb + off);
      float ds[16];
#pragma unroll
      for (int g4 = 0; g4 < 4; ++g4) {
        const int ql = sub * 32 + 8 * g4 + 4 * hf;  // first of 4 consecutive tile queries
        const f32x4 lt4 = *reinterpret_cast<const f32x4*>(st_lse_t + ql);
        const f32x4 ls4 = *reinterpret_cast<const f32x4*>(st_lse_s + ql);
        const f32x4 g4v = *reinterpret_cast<const f32x4*>(st_g + ql);
        f32x4 c4 = {};
        if constexpr (TEACHER) c4 = *reinterpret_cast<const f32x4*>(st_c + ql);
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const int i = 4 * g4 + e;
          const float pt = fast_exp2(fmaf(st[i], a.c_t, -lt4[e]));
          float v;
          if constexpr (TEACHER) {
            v = g4v[e] * pt * (scaled_diff(st[i], a.scale_t, ss[i], a.scale_s) - c4[e]);
          } else {
            const float ps = fast_exp2(fmaf(ss[i], a.c_s, -ls4[e]));
            v = g4v[e] * (ps - pt);
          }
          if (need_mask) {
            const int q = q0 + ql + e;
            const bool ok = q < a.Nq && (!CAUSAL || krow <= q + off);
            v = ok ? v : 0.f;
          }
          ds[i] = v;
        }
      }
      grad_product<T, DX, PX>(dacc, ds, lds_xT, sub, hf, r32);
    }
  }

  const float scale = TEACHER ? a.scale_t : a.scale_s;
  float* out = a.dk + (int64_t)bh * a.Nk * DX;
#pragma unroll
  for (int db = 0; db < DX / 32; ++db) {
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      const int k = k0w + acc_row(i, hf);
      if (k < a.Nk) out[(int64_t)k * DX + db * 32 + r32] = scale * dacc[db][i];
    }
  }
}

// ----------------------------------------------------------------------------------------------
template <typename T, int DT, int DS, bool C, bool TE>
static hipError_t launch_dq_t(const BwdArgs& a, hipStream_t s) {
  const int64_t nblk = (int64_t)((a.Nq + BwdTile<T>::BW - 1) / BwdTile<T>::BW) * a.B * a.H;
  if (nblk <= 0) return hipSuccess;
  if (nblk > 0x7fffffff) return hipErrorInvalidValue;
  hipLaunchKernelGGL((bwd_dq_kernel<T, DT, DS, C, TE>), dim3((unsigned)nblk), dim3(256), 0, s, a);
  return hipGetLastError();
}

template <typename T, int DT, int DS, bool C, bool TE>
static hipError_t launch_dk_t(const BwdArgs& a, hipStream_t s) {
  const int64_t nblk = (int64_t)((a.Nk + BwdTile<T>::BW - 1) / BwdTile<T>::BW) * a.B * a.H;
  if (nblk <= 0) return hipSuccess;
  if (nblk > 0x7fffffff) return hipErrorInvalidValue;
  hipLaunchKernelGGL((bwd_dk_kernel<T, DT, DS, C, TE>), dim3((unsigned)nblk), dim3(256), 0, s, a);
  return hipGetLastError();
}

template <bool DQ, typename T, int DT, int DS>
static hipError_t bwd_ct(const BwdArgs& a, bool causal, bool teacher, hipStream_t s) {
  if (DQ) {
    if (causal) return teacher ? launch_dq_t<T, DT, DS, true, true>(a, s) : launch_dq_t<T, DT, DS, true, false>(a, s);
    return teacher ? launch_dq_t<T, DT, DS, false, true>(a, s) : launch_dq_t<T, DT, DS, false, false>(a, s);
  }
  if (causal) return teacher ? launch_dk_t<T, DT, DS, true, true>(a, s) : launch_dk_t<T, DT, DS, true, false>(a, s);
  return teacher ? launch_dk_t<T, DT, DS, false, true>(a, s) : launch_dk_t<T, DT, DS, false, false>(a, s);
}

template <bool DQ, typename T>
static hipError_t bwd_d(const BwdArgs& a, int dt, int ds, bool causal, bool teacher, hipStream_t s) {
  if (dt == 128 && ds == 128) return bwd_ct<DQ, T, 128, 128>(a, causal, teacher, s);
  if (dt == 128 && ds == 64) return bwd_ct<DQ, T, 128, 64>(a, causal, teacher, s);
  if (dt == 64 && ds == 128) return bwd_ct<DQ, T, 64, 128>(a, causal, teacher, s);
  if (dt == 64 && ds == 64) return bwd_ct<DQ, T, 64, 64>(a, causal, teacher, s);
  return hipErrorInvalidValue;
}

hipError_t launch_bwd_dq(const BwdArgs& a, int dtype, int dt, int ds, bool causal, bool teacher, hipStream_t s) {
  if (dtype == 1) return bwd_d<true, __bf16>(a, dt, ds, causal, teacher, s);
  if (dtype == 0) return bwd_d<true, float>(a, dt, ds, causal, teacher, s);
  return hipErrorInvalidValue;
}

hipError_t launch_bwd_dk(const BwdArgs& a, int dtype, int dt, int ds, bool causal, bool teacher, hipStream_t s) {
  if (dtype == 1) return bwd_d<false, __bf16>(a, dt, ds, causal, teacher, s);
  if (dtype == 0) return bwd_d<false, float>(a, dt, ds, causal, teacher, s);
  return hipErrorInvalidValue;
}

}  // namespace skl
