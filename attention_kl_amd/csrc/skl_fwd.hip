// One-pass forward of the attention KL divergence on gfx950.
//
// StreamKL abstract (arXiv 2026), S4: the coupled two-distribution KL is reduced
// online, in one pass that streams query/key tiles through on-chip memory.  The
// online form used here follows from the definition: with per-row running
// maxima m_t, m_s of the teacher and student logits, running sums
// l_t = sum exp(a_j - m_t), l_s = sum exp(b_j - m_s) and the teacher-weighted
// accumulator acc = sum exp(a_j - m_t) (a_j - b_j), all rescaled when a maximum
// grows,
//     sum_j P_t,j (a_j - b_j) = acc / l_t,   KL = acc/l_t - (m_t + ln l_t) + (m_s + ln l_s).
// The row is closed as acc/l_t + (m_s - m_t) + ln(l_s/l_t), the same value
// with one log of a ratio instead of two large log-sum-exps that cancel.
//
// Work split: one workgroup = 4 wavefronts = 128 query rows of one (b, h); each
// wavefront keeps its 32 rows' Q_t, Q_s in registers as MFMA B operands and
// streams key tiles through LDS.  The logit tile is formed transposed
// (keys x queries) so each lane owns one query row and 16 of its keys: the two
// lane halves of a row keep separate running states over disjoint key subsets
// and are merged once at the end, so the key loop needs no cross-lane traffic.
#include "skl_device.hpp"
#include "skl_kernels.hpp"

namespace skl {

template <typename T>
struct FwdTile {
  static constexpr int BQ = 128;                       // query rows per workgroup
  static constexpr int BK = sizeof(T) == 2 ? 64 : 32;  // keys per LDS tile
};

template <typename T, int DT, int DS, bool CAUSAL>
__global__ __launch_bounds__(256) void fwd_kernel(const FwdArgs a) {
  constexpr int BQ = FwdTile<T>::BQ, BK = FwdTile<T>::BK, NT = 256;
  constexpr int PT = DT * (int)sizeof(T) + 16;  // padded LDS row pitch (bytes)
  constexpr int PS = DS * (int)sizeof(T) + 16;
  __shared__ __attribute__((aligned(16))) char lds[BK * (PT + PS)];
  char* lds_kt = lds;
  char* lds_ks = lds + BK * PT;

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6, hf = lane >> 5, r32 = lane & 31;
  const int nbh = a.B * a.H;
  const int nqb = (a.Nq + BQ - 1) / BQ;
  const int bh = blockIdx.x % nbh;
  const int qi = blockIdx.x / nbh;
  const int qb = CAUSAL ? (nqb - 1 - qi) : qi;  // causal: longest rows first
  const int b = bh / a.H, h = bh % a.H;
  const int off = a.Nk - a.Nq;

  const T* qt = reinterpret_cast<const T*>(a.qt) + b * a.sqt[0] + h * a.sqt[1];
  const T* kt = reinterpret_cast<const T*>(a.kt) + b * a.skt[0] + h * a.skt[1];
  const T* qs = reinterpret_cast<const T*>(a.qs) + b * a.sqs[0] + h * a.sqs[1];
  const T* ks = reinterpret_cast<const T*>(a.ks) + b * a.sks[0] + h * a.sks[1];

  const int q0w = qb * BQ + wave * 32;
  const int qrow = q0w + r32;
  u32x4 qt_r[DT * sizeof(T) / 32], qs_r[DS * sizeof(T) / 32];
  load_row_regs<T, DT>(qt_r, qt + (int64_t)qrow * a.sqt[2], qrow < a.Nq, hf);
  load_row_regs<T, DS>(qs_r, qs + (int64_t)qrow * a.sqs[2], qrow < a.Nq, hf);

  float m_t = kMaxInit, m_s = kMaxInit;  // running maxima, log2 units (logit * scale * log2 e)
  float l_t = 0.f, l_s = 0.f, acc = 0.f;

  const int q_last = min(a.Nq, (qb + 1) * BQ) - 1;
  const int kend = CAUSAL ? min(a.Nk, q_last + off + 1) : a.Nk;
  const int ntiles = (kend + BK - 1) / BK;

  for (int t = 0; t < ntiles; ++t) {
    const int k0 = t * BK;
    __syncthreads();
    stage_tile<T, DT, BK, NT, 0>(lds_kt, PT, nullptr, kt + (int64_t)k0 * a.skt[2], a.skt[2], a.Nk - k0, tid);
    stage_tile<T, DS, BK, NT, 0>(lds_ks, PS, nullptr, ks + (int64_t)k0 * a.sks[2], a.sks[2], a.Nk - k0, tid);
    __syncthreads();
#pragma unroll
    for (int sub = 0; sub < BK / 32; ++sub) {
      const int kb = k0 + sub * 32;
      if (kb >= a.Nk) break;
      if (CAUSAL && kb > q0w + 31 + off) break;  // no row of this wavefront reaches these keys
      f32x16 st = {}, ss = {};
      tile_dot_lds_a<T, DT>(st, lds_kt + (sub * 32 + r32) * PT, hf, qt_r);
      tile_dot_lds_a<T, DS>(ss, lds_ks + (sub * 32 + r32) * PS, hf, qs_r);

      float dif[16];  // (a - b) / scale_t, taken before masking so masked entries stay finite
#pragma unroll
      for (int i = 0; i < 16; ++i) dif[i] = fmaf(ss[i], -a.ratio, st[i]);
      const bool need_mask = (kb + 31 >= a.Nk) || (CAUSAL && kb + 31 > q0w + off);
      if (need_mask) {
#pragma unroll
        for (int i = 0; i < 16; ++i) {
          const int key = kb + acc_row(i, hf);
          const bool ok = key < a.Nk && (!CAUSAL || key <= qrow + off);
          if (!ok) {
            st[i] = -INFINITY;
            ss[i] = -INFINITY;
          }
        }
      }
      float mx = st[0], my = ss[0];
#pragma unroll
      for (int i = 1; i < 16; ++i) {
        mx = fmaxf(mx, st[i]);
        my = fmaxf(my, ss[i]);
      }
      const float mt_new = fmaxf(m_t, mx * a.c_t);
      const float ms_new = fmaxf(m_s, my * a.c_s);
      const float al_t = fast_exp2(m_t - mt_new);
      const float al_s = fast_exp2(m_s - ms_new);
      m_t = mt_new;
      m_s = ms_new;
      float pt = 0.f, ps = 0.f, pa = 0.f;
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        const float e = fast_exp2(fmaf(st[i], a.c_t, -mt_new));
        const float f = fast_exp2(fmaf(ss[i], a.c_s, -ms_new));
        pt += e;
        ps += f;
        pa = fmaf(e, dif[i], pa);
      }
      l_t = fmaf(l_t, al_t, pt);
      l_s = fmaf(l_s, al_s, ps);
      acc = fmaf(acc, al_t, pa);
    }
  }

  // Merge the two half-row states (disjoint key subsets) of each query row.
  const float o_mt = __shfl_xor(m_t, 32), o_lt = __shfl_xor(l_t, 32), o_acc = __shfl_xor(acc, 32);
  const float o_ms = __shfl_xor(m_s, 32), o_ls = __shfl_xor(l_s, 32);
  const float Mt = fmaxf(m_t, o_mt), Ms = fmaxf(m_s, o_ms);
  const float f1 = fast_exp2(m_t - Mt), f2 = fast_exp2(o_mt - Mt);
  const float g1 = fast_exp2(m_s - Ms), g2 = fast_exp2(o_ms - Ms);
  const float Lt = l_t * f1 + o_lt * f2;
  const float Ls = l_s * g1 + o_ls * g2;
  const float A = acc * f1 + o_acc * f2;

  if (hf == 0 && qrow < a.Nq) {
    // true divisions: Ls / Lt is exactly 1 when the two states are bitwise equal
    const int64_t o = ((int64_t)bh) * a.Nq + qrow;
    a.kl[o] = a.scale_t * (A / Lt) + kLn2 * ((Ms - Mt) + fast_log2(Ls / Lt));
    a.lse_t[o] = kLn2 * (Mt + fast_log2(Lt));
    a.lse_s[o] = kLn2 * (Ms + fast_log2(Ls));
  }
}

template <typename T, int DT, int DS, bool C>
static hipError_t launch_fwd_t(const FwdArgs& a, hipStream_t s) {
  const int64_t nqb = (a.Nq + FwdTile<T>::BQ - 1) / FwdTile<T>::BQ;
  const int64_t nblk = nqb * a.B * a.H;
  if (nblk <= 0) return hipSuccess;
  if (nblk > 0x7fffffff) return hipErrorInvalidValue;
  hipLaunchKernelGGL((fwd_kernel<T, DT, DS, C>), dim3((unsigned)nblk), dim3(256), 0, s, a);
  return hipGetLastError();
}

template <typename T, int DT, int DS>
static hipError_t fwd_c(const FwdArgs& a, bool causal, hipStream_t s) {
  return causal ? launch_fwd_t<T, DT, DS, true>(a, s) : launch_fwd_t<T, DT, DS, false>(a, s);
}

template <typename T>
static hipError_t fwd_d(const FwdArgs& a, int dt, int ds, bool causal, hipStream_t s) {
  if (dt == 128 && ds == 128) return fwd_c<T, 128, 128>(a, causal, s);
  if (dt == 128 && ds == 64) return fwd_c<T, 128, 64>(a, causal, s);
  if (dt == 64 && ds == 128) return fwd_c<T, 64, 128>(a, causal, s);
  if (dt == 64 && ds == 64) return fwd_c<T, 64, 64>(a, causal, s);
  return hipErrorInvalidValue;
}

hipError_t launch_fwd(const FwdArgs& a, int dtype, int dt, int ds, bool causal, hipStream_t s) {
  if (dtype == 1) return fwd_d<__bf16>(a, dt, ds, causal, s);
  if (dtype == 0) return fwd_d<float>(a, dt, ds, causal, s);
  return hipErrorInvalidValue;
}

}  // namespace skl
