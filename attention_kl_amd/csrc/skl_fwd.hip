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
//
// Schedule: key tiles are prefetched from HBM/L2 into registers one tile ahead
// and written to a double-buffered LDS ring (one barrier per tile).  Tiles that
// are fully allowed for every row of the workgroup run a software pipeline: the
// MFMAs of key subtile s+1 are issued in the same basic block as the exp/VALU
// work of subtile s, so the matrix cores and the VALU overlap.  The few tiles on
// the causal diagonal or past the ragged end run a separate masked loop.
#include "skl_device.hpp"
#include "skl_kernels.hpp"

namespace skl {

// Scheduling hint for one pipeline step: spread the MFMAs of the next subtile
// (with their LDS operand reads one step ahead) through the VALU work of the
// current one, so a single wavefront keeps the matrix core and the VALU busy.
#ifndef SKL_FWD_SCHED
#define SKL_FWD_SCHED 1
#endif
#if SKL_FWD_SCHED == 1
#define SKL_FWD_INTERLEAVE()                                          \
  do {                                                                \
    __builtin_amdgcn_sched_group_barrier(0x100, 2, 0);                \
    _Pragma("unroll") for (int _k = 0; _k < 16; ++_k) {               \
      __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);              \
      __builtin_amdgcn_sched_group_barrier(0x002, 5, 0);              \
      __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);              \
      __builtin_amdgcn_sched_group_barrier(0x002, 5, 0);              \
    }                                                                 \
  } while (0)
#elif SKL_FWD_SCHED == 2
#define SKL_FWD_INTERLEAVE()                                          \
  do {                                                                \
    _Pragma("unroll") for (int _k = 0; _k < 16; ++_k) {               \
      __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);              \
      __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);              \
      __builtin_amdgcn_sched_group_barrier(0x002, 10, 0);             \
    }                                                                 \
  } while (0)
#else
#define SKL_FWD_INTERLEAVE() \
  do {                       \
  } while (0)
#endif

template <typename T>
struct FwdTile {
  static constexpr int BQ = 128;                       // query rows per workgroup
  static constexpr int BK = sizeof(T) == 2 ? 64 : 32;  // keys per LDS tile
  static constexpr int NT = 256;
};

template <typename T, int DT, int DS>
constexpr int fwd_lds_bytes() {
  return 2 * FwdTile<T>::BK * ((DT + DS) * (int)sizeof(T) + 32);
}

// Per-lane running state of one query row over the keys this lane half sees.
struct RowState {
  float m_t, m_s;  // running maxima in log2 units (logit * scale * log2 e)
  float l_t, l_s, acc;
};

// Online update with one 32-key subtile: st/ss are the raw (unscaled) logits of this
// lane's 16 keys; masked keys are -inf in st/ss, dif = (a - b) / scale_t is finite.
__device__ __forceinline__ void online_update(RowState& s, const f32x16& st, const f32x16& ss, const float* dif,
                                              float c_t, float c_s) {
  float mx = fmaxf(st[0], st[1]), my = fmaxf(ss[0], ss[1]);
#pragma unroll
  for (int i = 2; i < 16; ++i) {
    mx = fmaxf(mx, st[i]);
    my = fmaxf(my, ss[i]);
  }
  const float mt_new = fmaxf(s.m_t, mx * c_t);
  const float ms_new = fmaxf(s.m_s, my * c_s);
  const float al_t = fast_exp2(s.m_t - mt_new);
  const float al_s = fast_exp2(s.m_s - ms_new);
  s.m_t = mt_new;
  s.m_s = ms_new;
  float pt = 0.f, ps = 0.f, pa = 0.f;
#pragma unroll
  for (int i = 0; i < 16; ++i) {
    const float e = fast_exp2(fmaf(st[i], c_t, -mt_new));
    const float f = fast_exp2(fmaf(ss[i], c_s, -ms_new));
    pt += e;
    ps += f;
    pa = fmaf(e, dif[i], pa);
  }
  s.l_t = fmaf(s.l_t, al_t, pt);
  s.l_s = fmaf(s.l_s, al_s, ps);
  s.acc = fmaf(s.acc, al_t, pa);
}

template <typename T, int DT, int DS, bool CAUSAL>
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(sizeof(T) == 2 ? 2 : 1, 2))) void fwd_kernel(const FwdArgs a) {
  constexpr int BQ = FwdTile<T>::BQ, BK = FwdTile<T>::BK, NT = FwdTile<T>::NT;
  constexpr int NSUB = BK / 32;
  constexpr int PT = DT * (int)sizeof(T) + 16;  // padded LDS row pitch (bytes)
  constexpr int PS = DS * (int)sizeof(T) + 16;
  constexpr int TILE = BK * (PT + PS);  // bytes of one K_t + K_s tile in LDS
  constexpr int NCT = DT * (int)sizeof(T) / 16, NCS = DS * (int)sizeof(T) / 16;  // 16-byte chunks per row
  constexpr int NLT = BK * NCT / NT, NLS = BK * NCS / NT;  // chunks per thread per tile
  static_assert(BK * NCT % NT == 0 && BK * NCS % NT == 0, "tile must split evenly over the workgroup");
  extern __shared__ __attribute__((aligned(16))) char lds[];

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6, hf = lane >> 5, r32 = lane & 31;
  const int nbh = a.B * a.H;
  const int nqb = (a.Nq + BQ - 1) / BQ;
  const int bh = blockIdx.x % nbh;
  const int qi = blockIdx.x / nbh;
  const int qb = CAUSAL ? (nqb - 1 - qi) : qi;  // causal: longest rows first
  const int b = bh / a.H, h = bh % a.H;
  const int off = a.Nk - a.Nq;

  const T* qt = reinterpret_cast<const T*>(a.qt) + b * a.sqt[0] + h * a.sqt[1];
  const char* kt = reinterpret_cast<const char*>(reinterpret_cast<const T*>(a.kt) + b * a.skt[0] + h * a.skt[1]);
  const T* qs = reinterpret_cast<const T*>(a.qs) + b * a.sqs[0] + h * a.sqs[1];
  const char* ks = reinterpret_cast<const char*>(reinterpret_cast<const T*>(a.ks) + b * a.sks[0] + h * a.sks[1]);
  const int64_t kt_pitch = a.skt[2] * (int64_t)sizeof(T), ks_pitch = a.sks[2] * (int64_t)sizeof(T);

  const int q0 = qb * BQ;
  const int q0w = q0 + wave * 32;
  const int qrow = q0w + r32;
  u32x4 qt_r[NCT / 2], qs_r[NCS / 2];
  load_row_regs<T, DT>(qt_r, qt + (int64_t)qrow * a.sqt[2], qrow < a.Nq, hf);
  load_row_regs<T, DS>(qs_r, qs + (int64_t)qrow * a.sqs[2], qrow < a.Nq, hf);

  RowState rs{kMaxInit, kMaxInit, 0.f, 0.f, 0.f};

  const int q_last = min(a.Nq, q0 + BQ) - 1;
  const int kend = CAUSAL ? min(a.Nk, q_last + off + 1) : a.Nk;
  const int ntiles = (kend + BK - 1) / BK;
  // tiles whose every key is allowed for every row of the workgroup
  const int t_full = min(ntiles, (CAUSAL ? min(a.Nk, q0 + off + 1) : a.Nk) / BK);

  // ---- K tile prefetch: registers one tile ahead, through buffer loads that return zero past
  // the last key (a scalar tile offset plus a loop-invariant per-lane offset: no address math)
  const __amdgpu_buffer_rsrc_t rk_t = make_rsrc(kt, (uint32_t)((a.Nk - 1) * kt_pitch + DT * (int)sizeof(T)));
  const __amdgpu_buffer_rsrc_t rk_s = make_rsrc(ks, (uint32_t)((a.Nk - 1) * ks_pitch + DS * (int)sizeof(T)));
  int vo_t[NLT], vo_s[NLS];
#pragma unroll
  for (int j = 0; j < NLT; ++j) {
    const int idx = tid + j * NT;
    vo_t[j] = (idx / NCT) * (int)kt_pitch + (idx % NCT) * 16;
  }
#pragma unroll
  for (int j = 0; j < NLS; ++j) {
    const int idx = tid + j * NT;
    vo_s[j] = (idx / NCS) * (int)ks_pitch + (idx % NCS) * 16;
  }
  u32x4 pf_t[NLT], pf_s[NLS];
  auto prefetch = [&](int tile) {
    const int so_t = tile * BK * (int)kt_pitch, so_s = tile * BK * (int)ks_pitch;
#pragma unroll
    for (int j = 0; j < NLT; ++j) pf_t[j] = buffer_load16(rk_t, vo_t[j], so_t);
#pragma unroll
    for (int j = 0; j < NLS; ++j) pf_s[j] = buffer_load16(rk_s, vo_s[j], so_s);
  };
  auto commit = [&](int tile) {
    char* base = lds + (tile & 1) * TILE;
#pragma unroll
    for (int j = 0; j < NLT; ++j) {
      const int idx = tid + j * NT, r = idx / NCT, c = idx % NCT;
      *reinterpret_cast<u32x4*>(base + r * PT + c * 16) = pf_t[j];
    }
#pragma unroll
    for (int j = 0; j < NLS; ++j) {
      const int idx = tid + j * NT, r = idx / NCS, c = idx % NCS;
      *reinterpret_cast<u32x4*>(base + BK * PT + r * PS + c * 16) = pf_s[j];
    }
  };
  auto logits = [&](f32x16& st, f32x16& ss, int tile, int sub) {
    const char* base = lds + (tile & 1) * TILE;
    st = f32x16{};
    ss = f32x16{};
    tile_dot_lds_a<T, DT>(st, base + (sub * 32 + r32) * PT, hf, qt_r);
    tile_dot_lds_a<T, DS>(ss, base + BK * PT + (sub * 32 + r32) * PS, hf, qs_r);
  };
  auto update_full = [&](const f32x16& st, const f32x16& ss) {
    float dif[16];
#pragma unroll
    for (int i = 0; i < 16; ++i) dif[i] = fmaf(ss[i], -a.ratio, st[i]);
    online_update(rs, st, ss, dif, a.c_t, a.c_s);
  };

  if (ntiles > 0) prefetch(0);

  // ---- pipelined loop over the fully allowed tiles.  Each step is straight-line code that issues
  // the MFMAs of the next key subtile and runs the exp/VALU update of the current one.
  if (t_full > 0) {
    commit(0);
    if (ntiles > 1) prefetch(1);
    __syncthreads();
    f32x16 cur_t, cur_s, nxt_t, nxt_s;
    logits(cur_t, cur_s, 0, 0);
    for (int t = 0; t < t_full; ++t) {
#pragma unroll
      for (int sub = 1; sub < NSUB; ++sub) {
        logits(nxt_t, nxt_s, t, sub);
        SKL_FWD_INTERLEAVE();
        update_full(cur_t, cur_s);
        cur_t = nxt_t;
        cur_s = nxt_s;
      }
      // publish tile t+1 (its buffer last held tile t-1, whose reads ended before the previous
      // barrier).  Unconditional so the step stays one basic block: past the last tile the
      // prefetch returns zeros and the commit fills a buffer no wave reads.
      commit(t + 1);
      prefetch(t + 2);
      __syncthreads();
      // first subtile of tile t+1; past the last full tile the result is discarded
      logits(nxt_t, nxt_s, t + 1, 0);
      SKL_FWD_INTERLEAVE();
      update_full(cur_t, cur_s);
      cur_t = nxt_t;
      cur_s = nxt_s;
    }
  }

  // ---- masked tail: causal diagonal tiles and the ragged end
  // (the pipelined loop already published tile t_full; buffer t&1 of a later tile last held tile
  // t-2, whose reads all finished before the barrier that published tile t-1)
  for (int t = t_full; t < ntiles; ++t) {
    if (t > t_full || t_full == 0) {
      commit(t);
      if (t + 1 < ntiles) prefetch(t + 1);
      __syncthreads();
    }
#pragma unroll
    for (int sub = 0; sub < NSUB; ++sub) {
      const int kb = t * BK + sub * 32;
      if (kb >= a.Nk) break;
      if (CAUSAL && kb > q0w + 31 + off) break;  // no row of this wavefront reaches these keys
      f32x16 st, ss;
      logits(st, ss, t, sub);
      float dif[16];
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        dif[i] = fmaf(ss[i], -a.ratio, st[i]);
        const int key = kb + acc_row(i, hf);
        const bool ok = key < a.Nk && (!CAUSAL || key <= qrow + off);
        st[i] = ok ? st[i] : -INFINITY;
        ss[i] = ok ? ss[i] : -INFINITY;
      }
      online_update(rs, st, ss, dif, a.c_t, a.c_s);
    }
  }

  // Merge the two half-row states (disjoint key subsets) of each query row.
  const float o_mt = __shfl_xor(rs.m_t, 32), o_lt = __shfl_xor(rs.l_t, 32), o_acc = __shfl_xor(rs.acc, 32);
  const float o_ms = __shfl_xor(rs.m_s, 32), o_ls = __shfl_xor(rs.l_s, 32);
  const float Mt = fmaxf(rs.m_t, o_mt), Ms = fmaxf(rs.m_s, o_ms);
  const float f1 = fast_exp2(rs.m_t - Mt), f2 = fast_exp2(o_mt - Mt);
  const float g1 = fast_exp2(rs.m_s - Ms), g2 = fast_exp2(o_ms - Ms);
  const float Lt = rs.l_t * f1 + o_lt * f2;
  const float Ls = rs.l_s * g1 + o_ls * g2;
  const float A = rs.acc * f1 + o_acc * f2;

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
  constexpr int lds = fwd_lds_bytes<T, DT, DS>();
  auto kern = fwd_kernel<T, DT, DS, C>;
  if (lds > 65536) {
    const hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void*>(kern),
                                             hipFuncAttributeMaxDynamicSharedMemorySize, lds);
    if (e != hipSuccess) return e;
  }
  hipLaunchKernelGGL(kern, dim3((unsigned)nblk), dim3(FwdTile<T>::NT), lds, s, a);
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
