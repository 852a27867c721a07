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
// One kernel template serves both halves.  Each workgroup owns 128 rows of the
// output (query rows for dQ, key rows for dK) and keeps their Q or K slices in
// registers as MFMA B operands; the other side streams through a double-buffered
// LDS ring.  Owning the output rows means no atomics and no workspace.  Both
// halves recompute both logit tiles.
//
// The logit tile is formed with the owned rows as columns, so each lane holds 16
// streamed rows of one owned row; that register block is directly the A operand
// of the gradient product (contraction over the streamed rows).  The B operand,
// the streamed tile read with the streamed rows as the contraction index, comes
// from the row-major LDS tile through transpose reads, so no transposed copy is
// stored.  bf16: dS enters the MFMA as hi + lo bf16 parts (two products), so its
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
  static constexpr int NT = 256;
};

template <typename T, int DT, int DS, bool OWN_Q>
constexpr int bwd_lds_bytes() {
  return 2 * (TileRing<T, DT, DS, BwdTile<T>::BS, BwdTile<T>::NT>::BYTES + (OWN_Q ? 0 : 4 * BwdTile<T>::BS * 4));
}

// out[db] += dS . X[:, 32 db .. 32 db + 31] for one 32-row streamed subtile.  dS is in the
// logit accumulator layout (lane = owned row, element i = streamed row acc_row(i, hf)); X is the
// streamed tile, row-major in LDS at `xt` with pitch PX bytes.
template <typename T, int DX, int PX>
__device__ __forceinline__ void grad_product(f32x16* out, const float* ds, const char* xt, int sub, int lane) {
  const int hf = lane >> 5, r32 = lane & 31;
  if constexpr (sizeof(T) == 2) {
    // transpose-read source lane: row 4*hf + (lane%16)/4 of each 16-row chunk, column 16*((lane/16)%2) + 4*(lane%4)
    const int trow = 4 * hf + ((lane & 15) >> 2);
    const int tcol = 16 * ((lane >> 4) & 1) + 4 * (lane & 3);
#pragma unroll
    for (int c = 0; c < 2; ++c) {
      u32x4 hi, lo;
      split_bf16x8(ds + 8 * c, hi, lo);
#pragma unroll
      for (int db = 0; db < DX / 32; ++db) {
        const char* p = xt + (sub * 32 + 16 * c + trow) * PX + (32 * db + tcol) * 2;
        const u32x2 p0 = lds_read_tr16(p), p1 = lds_read_tr16(p + 8 * PX);
        const u32x4 bop = {p0[0], p0[1], p1[0], p1[1]};
        mma_chunk<__bf16>(out[db], hi, bop);
        mma_chunk<__bf16>(out[db], lo, bop);
      }
    }
  } else {
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      const char* p = xt + (sub * 32 + acc_row(i, hf)) * PX + r32 * 4;
#pragma unroll
      for (int db = 0; db < DX / 32; ++db)
        out[db] = __builtin_amdgcn_mfma_f32_32x32x2f32(ds[i], *reinterpret_cast<const float*>(p + db * 128), out[db],
                                                        0, 0, 0);
    }
  }
}

// OWN_Q: the workgroup owns query rows and writes dQ; otherwise it owns key rows and writes dK.
// TEACHER: gradients of the teacher side (dQ_t / dK_t) instead of the student side.
template <typename T, int DT, int DS, bool CAUSAL, bool TEACHER, bool OWN_Q>
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(sizeof(T) == 2 ? 2 : 1, 2))) void bwd_kernel(
    const BwdArgs a) {
  constexpr int BW = BwdTile<T>::BW, BS = BwdTile<T>::BS, NT = BwdTile<T>::NT;
  constexpr int NSUB = BS / 32;
  constexpr int DX = TEACHER ? DT : DS;
  using Ring = TileRing<T, DT, DS, BS, NT>;
  constexpr int PT = Ring::PA, PS = Ring::PB;
  constexpr int STAT = OWN_Q ? 0 : 4 * BS * 4;  // streamed-query statistics (key-owner kernel)
  constexpr int SLOT = Ring::BYTES + STAT;
  extern __shared__ __attribute__((aligned(16))) char lds[];

  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6, hf = lane >> 5, r32 = lane & 31;
  const int nbh = a.B * a.H;
  const int n_own = OWN_Q ? a.Nq : a.Nk, n_str = OWN_Q ? a.Nk : a.Nq;
  const int nob = (n_own + BW - 1) / BW;
  const int bh = blockIdx.x % nbh;
  const int oi = blockIdx.x / nbh;
  // causal: the longest streams first (late query blocks for dQ, early key blocks for dK)
  const int ob = (CAUSAL && OWN_Q) ? (nob - 1 - oi) : oi;
  const int b = bh / a.H, h = bh % a.H;
  const int off = a.Nk - a.Nq;

  const T* qt = reinterpret_cast<const T*>(a.qt) + b * a.sqt[0] + h * a.sqt[1];
  const T* kt = reinterpret_cast<const T*>(a.kt) + b * a.skt[0] + h * a.skt[1];
  const T* qs = reinterpret_cast<const T*>(a.qs) + b * a.sqs[0] + h * a.sqs[1];
  const T* ks = reinterpret_cast<const T*>(a.ks) + b * a.sks[0] + h * a.sks[1];
  const T* own_t = OWN_Q ? qt : kt;
  const T* own_s = OWN_Q ? qs : ks;
  const T* str_t = OWN_Q ? kt : qt;
  const T* str_s = OWN_Q ? ks : qs;
  const int64_t own_pt = OWN_Q ? a.sqt[2] : a.skt[2], own_ps = OWN_Q ? a.sqs[2] : a.sks[2];
  const int64_t str_pt = OWN_Q ? a.skt[2] : a.sqt[2], str_ps = OWN_Q ? a.sks[2] : a.sqs[2];

  const int o0 = ob * BW;
  const int o0w = o0 + wave * 32;
  const int orow = o0w + r32;
  const bool ovalid = orow < n_own;
  u32x4 ot_r[DT * sizeof(T) / 32], os_r[DS * sizeof(T) / 32];
  load_row_regs<T, DT>(ot_r, own_t + (int64_t)orow * own_pt, ovalid, hf);
  load_row_regs<T, DS>(os_r, own_s + (int64_t)orow * own_ps, ovalid, hf);

  const float* lse_t_bh = a.lse_t + (int64_t)bh * a.Nq;
  const float* lse_s_bh = a.lse_s + (int64_t)bh * a.Nq;
  const float* g_bh = a.g + (int64_t)bh * a.Nq;
  const float* kl_bh = TEACHER ? a.kl + (int64_t)bh * a.Nq : nullptr;

  // query-owner: this lane's row statistics (log2 units), constant over the key stream
  float own_lt = 0.f, own_ls = 0.f, own_g = 0.f, own_c = 0.f;
  if constexpr (OWN_Q) {
    if (ovalid) {
      own_lt = lse_t_bh[orow] * kLog2e;
      own_ls = lse_s_bh[orow] * kLog2e;
      own_g = g_bh[orow];
      if constexpr (TEACHER) own_c = kl_bh[orow] + lse_t_bh[orow] - lse_s_bh[orow];
    }
  }

  // streamed range
  int t_begin, t_end;
  if constexpr (OWN_Q) {
    const int q_last = min(a.Nq, o0 + BW) - 1;
    const int kend = CAUSAL ? min(a.Nk, q_last + off + 1) : a.Nk;
    t_begin = 0;
    t_end = (kend + BS - 1) / BS;
  } else {
    const int qmin = CAUSAL ? max(0, o0 - off) : 0;  // first query that may see this block's first key
    t_begin = qmin / BS;
    t_end = (a.Nq + BS - 1) / BS;
  }

  Ring ring;
  ring.init(reinterpret_cast<const char*>(str_t), str_pt * (int64_t)sizeof(T), reinterpret_cast<const char*>(str_s),
            str_ps * (int64_t)sizeof(T), n_str, tid);
  // key-owner: per-tile statistics of the streamed queries, prefetched with the tile
  __amdgpu_buffer_rsrc_t r_lt, r_ls, r_g, r_kl;
  float pf_lt = 0.f, pf_ls = 0.f, pf_g = 0.f, pf_kl = 0.f;
  if constexpr (!OWN_Q) {
    r_lt = make_rsrc(lse_t_bh, (uint32_t)a.Nq * 4u);
    r_ls = make_rsrc(lse_s_bh, (uint32_t)a.Nq * 4u);
    r_g = make_rsrc(g_bh, (uint32_t)a.Nq * 4u);
    if constexpr (TEACHER) r_kl = make_rsrc(kl_bh, (uint32_t)a.Nq * 4u);
  }
  auto prefetch = [&](int t) {
    ring.prefetch(t * BS);
    if constexpr (!OWN_Q) {
      if (tid < BS) {
        const int so = t * BS * 4;
        pf_lt = __builtin_bit_cast(float, __builtin_amdgcn_raw_buffer_load_b32(r_lt, tid * 4, so, 0));
        pf_ls = __builtin_bit_cast(float, __builtin_amdgcn_raw_buffer_load_b32(r_ls, tid * 4, so, 0));
        pf_g = __builtin_bit_cast(float, __builtin_amdgcn_raw_buffer_load_b32(r_g, tid * 4, so, 0));
        if constexpr (TEACHER)
          pf_kl = __builtin_bit_cast(float, __builtin_amdgcn_raw_buffer_load_b32(r_kl, tid * 4, so, 0));
      }
    }
  };
  auto commit = [&](int t) {
    char* slot = lds + (t & 1) * SLOT;
    ring.commit(slot);
    if constexpr (!OWN_Q) {
      if (tid < BS) {
        float* st = reinterpret_cast<float*>(slot + Ring::BYTES);
        st[tid] = pf_lt * kLog2e;
        st[BS + tid] = pf_ls * kLog2e;
        st[2 * BS + tid] = pf_g;  // zero past the last query: those rows contribute nothing
        st[3 * BS + tid] = pf_kl + pf_lt - pf_ls;
      }
    }
  };

  f32x16 dacc[DX / 32];
#pragma unroll
  for (int db = 0; db < DX / 32; ++db) dacc[db] = f32x16{};

  if (t_begin < t_end) prefetch(t_begin);
  // (slot t&1 last held tile t-2, whose reads all finished before the barrier that published t-1)
  for (int t = t_begin; t < t_end; ++t) {
    commit(t);
    if (t + 1 < t_end) prefetch(t + 1);
    __syncthreads();
    const char* slot = lds + (t & 1) * SLOT;
    const char* tile_t = slot;
    const char* tile_s = slot + BS * PT;
    const float* stats = reinterpret_cast<const float*>(slot + Ring::BYTES);
#pragma unroll
    for (int sub = 0; sub < NSUB; ++sub) {
      const int sb = t * BS + sub * 32;  // first streamed row of this subtile
      // allowed(q, k): k <= q + off when causal; classify the 32 x 32 block of this wave
      bool skip, full;
      if constexpr (OWN_Q) {
        skip = sb >= n_str || (CAUSAL && sb > o0w + 31 + off);
        full = sb + 31 < n_str && (!CAUSAL || sb + 31 <= o0w + off);
      } else {
        skip = sb >= n_str || (CAUSAL && o0w > sb + 31 + off);
        full = sb + 31 < n_str && (!CAUSAL || o0w + 31 <= sb + off);
      }
      if (skip) continue;
      f32x16 st = {}, ss = {};
      tile_dot_lds_a<T, DT>(st, tile_t + (sub * 32 + r32) * PT, hf, ot_r);
      tile_dot_lds_a<T, DS>(ss, tile_s + (sub * 32 + r32) * PS, hf, os_r);
      float ds[16];
#pragma unroll
      for (int g4 = 0; g4 < 4; ++g4) {
        f32x4 lt4, ls4, gg4, cc4;
        if constexpr (OWN_Q) {
          lt4 = f32x4{own_lt, own_lt, own_lt, own_lt};
          ls4 = f32x4{own_ls, own_ls, own_ls, own_ls};
          gg4 = f32x4{own_g, own_g, own_g, own_g};
          cc4 = f32x4{own_c, own_c, own_c, own_c};
        } else {
          const int ql = sub * 32 + 8 * g4 + 4 * hf;
          lt4 = *reinterpret_cast<const f32x4*>(stats + ql);
          ls4 = *reinterpret_cast<const f32x4*>(stats + BS + ql);
          gg4 = *reinterpret_cast<const f32x4*>(stats + 2 * BS + ql);
          cc4 = TEACHER ? *reinterpret_cast<const f32x4*>(stats + 3 * BS + ql) : f32x4{};
        }
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const int i = 4 * g4 + e;
          const float pt = fast_exp2(fmaf(st[i], a.c_t, -lt4[e]));
          float v;
          if constexpr (TEACHER) {
            v = gg4[e] * pt * (scaled_diff(st[i], a.scale_t, ss[i], a.scale_s) - cc4[e]);
          } else {
            const float ps = fast_exp2(fmaf(ss[i], a.c_s, -ls4[e]));
            v = gg4[e] * (ps - pt);
          }
          if (!full) {
            const int sr = sb + acc_row(i, hf);
            const bool ok = sr < n_str && (!CAUSAL || (OWN_Q ? sr <= orow + off : orow <= sr + off));
            v = ok ? v : 0.f;
          }
          ds[i] = v;
        }
      }
      if constexpr (TEACHER)
        grad_product<T, DX, PT>(dacc, ds, tile_t, sub, lane);
      else
        grad_product<T, DX, PS>(dacc, ds, tile_s, sub, lane);
    }
  }

  const float scale = TEACHER ? a.scale_t : a.scale_s;
  float* out = (OWN_Q ? a.dq : a.dk) + (int64_t)bh * n_own * DX;
#pragma unroll
  for (int db = 0; db < DX / 32; ++db) {
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      const int r = o0w + acc_row(i, hf);
      if (r < n_own) out[(int64_t)r * DX + db * 32 + r32] = scale * dacc[db][i];
    }
  }
}

// ----------------------------------------------------------------------------------------------
template <typename T, int DT, int DS, bool C, bool TE, bool OWN_Q>
static hipError_t launch_bwd_t(const BwdArgs& a, hipStream_t s) {
  const int n_own = OWN_Q ? a.Nq : a.Nk;
  const int64_t nblk = (int64_t)((n_own + BwdTile<T>::BW - 1) / BwdTile<T>::BW) * a.B * a.H;
  if (nblk <= 0) return hipSuccess;
  if (nblk > 0x7fffffff) return hipErrorInvalidValue;
  constexpr int lds = bwd_lds_bytes<T, DT, DS, OWN_Q>();
  auto kern = bwd_kernel<T, DT, DS, C, TE, OWN_Q>;
  if (lds > 65536) {
    const hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void*>(kern),
                                             hipFuncAttributeMaxDynamicSharedMemorySize, lds);
    if (e != hipSuccess) return e;
  }
  hipLaunchKernelGGL(kern, dim3((unsigned)nblk), dim3(BwdTile<T>::NT), lds, s, a);
  return hipGetLastError();
}

template <bool OWN_Q, typename T, int DT, int DS>
static hipError_t bwd_ct(const BwdArgs& a, bool causal, bool teacher, hipStream_t s) {
  if (causal)
    return teacher ? launch_bwd_t<T, DT, DS, true, true, OWN_Q>(a, s) : launch_bwd_t<T, DT, DS, true, false, OWN_Q>(a, s);
  return teacher ? launch_bwd_t<T, DT, DS, false, true, OWN_Q>(a, s) : launch_bwd_t<T, DT, DS, false, false, OWN_Q>(a, s);
}

template <bool OWN_Q, typename T>
static hipError_t bwd_d(const BwdArgs& a, int dt, int ds, bool causal, bool teacher, hipStream_t s) {
  if (dt == 128 && ds == 128) return bwd_ct<OWN_Q, T, 128, 128>(a, causal, teacher, s);
  if (dt == 128 && ds == 64) return bwd_ct<OWN_Q, T, 128, 64>(a, causal, teacher, s);
  if (dt == 64 && ds == 128) return bwd_ct<OWN_Q, T, 64, 128>(a, causal, teacher, s);
  if (dt == 64 && ds == 64) return bwd_ct<OWN_Q, T, 64, 64>(a, causal, teacher, s);
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
