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
// Schedule: 32-key tiles reach LDS by buffer->LDS DMA into a 3-slot ring, two
// tiles ahead, one barrier per tile; three workgroups share a CU, so while one
// wavefront waits on its MFMAs the others run their exp/VALU work.  Keys a row
// may not see (causal diagonal, ragged end) are set to -inf in the logit tile
// under a wave-uniform branch, then every tile takes the same update.
#pragma once

#include "skl_device.hpp"
#include "skl_kernels.hpp"
#include <type_traits>

namespace skl {

// LDS operand reads in flight ahead of the logit MFMAs (bf16)
#ifndef FWD_LA
#define FWD_LA 4
#endif

template <typename T>
struct FwdTile {
  static constexpr int BQ = 128;  // query rows per workgroup (4 wavefronts x 32)
  static constexpr int BK = 32;   // keys per LDS tile (one 32 x 32 logit block per wavefront)
  static constexpr int NBUF = 3;  // LDS ring depth: tiles t+1 and t+2 are in flight while t is used
  static constexpr int NT = 256;
};

// Per-lane running state of one query row over the keys this lane half sees.
struct RowState {
  float m_t, m_s;  // running maxima in log2 units (logit * scale * log2 e)
  float l_t, l_s, acc;
};

// max(a, b, c) as one v_max3_f32.  Logits here are finite or -inf, never NaN, so the NaN
// quieting the compiler puts in front of fmaxf (one extra VALU op per operand that is not
// known to be quiet, such as an MFMA result) is not needed.
__device__ __forceinline__ float max3(float a, float b, float c) {
  float r;
  asm("v_max3_f32 %0, %1, %2, %3" : "=v"(r) : "v"(a), "v"(b), "v"(c));
  return r;
}

// Online update with one 32-key subtile: st/ss are the raw (unscaled) logits of this
// lane's 16 keys; masked keys are -inf in st/ss, dif = (a - b) / scale_t is finite.
__device__ __forceinline__ void online_update(RowState& s, const f32x16& st, const f32x16& ss, const float* dif,
                                              float c_t, float c_s) {
  float mx = max3(st[0], st[1], st[2]), my = max3(ss[0], ss[1], ss[2]);
#pragma unroll
  for (int i = 3; i < 15; i += 2) {
    mx = max3(mx, st[i], st[i + 1]);
    my = max3(my, ss[i], ss[i + 1]);
  }
  mx = max3(mx, st[15], mx);
  my = max3(my, ss[15], my);
  const float mt_new = max3(s.m_t, mx * c_t, s.m_t);
  const float ms_new = max3(s.m_s, my * c_s, s.m_s);
  const float al_t = fast_exp2(s.m_t - mt_new);
  const float al_s = fast_exp2(s.m_s - ms_new);
  s.m_t = mt_new;
  s.m_s = ms_new;
  // partial sums of this subtile, started from its first key
  float pt = fast_exp2(fmaf(st[0], c_t, -mt_new));
  float ps = fast_exp2(fmaf(ss[0], c_s, -ms_new));
  float pa = pt * dif[0];
#pragma unroll
  for (int i = 1; i < 16; ++i) {
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

// The same sums against a power-of-two reference instead of the running maximum: m_t, m_s hold
// integers, every exponent is taken relative to them, and every third tile ref_renorm moves the
// binary exponent of l into m (exact: a power-of-two scaling of l and acc).  No per-element maximum
// and no per-tile rescaling exps are needed.  It stays finite as long as no logit (log2 units)
// exceeds the reference by ~120, and keeps full precision unless a sum falls near the denormals;
// the kernel checks both at the end and reruns the tile loop with online_update when either fails.
__device__ __forceinline__ void ref_update(RowState& s, const f32x16& st, const f32x16& ss, const float* dif, float c_t,
                                           float c_s) {
  float pt = fast_exp2(fmaf(st[0], c_t, -s.m_t));
  float ps = fast_exp2(fmaf(ss[0], c_s, -s.m_s));
  float pa = pt * dif[0];
#pragma unroll
  for (int i = 1; i < 16; ++i) {
    const float e = fast_exp2(fmaf(st[i], c_t, -s.m_t));
    const float f = fast_exp2(fmaf(ss[i], c_s, -s.m_s));
    pt += e;
    ps += f;
    pa = fmaf(e, dif[i], pa);
  }
  s.l_t += pt;
  s.l_s += ps;
  s.acc += pa;
}

// l = l' 2^e with l' in [0.5, 1): m += e (0 sums keep e = 0); emin tracks the smallest e seen.
__device__ __forceinline__ void ref_renorm(RowState& s, int& emin) {
  const int et = __builtin_amdgcn_frexp_expf(s.l_t), es = __builtin_amdgcn_frexp_expf(s.l_s);
  s.l_t = __builtin_amdgcn_ldexpf(s.l_t, -et);
  s.acc = __builtin_amdgcn_ldexpf(s.acc, -et);
  s.l_s = __builtin_amdgcn_ldexpf(s.l_s, -es);
  s.m_t += (float)et;
  s.m_s += (float)es;
  emin = min(emin, min(et, es));
}

// Equal scales (s_t = s_s = s, so one c = s log2 e for both sides): the second MFMA chain continues
// from the teacher logits with the student queries negated, so it yields dd = q_t.k_t - q_s.k_s, the
// raw logit difference, and no per-element product forms it.  Both sides share one power-of-two
// reference m: x = c st - m, y = x - c dd = c ss - m, and acc sums e dd.  Per element: two exponent
// FMAs, two exp2, two sums and the accumulator FMA.
__device__ __forceinline__ void ref_update_eq(RowState& s, const f32x16& st, const f32x16& dd, float c) {
  float x = fmaf(st[0], c, -s.m_t);
  float pt = fast_exp2(x);
  float ps = fast_exp2(fmaf(dd[0], -c, x));
  float pa = pt * dd[0];
#pragma unroll
  for (int i = 1; i < 16; ++i) {
    x = fmaf(st[i], c, -s.m_t);
    const float e = fast_exp2(x);
    const float f = fast_exp2(fmaf(dd[i], -c, x));
    pt += e;
    ps += f;
    pa = fmaf(e, dd[i], pa);
  }
  s.l_t += pt;
  s.l_s += ps;
  s.acc += pa;
}

// The shared reference moves to the binary exponent of the larger sum (exact scalings); emin tracks
// the smallest exponent either sum had against the old reference (a sum near the denormals).  A side
// that sinks far below the other is caught at the end of the loop, where the smaller sum must stay
// within 2^-100 of the larger one (ref_gap_bad).
__device__ __forceinline__ void ref_renorm_eq(RowState& s, int& emin) {
  const int et = __builtin_amdgcn_frexp_expf(s.l_t), es = __builtin_amdgcn_frexp_expf(s.l_s);
  const int e = max(et, es);
  s.l_t = __builtin_amdgcn_ldexpf(s.l_t, -e);
  s.acc = __builtin_amdgcn_ldexpf(s.acc, -e);
  s.l_s = __builtin_amdgcn_ldexpf(s.l_s, -e);
  s.m_t += (float)e;
  s.m_s = s.m_t;
  emin = min(emin, min(et, es));
}

// End of the loop with a shared reference (the loop ends on a renormalisation, so the larger sum is in
// [0.5, 1)): a smaller sum below 2^-100 of it, or at zero, has lost its precision in this lane half,
// even where the merged row (the other half) looks normal.  Without this test a row of three tiles or
// fewer, whose only renormalisation leaves the student's sum a denormal, came out as -inf.
__device__ __forceinline__ bool ref_gap_bad(const RowState& s) {
  return fmaxf(s.l_t, s.l_s) > 0.f && fminf(s.l_t, s.l_s) < 0x1p-100f;
}

// Jensen-Shannon pass (second pass over the keys, with both log-sum-exps known from the KL
// forward).  Per row, with x = log2 P_t, y = log2 P_s, r = y - x and M = (P_t + P_s)/2:
//   log2(P_t/M) = w - max(r, 0),  log2(P_s/M) = w + min(r, 0),  w = 1 - log2(1 + 2^-|r|),
// which stays accurate when the two rows nearly agree (r near 0) and never forms log2 M itself.
// Each lane half sums P_t log2(P_t/M) and P_s log2(P_s/M) over its keys.
struct JsState {
  float at, as;
};

__device__ __forceinline__ void js_update(JsState& s, const f32x16& st, const f32x16& ss, float lt, float ls, float c_t,
                                          float c_s) {
  float at = 0.f, as = 0.f;
#pragma unroll
  for (int i = 0; i < 16; ++i) {
    const float x = fmaf(st[i], c_t, -lt), y = fmaf(ss[i], c_s, -ls);
    const float p = fast_exp2(x), q = fast_exp2(y);
    const float r = y - x;
    const float lp = (1.f - fast_log2(1.f + fast_exp2(-fabsf(r)))) - fmaxf(r, 0.f);  // log2(P_t/M)
    at = fmaf(p, lp, at);
    as = fmaf(q, lp + r, as);  // log2(P_s/M) = log2(P_t/M) + r
  }
  s.at += at;
  s.as += as;
}

// JS: the Jensen-Shannon pass instead of the KL forward (lse_t, lse_s are read; kl receives JS and
// js_t the teacher half KL(P_t || M)).  EQ (KL forward, bf16, scale_t == scale_s): the logit
// difference comes from the second MFMA chain (see ref_update_eq).
template <typename T, int DT, int DS, bool CAUSAL, bool JS, bool EQ>
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(sizeof(T) == 2 ? 3 : 1, 3))) void fwd_kernel(
    const FwdArgs a) {
  constexpr int BQ = FwdTile<T>::BQ, BK = FwdTile<T>::BK, NBUF = FwdTile<T>::NBUF, NT = FwdTile<T>::NT;
  constexpr int RBT = DT * (int)sizeof(T), RBS = DS * (int)sizeof(T);  // row bytes
  constexpr int TILE = BK * (RBT + RBS);                                  // one K_t + K_s tile
  constexpr int NCT = RBT / 16, NCS = RBS / 16;                           // 16-byte chunks per row
  using DmaT = DmaTile<BK, RBT, NT>;
  using DmaS = DmaTile<BK, RBS, NT>;
  constexpr int NI = DmaT::NI + DmaS::NI;  // DMA instructions per thread per tile
  // one array per ring slot: distinct objects let the compiler see that a DMA into one slot never
  // aliases reads of another, so it adds no wait beyond the explicit ones below
  __shared__ __attribute__((aligned(1024))) char slot0[TILE], slot1[TILE], slot2[TILE];
  static_assert(NBUF == 3, "one named array per ring slot");

  const int tid = threadIdx.x, lane = tid & 63, hf = lane >> 5, r32 = lane & 31;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);  // scalar: per-wave tests branch on SCC
  const int nbh = a.B * a.H;
  const int nqb = (a.mq + BQ - 1) / BQ;
  // Workgroups go to the eight XCDs round-robin (workgroup i to XCD i mod 8), each XCD with its own
  // L2.  When the grid splits evenly, XCD x takes the x-th eighth of the (head, query block) list in
  // order, so the workgroups resident on one XCD are query blocks of one head that read the same key
  // tiles from that L2 (each head's blocks still longest first); otherwise heads are interleaved.
  // Within an XCD the workgroups go to its CUs round-robin (position j to CU j mod the XCD's CUs), so
  // in a small grid with two workgroups per CU whose eighth holds whole heads, positions j and j + S/2
  // share a CU: with `fold`, the first half goes out longest first across the heads and the second
  // half shortest first, so each CU's two query blocks hold about the same number of key tiles
  // (head by head, causal, the CU of position 0 held the two longest).
  // Split (a.part): a head has nqb + nsb units, longest first: units 2i and 2i + 1 are the two key
  // halves of query block nqb-1-i (i < nsb), then come the whole blocks qsplit-1 .. 0.  Three
  // workgroups share a CU, at positions j, j + cpx and j + 2 cpx of the XCD's share: the share's units
  // are ranked by length across its heads and dealt out in a serpentine (ranks j, 2 cpx - 1 - j,
  // 2 cpx + j), so each CU mixes long and short units.
  const bool split = CAUSAL && !JS && a.part != nullptr && a.qsplit < nqb;
  const int nsb = split ? nqb - a.qsplit : 0;  // split blocks per head
  const int nun = nqb + nsb;                   // units per head
  const int nblk = (int)gridDim.x;
  const int S8 = nblk / 8, j8 = (int)(blockIdx.x / 8);
  int pos = j8;  // position in the XCD's eighth, head-major
  if (split) {
    if (S8 % nun == 0 && a.cpx > 0 && S8 % a.cpx == 0) {
      const int hs = S8 / nun;  // whole heads in the eighth
      const int k = j8 / a.cpx, r = j8 % a.cpx;
      const int rank = k * a.cpx + ((k & 1) ? a.cpx - 1 - r : r);
      pos = (rank % hs) * nun + rank / hs;
    }
  } else if (a.fold && S8 % nqb == 0 && S8 % 2 == 0) {
    const int hs = S8 / nqb;                                     // whole heads in the eighth
    const int pp = j8 < S8 / 2 ? j8 : (S8 + S8 / 2 - 1 - j8);  // rank by length
    pos = (pp % hs) * nqb + pp / hs;
  }
  const int L = (int)(blockIdx.x % 8) * S8 + pos;
  const bool xcd = nblk % 8 == 0;
  const int bh = xcd ? L / nun : blockIdx.x % nbh;
  const int ui = xcd ? L % nun : blockIdx.x / nbh;  // unit of the head
  int qi = ui, part = -1;                          // part: which key half of a split block, -1 whole
  if (split) {
    if (ui < 2 * nsb) {
      qi = ui / 2;
      part = ui % 2;
    } else {
      qi = ui - nsb;
    }
  }
  const int qb = CAUSAL ? (nqb - 1 - qi) : qi;  // causal: longest rows first
  const int b = bh / a.H, h = bh % a.H;
  const Segment sg = segment_of(a, b);
  const int nq = sg.nq, nk = sg.nk;
  const int q0 = qb * BQ;
  if (q0 >= nq) return;  // past the end of a shorter segment of a packed batch (whole workgroup)
  const int off = nk - nq;

  const T* qt = reinterpret_cast<const T*>(a.qt) + sg.bs * a.sqt[0] + h * a.sqt[1] + sg.q0 * a.sqt[2];
  // grouped-query attention: query head h reads key head h / g of each side
  const char* kt = reinterpret_cast<const char*>(reinterpret_cast<const T*>(a.kt) + sg.bs * a.skt[0] +
                                                 (h / a.gt) * a.skt[1] + sg.k0 * a.skt[2]);
  const T* qs = reinterpret_cast<const T*>(a.qs) + sg.bs * a.sqs[0] + h * a.sqs[1] + sg.q0 * a.sqs[2];
  const char* ks = reinterpret_cast<const char*>(reinterpret_cast<const T*>(a.ks) + sg.bs * a.sks[0] +
                                                 (h / a.gs) * a.sks[1] + sg.k0 * a.sks[2]);
  const int64_t kt_pitch = a.skt[2] * (int64_t)sizeof(T), ks_pitch = a.sks[2] * (int64_t)sizeof(T);

  const int q0w = q0 + wave * 32;
  const int qrow = q0w + r32;
  u32x4 qt_r[NCT / 2], qs_r[NCS / 2];
  load_row_regs<T, DT>(qt_r, qt + (int64_t)qrow * a.sqt[2], qrow < nq, hf);
  load_row_regs<T, DS>(qs_r, qs + (int64_t)qrow * a.sqs[2], qrow < nq, hf);
  static_assert(!EQ || (!JS && sizeof(T) == 2), "the difference chain serves the bf16 KL forward");
  if constexpr (EQ) {  // -q_s: flip the sign bit of both bf16 halves of every word (exact)
#pragma unroll
    for (int c = 0; c < NCS / 2; ++c) qs_r[c] ^= u32x4{0x80008000u, 0x80008000u, 0x80008000u, 0x80008000u};
  }

  constexpr int KL_FAST = 0, KL_EXACT = 1, JS_PASS = 2;  // modes of the tile loop
  RowState rs{kMaxInit, kMaxInit, 0.f, 0.f, 0.f};
  JsState js{0.f, 0.f};
  auto stat_index = [&]() -> int64_t { return ((int64_t)sg.bs * a.H + h) * a.Nq + sg.q0 + qrow; };  // row statistics
  float js_lt = 0.f, js_ls = 0.f;  // JS: the row's log-sum-exps in log2 units
  if constexpr (JS) {
    if (qrow < nq) {
      js_lt = a.lse_t[stat_index()] * kLog2e;
      js_ls = a.lse_s[stat_index()] * kLog2e;
    }
  }

  const int q_last = min(nq, q0 + BQ) - 1;
  const int kend = CAUSAL ? min(nk, q_last + off + 1) : nk;
  const int nt_all = max(kend + BK - 1, 0) / BK;  // 0 only for rows with no key (an invalid segment)
  // key tiles tb .. tb + ntiles - 1 (a half of a split block: the first or the rest); keys from klim
  // on belong to the other half
  const int tb = part == 1 ? nt_all / 2 : 0;
  const int ntiles = part == 0 ? nt_all / 2 : nt_all - tb;
  const int klim = min(nk, (tb + ntiles) * BK);

  // K tiles: buffer->LDS DMA (zero past the last key) into a NBUF-deep ring, two tiles ahead
  const u32x4 rk_t = rsrc_words(kt, nk > 0 ? (uint32_t)((nk - 1) * kt_pitch + RBT) : 0u);
  const u32x4 rk_s = rsrc_words(ks, nk > 0 ? (uint32_t)((nk - 1) * ks_pitch + RBS) : 0u);
  DmaT dma_t;
  DmaS dma_s;
  dma_t.init(kt_pitch, wave, lane);
  dma_s.init(ks_pitch, wave, lane);
  auto slot_ptr = [&](int slot) -> char* { return slot == 0 ? slot0 : (slot == 1 ? slot1 : slot2); };
  auto issue = [&](int tile, int slot) {
    const bool whole = (tile + 1) * BK <= nk;
    const uint32_t dst = slot == 0 ? lds_addr(slot0) : (slot == 1 ? lds_addr(slot1) : lds_addr(slot2));
    dma_t.issue(rk_t, tile * BK * (int)kt_pitch, whole, dst, wave);
    dma_s.issue(rk_s, tile * BK * (int)ks_pitch, whole, dst + BK * RBT, wave);
  };
  // this lane's operand chunk offsets (row r32 of a tile), loop-invariant
  int off_t[NCT / 2], off_s[NCS / 2];
  swz_operand_offsets<RBT, NCT / 2>(off_t, r32, hf);
  swz_operand_offsets<RBS, NCS / 2>(off_s, r32, hf);

  // The tile loop, for one mode: KL_FAST (ref_update), KL_EXACT (online_update) or JS_PASS.
  int emin = 0;
  auto tile_loop = [&](auto mode_tag) {
    constexpr int MODE = decltype(mode_tag)::value;
    // The compiler cannot see the DMAs in the hardware's vmcnt; retire every load of its own now,
    // so that none of its waits lands inside the loop, where it would also drain the DMA ring.
    wait_vmcnt<0>();
    issue(tb, 0);
    issue(tb + 1, 1);  // past the last tile a DMA returns zeros into a slot nobody reads
    // One step per tile; the loop is unrolled by the ring depth so every LDS address is a
    // per-lane base plus an immediate.  The tile count is rounded up to a multiple of the ring
    // depth: the extra tiles lie past every row's last key, so they are fully masked and leave the
    // state unchanged, and the unrolled body needs no guard (whose join would copy the state).
    const int ntiles_pad = (ntiles + NBUF - 1) / NBUF * NBUF;
    for (int t0 = 0; t0 < ntiles_pad; t0 += NBUF) {
#pragma unroll
      for (int u = 0; u < NBUF; ++u) {
        const int t = t0 + u;
        {
          wait_vmcnt<NI>();  // tile t has landed (tile t+1 may still be in flight)
          __syncthreads();   // ... for every wave; and every wave is done with tile t-1
          issue(tb + t + 2, (u + 2) % NBUF);  // into the slot that held tile t-1
          const char* tile = slot_ptr(u);
          const int kb = (tb + t) * BK;
          f32x16 st = {}, ss = {};
          if constexpr (EQ) {
            // ss holds dd = st - q_s.k_s: the student chain starts from the finished teacher logits
            tile_dot_swz<T, DT>(st, tile, off_t, qt_r);
            ss = st;
            tile_dot_swz<T, DS>(ss, tile + BK * RBT, off_s, qs_r);
            sched_read_ahead<(RBT + RBS) / 32, FWD_LA>();
          } else {
            // both chains interleaved, each operand read issued a few MFMAs ahead of its use: with the
            // reads one MFMA ahead each MFMA waited out an LDS latency, and the logit phase of a wave
            // took several times its matrix cycles
            tile_dot2_swz<T, DT, DS>(st, ss, tile, tile + BK * RBT, off_t, off_s, qt_r, qs_r);
            if constexpr (sizeof(T) == 2) sched_read_ahead<(RBT + RBS) / 32, FWD_LA>();
          }
          float dif[16];  // (a - b) / scale_t, taken before masking so masked entries stay finite
          if constexpr (!JS && !EQ) {
#pragma unroll
            for (int i = 0; i < 16; ++i) {
              dif[i] = fmaf(ss[i], -a.ratio, st[i]);
              // pin dif here, ahead of the masking branch: then no unmasked logit outlives the branch
              // and the masking below rewrites st/ss in place instead of copying them on every tile
              asm volatile("" : "+v"(dif[i]));
            }
          }
          // A tile that no row of this wavefront reaches (causal) goes through the masked path too:
          // with every key at -inf the update leaves the state bit for bit unchanged, and the loop
          // keeps one definition of the state (no copies at a join).  Such tiles are under 1% of
          // a causal problem's.
          const bool full = t < ntiles && kb + 31 < klim && (!CAUSAL || kb + 31 <= q0w + off);
          if (!full) {  // in place, so the update below has one copy of its state
            asm volatile("");  // keep this a branch: the compiler would otherwise select on every tile
#pragma unroll
            for (int i = 0; i < 16; ++i) {
              const int key = kb + acc_row(i, hf);
              const bool ok = key < klim && (!CAUSAL || key <= qrow + off);
              // JS: a large finite logit instead of -inf gives P_t = P_s = 0 with a finite r, so
              // the term is an exact zero rather than 0 * NaN
              st[i] = ok ? st[i] : (JS ? -1e30f : -INFINITY);
              if constexpr (!EQ) ss[i] = ok ? ss[i] : (JS ? -1e30f : -INFINITY);  // EQ: dd stays finite
            }
          }
          if constexpr (MODE == JS_PASS) {
            js_update(js, st, ss, js_lt, js_ls, a.c_t, a.c_s);
            asm volatile("" ::"v"(js.at), "v"(js.as));
          } else {
            if constexpr (MODE == KL_FAST && EQ) {
              ref_update_eq(rs, st, ss, a.c_t);
              if (u == NBUF - 1) ref_renorm_eq(rs, emin);
            } else if constexpr (MODE == KL_FAST) {
              ref_update(rs, st, ss, dif, a.c_t, a.c_s);
              if (u == NBUF - 1) ref_renorm(rs, emin);
            } else if constexpr (EQ) {  // the exact rerun takes the student logits back from dd
              f32x16 sl;
#pragma unroll
              for (int i = 0; i < 16; ++i) {
                sl[i] = st[i] - ss[i];
                dif[i] = ss[i];
              }
              online_update(rs, st, sl, dif, a.c_t, a.c_s);
            } else {
              online_update(rs, st, ss, dif, a.c_t, a.c_s);
            }
            // the new state exists before the next barrier: keeps each tile's update in its own step
            asm volatile("" ::"v"(rs.m_t), "v"(rs.m_s), "v"(rs.l_t), "v"(rs.l_s), "v"(rs.acc));
          }
        }
      }
    }
    wait_vmcnt<0>();  // no DMA may still target this workgroup's LDS when it exits (or is refilled)
  };

  if constexpr (JS) {
    tile_loop(std::integral_constant<int, JS_PASS>{});
    const float at = js.at + __shfl_xor(js.at, 32), as = js.as + __shfl_xor(js.as, 32);
    if (hf == 0 && qrow < nq) {
      a.kl[stat_index()] = 0.5f * kLn2 * (at + as);
      a.js_t[stat_index()] = kLn2 * at;
    }
    return;
  }

  // Merge the two half-row states (disjoint key subsets) of each query row; the references m are
  // running maxima or powers of two, the merge is the same.
  float Mt, Ms, Lt, Ls, A;
  auto merge = [&]() {
    const float o_mt = __shfl_xor(rs.m_t, 32), o_lt = __shfl_xor(rs.l_t, 32), o_acc = __shfl_xor(rs.acc, 32);
    const float o_ms = __shfl_xor(rs.m_s, 32), o_ls = __shfl_xor(rs.l_s, 32);
    Mt = fmaxf(rs.m_t, o_mt);
    Ms = fmaxf(rs.m_s, o_ms);
    const float f1 = fast_exp2(rs.m_t - Mt), f2 = fast_exp2(o_mt - Mt);
    const float g1 = fast_exp2(rs.m_s - Ms), g2 = fast_exp2(o_ms - Ms);
    Lt = rs.l_t * f1 + o_lt * f2;
    Ls = rs.l_s * g1 + o_ls * g2;
    A = rs.acc * f1 + o_acc * f2;
  };
  rs = RowState{0.f, 0.f, 0.f, 0.f, 0.f};  // power-of-two references start at 2^0
  tile_loop(std::integral_constant<int, KL_FAST>{});
  const bool half_bad = EQ && ref_gap_bad(rs);  // this lane half's own sums, before the merge
  merge();
  // A row whose sums left the safe range (an overflow, or a sum that came near the denormals) is
  // redone by the whole workgroup with running maxima; realistic logits never get there.
  const bool risky = half_bad || !(__builtin_isfinite(Lt) && __builtin_isfinite(Ls) && __builtin_isfinite(A)) ||
                     emin < -100 || (qrow < nq && (Lt == 0.f || Ls == 0.f));
  if (__syncthreads_or(risky)) {
    rs = RowState{kMaxInit, kMaxInit, 0.f, 0.f, 0.f};
    tile_loop(std::integral_constant<int, KL_EXACT>{});
    merge();
  }

  if (part >= 0) {  // a half of a split block: its row states go to the workspace (fwd_merge_kernel)
    if (hf == 0 && qrow < nq) {
      float* ps = a.part + ((int64_t)(bh * nsb + qb - a.qsplit) * 2 + part) * 5 * BQ + (qrow - q0);
      ps[0] = Mt;
      ps[BQ] = Ms;
      ps[2 * BQ] = Lt;
      ps[3 * BQ] = Ls;
      ps[4 * BQ] = A;
    }
    return;
  }
  if (hf == 0 && qrow < nq) {
    // true divisions: Ls / Lt is exactly 1 when the two states are bitwise equal
    const int64_t o = stat_index();
    a.kl[o] = a.scale_t * (A / Lt) + kLn2 * ((Ms - Mt) + fast_log2(Ls / Lt));
    a.lse_t[o] = kLn2 * (Mt + fast_log2(Lt));
    a.lse_s[o] = kLn2 * (Ms + fast_log2(Ls));
  }
}

// Rows of the split query blocks (dense batch): the two halves' row states (fwd_kernel, in part),
// merged in a fixed order (first half, then second) and closed as fwd_kernel closes a row.  One
// thread per row; nsb split blocks per head.
template <int bq>
__global__ __launch_bounds__(256) void fwd_merge_kernel(const FwdArgs a, int nsb) {
  const int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;  // (head, split block, row)
  if (i >= (int64_t)a.B * a.H * nsb * bq) return;
  const int r = (int)(i % bq);
  const int64_t u = i / bq;  // head * nsb + split block
  const int q = (a.qsplit + (int)(u % nsb)) * bq + r;
  if (q >= a.Nq) return;
  const float* p0 = a.part + u * 2 * 5 * bq + r;
  const float* p1 = p0 + 5 * bq;
  const float Mt = fmaxf(p0[0], p1[0]), Ms = fmaxf(p0[bq], p1[bq]);
  const float f0 = fast_exp2(p0[0] - Mt), f1 = fast_exp2(p1[0] - Mt);
  const float g0 = fast_exp2(p0[bq] - Ms), g1 = fast_exp2(p1[bq] - Ms);
  const float Lt = p0[2 * bq] * f0 + p1[2 * bq] * f1;
  const float Ls = p0[3 * bq] * g0 + p1[3 * bq] * g1;
  const float A = p0[4 * bq] * f0 + p1[4 * bq] * f1;
  const int64_t o = (u / nsb) * a.Nq + q;
  a.kl[o] = a.scale_t * (A / Lt) + kLn2 * ((Ms - Mt) + fast_log2(Ls / Lt));
  a.lse_t[o] = kLn2 * (Mt + fast_log2(Lt));
  a.lse_s[o] = kLn2 * (Ms + fast_log2(Ls));
}

// ----------------------------------------------------------------------------------------------
template <bool JS, typename T, int DT, int DS, bool C>
static hipError_t launch_fwd_t(const FwdArgs& args, hipStream_t s) {
  constexpr int BQ = FwdTile<T>::BQ;
  FwdArgs a = args;
  const int64_t nqb = (a.mq + BQ - 1) / BQ;
  // split key halves: causal dense KL forward only, from query block qsplit >= 1 on
  const bool split = C && !JS && a.part != nullptr && a.cu_q == nullptr && a.qsplit >= 1 && a.qsplit < nqb;
  if (!split) a.part = nullptr;
  const int64_t nsb = split ? nqb - a.qsplit : 0;
  const int64_t nblk = (nqb + nsb) * a.B * a.H;
  if (nblk <= 0) return hipSuccess;
  if (nblk > 0x7fffffff) return hipErrorInvalidValue;
  if constexpr (!JS && sizeof(T) == 2) {
    if (a.c_t == a.c_s && a.eq_ok) {
      hipLaunchKernelGGL((fwd_kernel<T, DT, DS, C, false, true>), dim3((unsigned)nblk), dim3(FwdTile<T>::NT), 0, s,
                         a);
    } else {
      hipLaunchKernelGGL((fwd_kernel<T, DT, DS, C, false, false>), dim3((unsigned)nblk), dim3(FwdTile<T>::NT), 0, s,
                         a);
    }
  } else {
    hipLaunchKernelGGL((fwd_kernel<T, DT, DS, C, JS, false>), dim3((unsigned)nblk), dim3(FwdTile<T>::NT), 0, s, a);
  }
  hipError_t e = hipGetLastError();
  if (e != hipSuccess || !split) return e;
  const int64_t rows = (int64_t)a.B * a.H * nsb * BQ;
  hipLaunchKernelGGL(fwd_merge_kernel<BQ>, dim3((unsigned)((rows + 255) / 256)), dim3(256), 0, s, a, (int)nsb);
  return hipGetLastError();
}

template <bool JS, typename T, int DT, int DS>
static hipError_t fwd_c(const FwdArgs& a, bool causal, hipStream_t s) {
  return causal ? launch_fwd_t<JS, T, DT, DS, true>(a, s) : launch_fwd_t<JS, T, DT, DS, false>(a, s);
}

template <bool JS, typename T>
static hipError_t fwd_d(const FwdArgs& a, int dt, int ds, bool causal, hipStream_t s) {
  if (dt == 128 && ds == 128) return fwd_c<JS, T, 128, 128>(a, causal, s);
  if (dt == 128 && ds == 64) return fwd_c<JS, T, 128, 64>(a, causal, s);
  if (dt == 64 && ds == 128) return fwd_c<JS, T, 64, 128>(a, causal, s);
  if (dt == 64 && ds == 64) return fwd_c<JS, T, 64, 64>(a, causal, s);
  return hipErrorInvalidValue;
}

// Launch the forward kernel (JS: its Jensen-Shannon pass).  dtype: 0 fp32, 1 bf16.
template <bool JS>
static hipError_t fwd_dispatch(const FwdArgs& a, int dtype, int dt, int ds, bool causal, hipStream_t s) {
  if (dtype == 1) return fwd_d<JS, __bf16>(a, dt, ds, causal, s);
  if (dtype == 0) return fwd_d<JS, float>(a, dt, ds, causal, s);
  return hipErrorInvalidValue;
}

}  // namespace skl
