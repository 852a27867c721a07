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
// One kernel template serves both halves.  Each wave owns 32 rows of the output
// (query rows for dQ, key rows for dK) and keeps their Q or K slices in registers
// as MFMA B operands; the other side streams through a 4-slot LDS ring filled by
// buffer->LDS DMA.  Owning the output rows means no atomics (grouped key heads
// may add a caller workspace of partial dK, summed in a fixed order).  Both halves
// recompute both logit tiles.
//
// The logit tile is formed with the owned rows as columns, so each lane holds 16
// streamed rows of one owned row; that register block is directly the A operand
// of the gradient product (contraction over the streamed rows).  The B operand,
// the streamed tile read with the streamed rows as the contraction index, comes
// from the LDS tile through transpose reads, so no transposed copy is stored.
// bf16 inputs: dS enters the MFMA rounded once to fp16 at a power-of-two scale
// against an fp16 copy of the streamed tile (2^-11 relative), or, for inputs
// outside that product's range, as hi + lo bf16 parts (two products, about 2^-16)
// instead of bf16's 2^-9.
//
// Per streamed tile s a wave runs a matrix phase, M(s) = gradient product of
// tile s-1 then the two logit products of tile s, and a vector phase, V(s) = the
// probabilities and dS of tile s.  bf16 workgroups have eight waves in two
// groups, one wave of each group per SIMD, working in periods that end at a
// workgroup barrier: in period s group 0 runs M(s) then V(s), group 1 V(s-1) then
// M(s), so on every SIMD one wave is in its matrix phase while the other is in
// its vector phase (ping-pong) and the matrix cores and the vector ALUs work at
// the same time; within a period each wave goes on to its second phase as soon
// as its first is done.
#pragma once

#include "skl_device.hpp"
#include "skl_kernels.hpp"
#include <type_traits>

namespace skl {

// a * sa - b * sb with both products rounded before the subtraction (no FMA contraction), so the
// result is exactly 0 when (a, sa) == (b, sb): identical teacher and student give zero gradients.
__device__ __forceinline__ float scaled_diff(float a, float sa, float b, float sb) {
#pragma clang fp contract(off)
  return a * sa - b * sb;
}

template <typename T>
struct BwdTile {
  static constexpr int NG = sizeof(T) == 2 ? 2 : 1;  // wave groups (two: ping-pong)
  static constexpr int NW = 4 * NG;                  // waves per workgroup
  static constexpr int NT = 64 * NW;
  static constexpr int BW = 32 * NW;  // owned rows per workgroup (32 per wave)
  static constexpr int BS = 32;       // streamed rows per LDS tile
  // LDS ring: tile s is read in phases 2s..2s+3 (ping-pong) or in step s (one group), while the
  // next PD = NBUF - 2 tiles are in flight
  static constexpr int NBUF = 4;
  static constexpr int PD = NBUF - 2;
  static_assert(BW == (sizeof(T) == 2 ? kBwdRowsBf16 : kBwdRowsF32), "rows per workgroup known to the launcher");
};

// dS of one 32 x 32 tile in the accumulator layout, kept from a vector phase to the next matrix
// phase as the gradient product's A operand: bf16 hi + lo chunks or fp16 chunks (bf16 inputs), or
// fp32 values.
template <typename T>
struct DsTile;
template <>
struct DsTile<__bf16> {
  u32x4 hi[2], lo[2], h[2];
  __device__ __forceinline__ void set(const float* v) {
    split_bf16x8(v, hi[0], lo[0]);
    split_bf16x8(v + 8, hi[1], lo[1]);
  }
  __device__ __forceinline__ void set16(const float* v) {
    h[0] = pack_f16x8(v);
    h[1] = pack_f16x8(v + 8);
  }
};
template <>
struct DsTile<float> {
  float v[16];
  __device__ __forceinline__ void set(const float* x) {
#pragma unroll
    for (int i = 0; i < 16; ++i) v[i] = x[i];
  }
  __device__ __forceinline__ void set16(const float* x) { set(x); }  // fp32 inputs have no fp16 product
};

// Per-lane byte offsets, inside a swizzled streamed tile of RB-byte rows, of the transpose-read
// sources of the gradient product: pass s in {0, 1} covers rows 8s + 4 hf + (lane%16)/4 (plus 16c
// for chunk c, an immediate), column 32 db + 16 ((lane/16)%2) + 4 (lane%4).
template <int RB, int DX>
__device__ __forceinline__ void tr_offsets(int (*off)[DX / 32], int lane) {
  const int trow = 4 * (lane >> 5) + ((lane & 15) >> 2);
  const int tcol = 16 * ((lane >> 4) & 1) + 4 * (lane & 3);  // element column inside a 32-wide block
#pragma unroll
  for (int sp = 0; sp < 2; ++sp) {
    const int row = trow + 8 * sp;
#pragma unroll
    for (int db = 0; db < DX / 32; ++db) {
      const int chunk = 4 * db + (tcol >> 3);
      off[sp][db] = row * RB + ((chunk ^ swz<RB>(row)) << 4) + (tcol & 7) * 2;
    }
  }
}

// Gradient-product B operands of chunk c (streamed rows 16c .. 16c + 15) of the streamed tile X
// at `xt` (row-major, swizzled): columns 32 db .. 32 db + 31 for each db, through transpose reads.
template <int DX, int RB>
__device__ __forceinline__ void grad_operands(u32x4* bop, const char* xt, const int (*toff)[DX / 32], int c) {
#pragma unroll
  for (int db = 0; db < DX / 32; ++db) {
    const u32x2 p0 = lds_read_tr16(xt + toff[0][db] + 16 * c * RB);
    const u32x2 p1 = lds_read_tr16(xt + toff[1][db] + 16 * c * RB);
    bop[db] = u32x4{p0[0], p0[1], p1[0], p1[1]};
  }
}
// out[db] += dS[:, chunk c] . B[db]: hi parts into every accumulator, then lo parts, so no MFMA
// waits on the one just before it.
template <int DX>
__device__ __forceinline__ void grad_mma(f32x16* out, const DsTile<__bf16>& ds, int c, const u32x4* bop) {
#pragma unroll
  for (int db = 0; db < DX / 32; ++db) mma_chunk<__bf16>(out[db], ds.hi[c], bop[db]);
#pragma unroll
  for (int db = 0; db < DX / 32; ++db) mma_chunk<__bf16>(out[db], ds.lo[c], bop[db]);
}

// out[db] += dS . X[:, 32 db .. 32 db + 31] for one 32-row streamed tile.  dS is in the logit
// accumulator layout (lane = owned row, element i = streamed row acc_row(i, hf)); X is the
// streamed tile of the side being differentiated, row-major and swizzled in LDS at `xt`.  F16: dS
// and X are fp16 (X at `xt` is the converted copy of the tile), one product; otherwise bf16 X and
// the hi + lo parts of dS.
template <typename T, int DX, int RB, bool F16 = false>
__device__ __forceinline__ void grad_product(f32x16* out, const DsTile<T>& ds, const char* xt,
                                             const int (*toff)[DX / 32], int lane) {
  if constexpr (F16) {
#pragma unroll
    for (int c = 0; c < 2; ++c) {
      u32x4 bop[DX / 32];
      grad_operands<DX, RB>(bop, xt, toff, c);
#pragma unroll
      for (int db = 0; db < DX / 32; ++db) mma_chunk<_Float16>(out[db], ds.h[c], bop[db]);
    }
  } else if constexpr (sizeof(T) == 2) {
#pragma unroll
    for (int c = 0; c < 2; ++c) {
      u32x4 bop[DX / 32];
      grad_operands<DX, RB>(bop, xt, toff, c);
      grad_mma<DX>(out, ds, c, bop);
    }
  } else {
    const int hf = lane >> 5, r32 = lane & 31;
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      const int row = acc_row(i, hf);
#pragma unroll
      for (int db = 0; db < DX / 32; ++db) {
        const int col = 32 * db + r32;  // fp32 element column; 4 per 16-byte chunk
        const float x = *reinterpret_cast<const float*>(xt + row * RB + ((((col >> 2) ^ swz<RB>(row))) << 4) +
                                                        (col & 3) * 4);
        out[db] = __builtin_amdgcn_mfma_f32_32x32x2f32(ds.v[i], x, out[db], 0, 0, 0);
      }
    }
  }
}

// Half `half` (HB bytes) of the gradient side of a streamed tile, converted from bf16 to fp16 in the
// same layout by the 256 lanes of one wave group (t = 0..255), in steps that the fast matrix phase
// spreads between its MFMAs: read, one step per word of two values, finish (write).  The conversion
// is exact for magnitudes in [2^-17, 2^16) and for zero (fp16 keeps 11 significant bits against
// bf16's 8); below, values round onto the fp16 subnormal grid (absolute error at most 2^-25), and
// from 2^16 on they become infinite.  finish() returns true when this lane's values leave that
// safe range: some magnitude reaches 2^16, or they are not all zero yet all below 2^-8 (so that an
// absolute error of 2^-25 could exceed 2^-17 of the largest of them).
template <int HB>
struct HalfToF16 {
  static constexpr int PER = HB / 256;  // bytes per lane
  static constexpr int NWD = PER / 4;   // words (two values each) per lane
  static_assert(PER == 16 || PER == 8, "tile half of 2 or 4 KB");
  uint32_t w[NWD], r[NWD];
  float m;
  int o;
  __device__ __forceinline__ void read(const char* src, int half, int t) {
    o = half * HB + PER * t;
    if constexpr (PER == 16) {
      const u32x4 v = lds_read16(src + o);
      w[0] = v[0], w[1] = v[1], w[2] = v[2], w[3] = v[3];
    } else {
      const u32x2 v = *reinterpret_cast<const u32x2*>(src + o);
      w[0] = v[0], w[1] = v[1];
    }
    m = 0.f;
  }
  __device__ __forceinline__ void step(int p) {
    const float f0 = __uint_as_float(w[p] << 16), f1 = __uint_as_float(w[p] & 0xffff0000u);
    const f16x2 h = {(_Float16)f0, (_Float16)f1};
    r[p] = __builtin_bit_cast(uint32_t, h);
    m = fmaxf(m, fmaxf(fabsf(f0), fabsf(f1)));
  }
  __device__ __forceinline__ bool finish(char* dst) {
    if constexpr (PER == 16)
      *reinterpret_cast<u32x4*>(dst + o) = u32x4{r[0], r[1], r[2], r[3]};
    else
      *reinterpret_cast<u32x2*>(dst + o) = u32x2{r[0], r[1]};
    return (m > 0.f && m < 0x1p-8f) || !(m < 0x1p16f);
  }
};

// A bound, below 2^e with e = frexp exponent of the result, on |dS| of the KL teacher gradients
// in row i.  With u = a - LSE_t <= 0 and v = b - LSE_s <= 0, dS = P_t (u - v - KL_i) and P_t = e^u:
// P_t |u| <= 1/e, and the log-sum inequality over the other keys gives P_t (u - v) <= KL_i + 1/e, so
// P_t |v| <= KL_i + 2/e and |dS| <= 2 KL_i + 3/e.  (The student's |dS| <= 1; both JS halves' <= 1.34.)
__device__ __forceinline__ float teacher_ds_bound(float kl) { return 2.f * fabsf(kl) + 1.11f; }

// log2|g| of a row weight, as the key owner folds it into the exponent offsets of the streamed
// queries.  A zero weight gives -1e30 instead of -inf: the offsets stay finite, so both exponents
// of such a row sink to about -1e30 and their probabilities to exact zeros, and their difference
// (the Jensen-Shannon form's log-ratio r) stays finite instead of inf - inf.
__device__ __forceinline__ float log2_weight(float g) { return fmaxf(fast_log2(fabsf(g)), -1.0e30f); }

// Wait until at most N of this wave's vector-memory operations are outstanding, N wave-uniform
// and below 16.
__device__ __forceinline__ void wait_vmcnt_upto(int n) {
  switch (n) {
    case 0: wait_vmcnt<0>(); break;
    case 1: wait_vmcnt<1>(); break;
    case 2: wait_vmcnt<2>(); break;
    case 3: wait_vmcnt<3>(); break;
    case 4: wait_vmcnt<4>(); break;
    case 5: wait_vmcnt<5>(); break;
    case 6: wait_vmcnt<6>(); break;
    case 7: wait_vmcnt<7>(); break;
    case 8: wait_vmcnt<8>(); break;
    case 9: wait_vmcnt<9>(); break;
    case 10: wait_vmcnt<10>(); break;
    case 11: wait_vmcnt<11>(); break;
    case 12: wait_vmcnt<12>(); break;
    case 13: wait_vmcnt<13>(); break;
    case 14: wait_vmcnt<14>(); break;
    default: wait_vmcnt<15>(); break;
  }
}

// OWN_Q: the workgroup owns query rows and writes dQ; otherwise it owns key rows and writes dK.
// TEACHER: gradients of the teacher side (dQ_t / dK_t) instead of the student side.
// GRP (key owner only): several query heads read each key head of the gradient's side.  It is a
// template flag, not just the run-time count, so that the one-head kernel has no pass loop around
// its tile loop: with one, the compiler schedules the tile loop's LDS reads less far ahead.
// JS: gradients of sum_i g_i JS_i (Jensen-Shannon divergence of the two rows) instead of sum_i g_i KL_i.
template <typename T, int DT, int DS, bool CAUSAL, bool TEACHER, bool OWN_Q, bool GRP, bool JS>
__global__ __launch_bounds__(BwdTile<T>::NT) __attribute__((amdgpu_waves_per_eu(sizeof(T) == 2 ? 2 : 1, 2))) void
bwd_kernel(const BwdArgs a) {
  using C = BwdTile<T>;
  constexpr int NG = C::NG, NW = C::NW, NT = C::NT, BW = C::BW, BS = C::BS, NBUF = C::NBUF, PD = C::PD;
  constexpr int DX = TEACHER ? DT : DS;
  constexpr int RBT = DT * (int)sizeof(T), RBS = DS * (int)sizeof(T), RBX = TEACHER ? RBT : RBS;
  constexpr int NCT = RBT / 16, NCS = RBS / 16;
  constexpr int TILE = BS * (RBT + RBS);
  // raw statistics of the streamed queries, 64 slots each: lse_t, lse_s, g, then kl (KL, teacher) or
  // js_t, js (JS)
  constexpr int STAT = OWN_Q ? 0 : (JS ? 5 : 4) * 256;
  constexpr int SLOT = TILE + STAT;
  using DmaT = DmaTile<BS, RBT, NT>;
  using DmaS = DmaTile<BS, RBS, NT>;
  constexpr int NI = DmaT::NI + DmaS::NI;             // tile DMA instructions per wave per tile
  constexpr int NIS = OWN_Q ? 0 : (JS ? 5 : (TEACHER ? 4 : 3));  // statistics DMA instructions (wave 0 only)
  constexpr int NRG = 4 * (DX / 32);                       // bf16 gradient product: LDS reads = MFMAs
  constexpr int NRL = (RBT + RBS) / 32;                    // bf16 logit products: LDS reads = MFMAs
  static_assert(SLOT % 256 == 0, "ring slots start on a 256-byte bank window");
  __shared__ __attribute__((aligned(1024))) char ring[NBUF][SLOT];
  // converted statistics (log2 units) of the streamed queries, per wave: in the ping-pong each wave
  // converts them in its own matrix phase of the tile, a phase before its vector phase reads them, so
  // no other wave takes part; with one group, in the vector phase itself
  constexpr bool MCONV = !OWN_Q && NG == 2;
  __shared__ __attribute__((aligned(16))) float wst[!OWN_Q ? NW : 1][4][32];
  // Fast gradient product (bf16 inputs): dS is rounded once to fp16 (2^-11 relative), scaled by a
  // power of two that keeps it inside the fp16 range (see teacher_ds_bound), and the gradient side
  // of each streamed tile is converted to fp16 in LDS (see HalfToF16), which halves the gradient
  // product's MFMA work against the bf16 hi + lo form.  Each group converts half of a tile during
  // its matrix phase of that tile; the copies of two consecutive tiles live at once.  A workgroup
  // that meets a value outside the conversion's safe range, or ends with a non-finite gradient, is
  // redone with the hi + lo form.
  constexpr bool FAST = sizeof(T) == 2;
  constexpr bool KLT = TEACHER && !JS;  // KL teacher gradients: dS bounded per row by the row's KL
  constexpr int HROW = BS * RBX;  // bytes of the gradient side of one streamed tile
  __shared__ __attribute__((aligned(1024))) char h16[FAST ? 2 : 1][FAST ? HROW : 16];
  __shared__ float gred[(FAST && !OWN_Q) ? NW : 1];  // per-wave maxima of |g| (key owner)

  const int tid0 = threadIdx.x;
  // wave index in a scalar register: every branch on it (and on the group) is a scalar branch, so a
  // barrier inside one is executed only by the waves that take it
  const int wave = __builtin_amdgcn_readfirstlane(tid0 >> 6);
  const int grp = NG == 2 ? (wave >> 2) : 0;
  // Heads: query head h reads teacher key head h / gt and student key head h / gs.  A query-owner
  // workgroup serves one query head.  A key-owner workgroup owns key rows of one key head of the
  // gradient's side and makes one pass over the stream of each of the GX query heads that read it,
  // accumulating its dK rows over the passes.
  static_assert(!(OWN_Q && GRP), "a query-owner workgroup serves one query head");
  const int GX = GRP ? (TEACHER ? a.gt : a.gs) : 1;
  const int HX = GRP ? a.H / GX : a.H;  // heads of the owned rows
  const int nbh = a.B * HX;
  const int nob = ((OWN_Q ? a.mq : a.mk) + BW - 1) / BW;
  // Paired (causal, dense, both kernels of a small problem side by side): workgroup slot oi of a head
  // runs block oi and then block nob-1-oi, a long causal stream and a short one, so that every slot
  // of the head streams about as many tiles; the middle block of an odd count runs alone.
  const int nsl = a.pair ? (nob + 1) / 2 : nob;  // workgroup slots per head
  // Workgroups go to the eight XCDs round-robin (workgroup i to XCD i mod 8), each with its own L2:
  // when the grid splits evenly (and keys are not grouped), XCD x takes the x-th eighth of the (head,
  // owned block) list, so its resident workgroups share one head's streamed tiles in L2.  In that
  // eighth the blocks go out head by head, longest stream first within a head; for a small grid
  // (len_major) whose eighth holds whole heads, longest first across those heads, so that the XCD's
  // longest streams all start first (for causal problems the block lengths differ up to N / 32 tiles).
  const int nblk = (int)gridDim.x;
  const int S8 = nblk / 8, j8 = (int)(blockIdx.x / 8);
  const int hs = (a.len_major && S8 % nsl == 0) ? S8 / nsl : 1;  // whole heads in an XCD's eighth
  const int L = (int)(blockIdx.x % 8) * S8 + (hs > 1 ? (j8 % hs) * nsl + j8 / hs : j8);
  const bool xcd = !GRP && nblk % 8 == 0;
  const int bh = xcd ? L / nsl : blockIdx.x % nbh;  // (batch, owned head)
  // grouped keys: the group's passes may be split over NSP workgroups (adjacent in launch order)
  const int NSP = GRP ? a.nsplit : 1;
  const int sp = GRP ? (blockIdx.x / nbh) % NSP : 0;
  const int oi0 = xcd ? L % nsl : (GRP ? blockIdx.x / nbh / NSP : blockIdx.x / nbh);
  const int njob = (CAUSAL && !GRP && a.pair && nob - 1 - oi0 != oi0) ? 2 : 1;
  for (int jb = 0; jb < njob; ++jb) {
    // no wave reads the LDS of the last block any more (its loop ended on a barrier): the ring may refill
    if (jb > 0) __syncthreads();
    const int oi = jb == 0 ? oi0 : nob - 1 - oi0;
    // Per block, the lane index comes from an opaque copy, so that nothing derived from it is
    // invariant over the loop: hoisted out of it, such values held registers through the tile loops
    // and spilled there.
    int tid = tid0;
    asm volatile("" : "+v"(tid));
    const int lane = tid & 63, hf = lane >> 5, r32 = lane & 31;
    // causal: the longest streams first (late query blocks for dQ, early key blocks for dK)
    const int ob = (CAUSAL && OWN_Q) ? (nob - 1 - oi) : oi;
    const int b = bh / HX, ho = bh % HX;
    const Segment sg = segment_of(a, b);
    const int n_own = OWN_Q ? sg.nq : sg.nk, n_str = OWN_Q ? sg.nk : sg.nq;
    if (ob * BW >= n_own) return;  // past the end of a shorter segment of a packed batch (whole workgroup)
    const int off = sg.nk - sg.nq;

    const int64_t own_pt = OWN_Q ? a.sqt[2] : a.skt[2], own_ps = OWN_Q ? a.sqs[2] : a.sks[2];
    const int64_t str_pt = (OWN_Q ? a.skt[2] : a.sqt[2]) * (int64_t)sizeof(T);
    const int64_t str_ps = (OWN_Q ? a.sks[2] : a.sqs[2]) * (int64_t)sizeof(T);

    const int o0 = ob * BW;
    const int o0w = o0 + wave * 32;
    const int orow = o0w + r32;
    const bool ovalid = orow < n_own;
    u32x4 ot_r[NCT / 2], os_r[NCS / 2];

    // Per query head hq (one pass): the streamed operands, this wave's owned rows of both sides (the
    // other side's key head can change from pass to pass), and the row statistics of head hq.
    const T *str_t, *str_s;
    const float *lse_t_bh, *lse_s_bh, *g_bh, *kl_bh, *js_bh;
    auto set_head = [&](const BwdArgs& A, int hq) {
      const T* qt = reinterpret_cast<const T*>(A.qt) + sg.bs * A.sqt[0] + hq * A.sqt[1] + sg.q0 * A.sqt[2];
      const T* kt = reinterpret_cast<const T*>(A.kt) + sg.bs * A.skt[0] + (hq / A.gt) * A.skt[1] + sg.k0 * A.skt[2];
      const T* qs = reinterpret_cast<const T*>(A.qs) + sg.bs * A.sqs[0] + hq * A.sqs[1] + sg.q0 * A.sqs[2];
      const T* ks = reinterpret_cast<const T*>(A.ks) + sg.bs * A.sks[0] + (hq / A.gs) * A.sks[1] + sg.k0 * A.sks[2];
      str_t = OWN_Q ? kt : qt;
      str_s = OWN_Q ? ks : qs;
      // the row offsets are formed from an opaque copy of orow in every pass: computed once before the
      // pass loop instead, they would hold registers through the tile loop that its LDS reads need
      int row = orow;
      asm volatile("" : "+v"(row));
      const bool valid = row < n_own;
      load_row_regs<T, DT>(ot_r, (OWN_Q ? qt : kt) + (int64_t)row * own_pt, valid, hf);
      load_row_regs<T, DS>(os_r, (OWN_Q ? qs : ks) + (int64_t)row * own_ps, valid, hf);
      const int64_t r0 = ((int64_t)sg.bs * A.H + hq) * A.Nq + sg.q0;
      lse_t_bh = A.lse_t + r0;
      lse_s_bh = A.lse_s + r0;
      g_bh = A.g + r0;
      kl_bh = (TEACHER || JS) ? A.kl + r0 : nullptr;  // KL, or (JS) the teacher half js_t
      js_bh = JS ? A.js + r0 : nullptr;
    };

    // query-owner: this lane's row statistics (log2 units), constant over the key stream
    float own_lt = 0.f, own_ls = 0.f, own_c = 0.f;

    // streamed range of the workgroup: tiles t_begin .. t_begin + ntile - 1 (ntile >= 1)
    int t_begin, t_end;
    if constexpr (OWN_Q) {
      const int q_last = min(n_own, o0 + BW) - 1;
      const int kend = CAUSAL ? min(n_str, q_last + off + 1) : n_str;
      t_begin = 0;
      t_end = (kend + BS - 1) / BS;
    } else {
      const int qmin = CAUSAL ? max(0, o0 - off) : 0;  // first query that may see this block's first key
      t_begin = qmin / BS;
      t_end = (n_str + BS - 1) / BS;
    }
    // never negative: the two groups' barrier counts (ntile + 2 each) stay equal even for rows
    // with no allowed key (an invalid segment of a packed batch)
    const int ntile = max(t_end - t_begin, 0);

    // ---- streamed tiles: buffer->LDS DMA into the ring, two tiles ahead
    u32x4 rs_t, rs_s, rst[5];
    auto set_rsrc = [&]() {  // buffer descriptors of the current head's streamed rows and statistics
      rs_t = rsrc_words(str_t, n_str > 0 ? (uint32_t)((n_str - 1) * str_pt + RBT) : 0u);
      rs_s = rsrc_words(str_s, n_str > 0 ? (uint32_t)((n_str - 1) * str_ps + RBS) : 0u);
      if constexpr (!OWN_Q) {
        rst[0] = rsrc_words(lse_t_bh, (uint32_t)n_str * 4u);
        rst[1] = rsrc_words(lse_s_bh, (uint32_t)n_str * 4u);
        rst[2] = rsrc_words(g_bh, (uint32_t)n_str * 4u);
        rst[3] = (TEACHER || JS) ? rsrc_words(kl_bh, (uint32_t)n_str * 4u) : rst[2];
        rst[4] = JS ? rsrc_words(js_bh, (uint32_t)n_str * 4u) : rst[2];
      }
    };
    DmaT dma_t;  // per-lane offsets set at the start of each run (below)
    DmaS dma_s;
    auto slot_ptr = [&](int u) -> char* { return ring[u]; };
    // This wave's share of tile s of the workgroup's stream into ring slot u, in two parts: part 0 the
    // teacher rows (and, key owner, the statistics), part 1 the student rows.
    auto issue_part = [&](int s, int u, auto part) {
      const int t = t_begin + s;
      const uint32_t sl = lds_addr(ring) + (uint32_t)(u * SLOT);
      const bool whole = (t + 1) * BS <= n_str;
      if constexpr (decltype(part)::value == 0) {
        dma_t.issue(rs_t, t * BS * (int)str_pt, whole, sl, wave);
        if constexpr (!OWN_Q) {
          if (wave == 0) {
            const int vo = (t * BS + lane) * 4;  // lanes 32..63 fetch the next tile's rows: unused
#pragma unroll
            for (int k = 0; k < NIS; ++k) dma_dword(rst[k], vo, sl + TILE + k * 256);
          }
        }
      } else {
        dma_s.issue(rs_s, t * BS * (int)str_ps, whole, sl + BS * RBT, wave);
      }
    };
    auto issue = [&](int s, int u) {
      issue_part(s, u, std::integral_constant<int, 0>{});
      issue_part(s, u, std::integral_constant<int, 1>{});
    };
    // this wave's DMA of the older of its two newest tiles has landed (the newest may be in flight)
    auto wait_tile = [&]() {
      if constexpr (NIS > 0) {
        if (wave == 0)
          wait_vmcnt<(PD - 1) * (NI + NIS)>();
        else
          wait_vmcnt<(PD - 1) * NI>();
      } else {
        wait_vmcnt<(PD - 1) * NI>();
      }
    };
    auto tile_state = [&](int s, bool& skip, bool& full) {
      const int sb = (t_begin + s) * BS;  // first streamed row of the tile
      if constexpr (OWN_Q) {
        skip = sb >= n_str || (CAUSAL && sb > o0w + 31 + off);
        full = sb + 31 < n_str && (!CAUSAL || sb + 31 <= o0w + off);
      } else {
        skip = sb >= n_str || (CAUSAL && o0w > sb + 31 + off);
        full = sb + 31 < n_str && (!CAUSAL || o0w + 31 <= sb + off);
      }
    };

    int off_t[NCT / 2], off_s[NCS / 2];  // logit-product operand offsets (row r32 of a tile)
    int toff[2][DX / 32];                 // transpose-read offsets of the gradient product
    // The per-lane offsets above and the DMA's are formed at the start of each run from an opaque copy
    // of the lane index: formed once, the compiler kept some of them through the fast run for the
    // hi + lo rerun and spilled them to scratch.
    auto set_offsets = [&]() {
      int ln = lane;
      asm volatile("" : "+v"(ln));
      dma_t.init(str_pt, wave, ln);
      dma_s.init(str_ps, wave, ln);
      swz_operand_offsets<RBT, NCT / 2>(off_t, ln & 31, ln >> 5);
      swz_operand_offsets<RBS, NCS / 2>(off_s, ln & 31, ln >> 5);
      tr_offsets<RBX, DX>(toff, ln);
    };

    f32x16 dacc[DX / 32];
#pragma unroll
    for (int db = 0; db < DX / 32; ++db) dacc[db] = f32x16{};
    f32x16 st = {}, ss = {};
    DsTile<T> dsr;  // dS of the last tile through the vector phase, for the gradient product

    // Key owner: statistics of the streamed query rows, converted per tile to the units the vector
    // phase uses.  The row weight g enters the exponents: g P = sgn(g) exp2(x - (LSE log2 e - log2|g|)),
    // so dS needs no per-element product with g; only a tile holding a negative weight multiplies by
    // the sign afterwards (g = 0 gives an exponent near -1e30 and a zero term, see log2_weight).
    //   0: LSE_t log2 e - log2|g|   1: LSE_s log2 e - log2|g|   2: sgn(g)
    //   3: KL: KL + LSE_t - LSE_s (teacher).  JS: the gradient side's half KL(P || M) in log2 units,
    //      js_t for the teacher and 2 js - js_t for the student
    constexpr int NSTAT = (TEACHER || JS) ? 4 : 3;
    // Fast path: dS is formed times 2^esh (an exponent offset, so no extra product): for the query
    // owner esh = 14 - e with 2^e above its rows' bound on |dS| before the row weight (e = 1, or per row
    // for KL teacher gradients), for the key owner 14 - e with 2^e above |g| times that bound for every
    // query the workgroup streams.  0 on the hi + lo path.
    float esh = 0.f;
    bool fast_run = false;
    auto convert_one = [&](int k, const float* raw) -> float {
      const float g = raw[128 + r32];
      if (k == 0) return raw[r32] * kLog2e - log2_weight(g) - esh;
      if (k == 1) return raw[64 + r32] * kLog2e - log2_weight(g) - esh;
      if (k == 2) return g;  // its sign is taken when stored
      if constexpr (JS) return (TEACHER ? raw[192 + r32] : fmaf(2.f, raw[256 + r32], -raw[192 + r32])) * kLog2e;
      return raw[192 + r32] + raw[r32] - raw[64 + r32];
    };
    // Ping-pong: each wave converts the statistics of tile s in its own matrix phase of that tile (the
    // tile landed before it, and the wave's VALU is mostly idle while its MFMAs run).  The two lane
    // halves hold the same 32 rows and split the statistics: half hf converts k = hf (the exponent
    // offsets) and k = 2 + hf (the sign of g; the KL or JS term when there are four).  The raw values
    // are read early (stats_read), converted and stored late (stats_store); tile_neg tells the vector
    // phase whether some row weight of the tile is negative.
    bool tile_neg = false;
    auto stats_read = [&](const char* sl) -> f32x4 {
      const float* raw = reinterpret_cast<const float*>(sl + TILE);
      float c3 = 0.f;
      if constexpr (JS) c3 = TEACHER ? raw[192 + r32] : fmaf(2.f, raw[256 + r32], -raw[192 + r32]);
      else if constexpr (TEACHER) c3 = raw[192 + r32] + raw[r32] - raw[64 + r32];
      return f32x4{raw[64 * hf + r32], raw[128 + r32], c3, 0.f};  // LSE of side hf, g, term 3
    };
    auto stats_store = [&](const f32x4& rv) {
      const float g = rv[1];
      wst[wave][hf][r32] = rv[0] * kLog2e - log2_weight(g) - esh;
      if (hf == 0)
        wst[wave][2][r32] = g < 0.f ? -1.f : 1.f;
      else if (NSTAT == 4)
        wst[wave][3][r32] = JS ? rv[2] * kLog2e : rv[2];
      tile_neg = __builtin_amdgcn_ballot_w64(g < 0.f) != 0;
    };

    // Vector work of tile s (ring slot u at sl): probabilities from the saved statistics, then dS.
    auto vector_phase = [&](int s, int u, const char* sl, auto f16c) {
      constexpr bool F16 = decltype(f16c)::value;
      bool skip, full;
      tile_state(s, skip, full);
      if (NG == 1 && skip) return;  // ping-pong: a skipped tile goes through the masked path (all zero)
      bool neg = false;  // some row weight of the tile is negative
      if constexpr (!OWN_Q && !MCONV) {  // statistics of the 32 streamed queries, converted by each wave
        const float* raw = reinterpret_cast<const float*>(sl + TILE);
#pragma unroll
        for (int k = 0; k < NSTAT; ++k) {
          const float v = convert_one(k, raw);
          wst[wave][k][r32] = k == 2 ? (v < 0.f ? -1.f : 1.f) : v;
        }
        neg = __builtin_amdgcn_ballot_w64(raw[128 + r32] < 0.f) != 0;
      }
      if constexpr (MCONV) neg = tile_neg;
      const int sb = (t_begin + s) * BS;
      float ds[16];
#pragma unroll
      for (int g4 = 0; g4 < 4; ++g4) {
        // The row weight is not applied here: the query owner scales each output row by it at the
        // store, the key owner has it folded into the statistics (sign below).
        f32x4 lt4, ls4, cc4;
        if constexpr (OWN_Q) {
          lt4 = f32x4{own_lt, own_lt, own_lt, own_lt};
          ls4 = f32x4{own_ls, own_ls, own_ls, own_ls};
          cc4 = f32x4{own_c, own_c, own_c, own_c};
        } else {
          const int ql = 8 * g4 + 4 * hf;
          const float(*cs)[32] = wst[wave];
          lt4 = *reinterpret_cast<const f32x4*>(&cs[0][ql]);
          ls4 = *reinterpret_cast<const f32x4*>(&cs[1][ql]);
          cc4 = (TEACHER || JS) ? *reinterpret_cast<const f32x4*>(&cs[3][ql]) : f32x4{};
        }
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const int i = 4 * g4 + e;
          float v;
          if constexpr (JS) {
            // P (log2(P/M) - KL(P || M) log2 e) of the gradient's side, with r = log2(P_s/P_t) and
            // log2(P_t/M) = w - max(r, 0), log2(P_s/M) = w + min(r, 0), w = 1 - log2(1 + 2^-|r|)
            const float x = fmaf(st[i], a.c_t, -lt4[e]), y = fmaf(ss[i], a.c_s, -ls4[e]);
            const float r = y - x;
            const float w = 1.f - fast_log2(1.f + fast_exp2(-fabsf(r)));
            v = TEACHER ? fast_exp2(x) * (w - fmaxf(r, 0.f) - cc4[e]) : fast_exp2(y) * (w + fminf(r, 0.f) - cc4[e]);
            ds[i] = v;
            continue;
          }
          const float pt = fast_exp2(fmaf(st[i], a.c_t, -lt4[e]));
          if constexpr (TEACHER) {
            v = pt * (scaled_diff(st[i], a.scale_t, ss[i], a.scale_s) - cc4[e]);
          } else {
            const float ps = fast_exp2(fmaf(ss[i], a.c_s, -ls4[e]));
            v = ps - pt;
          }
          ds[i] = v;
        }
      }
      if (neg) {  // key owner, a tile with a negative row weight: dS takes the sign of g
        asm volatile("");  // keep this a branch: taken only for such tiles
        const float(*cs)[32] = wst[wave];
#pragma unroll
        for (int g4 = 0; g4 < 4; ++g4) {
          const f32x4 sg4 = *reinterpret_cast<const f32x4*>(&cs[2][8 * g4 + 4 * hf]);
#pragma unroll
          for (int e = 0; e < 4; ++e) ds[4 * g4 + e] *= sg4[e];
        }
      }
      if (!full) {
#pragma unroll
        for (int i = 0; i < 16; ++i) {
          const int sr = sb + acc_row(i, hf);
          const bool ok = sr < n_str && (!CAUSAL || (OWN_Q ? sr <= orow + off : orow <= sr + off));
          ds[i] = ok ? ds[i] : 0.f;
        }
      }
      if constexpr (F16)
        dsr.set16(ds);
      else
        dsr.set(ds);
    };
    // Matrix-core work of tile s (ring slot at sl): the gradient product, and the two logit products.
    auto grad_phase = [&](int s, const char* sl) {
      bool skip, full;
      tile_state(s, skip, full);
      if (!skip) grad_product<T, DX, RBX>(dacc, dsr, TEACHER ? sl : sl + BS * RBT, toff, lane);
    };
    auto logit_phase = [&](int s, const char* sl) {
      bool skip, full;
      tile_state(s, skip, full);
      if (!skip) {
        st = f32x16{};
        ss = f32x16{};
        tile_dot2_swz<T, DT, DS>(st, ss, sl, sl + BS * RBT, off_t, off_s, ot_r, os_r);
        if constexpr (sizeof(T) == 2) sched_read_ahead<NRL, 4>();
      }
    };
    // Matrix phase of the ping-pong: gradient product of tile s-1 (slot sp), logit products of
    // tile s (slot sc), as one straight run of LDS reads and MFMAs so that the reads for the logit
    // products go out while the gradient MFMAs still run.  It has no branches: a tile that a wave
    // skips has an all-zero dS (its vector phase masks every element), at s = 0 the gradient
    // product adds a zero dS times ring slot 3 (zero-filled before the first barrier; tile 3 only
    // arrives in period 1), and at s = ntile the logit products (of a tile that has landed, so
    // finite) are not used.  Those cost under one percent of the MFMA work of a causal problem and
    // keep a single register assignment for the accumulators.
    auto matrix_phase = [&](const char* sp, const char* sc) {
      grad_product<T, DX, RBX>(dacc, dsr, TEACHER ? sp : sp + BS * RBT, toff, lane);
      st = f32x16{};
      ss = f32x16{};
      tile_dot2_swz<T, DT, DS>(st, ss, sc, sc + BS * RBT, off_t, off_s, ot_r, os_r);
      if constexpr (sizeof(T) == 2) sched_read_ahead<NRG + NRL, 6>();
    };
    bool risky = false;  // fast path: some converted value left the safe range (see HalfToF16)
    // Fast matrix phase: gradient product of tile s-1 from its fp16 copy at hp, logit products of
    // tile s (ring slot sc), and this group's half of tile s converted to fp16 at hd.  The order is
    // fixed by scheduling barriers: LDS reads go out LA logit steps (of two MFMAs) ahead of their
    // MFMAs; the conversion's read goes out with the first logit reads and its VALU steps ride behind
    // logit MFMAs from step CD on, when the value has arrived.  dma(part) queues the two parts of this
    // wave's share of a later tile behind the logit MFMAs of steps DM0 and DM1: a DMA instruction can
    // wait at issue while the memory pipeline takes other waves' DMA, and there the matrix core keeps
    // working through the MFMAs already issued.
    auto matrix_phase16 = [&](const char* hp, const char* sc, char* hd, int u, auto&& dma) {
      if constexpr (FAST) {
        // key owner: this wave converts the statistics of tile s here (see stats_read)
        constexpr int NDB = DX / 32, NT2 = RBT / 32, NS2 = RBS / 32, NM = NT2 > NS2 ? NT2 : NS2;
        constexpr int LA = 2, CD = 2, DM0 = 1, DM1 = NM > 4 ? 4 : NM - 1;
        using Conv = HalfToF16<HROW / 2>;
        const char* tt = sc;
        const char* ts = sc + BS * RBT;
        auto fence = [] { __builtin_amdgcn_sched_barrier(0); };
        u32x4 b0[NDB], b1[NDB];
        grad_operands<DX, RBX>(b0, hp, toff, 0);
        fence();
        grad_operands<DX, RBX>(b1, hp, toff, 1);
#pragma unroll
        for (int db = 0; db < NDB; ++db) mma_chunk<_Float16>(dacc[db], dsr.h[0], b0[db]);
        fence();
        u32x4 at[NM], as[NM];
        auto lread = [&](int c) {
          if (c < NT2) at[c] = lds_read16(tt + off_t[c]);
          if (c < NS2) as[c] = lds_read16(ts + off_s[c]);
        };
#pragma unroll
        for (int c = 0; c < LA; ++c) lread(c);
        Conv cv;
        cv.read(TEACHER ? tt : ts, grp, tid & 255);
        f32x4 rv = {};
        if constexpr (MCONV) rv = stats_read(sc);
#pragma unroll
        for (int db = 0; db < NDB; ++db) mma_chunk<_Float16>(dacc[db], dsr.h[1], b1[db]);
        fence();
        st = f32x16{};
        ss = f32x16{};
#pragma unroll
        for (int c = 0; c < NM; ++c) {
          if (c + LA < NM) lread(c + LA);
          if (c < NT2) mma_chunk<T>(st, at[c], ot_r[c]);
          if (c < NS2) mma_chunk<T>(ss, as[c], os_r[c]);
          if (c >= CD && c - CD < Conv::NWD) cv.step(c - CD);
          if (c - CD == Conv::NWD) risky |= cv.finish(hd);
          if (MCONV && c == NM - 2) stats_store(rv);
          if (c == DM0) dma(std::integral_constant<int, 0>{});
          if (c == DM1) dma(std::integral_constant<int, 1>{});
          fence();
        }
        if constexpr (NM - CD <= Conv::NWD) {  // short logit runs: whatever steps remain
#pragma unroll
          for (int p = NM - CD; p < Conv::NWD; ++p) cv.step(p);
          risky |= cv.finish(hd);
        }
      }
    };

    const int pbeg = GRP ? sp * GX / NSP : 0, pend = GRP ? (sp + 1) * GX / NSP : 1;
    // Every pass over the stream, into dacc; F16: with the fast gradient product.
    auto run = [&](auto f16c) {
      constexpr bool F16 = decltype(f16c)::value;
      set_offsets();
      // Key owner, fast path: the largest |g| (times the row's bound on |dS|) of the queries this
      // workgroup streams, over all its passes: for grouped keys read up front, otherwise while the
      // first tiles' DMA and the owned rows' loads are in flight (below).
      auto g_scan = [&]() {
        float gm = 0.f;
        for (int pass = pbeg; pass < pend; ++pass) {
          const int64_t r0 = ((int64_t)sg.bs * a.H + ho * GX + pass) * a.Nq + sg.q0;
          const float* gp = a.g + r0;
          for (int q = t_begin * BS + tid; q < n_str; q += 16 * NT) {  // 16 loads in flight per lane
            float v[16], c[16];
#pragma unroll
            for (int k = 0; k < 16; ++k) v[k] = gp[min(q + k * NT, n_str - 1)];  // unconditional loads
            if constexpr (KLT) {
#pragma unroll
              for (int k = 0; k < 16; ++k) c[k] = a.kl[r0 + min(q + k * NT, n_str - 1)];
            }
#pragma unroll
            for (int k = 0; k < 16; ++k) gm = fmaxf(gm, fabsf(v[k]) * (KLT ? teacher_ds_bound(c[k]) : 1.f));
          }
        }
#pragma unroll
        for (int o = 32; o > 0; o >>= 1) gm = fmaxf(gm, __shfl_xor(gm, o));
        if (lane == 0) gred[wave] = gm;
        __syncthreads();
#pragma unroll
        for (int w = 0; w < NW; ++w) gm = fmaxf(gm, gred[w]);
        esh = (float)(14 - __builtin_amdgcn_frexp_expf(gm));  // gm < 2^e, e = frexp exponent
      };
      if constexpr (F16 && !OWN_Q) {
        if constexpr (GRP) g_scan();
      } else {
        esh = F16 ? 13.f : 0.f;  // |dS| < 2 (KL student, either JS half); KL teacher rows: below
      }
      fast_run = F16;
      for (int pass = pbeg; pass < pend; ++pass) {
        set_head(a, ho * GX + pass);  // the owned rows' loads go out
        set_rsrc();
        // query owner: this row's statistics, loaded here (unconditionally, at a clamped row: a
        // load under a lane mask would be waited for where the masks join, before the DMA below)
        // and used after it
        float r_lt = 0.f, r_ls = 0.f, r_k = 0.f, r_j = 0.f;
        if constexpr (OWN_Q) {
          const int rr = min(orow, n_own - 1);
          r_lt = lse_t_bh[rr];
          r_ls = lse_s_bh[rr];
          if constexpr (TEACHER || JS) r_k = kl_bh[rr];  // KL, or (JS) the teacher half js_t
          if constexpr (JS) r_j = js_bh[rr];
        }
        // The first tiles' DMA goes out with these loads and the owned rows' (and the key owner's scan
        // of |g|): one memory round trip before the first period instead of two or three.  The
        // compiler's waits for its own loads also wait for these older DMAs, which the first period
        // needs anyway.
#pragma unroll
        for (int i = 0; i < PD; ++i) issue(i, i);  // past the last tile a DMA reads nothing, writes zeros
        if constexpr (F16 && !OWN_Q && !GRP) g_scan();
        if constexpr (OWN_Q) {
          if (ovalid) {
            // KL teacher: this row's own shift, 14 - e with 2^e above the row's bound on |dS|
            const float sh = (F16 && KLT) ? (float)(14 - __builtin_amdgcn_frexp_expf(teacher_ds_bound(r_k))) : esh;
            own_lt = r_lt * kLog2e - sh;
            own_ls = r_ls * kLog2e - sh;
            if constexpr (JS)
              own_c = (TEACHER ? r_k : fmaf(2.f, r_j, -r_k)) * kLog2e;
            else if constexpr (TEACHER)
              own_c = r_k + r_lt - r_ls;
          }
        }
        {
          float z[16] = {};
          if constexpr (F16)
            dsr.set16(z);
          else
            dsr.set(z);
        }
        if constexpr (F16) {  // zero the fp16 copy that the s = 0 gradient product reads (times a zero dS)
          static_assert(HROW % 16 == 0, "copy fill");
#pragma unroll
          for (int o = 16 * tid; o < HROW; o += 16 * NT) *reinterpret_cast<u32x4*>(h16[1] + o) = u32x4{};
        } else if constexpr (NG == 2) {  // zero the last slot: the s = 0 gradient product reads it (times a zero dS)
          static_assert(TILE % 16 == 0, "slot fill");
#pragma unroll
          for (int o = 16 * tid; o < TILE; o += 16 * NT) *reinterpret_cast<u32x4*>(ring[NBUF - 1] + o) = u32x4{};
        }
        // both first tiles and every load of the compiler's own have landed: none of its waits for
        // them falls inside the loop, where it would also drain the DMA ring
        wait_vmcnt<0>();
        __syncthreads();
        if constexpr (NG == 2) {
          // Periods s = 0 .. ntile, one workgroup barrier at the end of each.  In period s group 0 runs
          // the matrix phase of tile s, then its vector phase; group 1 runs the vector phase of tile s-1,
          // then the matrix phase of tile s, so on every SIMD one wave is in its matrix phase while the
          // other is in its vector phase, and each wave moves on to its second phase as soon as it is
          // done with the first.  No wave reads in a period what another wave writes in that period:
          // a matrix phase reads tile s (landed and published by the previous barrier) and the fp16
          // copy of tile s-1 (both halves written in period s-1), and writes its half of the copy of
          // tile s into the other buffer; the statistics are the wave's own.  Ring: both groups issue
          // their shares of tile s+PD in period s, into the slot of tile s-2, last read in period s-1
          // (fast path: within the matrix phase of tile s; hi + lo path: group 0 after its matrix
          // phase, group 1 before its vector phase of tile s-1); each wave waits for its share of
          // tile s+1 before the barrier that ends period s.  The last slot, read by the s = 0
          // gradient product of the hi + lo path, first receives a tile in period 1.
          if (!F16 && grp == 1) issue(PD, PD);  // group 1's share of tile PD (period 0 has no vector phase for it)
          for (int s0 = 0; s0 <= ntile; s0 += NBUF) {
#pragma unroll
            for (int u = 0; u < NBUF; ++u) {
              const int s = s0 + u;
              if (s <= ntile) {
                // matrix phase of tile s: first half of period s (group 0) or second half (group 1)
                if constexpr (F16) {
                  matrix_phase16(h16[(u + 1) & 1], slot_ptr(u), h16[u & 1], u,  // converts the statistics too
                                 [&](auto part) { issue_part(s + PD, (u + PD) % NBUF, part); });
                } else {
                  matrix_phase(slot_ptr((u + NBUF - 1) % NBUF), slot_ptr(u));
                  if constexpr (MCONV) stats_store(stats_read(slot_ptr(u)));  // tile s landed before this phase
                }
                if (grp == 1) {  // the end of period s for group 1
                  wait_tile();
                  __syncthreads();
                }
                // hi + lo path: group 0's share of tile s+PD after its matrix phase (issued at the start of
                // the period together with group 1's share, the DMA instructions of all eight waves
                // queued at once)
                if (!F16 && grp == 0) issue(s + PD, (u + PD) % NBUF);
                // vector phase of tile s: second half of period s (group 0) or first half of s+1 (group 1)
                if (s < ntile) {
                  if (!F16 && grp == 1) issue(s + PD + 1, (u + PD + 1) % NBUF);
                  vector_phase(s, u, slot_ptr(u), f16c);
                }
                if (grp == 0) {  // the end of period s for group 0 (ntile + 1 barriers for each group)
                  if (s < ntile) wait_tile();
                  __syncthreads();
                }
              }
            }
          }
        } else {
          // One group: each tile is finished within its step; tile s+PD is issued at the start of step s
          // and tile s+1 waited for at its end.
          for (int s0 = 0; s0 < ntile; s0 += NBUF) {
#pragma unroll
            for (int u = 0; u < NBUF; ++u) {
              const int s = s0 + u;
              if (s < ntile) {
                issue(s + PD, (u + PD) % NBUF);
                logit_phase(s, slot_ptr(u));
                vector_phase(s, u, slot_ptr(u), f16c);
                grad_phase(s, slot_ptr(u));
                wait_tile();
                __syncthreads();
              }
            }
          }
        }
        wait_vmcnt<0>();  // no DMA may still target the ring when it is refilled or the workgroup exits
        if (pass + 1 < pend) __syncthreads();  // all waves' DMAs have landed before the ring is refilled
      }
    };
    if constexpr (FAST) {
      run(std::true_type{});
      // a streamed value outside the fp16 conversion's safe range, or a non-finite gradient (a
      // non-finite input): redo the workgroup with the hi + lo product
      bool bad = risky;
#pragma unroll
      for (int db = 0; db < DX / 32; ++db)
#pragma unroll
        for (int i = 0; i < 16; ++i) bad |= !__builtin_isfinite(dacc[db][i]);
      if (__syncthreads_or(bad)) {
#pragma unroll
        for (int db = 0; db < DX / 32; ++db) dacc[db] = f32x16{};
        run(std::false_type{});
      }
    } else {
      run(std::false_type{});
    }


    // JS: dS above is in log2 units and lacks the 1/2 of each half: ln 2 / 2 goes into the scale
    const float scale = (TEACHER ? a.scale_t : a.scale_s) * (JS ? 0.5f * kLn2 : 1.f);
    // a split group writes its partial dK into its part of the workspace (same layout as dK)
    float* out = (OWN_Q ? a.dq : (GRP && NSP > 1 ? a.ws + sp * a.ws_part : a.dk)) +
                 (((int64_t)sg.bs * HX + ho) * (OWN_Q ? a.Nq : a.Nk) + (OWN_Q ? sg.q0 : sg.k0)) * DX;
    // query owner: dS was formed without the row weight (it is one factor per output row)
    float rscale[16];
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      const int r = o0w + acc_row(i, hf);
      // fast path: dS was formed times 2^esh, per row for the query owner of KL teacher gradients
      int sh = (int)esh;
      if (OWN_Q && KLT && fast_run && r < n_own) sh = 14 - __builtin_amdgcn_frexp_expf(teacher_ds_bound(kl_bh[r]));
      rscale[i] = OWN_Q ? (r < n_own ? ldexpf(scale * g_bh[r], -sh) : 0.f) : ldexpf(scale, -sh);
    }
#pragma unroll
    for (int db = 0; db < DX / 32; ++db) {
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        const int r = o0w + acc_row(i, hf);
        if (r < n_own) out[(int64_t)r * DX + db * 32 + r32] = rscale[i] * dacc[db][i];
      }
    }
  }
}

// ----------------------------------------------------------------------------------------------
template <bool JS, typename T, int DT, int DS, bool C, bool TE, bool OWN_Q>
static hipError_t launch_bwd_t(const BwdArgs& args, hipStream_t s) {
  BwdArgs a = args;
  const int n_own = OWN_Q ? a.mq : a.mk;  // longest segment (dense batch: all rows)
  // owned heads: query heads, or the key heads of the gradient's side
  const int gx = OWN_Q ? 1 : (TE ? a.gt : a.gs);
  const int64_t nob = (n_own + BwdTile<T>::BW - 1) / BwdTile<T>::BW;
  // pairs of owned blocks per workgroup: causal, dense and ungrouped only
  a.pair = (a.pair && C && gx == 1 && a.cu_q == nullptr) ? 1 : 0;
  const int64_t nblk = (a.pair ? (nob + 1) / 2 : nob) * a.B * (a.H / gx);
  if (nblk <= 0) return hipSuccess;
  if (nblk > 0x7fffffff) return hipErrorInvalidValue;
  if constexpr (!OWN_Q) {
    if (gx > 1) {
      constexpr int DX = TE ? DT : DS;
      const int64_t nb = a.cu_q ? 1 : a.B;
      const int64_t part = nb * (a.H / gx) * a.Nk * DX;  // floats of dK
      if (a.ws != nullptr && a.ws_floats >= part * gx && nb * (a.H / gx) <= 65535) {
        // the ungrouped kernel over every query head (it reads key head h / g of each side), each
        // head's contribution written to its own slice of an ungrouped dK in the workspace
        BwdArgs b = a;
        b.dk = a.ws;
        const int64_t nblk_h = nblk * gx;
        if (nblk_h > 0x7fffffff) return hipErrorInvalidValue;
        hipLaunchKernelGGL((bwd_kernel<T, DT, DS, C, TE, false, false, JS>), dim3((unsigned)nblk_h),
                           dim3(BwdTile<T>::NT), 0, s, b);
        hipError_t e = hipGetLastError();
        if (e != hipSuccess) return e;
        return launch_group_sum(a.dk, a.ws, nb * (a.H / gx), gx, (int64_t)a.Nk * DX, s);
      }
      BwdArgs b = a;
      b.nsplit = split_count(gx, nblk, part, a.ws, a.ws_floats);
      b.ws_part = part;
      if (nblk * b.nsplit > 0x7fffffff) return hipErrorInvalidValue;
      hipLaunchKernelGGL((bwd_kernel<T, DT, DS, C, TE, false, true, JS>), dim3((unsigned)(nblk * b.nsplit)),
                         dim3(BwdTile<T>::NT), 0, s, b);
      hipError_t e = hipGetLastError();
      if (e != hipSuccess || b.nsplit == 1) return e;
      return launch_sum_parts(a.dk, a.ws, b.nsplit, part, s);
    }
  }
  hipLaunchKernelGGL((bwd_kernel<T, DT, DS, C, TE, OWN_Q, false, JS>), dim3((unsigned)nblk), dim3(BwdTile<T>::NT), 0, s,
                     a);
  return hipGetLastError();
}

template <bool JS, bool OWN_Q, typename T, int DT, int DS>
static hipError_t bwd_ct(const BwdArgs& a, bool causal, bool teacher, hipStream_t s) {
  if (causal)
    return teacher ? launch_bwd_t<JS, T, DT, DS, true, true, OWN_Q>(a, s) : launch_bwd_t<JS, T, DT, DS, true, false, OWN_Q>(a, s);
  return teacher ? launch_bwd_t<JS, T, DT, DS, false, true, OWN_Q>(a, s) : launch_bwd_t<JS, T, DT, DS, false, false, OWN_Q>(a, s);
}

template <bool JS, bool OWN_Q, typename T>
static hipError_t bwd_d(const BwdArgs& a, int dt, int ds, bool causal, bool teacher, hipStream_t s) {
  if (dt == 128 && ds == 128) return bwd_ct<JS, OWN_Q, T, 128, 128>(a, causal, teacher, s);
  if (dt == 128 && ds == 64) return bwd_ct<JS, OWN_Q, T, 128, 64>(a, causal, teacher, s);
  if (dt == 64 && ds == 128) return bwd_ct<JS, OWN_Q, T, 64, 128>(a, causal, teacher, s);
  if (dt == 64 && ds == 64) return bwd_ct<JS, OWN_Q, T, 64, 64>(a, causal, teacher, s);
  return hipErrorInvalidValue;
}

// Launch the query-owner (OWN_Q) or key-owner backward kernel; JS: of the Jensen-Shannon divergence.
template <bool JS, bool OWN_Q>
static hipError_t bwd_dispatch(const BwdArgs& a, int dtype, int dt, int ds, bool causal, bool teacher, hipStream_t s) {
  if (dtype == 1) return bwd_d<JS, OWN_Q, __bf16>(a, dt, ds, causal, teacher, s);
  if (dtype == 0) return bwd_d<JS, OWN_Q, float>(a, dt, ds, causal, teacher, s);
  return hipErrorInvalidValue;
}

}  // namespace skl
