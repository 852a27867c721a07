// Device-side building blocks shared by the attention-KL kernels (gfx950 only).
//
// MFMA tile convention used everywhere (v_mfma_f32_32x32x16_bf16 and
// v_mfma_f32_32x32x2f32, 64-lane wavefront):
//   A operand  : lane l supplies row  m = l % 32 of the 32 x k block
//   B operand  : lane l supplies col  n = l % 32 of the k x 32 block
//   lane half  : hf = l / 32 supplies the second half of the k block
//   D (32x32)  : lane l holds column n = l % 32, rows  8*(i/4) + 4*hf + (i%4),  i = 0..15
// Operand rows are read as 16-byte chunks: lane half hf takes chunks 2c+hf of a
// row for step c.  A and B always use the same chunk-to-k mapping, so the
// contraction pairs the same feature index on both sides whatever the dtype.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace skl {

typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));
typedef _Float16 f16x2 __attribute__((ext_vector_type(2)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;
// Running maxima start here rather than at -inf so that a lane whose keys are all
// masked so far still rescales by exp2(0) = 1 instead of exp2(-inf + inf) = NaN.
constexpr float kMaxInit = -1.0e30f;

__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }
__device__ __forceinline__ float fast_log2(float x) { return __builtin_amdgcn_logf(x); }

// acc += A * B over one 16-byte chunk per lane of each operand.
template <typename T>
__device__ __forceinline__ void mma_chunk(f32x16& acc, const u32x4& a, const u32x4& b);

template <>
__device__ __forceinline__ void mma_chunk<__bf16>(f32x16& acc, const u32x4& a, const u32x4& b) {
  acc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, a), __builtin_bit_cast(bf16x8, b), acc,
                                                0, 0, 0);
}

template <>
__device__ __forceinline__ void mma_chunk<_Float16>(f32x16& acc, const u32x4& a, const u32x4& b) {
  acc = __builtin_amdgcn_mfma_f32_32x32x16_f16(__builtin_bit_cast(f16x8, a), __builtin_bit_cast(f16x8, b), acc, 0,
                                               0, 0);
}

template <>
__device__ __forceinline__ void mma_chunk<float>(f32x16& acc, const u32x4& a, const u32x4& b) {
  // Copy each lane element to a scalar before reinterpreting it: a bit-cast applied directly to
  // an ext-vector element reads the vector's first element.
  const uint32_t av[4] = {a[0], a[1], a[2], a[3]};
  const uint32_t bv[4] = {b[0], b[1], b[2], b[3]};
#pragma unroll
  for (int e = 0; e < 4; ++e)
    acc = __builtin_amdgcn_mfma_f32_32x32x2f32(__uint_as_float(av[e]), __uint_as_float(bv[e]), acc, 0, 0, 0);
}

__device__ __forceinline__ u32x4 lds_read16(const char* p) { return *reinterpret_cast<const u32x4*>(p); }

// Row of the 32x32 accumulator held in register i by lane half hf.
__device__ __forceinline__ int acc_row(int i, int hf) { return 8 * (i >> 2) + 4 * hf + (i & 3); }

// Load one row's operand chunks (2c + hf) from global memory, or zeros past the end.
template <typename T, int D>
__device__ __forceinline__ void load_row_regs(u32x4* regs, const T* row, bool valid, int hf) {
  constexpr int NC = D * (int)sizeof(T) / 16;
  const char* p = reinterpret_cast<const char*>(row);
#pragma unroll
  for (int c = 0; c < NC / 2; ++c) {
    regs[c] = valid ? *reinterpret_cast<const u32x4*>(p + (2 * c + hf) * 16) : u32x4{0u, 0u, 0u, 0u};
  }
}

// ---------------------------------------------------------------------------------------------
// Swizzled LDS tiles filled by buffer->LDS DMA (buffer_load_dwordx4 ... lds).
//
// A tile holds ROWS rows of RB bytes, unpadded; logical 16-byte chunk c of row r is stored at
// physical chunk c ^ swz(r).  One DMA instruction writes up to 64 lanes x 16 bytes contiguously at
// the wave's LDS address, so the swizzle is applied on the global side: each lane fetches the
// logical chunk that belongs at its physical slot.  Rows start on a 256-byte bank window (RB >= 256)
// or share one two to a window (RB == 128).  swz keeps both access patterns used here free of bank
// conflicts:
//  - MFMA operand reads (ds_read_b128, 16 lanes per cycle): 16 consecutive rows, one logical chunk;
//  - transpose reads (ds_read_b64_tr_b16, 32 lanes per cycle): rows R..R+3 (R % 4 == 0) times the
//    four logical chunks 4m..4m+3, so the four rows must land in four different 4-chunk blocks.
template <int RB>
__device__ __forceinline__ int swz(int r) {
  if constexpr (RB >= 256)
    return 4 * (r & 3) + ((r >> 2) & 3);
  else
    return 4 * ((r >> 1) & 1) + ((r >> 2) & 3);
}

template <int ROWS, int RB, int NT>
struct DmaTile {
  static constexpr int BYTES = ROWS * RB;
  static constexpr int NW = NT / 64;
  static constexpr int CH = BYTES / NW < 1024 ? BYTES / NW : 1024;  // bytes per wave per instruction
  static constexpr int LPW = CH / 16;                               // lanes taking part
  static constexpr int NI = BYTES / (NW * CH);                      // DMA instructions per wave per tile
  static_assert(CH % 256 == 0 && BYTES % (NW * CH) == 0, "tile must split into whole wave writes");
  int vo[NI];  // per-lane global byte offset inside the tile (relative to its first row)

  __device__ __forceinline__ void init(int64_t pitch, int wave, int lane) {
#pragma unroll
    for (int j = 0; j < NI; ++j) {
      const int o = (j * NW + wave) * CH + 16 * (lane % LPW);
      const int pr = o / RB, pc = (o % RB) / 16;
      vo[j] = pr * (int)pitch + ((pc ^ swz<RB>(pr)) * 16);
    }
  }
  // Queue the tile whose first row sits at byte offset `toff` of the buffer into LDS at byte
  // address `dst` (see lds_addr).
  // Issued as inline asm so that the compiler does not track these LDS writes: callers order
  // them with explicit vmcnt waits and barriers (the destination slot is never read while a DMA
  // into it can be in flight).  The asm has no output register.
  //
  // Only the VGPR offset of a buffer access is range-checked against num_records; the SGPR
  // offset is added after the check.  A tile that lies wholly inside the buffer (`whole`, a
  // wave-uniform flag) passes toff in the SGPR; any other tile (the ragged last one, or one past
  // the end) adds it to the VGPR offset, so its rows beyond the buffer arrive as zeros and no
  // byte outside the buffer is read.  The two asm strings differ so the branches stay separate.
  __device__ __forceinline__ void issue(const u32x4& rsrc, int toff, bool whole, uint32_t dst, int wave) const {
    const uint32_t base = dst;
    const bool on = LPW == 64 || (int)(threadIdx.x & 63) < LPW;  // lanes past LPW stay masked off
    const int stoff = __builtin_amdgcn_readfirstlane(toff);       // wave-uniform: keep it in an SGPR
    if (whole) {
#pragma unroll
      for (int j = 0; j < NI; ++j) {
        const uint32_t m0v = __builtin_amdgcn_readfirstlane(base + (uint32_t)((j * NW + wave) * CH));
        if (on)
          asm volatile("s_mov_b32 m0, %0\n\tbuffer_load_dwordx4 %1, %2, %3 offen lds ; whole tile"
                       :
                       : "s"(m0v), "v"(vo[j]), "s"(rsrc), "s"(stoff)
                       : "memory", "m0");
      }
    } else {
#pragma unroll
      for (int j = 0; j < NI; ++j) {
        const uint32_t m0v = __builtin_amdgcn_readfirstlane(base + (uint32_t)((j * NW + wave) * CH));
        if (on)
          asm volatile("s_mov_b32 m0, %0\n\tbuffer_load_dwordx4 %1, %2, %3 offen lds ; checked tile"
                       :
                       : "s"(m0v), "v"(vo[j] + toff), "s"(rsrc), "s"(0)
                       : "memory", "m0");
      }
    }
  }
};

// One dword per lane from byte offset `voff` of the buffer into LDS at byte address `dst` + 4 * lane
// (inline asm, untracked like DmaTile::issue).  The whole offset is range-checked: past num_records
// the lane writes zero.
__device__ __forceinline__ void dma_dword(const u32x4& rsrc, int voff, uint32_t dst) {
  const uint32_t m0v = __builtin_amdgcn_readfirstlane(dst);
  asm volatile("s_mov_b32 m0, %0\n\tbuffer_load_dword %1, %2, %3 offen lds"
               :
               : "s"(m0v), "v"(voff), "s"(rsrc), "s"(0)
               : "memory", "m0");
}

// LDS byte address of a __shared__ array (its first byte), for the DMA's M0.  Taken from the array
// itself, not from a generic pointer into it, so that the conversion needs no null check.
template <class A>
__device__ __forceinline__ uint32_t lds_addr(A& arr) {
  return (uint32_t)(uintptr_t)((__attribute__((address_space(3))) char*)&arr);
}

// Raw buffer descriptor words (base, stride 0, num_records = bytes, gfx9 data-format word)
// for DMA issued from inline asm.
__device__ __forceinline__ u32x4 rsrc_words(const void* base, uint32_t bytes) {
  const uint64_t p = reinterpret_cast<uint64_t>(base);
  return u32x4{(uint32_t)p, (uint32_t)(p >> 32) & 0xffffu, bytes, 0x00020000u};
}

// Wait until at most N buffer loads (including LDS DMA) of this wave are outstanding.
template <int N>
__device__ __forceinline__ void wait_vmcnt() {
  static_assert(N >= 0 && N < 64, "vmcnt range");
  // gfx9 encoding: vmcnt[3:0] | expcnt[6:4]=7 | lgkmcnt[11:8]=15 | vmcnt[5:4] at [15:14]
  __builtin_amdgcn_s_waitcnt((N & 15) | (7 << 4) | (15 << 8) | ((N >> 4) << 14));
}

// Per-lane LDS byte offsets of the MFMA operand chunks of row `row` of a swizzled tile: chunk
// 2c + hf for step c (the same chunk-to-k mapping as the register operands).
template <int RB, int NSTEP>
__device__ __forceinline__ void swz_operand_offsets(int* off, int row, int hf) {
  const int s = swz<RB>(row) ^ hf;  // (2c + hf) ^ swz == 2c ^ (hf ^ swz)
#pragma unroll
  for (int c = 0; c < NSTEP; ++c) off[c] = row * RB + (((2 * c) ^ s) << 4);
}

// 32x32 logit tile from a swizzled LDS tile (A rows) and register B rows.
template <typename T, int D>
__device__ __forceinline__ void tile_dot_swz(f32x16& acc, const char* tile, const int* off, const u32x4* b_regs) {
  constexpr int NC = D * (int)sizeof(T) / 16;
#pragma unroll
  for (int c = 0; c < NC / 2; ++c) mma_chunk<T>(acc, lds_read16(tile + off[c]), b_regs[c]);
}

// Scheduling groups for a straight run of N LDS operand reads feeding N MFMAs: the first P reads
// go out before any MFMA, then each pair of MFMAs is followed by the next pair of reads, so every
// read is issued about P MFMAs before its consumer.  Only instructions of the enclosing basic block
// are affected.
template <int N, int P>
__device__ __forceinline__ void sched_read_ahead() {
  static_assert(P <= N && (N - P) % 2 == 0, "read-ahead pattern");
  __builtin_amdgcn_sched_group_barrier(0x100, P, 0);  // DS reads
#pragma unroll
  for (int i = 0; i < (N - P) / 2; ++i) {
    __builtin_amdgcn_sched_group_barrier(0x008, 2, 0);  // MFMA
    __builtin_amdgcn_sched_group_barrier(0x100, 2, 0);
  }
  __builtin_amdgcn_sched_group_barrier(0x008, P, 0);
}

// Both 32x32 logit tiles of one step: st from the DT-feature rows at `tt`, ss from the DS-feature
// rows at `ts`, the two accumulation chains interleaved so that neither MFMA waits on its
// predecessor's result.  Operand reads: DT*sizeof(T)/32 + DS*sizeof(T)/32 ds_read_b128.
template <typename T, int DT, int DS>
__device__ __forceinline__ void tile_dot2_swz(f32x16& st, f32x16& ss, const char* tt, const char* ts,
                                              const int* off_t, const int* off_s, const u32x4* bt,
                                              const u32x4* bs) {
  constexpr int NT2 = DT * (int)sizeof(T) / 32, NS2 = DS * (int)sizeof(T) / 32;
  constexpr int NM = NT2 > NS2 ? NT2 : NS2;
#pragma unroll
  for (int c = 0; c < NM; ++c) {
    if (c < NT2) mma_chunk<T>(st, lds_read16(tt + off_t[c]), bt[c]);
    if (c < NS2) mma_chunk<T>(ss, lds_read16(ts + off_s[c]), bs[c]);
  }
}

// LDS transpose read (gfx950 ds_read_b64_tr_b16).  Within each group of 16 lanes, source
// lane r supplies the address of 4 consecutive 16-bit elements; result lane i receives
// element i%4 of source lanes i/4, i/4+4, i/4+8, i/4+12.  Pointing source lane r at row
// R0 + r/4, column C0 + 4(r%4) of a row-major tile hands lane i rows R0..R0+3 of column C0 + i.
__device__ __forceinline__ u32x2 lds_read_tr16(const char* p) {
  typedef short s16x4 __attribute__((ext_vector_type(4)));
  const s16x4 v = __builtin_amdgcn_ds_read_tr16_b64_v4i16((s16x4 __attribute__((address_space(3)))*)(p));
  return __builtin_bit_cast(u32x2, v);
}

// Split 8 fp32 values into bf16 hi + lo parts (v ~= hi + lo to about 2^-16 relative).  Each pair
// is rounded to bf16 once (hi); its two halves, widened back to fp32 by a shift and a mask, give
// the remainders, which are rounded again (lo).
__device__ __forceinline__ void split_bf16x8(const float* v, u32x4& hi, u32x4& lo) {
#pragma unroll
  for (int p = 0; p < 4; ++p) {
    const bf16x2 h = {(__bf16)v[2 * p], (__bf16)v[2 * p + 1]};
    const uint32_t hw = __builtin_bit_cast(uint32_t, h);
    const float r0 = v[2 * p] - __uint_as_float(hw << 16);
    const float r1 = v[2 * p + 1] - __uint_as_float(hw & 0xffff0000u);
    const bf16x2 l = {(__bf16)r0, (__bf16)r1};
    hi[p] = hw;
    lo[p] = __builtin_bit_cast(uint32_t, l);
  }
}

// 8 fp32 values rounded to fp16 (nearest even; beyond the fp16 range they become +-inf).
__device__ __forceinline__ u32x4 pack_f16x8(const float* v) {
  u32x4 r;
#pragma unroll
  for (int p = 0; p < 4; ++p) {
    const f16x2 h = {(_Float16)v[2 * p], (_Float16)v[2 * p + 1]};
    r[p] = __builtin_bit_cast(uint32_t, h);
  }
  return r;
}

// bf16 values, two per word, as fp32 (a shift or a mask of each half).
template <int NW>
__device__ __forceinline__ void widen_bf16(const uint32_t* w, float* f) {
#pragma unroll
  for (int p = 0; p < NW; ++p) {
    f[2 * p] = __uint_as_float(w[p] << 16);
    f[2 * p + 1] = __uint_as_float(w[p] & 0xffff0000u);
  }
}

}  // namespace skl
