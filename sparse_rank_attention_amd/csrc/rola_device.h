// rola_device.h -- device helpers shared by the gfx950 kernels of librola:
// bf16 and vector types, MFMA and cross-lane wrappers, direct global->LDS
// copies, LDS tile swizzles and transposed operand reads, and the 3-D
// rotary embedding.
#ifndef ROLA_DEVICE_H_
#define ROLA_DEVICE_H_

#include <hip/hip_runtime.h>
#include <stdint.h>

#include <type_traits>

#include "../../include/rola.h"
#include "rola_internal.h"

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __fp16 f16x8 __attribute__((ext_vector_type(8)));
typedef __fp16 f16x2 __attribute__((ext_vector_type(2)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef int i32x8 __attribute__((ext_vector_type(8)));

#define LDS_AS __attribute__((address_space(3)))
#define GLOBAL_AS __attribute__((address_space(1)))

namespace rola {


static __device__ __forceinline__ float bf2f(uint16_t h) {
  return __uint_as_float(((uint32_t)h) << 16);
}
static __device__ __forceinline__ float bflo(uint32_t w) { return __uint_as_float(w << 16); }
static __device__ __forceinline__ float bfhi(uint32_t w) { return __uint_as_float(w & 0xffff0000u); }

static __device__ __forceinline__ bf16x8 as_bf16x8(u32x4 u) { return __builtin_bit_cast(bf16x8, u); }
static __device__ __forceinline__ u32x4 as_u32x4(bf16x8 b) { return __builtin_bit_cast(u32x4, b); }

// Physical position of a key (or rank index) inside a 16-group of the
// transposed tiles: keys [0-3, 8-11, 4-7, 12-15] are stored at 0..15.
static __device__ __forceinline__ int perm16_key_of_pos(int p) {
  const int w = p & 15;
  const int k = (w < 4) ? w : (w < 8) ? w + 4 : (w < 12) ? w - 4 : w;
  return (p & ~15) | k;
}

static __device__ __forceinline__ float phi(float u) { return u > 0.0f ? u + 1.0f : __expf(u); }

// 2^x on the transcendental unit (v_exp_f32); results below the normal range
// flush to zero, which is harmless for softmax weights.
static __device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }

static __device__ __forceinline__ f32x16 mfma_bf16(bf16x8 a, bf16x8 b, f32x16 c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
}
static __device__ __forceinline__ f32x16 mfma_f16(f16x8 a, f16x8 b, f32x16 c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_f16(a, b, c, 0, 0, 0);
}

// e4m3 codes: round to nearest even, saturating at +-448
// (v_cvt_pk_fp8_f32; `hi` selects the upper 16 bits of `old`).
template <bool HI>
static __device__ __forceinline__ int cvt_fp8x2(float a, float b, int old) {
  return __builtin_amdgcn_cvt_pk_fp8_f32(a, b, old, HI);
}

// v_mfma_f32_32x32x64_f8f6f4 with both operands e4m3 and no block scales.
// Lane l holds 32 codes (8 dwords) of row (A) / column (B) l%32; A and B
// bytes with the same lane half and byte index meet at the same k.
static __device__ __forceinline__ f32x16 mfma_fp8(i32x8 a, i32x8 b, f32x16 c) {
  return __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(a, b, c, 0, 0, 0, 0, 0, 0);
}

static __device__ __forceinline__ float shfl_xor32(float v) { return __shfl_xor(v, 32, 64); }

// max / sum of a value and its partner lane l^32, on the VALU: the two
// halves of the wave are exchanged between two registers (v_permlane32_swap)
// and combined symmetrically, so every lane gets the pair result.
static __device__ __forceinline__ float pair_max32(float v) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
static __device__ __forceinline__ float pair_sum32(float v) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v), false, false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}

// Direct global->LDS copy of 16 bytes per lane: lane l of the wave writes
// lds_dst + 16*l (lds_dst is wave-uniform).  Issued from inline asm so that
// the compiler does not order every later LDS access after all pending
// copies (it would insert s_waitcnt vmcnt(0) and drain the prefetch rings);
// completion is awaited explicitly with s_waitcnt vmcnt before use.  M0 is
// saved and restored around the copy.
static __device__ __forceinline__ void lds_dma16(const void *gsrc, void *lds_dst) {
  const uint32_t base = __builtin_amdgcn_readfirstlane((uint32_t)(uintptr_t)(LDS_AS void *)lds_dst);
  uint32_t saved;
  asm volatile(
      "s_mov_b32 %0, m0\n\t"
      "s_mov_b32 m0, %1\n\t"
      "global_load_lds_dwordx4 %2, off\n\t"
      "s_mov_b32 m0, %0"
      : "=&s"(saved)
      : "s"(base), "v"(gsrc)
      : "memory");
}

// The same copy from a wave-uniform base address (held in an SGPR pair)
// plus a 32-bit per-lane byte offset (the global_load_lds saddr form): no
// per-lane 64-bit address arithmetic.
static __device__ __forceinline__ void lds_dma16_s(const void *base_ptr, uint32_t voff, void *lds_dst) {
  const uint32_t m = __builtin_amdgcn_readfirstlane((uint32_t)(uintptr_t)(LDS_AS void *)lds_dst);
  const uint64_t b64 = (uint64_t)(uintptr_t)base_ptr;
  // readfirstlane returns int: widen through uint32_t (no sign extension)
  const uint32_t lo = (uint32_t)__builtin_amdgcn_readfirstlane((uint32_t)b64);
  const uint32_t hi = (uint32_t)__builtin_amdgcn_readfirstlane((uint32_t)(b64 >> 32));
  const void *sbase = (const void *)(uintptr_t)(((uint64_t)hi << 32) | (uint64_t)lo);
  uint32_t saved;
  asm volatile(
      "s_mov_b32 %0, m0\n\t"
      "s_mov_b32 m0, %1\n\t"
      "global_load_lds_dwordx4 %2, %3\n\t"
      "s_mov_b32 m0, %0"
      : "=&s"(saved)
      : "s"(m), "v"(voff), "s"(sbase)
      : "memory");
}

// The same copy with the LDS destination given as a byte address in LDS
// (wave-uniform, formed by scalar arithmetic from the ring's base) and the
// global base in an SGPR pair.
static __device__ __forceinline__ void lds_dma16_m0(const void *sbase, uint32_t voff, uint32_t m0) {
  uint32_t saved;
  asm volatile(
      "s_mov_b32 %0, m0\n\t"
      "s_mov_b32 m0, %1\n\t"
      "global_load_lds_dwordx4 %2, %3\n\t"
      "s_mov_b32 m0, %0"
      : "=&s"(saved)
      : "s"(m0), "v"(voff), "s"(sbase)
      : "memory");
}

// LDS byte address of a shared array element (the array's own address space
// is LDS, so no null check is generated)
template <typename T>
static __device__ __forceinline__ uint32_t lds_addr(const T *p) {
  return (uint32_t)(uintptr_t)(const LDS_AS void *)p;
}

// LDS tile layouts: row-major [64 rows][D] bf16 in 16-byte chunks, chunk c
// of row r stored at c ^ swizzle(r).  K tiles (read as 16-byte MFMA rows)
// XOR with the row's low four bits (16 chunks per row at D=128, 8 at D=64);
// V tiles (read transposed, 8 bytes per lane) XOR with 4 * (row & 3), the
// four rows a transposed read spans.  Both were measured free of bank
// conflicts (SQ_LDS_BANK_CONFLICT = 0).
template <int D>
static __device__ __forceinline__ int swz_k(int r) { return r & (15 & (D / 8 - 1)); }
template <int D>
static __device__ __forceinline__ int swz_v(int r) { return (4 * (r & 3)) & (D / 8 - 1); }

static __device__ __forceinline__ void barrier_lds() {
  // all LDS reads of this wave retired, then a plain workgroup barrier (no
  // vmcnt wait: prefetches stay in flight across it)
  asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
}

template <int N>
static __device__ __forceinline__ void wait_vmcnt() {
  static_assert(N >= 0 && N < 64, "vmcnt range");
  __builtin_amdgcn_s_waitcnt((N & 15) | (0x7 << 4) | (0xF << 8) | (((N >> 4) & 3) << 14));
}

template <int OPS, int S>
static __device__ __forceinline__ void wait_tiles_in_flight(int tiles) {
  // wait until at most `tiles` later tiles (2*OPS DMA ops each) are outstanding
  if (S >= 4 && tiles >= 2) wait_vmcnt<(S >= 4 ? 4 * OPS : 0)>();
  else if (S >= 3 && tiles >= 1) wait_vmcnt<(S >= 3 ? 2 * OPS : 0)>();
  else wait_vmcnt<0>();
}

// wait until at most `tiles` (<= T) later tiles of PER DMA ops each are outstanding
template <int PER, int T>
static __device__ __forceinline__ void wait_tiles(int tiles) {
  if constexpr (T > 0) {
    if (tiles >= T) {
      wait_vmcnt<T * PER>();
      return;
    }
    wait_tiles<PER, T - 1>(tiles);
  } else {
    wait_vmcnt<0>();
  }
}

typedef short i16x4 __attribute__((ext_vector_type(4)));

// A operand V^T[d][keys] of a 32x32x16 MFMA step s (keys 16s..16s+15) and
// d-tile dt, read from a row-major V tile with the transposing LDS load: in
// each 16-lane group, lane i points at row kbase + i/4, dims dbase + 4*(i%4),
// and lane l receives rows kbase..kbase+3 of dim dbase + l%16.  Key order per
// lane group g: 16s + 4g + {0..3}, then 16s + 8 + 4g + {0..3} -- the order of
// the S^T accumulator rows that form the matching B operand.
template <int D>
static __device__ __forceinline__ bf16x8 vt_operand(const uint16_t *sV, int s, int dt, int lane) {
  const int g = lane >> 5, dhalf = (lane >> 4) & 1, i = lane & 15;
  const int dstart = 32 * dt + 16 * dhalf + 4 * (i & 3);
  const int c = dstart >> 3, sub = dstart & 7;
  const int r0 = 16 * s + 4 * g + (i >> 2), r1 = r0 + 8;
  const LDS_AS i16x4 *p0 = (const LDS_AS i16x4 *)(const LDS_AS uint16_t *)(sV + r0 * D + ((c ^ swz_v<D>(r0)) << 3) + sub);
  const LDS_AS i16x4 *p1 = (const LDS_AS i16x4 *)(const LDS_AS uint16_t *)(sV + r1 * D + ((c ^ swz_v<D>(r1)) << 3) + sub);
  const i16x4 a = __builtin_amdgcn_ds_read_tr16_b64_v4i16((LDS_AS i16x4 *)p0);
  const i16x4 b = __builtin_amdgcn_ds_read_tr16_b64_v4i16((LDS_AS i16x4 *)p1);
  typedef short i16x8 __attribute__((ext_vector_type(8)));
  const i16x8 ab = {a[0], a[1], a[2], a[3], b[0], b[1], b[2], b[3]};
  return __builtin_bit_cast(bf16x8, ab);
}

// The same operand from a precomputed lane address p (first four keys) and
// the element distance `half` to the second four keys (8 rows further).
static __device__ __forceinline__ bf16x8 vt_operand_at(const uint16_t *p, int half) {
  const i16x4 a = __builtin_amdgcn_ds_read_tr16_b64_v4i16((LDS_AS i16x4 *)(const LDS_AS uint16_t *)p);
  const i16x4 b = __builtin_amdgcn_ds_read_tr16_b64_v4i16((LDS_AS i16x4 *)(const LDS_AS uint16_t *)(p + half));
  typedef short i16x8 __attribute__((ext_vector_type(8)));
  const i16x8 ab = {a[0], a[1], a[2], a[3], b[0], b[1], b[2], b[3]};
  return __builtin_bit_cast(bf16x8, ab);
}

// 3-D rotary embedding: the t, h and w axes own dims [0, off1), [off1,
// off2), [off2, D); pair p of an axis with d_a dims turns by
// pos * theta^(-2p/d_a).  Angles are formed in fp32 and taken modulo one
// turn before the hardware sine/cosine (inputs in revolutions), so no table
// lookups (global loads) are needed inside the streaming loops.
using RopeArgsDev = RopeArgsHost;

// (t, h, w) of token n; n < 2^31 (the planner caps N far below), so the
// divisions are 32-bit
static __device__ __forceinline__ void token_pos(int64_t n, const RopeArgsDev &ra, int &pt, int &ph,
                                                 int &pw) {
  const uint32_t hw = (uint32_t)(ra.grid_h * ra.grid_w), gw = (uint32_t)ra.grid_w;
  const uint32_t n32 = (uint32_t)n;
  const uint32_t t = n32 / hw, rem = n32 - t * hw, hh = rem / gw;
  pt = (int)t;
  ph = (int)hh;
  pw = (int)(rem - hh * gw);
}

// inverse frequency of the pair starting at even dim d
static __device__ __forceinline__ float rope_freq(int d, const RopeArgsDev &ra) {
  // the fields are read into registers first: a per-lane choice between
  // struct fields would otherwise become a per-lane load of the arguments
  const int off1 = ra.off1, off2 = ra.off2, h0 = ra.half0, h1 = ra.half1, h2 = ra.half2;
  const int p = (d < off1 ? d : d < off2 ? d - off1 : d - off2) >> 1;
  const int da = 2 * (d < off1 ? h0 : d < off2 ? h1 : h2);
  return exp2f(-2.0f * (float)p / (float)da * ra.log2_theta);
}

// Rotate 8 consecutive dims (4 pairs) starting at d0 and round to bf16.
// freq[p]: inverse frequency of pair p (rope_freq(d0 + 2p)).
static __device__ __forceinline__ bf16x8 rope8(bf16x8 x, int d0, int pt, int ph, int pw,
                                               const float *freq, const RopeArgsDev &ra) {
  const u32x4 u = as_u32x4(x);
  bf16x8 y;
#pragma unroll
  for (int p = 0; p < 4; ++p) {
    const int d = d0 + 2 * p;
    const int pos = d < ra.off1 ? pt : (d < ra.off2 ? ph : pw);
    float rev = (float)pos * freq[p] * 0.15915494309189535f;  // angle / (2 pi)
    rev = rev - floorf(rev);
    const float cs = __builtin_amdgcn_cosf(rev), sn = __builtin_amdgcn_sinf(rev);
    const float x0 = bflo(u[p]), x1 = bfhi(u[p]);
    y[2 * p] = (__bf16)(x0 * cs - x1 * sn);
    y[2 * p + 1] = (__bf16)(x0 * sn + x1 * cs);
  }
  return y;
}

}  // namespace rola

#endif  // ROLA_DEVICE_H_
