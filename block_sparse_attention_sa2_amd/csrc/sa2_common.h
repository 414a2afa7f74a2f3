// Device helpers shared by the libsa2 kernels (gfx950 / CDNA4 only).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include <string>

#include "sa2.h"

namespace sa2 {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef short i16x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;

// ---------------------------------------------------------------------------
// Element types.  bf16 values are carried as their 16-bit patterns.
// ---------------------------------------------------------------------------
struct bf16_t { uint16_t bits; };

// Eight consecutive elements (16-byte aligned) as bf16 for the MFMA operands.
__device__ inline bf16x8 load8(const bf16_t* p) {
  return *reinterpret_cast<const bf16x8*>(p);
}
__device__ inline bf16x8 load8(const float* p) {
  const f32x4 a = *reinterpret_cast<const f32x4*>(p);
  const f32x4 b = *reinterpret_cast<const f32x4*>(p + 4);
  bf16x8 r;
  r[0] = (__bf16)a[0]; r[1] = (__bf16)a[1]; r[2] = (__bf16)a[2]; r[3] = (__bf16)a[3];
  r[4] = (__bf16)b[0]; r[5] = (__bf16)b[1]; r[6] = (__bf16)b[2]; r[7] = (__bf16)b[3];
  return r;
}

// Eight consecutive elements widened to fp64 (mask builder).
__device__ inline void load8_f64(const bf16_t* p, double* out) {
  const u32x4 w = *reinterpret_cast<const u32x4*>(p);
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    out[2 * i] = (double)__uint_as_float(w[i] << 16);
    out[2 * i + 1] = (double)__uint_as_float(w[i] & 0xffff0000u);
  }
}
__device__ inline void load8_f64(const float* p, double* out) {
  const f32x4 a = *reinterpret_cast<const f32x4*>(p);
  const f32x4 b = *reinterpret_cast<const f32x4*>(p + 4);
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    out[i] = (double)a[i];
    out[4 + i] = (double)b[i];
  }
}

// Four consecutive fp32 values stored in the output type (8/16 bytes).
__device__ inline void store4(bf16_t* p, float a, float b, float c, float d) {
  bf16x4 v;
  v[0] = (__bf16)a; v[1] = (__bf16)b; v[2] = (__bf16)c; v[3] = (__bf16)d;
  *reinterpret_cast<bf16x4*>(p) = v;
}
__device__ inline void store4(float* p, float a, float b, float c, float d) {
  f32x4 v;
  v[0] = a; v[1] = b; v[2] = c; v[3] = d;
  *reinterpret_cast<f32x4*>(p) = v;
}

// ---------------------------------------------------------------------------
// MFMA.  v_mfma_f32_32x32x16_bf16 register layout (wave64, h = lane / 32):
//   A operand: lane holds A[lane % 32][8h .. 8h+7]        (row, k)
//   B operand: lane holds B[8h .. 8h+7][lane % 32]        (k, col)
//   C/D:       element e of lane is C[8(e/4) + 4h + e%4][lane % 32]
// ---------------------------------------------------------------------------
__device__ inline f32x16 mfma32(bf16x8 a, bf16x8 b, f32x16 c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c, 0, 0, 0);
}

// ds_read_b64_tr_b16: within each group of 16 lanes, lane i receives element
// i % 4 of the 64-bit words addressed by lanes 4r + i/4, r = 0..3.  If lane j
// of the group addresses X[k0 + j/4][n0 + 4(j%4)] of a row-major LDS tile X,
// lane i receives X[k0 + r][n0 + i], r = 0..3: a column of X.
__device__ inline bf16x4 lds_read_tr(const uint16_t* p) {
  i16x4 r = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
      (__attribute__((address_space(3))) i16x4*)(p));
  return __builtin_bit_cast(bf16x4, r);
}

__device__ inline bf16x8 cat(bf16x4 a, bf16x4 b) {
  return __builtin_shufflevector(a, b, 0, 1, 2, 3, 4, 5, 6, 7);
}

__device__ inline bf16x8 lds_read8(const uint16_t* p) {
  return *reinterpret_cast<const bf16x8*>(p);
}

// ---------------------------------------------------------------------------
// Launch helpers
// ---------------------------------------------------------------------------

// Workgroups are dispatched round-robin over the 8 XCDs.  Remap the hardware
// id so that consecutive logical ids run on the same XCD (and share its L2).
__device__ inline int xcd_remap(int id, int n) {
  const int q = n / 8, r = n % 8;
  const int x = id % 8, local = id / 8;
  return x * q + min(x, r) + local;
}

// v and the value of the lane 32 apart, in lane-dependent order, through
// v_permlane32_swap (a VALU exchange of the two half-waves; no LDS trip).
// Swapping the upper half of one copy with the lower half of another leaves
// each lane holding its own value in one result and its partner's in the
// other, so symmetric combinations need no select.
__device__ inline void cross_half(float v, float& a, float& b) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v), false,
                                                  false);
  a = __uint_as_float(r[0]);
  b = __uint_as_float(r[1]);
}
// Stores 32 consecutive columns of one row held in the MFMA accumulator
// layout (element e of half-wave h at column 8(e/4) + 4h + e%4), scaled by
// mul and rounded to bf16, as two 16-byte stores per lane instead of four
// 8-byte ones: v_permlane32_swap hands each half-wave its partner's
// neighbouring four columns, so half-wave h writes columns 16j + 8h .. +7.
// The exchange runs on every lane; `valid` (the same for a lane and the lane
// 32 apart) guards only the stores.
__device__ inline uint32_t pack_bf16x2(float a, float b) {
  typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
  bf16x2_t v;
  v[0] = (__bf16)a;
  v[1] = (__bf16)b;
  return __builtin_bit_cast(uint32_t, v);
}
__device__ inline void store_row32(bf16_t* p, const f32x16& a, float mul, int h, bool valid) {
#pragma unroll
  for (int j = 0; j < 2; ++j) {
    uint32_t x[2], y[2];
#pragma unroll
    for (int w = 0; w < 2; ++w) {
      const int e0 = 8 * j + 2 * w, e1 = e0 + 4;   // a word of group 2j, the same of 2j + 1
      const auto r = __builtin_amdgcn_permlane32_swap(pack_bf16x2(a[e0] * mul, a[e0 + 1] * mul),
                                                      pack_bf16x2(a[e1] * mul, a[e1 + 1] * mul),
                                                      false, false);
      x[w] = r[0];   // half 0: its own group 2j; half 1: the partner's group 2j + 1
      y[w] = r[1];   // half 0: the partner's group 2j; half 1: its own group 2j + 1
    }
    if (valid) *reinterpret_cast<uint4*>(p + 16 * j + 8 * h) = make_uint4(x[0], x[1], y[0], y[1]);
  }
}
__device__ inline float wave_max32(float v) {  // max with the lane 32 apart
  float a, b;
  cross_half(v, a, b);
  return fmaxf(a, b);
}
__device__ inline float wave_sum32(float v) {  // sum with the lane 32 apart (same in both)
  float a, b;
  cross_half(v, a, b);
  return a + b;
}

}  // namespace sa2

// Host-side error reporting shared by the entry points.
namespace sa2 {
sa2_status fail(sa2_status st, const std::string& msg);
sa2_status check_launch(const char* what);
inline bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }
inline int cdiv(int a, int b) { return (a + b - 1) / b; }
}  // namespace sa2

namespace sa2 {
// Eight consecutive elements as fp32 (for the fp32 dot products of dO and O).
__device__ inline void load8_f32(const bf16_t* p, float* out) {
  const u32x4 w = *reinterpret_cast<const u32x4*>(p);
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    out[2 * i] = __uint_as_float(w[i] << 16);
    out[2 * i + 1] = __uint_as_float(w[i] & 0xffff0000u);
  }
}
__device__ inline void load8_f32(const float* p, float* out) {
  const f32x4 a = *reinterpret_cast<const f32x4*>(p);
  const f32x4 b = *reinterpret_cast<const f32x4*>(p + 4);
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    out[i] = a[i];
    out[4 + i] = b[i];
  }
}

__device__ inline bf16x8 zero8() {
  bf16x8 z;
#pragma unroll
  for (int i = 0; i < 8; ++i) z[i] = (__bf16)0.0f;
  return z;
}
__device__ inline f32x16 zero16() {
  f32x16 z;
#pragma unroll
  for (int i = 0; i < 16; ++i) z[i] = 0.0f;
  return z;
}
// Orders this wave's LDS writes before its later LDS reads by other lanes.
__device__ inline void wave_lds_sync() {
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
  __builtin_amdgcn_wave_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
}

// A value the compiler may keep in a scalar register (it is the same in every
// lane, e.g. the wave index).
__device__ inline int uniform(int x) { return __builtin_amdgcn_readfirstlane(x); }

// ---------------------------------------------------------------------------
// Direct global -> LDS copies through buffer resources.
//
// A raw buffer resource covers `bytes` bytes from `base`; a load whose offset
// (vector + scalar + immediate) is at or past `bytes` returns zeros, so rows
// past the end of a tensor arrive as zero rows with no clamping.  The
// buffer_load ... lds form writes lane l's bytes to LDS at M0 + IMM + size*l
// (M0: the LDS byte address of dst, the same in every lane); the immediate
// offset IMM moves the global address and the LDS address alike, the scalar
// offset only the global one.
//
// The copies are issued from inline assembly, so the compiler does not track
// them: it would otherwise make LDS reads that it cannot prove disjoint from
// a copy in flight wait for it (the transposing reads are such), which
// serialises the double buffers.  Every kernel therefore waits for its own
// copies explicitly (s_waitcnt vmcnt(0)) and then passes a workgroup barrier
// before it reads them, and issues no copy that it does not wait for.
// ---------------------------------------------------------------------------
typedef uint32_t rsrc_t __attribute__((ext_vector_type(4)));
#define SA2_AS3 __attribute__((address_space(3)))

__device__ inline rsrc_t make_rsrc(const void* base, uint32_t bytes) {
  const uint64_t a = reinterpret_cast<uint64_t>(base);
  rsrc_t r;
  r[0] = (uint32_t)a;
  r[1] = (uint32_t)(a >> 32);   // stride 0: a raw byte buffer
  r[2] = bytes;
  r[3] = 0x00020000u;           // 32-bit data format, no swizzle
  return r;
}
__device__ inline uint32_t lds_addr(const void* p) {
  return (uint32_t)reinterpret_cast<uintptr_t>((const SA2_AS3 void*)p);
}
template <int IMM>
__device__ inline void buf_lds16(rsrc_t r, const void* dst, uint32_t voff, uint32_t soff) {
  asm volatile("s_mov_b32 m0, %0\n\tbuffer_load_dwordx4 %1, %2, %3 offen offset:%4 lds"
               :: "s"(lds_addr(dst)), "v"(voff), "s"(r), "s"(soff), "i"(IMM) : "memory", "m0");
}
template <int IMM>
__device__ inline void buf_lds4(rsrc_t r, const void* dst, uint32_t voff, uint32_t soff) {
  asm volatile("s_mov_b32 m0, %0\n\tbuffer_load_dword %1, %2, %3 offen offset:%4 lds"
               :: "s"(lds_addr(dst)), "v"(voff), "s"(r), "s"(soff), "i"(IMM) : "memory", "m0");
}

// Unrolls f(integral_constant<int, I>) for I = B .. E-1, so that I can feed
// an immediate operand.
template <int I> struct Int { static constexpr int value = I; };
template <int B, int E, typename F>
__device__ inline void static_for(F&& f) {
  if constexpr (B < E) {
    f(Int<B>{});
    static_for<B + 1, E>(f);
  }
}

// ---------------------------------------------------------------------------
// Backward row statistics (bwd workspace).  Per head, rows are taken in
// groups of 32; group g holds [32 x log2-scaled LSE | 32 x Delta] (fp32), so
// one 256-byte copy brings both statistics of a 32-row slice.  A head has
// 4 * ceil(N / 128) groups: every row of every query block, padding included.
// ---------------------------------------------------------------------------
__host__ __device__ inline int stat_groups(int N) { return 4 * ((N + 127) / 128); }
__device__ inline size_t stat_lse2(int bh, int G, int row) {
  return ((size_t)bh * G + (row >> 5)) * 64 + (row & 31);
}
__device__ inline size_t stat_delta(int bh, int G, int row) { return stat_lse2(bh, G, row) + 32; }
}  // namespace sa2
