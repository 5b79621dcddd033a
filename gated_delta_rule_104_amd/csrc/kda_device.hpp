// Device-side building blocks shared by the libkda kernels (gfx950, wave64).
//
// MFMA tiles.  Every product in the kernels is built from 16x16 output tiles.
// For v_mfma_f32_16x16x{32,16}_bf16 and v_mfma_f32_16x16x4_f32 the accumulator
// of lane l holds rows 4*(l/16)+e (e = 0..3) of column l%16.  That layout is also
// the B-operand layout of a 16-deep contraction (lane l supplies k = 4*(l/16)+e of
// column l%16), so a tile produced by one product can feed the next one from
// registers with no data movement; the A operand then reads the matching k
// positions from LDS (see mma_ar_* below).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace kda {

typedef __bf16 bf16;
typedef __attribute__((__vector_size__(8 * sizeof(__bf16)))) __bf16 bf16x8;
typedef __attribute__((__vector_size__(4 * sizeof(__bf16)))) __bf16 bf16x4;
typedef __attribute__((__vector_size__(4 * sizeof(float)))) float f32x4;
typedef __attribute__((__vector_size__(4 * sizeof(uint32_t)))) uint32_t u32x4;
typedef __attribute__((__vector_size__(2 * sizeof(uint32_t)))) uint32_t u32x2;

__device__ __forceinline__ int lane_id() { return __builtin_amdgcn_mbcnt_hi(~0u, __builtin_amdgcn_mbcnt_lo(~0u, 0u)); }

// The lane id as a value the compiler must treat as freshly produced.  LDS
// addresses derived from it are then recomputed (a few integer ops) inside a
// loop instead of being hoisted out of it and pinned in registers.
__device__ __forceinline__ int fresh_lane(int l) {
  asm volatile("" : "+v"(l));
  return l;
}

// Workgroup barrier for LDS hand-off.  Waits only for this wave's LDS traffic
// (not for outstanding global loads, which are prefetches consumed later).
__device__ __forceinline__ void sync_lds() {
  asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
  __builtin_amdgcn_s_barrier();
  asm volatile("" ::: "memory");
}

// Order this wave's earlier LDS writes before its later LDS reads of data
// written by other lanes of the same wave.
__device__ __forceinline__ void wave_lds_fence() {
  asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
}

__device__ __forceinline__ float to_f32(bf16 x) { return (float)x; }
__device__ __forceinline__ float to_f32(float x) { return x; }
template <typename T> __device__ __forceinline__ T from_f32(float x);
template <> __device__ __forceinline__ bf16 from_f32<bf16>(float x) { return (bf16)x; }
template <> __device__ __forceinline__ float from_f32<float>(float x) { return x; }

// ---------------------------------------------------------------------------
// LDS tiles: rows of R bytes (R a power of two >= 16), 16-byte granules XOR-
// swizzled by the row index so that 16 lanes reading the same column range of
// 16 consecutive rows hit distinct banks.
template <int R>
__device__ __forceinline__ uint32_t swz(uint32_t row, uint32_t byte) {
  constexpr uint32_t G = R / 16;
  constexpr uint32_t MASK = (G < 16 ? G : 16) - 1;
  return row * R + ((((byte >> 4) ^ (row & MASK)) << 4) | (byte & 15u));
}

template <typename V>
__device__ __forceinline__ V lds_ld(const char* smem, uint32_t off) {
  return *reinterpret_cast<const V*>(smem + off);
}
template <typename V>
__device__ __forceinline__ void lds_st(char* smem, uint32_t off, V v) {
  *reinterpret_cast<V*>(smem + off) = v;
}

// ---------------------------------------------------------------------------
// MFMA wrappers.
__device__ __forceinline__ f32x4 mfma_bf16_k32(f32x4 acc, bf16x8 a, bf16x8 b) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, acc, 0, 0, 0);
}
__device__ __forceinline__ f32x4 mfma_bf16_k16(f32x4 acc, bf16x4 a, bf16x4 b) {
  return __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(a, b, acc, 0, 0, 0);
}
__device__ __forceinline__ f32x4 mfma_f32_k4(f32x4 acc, float a, float b) {
  return __builtin_amdgcn_mfma_f32_16x16x4f32(a, b, acc, 0, 0, 0);
}

__device__ __forceinline__ bf16x4 pack4(f32x4 t) {
  bf16x4 r;
  r[0] = (bf16)t[0]; r[1] = (bf16)t[1]; r[2] = (bf16)t[2]; r[3] = (bf16)t[3];
  return r;
}
__device__ __forceinline__ bf16x8 pack8(f32x4 lo, f32x4 hi) {
  bf16x8 r;
  r[0] = (bf16)lo[0]; r[1] = (bf16)lo[1]; r[2] = (bf16)lo[2]; r[3] = (bf16)lo[3];
  r[4] = (bf16)hi[0]; r[5] = (bf16)hi[1]; r[6] = (bf16)hi[2]; r[7] = (bf16)hi[3];
  return r;
}
__device__ __forceinline__ bf16x8 cat8(bf16x4 lo, bf16x4 hi) {
  bf16x8 r;
  r[0] = lo[0]; r[1] = lo[1]; r[2] = lo[2]; r[3] = lo[3];
  r[4] = hi[0]; r[5] = hi[1]; r[6] = hi[2]; r[7] = hi[3];
  return r;
}

__device__ __forceinline__ f32x4 zero4() { return f32x4{0.f, 0.f, 0.f, 0.f}; }

// ---------------------------------------------------------------------------
// Contractions whose A operand is an LDS tile of element type T (row-major,
// swizzled rows of R bytes) and whose B operand is a set of accumulator tiles in
// registers.  `bt[i]` holds k rows 16*i .. 16*i+15 of B for the lane's column.
//
// Operand fragments for the bf16 path use v_mfma_f32_16x16x32_bf16 with the k
// positions of lane group g = l/16 taken as {4g..4g+3} from tile 2m and
// {4g..4g+3} from tile 2m+1, i.e. k = 32m + 4g + p and 32m + 16 + 4g + p: the
// accumulator tiles pack straight into B fragments, and A reads two 8-byte
// pieces.  The fp32 path issues four 16x16x4 steps per 16-deep tile, step e
// taking k = 4g + e from the lane's accumulator register e.

// acc += A[r0 .. r0+15][k0 .. k0+32*nkb) * B  (bf16; bfr[m] = pack8(bt[2m], bt[2m+1]))
template <int R>
__device__ __forceinline__ f32x4 mma_ar_bf16(f32x4 acc, const char* smem, uint32_t base, int r0,
                                             int k0, const bf16x8* bfr, int nkb, int l) {
  const uint32_t row = r0 + (l & 15);
  const uint32_t g4 = 4 * (l >> 4);
  _Pragma("unroll") for (int m = 0; m < nkb; ++m) {
    const uint32_t kk = k0 + 32 * m + g4;
    bf16x4 lo = lds_ld<bf16x4>(smem, base + swz<R>(row, 2 * kk));
    bf16x4 hi = lds_ld<bf16x4>(smem, base + swz<R>(row, 2 * (kk + 16)));
    acc = mfma_bf16_k32(acc, cat8(lo, hi), bfr[m]);
  }
  return acc;
}

// acc += A[r0 .. r0+15][k0 .. k0+16*ntile) * B  (fp32; bt[i] accumulator tiles)
template <int R>
__device__ __forceinline__ f32x4 mma_ar_f32(f32x4 acc, const char* smem, uint32_t base, int r0,
                                            int k0, const f32x4* bt, int ntile, int l) {
  const uint32_t row = r0 + (l & 15);
  const uint32_t g4 = 4 * (l >> 4);
  _Pragma("unroll") for (int i = 0; i < ntile; ++i) {
    const uint32_t kk = k0 + 16 * i + g4;
    f32x4 a = lds_ld<f32x4>(smem, base + swz<R>(row, 4 * kk));
    acc = mfma_f32_k4(acc, a[0], bt[i][0]);
    acc = mfma_f32_k4(acc, a[1], bt[i][1]);
    acc = mfma_f32_k4(acc, a[2], bt[i][2]);
    acc = mfma_f32_k4(acc, a[3], bt[i][3]);
  }
  return acc;
}

// acc += A[ra0..+15][0..K) * B^T where B^T's rows rb0..+15 are stored like A
// (both LDS, k contiguous within a row).  bf16: 16x16x32 steps, k = 8g..8g+7.
template <int R>
__device__ __forceinline__ f32x4 mma_ll_bf16(f32x4 acc, const char* smem, uint32_t abase, int ra0,
                                             uint32_t bbase, int rb0, int K, int l) {
  const uint32_t g8 = 8 * (l >> 4);
  _Pragma("unroll") for (int k0 = 0; k0 < K; k0 += 32) {
    bf16x8 a = lds_ld<bf16x8>(smem, abase + swz<R>(ra0 + (l & 15), 2 * (k0 + g8)));
    bf16x8 b = lds_ld<bf16x8>(smem, bbase + swz<R>(rb0 + (l & 15), 2 * (k0 + g8)));
    acc = mfma_bf16_k32(acc, a, b);
  }
  return acc;
}

template <int R>
__device__ __forceinline__ f32x4 mma_ll_f32(f32x4 acc, const char* smem, uint32_t abase, int ra0,
                                            uint32_t bbase, int rb0, int K, int l) {
  const uint32_t g4 = 4 * (l >> 4);
  _Pragma("unroll") for (int k0 = 0; k0 < K; k0 += 16) {
    f32x4 a = lds_ld<f32x4>(smem, abase + swz<R>(ra0 + (l & 15), 4 * (k0 + g4)));
    f32x4 b = lds_ld<f32x4>(smem, bbase + swz<R>(rb0 + (l & 15), 4 * (k0 + g4)));
    acc = mfma_f32_k4(acc, a[0], b[0]);
    acc = mfma_f32_k4(acc, a[1], b[1]);
    acc = mfma_f32_k4(acc, a[2], b[2]);
    acc = mfma_f32_k4(acc, a[3], b[3]);
  }
  return acc;
}

}  // namespace kda
