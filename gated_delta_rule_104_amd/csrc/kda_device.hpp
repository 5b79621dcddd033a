// Device-side building blocks shared by the libkda kernels (gfx950, wave64).
//
// MFMA tiles.  Every product in the kernels is built from 16x16 output tiles.
// For v_mfma_f32_16x16x{32,16}_bf16 and v_mfma_f32_16x16x4_f32 the accumulator
// of lane l holds rows 4*(l/16)+e (e = 0..3) of column l%16.  That layout is also
// the B-operand layout of a 16-deep contraction (lane l supplies k = 4*(l/16)+e of
// column l%16), so a tile produced by one product can feed the next one from
// registers with no data movement; the A operand then reads the matching k
// positions from LDS.  For the 32-deep bf16 product a B fragment packs two such
// tiles, so lane group g supplies k = 4g..4g+3 and 16+4g..16+4g+3; LDS tiles
// read as the A operand of such products store every 32-wide k block in that
// order (kpos below), so that each A fragment is one 16-byte read.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace kda {

typedef __bf16 bf16;
typedef __attribute__((__vector_size__(8 * sizeof(__bf16)))) __bf16 bf16x8;
typedef __attribute__((__vector_size__(4 * sizeof(__bf16)))) __bf16 bf16x4;
typedef __attribute__((__vector_size__(4 * sizeof(float)))) float f32x4;
typedef __attribute__((__vector_size__(2 * sizeof(float)))) float f32x2;
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
// LDS tiles: rows of R bytes (R a power of two >= 16) made of 16-byte granules.
// A granule's position in its row is XORed with a function of the row index so
// that 16 lanes reading one logical granule of 16 consecutive rows (the MFMA
// operand pattern) spread over the banks.  The function depends only on
// row % 16, so row tile t of a tile sits at a fixed offset from tile 0.  The
// default suits 16-byte fragment reads; NARROW suits tiles read with 8-byte
// fragments (chosen by measuring gfx950's LDS bank-conflict counter on these
// access patterns):
//   default : row & (min(G, 16) - 1)                       (G = R / 16)
//   NARROW  : G = 8: (row & 7) ^ ((row >> 3) & 1);  G = 2: ((row >> 2) ^ (row >> 3)) & 1
template <int R, bool NARROW = false>
__device__ __forceinline__ uint32_t swz(uint32_t row, uint32_t byte) {
  constexpr uint32_t G = R / 16;
  uint32_t f;
  if constexpr (NARROW && G == 8) f = (row & 7u) ^ ((row >> 3) & 1u);
  else if constexpr (NARROW && G == 2) f = ((row >> 2) ^ (row >> 3)) & 1u;
  else f = row & ((G < 16 ? G : 16) - 1);
  return row * R + ((((byte >> 4) ^ f) << 4) | (byte & 15u));
}

template <typename V>
__device__ __forceinline__ V lds_ld(const char* smem, uint32_t off) {
  return *reinterpret_cast<const V*>(smem + off);
}
template <typename V>
__device__ __forceinline__ void lds_st(char* smem, uint32_t off, V v) {
  *reinterpret_cast<V*>(smem + off) = v;
}

// Transposing 8-byte LDS read of 16-bit elements (ds_read_b64_tr_b16, gfx950):
// see the chunk kernel's Kb^T fragments for the lane mapping.
__device__ __forceinline__ bf16x4 lds_tr16(const char* smem, uint32_t off) {
  typedef short s16x4 __attribute__((ext_vector_type(4)));
  typedef __attribute__((address_space(3))) s16x4 lds_s16x4;
  const s16x4 r = __builtin_amdgcn_ds_read_tr16_b64_v4i16(
      (lds_s16x4*)((__attribute__((address_space(3))) char*)const_cast<char*>(smem) + off));
  return __builtin_bit_cast(bf16x4, r);
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

typedef float f32x2v __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x2v __attribute__((ext_vector_type(2)));
typedef uint32_t u32x2v __attribute__((ext_vector_type(2)));

// fp32 -> bf16 (round to nearest even), two elements per conversion
__device__ __forceinline__ uint32_t cvt2(float a, float b) {
  return __builtin_bit_cast(uint32_t, __builtin_convertvector((f32x2v){a, b}, bf16x2v));
}
__device__ __forceinline__ bf16x4 pack4(f32x4 t) {
  return __builtin_bit_cast(bf16x4, (u32x2v){cvt2(t[0], t[1]), cvt2(t[2], t[3])});
}
__device__ __forceinline__ bf16x8 pack8(f32x4 lo, f32x4 hi) {
  bf16x8 r;
  r[0] = (bf16)lo[0]; r[1] = (bf16)lo[1]; r[2] = (bf16)lo[2]; r[3] = (bf16)lo[3];
  r[4] = (bf16)hi[0]; r[5] = (bf16)hi[1]; r[6] = (bf16)hi[2]; r[7] = (bf16)hi[3];
  return r;
}

// Position of k inside its row for tiles stored in that order: within each
// 32-wide block, granule g (8 elements) holds k = 4g..4g+3 then 16+4g..16+4g+3.
__host__ __device__ constexpr int kpos(int k) {
  return (k & ~31) | (((k & 15) >> 2) << 3) | ((k & 16) >> 2) | (k & 3);
}
static_assert(kpos(0) == 0 && kpos(3) == 3 && kpos(4) == 8 && kpos(16) == 4 && kpos(20) == 12 &&
                  kpos(31) == 31 && kpos(33) == 33 && kpos(48) == 36, "kpos");

__device__ __forceinline__ f32x4 zero4() { return f32x4{0.f, 0.f, 0.f, 0.f}; }

// ---------------------------------------------------------------------------
// Buffer resources, DPP row moves and raw 16-byte row loads.
typedef __amdgpu_buffer_rsrc_t rsrc_t;

// Raw buffer over [p, p + bytes): loads past the end return 0, stores are dropped.
__device__ __forceinline__ rsrc_t make_rsrc(const void* p, uint32_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(p), (short)0, (int)bytes, 0x00020000);
}
__device__ __forceinline__ u32x4 bload128(rsrc_t r, uint32_t off) {
  return __builtin_bit_cast(u32x4, __builtin_amdgcn_raw_buffer_load_b128(r, off, 0, 0));
}

// DPP moves within rows of 16 lanes (gfx9 encoding): row_shr:n shifts values
// n lanes up inside the row; lanes below n read 0 (bound control), so no old
// value has to be materialised.
template <int CTRL>
__device__ __forceinline__ float dpp(float x) {
  return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), CTRL, 0xF, 0xF, true));
}
constexpr int DPP_ROW_SHR = 0x110;
// integer moves: a rotation by 8 within each 16-lane row, and quad permutes
// that swap neighbouring lanes ([1,0,3,2]) and lane pairs ([2,3,0,1])
template <int CTRL>
__device__ __forceinline__ uint32_t dppu(uint32_t x) {
  return (uint32_t)__builtin_amdgcn_update_dpp(0, (int)x, CTRL, 0xF, 0xF, true);
}
constexpr int DPP_ROW_ROR8 = 0x128;
constexpr int DPP_QUAD_SWAP1 = 0xB1;
constexpr int DPP_QUAD_SWAP2 = 0x4E;

// Four lanes a, b, c, d hold the rows e = 0..3 of a 4 x 4 matrix of dwords
// (lane q: M[q][0..3]); afterwards lane q holds its column, M[0..3][q].  The
// partner across the first pair of lane pairs is reached with CTRL1 (a
// rotation by 8 within the row, or a quad permute), the neighbour with a quad
// swap; h and p are lane q's bits (q = 2h + p).
template <int CTRL1>
__device__ __forceinline__ u32x4 transpose4(u32x4 d, bool h, bool p) {
  uint32_t s0 = h ? d[0] : d[2], s1 = h ? d[1] : d[3];
  s0 = dppu<CTRL1>(s0);
  s1 = dppu<CTRL1>(s1);
  if (h) {
    d[0] = s0;
    d[1] = s1;
  } else {
    d[2] = s0;
    d[3] = s1;
  }
  s0 = p ? d[0] : d[1];
  s1 = p ? d[2] : d[3];
  s0 = dppu<DPP_QUAD_SWAP1>(s0);
  s1 = dppu<DPP_QUAD_SWAP1>(s1);
  if (p) {
    d[0] = s0;
    d[2] = s1;
  } else {
    d[1] = s0;
    d[3] = s1;
  }
  return d;
}

// 8 consecutive elements of a token row, as loaded from HBM.
template <typename T> struct Raw8 { u32x4 p[sizeof(T) / 2]; };

template <typename T>
__device__ __forceinline__ void raw_load(Raw8<T>& r, rsrc_t rs, uint32_t off) {
#pragma unroll
  for (int i = 0; i < (int)(sizeof(T) / 2); ++i) r.p[i] = bload128(rs, off + 16 * i);
}

template <typename T>
__device__ __forceinline__ void raw_f32(const Raw8<T>& r, float* out) {
  if constexpr (sizeof(T) == 2) {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      out[2 * i] = __uint_as_float(r.p[0][i] << 16);
      out[2 * i + 1] = __uint_as_float(r.p[0][i] & 0xffff0000u);
    }
  } else {
#pragma unroll
    for (int i = 0; i < 8; ++i) out[i] = __uint_as_float(r.p[i >> 2][i & 3]);
  }
}


}  // namespace kda
