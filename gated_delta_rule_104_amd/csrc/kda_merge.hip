// Sequential merge of per-segment results into true segment start states.
//
// The end state of a segment is affine in its start state, S_end = M S_start +
// S_zero_end, and one exchange of (S_zero_end, M) among the segments recovers
// every segment's exact start state ("Kimi K3 开源日来了", section
// "针对适配的 Infra", KDA context parallelism).  Per (b, h):
//     S = S_in;  for i in 0..G-1:  S_start[i] = S;  S = M[i] S + S_zero_end[i];
//     S_T = S.
//
// Workgroup = one head and 16 state columns, four waves; wave w computes row
// tiles w*D/64 .. of the new slice with fp32 matrix cores
// (v_mfma_f32_16x16x4_f32, full fp32 precision).  The slice of S is the B
// operand, kept in LDS in accumulator layout (lane l holds rows 4*(l/16)+e of
// column l%16 of each 16-row tile), so the A operand reads 4 consecutive
// entries of an M row per lane.  The next segment's M rows are fetched into
// registers while the current product runs.  The workgroups of one head sit on
// one XCD, so M is read from HBM once per head and shared through that L2.
//
// With segment records (the split prefill's), a segment whose map is exactly
// zero ends in its S_zero_end whatever its start: the chain restarts there, its
// M is neither read nor multiplied, and only the start states that a product
// made are written (the others are S_in or a S_zero_end, read from there).
#include "kda_device.hpp"
#include "kda_launch.hpp"

namespace kda {

template <int D>
// S_T may alias S_in: every read of S_in happens before the first barrier, every
// write of S_T after the last one, and each workgroup touches only its columns.
__global__ __launch_bounds__(256) void kda_merge_kernel(const float* S_in, const float* __restrict__ Z,
                                                        const float* __restrict__ M,
                                                        float* __restrict__ S_start, float* S_T,
                                                        int BH, int G, const uint32_t* __restrict__ flags) {
  constexpr int NT = D / 16;   // 16-row tiles of the state (= k tiles of the product)
  constexpr int RPW = NT / 4;  // row tiles per wave
  __shared__ f32x4 sS[NT][64];
  const int W = gridDim.x;
  int id = blockIdx.x;
  if ((W & 7) == 0) id = (blockIdx.x & 7) * (W >> 3) + (blockIdx.x >> 3);
  const int bh = id / NT, ct = id - bh * NT;
  const int wave = threadIdx.x >> 6, l = threadIdx.x & 63;
  const int g4 = 4 * (l >> 4), r16 = l & 15;
  const int col = 16 * ct + r16;
  const size_t hs = (size_t)bh * D * D;
  // offset of this lane's entry e of row tile rt in a D x D state
  auto at = [&](int rt, int e) -> size_t { return (size_t)(16 * rt + g4 + e) * D + col; };

  // this wave's row tiles of a state (null: zero) into the LDS slice
  auto slice_from = [&](const float* src) {
#pragma unroll
    for (int q = 0; q < RPW; ++q) {
      const int rt = wave * RPW + q;
      f32x4 x;
#pragma unroll
      for (int e = 0; e < 4; ++e) x[e] = src ? src[at(rt, e)] : 0.f;
      sS[rt][l] = x;
    }
  };
  // M rows of this wave's row tiles for segment i: a[q][t] = M[16 rt + r16][16 t + g4 .. +3]
  auto load_m = [&](f32x4 (*a)[NT], int i) {
    const float* Mi = M + ((size_t)i * BH + bh) * D * D;
#pragma unroll
    for (int q = 0; q < RPW; ++q)
#pragma unroll
      for (int t = 0; t < NT; ++t)
        a[q][t] = *reinterpret_cast<const f32x4*>(Mi + (size_t)(16 * (wave * RPW + q) + r16) * D + 16 * t + g4);
  };
  // one step: acc = M_i S + Z_i from the slice S in LDS (am holds M_i's rows)
  auto step = [&](const f32x4 (*am)[NT], int i, f32x4* acc, const f32x4* b) {
    const size_t gs = ((size_t)i * BH + bh) * D * D;
#pragma unroll
    for (int q = 0; q < RPW; ++q)
#pragma unroll
      for (int e = 0; e < 4; ++e) acc[q][e] = Z[gs + at(wave * RPW + q, e)];
#pragma unroll
    for (int q = 0; q < RPW; ++q)
#pragma unroll
      for (int t = 0; t < NT; ++t)
#pragma unroll
        for (int e = 0; e < 4; ++e) acc[q] = mfma_f32_k4(acc[q], am[q][t][e], b[t][e]);
  };
  auto slice_to_global = [&](float* dst) {
#pragma unroll
    for (int q = 0; q < RPW; ++q) {
      const int rt = wave * RPW + q;
      const f32x4 x = sS[rt][l];
#pragma unroll
      for (int e = 0; e < 4; ++e) dst[at(rt, e)] = x[e];
    }
  };

  if (flags) {
    // Segment records: start(i) is S_in for i = 0 and segment i-1's end
    // otherwise; that end is Z[i-1] when segment i-1's map vanished, and the
    // product M_{i-1} start(i-1) + Z[i-1] only when it did not.  So the chain
    // runs through the segments whose map did not vanish, each run starting
    // from the Z (or S_in) before it, and S_start[i] is written only where the
    // product made it.  Records are uniform over the workgroup.
    auto live = [&](int i) -> bool {
      const uint32_t* f = flags + ((size_t)i * BH + bh) * kFlagSlots;
      uint32_t x = 0u;
#pragma unroll
      for (int s = 0; s < D / 16; ++s) x |= f[s];
      return x != 0u;
    };
    bool have = false;  // the slice holds start(i)
    bool last_live = false;
    for (int i = 0; i < G; ++i) {
      last_live = live(i);
      if (!last_live) {
        have = false;
        continue;
      }
      if (!have) {
        slice_from(i == 0 ? (S_in ? S_in + hs : nullptr) : Z + ((size_t)(i - 1) * BH + bh) * D * D);
        __syncthreads();
        have = true;
      }
      f32x4 am[RPW][NT], b[NT], acc[RPW];
      load_m(am, i);
#pragma unroll
      for (int t = 0; t < NT; ++t) b[t] = sS[t][l];
      step(am, i, acc, b);
      __syncthreads();  // every wave has read the old slice
#pragma unroll
      for (int q = 0; q < RPW; ++q) sS[wave * RPW + q][l] = acc[q];
      if (i + 1 < G) {
        float* dst = S_start + ((size_t)(i + 1) * BH + bh) * D * D;
#pragma unroll
        for (int q = 0; q < RPW; ++q)
#pragma unroll
          for (int e = 0; e < 4; ++e) dst[at(wave * RPW + q, e)] = acc[q][e];
      }
      __syncthreads();
    }
    // S_T: the chain's last state, or the last segment's Z (S_in without segments)
    if (!last_live) {
      slice_from(G > 0 ? Z + ((size_t)(G - 1) * BH + bh) * D * D : (S_in ? S_in + hs : nullptr));
      __syncthreads();
    }
    slice_to_global(S_T + hs);
    return;
  }

  slice_from(S_in ? S_in + hs : nullptr);
  f32x4 am[RPW][NT];
  if (G > 0) load_m(am, 0);
  __syncthreads();

  for (int i = 0; i < G; ++i) {
    const size_t gs = ((size_t)i * BH + bh) * D * D;
    f32x4 b[NT];
#pragma unroll
    for (int t = 0; t < NT; ++t) b[t] = sS[t][l];
    if (S_start) {
#pragma unroll
      for (int q = 0; q < RPW; ++q)
#pragma unroll
        for (int e = 0; e < 4; ++e) S_start[gs + at(wave * RPW + q, e)] = b[wave * RPW + q][e];
    }
    f32x4 an[RPW][NT];
    if (i + 1 < G) load_m(an, i + 1);
    f32x4 acc[RPW];
    step(am, i, acc, b);
    __syncthreads();  // every wave has read the old slice
#pragma unroll
    for (int q = 0; q < RPW; ++q) sS[wave * RPW + q][l] = acc[q];
    __syncthreads();
    if (i + 1 < G) {
#pragma unroll
      for (int q = 0; q < RPW; ++q)
#pragma unroll
        for (int t = 0; t < NT; ++t) am[q][t] = an[q][t];
    }
  }
  slice_to_global(S_T + hs);
}

hipError_t launch_merge(const float* S_in, const float* Z, const float* M, float* S_start,
                        float* S_T, int BH, int G, int D, hipStream_t stream, const uint32_t* flags) {
  if (BH <= 0) return hipSuccess;
  const int nwg = BH * (D / 16);
  if (D == 128)
    hipLaunchKernelGGL((kda_merge_kernel<128>), dim3(nwg), dim3(256), 0, stream, S_in, Z, M, S_start, S_T, BH, G, flags);
  else if (D == 64)
    hipLaunchKernelGGL((kda_merge_kernel<64>), dim3(nwg), dim3(256), 0, stream, S_in, Z, M, S_start, S_T, BH, G, flags);
  else
    return hipErrorInvalidValue;
  return hipGetLastError();
}

}  // namespace kda
