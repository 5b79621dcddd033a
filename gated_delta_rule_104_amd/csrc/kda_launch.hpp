// Internal launch interface between the C-ABI layer (kda_api.hip) and the
// kernel translation units.  Host-side only types; no validation here.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>

namespace kda {

// One chunked pass over `G * BH` independent sequences of `Tseg` tokens each.
// Sequence s = g * BH + bh reads tokens [g*Tseg, (g+1)*Tseg) of head bh, whose
// rows start at token (bh * G + g) * Tseg of the [BH, G*Tseg, D] inputs.
struct ChunkArgs {
  const void* q;
  const void* k;
  const void* v;
  const void* la;
  const void* beta;
  const float* S0;  // prefill: start states [BH, D, D] or null
  void* o;          // prefill: outputs [BH, Tseg, D]
  float* S_out;     // prefill: S_T [BH, D, D]; segment pass: zero-start end states [G*BH, D, D]
  float* M_out;     // segment pass: transfer maps [G*BH, D, D]
  int BH;
  int G;
  int Tseg;
  int vsplit;       // workgroups per sequence (each owns 16*nc state columns)
};

// prefill: columns = D; segment pass: columns = 2*D (state + map).
// nc in {1, 2, 4}; nwg = G * BH * vsplit.
hipError_t launch_chunk(const ChunkArgs& a, bool bf16_io, int D, bool prefill, int nc, int nwg,
                        hipStream_t stream);

hipError_t launch_decode(const void* q, const void* k, const void* v, const void* la,
                         const void* beta, float* S, void* o, int NH, int D, bool bf16_io,
                         hipStream_t stream);

hipError_t launch_merge(const float* S_in, const float* Z, const float* M, float* S_start,
                        float* S_T, int BH, int G, int D, hipStream_t stream);

}  // namespace kda
