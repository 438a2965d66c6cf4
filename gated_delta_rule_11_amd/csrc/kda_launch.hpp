// kda_launch.hpp -- internal argument blocks between the C ABI layer and the
// kernel launchers.  All pointers are device pointers already validated by
// the ABI layer (non-null where required, sizes in the supported set).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace kda {

struct GateArgs {
  const void* z;
  const float* A;
  float g_min;
  float* G;
  int B, T, H, dk, chunk;
  bool z_bf16;
};

struct ChunkArgs {
  const void *q, *k, *v, *beta;
  const float* G;   // chunk-local sums (natural log) or nullptr when from_z
  const void* z;    // decay logits when from_z
  const float* A;
  float g_min;
  const float* S_in;  // may be nullptr (zero state)
  void* o;
  float* S_out;       // may be nullptr
  int B, T, H, dk, dv, chunk;
  float scale;
  bool in_bf16, out_bf16, from_z;
};

struct DecodeArgs {
  const void *q, *k, *v, *z, *beta;
  const float* A;
  float g_min;
  float* S;
  void* o;
  int N, H, dk, dv;
  float scale;
  bool in_bf16, out_bf16;
};

hipError_t launch_gate(const GateArgs& a, hipStream_t st);
hipError_t launch_decode(const DecodeArgs& a, hipStream_t st);
hipError_t launch_chunk_generic(const ChunkArgs& a, hipStream_t st);
// The MFMA path for bf16 inputs, dk = dv = 128, chunk = 64.  Returns
// hipErrorNotSupported (launching nothing) for any other shape.
hipError_t launch_chunk_mfma(const ChunkArgs& a, hipStream_t st);
bool chunk_mfma_supports(const ChunkArgs& a);

}  // namespace kda
