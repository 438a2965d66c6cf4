// kda_launch.hpp -- internal argument blocks between the C ABI layer and the
// kernel launchers.  All pointers are device pointers already validated by
// the ABI layer (non-null where required, sizes in the supported set).
#pragma once

#include <atomic>

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
  // Segment-parallel passes (MFMA path only; the defaults give the plain call).
  // Segment p covers chunks [p seg_chunks, (p + 1) seg_chunks) of every sequence.
  int nseg = 1;
  int seg_chunks = 0;       // 0: the whole sequence
  bool S_in_seg = false;    // S_in is [B, H, nseg, dk, dv]: one entry state per segment
  int S_out_mode = 0;       // 0: [B, H, dk, dv]; 1: [B, H, nseg, dk, dv]; 2: last segment into [B, H, dk, dv]
  bool S_identity = false;  // every segment starts from the identity (dv == dk)
  bool v_zero = false;      // values taken as zero (v is not read)
  bool o_skip = false;      // outputs are not written
  // Fused prologue: q, k un-normalised and beta a logit (normalised / sigmoid in-kernel).
  bool prologue = false;
  // Checkpoints for the backward pass: the state entering every 64-token block,
  // [B, H, ceil(T / 64), dk, dv] (MFMA path: segment instantiation, one segment).
  float* S_ckpt = nullptr;
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
  bool prologue = false;  // q, k un-normalised and beta a logit
};

struct ReplayArgs {
  const void *q, *k, *v, *z, *beta;  // [n_draft, N, H, d], beta [n_draft, N, H]
  const float* A;
  float g_min;
  const float* S_snap;  // [N, H, dk, dv], read only
  void* o;              // [n_draft, N, H, dv]
  float* S_commit;      // [N, H, dk, dv]
  const int* accepted;  // [N]
  int n_draft, N, H, dk, dv;
  float scale;
  bool in_bf16, out_bf16;
};

// Thread layout shared by the single-token kernels (decode, replay): thread
// (rg, j4) owns value columns 4 j4 .. 4 j4 + 3 of rows rg + NR i, i < RPT.
constexpr int decode_threads(int dk, int dv) { return (dk * dv / 4) < 256 ? (dk * dv / 4) : 256; }

template <int DK, int DV>
struct DecodeShape {
  static constexpr int NJ = DV / 4;                                  // column groups
  static constexpr int NTHREADS = decode_threads(DK, DV);
  static constexpr int NR = NTHREADS / NJ;                           // row groups
  static constexpr int RPT = DK / NR;                                // rows per thread
  static_assert(NR * RPT == DK, "rows must split evenly");
  static_assert(NJ * NR == NTHREADS, "threads must split evenly");
};

// Entry states of the segments: E_0 = S_in (or 0), E_{p+1} = M_p E_p + St_p.
struct SegScanArgs {
  const float* S_in;  // [BH, dk, dv] or nullptr
  const float* St;    // [BH, nseg - 1, dk, dv], end states from the zero state
  const float* M;     // [BH, nseg - 1, dk, dk], segment transitions
  float* E;           // [BH, nseg, dk, dv]
  int BH, nseg, dk, dv;
};

hipError_t launch_segscan(const SegScanArgs& a, hipStream_t st);

// Raise a kernel's dynamic LDS limit on the current device, once per device (the
// setting is per device); `done` is the kernel's bit set of devices already set up.
inline hipError_t set_lds_limit(const void* kern, int bytes, std::atomic<uint64_t>& done) {
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  const uint64_t bit = (dev >= 0 && dev < 64) ? (uint64_t{1} << dev) : 0;
  if (bit && (done.load(std::memory_order_relaxed) & bit)) return hipSuccess;
  e = hipFuncSetAttribute(kern, hipFuncAttributeMaxDynamicSharedMemorySize, bytes);
  if (e == hipSuccess && bit) done.fetch_or(bit, std::memory_order_relaxed);
  return e;
}

// Backward pass of the fused-gate prefill (fp32 gradients).
struct BwdArgs {
  const void *q, *k, *v, *beta, *z;  // [B, T, H, d], beta [B, T, H]
  const float* A;                    // [H, dk]
  float g_min;
  const void* d_o;                   // [B, T, H, dv]
  const float* dS_out;               // [B, H, dk, dv] or nullptr
  const float* ckpt;                 // [B, H, nblk, dk, dv]: state entering each 64-token block
  float* scratch;                    // [B, H, 3, dk, dv]: states entering sub-chunks 1..3 of a block
  float* dA_part;                    // [B, H, dk]
  float *grad_q, *grad_k, *grad_v, *grad_beta, *grad_z;  // fp32 gradients, layouts of the inputs
  float* grad_A;                                          // [H, dk]
  float* grad_S_in;                                       // [B, H, dk, dv] or nullptr
  int B, T, H, dk, dv;
  float scale;
  bool in_bf16, do_bf16;
  // [B, H, slices, 3, 2, 16, 16]: M = (I + L)^-1 and AL of the sub-chunks a block's
  // recompute formed, reused by its backward sweep (nullptr: formed again)
  float* mcache = nullptr;
};
constexpr int kBwdMCacheFloats = 3 * 2 * 16 * 16;  // per (b, h, slice)
int chunk_bwd_slices(int B, int H, int dv);
hipError_t launch_chunk_bwd(const BwdArgs& a, hipStream_t st);
hipError_t launch_gate(const GateArgs& a, hipStream_t st);
hipError_t launch_replay(const ReplayArgs& a, hipStream_t st);
hipError_t launch_decode(const DecodeArgs& a, hipStream_t st);
hipError_t launch_chunk_generic(const ChunkArgs& a, hipStream_t st);
// The MFMA path for bf16 inputs, dk = dv = 128, chunk = 64.  Returns
// hipErrorNotSupported (launching nothing) for any other shape.
hipError_t launch_chunk_mfma(const ChunkArgs& a, hipStream_t st);
bool chunk_mfma_supports(const ChunkArgs& a);

}  // namespace kda
