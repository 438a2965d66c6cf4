// kda_gate.hip -- bounded decay gate and chunk-local log-decay sums.
//
// G[b,t,h,c] = sum_{u = chunk start .. t} g_min * sigmoid(exp(A[h,c]) z[b,u,h,c])
// ("Kimi K3 reading notes", section 2: the scaled-sigmoid gate and its
// per-tile cumulative log-decay).  HBM-bound: 2 or 4 bytes in, 4 bytes out
// per element.
//
// One workgroup per (b, chunk, 256-element segment of a token row).  The
// H*dk elements of one token are contiguous, so a wavefront reads 64
// consecutive elements per token; each thread walks the chunk's tokens in
// order carrying its running sum.
#include "kda_common.hpp"
#include "kda_launch.hpp"

namespace kda {

template <typename Tin>
__global__ __launch_bounds__(256) void gate_kernel(const Tin* __restrict__ z, const float* __restrict__ A,
                                                   float gmin_l2e, float* __restrict__ G, int T, int HD,
                                                   int dk, int chunk, int nchunks, int nseg) {
  const int64_t bid = blockIdx.x;
  const int seg = static_cast<int>(bid % nseg);
  const int64_t rest = bid / nseg;
  const int ch = static_cast<int>(rest % nchunks);
  const int b = static_cast<int>(rest / nchunks);
  const int f = seg * 256 + static_cast<int>(threadIdx.x);  // element within the token row
  if (f >= HD) return;
  const int c = f % dk;
  const int h = f / dk;
  const float ea = __expf(A[h * dk + c]) * kLog2e;
  const int t0 = ch * chunk;
  const int t1 = min(T, t0 + chunk);
  float run = 0.f;  // log2 units
  for (int t = t0; t < t1; ++t) {
    const int64_t i = (static_cast<int64_t>(b) * T + t) * HD + f;
    run += gate_log2(io<Tin>::load(z, i), ea, gmin_l2e);
    G[i] = run * (1.0f / kLog2e);
  }
}

hipError_t launch_gate(const GateArgs& a, hipStream_t st) {
  const int HD = a.H * a.dk;
  const int nseg = (HD + 255) / 256;
  const int nchunks = (a.T + a.chunk - 1) / a.chunk;
  const int64_t nblocks = static_cast<int64_t>(a.B) * nchunks * nseg;
  if (nblocks == 0) return hipSuccess;
  if (nblocks > 0x7fffffffLL) return hipErrorInvalidConfiguration;
  const float gmin_l2e = a.g_min * kLog2e;
  if (a.z_bf16) {
    hipLaunchKernelGGL(gate_kernel<bf16_t>, dim3(static_cast<uint32_t>(nblocks)), dim3(256), 0, st,
                       static_cast<const bf16_t*>(a.z), a.A, gmin_l2e, a.G, a.T, HD, a.dk, a.chunk, nchunks, nseg);
  } else {
    hipLaunchKernelGGL(gate_kernel<float>, dim3(static_cast<uint32_t>(nblocks)), dim3(256), 0, st,
                       static_cast<const float*>(a.z), a.A, gmin_l2e, a.G, a.T, HD, a.dk, a.chunk, nchunks, nseg);
  }
  return hipGetLastError();
}

}  // namespace kda
