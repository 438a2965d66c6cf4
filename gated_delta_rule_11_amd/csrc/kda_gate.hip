// kda_gate.hip -- bounded decay gate and chunk-local log-decay sums.
//
// G[b,t,h,c] = sum_{u = chunk start .. t} g_min * sigmoid(exp(A[h,c]) z[b,u,h,c])
// ("Kimi K3 reading notes", section 2: the scaled-sigmoid gate and its
// per-tile cumulative log-decay).  HBM-bound: 2 or 4 bytes in, 4 bytes out
// per element.
//
// One workgroup per (b, chunk, 1024-element segment of a token row); each thread
// owns four consecutive elements of the row (one 8- or 16-byte load and one
// 16-byte store per token), walks the chunk's tokens in order carrying the four
// running sums, and issues the loads of eight tokens before it uses them, so that
// the loads of a thread overlap instead of waiting one token at a time.  Loads and
// stores are non-temporal: every byte is touched once, so nothing is kept in cache.
#include "kda_common.hpp"
#include "kda_launch.hpp"

namespace kda {

template <typename Tin> struct quad;
template <> struct quad<float> {
  typedef f32x4 raw;
  __device__ __forceinline__ static raw load(const float* p, int64_t i) {
    return __builtin_nontemporal_load(reinterpret_cast<const f32x4*>(p + i));
  }
  __device__ __forceinline__ static float at(const raw& r, int e) { return r[e]; }
};
template <> struct quad<bf16_t> {
  typedef uint32_t raw __attribute__((ext_vector_type(2)));
  __device__ __forceinline__ static raw load(const bf16_t* p, int64_t i) {
    return __builtin_nontemporal_load(reinterpret_cast<const raw*>(p + i));
  }
  __device__ __forceinline__ static float at(const raw& r, int e) {
    const uint32_t w = r[e >> 1];
    return __uint_as_float((e & 1) ? (w & 0xffff0000u) : (w << 16));
  }
};

constexpr int kGateSeg = 1024;  // row elements per workgroup (256 threads x 4)
constexpr int kGateAhead = 8;   // tokens whose loads are issued before their use

template <typename Tin>
__global__ __launch_bounds__(256) void gate_kernel(const Tin* __restrict__ z, const float* __restrict__ A,
                                                   float gmin_l2e, float* __restrict__ G, int T, int HD,
                                                   int dk, int chunk, int nchunks, int nseg) {
  using Q = quad<Tin>;
  const int64_t bid = blockIdx.x;
  const int seg = static_cast<int>(bid % nseg);
  const int64_t rest = bid / nseg;
  const int ch = static_cast<int>(rest % nchunks);
  const int b = static_cast<int>(rest / nchunks);
  const int f = seg * kGateSeg + 4 * static_cast<int>(threadIdx.x);  // first of the thread's four elements
  if (f >= HD) return;  // HD is a multiple of 16: a thread's four elements are all in the row or none
  const int h = f / dk, c = f % dk;  // c .. c + 3 lie in head h (dk is a multiple of 16)
  float ea[4];
#pragma unroll
  for (int e = 0; e < 4; ++e) ea[e] = __expf(A[h * dk + c + e]) * kLog2e;
  const int t0 = ch * chunk;
  const int t1 = min(T, t0 + chunk);
  const int64_t row0 = static_cast<int64_t>(b) * T;
  float run[4] = {0.f, 0.f, 0.f, 0.f};  // log2 units
  auto step = [&](const typename Q::raw& r, int t) {
    f32x4 out;
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      run[e] += gate_log2(Q::at(r, e), ea[e], gmin_l2e);
      out[e] = run[e] * (1.0f / kLog2e);
    }
    __builtin_nontemporal_store(out, reinterpret_cast<f32x4*>(G + (row0 + t) * HD + f));
  };
  int t = t0;
  for (; t + kGateAhead <= t1; t += kGateAhead) {
    typename Q::raw r[kGateAhead];
#pragma unroll
    for (int u = 0; u < kGateAhead; ++u) r[u] = Q::load(z, (row0 + t + u) * HD + f);
#pragma unroll
    for (int u = 0; u < kGateAhead; ++u) step(r[u], t + u);
  }
  for (; t < t1; ++t) step(Q::load(z, (row0 + t) * HD + f), t);
}

hipError_t launch_gate(const GateArgs& a, hipStream_t st) {
  const int HD = a.H * a.dk;
  const int nseg = (HD + kGateSeg - 1) / kGateSeg;
  const int nchunks = (a.T + a.chunk - 1) / a.chunk;
  const int64_t nblocks = static_cast<int64_t>(a.B) * nchunks * nseg;
  if (nblocks == 0) return hipSuccess;
  if (nblocks > 0x7fffffffLL) return hipErrorInvalidConfiguration;
  if (a.dk % 16 != 0) return hipErrorInvalidValue;  // every supported dk is a multiple of 16
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
