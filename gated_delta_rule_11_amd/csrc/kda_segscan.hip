// kda_segscan.hip -- entry states of the segments of a segment-parallel prefill.
//
// The fragment decomposition of "Kimi K3 reading notes", section 7: run from
// the zero state, segment p ends in S~_p; its transition (the map applied to
// an entry state, the product of the per-token maps (I - beta k k^T) Diag(alpha))
// is M_p.  The true entry states follow by a prefix scan over segments,
//   E_0 = S_in,  E_{p+1} = M_p E_p + S~_p,
// here in fp32, one workgroup per (b, h, 16-column block of the state), the
// column block of E held in LDS while the segments are walked in order.
// Layouts: St [BH, nseg - 1, dk, dv] and M [BH, nseg - 1, dk, dk] (the last
// segment's are never needed), E [BH, nseg, dk, dv].
#include "kda_common.hpp"
#include "kda_launch.hpp"

namespace kda {

constexpr int kScanCols = 16;

template <int DK>
__global__ __launch_bounds__(256) void segscan_kernel(const float* __restrict__ S_in, const float* __restrict__ St,
                                                       const float* __restrict__ M, float* __restrict__ E, int nseg,
                                                       int dv) {
  static_assert(DK * kScanCols == 256 * 8, "256 threads x 8 outputs");
  const int ncb = dv / kScanCols;
  const int bh = blockIdx.x / ncb;
  const int cb = blockIdx.x % ncb;
  const int tid = threadIdx.x;
  const int r = tid >> 1;          // state row (key channel)
  const int c8 = (tid & 1) * 8;    // first of this thread's 8 columns in the block
  __shared__ float Eb[DK][kScanCols];

  const int64_t sz = static_cast<int64_t>(DK) * dv;
  float e[8];
#pragma unroll
  for (int j = 0; j < 8; ++j)
    e[j] = S_in ? S_in[static_cast<int64_t>(bh) * sz + static_cast<int64_t>(r) * dv + cb * kScanCols + c8 + j] : 0.f;
  for (int p = 0; p < nseg; ++p) {
    const int64_t seg = static_cast<int64_t>(bh) * nseg + p;        // in E
    const int64_t sm = static_cast<int64_t>(bh) * (nseg - 1) + p;   // in St and M (p < nseg - 1 below)
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      E[seg * sz + static_cast<int64_t>(r) * dv + cb * kScanCols + c8 + j] = e[j];
      Eb[r][c8 + j] = e[j];
    }
    if (p + 1 == nseg) break;
    __syncthreads();
    const float* Mr = M + sm * DK * DK + static_cast<int64_t>(r) * DK;
    const float* Sr = St + sm * sz + static_cast<int64_t>(r) * dv + cb * kScanCols + c8;
    float acc[8];
#pragma unroll
    for (int j = 0; j < 8; ++j) acc[j] = Sr[j];
    for (int kk = 0; kk < DK; kk += 4) {
      const f32x4 m4 = *reinterpret_cast<const f32x4*>(Mr + kk);
#pragma unroll
      for (int q = 0; q < 4; ++q)
#pragma unroll
        for (int j = 0; j < 8; ++j) acc[j] += m4[q] * Eb[kk + q][c8 + j];
    }
    __syncthreads();
#pragma unroll
    for (int j = 0; j < 8; ++j) e[j] = acc[j];
  }
}

hipError_t launch_segscan(const SegScanArgs& a, hipStream_t st) {
  if (a.dk != 128 || a.dv % kScanCols) return hipErrorNotSupported;
  const int64_t nwg = static_cast<int64_t>(a.BH) * (a.dv / kScanCols);
  if (nwg == 0) return hipSuccess;
  hipLaunchKernelGGL(segscan_kernel<128>, dim3(static_cast<uint32_t>(nwg)), dim3(256), 0, st, a.S_in, a.St, a.M,
                     a.E, a.nseg, a.dv);
  return hipGetLastError();
}

}  // namespace kda
