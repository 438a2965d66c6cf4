// kda_segscan.hip -- entry states of the segments of a segment-parallel prefill.
//
// The fragment decomposition of "Kimi K3 reading notes", section 7: run from
// the zero state, segment p ends in S~_p; its transition (the map applied to
// an entry state, the product of the per-token maps (I - beta k k^T) Diag(alpha))
// is M_p.  The true entry states follow by a prefix scan over segments,
//   E_0 = S_in,  E_{p+1} = M_p E_p + S~_p.
// Layouts: St [BH, nseg - 1, dk, dv] and M [BH, nseg - 1, dk, dk] (the last
// segment's are never needed), E [BH, nseg, dk, dv].
//
// One workgroup per (b, h, 16-column block of the state), dk / 16 wavefronts,
// one 16-row tile of the block each.  Every column block of a head reads all of
// M_p, so the blocks of a head are given consecutive workgroup slots on one XCD
// (workgroups are dealt to the eight XCDs in turn): M_p then comes from HBM into
// one L2 per step instead of into eight.  Each step is a dk-deep product on fp32
// matrix cores (v_mfma_f32_16x16x4_f32): the wavefront's rows of M_p from global
// memory (fetched during the previous step), the column block of E_p from LDS,
// where it is kept transposed (column-major); two LDS copies alternate, so a
// step has one barrier.  Lane group g of a wavefront takes k = 16 q + 4 g ..
// 16 q + 4 g + 3 of its row in product q, so that one 16-byte load per lane reads
// 64 contiguous bytes of each of the 16 rows (with k = (dk / 4) g + ..., each
// load touched 64 separate lines and the address unit, not memory, bounded the
// step).  The steps are sequential; the loads of step p + 1 are in flight during
// step p.
#include <climits>

#include "kda_common.hpp"
#include "kda_launch.hpp"

namespace kda {

constexpr int kScanCols = 16;

template <int DK>
__global__ __launch_bounds__(DK * 4) void segscan_kernel(const float* __restrict__ S_in, const float* __restrict__ St,
                                                          const float* __restrict__ M, float* __restrict__ E, int nseg,
                                                          int dv, int nwork) {
  constexpr int ES = DK + 4;  // floats per transposed column (16-byte aligned rows)
  constexpr int KQ = DK / 16;  // products (16-byte groups of k) per lane
  const int ncb = dv / kScanCols;
  // work item of this workgroup: slot blockIdx / 8 of XCD blockIdx % 8 (the grid is a
  // multiple of 8; surplus workgroups leave at once)
  const int per_xcd = static_cast<int>(gridDim.x) / 8;
  const int wi = (blockIdx.x % 8) * per_xcd + blockIdx.x / 8;
  if (wi >= nwork) return;
  const int bh = wi / ncb;
  const int c0 = (wi % ncb) * kScanCols;
  const int w = threadIdx.x >> 6;  // row tile: rows 16 w .. 16 w + 15
  const int l = threadIdx.x & 63;
  const int lr = l & 15, lg = l >> 4;
  __shared__ __attribute__((aligned(16))) float ET[2][kScanCols][ES];

  const int64_t sz = static_cast<int64_t>(DK) * dv;
  // this lane's four outputs of the tile: rows 16 w + 4 lg + v, column c0 + lr
  const int64_t out0 = static_cast<int64_t>(16 * w + 4 * lg) * dv + c0 + lr;
  f32x4 e;
#pragma unroll
  for (int v = 0; v < 4; ++v) e[v] = S_in ? S_in[bh * sz + out0 + static_cast<int64_t>(v) * dv] : 0.f;

  // A operands of step p: M_p[16 w + lr][16 q + 4 lg + u]; B: E_p[16 q + 4 lg + u][c0 + lr] (q < KQ, u < 4)
  f32x4 a_nx[KQ], s_nx;
  auto fetch = [&](int p) __attribute__((always_inline)) {
    const int64_t sm = static_cast<int64_t>(bh) * (nseg - 1) + p;
    const f32x4* mr =
        reinterpret_cast<const f32x4*>(M + sm * DK * DK + static_cast<int64_t>(16 * w + lr) * DK + 4 * lg);
#pragma unroll
    for (int q = 0; q < KQ; ++q) a_nx[q] = mr[4 * q];
#pragma unroll
    for (int v = 0; v < 4; ++v) s_nx[v] = St[sm * sz + out0 + static_cast<int64_t>(v) * dv];
  };
  if (nseg > 1) fetch(0);

  for (int p = 0; p < nseg; ++p) {
    const int64_t seg = static_cast<int64_t>(bh) * nseg + p;
#pragma unroll
    for (int v = 0; v < 4; ++v) E[seg * sz + out0 + static_cast<int64_t>(v) * dv] = e[v];
    if (p + 1 == nseg) break;
    // E_p's column block, transposed, into this step's LDS copy
    float(*et)[ES] = ET[p & 1];
    *reinterpret_cast<f32x4*>(&et[lr][16 * w + 4 * lg]) = e;
    __syncthreads();
    f32x4 a[KQ];
#pragma unroll
    for (int q = 0; q < KQ; ++q) a[q] = a_nx[q];
    const f32x4 st = s_nx;
    if (p + 2 < nseg) fetch(p + 1);
    const f32x4* br = reinterpret_cast<const f32x4*>(&et[lr][4 * lg]);
    // four independent accumulators (k = 16 q + 4 lg + u by u) shorten the dependent
    // chain of products four times; they are summed at the end, in a fixed order
    f32x4 acc[4];
#pragma unroll
    for (int u = 0; u < 4; ++u) acc[u] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int q = 0; q < KQ; ++q) {
      const f32x4 b = br[4 * q];
#pragma unroll
      for (int u = 0; u < 4; ++u) acc[u] = __builtin_amdgcn_mfma_f32_16x16x4f32(a[q][u], b[u], acc[u], 0, 0, 0);
    }
    e = st + ((acc[0] + acc[1]) + (acc[2] + acc[3]));
  }
}

template <int DK>
static hipError_t launch_segscan_k(const SegScanArgs& a, hipStream_t st, int64_t nwg) {
  const int64_t grid = (nwg + 7) / 8 * 8;
  hipLaunchKernelGGL(segscan_kernel<DK>, dim3(static_cast<uint32_t>(grid)), dim3(DK * 4), 0, st, a.S_in, a.St, a.M,
                     a.E, a.nseg, a.dv, static_cast<int>(nwg));
  return hipGetLastError();
}

hipError_t launch_segscan(const SegScanArgs& a, hipStream_t st) {
  if (a.dv % kScanCols) return hipErrorNotSupported;
  const int64_t nwg = static_cast<int64_t>(a.BH) * (a.dv / kScanCols);
  if (nwg == 0 || a.nseg < 1) return hipSuccess;
  if (nwg > INT_MAX - 8) return hipErrorInvalidValue;
  switch (a.dk) {
    case 16: return launch_segscan_k<16>(a, st, nwg);
    case 32: return launch_segscan_k<32>(a, st, nwg);
    case 64: return launch_segscan_k<64>(a, st, nwg);
    case 128: return launch_segscan_k<128>(a, st, nwg);
  }
  return hipErrorNotSupported;
}

}  // namespace kda
