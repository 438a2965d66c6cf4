// kda_replay.hip -- speculative-decoding state replay in one launch.
//
// "Kimi K3: architecture, derivations and a pinned-source audit", section
// 10.3: the drafted tokens' inputs are cached, the state before the drafts is
// kept as a snapshot, and after verification the accepted prefix is replayed
// on chip.  One workgroup per (sequence n, head h) reads its fp32 state slice
// from the snapshot once, keeps it in registers across all n_draft drafted
// tokens (each step is the decode update of Eq. 1, "Kimi K3: the paper and
// proofs side by side", section 2.1.1, with the gate of "Kimi K3 reading
// notes", section 2), writes every drafted token's output, and stores the
// state to S_commit once, right after the step that completes the accepted
// prefix (before the first step when nothing is accepted).  The snapshot is
// never written.  HBM traffic per (n, h): one state read and one state write
// plus the drafted tokens' vectors, against n_draft of each for n_draft
// separate decode steps.
#include "kda_common.hpp"
#include "kda_launch.hpp"

namespace kda {

// Drafted tokens staged in LDS per group: their keys, queries, decays and values are
// read from HBM once per workgroup (coalesced, one element per thread) instead of by
// every thread that uses them, and each decay is formed once instead of once per
// value-column group.
constexpr int kReplayGroup = 8;

template <int DK, int DV, typename Tin, typename Tout>
__global__ __launch_bounds__(decode_threads(DK, DV), 3) void replay_kernel(
    const Tin* __restrict__ q, const Tin* __restrict__ k, const Tin* __restrict__ v,
    const Tin* __restrict__ z, const Tin* __restrict__ beta, const float* __restrict__ A, float gmin_l2e,
    const float* __restrict__ S_snap, Tout* __restrict__ o, float* __restrict__ S_commit,
    const int* __restrict__ accepted, int n_draft, int N, int H, float scale) {
  using Sh = DecodeShape<DK, DV>;
  constexpr int DG = kReplayGroup;
  const int nh = blockIdx.x;  // n * H + h
  const int n = nh / H;
  const int h = nh % H;
  const int tid = threadIdx.x;
  // thread (rg, j4) owns value columns 4 j4 .. 4 j4 + 3 of rows rg + NR i (the decode
  // step's layout, so that replaying a draft gives bit for bit what a decode step
  // gives); the staged keys, queries and decays are stored permuted, channel c at
  // position (c % NR) RPT + c / NR, so that a thread's rows are contiguous in LDS
  const int j4 = tid % Sh::NJ;
  const int rg = tid / Sh::NJ;
  const int r0 = Sh::RPT * rg;
  // accepted prefix length, clamped to [0, n_draft]
  const int m = min(max(accepted[n], 0), n_draft);

  __shared__ __attribute__((aligned(16))) float kS[DG][DK];
  __shared__ __attribute__((aligned(16))) float qS[DG][DK];
  __shared__ __attribute__((aligned(16))) float aS[DG][DK];  // decays alpha
  __shared__ __attribute__((aligned(16))) float vS[DG][DV];
  __shared__ float bS[DG];
  __shared__ float eaS[DK];  // e^A log2 e
  // two sets of reduction slots, alternating between steps: one barrier per step
  __shared__ float red_r[2][Sh::NR][DV];
  __shared__ float red_y[2][Sh::NR][DV];
  __shared__ float red_kq[2][Sh::NR];

  const f32x4* Sp = reinterpret_cast<const f32x4*>(S_snap + static_cast<int64_t>(nh) * DK * DV);
  f32x4* Cp = reinterpret_cast<f32x4*>(S_commit + static_cast<int64_t>(nh) * DK * DV);
  f32x4 s[Sh::RPT];
#pragma unroll
  for (int i = 0; i < Sh::RPT; ++i) s[i] = __builtin_nontemporal_load(&Sp[(rg + Sh::NR * i) * Sh::NJ + j4]);
  if (m == 0) {
#pragma unroll
    for (int i = 0; i < Sh::RPT; ++i) __builtin_nontemporal_store(s[i], &Cp[(rg + Sh::NR * i) * Sh::NJ + j4]);
  }
  for (int c = tid; c < DK; c += Sh::NTHREADS) eaS[c] = __expf(A[h * DK + c]) * kLog2e;

  for (int g0 = 0; g0 < n_draft; g0 += DG) {
    const int nd = min(DG, n_draft - g0);
    __syncthreads();  // the previous group's staged values are no longer read (and eaS is written)
    for (int e = tid; e < nd * DK; e += Sh::NTHREADS) {
      const int t = e / DK, c = e % DK;
      const int pc = (c % Sh::NR) * Sh::RPT + c / Sh::NR;
      const int64_t tok = (static_cast<int64_t>(g0 + t) * N + n) * H + h;
      kS[t][pc] = io<Tin>::load(k, tok * DK + c);
      qS[t][pc] = io<Tin>::load(q, tok * DK + c);
      aS[t][pc] = fast_exp2(gate_log2(io<Tin>::load(z, tok * DK + c), eaS[c], gmin_l2e));
    }
    for (int e = tid; e < nd * DV; e += Sh::NTHREADS) {
      const int t = e / DV, j = e % DV;
      vS[t][j] = io<Tin>::load(v, ((static_cast<int64_t>(g0 + t) * N + n) * H + h) * DV + j);
    }
    if (tid < nd) bS[tid] = io<Tin>::load(beta, (static_cast<int64_t>(g0 + tid) * N + n) * H + h);
    __syncthreads();

    for (int t = 0; t < nd; ++t) {
      const int tg = g0 + t;
      const int64_t tok = (static_cast<int64_t>(tg) * N + n) * H + h;
      const int buf = tg & 1;
      float r[4] = {0.f, 0.f, 0.f, 0.f}, y[4] = {0.f, 0.f, 0.f, 0.f};
      float kq = 0.f;
#pragma unroll
      for (int i = 0; i < Sh::RPT; ++i) {
        // the staged rows are read eight at a time: reading all 48 values ahead of the
        // products (the compiler's choice) kept the kernel at two wavefronts per SIMD
        // instead of the three the launch bound asks for
        if (i % 8 == 0 && i > 0) asm volatile("" ::: "memory");
        const float ac = aS[t][r0 + i], kc = kS[t][r0 + i], qc = qS[t][r0 + i];
        s[i].x *= ac; s[i].y *= ac; s[i].z *= ac; s[i].w *= ac;
        r[0] += kc * s[i].x; r[1] += kc * s[i].y; r[2] += kc * s[i].z; r[3] += kc * s[i].w;
        y[0] += qc * s[i].x; y[1] += qc * s[i].y; y[2] += qc * s[i].z; y[3] += qc * s[i].w;
        kq += kc * qc;
      }
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        red_r[buf][rg][4 * j4 + e] = r[e];
        red_y[buf][rg][4 * j4 + e] = y[e];
      }
      if (j4 == 0) red_kq[buf][rg] = kq;
      __syncthreads();
      float rt[4] = {0.f, 0.f, 0.f, 0.f}, yt[4] = {0.f, 0.f, 0.f, 0.f};
      float kqt = 0.f;
#pragma unroll 2
      for (int gg = 0; gg < Sh::NR; ++gg) {
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          rt[e] += red_r[buf][gg][4 * j4 + e];
          yt[e] += red_y[buf][gg][4 * j4 + e];
        }
        kqt += red_kq[buf][gg];
      }
      const float bt = bS[t];
      float ev[4];
#pragma unroll
      for (int e = 0; e < 4; ++e) ev[e] = bt * (vS[t][4 * j4 + e] - rt[e]);
#pragma unroll
      for (int i = 0; i < Sh::RPT; ++i) {
        const float kc = kS[t][r0 + i];
        s[i].x += kc * ev[0]; s[i].y += kc * ev[1]; s[i].z += kc * ev[2]; s[i].w += kc * ev[3];
      }
      if (rg == 0) {
#pragma unroll
        for (int e = 0; e < 4; ++e) io<Tout>::store(o, tok * DV + 4 * j4 + e, scale * (yt[e] + ev[e] * kqt));
      }
      if (tg + 1 == m) {
#pragma unroll
        for (int i = 0; i < Sh::RPT; ++i) __builtin_nontemporal_store(s[i], &Cp[(rg + Sh::NR * i) * Sh::NJ + j4]);
      }
    }
  }
}

template <int DK, int DV, typename Tin, typename Tout>
static hipError_t launch_replay_t(const ReplayArgs& a, hipStream_t st) {
  using Sh = DecodeShape<DK, DV>;
  hipLaunchKernelGGL((replay_kernel<DK, DV, Tin, Tout>), dim3(a.N * a.H), dim3(Sh::NTHREADS), 0, st,
                     static_cast<const Tin*>(a.q), static_cast<const Tin*>(a.k), static_cast<const Tin*>(a.v),
                     static_cast<const Tin*>(a.z), static_cast<const Tin*>(a.beta), a.A, a.g_min * kLog2e, a.S_snap,
                     static_cast<Tout*>(a.o), a.S_commit, a.accepted, a.n_draft, a.N, a.H, a.scale);
  return hipGetLastError();
}

template <int DK, int DV>
static hipError_t launch_replay_d(const ReplayArgs& a, hipStream_t st) {
  if (a.in_bf16)
    return a.out_bf16 ? launch_replay_t<DK, DV, bf16_t, bf16_t>(a, st) : launch_replay_t<DK, DV, bf16_t, float>(a, st);
  return a.out_bf16 ? launch_replay_t<DK, DV, float, bf16_t>(a, st) : launch_replay_t<DK, DV, float, float>(a, st);
}

template <int DK>
static hipError_t launch_replay_k(const ReplayArgs& a, hipStream_t st) {
  switch (a.dv) {
    case 16: return launch_replay_d<DK, 16>(a, st);
    case 32: return launch_replay_d<DK, 32>(a, st);
    case 64: return launch_replay_d<DK, 64>(a, st);
    case 128: return launch_replay_d<DK, 128>(a, st);
  }
  return hipErrorInvalidValue;
}

hipError_t launch_replay(const ReplayArgs& a, hipStream_t st) {
  switch (a.dk) {
    case 16: return launch_replay_k<16>(a, st);
    case 32: return launch_replay_k<32>(a, st);
    case 64: return launch_replay_k<64>(a, st);
    case 128: return launch_replay_k<128>(a, st);
  }
  return hipErrorInvalidValue;
}

}  // namespace kda
