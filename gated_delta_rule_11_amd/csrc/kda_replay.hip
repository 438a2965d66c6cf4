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

template <int DK, int DV, typename Tin>
struct ReplayToken {
  using Sh = DecodeShape<DK, DV>;
  float kc[Sh::RPT], qc[Sh::RPT], zc[Sh::RPT], vc[4], bt;

  __device__ __forceinline__ void load(const Tin* q, const Tin* k, const Tin* v, const Tin* z, const Tin* beta,
                                       int64_t tok, int rg, int j4) {
#pragma unroll
    for (int i = 0; i < Sh::RPT; ++i) {
      const int c = rg + Sh::NR * i;
      kc[i] = io<Tin>::load(k, tok * DK + c);
      qc[i] = io<Tin>::load(q, tok * DK + c);
      zc[i] = io<Tin>::load(z, tok * DK + c);
    }
#pragma unroll
    for (int e = 0; e < 4; ++e) vc[e] = io<Tin>::load(v, tok * DV + 4 * j4 + e);
    bt = io<Tin>::load(beta, tok);
  }
};

template <int DK, int DV, typename Tin, typename Tout>
__global__ __launch_bounds__(decode_threads(DK, DV)) void replay_kernel(
    const Tin* __restrict__ q, const Tin* __restrict__ k, const Tin* __restrict__ v,
    const Tin* __restrict__ z, const Tin* __restrict__ beta, const float* __restrict__ A, float gmin_l2e,
    const float* __restrict__ S_snap, Tout* __restrict__ o, float* __restrict__ S_commit,
    const int* __restrict__ accepted, int n_draft, int N, int H, float scale) {
  using Sh = DecodeShape<DK, DV>;
  const int nh = blockIdx.x;  // n * H + h
  const int n = nh / H;
  const int h = nh % H;
  const int tid = threadIdx.x;
  const int j4 = tid % Sh::NJ;
  const int rg = tid / Sh::NJ;
  // accepted prefix length, clamped to [0, n_draft]
  const int m = min(max(accepted[n], 0), n_draft);

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
  float ea[Sh::RPT];
#pragma unroll
  for (int i = 0; i < Sh::RPT; ++i) ea[i] = __expf(A[h * DK + rg + Sh::NR * i]) * kLog2e;

  ReplayToken<DK, DV, Tin> cur, nxt;
  if (n_draft > 0) cur.load(q, k, v, z, beta, static_cast<int64_t>(n) * H + h, rg, j4);
  for (int t = 0; t < n_draft; ++t) {
    const int64_t tok = (static_cast<int64_t>(t) * N + n) * H + h;
    // the next drafted token's vectors are in flight while this one is processed
    if (t + 1 < n_draft) nxt.load(q, k, v, z, beta, tok + static_cast<int64_t>(N) * H, rg, j4);
    const int buf = t & 1;

    float r[4] = {0.f, 0.f, 0.f, 0.f}, y[4] = {0.f, 0.f, 0.f, 0.f};
    float kq = 0.f;
#pragma unroll
    for (int i = 0; i < Sh::RPT; ++i) {
      const float ac = fast_exp2(gate_log2(cur.zc[i], ea[i], gmin_l2e));
      s[i].x *= ac; s[i].y *= ac; s[i].z *= ac; s[i].w *= ac;
      r[0] += cur.kc[i] * s[i].x; r[1] += cur.kc[i] * s[i].y; r[2] += cur.kc[i] * s[i].z; r[3] += cur.kc[i] * s[i].w;
      y[0] += cur.qc[i] * s[i].x; y[1] += cur.qc[i] * s[i].y; y[2] += cur.qc[i] * s[i].z; y[3] += cur.qc[i] * s[i].w;
      kq += cur.kc[i] * cur.qc[i];
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
#pragma unroll
    for (int g = 0; g < Sh::NR; ++g) {
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        rt[e] += red_r[buf][g][4 * j4 + e];
        yt[e] += red_y[buf][g][4 * j4 + e];
      }
      kqt += red_kq[buf][g];
    }
    float ev[4];
#pragma unroll
    for (int e = 0; e < 4; ++e) ev[e] = cur.bt * (cur.vc[e] - rt[e]);
#pragma unroll
    for (int i = 0; i < Sh::RPT; ++i) {
      s[i].x += cur.kc[i] * ev[0]; s[i].y += cur.kc[i] * ev[1]; s[i].z += cur.kc[i] * ev[2]; s[i].w += cur.kc[i] * ev[3];
    }
    if (rg == 0) {
#pragma unroll
      for (int e = 0; e < 4; ++e) io<Tout>::store(o, tok * DV + 4 * j4 + e, scale * (yt[e] + ev[e] * kqt));
    }
    if (t + 1 == m) {
#pragma unroll
      for (int i = 0; i < Sh::RPT; ++i) __builtin_nontemporal_store(s[i], &Cp[(rg + Sh::NR * i) * Sh::NJ + j4]);
    }
    if (t + 1 < n_draft) cur = nxt;
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
