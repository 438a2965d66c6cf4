// kda_decode.hip -- single-token KDA state update, in place, HBM-streaming.
//
// One workgroup per (sequence n, head h).  The fp32 state S[n,h] (dk x dv,
// rows = key channels) is read from HBM once, held in registers, updated and
// written back once:
//   alpha = exp(g_min * sigmoid(exp(A) z))                 (gate, inline)
//   D     = Diag(alpha) S                                  (decay rows)
//   r     = D^T k,  y = D^T q                              (one pass, two reductions over rows)
//   S'    = D + beta k (x) (v - r)                          (erase + write, Eq. 1)
//   o     = scale * S'^T q = scale * (y + beta (v - r) (k . q))
// Sources: Eq. 1 and its factorised update -- "Kimi K3: the paper and proofs
// side by side", section 2.1.1; the gate -- "Kimi K3 reading notes", section 2.
//
// With the fused prologue (NORM), q and k arrive un-normalised and beta as a
// logit: the sums of squares of k and q ride the same LDS reduction as r, y
// and k.q, and the normalisation is applied to those sums (r, y and k.q are
// linear in k and q), so the state pass is unchanged.
//
// Thread layout: thread (rg, j4) owns 4 consecutive value columns 4*j4..+3
// (one 16-byte access per row) of the rows rg + NR*i, i < RPT.  A wavefront
// therefore reads 64/NJ whole rows per access: contiguous 512-byte runs at
// dv = 128.  Column partial sums are reduced through LDS.
#include "kda_common.hpp"
#include "kda_launch.hpp"

namespace kda {

template <int DK, int DV, typename Tin, typename Tout, bool NORM>
__global__ __launch_bounds__(decode_threads(DK, DV)) void decode_step_kernel(
    const Tin* __restrict__ q, const Tin* __restrict__ k, const Tin* __restrict__ v,
    const Tin* __restrict__ z, const Tin* __restrict__ beta, const float* __restrict__ A,
    float gmin_l2e, float* __restrict__ S, Tout* __restrict__ o, int H, float scale) {
  using Sh = DecodeShape<DK, DV>;
  const int nh = blockIdx.x;  // n * H + h
  const int h = nh % H;
  const int tid = threadIdx.x;
  const int j4 = tid % Sh::NJ;
  const int rg = tid / Sh::NJ;

  __shared__ float red_r[Sh::NR][DV];
  __shared__ float red_y[Sh::NR][DV];
  __shared__ float red_kq[Sh::NR];
  __shared__ float red_nn[NORM ? 2 : 1][Sh::NR];  // |k|^2, |q|^2 partial sums

  const int64_t tok = static_cast<int64_t>(nh);
  f32x4* Sp = reinterpret_cast<f32x4*>(S + tok * DK * DV);

  // Issue all state loads first (the HBM stream), then the small vectors.
  f32x4 s[Sh::RPT];
#pragma unroll
  for (int i = 0; i < Sh::RPT; ++i) {
    const int c = rg + Sh::NR * i;
    s[i] = __builtin_nontemporal_load(&Sp[c * Sh::NJ + j4]);
  }

  float kc[Sh::RPT], qc[Sh::RPT], ac[Sh::RPT];
#pragma unroll
  for (int i = 0; i < Sh::RPT; ++i) {
    const int c = rg + Sh::NR * i;
    kc[i] = io<Tin>::load(k, tok * DK + c);
    qc[i] = io<Tin>::load(q, tok * DK + c);
    const float ea = __expf(A[h * DK + c]) * kLog2e;
    ac[i] = fast_exp2(gate_log2(io<Tin>::load(z, tok * DK + c), ea, gmin_l2e));
  }
  const float bt = NORM ? sigmoid_fast(io<Tin>::load(beta, tok)) : io<Tin>::load(beta, tok);

  // Decay rows, then partial column sums r = D^T k and y = D^T q.
  float r[4] = {0.f, 0.f, 0.f, 0.f}, y[4] = {0.f, 0.f, 0.f, 0.f};
  float kq = 0.f, kk = 0.f, qq = 0.f;
#pragma unroll
  for (int i = 0; i < Sh::RPT; ++i) {
    if (NORM) {
      kk += kc[i] * kc[i];
      qq += qc[i] * qc[i];
    }
    s[i].x *= ac[i]; s[i].y *= ac[i]; s[i].z *= ac[i]; s[i].w *= ac[i];
    r[0] += kc[i] * s[i].x; r[1] += kc[i] * s[i].y; r[2] += kc[i] * s[i].z; r[3] += kc[i] * s[i].w;
    y[0] += qc[i] * s[i].x; y[1] += qc[i] * s[i].y; y[2] += qc[i] * s[i].z; y[3] += qc[i] * s[i].w;
    kq += kc[i] * qc[i];
  }
#pragma unroll
  for (int e = 0; e < 4; ++e) {
    red_r[rg][4 * j4 + e] = r[e];
    red_y[rg][4 * j4 + e] = y[e];
  }
  if (j4 == 0) {
    red_kq[rg] = kq;
    if (NORM) {
      red_nn[0][rg] = kk;
      red_nn[NORM ? 1 : 0][rg] = qq;
    }
  }
  __syncthreads();
  float rt[4] = {0.f, 0.f, 0.f, 0.f}, yt[4] = {0.f, 0.f, 0.f, 0.f};
  float kqt = 0.f;
#pragma unroll
  for (int g = 0; g < Sh::NR; ++g) {
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      rt[e] += red_r[g][4 * j4 + e];
      yt[e] += red_y[g][4 * j4 + e];
    }
    kqt += red_kq[g];
  }
  // prologue: r, y and k.q were formed with the raw k and q; rescale them, and the
  // key that writes the state, by 1 / sqrt(|x|^2 + eps)
  float rk = 1.f;
  if (NORM) {
    float kkt = 0.f, qqt = 0.f;
#pragma unroll
    for (int g = 0; g < Sh::NR; ++g) {
      kkt += red_nn[0][g];
      qqt += red_nn[NORM ? 1 : 0][g];
    }
    rk = rsqrt_fast(kkt + kL2Eps);
    const float rq = rsqrt_fast(qqt + kL2Eps);
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      rt[e] *= rk;
      yt[e] *= rq;
    }
    kqt *= rk * rq;
  }

  // Correction e_j = beta (v_j - r_j); S' = D + k (x) e.
  float ev[4];
#pragma unroll
  for (int e = 0; e < 4; ++e) ev[e] = bt * (io<Tin>::load(v, tok * DV + 4 * j4 + e) - rt[e]);
  float ek[4];  // the normalised key's factor folded into the correction
#pragma unroll
  for (int e = 0; e < 4; ++e) ek[e] = NORM ? rk * ev[e] : ev[e];
#pragma unroll
  for (int i = 0; i < Sh::RPT; ++i) {
    const int c = rg + Sh::NR * i;
    f32x4 t = s[i];
    t.x += kc[i] * ek[0]; t.y += kc[i] * ek[1]; t.z += kc[i] * ek[2]; t.w += kc[i] * ek[3];
    __builtin_nontemporal_store(t, &Sp[c * Sh::NJ + j4]);
  }
  if (rg == 0) {
#pragma unroll
    for (int e = 0; e < 4; ++e) io<Tout>::store(o, tok * DV + 4 * j4 + e, scale * (yt[e] + ev[e] * kqt));
  }
}

template <int DK, int DV, typename Tin, typename Tout>
static hipError_t launch_decode_t(const DecodeArgs& a, hipStream_t st) {
  using Sh = DecodeShape<DK, DV>;
  auto kern = a.prologue ? decode_step_kernel<DK, DV, Tin, Tout, true> : decode_step_kernel<DK, DV, Tin, Tout, false>;
  hipLaunchKernelGGL(kern, dim3(a.N * a.H), dim3(Sh::NTHREADS), 0, st,
                     static_cast<const Tin*>(a.q), static_cast<const Tin*>(a.k), static_cast<const Tin*>(a.v),
                     static_cast<const Tin*>(a.z), static_cast<const Tin*>(a.beta), a.A, a.g_min * kLog2e, a.S,
                     static_cast<Tout*>(a.o), a.H, a.scale);
  return hipGetLastError();
}

template <int DK, int DV>
static hipError_t launch_decode_d(const DecodeArgs& a, hipStream_t st) {
  if (a.in_bf16) {
    return a.out_bf16 ? launch_decode_t<DK, DV, bf16_t, bf16_t>(a, st) : launch_decode_t<DK, DV, bf16_t, float>(a, st);
  }
  return a.out_bf16 ? launch_decode_t<DK, DV, float, bf16_t>(a, st) : launch_decode_t<DK, DV, float, float>(a, st);
}

template <int DK>
static hipError_t launch_decode_k(const DecodeArgs& a, hipStream_t st) {
  switch (a.dv) {
    case 16: return launch_decode_d<DK, 16>(a, st);
    case 32: return launch_decode_d<DK, 32>(a, st);
    case 64: return launch_decode_d<DK, 64>(a, st);
    case 128: return launch_decode_d<DK, 128>(a, st);
  }
  return hipErrorInvalidValue;
}

hipError_t launch_decode(const DecodeArgs& a, hipStream_t st) {
  switch (a.dk) {
    case 16: return launch_decode_k<16>(a, st);
    case 32: return launch_decode_k<32>(a, st);
    case 64: return launch_decode_k<64>(a, st);
    case 128: return launch_decode_k<128>(a, st);
  }
  return hipErrorInvalidValue;
}

}  // namespace kda
