// kda_chunk_generic.hip -- chunked KDA prefill for every supported shape and
// dtype, fp32 arithmetic on the vector ALUs.
//
// This is the path for fp32 inputs, for dk or dv below 128 and for chunk 16.
// It runs the chunkwise regrouping of Eq. 1 on sub-chunks of SC = 16 tokens
// (the 16-token tile of "Kimi K3 reading notes", section 2) with the state
// carried between sub-chunks.  A sub-chunk never straddles a chunk of the API
// (16 divides 16 and 64), so G's chunk-local sums give every decay ratio
// inside it.
//
// Algebra (derived from Eq. 1, "Kimi K3: the paper and proofs side by side",
// section 2.1.1; the regrouping is the chunkwise form that "Kimi K3:
// architecture, derivations and a pinned-source audit", section 4.5 names).
// Inside a sub-chunk with entry state S, per key channel c, with Gl_t the
// log-decay summed from the sub-chunk start through token t:
//   L[t,s] = beta_t sum_c k_tc k_sc 2^(Gl_tc - Gl_sc)      s < t
//   Tm     = (I + L)^-1 Diag(beta)                           (forward substitution)
//   W      = Tm (K * 2^Gl),  Ut = Tm V,  U = Ut - W S
//   P[t,s] = sum_c q_tc k_sc 2^(Gl_tc - Gl_sc)               s <= t
//   o      = scale ((Q * 2^Gl) S + P U)
//   S     <- Diag(2^Gl_last) S + (K * 2^(Gl_last - Gl))^T U
// Every power of two above has a non-positive exponent: Gl is non-increasing
// in t, so no overflow is possible for any g.
//
// Fused prologue (a.prologue): q and k arrive un-normalised and beta as a
// logit; each sub-chunk's rows are divided by sqrt(|x|^2 + 1e-6) in LDS and
// beta goes through the sigmoid, before any of the above.
//
// One workgroup (256 threads) per (b, h, slice of DVS value columns).  The
// value columns of the state evolve independently given (k, beta, alpha), so
// slicing changes no arithmetic.
#include "kda_common.hpp"
#include "kda_launch.hpp"

namespace kda {

namespace {
constexpr int SC = 16;
constexpr int NT = 256;
}  // namespace

template <int DK, int DVS, typename Tin, typename Tout, bool FROM_Z>
__global__ __launch_bounds__(NT) void chunk_generic_kernel(const ChunkArgs a) {
  const int nsl = a.dv / DVS;
  const int sl = blockIdx.x % nsl;
  const int bh = blockIdx.x / nsl;
  const int h = bh % a.H;
  const int b = bh / a.H;
  const int tid = threadIdx.x;
  const int j0 = sl * DVS;

  const Tin* q = static_cast<const Tin*>(a.q);
  const Tin* k = static_cast<const Tin*>(a.k);
  const Tin* v = static_cast<const Tin*>(a.v);
  const Tin* beta = static_cast<const Tin*>(a.beta);
  const Tin* z = static_cast<const Tin*>(a.z);
  Tout* o = static_cast<Tout*>(a.o);

  __shared__ float Ks[SC][DK], Qs[SC][DK], Gl[SC][DK], Ws[SC][DK];
  __shared__ float Vs[SC][DVS], Us[SC][DVS];
  __shared__ float Lm[SC][SC], Pm[SC][SC], Tm[SC][SC];
  __shared__ float bs[SC];
  __shared__ float rn[2][SC];  // prologue: 1 / sqrt(|k|^2 + eps), 1 / sqrt(|q|^2 + eps) per token
  __shared__ float Ss[DK][DVS];
  __shared__ float eaL[DK];

  const int64_t HDV = static_cast<int64_t>(a.H) * a.dv;
  const int64_t state_off = static_cast<int64_t>(bh) * DK * a.dv;
  const float gmin_l2e = a.g_min * kLog2e;

  for (int e = tid; e < DK * DVS; e += NT) {
    const int c = e / DVS, j = e % DVS;
    Ss[c][j] = a.S_in ? a.S_in[state_off + static_cast<int64_t>(c) * a.dv + j0 + j] : 0.f;
  }
  if (FROM_Z)
    for (int c = tid; c < DK; c += NT) eaL[c] = __expf(a.A[h * DK + c]) * kLog2e;
  __syncthreads();

  for (int t0 = 0; t0 < a.T; t0 += SC) {
    const int n = min(SC, a.T - t0);
    if (a.S_ckpt && t0 % 64 == 0) {  // backward checkpoint: the state entering this 64-token block
      float* ck = a.S_ckpt + (static_cast<int64_t>(bh) * ((a.T + 63) / 64) + t0 / 64) * DK * a.dv;
      for (int e = tid; e < DK * DVS; e += NT) ck[(e / DVS) * a.dv + j0 + e % DVS] = Ss[e / DVS][e % DVS];
    }
    // 1. load the sub-chunk; Gl = log2-decay summed from the sub-chunk start
    for (int e = tid; e < SC * DK; e += NT) {
      const int i = e / DK, c = e % DK;
      float kv = 0.f, qv = 0.f, gl = 0.f;
      if (i < n) {
        const int64_t row = (static_cast<int64_t>(b) * a.T + t0 + i) * a.H + h;
        kv = io<Tin>::load(k, row * DK + c);
        qv = io<Tin>::load(q, row * DK + c);
        if (FROM_Z) {
          gl = gate_log2(io<Tin>::load(z, row * DK + c), eaL[c], gmin_l2e);
        } else {
          gl = a.G[row * DK + c] * kLog2e;
          if (t0 % a.chunk != 0) {  // subtract the sum through token t0 - 1 (same chunk)
            const int64_t prev = (static_cast<int64_t>(b) * a.T + t0 - 1) * a.H + h;
            gl -= a.G[prev * DK + c] * kLog2e;
          }
        }
      }
      Ks[i][c] = kv;
      Qs[i][c] = qv;
      Gl[i][c] = gl;
    }
    for (int e = tid; e < SC * DVS; e += NT) {
      const int i = e / DVS, j = e % DVS;
      Vs[i][j] = i < n ? io<Tin>::load(v, (static_cast<int64_t>(b) * a.T + t0 + i) * HDV + static_cast<int64_t>(h) * a.dv + j0 + j) : 0.f;
    }
    if (tid < SC) {
      const float bl = tid < n ? io<Tin>::load(beta, (static_cast<int64_t>(b) * a.T + t0 + tid) * a.H + h) : 0.f;
      bs[tid] = tid < n ? (a.prologue ? sigmoid_fast(bl) : bl) : 0.f;
    }
    __syncthreads();
    if (a.prologue) {  // normalise the rows of k and q (rows past n are zero and stay zero)
      if (tid < 2 * SC) {
        const float* row = tid < SC ? Ks[tid] : Qs[tid - SC];
        float ss = 0.f;
        for (int c = 0; c < DK; ++c) ss += row[c] * row[c];
        rn[tid / SC][tid % SC] = rsqrt_fast(ss + kL2Eps);
      }
      __syncthreads();
      for (int e = tid; e < SC * DK; e += NT) {
        const int i = e / DK, c = e % DK;
        Ks[i][c] *= rn[0][i];
        Qs[i][c] *= rn[1][i];
      }
      __syncthreads();
    }
    if (FROM_Z) {  // per-token g -> running sums within the sub-chunk
      for (int c = tid; c < DK; c += NT)
        for (int i = 1; i < n; ++i) Gl[i][c] += Gl[i - 1][c];
      __syncthreads();
    }
    // 2. L (strictly lower, times beta_t) and P (lower incl. diagonal)
    for (int e = tid; e < SC * SC; e += NT) {
      const int i = e / SC, s = e % SC;
      float lk = 0.f, pq = 0.f;
      if (i < n && s <= i) {
        for (int c = 0; c < DK; ++c) {
          const float d = fast_exp2(Gl[i][c] - Gl[s][c]) * Ks[s][c];
          lk += Ks[i][c] * d;
          pq += Qs[i][c] * d;
        }
      }
      Lm[i][s] = (s < i) ? bs[i] * lk : 0.f;
      Pm[i][s] = pq;
    }
    __syncthreads();
    // 3. Tm = (I + L)^-1 Diag(beta): one column per thread, forward substitution
    if (tid < SC) {
      const int j = tid;
      float x[SC];
#pragma unroll
      for (int i = 0; i < SC; ++i) {
        float acc = (i == j) ? 1.f : 0.f;
        for (int m = 0; m < i; ++m) acc -= Lm[i][m] * x[m];
        x[i] = acc;
      }
#pragma unroll
      for (int i = 0; i < SC; ++i) Tm[i][j] = x[i] * bs[j];
    }
    __syncthreads();
    // 4. W = Tm (K * 2^Gl), Ut = Tm V
    for (int e = tid; e < SC * DK; e += NT) {
      const int i = e / DK, c = e % DK;
      float acc = 0.f;
      for (int s = 0; s <= i; ++s) acc += Tm[i][s] * Ks[s][c] * fast_exp2(Gl[s][c]);
      Ws[i][c] = acc;
    }
    for (int e = tid; e < SC * DVS; e += NT) {
      const int i = e / DVS, j = e % DVS;
      float acc = 0.f;
      for (int s = 0; s <= i; ++s) acc += Tm[i][s] * Vs[s][j];
      Us[i][j] = acc;
    }
    __syncthreads();
    // 5. U = Ut - W S
    for (int e = tid; e < SC * DVS; e += NT) {
      const int i = e / DVS, j = e % DVS;
      float acc = Us[i][j];
      for (int c = 0; c < DK; ++c) acc -= Ws[i][c] * Ss[c][j];
      Us[i][j] = acc;
    }
    __syncthreads();
    // 6. o = scale ((Q * 2^Gl) S + P U)
    for (int e = tid; e < SC * DVS; e += NT) {
      const int i = e / DVS, j = e % DVS;
      if (i < n && !a.o_skip) {
        float acc = 0.f;
        for (int c = 0; c < DK; ++c) acc += Qs[i][c] * fast_exp2(Gl[i][c]) * Ss[c][j];
        for (int s = 0; s <= i; ++s) acc += Pm[i][s] * Us[s][j];
        io<Tout>::store(o, (static_cast<int64_t>(b) * a.T + t0 + i) * HDV + static_cast<int64_t>(h) * a.dv + j0 + j,
                        a.scale * acc);
      }
    }
    __syncthreads();
    // 7. S <- Diag(2^Gl_last) S + (K * 2^(Gl_last - Gl))^T U
    for (int e = tid; e < DK * DVS; e += NT) {
      const int c = e / DVS, j = e % DVS;
      const float gl_last = Gl[n - 1][c];
      float acc = fast_exp2(gl_last) * Ss[c][j];
      for (int s = 0; s < n; ++s) acc += Ks[s][c] * fast_exp2(gl_last - Gl[s][c]) * Us[s][j];
      Ss[c][j] = acc;
    }
    __syncthreads();
  }
  if (a.S_out) {
    for (int e = tid; e < DK * DVS; e += NT) {
      const int c = e / DVS, j = e % DVS;
      a.S_out[state_off + static_cast<int64_t>(c) * a.dv + j0 + j] = Ss[c][j];
    }
  }
}

template <int DK, int DVS, typename Tin, typename Tout>
static hipError_t launch_cg_t(const ChunkArgs& a, hipStream_t st) {
  const int64_t nblocks = static_cast<int64_t>(a.B) * a.H * (a.dv / DVS);
  if (nblocks == 0) return hipSuccess;
  if (a.from_z)
    hipLaunchKernelGGL((chunk_generic_kernel<DK, DVS, Tin, Tout, true>), dim3(static_cast<uint32_t>(nblocks)),
                       dim3(NT), 0, st, a);
  else
    hipLaunchKernelGGL((chunk_generic_kernel<DK, DVS, Tin, Tout, false>), dim3(static_cast<uint32_t>(nblocks)),
                       dim3(NT), 0, st, a);
  return hipGetLastError();
}

template <int DK>
static hipError_t launch_cg_k(const ChunkArgs& a, hipStream_t st) {
  // value-column slice: 16 columns (the state slice and the sub-chunk fit LDS)
  if (a.in_bf16)
    return a.out_bf16 ? launch_cg_t<DK, 16, bf16_t, bf16_t>(a, st) : launch_cg_t<DK, 16, bf16_t, float>(a, st);
  return a.out_bf16 ? launch_cg_t<DK, 16, float, bf16_t>(a, st) : launch_cg_t<DK, 16, float, float>(a, st);
}

hipError_t launch_chunk_generic(const ChunkArgs& a, hipStream_t st) {
  switch (a.dk) {
    case 16: return launch_cg_k<16>(a, st);
    case 32: return launch_cg_k<32>(a, st);
    case 64: return launch_cg_k<64>(a, st);
    case 128: return launch_cg_k<128>(a, st);
  }
  return hipErrorInvalidValue;
}

}  // namespace kda
