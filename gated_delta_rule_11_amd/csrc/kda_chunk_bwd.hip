// kda_chunk_bwd.hip -- backward pass of the fused-gate KDA prefill, fp32 MFMA.
//
// The forward is Eq. 1 of "Kimi K3: the paper and proofs side by side",
// section 2.1.1, with the gate of "Kimi K3 reading notes", section 2, in the
// chunkwise regrouping (derived from Eq. 1; "Kimi K3: architecture,
// derivations and a pinned-source audit", section 4.5 names it).  Inside a
// sub-chunk of 16 tokens with entry state S, with G the log-decay summed from
// the sub-chunk start (natural log, in [16 g_min, 0]) and Gam = e^G:
//   Kt = K Gam, Kb = K / Gam, Qt = Q Gam, Kh = K Gam_last / Gam     (per channel)
//   AL = Kt Kb^T, L = Diag(beta) strict_lower(AL), P = lower(Qt Kb^T)
//   M = (I + L)^-1, T = M Diag(beta), W = T Kt, Ut = T V, U = Ut - W S
//   O = Qt S + P U,  S_next = Diag(Gam_last) S + Kh^T U
// Its derivative, given dO (times the output scale) and dS_next, is the chain
// rule through those steps in reverse:
//   dU = P^T dO + Kh dS_next
//   dS = Qt^T dO + Diag(Gam_last) dS_next - W^T dU                  (to the previous sub-chunk)
//   dQt = dO S^T + dP Kb,  dP = lower(dO U^T),  dKh = U dS_next^T,  dW = -dU S^T
//   dV = T^T dU,  dT = dU V^T + dW Kt^T,  dKt = T^T dW + dAL Kb
//   dbeta_s += sum_t dT[t][s] M[t][s],  dM = dT Diag(beta),  dL = -strict_lower(M^T dM M^T)
//   dbeta_t += sum_s dL[t][s] AL[t][s],  dAL = Diag(beta) dL,  dKb = dAL^T Kt + dP^T Qt
//   dq = dQt Gam,  dk = dKt Gam + dKb / Gam + dKh Gam_last / Gam
//   dG = dQt Qt + dKt Kt - dKb Kb - dKh Kh  (+ sum_t dKh Kh + dGam_last Gam_last at the last token)
//   dg = reverse cumulative sum of dG,  dz = dg g_min sigma (1 - sigma) e^A,  dA += (that) z
// With g >= -5 per token, Gam and 1/Gam stay within [e^-80, e^80] (fp32 normal
// range), so the products above are plain matrix products.
//
// One workgroup (8 wavefronts) per (b, h) walks the 64-token blocks in reverse.
// The forward left the state entering each block (checkpoints); the workgroup
// first recomputes the states entering the block's later sub-chunks (into a
// per-workgroup scratch, L2-resident), then runs the sub-chunks backwards.
// All products run on v_mfma_f32_16x16x4_f32 (fp32 operands, as the generic
// forward): lane i supplies A[i % 16][i / 16] and B[i / 16][i % 16] and holds
// D[4 (i / 16) + v][i % 16].  The state S and the running gradient dS are held
// in registers twice: by value-column tile (wavefront w owns columns 16 w..)
// for the products that contract over key channels, and transposed, by key-row
// tile, for those that contract over value channels.
#include "kda_common.hpp"
#include "kda_launch.hpp"

namespace kda {

namespace bw {
constexpr int SC = 16;   // sub-chunk
constexpr int CK = 64;   // checkpoint block
constexpr int NW = 8;    // wavefronts
constexpr int NT = NW * 64;

template <int DK, int DV>
struct Layout {
  static constexpr int RK = DK + 4;  // fp32 row strides
  static constexpr int RV = DV + 4;
  static constexpr int RS = 17;
  // [16][RK] tiles
  static constexpr int KT = 0, KB = KT + 16 * RK, QT = KB + 16 * RK, KH = QT + 16 * RK, W = KH + 16 * RK,
                       GG = W + 16 * RK, DQT = GG + 16 * RK, DKT = DQT + 16 * RK, DKB = DKT + 16 * RK,
                       DKH = DKB + 16 * RK, DW = DKH + 16 * RK;
  // [16][RV] tiles
  static constexpr int V = DW + 16 * RK, DO = V + 16 * RV, U = DO + 16 * RV, DU = U + 16 * RV;
  // [16][RS] small matrices
  static constexpr int AL = DU + 16 * RV, L = AL + 16 * RS, P = L + 16 * RS, M = P + 16 * RS, TT = M + 16 * RS,
                       DP = TT + 16 * RS, DT0 = DP + 16 * RS, DT1 = DT0 + 16 * RS, DM = DT1 + 16 * RS,
                       Y = DM + 16 * RS, DAL = Y + 16 * RS;
  // vectors
  static constexpr int BETA = DAL + 16 * RS, GL = BETA + 16, DGL = GL + DK;
  static constexpr int FLOATS = DGL + DK;
  static constexpr int BYTES = FLOATS * 4;
  static_assert(BYTES <= 160 * 1024, "LDS budget");
};
}  // namespace bw

__device__ __forceinline__ f32x4 mma4(float a, float b, f32x4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x4f32(a, b, c, 0, 0, 0);
}

__device__ __forceinline__ void bw_barrier() {
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup");
  __builtin_amdgcn_s_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup");
}

template <int DK, int DV, typename Tin, typename Tdo>
__global__ __launch_bounds__(bw::NT) void chunk_bwd_kernel(const BwdArgs a) {
  using namespace bw;
  using Ly = Layout<DK, DV>;
  constexpr int NKT = DK / 16, NVT = DV / 16;
  constexpr int RK = Ly::RK, RV = Ly::RV, RS = Ly::RS;
  extern __shared__ __attribute__((aligned(16))) float sm[];
  float* sKt = sm + Ly::KT;
  float* sKb = sm + Ly::KB;
  float* sQt = sm + Ly::QT;
  float* sKh = sm + Ly::KH;
  float* sW = sm + Ly::W;
  float* sG = sm + Ly::GG;
  float* sdQt = sm + Ly::DQT;
  float* sdKt = sm + Ly::DKT;
  float* sdKb = sm + Ly::DKB;
  float* sdKh = sm + Ly::DKH;
  float* sdW = sm + Ly::DW;
  float* sV = sm + Ly::V;
  float* sdO = sm + Ly::DO;
  float* sU = sm + Ly::U;
  float* sdU = sm + Ly::DU;
  float* sAL = sm + Ly::AL;
  float* sL = sm + Ly::L;
  float* sP = sm + Ly::P;
  float* sM = sm + Ly::M;
  float* sT = sm + Ly::TT;
  float* sdP = sm + Ly::DP;
  float* sdT0 = sm + Ly::DT0;
  float* sdT1 = sm + Ly::DT1;
  float* sdM = sm + Ly::DM;
  float* sY = sm + Ly::Y;
  float* sdAL = sm + Ly::DAL;
  float* sBeta = sm + Ly::BETA;
  float* sGl = sm + Ly::GL;
  float* sdGl = sm + Ly::DGL;

  const int bh = blockIdx.x;
  const int h = bh % a.H, b = bh / a.H;
  const int T = a.T, H = a.H;
  const int wv = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  // Lane coordinates are re-derived through an opaque copy after every barrier,
  // so that the LDS and global addresses built from them are formed where they
  // are used instead of being hoisted out of the loops and held in registers.
  int tid, ln, g4, r16;
  auto relane = [&]() {
    int t = threadIdx.x;
    asm volatile("" : "+v"(t));
    tid = t;
    ln = t & 63;
    g4 = ln >> 4;
    r16 = ln & 15;
  };
  relane();
  const bool own_j = wv < NVT;  // value-column tile jt = wv (state by columns)
  const bool own_c = wv < NKT;  // key-row tile ct = wv (state transposed)
  const int jt = wv, ct = wv;
  const int nblk = (T + CK - 1) / CK;
  const int64_t SZ = static_cast<int64_t>(DK) * DV;
  const float* ckpt = a.ckpt + static_cast<int64_t>(bh) * nblk * SZ;
  float* scratch = a.scratch + static_cast<int64_t>(bh) * 3 * SZ;
  const Tin* q = static_cast<const Tin*>(a.q);
  const Tin* k = static_cast<const Tin*>(a.k);
  const Tin* v = static_cast<const Tin*>(a.v);
  const Tin* z = static_cast<const Tin*>(a.z);
  const Tin* beta = static_cast<const Tin*>(a.beta);
  const Tdo* d_o = static_cast<const Tdo*>(a.d_o);
  const float g_min = a.g_min;

  // state by value-column tile: Sc[ct'][v] = S[16 ct' + 4 g4 + v][16 jt + r16]
  // state transposed by key-row tile: St[jt'][v] = S[16 ct + r16][16 jt' + 4 g4 + v]
  f32x4 Sc[NKT], St[NVT], dSc[NKT], dSt[NVT];
  auto load_state = [&](const float* src, f32x4 (&C)[NKT], f32x4 (&Tr)[NVT]) {
#pragma unroll
    for (int c2 = 0; c2 < NKT; ++c2)
#pragma unroll
      for (int e = 0; e < 4; ++e) C[c2][e] = (own_j && src) ? src[(16 * c2 + 4 * g4 + e) * DV + 16 * jt + r16] : 0.f;
#pragma unroll
    for (int j2 = 0; j2 < NVT; ++j2) {
      if (own_c && src) {
        Tr[j2] = *reinterpret_cast<const f32x4*>(src + (16 * ct + r16) * DV + 16 * j2 + 4 * g4);
      } else {
        Tr[j2] = f32x4{0.f, 0.f, 0.f, 0.f};
      }
    }
  };

  float dA_acc = 0.f;  // thread c < DK: this (b, h)'s part of dA[h][c]
  const float eA = tid < DK ? __expf(a.A[h * DK + tid]) : 0.f;

  // ---- sub-chunk inputs into LDS; BWD also loads q and dO
  auto load_sub = [&](int t0, int n, bool BWD) {
    if (tid < DK) {  // key channel c: gate, running log-decay, scaled keys (and queries)
      const int c = tid;
      float G = 0.f;
#pragma unroll 2
      for (int t = 0; t < SC; ++t) {
        const bool ok = t < n;
        const int64_t row = (static_cast<int64_t>(b) * T + t0 + t) * H + h;
        const float kv = ok ? io<Tin>::load(k, row * DK + c) : 0.f;
        const float zv = ok ? io<Tin>::load(z, row * DK + c) : 0.f;
        const float g = ok ? g_min / (1.f + __expf(-eA * zv)) : 0.f;
        G += g;
        const float Gm = __expf(G);
        sKt[t * RK + c] = kv * Gm;
        sKb[t * RK + c] = kv * __expf(-G);
        sG[t * RK + c] = G;
        if (BWD) sQt[t * RK + c] = (ok ? io<Tin>::load(q, row * DK + c) : 0.f) * Gm;
      }
      const float gl = __expf(G);
      sGl[c] = gl;
      // Kh = k e^(G_last - G) = Kb e^(G_last)
#pragma unroll 4
      for (int t = 0; t < SC; ++t) sKh[t * RK + c] = sKb[t * RK + c] * gl;
    } else if (tid < DK + DV) {  // value column j
      const int j = tid - DK;
#pragma unroll
      for (int t = 0; t < SC; ++t) {
        const bool ok = t < n;
        const int64_t row = (static_cast<int64_t>(b) * T + t0 + t) * H + h;
        sV[t * RV + j] = ok ? io<Tin>::load(v, row * DV + j) : 0.f;
        if (BWD) sdO[t * RV + j] = ok ? a.scale * io<Tdo>::load(d_o, row * DV + j) : 0.f;
      }
    } else if (tid >= 256 && tid < 256 + SC) {
      const int t = tid - 256;
      sBeta[t] = t < n ? io<Tin>::load(beta, (static_cast<int64_t>(b) * T + t0 + t) * H + h) : 0.f;
    }
  };

  // ---- AL = Kt Kb^T (wave 0), AP = Qt Kb^T (wave 1, BWD); masked L, P
  auto lp = [&](bool BWD) {
    if (wv == 0 || (BWD && wv == 1)) {
      const float* X = wv == 0 ? sKt : sQt;
      f32x4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll 8
      for (int kb = 0; kb < DK / 4; ++kb) acc = mma4(X[r16 * RK + 4 * kb + g4], sKb[r16 * RK + 4 * kb + g4], acc);
      // acc[e] = X[t][s] with t = 4 g4 + e, s = r16
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const int t = 4 * g4 + e, s = r16;
        if (wv == 0) {
          sAL[t * RS + s] = acc[e];
          sL[t * RS + s] = s < t ? sBeta[t] * acc[e] : 0.f;
        } else {
          sP[t * RS + s] = s <= t ? acc[e] : 0.f;
        }
      }
    }
  };

  // ---- M = (I + L)^-1 (forward substitution, one column per lane), T = M Diag(beta)
  auto inverse = [&]() {
    if (wv == 0 && ln < SC) {
      const int s = ln;
      float x[SC];
#pragma unroll
      for (int t = 0; t < SC; ++t) {
        float acc = (t == s) ? 1.f : 0.f;
#pragma unroll
        for (int m = 0; m < t; ++m) acc -= sL[t * RS + m] * x[m];
        x[t] = acc;
        __builtin_amdgcn_sched_barrier(0);  // keep each row's reads with its row
      }
      const float bs = sBeta[s];
#pragma unroll
      for (int t = 0; t < SC; ++t) {
        sM[t * RS + s] = x[t];
        sT[t * RS + s] = x[t] * bs;
      }
    }
  };

  // ---- W[:, ct] = T Kt[:, ct] -> LDS; Ut[:, jt] = T V[:, jt] -> registers
  auto w_ut = [&](f32x4& Ut) {
    if (own_c) {
      f32x4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int kb = 0; kb < 4; ++kb) acc = mma4(sT[r16 * RS + 4 * kb + g4], sKt[(4 * kb + g4) * RK + 16 * ct + r16], acc);
#pragma unroll
      for (int e = 0; e < 4; ++e) sW[(4 * g4 + e) * RK + 16 * ct + r16] = acc[e];
    }
    Ut = f32x4{0.f, 0.f, 0.f, 0.f};
    if (own_j) {
#pragma unroll
      for (int kb = 0; kb < 4; ++kb) Ut = mma4(sT[r16 * RS + 4 * kb + g4], sV[(4 * kb + g4) * RV + 16 * jt + r16], Ut);
    }
  };

  // ---- X[:, jt] += sum_c A[t][c] Y[c][jt] with Y held by columns (B operand = the lane's element e)
  auto over_c = [&](const float* Asrc, const f32x4 (&Y)[NKT], f32x4 acc) {
#pragma unroll
    for (int c2 = 0; c2 < NKT; ++c2) {
#pragma unroll
      for (int e = 0; e < 4; ++e) acc = mma4(Asrc[r16 * RK + 16 * c2 + 4 * g4 + e], Y[c2][e], acc);
      __builtin_amdgcn_sched_barrier(0);  // bound how far operand reads run ahead (registers)
    }
    return acc;
  };
  // ---- X[:, ct] += sum_j A[t][j] Y[ct][j] with Y held transposed
  auto over_j = [&](const float* Asrc, const f32x4 (&Y)[NVT], f32x4 acc) {
#pragma unroll
    for (int j2 = 0; j2 < NVT; ++j2) {
#pragma unroll
      for (int e = 0; e < 4; ++e) acc = mma4(Asrc[r16 * RV + 16 * j2 + 4 * g4 + e], Y[j2][e], acc);
      __builtin_amdgcn_sched_barrier(0);
    }
    return acc;
  };

  // dS_out
  load_state(a.dS_out ? a.dS_out + static_cast<int64_t>(bh) * SZ : nullptr, dSc, dSt);

  for (int blk = nblk - 1; blk >= 0; --blk) {
    const int b0 = blk * CK;
    const int nsub = min(CK, T - b0 + 0) > 0 ? (min(CK, T - b0) + SC - 1) / SC : 0;

    // ===== recompute the states entering sub-chunks 1 .. nsub-1 of the block
    load_state(ckpt + static_cast<int64_t>(blk) * SZ, Sc, St);
    for (int s = 0; s + 1 < nsub; ++s) {
      const int t0 = b0 + s * SC;
      const int n = min(SC, T - t0);
      bw_barrier();
      relane();
      load_sub(t0, n, false);
      bw_barrier();
      relane();
      lp(false);
      bw_barrier();
      relane();
      inverse();
      bw_barrier();
      relane();
      f32x4 Ut;
      w_ut(Ut);
      bw_barrier();
      relane();
      if (own_j) {
        // U[:, jt] = Ut - W S[:, jt];  S_next[c][jt] = Gam_last[c] S + sum_t Kh[t][c] U[t][jt]
        f32x4 negU = over_c(sW, Sc, f32x4{-Ut[0], -Ut[1], -Ut[2], -Ut[3]});  // = W S - Ut = -U
        float* dst = scratch + static_cast<int64_t>(s) * SZ;
#pragma unroll
        for (int c2 = 0; c2 < NKT; ++c2) {
          f32x4 acc;
#pragma unroll
          for (int e = 0; e < 4; ++e) acc[e] = sGl[16 * c2 + 4 * g4 + e] * Sc[c2][e];
#pragma unroll
          for (int e = 0; e < 4; ++e) acc = mma4(-sKh[(4 * g4 + e) * RK + 16 * c2 + r16], negU[e], acc);
          Sc[c2] = acc;
#pragma unroll
          for (int e = 0; e < 4; ++e) dst[(16 * c2 + 4 * g4 + e) * DV + 16 * jt + r16] = acc[e];
          __builtin_amdgcn_sched_barrier(0);
        }
      }
    }

    // ===== sub-chunks of the block, last first (the barrier at the top of each
    // makes the scratch states written above visible to every wavefront)
    for (int s = nsub - 1; s >= 0; --s) {
      const int t0 = b0 + s * SC;
      const int n = min(SC, T - t0);
      bw_barrier();
      relane();  // scratch states written, LDS free
      load_state(s == 0 ? ckpt + static_cast<int64_t>(blk) * SZ : scratch + static_cast<int64_t>(s - 1) * SZ, Sc,
                 St);
      load_sub(t0, n, true);
      bw_barrier();
      relane();
      lp(true);
      bw_barrier();
      relane();
      inverse();
      bw_barrier();
      relane();
      f32x4 Ut;
      w_ut(Ut);
      bw_barrier();
      relane();

      // ---- U, dU (by value-column tile); dQt (by key-row tile)
      f32x4 Uc = {0.f, 0.f, 0.f, 0.f}, dUc = {0.f, 0.f, 0.f, 0.f}, dQt = {0.f, 0.f, 0.f, 0.f};
      if (own_j) {
        const f32x4 WS = over_c(sW, Sc, f32x4{0.f, 0.f, 0.f, 0.f});
#pragma unroll
        for (int e = 0; e < 4; ++e) Uc[e] = Ut[e] - WS[e];
        // dU = P^T dO + Kh dS_next
        f32x4 acc = over_c(sKh, dSc, f32x4{0.f, 0.f, 0.f, 0.f});
#pragma unroll
        for (int kb = 0; kb < 4; ++kb) acc = mma4(sP[(4 * kb + g4) * RS + r16], sdO[(4 * kb + g4) * RV + 16 * jt + r16], acc);
        dUc = acc;
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          sU[(4 * g4 + e) * RV + 16 * jt + r16] = Uc[e];
          sdU[(4 * g4 + e) * RV + 16 * jt + r16] = dUc[e];
        }
      }
      if (own_c) dQt = over_j(sdO, St, dQt);  // dO S^T
      bw_barrier();
      relane();

      // ---- dKh, dW, dGam_last (by key-row tile); dP (wave 0); then dS in both layouts
      if (own_c) {
        const f32x4 dKh = over_j(sU, dSt, f32x4{0.f, 0.f, 0.f, 0.f});
        const f32x4 ndW = over_j(sdU, St, f32x4{0.f, 0.f, 0.f, 0.f});  // dU S^T = -dW
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          sdKh[(4 * g4 + e) * RK + 16 * ct + r16] = dKh[e];
          sdW[(4 * g4 + e) * RK + 16 * ct + r16] = -ndW[e];
        }
        float part = 0.f;  // sum_j dS_next[c][j] S[c][j], c = 16 ct + r16
#pragma unroll
        for (int j2 = 0; j2 < NVT; ++j2)
#pragma unroll
          for (int e = 0; e < 4; ++e) part += dSt[j2][e] * St[j2][e];
        part += __shfl_xor(part, 16);
        part += __shfl_xor(part, 32);
        if (g4 == 0) sdGl[16 * ct + r16] = part;
      }
      if (wv == NW - 1) {  // dP = lower(dO U^T)
        f32x4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll 8
        for (int kb = 0; kb < DV / 4; ++kb) acc = mma4(sdO[r16 * RV + 4 * kb + g4], sU[r16 * RV + 4 * kb + g4], acc);
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const int t = 4 * g4 + e;
          sdP[t * RS + r16] = r16 <= t ? acc[e] : 0.f;
        }
      }
      // dS = Qt^T dO + Diag(Gam_last) dS_next - W^T dU
      if (own_j) {
#pragma unroll
        for (int c2 = 0; c2 < NKT; ++c2) {
          f32x4 acc;
#pragma unroll
          for (int e = 0; e < 4; ++e) acc[e] = sGl[16 * c2 + 4 * g4 + e] * dSc[c2][e];
#pragma unroll
          for (int kb = 0; kb < 4; ++kb)
            acc = mma4(sQt[(4 * kb + g4) * RK + 16 * c2 + r16], sdO[(4 * kb + g4) * RV + 16 * jt + r16], acc);
#pragma unroll
          for (int e = 0; e < 4; ++e) acc = mma4(-sW[(4 * g4 + e) * RK + 16 * c2 + r16], dUc[e], acc);
          dSc[c2] = acc;
          __builtin_amdgcn_sched_barrier(0);
        }
      }
      if (own_c) {
        const float gl = sGl[16 * ct + r16];
#pragma unroll
        for (int j2 = 0; j2 < NVT; ++j2) {
          f32x4 acc;
#pragma unroll
          for (int e = 0; e < 4; ++e) acc[e] = gl * dSt[j2][e];
#pragma unroll
          for (int kb = 0; kb < 4; ++kb) {
            acc = mma4(sdO[(4 * kb + g4) * RV + 16 * j2 + r16], sQt[(4 * kb + g4) * RK + 16 * ct + r16], acc);
            acc = mma4(-sdU[(4 * kb + g4) * RV + 16 * j2 + r16], sW[(4 * kb + g4) * RK + 16 * ct + r16], acc);
          }
          dSt[j2] = acc;
          __builtin_amdgcn_sched_barrier(0);
        }
      }
      bw_barrier();
      relane();

      // ---- dV (by value-column tile, stored); dT parts (waves 6, 7); dKt from W (by key-row tile)
      if (own_j) {
        f32x4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int e = 0; e < 4; ++e) acc = mma4(sT[(4 * g4 + e) * RS + r16], dUc[e], acc);
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const int t = 4 * g4 + e;
          if (t < n) a.grad_v[((static_cast<int64_t>(b) * T + t0 + t) * H + h) * DV + 16 * jt + r16] = acc[e];
        }
      }
      if (wv == NW - 2 || wv == NW - 1) {
        f32x4 acc = {0.f, 0.f, 0.f, 0.f};
        if (wv == NW - 2) {  // dU V^T
#pragma unroll 8
          for (int kb = 0; kb < DV / 4; ++kb) acc = mma4(sdU[r16 * RV + 4 * kb + g4], sV[r16 * RV + 4 * kb + g4], acc);
        } else {  // dW Kt^T
#pragma unroll 8
          for (int kb = 0; kb < DK / 4; ++kb) acc = mma4(sdW[r16 * RK + 4 * kb + g4], sKt[r16 * RK + 4 * kb + g4], acc);
        }
        float* dst = wv == NW - 2 ? sdT0 : sdT1;
#pragma unroll
        for (int e = 0; e < 4; ++e) dst[(4 * g4 + e) * RS + r16] = acc[e];
      }
      f32x4 dKt = {0.f, 0.f, 0.f, 0.f};
      if (own_c) {
#pragma unroll
        for (int kb = 0; kb < 4; ++kb)
          dKt = mma4(sT[(4 * kb + g4) * RS + r16], sdW[(4 * kb + g4) * RK + 16 * ct + r16], dKt);
      }
      bw_barrier();
      relane();

      // ---- dM = dT Diag(beta) -> LDS (wave 0)
      if (wv == 0) {
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const int t = 4 * g4 + e;
          sdM[t * RS + r16] = (sdT0[t * RS + r16] + sdT1[t * RS + r16]) * sBeta[r16];
        }
      }
      bw_barrier();
      relane();
      // Y = M^T dM (wave 0)
      if (wv == 0) {
        f32x4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int kb = 0; kb < 4; ++kb) acc = mma4(sM[(4 * kb + g4) * RS + r16], sdM[(4 * kb + g4) * RS + r16], acc);
#pragma unroll
        for (int e = 0; e < 4; ++e) sY[(4 * g4 + e) * RS + r16] = acc[e];
      }
      bw_barrier();
      relane();
      // dL = -strict_lower(Y M^T) (over dM, free again); dAL = Diag(beta) dL (wave 0)
      if (wv == 0) {
        f32x4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int kb = 0; kb < 4; ++kb) acc = mma4(sY[r16 * RS + 4 * kb + g4], sM[r16 * RS + 4 * kb + g4], acc);
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const int t = 4 * g4 + e;
          const float dl = r16 < t ? -acc[e] : 0.f;
          sdM[t * RS + r16] = dl;
          sdAL[t * RS + r16] = dl * sBeta[t];
        }
      }
      bw_barrier();
      relane();
      // dbeta_u = sum_t dT[t][u] M[t][u] + sum_s dL[u][s] AL[u][s] (lanes 0..15 of wave 1)
      if (wv == 1 && ln < SC) {
        const int u = ln;
        float db = 0.f;
#pragma unroll
        for (int t = 0; t < SC; ++t) db += (sdT0[t * RS + u] + sdT1[t * RS + u]) * sM[t * RS + u];
#pragma unroll
        for (int s2 = 0; s2 < SC; ++s2) db += sdM[u * RS + s2] * sAL[u * RS + s2];
        if (u < n) a.grad_beta[(static_cast<int64_t>(b) * T + t0 + u) * H + h] = db;
      }

      // ---- dKt += dAL Kb; dKb = dAL^T Kt + dP^T Qt; dQt += dP Kb (by key-row tile)
      if (own_c) {
#pragma unroll
        for (int kb = 0; kb < 4; ++kb) {
          dKt = mma4(sdAL[r16 * RS + 4 * kb + g4], sKb[(4 * kb + g4) * RK + 16 * ct + r16], dKt);
          dQt = mma4(sdP[r16 * RS + 4 * kb + g4], sKb[(4 * kb + g4) * RK + 16 * ct + r16], dQt);
        }
        f32x4 dKb = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int kb = 0; kb < 4; ++kb) {
          dKb = mma4(sdAL[(4 * kb + g4) * RS + r16], sKt[(4 * kb + g4) * RK + 16 * ct + r16], dKb);
          dKb = mma4(sdP[(4 * kb + g4) * RS + r16], sQt[(4 * kb + g4) * RK + 16 * ct + r16], dKb);
        }
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const int o = (4 * g4 + e) * RK + 16 * ct + r16;
          sdKt[o] = dKt[e];
          sdKb[o] = dKb[e];
          sdQt[o] = dQt[e];
        }
      }
      bw_barrier();
      relane();

      // ---- per key channel: dq, dk, dG -> dg (reverse cumulative sum) -> dz, dA
      if (tid < DK) {
        const int c = tid;
        const float gl = sGl[c];
        float tail = 0.f;
#pragma unroll 2
        for (int t = 0; t < SC; ++t) {
          const int o = t * RK + c;
          const float Gm = __expf(sG[o]);
          const float dqt = sdQt[o], dkt = sdKt[o], dkb = sdKb[o], dkh = sdKh[o];
          const float Kh_ = sKh[o];
          sG[o] = dqt * sQt[o] + dkt * sKt[o] - dkb * sKb[o] - dkh * Kh_;  // dG (G is no longer needed)
          tail += dkh * Kh_;
          if (t < n) {
            const int64_t row = (static_cast<int64_t>(b) * T + t0 + t) * H + h;
            a.grad_q[row * DK + c] = dqt * Gm;
            a.grad_k[row * DK + c] = dkt * Gm + dkb / Gm + dkh * gl / Gm;
          }
        }
        float run = tail + sdGl[c] * gl;  // dG at the last token also carries Gam_last's uses
#pragma unroll 2
        for (int t = SC - 1; t >= 0; --t) {
          run += sG[t * RK + c];
          if (t < n) {
            const int64_t row = (static_cast<int64_t>(b) * T + t0 + t) * H + h;
            const float zv = io<Tin>::load(z, row * DK + c);
            const float sg = 1.f / (1.f + __expf(-eA * zv));
            const float dx = run * g_min * sg * (1.f - sg);
            a.grad_z[row * DK + c] = dx * eA;
            dA_acc += dx * eA * zv;
          }
        }
      }
    }
  }

  if (a.grad_S_in && own_j) {
    float* dst = a.grad_S_in + static_cast<int64_t>(bh) * SZ;
#pragma unroll
    for (int c2 = 0; c2 < NKT; ++c2)
#pragma unroll
      for (int e = 0; e < 4; ++e) dst[(16 * c2 + 4 * g4 + e) * DV + 16 * jt + r16] = dSc[c2][e];
  }
  if (tid < DK) a.dA_part[static_cast<int64_t>(bh) * DK + tid] = dA_acc;
}

// dA[h][c] = sum over b of the per-(b, h) parts (fixed order: deterministic)
__global__ void dA_reduce_kernel(const float* __restrict__ part, float* __restrict__ dA, int B, int H, int dk) {
  const int i = blockIdx.x * blockDim.x + threadIdx.x;
  if (i >= H * dk) return;
  const int h = i / dk, c = i % dk;
  float s = 0.f;
  for (int b = 0; b < B; ++b) s += part[(static_cast<int64_t>(b) * H + h) * dk + c];
  dA[i] = s;
}

template <int DK, int DV, typename Tin, typename Tdo>
static hipError_t launch_bwd_t(const BwdArgs& a, hipStream_t st) {
  auto kern = chunk_bwd_kernel<DK, DV, Tin, Tdo>;
  constexpr int bytes = bw::Layout<DK, DV>::BYTES;
  static bool attr_set = false;
  if (!attr_set) {
    hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void*>(kern),
                                       hipFuncAttributeMaxDynamicSharedMemorySize, bytes);
    if (e != hipSuccess) return e;
    attr_set = true;
  }
  hipLaunchKernelGGL(kern, dim3(a.B * a.H), dim3(bw::NT), bytes, st, a);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  const int n = a.H * a.dk;
  hipLaunchKernelGGL(dA_reduce_kernel, dim3((n + 255) / 256), dim3(256), 0, st, a.dA_part, a.grad_A, a.B, a.H, a.dk);
  return hipGetLastError();
}

template <int DK, int DV>
static hipError_t launch_bwd_d(const BwdArgs& a, hipStream_t st) {
  if (a.in_bf16)
    return a.do_bf16 ? launch_bwd_t<DK, DV, bf16_t, bf16_t>(a, st) : launch_bwd_t<DK, DV, bf16_t, float>(a, st);
  return a.do_bf16 ? launch_bwd_t<DK, DV, float, bf16_t>(a, st) : launch_bwd_t<DK, DV, float, float>(a, st);
}

template <int DK>
static hipError_t launch_bwd_k(const BwdArgs& a, hipStream_t st) {
  switch (a.dv) {
    case 16: return launch_bwd_d<DK, 16>(a, st);
    case 32: return launch_bwd_d<DK, 32>(a, st);
    case 64: return launch_bwd_d<DK, 64>(a, st);
    case 128: return launch_bwd_d<DK, 128>(a, st);
  }
  return hipErrorInvalidValue;
}

hipError_t launch_chunk_bwd(const BwdArgs& a, hipStream_t st) {
  if (static_cast<int64_t>(a.B) * a.H == 0) return hipSuccess;
  switch (a.dk) {
    case 16: return launch_bwd_k<16>(a, st);
    case 32: return launch_bwd_k<32>(a, st);
    case 64: return launch_bwd_k<64>(a, st);
    case 128: return launch_bwd_k<128>(a, st);
  }
  return hipErrorInvalidValue;
}

}  // namespace kda
