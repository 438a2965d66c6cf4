// kda_chunk_bwd.hip -- backward pass of the fused-gate KDA prefill on matrix cores.
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
// One workgroup (8 wavefronts) per (b, h), or per (b, h, half of the value columns)
// when B*H alone would leave compute units idle, walks the 64-token blocks in
// reverse.  The forward left the state entering each block (checkpoints); the
// workgroup first recomputes the states entering the block's later sub-chunks (into
// a per-workgroup scratch, L2-resident), then runs the sub-chunks backwards.  With
// two slices, each adds its part of the key-side gradients into zero-filled outputs.
// M = (I + L)^-1 is a product of four factors formed by repeated squaring, on fp32
// matrix cores for every input dtype.
// fp32 inputs: every product runs on v_mfma_f32_16x16x4_f32 (fp32 operands): lane
// i supplies A[i % 16][i / 16] and B[i / 16][i % 16] and holds D[4 (i / 16) + v][i % 16].
// bf16 inputs: the products run on v_mfma_f32_16x16x16_bf16 (bf16 operands, fp32
// accumulation) with the same lane layout, lane group g holding k = 4 g .. 4 g + 3,
// except dKt = T^T dW, the dL-free parts of dQt and dKb, dP, dT and the M, dM, Y, dL
// chain, which stay fp32 for every input dtype: dbeta and dG sum products of these with
// the inputs whose terms cancel.  The state S and the running gradient dS are held
// in registers twice: by value-column tile (wavefront w owns columns 16 w..)
// for the products that contract over key channels, and transposed, by key-row
// tile, for those that contract over value channels.
#include <type_traits>

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
                       GG = W + 16 * RK, DKH = GG + 16 * RK, DW = DKH + 16 * RK;
  // [16][RV] tiles
  static constexpr int V = DW + 16 * RK, DO = V + 16 * RV, U = DO + 16 * RV, DU = U + 16 * RV;
  // [16][RS] small matrices
  static constexpr int AL = DU + 16 * RV, L = AL + 16 * RS, P = L + 16 * RS, M = P + 16 * RS, TT = M + 16 * RS,
                       DP = TT + 16 * RS, DT0 = DP + 16 * RS, DT1 = DT0 + 16 * RS,
                       DT2 = DT1 + 16 * RS, DAL = DT2 + 16 * RS;
  // vectors
  static constexpr int BETA = DAL + 16 * RS, GL = BETA + 16, DGL = GL + DK, EA = DGL + DK;
  // [16][RK]: sigma(e^A z) and e^A z of the sub-chunk, kept for the gate's derivative
  static constexpr int SG = EA + DK, XZ = SG + 16 * RK;
  // [16][LS]: L^T for the inverse's column reads (LS a multiple of 4: 16-byte rows)
  static constexpr int LS = 20, LT = XZ + 16 * RK;
  static constexpr int FLOATS = LT + 16 * LS;
  static constexpr int BYTES = FLOATS * 4;
  static_assert(BYTES <= 160 * 1024, "LDS budget");
};
}  // namespace bw

// Four consecutive elements (16-byte aligned for fp32, 8-byte for bf16), loaded raw
// (so that a prefetch does not wait for its data) and widened to fp32 where used.
typedef uint32_t u32x2_t __attribute__((ext_vector_type(2)));
template <typename T> struct io4;
template <> struct io4<float> {
  typedef f32x4 raw;
  __device__ __forceinline__ static raw load(const float* p, int64_t i) { return *reinterpret_cast<const f32x4*>(p + i); }
  __device__ __forceinline__ static f32x4 wide(raw r) { return r; }
};
template <> struct io4<bf16_t> {
  typedef u32x2_t raw;
  __device__ __forceinline__ static raw load(const bf16_t* p, int64_t i) {
    return *reinterpret_cast<const u32x2_t*>(p + i);
  }
  __device__ __forceinline__ static f32x4 wide(raw u) {
    return f32x4{__uint_as_float(u[0] << 16), __uint_as_float(u[0] & 0xffff0000u), __uint_as_float(u[1] << 16),
                 __uint_as_float(u[1] & 0xffff0000u)};
  }
};
template <typename T> struct io1;
template <> struct io1<float> {
  typedef float raw;
  __device__ __forceinline__ static raw load(const float* p, int64_t i) { return p[i]; }
  __device__ __forceinline__ static float wide(raw r) { return r; }
};
template <> struct io1<bf16_t> {
  typedef uint16_t raw;
  __device__ __forceinline__ static raw load(const bf16_t* p, int64_t i) { return p[i].bits; }
  __device__ __forceinline__ static float wide(raw r) { return bf16_to_f32(r); }
};

__device__ __forceinline__ f32x4 mma4(float a, float b, f32x4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x4f32(a, b, c, 0, 0, 0);
}
typedef short s16x4_t __attribute__((ext_vector_type(4)));
typedef float f32x2_t __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
// four floats -> four bf16 (round to nearest even), the A or B operand of one lane
__device__ __forceinline__ s16x4_t bw_bf4(f32x4 x) {
  const u32x2_t r = {__builtin_bit_cast(uint32_t, __builtin_convertvector(f32x2_t{x[0], x[1]}, bf16x2_t)),
                     __builtin_bit_cast(uint32_t, __builtin_convertvector(f32x2_t{x[2], x[3]}, bf16x2_t))};
  return __builtin_bit_cast(s16x4_t, r);
}
// 16 x 16 x 16 product, lane group g holding k = 4 g .. 4 g + 3 of both operands
__device__ __forceinline__ f32x4 mma16bf(f32x4 a, f32x4 b, f32x4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(bw_bf4(a), bw_bf4(b), c, 0, 0, 0);
}

// Four consecutive fp32 values of a 17-float-stride row (not 16-byte aligned).
__device__ __forceinline__ f32x4 rows4(const float* p) {
  f32x4 r;
  r[0] = p[0]; r[1] = p[1]; r[2] = p[2]; r[3] = p[3];
  return r;
}

// Workgroup barrier ordering LDS only: the next sub-chunk's inputs stay in flight across it.
__device__ __forceinline__ void bw_barrier() {
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup", "local");
  __builtin_amdgcn_s_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup", "local");
}
// Workgroup barrier that also orders global memory (the recomputed states in the scratch).
__device__ __forceinline__ void bw_barrier_global() {
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup");
  __builtin_amdgcn_s_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup");
}

template <int DK, int DV, int NSP, typename Tin, typename Tdo>
__global__ __launch_bounds__(bw::NT) void chunk_bwd_kernel(const BwdArgs a) {
  using namespace bw;
  // bf16 inputs: bf16 operands for the products the file header lists, fp32 accumulation
  constexpr bool BF = std::is_same<Tin, bf16_t>::value;
  constexpr int DVS = DV / NSP;  // value columns of this workgroup's slice
  using Ly = Layout<DK, DVS>;
  constexpr int NKT = DK / 16, NVT = DVS / 16;
  constexpr int RK = Ly::RK, RV = Ly::RV, RS = Ly::RS;
  extern __shared__ __attribute__((aligned(16))) float sm[];
  float* sKt = sm + Ly::KT;
  float* sKb = sm + Ly::KB;
  float* sQt = sm + Ly::QT;
  float* sKh = sm + Ly::KH;
  float* sW = sm + Ly::W;
  float* sG = sm + Ly::GG;
  float* sdKh = sm + Ly::DKH;
  float* sdW = sm + Ly::DW;
  float* sV = sm + Ly::V;
  float* sdO = sm + Ly::DO;
  float* sU = sm + Ly::U;
  float* sdU = sm + Ly::DU;
  float* sAL = sm + Ly::AL;
  float* sP = sm + Ly::P;
  float* sM = sm + Ly::M;
  float* sT = sm + Ly::TT;
  float* sdP = sm + Ly::DP;
  float* sdT0 = sm + Ly::DT0;
  float* sdT1 = sm + Ly::DT1;
  float* sdT2 = sm + Ly::DT2;
  float* sdAL = sm + Ly::DAL;
  float* sBeta = sm + Ly::BETA;
  float* sGl = sm + Ly::GL;
  float* sdGl = sm + Ly::DGL;
  float* sEA = sm + Ly::EA;
  float* sSig = sm + Ly::SG;
  float* sXz = sm + Ly::XZ;
  float* sLt = sm + Ly::LT;

  const int bh = blockIdx.x / NSP, sp = blockIdx.x % NSP;
  const int h = bh % a.H, b = bh / a.H;
  const int T = a.T, H = a.H;
  const int j0 = sp * DVS;  // first value column of the slice
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
  const bool own_j = wv < NVT;  // value-column tile jt = wv of the slice (state by columns)
  const bool own_c = wv < NKT;  // key-row tile ct = wv (state transposed)
  const int jt = wv, ct = wv;
  // wavefronts with no value tile of their own take the 16 x 16 products
  constexpr int W_DP = NW - 1, W_DT0 = NW - 2, W_DT1 = NW - 3, W_DT2 = NW - 4;
  // dW Kt^T over the key channels in two halves, on two wavefronts of different SIMDs
  // (from d_k = 32 on: each half's lane-group quarter stays a multiple of four channels)
  constexpr bool kSplitDT1 = DK >= 32;
  const int nblk = (T + CK - 1) / CK;
  const int64_t SZ = static_cast<int64_t>(DK) * DV;
  const float* ckpt = a.ckpt + static_cast<int64_t>(bh) * nblk * SZ;
  float* scratch = a.scratch + static_cast<int64_t>(bh) * 3 * SZ;  // the slices write disjoint columns
  float* const mcache = a.mcache ? a.mcache + (static_cast<int64_t>(bh) * NSP + sp) * kBwdMCacheFloats : nullptr;
  const Tin* q = static_cast<const Tin*>(a.q);
  const Tin* k = static_cast<const Tin*>(a.k);
  const Tin* v = static_cast<const Tin*>(a.v);
  const Tin* z = static_cast<const Tin*>(a.z);
  const Tin* beta = static_cast<const Tin*>(a.beta);
  const Tdo* d_o = static_cast<const Tdo*>(a.d_o);
  const float g_min = a.g_min;
  // key-side gradients: the whole value range (one slice), or, with two slices, this
  // slice's part of it, added into the zero-filled outputs (two addends onto zero: the
  // same sum in either order, so the result does not depend on which slice adds first)
  float* const gq = a.grad_q;
  float* const gk = a.grad_k;
  float* const gz = a.grad_z;
  float* const gbeta = a.grad_beta;
  auto put = [](float* p, float x) {
    if constexpr (NSP == 2) {
      unsafeAtomicAdd(p, x);
    } else {
      *p = x;
    }
  };

  // state by value-column tile: Sc[ct'][e] = S[16 ct' + 4 g4 + e][j0 + 16 jt + r16]
  // state transposed by key-row tile: St[jt'][e] = S[16 ct + r16][j0 + 16 jt' + 4 g4 + e]
  f32x4 Sc[NKT], St[NVT], dSc[NKT], dSt[NVT];
  auto load_state = [&](const float* src, f32x4 (&C)[NKT], f32x4 (&Tr)[NVT]) {
#pragma unroll
    for (int c2 = 0; c2 < NKT; ++c2)
#pragma unroll
      for (int e = 0; e < 4; ++e)
        C[c2][e] = (own_j && src) ? src[(16 * c2 + 4 * g4 + e) * DV + j0 + 16 * jt + r16] : 0.f;
#pragma unroll
    for (int j2 = 0; j2 < NVT; ++j2) {
      if (own_c && src) {
        Tr[j2] = *reinterpret_cast<const f32x4*>(src + (16 * ct + r16) * DV + j0 + 16 * j2 + 4 * g4);
      } else {
        Tr[j2] = f32x4{0.f, 0.f, 0.f, 0.f};
      }
    }
  };

  float dA_acc = 0.f;  // key-row-tile lanes (g4, r16): part of dA[h][16 ct + r16]

  // ---- sub-chunk inputs.  The raw values of the next sub-chunk in processing order are
  // loaded into registers while the current one is processed, four consecutive channels
  // per load (token offsets clamped to the sub-chunk's last valid token, padding zeroed
  // later: no branch around a load).
  constexpr int NQK = SC * DK / 4, NQV = SC * DVS / 4;  // quads of the key side, the value side
  static_assert(NQK <= NT && NQV <= NT, "one quad per thread");
  typename io4<Tin>::raw pk = {}, pz = {}, pq = {}, pv = {};
  typename io4<Tdo>::raw po = {};
  typename io1<Tin>::raw pb = {};
  auto fetch = [&](int t0, int n, bool BWD) {
    {
      const int e = min(tid, NQK - 1) * 4, t = e / DK, c = e % DK;
      const int64_t row = (static_cast<int64_t>(b) * T + t0 + min(t, n - 1)) * H + h;
      pk = io4<Tin>::load(k, row * DK + c);
      pz = io4<Tin>::load(z, row * DK + c);
      if (BWD) pq = io4<Tin>::load(q, row * DK + c);
    }
    {
      const int e = min(tid, NQV - 1) * 4, t = e / DVS, j = e % DVS;
      const int64_t row = (static_cast<int64_t>(b) * T + t0 + min(t, n - 1)) * H + h;
      pv = io4<Tin>::load(v, row * DV + j0 + j);
      if (BWD) po = io4<Tdo>::load(d_o, row * DV + j0 + j);
    }
    pb = io1<Tin>::load(beta, (static_cast<int64_t>(b) * T + t0 + min(ln & 15, n - 1)) * H + h);
  };
  // the sub-chunk after (blk, s, BWD) in processing order: each block recomputes its
  // sub-chunks 0 .. nsub-2 forwards, then runs nsub-1 .. 0 backwards; blocks go last first
  auto nsub_of = [&](int blk) { return (min(CK, T - blk * CK) + SC - 1) / SC; };
  auto fetch_after = [&](int blk, int s, bool BWD) {
    const int ns = nsub_of(blk);
    int nb = blk, nsb;
    bool nbwd;
    if (!BWD) {
      nbwd = s + 1 >= ns - 1;
      nsb = nbwd ? ns - 1 : s + 1;
    } else if (s > 0) {
      nbwd = true;
      nsb = s - 1;
    } else {
      if (blk == 0) return;
      nb = blk - 1;
      const int ns2 = nsub_of(nb);
      nbwd = ns2 == 1;
      nsb = 0;  // its first recompute sub-chunk, or its only sub-chunk
    }
    const int t0 = nb * CK + nsb * SC;
    fetch(t0, min(SC, T - t0), nbwd);
  };

  // ---- sub-chunk (blk, s) into LDS from the prefetched registers; BWD also takes q and dO.
  // Two steps: every thread stores its elements and computes the gate; four lanes per key
  // channel sum the log-decay over the tokens and scale the channel's elements.
  auto load_sub = [&](int blk, int s, int t0, int n, bool BWD) {
    const auto kr = pk, zr = pz, qr = pq, vr = pv;
    const auto orw = po;
    const auto br = pb;
    fetch_after(blk, s, BWD);
    if (tid < NQK) {
      const int e = tid * 4, t = e / DK, c = e % DK;
      const bool ok = t < n;
      const f32x4 kv = io4<Tin>::wide(kr), zv = io4<Tin>::wide(zr), qv = io4<Tin>::wide(qr);
      const int o = t * RK + c;
      f32x4 gg, sg4, xz;
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        xz[i] = sEA[c + i] * zv[i];
        sg4[i] = fast_rcp(1.f + __expf(-xz[i]));
        gg[i] = ok ? g_min * sg4[i] : 0.f;
      }
      const f32x4 zero = {0.f, 0.f, 0.f, 0.f};
      *reinterpret_cast<f32x4*>(sKt + o) = ok ? kv : zero;  // raw until step 3
      if (BWD) *reinterpret_cast<f32x4*>(sQt + o) = ok ? qv : zero;
      *reinterpret_cast<f32x4*>(sG + o) = gg;
      *reinterpret_cast<f32x4*>(sSig + o) = sg4;
      *reinterpret_cast<f32x4*>(sXz + o) = xz;
    }
    if (tid < NQV) {
      const int e = tid * 4, t = e / DVS, j = e % DVS;
      const bool ok = t < n;
      const f32x4 vv = io4<Tin>::wide(vr), ov = io4<Tdo>::wide(orw);
      const f32x4 zero = {0.f, 0.f, 0.f, 0.f};
      *reinterpret_cast<f32x4*>(sV + t * RV + j) = ok ? vv : zero;
      if (BWD) *reinterpret_cast<f32x4*>(sdO + t * RV + j) = ok ? a.scale * ov : zero;
    }
    if (tid < SC) sBeta[tid] = tid < n ? io1<Tin>::wide(br) : 0.f;
    bw_barrier();
    relane();
    if (tid < 4 * DK) {
      // running log-decay over the sub-chunk, four lanes per key channel with four tokens
      // each: lane r of the quad continues the sum from lane r - 1's last value, in token
      // order, then every lane scales its own four elements
      const int c = tid >> 2, qd = tid & 3;
      float gv[4], Gv[4], G = 0.f;
#pragma unroll
      for (int i = 0; i < 4; ++i) gv[i] = sG[(4 * qd + i) * RK + c];
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        if (qd == r) {
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            G += gv[i];
            Gv[i] = G;
          }
        }
        G = __shfl(G, (ln & ~3) + r);
      }
      const float gl = __expf(G);  // e^(G_last)
      if (qd == 0) sGl[c] = gl;
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int o = (4 * qd + i) * RK + c;
        const float kv = sKt[o];
        const float Gm = __expf(Gv[i]), Gi = __expf(-Gv[i]);
        const float kb = kv * Gi;
        sG[o] = Gv[i];
        sKt[o] = kv * Gm;
        sKb[o] = kb;
        sKh[o] = kb * gl;  // k e^(G_last - G)
        if (BWD) sQt[o] = sQt[o] * Gm;
      }
    }
  };

  // ---- 16 x 16 tile: sum over K of A[r][k] B[c][k] (both row-major with stride RSTR).
  // Any assignment of the K channels to the K / 4 products' lane groups gives the same
  // sum; lane group g4 takes channels (K / 4) g4 .. (K / 4) g4 + K / 4 - 1, so each lane
  // reads its operands as contiguous 16-byte vectors.  MBF: bf16 operands (bf16 inputs
  // only); dP and dT take fp32 operands for every input dtype, since dbeta and the gate's
  // derivative are sums of their elements' products whose terms can cancel.
  auto mm_nt = [&](const float* Ap, const float* Bp, auto k_c, int RSTR, auto bf_c) {
    constexpr int K = decltype(k_c)::value, KQ = K / 4;
    constexpr bool MBF = BF && decltype(bf_c)::value;
    static_assert(KQ % 4 == 0, "16-byte operand reads");
    const float* ar = Ap + r16 * RSTR + KQ * g4;
    const float* br = Bp + r16 * RSTR + KQ * g4;
    f32x4 acc0 = {0.f, 0.f, 0.f, 0.f}, acc1 = {0.f, 0.f, 0.f, 0.f};
    // the reads of the next four channels go out before the products of the current ones
    f32x4 av = *reinterpret_cast<const f32x4*>(ar), bv = *reinterpret_cast<const f32x4*>(br);
#pragma unroll
    for (int qd = 0; qd < KQ / 4; ++qd) {
      f32x4 an = av, bn = bv;
      if (qd + 1 < KQ / 4) {
        an = *reinterpret_cast<const f32x4*>(ar + 4 * qd + 4);
        bn = *reinterpret_cast<const f32x4*>(br + 4 * qd + 4);
      }
      if constexpr (MBF) {
        if (qd & 1)
          acc1 = mma16bf(av, bv, acc1);
        else
          acc0 = mma16bf(av, bv, acc0);
      } else {
        acc0 = mma4(av[0], bv[0], acc0);
        acc1 = mma4(av[1], bv[1], acc1);
        acc0 = mma4(av[2], bv[2], acc0);
        acc1 = mma4(av[3], bv[3], acc1);
      }
      av = an;
      bv = bn;
    }
    return acc0 + acc1;
  };

  // ---- wave 0: AL = Kt Kb^T, then M = (I + L)^-1 and T = M Diag(beta); wave 1 (BWD):
  // P = lower(Qt Kb^T).  The inverse is a product of four factors formed by repeated
  // squaring on fp32 matrix cores (below).
  // cw (recompute): also leave M and AL in the cache slot; cached (backward): take M and
  // AL as prefetched from the slot the recompute filled instead of forming them again.
  f32x4 pre_m = {}, pre_al = {};  // wave 0: lane (g4, r16) holds row 4 g4 + e, column r16
  auto prefetch_m = [&](const float* cr) {
    if (wv == 0) {
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        pre_m[e] = cr[(4 * g4 + e) * 16 + r16];
        pre_al[e] = cr[256 + (4 * g4 + e) * 16 + r16];
      }
    }
  };
  auto lp_inverse = [&](bool BWD, float* cw, bool cached) {
    if (wv == 0 && cached) {
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const int t = 4 * g4 + e;
        sM[t * RS + r16] = pre_m[e];
        sT[t * RS + r16] = pre_m[e] * sBeta[r16];
        sAL[t * RS + r16] = pre_al[e];
      }
      return;
    }
    if (wv == 0 || (BWD && wv == 1)) {
      const f32x4 acc = mm_nt(wv == 0 ? sKt : sQt, sKb, std::integral_constant<int, DK>{}, RK, std::true_type{});
      // acc[e] = X[t][s] with t = 4 g4 + e, s = r16
      if (wv == 1) {
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const int t = 4 * g4 + e;
          sP[t * RS + r16] = r16 <= t ? acc[e] : 0.f;
        }
      } else {
        f32x4 lv;
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const int t = 4 * g4 + e;
          if (BWD) sAL[t * RS + r16] = acc[e];
          if (cw) cw[256 + t * 16 + r16] = acc[e];
          lv[e] = r16 < t ? sBeta[t] * acc[e] : 0.f;
        }
        // M = (I + L)^-1 = (I + N)(I + N^2)(I + N^4)(I + N^8) with N = -L (strictly lower
        // triangular, so N^16 = 0), on matrix cores.  Matrices are held in the accumulator
        // layout (lane (g4, r16): rows 4 g4 .. 4 g4 + 3 of column r16), each product's left
        // factor as its transpose in that layout; L^T comes through an fp32 copy in LDS
        // (written and read by this wavefront only, in order).
        *reinterpret_cast<f32x4*>(sLt + r16 * Ly::LS + 4 * g4) = lv;  // sLt[s][t] = L[t][s]
        f32x4 nn, nt, id;
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          nn[e] = -lv[e];
          nt[e] = -sLt[(4 * g4 + e) * Ly::LS + r16];
          id[e] = (4 * g4 + e == r16) ? 1.f : 0.f;
        }
        // c + X Y, given X^T and Y in the accumulator layout (k = 4 g4 + v in step v)
        auto mm16 = [](f32x4 xt, f32x4 y, f32x4 c) {
#pragma unroll
          for (int v = 0; v < 4; ++v) c = mma4(xt[v], y[v], c);
          return c;
        };
        const f32x4 zero = {0.f, 0.f, 0.f, 0.f};
        f32x4 pm = id + nn, pt = id + nt;  // I + N and its transpose
#pragma unroll
        for (int lev = 0; lev < 3; ++lev) {
          const f32x4 n2 = mm16(nt, nn, zero);             // N^(2^(lev+1))
          const f32x4 pn = mm16(pt, n2, pm);               // P (I + that)
          if (lev < 2) {
            const f32x4 n2t = mm16(nn, nt, zero);          // its transpose
            pt = mm16(n2, pt, pt);                         // and P's
            nt = n2t;
          }
          nn = n2;
          pm = pn;
        }
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const int t = 4 * g4 + e;
          sM[t * RS + r16] = pm[e];
          sT[t * RS + r16] = pm[e] * sBeta[r16];
          if (cw) cw[t * 16 + r16] = pm[e];
        }
      }
    }
  };

  // ---- W[:, ct] = T Kt[:, ct] -> LDS; Ut[:, jt] = T V[:, jt] -> registers
  auto w_ut = [&](f32x4& Ut) {
    if (own_c) {
      f32x4 acc = {0.f, 0.f, 0.f, 0.f};
      if constexpr (BF) {
        f32x4 bv;
#pragma unroll
        for (int e = 0; e < 4; ++e) bv[e] = sKt[(4 * g4 + e) * RK + 16 * ct + r16];
        acc = mma16bf(rows4(sT + r16 * RS + 4 * g4), bv, acc);
      } else {
#pragma unroll
        for (int kb = 0; kb < 4; ++kb)
          acc = mma4(sT[r16 * RS + 4 * kb + g4], sKt[(4 * kb + g4) * RK + 16 * ct + r16], acc);
      }
#pragma unroll
      for (int e = 0; e < 4; ++e) sW[(4 * g4 + e) * RK + 16 * ct + r16] = acc[e];
    }
    Ut = f32x4{0.f, 0.f, 0.f, 0.f};
    if (own_j) {
      if constexpr (BF) {
        f32x4 bv;
#pragma unroll
        for (int e = 0; e < 4; ++e) bv[e] = sV[(4 * g4 + e) * RV + 16 * jt + r16];
        Ut = mma16bf(rows4(sT + r16 * RS + 4 * g4), bv, Ut);
      } else {
#pragma unroll
        for (int kb = 0; kb < 4; ++kb)
          Ut = mma4(sT[r16 * RS + 4 * kb + g4], sV[(4 * kb + g4) * RV + 16 * jt + r16], Ut);
      }
    }
  };

  // ---- X[:, jt] += sum_c A[t][c] Y[c][jt], Y held by columns (B operand = the lane's element e);
  // two accumulators so that consecutive products do not wait on each other
  auto over_c = [&](const float* Asrc, const f32x4 (&Y)[NKT], f32x4 acc) {
    f32x4 acc2 = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int c2 = 0; c2 < NKT; ++c2) {
      if constexpr (BF) {
        const f32x4 av = *reinterpret_cast<const f32x4*>(Asrc + r16 * RK + 16 * c2 + 4 * g4);
        if (c2 & 1)
          acc2 = mma16bf(av, Y[c2], acc2);
        else
          acc = mma16bf(av, Y[c2], acc);
      } else {
#pragma unroll
        for (int e = 0; e < 4; e += 2) {
          acc = mma4(Asrc[r16 * RK + 16 * c2 + 4 * g4 + e], Y[c2][e], acc);
          acc2 = mma4(Asrc[r16 * RK + 16 * c2 + 4 * g4 + e + 1], Y[c2][e + 1], acc2);
        }
      }
    }
    return acc + acc2;
  };
  // ---- X[:, ct] += sum_j A[t][j] Y[ct][j], Y held transposed
  auto over_j = [&](const float* Asrc, const f32x4 (&Y)[NVT], f32x4 acc) {
    f32x4 acc2 = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int j2 = 0; j2 < NVT; ++j2) {
      if constexpr (BF) {
        const f32x4 av = *reinterpret_cast<const f32x4*>(Asrc + r16 * RV + 16 * j2 + 4 * g4);
        if (j2 & 1)
          acc2 = mma16bf(av, Y[j2], acc2);
        else
          acc = mma16bf(av, Y[j2], acc);
      } else {
#pragma unroll
        for (int e = 0; e < 4; e += 2) {
          acc = mma4(Asrc[r16 * RV + 16 * j2 + 4 * g4 + e], Y[j2][e], acc);
          acc2 = mma4(Asrc[r16 * RV + 16 * j2 + 4 * g4 + e + 1], Y[j2][e + 1], acc2);
        }
      }
    }
    return acc + acc2;
  };


  if (tid < DK) sEA[tid] = __expf(a.A[h * DK + tid]);
  // dS_out
  load_state(a.dS_out ? a.dS_out + static_cast<int64_t>(bh) * SZ : nullptr, dSc, dSt);

  if (nblk > 0) {  // the first sub-chunk in processing order
    const int ns = nsub_of(nblk - 1);
    const int t0 = (nblk - 1) * CK + (ns > 1 ? 0 : ns - 1) * SC;
    fetch(t0, min(SC, T - t0), ns == 1);
  }
  for (int blk = nblk - 1; blk >= 0; --blk) {
    const int b0 = blk * CK;
    const int nsub = (min(CK, T - b0) + SC - 1) / SC;

    // ===== recompute the states entering sub-chunks 1 .. nsub-1 of the block
    load_state(ckpt + static_cast<int64_t>(blk) * SZ, Sc, St);
    for (int s = 0; s + 1 < nsub; ++s) {
      const int t0 = b0 + s * SC;
      const int n = min(SC, T - t0);
      bw_barrier();
      relane();
      load_sub(blk, s, t0, n, false);
      bw_barrier();
      relane();
      lp_inverse(false, mcache ? mcache + s * 512 : nullptr, false);
      bw_barrier();
      relane();
      f32x4 Ut;
      w_ut(Ut);
      bw_barrier();
      relane();
      if (own_j) {
        // U[:, jt] = Ut - W S[:, jt];  S_next[c][jt] = Gam_last[c] S + sum_t Kh[t][c] U[t][jt]
        const f32x4 negU = over_c(sW, Sc, f32x4{-Ut[0], -Ut[1], -Ut[2], -Ut[3]});  // = W S - Ut = -U
        float* dst = scratch + static_cast<int64_t>(s) * SZ;
#pragma unroll
        for (int c2 = 0; c2 < NKT; ++c2) {
          f32x4 acc;
#pragma unroll
          for (int e = 0; e < 4; ++e) acc[e] = sGl[16 * c2 + 4 * g4 + e] * Sc[c2][e];
          if constexpr (BF) {
            f32x4 av;
#pragma unroll
            for (int e = 0; e < 4; ++e) av[e] = -sKh[(4 * g4 + e) * RK + 16 * c2 + r16];
            acc = mma16bf(av, negU, acc);
          } else {
#pragma unroll
            for (int e = 0; e < 4; ++e) acc = mma4(-sKh[(4 * g4 + e) * RK + 16 * c2 + r16], negU[e], acc);
          }
          Sc[c2] = acc;
#pragma unroll
          for (int e = 0; e < 4; ++e) dst[(16 * c2 + 4 * g4 + e) * DV + j0 + 16 * jt + r16] = acc[e];
        }
      }
    }

    bw_barrier_global();  // the recomputed states in the scratch, visible to every wavefront
    relane();

    // ===== sub-chunks of the block, last first
    for (int s = nsub - 1; s >= 0; --s) {
      const int t0 = b0 + s * SC;
      const int n = min(SC, T - t0);
      bw_barrier();
      relane();
      load_state(s == 0 ? ckpt + static_cast<int64_t>(blk) * SZ : scratch + static_cast<int64_t>(s - 1) * SZ, Sc,
                 St);
      load_sub(blk, s, t0, n, true);
      bw_barrier();
      relane();
      lp_inverse(true, nullptr, mcache && s + 1 < nsub);
      if (mcache && s > 0) prefetch_m(mcache + (s - 1) * 512);  // for the next sub-chunk
      bw_barrier();
      relane();
      f32x4 Ut;
      w_ut(Ut);
      bw_barrier();
      relane();

      // ---- U, dU (by value-column tile); dQt = dO S^T (by key-row tile)
      f32x4 dUc = {0.f, 0.f, 0.f, 0.f}, dQt = {0.f, 0.f, 0.f, 0.f};
      if (own_j) {
        const f32x4 WS = over_c(sW, Sc, f32x4{0.f, 0.f, 0.f, 0.f});
        // dU = P^T dO + Kh dS_next
        f32x4 acc = over_c(sKh, dSc, f32x4{0.f, 0.f, 0.f, 0.f});
        if constexpr (BF) {
          f32x4 av, bv;
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            av[e] = sP[(4 * g4 + e) * RS + r16];
            bv[e] = sdO[(4 * g4 + e) * RV + 16 * jt + r16];
          }
          acc = mma16bf(av, bv, acc);
        } else {
#pragma unroll
          for (int kb = 0; kb < 4; ++kb)
            acc = mma4(sP[(4 * kb + g4) * RS + r16], sdO[(4 * kb + g4) * RV + 16 * jt + r16], acc);
        }
        dUc = acc;
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          sU[(4 * g4 + e) * RV + 16 * jt + r16] = Ut[e] - WS[e];
          sdU[(4 * g4 + e) * RV + 16 * jt + r16] = dUc[e];
        }
      }
      if (own_c) dQt = over_j(sdO, St, dQt);
      bw_barrier();
      relane();

      // ---- dKh, dW, dGam_last (key-row tiles); dP, dU V^T (16 x 16); dS in both layouts
      if (own_c) {
        const f32x4 dKh = over_j(sU, dSt, f32x4{0.f, 0.f, 0.f, 0.f});
        const f32x4 ndW = over_j(sdU, St, f32x4{0.f, 0.f, 0.f, 0.f});  // dU S^T = -dW
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          sdKh[(4 * g4 + e) * RK + 16 * ct + r16] = dKh[e];
          sdW[(4 * g4 + e) * RK + 16 * ct + r16] = -ndW[e];
        }
        float part = 0.f;  // sum over the slice's j of dS_next[c][j] S[c][j], c = 16 ct + r16
#pragma unroll
        for (int j2 = 0; j2 < NVT; ++j2)
#pragma unroll
          for (int e = 0; e < 4; ++e) part += dSt[j2][e] * St[j2][e];
        part += __shfl_xor(part, 16);
        part += __shfl_xor(part, 32);
        if (g4 == 0) sdGl[16 * ct + r16] = part;
      }
      if (wv == W_DP) {  // dP = lower(dO U^T)
        const f32x4 acc = mm_nt(sdO, sU, std::integral_constant<int, DVS>{}, RV, std::false_type{});
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const int t = 4 * g4 + e;
          sdP[t * RS + r16] = r16 <= t ? acc[e] : 0.f;
        }
      }
      if (wv == W_DT0) {  // dU V^T
        const f32x4 acc = mm_nt(sdU, sV, std::integral_constant<int, DVS>{}, RV, std::false_type{});
#pragma unroll
        for (int e = 0; e < 4; ++e) sdT0[(4 * g4 + e) * RS + r16] = acc[e];
      }
      // dS = Qt^T dO + Diag(Gam_last) dS_next - W^T dU
      if (own_j) {
#pragma unroll
        for (int c2 = 0; c2 < NKT; ++c2) {
          f32x4 acc, acc2 = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
          for (int e = 0; e < 4; ++e) acc[e] = sGl[16 * c2 + 4 * g4 + e] * dSc[c2][e];
          if constexpr (BF) {
            f32x4 av, bv, wv4;
#pragma unroll
            for (int e = 0; e < 4; ++e) {
              av[e] = sQt[(4 * g4 + e) * RK + 16 * c2 + r16];
              bv[e] = sdO[(4 * g4 + e) * RV + 16 * jt + r16];
              wv4[e] = -sW[(4 * g4 + e) * RK + 16 * c2 + r16];
            }
            acc = mma16bf(av, bv, acc);
            acc2 = mma16bf(wv4, dUc, acc2);
          } else {
#pragma unroll
            for (int kb = 0; kb < 4; ++kb)
              acc = mma4(sQt[(4 * kb + g4) * RK + 16 * c2 + r16], sdO[(4 * kb + g4) * RV + 16 * jt + r16], acc);
#pragma unroll
            for (int e = 0; e < 4; ++e) acc2 = mma4(-sW[(4 * g4 + e) * RK + 16 * c2 + r16], dUc[e], acc2);
          }
          dSc[c2] = acc + acc2;
        }
      }
      if (own_c) {
        const float gl = sGl[16 * ct + r16];
#pragma unroll
        for (int j2 = 0; j2 < NVT; ++j2) {
          f32x4 acc, acc2 = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
          for (int e = 0; e < 4; ++e) acc[e] = gl * dSt[j2][e];
          if constexpr (BF) {
            f32x4 a1, b1, a2, b2;
#pragma unroll
            for (int e = 0; e < 4; ++e) {
              a1[e] = sdO[(4 * g4 + e) * RV + 16 * j2 + r16];
              b1[e] = sQt[(4 * g4 + e) * RK + 16 * ct + r16];
              a2[e] = -sdU[(4 * g4 + e) * RV + 16 * j2 + r16];
              b2[e] = sW[(4 * g4 + e) * RK + 16 * ct + r16];
            }
            acc = mma16bf(a1, b1, acc);
            acc2 = mma16bf(a2, b2, acc2);
          } else {
#pragma unroll
            for (int kb = 0; kb < 4; ++kb) {
              acc = mma4(sdO[(4 * kb + g4) * RV + 16 * j2 + r16], sQt[(4 * kb + g4) * RK + 16 * ct + r16], acc);
              acc2 = mma4(-sdU[(4 * kb + g4) * RV + 16 * j2 + r16], sW[(4 * kb + g4) * RK + 16 * ct + r16], acc2);
            }
          }
          dSt[j2] = acc + acc2;
        }
      }
      bw_barrier();
      relane();

      // ---- dV (value-column tiles, stored); dT's second part dW Kt^T; dKt = T^T dW (key-row tiles)
      if (own_j) {
        f32x4 acc = {0.f, 0.f, 0.f, 0.f};
        if constexpr (BF) {
          f32x4 av;
#pragma unroll
          for (int e = 0; e < 4; ++e) av[e] = sT[(4 * g4 + e) * RS + r16];
          acc = mma16bf(av, dUc, acc);
        } else {
#pragma unroll
          for (int e = 0; e < 4; ++e) acc = mma4(sT[(4 * g4 + e) * RS + r16], dUc[e], acc);
        }
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const int t = 4 * g4 + e;
          if (t < n) a.grad_v[((static_cast<int64_t>(b) * T + t0 + t) * H + h) * DV + j0 + 16 * jt + r16] = acc[e];
        }
      }
      if constexpr (kSplitDT1) {  // dW Kt^T, channels 0 .. DK/2 - 1 and DK/2 .. DK - 1
        if (wv == W_DT1 || wv == W_DT2) {
          const int k0 = wv == W_DT1 ? 0 : DK / 2;
          const f32x4 acc = mm_nt(sdW + k0, sKt + k0, std::integral_constant<int, DK / 2>{}, RK, std::false_type{});
          float* dst = wv == W_DT1 ? sdT1 : sdT2;
#pragma unroll
          for (int e = 0; e < 4; ++e) dst[(4 * g4 + e) * RS + r16] = acc[e];
        }
      } else if (wv == W_DT1) {  // dW Kt^T
        const f32x4 acc = mm_nt(sdW, sKt, std::integral_constant<int, DK>{}, RK, std::false_type{});
#pragma unroll
        for (int e = 0; e < 4; ++e) sdT1[(4 * g4 + e) * RS + r16] = acc[e];
      }
      f32x4 dKt = {0.f, 0.f, 0.f, 0.f}, dKb = {0.f, 0.f, 0.f, 0.f};
      if (own_c) {
        // fp32 products for every input dtype: the gate's derivative takes differences
        // of these gradients' terms that cancel
#pragma unroll
        for (int kb = 0; kb < 4; ++kb) {
          dKt = mma4(sT[(4 * kb + g4) * RS + r16], sdW[(4 * kb + g4) * RK + 16 * ct + r16], dKt);
          // the parts of dQt and dKb that do not wait for dL
          dQt = mma4(sdP[r16 * RS + 4 * kb + g4], sKb[(4 * kb + g4) * RK + 16 * ct + r16], dQt);
          dKb = mma4(sdP[(4 * kb + g4) * RS + r16], sQt[(4 * kb + g4) * RK + 16 * ct + r16], dKb);
        }
      }
      bw_barrier();
      relane();

      // ---- wave 0: dM = dT Diag(beta), Y = M^T dM, dL = -strict_lower(Y M^T), dAL = Diag(beta) dL,
      // dbeta; one wavefront end to end, the 16 x 16 matrices in registers in the accumulator
      // layout (lane (g4, r16): rows 4 g4 .. 4 g4 + 3 of column r16; a product takes its left
      // factor as that factor's transpose in that layout): Y^T = dM^T M, then Y M^T, and its
      // transpose M Y^T for dbeta's row sums.
      if (wv == 0) {
        f32x4 dt, dm, ma, mt, alt;
        const float bu = sBeta[r16];
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const int t = 4 * g4 + e;
          dt[e] = sdT0[t * RS + r16] + sdT1[t * RS + r16];
          if constexpr (kSplitDT1) dt[e] += sdT2[t * RS + r16];
          dm[e] = dt[e] * bu;
          ma[e] = sM[t * RS + r16];    // M
          mt[e] = sM[r16 * RS + t];    // M^T
          alt[e] = sAL[r16 * RS + t];  // AL^T
        }
        auto mm16 = [](f32x4 xt, f32x4 y, f32x4 c) {
#pragma unroll
          for (int v = 0; v < 4; ++v) c = mma4(xt[v], y[v], c);
          return c;
        };
        const f32x4 zero = {0.f, 0.f, 0.f, 0.f};
        const f32x4 yt = mm16(dm, ma, zero);    // Y^T = dM^T M
        const f32x4 acc = mm16(yt, mt, zero);   // Y M^T
        const f32x4 acct = mm16(mt, yt, zero);  // M Y^T = (Y M^T)^T
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const int t = 4 * g4 + e;
          sdAL[t * RS + r16] = (r16 < t ? -acc[e] : 0.f) * sBeta[t];
        }
        // dbeta_u = sum_t dT[t][u] M[t][u] + sum_s dL[u][s] AL[u][s]: column u's sums of
        // dT o M and of (dL o AL)^T (lane (g4, r16) holds dL[r16][4 g4 + e] in acct), each
        // over the lane's four rows and then over the four lane groups
        float cs = dt[0] * ma[0] + dt[1] * ma[1] + dt[2] * ma[2] + dt[3] * ma[3];
        float rs = 0.f;
#pragma unroll
        for (int e = 0; e < 4; ++e) rs += (4 * g4 + e < r16 ? -acct[e] : 0.f) * alt[e];
        cs += __shfl_xor(cs, 16);
        rs += __shfl_xor(rs, 16);
        cs += __shfl_xor(cs, 32);
        rs += __shfl_xor(rs, 32);
        if (ln < SC) {
          const int u = ln;  // = r16: lane group 0
          if (u < n) put(&gbeta[(static_cast<int64_t>(b) * T + t0 + u) * H + h], cs + rs);
        }
      }
      bw_barrier();
      relane();

      // ---- dKt += dAL Kb; dKb += dAL^T Kt (key-row tiles); then, from the accumulators,
      // dq, dk and dG of the wavefront's 16 key channels: lane (g4, r16) holds tokens
      // 4 g4 .. 4 g4 + 3 of channel c = 16 ct + r16.  dg = reverse cumulative sum of dG over
      // the sub-chunk (the last token also carries Gam_last's uses), dz = dg g_min sigma
      // (1 - sigma) e^A and dA += dz z: suffix sums in a lane, then across the lane groups.
      if (own_c) {
#pragma unroll
        for (int kb = 0; kb < 4; ++kb) {
          dKt = mma4(sdAL[r16 * RS + 4 * kb + g4], sKb[(4 * kb + g4) * RK + 16 * ct + r16], dKt);
          dKb = mma4(sdAL[(4 * kb + g4) * RS + r16], sKt[(4 * kb + g4) * RK + 16 * ct + r16], dKb);
        }
        const int c = 16 * ct + r16;
        float dg[4], tail = 0.f;
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const int t = 4 * g4 + e;
          const int o = t * RK + c;
          const float Gm = __expf(sG[o]), Gi = __expf(-sG[o]);
          const float dkh = sdKh[o], kh = sKh[o];
          dg[e] = dQt[e] * sQt[o] + dKt[e] * sKt[o] - dKb[e] * sKb[o] - dkh * kh;
          tail += dkh * kh;
          if (t < n) {
            const int64_t row = (static_cast<int64_t>(b) * T + t0 + t) * H + h;
            put(&gq[row * DK + c], dQt[e] * Gm);
            put(&gk[row * DK + c], dKt[e] * Gm + (dKb[e] + dkh * sGl[c]) * Gi);
          }
        }
#pragma unroll
        for (int i = 2; i >= 0; --i) dg[i] += dg[i + 1];  // suffix sums within the lane's tokens
        tail += __shfl_xor(tail, 16);
        tail += __shfl_xor(tail, 32);
        float later = 0.f;  // the sums of the later lane groups (later tokens)
#pragma unroll
        for (int r = 1; r < 4; ++r) {
          const float x = __shfl(dg[0], r16 + 16 * r);
          later += r > g4 ? x : 0.f;
        }
        const float base = sdGl[c] * sGl[c] + tail + later;
        const float ea = sEA[c];
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const int t = 4 * g4 + i;
          if (t < n) {
            const int o = t * RK + c;
            const float sg = sSig[o];
            const float dx = (base + dg[i]) * g_min * sg * (1.f - sg);
            put(&gz[((static_cast<int64_t>(b) * T + t0 + t) * H + h) * DK + c], dx * ea);
            dA_acc += dx * sXz[o];
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
      for (int e = 0; e < 4; ++e) dst[(16 * c2 + 4 * g4 + e) * DV + j0 + 16 * jt + r16] = dSc[c2][e];
  }
  // dA: the four lane groups of each key channel hold parts over their tokens
  dA_acc += __shfl_xor(dA_acc, 16);
  dA_acc += __shfl_xor(dA_acc, 32);
  if (own_c && g4 == 0) a.dA_part[(static_cast<int64_t>(bh) * NSP + sp) * DK + 16 * ct + r16] = dA_acc;
}

// Zero fill (a kernel rather than a memset, so that the launch sequence can be captured).
__global__ void zero_kernel(float* __restrict__ out, int64_t n) {
  const int64_t i4 = (static_cast<int64_t>(blockIdx.x) * blockDim.x + threadIdx.x) * 4;
  if (i4 + 4 <= n) {
    *reinterpret_cast<f32x4*>(out + i4) = f32x4{0.f, 0.f, 0.f, 0.f};
  } else {
    for (int64_t i = i4; i < n; ++i) out[i] = 0.f;
  }
}

// dA[h][c] = sum over b of the per-(b, h) parts (fixed order: deterministic)
__global__ void dA_reduce_kernel(const float* __restrict__ part, float* __restrict__ dA, int B, int H, int dk,
                                 int nsp) {
  const int i = blockIdx.x * blockDim.x + threadIdx.x;
  if (i >= H * dk) return;
  const int h = i / dk, c = i % dk;
  float s = 0.f;
  for (int b = 0; b < B; ++b)
    for (int p = 0; p < nsp; ++p) s += part[((static_cast<int64_t>(b) * H + h) * nsp + p) * dk + c];
  dA[i] = s;
}

template <int DK, int DV, int NSP, typename Tin, typename Tdo>
static hipError_t launch_bwd_t(const BwdArgs& a, hipStream_t st) {
  auto kern = chunk_bwd_kernel<DK, DV, NSP, Tin, Tdo>;
  constexpr int bytes = bw::Layout<DK, DV / NSP>::BYTES;
  static std::atomic<uint64_t> lds_set{0};
  hipError_t e = set_lds_limit(reinterpret_cast<const void*>(kern), bytes, lds_set);
  if (e != hipSuccess) return e;
  if (NSP == 2) {  // the two slices add into zero-filled key-side gradients
    const int64_t ntok = static_cast<int64_t>(a.B) * a.T * a.H;
    const struct { float* out; int64_t n; } fills[] = {
        {a.grad_q, ntok * a.dk}, {a.grad_k, ntok * a.dk}, {a.grad_z, ntok * a.dk}, {a.grad_beta, ntok}};
    for (const auto& f : fills) {
      if (f.n == 0) continue;
      const int64_t nthr = (f.n + 3) / 4;
      hipLaunchKernelGGL(zero_kernel, dim3(static_cast<uint32_t>((nthr + 255) / 256)), dim3(256), 0, st, f.out, f.n);
    }
    e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  hipLaunchKernelGGL(kern, dim3(static_cast<uint32_t>(static_cast<int64_t>(a.B) * a.H * NSP)), dim3(bw::NT), bytes,
                     st, a);
  e = hipGetLastError();
  if (e != hipSuccess) return e;
  const int n = a.H * a.dk;
  hipLaunchKernelGGL(dA_reduce_kernel, dim3((n + 255) / 256), dim3(256), 0, st, a.dA_part, a.grad_A, a.B, a.H, a.dk,
                     NSP);
  return hipGetLastError();
}

template <int DK, int DV, int NSP>
static hipError_t launch_bwd_s(const BwdArgs& a, hipStream_t st) {
  if (a.in_bf16)
    return a.do_bf16 ? launch_bwd_t<DK, DV, NSP, bf16_t, bf16_t>(a, st) : launch_bwd_t<DK, DV, NSP, bf16_t, float>(a, st);
  return a.do_bf16 ? launch_bwd_t<DK, DV, NSP, float, bf16_t>(a, st) : launch_bwd_t<DK, DV, NSP, float, float>(a, st);
}

template <int DK, int DV>
static hipError_t launch_bwd_d(const BwdArgs& a, hipStream_t st) {
  if constexpr (DV >= 64) {
    if (chunk_bwd_slices(a.B, a.H, a.dv) == 2) return launch_bwd_s<DK, DV, 2>(a, st);  // two value slices
  }
  return launch_bwd_s<DK, DV, 1>(a, st);
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

int chunk_bwd_slices(int B, int H, int dv) {
  // two value slices when one workgroup per (b, h) would leave compute units idle
  return (dv >= 64 && static_cast<int64_t>(B) * H < 256) ? 2 : 1;
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
