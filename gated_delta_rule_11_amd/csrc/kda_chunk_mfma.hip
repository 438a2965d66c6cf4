// kda_chunk_mfma.hip -- fused chunked KDA prefill on bf16 MFMA (gfx950).
//
// Shape: bf16 q, k, v, z (or fp32 G), d_k = d_v = 128, chunks of C = 64 tokens
// made of four 16-token tiles.  One workgroup (4 wavefronts) per (b, h,
// slice of DVS value columns); the fp32 state slice S[128 x DVS] lives in
// MFMA accumulator registers for the whole sequence and is carried chunk to
// chunk.  The value columns of the state evolve independently given (k,
// beta, alpha), so slicing changes no arithmetic; the chunk-local work that
// does not depend on v (gate, decays, L, P, W) is repeated per slice.
//
// Per chunk, with entry state S, tile i = tokens 16i..16i+15, per key
// channel c, alpha from the bounded gate (Eq. 5, "Kimi K3 reading notes",
// section 2) and the recurrence of Eq. 1 ("Kimi K3: the paper and proofs side
// by side", section 2.1.1) regrouped over the chunk (the chunkwise form named
// on "Kimi K3: architecture, derivations and a pinned-source audit", 4.5):
//   r_t   = prod of alpha over tile tokens <= t    (in (0,1])
//   sf_t  = prod of alpha over tile tokens  > t    (in (0,1])
//   D_i   = prod of alpha over tile i; eB_i = prod_{i'<i} D_i'; af_i = prod_{i'>i} D_i'
//   exp(G_t - G_s) = r_t * f_ij * sf_s  with f_ij = prod_{j<i'<i} D_i' (s in tile j < i)
//                                         or f_ii = 1 / D_i (same tile; <= e^80)
//   L[t,s] = beta_t sum_c k_tc k_sc exp(G_tc - G_sc) (s < t),  P[t,s] = sum_c q_tc k_sc exp(..) (s <= t)
//   (I + L) [W | Ut] = Diag(beta) [K*Gamma | V]      (block forward substitution)
//   U = Ut - W S ;  O = (Q*Gamma) S + P U ;  S <- Diag(Gamma_C) S + (K*Gamma_C/Gamma)^T U
// Gamma_t = eB_i r_t, Gamma_C / Gamma_s = af_j sf_s.  The bounded gate keeps
// every factor representable: only the same-tile reciprocal exceeds one, and
// a 16-token tile's log-decay is above 16 g_min >= -88.
//
// MFMA usage: v_mfma_f32_16x16x32_bf16 for the channel contractions that read
// both operands from LDS (L and P), v_mfma_f32_16x16x16_bf16 elsewhere.  For
// the 16x16x16 shape the accumulator layout (lane l holds rows 4(l/16)+v of
// column l%16) equals the B-operand layout, so the state, the solve's partial
// results and U feed the next product straight from registers.
#include "kda_common.hpp"
#include "kda_launch.hpp"

namespace kda {

namespace mf {
constexpr int C = 64;          // chunk
constexpr int DK = 128;        // key / value head dim
constexpr int NTH = 256;       // 4 wavefronts
constexpr int RS = DK + 8;     // row stride (bf16 elements) of [token][channel] tiles
constexpr int TS = C + 8;      // row stride of [channel][token] tiles
constexpr int XS = 24;         // row stride of the 16x16 diagonal inverses
constexpr int LDS_ = 20;       // row stride (floats) of the fp32 diagonal L blocks

template <int DVS>
struct Layout {
  static constexpr int KR = 0;                          // [64][RS]  k r       (later: -W)
  static constexpr int QR = KR + C * RS * 2;            // [64][RS]  q r
  static constexpr int KC = QR + C * RS * 2;            // [64][RS]  k sf
  static constexpr int QT = KC + C * RS * 2;            // [64][RS]  q Gamma
  static constexpr int KTT = QT + C * RS * 2;           // [128][TS] (k Gamma)^T
  static constexpr int KHT = KTT + DK * TS * 2;         // [128][TS] (k Gamma_C/Gamma)^T
  static constexpr int VT = KHT + DK * TS * 2;          // [DVS][TS] v^T
  static constexpr int LM = VT + DVS * TS * 2;          // [64][TS]  -L (off-diagonal tiles)
  static constexpr int PM = LM + C * TS * 2;            // [64][TS]  P
  static constexpr int XM = PM + C * TS * 2;            // [4][16][XS] diagonal inverses
  static constexpr int LD = XM + 4 * 16 * XS * 2;       // [4][16][LDS_] fp32 diagonal L
  static constexpr int DT = LD + 4 * 16 * LDS_ * 4;     // [4][128] fp32 tile decays
  static constexpr int GC = DT + 4 * DK * 4;            // [128] fp32 chunk decay
  static constexpr int BT = GC + DK * 4;                // [64] fp32 beta
  static constexpr int BYTES = BT + C * 4;
  static_assert(BYTES <= 160 * 1024, "LDS budget");
};
}  // namespace mf

typedef short s16x4 __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

__device__ __forceinline__ uint16_t f2bf(float f) { return __builtin_bit_cast(uint16_t, static_cast<__bf16>(f)); }
__device__ __forceinline__ float bflo(uint32_t u) { return __uint_as_float(u << 16); }
__device__ __forceinline__ float bfhi(uint32_t u) { return __uint_as_float(u & 0xffff0000u); }
__device__ __forceinline__ uint32_t pack2(float a, float b) {
  return static_cast<uint32_t>(f2bf(a)) | (static_cast<uint32_t>(f2bf(b)) << 16);
}
__device__ __forceinline__ s16x4 cvt4(f32x4 x) {
  u32x2 r;
  r[0] = pack2(x[0], x[1]);
  r[1] = pack2(x[2], x[3]);
  return __builtin_bit_cast(s16x4, r);
}
__device__ __forceinline__ s16x4 lds64(const uint16_t* p) {
  return __builtin_bit_cast(s16x4, *reinterpret_cast<const u32x2*>(p));
}
__device__ __forceinline__ u32x4 lds128(const uint16_t* p) { return *reinterpret_cast<const u32x4*>(p); }
__device__ __forceinline__ f32x4 mma16(s16x4 a, s16x4 b, f32x4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(a, b, c, 0, 0, 0);
}
__device__ __forceinline__ f32x4 mma32(u32x4 a, u32x4 b, f32x4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, a), __builtin_bit_cast(bf16x8, b), c,
                                                 0, 0, 0);
}

// Tile pairs (i, j <= i) of the L / P products, per wavefront.
__constant__ int8_t kPairs[4][3][2] = {{{0, 0}, {3, 0}, {3, 1}},
                                       {{1, 0}, {1, 1}, {3, 2}},
                                       {{2, 0}, {2, 1}, {-1, -1}},
                                       {{2, 2}, {3, 3}, {-1, -1}}};

template <int DVS, bool FROM_Z, typename Tout>
__global__ __launch_bounds__(mf::NTH) void chunk_mfma_kernel(const ChunkArgs a, int ns, int xcd_map) {
  using namespace mf;
  using Ly = Layout<DVS>;
  constexpr int NJT = DVS / 16;              // value-column tiles in the slice
  constexpr int JPW = (NJT + 3) / 4;         // value-column tiles per wavefront (max)

  extern __shared__ __attribute__((aligned(16))) unsigned char smem[];
  uint16_t* sKR = reinterpret_cast<uint16_t*>(smem + Ly::KR);
  uint16_t* sW = sKR;  // -W overwrites k r once L and P are done
  uint16_t* sQR = reinterpret_cast<uint16_t*>(smem + Ly::QR);
  uint16_t* sKC = reinterpret_cast<uint16_t*>(smem + Ly::KC);
  uint16_t* sQt = reinterpret_cast<uint16_t*>(smem + Ly::QT);
  uint16_t* sKtT = reinterpret_cast<uint16_t*>(smem + Ly::KTT);
  uint16_t* sKhT = reinterpret_cast<uint16_t*>(smem + Ly::KHT);
  uint16_t* sVT = reinterpret_cast<uint16_t*>(smem + Ly::VT);
  uint16_t* sLm = reinterpret_cast<uint16_t*>(smem + Ly::LM);
  uint16_t* sP = reinterpret_cast<uint16_t*>(smem + Ly::PM);
  uint16_t* sX = reinterpret_cast<uint16_t*>(smem + Ly::XM);
  float* sLd = reinterpret_cast<float*>(smem + Ly::LD);
  float* sD = reinterpret_cast<float*>(smem + Ly::DT);
  float* sGC = reinterpret_cast<float*>(smem + Ly::GC);
  float* sBeta = reinterpret_cast<float*>(smem + Ly::BT);

  // workgroup -> (b*H + h, slice); slices of one head share an XCD (and its L2)
  int bh, sl;
  {
    const int x = blockIdx.x;
    if (xcd_map) {
      const int idx = x >> 3;
      sl = idx % ns;
      bh = (idx / ns) * 8 + (x & 7);
    } else {
      sl = x % ns;
      bh = x / ns;
    }
  }
  const int h = bh % a.H;
  const int b = bh / a.H;
  const int j0 = sl * DVS;
  const int T = a.T;
  const int H = a.H;
  const int wv = threadIdx.x >> 6;
  const int ln = threadIdx.x & 63;
  const int g4 = ln >> 4;   // MFMA lane group
  const int r16 = ln & 15;  // MFMA lane row/column
  const int c0 = 2 * ln;    // gate layout: channels c0, c0+1

  const uint32_t* kq32 = static_cast<const uint32_t*>(a.q);
  const uint32_t* kk32 = static_cast<const uint32_t*>(a.k);
  const uint32_t* kz32 = static_cast<const uint32_t*>(a.z);
  const uint16_t* vv = static_cast<const uint16_t*>(a.v);
  const uint16_t* bb = static_cast<const uint16_t*>(a.beta);
  Tout* o = static_cast<Tout*>(a.o);

  // gate constants for the lane's two channels (log2 units)
  float ea0 = 0.f, ea1 = 0.f;
  const float gmin_l2e = a.g_min * kLog2e;
  if (FROM_Z) {
    ea0 = __expf(a.A[h * DK + c0]) * kLog2e;
    ea1 = __expf(a.A[h * DK + c0 + 1]) * kLog2e;
  }

  // fp32 state slice: S[u][ct] holds rows 16ct + 4 g4 + v, column 16 (wv + 4u) + r16
  f32x4 S[JPW][8];
#pragma unroll
  for (int u = 0; u < JPW; ++u) {
    const int jt = wv + 4 * u;
#pragma unroll
    for (int ct = 0; ct < 8; ++ct) {
#pragma unroll
      for (int v = 0; v < 4; ++v) {
        float x = 0.f;
        if (jt < NJT && a.S_in)
          x = a.S_in[(static_cast<int64_t>(bh) * DK + 16 * ct + 4 * g4 + v) * DK + j0 + 16 * jt + r16];
        S[u][ct][v] = x;
      }
    }
  }

  for (int t0 = 0; t0 < T; t0 += C) {
    const int n = min(C, T - t0);
    const int64_t row0 = (static_cast<int64_t>(b) * T + t0) * H + h;  // token t0's row index

    // ---------------- phase 1: gate, decays, operand tiles ----------------
    {
      const int i = wv;  // this wavefront's tile
      uint32_t kp[16], qp[16];
      float r0[16], r1[16], f0[16], f1[16];
      float D0 = 1.f, D1 = 1.f;
      if (FROM_Z) {
        float al0[16], al1[16];
#pragma unroll
        for (int tt = 0; tt < 16; ++tt) {
          const int t = 16 * i + tt;
          if (t < n) {
            const int64_t e = ((row0 + static_cast<int64_t>(t) * H) * DK + c0) >> 1;
            kp[tt] = kk32[e];
            qp[tt] = kq32[e];
            const uint32_t zp = kz32[e];
            al0[tt] = fast_exp2(gate_log2(bflo(zp), ea0, gmin_l2e));
            al1[tt] = fast_exp2(gate_log2(bfhi(zp), ea1, gmin_l2e));
          } else {
            kp[tt] = 0u;
            qp[tt] = 0u;
            al0[tt] = 1.f;
            al1[tt] = 1.f;
          }
        }
#pragma unroll
        for (int tt = 0; tt < 16; ++tt) {
          D0 *= al0[tt];
          D1 *= al1[tt];
          r0[tt] = D0;
          r1[tt] = D1;
        }
        float s0 = 1.f, s1 = 1.f;
#pragma unroll
        for (int tt = 15; tt >= 0; --tt) {
          f0[tt] = s0;
          f1[tt] = s1;
          s0 *= al0[tt];
          s1 *= al1[tt];
        }
      } else {
        // chunk-local sums G (natural log) -> log2 within this tile
        float G0[16], G1[16];
        const float2* G2 = reinterpret_cast<const float2*>(a.G);
        float base0 = 0.f, base1 = 0.f;
        if (i > 0 && 16 * i < n) {
          const float2 gb = G2[((row0 + static_cast<int64_t>(16 * i - 1) * H) * DK + c0) >> 1];
          base0 = gb.x * kLog2e;
          base1 = gb.y * kLog2e;
        }
        float last0 = base0, last1 = base1;
#pragma unroll
        for (int tt = 0; tt < 16; ++tt) {
          const int t = 16 * i + tt;
          if (t < n) {
            const int64_t e = ((row0 + static_cast<int64_t>(t) * H) * DK + c0) >> 1;
            kp[tt] = kk32[e];
            qp[tt] = kq32[e];
            const float2 gg = G2[e];
            G0[tt] = gg.x * kLog2e;
            G1[tt] = gg.y * kLog2e;
            last0 = G0[tt];
            last1 = G1[tt];
          } else {
            kp[tt] = 0u;
            qp[tt] = 0u;
            G0[tt] = last0;
            G1[tt] = last1;
          }
        }
#pragma unroll
        for (int tt = 0; tt < 16; ++tt) {
          r0[tt] = fast_exp2(G0[tt] - base0);
          r1[tt] = fast_exp2(G1[tt] - base1);
          f0[tt] = fast_exp2(last0 - G0[tt]);
          f1[tt] = fast_exp2(last1 - G1[tt]);
        }
        D0 = fast_exp2(last0 - base0);
        D1 = fast_exp2(last1 - base1);
      }
      sD[i * DK + c0] = D0;
      sD[i * DK + c0 + 1] = D1;
      if (ln < 16) {
        const int t = 16 * i + ln;
        sBeta[t] = t < n ? bf16_to_f32(bb[row0 + static_cast<int64_t>(t) * H]) : 0.f;
      }
#pragma unroll
      for (int tt = 0; tt < 16; ++tt) {
        const int t = 16 * i + tt;
        const float k0 = bflo(kp[tt]), k1 = bfhi(kp[tt]);
        const float q0 = bflo(qp[tt]), q1 = bfhi(qp[tt]);
        *reinterpret_cast<uint32_t*>(&sKR[t * RS + c0]) = pack2(k0 * r0[tt], k1 * r1[tt]);
        *reinterpret_cast<uint32_t*>(&sQR[t * RS + c0]) = pack2(q0 * r0[tt], q1 * r1[tt]);
        *reinterpret_cast<uint32_t*>(&sKC[t * RS + c0]) = pack2(k0 * f0[tt], k1 * f1[tt]);
      }
      // v^T for the slice's columns: lane -> columns ln*(DVS/64).. (DVS >= 64) or ln (< DVS)
      constexpr int VPL = DVS >= 64 ? DVS / 64 : 1;
      if (ln * VPL < DVS) {
#pragma unroll
        for (int cc = 0; cc < VPL; ++cc) {
          const int jc = ln * VPL + cc;
          uint32_t w[8];
#pragma unroll
          for (int tp = 0; tp < 8; ++tp) {
            uint32_t lo = 0u, hi = 0u;
            const int t = 16 * i + 2 * tp;
            if (t < n) lo = vv[(row0 + static_cast<int64_t>(t) * H) * DK + j0 + jc];
            if (t + 1 < n) hi = vv[(row0 + static_cast<int64_t>(t + 1) * H) * DK + j0 + jc];
            w[tp] = lo | (hi << 16);
          }
          u32x4* dst = reinterpret_cast<u32x4*>(&sVT[jc * TS + 16 * i]);
          dst[0] = u32x4{w[0], w[1], w[2], w[3]};
          dst[1] = u32x4{w[4], w[5], w[6], w[7]};
        }
      }
      __syncthreads();
      float eB0 = 1.f, eB1 = 1.f, af0 = 1.f, af1 = 1.f, gc0 = 1.f, gc1 = 1.f;
#pragma unroll
      for (int ii = 0; ii < 4; ++ii) {
        const float d0 = sD[ii * DK + c0], d1 = sD[ii * DK + c0 + 1];
        if (ii < i) { eB0 *= d0; eB1 *= d1; }
        if (ii > i) { af0 *= d0; af1 *= d1; }
        gc0 *= d0;
        gc1 *= d1;
      }
      if (wv == 0) {
        sGC[c0] = gc0;
        sGC[c0 + 1] = gc1;
      }
      uint32_t kt0[8], kt1[8], kh0[8], kh1[8];
#pragma unroll
      for (int tt = 0; tt < 16; ++tt) {
        const int t = 16 * i + tt;
        const float k0 = bflo(kp[tt]), k1 = bfhi(kp[tt]);
        const float q0 = bflo(qp[tt]), q1 = bfhi(qp[tt]);
        *reinterpret_cast<uint32_t*>(&sQt[t * RS + c0]) = pack2(q0 * r0[tt] * eB0, q1 * r1[tt] * eB1);
        const uint32_t a0 = f2bf(k0 * r0[tt] * eB0), a1 = f2bf(k1 * r1[tt] * eB1);
        const uint32_t b0 = f2bf(k0 * f0[tt] * af0), b1 = f2bf(k1 * f1[tt] * af1);
        if (tt & 1) {
          kt0[tt >> 1] |= a0 << 16; kt1[tt >> 1] |= a1 << 16;
          kh0[tt >> 1] |= b0 << 16; kh1[tt >> 1] |= b1 << 16;
        } else {
          kt0[tt >> 1] = a0; kt1[tt >> 1] = a1;
          kh0[tt >> 1] = b0; kh1[tt >> 1] = b1;
        }
      }
      u32x4* d;
      d = reinterpret_cast<u32x4*>(&sKtT[c0 * TS + 16 * i]);
      d[0] = u32x4{kt0[0], kt0[1], kt0[2], kt0[3]}; d[1] = u32x4{kt0[4], kt0[5], kt0[6], kt0[7]};
      d = reinterpret_cast<u32x4*>(&sKtT[(c0 + 1) * TS + 16 * i]);
      d[0] = u32x4{kt1[0], kt1[1], kt1[2], kt1[3]}; d[1] = u32x4{kt1[4], kt1[5], kt1[6], kt1[7]};
      d = reinterpret_cast<u32x4*>(&sKhT[c0 * TS + 16 * i]);
      d[0] = u32x4{kh0[0], kh0[1], kh0[2], kh0[3]}; d[1] = u32x4{kh0[4], kh0[5], kh0[6], kh0[7]};
      d = reinterpret_cast<u32x4*>(&sKhT[(c0 + 1) * TS + 16 * i]);
      d[0] = u32x4{kh1[0], kh1[1], kh1[2], kh1[3]}; d[1] = u32x4{kh1[4], kh1[5], kh1[6], kh1[7]};
    }
    __syncthreads();

    // ---------------- phase 2: L and P tiles ----------------
#pragma unroll
    for (int p = 0; p < 3; ++p) {
      const int i = kPairs[wv][p][0];
      const int j = kPairs[wv][p][1];
      if (i < 0) continue;
      f32x4 accL = {0.f, 0.f, 0.f, 0.f}, accP = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int kb = 0; kb < 4; ++kb) {
        const int cb = 32 * kb + 8 * g4;
        float f[8];
        if (i == j) {
#pragma unroll
          for (int v = 0; v < 8; ++v) f[v] = fast_rcp(sD[i * DK + cb + v]);
        } else {
#pragma unroll
          for (int v = 0; v < 8; ++v) f[v] = 1.f;
          for (int ii = j + 1; ii < i; ++ii) {
#pragma unroll
            for (int v = 0; v < 8; ++v) f[v] *= sD[ii * DK + cb + v];
          }
        }
        const u32x4 kc = lds128(&sKC[(16 * j + r16) * RS + cb]);
        u32x4 A;
#pragma unroll
        for (int w2 = 0; w2 < 4; ++w2)
          A[w2] = pack2(bflo(kc[w2]) * f[2 * w2], bfhi(kc[w2]) * f[2 * w2 + 1]);
        const u32x4 Bk = lds128(&sKR[(16 * i + r16) * RS + cb]);
        const u32x4 Bq = lds128(&sQR[(16 * i + r16) * RS + cb]);
        accL = mma32(A, Bk, accL);
        accP = mma32(A, Bq, accP);
      }
      // lane holds L^T / P^T at rows s = 16j + 4 g4 + v, column t = 16i + r16
      const int t = 16 * i + r16;
      const float bt = sBeta[t];
      f32x4 pv;
      if (i == j) {
#pragma unroll
        for (int v = 0; v < 4; ++v) {
          const int s = 4 * g4 + v;
          sLd[(i * 16 + r16) * LDS_ + s] = s < r16 ? bt * accL[v] : 0.f;
          pv[v] = s <= r16 ? accP[v] : 0.f;
        }
      } else {
        f32x4 nl;
#pragma unroll
        for (int v = 0; v < 4; ++v) nl[v] = -bt * accL[v];
        *reinterpret_cast<s16x4*>(&sLm[t * TS + 16 * j + 4 * g4]) = cvt4(nl);
        pv = accP;
      }
      *reinterpret_cast<s16x4*>(&sP[t * TS + 16 * j + 4 * g4]) = cvt4(pv);
    }
    __syncthreads();

    // ---------------- phase 3: diagonal inverses X_ii = (I + L_ii)^-1 ----------------
    if (ln < 16) {
      const int i = wv, jj = ln;
      const float* Ld = sLd + i * 16 * LDS_;
      float x[16];
#pragma unroll
      for (int r = 0; r < 16; ++r) {
        float acc = (r == jj) ? 1.f : 0.f;
#pragma unroll
        for (int m = 0; m < r; ++m) acc -= Ld[r * LDS_ + m] * x[m];
        x[r] = acc;
      }
#pragma unroll
      for (int r = 0; r < 16; ++r) sX[(i * 16 + r) * XS + jj] = f2bf(x[r]);
    }
    __syncthreads();

    // ---------------- phase 4: (I + L) [W | Ut] = Diag(beta) [K Gamma | V] ----------------
    f32x4 Ut[JPW][4];
#pragma unroll
    for (int col = 0; col < 2 + JPW; ++col) {
      // columns 0,1: key-channel tiles 2wv, 2wv+1 of W; then value tiles wv + 4u of Ut
      const bool is_w = col < 2;
      const int u = col - 2;
      const int ct = is_w ? 2 * wv + col : wv + 4 * u;
      if (!is_w && ct >= NJT) continue;
      const uint16_t* Y = is_w ? sKtT : sVT;
      f32x4 Z[4];
      s16x4 Zb[4];
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const s16x4 yv = lds64(&Y[(16 * ct + r16) * TS + 16 * i + 4 * g4]);
        f32x4 acc;
#pragma unroll
        for (int v = 0; v < 4; ++v)
          acc[v] = sBeta[16 * i + 4 * g4 + v] * bf16_to_f32(static_cast<uint16_t>(yv[v]));
#pragma unroll
        for (int j = 0; j < i; ++j) acc = mma16(lds64(&sLm[(16 * i + r16) * TS + 16 * j + 4 * g4]), Zb[j], acc);
        const f32x4 zero = {0.f, 0.f, 0.f, 0.f};
        Z[i] = mma16(lds64(&sX[(16 * i + r16) * XS + 4 * g4]), cvt4(acc), zero);
        Zb[i] = cvt4(Z[i]);
      }
      if (is_w) {
#pragma unroll
        for (int i = 0; i < 4; ++i)
#pragma unroll
          for (int v = 0; v < 4; ++v) sW[(16 * i + 4 * g4 + v) * RS + 16 * ct + r16] = f2bf(-Z[i][v]);
      } else {
#pragma unroll
        for (int i = 0; i < 4; ++i) Ut[u][i] = Z[i];
      }
    }
    __syncthreads();

    // ---------------- phases 5-7: U, outputs, state update (per owned value tile) ----------------
#pragma unroll
    for (int u = 0; u < JPW; ++u) {
      const int jt = wv + 4 * u;
      if (jt >= NJT) continue;
      s16x4 Sb[8];
#pragma unroll
      for (int ct = 0; ct < 8; ++ct) Sb[ct] = cvt4(S[u][ct]);
      // U = Ut + (-W) S
      s16x4 Ub[4];
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        f32x4 acc = Ut[u][i];
#pragma unroll
        for (int ct = 0; ct < 8; ++ct) acc = mma16(lds64(&sW[(16 * i + r16) * RS + 16 * ct + 4 * g4]), Sb[ct], acc);
        Ub[i] = cvt4(acc);
      }
      // O = (Q Gamma) S + P U
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        f32x4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int ct = 0; ct < 8; ++ct) acc = mma16(lds64(&sQt[(16 * i + r16) * RS + 16 * ct + 4 * g4]), Sb[ct], acc);
#pragma unroll
        for (int m = 0; m <= i; ++m) acc = mma16(lds64(&sP[(16 * i + r16) * TS + 16 * m + 4 * g4]), Ub[m], acc);
#pragma unroll
        for (int v = 0; v < 4; ++v) {
          const int t = 16 * i + 4 * g4 + v;
          if (t < n)
            io<Tout>::store(o, (row0 + static_cast<int64_t>(t) * H) * DK + j0 + 16 * jt + r16, a.scale * acc[v]);
        }
      }
      // S <- Diag(Gamma_C) S + (K Gamma_C / Gamma)^T U
#pragma unroll
      for (int ct = 0; ct < 8; ++ct) {
        f32x4 acc;
#pragma unroll
        for (int v = 0; v < 4; ++v) acc[v] = S[u][ct][v] * sGC[16 * ct + 4 * g4 + v];
#pragma unroll
        for (int m = 0; m < 4; ++m) acc = mma16(lds64(&sKhT[(16 * ct + r16) * TS + 16 * m + 4 * g4]), Ub[m], acc);
        S[u][ct] = acc;
      }
    }
    __syncthreads();
  }

  if (a.S_out) {
#pragma unroll
    for (int u = 0; u < JPW; ++u) {
      const int jt = wv + 4 * u;
      if (jt >= NJT) continue;
#pragma unroll
      for (int ct = 0; ct < 8; ++ct)
#pragma unroll
        for (int v = 0; v < 4; ++v)
          a.S_out[(static_cast<int64_t>(bh) * DK + 16 * ct + 4 * g4 + v) * DK + j0 + 16 * jt + r16] = S[u][ct][v];
    }
  }
}

bool chunk_mfma_supports(const ChunkArgs& a) {
  return a.in_bf16 && a.dk == 128 && a.dv == 128 && a.chunk == 64;
}

template <int DVS, bool FROM_Z, typename Tout>
static hipError_t launch_mfma_t(const ChunkArgs& a, hipStream_t st, int ns) {
  auto kern = chunk_mfma_kernel<DVS, FROM_Z, Tout>;
  constexpr int bytes = mf::Layout<DVS>::BYTES;
  static bool attr_set = false;  // set once per instantiation (idempotent if raced)
  if (!attr_set) {
    hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void*>(kern),
                                       hipFuncAttributeMaxDynamicSharedMemorySize, bytes);
    if (e != hipSuccess) return e;
    attr_set = true;
  }
  const int64_t nbh = static_cast<int64_t>(a.B) * a.H;
  const int64_t nblocks = nbh * ns;
  const int xcd_map = (nbh % 8 == 0) ? 1 : 0;
  hipLaunchKernelGGL(kern, dim3(static_cast<uint32_t>(nblocks)), dim3(mf::NTH), bytes, st, a, ns, xcd_map);
  return hipGetLastError();
}

template <int DVS>
static hipError_t launch_mfma_d(const ChunkArgs& a, hipStream_t st, int ns) {
  if (a.from_z)
    return a.out_bf16 ? launch_mfma_t<DVS, true, bf16_t>(a, st, ns) : launch_mfma_t<DVS, true, float>(a, st, ns);
  return a.out_bf16 ? launch_mfma_t<DVS, false, bf16_t>(a, st, ns) : launch_mfma_t<DVS, false, float>(a, st, ns);
}

hipError_t launch_chunk_mfma(const ChunkArgs& a, hipStream_t st) {
  if (!chunk_mfma_supports(a)) return hipErrorNotSupported;
  const int64_t nbh = static_cast<int64_t>(a.B) * a.H;
  if (nbh == 0) return hipSuccess;
  // value-column slices: enough workgroups to cover the 256 compute units,
  // at most 64 columns per slice (the state slice then fits the registers)
  int ns = 2;
  while (ns < 8 && nbh * ns < 256) ns *= 2;
  if (nbh * ns > 0x7fffffffLL) return hipErrorInvalidConfiguration;
  switch (ns) {
    case 2: return launch_mfma_d<64>(a, st, 2);
    case 4: return launch_mfma_d<32>(a, st, 4);
    default: return launch_mfma_d<16>(a, st, 8);
  }
}

}  // namespace kda
