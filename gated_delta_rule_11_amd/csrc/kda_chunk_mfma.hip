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
constexpr int LTS = 20;        // row stride (floats) of the transposed fp32 diagonal L blocks

// pair (i, j <= i) of 16-token tiles -> slot of its anchored key tile
__host__ __device__ constexpr int slot(int i, int j) { return i * (i + 1) / 2 + j; }

template <int DVS>
struct Layout {
  static constexpr int KR = 0;                          // [64][RS]  k r       (later: -W)
  static constexpr int QR = KR + C * RS * 2;            // [64][RS]  q r
  static constexpr int KA = QR + C * RS * 2;            // [10][16][RS] anchored keys k e^(B_i - G)
  static constexpr int QT = KA + 10 * 16 * RS * 2;      // [64][RS]  q Gamma
  static constexpr int KHT = QT + C * RS * 2;           // [128][TS] (k Gamma_C/Gamma)^T
  static constexpr int VT = KHT + DK * TS * 2;          // [DVS][TS] v^T
  static constexpr int LM = VT + DVS * TS * 2;          // [64][TS]  -L (off-diagonal tiles)
  static constexpr int PM = LM + C * TS * 2;            // [64][TS]  P
  static constexpr int XM = PM + C * TS * 2;            // [4][16][XS] diagonal inverses (bf16)
  static constexpr int LT = XM + 4 * 16 * XS * 2;       // [4][16][LTS] fp32 diagonal L, transposed
  static constexpr int DT = LT + 4 * 16 * LTS * 4;      // [4][128] fp32 tile decays D_i
  static constexpr int EB = DT + 4 * DK * 4;            // [4][128] fp32 decay before tile i
  static constexpr int GC = EB + 4 * DK * 4;            // [128] fp32 chunk decay
  static constexpr int BT = GC + DK * 4;                // [64] fp32 beta
  static constexpr int BYTES = BT + C * 4;
  static_assert(BYTES <= 160 * 1024, "LDS budget");
};

// Raw buffer resource: base, byte range.  The hardware range check covers the
// per-lane offset only, not the scalar (token) offset, so every token offset
// used below is clamped to the chunk's last valid token by construction.
constexpr int kRsrcFlags = 0x00020000;
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
__device__ __forceinline__ u32x4 cat(s16x4 lo, s16x4 hi) {
  const u32x2 l = __builtin_bit_cast(u32x2, lo), h = __builtin_bit_cast(u32x2, hi);
  return u32x4{l[0], l[1], h[0], h[1]};
}
__device__ __forceinline__ f32x4 mma16(s16x4 a, s16x4 b, f32x4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(a, b, c, 0, 0, 0);
}
// 16x16x32: lane group g holds k = 8g..8g+7 of both operands, so any
// consistent assignment of channels to those slots gives the same product.
__device__ __forceinline__ f32x4 mma32(u32x4 a, u32x4 b, f32x4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, a), __builtin_bit_cast(bf16x8, b), c,
                                                 0, 0, 0);
}
__device__ __forceinline__ __amdgpu_buffer_rsrc_t rsrc(const void* base, int64_t bytes) {
  const int nrec = bytes > 0x7fffffffLL ? 0x7fffffff : static_cast<int>(bytes);
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), static_cast<short>(0), nrec, mf::kRsrcFlags);
}
__device__ __forceinline__ uint32_t bload32(__amdgpu_buffer_rsrc_t r, int voff, int soff) {
  return __builtin_amdgcn_raw_buffer_load_b32(r, voff, soff, 0);
}

// One wavefront's raw inputs for its 16-token tile of a chunk (gate layout:
// lane -> channels 2*lane, 2*lane+1), loaded ahead of use.
template <int DVS>
struct RawTile {
  static constexpr int VPL = DVS >= 64 ? DVS / 64 : 1;  // value columns per lane
  uint32_t k[16], q[16], zg[16], zg2[16];  // bf16 pairs; z (bf16 pairs) or G (fp32 x, fp32 y)
  uint32_t gb0, gb1;                       // G at the token before the tile (G input only)
  uint32_t v[VPL][16];
  uint32_t beta;
};

template <int DVS, bool FROM_Z>
__device__ __forceinline__ void load_tile(RawTile<DVS>& R, const ChunkArgs& a, int b, int h, int t0, int i, int ln,
                                          int j0) {
  using namespace mf;
  const int T = a.T, H = a.H;
  const int n = min(C, T - t0);
  const int64_t row0 = (static_cast<int64_t>(b) * T + t0) * H + h;
  const int64_t span = static_cast<int64_t>(n - 1) * H + 1;
  const int rowb = H * DK * 2;
  const int c0 = 2 * ln;
  const auto rq = rsrc(static_cast<const uint16_t*>(a.q) + row0 * DK, span * DK * 2);
  const auto rk = rsrc(static_cast<const uint16_t*>(a.k) + row0 * DK, span * DK * 2);
  const auto rv = rsrc(static_cast<const uint16_t*>(a.v) + row0 * DK + j0, span * DK * 2);
  const auto rb = rsrc(static_cast<const uint16_t*>(a.beta) + row0, span * 2);
  // padded tokens read the last valid token and are masked by the consumer
#pragma unroll
  for (int tt = 0; tt < 16; ++tt) {
    const int so = min(16 * i + tt, n - 1) * rowb;
    R.k[tt] = bload32(rk, c0 * 2, so);
    R.q[tt] = bload32(rq, c0 * 2, so);
  }
  if (FROM_Z) {
    const auto rz = rsrc(static_cast<const uint16_t*>(a.z) + row0 * DK, span * DK * 2);
#pragma unroll
    for (int tt = 0; tt < 16; ++tt) R.zg[tt] = bload32(rz, c0 * 2, min(16 * i + tt, n - 1) * rowb);
  } else {
    const auto rg = rsrc(a.G + row0 * DK, span * DK * 4);
#pragma unroll
    for (int tt = 0; tt < 16; ++tt) {
      const u32x2 g = __builtin_bit_cast(
          u32x2, __builtin_amdgcn_raw_buffer_load_b64(rg, c0 * 4, min(16 * i + tt, n - 1) * rowb * 2, 0));
      R.zg[tt] = g[0];
      R.zg2[tt] = g[1];
    }
    const u32x2 gb = __builtin_bit_cast(
        u32x2, __builtin_amdgcn_raw_buffer_load_b64(rg, c0 * 4, min(max(16 * i - 1, 0), n - 1) * rowb * 2, 0));
    R.gb0 = gb[0];
    R.gb1 = gb[1];
  }
  constexpr int VPL = RawTile<DVS>::VPL;
  if (ln * VPL < DVS) {
#pragma unroll
    for (int cc = 0; cc < VPL; ++cc)
#pragma unroll
      for (int tt = 0; tt < 16; ++tt)
        R.v[cc][tt] = __builtin_amdgcn_raw_buffer_load_b16(rv, (ln * VPL + cc) * 2, min(16 * i + tt, n - 1) * rowb, 0);
  }
  if (ln < 16) R.beta = __builtin_amdgcn_raw_buffer_load_b16(rb, min(16 * i + ln, n - 1) * H * 2, 0, 0);
}

// Tile pairs (i, j < i) of the L / P products per wavefront; each wavefront's
// diagonal pair (wv, wv) is handled first and separately.
__constant__ int8_t kOffPairs[4][2][2] = {{{3, 0}, {3, 1}}, {{1, 0}, {3, 2}}, {{2, 0}, {-1, -1}}, {{2, 1}, {-1, -1}}};

template <int DVS, bool FROM_Z, typename Tout>
__global__ __launch_bounds__(mf::NTH) void chunk_mfma_kernel(const ChunkArgs a, int ns, int xcd_map) {
  using namespace mf;
  using Ly = Layout<DVS>;
  constexpr int NJT = DVS / 16;              // value-column tiles in the slice
  constexpr int JPW = (NJT + 3) / 4;         // value-column tiles per wavefront (max)
  constexpr int ES = sizeof(Tout);

  extern __shared__ __attribute__((aligned(16))) unsigned char smem[];
  uint16_t* sKR = reinterpret_cast<uint16_t*>(smem + Ly::KR);
  uint16_t* sW = sKR;  // -W overwrites k r column by column (each wavefront its own columns)
  uint16_t* sQR = reinterpret_cast<uint16_t*>(smem + Ly::QR);
  uint16_t* sKA = reinterpret_cast<uint16_t*>(smem + Ly::KA);
  uint16_t* sQt = reinterpret_cast<uint16_t*>(smem + Ly::QT);
  uint16_t* sKhT = reinterpret_cast<uint16_t*>(smem + Ly::KHT);
  uint16_t* sVT = reinterpret_cast<uint16_t*>(smem + Ly::VT);
  uint16_t* sLm = reinterpret_cast<uint16_t*>(smem + Ly::LM);
  uint16_t* sP = reinterpret_cast<uint16_t*>(smem + Ly::PM);
  uint16_t* sX = reinterpret_cast<uint16_t*>(smem + Ly::XM);
  float* sLT = reinterpret_cast<float*>(smem + Ly::LT);
  float* sD = reinterpret_cast<float*>(smem + Ly::DT);
  float* sEB = reinterpret_cast<float*>(smem + Ly::EB);
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
  const int wv = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int ln = threadIdx.x & 63;
  const int g4 = ln >> 4;   // MFMA lane group
  const int r16 = ln & 15;  // MFMA lane row/column
  const int c0 = 2 * ln;    // gate layout: channels c0, c0+1

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

  RawTile<DVS> raw;
  if (T > 0) load_tile<DVS, FROM_Z>(raw, a, b, h, 0, wv, ln, j0);

  for (int t0 = 0; t0 < T; t0 += C) {
    const int n = min(C, T - t0);
    const int64_t row0 = (static_cast<int64_t>(b) * T + t0) * H + h;  // token t0's row index
    const int64_t span = static_cast<int64_t>(n - 1) * H + 1;         // rows this chunk may touch

    // ---------------- phase 1: gate, decays, operand tiles ----------------
    const int i1 = wv;  // this wavefront's tile
    uint32_t kp[16], qp[16];
    float r0[16], r1[16], f0[16], f1[16];
    float D0 = 1.f, D1 = 1.f;
    {
      const int i = i1;
#pragma unroll
      for (int tt = 0; tt < 16; ++tt) {
        const bool valid = 16 * i + tt < n;
        kp[tt] = valid ? raw.k[tt] : 0u;
        qp[tt] = valid ? raw.q[tt] : 0u;
      }
      if (FROM_Z) {
        float al0[16], al1[16];
#pragma unroll
        for (int tt = 0; tt < 16; ++tt) {
          const bool valid = 16 * i + tt < n;
          al0[tt] = valid ? fast_exp2(gate_log2(bflo(raw.zg[tt]), ea0, gmin_l2e)) : 1.f;
          al1[tt] = valid ? fast_exp2(gate_log2(bfhi(raw.zg[tt]), ea1, gmin_l2e)) : 1.f;
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
        // chunk-local sums G (natural log, fp32) -> log2 within this tile
        float G0[16], G1[16];
        float base0 = 0.f, base1 = 0.f;
        if (i > 0 && 16 * i < n) {
          base0 = __uint_as_float(raw.gb0) * kLog2e;
          base1 = __uint_as_float(raw.gb1) * kLog2e;
        }
        float last0 = base0, last1 = base1;
#pragma unroll
        for (int tt = 0; tt < 16; ++tt) {
          if (16 * i + tt < n) {
            G0[tt] = __uint_as_float(raw.zg[tt]) * kLog2e;
            G1[tt] = __uint_as_float(raw.zg2[tt]) * kLog2e;
            last0 = G0[tt];
            last1 = G1[tt];
          } else {
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
        sBeta[t] = t < n ? bf16_to_f32(static_cast<uint16_t>(raw.beta)) : 0.f;
      }
#pragma unroll
      for (int tt = 0; tt < 16; ++tt) {
        const int t = 16 * i + tt;
        *reinterpret_cast<uint32_t*>(&sKR[t * RS + c0]) = pack2(bflo(kp[tt]) * r0[tt], bfhi(kp[tt]) * r1[tt]);
        *reinterpret_cast<uint32_t*>(&sQR[t * RS + c0]) = pack2(bflo(qp[tt]) * r0[tt], bfhi(qp[tt]) * r1[tt]);
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
            const int t = 16 * i + 2 * tp;
            const uint32_t lo = t < n ? (raw.v[cc][2 * tp] & 0xffffu) : 0u;
            const uint32_t hi = t + 1 < n ? (raw.v[cc][2 * tp + 1] & 0xffffu) : 0u;
            w[tp] = lo | (hi << 16);
          }
          u32x4* dst = reinterpret_cast<u32x4*>(&sVT[jc * TS + 16 * i]);
          dst[0] = u32x4{w[0], w[1], w[2], w[3]};
          dst[1] = u32x4{w[4], w[5], w[6], w[7]};
        }
      }
    }
    __syncthreads();
    {
      const int i = i1;
      float d0[4], d1[4];
#pragma unroll
      for (int ii = 0; ii < 4; ++ii) {
        d0[ii] = sD[ii * DK + c0];
        d1[ii] = sD[ii * DK + c0 + 1];
      }
      float eB0 = 1.f, eB1 = 1.f, af0 = 1.f, af1 = 1.f;
#pragma unroll
      for (int ii = 0; ii < 4; ++ii) {
        if (ii < i) { eB0 *= d0[ii]; eB1 *= d1[ii]; }
        if (ii > i) { af0 *= d0[ii]; af1 *= d1[ii]; }
      }
      sEB[i * DK + c0] = eB0;
      sEB[i * DK + c0 + 1] = eB1;
      if (i == 0) {
        sGC[c0] = af0 * D0;
        sGC[c0 + 1] = af1 * D1;
      }
      // q Gamma (token-major) and (k Gamma_C / Gamma)^T (channel-major)
      uint32_t kh0[8], kh1[8];
#pragma unroll
      for (int tt = 0; tt < 16; ++tt) {
        const int t = 16 * i + tt;
        *reinterpret_cast<uint32_t*>(&sQt[t * RS + c0]) =
            pack2(bflo(qp[tt]) * r0[tt] * eB0, bfhi(qp[tt]) * r1[tt] * eB1);
        const uint32_t b0 = f2bf(bflo(kp[tt]) * f0[tt] * af0), b1 = f2bf(bfhi(kp[tt]) * f1[tt] * af1);
        if (tt & 1) {
          kh0[tt >> 1] |= b0 << 16; kh1[tt >> 1] |= b1 << 16;
        } else {
          kh0[tt >> 1] = b0; kh1[tt >> 1] = b1;
        }
      }
      u32x4* d = reinterpret_cast<u32x4*>(&sKhT[c0 * TS + 16 * i]);
      d[0] = u32x4{kh0[0], kh0[1], kh0[2], kh0[3]}; d[1] = u32x4{kh0[4], kh0[5], kh0[6], kh0[7]};
      d = reinterpret_cast<u32x4*>(&sKhT[(c0 + 1) * TS + 16 * i]);
      d[0] = u32x4{kh1[0], kh1[1], kh1[2], kh1[3]}; d[1] = u32x4{kh1[4], kh1[5], kh1[6], kh1[7]};
      // anchored keys of this tile (j = i) for every tile m >= i:
      //   k_s e^(B_m - G_s) = (k_s sf_s) * (m == i ? 1 / D_i : prod_{i < ii < m} D_ii)
      for (int m = i; m < 4; ++m) {
        float fa0, fa1;
        if (m == i) {
          fa0 = fast_rcp(D0);
          fa1 = fast_rcp(D1);
        } else {
          fa0 = 1.f;
          fa1 = 1.f;
#pragma unroll
          for (int ii = 0; ii < 4; ++ii)
            if (ii > i && ii < m) { fa0 *= d0[ii]; fa1 *= d1[ii]; }
        }
        uint16_t* dst = sKA + slot(m, i) * 16 * RS + c0;
#pragma unroll
        for (int tt = 0; tt < 16; ++tt)
          *reinterpret_cast<uint32_t*>(dst + tt * RS) =
              pack2(bflo(kp[tt]) * f0[tt] * fa0, bfhi(kp[tt]) * f1[tt] * fa1);
      }
    }
    // the next chunk's raw tile is fetched now and lands during phases 2-4
    if (t0 + C < T) load_tile<DVS, FROM_Z>(raw, a, b, h, t0 + C, wv, ln, j0);
    __syncthreads();

    // ---------------- phase 2: L and P tiles, diagonal inverses ----------------
    {
      // L^T / P^T tile for pair (i, j): rows s of tile j, columns t of tile i
      auto lp_tile = [&](int i, int j, f32x4& accL, f32x4& accP) {
        accL = f32x4{0.f, 0.f, 0.f, 0.f};
        accP = f32x4{0.f, 0.f, 0.f, 0.f};
        const uint16_t* Ar = sKA + (slot(i, j) * 16 + r16) * RS;
#pragma unroll
        for (int kb = 0; kb < 4; ++kb) {
          const int cb = 32 * kb + 8 * g4;
          const u32x4 A = lds128(Ar + cb);
          accL = mma32(A, lds128(&sKR[(16 * i + r16) * RS + cb]), accL);
          accP = mma32(A, lds128(&sQR[(16 * i + r16) * RS + cb]), accP);
        }
      };
      const int i = wv;
      f32x4 dL, dP;
      lp_tile(i, i, dL, dP);
      // lane holds L^T / P^T at rows s = 4 g4 + v, column t = r16 (both in tile i)
      {
        const float bt = sBeta[16 * i + r16];
        f32x4 pv;
#pragma unroll
        for (int v = 0; v < 4; ++v) {
          const int s = 4 * g4 + v;
          sLT[(i * 16 + s) * LTS + r16] = s < r16 ? bt * dL[v] : 0.f;  // L[t][s] stored at [s][t]
          pv[v] = s <= r16 ? dP[v] : 0.f;
        }
        *reinterpret_cast<s16x4*>(&sP[(16 * i + r16) * TS + 16 * i + 4 * g4]) = cvt4(pv);
      }
      // off-diagonal pairs of this wavefront (issued before the inverse so they overlap it)
      f32x4 oL[2], oP[2];
#pragma unroll
      for (int p = 0; p < 2; ++p) {
        const int pi = kOffPairs[wv][p][0], pj = kOffPairs[wv][p][1];
        if (pi >= 0) lp_tile(pi, pj, oL[p], oP[p]);
      }
      // X_ii = (I + L_ii)^-1, one column per lane (lanes 0..15), right-looking
      __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
      __builtin_amdgcn_wave_barrier();
      __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
      if (ln < 16) {
        const float* Lt = sLT + i * 16 * LTS;
        float x[16];
#pragma unroll
        for (int r = 0; r < 16; ++r) x[r] = (r == ln) ? 1.f : 0.f;
#pragma unroll
        for (int m = 0; m < 15; ++m) {
#pragma unroll
          for (int r = m + 1; r < 16; ++r) x[r] -= Lt[m * LTS + r] * x[m];
        }
#pragma unroll
        for (int r = 0; r < 16; ++r) sX[(16 * i + r) * XS + ln] = f2bf(x[r]);
      }
#pragma unroll
      for (int p = 0; p < 2; ++p) {
        const int pi = kOffPairs[wv][p][0], pj = kOffPairs[wv][p][1];
        if (pi < 0) continue;
        const int t = 16 * pi + r16;
        const float bt = sBeta[t];
        f32x4 nl;
#pragma unroll
        for (int v = 0; v < 4; ++v) nl[v] = -bt * oL[p][v];
        *reinterpret_cast<s16x4*>(&sLm[t * TS + 16 * pj + 4 * g4]) = cvt4(nl);
        *reinterpret_cast<s16x4*>(&sP[t * TS + 16 * pj + 4 * g4]) = cvt4(oP[p]);
      }
    }
    __syncthreads();

    // ---------------- phase 3: (I + L) [W | Ut] = Diag(beta) [K Gamma | V] ----------------
    // columns: 0, 1 -> key-channel tiles 2wv, 2wv+1 of W; 2.. -> value tiles wv + 4u of Ut
    constexpr int NCOL = 2 + JPW;
    f32x4 Z[NCOL][4];
    {
      s16x4 Zb[NCOL][4];
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        float bt[4];
#pragma unroll
        for (int v = 0; v < 4; ++v) bt[v] = sBeta[16 * i + 4 * g4 + v];
#pragma unroll
        for (int col = 0; col < NCOL; ++col) {
          const bool is_w = col < 2;
          const int ct = is_w ? 2 * wv + col : wv + 4 * (col - 2);
          if (!is_w && ct >= NJT) continue;
          f32x4 acc;
          if (is_w) {  // K Gamma = (k r) * eB_i, rows t = 16i + 4 g4 + v, channel 16 ct + r16
            const float e = sEB[i * DK + 16 * ct + r16];
#pragma unroll
            for (int v = 0; v < 4; ++v)
              acc[v] = bt[v] * e * bf16_to_f32(sKR[(16 * i + 4 * g4 + v) * RS + 16 * ct + r16]);
          } else {
            const s16x4 yv = lds64(&sVT[(16 * ct + r16) * TS + 16 * i + 4 * g4]);
#pragma unroll
            for (int v = 0; v < 4; ++v) acc[v] = bt[v] * bf16_to_f32(static_cast<uint16_t>(yv[v]));
          }
#pragma unroll
          for (int j = 0; j < i; ++j)
            acc = mma16(lds64(&sLm[(16 * i + r16) * TS + 16 * j + 4 * g4]), Zb[col][j], acc);
          const f32x4 zero = {0.f, 0.f, 0.f, 0.f};
          Z[col][i] = mma16(lds64(&sX[(16 * i + r16) * XS + 4 * g4]), cvt4(acc), zero);
          Zb[col][i] = cvt4(Z[col][i]);
        }
      }
      // -W into the k r storage (this wavefront's own channel columns; all their reads are done)
#pragma unroll
      for (int col = 0; col < 2; ++col) {
        const int ct = 2 * wv + col;
#pragma unroll
        for (int i = 0; i < 4; ++i)
#pragma unroll
          for (int v = 0; v < 4; ++v) sW[(16 * i + 4 * g4 + v) * RS + 16 * ct + r16] = f2bf(-Z[col][i][v]);
      }
    }
    __syncthreads();

    // ---------------- phase 4: U, outputs, state update (per owned value tile) ----------------
    const auto ro = rsrc(static_cast<Tout*>(a.o) + row0 * DK + j0, (span - 1) * DK * ES + DVS * ES);
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
        f32x4 acc = Z[2 + u][i];
        const uint16_t* Wr = &sW[(16 * i + r16) * RS + 4 * g4];
#pragma unroll
        for (int cp = 0; cp < 4; ++cp)
          acc = mma32(cat(lds64(Wr + 32 * cp), lds64(Wr + 32 * cp + 16)), cat(Sb[2 * cp], Sb[2 * cp + 1]), acc);
        Ub[i] = cvt4(acc);
      }
      // O = (Q Gamma) S + P U
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        f32x4 acc = {0.f, 0.f, 0.f, 0.f};
        const uint16_t* Qr = &sQt[(16 * i + r16) * RS + 4 * g4];
#pragma unroll
        for (int cp = 0; cp < 4; ++cp)
          acc = mma32(cat(lds64(Qr + 32 * cp), lds64(Qr + 32 * cp + 16)), cat(Sb[2 * cp], Sb[2 * cp + 1]), acc);
        const uint16_t* Pr = &sP[(16 * i + r16) * TS + 4 * g4];
#pragma unroll
        for (int m = 0; m + 1 <= i; m += 2)
          acc = mma32(cat(lds64(Pr + 16 * m), lds64(Pr + 16 * m + 16)), cat(Ub[m], Ub[m + 1]), acc);
        // the unpaired last tile runs on the same 16x16x32 shape, zero-padded: an
        // accumulator produced by one MFMA shape is never fed to the other shape
        if ((i & 1) == 0) acc = mma32(cat(lds64(Pr + 16 * i), s16x4{0, 0, 0, 0}), cat(Ub[i], s16x4{0, 0, 0, 0}), acc);
#pragma unroll
        for (int v = 0; v < 4; ++v) {
          const int t = 16 * i + 4 * g4 + v;
          if (t < n) {
            const int voff = (t * H * DK + 16 * jt + r16) * ES;
            if (ES == 2)
              __builtin_amdgcn_raw_buffer_store_b16(f2bf(a.scale * acc[v]), ro, voff, 0, 0);
            else
              __builtin_amdgcn_raw_buffer_store_b32(__float_as_uint(a.scale * acc[v]), ro, voff, 0, 0);
          }
        }
      }
      // S <- Diag(Gamma_C) S + (K Gamma_C / Gamma)^T U
#pragma unroll
      for (int ct = 0; ct < 8; ++ct) {
        f32x4 acc;
#pragma unroll
        for (int v = 0; v < 4; ++v) acc[v] = S[u][ct][v] * sGC[16 * ct + 4 * g4 + v];
        const uint16_t* Kr = &sKhT[(16 * ct + r16) * TS + 4 * g4];
        acc = mma32(cat(lds64(Kr), lds64(Kr + 16)), cat(Ub[0], Ub[1]), acc);
        acc = mma32(cat(lds64(Kr + 32), lds64(Kr + 48)), cat(Ub[2], Ub[3]), acc);
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
  // H bound: one chunk's byte span must fit the 32-bit buffer offsets
  return a.in_bf16 && a.dk == 128 && a.dv == 128 && a.chunk == 64 && a.H <= 65536;
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
