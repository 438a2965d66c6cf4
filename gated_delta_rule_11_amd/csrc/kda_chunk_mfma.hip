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

// Registers carried across barriers.  Chain and gate wavefronts give the same
// slots different meanings, so the compiler allocates one register per slot
// instead of one per role:
//   chain: [0,32) state S (fp32)  [32,48) Ut  [48,64) S as bf16  [64,72) U as bf16
//   gate, raw tile of the next chunk (phases 2-3):
//          [0,16) k  [16,32) q  [32,48) z or G.x;  decay logits: [48,64) v, 64 beta;
//          chunk-local sums: [48,64) G.y  [64,80) v  80 beta  81,82 G before the tile
//   gate, A1 -> A2: [0,16) bf16(k r)  [16,32) bf16(q r)  [32,48) bf16(k sf)  48,49 tile decays
//   gate, A2 -> B : [0,16) bf16(q Gamma)  [16,32) (k Gamma_C/Gamma)^T pairs  32,33 Gamma_C
template <bool FROM_Z> struct XL {
  static constexpr int V = FROM_Z ? 48 : 64;     // value column, 16 tokens
  static constexpr int BETA = FROM_Z ? 64 : 80;
  static constexpr int GB = 81;                  // G before the tile (two channels)
  static constexpr int N = FROM_Z ? 72 : 84;     // slots (chain uses 72)
};

// Raw inputs of one wavefront's 16-token tile (gate layout: lane -> channels
// 2 lane, 2 lane + 1; value column lane), token offsets clamped to the chunk.
template <int DVS, bool FROM_Z>
__device__ __forceinline__ void load_tile(uint32_t (&X)[XL<FROM_Z>::N], const ChunkArgs& a, int b, int h, int t0, int i, int ln,
                                          int j0) {
  using namespace mf;
  static_assert(DVS <= 64, "one value column per lane");
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
#pragma unroll
  for (int tt = 0; tt < 16; ++tt) {
    const int so = min(16 * i + tt, n - 1) * rowb;
    X[tt] = bload32(rk, c0 * 2, so);
    X[16 + tt] = bload32(rq, c0 * 2, so);
  }
  if (FROM_Z) {
    const auto rz = rsrc(static_cast<const uint16_t*>(a.z) + row0 * DK, span * DK * 2);
#pragma unroll
    for (int tt = 0; tt < 16; ++tt) X[32 + tt] = bload32(rz, c0 * 2, min(16 * i + tt, n - 1) * rowb);
  } else {
    const auto rg = rsrc(a.G + row0 * DK, span * DK * 4);
#pragma unroll
    for (int tt = 0; tt < 16; ++tt) {
      const u32x2 g = __builtin_bit_cast(
          u32x2, __builtin_amdgcn_raw_buffer_load_b64(rg, c0 * 4, min(16 * i + tt, n - 1) * rowb * 2, 0));
      X[32 + tt] = g[0];
      X[48 + tt] = g[1];
    }
    const u32x2 gb = __builtin_bit_cast(
        u32x2, __builtin_amdgcn_raw_buffer_load_b64(rg, c0 * 4, min(max(16 * i - 1, 0), n - 1) * rowb * 2, 0));
    X[XL<FROM_Z>::GB] = gb[0];
    X[XL<FROM_Z>::GB + 1] = gb[1];
  }
  if (ln < DVS) {
#pragma unroll
    for (int tt = 0; tt < 16; ++tt)
      X[XL<FROM_Z>::V + tt] = __builtin_amdgcn_raw_buffer_load_b16(rv, ln * 2, min(16 * i + tt, n - 1) * rowb, 0);
  }
  if (ln < 16)
    X[XL<FROM_Z>::BETA] = __builtin_amdgcn_raw_buffer_load_b16(rb, min(16 * i + ln, n - 1) * H * 2, 0, 0);
}

// Off-diagonal tile pairs (i, j < i) of the L / P products, per gate wavefront.
__constant__ int8_t kOffPairs8[4][2][2] = {{{1, 0}, {3, 0}}, {{2, 1}, {3, 1}}, {{3, 2}, {-1, -1}}, {{2, 0}, {-1, -1}}};

// Eight wavefronts, software-pipelined over chunks.
//   chain wavefronts 0..3: own value tile w of the state slice; run phases 2-4 of chunk n.
//   gate  wavefronts 4..7: own 16-token tile w-4; prefetch, gate and build the operand
//                          tiles of chunk n+1 while the chain wavefronts update the state.
// Per chunk n (every barrier is reached by all eight wavefronts):
//   B : gate: write q Gamma, (k Gamma_C/Gamma)^T, Gamma_C of chunk n
//   2 : all : L, P tiles; chain: diagonal tiles + inverses; gate: off-diagonal tiles
//   3 : all : (I + L)[W | Ut] = Diag(beta)[K Gamma | V]; W tile w per wavefront, Ut on chain
//   A1: chain: U = Ut - W S        | gate: gate and decays of chunk n+1, tile decays -> LDS
//   A2: chain: O, state update     | gate: k r, q r, anchored keys, v^T, beta, eB of chunk n+1
template <int DVS, bool FROM_Z, typename Tout>
__global__ __launch_bounds__(512) void chunk_mfma_kernel(const ChunkArgs a, int ns, int xcd_map) {
  using namespace mf;
  using Ly = Layout<DVS>;
  constexpr int NJT = DVS / 16;  // value-column tiles in the slice (chain wavefront w owns tile w)
  constexpr int ES = sizeof(Tout);

  extern __shared__ __attribute__((aligned(16))) unsigned char smem[];
  uint16_t* sKR = reinterpret_cast<uint16_t*>(smem + Ly::KR);
  uint16_t* sW = sKR;  // -W overwrites k r column tile by column tile (one wavefront per tile)
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
  const bool chain = wv < 4;
  const int gi = wv - 4;    // gate wavefront's tile
  // Lane coordinates are re-derived through an opaque copy at every phase so
  // that the addresses built from them are computed where they are used
  // instead of being hoisted out of the chunk loop and held in registers.
  int ln, g4, r16, c0;
  auto relane = [&]() {
    int l = threadIdx.x & 63;
    asm volatile("" : "+v"(l));
    ln = l;
    g4 = l >> 4;   // MFMA lane group
    r16 = l & 15;  // MFMA lane row/column
    c0 = 2 * l;    // gate layout: channels c0, c0+1
  };
  relane();
  const int nch = (T + C - 1) / C;
  const bool owns_v = chain && wv < NJT;

  float ea0 = 0.f, ea1 = 0.f;
  const float gmin_l2e = a.g_min * kLog2e;
  if (FROM_Z && !chain) {
    ea0 = __expf(a.A[h * DK + c0]) * kLog2e;
    ea1 = __expf(a.A[h * DK + c0 + 1]) * kLog2e;
  }

  constexpr int NX = XL<FROM_Z>::N;
  uint32_t X[NX];
#pragma unroll
  for (int e = 0; e < NX; ++e) X[e] = 0u;
  // chain: state slice S[ct] = X[4ct .. 4ct+3], rows 16ct + 4 g4 + v, column 16 wv + r16 of the slice
#pragma unroll
  for (int ct = 0; ct < 8; ++ct)
#pragma unroll
    for (int v = 0; v < 4; ++v)
      if (owns_v && a.S_in)
        X[4 * ct + v] = __float_as_uint(
            a.S_in[(static_cast<int64_t>(bh) * DK + 16 * ct + 4 * g4 + v) * DK + j0 + 16 * wv + r16]);

  // gate, within-tile decay products, tile decays -> sD; q r -> sQR, v^T, beta (gate, chunk tc)
  auto gate_a1 = [&](int tc) {
    using L = XL<FROM_Z>;
    const int n = min(C, T - tc);
    const int i = gi;
    if (ln < 16) {
      const int t = 16 * i + ln;
      sBeta[t] = t < n ? bf16_to_f32(static_cast<uint16_t>(X[L::BETA])) : 0.f;
    }
    if (ln < DVS) {  // v^T, value column ln of the slice, tokens of this tile
      uint32_t w[8];
#pragma unroll
      for (int tp = 0; tp < 8; ++tp) {
        const int t = 16 * i + 2 * tp;
        const uint32_t lo = t < n ? (X[L::V + 2 * tp] & 0xffffu) : 0u;
        const uint32_t hi = t + 1 < n ? (X[L::V + 2 * tp + 1] & 0xffffu) : 0u;
        w[tp] = lo | (hi << 16);
      }
      u32x4* dv = reinterpret_cast<u32x4*>(&sVT[ln * TS + 16 * i]);
      dv[0] = u32x4{w[0], w[1], w[2], w[3]};
      dv[1] = u32x4{w[4], w[5], w[6], w[7]};
    }
    uint32_t kr[16], qr[16], ks[16];
    float D0, D1;
    if (FROM_Z) {
      float al0[16], al1[16];
#pragma unroll
      for (int tt = 0; tt < 16; ++tt) {
        const bool valid = 16 * i + tt < n;
        al0[tt] = valid ? fast_exp2(gate_log2(bflo(X[32 + tt]), ea0, gmin_l2e)) : 1.f;
        al1[tt] = valid ? fast_exp2(gate_log2(bfhi(X[32 + tt]), ea1, gmin_l2e)) : 1.f;
      }
      float p0 = 1.f, p1 = 1.f;  // prefix products r_t
#pragma unroll
      for (int tt = 0; tt < 16; ++tt) {
        const bool valid = 16 * i + tt < n;
        p0 *= al0[tt];
        p1 *= al1[tt];
        const uint32_t k = valid ? X[tt] : 0u, q = valid ? X[16 + tt] : 0u;
        kr[tt] = pack2(bflo(k) * p0, bfhi(k) * p1);
        qr[tt] = pack2(bflo(q) * p0, bfhi(q) * p1);
      }
      float s0 = 1.f, s1 = 1.f;  // exclusive suffix products sf_t
#pragma unroll
      for (int tt = 15; tt >= 0; --tt) {
        const uint32_t k = 16 * i + tt < n ? X[tt] : 0u;
        ks[tt] = pack2(bflo(k) * s0, bfhi(k) * s1);
        s0 *= al0[tt];
        s1 *= al1[tt];
      }
      D0 = s0;
      D1 = s1;
    } else {
      // chunk-local sums G (natural log, fp32) in [32,48) and [48,64); log2 within this tile
      float base0 = 0.f, base1 = 0.f;
      if (i > 0 && 16 * i < n) {
        base0 = __uint_as_float(X[L::GB]) * kLog2e;
        base1 = __uint_as_float(X[L::GB + 1]) * kLog2e;
      }
      float last0 = base0, last1 = base1;
#pragma unroll
      for (int tt = 0; tt < 16; ++tt) {
        if (16 * i + tt < n) {
          last0 = __uint_as_float(X[32 + tt]) * kLog2e;
          last1 = __uint_as_float(X[48 + tt]) * kLog2e;
        }
      }
#pragma unroll
      for (int tt = 0; tt < 16; ++tt) {
        const bool valid = 16 * i + tt < n;
        const float G0 = valid ? __uint_as_float(X[32 + tt]) * kLog2e : last0;
        const float G1 = valid ? __uint_as_float(X[48 + tt]) * kLog2e : last1;
        const float r0 = fast_exp2(G0 - base0), r1 = fast_exp2(G1 - base1);
        const uint32_t k = valid ? X[tt] : 0u, q = valid ? X[16 + tt] : 0u;
        kr[tt] = pack2(bflo(k) * r0, bfhi(k) * r1);
        qr[tt] = pack2(bflo(q) * r0, bfhi(q) * r1);
        ks[tt] = pack2(bflo(k) * fast_exp2(last0 - G0), bfhi(k) * fast_exp2(last1 - G1));
      }
      D0 = fast_exp2(last0 - base0);
      D1 = fast_exp2(last1 - base1);
    }
#pragma unroll
    for (int tt = 0; tt < 16; ++tt) {
      *reinterpret_cast<uint32_t*>(&sQR[(16 * i + tt) * RS + c0]) = qr[tt];
      X[tt] = kr[tt];
      X[16 + tt] = qr[tt];
      X[32 + tt] = ks[tt];
    }
    sD[i * DK + c0] = D0;
    sD[i * DK + c0 + 1] = D1;
    X[48] = __float_as_uint(D0);
    X[49] = __float_as_uint(D1);
  };

  // k r, anchored keys, eB (gate, chunk tc; sD complete and the k r storage free)
  auto gate_a2 = [&]() {
    const int i = gi;
    const float D0 = __uint_as_float(X[48]), D1 = __uint_as_float(X[49]);
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
    // anchored keys of tile i for every tile m >= i:
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
        *reinterpret_cast<uint32_t*>(dst + tt * RS) = pack2(bflo(X[32 + tt]) * fa0, bfhi(X[32 + tt]) * fa1);
    }
    uint32_t qt[16], kh[16];
#pragma unroll
    for (int tt = 0; tt < 16; ++tt) {
      *reinterpret_cast<uint32_t*>(&sKR[(16 * i + tt) * RS + c0]) = X[tt];
      qt[tt] = pack2(bflo(X[16 + tt]) * eB0, bfhi(X[16 + tt]) * eB1);
    }
#pragma unroll
    for (int tp = 0; tp < 8; ++tp) {
      const uint32_t a0 = X[32 + 2 * tp], a1 = X[33 + 2 * tp];
      kh[tp] = pack2(bflo(a0) * af0, bflo(a1) * af0);
      kh[8 + tp] = pack2(bfhi(a0) * af1, bfhi(a1) * af1);
    }
#pragma unroll
    for (int e = 0; e < 16; ++e) {
      X[e] = qt[e];
      X[16 + e] = kh[e];
    }
    X[32] = __float_as_uint(af0 * D0);  // Gamma_C, used by tile 0's wavefront only
    X[33] = __float_as_uint(af1 * D1);
  };

  // tiles the state chain reads until the end of a chunk (written once it is done)
  auto gate_b = [&]() {
    const int i = gi;
#pragma unroll
    for (int tt = 0; tt < 16; ++tt) *reinterpret_cast<uint32_t*>(&sQt[(16 * i + tt) * RS + c0]) = X[tt];
    u32x4* d = reinterpret_cast<u32x4*>(&sKhT[c0 * TS + 16 * i]);
    d[0] = u32x4{X[16], X[17], X[18], X[19]};
    d[1] = u32x4{X[20], X[21], X[22], X[23]};
    d = reinterpret_cast<u32x4*>(&sKhT[(c0 + 1) * TS + 16 * i]);
    d[0] = u32x4{X[24], X[25], X[26], X[27]};
    d[1] = u32x4{X[28], X[29], X[30], X[31]};
    if (i == 0) {
      sGC[c0] = __uint_as_float(X[32]);
      sGC[c0 + 1] = __uint_as_float(X[33]);
    }
  };

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

  // ---- prologue: operand tiles of chunk 0
  if (!chain && T > 0) {
    load_tile<DVS, FROM_Z>(X, a, b, h, 0, gi, ln, j0);
    gate_a1(0);
  }
  __syncthreads();
  if (!chain && T > 0) gate_a2();
  __syncthreads();

  for (int ch = 0; ch < nch; ++ch) {
    relane();
    const int t0 = ch * C;
    const int n = min(C, T - t0);
    const int64_t row0 = (static_cast<int64_t>(b) * T + t0) * H + h;
    const int64_t span = static_cast<int64_t>(n - 1) * H + 1;
    const bool more = ch + 1 < nch;

    // ---------------- B: tiles the state chain reads ----------------
    if (!chain) gate_b();
    __syncthreads();
    relane();

    // ---------------- 2: L and P tiles, diagonal inverses ----------------
    if (chain) {
      const int i = wv;
      f32x4 dL, dP;
      lp_tile(i, i, dL, dP);
      const float bt = sBeta[16 * i + r16];
      f32x4 pv;
#pragma unroll
      for (int v = 0; v < 4; ++v) {
        const int s = 4 * g4 + v;
        sLT[(i * 16 + s) * LTS + r16] = s < r16 ? bt * dL[v] : 0.f;  // L[t][s] stored at [s][t]
        pv[v] = s <= r16 ? dP[v] : 0.f;
      }
      *reinterpret_cast<s16x4*>(&sP[(16 * i + r16) * TS + 16 * i + 4 * g4]) = cvt4(pv);
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
    } else {
      // prefetch the next chunk's raw tile; it lands during phases 2-3
      if (more) load_tile<DVS, FROM_Z>(X, a, b, h, t0 + C, gi, ln, j0);
#pragma unroll
      for (int p = 0; p < 2; ++p) {
        const int pi = kOffPairs8[gi][p][0], pj = kOffPairs8[gi][p][1];
        if (pi < 0) continue;
        f32x4 oL, oP;
        lp_tile(pi, pj, oL, oP);
        const int t = 16 * pi + r16;
        const float bt = sBeta[t];
        f32x4 nl;
#pragma unroll
        for (int v = 0; v < 4; ++v) nl[v] = -bt * oL[v];
        *reinterpret_cast<s16x4*>(&sLm[t * TS + 16 * pj + 4 * g4]) = cvt4(nl);
        *reinterpret_cast<s16x4*>(&sP[t * TS + 16 * pj + 4 * g4]) = cvt4(oP);
      }
    }
    __syncthreads();
    relane();

    // ---------------- 3: (I + L) [W | Ut] = Diag(beta) [K Gamma | V] ----------------
    {
      // column 0: key-channel tile wv of W (every wavefront); column 1: value tile wv (chain)
      f32x4 Z[2][4];
      s16x4 Zb[2][4];
      const int ncol = owns_v ? 2 : 1;
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        float bt[4];
#pragma unroll
        for (int v = 0; v < 4; ++v) bt[v] = sBeta[16 * i + 4 * g4 + v];
#pragma unroll
        for (int col = 0; col < 2; ++col) {
          if (col >= ncol) continue;
          f32x4 acc;
          if (col == 0) {  // K Gamma = (k r) * eB_i, rows t = 16i + 4 g4 + v, channel 16 wv + r16
            const float e = sEB[i * DK + 16 * wv + r16];
#pragma unroll
            for (int v = 0; v < 4; ++v)
              acc[v] = bt[v] * e * bf16_to_f32(sKR[(16 * i + 4 * g4 + v) * RS + 16 * wv + r16]);
          } else {
            const s16x4 yv = lds64(&sVT[(16 * wv + r16) * TS + 16 * i + 4 * g4]);
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
      // -W over this wavefront's own k r column tile (all its reads of it are done)
#pragma unroll
      for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int v = 0; v < 4; ++v) sW[(16 * i + 4 * g4 + v) * RS + 16 * wv + r16] = f2bf(-Z[0][i][v]);
      if (owns_v) {
#pragma unroll
        for (int i = 0; i < 4; ++i)
#pragma unroll
          for (int v = 0; v < 4; ++v) X[32 + 4 * i + v] = __float_as_uint(Z[1][i][v]);
      }
    }
    __syncthreads();
    relane();

    // ---------------- A1: chain U = Ut + (-W) S  |  gate: next chunk's gate ----------------
    if (owns_v) {
      s16x4 Sb[8];
#pragma unroll
      for (int ct = 0; ct < 8; ++ct) {
        f32x4 sv;
#pragma unroll
        for (int v = 0; v < 4; ++v) sv[v] = __uint_as_float(X[4 * ct + v]);
        Sb[ct] = cvt4(sv);
      }
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        f32x4 acc;
#pragma unroll
        for (int v = 0; v < 4; ++v) acc[v] = __uint_as_float(X[32 + 4 * i + v]);
        const uint16_t* Wr = &sW[(16 * i + r16) * RS + 4 * g4];
#pragma unroll
        for (int cp = 0; cp < 4; ++cp)
          acc = mma32(cat(lds64(Wr + 32 * cp), lds64(Wr + 32 * cp + 16)), cat(Sb[2 * cp], Sb[2 * cp + 1]), acc);
        const u32x2 ub = __builtin_bit_cast(u32x2, cvt4(acc));
        X[64 + 2 * i] = ub[0];
        X[65 + 2 * i] = ub[1];
      }
#pragma unroll
      for (int ct = 0; ct < 8; ++ct) {
        const u32x2 sb = __builtin_bit_cast(u32x2, Sb[ct]);
        X[48 + 2 * ct] = sb[0];
        X[49 + 2 * ct] = sb[1];
      }
    } else if (!chain && more) {
      gate_a1(t0 + C);
    }
    __syncthreads();
    relane();

    // ---------------- A2: chain outputs and state update  |  gate: next chunk's tiles ----------------
    if (owns_v) {
      s16x4 Sb[8], Ub[4];
#pragma unroll
      for (int ct = 0; ct < 8; ++ct) Sb[ct] = __builtin_bit_cast(s16x4, u32x2{X[48 + 2 * ct], X[49 + 2 * ct]});
#pragma unroll
      for (int i = 0; i < 4; ++i) Ub[i] = __builtin_bit_cast(s16x4, u32x2{X[64 + 2 * i], X[65 + 2 * i]});
      const auto ro = rsrc(static_cast<Tout*>(a.o) + row0 * DK + j0, (span - 1) * DK * ES + DVS * ES);
      const s16x4 z4 = {0, 0, 0, 0};
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
        if ((i & 1) == 0) acc = mma32(cat(lds64(Pr + 16 * i), z4), cat(Ub[i], z4), acc);
#pragma unroll
        for (int v = 0; v < 4; ++v) {
          const int t = 16 * i + 4 * g4 + v;
          if (t < n) {
            const int voff = (t * H * DK + 16 * wv + r16) * ES;
            if (ES == 2)
              __builtin_amdgcn_raw_buffer_store_b16(f2bf(a.scale * acc[v]), ro, voff, 0, 0);
            else
              __builtin_amdgcn_raw_buffer_store_b32(__float_as_uint(a.scale * acc[v]), ro, voff, 0, 0);
          }
        }
      }
#pragma unroll
      for (int ct = 0; ct < 8; ++ct) {
        f32x4 acc;
#pragma unroll
        for (int v = 0; v < 4; ++v) acc[v] = __uint_as_float(X[4 * ct + v]) * sGC[16 * ct + 4 * g4 + v];
        const uint16_t* Kr = &sKhT[(16 * ct + r16) * TS + 4 * g4];
        acc = mma32(cat(lds64(Kr), lds64(Kr + 16)), cat(Ub[0], Ub[1]), acc);
        acc = mma32(cat(lds64(Kr + 32), lds64(Kr + 48)), cat(Ub[2], Ub[3]), acc);
#pragma unroll
        for (int v = 0; v < 4; ++v) X[4 * ct + v] = __float_as_uint(acc[v]);
      }
    } else if (!chain && more) {
      gate_a2();
    }
    __syncthreads();
    relane();
  }

  relane();
  if (a.S_out && owns_v) {
#pragma unroll
    for (int ct = 0; ct < 8; ++ct)
#pragma unroll
      for (int v = 0; v < 4; ++v)
        a.S_out[(static_cast<int64_t>(bh) * DK + 16 * ct + 4 * g4 + v) * DK + j0 + 16 * wv + r16] =
            __uint_as_float(X[4 * ct + v]);
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
  hipLaunchKernelGGL(kern, dim3(static_cast<uint32_t>(nblocks)), dim3(512), bytes, st, a, ns, xcd_map);
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
