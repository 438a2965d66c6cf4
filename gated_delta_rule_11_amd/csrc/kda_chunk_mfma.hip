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
#include <type_traits>

#include "kda_common.hpp"
#include "kda_launch.hpp"

namespace kda {

namespace mf {
constexpr int C = 64;          // chunk
constexpr int DK = 128;        // key / value head dim
constexpr int RS = DK + 8;     // row stride (bf16 elements) of [token][channel] tiles
constexpr int TS = C + 8;      // row stride of [channel][token] tiles
constexpr int XS = 24;         // row stride of the 16x16 diagonal inverses
constexpr int LFS = 20;        // row stride (floats) of the fp32 (L_ii)^T copies: conflict-free column writes

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
  static constexpr int DT = XM + 4 * 16 * XS * 2;       // [4][128] fp32 tile decays D_i
  static constexpr int EB = DT + 4 * DK * 4;            // [4][128] fp32 decay before tile i
  static constexpr int GC = EB + 4 * DK * 4;            // [128] fp32 chunk decay
  static constexpr int BT = GC + DK * 4;                // [64] fp32 beta
  static constexpr int LF = BT + C * 4;                 // [4][16][LFS] fp32 (L_ii)^T, one per chain wavefront
  static constexpr int BYTES = LF + 4 * 16 * LFS * 4;
  static_assert(BYTES <= 160 * 1024, "LDS budget");
};

// Raw buffer resource: base, byte range.  The hardware range check covers the
// per-lane offset only, not the scalar (token) offset, so every token offset
// used below is clamped to the chunk's last valid token by construction.
constexpr int kRsrcFlags = 0x00020000;
}  // namespace mf

typedef short s16x4 __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

__device__ __forceinline__ uint16_t f2bf(float f) { return __builtin_bit_cast(uint16_t, static_cast<__bf16>(f)); }
__device__ __forceinline__ float bflo(uint32_t u) { return __uint_as_float(u << 16); }
__device__ __forceinline__ float bfhi(uint32_t u) { return __uint_as_float(u & 0xffff0000u); }
typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
// two floats -> two bf16 (a low, b high), round to nearest even, one v_cvt_pk_bf16_f32
__device__ __forceinline__ uint32_t pack2(float a, float b) {
  return __builtin_bit_cast(uint32_t, __builtin_convertvector(f32x2{a, b}, bf16x2));
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
// One 8-byte LDS read per call, for the state chain's operand reads in A1 and A2.  They
// go through a volatile LDS pointer so that the compiler keeps each one a single
// ds_read_b64: paired into one ds_read2_b64 (two addresses 32 bytes apart, as these
// tiles are read), the same lanes take eight cycles of bank conflicts per instruction
// on gfx950, while two separate reads at these strides take none (measured with the
// LDS bank-conflict counter).  Elsewhere (the solve) the pairing stays: there the
// volatile reads' fixed order cost more than the conflicts.
typedef __attribute__((address_space(3))) const volatile u32x2 lds_u32x2;
__device__ __forceinline__ s16x4 lds64u(const uint16_t* p) {
  const u32x2 v = *(lds_u32x2*)(p);  // a plain volatile load (a bit-cast of the lvalue would drop it)
  return __builtin_bit_cast(s16x4, v);
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
// Workgroup barrier that orders LDS only.  No wavefront reads another's global
// memory writes inside the kernel, so global loads in flight (the next chunk's
// prefetch) stay in flight across it instead of being drained at every barrier.
__device__ __forceinline__ void lds_barrier() {
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup", "local");
  __builtin_amdgcn_s_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup", "local");
}
__device__ __forceinline__ __amdgpu_buffer_rsrc_t rsrc(const void* base, int64_t bytes) {
  const int nrec = bytes > 0x7fffffffLL ? 0x7fffffff : static_cast<int>(bytes);
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), static_cast<short>(0), nrec, mf::kRsrcFlags);
}
__device__ __forceinline__ uint32_t bload32(__amdgpu_buffer_rsrc_t r, int voff, int soff) {
  return __builtin_amdgcn_raw_buffer_load_b32(r, voff, soff, 0);
}

// Raw inputs of one 16-token tile, held by its gate wavefront from the load to the
// gate.  Lane layout of the gate wavefronts: lane l takes tokens 8 (l >> 5) .. +7 of
// the tile (its half) and key channels 4 (l & 31) .. +3, so a token row of one
// tensor is one 8-byte load per lane over 32 lanes (two token rows per
// instruction); value columns 2 (l & 31), +1 of the slice, 4 bytes per token.
template <bool FROM_Z> struct RawTile {
  u32x2 k[8], q[8];              // bf16 quads
  u32x2 z[FROM_Z ? 8 : 1];       // decay logits (bf16 quads)
  f32x4 g[FROM_Z ? 1 : 8];       // chunk-local G of the four channels
  f32x4 gb;                      // G before the tile (G path)
  uint32_t v[8];                 // two value columns, bf16 pair
  uint32_t beta;                 // beta of tile token l (lanes 0..15)
};

// Raw inputs of one wavefront's 16-token tile, token offsets clamped to the chunk,
// in four parts (keys; queries; gate inputs; values and beta) so that the loads
// of a tile can go out in different phases.  The token offset is part of the
// per-lane offset (the two halves of the wavefront read different tokens), which
// the buffer resource's range check covers.
template <int DVS, bool FROM_Z, int PART, bool SEG>
__device__ __forceinline__ void load_part(RawTile<FROM_Z>& R, const ChunkArgs& a, int b, int h, int t0, int i,
                                          int ln, int j0) {
  using namespace mf;
  static_assert(DVS <= 64, "two value columns per lane of a half-wavefront");
  const int T = a.T, H = a.H;
  const int n = min(C, T - t0);
  const int64_t row0 = (static_cast<int64_t>(b) * T + t0) * H + h;
  const int64_t span = static_cast<int64_t>(n - 1) * H + 1;
  const int rowb = H * DK * 2;
  const int tb = 16 * i + 8 * (ln >> 5);  // first token of this lane's half of the tile
  const int cq = ln & 31;
  if constexpr (PART == 0 || PART == 1) {
    const auto r = rsrc(static_cast<const uint16_t*>(PART == 0 ? a.k : a.q) + row0 * DK, span * DK * 2);
#pragma unroll
    for (int tt = 0; tt < 8; ++tt) {
      const u32x2 x = __builtin_bit_cast(
          u32x2, __builtin_amdgcn_raw_buffer_load_b64(r, min(tb + tt, n - 1) * rowb + 8 * cq, 0, 0));
      if constexpr (PART == 0)
        R.k[tt] = x;
      else
        R.q[tt] = x;
    }
  } else if constexpr (PART == 2) {
    if constexpr (FROM_Z) {
      const auto rz = rsrc(static_cast<const uint16_t*>(a.z) + row0 * DK, span * DK * 2);
#pragma unroll
      for (int tt = 0; tt < 8; ++tt)
        R.z[tt] = __builtin_bit_cast(
            u32x2, __builtin_amdgcn_raw_buffer_load_b64(rz, min(tb + tt, n - 1) * rowb + 8 * cq, 0, 0));
    } else {
      const auto rg = rsrc(a.G + row0 * DK, span * DK * 4);
#pragma unroll
      for (int tt = 0; tt < 8; ++tt)
        R.g[tt] = __builtin_bit_cast(
            f32x4, __builtin_amdgcn_raw_buffer_load_b128(rg, min(tb + tt, n - 1) * rowb * 2 + 16 * cq, 0, 0));
      R.gb = __builtin_bit_cast(
          f32x4, __builtin_amdgcn_raw_buffer_load_b128(rg, min(max(16 * i - 1, 0), n - 1) * rowb * 2 + 16 * cq, 0, 0));
    }
  } else {
    const auto rv = rsrc(static_cast<const uint16_t*>(a.v) + row0 * DK + j0, span * DK * 2);
    const auto rb = rsrc(static_cast<const uint16_t*>(a.beta) + row0, span * 2);
    if (cq < DVS / 2) {
#pragma unroll
      for (int tt = 0; tt < 8; ++tt)
        R.v[tt] = (SEG && a.v_zero) ? 0u
                                    : __builtin_amdgcn_raw_buffer_load_b32(rv, min(tb + tt, n - 1) * rowb + 4 * cq, 0, 0);
    }
    if (ln < 16) R.beta = __builtin_amdgcn_raw_buffer_load_b16(rb, min(16 * i + ln, n - 1) * H * 2, 0, 0);
  }
}

template <int DVS, bool FROM_Z, bool SEG, bool STO>
__device__ __forceinline__ void load_tile(RawTile<FROM_Z>& R, const ChunkArgs& a, int b, int h, int t0, int i,
                                          int ln, int j0) {
  load_part<DVS, FROM_Z, 0, SEG>(R, a, b, h, t0, i, ln, j0);
  if constexpr (!STO) load_part<DVS, FROM_Z, 1, SEG>(R, a, b, h, t0, i, ln, j0);
  load_part<DVS, FROM_Z, 2, SEG>(R, a, b, h, t0, i, ln, j0);
  load_part<DVS, FROM_Z, 3, SEG>(R, a, b, h, t0, i, ln, j0);
}

// Per-token sums over the 32 lanes of a half-wavefront, for the fused prologue's
// norms.  v[t] is this lane's part of token t's sum (t < 8, tokens of its half);
// the result in lane l is the total of token (l >> 2) & 7 of its half.  Each step
// pairs every lane with one partner of the same half, keeps half of the tokens it
// still carries and adds the partner's part of them: lanes l and l ^ 16 (swap of
// the odd and even 16-lane rows), l and 15 - l within a row, l and 7 - l within an
// 8-lane half row; the last two steps sum the quad.  The partners' lane offsets,
// {16, 15, 7, 2, 1}, span the 32 lanes of the half once.
__device__ __forceinline__ float half_token_sums8(const float (&v)[8], int ln) {
  float w[4];  // token m + 4 (lane bit 4)
#pragma unroll
  for (int m = 0; m < 4; ++m) {
    const auto s = __builtin_amdgcn_permlane16_swap(__float_as_uint(v[m]), __float_as_uint(v[m + 4]), false, false);
    w[m] = __uint_as_float(s[0]) + __uint_as_float(s[1]);
  }
  const bool b3 = (ln & 8) != 0, b2 = (ln & 4) != 0;
  float y[2];  // token m + 2 (bit 3) + 4 (bit 4)
#pragma unroll
  for (int m = 0; m < 2; ++m) {
    const float keep = b3 ? w[m + 2] : w[m], send = b3 ? w[m] : w[m + 2];
    y[m] = keep + __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(send), 0x140, 0xf, 0xf, false));
  }
  const float keep = b2 ? y[1] : y[0], send = b2 ? y[0] : y[1];
  float z = keep + __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(send), 0x141, 0xf, 0xf, false));
  z += __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(z), 0x4E, 0xf, 0xf, false));  // quad [2,3,0,1]
  z += __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(z), 0xB1, 0xf, 0xf, false));  // quad [1,0,3,2]
  return z;
}

// The value of x in lane l ^ 32 (the other half of the wavefront).
__device__ __forceinline__ float other_half(float x, int ln) {
  const auto s = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return __uint_as_float((ln & 32) ? s[0] : s[1]);
}

// Off-diagonal tile pairs (i, j < i) of the L / P products, per gate wavefront.
__constant__ int8_t kOffPairs8[4][2][2] = {{{1, 0}, {3, 0}}, {{2, 1}, {3, 1}}, {{3, 2}, {-1, -1}}, {{2, 0}, {-1, -1}}};

// Eight wavefronts in two roles, software-pipelined over chunks.
//   chain wavefronts 0..3: own value tile w of the state slice; run phases 2-4 of chunk n.
//   gate  wavefronts 4..7: own 16-token tile w-4; prefetch, gate and build the operand
//                          tiles of chunk n+1 while the chain wavefronts update the state.
// Each role runs its own loop (no register of one role is merged with the other's),
// and both loops pass the same barriers:
//   2 : all : L, P tiles; chain: diagonal tiles + inverses; gate: (k Gamma_C/Gamma)^T and
//             Gamma_C of chunk n (read in A2), off-diagonal tiles and
//             the prefetch of chunk n+1 (in flight until A1)
//   3 : all : (I + L)[W | Ut] = Diag(beta)[K Gamma | V]; W tile w per wavefront, Ut on chain
//   A1: chain: U = Ut - W S, (q Gamma) S   | gate: gate and decays of chunk n+1, k sf
//   A2: chain: O += P U, state update      | gate: k r, q r, q Gamma, eB, anchored keys (all but
//                                          |       adjacent pairs) of chunk n+1
//
// SEG instantiations serve the passes of the segment-parallel form (one
// workgroup per segment; identity entry state, zero values, outputs skipped,
// per-segment states); the plain instantiation compiles all of that out.
// NORM instantiations fuse the prologue: the gate wavefronts take each token's
// key and query norms (lane reductions) into the factors the raw keys and queries
// are multiplied by anyway, and compute beta = sigmoid(logit).  The query is
// normalised before its decay factor is applied: a raw query scaled by the decay
// of a saturated tile (down to e^-80) could fall below the smallest normal
// number and lose its precision.
//
// STO (state only) instantiations serve the segment passes that write no outputs
// (end states, transitions, backward checkpoints): no queries are loaded and neither
// P nor (q Gamma) S is formed.
template <int DVS, bool FROM_Z, typename Tout, bool SEG, bool NORM, bool STO>
__global__ __launch_bounds__(512) void chunk_mfma_kernel(const ChunkArgs a, int ns, int xcd_map) {
  using namespace mf;
  static_assert(!NORM || FROM_Z, "the fused prologue runs with the fused gate");
  static_assert(!STO || SEG, "state-only passes are segment passes");
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
  float* sD = reinterpret_cast<float*>(smem + Ly::DT);
  float* sEB = reinterpret_cast<float*>(smem + Ly::EB);
  float* sGC = reinterpret_cast<float*>(smem + Ly::GC);
  float* sBeta = reinterpret_cast<float*>(smem + Ly::BT);
  float* sLf = reinterpret_cast<float*>(smem + Ly::LF);

  // workgroup -> ((b*H + h) * nseg + segment, slice); the slices of one head and
  // segment share an XCD (and its L2)
  int bh, sl, sg;
  {
    const int x = blockIdx.x;
    int bhs;
    if (xcd_map) {
      const int idx = x >> 3;
      sl = idx % ns;
      bhs = (idx / ns) * 8 + (x & 7);
    } else {
      sl = x % ns;
      bhs = x / ns;
    }
    bh = SEG ? bhs / a.nseg : bhs;
    sg = SEG ? bhs % a.nseg : 0;
  }
  const int h = bh % a.H;
  const int b = bh / a.H;
  const int j0 = sl * DVS;
  const int T = a.T;
  const int H = a.H;
  const int wv = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  // Lane coordinates are re-derived through an opaque copy at every phase so
  // that the addresses built from them are computed where they are used
  // instead of being hoisted out of the chunk loop and held in registers.
  int ln, g4, r16, c0;
  auto relane = [&]() __attribute__((always_inline)) {
    int l = threadIdx.x & 63;
    asm volatile("" : "+v"(l));
    ln = l;
    g4 = l >> 4;   // MFMA lane group
    r16 = l & 15;  // MFMA lane row/column
    c0 = 4 * (l & 31);  // gate layout: channels c0 .. c0+3 (tokens of half l >> 5)
  };
  relane();
  // this workgroup's chunks: segment sg of the sequence (all of it for one segment)
  const int nch_all = (T + C - 1) / C;
  const int seg_chunks = (SEG && a.seg_chunks > 0) ? a.seg_chunks : nch_all;
  const int c_begin = SEG ? min(sg * seg_chunks, nch_all) : 0;
  const int nch = SEG ? min(c_begin + seg_chunks, nch_all) : nch_all;

  // L^T / P^T tile for pair (i, j): rows s of tile j, columns t of tile i
  auto lp_tile = [&](int i, int j, f32x4& accL, f32x4& accP) __attribute__((always_inline)) {
    accL = f32x4{0.f, 0.f, 0.f, 0.f};
    accP = f32x4{0.f, 0.f, 0.f, 0.f};
    const uint16_t* Ar = sKA + (slot(i, j) * 16 + r16) * RS;
#pragma unroll
    for (int kb = 0; kb < 4; ++kb) {
      const int cb = 32 * kb + 8 * g4;
      const u32x4 A = lds128(Ar + cb);
      accL = mma32(A, lds128(&sKR[(16 * i + r16) * RS + cb]), accL);
      if constexpr (!STO) accP = mma32(A, lds128(&sQR[(16 * i + r16) * RS + cb]), accP);
    }
  };

  // (I + L)[W | Ut] = Diag(beta)[K Gamma | V] by forward substitution over the
  // four diagonal blocks: column 0 is key-channel tile wv of W (every wavefront),
  // column 1 value tile wv (chain wavefronts owning one).  -W goes over this
  // wavefront's own k r column tile (all its reads of it are done); Ut is returned.
  auto solve = [&](auto ncol_c, f32x4 (&Ut)[4]) {
    constexpr int ncol = decltype(ncol_c)::value;
    f32x4 Z[ncol][4];
    s16x4 Zb[ncol][4];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      float bt[4];
#pragma unroll
      for (int v = 0; v < 4; ++v) bt[v] = sBeta[16 * i + 4 * g4 + v];
#pragma unroll
      for (int col = 0; col < ncol; ++col) {
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
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
      for (int v = 0; v < 4; ++v) sW[(16 * i + 4 * g4 + v) * RS + 16 * wv + r16] = f2bf(-Z[0][i][v]);
    if constexpr (ncol == 2) {
#pragma unroll
      for (int i = 0; i < 4; ++i) Ut[i] = Z[1][i];
    }
  };

  if (wv < 4) {
    // =========================== chain wavefronts ===========================
    const bool owns_v = wv < NJT;
    // state slice S[ct][v]: row 16 ct + 4 g4 + v, column 16 wv + r16 of the slice
    f32x4 S[8];
#pragma unroll
    for (int ct = 0; ct < 8; ++ct)
#pragma unroll
      for (int v = 0; v < 4; ++v)
        S[ct][v] = !owns_v                ? 0.f
                   : (SEG && a.S_identity) ? ((16 * ct + 4 * g4 + v == j0 + 16 * wv + r16) ? 1.f : 0.f)
                   : a.S_in                ? a.S_in[((SEG && a.S_in_seg ? static_cast<int64_t>(bh) * a.nseg + sg
                                                                        : static_cast<int64_t>(bh)) * DK +
                                                     16 * ct + 4 * g4 + v) * DK + j0 + 16 * wv + r16]
                                           : 0.f;
    lds_barrier();  // prologue: operand tiles of chunk 0 (gate wavefronts)
    lds_barrier();

    for (int ch = c_begin; ch < nch; ++ch) {
      const int t0 = ch * C;
      const int n = min(C, T - t0);
      const int64_t row0 = (static_cast<int64_t>(b) * T + t0) * H + h;
      const int64_t span = static_cast<int64_t>(n - 1) * H + 1;

      if (SEG && a.S_ckpt && owns_v) {  // backward checkpoint: the state entering this chunk
        float* ck = a.S_ckpt + (static_cast<int64_t>(bh) * nch_all + ch) * DK * DK;
#pragma unroll
        for (int ct = 0; ct < 8; ++ct)
#pragma unroll
          for (int v = 0; v < 4; ++v) ck[(16 * ct + 4 * g4 + v) * DK + j0 + 16 * wv + r16] = S[ct][v];
      }
      relane();

      // ---- 2: diagonal L, P tiles of tile wv and the inverse of (I + L_ii)
      {
        const int i = wv;
        f32x4 dL, dP;
        lp_tile(i, i, dL, dP);
        const float bt = sBeta[16 * i + r16];
        // lane (t = r16, g4): P[t][s] and beta_t L[t][s] for s = 4 g4 + v (masked)
        f32x4 pv;
        float lv[4];
#pragma unroll
        for (int v = 0; v < 4; ++v) {
          const int s = 4 * g4 + v;
          lv[v] = s < r16 ? bt * dL[v] : 0.f;
          pv[v] = s <= r16 ? dP[v] : 0.f;
        }
        if constexpr (!STO) *reinterpret_cast<s16x4*>(&sP[(16 * i + r16) * TS + 16 * i + 4 * g4]) = cvt4(pv);
        // X_ii = (I + L_ii)^-1, one column per lane (lanes 0..15), right-looking: once x[m]
        // is final, column m of L is applied to the rows below it.  The columns of L come
        // from this wavefront's fp32 copy of (L_ii)^T in LDS, read at wave-uniform addresses
        // (broadcasts); only this wavefront touches the copy, and its LDS accesses complete
        // in order, so no barrier is needed between the writes and the reads.
        float* Lt = sLf + wv * 16 * LFS;
#pragma unroll
        for (int v = 0; v < 4; ++v) Lt[(4 * g4 + v) * LFS + r16] = lv[v];
        float x[16];
#pragma unroll
        for (int r = 0; r < 16; ++r) x[r] = (r == ln) ? 1.f : 0.f;
#pragma unroll
        for (int m = 0; m < 15; ++m) {
#pragma unroll
          for (int q4 = (m + 1) / 4; q4 < 4; ++q4) {
            const f32x4 l4 = *reinterpret_cast<const f32x4*>(Lt + m * LFS + 4 * q4);
#pragma unroll
            for (int u = 0; u < 4; ++u)
              if (4 * q4 + u > m) x[4 * q4 + u] -= l4[u] * x[m];
          }
        }
        if (ln < 16) {
#pragma unroll
          for (int r = 0; r < 16; ++r) sX[(16 * i + r) * XS + ln] = f2bf(x[r]);
        }
      }
      lds_barrier();
      relane();

      // ---- 3: W column tile wv, and Ut for the owned value tile
      f32x4 Ut[4];
      if (owns_v)
        solve(std::integral_constant<int, 2>{}, Ut);
      else
        solve(std::integral_constant<int, 1>{}, Ut);
      lds_barrier();
      relane();

      // ---- A1: U = Ut + (-W) S, O = (q Gamma) S + P U (stored)
      s16x4 Sb[8], Ub[4];
      f32x4 O[4];
      if (owns_v) {
#pragma unroll
        for (int ct = 0; ct < 8; ++ct) Sb[ct] = cvt4(S[ct]);
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          f32x4 acc = Ut[i];
          const uint16_t* Wr = &sW[(16 * i + r16) * RS + 4 * g4];
#pragma unroll
          for (int cp = 0; cp < 4; ++cp)
            acc = mma32(cat(lds64u(Wr + 32 * cp), lds64u(Wr + 32 * cp + 16)), cat(Sb[2 * cp], Sb[2 * cp + 1]), acc);
          Ub[i] = cvt4(acc);
        }
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          f32x4 acc = {0.f, 0.f, 0.f, 0.f};
          const uint16_t* Qr = &sQt[(16 * i + r16) * RS + 4 * g4];
          if constexpr (!STO) {
#pragma unroll
            for (int cp = 0; cp < 4; ++cp)
              acc = mma32(cat(lds64u(Qr + 32 * cp), lds64u(Qr + 32 * cp + 16)), cat(Sb[2 * cp], Sb[2 * cp + 1]), acc);
          }
          O[i] = acc;
        }
        // the intra-chunk part, O += P U, and the output stores: U of this value tile is
        // complete here, and P was written in phase 2 (the gate wavefronts are the longer
        // side of this phase, the state chain of A2)
        if (!STO && !(SEG && a.o_skip)) {  // outputs (passes that only need states skip them)
          const auto ro = rsrc(static_cast<Tout*>(a.o) + row0 * DK + j0, (span - 1) * DK * ES + DVS * ES);
          const s16x4 z4 = {0, 0, 0, 0};
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            f32x4 acc = O[i];
            const uint16_t* Pr = &sP[(16 * i + r16) * TS + 4 * g4];
#pragma unroll
            for (int m = 0; m + 1 <= i; m += 2)
              acc = mma32(cat(lds64u(Pr + 16 * m), lds64u(Pr + 16 * m + 16)), cat(Ub[m], Ub[m + 1]), acc);
            // the unpaired last tile runs on the same 16x16x32 shape, zero-padded: an
            // accumulator produced by one MFMA shape is never fed to the other shape
            if ((i & 1) == 0) acc = mma32(cat(lds64u(Pr + 16 * i), z4), cat(Ub[i], z4), acc);
            // rows t >= n lie past the end of the resource's range (H * DK >= DVS), so
            // the hardware drops their stores: no branch splits the MFMA sequence
#pragma unroll
            for (int v = 0; v < 4; ++v) {
              const int t = 16 * i + 4 * g4 + v;
              const int voff = (t * H * DK + 16 * wv + r16) * ES;
              const float ov = a.scale * acc[v];
              if (ES == 2)
                __builtin_amdgcn_raw_buffer_store_b16(f2bf(ov), ro, voff, 0, 0);
              else
                __builtin_amdgcn_raw_buffer_store_b32(__float_as_uint(ov), ro, voff, 0, 0);
            }
          }
        }
      }
      lds_barrier();
      relane();

      // ---- A2: S = Diag(Gamma_C) S + (K Gamma_C / Gamma)^T U
      if (owns_v) {
#pragma unroll
        for (int ct = 0; ct < 8; ++ct) {
          f32x4 acc;
#pragma unroll
          for (int v = 0; v < 4; ++v) acc[v] = S[ct][v] * sGC[16 * ct + 4 * g4 + v];
          const uint16_t* Kr = &sKhT[(16 * ct + r16) * TS + 4 * g4];
          acc = mma32(cat(lds64u(Kr), lds64u(Kr + 16)), cat(Ub[0], Ub[1]), acc);
          acc = mma32(cat(lds64u(Kr + 32), lds64u(Kr + 48)), cat(Ub[2], Ub[3]), acc);
          S[ct] = acc;
        }
      }
      lds_barrier();
    }

    relane();
    // final state: per (b, h); per (b, h, segment); or from the last segment only
    if (a.S_out && owns_v && (!SEG || a.S_out_mode != 2 || sg == a.nseg - 1)) {
      const int64_t base = (SEG && a.S_out_mode == 1) ? static_cast<int64_t>(bh) * a.nseg + sg : bh;
#pragma unroll
      for (int ct = 0; ct < 8; ++ct)
#pragma unroll
        for (int v = 0; v < 4; ++v)
          a.S_out[(base * DK + 16 * ct + 4 * g4 + v) * DK + j0 + 16 * wv + r16] = S[ct][v];
    }
  } else {
    // =========================== gate wavefronts ============================
    // The gate wavefronts are the longer side of every phase but A1: there they
    // yield instruction issue to the state-chain wavefront sharing their SIMD
    // (its U and (q Gamma) S products), elsewhere they take it.
    //
    // Lane layout: lane l holds tokens 8 gh .. 8 gh + 7 of its tile (gh = l >> 5, the
    // half) for channels c0 .. c0 + 3; products along the tile's tokens are formed
    // within each half and joined across the halves (lanes l and l ^ 32).
    __builtin_amdgcn_s_setprio(2);
    const int i = wv - 4;  // this wavefront's 16-token tile
    float ea[4] = {0.f, 0.f, 0.f, 0.f};
    const float gmin_l2e = a.g_min * kLog2e;
    if constexpr (FROM_Z) {
#pragma unroll
      for (int j = 0; j < 4; ++j) ea[j] = __expf(a.A[h * DK + c0 + j]) * kLog2e;
    }
    RawTile<FROM_Z> R;
    u32x2 ks[8];                // A1 -> A2: bf16 quads of k sf
    float rp[8][4];             // A1 -> A2: within-tile prefix products r (0 past the sequence's end)
    float nkt[8];               // A1 -> A2 (prologue): key normalisers of this lane's tokens
    float Dt[4] = {1.f, 1.f, 1.f, 1.f};  // A1 -> A2: decay over the tile
    u32x4 kh[4];                         // A2 -> 2: (k Gamma_C / Gamma)^T, 8 tokens per channel
    float gc[4] = {1.f, 1.f, 1.f, 1.f};  // A2 -> 2: Gamma_C (written by tile 0's wavefront)
    float nqt[8];                        // A1 -> A2 (prologue): query normalisers of this lane's tokens
    auto q4 = [](u32x2 x, int j) __attribute__((always_inline)) {  // channel j of a bf16 quad
      return (j & 1) ? bfhi(x[j >> 1]) : bflo(x[j >> 1]);
    };
    auto pack4 = [](float x0, float x1, float x2, float x3) __attribute__((always_inline)) {
      return u32x2{pack2(x0, x1), pack2(x2, x3)};
    };

    // gate of chunk tc: within-tile decay products, tile decays -> sD; q r -> sQR, v^T, beta
    // FULL: every token of the chunk is valid (all chunks but a ragged last one)
    auto gate_a1 = [&](int tc, auto full_c) __attribute__((always_inline)) {
      constexpr bool FULL = decltype(full_c)::value;
      const int n = FULL ? C : min(C, T - tc);
      const int gh = ln >> 5;
      const int tb = 16 * i + 8 * gh;  // chunk-local token of this lane's first
      if (ln < 16) {
        const int t = 16 * i + ln;
        const float bl = bf16_to_f32(static_cast<uint16_t>(R.beta));
        sBeta[t] = (FULL || t < n) ? (NORM ? sigmoid_fast(bl) : bl) : 0.f;
      }
      if ((ln & 31) < DVS / 2) {  // v^T: value columns 2 (l & 31), +1 of the slice, this half's tokens
        uint32_t lo[4], hi[4];
#pragma unroll
        for (int tp = 0; tp < 4; ++tp) {
          const int t = tb + 2 * tp;
          const uint32_t v0 = (FULL || t < n) ? R.v[2 * tp] : 0u;
          const uint32_t v1 = (FULL || t + 1 < n) ? R.v[2 * tp + 1] : 0u;
          lo[tp] = (v0 & 0xffffu) | (v1 << 16);
          hi[tp] = (v0 >> 16) | (v1 & 0xffff0000u);
        }
        const int col = 2 * (ln & 31);
        *reinterpret_cast<u32x4*>(&sVT[col * TS + tb]) = u32x4{lo[0], lo[1], lo[2], lo[3]};
        *reinterpret_cast<u32x4*>(&sVT[(col + 1) * TS + tb]) = u32x4{hi[0], hi[1], hi[2], hi[3]};
      }
      // prologue: 1 / sqrt(|x_t|^2 + eps) of this half's keys and queries
      float nk[8], nq[8];
#pragma unroll
      for (int tt = 0; tt < 8; ++tt) nk[tt] = nq[tt] = 1.f;
      if constexpr (NORM) {
        float pk[8], pq[8];
        // sums of squares of this lane's four channels: the quad is bit-cast whole and
        // split with vector shuffles (no bit-cast of a single vector element)
        auto sumsq = [](u32x2 x) __attribute__((always_inline)) {
          const bf16x4 b = __builtin_bit_cast(bf16x4, x);
          const bf16x2 lo = __builtin_shufflevector(b, b, 0, 1), hi = __builtin_shufflevector(b, b, 2, 3);
          return __builtin_amdgcn_fdot2_f32_bf16(hi, hi, __builtin_amdgcn_fdot2_f32_bf16(lo, lo, 0.f, false), false);
        };
#pragma unroll
        for (int tt = 0; tt < 8; ++tt) pk[tt] = sumsq(R.k[tt]);
        const float rkl = rsqrt_fast(half_token_sums8(pk, ln) + kL2Eps);
#pragma unroll
        for (int tt = 0; tt < 8; ++tt) {
          const float n0 = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(rkl), 4 * tt));
          const float n1 = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(rkl), 32 + 4 * tt));
          nk[tt] = gh ? n1 : n0;
        }
        if constexpr (!STO) {  // state-only passes load no queries
#pragma unroll
          for (int tt = 0; tt < 8; ++tt) pq[tt] = sumsq(R.q[tt]);
          const float rql = rsqrt_fast(half_token_sums8(pq, ln) + kL2Eps);
#pragma unroll
          for (int tt = 0; tt < 8; ++tt) {
            const float m0 = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(rql), 4 * tt));
            const float m1 = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(rql), 32 + 4 * tt));
            nq[tt] = gh ? m1 : m0;
          }
        }
      }
      // r (prefix products up to and including t) and sf (products after t), within
      // the tile: E / F carry the other half's product into the first / second half
      float rr[8][4], sfv[8][4];
      if constexpr (FROM_Z) {
        float al[8][4];
#pragma unroll
        for (int tt = 0; tt < 8; ++tt) {
          const bool valid = FULL || tb + tt < n;
#pragma unroll
          for (int j = 0; j < 4; ++j)
            al[tt][j] = valid ? fast_exp2(gate_log2(q4(R.z[tt], j), ea[j], gmin_l2e)) : 1.f;
        }
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          float P = 1.f;  // this half's product
#pragma unroll
          for (int tt = 0; tt < 8; ++tt) P *= al[tt][j];
          const float Po = other_half(P, ln);
          Dt[j] = gh ? Po * P : P * Po;  // first half's product times the second's, in both halves
          float p = gh ? Po : 1.f;
#pragma unroll
          for (int tt = 0; tt < 8; ++tt) {
            p *= al[tt][j];
            rr[tt][j] = p;
          }
          float sf = gh ? 1.f : Po;
#pragma unroll
          for (int tt = 7; tt >= 0; --tt) {
            sfv[tt][j] = sf;
            sf *= al[tt][j];
          }
        }
      } else {
        // chunk-local sums G (natural log, fp32); log2 within this tile: r = 2^(G - base),
        // sf = 2^(last - G), D = 2^(last - base), with base = G before the tile and last = G
        // at the tile's last valid token
        const bool any = FULL || 16 * i < n;
        const bool mine = FULL || tb < n;  // this half holds a valid token
        const int tl = FULL ? 7 : min(7, max(0, n - 1 - tb));
        float base[4], mylast[4], last[4];
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          base[j] = (i > 0 && any) ? R.gb[j] * kLog2e : 0.f;
          float g_tl = 0.f;
#pragma unroll
          for (int tt = 0; tt < 8; ++tt)
            if (tt == tl) g_tl = R.g[tt][j] * kLog2e;
          mylast[j] = mine ? g_tl : base[j];
          const float other = other_half(mylast[j], ln);
          // the second half's last valid token is the tile's, when that half has one
          const bool second_valid = FULL || 16 * i + 8 < n;
          last[j] = gh ? (second_valid ? mylast[j] : other) : (second_valid ? other : mylast[j]);
          Dt[j] = fast_exp2(last[j] - base[j]);
        }
#pragma unroll
        for (int tt = 0; tt < 8; ++tt) {
          const bool valid = FULL || tb + tt < n;
#pragma unroll
          for (int j = 0; j < 4; ++j) {
            const float G = valid ? R.g[tt][j] * kLog2e : last[j];
            rr[tt][j] = fast_exp2(G - base[j]);
            sfv[tt][j] = fast_exp2(last[j] - G);
          }
        }
      }
      // k sf now (the other tiles' wavefronts read it in A2); k r and q r are formed in
      // A2, where the gate wavefronts have more room, from the raw keys and queries and r
#pragma unroll
      for (int tt = 0; tt < 8; ++tt) {
        const bool valid = FULL || tb + tt < n;
        const u32x2 k = valid ? R.k[tt] : u32x2{0u, 0u};
        ks[tt] = pack4(q4(k, 0) * (sfv[tt][0] * nk[tt]), q4(k, 1) * (sfv[tt][1] * nk[tt]),
                       q4(k, 2) * (sfv[tt][2] * nk[tt]), q4(k, 3) * (sfv[tt][3] * nk[tt]));
#pragma unroll
        for (int j = 0; j < 4; ++j) rp[tt][j] = valid ? rr[tt][j] : 0.f;
        nkt[tt] = nk[tt];
        nqt[tt] = nq[tt];
      }
      // k sf of this tile is the anchored-key slot (i + 1, i) as it stands (no tile
      // in between); the scaled slots read it back in the next phase
      if (i < 3) {
#pragma unroll
        for (int tt = 0; tt < 8; ++tt)
          *reinterpret_cast<u32x2*>(&sKA[(slot(i + 1, i) * 16 + 8 * gh + tt) * RS + c0]) = ks[tt];
      }
      if (gh == 0) *reinterpret_cast<f32x4*>(&sD[i * DK + c0]) = f32x4{Dt[0], Dt[1], Dt[2], Dt[3]};
    };

    // k r, anchored keys, eB (sD complete and the k r storage free)
    auto gate_a2 = [&]() __attribute__((always_inline)) {
      const int gh = ln >> 5;
      f32x4 dd[4];
#pragma unroll
      for (int ii = 0; ii < 4; ++ii) dd[ii] = *reinterpret_cast<const f32x4*>(&sD[ii * DK + c0]);
      float eB[4] = {1.f, 1.f, 1.f, 1.f}, af[4] = {1.f, 1.f, 1.f, 1.f};
#pragma unroll
      for (int ii = 0; ii < 4; ++ii)
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          if (ii < i) eB[j] *= dd[ii][j];
          if (ii > i) af[j] *= dd[ii][j];
        }
      if (gh == 0) *reinterpret_cast<f32x4*>(&sEB[i * DK + c0]) = f32x4{eB[0], eB[1], eB[2], eB[3]};
      // anchored keys of the diagonal pair, (k_s sf_s) / D_i
      {
        float f[4];
#pragma unroll
        for (int j = 0; j < 4; ++j) f[j] = fast_rcp(Dt[j]);
        uint16_t* dst = sKA + (slot(i, i) * 16 + 8 * gh) * RS + c0;
#pragma unroll
        for (int tt = 0; tt < 8; ++tt)
          *reinterpret_cast<u32x2*>(dst + tt * RS) =
              pack4(q4(ks[tt], 0) * f[0], q4(ks[tt], 1) * f[1], q4(ks[tt], 2) * f[2], q4(ks[tt], 3) * f[3]);
      }
      // anchored keys two or three tiles apart, k_s e^(B_m - G_s) = (k_s sf_s) prod_{j < ii < m} D_ii,
      // one slot per wavefront of tiles 1..3: (3,1), (2,0), (3,0); k sf of tile j is read
      // back from slot (j + 1, j)
      if (i > 0) {
        const int m = i == 2 ? 2 : 3;
        const int j = i == 1 ? 1 : 0;
        float fa[4] = {1.f, 1.f, 1.f, 1.f};
#pragma unroll
        for (int ii = 0; ii < 4; ++ii)
#pragma unroll
          for (int c = 0; c < 4; ++c)
            if (ii > j && ii < m) fa[c] *= dd[ii][c];
        const uint16_t* src = sKA + (slot(j + 1, j) * 16 + 8 * gh) * RS + c0;
        uint16_t* dst = sKA + (slot(m, j) * 16 + 8 * gh) * RS + c0;
        u32x2 w[8];
#pragma unroll
        for (int tt = 0; tt < 8; ++tt) w[tt] = *reinterpret_cast<const u32x2*>(src + tt * RS);
#pragma unroll
        for (int tt = 0; tt < 8; ++tt)
          *reinterpret_cast<u32x2*>(dst + tt * RS) =
              pack4(q4(w[tt], 0) * fa[0], q4(w[tt], 1) * fa[1], q4(w[tt], 2) * fa[2], q4(w[tt], 3) * fa[3]);
      }
#pragma unroll
      for (int tt = 0; tt < 8; ++tt) {
        const int row = 16 * i + 8 * gh + tt;
        const u32x2 k = R.k[tt];
        *reinterpret_cast<u32x2*>(&sKR[row * RS + c0]) =
            pack4(q4(k, 0) * (rp[tt][0] * nkt[tt]), q4(k, 1) * (rp[tt][1] * nkt[tt]),
                  q4(k, 2) * (rp[tt][2] * nkt[tt]), q4(k, 3) * (rp[tt][3] * nkt[tt]));
        if constexpr (!STO) {
          // q r (read by the next phase 2) and q Gamma (read by the next A1); the state
          // chain's reads of the current chunk's q Gamma ended with A1
          // (prologue: the query's normaliser taken into the same factor)
          const u32x2 q = R.q[tt];
          const float nq = nqt[tt];
          *reinterpret_cast<u32x2*>(&sQR[row * RS + c0]) =
              pack4(q4(q, 0) * (rp[tt][0] * nq), q4(q, 1) * (rp[tt][1] * nq), q4(q, 2) * (rp[tt][2] * nq),
                    q4(q, 3) * (rp[tt][3] * nq));
          *reinterpret_cast<u32x2*>(&sQt[row * RS + c0]) =
              pack4(q4(q, 0) * (rp[tt][0] * nq * eB[0]), q4(q, 1) * (rp[tt][1] * nq * eB[1]),
                    q4(q, 2) * (rp[tt][2] * nq * eB[2]), q4(q, 3) * (rp[tt][3] * nq * eB[3]));
        }
      }
      // (k Gamma_C / Gamma)^T of this half's tokens: channel c0 + j, tokens 8 gh .. + 7
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        uint32_t w[4];
#pragma unroll
        for (int tp = 0; tp < 4; ++tp) w[tp] = pack2(q4(ks[2 * tp], j) * af[j], q4(ks[2 * tp + 1], j) * af[j]);
        kh[j] = u32x4{w[0], w[1], w[2], w[3]};
      }
#pragma unroll
      for (int j = 0; j < 4; ++j) gc[j] = af[j] * Dt[j];
    };

    // tiles the state chain reads in A2 (written once the previous chunk's A2 is done)
    auto gate_b = [&]() __attribute__((always_inline)) {
      const int gh = ln >> 5;
#pragma unroll
      for (int j = 0; j < 4; ++j) *reinterpret_cast<u32x4*>(&sKhT[(c0 + j) * TS + 16 * i + 8 * gh]) = kh[j];
      if (i == 0 && gh == 0) *reinterpret_cast<f32x4*>(&sGC[c0]) = f32x4{gc[0], gc[1], gc[2], gc[3]};
    };

    // ---- prologue: operand tiles of chunk 0
    if (c_begin < nch) {
      load_tile<DVS, FROM_Z, SEG, STO>(R, a, b, h, c_begin * C, i, ln, j0);
      if (T - c_begin * C >= C)
        gate_a1(c_begin * C, std::true_type{});
      else
        gate_a1(c_begin * C, std::false_type{});
    }
    lds_barrier();
    relane();
    if (c_begin < nch) gate_a2();
    lds_barrier();

    for (int ch = c_begin; ch < nch; ++ch) {
      const int t0 = ch * C;
      const bool more = ch + 1 < nch;

      relane();
      gate_b();

      // ---- 2: off-diagonal L, P tiles; keys, queries and gate inputs of the next chunk,
      // in flight until A1.  All workgroups load at once here and the loads issue only
      // as fast as memory takes them, so this phase (which waits for the state chain)
      // carries most of them; values and beta follow in phase 3.
      if (more) {
        load_part<DVS, FROM_Z, 0, SEG>(R, a, b, h, t0 + C, i, ln, j0);
        if constexpr (!STO) load_part<DVS, FROM_Z, 1, SEG>(R, a, b, h, t0 + C, i, ln, j0);
        load_part<DVS, FROM_Z, 2, SEG>(R, a, b, h, t0 + C, i, ln, j0);
      }
#pragma unroll
      for (int p = 0; p < 2; ++p) {
        const int pi = kOffPairs8[i][p][0], pj = kOffPairs8[i][p][1];
        if (pi < 0) continue;
        f32x4 oL, oP;
        lp_tile(pi, pj, oL, oP);
        const int t = 16 * pi + r16;
        const float bt = sBeta[t];
        f32x4 nl;
#pragma unroll
        for (int v = 0; v < 4; ++v) nl[v] = -bt * oL[v];
        *reinterpret_cast<s16x4*>(&sLm[t * TS + 16 * pj + 4 * g4]) = cvt4(nl);
        if constexpr (!STO) *reinterpret_cast<s16x4*>(&sP[t * TS + 16 * pj + 4 * g4]) = cvt4(oP);
      }
      lds_barrier();
      relane();

      // ---- 3: W column tile wv
      if (more) load_part<DVS, FROM_Z, 3, SEG>(R, a, b, h, t0 + C, i, ln, j0);
      {
        f32x4 unused[4];
        solve(std::integral_constant<int, 1>{}, unused);
      }
      lds_barrier();
      relane();

      // ---- A1: gate of the next chunk
      __builtin_amdgcn_s_setprio(0);
      if (more) {
        if (T - (t0 + C) >= C)
          gate_a1(t0 + C, std::true_type{});
        else
          gate_a1(t0 + C, std::false_type{});
      }
      lds_barrier();
      relane();

      // ---- A2: operand tiles of the next chunk
      __builtin_amdgcn_s_setprio(2);
      if (more) gate_a2();
      lds_barrier();
    }
  }
}

bool chunk_mfma_supports(const ChunkArgs& a) {
  // H bound: one chunk's byte span must fit the 32-bit buffer offsets
  return a.in_bf16 && a.dk == 128 && a.dv == 128 && a.chunk == 64 && a.H <= 65536;
}

template <int DVS, bool FROM_Z, typename Tout, bool SEG, bool NORM = false, bool STO = false>
static hipError_t launch_mfma_t(const ChunkArgs& a, hipStream_t st, int ns) {
  auto kern = chunk_mfma_kernel<DVS, FROM_Z, Tout, SEG, NORM, STO>;
  constexpr int bytes = mf::Layout<DVS>::BYTES;
  static std::atomic<uint64_t> lds_set{0};
  const hipError_t e = set_lds_limit(reinterpret_cast<const void*>(kern), bytes, lds_set);
  if (e != hipSuccess) return e;
  const int64_t nbh = static_cast<int64_t>(a.B) * a.H * a.nseg;  // (b, h, segment) units
  const int64_t nblocks = nbh * ns;
  const int xcd_map = (nbh % 8 == 0) ? 1 : 0;
  hipLaunchKernelGGL(kern, dim3(static_cast<uint32_t>(nblocks)), dim3(512), bytes, st, a, ns, xcd_map);
  return hipGetLastError();
}

template <int DVS>
static hipError_t launch_mfma_d(const ChunkArgs& a, hipStream_t st, int ns) {
  const bool seg = a.nseg > 1 || a.seg_chunks > 0 || a.S_in_seg || a.S_out_mode != 0 || a.S_identity ||
                   a.v_zero || a.o_skip || a.S_ckpt;
  if (a.prologue) {  // fused prologue: fused gate, one pass or segment passes
    if (!a.from_z) return hipErrorNotSupported;
    if (seg) {
      if (a.o_skip) return launch_mfma_t<DVS, true, bf16_t, true, true, true>(a, st, ns);
      return a.out_bf16 ? launch_mfma_t<DVS, true, bf16_t, true, true>(a, st, ns)
                        : launch_mfma_t<DVS, true, float, true, true>(a, st, ns);
    }
    return a.out_bf16 ? launch_mfma_t<DVS, true, bf16_t, false, true>(a, st, ns)
                      : launch_mfma_t<DVS, true, float, false, true>(a, st, ns);
  }
  if (seg) {  // segment passes, with the fused gate or a precomputed G
    if (a.from_z) {
      if (a.o_skip) return launch_mfma_t<DVS, true, bf16_t, true, false, true>(a, st, ns);  // no outputs
      return a.out_bf16 ? launch_mfma_t<DVS, true, bf16_t, true>(a, st, ns)
                        : launch_mfma_t<DVS, true, float, true>(a, st, ns);
    }
    if (a.o_skip) return launch_mfma_t<DVS, false, bf16_t, true, false, true>(a, st, ns);
    return a.out_bf16 ? launch_mfma_t<DVS, false, bf16_t, true>(a, st, ns)
                      : launch_mfma_t<DVS, false, float, true>(a, st, ns);
  }
  if (a.from_z)
    return a.out_bf16 ? launch_mfma_t<DVS, true, bf16_t, false>(a, st, ns)
                      : launch_mfma_t<DVS, true, float, false>(a, st, ns);
  return a.out_bf16 ? launch_mfma_t<DVS, false, bf16_t, false>(a, st, ns)
                    : launch_mfma_t<DVS, false, float, false>(a, st, ns);
}

hipError_t launch_chunk_mfma(const ChunkArgs& a, hipStream_t st) {
  if (!chunk_mfma_supports(a)) return hipErrorNotSupported;
  const int64_t nbh = static_cast<int64_t>(a.B) * a.H * a.nseg;  // (b, h, segment) units
  if (nbh == 0) return hipSuccess;
  // value-column slices: at most 64 columns per slice (the state slice then fits the
  // registers); narrower slices only while the grid still fits one workgroup per
  // compute unit (256), since every slice repeats the gate wavefronts' work and a
  // second round of workgroups would double the time
  int ns = 2;
  while (ns < 8 && nbh * ns * 2 <= 256) ns *= 2;
  if (nbh * ns > 0x7fffffffLL) return hipErrorInvalidConfiguration;
  switch (ns) {
    case 2: return launch_mfma_d<64>(a, st, 2);
    case 4: return launch_mfma_d<32>(a, st, 4);
    default: return launch_mfma_d<16>(a, st, 8);
  }
}

}  // namespace kda
