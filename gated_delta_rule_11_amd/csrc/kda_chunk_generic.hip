// kda_chunk_generic.hip -- chunked KDA prefill for every supported shape outside
// the bf16 matrix-core kernel's (fp32 inputs, dk or dv below 128, chunk 16).
// fp32 arithmetic throughout; every product runs on fp32 matrix cores
// (v_mfma_f32_16x16x4_f32).
//
// The chunkwise regrouping of Eq. 1 ("Kimi K3: the paper and proofs side by
// side", section 2.1.1; the chunkwise form of "Kimi K3: architecture,
// derivations and a pinned-source audit", section 4.5) on tiles of 16 tokens
// (the tile of "Kimi K3 reading notes", section 2), the state carried between
// tiles.  A tile never straddles an API chunk (16 divides 16 and 64), so G's
// chunk-local sums give every decay ratio inside it.  Inside a tile with entry
// state S, per key channel c, Gl_t is the log2-decay summed from the tile start
// through token t, and a = Gl_7 anchors the tile:
//   L[t,s] = beta_t sum_c (k_tc 2^(Gl_tc - a_c)) (k_sc 2^(a_c - Gl_sc))    s < t
//   P[t,s] =        sum_c (q_tc 2^(Gl_tc - a_c)) (k_sc 2^(a_c - Gl_sc))    s <= t
//   X = (I + L)^-1,  Tm = X Diag(beta)
//   U = Tm (V - (K * 2^Gl) S)                 (= Tm V - W S with W = Tm (K * 2^Gl))
//   o = scale ((Q * 2^Gl) S + P U)
//   S <- Diag(2^Gl_15) S + (K * 2^(Gl_15 - Gl))^T U
// With g >= g_min >= -5 every exponent lies within 58 of zero (the anchor is
// mid-tile), so no factor over- or underflows; a caller's own G obeys the tile
// bound the header states.  Tokens past the end of the sequence enter as
// k = q = v = beta = g = 0, which leaves S and the valid rows unchanged.
//
// Fused prologue (a.prologue): q and k arrive un-normalised, beta as a logit.
// The products above are formed from the raw rows and the norms applied to
// their rows and columns afterwards (L -> Diag(rk) L Diag(rk), P -> Diag(rq) P
// Diag(rk), and the rows of (K * 2^Gl) S, (Q * 2^Gl) S and U), with
// r = 1 / sqrt(|x|^2 + 1e-6).
//
// One workgroup of nine wavefronts per (b, h, slice of DVS value columns), a
// pipeline of three stages one tile apart with one barrier per step (step n:
// stage 1 on tile n, stage 2 on tile n - 1, stage 3 on tile n - 2):
//   1  key wavefronts 0-3; wavefront w takes key-channel tiles w, w + 4: gate
//      and decay sums, the anchored factors, its part of L and P (matrix cores,
//      each lane holding one token's four channels of a tile), q 2^Gl,
//      -k 2^Gl, k 2^(Gl_15 - Gl) and the tile's values into LDS;
//   2  one wavefront (an idle state slot's, else the ninth): L and P summed over
//      the parts and masked, X = (I + L)^-1 (by repeated squaring on fp32 matrix
//      cores where the solve has its SIMD to itself, else row by row by back
//      substitution on the vector unit), Tm and P into LDS;
//   3  state wavefronts 4 .. 4 + DVS/16 - 1, each owning 16 value columns and
//      that dk x 16 block of the state in its accumulators: (K 2^Gl) S and
//      (Q 2^Gl) S, U, o and the state update.
// LDS holds three copies of the per-tile data, by tile index mod 3.  Only the
// key wavefronts load from memory (one tile ahead), so the state wavefronts
// never wait behind their own output stores.  The four SIMDs of a compute unit
// are the limit: a key wavefront's vector work and a state wavefront's matrix
// instructions on one SIMD do not overlap much, so work is kept off the busiest
// SIMDs rather than duplicated.
#include <type_traits>

#include "kda_common.hpp"
#include "kda_launch.hpp"

namespace kda {

namespace {

constexpr int NT = 576;        // four key-role, four state-role wavefronts and one more
constexpr int KH_STRIDE = 20;  // floats per transposed row: 16 tokens + 4 (16-byte rows, no bank conflicts)

template <int DK, int DVS>
struct TileLds {
  static constexpr int NCT = DK / 16;              // key-channel tiles
  static constexpr int NP = NCT < 4 ? NCT : 4;     // wavefronts holding key tiles
  float lp[NP][2][16][16];                         // partial L and P (rows t, columns s)
  f32x4 qg[NCT][64];                               // q 2^Gl, lane (t, group) order
  f32x4 kg[NCT][64];                               // -k 2^Gl, same order
  f32x4 tm[64];                                    // Tm, row t, columns 4 group .. 4 group + 3
  f32x4 pm[64];                                    // P (masked), same order
  float kh[DK][KH_STRIDE];                         // k 2^(Gl_15 - Gl), channel rows, token columns
  float vt[DVS][KH_STRIDE];                        // values of the slice, column rows, token columns
  float el[DK];                                    // 2^Gl_15 per channel
  float beta[16];
  float rk[16], rq[16];                            // prologue: 1 / |k|, 1 / |q| per token
  float nrm[NP][2][16];                            // prologue: partial |k|^2 and |q|^2 per token
};

typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

// Four consecutive elements of a row, kept raw while the load is in flight.
template <typename T> struct Row4;
template <> struct Row4<float> {
  typedef f32x4 raw;
  __device__ __forceinline__ static raw load(const float* p) { return *reinterpret_cast<const f32x4*>(p); }
  __device__ __forceinline__ static f32x4 cvt(raw r) { return r; }
};
template <> struct Row4<bf16_t> {
  typedef u32x2 raw;
  __device__ __forceinline__ static raw load(const bf16_t* p) { return *reinterpret_cast<const u32x2*>(p); }
  __device__ __forceinline__ static f32x4 cvt(raw r) {
    return f32x4{__uint_as_float(r.x << 16), __uint_as_float(r.x & 0xffff0000u), __uint_as_float(r.y << 16),
                 __uint_as_float(r.y & 0xffff0000u)};
  }
};
template <typename T> struct One;
template <> struct One<float> {
  typedef float raw;
  __device__ __forceinline__ static raw load(const float* p) { return *p; }
  __device__ __forceinline__ static float cvt(raw r) { return r; }
};
template <> struct One<bf16_t> {
  typedef uint16_t raw;
  __device__ __forceinline__ static raw load(const bf16_t* p) { return p->bits; }
  __device__ __forceinline__ static float cvt(raw r) { return bf16_to_f32(r); }
};

__device__ __forceinline__ f32x4 mfma4(float a, float b, f32x4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x4f32(a, b, c, 0, 0, 0);
}
typedef short s16x4 __attribute__((ext_vector_type(4)));
typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
// four floats -> four bf16, round to nearest even (two v_cvt_pk_bf16_f32)
__device__ __forceinline__ s16x4 bf4(f32x4 x) {
  const u32x2 r = {__builtin_bit_cast(uint32_t, __builtin_convertvector(f32x2{x[0], x[1]}, bf16x2)),
                   __builtin_bit_cast(uint32_t, __builtin_convertvector(f32x2{x[2], x[3]}, bf16x2))};
  return __builtin_bit_cast(s16x4, r);
}
// One 16 x 16 x 16 product whose lane (row or column l % 16, group g = l / 16) holds
// k = 4 g .. 4 g + 3 of both operands, the layout of every product here: four fp32
// 16x16x4 products (k = 4 g + r in step r), or, for bf16 inputs (BF), one bf16
// 16x16x16 product of the operands rounded to bf16 (fp32 accumulation).
template <bool BF>
__device__ __forceinline__ f32x4 mm16(f32x4 a, f32x4 b, f32x4 c) {
  if constexpr (BF) {
    return __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(bf4(a), bf4(b), c, 0, 0, 0);
  } else {
#pragma unroll
    for (int r = 0; r < 4; ++r) c = mfma4(a[r], b[r], c);
    return c;
  }
}
template <bool BF>
__device__ __forceinline__ f32x4 mm16b(f32x4 a, s16x4 b_bf, f32x4 b, f32x4 c) {  // b already rounded (BF)
  if constexpr (BF) {
    return __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(bf4(a), b_bf, c, 0, 0, 0);
  } else {
    return mm16<false>(a, b, c);
  }
}
// inclusive prefix sum over the 16 lanes of a DPP row (lanes 16 r .. 16 r + 15)
__device__ __forceinline__ float row_prefix16(float x) {
  x += __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), 0x111, 0xf, 0xf, true));  // row_shr:1
  x += __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), 0x112, 0xf, 0xf, true));  // row_shr:2
  x += __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), 0x114, 0xf, 0xf, true));  // row_shr:4
  x += __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(x), 0x118, 0xf, 0xf, true));  // row_shr:8
  return x;
}
// lanes 7 and 15 of each 16-lane row, to the whole row (ds_swizzle bit mode within
// 32-lane halves: lane' = (lane & 0x10) | 7 and (lane & 0x10) | 15)
__device__ __forceinline__ float row_lane7(float x) {
  return __int_as_float(__builtin_amdgcn_ds_swizzle(__float_as_int(x), 0x10 | (7 << 5)));
}
__device__ __forceinline__ float row_lane15(float x) {
  return __int_as_float(__builtin_amdgcn_ds_swizzle(__float_as_int(x), 0x10 | (15 << 5)));
}
// Orders a prefetch after the last use of the registers it refills: the value
// is an operand (so it is computed before this point) and memory is clobbered
// (so no load moves above it).  Without it the compiler issues the next tile's
// loads first, into other registers, and copies them back at the end of the
// step, which waits for the loads there.
__device__ __forceinline__ void settle(f32x4& x) { asm volatile("" : "+v"(x)::"memory"); }
__device__ __forceinline__ void settle(float& x) { asm volatile("" : "+v"(x)::"memory"); }
__device__ __forceinline__ float sel4(int g, float a0, float a1, float a2, float a3) {
  return g == 0 ? a0 : (g == 1 ? a1 : (g == 2 ? a2 : a3));
}

}  // namespace

template <int DK, int DVS, typename Tin, bool FROM_Z>
__global__ __launch_bounds__(NT) void chunk_tile_kernel(const ChunkArgs a) {
  using Lds = TileLds<DK, DVS>;
  constexpr bool BF = std::is_same<Tin, bf16_t>::value;  // bf16 products for bf16 inputs
  constexpr int NCT = Lds::NCT, NP = Lds::NP;
  constexpr int CPW = (NCT + 3) / 4;  // key tiles per key wavefront
  constexpr int VPL = DVS / 16;       // values per key-role lane per tile
  extern __shared__ __attribute__((aligned(16))) unsigned char smem[];
  Lds* lds = reinterpret_cast<Lds*>(smem);                         // three copies, by tile index mod 3
  float* lsol = reinterpret_cast<float*>(smem + 3 * sizeof(Lds));  // [16][16]: stage 2's L

  // workgroup -> ((b*H + h) * nseg + segment, slice)
  const int nsl = a.dv / DVS;
  const int sl = blockIdx.x % nsl;
  const int bhs = blockIdx.x / nsl;
  const int bh = bhs / a.nseg, sg = bhs % a.nseg;
  const int h = bh % a.H;
  const int b = bh / a.H;
  const int w = threadIdx.x >> 6;
  const int l = threadIdx.x & 63;
  const int li = l & 15, lg = l >> 4;
  const bool key_role = w < 4;
  const int kw = w, sw = w - 4;  // index within the role
  const bool key_wave = key_role && kw < NP;
  const bool state_wave = !key_role && sw < DVS / 16;
  // stage 2 runs on an idle state slot's SIMD when there is one (wavefront w sits on
  // SIMD w mod 4), else on a ninth wavefront
  const int solve_w = DVS < 64 ? 7 : 8;
  // The solve's SIMD is otherwise idle when it runs in state slot 7 and key wavefront 3
  // has no key tile (d_k <= 48): there X = (I + L)^-1 goes to the matrix cores (a short
  // dependent chain of products); elsewhere the SIMD's matrix pipe is busy with a key or
  // state wavefront's products and the back substitution on the vector unit is faster.
  constexpr bool kMfmaSolve = DVS < 64 && NCT <= 3;
  const bool norm = a.prologue;
  // this workgroup's tokens: segment sg (chunk-aligned, so tile-aligned), or the whole sequence
  const int64_t seg_len = a.seg_chunks > 0 ? static_cast<int64_t>(a.seg_chunks) * a.chunk : a.T;
  const int t_begin = static_cast<int>(min(static_cast<int64_t>(sg) * seg_len, static_cast<int64_t>(a.T)));
  const int t_end = static_cast<int>(min(t_begin + seg_len, static_cast<int64_t>(a.T)));
  const int ntiles = (t_end - t_begin + 15) / 16;
  const int last_t0 = t_begin + 16 * (ntiles - 1);

  const Tin* q = static_cast<const Tin*>(a.q);
  const Tin* k = static_cast<const Tin*>(a.k);
  const Tin* v = static_cast<const Tin*>(a.v);
  const Tin* beta = static_cast<const Tin*>(a.beta);
  const Tin* z = static_cast<const Tin*>(a.z);
  const int64_t HDK = static_cast<int64_t>(a.H) * DK;
  const int64_t HDV = static_cast<int64_t>(a.H) * a.dv;
  const int64_t seq0 = static_cast<int64_t>(b) * a.T;  // first token row of this sequence
  const float gmin_l2e = a.g_min * kLog2e;

  if (key_role) {
    // ---- stage 1: key wavefront kw holds key tiles kw and kw + 4 (< NCT by construction)
    float eal[CPW][4];  // exp(A) log2 e of this lane's channels
#pragma unroll
    for (int m = 0; m < CPW; ++m)
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int ct = kw + 4 * m;
        eal[m][r] = (FROM_Z && key_wave && ct < NCT) ? __expf(a.A[h * DK + 16 * ct + 4 * lg + r]) * kLog2e : 0.f;
      }
    // values: lane kw * 64 + l loads VPL consecutive columns of token (kw * 64 + l) / 16
    const int vq = 64 * kw + l;
    const int vtok = vq >> 4, vc0 = (vq & 15) * VPL;
    // Inputs are fetched one tile ahead.  Loads are unconditional (rows clamped into
    // the sequence, key tiles into range, the last tile fetched again at the end): a
    // load under a branch would make the compiler copy its result at the join and
    // wait for it there.
    struct In {
      typename Row4<Tin>::raw k[CPW], q[CPW], z[CPW];
      f32x4 g[CPW], gp[CPW];
      typename One<Tin>::raw b, v[VPL];
    };
    // values taken as zero (a transition pass) are not read: the loads then go to q,
    // in range, and their results are dropped
    const Tin* vsrc = a.v_zero ? q : v;
    const int64_t vrow_len = a.v_zero ? static_cast<int64_t>(DK) : a.dv;
    auto fetch = [&](In& R, int t0) __attribute__((always_inline)) {
      const int n = min(16, t_end - t0);
      const int64_t row = seq0 + t0 + min(li, n - 1);
#pragma unroll
      for (int m = 0; m < CPW; ++m) {
        const int ct = min(kw + 4 * m, NCT - 1);
        const int64_t e = (row * a.H + h) * DK + 16 * ct + 4 * lg;
        R.k[m] = Row4<Tin>::load(k + e);
        R.q[m] = Row4<Tin>::load(q + e);
        if (FROM_Z) {
          R.z[m] = Row4<Tin>::load(z + e);
        } else {
          // G through the token before the tile (same chunk; at t0 = 0 the tile's own
          // first row is read, and unused)
          R.g[m] = *reinterpret_cast<const f32x4*>(a.G + e);
          R.gp[m] = *reinterpret_cast<const f32x4*>(a.G + e - static_cast<int64_t>(min(li, n - 1) + (t0 > 0)) * HDK);
        }
      }
      R.b = One<Tin>::load(beta + row * a.H + h);
      const int64_t vrow = seq0 + t0 + min(vtok, n - 1);
#pragma unroll
      for (int e = 0; e < VPL; ++e)
        R.v[e] = One<Tin>::load(vsrc + (vrow * a.H + h) * vrow_len + sl * DVS + vc0 + e);
    };

    auto step = [&](In& R, int it) __attribute__((always_inline)) {
      Lds& cur = lds[it % 3];
      const int t0 = t_begin + 16 * it;
      const int n = min(16, t_end - t0);
      const bool valid = li < n;
      f32x4 kk[CPW], qq[CPW], gl[CPW];
#pragma unroll
      for (int m = 0; m < CPW; ++m) {
        kk[m] = Row4<Tin>::cvt(R.k[m]);
        qq[m] = Row4<Tin>::cvt(R.q[m]);
        if (FROM_Z) {
          const f32x4 zz = Row4<Tin>::cvt(R.z[m]);
#pragma unroll
          for (int r = 0; r < 4; ++r) {
            const float g = gate_log2(zz[r], eal[m][r], gmin_l2e);
            gl[m][r] = valid ? g : 0.f;
          }
        } else {
#pragma unroll
          for (int r = 0; r < 4; ++r) gl[m][r] = (R.g[m][r] - (t0 % a.chunk != 0 ? R.gp[m][r] : 0.f)) * kLog2e;
        }
      }
      float bval = One<Tin>::cvt(R.b);
      float vv[VPL];
#pragma unroll
      for (int e = 0; e < VPL; ++e) {
        vv[e] = (vtok < n && !a.v_zero) ? One<Tin>::cvt(R.v[e]) : 0.f;
        settle(vv[e]);
      }
#pragma unroll
      for (int m = 0; m < CPW; ++m) {
        settle(kk[m]);
        settle(qq[m]);
        settle(gl[m]);
      }
      settle(bval);
      fetch(R, min(t0 + 16, last_t0));
      if (norm) bval = sigmoid_fast(bval);

#pragma unroll
      for (int e = 0; e < VPL; ++e) cur.vt[vc0 + e][vtok] = vv[e];
      if (key_wave) {  // anchored factors, partial L and P, operand tiles into LDS
        // decay sums and the row broadcasts of the anchor and the tile total first: a
        // broadcast issued after an LDS write would wait for the write (the LDS counter
        // is in order)
        f32x4 g[CPW], anc[CPW], last[CPW];
#pragma unroll
        for (int m = 0; m < CPW; ++m)
#pragma unroll
          for (int r = 0; r < 4; ++r) g[m][r] = FROM_Z ? row_prefix16(gl[m][r]) : gl[m][r];
#pragma unroll
        for (int m = 0; m < CPW; ++m)
#pragma unroll
          for (int r = 0; r < 4; ++r) {
            anc[m][r] = row_lane7(g[m][r]);
            last[m][r] = row_lane15(g[m][r]);
          }
        f32x4 accL = {0.f, 0.f, 0.f, 0.f}, accP = {0.f, 0.f, 0.f, 0.f};
        float ssk = 0.f, ssq = 0.f;
        f32x4 qgv[CPW], kgv[CPW], khv[CPW], elv[CPW];
#pragma unroll
        for (int m = 0; m < CPW; ++m) {
          f32x4 kf, kb, qf;
#pragma unroll
          for (int r = 0; r < 4; ++r) {
            const float kv = valid ? kk[m][r] : 0.f;
            const float qv = valid ? qq[m][r] : 0.f;
            ssk += kv * kv;
            ssq += qv * qv;
            const float d = g[m][r] - anc[m][r];
            const float f = fast_exp2(d), fi = fast_exp2(-d), eg = fast_exp2(g[m][r]);
            kf[r] = kv * f;
            kb[r] = kv * fi;
            qf[r] = qv * f;
            qgv[m][r] = qv * eg;
            kgv[m][r] = -(kv * eg);
            khv[m][r] = kv * fast_exp2(last[m][r] - g[m][r]);
            elv[m][r] = fast_exp2(last[m][r]);
          }
          accL = mm16<BF>(kf, kb, accL);
          accP = mm16<BF>(qf, kb, accP);
        }
#pragma unroll
        for (int m = 0; m < CPW; ++m) {
          const int ct = kw + 4 * m;
          cur.qg[ct][l] = qgv[m];
          cur.kg[ct][l] = kgv[m];
#pragma unroll
          for (int r = 0; r < 4; ++r) cur.kh[16 * ct + 4 * lg + r][li] = khv[m][r];
        }
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          cur.lp[kw][0][4 * lg + r][li] = accL[r];
          cur.lp[kw][1][4 * lg + r][li] = accP[r];
        }
        if (li == 0)
#pragma unroll
          for (int m = 0; m < CPW; ++m) *reinterpret_cast<f32x4*>(&cur.el[16 * (kw + 4 * m) + 4 * lg]) = elv[m];
        if (norm) {
          ssk += __shfl_xor(ssk, 16);
          ssk += __shfl_xor(ssk, 32);
          ssq += __shfl_xor(ssq, 16);
          ssq += __shfl_xor(ssq, 32);
          if (lg == 0) {
            cur.nrm[kw][0][li] = ssk;
            cur.nrm[kw][1][li] = ssq;
          }
        }
      }
      if (kw == 0 && lg == 0) cur.beta[li] = valid ? bval : 0.f;
      __syncthreads();
    };

    In R;
    if (ntiles > 0) fetch(R, t_begin);
    for (int it = 0; it < ntiles; ++it) step(R, it);
    __syncthreads();
    __syncthreads();
  } else if (w == solve_w) {
    // ---- stage 2 on tile m at step m + 1: L and P summed over the key parts and
    // masked, X = (I + L)^-1, Tm = X Diag(beta); Tm, P and the prologue's
    // norms into LDS.  This wavefront shares its SIMD with others and would lose most
    // issue cycles to them (older wavefronts issue first): it runs at the highest
    // issue priority.
    __builtin_amdgcn_s_setprio(3);
    __syncthreads();
    for (int m = 0; m < ntiles; ++m) {
      Lds& cur = lds[m % 3];
      f32x4 Lr = {0.f, 0.f, 0.f, 0.f}, Pr = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int p = 0; p < NP; ++p) {
        Lr += *reinterpret_cast<const f32x4*>(&cur.lp[p][0][li][4 * lg]);
        Pr += *reinterpret_cast<const f32x4*>(&cur.lp[p][1][li][4 * lg]);
      }
      f32x4 rk4 = {1.f, 1.f, 1.f, 1.f};
      float rk1 = 1.f, rq1 = 1.f;
      if (norm) {
        f32x4 sk = {0.f, 0.f, 0.f, 0.f};
        float s1k = 0.f, s1q = 0.f;
#pragma unroll
        for (int p = 0; p < NP; ++p) {
          sk += *reinterpret_cast<const f32x4*>(&cur.nrm[p][0][4 * lg]);
          s1k += cur.nrm[p][0][li];
          s1q += cur.nrm[p][1][li];
        }
#pragma unroll
        for (int r = 0; r < 4; ++r) rk4[r] = rsqrt_fast(sk[r] + kL2Eps);
        rk1 = rsqrt_fast(s1k + kL2Eps);
        rq1 = rsqrt_fast(s1q + kL2Eps);
        if (lg == 0) {
          cur.rk[li] = rk1;
          cur.rq[li] = rq1;
        }
      }
      const float bt = cur.beta[li];
      const f32x4 bs4 = *reinterpret_cast<const f32x4*>(&cur.beta[4 * lg]);
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int s = 4 * lg + r;
        Lr[r] = s < li ? bt * rk1 * Lr[r] * rk4[r] : 0.f;
        Pr[r] = s <= li ? rq1 * Pr[r] * rk4[r] : 0.f;
      }
      f32x4 tm;  // Tm = X Diag(beta): row li, columns 4 lg + r
      if constexpr (kMfmaSolve) {
        // X^T = (I + M)(I + M^2)(I + M^4)(I + M^8) with M = -L^T (strictly upper triangular,
        // so M^16 = 0): three squarings and three products on fp32 matrix cores, whatever
        // the input dtype.  Each matrix and its transpose are kept in the products' lane
        // layout (lane (lg, li): rows 4 lg .. 4 lg + 3 of column li; a product takes its left
        // factor as that factor's transpose in that layout).  Lr is L^T in it; L itself comes
        // through LDS (the LDS operations of one wavefront complete in order).
        *reinterpret_cast<f32x4*>(lsol + 16 * li + 4 * lg) = Lr;  // lsol[t][s] = L[t][s]
        f32x4 nn, nt, id;
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          nn[r] = -Lr[r];
          nt[r] = -lsol[(4 * lg + r) * 16 + li];
          id[r] = (4 * lg + r == li) ? 1.f : 0.f;
        }
        const f32x4 zero = {0.f, 0.f, 0.f, 0.f};
        f32x4 pm = id + nn, pt = id + nt;  // I + M and its transpose
#pragma unroll
        for (int lev = 0; lev < 3; ++lev) {
          const f32x4 n2 = mm16<false>(nt, nn, zero);  // M^(2^(lev+1))
          const f32x4 pn = mm16<false>(pt, n2, pm);    // P (I + that)
          if (lev < 2) {
            const f32x4 n2t = mm16<false>(nn, nt, zero);
            pt = mm16<false>(n2, pt, pt);
            nt = n2t;
          }
          nn = n2;
          pm = pn;
        }
#pragma unroll
        for (int r = 0; r < 4; ++r) tm[r] = pm[r] * bs4[r];
      } else {
        // row li of X: x_j = [j == li] - sum_{m > j} x_m L[m][j], m from 15 down.  With
        // acc_j started at -[j == li], x_m = -acc_m for every lane (rows above li stay 0).
        // L goes through LDS (the LDS operations of one wavefront complete in order),
        // whose rows every lane reads as broadcasts, all before the substitution starts.
        *reinterpret_cast<f32x4*>(lsol + 16 * li + 4 * lg) = Lr;
        f32x4 lrow[16][4];
#pragma unroll
        for (int mm = 1; mm < 16; ++mm)
#pragma unroll
          for (int j4 = 0; j4 < mm; j4 += 4) lrow[mm][j4 / 4] = *reinterpret_cast<const f32x4*>(lsol + 16 * mm + j4);
        float acc[16];
#pragma unroll
        for (int j = 0; j < 16; ++j) acc[j] = li == j ? -1.f : 0.f;
#pragma unroll
        for (int mm = 15; mm >= 1; --mm)
#pragma unroll
          for (int j = 0; j < mm; ++j) acc[j] = fmaf(-acc[mm], lrow[mm][j / 4][j % 4], acc[j]);
#pragma unroll
        for (int r = 0; r < 4; ++r) tm[r] = -sel4(lg, acc[r], acc[4 + r], acc[8 + r], acc[12 + r]) * bs4[r];
      }
      cur.tm[l] = tm;
      cur.pm[l] = Pr;
      __syncthreads();
    }
    __syncthreads();
  } else if (state_wave) {
    // ---- stage 2 (tile it + 1) and stage 3 (tile it) at step it + 2
    const int jcol = sl * DVS + 16 * sw + li;
    const int64_t soff = static_cast<int64_t>(4 * lg) * a.dv + jcol;  // within one state
    const int64_t sin_base = static_cast<int64_t>(a.S_in_seg ? bhs : bh) * DK * a.dv;
    f32x4 S[NCT];  // rows 16 ct + 4 lg + r of value column jcol of the state
#pragma unroll
    for (int ct = 0; ct < NCT; ++ct)
#pragma unroll
      for (int r = 0; r < 4; ++r)
        S[ct][r] = a.S_identity ? (16 * ct + 4 * lg + r == jcol ? 1.f : 0.f)
                   : a.S_in     ? a.S_in[sin_base + soff + static_cast<int64_t>(16 * ct + r) * a.dv]
                                : 0.f;

    __syncthreads();
    __syncthreads();
    for (int it = 0; it < ntiles; ++it) {
      const Lds& cur = lds[it % 3];
      const int t0 = t_begin + 16 * it;
      const int n = min(16, t_end - t0);
      if (a.S_ckpt && t0 % 64 == 0) {  // backward checkpoint (one segment): the state entering this 64-token block
        float* ck = a.S_ckpt + (static_cast<int64_t>(bh) * ((a.T + 63) / 64) + t0 / 64) * DK * a.dv;
#pragma unroll
        for (int ct = 0; ct < NCT; ++ct)
#pragma unroll
          for (int r = 0; r < 4; ++r) ck[(16 * ct + 4 * lg + r) * a.dv + jcol] = S[ct][r];
      }
      // (-K 2^Gl) S and (Q 2^Gl) S: lane (t, g) supplies token t's channels 16 ct + 4 g + r;
      // two accumulators each (even and odd k steps) halve the dependent chains
      f32x4 ya[2] = {{0.f, 0.f, 0.f, 0.f}, {0.f, 0.f, 0.f, 0.f}};
      f32x4 oa[2] = {{0.f, 0.f, 0.f, 0.f}, {0.f, 0.f, 0.f, 0.f}};
#pragma unroll
      for (int ct = 0; ct < NCT; ++ct) {
        const f32x4 kgv = cur.kg[ct][l];
        const f32x4 qgv = cur.qg[ct][l];
        if constexpr (BF) {
          const s16x4 sb = bf4(S[ct]);
          ya[ct & 1] = mm16b<true>(kgv, sb, S[ct], ya[ct & 1]);
          oa[ct & 1] = mm16b<true>(qgv, sb, S[ct], oa[ct & 1]);
        } else {
#pragma unroll
          for (int r = 0; r < 4; ++r) {
            ya[r & 1] = mfma4(kgv[r], S[ct][r], ya[r & 1]);
            oa[r & 1] = mfma4(qgv[r], S[ct][r], oa[r & 1]);
          }
        }
      }
      f32x4 y = ya[0] + ya[1], oacc = oa[0] + oa[1];
      const f32x4 vin = *reinterpret_cast<const f32x4*>(&cur.vt[16 * sw + li][4 * lg]);  // rows 4 lg + r
      const f32x4 tm = cur.tm[l];
      const f32x4 pm = cur.pm[l];
      f32x4 rk4 = {1.f, 1.f, 1.f, 1.f}, rq4 = {1.f, 1.f, 1.f, 1.f};
      if (norm) {
        rk4 = *reinterpret_cast<const f32x4*>(&cur.rk[4 * lg]);
        rq4 = *reinterpret_cast<const f32x4*>(&cur.rq[4 * lg]);
      }
      y = vin + rk4 * y;
      // U = Tm Y (rows 4 lg + r)
      const f32x4 u = mm16<BF>(tm, y, f32x4{0.f, 0.f, 0.f, 0.f});
      // S <- Diag(2^Gl_15) S + (K 2^(Gl_15 - Gl))^T U
      const f32x4 uk = u * rk4;
#pragma unroll
      for (int ct = 0; ct < NCT; ++ct) {
        const f32x4 el4 = *reinterpret_cast<const f32x4*>(&cur.el[16 * ct + 4 * lg]);
        const f32x4 khv = *reinterpret_cast<const f32x4*>(&cur.kh[16 * ct + li][4 * lg]);
        S[ct] = mm16<BF>(khv, uk, S[ct] * el4);
      }
      // o = scale (Q 2^Gl S + P U)
      if (!a.o_skip) {
        oacc *= rq4;
        oacc = mm16<BF>(pm, u, oacc);
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          const int t = 4 * lg + r;
          if (t < n) {
            const int64_t oi = (seq0 + t0 + t) * HDV + static_cast<int64_t>(h) * a.dv + jcol;
            if (a.out_bf16)
              io<bf16_t>::store(static_cast<bf16_t*>(a.o), oi, a.scale * oacc[r]);
            else
              io<float>::store(static_cast<float*>(a.o), oi, a.scale * oacc[r]);
          }
        }
      }
      __syncthreads();
    }
    // final state: per (b, h); per (b, h, segment); or from the last segment only
    if (a.S_out && (a.S_out_mode != 2 || sg == a.nseg - 1)) {
      const int64_t sout_base = static_cast<int64_t>(a.S_out_mode == 1 ? bhs : bh) * DK * a.dv;
#pragma unroll
      for (int ct = 0; ct < NCT; ++ct)
#pragma unroll
        for (int r = 0; r < 4; ++r) a.S_out[sout_base + soff + static_cast<int64_t>(16 * ct + r) * a.dv] = S[ct][r];
    }
  } else {
    for (int it = 0; it < ntiles + 2; ++it) __syncthreads();
  }
}

namespace {

// Value columns per workgroup: 64 (one 16-column block per state wavefront),
// halved while the grid has fewer workgroups than compute units, down to 16.
int tile_slice_cols(const ChunkArgs& a) {
  int dvs = a.dv < 64 ? a.dv : 64;
  const int64_t units = static_cast<int64_t>(a.B) * a.H * a.nseg;  // (b, h, segment)
  while (dvs > 16 && units * (a.dv / dvs) < 256) dvs /= 2;
  return dvs;
}

template <int DK, int DVS, typename Tin, bool FROM_Z>
hipError_t launch_tile_t(const ChunkArgs& a, hipStream_t st) {
  static std::atomic<uint64_t> lds_set{0};
  auto kern = chunk_tile_kernel<DK, DVS, Tin, FROM_Z>;
  const int bytes = 3 * static_cast<int>(sizeof(TileLds<DK, DVS>)) + 256 * 4;
  const hipError_t e = set_lds_limit(reinterpret_cast<const void*>(kern), bytes, lds_set);
  if (e != hipSuccess) return e;
  const int64_t nblocks = static_cast<int64_t>(a.B) * a.H * a.nseg * (a.dv / DVS);
  if (nblocks > 0x7fffffffLL) return hipErrorInvalidConfiguration;
  hipLaunchKernelGGL(kern, dim3(static_cast<uint32_t>(nblocks)), dim3(NT), bytes, st, a);
  return hipGetLastError();
}

template <int DK, int DVS>
hipError_t launch_tile_v(const ChunkArgs& a, hipStream_t st) {
  if (a.in_bf16)
    return a.from_z ? launch_tile_t<DK, DVS, bf16_t, true>(a, st) : launch_tile_t<DK, DVS, bf16_t, false>(a, st);
  return a.from_z ? launch_tile_t<DK, DVS, float, true>(a, st) : launch_tile_t<DK, DVS, float, false>(a, st);
}

template <int DK>
hipError_t launch_tile_k(const ChunkArgs& a, hipStream_t st) {
  switch (tile_slice_cols(a)) {
    case 16: return launch_tile_v<DK, 16>(a, st);
    case 32: return launch_tile_v<DK, 32>(a, st);
    case 64: return launch_tile_v<DK, 64>(a, st);
  }
  return hipErrorInvalidValue;
}

}  // namespace

hipError_t launch_chunk_generic(const ChunkArgs& a, hipStream_t st) {
  if (static_cast<int64_t>(a.B) * a.H * a.nseg == 0) return hipSuccess;
  if (a.S_identity && a.dv != a.dk) return hipErrorInvalidValue;
  if (a.dv % 16 || a.dv < 16 || a.dv > 128) return hipErrorInvalidValue;
  switch (a.dk) {
    case 16: return launch_tile_k<16>(a, st);
    case 32: return launch_tile_k<32>(a, st);
    case 64: return launch_tile_k<64>(a, st);
    case 128: return launch_tile_k<128>(a, st);
  }
  return hipErrorInvalidValue;
}

}  // namespace kda
