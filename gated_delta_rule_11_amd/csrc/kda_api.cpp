// kda_api.cpp -- the C ABI of libkda.so (declared in include/kda.h).
//
// Every entry point validates its arguments on the host first; on any error
// it returns a status and launches nothing.  Launches are asynchronous on the
// caller's stream.
#include <hip/hip_runtime.h>
#include <math.h>
#include <stdint.h>

#include <atomic>
#include <initializer_list>

#include "../../include/kda.h"
#include "kda_launch.hpp"

namespace {

constexpr int64_t kMaxElems = int64_t(1) << 62;

bool dim_ok(int d) { return d == 16 || d == 32 || d == 64 || d == 128; }
bool dtype_ok(int t) { return t == KDA_F32 || t == KDA_BF16; }
size_t esize(int t) { return t == KDA_BF16 ? 2 : 4; }

struct Range {
  const void* p;
  int64_t bytes;
};

// True when two non-empty byte ranges overlap.
bool overlap(Range a, Range b) {
  if (!a.p || !b.p || a.bytes <= 0 || b.bytes <= 0) return false;
  const uintptr_t a0 = reinterpret_cast<uintptr_t>(a.p), b0 = reinterpret_cast<uintptr_t>(b.p);
  return a0 < b0 + static_cast<uintptr_t>(b.bytes) && b0 < a0 + static_cast<uintptr_t>(a.bytes);
}

// Checks B, T, H, dk, dv and returns false when a size is out of range (negative
// B or T; H, dk or dv below 1) or any product overflows the supported index range.
// The head dims are checked here, before the products below divide by them.  T is
// kept 64 below INT_MAX so that token offsets rounded up to a whole chunk (T + 63,
// a chunk start + 64) stay within 32 bits in the kernels.
constexpr int64_t kMaxT = 0x7fffffffLL - 64;
bool sizes_ok(int64_t B, int64_t T, int64_t H, int64_t dk, int64_t dv) {
  if (B < 0 || T < 0 || H < 1 || dk < 1 || dv < 1 || T > kMaxT) return false;
  if (B * H > 0x7fffffffLL) return false;
  if (H * dk > 0x7fffffffLL || H * dv > 0x7fffffffLL) return false;
  if (B > 0 && T > 0 && B * T > kMaxElems / (H * (dk > dv ? dk : dv))) return false;
  if (B * H > kMaxElems / (dk * dv)) return false;
  return true;
}

kda_status from_hip(hipError_t e) { return e == hipSuccess ? KDA_OK : KDA_ERR_HIP; }

// g_min accepted by the gate and the chunked prefill (the pages fix -5): 16 g_min >= -80
// keeps the decay of any 16-token tile and its reciprocal normal fp32 numbers with room to
// spare, so that a unit-norm query or key component down to about 1e-3 times that decay is
// still a normal number (the matrix-core kernel anchors its decay factors at tile starts).
constexpr float kGminFloor = -5.0f;
bool gmin_ok(float g) { return isfinite(g) && g <= 0.f && g >= kGminFloor; }

bool aligned(const void* p, uintptr_t a) { return (reinterpret_cast<uintptr_t>(p) & (a - 1)) == 0; }

// Tensor bases 16-byte aligned, beta to its element size (NULL passes).
bool all_aligned(std::initializer_list<const void*> vec16, const void* beta, size_t beta_size) {
  for (const void* p : vec16)
    if (!aligned(p, 16)) return false;
  return aligned(beta, beta_size);
}

}  // namespace

extern "C" {

const char* kda_status_string(int s) {
  switch (s) {
    case KDA_OK: return "KDA_OK";
    case KDA_ERR_NULL: return "KDA_ERR_NULL: a required pointer is NULL";
    case KDA_ERR_SHAPE: return "KDA_ERR_SHAPE: a size is negative or too large";
    case KDA_ERR_DTYPE: return "KDA_ERR_DTYPE: unknown dtype";
    case KDA_ERR_WORKSPACE: return "KDA_ERR_WORKSPACE: the workspace is smaller than required";
    case KDA_ERR_UNSUPPORTED: return "KDA_ERR_UNSUPPORTED: head dim, chunk or parameter outside the supported set";
    case KDA_ERR_HIP: return "KDA_ERR_HIP: the HIP runtime reported a launch error";
    case KDA_ERR_ALIAS: return "KDA_ERR_ALIAS: an output overlaps an input";
    case KDA_ERR_ALIGN: return "KDA_ERR_ALIGN: a tensor pointer is not 16-byte aligned";
  }
  return "unknown kda_status";
}

int kda_version(void) { return 200; }

int kda_chunk_uses_mfma(kda_dtype in_dtype, int dk, int dv, int chunk) {
  kda::ChunkArgs a{};
  a.dk = dk; a.dv = dv; a.chunk = chunk; a.in_bf16 = in_dtype == KDA_BF16;
  return dtype_ok(in_dtype) && kda::chunk_mfma_supports(a) ? 1 : 0;
}

kda_status kda_gate(const void* z, kda_dtype z_dtype, const float* A, float g_min, int B, int T, int H, int dk,
                    int chunk, float* G, void* stream) {
  if (!dtype_ok(z_dtype)) return KDA_ERR_DTYPE;
  if (!sizes_ok(B, T, H, dk, dk)) return KDA_ERR_SHAPE;
  if (!dim_ok(dk) || !(chunk == 1 || chunk == 16 || chunk == 64)) return KDA_ERR_UNSUPPORTED;
  if (!gmin_ok(g_min)) return KDA_ERR_UNSUPPORTED;
  const int64_t n = int64_t(B) * T * H * dk;
  if (n == 0) return KDA_OK;
  if (!z || !A || !G) return KDA_ERR_NULL;
  if (!all_aligned({z, A, G}, nullptr, 1)) return KDA_ERR_ALIGN;
  const Range rG{G, n * 4};
  if (overlap(rG, Range{z, n * int64_t(esize(z_dtype))}) || overlap(rG, Range{A, int64_t(H) * dk * 4}))
    return KDA_ERR_ALIAS;
  kda::GateArgs a{z, A, g_min, G, B, T, H, dk, chunk, z_dtype == KDA_BF16};
  return from_hip(kda::launch_gate(a, static_cast<hipStream_t>(stream)));
}

}  // extern "C"

// ---------------------------------------------------------------------------
// Allocation-free prefill for callers that cannot allocate device memory.
//
// The scratch memory of the segment-parallel form lives in a file-scope device
// array instead of a caller workspace.  Its size bounds the automatic form's
// need: that form cuts B*H sequences into at most 256 / (2 B H) segments, so
// (b, h, segment) units never exceed 128, each needing at most three 128 x 128
// fp32 matrices (end state, transition, entry state): 128 * 3 * 64 KiB = 24 MiB.
// The loader gives every device its own copy; host code uses the address
// hipGetSymbolAddress returns on each device, never the array's name.
constexpr size_t kScratchBytes = KDA_NOALLOC_SCRATCH_BYTES;
static_assert(kScratchBytes == size_t(128) * 3 * 128 * 128 * 4, "the automatic form's largest need");
static __device__ __align__(256) unsigned char scratch[kScratchBytes];

namespace {
constexpr int kMaxDevices = 64;
std::atomic<void*> g_scratch[kMaxDevices];

// The current device's copy of `scratch` (looked up once per device), or nullptr.
void* scratch_on_current_device(hipError_t* err) {
  int dev = 0;
  *err = hipGetDevice(&dev);
  if (*err != hipSuccess) return nullptr;
  if (dev < 0 || dev >= kMaxDevices) {
    *err = hipErrorInvalidDevice;
    return nullptr;
  }
  void* p = g_scratch[dev].load(std::memory_order_acquire);
  if (p) return p;
  *err = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
  if (*err != hipSuccess || !p) {
    if (*err == hipSuccess) *err = hipErrorInvalidSymbol;
    return nullptr;
  }
  g_scratch[dev].store(p, std::memory_order_release);
  return p;
}
}  // namespace

namespace {

// Segments of a segment-parallel prefill: `seg_chunks` chunks each (more segments
// than chunks: one chunk each), `nseg` of them non-empty.  In 64 bits, since the
// requested count may be as large as INT_MAX.
struct SegLayout {
  int nseg;
  int seg_chunks;
};
SegLayout seg_layout(int64_t nch, int64_t segments) {
  if (segments < 1) segments = 1;
  const int64_t sc = (nch + segments - 1) / segments;
  if (sc <= 0) return {1, 0};
  return {int((nch + sc - 1) / sc), int(sc)};
}

// Workspace of the segment-parallel form, in floats: the end states from the zero
// state St and the transitions M of every segment but the last (whose are never
// used), then the entry states E of every segment.
int64_t seg_ws_floats(int64_t bh, int64_t nseg, int64_t dk, int64_t dv) {
  if (nseg <= 1) return 0;
  return bh * ((nseg - 1) * (dk * dv + dk * dk) + nseg * dk * dv);
}

// Launch form the chunked prefill picks from the sizes alone.  One pass runs one
// workgroup per (b, h, value-column slice) and walks the whole sequence; when B*H
// is too small to occupy the compute units even with narrow slices, the sequence is
// cut into segments ("Kimi K3 reading notes", section 7).  The segment-parallel form
// does about three passes' work (end states, transitions, then outputs), so it pays
// only once it multiplies the parallelism well beyond that: here when at least
// kMinSegs segments of at least kMinSegTokens tokens each fit, with the 64-column
// slices per (b, h, segment) of the widest launch (d_v / 64 of them, at least one)
// filling kFillUnits.  The rule depends on the sizes only, not on the input dtype
// (both kernels slice d_v = 128 into two 64-column slices at their widest).
constexpr int64_t kFillUnits = 256;   // compute units of the MI355X
constexpr int64_t kMinSegs = 4;
constexpr int64_t kMinSegTokens = 256;
int64_t auto_segments(int64_t B, int64_t T, int64_t H, int dk, int dv, int chunk) {
  (void)dk;
  const int64_t bh = B * H, nch = (T + chunk - 1) / chunk;
  if (bh <= 0 || nch <= 0) return 1;
  const int64_t per = dv >= 64 ? dv / 64 : 1;
  const int64_t min_chunks = kMinSegTokens / chunk;
  int64_t segs = kFillUnits / (per * bh);
  segs = segs < nch / min_chunks ? segs : nch / min_chunks;
  return segs >= kMinSegs ? segs : 1;
}

bool chunk_args_ok(int B, int T, int H, int dk, int dv, int chunk) {
  return sizes_ok(B, T, H, dk, dv) && dim_ok(dk) && dim_ok(dv) && (chunk == 16 || chunk == 64);
}

// `segments` > 0: exactly that many segments (kda_chunk_fwd_z_segmented); 0: the
// automatic choice, whose workspace kda_chunk_fwd_workspace_bytes sizes; < 0: an
// invalid count (KDA_ERR_SHAPE).
kda_status chunk_common(const void* q, const void* k, const void* v, const void* beta, const void* z,
                        kda_dtype in_dtype, const float* G, const float* A, float g_min, const float* S_in, void* o,
                        kda_dtype o_dtype, float* S_out, int B, int T, int H, int dk, int dv, int chunk, float scale,
                        bool from_z, int segments, void* ws, size_t ws_bytes, bool prologue, void* stream,
                        bool static_scratch = false) {
  if (!dtype_ok(in_dtype) || !dtype_ok(o_dtype)) return KDA_ERR_DTYPE;
  if (!sizes_ok(B, T, H, dk, dv)) return KDA_ERR_SHAPE;
  if (!dim_ok(dk) || !dim_ok(dv) || !(chunk == 16 || chunk == 64)) return KDA_ERR_UNSUPPORTED;
  if (!isfinite(scale)) return KDA_ERR_UNSUPPORTED;
  if (from_z && !gmin_ok(g_min)) return KDA_ERR_UNSUPPORTED;
  if (segments < 0) return KDA_ERR_SHAPE;
  const int64_t bh = int64_t(B) * H;
  const int64_t ntok = bh * T;
  const int64_t nstate = bh * dk * dv;
  const int64_t nch = (int64_t(T) + chunk - 1) / chunk;
  // the caller's workspace must hold what the chosen form needs
  const bool auto_form = segments == 0;
  const SegLayout lay = seg_layout(nch, auto_form ? auto_segments(B, T, H, dk, dv, chunk) : segments);
  const int64_t need = seg_ws_floats(bh, lay.nseg, dk, dv) * 4;
  if (bh == 0) return KDA_OK;
  if (ntok > 0) {
    if (!q || !k || !v || !beta || !o) return KDA_ERR_NULL;
    if (from_z ? (!z || !A) : !G) return KDA_ERR_NULL;
  }
  if (static_scratch) ws = nullptr;  // the library's own array, looked up after validation
  if (need > 0 && !ws && !static_scratch) return KDA_ERR_NULL;
  if (!all_aligned({q, k, v, z, G, A, o, S_in, S_out, need > 0 ? ws : nullptr}, beta, esize(in_dtype)))
    return KDA_ERR_ALIGN;
  if (ws_bytes < size_t(need)) return KDA_ERR_WORKSPACE;
  const int64_t ein = esize(in_dtype);
  const Range rq{q, ntok * dk * ein}, rk{k, ntok * dk * ein}, rv{v, ntok * dv * ein}, rb{beta, ntok * ein};
  const Range rz{from_z ? z : nullptr, ntok * dk * ein}, rG{from_z ? nullptr : G, ntok * dk * 4};
  const Range rA{from_z ? A : nullptr, int64_t(H) * dk * 4};
  const Range ro{o, ntok * dv * int64_t(esize(o_dtype))};
  const Range rSi{S_in, nstate * 4}, rSo{S_out, nstate * 4};
  const Range rw{need > 0 ? ws : nullptr, need};
  for (Range in : {rq, rk, rv, rb, rz, rG, rA, rSi})
    if (overlap(ro, in)) return KDA_ERR_ALIAS;
  for (Range in : {rq, rk, rv, rb, rz, rG, rA, ro})
    if (overlap(rSo, in)) return KDA_ERR_ALIAS;
  if (overlap(rSo, rSi) && S_out != S_in) return KDA_ERR_ALIAS;
  for (Range in : {rq, rk, rv, rb, rz, rG, rA, ro, rSi, rSo})
    if (overlap(rw, in)) return KDA_ERR_ALIAS;
  if (static_scratch && need > 0) {
    hipError_t e = hipSuccess;
    ws = scratch_on_current_device(&e);
    if (!ws) return KDA_ERR_HIP;
  }

  kda::ChunkArgs a{};
  a.q = q; a.k = k; a.v = v; a.beta = beta; a.G = from_z ? nullptr : G; a.z = from_z ? z : nullptr;
  a.A = from_z ? A : nullptr; a.g_min = g_min; a.S_in = S_in; a.o = o; a.S_out = S_out;
  a.B = B; a.T = T; a.H = H; a.dk = dk; a.dv = dv; a.chunk = chunk; a.scale = scale;
  a.in_bf16 = in_dtype == KDA_BF16; a.out_bf16 = o_dtype == KDA_BF16; a.from_z = from_z;
  a.prologue = prologue;
  hipStream_t st = static_cast<hipStream_t>(stream);
  // bf16, d = 128, chunk 64 on the bf16 matrix-core kernel; every other shape on the
  // fp32 matrix-core tile kernel
  const bool mfma = kda::chunk_mfma_supports(a);
  auto launch = [&](const kda::ChunkArgs& c) {
    return mfma ? kda::launch_chunk_mfma(c, st) : kda::launch_chunk_generic(c, st);
  };
  if (lay.nseg <= 1) return from_hip(launch(a));

  // Segment-parallel form ("Kimi K3 reading notes", section 7): the segments but the
  // last from the zero state (end states St) and from the identity with zero values
  // (transitions M), the entry states E by a scan, then every segment from its entry
  // state, writing the outputs and, from the last one, the final state.
  const int nseg = lay.nseg;
  float* St = static_cast<float*>(ws);
  float* M = St + bh * (nseg - 1) * dk * dv;
  float* E = M + bh * (nseg - 1) * dk * dk;
  a.seg_chunks = lay.seg_chunks;
  kda::ChunkArgs pa = a;  // pass A: end states from the zero state
  pa.nseg = nseg - 1; pa.S_in = nullptr; pa.S_out = St; pa.S_out_mode = 1; pa.o_skip = true;
  kda::ChunkArgs pb = pa;  // pass B: transitions (identity entry state, zero values, dk columns)
  pb.S_identity = true; pb.v_zero = true; pb.S_out = M; pb.dv = dk;
  kda::ChunkArgs pc = a;  // pass C: outputs and the final state from the true entry states
  pc.nseg = nseg; pc.S_in = E; pc.S_in_seg = true; pc.S_out_mode = 2;
  const kda::SegScanArgs sa{S_in, St, M, E, int(bh), nseg, dk, dv};
  hipError_t e = launch(pa);
  if (e == hipSuccess) e = launch(pb);
  if (e == hipSuccess) e = kda::launch_segscan(sa, st);
  if (e == hipSuccess) e = launch(pc);
  return from_hip(e);
}

}  // namespace

extern "C" {

size_t kda_chunk_fwd_workspace_bytes(int B, int T, int H, int dk, int dv, int chunk) {
  if (!chunk_args_ok(B, T, H, dk, dv, chunk)) return 0;
  const int64_t nch = (int64_t(T) + chunk - 1) / chunk;
  const SegLayout lay = seg_layout(nch, auto_segments(B, T, H, dk, dv, chunk));
  return size_t(seg_ws_floats(int64_t(B) * H, lay.nseg, dk, dv)) * 4;
}

kda_status kda_chunk_fwd(const void* q, const void* k, const void* v, const void* beta, kda_dtype in_dtype,
                         const float* G, const float* S_in, void* o, kda_dtype o_dtype, float* S_out, int B, int T,
                         int H, int dk, int dv, int chunk, float scale, void* workspace, size_t workspace_bytes,
                         void* stream) {
  return chunk_common(q, k, v, beta, nullptr, in_dtype, G, nullptr, -5.0f, S_in, o, o_dtype, S_out, B, T, H, dk, dv,
                      chunk, scale, false, 0, workspace, workspace_bytes, false, stream);
}

size_t kda_chunk_fwd_z_segmented_workspace_bytes(int B, int H, int dk, int dv, int segments) {
  if (B < 0 || H < 0 || dk < 0 || dv < 0 || segments < 1) return 0;
  return size_t(seg_ws_floats(int64_t(B) * H, segments, dk, dv)) * 4;
}

kda_status kda_chunk_fwd_z_segmented(const void* q, const void* k, const void* v, const void* beta, const void* z,
                                     kda_dtype in_dtype, const float* A, float g_min, const float* S_in, void* o,
                                     kda_dtype o_dtype, float* S_out, int B, int T, int H, int dk, int dv, int chunk,
                                     float scale, int segments, void* workspace, size_t workspace_bytes,
                                     void* stream) {
  // a count below one is a shape error (reported after the dtype checks, as every size)
  return chunk_common(q, k, v, beta, z, in_dtype, nullptr, A, g_min, S_in, o, o_dtype, S_out, B, T, H, dk, dv, chunk,
                      scale, true, segments < 1 ? -1 : segments, workspace, workspace_bytes, false, stream);
}

size_t kda_chunk_bwd_z_workspace_bytes(int B, int T, int H, int dk, int dv) {
  if (B < 0 || T < 0 || H < 0 || dk < 0 || dv < 0) return 0;
  const size_t bh = size_t(B) * size_t(H), sz = size_t(dk) * size_t(dv);
  const size_t nblk = (size_t(T) + 63) / 64;
  const size_t nsp = size_t(kda::chunk_bwd_slices(B, H, dv));
  const size_t mcache = bh * nsp * size_t(kda::kBwdMCacheFloats);  // recompute's M and AL
  return (bh * (nblk + 3) * sz + bh * nsp * size_t(dk) + mcache) * 4;
}

kda_status kda_chunk_bwd_z(const void* q, const void* k, const void* v, const void* beta, const void* z,
                           kda_dtype in_dtype, const float* A, float g_min, const float* S_in, const void* d_o,
                           kda_dtype do_dtype, const float* dS_out, float* dq, float* dk_, float* dv_, float* dbeta,
                           float* dz, float* dA, float* dS_in, int B, int T, int H, int dk, int dv, float scale,
                           void* workspace, size_t workspace_bytes, void* stream) {
  if (!dtype_ok(in_dtype) || !dtype_ok(do_dtype)) return KDA_ERR_DTYPE;
  if (!sizes_ok(B, T, H, dk, dv)) return KDA_ERR_SHAPE;
  if (!dim_ok(dk) || !dim_ok(dv)) return KDA_ERR_UNSUPPORTED;
  if (!isfinite(scale) || !isfinite(g_min) || g_min > 0.f || g_min < -5.f) return KDA_ERR_UNSUPPORTED;
  const int64_t ntok = int64_t(B) * T * H, bh = int64_t(B) * H;
  if (bh == 0) return KDA_OK;
  if (!A || !dA) return KDA_ERR_NULL;
  if (ntok > 0 && (!q || !k || !v || !beta || !z || !d_o || !dq || !dk_ || !dv_ || !dbeta || !dz))
    return KDA_ERR_NULL;
  if (!workspace) return KDA_ERR_NULL;
  if (!all_aligned({q, k, v, z, A, S_in, d_o, dS_out, dq, dk_, dv_, dz, dA, dS_in, workspace}, beta,
                   esize(in_dtype)) ||
      !aligned(dbeta, 4))
    return KDA_ERR_ALIGN;
  if (workspace_bytes < kda_chunk_bwd_z_workspace_bytes(B, T, H, dk, dv)) return KDA_ERR_WORKSPACE;
  const int64_t ein = esize(in_dtype), edo = esize(do_dtype), nstate = bh * dk * dv;
  const Range ins[] = {{q, ntok * dk * ein}, {k, ntok * dk * ein}, {v, ntok * dv * ein}, {beta, ntok * ein},
                       {z, ntok * dk * ein}, {A, int64_t(H) * dk * 4}, {S_in, nstate * 4}, {d_o, ntok * dv * edo},
                       {dS_out, nstate * 4}};
  const Range outs[] = {{dq, ntok * dk * 4}, {dk_, ntok * dk * 4}, {dv_, ntok * dv * 4}, {dbeta, ntok * 4},
                        {dz, ntok * dk * 4}, {dA, int64_t(H) * dk * 4}, {dS_in, nstate * 4},
                        {workspace, int64_t(kda_chunk_bwd_z_workspace_bytes(B, T, H, dk, dv))}};
  for (const Range& o : outs) {
    for (const Range& in : ins)
      if (overlap(o, in)) return KDA_ERR_ALIAS;
    for (const Range& o2 : outs)
      if (&o2 != &o && overlap(o, o2)) return KDA_ERR_ALIAS;
  }
  hipStream_t st = static_cast<hipStream_t>(stream);
  const int64_t nblk = (int64_t(T) + 63) / 64;
  float* ckpt = static_cast<float*>(workspace);
  float* sub_states = ckpt + bh * nblk * dk * dv;
  float* dA_part = sub_states + bh * 3 * dk * dv;
  const int nsp = kda::chunk_bwd_slices(B, H, dv);
  float* mcache = dA_part + bh * nsp * dk;
  // forward pass that only leaves the state entering every 64-token block
  kda::ChunkArgs f{};
  f.q = q; f.k = k; f.v = v; f.beta = beta; f.z = z; f.A = A; f.g_min = g_min; f.S_in = S_in;
  f.o = dq;  // never written (outputs skipped)
  f.S_out = nullptr; f.B = B; f.T = T; f.H = H; f.dk = dk; f.dv = dv; f.chunk = 64; f.scale = scale;
  f.in_bf16 = in_dtype == KDA_BF16; f.out_bf16 = false; f.from_z = true; f.o_skip = true; f.S_ckpt = ckpt;
  hipError_t e = kda::chunk_mfma_supports(f) ? kda::launch_chunk_mfma(f, st) : kda::launch_chunk_generic(f, st);
  if (e != hipSuccess) return from_hip(e);
  kda::BwdArgs bwa{q, k, v, beta, z, A, g_min, d_o, dS_out, ckpt, sub_states, dA_part, dq, dk_, dv_, dbeta, dz, dA,
                   dS_in, B, T, H, dk, dv, scale, in_dtype == KDA_BF16, do_dtype == KDA_BF16};
  bwa.mcache = mcache;
  return from_hip(kda::launch_chunk_bwd(bwa, st));
}

kda_status kda_chunk_fwd_z_prologue(const void* q, const void* k, const void* v, const void* beta_logit,
                                    const void* z, kda_dtype in_dtype, const float* A, float g_min,
                                    const float* S_in, void* o, kda_dtype o_dtype, float* S_out, int B, int T, int H,
                                    int dk, int dv, int chunk, float scale, void* workspace, size_t workspace_bytes,
                                    void* stream) {
  return chunk_common(q, k, v, beta_logit, z, in_dtype, nullptr, A, g_min, S_in, o, o_dtype, S_out, B, T, H, dk, dv,
                      chunk, scale, true, 0, workspace, workspace_bytes, true, stream);
}

kda_status kda_chunk_fwd_z(const void* q, const void* k, const void* v, const void* beta, const void* z,
                           kda_dtype in_dtype, const float* A, float g_min, const float* S_in, void* o,
                           kda_dtype o_dtype, float* S_out, int B, int T, int H, int dk, int dv, int chunk,
                           float scale, void* workspace, size_t workspace_bytes, void* stream) {
  return chunk_common(q, k, v, beta, z, in_dtype, nullptr, A, g_min, S_in, o, o_dtype, S_out, B, T, H, dk, dv, chunk,
                      scale, true, 0, workspace, workspace_bytes, false, stream);
}

static kda_status decode_common(const void* q, const void* k, const void* v, const void* z, const void* beta,
                                kda_dtype in_dtype, const float* A, float g_min, float* S, void* o,
                                kda_dtype o_dtype, int N, int H, int dk, int dv, float scale, bool prologue,
                                void* stream) {
  if (!dtype_ok(in_dtype) || !dtype_ok(o_dtype)) return KDA_ERR_DTYPE;
  if (!sizes_ok(N, 1, H, dk, dv)) return KDA_ERR_SHAPE;
  if (!dim_ok(dk) || !dim_ok(dv)) return KDA_ERR_UNSUPPORTED;
  if (!isfinite(g_min) || g_min > 0.f || !isfinite(scale)) return KDA_ERR_UNSUPPORTED;
  const int64_t nh = int64_t(N) * H;
  if (nh == 0) return KDA_OK;
  if (!q || !k || !v || !z || !beta || !A || !S || !o) return KDA_ERR_NULL;
  if (!all_aligned({q, k, v, z, A, S, o}, beta, esize(in_dtype))) return KDA_ERR_ALIGN;
  const int64_t ein = esize(in_dtype);
  const Range rS{S, nh * dk * dv * 4}, ro{o, nh * dv * int64_t(esize(o_dtype))};
  const Range ins[] = {{q, nh * dk * ein}, {k, nh * dk * ein}, {v, nh * dv * ein}, {z, nh * dk * ein},
                       {beta, nh * ein}, {A, int64_t(H) * dk * 4}};
  for (const Range& in : ins)
    if (overlap(rS, in) || overlap(ro, in)) return KDA_ERR_ALIAS;
  if (overlap(rS, ro)) return KDA_ERR_ALIAS;
  kda::DecodeArgs a{q, k, v, z, beta, A, g_min, S, o, N, H, dk, dv, scale, in_dtype == KDA_BF16,
                    o_dtype == KDA_BF16, prologue};
  return from_hip(kda::launch_decode(a, static_cast<hipStream_t>(stream)));
}

kda_status kda_decode_step(const void* q, const void* k, const void* v, const void* z, const void* beta,
                           kda_dtype in_dtype, const float* A, float g_min, float* S, void* o, kda_dtype o_dtype,
                           int N, int H, int dk, int dv, float scale, void* stream) {
  return decode_common(q, k, v, z, beta, in_dtype, A, g_min, S, o, o_dtype, N, H, dk, dv, scale, false, stream);
}

kda_status kda_decode_step_prologue(const void* q, const void* k, const void* v, const void* z, const void* beta,
                                    kda_dtype in_dtype, const float* A, float g_min, float* S, void* o,
                                    kda_dtype o_dtype, int N, int H, int dk, int dv, float scale, void* stream) {
  return decode_common(q, k, v, z, beta, in_dtype, A, g_min, S, o, o_dtype, N, H, dk, dv, scale, true, stream);
}

kda_status kda_decode_replay(const void* q, const void* k, const void* v, const void* z, const void* beta,
                             kda_dtype in_dtype, const float* A, float g_min, const float* S_snapshot,
                             const int* accepted, void* o, kda_dtype o_dtype, float* S_commit, int n_draft, int N,
                             int H, int dk, int dv, float scale, void* stream) {
  if (!dtype_ok(in_dtype) || !dtype_ok(o_dtype)) return KDA_ERR_DTYPE;
  if (!sizes_ok(N, n_draft, H, dk, dv)) return KDA_ERR_SHAPE;
  if (!dim_ok(dk) || !dim_ok(dv)) return KDA_ERR_UNSUPPORTED;
  if (!isfinite(g_min) || g_min > 0.f || !isfinite(scale)) return KDA_ERR_UNSUPPORTED;
  const int64_t nh = int64_t(N) * H;
  if (nh == 0) return KDA_OK;
  if (!A || !S_snapshot || !accepted || !S_commit) return KDA_ERR_NULL;
  if (n_draft > 0 && (!q || !k || !v || !z || !beta || !o)) return KDA_ERR_NULL;
  if (!all_aligned({A, S_snapshot, S_commit}, nullptr, 1) || reinterpret_cast<uintptr_t>(accepted) % 4)
    return KDA_ERR_ALIGN;
  if (n_draft > 0 && !all_aligned({q, k, v, z, o}, beta, esize(in_dtype))) return KDA_ERR_ALIGN;
  const int64_t ein = esize(in_dtype), nt = nh * n_draft;
  const Range rC{S_commit, nh * dk * dv * 4}, ro{o, nt * dv * int64_t(esize(o_dtype))};
  const Range ins[] = {{q, nt * dk * ein}, {k, nt * dk * ein}, {v, nt * dv * ein}, {z, nt * dk * ein},
                       {beta, nt * ein}, {A, int64_t(H) * dk * 4}, {S_snapshot, nh * dk * dv * 4},
                       {accepted, int64_t(N) * 4}};
  for (const Range& in : ins)
    if (overlap(rC, in) || overlap(ro, in)) return KDA_ERR_ALIAS;
  if (overlap(rC, ro)) return KDA_ERR_ALIAS;
  kda::ReplayArgs a{q,        k,          v,     z, beta, A, g_min, S_snapshot, o, S_commit, accepted, n_draft, N, H,
                    dk,       dv,         scale, in_dtype == KDA_BF16, o_dtype == KDA_BF16};
  return from_hip(kda::launch_replay(a, static_cast<hipStream_t>(stream)));
}

kda_status kda_chunk_fwd_z_noalloc(const void* q, const void* k, const void* v, const void* beta, const void* z,
                                   kda_dtype in_dtype, const float* A, float g_min, const float* S_in, void* o,
                                   kda_dtype o_dtype, float* S_out, int B, int T, int H, int dk, int dv, int chunk,
                                   float scale, void* stream) {
  // a need beyond the static array is reported as a workspace error (chunk_common
  // compares it with the array's size, after the argument checks)
  return chunk_common(q, k, v, beta, z, in_dtype, nullptr, A, g_min, S_in, o, o_dtype, S_out, B, T, H, dk, dv, chunk,
                      scale, true, 0, nullptr, kScratchBytes, false, stream, true);
}

}  // extern "C"
