// Gated DeltaNet with the CPR schedule on MI355X (gfx950): kernels and C ABI.
//
// The layer and the schedule are described in include/gdn.h.  Two pieces of
// arithmetic exist, and each is executed by exactly one piece of device code,
// whichever entry point runs it:
//
//   R  the token step (one token, one value head, the d_v rows of the state
//      spread one per lane).  Run by k_rec (prefill / trainer forward, state in
//      registers for a whole chunk) and by k_decode (state streamed from HBM).
//   B  the chunk form, giving the state at the end of a full chunk from the
//      state at its start.  Run by k_wy (chunk factors W, U, G; parallel over
//      chunks) and k_scan (the state update; sequential over the chunks of a
//      sequence), both for prefill and for the decode resync.
//
// Equality of bits between prefill and decode rests on: identical IEEE
// operation sequences per output element (the build uses -ffp-contract=off;
// every fused multiply-add is an explicit fmaf), the same expf / sqrtf, the
// same fixed summation orders, and per-item work that never depends on the
// launch's grid or on other items.  gdn_contract_id() names this contract.

#include <hip/hip_runtime.h>

#include <cstdint>
#include <cstring>
#include <mutex>
#include <string>
#include <vector>

#ifndef GDN_SOURCE_DIGEST
#define GDN_SOURCE_DIGEST "unversioned"
#endif
#include "gdn.h"
#include "gdn_plan.h"

// Fixed device scratch of gdn_decode_step_noalloc (the resync's chunk factors),
// for callers that cannot allocate device memory.  Each GPU the library runs
// on holds its own copy until the process ends.  Host code never passes this
// name to a kernel (on the host it is only a stand-in for the symbol): the
// array's address on a device comes from hipGetSymbolAddress (scratch_ptr).
static __device__ __align__(256) unsigned char scratch[GDN_NOALLOC_SCRATCH_BYTES];

namespace {

using bf16_t = uint16_t;

// Read-only, wave-uniform operands are read through the constant address
// space so the compiler issues scalar loads (the values land in SGPRs and feed
// the VALU directly).
using cfloat_p = const __attribute__((address_space(4))) float*;
__device__ __forceinline__ cfloat_p as_const(const float* p) {
  return reinterpret_cast<cfloat_p>(reinterpret_cast<uintptr_t>(p));
}

__device__ __forceinline__ float ldin(const float* p) { return *p; }
__device__ __forceinline__ float ldin(const bf16_t* p) {
  return __uint_as_float(static_cast<uint32_t>(*p) << 16);
}

// Component-wise select of float4 values (a ternary on the struct can turn
// into a select of addresses in private memory).
__device__ __forceinline__ float4 sel4(bool c, float4 a, float4 b) {
  return float4{c ? a.x : b.x, c ? a.y : b.y, c ? a.z : b.z, c ? a.w : b.w};
}

// Raw buffer access: a 4-dword resource over [base, base + bytes) in SGPRs,
// a per-lane byte offset and a wave-uniform byte offset.  Accesses outside
// the range read 0 / are dropped by the hardware.
using brsrc_t = __amdgpu_buffer_rsrc_t;
constexpr int kBufWord3 = 0x00020000;  // raw 32-bit data format (gfx9 family)
__device__ __forceinline__ brsrc_t make_rsrc(const void* base, uint32_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), static_cast<short>(0),
                                           static_cast<int>(bytes), kBufWord3);
}
__device__ __forceinline__ float ldbuf(brsrc_t r, uint32_t voff, uint32_t soff, const float*) {
  return __uint_as_float(__builtin_amdgcn_raw_buffer_load_b32(r, voff, soff, 0));
}
typedef float v4f __attribute__((ext_vector_type(4)));
__device__ __forceinline__ void stbuf4(v4f x, brsrc_t r, uint32_t voff, uint32_t soff) {
  __builtin_amdgcn_raw_buffer_store_b128(
      __builtin_bit_cast(uint32_t __attribute__((ext_vector_type(4))), x), r, voff, soff, 0);
}
__device__ __forceinline__ void stbuf(float x, brsrc_t r, uint32_t voff, uint32_t soff) {
  __builtin_amdgcn_raw_buffer_store_b32(__float_as_uint(x), r, voff, soff, 0);
}
__device__ __forceinline__ float4 ldbuf4(brsrc_t r, uint32_t voff, uint32_t soff) {
  const auto x = __builtin_amdgcn_raw_buffer_load_b128(r, voff, soff, 0);
  return float4{__uint_as_float(x[0]), __uint_as_float(x[1]), __uint_as_float(x[2]),
                __uint_as_float(x[3])};
}
__device__ __forceinline__ float ldbuf(brsrc_t r, uint32_t voff, uint32_t soff, const bf16_t*) {
  const uint16_t x = __builtin_amdgcn_raw_buffer_load_b16(r, voff, soff, 0);
  return __uint_as_float(static_cast<uint32_t>(x) << 16);
}
// Four consecutive input elements as floats: 16 bytes (fp32) or 8 (bf16).
__device__ __forceinline__ float4 ldbuf4in(brsrc_t r, uint32_t voff, uint32_t soff, const float*) {
  return ldbuf4(r, voff, soff);
}
__device__ __forceinline__ float4 ldbuf4in(brsrc_t r, uint32_t voff, uint32_t soff, const bf16_t*) {
  const auto x = __builtin_amdgcn_raw_buffer_load_b64(r, voff, soff, 0);
  return float4{__uint_as_float(x[0] << 16), __uint_as_float(x[0] & 0xffff0000u), __uint_as_float(x[1] << 16),
                __uint_as_float(x[1] & 0xffff0000u)};
}

// Largest n in [0, N) with arr[n] <= x (arr non-decreasing, arr[0] = 0): the
// sequence that owns slot x.  Uniform across the block.
__device__ __forceinline__ int find_seq(const int32_t* __restrict__ arr, int N, int64_t x) {
  int lo = 0, hi = N - 1;
  while (lo < hi) {
    const int mid = (lo + hi + 1) >> 1;
    if (arr[mid] <= x) lo = mid; else hi = mid - 1;
  }
  return lo;
}

// ---------------------------------------------------------------------------
// L2 normalisation of one d-vector (d <= 128) by one full wave of 64 lanes.
// Lane l holds elements l and l + 64.  The sum of squares is combined by a
// butterfly, after which every lane holds the same value.  Every kernel that
// needs a normalised q or k goes through l2norm_vals (directly or through
// l2norm_wave), so all of them see the same bits.
// The arithmetic on already loaded elements x0 = x[l], x1 = x[l + 64]:
template <int D>
__device__ __forceinline__ void l2norm_vals(float x0, float x1, float mul, int do_norm, float& y0,
                                            float& y1) {
  if (do_norm) {
    float ss = fmaf(x1, x1, x0 * x0);
#pragma unroll
    for (int m = 32; m >= 1; m >>= 1) ss += __shfl_xor(ss, m, 64);
    const float r = 1.0f / sqrtf(ss + gdn::kNormEps);
    x0 = x0 * r;
    x1 = x1 * r;
  }
  y0 = x0 * mul;
  y1 = x1 * mul;
}
// The same normalisation at d = 128 with sixteen lanes per vector, so that a
// lane loads and stores its elements 8 or 16 bytes at a time: lane lam of the
// group holds elements 4 lam + i (lo) and 64 + 4 lam + i (hi), i = 0..3.  The
// sums are those of l2norm_vals: leaf l = fmaf(x[l + 64], x[l + 64], x[l] x[l]),
// then pairs (l, l ^ m) for m = 32, 16, 8, 4, 2, 1.  With l = 4 lam + i the
// pairs for m = 32 .. 4 are lanes lam ^ 8 .. lam ^ 1 with the same i, and for
// m = 2, 1 they are i ^ 2, i ^ 1 within the lane; a pair's sum does not depend
// on which of the two adds, so every result has l2norm_vals' bits.
__device__ __forceinline__ void l2norm_quads(float4& lo, float4& hi, float mul, int do_norm) {
  if (do_norm) {
    float e0 = fmaf(hi.x, hi.x, lo.x * lo.x), e1 = fmaf(hi.y, hi.y, lo.y * lo.y);
    float e2 = fmaf(hi.z, hi.z, lo.z * lo.z), e3 = fmaf(hi.w, hi.w, lo.w * lo.w);
#pragma unroll
    for (int m = 8; m >= 1; m >>= 1) {
      e0 += __shfl_xor(e0, m, 64);
      e1 += __shfl_xor(e1, m, 64);
      e2 += __shfl_xor(e2, m, 64);
      e3 += __shfl_xor(e3, m, 64);
    }
    const float r = 1.0f / sqrtf(((e0 + e2) + (e1 + e3)) + gdn::kNormEps);
    lo = float4{lo.x * r, lo.y * r, lo.z * r, lo.w * r};
    hi = float4{hi.x * r, hi.y * r, hi.z * r, hi.w * r};
  }
  lo = float4{lo.x * mul, lo.y * mul, lo.z * mul, lo.w * mul};
  hi = float4{hi.x * mul, hi.y * mul, hi.z * mul, hi.w * mul};
}
// Four consecutive input elements as floats (16 bytes fp32, 8 bytes bf16).
__device__ __forceinline__ float4 ld4in(const float* p) { return *reinterpret_cast<const float4*>(p); }
__device__ __forceinline__ float4 ld4in(const bf16_t* p) {
  const uint2 x = *reinterpret_cast<const uint2*>(p);
  return float4{__uint_as_float(x.x << 16), __uint_as_float(x.x & 0xffff0000u), __uint_as_float(x.y << 16),
                __uint_as_float(x.y & 0xffff0000u)};
}
template <int D, typename TIn>
__device__ __forceinline__ void l2norm_wave(const TIn* __restrict__ x, float mul, int do_norm,
                                            float& y0, float& y1) {
  const int l = threadIdx.x & 63;
  const float x0 = (l < D) ? ldin(x + l) : 0.0f;
  const float x1 = (D > 64) ? ldin(x + l + 64) : 0.0f;
  l2norm_vals<D>(x0, x1, mul, do_norm, y0, y1);
}

// ---------------------------------------------------------------------------
// Device planner: per-sequence prefix counts of chunks (ceil) and full chunks
// (floor).  One thread; N is small next to the token count.  It runs in the
// first thread of the prep kernel (one launch fewer on the path), or alone in
// k_plan when there is nothing to normalise.
struct PlanArgs {
  const int32_t* cu;  // nullptr: no plan
  int N, C;
  int32_t* cu_chunks;
  int32_t* cu_full;
};
__device__ __forceinline__ void plan_counts(const PlanArgs& p) {
  int32_t a = 0, b = 0;
  p.cu_chunks[0] = 0;
  p.cu_full[0] = 0;
  for (int n = 0; n < p.N; ++n) {
    int32_t L = p.cu[n + 1] - p.cu[n];
    if (L < 0) L = 0;
    a += (L + p.C - 1) / p.C;
    b += L / p.C;
    p.cu_chunks[n + 1] = a;
    p.cu_full[n + 1] = b;
  }
}
__global__ void k_plan(const int32_t* __restrict__ cu, int N, int C, int32_t* __restrict__ cu_chunks,
                       int32_t* __restrict__ cu_full) {
  if (blockIdx.x != 0 || threadIdx.x != 0) return;
  plan_counts(PlanArgs{cu, N, C, cu_chunks, cu_full});
}

// Sequences by length, longest first (ties by index): order[rank] = n.  One
// thread per sequence counts the sequences ranked ahead of it.
__global__ void k_order(const int32_t* __restrict__ cu, int N, int32_t* __restrict__ order) {
  const int n = blockIdx.x * blockDim.x + threadIdx.x;
  if (n >= N) return;
  const int32_t Ln = cu[n + 1] - cu[n];
  int rank = 0;
  for (int m = 0; m < N; ++m) {
    const int32_t Lm = cu[m + 1] - cu[m];
    rank += (Lm > Ln || (Lm == Ln && m < n)) ? 1 : 0;
  }
  order[rank] = n;
}

// ---------------------------------------------------------------------------
// Prep: normalised k and q (times scale) in fp32, written head-major and
// interleaved: qk[hq][t][0][:] = k-hat, qk[hq][t][1][:] = q-hat.  A chunk's
// key/query stream for one head is then a single contiguous run, read by
// k_rec as wave-uniform scalar loads.  Each wave normalises kPrepVecs
// consecutive (token, q/k head) vectors, after loading all of them: at
// d = 128 four at a time with l2norm_quads, else one at a time with the lanes
// and arithmetic of l2norm_wave.
constexpr int kPrepVecs = 4;
// (g, beta) of each value head in token order, gb[h][t] = (g[t][h], beta[t][h]):
// the token step then reads a token's pair with one 8-byte scalar load, eight
// tokens to a cache line (in [t][h] order each token's pair is a new line for
// every wave of the head).  Null: not written.
struct GbArgs {
  const float* g;
  const float* beta;
  float* gb;
  int H_v;
};
template <int D, typename TIn>
__global__ __launch_bounds__(256) void k_prep(const TIn* __restrict__ q, const TIn* __restrict__ k,
                                              float* __restrict__ qk, int64_t T, int H_qk,
                                              float scale, int l2, PlanArgs plan, GbArgs gb) {
  if (plan.cu && blockIdx.x == 0 && threadIdx.x == 0) plan_counts(plan);
  if (gb.gb) {
    const int64_t n = T * gb.H_v;
    for (int64_t e = static_cast<int64_t>(blockIdx.x) * 256 + threadIdx.x; e < n;
         e += static_cast<int64_t>(gridDim.x) * 256) {
      const int64_t t = e / gb.H_v;
      const int64_t h = e - t * gb.H_v;
      *reinterpret_cast<float2*>(gb.gb + (h * T + t) * 2) = float2{gb.g[e], gb.beta[e]};
    }
  }
  const int64_t nvec = T * H_qk;
  const int64_t vec0 = (static_cast<int64_t>(blockIdx.x) * 4 + (threadIdx.x >> 6)) * kPrepVecs;
  if (vec0 >= nvec) return;
  const int l = threadIdx.x & 63;
  if constexpr (D == 128) {
    static_assert(kPrepVecs % 4 == 0, "whole lane groups");
    constexpr int NR = kPrepVecs / 4;  // rounds of four vectors
    const int lg = l >> 4, lam = l & 15;
    float4 klo[NR], khi[NR], qlo[NR], qhi[NR];
#pragma unroll
    for (int r = 0; r < NR; ++r) {
      const int64_t vr = vec0 + 4 * r + lg;
      const int64_t vec = vr < nvec ? vr : nvec - 1;  // t * H_qk + hq
      klo[r] = ld4in(k + vec * D + 4 * lam);
      khi[r] = ld4in(k + vec * D + 64 + 4 * lam);
      qlo[r] = ld4in(q + vec * D + 4 * lam);
      qhi[r] = ld4in(q + vec * D + 64 + 4 * lam);
    }
    // (token, head) of vec0 once per wave; the lane's vector is a few past it
    const int64_t t0 = vec0 / H_qk;
    const int h0 = static_cast<int>(vec0 - t0 * H_qk);
#pragma unroll
    for (int r = 0; r < NR; ++r) {
      const int64_t vec = vec0 + 4 * r + lg;
      l2norm_quads(klo[r], khi[r], 1.0f, l2);  // every lane: the shuffles read all of them
      l2norm_quads(qlo[r], qhi[r], scale, l2);
      if (vec < nvec) {
        const int off = h0 + 4 * r + lg;  // < H_qk + kPrepVecs
        const int64_t t = t0 + off / H_qk;
        const int hq = off % H_qk;
        float* out = qk + (static_cast<int64_t>(hq) * T + t) * 2 * D;
        *reinterpret_cast<float4*>(out + 4 * lam) = klo[r];
        *reinterpret_cast<float4*>(out + 64 + 4 * lam) = khi[r];
        *reinterpret_cast<float4*>(out + D + 4 * lam) = qlo[r];
        *reinterpret_cast<float4*>(out + D + 64 + 4 * lam) = qhi[r];
      }
    }
    return;
  }
  float k0[kPrepVecs], k1[kPrepVecs], q0[kPrepVecs], q1[kPrepVecs];
#pragma unroll
  for (int v = 0; v < kPrepVecs; ++v) {
    const int64_t vec = vec0 + v < nvec ? vec0 + v : nvec - 1;  // t * H_qk + hq
    k0[v] = (l < D) ? ldin(k + vec * D + l) : 0.0f;
    k1[v] = (D > 64) ? ldin(k + vec * D + l + 64) : 0.0f;
    q0[v] = (l < D) ? ldin(q + vec * D + l) : 0.0f;
    q1[v] = (D > 64) ? ldin(q + vec * D + l + 64) : 0.0f;
  }
#pragma unroll
  for (int v = 0; v < kPrepVecs; ++v) {
    const int64_t vec = vec0 + v;
    if (vec >= nvec) break;  // uniform over the wave
    const int64_t t = vec / H_qk;
    const int hq = static_cast<int>(vec - t * H_qk);
    float* out = qk + (static_cast<int64_t>(hq) * T + t) * 2 * D;
    float y0, y1;
    l2norm_vals<D>(k0[v], k1[v], 1.0f, l2, y0, y1);
    if (l < D) out[l] = y0;
    if (D > 64) out[l + 64] = y1;
    l2norm_vals<D>(q0[v], q1[v], scale, l2, y0, y1);
    if (l < D) out[D + l] = y0;
    if (D > 64) out[D + l + 64] = y1;
  }
}
__host__ __device__ constexpr int64_t prep_blocks(int64_t nvec) {
  return (nvec + 4 * kPrepVecs - 1) / (4 * kPrepVecs);
}

// ---------------------------------------------------------------------------
// B, part 1 -- chunk factors.  For one full chunk of one value head, with
// G_p the running fp32 sum of g (p ascending) and gam_p = exp(G_p):
//   A_pr = beta_p * ((k_p . k_r) * exp(G_p - G_r))      p > r
//   w_p  = beta_p gam_p k_p - sum_{r<p} A_pr w_r        (r ascending)
//   u_p  = beta_p v_p       - sum_{r<p} A_pr u_r
// Writes W, U [C, D] and G [C].  Items: every full chunk of a prefill
// (RESYNC = false) or, for decode, every (sequence, head) whose chunk just
// completed (pos == 0 after the token step), reading the chunk buffers.
struct ChunkIO {
  const float* khat;   // normalised keys, fp32 (see k_wy for the addressing)
  const void* v;       // values, in_dtype, token stride H_v * D
  const float* beta;   // token stride H_v
  const float* g;      // token stride H_v
  const int32_t* cu;   // prefill: cu_seqlens
  const int32_t* cu_full;
  const int32_t* pos;  // resync: cache pos [N, H_v]
  float* W;
  float* U;
  float* G;
  int N, H_qk, H_v;
  int64_t T;           // prefill: total tokens (bounds); resync: N * C
  int64_t max_slot;    // W/U/G slots available
};

// Start of the normalised keys of a chunk and the stride between its tokens:
// prefill reads the prep layout [H_qk][T][2][D], resync the cache buffer
// [N][C][H_qk][D].  Only the addressing differs; the values are the same bits.
template <int D, bool RESYNC>
__device__ __forceinline__ const float* key_rows(const float* base, int64_t T, int H_qk, int hq,
                                                 int64_t tok0, int64_t& stride) {
  if (RESYNC) {
    stride = static_cast<int64_t>(H_qk) * D;
    return base + (tok0 * H_qk + hq) * D;
  }
  stride = 2 * D;
  return base + (static_cast<int64_t>(hq) * T + tok0) * 2 * D;
}

// Item modes of the chunk-form kernels.  kFull: the full chunks of a prefill
// (W/U/G slots = full-chunk slots).  kResync: the decode buffers.  kAll: every
// chunk of every sequence, the last one possibly partial (trainer forward;
// W/U/G slots = chunk slots).  A partial chunk of L < C tokens is padded with
// rows k = 0, v = 0, beta = 0, g = 0, which leaves the chunk algebra exact;
// a full chunk executes the same operations in every mode.
enum Mode { kFull = 0, kResync = 1, kAll = 2 };

// Chunk-factor blocks, grid (8 G ceil(items / 8), H_qk): the G value heads of
// a q/k group read the same keys, so the blocks of one group and item go out
// 8 apart and land on the same XCD (blocks are dispatched round-robin over the
// 8 XCDs) at about the same time; the later ones find the keys in its L2.
// Items past the last one exit in the kernels' range checks.
__device__ __forceinline__ void wy_item(int G, int64_t& item, int& h) {
  const int64_t x = blockIdx.x;
  item = (x / (8 * G)) * 8 + x % 8;
  h = static_cast<int>(blockIdx.y) * G + static_cast<int>((x / 8) % G);
}

template <int D, int C, typename TIn, int MODE>
__global__ __launch_bounds__(256) void k_wy(ChunkIO io) {
  constexpr bool RESYNC = MODE == kResync;
  constexpr int NT = 256;
  __shared__ float sK[C][D + 1];
  __shared__ float sA[C][C + 1];
  __shared__ float sY[C][2 * D];  // column t: W (t < D) or U (t >= D); owned by thread t
  __shared__ float sB[C], sG[C], sBG[C];
  const int tid = threadIdx.x;
  int64_t item;
  int h;
  wy_item(io.H_v / io.H_qk, item, h);
  const int hq = h / (io.H_v / io.H_qk);
  int64_t tok0, slot;
  int L = C;
  if (MODE == kResync) {
    if (item >= io.N) return;
    const int n = static_cast<int>(item);
    if (io.pos[static_cast<int64_t>(n) * io.H_v + h] != 0) return;
    tok0 = static_cast<int64_t>(n) * C;
    slot = n;
  } else if (MODE == kFull) {
    slot = item;
    if (slot >= io.cu_full[io.N]) return;
    const int n = find_seq(io.cu_full, io.N, slot);
    tok0 = static_cast<int64_t>(io.cu[n]) + static_cast<int64_t>(slot - io.cu_full[n]) * C;
  } else {
    slot = item;
    if (slot >= io.cu_full[io.N]) return;  // cu_full holds the chunk prefix in this mode
    const int n = find_seq(io.cu_full, io.N, slot);
    tok0 = static_cast<int64_t>(io.cu[n]) + static_cast<int64_t>(slot - io.cu_full[n]) * C;
    const int64_t rem = static_cast<int64_t>(io.cu[n + 1]) - tok0;
    L = rem < C ? static_cast<int>(rem) : C;
    if (L <= 0) return;
  }
  if (tok0 < 0 || tok0 + L > io.T || slot >= io.max_slot) return;

  const TIn* v = static_cast<const TIn*>(io.v);
  int64_t kst;
  const float* krow = key_rows<D, RESYNC>(io.khat, io.T, io.H_qk, hq, tok0, kst);
  for (int e = tid; e < C * D; e += NT) {
    const int p = e / D, i = e % D;
    sK[p][i] = p < L ? krow[p * kst + i] : 0.0f;
  }
  if (tid < C) sB[tid] = tid < L ? io.beta[(tok0 + tid) * io.H_v + h] : 0.0f;
  if (tid == 0) {
    float acc = 0.0f;
    for (int p = 0; p < C; ++p) {
      acc = acc + (p < L ? io.g[(tok0 + p) * io.H_v + h] : 0.0f);
      sG[p] = acc;
    }
  }
  __syncthreads();
  if (tid < C) sBG[tid] = sB[tid] * expf(sG[tid]);
  for (int e = tid; e < C * C; e += NT) {
    const int p = e / C, r = e % C;
    float a = 0.0f;
    if (r < p) {
      float dot = 0.0f;
#pragma unroll 8
      for (int i = 0; i < D; ++i) dot = fmaf(sK[p][i], sK[r][i], dot);
      a = sB[p] * (dot * expf(sG[p] - sG[r]));
    }
    sA[p][r] = a;
  }
  __syncthreads();
  // forward substitution: thread j < D owns column j of W, thread D + j of U
  if (tid < 2 * D) {
    const bool isW = tid < D;
    const int j = isW ? tid : tid - D;
    float* out = (isW ? io.W : io.U) + (slot * io.H_v + h) * static_cast<int64_t>(C) * D;
    for (int p = 0; p < C; ++p) {
      const float vx = p < L ? ldin(v + (tok0 + p) * io.H_v * D + static_cast<int64_t>(h) * D + j)
                             : 0.0f;
      float x = isW ? sBG[p] * sK[p][j] : sB[p] * vx;
      for (int r = 0; r < p; ++r) x = fmaf(-sA[p][r], sY[r][tid], x);
      sY[p][tid] = x;
      out[static_cast<int64_t>(p) * D + j] = x;
    }
  }
  if (tid < C) io.G[(slot * io.H_v + h) * C + tid] = sG[tid];
}

// ---------------------------------------------------------------------------
// B, part 2 -- the state update over one full chunk, for a tile of TILE rows
// (d_v indices) of the state; rows evolve independently, so tiling is exact.
//   Delta_pj = U_pj - sum_i W_pi S_ji                 (i ascending)
//   Dt_pj    = Delta_pj * exp(G_last - G_p)
//   S'_ji    = exp(G_last) S_ji  then  += Dt_pj k_pi   (p ascending, fmaf)
// Prefill (RESYNC = false): one block per (sequence, head, tile) walks the
// sequence's full chunks, storing each chunk-start state, the tail chunk's
// start state, and the final state when the sequence ends on a chunk edge.
// Resync: one step from cache S_chunk for each (sequence, head) with pos == 0,
// writing S_chunk = S_run = result.
// Row quads.  At d = 128 outside the all-chunks mode, the prefill's
// chunk-start states [d][d] keep each run of four consecutive rows of a
// column together: element (r, j) sits at ((r / 4) d + j) 4 + r % 4.  A lane
// that holds rows 4 q .. 4 q + 3 of column j (the scan's accumulator layout,
// the token step's row part) then moves them with one 16-byte access, and
// consecutive columns are consecutive 16-byte words.
struct ScanIO {
  const float* khat;     // prefill: prep keys; resync: cache kbuf
  const float* W;
  const float* U;
  const float* G;
  const int32_t* cu;
  const int32_t* cu_chunks;
  const int32_t* cu_full;
  const float* h0;       // nullable
  float* states;         // prefill chunk-start states
  float* hT;             // nullable
  float* Dl;             // kAll: Delta of every chunk [slot][H_v][C][D]
  float* hT_tail;        // kAll, nullable: the chunk-form final state of a
                         // sequence whose last chunk is partial
  // cache (nullable in prefill)
  float* S_run;
  float* S_chunk;
  int32_t* pos;
  int N, H_qk, H_v;
  int64_t T;
  int64_t max_state_slot, max_full_slot;
  const int32_t* order;  // nullable: sequences longest first (d = 128 scan)
};

template <int D, int C, int TILE, int MODE>
__global__ __launch_bounds__(256) void k_scan(ScanIO io) {
  constexpr bool RESYNC = MODE == kResync;
  constexpr int NT = 256;
  constexpr int NTILE = D / TILE;
  __shared__ float sS[TILE][D + 1];
  __shared__ float sW[C][D];
  __shared__ float sK[C][D];
  __shared__ float sD[C][TILE + 1];
  __shared__ float sG[C];
  const int tid = threadIdx.x;
  const int tile = blockIdx.x % NTILE;
  const int h = (blockIdx.x / NTILE) % io.H_v;
  const int n = blockIdx.x / (NTILE * io.H_v);
  if (n >= io.N) return;
  const int hq = h / (io.H_v / io.H_qk);
  const int j0 = tile * TILE;
  const int64_t DD = static_cast<int64_t>(D) * D;
  const int64_t nh = static_cast<int64_t>(n) * io.H_v + h;

  int64_t tok0 = 0, nsteps = 1, L = 0, slot0 = 0, fslot0 = 0, nchunks = 0;
  if (RESYNC) {
    if (io.pos[nh] != 0) return;
    fslot0 = n;
  } else {
    tok0 = io.cu[n];
    L = static_cast<int64_t>(io.cu[n + 1]) - tok0;
    if (L < 0 || tok0 < 0 || tok0 + L > io.T) return;
    nchunks = (L + C - 1) / C;
    nsteps = MODE == kAll ? nchunks : L / C;
    slot0 = io.cu_chunks[n];
    fslot0 = MODE == kAll ? slot0 : io.cu_full[n];
    if (slot0 + nchunks > io.max_state_slot || fslot0 + nsteps > io.max_full_slot) return;
  }

  // load the starting state tile: S_ji = stored[i][j]
  const float* src = RESYNC ? io.S_chunk + nh * DD : (io.h0 ? io.h0 + nh * DD : nullptr);
  for (int e = tid; e < TILE * D; e += NT) {
    const int i = e / TILE, jj = e % TILE;
    sS[jj][i] = src ? src[static_cast<int64_t>(i) * D + j0 + jj] : 0.0f;
  }
  __syncthreads();

  for (int64_t c = 0; c < nsteps; ++c) {
    if (!RESYNC) {  // chunk-start state of chunk c
      float* dst = io.states + ((slot0 + c) * io.H_v + h) * DD;
      for (int e = tid; e < TILE * D; e += NT) {
        const int i = e / TILE, jj = e % TILE;
        dst[static_cast<int64_t>(i) * D + j0 + jj] = sS[jj][i];
      }
    }
    const int64_t fs = fslot0 + c;
    const float* Wc = io.W + (fs * io.H_v + h) * static_cast<int64_t>(C) * D;
    const float* Uc = io.U + (fs * io.H_v + h) * static_cast<int64_t>(C) * D;
    const float* Gc = io.G + (fs * io.H_v + h) * C;
    const int64_t ktok0 = RESYNC ? static_cast<int64_t>(n) * C : tok0 + c * C;
    int64_t kst;
    const float* krow = key_rows<D, RESYNC>(io.khat, io.T, io.H_qk, hq, ktok0, kst);
    const int64_t rows = RESYNC ? C : (L - c * C < C ? L - c * C : C);  // < C: padded tail
    for (int e = tid; e < C * D; e += NT) {
      const int p = e / D, i = e % D;
      sW[p][i] = Wc[e];
      sK[p][i] = p < rows ? krow[p * kst + i] : 0.0f;
    }
    if (tid < C) sG[tid] = Gc[tid];
    __syncthreads();
    const float glast = sG[C - 1];
    for (int e = tid; e < C * TILE; e += NT) {
      const int p = e / TILE, jj = e % TILE;
      float acc = 0.0f;
#pragma unroll 8
      for (int i = 0; i < D; ++i) acc = fmaf(sW[p][i], sS[jj][i], acc);
      const float delta = Uc[static_cast<int64_t>(p) * D + j0 + jj] - acc;
      if (MODE == kAll) io.Dl[((fs * io.H_v + h) * C + p) * static_cast<int64_t>(D) + j0 + jj] = delta;
      sD[p][jj] = delta * expf(glast - sG[p]);
    }
    __syncthreads();
    const float gam = expf(glast);
    for (int e = tid; e < TILE * D; e += NT) {
      const int jj = e / D, i = e % D;
      float acc = gam * sS[jj][i];
#pragma unroll 8
      for (int p = 0; p < C; ++p) acc = fmaf(sD[p][jj], sK[p][i], acc);
      sS[jj][i] = acc;  // each (jj, i) is read and written by this thread only
    }
    __syncthreads();
  }

  if (RESYNC) {
    float* d1 = io.S_chunk + nh * DD;
    float* d2 = io.S_run + nh * DD;
    for (int e = tid; e < TILE * D; e += NT) {
      const int i = e / TILE, jj = e % TILE;
      const float x = sS[jj][i];
      d1[static_cast<int64_t>(i) * D + j0 + jj] = x;
      d2[static_cast<int64_t>(i) * D + j0 + jj] = x;
    }
    return;
  }
  const bool tail = (L % C) != 0;
  if (MODE == kAll && tail) return;  // the tail's start state was stored in the loop
  for (int e = tid; e < TILE * D; e += NT) {
    const int i = e / TILE, jj = e % TILE;
    const int64_t off = static_cast<int64_t>(i) * D + j0 + jj;
    const float x = sS[jj][i];
    if (tail) {
      io.states[((slot0 + nsteps) * io.H_v + h) * DD + off] = x;  // tail chunk start
      if (io.S_chunk) io.S_chunk[nh * DD + off] = x;
    } else {
      if (io.hT) io.hT[nh * DD + off] = x;
      if (io.S_chunk) {
        io.S_chunk[nh * DD + off] = x;
        io.S_run[nh * DD + off] = x;
      }
    }
  }
  if (io.pos && tile == 0 && tid == 0) io.pos[nh] = static_cast<int32_t>(L % C);
}

// ---------------------------------------------------------------------------
// Matrix-core helpers.  mfma4 is v_mfma_f32_16x16x4_f32 on one 16 x 16 tile:
// lane l supplies A[l % 16][l / 16] and B[l / 16][l % 16], and holds
// D[4 (l / 16) + r][l % 16] in accumulator register r.

__device__ __forceinline__ v4f mfma4(float a, float b, v4f c) {
  return __builtin_amdgcn_mfma_f32_16x16x4f32(a, b, c, 0, 0, 0);
}

// Launches are padded to a multiple of 8 blocks; consecutive virtual block
// ids land on the same XCD (blocks are dispatched round-robin over the 8 XCDs)
// so the tiles of one head, and the heads of one q/k group, share an L2.
__device__ __forceinline__ int64_t xcd_block(int64_t nb8) {
  const int64_t b = blockIdx.x;
  return (b % 8) * (nb8 / 8) + b / 8;
}

// Matrix-core products of fp32 operands from bf16 parts.  A value x is
// written as three bf16 parts, x = hi + mid + lo exactly: hi is x rounded to
// nearest bf16; the residual x - hi is exact in fp32 (hi is within a factor
// two of x) and has at most 16 significant bits; mid is that residual rounded
// to nearest, and what is left has at most 8 significant bits, so lo holds it
// exactly (for |x| above about 2^-110; smaller parts meet the bf16 range).
// |mid| <= 2^-8 |x| and |lo| <= 2^-16 |x|, so of the nine part products of
// a b the six kept,
//   ah bh, ah bm, ah bl, am bh, am bm, al bh,
// leave out three whose sum is below 2^-23 |a b| and of either sign.  Each
// part product is exact in fp32; v_mfma_f32_16x16x32_bf16 sums them into an
// fp32 accumulator.  Parts are packed two per 32-bit word, the lower element
// in the low half, and a lane's eight elements of one part fill four words.
typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
typedef float f32x2_t __attribute__((ext_vector_type(2)));
typedef uint32_t u32x4_t __attribute__((ext_vector_type(4)));
struct Parts {
  u32x4_t p[3];  // hi, mid, lo
};

__device__ __forceinline__ uint32_t pack_bf16(float a, float b) {
  return __builtin_bit_cast(uint32_t, __builtin_convertvector(f32x2_t{a, b}, bf16x2_t));
}
__device__ __forceinline__ void split_pair(float x0, float x1, uint32_t& h, uint32_t& m, uint32_t& l) {
  h = pack_bf16(x0, x1);
  const float r0 = x0 - __uint_as_float(h << 16), r1 = x1 - __uint_as_float(h & 0xffff0000u);
  m = pack_bf16(r0, r1);
  const float s0 = r0 - __uint_as_float(m << 16), s1 = r1 - __uint_as_float(m & 0xffff0000u);
  l = pack_bf16(s0, s1);  // exact
}
// parts of x[0..7] and of y[0..7], stage by stage over all sixteen values
// (neighbouring instructions are then independent)
__device__ __forceinline__ void split8x2(const float (&x)[8], const float (&y)[8], Parts& px, Parts& py) {
  float v[16], r[16];
  uint32_t h[8], m[8], l[8];
#pragma unroll
  for (int k = 0; k < 8; ++k) v[k] = x[k], v[8 + k] = y[k];
#pragma unroll
  for (int k = 0; k < 8; ++k) h[k] = pack_bf16(v[2 * k], v[2 * k + 1]);
#pragma unroll
  for (int k = 0; k < 8; ++k) {
    r[2 * k] = v[2 * k] - __uint_as_float(h[k] << 16);
    r[2 * k + 1] = v[2 * k + 1] - __uint_as_float(h[k] & 0xffff0000u);
  }
#pragma unroll
  for (int k = 0; k < 8; ++k) m[k] = pack_bf16(r[2 * k], r[2 * k + 1]);
#pragma unroll
  for (int k = 0; k < 8; ++k) {
    r[2 * k] = r[2 * k] - __uint_as_float(m[k] << 16);
    r[2 * k + 1] = r[2 * k + 1] - __uint_as_float(m[k] & 0xffff0000u);
  }
#pragma unroll
  for (int k = 0; k < 8; ++k) l[k] = pack_bf16(r[2 * k], r[2 * k + 1]);  // exact
#pragma unroll
  for (int k = 0; k < 4; ++k) {
    px.p[0][k] = h[k], px.p[1][k] = m[k], px.p[2][k] = l[k];
    py.p[0][k] = h[4 + k], py.p[1][k] = m[4 + k], py.p[2][k] = l[4 + k];
  }
}
// parts of x[0..7]
__device__ __forceinline__ Parts split8(const float (&x)[8]) {
  Parts r;
#pragma unroll
  for (int k = 0; k < 4; ++k) {
    uint32_t h, m, l;
    split_pair(x[2 * k], x[2 * k + 1], h, m, l);
    r.p[0][k] = h, r.p[1][k] = m, r.p[2][k] = l;
  }
  return r;
}
// parts of the eight values {x[0..3], y[0..3]} (two accumulator tiles)
__device__ __forceinline__ Parts split8(v4f x, v4f y) {
  const float v[8] = {x[0], x[1], x[2], x[3], y[0], y[1], y[2], y[3]};
  return split8(v);
}
// v_mfma_f32_16x16x32_bf16: lane l supplies A[l % 16][8 (l / 16) + e] and
// B[8 (l / 16) + e][l % 16] for e = 0..7, and holds D[4 (l / 16) + r][l % 16]
// in accumulator register r (the same output layout as mfma4).
__device__ __forceinline__ v4f mfma_bf(u32x4_t a, u32x4_t b, v4f c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8_t, a), __builtin_bit_cast(bf16x8_t, b),
                                                 c, 0, 0, 0);
}

// Scheduling pattern for a region of NM products: its NR LDS reads first, then
// each product followed by up to three VALU instructions.
template <int NM, int NR>
__device__ __forceinline__ void mfma_valu_pattern() {
  __builtin_amdgcn_sched_group_barrier(0x100, NR, 0);  // LDS reads
  __builtin_amdgcn_sched_group_barrier(0x002, 8, 0);   // VALU
#pragma unroll
  for (int i = 0; i < NM; ++i) {
    __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);  // MFMA
    __builtin_amdgcn_sched_group_barrier(0x002, 3, 0);  // VALU
  }
}

// B, part 2 on the matrix cores (d = 128, C = 64): the chunk-state scan
//   Delta = U - W S^T,   S' = gam_C S + sum_p lam_p Delta_p k_p^T
// (gam_C = exp(G_C), lam_p = exp(G_C - G_p)), sequential over the chunks of a
// sequence, with fp32 operands as bf16 parts (above).  A block of NW waves (4
// or 8) owns 16 NW columns j of d_v of one (sequence, head); wave w holds S^T
// (rows i of d_k, its 16 columns j) as eight 16 x 16 accumulator tiles.
// Every column is computed the same way whatever the block width.
//
// Contraction order.  A k block of 32 (kb) is spread over the lanes so that
// both products take their B operand from accumulator tiles: lane group g
// supplies, as element e, k = 32 kb + 16 (e / 4) + 4 g + e % 4, which is
// register e % 4 of tile 2 kb + e / 4 of the state (Delta, k = i) or of
// lam * Delta (S', k = p).  The A operands (W rows p, columns i; K^T rows i,
// columns p) sit in LDS as parts in that same element order, so a lane reads
// each part of its eight elements as one 16-byte word.  Summation orders:
// Delta starts from -U and adds, for kb = 0..3, the six part products in the
// order listed above (it is kept negated; S' takes lam * Delta from
// (-lam) * (-Delta)); S' starts from gam_C S and adds, for the two k blocks of
// p, the same six.
//
// Staging.  W and G of chunk c + 1 are loaded at the end of chunk c - 1's S'
// products and W goes to LDS (as parts) during chunk c's S' products; K of chunk c + 1 is
// loaded during chunk c's S' products and written during chunk c + 1's Delta
// products.  The W and K^T buffers are then each written while the other is
// read, with two barriers per chunk, and every load has a whole phase to
// arrive.  Past the last chunk the loads reload the last chunk's operands,
// which nothing reads: the loop body has no branches.  Decode resync runs
// this same kernel on the chunk buffers.
template <int C, int MODE, int NW>
__global__ __launch_bounds__(64 * NW) __attribute__((amdgpu_waves_per_eu(NW / 4))) void k_scan_mfma(ScanIO io,
                                                                                            int64_t nblocks,
                                                                                            int64_t nb8) {
  constexpr int D = 128;
  // 32-bit words per LDS row: 16 (W) or 8 (K^T) groups of three 16-byte
  // parts, plus 16 bytes (rows l and l + 1 of a read then start 4 banks apart)
  constexpr int WR = 16 * 12 + 4, KR = 8 * 12 + 4;
  constexpr int NB = D / (16 * NW);  // blocks per (sequence, head)
  constexpr int NR = 16 / NW;        // W rows per thread (one group of 8 columns each)
  constexpr int KC = 16 / NW;        // K^T rows (key columns i) per thread (one group of 8 keys each)
  constexpr int KCS = D / KC;        // threads per key group
  static_assert(C == 64 && (NW == 4 || NW == 8), "tiling assumes C = 64, D = 128");
  constexpr bool RESYNC = MODE == kResync;
  __shared__ __attribute__((aligned(16))) uint32_t sW[C * WR];  // W[p][group of i][part][8]
  __shared__ __attribute__((aligned(16))) uint32_t sK[D * KR];  // K^T[i][group of p][part][8]
  __shared__ float sLam[C];                                     // -lam_p
  const int tid = threadIdx.x, lane = tid & 63, l16 = lane & 15, g = lane >> 4;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
  // ordered launches keep the dispatch order, so the longest sequences start
  // first on every XCD; virtual blocks 2 p and 2 p + 1 (the two halves of a
  // head, or two heads of a q/k group) go out 8 blocks apart, i.e. to the same
  // XCD at about the same time, and share their W and K (K) through its L2
  // (the grid is then a multiple of 16 blocks)
  const int64_t bx = blockIdx.x;
  const int64_t vb = io.order ? ((bx / 16) * 8 + bx % 8) * 2 + (bx / 8) % 2 : xcd_block(nb8);
  if (vb >= nblocks) return;
  const int half = static_cast<int>(vb % NB);
  const int h = static_cast<int>((vb / NB) % io.H_v);
  int n = static_cast<int>(vb / (NB * io.H_v));
  if (n >= io.N) return;
  if (io.order) n = io.order[n];  // longest sequences first: their chains start earliest
  const int hq = h / (io.H_v / io.H_qk);
  const int j = 16 * NW * half + 16 * w + l16;  // this lane's column of d_v
  const int64_t DD = static_cast<int64_t>(D) * D, CD = static_cast<int64_t>(C) * D;
  const int64_t nh = static_cast<int64_t>(n) * io.H_v + h;

  int64_t tok0 = 0, nsteps = 1, L = 0, slot0 = 0, fslot0 = 0, nchunks = 0;
  if (RESYNC) {
    if (io.pos[nh] != 0) return;
    fslot0 = n;
  } else {
    tok0 = io.cu[n];
    L = static_cast<int64_t>(io.cu[n + 1]) - tok0;
    if (L < 0 || tok0 < 0 || tok0 + L > io.T) return;
    nchunks = (L + C - 1) / C;
    nsteps = MODE == kAll ? nchunks : L / C;
    slot0 = io.cu_chunks[n];
    fslot0 = MODE == kAll ? slot0 : io.cu_full[n];
    if (slot0 + nchunks > io.max_state_slot || fslot0 + nsteps > io.max_full_slot) return;
  }
  // buffer offsets (bytes): lane part in a VGPR, wave-uniform part in an SGPR
  const uint32_t fj = 4u * static_cast<uint32_t>(4 * g * D + j);  // (row 4 g, column j) of [.][D]
  const uint32_t fq4 = 16u * static_cast<uint32_t>(g * D + j);     // (quad g, column j) in row quads
  const uint32_t kst = RESYNC ? static_cast<uint32_t>(io.H_qk) * D * 4u : 2 * D * 4u;  // key row stride
  // W staging: rows wr0 .. wr0 + NR - 1, column group wg (columns 32 (wg / 4)
  // + 4 (wg % 4) + 0..3 and + 16 + 0..3, elements 0..7 of the group)
  const int wg = tid & 15, wr0 = (tid >> 4) * NR;
  const uint32_t fw = 4u * static_cast<uint32_t>(wr0 * D + 32 * (wg >> 2) + 4 * (wg & 3));
  // K staging: key group kg (keys p = 32 (kg / 4) + 16 (e / 4) + 4 (kg % 4) +
  // e % 4 for e = 0..7) at columns KC kc .. KC kc + KC - 1, one 4 KC-byte load
  // per key (consecutive lanes take consecutive columns: coalesced).  In LDS
  // the group of row i sits at slot kg ^ ((i / 8) % 8): the writes (rows KC
  // apart in consecutive lanes) and the A-operand reads are both free of bank
  // conflicts.
  const int kg = tid / KCS, kc = tid % KCS;
  const uint32_t fk = static_cast<uint32_t>(32 * (kg >> 2) + 4 * (kg & 3)) * kst + 4u * KC * kc;
  const int kslot = kg ^ (((KC * kc) >> 3) & 7);  // the same for the thread's KC rows
  struct OpRes {
    brsrc_t rk, rw, ru;
    int64_t sh;
  };
  auto op_res = [&](int64_t c) {
    OpRes r;
    r.sh = (fslot0 + c) * io.H_v + h;
    const int rows = RESYNC ? C : static_cast<int>(L - c * C < C ? L - c * C : C);
    const float* kb = RESYNC ? io.khat + (static_cast<int64_t>(n) * C * io.H_qk + hq) * D
                             : io.khat + (static_cast<int64_t>(hq) * io.T + tok0 + c * C) * 2 * D;
    r.rk = make_rsrc(kb, static_cast<uint32_t>(rows) * kst);  // rows past the end read 0
    r.rw = make_rsrc(io.W + r.sh * CD, C * D * 4u);
    r.ru = make_rsrc(io.U + r.sh * CD, C * D * 4u);
    return r;
  };
  float pw[NR][8], pk[8][KC];
  float un[4][4];
  float gvn = 0.0f, glastn = 0.0f;
  auto load_w = [&](const OpRes& rs) {  // W rows wr0 + m, and G (element lane of every wave)
#pragma unroll
    for (int m = 0; m < NR; ++m)
#pragma unroll
      for (int hf = 0; hf < 2; ++hf) {
        const float4 x = ldbuf4(rs.rw, fw, static_cast<uint32_t>(m * D * 4 + 64 * hf));
        pw[m][4 * hf] = x.x, pw[m][4 * hf + 1] = x.y, pw[m][4 * hf + 2] = x.z, pw[m][4 * hf + 3] = x.w;
      }
    gvn = io.G[rs.sh * C + lane];
    glastn = io.G[rs.sh * C + C - 1];
  };
  auto load_k = [&](const OpRes& rs) {
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      const uint32_t so = static_cast<uint32_t>(16 * (e >> 2) + (e & 3)) * kst;
      if constexpr (KC == 4) {
        const float4 x = ldbuf4(rs.rk, fk, so);
        pk[e][0] = x.x, pk[e][1] = x.y, pk[e][2] = x.z, pk[e][3] = x.w;
      } else {
        const auto x = __builtin_amdgcn_raw_buffer_load_b64(rs.rk, fk, so, 0);
        pk[e][0] = __uint_as_float(x[0]), pk[e][1] = __uint_as_float(x[1]);
      }
    }
  };
  auto load_u = [&](const OpRes& rs, int m) {  // part m of 8: two of the U values
#pragma unroll
    for (int e = 0; e < 2; ++e) {
      const int pb = m / 2, r = 2 * (m % 2) + e;
      un[pb][r] = ldbuf(rs.ru, fj, static_cast<uint32_t>((16 * pb + r) * D * 4), static_cast<const float*>(nullptr));
    }
  };
  auto put_w = [&](int m) {  // W parts of row wr0 + m
    const Parts x = split8(pw[m]);
    uint32_t* d = &sW[(wr0 + m) * WR + 12 * wg];
#pragma unroll
    for (int q = 0; q < 3; ++q) *reinterpret_cast<u32x4_t*>(d + 4 * q) = x.p[q];
  };
  auto put_lam = [&]() { sLam[lane] = -expf(glastn - gvn); };  // every wave writes the row: no branch
  auto put_k = [&](int c, const Parts& y) {  // K^T parts of key column KC kc + c
    uint32_t* d = &sK[(KC * kc + c) * KR + 12 * kslot];
#pragma unroll
    for (int q = 0; q < 3; ++q) *reinterpret_cast<u32x4_t*>(d + 4 * q) = y.p[q];
  };
  auto k_col = [&](float (&x)[8], int c) {
#pragma unroll
    for (int e = 0; e < 8; ++e) x[e] = pk[e][c];
  };
  auto put_w_parts = [&](int m, const Parts& x) {  // W parts of row wr0 + m
    uint32_t* d = &sW[(wr0 + m) * WR + 12 * wg];
#pragma unroll
    for (int q = 0; q < 3; ++q) *reinterpret_cast<u32x4_t*>(d + 4 * q) = x.p[q];
  };
  auto tiles8 = [](float (&x)[8], v4f a, v4f b) {
#pragma unroll
    for (int e = 0; e < 4; ++e) x[e] = a[e], x[4 + e] = b[e];
  };

  // S^T tiles (i = 16 ib + 4 g + r, j)
  v4f st[8];
  {
    const float* src = RESYNC ? io.S_chunk + nh * DD : (io.h0 ? io.h0 + nh * DD : nullptr);
    const brsrc_t rs = make_rsrc(src ? src : io.W, src ? D * D * 4u : 0u);  // no h0: reads 0
#pragma unroll
    for (int ib = 0; ib < 8; ++ib)
#pragma unroll
      for (int r = 0; r < 4; ++r)
        st[ib][r] = ldbuf(rs, fj, static_cast<uint32_t>((16 * ib + r) * D * 4), static_cast<const float*>(nullptr));
  }
  auto store_state = [&](float* dst) {
    const brsrc_t rd = make_rsrc(dst, D * D * 4u);
#pragma unroll
    for (int ib = 0; ib < 8; ++ib)
#pragma unroll
      for (int r = 0; r < 4; ++r) stbuf(st[ib][r], rd, fj, static_cast<uint32_t>((16 * ib + r) * D * 4));
  };
  // a chunk-start state: row quads outside the all-chunks mode
  auto store_start_tile = [&](const brsrc_t& rd, int ib) {
    if constexpr (MODE != kAll) {
      stbuf4(st[ib], rd, fq4, static_cast<uint32_t>(ib) * 4 * D * 16);
    } else {
#pragma unroll
      for (int r = 0; r < 4; ++r) stbuf(st[ib][r], rd, fj, static_cast<uint32_t>((16 * ib + r) * D * 4));
    }
  };

  float glast = 0.0f;  // G at the end of the current chunk
  if (nsteps > 0) {    // chunk 0's W and lam to LDS, its K and U in registers
    const OpRes rs = op_res(0);
    load_w(rs);
    load_k(rs);
#pragma unroll
    for (int m = 0; m < 8; ++m) load_u(rs, m);
#pragma unroll
    for (int m = 0; m < NR; ++m) put_w(m);
    put_lam();
    glast = glastn;
    load_w(op_res(nsteps > 1 ? 1 : 0));  // chunk 1's W and G: to LDS during chunk 0's S' products
  }
  v4f dl[4];  // -Delta tiles (p = 16 pb + 4 g + r, j), started from -U
#pragma unroll
  for (int pb = 0; pb < 4; ++pb)
#pragma unroll
    for (int r = 0; r < 4; ++r) dl[pb][r] = -un[pb][r];
  Parts b = split8(st[0], st[1]);  // B parts of Delta's first k block
  __syncthreads();
  // A operands: part q of W rows 16 pb + l16 in k block kb, of K^T rows
  // 16 (4 h2 + t) + l16 in k block kp
  auto read_w = [&](u32x4_t (&x)[4], int kb, int q) {
#pragma unroll
    for (int pb = 0; pb < 4; ++pb)
      x[pb] = *reinterpret_cast<const u32x4_t*>(&sW[(16 * pb + l16) * WR + 12 * (4 * kb + g) + 4 * q]);
  };
  auto read_k = [&](u32x4_t (&x)[4], int kp, int h2, int q) {
#pragma unroll
    for (int t = 0; t < 4; ++t) {
      const int i = 16 * (4 * h2 + t) + l16;  // slot of group 4 kp + g in row i (see the K staging)
      x[t] = *reinterpret_cast<const u32x4_t*>(&sK[i * KR + 12 * ((4 * kp + g) ^ ((i >> 3) & 7)) + 4 * q]);
    }
  };
  // Each k block's products form one scheduling region with VALU work that
  // does not depend on them (B parts of a later block, a share of the operand
  // staging, the gam scaling of state tiles already used), one product to a
  // few VALU instructions, so that the matrix core and the VALU run side by
  // side.  Part 0 of a block's A operand is read one region ahead, parts 1
  // and 2 at the start of their region (part 0's products cover them).
  for (int64_t c = 0; c < nsteps; ++c) {
    const int64_t fs = fslot0 + c;
    const bool more = c + 1 < nsteps;
    const OpRes nres = op_res(more ? c + 1 : c);
    const brsrc_t rst = RESYNC ? make_rsrc(io.W, 0u)  // no chunk-start states in resync
                               : make_rsrc(io.states + ((slot0 + c) * io.H_v + h) * DD, D * D * 4u);
    const float gam = expf(glast);
    float nlam[4][4];
    u32x4_t a0[4];
    read_w(a0, 0, 0);
    __builtin_amdgcn_sched_barrier(0);
    // ---- -Delta = -U + W S^T, k = i (the four tiles' chains are
    // interleaved; each keeps its own k order)
#pragma unroll
    for (int kb = 0; kb < 4; ++kb) {
      u32x4_t a1[4], a2[4], an[4];
      read_w(a1, kb, 1);
      read_w(a2, kb, 2);
      if (kb + 1 < 4) read_w(an, kb + 1, 0);
      // the next block's B parts and, on some blocks, a column of chunk c's
      // K^T (its buffer was last read by chunk c - 1)
      Parts bn = b;
      if (kb % (4 / KC) == 0) {
        float xk[8], xb[8];
        k_col(xk, kb / (4 / KC));
        Parts pk2;
        if (kb + 1 < 4) {
          tiles8(xb, st[2 * kb + 2], st[2 * kb + 3]);
          split8x2(xb, xk, bn, pk2);
        } else {
          pk2 = split8(xk);
        }
        put_k(kb / (4 / KC), pk2);
      } else if (kb + 1 < 4) {
        bn = split8(st[2 * kb + 2], st[2 * kb + 3]);
      }
      // tiles 2 kb, 2 kb + 1 of the chunk-start state (a store, dropped in
      // resync) and two parts of chunk c + 1's U.  The all-chunks mode then
      // scales them by gam_C for S' here; the others store 16 bytes per lane
      // and scale past the next barrier, so that no write of a wide store's
      // data registers follows it closely.
      if (!RESYNC) {
        store_start_tile(rst, 2 * kb);
        store_start_tile(rst, 2 * kb + 1);
      }
      if constexpr (MODE == kAll) {
        st[2 * kb] = gam * st[2 * kb];
        st[2 * kb + 1] = gam * st[2 * kb + 1];
      }
      load_u(nres, 2 * kb);
      load_u(nres, 2 * kb + 1);
      if (kb == 3) {  // -lam of the chunk's rows, read beside the last block's products
#pragma unroll
        for (int pb = 0; pb < 4; ++pb)
#pragma unroll
          for (int r = 0; r < 4; ++r) nlam[pb][r] = sLam[16 * pb + 4 * g + r];
      }
#pragma unroll
      for (int bq = 0; bq < 3; ++bq)  // A part 0 with B parts 0..2, part 1 with 0..1, part 2 with 0
#pragma unroll
        for (int pb = 0; pb < 4; ++pb) dl[pb] = mfma_bf(a0[pb], b.p[bq], dl[pb]);
#pragma unroll
      for (int bq = 0; bq < 2; ++bq)
#pragma unroll
        for (int pb = 0; pb < 4; ++pb) dl[pb] = mfma_bf(a1[pb], b.p[bq], dl[pb]);
#pragma unroll
      for (int pb = 0; pb < 4; ++pb) dl[pb] = mfma_bf(a2[pb], b.p[0], dl[pb]);
      if (kb + 1 < 4) mfma_valu_pattern<24, 12>();
      else mfma_valu_pattern<24, 8>();
      __builtin_amdgcn_sched_barrier(0);
      b = bn;
#pragma unroll
      for (int pb = 0; pb < 4; ++pb) a0[pb] = an[pb];
    }
    if (MODE == kAll) {
      const brsrc_t rd = make_rsrc(io.Dl + (fs * io.H_v + h) * CD, C * D * 4u);
#pragma unroll
      for (int pb = 0; pb < 4; ++pb)
#pragma unroll
        for (int r = 0; r < 4; ++r) stbuf(-dl[pb][r], rd, fj, static_cast<uint32_t>((16 * pb + r) * D * 4));
    }
    // lam * Delta = (-lam) * (-Delta)
#pragma unroll
    for (int pb = 0; pb < 4; ++pb)
#pragma unroll
      for (int r = 0; r < 4; ++r) dl[pb][r] = dl[pb][r] * nlam[pb][r];
    __syncthreads();  // chunk c's K^T written; its W and lam read by every wave
    // ---- S'^T (i, j) = gam_C S^T + K^T (lam Delta), k = p (outside the
    // all-chunks mode tiles 0..3 are scaled by gam_C here, tiles 4..7 beside
    // the first products, into tiles 0..3)
    if constexpr (MODE != kAll) {
#pragma unroll
      for (int ib = 0; ib < 4; ++ib) st[ib] = gam * st[ib];
    }
    read_k(a0, 0, 0, 0);
    put_lam();  // chunk c + 1's (chunk c's was read before the barrier)
    glast = more ? glastn : glast;
    load_k(nres);  // chunk c + 1's K: to LDS during its Delta products
    Parts b0 = b, b1 = b;
    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
    for (int it = 0; it < 4; ++it) {  // k block kp, tiles 4 h2 .. 4 h2 + 3
      const int kp = it / 2, h2 = it % 2;
      u32x4_t a1[4], a2[4], an[4];
      read_k(a1, kp, h2, 1);
      read_k(a2, kp, h2, 2);
      if (it + 1 < 4) read_k(an, (it + 1) / 2, (it + 1) % 2, 0);
      // chunk c + 1's W rows (chunk c's was read before the barrier), with
      // the second block's B parts, and the next chunk's first B parts
      // (tiles 0..3 are final) and -U
      if (it == 0) {
        b0 = split8(dl[0], dl[1]);
        if constexpr (MODE != kAll) {
#pragma unroll
          for (int ib = 4; ib < 8; ++ib) st[ib] = gam * st[ib];
        }
      }
      const bool wrow = it % (4 / NR) == 0;
      if (it == 1 || it == 3) {
        float xb[8];
        if (it == 1) tiles8(xb, dl[2], dl[3]);
        else tiles8(xb, st[0], st[1]);
        Parts& pb2 = it == 1 ? b1 : b;
        if (wrow) {
          Parts pw2;
          split8x2(xb, pw[it / (4 / NR)], pb2, pw2);
          put_w_parts(it / (4 / NR), pw2);
        } else {
          pb2 = split8(xb);
        }
      } else if (wrow) {
        put_w(it / (4 / NR));
      }
      if (it == 2) {
#pragma unroll
        for (int pb = 0; pb < 4; ++pb)
#pragma unroll
          for (int r = 0; r < 4; ++r) dl[pb][r] = -un[pb][r];
      }
      const Parts& bb = kp == 0 ? b0 : b1;
#pragma unroll
      for (int bq = 0; bq < 3; ++bq)
#pragma unroll
        for (int t = 0; t < 4; ++t) st[4 * h2 + t] = mfma_bf(a0[t], bb.p[bq], st[4 * h2 + t]);
#pragma unroll
      for (int bq = 0; bq < 2; ++bq)
#pragma unroll
        for (int t = 0; t < 4; ++t) st[4 * h2 + t] = mfma_bf(a1[t], bb.p[bq], st[4 * h2 + t]);
#pragma unroll
      for (int t = 0; t < 4; ++t) st[4 * h2 + t] = mfma_bf(a2[t], bb.p[0], st[4 * h2 + t]);
      if (it + 1 < 4) mfma_valu_pattern<24, 12>();
      else mfma_valu_pattern<24, 8>();
      __builtin_amdgcn_sched_barrier(0);
#pragma unroll
      for (int t = 0; t < 4; ++t) a0[t] = an[t];
    }
    // chunk c + 2's W and G, issued where the wave waits at the barrier anyway
    // rather than among the products, where each memory instruction held up
    // the products behind it (to LDS during chunk c + 1's S' products)
    load_w(op_res(c + 2 < nsteps ? c + 2 : nsteps - 1));
    __syncthreads();  // chunk c's K^T read; chunk c + 1's W and lam written
  }

  if (RESYNC) {
    store_state(io.S_chunk + nh * DD);
    store_state(io.S_run + nh * DD);
    return;
  }
  const bool tail = (L % C) != 0;
  if (MODE == kAll && tail) {
    if (io.hT_tail) store_state(io.hT_tail + nh * DD);
    return;
  }
  if (tail) {
    {  // tail chunk start
      const brsrc_t rd = make_rsrc(io.states + ((slot0 + nsteps) * io.H_v + h) * DD, D * D * 4u);
#pragma unroll
      for (int ib = 0; ib < 8; ++ib) store_start_tile(rd, ib);
    }
    if (io.S_chunk) store_state(io.S_chunk + nh * DD);
  } else {
    if (io.hT) store_state(io.hT + nh * DD);
    if (io.S_chunk) {
      store_state(io.S_chunk + nh * DD);
      store_state(io.S_run + nh * DD);
    }
  }
  if (io.pos && half == 0 && tid == 0) io.pos[nh] = static_cast<int32_t>(L % C);
}

// ---------------------------------------------------------------------------
// B, part 1 on the matrix cores (d = 128, C = 64).  Same quantities as k_wy:
//   A_pr = beta_p * ((k_p . k_r) * exp(G_p - G_r))   (p > r)
//   [W | U] = (I + A)^-1 [diag(beta gam) K | diag(beta) V]
// The Gram matrix comes from v_mfma_f32_16x16x4_f32 (i-steps s = 0..31, lane
// group g supplying i = 32 g + s).  The solve is blocked by 16 rows: block
// row b starts from its right-hand side, subtracts A[b][c] Y[c] for the solved
// blocks c < b on the matrix cores (k-steps s = 0..3, group g supplying row
// 4 g + s of block c), then multiplies by the inverse of its unit lower
// triangular diagonal block, T_b = (I + A_bb)^-1, also on the matrix cores.
// Each T_b is formed once per chunk by forward substitution on the identity
// (row by row, each solved row broadcast across the wave with a shuffle).
// Wave w owns 64 columns: W[:, 64w..] for w < 2, U[:, 64(w-2)..] for w >= 2.
// Decode resync runs this same kernel.
template <int C, typename TIn, int MODE>
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(4))) void k_wy_mfma(ChunkIO io) {
  constexpr int D = 128;
  constexpr int KS = D + 4;  // row stride of sK
  constexpr int AS = C + 4;  // row stride of sA
  static_assert(C == 64, "tiling assumes C = 64");
  constexpr bool RESYNC = MODE == kResync;
  // A takes K's space once the Gram products have read K (34.5 KB of LDS per
  // block: four blocks per CU)
  static_assert(C * AS <= C * KS, "A fits in K's space");
  __shared__ __attribute__((aligned(16))) float sK[C * KS];
  float* sA = sK;
  __shared__ float sB[C], sG[C], sBG[C];
  const int tid = threadIdx.x, lane = tid & 63;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);  // wave index, uniform
  const int l16 = lane & 15, g = lane >> 4;
  int64_t item;
  int h;
  wy_item(io.H_v / io.H_qk, item, h);
  const int hq = h / (io.H_v / io.H_qk);
  int64_t tok0, slot;
  int L = C;
  if (MODE == kResync) {
    if (item >= io.N) return;
    const int n = static_cast<int>(item);
    if (io.pos[static_cast<int64_t>(n) * io.H_v + h] != 0) return;
    tok0 = static_cast<int64_t>(n) * C;
    slot = n;
  } else {
    slot = item;
    if (slot >= io.cu_full[io.N]) return;
    const int n = find_seq(io.cu_full, io.N, slot);
    tok0 = static_cast<int64_t>(io.cu[n]) + static_cast<int64_t>(slot - io.cu_full[n]) * C;
    if (MODE == kAll) {
      const int64_t rem = static_cast<int64_t>(io.cu[n + 1]) - tok0;
      L = rem < C ? static_cast<int>(rem) : C;
      if (L <= 0) return;
    }
  }
  if (tok0 < 0 || tok0 + L > io.T || slot >= io.max_slot) return;

  int64_t kst;
  const float* krow = key_rows<D, RESYNC>(io.khat, io.T, io.H_qk, hq, tok0, kst);
  const bool isW = w < 2;
  const int cbase = 64 * (w & 1);
  const TIn* v = static_cast<const TIn*>(io.v) + tok0 * io.H_v * D + static_cast<int64_t>(h) * D;
  // Every column of W and U is solved on its own, so which lane holds which
  // column is free: in a wave's tile ct, lane l16 holds column
  // cbase + 4 l16 + ct, i.e. a lane's four tiles are four adjacent columns,
  // read and written 16 (8) bytes at a time.  Right-hand-side sources, (row
  // 16 bi + 4 g + r, that column): V straight from memory for the U waves
  // (rows past a partial chunk's end are outside the buffer range and read
  // 0), K from LDS for the W waves below.
  const int col4 = cbase + 4 * l16;
  // K (and beta, g) are loaded first and V last: loads complete in order, so
  // the K staging below waits for K alone and V lands during the Gram products
  float bx = 0.0f, gx = 0.0f;
  if (tid < C) {
    const int pc = tid < L ? tid : L - 1;
    bx = io.beta[(tok0 + pc) * io.H_v + h];
    gx = io.g[(tok0 + pc) * io.H_v + h];
  }
  constexpr int NK = (C * (D / 4)) / 256;
  static_assert(NK * 256 == C * (D / 4), "whole rounds");
  float4 kx[NK];
#pragma unroll
  for (int e_ = 0; e_ < NK; ++e_) {
    const int e = tid + 256 * e_;
    const int p = e / (D / 4), i4 = e % (D / 4);
    const int pc = p < L ? p : L - 1;
    kx[e_] = *reinterpret_cast<const float4*>(krow + pc * kst + 4 * i4);
  }
  float rpre[4][4][4];
  if (!isW) {  // wave-uniform
    constexpr uint32_t ES = sizeof(TIn);
    const uint32_t rs = static_cast<uint32_t>(io.H_v) * D * ES;  // row stride, bytes
    const brsrc_t rv = make_rsrc(v, static_cast<uint32_t>(L - 1) * rs + D * ES);
    const uint32_t vo = static_cast<uint32_t>(4 * g) * rs + static_cast<uint32_t>(col4) * ES;
    // A partial chunk (only in the all-chunks mode) relies on the range check
    // for its missing rows, so there the row is part of the lane offset (the
    // hardware range-checks the lane offset, not the scalar one); a full chunk
    // keeps the row in the scalar offset.  The branch is uniform per block.
    const bool full = MODE != kAll || L == C;
#pragma unroll
    for (int bi = 0; bi < 4; ++bi)
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const uint32_t ro = static_cast<uint32_t>(16 * bi + r) * rs;
        const float4 x = ldbuf4in(rv, full ? vo : vo + ro, full ? ro : 0u, static_cast<const TIn*>(nullptr));
        rpre[bi][0][r] = x.x;
        rpre[bi][1][r] = x.y;
        rpre[bi][2][r] = x.z;
        rpre[bi][3][r] = x.w;
      }
  }
#pragma unroll
  for (int e_ = 0; e_ < NK; ++e_) {
    const int e = tid + 256 * e_;
    const int p = e / (D / 4), i4 = e % (D / 4);
    *reinterpret_cast<float4*>(sK + p * KS + 4 * i4) = sel4(p < L, kx[e_], float4{0.0f, 0.0f, 0.0f, 0.0f});
  }
  if (tid < C) {
    sB[tid] = tid < L ? bx : 0.0f;
    sBG[tid] = tid < L ? gx : 0.0f;  // raw g for now
  }
  __syncthreads();
  if (isW) {  // wave-uniform
#pragma unroll
    for (int bi = 0; bi < 4; ++bi)
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const float4 x = *reinterpret_cast<const float4*>(sK + (16 * bi + 4 * g + r) * KS + col4);
        rpre[bi][0][r] = x.x;
        rpre[bi][1][r] = x.y;
        rpre[bi][2][r] = x.z;
        rpre[bi][3][r] = x.w;
      }
  }
  if (tid == 0) {  // running sum of g, p ascending
    float acc = 0.0f;
    for (int p = 0; p < C; ++p) {
      acc = acc + sBG[p];
      sG[p] = acc;
    }
  }
  __syncthreads();
  if (tid < C) sBG[tid] = sB[tid] * expf(sG[tid]);
  // Gram tiles (row block rb, column block cb <= rb): rows p = 16 rb + 4 g + r,
  // columns r' = 16 cb + l16.  The ten lower tiles are spread 3/3/2/2 over the
  // waves; each tile's k-steps run in the same order whichever wave owns it.
  // Tiles above the diagonal block are never read.
  {
    constexpr int kTiles = 3;
    int trb[kTiles], tcb[kTiles];
    const int nt = w < 2 ? 3 : 2;
    if (w == 0) { trb[0] = 0; tcb[0] = 0; trb[1] = 3; tcb[1] = 3; trb[2] = 3; tcb[2] = 0; }
    else if (w == 1) { trb[0] = 1; tcb[0] = 1; trb[1] = 2; tcb[1] = 2; trb[2] = 3; tcb[2] = 1; }
    else if (w == 2) { trb[0] = 1; tcb[0] = 0; trb[1] = 3; tcb[1] = 2; trb[2] = 0; tcb[2] = 0; }
    else { trb[0] = 2; tcb[0] = 0; trb[1] = 2; tcb[1] = 1; trb[2] = 0; tcb[2] = 0; }
    v4f kk[kTiles];
#pragma unroll
    for (int t = 0; t < kTiles; ++t) kk[t] = v4f{0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
    for (int s4 = 0; s4 < 8; ++s4) {
#pragma unroll
      for (int t = 0; t < kTiles; ++t) {
        if (t >= nt) continue;
        const float4 a4 = *reinterpret_cast<const float4*>(sK + (16 * trb[t] + l16) * KS + 32 * g + 4 * s4);
        const float4 b4 = *reinterpret_cast<const float4*>(sK + (16 * tcb[t] + l16) * KS + 32 * g + 4 * s4);
        kk[t] = mfma4(a4.x, b4.x, kk[t]);
        kk[t] = mfma4(a4.y, b4.y, kk[t]);
        kk[t] = mfma4(a4.z, b4.z, kk[t]);
        kk[t] = mfma4(a4.w, b4.w, kk[t]);
      }
    }
    __syncthreads();  // every wave's Gram reads of K are done: A overwrites K
#pragma unroll
    for (int t = 0; t < kTiles; ++t) {
      if (t >= nt) continue;
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int p = 16 * trb[t] + 4 * g + r, q = 16 * tcb[t] + l16;
        // operands read and exp taken unconditionally: a select, not a branch
        const float gpq = expf(sG[p] - sG[q]);
        const float a = sB[p] * (kk[t][r] * gpq);
        sA[p * AS + q] = q < p ? a : 0.0f;
      }
    }
  }
  __syncthreads();
  // T_b = (I + A_bb)^-1 for the diagonal 16 x 16 blocks: wave w inverts block
  // w by forward substitution on the identity (pivot rows 0..14 in order; the
  // coefficients at or above the pivot are the diagonal tile's zeros), holding
  // T[4 g + r][l16] in register r, and stores it row-major in an upper tile of
  // A (those tiles are never read as A).
  constexpr int kTRow[4] = {0, 0, 0, 1}, kTCol[4] = {1, 2, 3, 2};
  {
    const int tb = w;
    v4f t;
#pragma unroll
    for (int r = 0; r < 4; ++r) t[r] = 4 * g + r == l16 ? 1.0f : 0.0f;
#pragma unroll
    for (int pp = 0; pp < 15; ++pp) {
      float a[4];
#pragma unroll
      for (int r = 0; r < 4; ++r) a[r] = sA[(16 * tb + 4 * g + r) * AS + 16 * tb + pp];
      const float y = __shfl(t[pp & 3], l16 + 16 * (pp >> 2), 64);
#pragma unroll
      for (int r = 0; r < 4; ++r) t[r] = fmaf(-a[r], y, t[r]);
    }
    const int trow = tb == 3 ? 1 : 0, tcol = tb == 3 ? 2 : tb + 1;
#pragma unroll
    for (int r = 0; r < 4; ++r) sA[(16 * trow + 4 * g + r) * AS + 16 * tcol + l16] = t[r];
  }
  __syncthreads();
  float* out = (isW ? io.W : io.U) + (slot * io.H_v + h) * static_cast<int64_t>(C) * D;
  v4f Y[4][4];  // [row block][column tile], accumulator layout
#pragma unroll
  for (int bi = 0; bi < 4; ++bi) {
    v4f acc[4];
#pragma unroll
    for (int ct = 0; ct < 4; ++ct)
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int p = 16 * bi + 4 * g + r;
        const float wv = sBG[p] * rpre[bi][ct][r], uv = sB[p] * rpre[bi][ct][r];
        acc[ct][r] = isW ? wv : uv;
      }
#pragma unroll
    for (int bj = 0; bj < bi; ++bj)
#pragma unroll
      for (int s4 = 0; s4 < 4; ++s4) {
        const float a = -sA[(16 * bi + l16) * AS + 16 * bj + 4 * g + s4];
#pragma unroll
        for (int ct = 0; ct < 4; ++ct) acc[ct] = mfma4(a, Y[bj][ct][s4], acc[ct]);
      }
    // the block's rows: Y_bi = T_bi (right-hand side - sum_bj A_bi,bj Y_bj) on
    // the matrix cores, k-steps r = 0..3 with lane group g supplying row 4 g + r
    {
      const float4 tl = *reinterpret_cast<const float4*>(sA + (16 * kTRow[bi] + l16) * AS +
                                                          16 * kTCol[bi] + 4 * g);
      v4f yv[4];
#pragma unroll
      for (int ct = 0; ct < 4; ++ct) yv[ct] = v4f{0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
      for (int ct = 0; ct < 4; ++ct) yv[ct] = mfma4(tl.x, acc[ct][0], yv[ct]);
#pragma unroll
      for (int ct = 0; ct < 4; ++ct) yv[ct] = mfma4(tl.y, acc[ct][1], yv[ct]);
#pragma unroll
      for (int ct = 0; ct < 4; ++ct) yv[ct] = mfma4(tl.z, acc[ct][2], yv[ct]);
#pragma unroll
      for (int ct = 0; ct < 4; ++ct) yv[ct] = mfma4(tl.w, acc[ct][3], yv[ct]);
#pragma unroll
      for (int ct = 0; ct < 4; ++ct) acc[ct] = yv[ct];
    }
#pragma unroll
    for (int ct = 0; ct < 4; ++ct) Y[bi][ct] = acc[ct];
#pragma unroll
    for (int r = 0; r < 4; ++r)
      *reinterpret_cast<float4*>(out + static_cast<int64_t>(16 * bi + 4 * g + r) * D + col4) =
          float4{acc[0][r], acc[1][r], acc[2][r], acc[3][r]};
  }
  if (tid < C) io.G[(slot * io.H_v + h) * C + tid] = sG[tid];
}

// ---------------------------------------------------------------------------
// R -- the token step, per lane = one row j (a d_v index) of the state, the
// row's d_k entries in registers s[0..D).  For a token with a = s . k (taken
// on the state before the token):
//   alpha = expf(g);  u = alpha * a;  delta = beta * (v_j - u)
//   s_i   = fmaf(delta, k_i, alpha * s_i)             i ascending
//   o_j   = sum_i s_i q_i  (fmaf chain from 0, i ascending, updated s)
// and the next token's a is the same kind of chain over the updated s.  The
// key and query vectors are wave-uniform operands.
template <int D, typename P>
__device__ __forceinline__ float row_dot(const float (&s)[D], P x) {
  float a = 0.0f;
#pragma unroll
  for (int i = 0; i < D; ++i) {
    a = fmaf(s[i], x[i], a);
    if ((i & 7) == 7) asm volatile("" : "+v"(a));  // keep operand reads in blocks
  }
  return a;
}

// The decode form of one token of R (same operations and order as k_rec's
// pass, without the next-token chain): s_i = fmaf(delta, k_i, alpha * s_i);
// o += s_i * q_i.  k, q are in LDS; reads are kept in blocks of 8 so the
// operands do not all become live at once.
template <int D>
__device__ __forceinline__ float r_update_lds(float (&s)[D], const float* k, const float* q,
                                              float alpha, float delta) {
  float o = 0.0f;
#pragma unroll
  for (int i = 0; i < D; ++i) {
    s[i] = fmaf(delta, k[i], alpha * s[i]);
    o = fmaf(s[i], q[i], o);
    if ((i & 7) == 7) {
      asm volatile("" : "+v"(o));
      __builtin_amdgcn_sched_barrier(0);
    }
  }
  return o;
}

// Operands of one RB-element block of a token: k_i, q_i and the next token's
// k_i, as wave-uniform scalar loads.
constexpr int RB = 16;
struct OpBlock {
  float k[RB], q[RB], n[RB];
};
template <int D>  // D: full head dimension (offset of q after k)
__device__ __forceinline__ void load_block(OpBlock& x, cfloat_p kq, cfloat_p kn, int b) {
#pragma unroll
  for (int r = 0; r < RB; ++r) {
    x.k[r] = kq[b * RB + r];
    x.q[r] = kq[D + b * RB + r];
    x.n[r] = kn[b * RB + r];
  }
}

// One token of R over a lane's row, operands as wave-uniform scalar loads:
//   s_i = fmaf(delta, k_i, alpha * s_i);  o += s_i * q_i;  an += s_i * kn_i,
// each chain in ascending i.  kq points at the token's [k | q] pair, kn at
// the next token's k.  The row is walked in blocks of RB elements (one
// scalar-load wait per block, so RB is as large as the SGPR file allows); at every
// block edge an empty asm pins the accumulator chains and a scheduling
// barrier stops the compiler from hoisting more scalar loads than the SGPR
// file holds.  Neither changes any operation or its order.  (Prefetching a
// block ahead measured slower: scalar loads complete out of order, so every
// wait is an all-outstanding wait.)  After each block's wait the pass
// touches the next token's query line and the key line two tokens ahead
// (p0, p1; folded into `sink` one block later, so the next block's wait
// retires them): the following tokens' operand loads then hit the scalar
// cache.  With SPREAD (four waves share the stream: two value heads, two
// row parts) each of them touches only the lines of block toff / RB, once
// per token: every line is still touched, with a quarter of the requests to
// the scalar cache that all the waves share.  The reads stay inside the prep
// buffer's two spare token rows.
template <int DK, int D, bool SPREAD>  // DK: elements of the row this lane holds; D: head dimension
__device__ __forceinline__ void r_token_pass(float (&s)[DK], cfloat_p kq, cfloat_p kn, float alpha,
                                             float delta, float& o, float& an, uint32_t& p0,
                                             uint32_t& p1, uint32_t& sink, int toff) {
  constexpr int NB = DK / RB;
  static_assert(DK % RB == 0, "row part must be whole operand blocks");
#pragma unroll
  for (int b = 0; b < NB; ++b) {
    OpBlock x;
    load_block<D>(x, kq, kn, b);
    {
      const int i = b * RB;
      s[i] = fmaf(delta, x.k[0], alpha * s[i]);
      o = fmaf(s[i], x.q[0], o);
      an = fmaf(s[i], x.n[0], an);
    }
    __builtin_amdgcn_sched_barrier(0);
    if (!SPREAD || b == 0) {  // (SPREAD: the waves sharing the stream split its lines)
      sink ^= p0 ^ p1;
      p0 = __float_as_uint(kq[2 * D + D + (SPREAD ? toff : b * RB)]);
      p1 = __float_as_uint(kq[4 * D + (SPREAD ? toff : b * RB)]);
    }
    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
    for (int r = 1; r < RB; ++r) {
      const int i = b * RB + r;
      s[i] = fmaf(delta, x.k[r], alpha * s[i]);
      o = fmaf(s[i], x.q[r], o);
      an = fmaf(s[i], x.n[r], an);
    }
    asm volatile("" : "+v"(o), "+v"(an));
    __builtin_amdgcn_sched_barrier(0);
  }
}

struct RecIO {
  const float* qk;   // prep layout [H_qk][T][2][D]
  const void* v;
  const float* beta;
  const float* g;
  const float* gb;   // (g, beta) per value head in token order [H_v][T][2]
  const int32_t* cu;
  const int32_t* cu_chunks;
  const float* states;  // prefill at d = 128: row quads
  float* o;
  float* hT;       // nullable
  // cache (nullable): the tail chunk leaves its running state and tokens
  float* S_run;
  float* kbuf;
  void* vbuf;
  float* bbuf;
  float* gbuf;
  int N, H_qk, H_v;
  int64_t T, max_state_slot;
};

// How the token step splits a head's state over waves: 64-row parts of d_v
// (one row per lane) and, at d = 128, two 64-element halves of d_k.  With the
// d_k split, every dot product of R is the sum of two partial chains,
//   x = chain(i = 0 .. 63) + chain(i = 64 .. 127),
// each an ascending fmaf chain from 0; the wave pair holding the two halves of
// the same rows exchanges its partials through LDS.  The decode step forms
// the same two chains and the same sum.
template <int D>
struct RowSplit {
  static constexpr int NH = (D + 63) / 64;   // row parts
  static constexpr int KS = D >= 128 ? 2 : 1; // d_k parts
  static constexpr int DK = D / KS;          // elements per lane
  static constexpr int WPH = NH * KS;        // waves per value head
};

// Blocks over (chunk, q/k head, z): each block holds `hpb` value heads of the
// group (waves = hpb * waves per head, at most 8), so the waves that read the
// same key/query stream share a CU and its scalar cache; blockIdx.z continues
// a group of more heads.  Wave (head, row part, d_k part) = index within the
// block in that order, d_k part fastest.
template <int D, int C, typename TIn, bool SPREAD, bool QUAD>  // QUAD: states in row quads
__global__ __launch_bounds__(512) __attribute__((amdgpu_waves_per_eu(6))) void k_rec(RecIO io, int hpb) {
  using RS = RowSplit<D>;
  constexpr int DK = RS::DK, KS = RS::KS, NH = RS::NH;
  constexpr int NW = 8 / KS;       // (head, row part) pairs per block, at most
  __shared__ float xa[2][8][64];  // partial dots (parity, wave, lane)
  __shared__ float xo[2][8][64];
  // the chunk's v rows of each (head, row part); fp32 values at d = 128 are
  // staged half a chunk at a time so that three blocks fit a CU's LDS
  constexpr int SC = (sizeof(TIn) == 4 && D == 128) ? C / 2 : C;
  __shared__ TIn sv[NW][SC][64];
  __shared__ float2 sgb[8][C];  // (g, beta) of the block's heads, token order
  const int slot = blockIdx.x;
  const int wl = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int wv = blockIdx.z * hpb * RS::WPH + wl;
  const int kh = wv % KS, rh = (wv / KS) % NH;
  const int G = io.H_v / io.H_qk;
  const int h = blockIdx.y * G + wv / RS::WPH;
  const int wp = wl / KS;  // (head, row part) pair within the block
  const int toff = SPREAD ? (wp & 3) * RB : 0;  // the touch lines of this wave (SPREAD)
  const int lane = threadIdx.x & 63;
  const int j = rh * 64 + lane;
  const bool act = D % 64 == 0 || j < D;
  if (slot >= io.cu_chunks[io.N] || slot >= io.max_state_slot) return;  // whole block
  const int n = find_seq(io.cu_chunks, io.N, slot);
  const int hq = h / G;
  const int64_t c = slot - io.cu_chunks[n];
  const int64_t tok0 = static_cast<int64_t>(io.cu[n]) + c * C;
  const int64_t end = io.cu[n + 1];
  if (tok0 < 0 || end > io.T || tok0 >= end) return;  // whole block
  const int L = static_cast<int>(end - tok0 < C ? end - tok0 : C);
  const int64_t DD = static_cast<int64_t>(D) * D;
  const int vs = io.H_v * D;  // < 2^20 (host-checked)
  const int i0 = kh * DK;     // first d_k element of this wave
  // Token operands of the chunk: g and beta from LDS (one broadcast read per
  // token, so that the scalar cache serves only the key/query stream), v from
  // LDS, o through a buffer resource over the chunk's rows (lane offset in a
  // VGPR, token offset in an SGPR).
  float* obase = io.o + (tok0 * io.H_v + h) * D;
  const uint32_t otok = static_cast<uint32_t>(vs) * 4u;
  const brsrc_t orr = make_rsrc(obase, static_cast<uint32_t>(L - 1) * otok + D * 4u);
  // inactive lanes (D < 64) read row 0 and store nothing; buffer offsets are
  // the lane's part in a VGPR and the row part's and token's in an SGPR
  const int jc = act ? j : 0;
  const uint32_t lo4 = static_cast<uint32_t>(lane) * 4u;
  const uint32_t ro = static_cast<uint32_t>(rh * 64) * 4u;
  {  // stage v: pair q of the block is (head q / NH of the block, row part q % NH)
    const int npair = static_cast<int>(blockDim.x >> 6) / KS;
    const TIn* vin = static_cast<const TIn*>(io.v);
    const int hb = blockIdx.y * G + blockIdx.z * hpb;  // first head of the block
    for (int e = threadIdx.x; e < npair * SC * 64; e += blockDim.x) {
      const int q = e / (SC * 64), tt = (e / 64) % SC, ll = e % 64;
      const int row = (q % NH) * 64 + ll;
      const int tc = tt < L ? tt : L - 1;
      sv[q][tt][ll] = row < D ? vin[(tok0 + tc) * io.H_v * D + static_cast<int64_t>(hb + q / NH) * D + row]
                              : TIn(0);
    }
    for (int e = threadIdx.x; e < hpb * C; e += blockDim.x) {
      const int hh = e / C, tt = e % C;
      const int tc = tt < L ? tt : L - 1;
      sgb[hh][tt] = *reinterpret_cast<const float2*>(io.gb + ((static_cast<int64_t>(hb + hh) * io.T) + tok0 + tc) * 2);
    }
  }
  __syncthreads();
  const int hl = wl / RS::WPH;  // the wave's head within the block

  float s[DK];
  const float* st = io.states + (static_cast<int64_t>(slot) * io.H_v + h) * DD;
  if constexpr (QUAD) {  // rows i0 + 4 m .. + 3 of column jc in 16 bytes
#pragma unroll
    for (int m = 0; m < DK / 4; ++m) {
      const float4 x = *reinterpret_cast<const float4*>(st + (static_cast<int64_t>(i0 / 4 + m) * D + jc) * 4);
      s[4 * m] = x.x, s[4 * m + 1] = x.y, s[4 * m + 2] = x.z, s[4 * m + 3] = x.w;
    }
  } else {
#pragma unroll
    for (int i = 0; i < DK; ++i) s[i] = st[static_cast<int64_t>(i0 + i) * D + jc];
  }

  // key (t) / query (t) / key (t+1) streams, 2*D floats per token
  cfloat_p kq = as_const(io.qk + (static_cast<int64_t>(hq) * io.T + tok0) * 2 * D + i0);
  float a = row_dot<DK>(s, kq);
  if constexpr (KS == 2) {
    xa[1][wl][lane] = a;
    __syncthreads();
    a = a + xa[1][wl ^ 1][lane];
  }
  // g, beta and v are loaded one token ahead; the last token reloads itself
  // rather than reading past the chunk
  uint32_t pp0 = 0, pp1 = 0, psink = 0;
  float gn = sgb[hl][0].x, bn = sgb[hl][0].y, vn = ldin(&sv[wp][0][lane]);
  for (int t = 0; t < L; ++t) {
    const float alpha = expf(gn);
    const float b = bn;
    const float vj = vn;
    const int tn = t + 1 < L ? t + 1 : t;
    {
      const float2 x = sgb[hl][tn];
      gn = x.x;
      bn = x.y;
    }
    if constexpr (SC < C) {
      // the second half: every wave read its last first-half row (token SC - 1)
      // one token ahead, before the previous token's exchange barrier
      if (t == SC - 1 && L > SC) {  // tokens SC .. C - 1 (past the end: the last)
        const int npair = static_cast<int>(blockDim.x >> 6) / KS;
        const TIn* vin = static_cast<const TIn*>(io.v);
        const int hb = blockIdx.y * G + blockIdx.z * hpb;
        for (int e = threadIdx.x; e < npair * SC * 64; e += blockDim.x) {
          const int q = e / (SC * 64), tt = (e / 64) % SC, ll = e % 64;
          const int row = (q % NH) * 64 + ll;
          const int tc = SC + tt < L ? SC + tt : L - 1;
          sv[q][tt][ll] = row < D ? vin[(tok0 + tc) * io.H_v * D +
                                        static_cast<int64_t>(hb + q / NH) * D + row]
                                  : TIn(0);
        }
        __syncthreads();
      }
      vn = ldin(&sv[wp][tn >= SC ? tn - SC : tn][lane]);
    } else {
      vn = ldin(&sv[wp][tn][lane]);
    }
    const float u = alpha * a;
    const float delta = b * (vj - u);
    cfloat_p kn = kq + 2 * D;  // past the chunk's end on its last token: read, never used
    float o = 0.0f, an = 0.0f;
    r_token_pass<DK, D, SPREAD>(s, kq, kn, alpha, delta, o, an, pp0, pp1, psink, toff);
    if constexpr (KS == 2) {
      const int par = t & 1;  // a slot is rewritten two barriers after it was read
      xa[par][wl][lane] = an;
      xo[par][wl][lane] = o;
      __syncthreads();
      an = an + xa[par][wl ^ 1][lane];
      o = o + xo[par][wl ^ 1][lane];
    }
    if (act && kh == 0) stbuf(o, orr, lo4, static_cast<uint32_t>(t) * otok + ro);
    a = an;
    kq += 2 * D;
    // opaque to the optimizer: otherwise it forwards this token's kn loads to
    // the next token's k loads and must keep the values live across iterations
    asm volatile("" : "+s"(kq));
  }
  asm volatile("" :: "s"(psink ^ pp0 ^ pp1));
  if (L == C) return;
  // tail chunk: the running state is the sequence's final state, and the
  // partial chunk's tokens go to the decode buffers
  const int64_t nh = static_cast<int64_t>(n) * io.H_v + h;
  if (act && io.hT) {
#pragma unroll
    for (int i = 0; i < DK; ++i) io.hT[nh * DD + static_cast<int64_t>(i0 + i) * D + j] = s[i];
  }
  if (!io.S_run) return;
  if (act) {
#pragma unroll
    for (int i = 0; i < DK; ++i) io.S_run[nh * DD + static_cast<int64_t>(i0 + i) * D + j] = s[i];
  }
  if (kh != 0) return;
  TIn* vb = static_cast<TIn*>(io.vbuf);
  const TIn* vin = static_cast<const TIn*>(io.v);
  for (int t = 0; t < L; ++t) {
    const int64_t tk = tok0 + t;
    const int64_t bi = static_cast<int64_t>(n) * C + t;
    if (act) {
      vb[(bi * io.H_v + h) * D + j] = vin[(tk * io.H_v + h) * D + j];
      if (h % G == 0)
        io.kbuf[(bi * io.H_qk + hq) * D + j] =
            io.qk[((static_cast<int64_t>(hq) * io.T + tk) * 2) * D + j];
    }
    if (j == 0) {
      io.bbuf[bi * io.H_v + h] = io.beta[tk * io.H_v + h];
      io.gbuf[bi * io.H_v + h] = io.g[tk * io.H_v + h];
    }
  }
}

// ---------------------------------------------------------------------------
// Decode token step: one block of max(D, 64) lanes per (sequence, value
// head); lane j owns row j.  Wave 0 normalises the token's q and k with
// l2norm_wave (same bits as k_prep), then every lane runs R on its row of
// S_run, exactly as k_rec does, and the token is appended to the chunk
// buffers.  pos advances; it wraps to 0 when the chunk is complete, which is
// what the resync launches test.
struct DecIO {
  const void* q;
  const void* k;
  const void* v;
  const float* beta;
  const float* g;
  float* o;
  float* S_run;
  float* kbuf;
  void* vbuf;
  float* bbuf;
  float* gbuf;
  int32_t* pos;
  int N, H_qk, H_v, l2;
  float scale;
};

// One decode token per (sequence, value head) block; waves split the state as
// in k_rec (row parts, and d_k halves at d = 128, whose partial dots are
// summed in the same order).  CPR = false is the plain recurrent decode of the
// native-mixed baseline: the same token step on S_run, no chunk buffers, no
// position, no resync.
template <int D, int C, typename TIn, bool CPR = true>
__global__ __launch_bounds__(256) void k_decode(DecIO io) {
  using RS = RowSplit<D>;
  constexpr int DK = RS::DK, KS = RS::KS;
  static_assert(RS::WPH <= 4, "one block of at most 4 waves per head");
  __shared__ float sq[D < 64 ? 64 : D];
  __shared__ float sk[D < 64 ? 64 : D];
  __shared__ float xa[4][64];
  __shared__ float xo[4][64];
  const int n = blockIdx.x;
  const int h = blockIdx.y;
  const int wl = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int kh = wl % KS, rh = wl / KS;
  const int lane = threadIdx.x & 63;
  const int j = rh * 64 + lane;
  const bool act = j < D;
  const int G = io.H_v / io.H_qk;
  const int hq = h / G;
  const int64_t nh = static_cast<int64_t>(n) * io.H_v + h;
  const int64_t DD = static_cast<int64_t>(D) * D;
  const int i0 = kh * DK;
  int p = 0;
  if constexpr (CPR) {
    p = io.pos[nh];
    p = p < 0 ? 0 : (p >= C ? C - 1 : p);
  }
  if (threadIdx.x < 64) {
    const TIn* q = static_cast<const TIn*>(io.q) + (static_cast<int64_t>(n) * io.H_qk + hq) * D;
    const TIn* k = static_cast<const TIn*>(io.k) + (static_cast<int64_t>(n) * io.H_qk + hq) * D;
    float y0, y1;
    l2norm_wave<D>(q, io.scale, io.l2, y0, y1);
    if (lane < D) sq[lane] = y0;
    if (D > 64) sq[lane + 64] = y1;
    l2norm_wave<D>(k, 1.0f, io.l2, y0, y1);
    if (lane < D) sk[lane] = y0;
    if (D > 64) sk[lane + 64] = y1;
  }
  const int jc = act ? j : 0;
  float s[DK];
  float* sr = io.S_run + nh * DD;
#pragma unroll
  for (int i = 0; i < DK; ++i) s[i] = sr[static_cast<int64_t>(i0 + i) * D + jc];
  __syncthreads();
  const TIn* v = static_cast<const TIn*>(io.v);
  const float gt = io.g[nh];
  const float alpha = expf(gt);
  const float b = io.beta[nh];
  const float vj = ldin(v + nh * D + jc);
  float a = row_dot<DK>(s, static_cast<const float*>(sk) + i0);
  if constexpr (KS == 2) {
    xa[wl][lane] = a;
    __syncthreads();
    a = a + xa[wl ^ 1][lane];
  }
  const float u = alpha * a;
  const float delta = b * (vj - u);
  float o = r_update_lds<DK>(s, sk + i0, sq + i0, alpha, delta);
  if constexpr (KS == 2) {
    xo[wl][lane] = o;
    __syncthreads();
    o = o + xo[wl ^ 1][lane];
  }
  if (act) {
#pragma unroll
    for (int i = 0; i < DK; ++i) sr[static_cast<int64_t>(i0 + i) * D + j] = s[i];
    if (kh == 0) {
      io.o[nh * D + j] = o;
      if constexpr (CPR) {
        const int64_t bt = static_cast<int64_t>(n) * C + p;
        static_cast<TIn*>(io.vbuf)[(bt * io.H_v + h) * D + j] = v[nh * D + j];
        if (h % G == 0) io.kbuf[(bt * io.H_qk + hq) * D + j] = sk[j];
        if (j == 0) {
          io.bbuf[bt * io.H_v + h] = b;
          io.gbuf[bt * io.H_v + h] = gt;
        }
      }
    }
  }
  if constexpr (CPR) {
    __syncthreads();  // every lane has read pos
    if (threadIdx.x == 0) io.pos[nh] = (p + 1 == C) ? 0 : p + 1;
  }
}

// ---------------------------------------------------------------------------
// Backward (gdn_fwd_bwd).  The gradient of the layer as a function, computed
// through its chunk form (the forward's chunk factors W, U, G, its
// chunk-start states S and Delta = U - W S^T are kept from the forward).  Per
// chunk of L rows (padded to C with zero rows), P = (Q K^T) . Gam (r <= p),
// Gam_pr = exp(G_p - G_r), gam_p = exp(G_p), lam_p = exp(G_last - G_p), and
// dS' the gradient of the state at the chunk's end:
//   dDelta = P^T dO + diag(lam) K dS'^T
//   dS     = gam_last dS' + sum_p gam_p dO_p q_p^T - sum_p dDelta_p W_p^T
// (the reverse scan over chunks), then per chunk the gradients of q, k, v,
// beta and g through O, the state update and the WY solve.  No atomics; every
// sum has a fixed order, so the result is reproducible bit for bit.
struct BwdIO {
  const float* qk;        // prep layout [H_qk][T][2][D] (k-hat, q-hat)
  const void* q;          // raw inputs (norm backward)
  const void* k;
  const void* v;
  const float* beta;
  const float* g;
  const float* dO;        // [T][H_v][D]
  const float* dhT;       // nullable [N][H_v][D][D]
  const int32_t* cu;
  const int32_t* cu_chunks;
  const float* W;         // [slot][H_v][C][D]
  const float* U;
  const float* G;         // [slot][H_v][C]
  const float* states;    // [slot][H_v][D][D] chunk-start states (stored layout)
  const float* Dl;        // [slot][H_v][C][D] Delta
  float* E;               // [slot][H_v][C][D] P^T dO
  float* dstates;         // [slot][H_v][D][D] gradient of each chunk's end state
  float* dD;              // [slot][H_v][C][D] dDelta, then dX_u
  // d = 16 only (the d = 128 chunk kernel forms these itself; null there):
  float* SdO;             // [slot][H_v][C][D] S^T dO_p
  float* DsD;             // [slot][H_v][C][D] dS'^T Delta_p
  float* SdD;             // [slot][H_v][C][D] S^T dDelta_p, then dX_w
  float* dqv;             // [T][H_v][D] per value head
  float* dkv;             // [T][H_v][D]
  void* dv;               // [T][H_v][D], fp32 or (grad_bf16) bf16
  float* dbeta;           // [T][H_v]
  float* dg;              // [T][H_v]
  void* dq;               // [T][H_qk][D], fp32 or (grad_bf16) bf16
  void* dk;
  float* dh0;             // [N][H_v][D][D]
  int N, H_qk, H_v, l2;
  int grad_bf16;          // dq, dk, dv as bf16 (round to nearest even)
  float scale;
  int64_t T, max_state_slot;
};

// Element i of a gradient output: fp32, or bf16 rounded to nearest even from
// the fp32 value (a NaN stays a NaN).
__device__ __forceinline__ void st_grad(void* base, int64_t i, float x, int bf16) {
  if (bf16) {
    const uint32_t u = __float_as_uint(x);
    const uint32_t r = (u & 0x7fffffffu) > 0x7f800000u ? (u >> 16) | 0x40u
                                                        : (u + 0x7fffu + ((u >> 16) & 1u)) >> 16;
    static_cast<uint16_t*>(base)[i] = static_cast<uint16_t>(r);
  } else {
    static_cast<float*>(base)[i] = x;
  }
}

// Chunk item of a backward kernel over every chunk and value head, grid
// (8 G ceil(chunks / 8), H_qk) grouped as the chunk factors' (the value heads
// of a q/k group, which read the same q-hat and k-hat rows, 8 blocks apart).
template <int C>
__device__ __forceinline__ bool bwd_item(const BwdIO& io, int64_t& slot, int& h, int64_t& tok0, int& L) {
  wy_item(io.H_v / io.H_qk, slot, h);
  if (slot >= io.cu_chunks[io.N] || slot >= io.max_state_slot) return false;
  const int n = find_seq(io.cu_chunks, io.N, slot);
  tok0 = static_cast<int64_t>(io.cu[n]) + (slot - io.cu_chunks[n]) * C;
  const int64_t end = io.cu[n + 1];
  if (tok0 < 0 || end > io.T || tok0 >= end) return false;
  L = static_cast<int>(end - tok0 < C ? end - tok0 : C);
  return true;
}

// E = P^T dO for one chunk and value head.
template <int D, int C>
__global__ __launch_bounds__(256) void k_bwd_prep(BwdIO io) {
  constexpr int NT = 256;
  __shared__ float sQ[C][D + 1];
  __shared__ float sK[C][D + 1];
  __shared__ float sP[C][C + 1];
  __shared__ float sG[C];
  int64_t slot, tok0;
  int L, h;
  if (!bwd_item<C>(io, slot, h, tok0, L)) return;
  const int tid = threadIdx.x, hq = h / (io.H_v / io.H_qk);
  const float* kq = io.qk + (static_cast<int64_t>(hq) * io.T + tok0) * 2 * D;
  for (int e = tid; e < C * D; e += NT) {
    const int p = e / D, i = e % D;
    sK[p][i] = p < L ? kq[p * 2 * D + i] : 0.0f;
    sQ[p][i] = p < L ? kq[p * 2 * D + D + i] : 0.0f;
  }
  if (tid < C) sG[tid] = io.G[(slot * io.H_v + h) * C + tid];
  __syncthreads();
  for (int e = tid; e < C * C; e += NT) {
    const int p = e / C, r = e % C;
    float x = 0.0f;
    if (r <= p && p < L) {
      float d = 0.0f;
      for (int i = 0; i < D; ++i) d = fmaf(sQ[p][i], sK[r][i], d);
      x = d * expf(sG[p] - sG[r]);
    }
    sP[p][r] = x;
  }
  __syncthreads();
  const float* dO = io.dO + (tok0 * io.H_v + h) * D;
  float* E = io.E + (slot * io.H_v + h) * static_cast<int64_t>(C) * D;
  for (int e = tid; e < C * D; e += NT) {
    const int r = e / D, j = e % D;
    float acc = 0.0f;
    for (int p = r; p < L; ++p) acc = fmaf(sP[p][r], dO[static_cast<int64_t>(p) * io.H_v * D + j], acc);
    E[e] = acc;
  }
}

// Reverse scan of the state gradient over the chunks of a sequence, for a
// tile of TILE rows (d_v indices) -- rows are independent here too.
template <int D, int C, int TILE>
__global__ __launch_bounds__(256) void k_bwd_scan(BwdIO io) {
  constexpr int NT = 256;
  constexpr int NTILE = D / TILE;
  __shared__ float sS[TILE][D + 1];  // dS' rows: sS[jj][i] = stored[i][j0 + jj]
  __shared__ float sK[C][D];
  __shared__ float sQ[C][D];
  __shared__ float sW[C][D];
  __shared__ float sDD[C][TILE + 1];
  __shared__ float sO[C][TILE + 1];
  __shared__ float sG[C];
  const int tid = threadIdx.x;
  const int tile = blockIdx.x % NTILE;
  const int h = (blockIdx.x / NTILE) % io.H_v;
  const int n = blockIdx.x / (NTILE * io.H_v);
  if (n >= io.N) return;
  const int hq = h / (io.H_v / io.H_qk);
  const int j0 = tile * TILE;
  const int64_t DD = static_cast<int64_t>(D) * D;
  const int64_t nh = static_cast<int64_t>(n) * io.H_v + h;
  const int64_t s0 = io.cu[n];
  const int64_t Lseq = static_cast<int64_t>(io.cu[n + 1]) - s0;
  if (Lseq < 0 || s0 < 0 || s0 + Lseq > io.T) return;
  const int64_t nchunks = (Lseq + C - 1) / C;
  const int64_t slot0 = io.cu_chunks[n];
  if (slot0 + nchunks > io.max_state_slot) return;

  for (int e = tid; e < TILE * D; e += NT) {
    const int i = e / TILE, jj = e % TILE;
    sS[jj][i] = io.dhT ? io.dhT[nh * DD + static_cast<int64_t>(i) * D + j0 + jj] : 0.0f;
  }
  __syncthreads();
  for (int64_t c = nchunks - 1; c >= 0; --c) {
    const int64_t slot = slot0 + c;
    const int64_t tok0 = s0 + c * C;
    const int rows = static_cast<int>(Lseq - c * C < C ? Lseq - c * C : C);
    float* dst = io.dstates + (slot * io.H_v + h) * DD;
    for (int e = tid; e < TILE * D; e += NT) {
      const int i = e / TILE, jj = e % TILE;
      dst[static_cast<int64_t>(i) * D + j0 + jj] = sS[jj][i];
    }
    const float* kq = io.qk + (static_cast<int64_t>(hq) * io.T + tok0) * 2 * D;
    const float* Wc = io.W + (slot * io.H_v + h) * static_cast<int64_t>(C) * D;
    for (int e = tid; e < C * D; e += NT) {
      const int p = e / D, i = e % D;
      sK[p][i] = p < rows ? kq[p * 2 * D + i] : 0.0f;
      sQ[p][i] = p < rows ? kq[p * 2 * D + D + i] : 0.0f;
      sW[p][i] = Wc[e];
    }
    if (tid < C) sG[tid] = io.G[(slot * io.H_v + h) * C + tid];
    __syncthreads();
    for (int e = tid; e < C * TILE; e += NT) {
      const int p = e / TILE, jj = e % TILE;
      sO[p][jj] = p < rows ? expf(sG[p]) * io.dO[((tok0 + p) * io.H_v + h) * D + j0 + jj] : 0.0f;
    }
    const float glast = sG[C - 1];
    const float* Ec = io.E + (slot * io.H_v + h) * static_cast<int64_t>(C) * D;
    float* dDc = io.dD + (slot * io.H_v + h) * static_cast<int64_t>(C) * D;
    for (int e = tid; e < C * TILE; e += NT) {
      const int p = e / TILE, jj = e % TILE;
      float d = 0.0f;
      for (int i = 0; i < D; ++i) d = fmaf(sK[p][i], sS[jj][i], d);
      const float x = Ec[static_cast<int64_t>(p) * D + j0 + jj] + expf(glast - sG[p]) * d;
      sDD[p][jj] = x;
      dDc[static_cast<int64_t>(p) * D + j0 + jj] = x;
    }
    __syncthreads();
    const float gl = expf(glast);
    for (int e = tid; e < TILE * D; e += NT) {
      const int jj = e / D, i = e % D;
      float acc = gl * sS[jj][i];
      for (int p = 0; p < C; ++p) acc = fmaf(sO[p][jj], sQ[p][i], acc);
      for (int p = 0; p < C; ++p) acc = fmaf(-sDD[p][jj], sW[p][i], acc);
      sS[jj][i] = acc;
    }
    __syncthreads();
  }
  for (int e = tid; e < TILE * D; e += NT) {
    const int i = e / TILE, jj = e % TILE;
    io.dh0[nh * DD + static_cast<int64_t>(i) * D + j0 + jj] = sS[jj][i];
  }
}

// The three state products of a chunk: out_p[i] = sum_j X[i][j] Y_p[j] for
// (X, Y) = (S, dO) -> SdO, (S, dDelta) -> SdD, (dS', Delta) -> DsD.
template <int D, int C>
__global__ __launch_bounds__(256) void k_bwd_mm(BwdIO io) {
  constexpr int NT = 256;
  __shared__ float sM[D][D + 1];
  __shared__ float sY[C][D + 1];
  int64_t slot, tok0;
  int L, h;
  if (!bwd_item<C>(io, slot, h, tok0, L)) return;
  const int tid = threadIdx.x;
  const int64_t DD = static_cast<int64_t>(D) * D;
  const int64_t CD = static_cast<int64_t>(C) * D;
  const int64_t sh = slot * io.H_v + h;
  for (int prod = 0; prod < 3; ++prod) {
    if (prod != 1) {
      const float* X = (prod == 0 ? io.states : io.dstates) + sh * DD;
      for (int e = tid; e < D * D; e += NT) sM[e / D][e % D] = X[e];
    }
    for (int e = tid; e < C * D; e += NT) {
      const int p = e / D, j = e % D;
      float y = 0.0f;
      if (p < L) {
        if (prod == 0) y = io.dO[((tok0 + p) * io.H_v + h) * D + j];
        else if (prod == 1) y = io.dD[sh * CD + e];
        else y = io.Dl[sh * CD + e];
      }
      sY[p][j] = y;
    }
    __syncthreads();
    float* out = (prod == 0 ? io.SdO : prod == 1 ? io.SdD : io.DsD) + sh * CD;
    for (int e = tid; e < C * D; e += NT) {
      const int p = e / D, i = e % D;
      float acc = 0.0f;
      for (int j = 0; j < D; ++j) acc = fmaf(sM[i][j], sY[p][j], acc);
      out[e] = acc;
    }
    __syncthreads();
  }
}

// Per chunk and value head: gradients of q-hat, k-hat (per value head), v,
// beta and g.
template <int D, int C, typename TIn>
__global__ __launch_bounds__(256) void k_bwd_chunk(BwdIO io) {
  constexpr int NT = 256;
  constexpr int CP = C + 1;
  constexpr int DP = D + 1;
  // LDS: K | Q QK Z (later reused as Y = [dX_w | dX_u]) | KK | A | dA | vectors
  __shared__ float lds[C * DP + (C * DP + 2 * C * CP) + 3 * C * CP + 8 * C + 256];
  float (*sK)[DP] = reinterpret_cast<float (*)[DP]>(lds);
  float (*sQ)[DP] = reinterpret_cast<float (*)[DP]>(lds + C * DP);
  float (*sQK)[CP] = reinterpret_cast<float (*)[CP]>(lds + 2 * C * DP);
  float (*sZ)[CP] = reinterpret_cast<float (*)[CP]>(lds + 2 * C * DP + C * CP);
  float (*sY)[2 * D] = reinterpret_cast<float (*)[2 * D]>(lds + C * DP);  // after Q, QK, Z die
  float (*sKK)[CP] = reinterpret_cast<float (*)[CP]>(lds + 2 * C * DP + 2 * C * CP);
  float (*sA)[CP] = reinterpret_cast<float (*)[CP]>(lds + 2 * C * DP + 3 * C * CP);
  float (*sdA)[CP] = reinterpret_cast<float (*)[CP]>(lds + 2 * C * DP + 4 * C * CP);
  float* vec = lds + 2 * C * DP + 5 * C * CP;
  float* sG = vec;
  float* sB = vec + C;
  float* sGam = vec + 2 * C;
  float* sLam = vec + 3 * C;
  float* sdG = vec + 4 * C;
  float* sdB = vec + 5 * C;
  float* red = vec + 8 * C;  // 256 partial sums
  static_assert(C * DP + 2 * C * CP >= C * 2 * D, "Y must fit in the Q/QK/Z region");

  int64_t slot, tok0;
  int L, h;
  if (!bwd_item<C>(io, slot, h, tok0, L)) return;
  const int tid = threadIdx.x, hq = h / (io.H_v / io.H_qk);
  const int64_t DD = static_cast<int64_t>(D) * D;
  const int64_t CD = static_cast<int64_t>(C) * D;
  const int64_t sh = slot * io.H_v + h;
  const float* kq = io.qk + (static_cast<int64_t>(hq) * io.T + tok0) * 2 * D;
  for (int e = tid; e < C * D; e += NT) {
    const int p = e / D, i = e % D;
    sK[p][i] = p < L ? kq[p * 2 * D + i] : 0.0f;
    sQ[p][i] = p < L ? kq[p * 2 * D + D + i] : 0.0f;
  }
  if (tid < C) {
    sG[tid] = io.G[sh * C + tid];
    sB[tid] = tid < L ? io.beta[(tok0 + tid) * io.H_v + h] : 0.0f;
  }
  // <S, dS'> (fixed-order block reduction)
  {
    const float* M = io.states + sh * DD;
    const float* dM = io.dstates + sh * DD;
    float part = 0.0f;
    for (int e = tid; e < D * D; e += NT) part = fmaf(M[e], dM[e], part);
    red[tid] = part;
  }
  __syncthreads();
  const float glast = sG[C - 1];
  if (tid < C) {
    sGam[tid] = expf(sG[tid]);
    sLam[tid] = expf(glast - sG[tid]);
  }
  for (int w = NT / 2; w >= 1; w >>= 1) {
    if (tid < w) red[tid] = red[tid] + red[tid + w];
    __syncthreads();
  }
  const float MdM = red[0];
  const float* dO = io.dO + (tok0 * io.H_v + h) * D;
  const float* Dl = io.Dl + sh * CD;
  for (int e = tid; e < C * C; e += NT) {
    const int p = e / C, r = e % C;
    float qk = 0.0f, kk = 0.0f, a = 0.0f, z = 0.0f;
    if (r <= p && p < L) {
      const float gam = expf(sG[p] - sG[r]);
      float dqk = 0.0f, dkk = 0.0f, dp = 0.0f;
      for (int i = 0; i < D; ++i) {
        dqk = fmaf(sQ[p][i], sK[r][i], dqk);
        dkk = fmaf(sK[p][i], sK[r][i], dkk);
        dp = fmaf(dO[static_cast<int64_t>(p) * io.H_v * D + i], Dl[static_cast<int64_t>(r) * D + i], dp);
      }
      qk = dqk;
      z = dp * gam;
      if (r < p) {
        kk = dkk;
        a = sB[p] * (dkk * gam);
      }
    }
    sQK[p][r] = qk;
    sZ[p][r] = z;
    sKK[p][r] = kk;
    sA[p][r] = a;
  }
  __syncthreads();
  const float* SdO = io.SdO + sh * CD;
  const float* DsD = io.DsD + sh * CD;
  // dq-hat and the Q / DsD parts of dk-hat
  for (int e = tid; e < C * D; e += NT) {
    const int p = e / D, i = e % D;
    if (p >= L) continue;
    float aq = sGam[p] * SdO[e];
    for (int r = 0; r <= p; ++r) aq = fmaf(sZ[p][r], sK[r][i], aq);
    io.dqv[((tok0 + p) * io.H_v + h) * D + i] = aq;
    float ak = sLam[p] * DsD[e];
    for (int q = p; q < L; ++q) ak = fmaf(sZ[q][p], sQ[q][i], ak);
    io.dkv[((tok0 + p) * io.H_v + h) * D + i] = ak;
  }
  // dG terms from O and from the state update (needs Q, QK, Z, DsD, SdO)
  if (tid < C) {
    const int p = tid;
    float x = 0.0f;
    if (p < L) {
      float qs = 0.0f, kd = 0.0f;
      for (int i = 0; i < D; ++i) {
        qs = fmaf(sQ[p][i], SdO[static_cast<int64_t>(p) * D + i], qs);
        kd = fmaf(sK[p][i], DsD[static_cast<int64_t>(p) * D + i], kd);
      }
      x = sGam[p] * qs - sLam[p] * kd;
      for (int r = 0; r < p; ++r) x = fmaf(sZ[p][r], sQK[p][r], x);
      for (int q = p + 1; q < L; ++q) x = fmaf(-sZ[q][p], sQK[q][p], x);
      if (p == L - 1) {
        float s = sGam[C - 1] * MdM;
        for (int q = 0; q < L; ++q) {
          float kd2 = 0.0f;
          for (int i = 0; i < D; ++i)
            kd2 = fmaf(sK[q][i], DsD[static_cast<int64_t>(q) * D + i], kd2);
          s = fmaf(sLam[q], kd2, s);
        }
        x = x + s;
      }
    }
    sdG[p] = x;
  }
  __syncthreads();  // Q, QK, Z are dead from here; their space holds Y
  // back substitution (I + A)^T Y = [dW | dU], dW = -SdD, dU = dDelta;
  // thread t owns column t (t < D: dX_w, else dX_u)
  if (tid < 2 * D) {
    const int t = tid;
    const bool isW = t < D;
    const int col = isW ? t : t - D;
    const float* rhs = isW ? io.SdD + sh * CD : io.dD + sh * CD;
    for (int p = C - 1; p >= 0; --p) {
      float y = 0.0f;
      if (p < L) {
        y = isW ? -rhs[static_cast<int64_t>(p) * D + col] : rhs[static_cast<int64_t>(p) * D + col];
        for (int r = p + 1; r < L; ++r) y = fmaf(-sA[r][p], sY[r][t], y);
      }
      sY[p][t] = y;
    }
  }
  __syncthreads();
  // dA_pr = -(dX_w,p . W_r + dX_u,p . U_r), r < p
  const float* Wc = io.W + sh * CD;
  const float* Uc = io.U + sh * CD;
  for (int e = tid; e < C * C; e += NT) {
    const int p = e / C, r = e % C;
    float x = 0.0f;
    if (r < p && p < L) {
      float a = 0.0f;
      for (int i = 0; i < D; ++i) a = fmaf(sY[p][i], Wc[static_cast<int64_t>(r) * D + i], a);
      for (int i = 0; i < D; ++i) a = fmaf(sY[p][D + i], Uc[static_cast<int64_t>(r) * D + i], a);
      x = -a;
    }
    sdA[p][r] = x;
  }
  __syncthreads();
  // dbeta and the remaining dG terms
  if (tid < C) {
    const int p = tid;
    float db = 0.0f, dgp = sdG[p];
    if (p < L) {
      const TIn* vin = static_cast<const TIn*>(io.v) + ((tok0 + p) * io.H_v + h) * D;
      float xk = 0.0f, uv = 0.0f;
      for (int i = 0; i < D; ++i) {
        xk = fmaf(sY[p][i], sK[p][i], xk);
        uv = fmaf(sY[p][D + i], ldin(vin + i), uv);
      }
      db = sGam[p] * xk + uv;
      dgp = fmaf(sB[p] * sGam[p], xk, dgp);
      for (int r = 0; r < p; ++r) {
        db = fmaf(sdA[p][r], sKK[p][r] * expf(sG[p] - sG[r]), db);
        dgp = fmaf(sdA[p][r], sA[p][r], dgp);
      }
      for (int q = p + 1; q < L; ++q) dgp = fmaf(-sdA[q][p], sA[q][p], dgp);
    }
    sdB[p] = db;
    sdG[p] = dgp;
  }
  __syncthreads();
  // dA -> gradient of k_p . k_r  (E2_pr = dA_pr beta_p Gam_pr), in place
  for (int e = tid; e < C * C; e += NT) {
    const int p = e / C, r = e % C;
    if (r < p && p < L) sdA[p][r] = sdA[p][r] * sB[p] * expf(sG[p] - sG[r]);
  }
  __syncthreads();
  for (int e = tid; e < C * D; e += NT) {
    const int p = e / D, i = e % D;
    if (p >= L) continue;
    const int64_t o = ((tok0 + p) * io.H_v + h) * D + i;
    float ak = io.dkv[o];
    ak = fmaf(sB[p] * sGam[p], sY[p][i], ak);
    for (int r = 0; r < p; ++r) ak = fmaf(sdA[p][r], sK[r][i], ak);
    for (int q = p + 1; q < L; ++q) ak = fmaf(sdA[q][p], sK[q][i], ak);
    io.dkv[o] = ak;
    st_grad(io.dv, o, sB[p] * sY[p][D + i], io.grad_bf16);
  }
  if (tid == 0) {  // dg = reverse running sum of dG within the chunk
    float acc = 0.0f;
    for (int p = L - 1; p >= 0; --p) {
      acc = acc + sdG[p];
      io.dg[(tok0 + p) * io.H_v + h] = acc;
      io.dbeta[(tok0 + p) * io.H_v + h] = sdB[p];
    }
  }
}

// ---------------------------------------------------------------------------
// Matrix-core forms of the backward for d = 128, C = 64.  The gradient is the
// same as above; sums are taken on v_mfma_f32_16x16x4_f32 in a fixed order.
// Tile helpers: one 16 x 16 output tile in accumulator layout (lane l holds
// rows 4g + r, column l16; g = l / 16), K summed in steps of 4 with lane group
// g supplying k = g K/4 + s, s = 0 .. K/4 - 1.
//   mma_nt: a -> A[m0 + l16][0], b -> B[n0 + l16][0], both k-contiguous
//   mma_nn: a -> A[m0 + l16][0] k-contiguous; b -> B[0][n0 + l16], row stride
//           ldb; rows of B at or past `brows` read row brows - 1 (in bounds)
//   mma_tn: a -> At[0][m0 + l16] (A given transposed, row stride lda); b as nn
template <int K>
__device__ __forceinline__ v4f mma_nt(v4f acc, const float* a, const float* b, int g) {
  a += g * (K / 4);
  b += g * (K / 4);
#pragma unroll
  for (int s4 = 0; s4 < K / 16; ++s4) {
    const float4 x = *reinterpret_cast<const float4*>(a + 4 * s4);
    const float4 y = *reinterpret_cast<const float4*>(b + 4 * s4);
    acc = mfma4(x.x, y.x, acc);
    acc = mfma4(x.y, y.y, acc);
    acc = mfma4(x.z, y.z, acc);
    acc = mfma4(x.w, y.w, acc);
  }
  return acc;
}
// mma_nt with the B operand already in registers: b[s4] holds what mma_nt
// would read at b + g K/4 + 4 s4
template <int K>
__device__ __forceinline__ v4f mma_nt_rb(v4f acc, const float* a, const float4* b, int g) {
  a += g * (K / 4);
#pragma unroll
  for (int s4 = 0; s4 < K / 16; ++s4) {
    const float4 x = *reinterpret_cast<const float4*>(a + 4 * s4);
    acc = mfma4(x.x, b[s4].x, acc);
    acc = mfma4(x.y, b[s4].y, acc);
    acc = mfma4(x.z, b[s4].z, acc);
    acc = mfma4(x.w, b[s4].w, acc);
  }
  return acc;
}
template <int K>
__device__ __forceinline__ v4f mma_nn(v4f acc, const float* a, const float* b, int ldb, int brows,
                                      int g) {
  a += g * (K / 4);
#pragma unroll
  for (int s4 = 0; s4 < K / 16; ++s4) {
    const float4 x = *reinterpret_cast<const float4*>(a + 4 * s4);
    float y[4];
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      int k = g * (K / 4) + 4 * s4 + q;
      k = k < brows ? k : brows - 1;
      y[q] = b[static_cast<int64_t>(k) * ldb];
    }
    acc = mfma4(x.x, y[0], acc);
    acc = mfma4(x.y, y[1], acc);
    acc = mfma4(x.z, y[2], acc);
    acc = mfma4(x.w, y[3], acc);
  }
  return acc;
}
template <int K>
__device__ __forceinline__ v4f mma_tn(v4f acc, const float* a, int lda, const float* b, int ldb,
                                      int brows, int g) {
#pragma unroll
  for (int s = 0; s < K / 4; ++s) {
    const int k = g * (K / 4) + s;
    const int kb = k < brows ? k : brows - 1;
    acc = mfma4(a[k * lda], b[static_cast<int64_t>(kb) * ldb], acc);
  }
  return acc;
}

// E = P^T dO on the matrix cores.
template <int C>
__global__ __launch_bounds__(256) void k_bwd_prep_m(BwdIO io) {
  constexpr int D = 128, S1 = D + 4, S2 = C + 4;
  static_assert(C == 64, "tiling assumes C = 64");
  __shared__ __attribute__((aligned(16))) float lds[2 * C * S1];  // Q | K, then dO | P^T
  __shared__ float sG[C];
  float* sQ = lds;
  float* sK = lds + C * S1;
  float* sO = lds;             // [C][S1]
  float* PT = lds + C * S1;    // [C][S2]
  static_assert(C * S2 <= C * S1, "LDS reuse");
  int64_t slot, tok0;
  int L, h;
  if (!bwd_item<C>(io, slot, h, tok0, L)) return;
  const int tid = threadIdx.x, lane = tid & 63, l16 = lane & 15, g = lane >> 4;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int hq = h / (io.H_v / io.H_qk);
  const int64_t sh = slot * io.H_v + h;
  const float* kq = io.qk + (static_cast<int64_t>(hq) * io.T + tok0) * 2 * D;
  static_assert((C * (D / 4)) % 256 == 0, "whole rounds");
#pragma unroll
  for (int e_ = 0; e_ < (C * (D / 4)) / 256; ++e_) {
    const int e = tid + 256 * e_;
    const int p = e / (D / 4), i4 = e % (D / 4);
    const int pc = p < L ? p : L - 1;
    const float4 k4 = *reinterpret_cast<const float4*>(kq + pc * 2 * D + 4 * i4);
    const float4 q4 = *reinterpret_cast<const float4*>(kq + pc * 2 * D + D + 4 * i4);
    const float4 z = {0.0f, 0.0f, 0.0f, 0.0f};
    *reinterpret_cast<float4*>(sK + p * S1 + 4 * i4) = sel4(p < L, k4, z);
    *reinterpret_cast<float4*>(sQ + p * S1 + 4 * i4) = sel4(p < L, q4, z);
  }
  if (tid < C) sG[tid] = io.G[sh * C + tid];
  // dO rows, fetched now (after the loads the products wait for) and staged
  // once Q and K are dead
  const float* dO = io.dO + (tok0 * io.H_v + h) * D;
  float4 po[(C * (D / 4)) / 256];
#pragma unroll
  for (int e_ = 0; e_ < (C * (D / 4)) / 256; ++e_) {
    const int e = tid + 256 * e_;
    const int p = e / (D / 4), i4 = e % (D / 4);
    const int pc = p < L ? p : L - 1;
    po[e_] = *reinterpret_cast<const float4*>(dO + static_cast<int64_t>(pc) * io.H_v * D + 4 * i4);
  }
  __syncthreads();
  float P[4][4];  // rows p = 16 w + 4 g + r, columns r' = 16 nb + l16
#pragma unroll
  for (int nb = 0; nb < 4; ++nb) {
    v4f acc = {0.0f, 0.0f, 0.0f, 0.0f};
    if (nb <= w) acc = mma_nt<D>(acc, sQ + (16 * w + l16) * S1, sK + (16 * nb + l16) * S1, g);
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const int pp = 16 * w + 4 * g + r, qq = 16 * nb + l16;
      const float x = acc[r] * expf(sG[pp] - sG[qq]);
      P[nb][r] = (nb <= w && qq <= pp && pp < L) ? x : 0.0f;
    }
  }
  __syncthreads();  // Q and K are dead
#pragma unroll
  for (int nb = 0; nb < 4; ++nb)
#pragma unroll
    for (int r = 0; r < 4; ++r) PT[(16 * nb + l16) * S2 + 16 * w + 4 * g + r] = P[nb][r];
#pragma unroll
  for (int e_ = 0; e_ < (C * (D / 4)) / 256; ++e_) {
    const int e = tid + 256 * e_;
    const int p = e / (D / 4), i4 = e % (D / 4);
    *reinterpret_cast<float4*>(sO + p * S1 + 4 * i4) = sel4(p < L, po[e_], float4{0.0f, 0.0f, 0.0f, 0.0f});
  }
  __syncthreads();
  float* E = io.E + sh * static_cast<int64_t>(C) * D;
#pragma unroll
  for (int nb = 0; nb < D / 16; ++nb) {
    v4f acc = {0.0f, 0.0f, 0.0f, 0.0f};
    acc = mma_nn<C>(acc, PT + (16 * w + l16) * S2, sO + 16 * nb + l16, S1, C, g);
#pragma unroll
    for (int r = 0; r < 4; ++r) E[(16 * w + 4 * g + r) * D + 16 * nb + l16] = acc[r];
  }
}

// Native-mixed baseline (not the CPR contract): the outputs of one chunk and
// value head in chunk form on the matrix cores,
//   O = diag(gam) Q S_c^T + P Delta,   P_pr = (q_p . k_r) exp(G_p - G_r), r <= p,
// from the chunk-start state S_c (stored [d_k][d_v]) and Delta = U - W S_c^T
// of the chunk scan.  P is built in LDS by pairs of waves; wave w then owns
// the 16 output columns j = 16 w + l16 for all 64 rows, with S_c and Delta
// streamed as B operands (k = i, then k = r).
template <int C>
__global__ __launch_bounds__(512) void k_chunk_o_m(BwdIO io) {
  constexpr int D = 128, S1 = D + 4, S2 = C + 4;
  static_assert(C == 64, "tiling assumes C = 64");
  __shared__ __attribute__((aligned(16))) float sQ[C * S1];
  __shared__ __attribute__((aligned(16))) float sK[C * S1];
  __shared__ __attribute__((aligned(16))) float sP[C * S2];
  __shared__ float sG[C], sGam[C];
  int64_t slot, tok0;
  int L, h;
  if (!bwd_item<C>(io, slot, h, tok0, L)) return;
  const int tid = threadIdx.x, lane = tid & 63, l16 = lane & 15, g = lane >> 4;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);  // 0..7
  const int hq = h / (io.H_v / io.H_qk);
  const int64_t sh = slot * io.H_v + h;
  const int64_t DD = static_cast<int64_t>(D) * D, CD = static_cast<int64_t>(C) * D;
  const float* kq = io.qk + (static_cast<int64_t>(hq) * io.T + tok0) * 2 * D;
  const float4 z4 = {0.0f, 0.0f, 0.0f, 0.0f};
  static_assert((C * (D / 4)) % 512 == 0, "whole rounds");
#pragma unroll
  for (int e_ = 0; e_ < (C * (D / 4)) / 512; ++e_) {
    const int e = tid + 512 * e_;
    const int p = e / (D / 4), i4 = e % (D / 4);
    const int pc = p < L ? p : L - 1;
    const float4 k4 = *reinterpret_cast<const float4*>(kq + pc * 2 * D + 4 * i4);
    const float4 q4 = *reinterpret_cast<const float4*>(kq + pc * 2 * D + D + 4 * i4);
    *reinterpret_cast<float4*>(sK + p * S1 + 4 * i4) = sel4(p < L, k4, z4);
    *reinterpret_cast<float4*>(sQ + p * S1 + 4 * i4) = sel4(p < L, q4, z4);
  }
  if (tid < C) {
    const float gv = io.G[sh * C + tid];
    sG[tid] = gv;
    sGam[tid] = expf(gv);
  }
  __syncthreads();
  // P tiles (row block tmb, column blocks tnb0 and tnb0 + 2), r <= p
  const int tmb = w >> 1, tnb0 = w & 1;
#pragma unroll
  for (int t = 0; t < 2; ++t) {
    const int nb = tnb0 + 2 * t;
    v4f acc = {0.0f, 0.0f, 0.0f, 0.0f};
    if (nb <= tmb) acc = mma_nt<D>(acc, sQ + (16 * tmb + l16) * S1, sK + (16 * nb + l16) * S1, g);
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const int pp = 16 * tmb + 4 * g + r, qq = 16 * nb + l16;
      const float x = acc[r] * expf(sG[pp] - sG[qq]);
      sP[pp * S2 + qq] = (nb <= tmb && qq <= pp && pp < L) ? x : 0.0f;
    }
  }
  __syncthreads();
  // O tiles (p = 16 pb + 4 g + r, j): Q S_c^T (k = i = g D/4 + s), scaled by
  // gam_p, then + P Delta (k = r = g C/4 + s)
  const int j = 16 * w + l16;
  const float* Sc = io.states + sh * DD + j;
  const float* Dc = io.Dl + sh * CD + j;
  v4f acc[4];
#pragma unroll
  for (int pb = 0; pb < 4; ++pb) acc[pb] = v4f{0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
  for (int s4 = 0; s4 < D / 16; ++s4) {
    float b[4];
#pragma unroll
    for (int c = 0; c < 4; ++c) b[c] = Sc[static_cast<int64_t>(g * (D / 4) + 4 * s4 + c) * D];
#pragma unroll
    for (int pb = 0; pb < 4; ++pb) {
      const float4 a = *reinterpret_cast<const float4*>(sQ + (16 * pb + l16) * S1 + g * (D / 4) + 4 * s4);
      acc[pb] = mfma4(a.x, b[0], acc[pb]);
      acc[pb] = mfma4(a.y, b[1], acc[pb]);
      acc[pb] = mfma4(a.z, b[2], acc[pb]);
      acc[pb] = mfma4(a.w, b[3], acc[pb]);
    }
  }
#pragma unroll
  for (int pb = 0; pb < 4; ++pb)
#pragma unroll
    for (int r = 0; r < 4; ++r) acc[pb][r] = sGam[16 * pb + 4 * g + r] * acc[pb][r];
#pragma unroll
  for (int s4 = 0; s4 < C / 16; ++s4) {
    float b[4];
#pragma unroll
    for (int c = 0; c < 4; ++c) b[c] = Dc[static_cast<int64_t>(g * (C / 4) + 4 * s4 + c) * D];
#pragma unroll
    for (int pb = 0; pb < 4; ++pb) {
      const float4 a = *reinterpret_cast<const float4*>(sP + (16 * pb + l16) * S2 + g * (C / 4) + 4 * s4);
      acc[pb] = mfma4(a.x, b[0], acc[pb]);
      acc[pb] = mfma4(a.y, b[1], acc[pb]);
      acc[pb] = mfma4(a.z, b[2], acc[pb]);
      acc[pb] = mfma4(a.w, b[3], acc[pb]);
    }
  }
  const int64_t vs = static_cast<int64_t>(io.H_v) * D;
#pragma unroll
  for (int pb = 0; pb < 4; ++pb)
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const int p = 16 * pb + 4 * g + r;
      if (p < L) io.dqv[(tok0 + p) * vs + static_cast<int64_t>(h) * D + j] = acc[pb][r];
    }
}

// Reverse scan of the state gradient on the matrix cores, one block of 8
// waves per (sequence, value head):
//   dDelta = E + diag(lam) K dS'^T,   dS = gam_last dS' + (gam dO)^T Q - dDelta^T W,
// with fp32 operands as bf16 parts (as in the chunk scan).  The state
// gradient is held transposed (rows i of d_k, columns j of d_v) in
// accumulator layout: wave w owns columns j = 16 w .. 16 w + 15 as eight
// 16 x 16 tiles (ib = 0..7).  A k block of 32 is spread over the lanes as in
// the chunk scan (lane group g supplies element e as k = 32 kb + 16 (e / 4) +
// 4 g + e % 4, register e % 4 of tile 2 kb + e / 4), so dDelta (k = i) takes
// the state, and the update (k = p) takes gam dO and dDelta, straight from
// accumulator tiles split into parts.  Summation orders: dDelta's products
// start from 0 and add, for kb = 0..3, the six part products (then
// fmaf(lam, ., E)); the update starts from gam_last dS' and adds the six
// part products of Q^T (gam dO) for the two k blocks of p, then those of
// (-W^T) dDelta.  (Two waves share a SIMD, so a block's A operand is read at
// the start of its region: the other wave's products cover the reads.)  Per chunk, K (rows p, groups of i), and Q^T and -W^T (rows
// i, groups of p; group slots XOR-swizzled by row as in the chunk scan) sit
// in LDS as parts.  K is read only by the dDelta products and Q, W only by
// the update, so each is written while the other is read: the previous
// chunk's K is loaded during this chunk's dDelta products and split into LDS
// beside the update's; its Q, W and G are loaded during the update and split
// into LDS beside the next chunk's dDelta products.  Each k block's products
// are one scheduling region with that VALU work.  Two barriers per chunk and
// no branch in the loop (past chunk 0 the loads reload chunk 0).
template <int C>
__global__ __launch_bounds__(512) void k_bwd_scan_m(BwdIO io) {
  constexpr int D = 128;
  constexpr int WR = 16 * 12 + 4, KR = 8 * 12 + 4;  // words per LDS row (parts + 16 bytes)
  static_assert(C == 64, "tiling assumes C = 64, D = 128");
  __shared__ __attribute__((aligned(16))) uint32_t sK[C * WR];  // K[p][group of i][part][8]
  __shared__ __attribute__((aligned(16))) uint32_t sQ[D * KR];  // Q^T[i][slot of p group][part][8]
  __shared__ __attribute__((aligned(16))) uint32_t sW[D * KR];  // -W^T, the same way
  __shared__ float sGam[C], sLam[C];
  const int tid = threadIdx.x, lane = tid & 63, l16 = lane & 15, g = lane >> 4;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
  // (sequence, head) pairs 2 p, 2 p + 1 (two heads of a q/k group when the
  // group has two) go out 8 blocks apart, to one XCD at about the same time,
  // and share the q-hat and k-hat rows through its L2 (grid: 16 | blocks)
  const int64_t bx = blockIdx.x;
  const int64_t nh = ((bx / 16) * 8 + bx % 8) * 2 + (bx / 8) % 2;
  const int n = static_cast<int>(nh / io.H_v), h = static_cast<int>(nh % io.H_v);
  if (n >= io.N) return;
  const int hq = h / (io.H_v / io.H_qk);
  const int64_t DD = static_cast<int64_t>(D) * D, CD = static_cast<int64_t>(C) * D;
  const int64_t s0 = io.cu[n];
  const int64_t Lseq = static_cast<int64_t>(io.cu[n + 1]) - s0;
  if (Lseq < 0 || s0 < 0 || s0 + Lseq > io.T) return;
  const int64_t nchunks = (Lseq + C - 1) / C;
  const int64_t slot0 = io.cu_chunks[n];
  if (slot0 + nchunks > io.max_state_slot) return;
  const int j = 16 * w + l16;  // this lane's column of d_v

  // Buffer offsets (bytes): a lane part in a VGPR, a wave-uniform part in an
  // SGPR.  Rows past a partial chunk's end are outside the range of the
  // chunk's K/Q and dO resources (range-checked lane offsets) and read 0.
  const uint32_t fj = 4u * static_cast<uint32_t>(4 * g * D + j);   // (p or i = 4 g, j) of [.][D]
  const uint32_t ostride = static_cast<uint32_t>(io.H_v) * D * 4u;  // dO row stride
  const uint32_t fo = 4u * static_cast<uint32_t>(j) + static_cast<uint32_t>(4 * g) * ostride;
  // K staging: rows kr0, kr0 + 1, column group kgp (columns 32 (kgp / 4) +
  // 4 (kgp % 4) + 0..3 and + 16 + 0..3)
  const int kgp = tid & 15, kr0 = (tid >> 4) * 2;
  const uint32_t fk = 4u * static_cast<uint32_t>(kr0 * 2 * D + 32 * (kgp >> 2) + 4 * (kgp & 3));
  // Q and W staging: key group qg (keys p = 32 (qg / 4) + 16 (e / 4) +
  // 4 (qg % 4) + e % 4), columns 2 qc, 2 qc + 1 (8 bytes per key: coalesced)
  const int qg = tid >> 6, qc = tid & 63;
  const int qslot = qg ^ (((2 * qc) >> 3) & 7);  // the same for both columns
  const int qp0 = 32 * (qg >> 2) + 4 * (qg & 3);
  auto rows_of = [&](int64_t c) { return static_cast<int>(Lseq - c * C < C ? Lseq - c * C : C); };
  struct OpRes {
    brsrc_t rq, rw;
    int64_t sh;
  };
  auto op_res = [&](int64_t c) {
    OpRes r;
    r.sh = (slot0 + c) * io.H_v + h;
    const int rows = rows_of(c);
    r.rq = make_rsrc(io.qk + (static_cast<int64_t>(hq) * io.T + s0 + c * C) * 2 * D,
                     static_cast<uint32_t>(rows) * 2 * D * 4u);
    r.rw = make_rsrc(io.W + r.sh * CD, C * D * 4u);
    return r;
  };
  float pk[2][8], pq[8][2], pw[8][2];
  float gvn = 0.0f, glastn = 0.0f;  // G[lane] and G[C - 1]
  auto load_k = [&](const OpRes& rs) {
#pragma unroll
    for (int m = 0; m < 2; ++m)
#pragma unroll
      for (int hf = 0; hf < 2; ++hf) {
        const float4 x = ldbuf4(rs.rq, fk + static_cast<uint32_t>(m * 2 * D * 4 + 64 * hf), 0u);
        pk[m][4 * hf] = x.x, pk[m][4 * hf + 1] = x.y, pk[m][4 * hf + 2] = x.z, pk[m][4 * hf + 3] = x.w;
      }
  };
  auto load_qw = [&](const OpRes& rs) {
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      const uint32_t p = static_cast<uint32_t>(qp0 + 16 * (e >> 2) + (e & 3));
      const auto xq = __builtin_amdgcn_raw_buffer_load_b64(rs.rq, (p * 2 * D + D + 2 * qc) * 4u, 0u, 0);
      const auto xw = __builtin_amdgcn_raw_buffer_load_b64(rs.rw, (p * D + 2 * qc) * 4u, 0u, 0);  // padded rows of W are 0
      pq[e][0] = __uint_as_float(xq[0]), pq[e][1] = __uint_as_float(xq[1]);
      pw[e][0] = __uint_as_float(xw[0]), pw[e][1] = __uint_as_float(xw[1]);
    }
    gvn = io.G[rs.sh * C + lane];
    glastn = io.G[rs.sh * C + C - 1];
  };
  auto put_k = [&](int m, const Parts& y) {  // row kr0 + m
    uint32_t* d = &sK[(kr0 + m) * WR + 12 * kgp];
#pragma unroll
    for (int q = 0; q < 3; ++q) *reinterpret_cast<u32x4_t*>(d + 4 * q) = y.p[q];
  };
  auto put_t = [&](uint32_t* base, int c, const Parts& y) {  // column 2 qc + c of Q^T or -W^T
    uint32_t* d = &base[(2 * qc + c) * KR + 12 * qslot];
#pragma unroll
    for (int q = 0; q < 3; ++q) *reinterpret_cast<u32x4_t*>(d + 4 * q) = y.p[q];
  };
  auto col = [](float (&x)[8], const float (&src)[8][2], int c, bool neg) {
#pragma unroll
    for (int e = 0; e < 8; ++e) x[e] = neg ? -src[e][c] : src[e][c];
  };
  auto put_gl = [&]() {  // every wave writes the same values (no branch)
    // the lane index is re-derived here so that the two LDS addresses are
    // formed where they are used instead of being kept (and spilled) across
    // the loop
    int l = lane;
    asm volatile("" : "+v"(l));
    sLam[l] = expf(glastn - gvn);
    sGam[l] = expf(gvn);
  };
  // E and dO of a chunk in accumulator layout: (p = 16 pb + 4 g + r, j)
  auto load_ed = [&](float (&e)[4][4], float (&d)[4][4], int64_t c) {
    const int64_t sh = (slot0 + c) * io.H_v + h;
    const int rows = rows_of(c);
    const brsrc_t re = make_rsrc(io.E + sh * CD, C * D * 4u);
    const brsrc_t ro = make_rsrc(io.dO + ((s0 + c * C) * io.H_v + h) * D,
                                 static_cast<uint32_t>(rows - 1) * ostride + D * 4u);
#pragma unroll
    for (int pb = 0; pb < 4; ++pb)
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        e[pb][r] = ldbuf(re, fj, static_cast<uint32_t>((16 * pb + r) * D * 4), static_cast<const float*>(nullptr));
        d[pb][r] = ldbuf(ro, fo + static_cast<uint32_t>(16 * pb + r) * ostride, 0u,
                         static_cast<const float*>(nullptr));
      }
  };
  auto tiles8 = [](float (&x)[8], v4f a, v4f b) {
#pragma unroll
    for (int e = 0; e < 4; ++e) x[e] = a[e], x[4 + e] = b[e];
  };
  // A operands: part q of K rows 16 pb + l16 in k block kb; of Q^T or -W^T
  // rows 16 (4 h2 + t) + l16 in k block kp
  auto read_k = [&](u32x4_t (&x)[4], int kb, int q) {
#pragma unroll
    for (int pb = 0; pb < 4; ++pb)
      x[pb] = *reinterpret_cast<const u32x4_t*>(&sK[(16 * pb + l16) * WR + 12 * (4 * kb + g) + 4 * q]);
  };
  auto read_t = [&](u32x4_t (&x)[4], const uint32_t* base, int kp, int h2, int q) {
#pragma unroll
    for (int t = 0; t < 4; ++t) {
      const int i = 16 * (4 * h2 + t) + l16;
      x[t] = *reinterpret_cast<const u32x4_t*>(&base[i * KR + 12 * ((4 * kp + g) ^ ((i >> 3) & 7)) + 4 * q]);
    }
  };

  // state gradient dS'^T tiles: (i = 16 ib + 4 g + r, j)
  v4f st[8];
  {
    const brsrc_t rh = make_rsrc(io.dhT ? io.dhT + nh * DD : io.dh0, io.dhT ? D * D * 4u : 0u);
#pragma unroll
    for (int ib = 0; ib < 8; ++ib)
#pragma unroll
      for (int r = 0; r < 4; ++r)  // no dhT: an empty range reads 0
        st[ib][r] = ldbuf(rh, fj, static_cast<uint32_t>((16 * ib + r) * D * 4), static_cast<const float*>(nullptr));
  }

  float glast = 0.0f;  // G at the end of the current chunk
  if (nchunks > 0) {   // the last chunk's K to LDS; its Q, W and G in registers
    const OpRes rs = op_res(nchunks - 1);
    load_k(rs);
    load_qw(rs);
#pragma unroll
    for (int m = 0; m < 2; ++m) put_k(m, split8(pk[m]));
    glast = glastn;
  }
  Parts b = split8(st[0], st[1]);  // B parts of dDelta's first k block
  __syncthreads();
  for (int64_t c = nchunks - 1; c >= 0; --c) {
    const int64_t sh = (slot0 + c) * io.H_v + h;
    const int rows = rows_of(c);
    const OpRes nres = op_res(c > 0 ? c - 1 : c);  // the next chunk (c - 1), or chunk 0 again
    put_gl();  // this chunk's lam and gam (the previous ones were read before the last barrier)
    float ec[4][4], dc[4][4];  // land while dDelta is computed
    load_ed(ec, dc, c);
    const brsrc_t rs = make_rsrc(io.dstates + sh * DD, D * D * 4u);
    v4f dd[4];
#pragma unroll
    for (int pb = 0; pb < 4; ++pb) dd[pb] = v4f{0.0f, 0.0f, 0.0f, 0.0f};
    __builtin_amdgcn_sched_barrier(0);
    // ---- dDelta tiles (p = 16 pb + 4 g + r, j): k = i; beside them this
    // chunk's Q and -W go to LDS as parts, a column per block
#pragma unroll
    for (int kb = 0; kb < 4; ++kb) {
      u32x4_t a0[4], a1[4], a2[4];
      read_k(a0, kb, 0);
      read_k(a1, kb, 1);
      read_k(a2, kb, 2);
      Parts bn = b, pt;
      {
        float xt[8];
        col(xt, kb < 2 ? pq : pw, kb & 1, kb >= 2);
        if (kb + 1 < 4) {
          float xb[8];
          tiles8(xb, st[2 * kb + 2], st[2 * kb + 3]);
          split8x2(xb, xt, bn, pt);
        } else {
          pt = split8(xt);
        }
        put_t(kb < 2 ? sQ : sW, kb & 1, pt);
      }
      // the incoming state gradient (a store), tiles 2 kb and 2 kb + 1
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        const int ib = 2 * kb + e / 4, r = e % 4;
        stbuf(st[ib][r], rs, fj, static_cast<uint32_t>((16 * ib + r) * D * 4));
      }
#pragma unroll
      for (int bq = 0; bq < 3; ++bq)
#pragma unroll
        for (int pb = 0; pb < 4; ++pb) dd[pb] = mfma_bf(a0[pb], b.p[bq], dd[pb]);
#pragma unroll
      for (int bq = 0; bq < 2; ++bq)
#pragma unroll
        for (int pb = 0; pb < 4; ++pb) dd[pb] = mfma_bf(a1[pb], b.p[bq], dd[pb]);
#pragma unroll
      for (int pb = 0; pb < 4; ++pb) dd[pb] = mfma_bf(a2[pb], b.p[0], dd[pb]);
      mfma_valu_pattern<24, 12>();
      __builtin_amdgcn_sched_barrier(0);
      b = bn;
    }
    __syncthreads();  // every wave has read this chunk's K; Q, W, sGam and sLam are written
    const brsrc_t rd = make_rsrc(io.dD + sh * CD, C * D * 4u);
#pragma unroll
    for (int pb = 0; pb < 4; ++pb)
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int p = 16 * pb + 4 * g + r;
        const float v = fmaf(sLam[p], dd[pb][r], ec[pb][r]);
        dd[pb][r] = p < rows ? v : 0.0f;
        stbuf(dd[pb][r], rd, fj, static_cast<uint32_t>((16 * pb + r) * D * 4));
        dc[pb][r] = sGam[p] * dc[pb][r];  // gam dO
      }
    // ---- dS^T = gam_last dS'^T + Q^T (gam dO) - W^T dDelta: k = p from
    // registers; beside the products the next chunk's K goes to LDS as parts
    const float gl = expf(glast);
#pragma unroll
    for (int ib = 0; ib < 8; ++ib) st[ib] = gl * st[ib];
    load_k(nres);  // the next chunk's K: to LDS beside these products
    Parts bq0 = b, bq1 = b, bw0 = b, bw1 = b;
    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
    for (int it = 0; it < 8; ++it) {  // op (Q, then W), k block kp, tiles 4 h2 .. 4 h2 + 3
      const int op = it / 4, kp = (it / 2) % 2, h2 = it % 2;
      const uint32_t* src = op == 0 ? sQ : sW;
      u32x4_t a0[4], a1[4], a2[4];
      read_t(a0, src, kp, h2, 0);
      read_t(a1, src, kp, h2, 1);
      read_t(a2, src, kp, h2, 2);
      if (it == 0) {
        float x[8], y[8];
        tiles8(x, v4f{dc[0][0], dc[0][1], dc[0][2], dc[0][3]}, v4f{dc[1][0], dc[1][1], dc[1][2], dc[1][3]});
        tiles8(y, v4f{dc[2][0], dc[2][1], dc[2][2], dc[2][3]}, v4f{dc[3][0], dc[3][1], dc[3][2], dc[3][3]});
        split8x2(x, y, bq0, bq1);
      }
      if (it == 3 || it == 4) {  // dDelta's k block it - 3 with the next chunk's K row it - 3
        float x[8];
        tiles8(x, dd[2 * (it - 3)], dd[2 * (it - 3) + 1]);
        split8x2(x, pk[it - 3], it == 3 ? bw0 : bw1, b);
        put_k(it - 3, b);
      }
      if (it == 7) b = split8(st[0], st[1]);  // the next chunk's first B parts (tiles 0..3 are final)
      const Parts& bb = op == 0 ? (kp == 0 ? bq0 : bq1) : (kp == 0 ? bw0 : bw1);
#pragma unroll
      for (int bq = 0; bq < 3; ++bq)
#pragma unroll
        for (int t = 0; t < 4; ++t) st[4 * h2 + t] = mfma_bf(a0[t], bb.p[bq], st[4 * h2 + t]);
#pragma unroll
      for (int bq = 0; bq < 2; ++bq)
#pragma unroll
        for (int t = 0; t < 4; ++t) st[4 * h2 + t] = mfma_bf(a1[t], bb.p[bq], st[4 * h2 + t]);
#pragma unroll
      for (int t = 0; t < 4; ++t) st[4 * h2 + t] = mfma_bf(a2[t], bb.p[0], st[4 * h2 + t]);
      mfma_valu_pattern<24, 12>();
      __builtin_amdgcn_sched_barrier(0);
      if (it == 3) load_qw(nres);  // the next chunk's Q, W and G: to LDS beside its dDelta products
    }
    glast = glastn;
    __syncthreads();  // every wave has read this chunk's Q, W, sGam and sLam; the next K is written
  }
  const brsrc_t rh0 = make_rsrc(io.dh0 + nh * DD, D * D * 4u);
#pragma unroll
  for (int ib = 0; ib < 8; ++ib)
#pragma unroll
    for (int r = 0; r < 4; ++r) stbuf(st[ib][r], rh0, fj, static_cast<uint32_t>((16 * ib + r) * D * 4));
}

// Sum of a value over the 4 lanes of a quad (lanes 4k .. 4k+3 of a wave) as
// (x0 + x1) + (x2 + x3); additions commute, so all four lanes get the same bits.
__device__ __forceinline__ float quad_sum(float x) {
  x = x + __shfl_xor(x, 1, 64);
  return x + __shfl_xor(x, 2, 64);
}

// Sum of a value over the 8 lanes of an octet (lanes 8k .. 8k+7 of a wave) as
// a butterfly; additions commute, so all eight lanes get the same bits.
__device__ __forceinline__ float oct_sum(float x) {
  x = x + __shfl_xor(x, 1, 64);
  x = x + __shfl_xor(x, 2, 64);
  return x + __shfl_xor(x, 4, 64);
}

// Per chunk and value head, on the matrix cores: gradients of q-hat, k-hat
// (per value head), v, beta and g.  Eight waves (two per SIMD) share the LDS
// tiles; row reductions use 8 lanes per row.  The chunk's three state
// products and <S, dS'> are formed here first, from S and dS' streamed out of
// memory once (so they never make a round trip through memory):
//   SdO[p][n] = sum_k dO[p][k] S[n][k]      SdD[p][n] = sum_k dDelta[p][k] S[n][k]
//   DsD[p][n] = sum_k Delta[p][k] dS'[n][k]  MdM = sum_{n,k} S[n][k] dS'[n][k]
// with S, dS' in their stored layout: wave w streams rows n = 16 w + l16,
// which are its own output columns.  These products and Z = dO Delta^T take
// their fp32 operands as three bf16 parts on v_mfma_f32_16x16x32_bf16 (the six
// part products of the chunk scan, in the same order), k = 32 kb + 8 g + e for
// element e of lane group g: dO, Delta and dDelta are split once into LDS
// (row p, group k / 8, part, eight elements in 16 bytes), a wave's S and dS'
// rows in registers.
__device__ __forceinline__ v4f mfma_six(const Parts& a, const Parts& b, v4f c) {
  c = mfma_bf(a.p[0], b.p[0], c);
  c = mfma_bf(a.p[0], b.p[1], c);
  c = mfma_bf(a.p[0], b.p[2], c);
  c = mfma_bf(a.p[1], b.p[0], c);
  c = mfma_bf(a.p[1], b.p[1], c);
  return mfma_bf(a.p[2], b.p[0], c);
}
template <int C, typename TIn>
__global__ __launch_bounds__(512) void k_bwd_chunk_m(BwdIO io) {
  constexpr int D = 128, CS = C + 4, KS = D + 4, YS = 2 * D + 4;
  static_assert(C == 64, "tiling assumes C = 64");
  // One LDS pool (words):
  //   Z [0, C CS), QK (later F = E2 + E2^T), KG = (k_p . k_r) Gam_pr (r < p),
  //   K [3 C CS, + C KS), Y [3 C CS + C KS, + 2 C KS): Q | R, then Y;
  // R holds DsD, then SdO, for row reads.  Before the Z phase ends the pool
  // holds the parts of dDelta, dO and Delta from word 0 (PT words each).
  constexpr int PR = 16 * 12 + 4;  // words per parts row: 16 groups x 3 parts x 16 bytes, + 16 bytes
  constexpr int PT = C * PR;
  constexpr int oQK = C * CS, oKG = 2 * C * CS, oK = 3 * C * CS, oY = oK + C * KS;
  constexpr int NPOOL = oY + 2 * C * KS;
  static_assert(3 * PT <= NPOOL && C * YS <= 2 * C * KS, "pool layout");
  static_assert(C * CS <= PT, "Z is written over dDelta's parts only");
  __shared__ __attribute__((aligned(16))) float pool[NPOOL];
  uint32_t* const pdD = reinterpret_cast<uint32_t*>(pool);
  uint32_t* const pdO = pdD + PT;
  uint32_t* const pDl = pdD + 2 * PT;
  float* const sZ = pool;
  float* const sQK = pool + oQK;
  float* const sKG = pool + oKG;
  float* const sK = pool + oK;
  float* const sY = pool + oY;
  float* const sQ = sY;
  float* const sR = sY + C * KS;
  __shared__ float red[8];
  __shared__ float sG[C], sB[C], sGam[C], sdB[C];
  __shared__ __attribute__((aligned(16))) float sLam[C], skd[C];
  __shared__ __attribute__((aligned(16))) float sdG[C];
  int64_t slot, tok0;
  int L, h;
  if (!bwd_item<C>(io, slot, h, tok0, L)) return;
  const int tid = threadIdx.x, lane = tid & 63, l16 = lane & 15, g = lane >> 4;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);  // 0..7
  const int hq = h / (io.H_v / io.H_qk);
  const int64_t CD = static_cast<int64_t>(C) * D;
  const int64_t sh = slot * io.H_v + h;
  const int64_t vs = static_cast<int64_t>(io.H_v) * D;
  const float* kq = io.qk + (static_cast<int64_t>(hq) * io.T + tok0) * 2 * D;
  const float* dO = io.dO + (tok0 * io.H_v + h) * D;
  const float* Dl = io.Dl + sh * CD;
  const float* dDl = io.dD + sh * CD;
  const float* Wc = io.W + sh * CD;
  const float* Uc = io.U + sh * CD;
  const float4 z4 = {0.0f, 0.0f, 0.0f, 0.0f};
  auto crow = [&](int p) { return p < L ? p : L - 1; };
  // C x C tiles of wave w: row block mb = w / 2, column blocks nb = w % 2 and w % 2 + 2
  const int tmb = w >> 1, tnb0 = w & 1;
  const int col = 16 * w + l16;
  if (tid < C) {
    sG[tid] = io.G[sh * C + tid];
    const float bx = io.beta[(tok0 + crow(tid)) * io.H_v + h];
    sB[tid] = tid < L ? bx : 0.0f;
  }
  // dO, Delta, dDelta split into parts: thread t takes (row, group) pairs t and
  // t + 512, row = pair / 16, eight elements from k = 8 (pair % 16); rows past
  // the chunk's end are 0
  {
    float4 x[3][2][2];
#pragma unroll
    for (int j = 0; j < 2; ++j) {
      const int pair = tid + 512 * j, p = pair >> 4, q = pair & 15, pc = crow(p);
#pragma unroll
      for (int hf = 0; hf < 2; ++hf) {
        x[0][j][hf] = *reinterpret_cast<const float4*>(dDl + p * D + 8 * q + 4 * hf);
        x[1][j][hf] = *reinterpret_cast<const float4*>(dO + pc * vs + 8 * q + 4 * hf);
        x[2][j][hf] = *reinterpret_cast<const float4*>(Dl + p * D + 8 * q + 4 * hf);
      }
    }
#pragma unroll
    for (int j = 0; j < 2; ++j) {
      const int pair = tid + 512 * j, p = pair >> 4, q = pair & 15;
#pragma unroll
      for (int m = 0; m < 3; ++m) {
        const float4 a = sel4(p < L, x[m][j][0], z4), b = sel4(p < L, x[m][j][1], z4);
        const Parts y = split8(v4f{a.x, a.y, a.z, a.w}, v4f{b.x, b.y, b.z, b.w});
        uint32_t* d = pdD + m * PT + p * PR + 12 * q;
#pragma unroll
        for (int t = 0; t < 3; ++t) *reinterpret_cast<u32x4_t*>(d + 4 * t) = y.p[t];
      }
    }
  }
  // this lane's S and dS' row pieces (k = 32 kb + 8 g .. + 7), one k block ahead
  const int64_t DD = static_cast<int64_t>(D) * D;
  const float* xs1 = io.states + sh * DD + col * D + 8 * g;
  const float* xs2 = io.dstates + sh * DD + col * D + 8 * g;
  float4 c1[2], c2[2], n1[2], n2[2];
#pragma unroll
  for (int hf = 0; hf < 2; ++hf) {
    c1[hf] = *reinterpret_cast<const float4*>(xs1 + 4 * hf);
    c2[hf] = *reinterpret_cast<const float4*>(xs2 + 4 * hf);
  }
  // dDelta's column col, the back substitution's right-hand side for tile 1
  float rh[4][2][4];
#pragma unroll
  for (int bi = 0; bi < 4; ++bi)
#pragma unroll
    for (int r = 0; r < 4; ++r) rh[bi][1][r] = dDl[(16 * bi + 4 * g + r) * D + col];
  __syncthreads();
  const float glast = sG[C - 1];
  if (tid < C) {
    sGam[tid] = expf(sG[tid]);
    sLam[tid] = expf(glast - sG[tid]);
  }
  // ---- the state products (accumulator layout: rows 16 mb + 4 g + r, column col)
  v4f acc[3][4];  // SdO, SdD, DsD
#pragma unroll
  for (int pr = 0; pr < 3; ++pr)
#pragma unroll
    for (int mb = 0; mb < 4; ++mb) acc[pr][mb] = v4f{0.0f, 0.0f, 0.0f, 0.0f};
  float mdm = 0.0f;
#pragma unroll
  for (int kb = 0; kb < 4; ++kb) {
    if (kb + 1 < 4) {
#pragma unroll
      for (int hf = 0; hf < 2; ++hf) {
        n1[hf] = *reinterpret_cast<const float4*>(xs1 + 32 * (kb + 1) + 4 * hf);
        n2[hf] = *reinterpret_cast<const float4*>(xs2 + 32 * (kb + 1) + 4 * hf);
      }
    }
#pragma unroll
    for (int hf = 0; hf < 2; ++hf) {
      mdm = fmaf(c1[hf].x, c2[hf].x, mdm);
      mdm = fmaf(c1[hf].y, c2[hf].y, mdm);
      mdm = fmaf(c1[hf].z, c2[hf].z, mdm);
      mdm = fmaf(c1[hf].w, c2[hf].w, mdm);
    }
    const Parts b1 = split8(v4f{c1[0].x, c1[0].y, c1[0].z, c1[0].w}, v4f{c1[1].x, c1[1].y, c1[1].z, c1[1].w});
    const Parts b2 = split8(v4f{c2[0].x, c2[0].y, c2[0].z, c2[0].w}, v4f{c2[1].x, c2[1].y, c2[1].z, c2[1].w});
#pragma unroll
    for (int mb = 0; mb < 4; ++mb) {
      const int ro = (16 * mb + l16) * PR + 12 * (4 * kb + g);
      Parts a0, a1, a2;
#pragma unroll
      for (int t = 0; t < 3; ++t) {
        a0.p[t] = *reinterpret_cast<const u32x4_t*>(pdO + ro + 4 * t);
        a1.p[t] = *reinterpret_cast<const u32x4_t*>(pdD + ro + 4 * t);
        a2.p[t] = *reinterpret_cast<const u32x4_t*>(pDl + ro + 4 * t);
      }
      acc[0][mb] = mfma_six(a0, b1, acc[0][mb]);
      acc[1][mb] = mfma_six(a1, b1, acc[1][mb]);
      acc[2][mb] = mfma_six(a2, b2, acc[2][mb]);
    }
    if (kb + 1 < 4) {
#pragma unroll
      for (int hf = 0; hf < 2; ++hf) c1[hf] = n1[hf], c2[hf] = n2[hf];
    }
  }
  // <S, dS'>: wave butterfly, then the 8 wave sums in ascending order (tid 0)
#pragma unroll
  for (int off = 32; off >= 1; off >>= 1) mdm = mdm + __shfl_xor(mdm, off, 64);
  if (lane == 0) red[w] = mdm;
  // -SdD's column col: the back substitution's right-hand side for tile 0
  float pS[4][4], pD[4][4];
#pragma unroll
  for (int mb = 0; mb < 4; ++mb)
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      pS[mb][r] = acc[0][mb][r];
      rh[mb][0][r] = acc[1][mb][r];
      pD[mb][r] = acc[2][mb][r];
    }
  // Q and K, fetched during the Z products and written once dO's and Delta's
  // parts are dead
  static_assert((C * (D / 4)) % 512 == 0, "whole rounds");
  constexpr int NR = (C * (D / 4)) / 512;  // float4 of a C x D tile per thread
  float4 pq[NR], pk[NR];
#pragma unroll
  for (int e_ = 0; e_ < NR; ++e_) {
    const int e = tid + 512 * e_;
    const int p = e / (D / 4), i4 = e % (D / 4), pc = crow(p);
    pk[e_] = *reinterpret_cast<const float4*>(kq + pc * 2 * D + 4 * i4);
    pq[e_] = *reinterpret_cast<const float4*>(kq + pc * 2 * D + D + 4 * i4);
  }
  __syncthreads();  // dDelta's parts are dead: Z takes their place
  float MdM = 0.0f;  // thread 0's
  if (tid == 0) {
#pragma unroll
    for (int q = 0; q < 8; ++q) MdM = MdM + red[q];
  }
  // ---- Z = (dO Delta^T) . Gam, masked r <= p
#pragma unroll
  for (int t = 0; t < 2; ++t) {
    const int nb = tnb0 + 2 * t;
    v4f dp = {0.0f, 0.0f, 0.0f, 0.0f};
    if (nb <= tmb) {
#pragma unroll
      for (int kb = 0; kb < 4; ++kb) {
        const int ra = (16 * tmb + l16) * PR + 12 * (4 * kb + g), rb = (16 * nb + l16) * PR + 12 * (4 * kb + g);
        Parts a, b;
#pragma unroll
        for (int q = 0; q < 3; ++q) {
          a.p[q] = *reinterpret_cast<const u32x4_t*>(pdO + ra + 4 * q);
          b.p[q] = *reinterpret_cast<const u32x4_t*>(pDl + rb + 4 * q);
        }
        dp = mfma_six(a, b, dp);
      }
    }
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const int pp = 16 * tmb + 4 * g + r, qq = 16 * nb + l16;
      const float gam = expf(sG[pp] - sG[qq]);
      sZ[pp * CS + qq] = (nb <= tmb && qq <= pp && pp < L) ? dp[r] * gam : 0.0f;
    }
  }
  __syncthreads();  // dO and Delta are dead
#pragma unroll
  for (int e_ = 0; e_ < NR; ++e_) {
    const int e = tid + 512 * e_;
    const int p = e / (D / 4), i4 = e % (D / 4);
    *reinterpret_cast<float4*>(sK + p * KS + 4 * i4) = sel4(p < L, pk[e_], z4);
    *reinterpret_cast<float4*>(sQ + p * KS + 4 * i4) = sel4(p < L, pq[e_], z4);
  }
  // DsD for the row reads of the dG term through the state update
#pragma unroll
  for (int mb = 0; mb < 4; ++mb)
#pragma unroll
    for (int r = 0; r < 4; ++r) sR[(16 * mb + 4 * g + r) * KS + col] = pD[mb][r];
  __syncthreads();
  // k . DsD per row (8 lanes per row, each a 16-element chain over its part)
  {
    const int pp = tid >> 3, part = tid & 7;
    float kd = 0.0f;
#pragma unroll
    for (int m = 0; m < 4; ++m) {
      const int i = 16 * part + 4 * m;
      const float4 rD = *reinterpret_cast<const float4*>(sR + pp * KS + i);
      kd = fmaf(sK[pp * KS + i], rD.x, kd);
      kd = fmaf(sK[pp * KS + i + 1], rD.y, kd);
      kd = fmaf(sK[pp * KS + i + 2], rD.z, kd);
      kd = fmaf(sK[pp * KS + i + 3], rD.w, kd);
    }
    kd = oct_sum(kd);
    if (part == 0) skd[pp] = pp < L ? kd : 0.0f;
  }
  // ---- QK (r <= p) and KK Gam (r < p)
#pragma unroll
  for (int t = 0; t < 2; ++t) {
    const int nb = tnb0 + 2 * t;
    v4f qk = {0.0f, 0.0f, 0.0f, 0.0f}, kk = qk;
    if (nb <= tmb) {
      qk = mma_nt<D>(qk, sQ + (16 * tmb + l16) * KS, sK + (16 * nb + l16) * KS, g);
      kk = mma_nt<D>(kk, sK + (16 * tmb + l16) * KS, sK + (16 * nb + l16) * KS, g);
    }
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const int pp = 16 * tmb + 4 * g + r, qq = 16 * nb + l16;
      const float gam = expf(sG[pp] - sG[qq]);
      const bool in = nb <= tmb && qq <= pp && pp < L;
      sQK[pp * CS + qq] = in ? qk[r] : 0.0f;
      sKG[pp * CS + qq] = (in && qq < pp) ? kk[r] * gam : 0.0f;
    }
  }
  __syncthreads();  // the DsD row reads are done
  // SdO, for the row reads of the dG terms below
#pragma unroll
  for (int mb = 0; mb < 4; ++mb)
#pragma unroll
    for (int r = 0; r < 4; ++r) sR[(16 * mb + 4 * g + r) * KS + col] = pS[mb][r];
  // ---- dq-hat = gam SdO + Z K  and  dk-hat (partial) = lam DsD + Z^T Q; wave w
  // owns columns i = 16 w + l16, all four row blocks
  v4f dk[4];
#pragma unroll
  for (int mb = 0; mb < 4; ++mb) {
    v4f aq, ak;
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const int pp = 16 * mb + 4 * g + r;
      aq[r] = sGam[pp] * pS[mb][r];
      ak[r] = sLam[pp] * pD[mb][r];
    }
    aq = mma_nn<C>(aq, sZ + (16 * mb + l16) * CS, sK + col, KS, C, g);
    ak = mma_tn<C>(ak, sZ + 16 * mb + l16, CS, sQ + col, KS, C, g);
    dk[mb] = ak;
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const int pp = 16 * mb + 4 * g + r;
      if (pp < L) io.dqv[(tok0 + pp) * vs + static_cast<int64_t>(h) * D + col] = aq[r];
    }
  }
  __syncthreads();  // the SdO tile is written
  // ---- dG terms through O and the state update (8 lanes per row)
  {
    const int pp = tid >> 3, part = tid & 7;
    float qs = 0.0f, zq = 0.0f;
#pragma unroll
    for (int m = 0; m < 4; ++m) {
      const int i = 16 * part + 4 * m;
      const float4 rS = *reinterpret_cast<const float4*>(sR + pp * KS + i);
      qs = fmaf(sQ[pp * KS + i], rS.x, qs);
      qs = fmaf(sQ[pp * KS + i + 1], rS.y, qs);
      qs = fmaf(sQ[pp * KS + i + 2], rS.z, qs);
      qs = fmaf(sQ[pp * KS + i + 3], rS.w, qs);
    }
#pragma unroll
    for (int r = 8 * part; r < 8 * part + 8; ++r) {
      // both candidates read (in bounds), then selected: no divergent branch
      const bool lo = r < pp;
      const float z1 = sZ[pp * CS + r], q1 = sQK[pp * CS + r];
      const float z2 = sZ[r * CS + pp], q2 = sQK[r * CS + pp];
      const float t = fmaf(lo ? z1 : -z2, lo ? q1 : q2, zq);
      zq = r != pp ? t : zq;
    }
    qs = oct_sum(qs);
    zq = oct_sum(zq);
    if (part == 0) sdG[pp] = pp < L ? (sGam[pp] * qs - sLam[pp] * skd[pp]) + zq : 0.0f;
  }
  __syncthreads();  // Q, SdO, QK, Z reads done; Y may overwrite them
  if (tid == 0) {
    // rows q < L in ascending order; both rows are read 16 bytes at a time
    // first, and rows past L keep sacc (a select, not a shorter loop)
    float sacc = sGam[C - 1] * MdM;
#pragma unroll
    for (int q4 = 0; q4 < C / 4; ++q4) {
      const float4 lm = *reinterpret_cast<const float4*>(sLam + 4 * q4);
      const float4 kd = *reinterpret_cast<const float4*>(skd + 4 * q4);
      sacc = 4 * q4 < L ? fmaf(lm.x, kd.x, sacc) : sacc;
      sacc = 4 * q4 + 1 < L ? fmaf(lm.y, kd.y, sacc) : sacc;
      sacc = 4 * q4 + 2 < L ? fmaf(lm.z, kd.z, sacc) : sacc;
      sacc = 4 * q4 + 3 < L ? fmaf(lm.w, kd.w, sacc) : sacc;
    }
    sdG[L - 1] = sdG[L - 1] + sacc;
  }
  // ---- back substitution (I + A)^T Y = [-SdD | dDelta], A_pr = beta_p KG_pr,
  // blocked by 16 rows from the bottom; wave w owns columns col of -SdD (tile
  // ct = 0) and of dDelta (ct = 1); every column is solved on its own
  // W and U rows of this wave's first dA tile, fetched while the back
  // substitution runs (the wave with no first tile fetches a valid row block)
  float4 pw[D / 16], pu[D / 16];
  {
    const int nb = tnb0 <= tmb ? tnb0 : 0;
    const float* wr = Wc + (16 * nb + l16) * D + g * (D / 4);
    const float* ur = Uc + (16 * nb + l16) * D + g * (D / 4);
#pragma unroll
    for (int s4 = 0; s4 < D / 16; ++s4) {
      pw[s4] = *reinterpret_cast<const float4*>(wr + 4 * s4);
      pu[s4] = *reinterpret_cast<const float4*>(ur + 4 * s4);
    }
  }
  // and this thread's v segment for dbeta (row tid / 8, 16 elements)
  float pv[16];
  {
    const int pp = tid >> 3, part = tid & 7;
    const TIn* vin = static_cast<const TIn*>(io.v) + (tok0 + crow(pp)) * vs +
                     static_cast<int64_t>(h) * D + 16 * part;
#pragma unroll
    for (int i = 0; i < 16; ++i) pv[i] = ldin(vin + i);
  }
  // T_b = (I + A_bb)^-1 for the four diagonal 16 x 16 blocks: wave b < 4
  // inverts block b by forward substitution on the identity (pivots 0..14 in
  // order; a pivot's coefficients for rows at or above it are the masked
  // tile's zeros), holding T[4 g + r][l16] in register r, and leaves it in Z's
  // place (free until dA) for every wave: block bi's rows are then
  // Y_bi = T_bi^T (right-hand side - sum_bj A_bj,bi^T Y_bj) on the matrix cores
  float* const sT = sZ;  // [4][16][16]
  if (w < 4) {  // wave-uniform
    const int tb = w;
    v4f t;
#pragma unroll
    for (int r = 0; r < 4; ++r) t[r] = 4 * g + r == l16 ? 1.0f : 0.0f;
#pragma unroll
    for (int pp = 0; pp < 15; ++pp) {
      float a[4];
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int row = 16 * tb + 4 * g + r;
        a[r] = sB[row] * sKG[row * CS + 16 * tb + pp];
      }
      const float y = __shfl(t[pp & 3], l16 + 16 * (pp >> 2), 64);
#pragma unroll
      for (int r = 0; r < 4; ++r) t[r] = fmaf(-a[r], y, t[r]);
    }
#pragma unroll
    for (int r = 0; r < 4; ++r) sT[tb * 256 + (4 * g + r) * 16 + l16] = t[r];
  }
  __syncthreads();
  {
    v4f Y[4][2];
#pragma unroll
    for (int bi = 3; bi >= 0; --bi) {
      v4f acc[2];
#pragma unroll
      for (int ct = 0; ct < 2; ++ct)
#pragma unroll
        for (int r = 0; r < 4; ++r) {
          const int pp = 16 * bi + 4 * g + r;
          const float x = (ct == 0 ? -1.0f : 1.0f) * rh[bi][ct][r];
          acc[ct][r] = pp < L ? x : 0.0f;
        }
#pragma unroll
      for (int bj = bi + 1; bj < 4; ++bj)
#pragma unroll
        for (int s4 = 0; s4 < 4; ++s4) {
          const int rr = 16 * bj + 4 * g + s4;
          const float a = -(sB[rr] * sKG[rr * CS + 16 * bi + l16]);
#pragma unroll
          for (int ct = 0; ct < 2; ++ct) acc[ct] = mfma4(a, Y[bj][ct][s4], acc[ct]);
        }
      // Y_bi = T_bi^T acc: k-step s takes T[4 g + s][l16] (lane group g) and
      // acc row 4 g + s, which this lane holds in register s
      {
        float tA[4];
#pragma unroll
        for (int s2 = 0; s2 < 4; ++s2) tA[s2] = sT[bi * 256 + (4 * g + s2) * 16 + l16];
#pragma unroll
        for (int ct = 0; ct < 2; ++ct) {
          v4f y = {0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
          for (int s2 = 0; s2 < 4; ++s2) y = mfma4(tA[s2], acc[ct][s2], y);
          acc[ct] = y;
        }
      }
#pragma unroll
      for (int ct = 0; ct < 2; ++ct) {
        Y[bi][ct] = acc[ct];
#pragma unroll
        for (int r = 0; r < 4; ++r) sY[(16 * bi + 4 * g + r) * YS + ct * D + col] = acc[ct][r];
      }
    }
  }
  __syncthreads();
  // ---- dA = -(dX_w W^T + dX_u U^T), strictly lower; written over Z
#pragma unroll
  for (int t = 0; t < 2; ++t) {
    const int nb = tnb0 + 2 * t;
    v4f acc = {0.0f, 0.0f, 0.0f, 0.0f};
    if (nb <= tmb) {
      // each half's registers are refilled with the next tile's rows as soon
      // as its products are issued
      const bool next = t == 0 && nb + 2 <= tmb;
      acc = mma_nt_rb<D>(acc, sY + (16 * tmb + l16) * YS, pw, g);
      if (next) {
#pragma unroll
        for (int s4 = 0; s4 < D / 16; ++s4)
          pw[s4] = *reinterpret_cast<const float4*>(Wc + (16 * (nb + 2) + l16) * D + g * (D / 4) + 4 * s4);
      }
      acc = mma_nt_rb<D>(acc, sY + (16 * tmb + l16) * YS + D, pu, g);
      if (next) {
#pragma unroll
        for (int s4 = 0; s4 < D / 16; ++s4)
          pu[s4] = *reinterpret_cast<const float4*>(Uc + (16 * (nb + 2) + l16) * D + g * (D / 4) + 4 * s4);
      }
    }
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const int pp = 16 * tmb + 4 * g + r, qq = 16 * nb + l16;
      sZ[pp * CS + qq] = (nb <= tmb && qq < pp && pp < L) ? -acc[r] : 0.0f;
    }
  }
  __syncthreads();
  // ---- dbeta and the remaining dG terms (8 lanes per row); F = E2 + E2^T
  {
    const int pp = tid >> 3, part = tid & 7;
    float xk = 0.0f, uv = 0.0f, da = 0.0f, dga = 0.0f;
#pragma unroll
    for (int i = 16 * part; i < 16 * part + 16; ++i) {
      xk = fmaf(sY[pp * YS + i], sK[pp * KS + i], xk);
      uv = fmaf(sY[pp * YS + D + i], pv[i - 16 * part], uv);
    }
#pragma unroll
    for (int r = 8 * part; r < 8 * part + 8; ++r) {
      // both candidates read (in bounds), then selected: no divergent branch
      const bool lo = r < pp;
      const float z1 = sZ[pp * CS + r], k1 = sKG[pp * CS + r];
      const float z2 = sZ[r * CS + pp], k2 = sKG[r * CS + pp], b2 = sB[r];
      const float ta = fmaf(z1, k1, da);
      const float tg = lo ? fmaf(z1, sB[pp] * k1, dga) : fmaf(-z2, b2 * k2, dga);
      da = lo ? ta : da;
      dga = r != pp ? tg : dga;
    }
    xk = oct_sum(xk);
    uv = oct_sum(uv);
    da = oct_sum(da);
    dga = oct_sum(dga);
    if (part == 0) {
      const float db = (sGam[pp] * xk + uv) + da;
      const float dgp = fmaf(sB[pp] * sGam[pp], xk, sdG[pp]) + dga;
      sdB[pp] = pp < L ? db : 0.0f;
      sdG[pp] = pp < L ? dgp : 0.0f;
    }
  }
  static_assert((C * C) % 512 == 0, "whole rounds");
#pragma unroll
  for (int e_ = 0; e_ < (C * C) / 512; ++e_) {
    const int e = tid + 512 * e_;
    const int pp = e / C, q = e % C;
    const int hi = pp > q ? pp : q, lo = pp > q ? q : pp;
    const float f = sZ[hi * CS + lo] * sB[hi] * expf(sG[hi] - sG[lo]);
    sQK[pp * CS + q] = pp == q ? 0.0f : f;
  }
  __syncthreads();
  // ---- dk-hat += beta gam dX_w + F K ; dv = beta dX_u
#pragma unroll
  for (int mb = 0; mb < 4; ++mb) {
    v4f ak = dk[mb];
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const int pp = 16 * mb + 4 * g + r;
      ak[r] = fmaf(sB[pp] * sGam[pp], sY[pp * YS + col], ak[r]);
    }
    ak = mma_nn<C>(ak, sQK + (16 * mb + l16) * CS, sK + col, KS, C, g);
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const int pp = 16 * mb + 4 * g + r;
      if (pp < L) io.dkv[(tok0 + pp) * vs + static_cast<int64_t>(h) * D + col] = ak[r];
    }
  }
  static_assert((C * D) % 512 == 0, "whole rounds");
#pragma unroll
  for (int e_ = 0; e_ < (C * D) / 512; ++e_) {
    const int e = tid + 512 * e_;
    const int pp = e / D, j = e % D;
    if (pp < L)
      st_grad(io.dv, (tok0 + pp) * vs + static_cast<int64_t>(h) * D + j, sB[pp] * sY[pp * YS + D + j],
              io.grad_bf16);
  }
  // dg: reverse running sum over the chunk (p descending), taken by one lane
  // from registers; then every lane stores its token
  if (tid == 0) {
    float x[C];
#pragma unroll
    for (int q4 = 0; q4 < C / 4; ++q4) {
      const float4 t4 = *reinterpret_cast<const float4*>(sdG + 4 * q4);
      x[4 * q4] = t4.x;
      x[4 * q4 + 1] = t4.y;
      x[4 * q4 + 2] = t4.z;
      x[4 * q4 + 3] = t4.w;
    }
    float acc = 0.0f;
#pragma unroll
    for (int pp = C - 1; pp >= 0; --pp) {  // rows at or past L hold 0: acc + 0 is exact
      acc = acc + x[pp];
      x[pp] = acc;
    }
#pragma unroll
    for (int q4 = 0; q4 < C / 4; ++q4)
      *reinterpret_cast<float4*>(sdG + 4 * q4) = float4{x[4 * q4], x[4 * q4 + 1], x[4 * q4 + 2], x[4 * q4 + 3]};
  }
  __syncthreads();
  if (tid < L) {
    io.dg[(tok0 + tid) * io.H_v + h] = sdG[tid];
    io.dbeta[(tok0 + tid) * io.H_v + h] = sdB[tid];
  }
}

// Sum over the value heads of each group (ascending head order), then the L2
// norm backward: dx = s r (dxh - n (n . dxh)), n = x r, r = (sum x^2 + eps)^-1/2.
// Each wave takes kQkVecs consecutive (token, q/k head) vectors; their loads
// are issued together, and every vector keeps the lanes and order of the
// one-vector form.
constexpr int kQkVecs = 4;
template <int D, typename TIn>
__global__ __launch_bounds__(256) void k_bwd_qk(BwdIO io) {
  const int64_t nvec = io.T * io.H_qk;
  const int64_t vec0 = (static_cast<int64_t>(blockIdx.x) * 4 + (threadIdx.x >> 6)) * kQkVecs;
  if (vec0 >= nvec) return;
  const int G = io.H_v / io.H_qk;
  const int l = threadIdx.x & 63;
  int64_t vecs[kQkVecs];  // t * H_qk + hq, clamped into range (extra ones are not stored)
#pragma unroll
  for (int v = 0; v < kQkVecs; ++v) vecs[v] = vec0 + v < nvec ? vec0 + v : nvec - 1;
  for (int which = 0; which < 2; ++which) {  // 0: q, 1: k
    const float* src = which == 0 ? io.dqv : io.dkv;
    float g0[kQkVecs], g1[kQkVecs], x0[kQkVecs], x1[kQkVecs];
#pragma unroll
    for (int v = 0; v < kQkVecs; ++v) {
      g0[v] = 0.0f;
      g1[v] = 0.0f;
      const TIn* x = static_cast<const TIn*>(which == 0 ? io.q : io.k) + vecs[v] * D;
      x0[v] = l < D ? ldin(x + l) : 0.0f;
      x1[v] = D > 64 ? ldin(x + l + 64) : 0.0f;
    }
    for (int gg = 0; gg < G; ++gg) {
#pragma unroll
      for (int v = 0; v < kQkVecs; ++v) {
        const int64_t t = vecs[v] / io.H_qk;
        const int hq = static_cast<int>(vecs[v] - t * io.H_qk);
        const float* row = src + (t * io.H_v + static_cast<int64_t>(hq) * G + gg) * D;
        if (l < D) g0[v] = g0[v] + row[l];
        if (D > 64) g1[v] = g1[v] + row[l + 64];
      }
    }
    const float mul = which == 0 ? io.scale : 1.0f;
    void* dst = which == 0 ? io.dq : io.dk;
#pragma unroll
    for (int v = 0; v < kQkVecs; ++v) {
      if (vec0 + v >= nvec) break;  // uniform over the wave
      const int64_t d0 = (vec0 + v) * D;
      if (io.l2) {
        float ss = fmaf(x1[v], x1[v], x0[v] * x0[v]);
#pragma unroll
        for (int m = 32; m >= 1; m >>= 1) ss += __shfl_xor(ss, m, 64);
        const float r = 1.0f / sqrtf(ss + gdn::kNormEps);
        const float n0 = x0[v] * r, n1 = x1[v] * r;
        float dot = fmaf(n1, g1[v], n0 * g0[v]);
#pragma unroll
        for (int m = 32; m >= 1; m >>= 1) dot += __shfl_xor(dot, m, 64);
        if (l < D) st_grad(dst, d0 + l, mul * r * (g0[v] - n0 * dot), io.grad_bf16);
        if (D > 64) st_grad(dst, d0 + l + 64, mul * r * (g1[v] - n1 * dot), io.grad_bf16);
      } else {
        if (l < D) st_grad(dst, d0 + l, mul * g0[v], io.grad_bf16);
        if (D > 64) st_grad(dst, d0 + l + 64, mul * g1[v], io.grad_bf16);
      }
    }
  }
}

// ---------------------------------------------------------------------------
// Prefill continuation.  Sequence n of the extended batch is the p_n tokens
// already in its cache's chunk buffers (p_n = pos of head 0, clamped into
// [0, C) as the decode step clamps it) followed by its new tokens.  The
// extended batch then goes through the prefill kernels from the chunk-start
// state S_chunk, which makes every new token's output and the final state
// those of one prefill over the whole history.
__global__ void k_cont_plan(const int32_t* __restrict__ cu, const int32_t* __restrict__ pos,
                            int N, int H_v, int C, int32_t* __restrict__ cu_ext,
                            int32_t* __restrict__ cu_chunks, int32_t* __restrict__ cu_full) {
  if (blockIdx.x != 0 || threadIdx.x != 0) return;
  int32_t e = 0, a = 0, b = 0;
  cu_ext[0] = 0;
  cu_chunks[0] = 0;
  cu_full[0] = 0;
  for (int n = 0; n < N; ++n) {
    int32_t p = pos[static_cast<int64_t>(n) * H_v];
    p = p < 0 ? 0 : (p >= C ? C - 1 : p);
    int32_t L = cu[n + 1] - cu[n];
    L = (L < 0 ? 0 : L) + p;
    e += L;
    a += (L + C - 1) / C;
    b += L / C;
    cu_ext[n + 1] = e;
    cu_chunks[n + 1] = a;
    cu_full[n + 1] = b;
  }
}

struct ContIO {
  const void* q;
  const void* k;
  const void* v;
  const float* beta;
  const float* g;
  const int32_t* cu;      // new tokens
  const int32_t* cu_ext;  // buffered + new tokens
  const float* kbuf;
  const void* vbuf;
  const float* bbuf;
  const float* gbuf;
  float* qk;              // prep layout of the extended batch
  void* v_ext;
  float* b_ext;
  float* g_ext;
  float* gb;              // (g, beta) of the extended batch per value head, token order
  const float* o_ext;
  float* o;
  int N, H_qk, H_v, C, l2;
  float scale;
  int64_t T, T_ext;       // rows of the new and of the extended batch (bounds)
};

// Extended-batch inputs, one wave per (extended row, q/k head): buffered rows
// copy the cache's normalised key (the query of a buffered row only feeds an
// output that is discarded: 0), value, beta and g; new rows normalise q and k
// with the lanes and arithmetic of k_prep and copy v, beta and g.
template <int D, typename TIn>
__global__ __launch_bounds__(256) void k_cont_gather(ContIO io) {
  const int64_t vec = static_cast<int64_t>(blockIdx.x) * 4 + (threadIdx.x >> 6);
  if (vec >= io.T_ext * io.H_qk) return;
  const int64_t e = vec / io.H_qk;
  const int hq = static_cast<int>(vec - e * io.H_qk);
  if (e >= io.cu_ext[io.N]) return;  // uniform over the wave
  const int n = find_seq(io.cu_ext, io.N, e);
  const int64_t r = e - io.cu_ext[n];
  const int64_t p = static_cast<int64_t>(io.cu_ext[n + 1] - io.cu_ext[n]) - (io.cu[n + 1] - io.cu[n]);
  const int l = threadIdx.x & 63;
  const int G = io.H_v / io.H_qk;
  float* out = io.qk + (static_cast<int64_t>(hq) * io.T_ext + e) * 2 * D;
  const TIn* vin;
  const float *bin, *gin;
  int64_t vrow, brow;  // row index of v (x H_v) and of beta / g (x H_v) in their source
  if (r < p) {
    const int64_t bt = static_cast<int64_t>(n) * io.C + r;
    const float* kb = io.kbuf + (bt * io.H_qk + hq) * D;
    if (l < D) {
      out[l] = kb[l];
      out[D + l] = 0.0f;
    }
    if (D > 64) {
      out[l + 64] = kb[l + 64];
      out[D + l + 64] = 0.0f;
    }
    vin = static_cast<const TIn*>(io.vbuf);
    bin = io.bbuf;
    gin = io.gbuf;
    vrow = brow = bt;
  } else {
    const int64_t src = io.cu[n] + (r - p);
    const TIn* kx = static_cast<const TIn*>(io.k) + (src * io.H_qk + hq) * D;
    const TIn* qx = static_cast<const TIn*>(io.q) + (src * io.H_qk + hq) * D;
    const float k0 = (l < D) ? ldin(kx + l) : 0.0f, k1 = (D > 64) ? ldin(kx + l + 64) : 0.0f;
    const float q0 = (l < D) ? ldin(qx + l) : 0.0f, q1 = (D > 64) ? ldin(qx + l + 64) : 0.0f;
    float y0, y1;
    l2norm_vals<D>(k0, k1, 1.0f, io.l2, y0, y1);
    if (l < D) out[l] = y0;
    if (D > 64) out[l + 64] = y1;
    l2norm_vals<D>(q0, q1, io.scale, io.l2, y0, y1);
    if (l < D) out[D + l] = y0;
    if (D > 64) out[D + l + 64] = y1;
    vin = static_cast<const TIn*>(io.v);
    bin = io.beta;
    gin = io.g;
    vrow = brow = src;
  }
  TIn* vo = static_cast<TIn*>(io.v_ext);
  for (int hh = 0; hh < G; ++hh) {
    const int h = hq * G + hh;
    const TIn* vs = vin + (vrow * io.H_v + h) * D;
    TIn* vd = vo + (e * io.H_v + h) * D;
    if (l < D) vd[l] = vs[l];
    if (D > 64) vd[l + 64] = vs[l + 64];
    if (l == 0) {
      const float bx = bin[brow * io.H_v + h], gx = gin[brow * io.H_v + h];
      io.b_ext[e * io.H_v + h] = bx;
      io.g_ext[e * io.H_v + h] = gx;
      *reinterpret_cast<float2*>(io.gb + (static_cast<int64_t>(h) * io.T_ext + e) * 2) = float2{gx, bx};
    }
  }
}

// The new tokens' outputs from the extended batch's, one float4 per thread.
template <int D>
__global__ __launch_bounds__(256) void k_cont_scatter(ContIO io) {
  const int64_t per = static_cast<int64_t>(io.H_v) * D / 4;
  const int64_t x = static_cast<int64_t>(blockIdx.x) * 256 + threadIdx.x;
  if (x >= io.T * per) return;
  const int64_t s = x / per, rem = x - s * per;
  const int n = find_seq(io.cu, io.N, s);
  const int64_t p = static_cast<int64_t>(io.cu_ext[n + 1] - io.cu_ext[n]) - (io.cu[n + 1] - io.cu[n]);
  const int64_t e = io.cu_ext[n] + p + (s - io.cu[n]);
  if (e < 0 || e >= io.T_ext) return;
  reinterpret_cast<float4*>(io.o)[s * per + rem] = reinterpret_cast<const float4*>(io.o_ext)[e * per + rem];
}

// ---------------------------------------------------------------------------
// Cache init: S_run = S_chunk = h0 (or 0), pos = 0.  Plain fill kernel (no
// memset nodes, so the call is safe to capture in a graph).
__global__ void k_cache_init(const float* __restrict__ h0, float* __restrict__ S_run,
                             float* __restrict__ S_chunk, int32_t* __restrict__ pos,
                             int64_t n_state, int64_t n_pos) {
  const int64_t stride = static_cast<int64_t>(gridDim.x) * blockDim.x;
  for (int64_t e = static_cast<int64_t>(blockIdx.x) * blockDim.x + threadIdx.x; e < n_state;
       e += stride) {
    const float x = h0 ? h0[e] : 0.0f;
    S_run[e] = x;
    S_chunk[e] = x;
  }
  for (int64_t e = static_cast<int64_t>(blockIdx.x) * blockDim.x + threadIdx.x; e < n_pos;
       e += stride)
    pos[e] = 0;
}

// ---------------------------------------------------------------------------
// Kernel timing: optional HIP events around every launch.
struct ProfRec {
  const char* name;
  hipEvent_t a, b;
};
struct Profiler {
  std::mutex mu;
  bool on = false;
  std::string filter;  // only launches whose name contains it (empty: all)
  std::vector<ProfRec> recs;
  std::vector<hipEvent_t> pool;
  hipEvent_t get() {
    if (!pool.empty()) {
      hipEvent_t e = pool.back();
      pool.pop_back();
      return e;
    }
    // timing-only events: no system-scope fence (no cache writeback and
    // invalidation around the timed launches); they are read only after the
    // caller has synchronised the device
    hipEvent_t e = nullptr;
    if (hipEventCreateWithFlags(&e, hipEventDisableSystemFence) != hipSuccess) return nullptr;
    return e;
  }
};
Profiler& prof() {
  static Profiler p;
  return p;
}

// Brackets the launches made in its scope with events when timing is on.
class Timed {
 public:
  Timed(const char* name, hipStream_t st) : st_(st) {
    Profiler& p = prof();
    std::lock_guard<std::mutex> g(p.mu);
    if (!p.on) return;
    if (!p.filter.empty() && std::strstr(name, p.filter.c_str()) == nullptr) return;
    rec_.name = name;
    rec_.a = p.get();
    rec_.b = p.get();
    if (rec_.a && rec_.b) {
      (void)hipEventRecord(rec_.a, st_);
      active_ = true;
    }
  }
  ~Timed() {
    if (!active_) return;
    (void)hipEventRecord(rec_.b, st_);
    Profiler& p = prof();
    std::lock_guard<std::mutex> g(p.mu);
    p.recs.push_back(rec_);
  }

 private:
  hipStream_t st_;
  ProfRec rec_{};
  bool active_ = false;
};

// ---------------------------------------------------------------------------
// Host orchestration.

constexpr int kTile128 = 32;  // state rows per k_scan block at d = 128

template <int D>
constexpr int scan_tile() { return D == 128 ? kTile128 : D; }

// Blocks of the persistent backward kernels: one per CU.
constexpr int64_t kPersistentBlocks = 256;

// Value heads per k_rec block: as many of the group as fit in 8 waves and
// divide the group evenly (the group has at most 8 heads).
template <int D>
int rec_heads_per_block(int G) {
  int hpb = 8 / RowSplit<D>::WPH;
  while (hpb > 1 && G % hpb != 0) --hpb;
  return hpb < G ? hpb : G;
}

// Grid of the kernels over every chunk and value head (see wy_item).
dim3 chunk_grid(int64_t chunks, const gdn_shape_t* s) {
  const int64_t G = s->H_v / s->H_qk;
  const int64_t c = chunks > 0 ? chunks : 1;
  return dim3(static_cast<unsigned>((c + 7) / 8 * 8 * G), static_cast<unsigned>(s->H_qk));
}

// Whether the waves of a token-step block that share a key/query stream are
// four (two value heads, two row parts at d = 128, one operand block each),
// so that they can split the prefetch touches.
template <int D>
bool rec_spread(int hpb) {
  return D == 128 && RowSplit<D>::NH * hpb == 4 && RowSplit<D>::DK / RB == 4;
}

// The chunk factors: matrix-core kernel at d = 128, the VALU kernel at d = 16.
template <int D, int C, typename TIn, int MODE>
void launch_wy(const ChunkIO& io, int64_t items, int H_v, hipStream_t st) {
  if (items <= 0) return;
  const int64_t G = H_v / io.H_qk;
  const dim3 grid(static_cast<unsigned>((items + 7) / 8 * 8 * G), io.H_qk);
  if constexpr (D == 128)
    hipLaunchKernelGGL((k_wy_mfma<C, TIn, MODE>), grid, dim3(256), 0, st, io);
  else
    hipLaunchKernelGGL((k_wy<D, C, TIn, MODE>), grid, dim3(256), 0, st, io);
}

// The chunk-state scan: matrix-core kernel at d = 128, the VALU kernel at d = 16.
template <int D, int C, int MODE>
void launch_scan(const ScanIO& io, int64_t N, int H_v, hipStream_t st) {
  constexpr int TILE = scan_tile<D>();
  const int64_t blocks = N * H_v * (D / TILE);
  if (blocks <= 0) return;
  if constexpr (D == 128) {  // blocks of 64 columns of d_v
    // Half a head per block of 4 waves, one block per CU (its LDS keeps two
    // off a CU), while they are no more than the CUs: each chain then has a
    // SIMD per wave.  Past that, a head per block of 8 waves, which stages
    // each chunk's W and K once for all 128 columns.
    const bool wide = N * H_v * 2 > kPersistentBlocks;
    const int64_t mblocks = N * H_v * (wide ? 1 : 2);
    const int64_t nb8 = (mblocks + 7) / 8 * 8;
    const int64_t grid = io.order ? (mblocks + 15) / 16 * 16 : nb8;
    if (wide)
      hipLaunchKernelGGL((k_scan_mfma<C, MODE, 8>), dim3(static_cast<unsigned>(grid)), dim3(512), 0, st,
                         io, mblocks, nb8);
    else
      hipLaunchKernelGGL((k_scan_mfma<C, MODE, 4>), dim3(static_cast<unsigned>(grid)), dim3(256), 0, st,
                         io, mblocks, nb8);
  } else {
    hipLaunchKernelGGL((k_scan<D, C, TILE, MODE>), dim3(static_cast<unsigned>(blocks)), dim3(256),
                       0, st, io);
  }
}

// Longest-first order of the chunk scan's sequences when its blocks need
// several rounds of the GPU (more than two per CU): the longest chains then
// start first.  The scan of each (sequence, head) is the same either way.
const int32_t* scan_order(const int32_t* cu, int32_t N, int H_v, const gdn::Layout& L, char* ws,
                          hipStream_t st) {
  if (N < 2 || L.order == 0 || static_cast<int64_t>(N) * H_v * 2 <= 2 * kPersistentBlocks)
    return nullptr;
  int32_t* order = reinterpret_cast<int32_t*>(ws + L.order);
  Timed t_("k_plan", st);
  hipLaunchKernelGGL(k_order, dim3(static_cast<unsigned>((N + 255) / 256)), dim3(256), 0, st, cu, N,
                     order);
  return order;
}

// The chunk plan and the prep layout: one prep launch whose first thread
// also writes the plan, or the planner alone when there are no tokens.
template <int D, typename TIn>
void launch_plan_prep(const gdn_shape_t* s, int32_t N, const gdn::Counts& cnt, const int32_t* cu,
                      const void* q, const void* k, float* qk, int32_t* cu_chunks, int32_t* cu_full,
                      GbArgs gb, hipStream_t st) {
  const int64_t nvec = cnt.T * s->H_qk;
  if (nvec <= 0) {
    Timed t_("k_plan", st);
    hipLaunchKernelGGL(k_plan, dim3(1), dim3(64), 0, st, cu, N, s->C, cu_chunks, cu_full);
    return;
  }
  Timed t_("k_prep", st);
  hipLaunchKernelGGL((k_prep<D, TIn>), dim3(static_cast<unsigned>(prep_blocks(nvec))), dim3(256), 0, st,
                     static_cast<const TIn*>(q), static_cast<const TIn*>(k), qk, cnt.T, s->H_qk,
                     s->scale, s->qk_l2norm, PlanArgs{cu, N, s->C, cu_chunks, cu_full}, gb);
}

template <int D, int C, typename TIn>
int launch_prefill(const gdn_shape_t* s, int32_t N, const gdn::Counts& cnt, const gdn::Layout& L,
                   const int32_t* cu, const void* q, const void* k, const void* v,
                   const float* beta, const float* g, const float* h0, float* o, float* hT,
                   const gdn_cache_t* cache, char* ws, hipStream_t st, bool gathered = false) {
  // gathered: the chunk plan and the prep layout are already in ws (prefill
  // continuation); q and k are then not read
  int32_t* cu_chunks = reinterpret_cast<int32_t*>(ws + L.cu_chunks);
  int32_t* cu_full = reinterpret_cast<int32_t*>(ws + L.cu_full);
  float* qk = reinterpret_cast<float*>(ws + L.qk);
  float* W = reinterpret_cast<float*>(ws + L.W);
  float* U = reinterpret_cast<float*>(ws + L.U);
  float* Gs = reinterpret_cast<float*>(ws + L.G);
  float* states = reinterpret_cast<float*>(ws + L.states);

  float* gbp = reinterpret_cast<float*>(ws + L.gb);
  if (!gathered)
    launch_plan_prep<D, TIn>(s, N, cnt, cu, q, k, qk, cu_chunks, cu_full, GbArgs{g, beta, gbp, s->H_v}, st);
  if (cnt.full > 0) {
    ChunkIO io{};
    io.khat = qk; io.v = v; io.beta = beta; io.g = g; io.cu = cu; io.cu_full = cu_full;
    io.W = W; io.U = U; io.G = Gs;
    io.N = N; io.H_qk = s->H_qk; io.H_v = s->H_v; io.T = cnt.T; io.max_slot = L.full_slots;
    Timed t_("k_wy", st);
    launch_wy<D, C, TIn, kFull>(io, cnt.full, s->H_v, st);
  }
  {
    ScanIO io{};
    io.khat = qk; io.W = W; io.U = U; io.G = Gs; io.cu = cu; io.cu_chunks = cu_chunks;
    io.cu_full = cu_full; io.h0 = h0; io.states = states; io.hT = hT;
    if (cache) { io.S_run = cache->S_run; io.S_chunk = cache->S_chunk; io.pos = cache->pos; }
    io.N = N; io.H_qk = s->H_qk; io.H_v = s->H_v; io.T = cnt.T;
    io.max_state_slot = L.state_slots; io.max_full_slot = L.full_slots;
    io.order = scan_order(cu, N, s->H_v, L, ws, st);
    if (N > 0) {
      Timed t_("k_scan", st);
      launch_scan<D, C, kFull>(io, N, s->H_v, st);
    }
  }
  if (cnt.chunks > 0) {
    RecIO io{};
    io.qk = qk; io.v = v; io.beta = beta; io.g = g; io.gb = gbp; io.cu = cu;
    io.cu_chunks = cu_chunks; io.states = states; io.o = o; io.hT = hT;
    if (cache) {
      io.S_run = cache->S_run; io.kbuf = cache->kbuf; io.vbuf = cache->vbuf;
      io.bbuf = cache->bbuf; io.gbuf = cache->gbuf;
    }
    io.N = N; io.H_qk = s->H_qk; io.H_v = s->H_v; io.T = cnt.T; io.max_state_slot = L.state_slots;
    Timed t_("k_rec", st);
    const int G = s->H_v / s->H_qk;
    const int hpb = rec_heads_per_block<D>(G);
    const dim3 rgrid(static_cast<unsigned>(cnt.chunks), s->H_qk, G / hpb), rblock(64 * RowSplit<D>::WPH * hpb);
    if (rec_spread<D>(hpb))
      hipLaunchKernelGGL((k_rec<D, C, TIn, true, D == 128>), rgrid, rblock, 0, st, io, hpb);
    else
      hipLaunchKernelGGL((k_rec<D, C, TIn, false, D == 128>), rgrid, rblock, 0, st, io, hpb);
  }
  return hipGetLastError() == hipSuccess ? GDN_OK : GDN_ERR_HIP;
}

template <int D, int C, typename TIn>
int launch_prefill_continue(const gdn_shape_t* s, int32_t N, const gdn::Counts& cnt,
                            const gdn::Counts& cntx, const gdn::Layout& L, const int32_t* cu,
                            const void* q, const void* k, const void* v, const float* beta,
                            const float* g, const gdn_cache_t* cache, float* o, float* hT,
                            char* ws, hipStream_t st) {
  int32_t* cu_ext = reinterpret_cast<int32_t*>(ws + L.cu_ext);
  ContIO io{};
  io.q = q; io.k = k; io.v = v; io.beta = beta; io.g = g; io.cu = cu; io.cu_ext = cu_ext;
  io.kbuf = cache->kbuf; io.vbuf = cache->vbuf; io.bbuf = cache->bbuf; io.gbuf = cache->gbuf;
  io.qk = reinterpret_cast<float*>(ws + L.qk);
  io.v_ext = ws + L.v_ext;
  io.b_ext = reinterpret_cast<float*>(ws + L.b_ext);
  io.g_ext = reinterpret_cast<float*>(ws + L.g_ext);
  io.gb = reinterpret_cast<float*>(ws + L.gb);
  io.o_ext = reinterpret_cast<float*>(ws + L.o_ext);
  io.o = o;
  io.N = N; io.H_qk = s->H_qk; io.H_v = s->H_v; io.C = C; io.l2 = s->qk_l2norm;
  io.scale = s->scale; io.T = cnt.T; io.T_ext = cntx.T;
  {
    Timed t_("k_cont_plan", st);
    hipLaunchKernelGGL(k_cont_plan, dim3(1), dim3(64), 0, st, cu, cache->pos, N, s->H_v, C, cu_ext,
                       reinterpret_cast<int32_t*>(ws + L.cu_chunks),
                       reinterpret_cast<int32_t*>(ws + L.cu_full));
  }
  const int64_t nvec = cntx.T * s->H_qk;
  if (nvec > 0) {
    Timed t_("k_cont_gather", st);
    hipLaunchKernelGGL((k_cont_gather<D, TIn>), dim3(static_cast<unsigned>((nvec + 3) / 4)),
                       dim3(256), 0, st, io);
  }
  const int rc = launch_prefill<D, C, TIn>(s, N, cntx, L, cu_ext, nullptr, nullptr, io.v_ext,
                                           io.b_ext, io.g_ext, cache->S_chunk,
                                           reinterpret_cast<float*>(ws + L.o_ext), hT, cache, ws, st,
                                           true);
  if (rc != GDN_OK) return rc;
  const int64_t n4 = cnt.T * s->H_v * (D / 4);
  if (n4 > 0) {
    Timed t_("k_cont_scatter", st);
    hipLaunchKernelGGL((k_cont_scatter<D>), dim3(static_cast<unsigned>((n4 + 255) / 256)), dim3(256),
                       0, st, io);
  }
  return hipGetLastError() == hipSuccess ? GDN_OK : GDN_ERR_HIP;
}

// The decode token step of N sequences (no workspace).
template <int D, int C, typename TIn>
void launch_token_step(const gdn_shape_t* s, int32_t N, const void* q, const void* k,
                       const void* v, const float* beta, const float* g, const gdn_cache_t* cache,
                       float* o, hipStream_t st) {
  DecIO io{};
  io.q = q; io.k = k; io.v = v; io.beta = beta; io.g = g; io.o = o;
  io.S_run = cache->S_run; io.kbuf = cache->kbuf; io.vbuf = cache->vbuf;
  io.bbuf = cache->bbuf; io.gbuf = cache->gbuf; io.pos = cache->pos;
  io.N = N; io.H_qk = s->H_qk; io.H_v = s->H_v; io.l2 = s->qk_l2norm; io.scale = s->scale;
  Timed t_("k_decode", st);
  hipLaunchKernelGGL((k_decode<D, C, TIn>), dim3(N, s->H_v), dim3(64 * RowSplit<D>::WPH), 0, st, io);
}

// The decode resync of the N sequences of `cache` (the chunk form on their
// chunk buffers; only those whose chunk just completed do any work), with the
// chunk factors in W, U [N, H_v, C, D] and G [N, H_v, C].  Every (sequence,
// head) is computed on its own, so a cache viewed from sequence n0 on
// (cache_from) gives the same bits as the whole batch.
template <int D, int C, typename TIn>
void launch_resync(const gdn_shape_t* s, int32_t N, const gdn_cache_t* cache, float* W, float* U,
                   float* Gs, hipStream_t st) {
  ChunkIO ci{};
  ci.khat = cache->kbuf; ci.v = cache->vbuf; ci.beta = cache->bbuf; ci.g = cache->gbuf;
  ci.pos = cache->pos; ci.W = W; ci.U = U; ci.G = Gs;
  ci.N = N; ci.H_qk = s->H_qk; ci.H_v = s->H_v;
  ci.T = static_cast<int64_t>(N) * C; ci.max_slot = N;
  {
    Timed t_("k_wy_resync", st);
    launch_wy<D, C, TIn, kResync>(ci, N, s->H_v, st);
  }
  ScanIO si{};
  si.khat = cache->kbuf; si.W = W; si.U = U; si.G = Gs;
  si.S_run = cache->S_run; si.S_chunk = cache->S_chunk; si.pos = cache->pos;
  si.N = N; si.H_qk = s->H_qk; si.H_v = s->H_v; si.max_full_slot = N;
  Timed t_("k_scan_resync", st);
  launch_scan<D, C, kResync>(si, N, s->H_v, st);
}

template <int D, int C, typename TIn>
int launch_decode(const gdn_shape_t* s, int32_t N, const gdn::Layout& L, const void* q,
                  const void* k, const void* v, const float* beta, const float* g,
                  const gdn_cache_t* cache, bool resync, float* o, char* ws, hipStream_t st) {
  launch_token_step<D, C, TIn>(s, N, q, k, v, beta, g, cache, o, st);
  if (resync)
    launch_resync<D, C, TIn>(s, N, cache, reinterpret_cast<float*>(ws + L.W),
                             reinterpret_cast<float*>(ws + L.U), reinterpret_cast<float*>(ws + L.G),
                             st);
  return hipGetLastError() == hipSuccess ? GDN_OK : GDN_ERR_HIP;
}

// The native-mixed baseline's decode: the plain token step on a state.
template <int D, int C, typename TIn>
int launch_decode_native(const gdn_shape_t* s, int32_t N, const void* q, const void* k,
                         const void* v, const float* beta, const float* g, float* S, float* o,
                         hipStream_t st) {
  DecIO io{};
  io.q = q; io.k = k; io.v = v; io.beta = beta; io.g = g; io.o = o; io.S_run = S;
  io.N = N; io.H_qk = s->H_qk; io.H_v = s->H_v; io.l2 = s->qk_l2norm; io.scale = s->scale;
  Timed t_("k_decode_native", st);
  hipLaunchKernelGGL((k_decode<D, C, TIn, false>), dim3(N, s->H_v), dim3(64 * RowSplit<D>::WPH), 0,
                     st, io);
  return hipGetLastError() == hipSuccess ? GDN_OK : GDN_ERR_HIP;
}

// The cache of sequences [n0, N) of `c`, as a cache of its own.
gdn_cache_t cache_from(const gdn_cache_t* c, const gdn_shape_t* s, int64_t n0) {
  const int64_t d = s->d_k, C = s->C, Hq = s->H_qk, Hv = s->H_v;
  const int64_t in = s->in_dtype == GDN_BF16 ? 2 : 4;
  gdn_cache_t r = *c;
  r.S_run = c->S_run + n0 * Hv * d * d;
  r.S_chunk = c->S_chunk + n0 * Hv * d * d;
  r.kbuf = c->kbuf + n0 * C * Hq * d;
  r.vbuf = static_cast<char*>(c->vbuf) + n0 * C * Hv * d * in;
  r.bbuf = c->bbuf + n0 * C * Hv;
  r.gbuf = c->gbuf + n0 * C * Hv;
  r.pos = c->pos + n0 * Hv;
  return r;
}

// gdn_decode_step_noalloc: the token step of all N sequences, then the resync
// in groups of `group` sequences whose chunk factors take turns in the fixed
// scratch (in stream order, each group's scan has read them before the next
// group's chunk-factor launch overwrites them).  With pos_host, groups with no
// completing chunk are skipped.
template <int D, int C, typename TIn>
int launch_decode_noalloc(const gdn_shape_t* s, int32_t N, int32_t group, const gdn::Layout& Lg,
                          const void* q, const void* k, const void* v, const float* beta,
                          const float* g, const gdn_cache_t* cache, bool resync,
                          const int32_t* pos_host, float* o, char* scr, hipStream_t st) {
  launch_token_step<D, C, TIn>(s, N, q, k, v, beta, g, cache, o, st);
  for (int32_t n0 = 0; resync && n0 < N; n0 += group) {
    const int32_t m = N - n0 < group ? N - n0 : group;
    if (pos_host) {
      bool any = false;
      for (int64_t e = static_cast<int64_t>(n0) * s->H_v; e < static_cast<int64_t>(n0 + m) * s->H_v; ++e)
        any = any || pos_host[e] + 1 == C;
      if (!any) continue;
    }
    const gdn_cache_t sub = cache_from(cache, s, n0);
    launch_resync<D, C, TIn>(s, m, &sub, reinterpret_cast<float*>(scr + Lg.W),
                             reinterpret_cast<float*>(scr + Lg.U), reinterpret_cast<float*>(scr + Lg.G),
                             st);
  }
  return hipGetLastError() == hipSuccess ? GDN_OK : GDN_ERR_HIP;
}

// native: the native-mixed baseline's trainer step, whose forward outputs come
// from the chunk form (k_chunk_o over every chunk, the final state of a
// sequence with a partial last chunk from the chunk-state scan) instead of the
// token recurrence; the backward is the same.  d = 128 only.
template <int D, int C, typename TIn>
int launch_fwd_bwd(const gdn_shape_t* s, int32_t N, const gdn::Counts& cnt, const gdn::Layout& L,
                   const int32_t* cu, const void* q, const void* k, const void* v,
                   const float* beta, const float* g, const float* h0, const float* dO,
                   const float* dhT, float* o, float* hT, void* dq, void* dk, void* dv,
                   int grad_bf16, float* dbeta, float* dg, float* dh0, char* ws, hipStream_t st,
                   bool native = false) {
  if (native && D != 128) return GDN_ERR_UNSUPPORTED;
  int32_t* cu_chunks = reinterpret_cast<int32_t*>(ws + L.cu_chunks);
  int32_t* cu_full = reinterpret_cast<int32_t*>(ws + L.cu_full);
  float* qk = reinterpret_cast<float*>(ws + L.qk);
  float* W = reinterpret_cast<float*>(ws + L.W);
  float* U = reinterpret_cast<float*>(ws + L.U);
  float* Gs = reinterpret_cast<float*>(ws + L.G);
  float* states = reinterpret_cast<float*>(ws + L.states);
  float* Dl = reinterpret_cast<float*>(ws + L.Dl);
  float* gbp = reinterpret_cast<float*>(ws + L.gb);
  launch_plan_prep<D, TIn>(s, N, cnt, cu, q, k, qk, cu_chunks, cu_full, GbArgs{g, beta, gbp, s->H_v}, st);
  if (cnt.chunks > 0) {
    ChunkIO io{};
    io.khat = qk; io.v = v; io.beta = beta; io.g = g; io.cu = cu; io.cu_full = cu_chunks;
    io.W = W; io.U = U; io.G = Gs;
    io.N = N; io.H_qk = s->H_qk; io.H_v = s->H_v; io.T = cnt.T; io.max_slot = L.state_slots;
    Timed t_("k_wy", st);
    launch_wy<D, C, TIn, kAll>(io, cnt.chunks, s->H_v, st);
  }
  constexpr int TILE = scan_tile<D>();
  const int64_t sblocks = static_cast<int64_t>(N) * s->H_v * (D / TILE);
  if (sblocks > 0) {
    ScanIO io{};
    io.khat = qk; io.W = W; io.U = U; io.G = Gs; io.cu = cu; io.cu_chunks = cu_chunks;
    io.cu_full = cu_full; io.h0 = h0; io.states = states; io.hT = hT; io.Dl = Dl;
    if (native) io.hT_tail = hT;
    io.N = N; io.H_qk = s->H_qk; io.H_v = s->H_v; io.T = cnt.T;
    io.max_state_slot = L.state_slots; io.max_full_slot = L.state_slots;
    io.order = scan_order(cu, N, s->H_v, L, ws, st);
    Timed t_("k_scan", st);
    launch_scan<D, C, kAll>(io, N, s->H_v, st);
  }
  if (native && cnt.chunks > 0) {
    if constexpr (D == 128) {
      BwdIO b{};
      b.qk = qk; b.cu = cu; b.cu_chunks = cu_chunks; b.G = Gs; b.states = states; b.Dl = Dl;
      b.dqv = o;  // k_chunk_o's output
      b.N = N; b.H_qk = s->H_qk; b.H_v = s->H_v; b.T = cnt.T; b.max_state_slot = L.state_slots;
      Timed t_("k_chunk_o", st);
      hipLaunchKernelGGL((k_chunk_o_m<C>), chunk_grid(cnt.chunks, s),
                         dim3(512), 0, st, b);
    }
  } else if (cnt.chunks > 0) {
    RecIO io{};
    io.qk = qk; io.v = v; io.beta = beta; io.g = g; io.gb = gbp; io.cu = cu;
    io.cu_chunks = cu_chunks; io.states = states; io.o = o; io.hT = hT;
    io.N = N; io.H_qk = s->H_qk; io.H_v = s->H_v; io.T = cnt.T; io.max_state_slot = L.state_slots;
    Timed t_("k_rec", st);
    const int G = s->H_v / s->H_qk;
    const int hpb = rec_heads_per_block<D>(G);
    const dim3 rgrid(static_cast<unsigned>(cnt.chunks), s->H_qk, G / hpb), rblock(64 * RowSplit<D>::WPH * hpb);
    if (rec_spread<D>(hpb))
      hipLaunchKernelGGL((k_rec<D, C, TIn, true, false>), rgrid, rblock, 0, st, io, hpb);
    else
      hipLaunchKernelGGL((k_rec<D, C, TIn, false, false>), rgrid, rblock, 0, st, io, hpb);
  }
  // backward
  BwdIO b{};
  b.qk = qk; b.q = q; b.k = k; b.v = v; b.beta = beta; b.g = g; b.dO = dO; b.dhT = dhT;
  b.cu = cu; b.cu_chunks = cu_chunks; b.W = W; b.U = U; b.G = Gs; b.states = states; b.Dl = Dl;
  b.E = reinterpret_cast<float*>(ws + L.E);
  b.dstates = reinterpret_cast<float*>(ws + L.dstates);
  b.dD = reinterpret_cast<float*>(ws + L.dD);
  if (L.SdO) {  // (not allocated at d = 128)
    b.SdO = reinterpret_cast<float*>(ws + L.SdO);
    b.DsD = reinterpret_cast<float*>(ws + L.DsD);
    b.SdD = reinterpret_cast<float*>(ws + L.SdD);
  }
  b.dqv = reinterpret_cast<float*>(ws + L.dqv);
  b.dkv = reinterpret_cast<float*>(ws + L.dkv);
  b.dv = dv; b.dbeta = dbeta; b.dg = dg; b.dq = dq; b.dk = dk; b.dh0 = dh0;
  b.grad_bf16 = grad_bf16;
  b.N = N; b.H_qk = s->H_qk; b.H_v = s->H_v; b.l2 = s->qk_l2norm; b.scale = s->scale;
  b.T = cnt.T; b.max_state_slot = L.state_slots;
  const dim3 cgrid = chunk_grid(cnt.chunks, s);
  if (cnt.chunks > 0) {
    Timed t_("k_bwd_prep", st);
    if constexpr (D == 128)
      hipLaunchKernelGGL((k_bwd_prep_m<C>), cgrid, dim3(256), 0, st, b);
    else
      hipLaunchKernelGGL((k_bwd_prep<D, C>), cgrid, dim3(256), 0, st, b);
  }
  if (sblocks > 0) {
    Timed t_("k_bwd_scan", st);
    if constexpr (D == 128) {
      hipLaunchKernelGGL((k_bwd_scan_m<C>), dim3(static_cast<unsigned>((N * s->H_v + 15) / 16 * 16)), dim3(512), 0,
                         st, b);
    } else {
      hipLaunchKernelGGL((k_bwd_scan<D, C, TILE>), dim3(static_cast<unsigned>(sblocks)),
                         dim3(256), 0, st, b);
    }
  }
  if (cnt.chunks > 0) {
    if constexpr (D != 128) {  // (at d = 128 the chunk kernel forms the state products itself)
      Timed t_("k_bwd_mm", st);
      hipLaunchKernelGGL((k_bwd_mm<D, C>), cgrid, dim3(256), 0, st, b);
    }
    {
      Timed t_("k_bwd_chunk", st);
      if constexpr (D == 128)
        hipLaunchKernelGGL((k_bwd_chunk_m<C, TIn>), cgrid, dim3(512), 0, st, b);
      else
        hipLaunchKernelGGL((k_bwd_chunk<D, C, TIn>), cgrid, dim3(256), 0, st, b);
    }
  }
  const int64_t nvec = cnt.T * s->H_qk;
  if (nvec > 0) {
    Timed t_("k_bwd_qk", st);
    hipLaunchKernelGGL((k_bwd_qk<D, TIn>),
                       dim3(static_cast<unsigned>((nvec + 4 * kQkVecs - 1) / (4 * kQkVecs))),
                       dim3(256), 0, st, b);
  }
  return hipGetLastError() == hipSuccess ? GDN_OK : GDN_ERR_HIP;
}

// Native-mixed baseline prefill: the trainer forward's chunk kernels over every
// chunk, then chunk-form outputs.  d = 128 only.
template <int D, int C, typename TIn>
int launch_prefill_chunked(const gdn_shape_t* s, int32_t N, const gdn::Counts& cnt,
                           const gdn::Layout& L, const int32_t* cu, const void* q, const void* k,
                           const void* v, const float* beta, const float* g, const float* h0,
                           float* o, float* hT, char* ws, hipStream_t st) {
  if constexpr (D != 128) {
    return GDN_ERR_UNSUPPORTED;
  } else {
    int32_t* cu_chunks = reinterpret_cast<int32_t*>(ws + L.cu_chunks);
    int32_t* cu_full = reinterpret_cast<int32_t*>(ws + L.cu_full);
    float* qk = reinterpret_cast<float*>(ws + L.qk);
    float* W = reinterpret_cast<float*>(ws + L.W);
    float* U = reinterpret_cast<float*>(ws + L.U);
    float* Gs = reinterpret_cast<float*>(ws + L.G);
    float* states = reinterpret_cast<float*>(ws + L.states);
    float* Dl = reinterpret_cast<float*>(ws + L.Dl);
    launch_plan_prep<D, TIn>(s, N, cnt, cu, q, k, qk, cu_chunks, cu_full, GbArgs{}, st);
    if (cnt.chunks > 0) {
      ChunkIO io{};
      io.khat = qk; io.v = v; io.beta = beta; io.g = g; io.cu = cu; io.cu_full = cu_chunks;
      io.W = W; io.U = U; io.G = Gs;
      io.N = N; io.H_qk = s->H_qk; io.H_v = s->H_v; io.T = cnt.T; io.max_slot = L.state_slots;
      Timed t_("k_wy", st);
      launch_wy<D, C, TIn, kAll>(io, cnt.chunks, s->H_v, st);
    }
    if (N > 0) {
      ScanIO io{};
      io.khat = qk; io.W = W; io.U = U; io.G = Gs; io.cu = cu; io.cu_chunks = cu_chunks;
      io.cu_full = cu_full; io.h0 = h0; io.states = states; io.hT = hT; io.hT_tail = hT;
      io.Dl = Dl;
      io.N = N; io.H_qk = s->H_qk; io.H_v = s->H_v; io.T = cnt.T;
      io.max_state_slot = L.state_slots; io.max_full_slot = L.state_slots;
      io.order = scan_order(cu, N, s->H_v, L, ws, st);
      Timed t_("k_scan", st);
      launch_scan<D, C, kAll>(io, N, s->H_v, st);
    }
    if (cnt.chunks > 0) {
      BwdIO b{};
      b.qk = qk; b.cu = cu; b.cu_chunks = cu_chunks; b.G = Gs; b.states = states; b.Dl = Dl;
      b.dqv = o;
      b.N = N; b.H_qk = s->H_qk; b.H_v = s->H_v; b.T = cnt.T; b.max_state_slot = L.state_slots;
      Timed t_("k_chunk_o", st);
      hipLaunchKernelGGL((k_chunk_o_m<C>), chunk_grid(cnt.chunks, s),
                         dim3(512), 0, st, b);
    }
    return hipGetLastError() == hipSuccess ? GDN_OK : GDN_ERR_HIP;
  }
}

// Device address of `scratch` on the current device.  Looked up once per
// device, with that device current, and kept: every GPU holds its own copy of
// the array at its own address.
int scratch_ptr(char** out) {
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0) return GDN_ERR_HIP;
  static std::mutex mu;
  static std::vector<char*> ptrs;
  std::lock_guard<std::mutex> lock(mu);
  if (static_cast<size_t>(dev) >= ptrs.size()) ptrs.resize(static_cast<size_t>(dev) + 1, nullptr);
  if (!ptrs[dev]) {
    void* p = nullptr;
    if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || !p) return GDN_ERR_HIP;
    ptrs[dev] = static_cast<char*>(p);
  }
  *out = ptrs[dev];
  return GDN_OK;
}

// Sequences whose resync chunk factors fit the fixed scratch together (at most
// N; 0 if not even one sequence's do).
int32_t noalloc_group(const gdn_shape_t* s, int32_t N) {
  constexpr size_t cap = GDN_NOALLOC_SCRATCH_BYTES;
  const size_t per = static_cast<size_t>(s->H_v) * s->C * (2 * static_cast<size_t>(s->d_k) + 1) * 4;
  int64_t m = static_cast<int64_t>(cap / per);
  if (m > N) m = N;
  while (m > 0 && gdn::layout(s, static_cast<int32_t>(m), 0, GDN_OP_DECODE).total > cap) --m;
  return static_cast<int32_t>(m);
}

// Calls f.template operator()<D, C, TIn>() for the shape's compiled variant.
template <typename F>
int dispatch(const gdn_shape_t* s, F&& f) {
  if (s->d_k == 128 && s->C == 64) {
    if (s->in_dtype == GDN_BF16) return f.template operator()<128, 64, bf16_t>();
    return f.template operator()<128, 64, float>();
  }
  if (s->d_k == 16 && s->C == 16) {
    if (s->in_dtype == GDN_BF16) return f.template operator()<16, 16, bf16_t>();
    return f.template operator()<16, 16, float>();
  }
  return GDN_ERR_UNSUPPORTED;
}

// The host copy of cu_seqlens: the caller's, or, when cu_host is NULL, one
// read back from the device copy (a copy enqueued on the stream and waited
// for; the values are then validated like a caller's).
int host_cu(const int32_t* cu_dev, const int32_t* cu_host, int32_t N, hipStream_t st,
            std::vector<int32_t>& buf, const int32_t** out) {
  if (cu_host) {
    *out = cu_host;
    return GDN_OK;
  }
  if (N < 0 || !cu_dev) return GDN_ERR_INVALID_ARG;
  buf.assign(static_cast<size_t>(N) + 1, 0);
  if (hipMemcpyAsync(buf.data(), cu_dev, buf.size() * sizeof(int32_t), hipMemcpyDeviceToHost,
                     st) != hipSuccess ||
      hipStreamSynchronize(st) != hipSuccess)
    return GDN_ERR_HIP;
  *out = buf.data();
  return GDN_OK;
}

}  // namespace

extern "C" {

size_t gdn_workspace_bytes(const gdn_shape_t* shape, int32_t n_seqs, int64_t total_tokens,
                           int32_t op) {
  if (gdn::check_shape(shape) != GDN_OK || n_seqs < 0) return 0;
  if (op == GDN_OP_DECODE) total_tokens = 0;
  if (total_tokens < 0) return 0;
  return gdn::layout(shape, n_seqs, total_tokens, op).total;
}

int gdn_cache_init(const gdn_shape_t* shape, int32_t n_seqs, const float* h0, gdn_cache_t* cache,
                   void* stream) {
  int rc = gdn::check_shape(shape);
  if (rc != GDN_OK) return rc;
  if (n_seqs < 0 || !gdn::aligned16({h0})) return GDN_ERR_INVALID_ARG;
  if ((rc = gdn::check_cache(cache)) != GDN_OK) return rc;
  if (n_seqs == 0) return GDN_OK;
  const int64_t n_state =
      static_cast<int64_t>(n_seqs) * shape->H_v * shape->d_k * static_cast<int64_t>(shape->d_v);
  const int64_t n_pos = static_cast<int64_t>(n_seqs) * shape->H_v;
  int64_t blocks = (n_state + 255) / 256;
  if (blocks > 65536) blocks = 65536;
  Timed t_("k_cache_init", static_cast<hipStream_t>(stream));
  hipLaunchKernelGGL(k_cache_init, dim3(static_cast<unsigned>(blocks)), dim3(256), 0,
                     static_cast<hipStream_t>(stream), h0, cache->S_run, cache->S_chunk,
                     cache->pos, n_state, n_pos);
  return hipGetLastError() == hipSuccess ? GDN_OK : GDN_ERR_HIP;
}

int gdn_prefill(const gdn_shape_t* shape, int32_t n_seqs, const int32_t* cu_seqlens_dev,
                const int32_t* cu_seqlens_host, const void* q, const void* k, const void* v,
                const float* beta, const float* g, const float* h0, float* o, float* hT,
                gdn_cache_t* cache, void* ws, size_t ws_bytes, void* stream) {
  int rc = gdn::check_shape(shape);
  if (rc != GDN_OK) return rc;
  if (n_seqs < 0 || !cu_seqlens_dev) return GDN_ERR_INVALID_ARG;
  if (!gdn::aligned16({q, k, v, beta, g, h0, o, hT})) return GDN_ERR_INVALID_ARG;
  if (cache && (rc = gdn::check_cache(cache)) != GDN_OK) return rc;
  std::vector<int32_t> cu_buf;
  if ((rc = host_cu(cu_seqlens_dev, cu_seqlens_host, n_seqs, static_cast<hipStream_t>(stream),
                    cu_buf, &cu_seqlens_host)) != GDN_OK)
    return rc;
  gdn::Counts cnt;
  if ((rc = gdn::count_chunks(cu_seqlens_host, n_seqs, shape->C, &cnt)) != GDN_OK) return rc;
  if (cnt.T > 0 && (!q || !k || !v || !beta || !g || !o)) return GDN_ERR_INVALID_ARG;
  const gdn::Layout L = gdn::layout(shape, n_seqs, cnt.T, GDN_OP_PREFILL);
  if (!ws || ws_bytes < L.total) return GDN_ERR_WORKSPACE;
  if (n_seqs == 0) return GDN_OK;
  hipStream_t st = static_cast<hipStream_t>(stream);
  char* w = static_cast<char*>(ws);
  return dispatch(shape, [&]<int D, int C, typename TIn>() {
    return launch_prefill<D, C, TIn>(shape, n_seqs, cnt, L, cu_seqlens_dev, q, k, v, beta, g, h0,
                                     o, hT, cache, w, st);
  });
}

int gdn_prefill_continue(const gdn_shape_t* shape, int32_t n_seqs, const int32_t* cu_seqlens_dev,
                         const int32_t* cu_seqlens_host, const int32_t* pos_host, const void* q,
                         const void* k, const void* v, const float* beta, const float* g,
                         gdn_cache_t* cache, float* o, float* hT, void* ws, size_t ws_bytes,
                         void* stream) {
  int rc = gdn::check_shape(shape);
  if (rc != GDN_OK) return rc;
  if (n_seqs < 0 || !cu_seqlens_dev || (n_seqs > 0 && !pos_host)) return GDN_ERR_INVALID_ARG;
  if ((rc = gdn::check_cache(cache)) != GDN_OK) return rc;
  if (!gdn::aligned16({q, k, v, beta, g, o, hT})) return GDN_ERR_INVALID_ARG;
  std::vector<int32_t> cu_buf;
  if ((rc = host_cu(cu_seqlens_dev, cu_seqlens_host, n_seqs, static_cast<hipStream_t>(stream),
                    cu_buf, &cu_seqlens_host)) != GDN_OK)
    return rc;
  gdn::Counts cnt;
  if ((rc = gdn::count_chunks(cu_seqlens_host, n_seqs, shape->C, &cnt)) != GDN_OK) return rc;
  if (cnt.T > 0 && (!q || !k || !v || !beta || !g || !o)) return GDN_ERR_INVALID_ARG;
  // the extended batch: each sequence's buffered tokens, then its new ones
  std::vector<int32_t> cux(static_cast<size_t>(n_seqs) + 1, 0);
  for (int32_t n = 0; n < n_seqs; ++n) {
    const int32_t p = pos_host[n];
    if (p < 0 || p >= shape->C) return GDN_ERR_INVALID_ARG;
    const int64_t e = static_cast<int64_t>(cux[n]) + p + (cu_seqlens_host[n + 1] - cu_seqlens_host[n]);
    if (e > INT32_MAX) return GDN_ERR_INVALID_ARG;
    cux[n + 1] = static_cast<int32_t>(e);
  }
  gdn::Counts cntx;
  if ((rc = gdn::count_chunks(cux.data(), n_seqs, shape->C, &cntx)) != GDN_OK) return rc;
  const gdn::Layout L = gdn::layout(shape, n_seqs, cnt.T, GDN_OP_PREFILL_CONTINUE);
  if (!ws || ws_bytes < L.total) return GDN_ERR_WORKSPACE;
  if (n_seqs == 0) return GDN_OK;
  hipStream_t st = static_cast<hipStream_t>(stream);
  char* w = static_cast<char*>(ws);
  return dispatch(shape, [&]<int D, int C, typename TIn>() {
    return launch_prefill_continue<D, C, TIn>(shape, n_seqs, cnt, cntx, L, cu_seqlens_dev, q, k, v,
                                              beta, g, cache, o, hT, w, st);
  });
}

}  // extern "C"

namespace {
// Argument checks shared by the two decode entry points; *resync tells
// whether some sequence may complete its chunk (always, without pos_host).
int check_decode(const gdn_shape_t* shape, int32_t n_seqs, const void* q, const void* k,
                 const void* v, const float* beta, const float* g, const gdn_cache_t* cache,
                 const int32_t* pos_host, const float* o, bool* resync) {
  int rc = gdn::check_shape(shape);
  if (rc != GDN_OK) return rc;
  if (n_seqs < 0) return GDN_ERR_INVALID_ARG;
  if ((rc = gdn::check_cache(cache)) != GDN_OK) return rc;
  if (n_seqs > 0 && (!q || !k || !v || !beta || !g || !o)) return GDN_ERR_INVALID_ARG;
  if (!gdn::aligned16({q, k, v, beta, g, o})) return GDN_ERR_INVALID_ARG;
  if (n_seqs > 65535) return GDN_ERR_UNSUPPORTED;  // grid.x of the per-sequence launches
  *resync = true;
  if (pos_host) {
    *resync = false;
    const int64_t np = static_cast<int64_t>(n_seqs) * shape->H_v;
    for (int64_t e = 0; e < np; ++e) {
      if (pos_host[e] < 0 || pos_host[e] >= shape->C) return GDN_ERR_INVALID_ARG;
      if (pos_host[e] + 1 == shape->C) *resync = true;
    }
  }
  return GDN_OK;
}
}  // namespace

extern "C" {

int gdn_decode_step(const gdn_shape_t* shape, int32_t n_seqs, const void* q, const void* k,
                    const void* v, const float* beta, const float* g, gdn_cache_t* cache,
                    const int32_t* pos_host, float* o, void* ws, size_t ws_bytes, void* stream) {
  bool resync = true;
  int rc = check_decode(shape, n_seqs, q, k, v, beta, g, cache, pos_host, o, &resync);
  if (rc != GDN_OK) return rc;
  const gdn::Layout L = gdn::layout(shape, n_seqs, 0, GDN_OP_DECODE);
  if (!ws || ws_bytes < L.total) return GDN_ERR_WORKSPACE;
  if (n_seqs == 0) return GDN_OK;
  hipStream_t st = static_cast<hipStream_t>(stream);
  char* w = static_cast<char*>(ws);
  return dispatch(shape, [&]<int D, int C, typename TIn>() {
    return launch_decode<D, C, TIn>(shape, n_seqs, L, q, k, v, beta, g, cache, resync, o, w, st);
  });
}

int gdn_decode_step_noalloc(const gdn_shape_t* shape, int32_t n_seqs, const void* q,
                            const void* k, const void* v, const float* beta, const float* g,
                            gdn_cache_t* cache, const int32_t* pos_host, float* o, void* stream) {
  bool resync = true;
  int rc = check_decode(shape, n_seqs, q, k, v, beta, g, cache, pos_host, o, &resync);
  if (rc != GDN_OK) return rc;
  if (n_seqs == 0) return GDN_OK;
  const int32_t group = noalloc_group(shape, n_seqs);
  if (group < 1) return GDN_ERR_WORKSPACE;  // one sequence's resync exceeds the scratch
  char* scr = nullptr;
  if ((rc = scratch_ptr(&scr)) != GDN_OK) return rc;
  const gdn::Layout Lg = gdn::layout(shape, group, 0, GDN_OP_DECODE);
  hipStream_t st = static_cast<hipStream_t>(stream);
  return dispatch(shape, [&]<int D, int C, typename TIn>() {
    return launch_decode_noalloc<D, C, TIn>(shape, n_seqs, group, Lg, q, k, v, beta, g, cache,
                                            resync, pos_host, o, scr, st);
  });
}

}  // extern "C"

namespace {
int fwd_bwd_entry(const gdn_shape_t* shape, int32_t n_seqs, const int32_t* cu_seqlens_dev,
                  const int32_t* cu_seqlens_host, const void* q, const void* k, const void* v,
                  const float* beta, const float* g, const float* h0, const float* dO,
                  const float* dhT, float* o, float* hT, int32_t grad_dtype, void* dq, void* dk,
                  void* dv, float* dbeta, float* dg, float* dh0, void* ws, size_t ws_bytes,
                  void* stream, bool native) {
  int rc = gdn::check_shape(shape);
  if (rc != GDN_OK) return rc;
  if (native && shape->d_k != 128) return GDN_ERR_UNSUPPORTED;
  if (grad_dtype != GDN_F32 && grad_dtype != GDN_BF16) return GDN_ERR_INVALID_ARG;
  if (n_seqs < 0 || !cu_seqlens_dev) return GDN_ERR_INVALID_ARG;
  if (n_seqs > 0 && (!hT || !dh0)) return GDN_ERR_INVALID_ARG;
  if (!gdn::aligned16({q, k, v, beta, g, h0, dO, dhT, o, hT, dq, dk, dv, dbeta, dg, dh0}))
    return GDN_ERR_INVALID_ARG;
  std::vector<int32_t> cu_buf;
  if ((rc = host_cu(cu_seqlens_dev, cu_seqlens_host, n_seqs, static_cast<hipStream_t>(stream),
                    cu_buf, &cu_seqlens_host)) != GDN_OK)
    return rc;
  gdn::Counts cnt;
  if ((rc = gdn::count_chunks(cu_seqlens_host, n_seqs, shape->C, &cnt)) != GDN_OK) return rc;
  if (cnt.T > 0 && (!q || !k || !v || !beta || !g || !o || !dO || !dq || !dk || !dv || !dbeta ||
                    !dg))
    return GDN_ERR_INVALID_ARG;
  const gdn::Layout L = gdn::layout(shape, n_seqs, cnt.T, GDN_OP_FWD_BWD);
  if (!ws || ws_bytes < L.total) return GDN_ERR_WORKSPACE;
  if (n_seqs == 0) return GDN_OK;
  hipStream_t st = static_cast<hipStream_t>(stream);
  char* w = static_cast<char*>(ws);
  const int bf16 = grad_dtype == GDN_BF16 ? 1 : 0;
  return dispatch(shape, [&]<int D, int C, typename TIn>() {
    return launch_fwd_bwd<D, C, TIn>(shape, n_seqs, cnt, L, cu_seqlens_dev, q, k, v, beta, g, h0,
                                     dO, dhT, o, hT, dq, dk, dv, bf16, dbeta, dg, dh0, w, st,
                                     native);
  });
}
}  // namespace

extern "C" {

int gdn_fwd_bwd_ex(const gdn_shape_t* shape, int32_t n_seqs, const int32_t* cu_seqlens_dev,
                   const int32_t* cu_seqlens_host, const void* q, const void* k, const void* v,
                   const float* beta, const float* g, const float* h0, const float* dO,
                   const float* dhT, float* o, float* hT, int32_t grad_dtype, void* dq, void* dk,
                   void* dv, float* dbeta, float* dg, float* dh0, void* ws, size_t ws_bytes,
                   void* stream) {
  return fwd_bwd_entry(shape, n_seqs, cu_seqlens_dev, cu_seqlens_host, q, k, v, beta, g, h0, dO,
                       dhT, o, hT, grad_dtype, dq, dk, dv, dbeta, dg, dh0, ws, ws_bytes, stream,
                       false);
}

int gdn_fwd_bwd_chunked(const gdn_shape_t* shape, int32_t n_seqs, const int32_t* cu_seqlens_dev,
                        const int32_t* cu_seqlens_host, const void* q, const void* k,
                        const void* v, const float* beta, const float* g, const float* h0,
                        const float* dO, const float* dhT, float* o, float* hT, float* dq,
                        float* dk, float* dv, float* dbeta, float* dg, float* dh0, void* ws,
                        size_t ws_bytes, void* stream) {
  return fwd_bwd_entry(shape, n_seqs, cu_seqlens_dev, cu_seqlens_host, q, k, v, beta, g, h0, dO,
                       dhT, o, hT, GDN_F32, dq, dk, dv, dbeta, dg, dh0, ws, ws_bytes, stream, true);
}

int gdn_decode_step_native(const gdn_shape_t* shape, int32_t n_seqs, const void* q, const void* k,
                           const void* v, const float* beta, const float* g, float* S, float* o,
                           void* stream) {
  int rc = gdn::check_shape(shape);
  if (rc != GDN_OK) return rc;
  if (n_seqs < 0) return GDN_ERR_INVALID_ARG;
  if (n_seqs > 0 && (!q || !k || !v || !beta || !g || !S || !o)) return GDN_ERR_INVALID_ARG;
  if (!gdn::aligned16({q, k, v, beta, g, S, o})) return GDN_ERR_INVALID_ARG;
  if (n_seqs > 65535) return GDN_ERR_UNSUPPORTED;  // grid.x
  if (n_seqs == 0) return GDN_OK;
  hipStream_t st = static_cast<hipStream_t>(stream);
  return dispatch(shape, [&]<int D, int C, typename TIn>() {
    return launch_decode_native<D, C, TIn>(shape, n_seqs, q, k, v, beta, g, S, o, st);
  });
}

int gdn_fwd_bwd(const gdn_shape_t* shape, int32_t n_seqs, const int32_t* cu_seqlens_dev,
                const int32_t* cu_seqlens_host, const void* q, const void* k, const void* v,
                const float* beta, const float* g, const float* h0, const float* dO,
                const float* dhT, float* o, float* hT, float* dq, float* dk, float* dv,
                float* dbeta, float* dg, float* dh0, void* ws, size_t ws_bytes, void* stream) {
  return gdn_fwd_bwd_ex(shape, n_seqs, cu_seqlens_dev, cu_seqlens_host, q, k, v, beta, g, h0, dO,
                        dhT, o, hT, GDN_F32, dq, dk, dv, dbeta, dg, dh0, ws, ws_bytes, stream);
}

int gdn_prefill_chunked(const gdn_shape_t* shape, int32_t n_seqs, const int32_t* cu_seqlens_dev,
                        const int32_t* cu_seqlens_host, const void* q, const void* k,
                        const void* v, const float* beta, const float* g, const float* h0,
                        float* o, float* hT, void* ws, size_t ws_bytes, void* stream) {
  int rc = gdn::check_shape(shape);
  if (rc != GDN_OK) return rc;
  if (shape->d_k != 128) return GDN_ERR_UNSUPPORTED;
  if (n_seqs < 0 || !cu_seqlens_dev) return GDN_ERR_INVALID_ARG;
  if (!gdn::aligned16({q, k, v, beta, g, h0, o, hT})) return GDN_ERR_INVALID_ARG;
  std::vector<int32_t> cu_buf;
  if ((rc = host_cu(cu_seqlens_dev, cu_seqlens_host, n_seqs, static_cast<hipStream_t>(stream),
                    cu_buf, &cu_seqlens_host)) != GDN_OK)
    return rc;
  gdn::Counts cnt;
  if ((rc = gdn::count_chunks(cu_seqlens_host, n_seqs, shape->C, &cnt)) != GDN_OK) return rc;
  if (cnt.T > 0 && (!q || !k || !v || !beta || !g || !o)) return GDN_ERR_INVALID_ARG;
  const gdn::Layout L = gdn::layout(shape, n_seqs, cnt.T, GDN_OP_PREFILL_CHUNKED);
  if (!ws || ws_bytes < L.total) return GDN_ERR_WORKSPACE;
  if (n_seqs == 0) return GDN_OK;
  hipStream_t st = static_cast<hipStream_t>(stream);
  char* w = static_cast<char*>(ws);
  return dispatch(shape, [&]<int D, int C, typename TIn>() {
    return launch_prefill_chunked<D, C, TIn>(shape, n_seqs, cnt, L, cu_seqlens_dev, q, k, v, beta,
                                             g, h0, o, hT, w, st);
  });
}

int gdn_profile_enable(int on) {
  Profiler& p = prof();
  std::lock_guard<std::mutex> g(p.mu);
  p.on = on != 0;
  return GDN_OK;
}

int gdn_profile_filter(const char* kernel) {
  Profiler& p = prof();
  std::lock_guard<std::mutex> g(p.mu);
  p.filter = kernel ? kernel : "";
  return GDN_OK;
}

int gdn_profile_read(const char* kernel, double* total_ms, int64_t* launches) {
  if (!total_ms || !launches) return GDN_ERR_INVALID_ARG;
  Profiler& p = prof();
  std::lock_guard<std::mutex> g(p.mu);
  double ms = 0.0;
  int64_t cnt = 0;
  int rc = GDN_OK;
  std::vector<ProfRec> keep;
  for (const ProfRec& r : p.recs) {
    const bool match = !kernel || !kernel[0] || std::strstr(r.name, kernel) != nullptr;
    if (!match) {
      keep.push_back(r);
      continue;
    }
    float t = 0.0f;
    if (hipEventSynchronize(r.b) != hipSuccess || hipEventElapsedTime(&t, r.a, r.b) != hipSuccess)
      rc = GDN_ERR_HIP;
    ms += t;
    ++cnt;
    p.pool.push_back(r.a);
    p.pool.push_back(r.b);
  }
  p.recs.swap(keep);
  *total_ms = ms;
  *launches = cnt;
  return rc;
}

const char* gdn_contract_id(void) {
  return "gdn-cpr/v11;eps=1e-6;claims=d16C16,d128C64;R=lane-row,dk-halves-at-d128,fmaf-asc,o-after-update;"
         "B=mfma16x16x4-wy-blocked16-diaginv,bf16x3-mfma16x16x32-scan-regB;prep=wave-butterfly;"
         "bwd=bf16x3-mfma16x16x32-scan-stateproducts-Z;src=" GDN_SOURCE_DIGEST;
}

int gdn_contract_check(const char* id) {
  if (!id) return GDN_ERR_INVALID_ARG;
  return std::strcmp(id, gdn_contract_id()) == 0 ? GDN_OK : GDN_ERR_UNSUPPORTED;
}

const char* gdn_error_string(int status) {
  switch (status) {
    case GDN_OK: return "ok";
    case GDN_ERR_INVALID_ARG: return "invalid argument";
    case GDN_ERR_UNSUPPORTED: return "shape outside the compiled claims";
    case GDN_ERR_WORKSPACE: return "workspace missing or too small";
    case GDN_ERR_HIP: return "HIP runtime error";
    default: return "unknown status";
  }
}

}  // extern "C"
