// Host-side argument validation and workspace layout.  Pure C++ (no HIP), so
// the same code is built into libgdn.so and into a sanitizer-instrumented
// host test.
#pragma once

#include <cstddef>
#include <cstdint>
#include <initializer_list>

#include "gdn.h"

namespace gdn {

constexpr float kNormEps = 1e-6f;  // inside the L2 norm: x / sqrt(sum x^2 + eps)
constexpr size_t kAlign = 256;     // every workspace region starts on 256 bytes

// Shapes the library is compiled for (the "claims"): d_k == d_v == d, chunk C.
struct Claim {
  int d, C;
};
constexpr Claim kClaims[] = {{16, 16}, {128, 64}};

// Per-call counts derived from cu_seqlens on the host.
struct Counts {
  int64_t T = 0;       // total tokens
  int64_t chunks = 0;  // sum over sequences of ceil(L / C)
  int64_t full = 0;    // sum over sequences of floor(L / C)
};

// Byte offsets of the regions of one call's workspace.  A region of size 0 is
// absent.  Slots are indexed by "chunk slot": prefix sum over sequences of
// their chunk counts (all chunks for states, full chunks for W/U/G).
struct Layout {
  size_t cu_chunks = 0;  // int32 [N+1]  prefix of ceil(L/C)
  size_t cu_full = 0;    // int32 [N+1]  prefix of floor(L/C)
  size_t qk = 0;         // f32 [H_qk, T, 2, d]  normalised k, q per token
  size_t W = 0;          // f32 [full_slots, H_v, C, d]
  size_t U = 0;          // f32 [full_slots, H_v, C, d]
  size_t G = 0;          // f32 [full_slots, H_v, C]
  size_t states = 0;     // f32 [state_slots, H_v, d, d]  chunk-start states
  size_t order = 0;      // int32 [N]  sequences longest first (chunk scan)
  size_t gb = 0;         // f32 [H_v, T, 2]  (g, beta) of each value head in token order
  // trainer forward + backward only (W, U, G then use chunk slots)
  size_t Dl = 0;         // f32 [state_slots, H_v, C, d]  Delta = U - W S^T
  size_t E = 0;          // f32 [state_slots, H_v, C, d]  P^T dO
  size_t dstates = 0;    // f32 [state_slots, H_v, d, d]  gradient at chunk ends
  size_t dD = 0;         // f32 [state_slots, H_v, C, d]  dDelta, then dX_u
  size_t SdO = 0;        // f32 [state_slots, H_v, C, d]
  size_t DsD = 0;        // f32 [state_slots, H_v, C, d]
  size_t SdD = 0;        // f32 [state_slots, H_v, C, d]  then dX_w
  size_t dqv = 0;        // f32 [T, H_v, d]  per value head dq-hat
  size_t dkv = 0;        // f32 [T, H_v, d]  per value head dk-hat
  // prefill continuation only: the extended batch (buffered + new tokens of
  // every sequence, T' <= T + N (C - 1) rows) and its outputs
  size_t cu_ext = 0;     // int32 [N+1]  prefix of buffered + new tokens
  size_t v_ext = 0;      // in_dtype [T', H_v, d]
  size_t b_ext = 0;      // f32 [T', H_v]
  size_t g_ext = 0;      // f32 [T', H_v]
  size_t o_ext = 0;      // f32 [T', H_v, d]
  size_t total = 0;
  int64_t full_slots = 0, state_slots = 0;
};

// GDN_OK, GDN_ERR_INVALID_ARG or GDN_ERR_UNSUPPORTED.
int check_shape(const gdn_shape_t* s);

// Validates cu_seqlens on the host (starts at 0, non-decreasing) and counts
// tokens and chunks.  GDN_OK or GDN_ERR_INVALID_ARG.
int count_chunks(const int32_t* cu_host, int32_t n_seqs, int32_t C, Counts* out);

// Workspace layout for an op, sized from (n_seqs, total_tokens) only, so that
// gdn_workspace_bytes needs no cu_seqlens: slots are bounded by T/C + N.
Layout layout(const gdn_shape_t* s, int32_t n_seqs, int64_t total_tokens, int op);

// Checks the pointer fields of a decode cache (all must be non-NULL).
int check_cache(const gdn_cache_t* c);
// True if every pointer is 16-byte aligned (NULL counts as aligned).
bool aligned16(std::initializer_list<const void*> ptrs);

}  // namespace gdn
