// Host-side validation and workspace layout (pure C++).
#include "gdn_plan.h"

#include <cmath>
#include <limits>

namespace gdn {

int check_shape(const gdn_shape_t* s) {
  if (!s) return GDN_ERR_INVALID_ARG;
  if (s->H_qk <= 0 || s->H_v <= 0 || s->d_k <= 0 || s->d_v <= 0 || s->C <= 0)
    return GDN_ERR_INVALID_ARG;
  if (s->qk_l2norm != 0 && s->qk_l2norm != 1) return GDN_ERR_INVALID_ARG;
  if (!std::isfinite(s->scale)) return GDN_ERR_INVALID_ARG;
  if (s->in_dtype != GDN_F32 && s->in_dtype != GDN_BF16) return GDN_ERR_UNSUPPORTED;
  if (s->H_v % s->H_qk != 0) return GDN_ERR_UNSUPPORTED;
  if (s->H_v / s->H_qk > 8) return GDN_ERR_UNSUPPORTED;  // token-step block: <= 16 waves
  if (s->d_k != s->d_v) return GDN_ERR_UNSUPPORTED;
  // keep every [.., H, d] row offset well inside 32 bits per token
  if (static_cast<int64_t>(s->H_v) * s->d_v > (1 << 20)) return GDN_ERR_UNSUPPORTED;
  for (const Claim& c : kClaims)
    if (c.d == s->d_k && c.C == s->C) return GDN_OK;
  return GDN_ERR_UNSUPPORTED;
}

int count_chunks(const int32_t* cu, int32_t n_seqs, int32_t C, Counts* out) {
  if (!cu || !out || n_seqs < 0 || C <= 0) return GDN_ERR_INVALID_ARG;
  if (cu[0] != 0) return GDN_ERR_INVALID_ARG;
  Counts r;
  for (int32_t n = 0; n < n_seqs; ++n) {
    const int64_t L = static_cast<int64_t>(cu[n + 1]) - cu[n];
    if (L < 0) return GDN_ERR_INVALID_ARG;
    r.chunks += (L + C - 1) / C;
    r.full += L / C;
  }
  r.T = cu[n_seqs];
  *out = r;
  return GDN_OK;
}

static size_t take(size_t* cursor, size_t bytes) {
  const size_t at = *cursor;
  *cursor += (bytes + kAlign - 1) / kAlign * kAlign;
  return at;
}

Layout layout(const gdn_shape_t* s, int32_t N, int64_t T, int op) {
  Layout L;
  if (check_shape(s) != GDN_OK || N < 0 || T < 0) return L;
  const size_t d = static_cast<size_t>(s->d_k), C = static_cast<size_t>(s->C);
  const size_t Hq = static_cast<size_t>(s->H_qk), Hv = static_cast<size_t>(s->H_v);
  const size_t f = sizeof(float);
  size_t cur = kAlign;  // offset 0 is never handed out
  if (op == GDN_OP_DECODE) {
    L.full_slots = N;
    L.state_slots = 0;
    L.W = take(&cur, N * Hv * C * d * f);
    L.U = take(&cur, N * Hv * C * d * f);
    L.G = take(&cur, N * Hv * C * f);
    L.total = cur;
    return L;
  }
  if (op != GDN_OP_PREFILL && op != GDN_OP_FWD_BWD && op != GDN_OP_PREFILL_CHUNKED &&
      op != GDN_OP_PREFILL_CONTINUE)
    return Layout{};
  // the continuation re-runs each sequence's up to C - 1 buffered tokens
  if (op == GDN_OP_PREFILL_CONTINUE) T += static_cast<int64_t>(N) * (static_cast<int64_t>(C) - 1);
  const bool all_chunks = op != GDN_OP_PREFILL && op != GDN_OP_PREFILL_CONTINUE;
  L.full_slots = T / static_cast<int64_t>(C);
  L.state_slots = T / static_cast<int64_t>(C) + N;
  L.cu_chunks = take(&cur, (N + 1) * sizeof(int32_t));
  L.cu_full = take(&cur, (N + 1) * sizeof(int32_t));
  // two spare token rows: the token step reads (prefetches) up to two tokens
  // past the end of a chunk; those values are never used
  L.qk = take(&cur, (T * Hq + 2) * 2 * d * f);
  const int64_t wu_slots = all_chunks ? L.state_slots : L.full_slots;
  L.W = take(&cur, wu_slots * Hv * C * d * f);
  L.U = take(&cur, wu_slots * Hv * C * d * f);
  L.G = take(&cur, wu_slots * Hv * C * f);
  L.states = take(&cur, L.state_slots * Hv * d * d * f);
  L.order = take(&cur, static_cast<size_t>(N) * sizeof(int32_t) + 1);
  if (op != GDN_OP_PREFILL_CHUNKED) L.gb = take(&cur, T * Hv * 2 * f);  // read by the token step
  if (op == GDN_OP_PREFILL_CHUNKED) L.Dl = take(&cur, L.state_slots * Hv * C * d * f);
  if (op == GDN_OP_FWD_BWD) {
    const size_t cd = L.state_slots * Hv * C * d * f;
    L.Dl = take(&cur, cd);
    L.E = take(&cur, cd);
    L.dstates = take(&cur, L.state_slots * Hv * d * d * f);
    L.dD = take(&cur, cd);
    if (d != 128) {  // at d = 128 the backward chunk kernel forms these itself
      L.SdO = take(&cur, cd);
      L.DsD = take(&cur, cd);
      L.SdD = take(&cur, cd);
    }
    L.dqv = take(&cur, T * Hv * d * f);
    L.dkv = take(&cur, T * Hv * d * f);
  }
  if (op == GDN_OP_PREFILL_CONTINUE) {
    const size_t in = s->in_dtype == GDN_BF16 ? 2 : 4;
    L.cu_ext = take(&cur, (N + 1) * sizeof(int32_t));
    L.v_ext = take(&cur, T * Hv * d * in);
    L.b_ext = take(&cur, T * Hv * f);
    L.g_ext = take(&cur, T * Hv * f);
    L.o_ext = take(&cur, T * Hv * d * f);
  }
  L.total = cur;
  return L;
}

int check_cache(const gdn_cache_t* c) {
  if (!c || !c->S_run || !c->S_chunk || !c->kbuf || !c->vbuf || !c->bbuf || !c->gbuf ||
      !c->pos)
    return GDN_ERR_INVALID_ARG;
  if (!aligned16({c->S_run, c->S_chunk, c->kbuf, c->vbuf, c->bbuf, c->gbuf, c->pos}))
    return GDN_ERR_INVALID_ARG;
  return GDN_OK;
}

bool aligned16(std::initializer_list<const void*> ptrs) {
  for (const void* p : ptrs)
    if ((reinterpret_cast<uintptr_t>(p) & 15u) != 0) return false;  // NULL passes
  return true;
}

}  // namespace gdn
