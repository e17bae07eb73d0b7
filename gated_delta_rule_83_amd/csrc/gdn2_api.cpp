// gdn2_api.cpp -- the C ABI of libgdn2 (include/gdn2.h): argument checks,
// then a launch on the caller's stream. Nothing here allocates device memory
// or keeps state between calls.
#include "gdn2.h"

#include <stdint.h>

#include "gdn2_internal.hpp"
#include "gdn2_range.hpp"

namespace {

bool supported_dim(int d) { return d == 16 || d == 32 || d == 64 || d == 128; }
bool supported_chunk(int c) { return c == 16 || c == 32 || c == 64; }

struct Range {
  uintptr_t lo, hi;  // [lo, hi)
};

Range range_of(const void *p, size_t bytes) {
  const uintptr_t lo = reinterpret_cast<uintptr_t>(p);
  return Range{lo, lo + bytes};
}

bool overlaps(Range x, Range y) {
  return x.lo != x.hi && y.lo != y.hi && x.lo < y.hi && y.lo < x.hi;
}

bool aligned16(const void *p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }
// One fp32 per token and value head (beta, alpha and their gradients) is read
// and written as single floats: 4-byte alignment, so that a view starting at
// any token of a [T, H_v] tensor is accepted.
bool aligned4(const void *p) { return (reinterpret_cast<uintptr_t>(p) & 3u) == 0; }

// Common description checks; `decode` additionally requires T == 1.
gdn2_status check_desc(const gdn2_desc *d, bool decode) {
  if (!d) return GDN2_ERR_NULL_POINTER;
  if (d->dtype != GDN2_F32 && d->dtype != GDN2_BF16) return GDN2_ERR_BAD_DTYPE;
  if (d->B < 0 || d->T < 0 || d->H_qk < 1 || d->H_v < 1 || d->d_k < 1 || d->d_v < 1 ||
      d->chunk < 1)
    return GDN2_ERR_BAD_SHAPE;
  if (d->H_v % d->H_qk != 0) return GDN2_ERR_BAD_SHAPE;
  if (decode && d->T != 1) return GDN2_ERR_BAD_SHAPE;
  if (!supported_dim(d->d_k) || !supported_dim(d->d_v)) return GDN2_ERR_UNSUPPORTED;
  if (!decode && !supported_chunk(d->chunk)) return GDN2_ERR_UNSUPPORTED;
  // the prefill's buffer descriptors span one chunk of token rows: the
  // widest row times the longest chunk must fit their 31-bit range
  if (!decode && !gdn2::window_fits(d->H_qk, d->H_v, d->d_k, d->d_v)) return GDN2_ERR_UNSUPPORTED;
  return GDN2_OK;
}

}  // namespace

extern "C" {

int gdn2_version(void) { return 10000; }

const char *gdn2_status_string(gdn2_status s) {
  switch (s) {
    case GDN2_OK: return "ok";
    case GDN2_ERR_NULL_POINTER: return "a required pointer is NULL";
    case GDN2_ERR_BAD_SHAPE: return "invalid shape, or a tensor pointer not 16-byte aligned";
    case GDN2_ERR_UNSUPPORTED: return "unsupported head dimension or chunk length, or token rows too wide for a chunk's buffer range";
    case GDN2_ERR_BAD_DTYPE: return "unknown dtype";
    case GDN2_ERR_WORKSPACE: return "workspace too small";
    case GDN2_ERR_HIP: return "HIP runtime error at launch";
    case GDN2_ERR_ALIAS: return "output or workspace overlaps an input, the state or each other";
    case GDN2_ERR_SCRATCH: return "the problem needs more scratch than the allocation-free entry point's static buffer";
  }
  return "unknown status";
}

namespace {

gdn2::PrefillArgs prefill_args(const gdn2_desc *d) {
  gdn2::PrefillArgs p{};
  p.B = d->B; p.T = d->T; p.H_qk = d->H_qk; p.H_v = d->H_v; p.d_k = d->d_k; p.d_v = d->d_v;
  p.chunk = d->chunk;
  p.bf16 = d->dtype == GDN2_BF16;
  p.nct = gdn2::prefill_pick_nct(d->B, d->H_v, d->d_v);
  return p;
}

gdn2_status backward_general(const gdn2_desc *d, const int32_t *cu, const void *q, const void *k, const void *v,
                             const void *a, const void *b, const void *w, const float *S0, const void *dO,
                             const float *dS_T, void *dq, void *dk, void *dv, void *da, void *db, void *dw,
                             float *dS0, void *workspace, size_t workspace_bytes, void *stream, bool varlen,
                             int form);

// gdn2_chunk_forward and gdn2_chunk_forward_preact: per-channel gates, fp32
// activated values or pre-activations in the input dtype. ws_cap: largest
// workspace the split may plan for (0: no limit).
gdn2_status forward_general(const gdn2_desc *d, const void *q, const void *k, const void *v, const void *a,
                            const void *b, const void *w, const float *S0, void *o, float *S_T, void *workspace,
                            size_t workspace_bytes, void *stream, bool preact, size_t ws_cap = 0);

size_t workspace_bytes_capped(const gdn2_desc *desc, size_t ws_cap) {
  if (check_desc(desc, false) != GDN2_OK) return 0;
  gdn2::PrefillArgs a = prefill_args(desc);
  a.ws_cap = ws_cap;
  return gdn2::prefill_plan(a).ws_bytes;
}

}  // namespace

size_t gdn2_chunk_forward_workspace_bytes(const gdn2_desc *desc) {
  // nonzero only when long sequences are split across workgroups
  return workspace_bytes_capped(desc, 0);
}

gdn2_status gdn2_chunk_forward_plan(const gdn2_desc *desc, int32_t *chunk_run, int32_t *segments) {
  const gdn2_status st = check_desc(desc, false);
  if (st != GDN2_OK) return st;
  const gdn2::PrefillPlan pl = gdn2::prefill_plan(prefill_args(desc));
  if (chunk_run) *chunk_run = pl.chunk;
  if (segments) *segments = pl.nseg;
  return GDN2_OK;
}

gdn2_status gdn2_chunk_forward(const gdn2_desc *d, const void *q, const void *k, const void *v,
                               const float *a, const float *b, const float *w, const float *S0,
                               void *o, float *S_T, void *workspace, size_t workspace_bytes,
                               void *stream) {
  return forward_general(d, q, k, v, a, b, w, S0, o, S_T, workspace, workspace_bytes, stream, false);
}

gdn2_status gdn2_chunk_forward_preact(const gdn2_desc *d, const void *q, const void *k, const void *v,
                                      const void *a_pre, const void *b_pre, const void *w_pre, const float *S0,
                                      void *o, float *S_T, void *workspace, size_t workspace_bytes,
                                      void *stream) {
  return forward_general(d, q, k, v, a_pre, b_pre, w_pre, S0, o, S_T, workspace, workspace_bytes, stream, true);
}

}  // extern "C"

namespace {

gdn2_status forward_general(const gdn2_desc *d, const void *q, const void *k, const void *v, const void *a,
                            const void *b, const void *w, const float *S0, void *o, float *S_T, void *workspace,
                            size_t workspace_bytes, void *stream, bool preact, size_t ws_cap) {
  gdn2_status st = check_desc(d, false);
  if (st != GDN2_OK) return st;
  const size_t ws_need = workspace_bytes_capped(d, ws_cap);
  if (ws_need > 0 && (!workspace || workspace_bytes < ws_need)) return GDN2_ERR_WORKSPACE;
  const size_t B = (size_t)d->B, T = (size_t)d->T, Hqk = (size_t)d->H_qk, Hv = (size_t)d->H_v;
  const size_t dk = (size_t)d->d_k, dv = (size_t)d->d_v;
  const size_t es = d->dtype == GDN2_BF16 ? 2 : 4;
  if (B == 0) return GDN2_OK;
  const bool tokens = T > 0;
  if (tokens && (!q || !k || !v || !a || !b || !w || !o)) return GDN2_ERR_NULL_POINTER;
  const void *ptrs[] = {q, k, v, a, b, w, S0, o, S_T};
  for (const void *p : ptrs)
    if (p && !aligned16(p)) return GDN2_ERR_BAD_SHAPE;

  const Range rq = range_of(q, B * T * Hqk * dk * es), rk = range_of(k, B * T * Hqk * dk * es);
  const Range rv = range_of(v, B * T * Hv * dv * es);
  const size_t gs = preact ? es : 4;  // gate element bytes
  const Range ra = range_of(a, B * T * Hv * dk * gs), rb = range_of(b, B * T * Hv * dk * gs);
  const Range rw = range_of(w, B * T * Hv * dv * gs);
  const Range ro = range_of(o, B * T * Hv * dv * es);
  const Range rs0 = range_of(S0, S0 ? B * Hv * dk * dv * 4 : 0);
  const Range rst = range_of(S_T, S_T ? B * Hv * dk * dv * 4 : 0);
  const Range ins[] = {rq, rk, rv, ra, rb, rw, rs0, rst};
  if (tokens)
    for (const Range &r : ins)
      if (overlaps(ro, r)) return GDN2_ERR_ALIAS;
  if (ws_need > 0) {
    if (!aligned16(workspace)) return GDN2_ERR_BAD_SHAPE;
    const Range rws = range_of(workspace, ws_need);
    for (const Range &r : ins)
      if (overlaps(rws, r)) return GDN2_ERR_ALIAS;
    if (overlaps(rws, ro)) return GDN2_ERR_ALIAS;
  }
  // S_T may alias S0 exactly (in-place), but not partially.
  if (S0 && S_T && overlaps(rs0, rst) && S0 != S_T) return GDN2_ERR_ALIAS;

  gdn2::PrefillArgs p = prefill_args(d);
  p.q = q; p.k = k; p.v = v; p.S0 = S0; p.o = o; p.S_T = S_T;
  p.a = static_cast<const float *>(a);  // pre-activations in the input dtype when preact
  p.b = static_cast<const float *>(b);
  p.w = static_cast<const float *>(w);
  p.preact = preact;
  p.workspace = workspace;
  p.workspace_bytes = workspace_bytes;
  p.ws_cap = ws_cap;
  const hipError_t e = gdn2::launch_prefill(p, reinterpret_cast<hipStream_t>(stream));
  return e == hipSuccess ? GDN2_OK : GDN2_ERR_HIP;
}

}  // namespace

namespace gdn2 {

// gdn2_chunk_forward with the split planned within a workspace of at most
// ws_cap bytes (the allocation-free entry point's static scratch).
size_t chunk_forward_workspace_capped(const gdn2_desc *desc, size_t ws_cap) {
  return workspace_bytes_capped(desc, ws_cap);
}

gdn2_status chunk_forward_capped(const gdn2_desc *d, const void *q, const void *k, const void *v, const float *a,
                                 const float *b, const float *w, const float *S0, void *o, float *S_T,
                                 void *workspace, size_t workspace_bytes, size_t ws_cap, void *stream) {
  return forward_general(d, q, k, v, a, b, w, S0, o, S_T, workspace, workspace_bytes, stream, false, ws_cap);
}

}  // namespace gdn2


namespace {

// Coupled gates (beta [B, T, H_v]); a is [B, T, H_v, d_k], or [B, T, H_v]
// with scalar_decay.
gdn2_status forward_scalar_gates(const gdn2_desc *d, const void *q, const void *k, const void *v,
                                 const float *a, const float *beta, const float *S0, void *o, float *S_T,
                                 void *workspace, size_t workspace_bytes, void *stream, bool scalar_decay) {
  gdn2_status st = check_desc(d, false);
  if (st != GDN2_OK) return st;
  const size_t ws_need = gdn2_chunk_forward_workspace_bytes(d);
  if (ws_need > 0 && (!workspace || workspace_bytes < ws_need)) return GDN2_ERR_WORKSPACE;
  const size_t B = (size_t)d->B, T = (size_t)d->T, Hqk = (size_t)d->H_qk, Hv = (size_t)d->H_v;
  const size_t dk = (size_t)d->d_k, dv = (size_t)d->d_v;
  const size_t es = d->dtype == GDN2_BF16 ? 2 : 4;
  if (B == 0) return GDN2_OK;
  const bool tokens = T > 0;
  if (tokens && (!q || !k || !v || !a || !beta || !o)) return GDN2_ERR_NULL_POINTER;
  const void *ptrs[] = {q, k, v, scalar_decay ? nullptr : a, S0, o, S_T};
  for (const void *p : ptrs)
    if (p && !aligned16(p)) return GDN2_ERR_BAD_SHAPE;
  if ((scalar_decay && a && !aligned4(a)) || (beta && !aligned4(beta))) return GDN2_ERR_BAD_SHAPE;
  const Range rq = range_of(q, B * T * Hqk * dk * es), rk = range_of(k, B * T * Hqk * dk * es);
  const Range rv = range_of(v, B * T * Hv * dv * es);
  const Range ra = range_of(a, B * T * Hv * (scalar_decay ? 1 : dk) * 4), rbeta = range_of(beta, B * T * Hv * 4);
  const Range ro = range_of(o, B * T * Hv * dv * es);
  const Range rs0 = range_of(S0, S0 ? B * Hv * dk * dv * 4 : 0);
  const Range rst = range_of(S_T, S_T ? B * Hv * dk * dv * 4 : 0);
  const Range ins[] = {rq, rk, rv, ra, rbeta, rs0, rst};
  if (tokens)
    for (const Range &r : ins)
      if (overlaps(ro, r)) return GDN2_ERR_ALIAS;
  if (S0 && S_T && overlaps(rs0, rst) && S0 != S_T) return GDN2_ERR_ALIAS;
  if (ws_need > 0) {
    if (!aligned16(workspace)) return GDN2_ERR_BAD_SHAPE;
    const Range rws = range_of(workspace, ws_need);
    for (const Range &r : ins)
      if (overlaps(rws, r)) return GDN2_ERR_ALIAS;
    if (overlaps(rws, ro)) return GDN2_ERR_ALIAS;
  }
  gdn2::PrefillArgs p = prefill_args(d);
  p.q = q; p.k = k; p.v = v; p.a = a; p.b = beta; p.w = beta; p.S0 = S0; p.o = o; p.S_T = S_T;
  p.workspace = workspace;
  p.workspace_bytes = workspace_bytes;
  p.coupled = true;
  p.scalar_decay = scalar_decay;
  const hipError_t e = gdn2::launch_prefill(p, reinterpret_cast<hipStream_t>(stream));
  return e == hipSuccess ? GDN2_OK : GDN2_ERR_HIP;
}

}  // namespace

extern "C" {

gdn2_status gdn2_chunk_forward_coupled(const gdn2_desc *d, const void *q, const void *k, const void *v,
                                       const float *a, const float *beta, const float *S0, void *o,
                                       float *S_T, void *workspace, size_t workspace_bytes, void *stream) {
  return forward_scalar_gates(d, q, k, v, a, beta, S0, o, S_T, workspace, workspace_bytes, stream, false);
}

gdn2_status gdn2_chunk_forward_scalar(const gdn2_desc *d, const void *q, const void *k, const void *v,
                                      const float *a, const float *beta, const float *S0, void *o,
                                      float *S_T, void *workspace, size_t workspace_bytes, void *stream) {
  return forward_scalar_gates(d, q, k, v, a, beta, S0, o, S_T, workspace, workspace_bytes, stream, true);
}

gdn2_status gdn2_chunk_forward_varlen(const gdn2_desc *d, const int32_t *cu_seqlens, const void *q,
                                      const void *k, const void *v, const float *a, const float *b,
                                      const float *w, const float *S0, void *o, float *S_T, void *stream) {
  return gdn2_chunk_forward_varlen_gates(d, cu_seqlens, GDN2_GATES_CHANNEL, q, k, v, a, b, w, S0, o, S_T, stream);
}

gdn2_status gdn2_chunk_forward_varlen_gates(const gdn2_desc *d, const int32_t *cu_seqlens, gdn2_gates gates,
                                            const void *q, const void *k, const void *v, const void *a,
                                            const void *b, const void *w, const float *S0, void *o, float *S_T,
                                            void *stream) {
  gdn2_status st = check_desc(d, false);
  if (st != GDN2_OK) return st;
  if (gates != GDN2_GATES_CHANNEL && gates != GDN2_GATES_PREACT && gates != GDN2_GATES_COUPLED &&
      gates != GDN2_GATES_SCALAR)
    return GDN2_ERR_UNSUPPORTED;
  const bool preact = gates == GDN2_GATES_PREACT;
  const bool coupled = gates == GDN2_GATES_COUPLED || gates == GDN2_GATES_SCALAR;
  const size_t B = (size_t)d->B, T = (size_t)d->T, Hqk = (size_t)d->H_qk, Hv = (size_t)d->H_v;
  const size_t dk = (size_t)d->d_k, dv = (size_t)d->d_v;
  const size_t es = d->dtype == GDN2_BF16 ? 2 : 4;
  if (B == 0) return GDN2_OK;
  if (!cu_seqlens) return GDN2_ERR_NULL_POINTER;
  const bool tokens = T > 0;
  if (tokens && (!q || !k || !v || !a || !b || !o)) return GDN2_ERR_NULL_POINTER;
  if (tokens && !coupled && !w) return GDN2_ERR_NULL_POINTER;
  if (coupled) w = nullptr;  // the write gate is beta
  const bool sa = gates == GDN2_GATES_SCALAR;  // a is one scalar per token and value head
  const void *ptrs[] = {q, k, v, sa ? nullptr : a, coupled ? nullptr : b, w, S0, o, S_T};
  for (const void *p : ptrs)
    if (p && !aligned16(p)) return GDN2_ERR_BAD_SHAPE;
  if ((sa && a && !aligned4(a)) || (coupled && b && !aligned4(b))) return GDN2_ERR_BAD_SHAPE;
  // token tensors hold T tokens in all (packed sequences); gate elements per
  // channel, or one per token and value head (beta; alpha in the scalar form)
  const size_t gs = preact ? es : 4;
  const size_t na = gates == GDN2_GATES_SCALAR ? T * Hv : T * Hv * dk, nb = coupled ? T * Hv : T * Hv * dk;
  const Range rq = range_of(q, T * Hqk * dk * es), rk = range_of(k, T * Hqk * dk * es);
  const Range rv = range_of(v, T * Hv * dv * es);
  const Range ra = range_of(a, na * gs), rb = range_of(b, nb * gs);
  const Range rw = range_of(w, coupled ? 0 : T * Hv * dv * gs);
  const Range ro = range_of(o, T * Hv * dv * es);
  const Range rs0 = range_of(S0, S0 ? B * Hv * dk * dv * 4 : 0);
  const Range rst = range_of(S_T, S_T ? B * Hv * dk * dv * 4 : 0);
  const Range rcu = range_of(cu_seqlens, (B + 1) * sizeof(int32_t));
  const Range ins[] = {rq, rk, rv, ra, rb, rw, rs0, rst, rcu};
  if (tokens)
    for (const Range &r : ins)
      if (overlaps(ro, r)) return GDN2_ERR_ALIAS;
  if (S_T && overlaps(rst, rcu)) return GDN2_ERR_ALIAS;
  if (S0 && S_T && overlaps(rs0, rst) && S0 != S_T) return GDN2_ERR_ALIAS;

  gdn2::PrefillArgs p = prefill_args(d);
  p.q = q; p.k = k; p.v = v; p.S0 = S0; p.o = o; p.S_T = S_T;
  p.a = static_cast<const float *>(a);  // input dtype when preact
  p.b = static_cast<const float *>(b);
  p.w = static_cast<const float *>(coupled ? b : w);
  p.coupled = coupled;
  p.scalar_decay = gates == GDN2_GATES_SCALAR;
  p.preact = preact;
  p.cu_seqlens = cu_seqlens;
  const hipError_t e = gdn2::launch_prefill(p, reinterpret_cast<hipStream_t>(stream));
  return e == hipSuccess ? GDN2_OK : GDN2_ERR_HIP;
}

gdn2_status gdn2_decode_step(const gdn2_desc *d, const void *q, const void *k, const void *v,
                             const float *a, const float *b, const float *w, float *S, void *o,
                             void *stream) {
  return gdn2_decode_step_gates(d, GDN2_GATES_CHANNEL, q, k, v, a, b, w, S, o, stream);
}

gdn2_status gdn2_decode_step_gates(const gdn2_desc *d, gdn2_gates gates, const void *q, const void *k,
                                   const void *v, const void *a, const void *b, const void *w, float *S, void *o,
                                   void *stream) {
  gdn2_status st = check_desc(d, true);
  if (st != GDN2_OK) return st;
  int form;
  switch (gates) {
    case GDN2_GATES_CHANNEL: form = gdn2::kGateGeneral; break;
    case GDN2_GATES_PREACT: form = gdn2::kGatePre; break;
    case GDN2_GATES_COUPLED: form = gdn2::kGateCoupled; break;
    case GDN2_GATES_SCALAR: form = gdn2::kGateScalar; break;
    default: return GDN2_ERR_UNSUPPORTED;
  }
  const bool coupled = form == gdn2::kGateCoupled || form == gdn2::kGateScalar;
  const bool sa = form == gdn2::kGateScalar;
  const size_t B = (size_t)d->B, Hqk = (size_t)d->H_qk, Hv = (size_t)d->H_v;
  const size_t dk = (size_t)d->d_k, dv = (size_t)d->d_v;
  const size_t es = d->dtype == GDN2_BF16 ? 2 : 4;
  if (B == 0) return GDN2_OK;
  if (!q || !k || !v || !a || !b || !S || !o) return GDN2_ERR_NULL_POINTER;
  if (!coupled && !w) return GDN2_ERR_NULL_POINTER;
  if (coupled) w = nullptr;  // the write gate is beta
  const void *ptrs[] = {q, k, v, sa ? nullptr : a, coupled ? nullptr : b, w, S, o};
  for (const void *p : ptrs)
    if (p && !aligned16(p)) return GDN2_ERR_BAD_SHAPE;
  if ((sa && !aligned4(a)) || (coupled && !aligned4(b))) return GDN2_ERR_BAD_SHAPE;
  const size_t gs = form == gdn2::kGatePre ? es : 4;  // gate element bytes
  const Range ro = range_of(o, B * Hv * dv * es);
  const Range ins[] = {range_of(q, B * Hqk * dk * es), range_of(k, B * Hqk * dk * es),
                       range_of(v, B * Hv * dv * es),  range_of(a, B * Hv * (sa ? 1 : dk) * gs),
                       range_of(b, B * Hv * (coupled ? 1 : dk) * gs), range_of(w, coupled ? 0 : B * Hv * dv * gs),
                       range_of(S, B * Hv * dk * dv * 4)};
  for (const Range &r : ins)
    if (overlaps(ro, r)) return GDN2_ERR_ALIAS;

  gdn2::DecodeArgs p;
  p.B = d->B; p.H_qk = d->H_qk; p.H_v = d->H_v; p.d_k = d->d_k; p.d_v = d->d_v;
  p.bf16 = d->dtype == GDN2_BF16;
  p.q = q; p.k = k; p.v = v; p.a = a; p.b = b; p.w = w; p.gate_form = form; p.S = S; p.o = o;
  const hipError_t e = gdn2::launch_decode(p, reinterpret_cast<hipStream_t>(stream));
  return e == hipSuccess ? GDN2_OK : GDN2_ERR_HIP;
}

}  // extern "C"

extern "C" {

size_t gdn2_chunk_backward_workspace_bytes(const gdn2_desc *d) {
  if (check_desc(d, false) != GDN2_OK) return 0;
  return gdn2::backward_workspace_bytes_split(d->B, d->T, d->H_qk, d->H_v, d->d_k, d->d_v, d->dtype == GDN2_BF16);
}

size_t gdn2_chunk_backward_varlen_workspace_bytes(const gdn2_desc *d) {
  if (check_desc(d, false) != GDN2_OK) return 0;
  return gdn2::backward_workspace_bytes(d->B, (size_t)d->T, d->H_v, d->d_k, d->d_v);
}

gdn2_status gdn2_chunk_backward(const gdn2_desc *d, const void *q, const void *k, const void *v,
                                const float *a, const float *b, const float *w, const float *S0,
                                const void *dO, const float *dS_T, void *dq, void *dk, void *dv, float *da,
                                float *db, float *dw, float *dS0, void *workspace, size_t workspace_bytes,
                                void *stream) {
  return backward_general(d, nullptr, q, k, v, a, b, w, S0, dO, dS_T, dq, dk, dv, da, db, dw, dS0, workspace,
                          workspace_bytes, stream, false, gdn2::kGateGeneral);
}

gdn2_status gdn2_chunk_backward_preact(const gdn2_desc *d, const void *q, const void *k, const void *v,
                                       const void *a_pre, const void *b_pre, const void *w_pre, const float *S0,
                                       const void *dO, const float *dS_T, void *dq, void *dk, void *dv,
                                       void *da_pre, void *db_pre, void *dw_pre, float *dS0, void *workspace,
                                       size_t workspace_bytes, void *stream) {
  return backward_general(d, nullptr, q, k, v, a_pre, b_pre, w_pre, S0, dO, dS_T, dq, dk, dv, da_pre, db_pre, dw_pre,
                          dS0, workspace, workspace_bytes, stream, false, gdn2::kGatePre);
}

gdn2_status gdn2_chunk_backward_coupled(const gdn2_desc *d, const void *q, const void *k, const void *v,
                                        const float *a, const float *beta, const float *S0, const void *dO,
                                        const float *dS_T, void *dq, void *dk, void *dv, float *da, float *dbeta,
                                        float *dS0, void *workspace, size_t workspace_bytes, void *stream) {
  return backward_general(d, nullptr, q, k, v, a, beta, nullptr, S0, dO, dS_T, dq, dk, dv, da, dbeta, nullptr, dS0,
                          workspace, workspace_bytes, stream, false, gdn2::kGateCoupled);
}

gdn2_status gdn2_chunk_backward_scalar(const gdn2_desc *d, const void *q, const void *k, const void *v,
                                       const float *alpha, const float *beta, const float *S0, const void *dO,
                                       const float *dS_T, void *dq, void *dk, void *dv, float *dalpha, float *dbeta,
                                       float *dS0, void *workspace, size_t workspace_bytes, void *stream) {
  return backward_general(d, nullptr, q, k, v, alpha, beta, nullptr, S0, dO, dS_T, dq, dk, dv, dalpha, dbeta,
                          nullptr, dS0, workspace, workspace_bytes, stream, false, gdn2::kGateScalar);
}

gdn2_status gdn2_chunk_backward_varlen(const gdn2_desc *d, const int32_t *cu_seqlens, const void *q, const void *k,
                                       const void *v, const float *a, const float *b, const float *w,
                                       const float *S0, const void *dO, const float *dS_T, void *dq, void *dk,
                                       void *dv, float *da, float *db, float *dw, float *dS0, void *workspace,
                                       size_t workspace_bytes, void *stream) {
  return backward_general(d, cu_seqlens, q, k, v, a, b, w, S0, dO, dS_T, dq, dk, dv, da, db, dw, dS0, workspace,
                          workspace_bytes, stream, true, gdn2::kGateGeneral);
}

gdn2_status gdn2_chunk_backward_varlen_gates(const gdn2_desc *d, const int32_t *cu_seqlens, gdn2_gates gates,
                                             const void *q, const void *k, const void *v, const void *a,
                                             const void *b, const void *w, const float *S0, const void *dO,
                                             const float *dS_T, void *dq, void *dk, void *dv, void *da, void *db,
                                             void *dw, float *dS0, void *workspace, size_t workspace_bytes,
                                             void *stream) {
  int form;
  switch (gates) {
    case GDN2_GATES_CHANNEL: form = gdn2::kGateGeneral; break;
    case GDN2_GATES_PREACT: form = gdn2::kGatePre; break;
    case GDN2_GATES_COUPLED: form = gdn2::kGateCoupled; break;
    case GDN2_GATES_SCALAR: form = gdn2::kGateScalar; break;
    default: {
      const gdn2_status sd = check_desc(d, false);
      return sd != GDN2_OK ? sd : GDN2_ERR_UNSUPPORTED;
    }
  }
  return backward_general(d, cu_seqlens, q, k, v, a, b, w, S0, dO, dS_T, dq, dk, dv, da, db, dw, dS0, workspace,
                          workspace_bytes, stream, true, form);
}

}  // extern "C"

namespace {

// gdn2_chunk_backward and gdn2_chunk_backward_varlen (cu_seqlens non-null:
// B sequences packed along T tokens).
gdn2_status backward_general(const gdn2_desc *d, const int32_t *cu, const void *q, const void *k, const void *v,
                             const void *a, const void *b, const void *w, const float *S0, const void *dO,
                             const float *dS_T, void *dq, void *dk, void *dv, void *da, void *db, void *dw,
                             float *dS0, void *workspace, size_t workspace_bytes, void *stream, bool varlen,
                             int form) {
  const bool preact = form == gdn2::kGatePre, coupled = form == gdn2::kGateCoupled || form == gdn2::kGateScalar;
  gdn2_status st = check_desc(d, false);
  if (st != GDN2_OK) return st;
  const size_t B = (size_t)d->B, T = (size_t)d->T, Hqk = (size_t)d->H_qk, Hv = (size_t)d->H_v;
  const size_t dkk = (size_t)d->d_k, dvv = (size_t)d->d_v;
  const size_t es = d->dtype == GDN2_BF16 ? 2 : 4;
  if (B == 0) return GDN2_OK;
  if (varlen && !cu) return GDN2_ERR_NULL_POINTER;
  const size_t BT = varlen ? T : B * T;  // tokens in all
  const size_t ws_need = varlen ? gdn2::backward_workspace_bytes(d->B, BT, d->H_v, d->d_k, d->d_v)
                                : gdn2::backward_workspace_bytes_split(d->B, d->T, d->H_qk, d->H_v, d->d_k, d->d_v,
                                                                        d->dtype == GDN2_BF16);
  if (ws_need > 0 && (!workspace || workspace_bytes < ws_need)) return GDN2_ERR_WORKSPACE;
  const bool tokens = BT > 0;
  if (tokens && (!q || !k || !v || !a || !b || !dO || !dq || !dk || !dv || !da || !db))
    return GDN2_ERR_NULL_POINTER;
  if (tokens && !coupled && (!w || !dw)) return GDN2_ERR_NULL_POINTER;
  if (coupled) w = dw = nullptr;  // the write gate is beta
  const bool sa = form == gdn2::kGateScalar;  // a, da one scalar per token and value head
  const void *ptrs[] = {q, k, v, sa ? nullptr : a, coupled ? nullptr : b, w, S0, dO, dS_T, dq, dk, dv,
                        sa ? nullptr : da, coupled ? nullptr : db, dw, dS0};
  for (const void *p : ptrs)
    if (p && !aligned16(p)) return GDN2_ERR_BAD_SHAPE;
  const void *scalars[] = {sa ? a : nullptr, sa ? da : nullptr, coupled ? b : nullptr, coupled ? db : nullptr};
  for (const void *p : scalars)
    if (p && !aligned4(p)) return GDN2_ERR_BAD_SHAPE;
  if (ws_need > 0 && (reinterpret_cast<uintptr_t>(workspace) & 255u) != 0) return GDN2_ERR_BAD_SHAPE;

  const size_t nqk = BT * Hqk * dkk, nab = BT * Hv * dkk, nvw = BT * Hv * dvv, ns = B * Hv * dkk * dvv;
  const size_t gs = preact ? es : 4;  // gate (and gate gradient) element bytes
  // gate elements: per channel, or one per token and value head (beta; alpha in the scalar form)
  const size_t na = form == gdn2::kGateScalar ? BT * Hv : nab, nb = coupled ? BT * Hv : nab;
  const size_t nw = coupled ? 0 : nvw;
  const Range ins[] = {range_of(q, nqk * es),  range_of(k, nqk * es), range_of(v, nvw * es),
                       range_of(a, na * gs),  range_of(b, nb * gs), range_of(w, nw * gs),
                       range_of(S0, S0 ? ns * 4 : 0), range_of(dO, nvw * es),
                       range_of(dS_T, dS_T ? ns * 4 : 0), range_of(cu, varlen ? (B + 1) * sizeof(int32_t) : 0)};
  const Range outs[] = {range_of(dq, nqk * es), range_of(dk, nqk * es), range_of(dv, nvw * es),
                        range_of(da, na * gs), range_of(db, nb * gs), range_of(dw, nw * gs),
                        range_of(dS0, dS0 ? ns * 4 : 0), range_of(workspace, ws_need)};
  constexpr int NO = sizeof(outs) / sizeof(outs[0]);
  for (int i = 0; i < NO; ++i) {
    for (const Range &r : ins) {
      // dS0 may replace dS_T exactly (each element is read before it is written)
      if (i == 6 && dS0 && dS0 == dS_T && r.lo == reinterpret_cast<uintptr_t>(dS_T)) continue;
      if (overlaps(outs[i], r)) return GDN2_ERR_ALIAS;
    }
    for (int j = i + 1; j < NO; ++j)
      if (overlaps(outs[i], outs[j])) return GDN2_ERR_ALIAS;
  }

  gdn2::BackwardArgs p{};
  p.B = d->B; p.T = d->T; p.H_qk = d->H_qk; p.H_v = d->H_v; p.d_k = d->d_k; p.d_v = d->d_v;
  p.bf16 = d->dtype == GDN2_BF16;
  p.q = q; p.k = k; p.v = v; p.S0 = S0; p.dO = dO; p.dST = dS_T;
  p.a = static_cast<const float *>(a);  // pre-activations in the input dtype when preact
  p.b = static_cast<const float *>(b);
  p.w = static_cast<const float *>(w);
  p.dq = dq; p.dk = dk; p.dv = dv; p.dS0 = dS0;
  p.da = static_cast<float *>(da);
  p.db = static_cast<float *>(db);
  p.dw = static_cast<float *>(dw);
  p.gate_form = form;
  p.workspace = workspace;
  p.workspace_bytes = ws_need;  // the part checked against the other buffers
  p.cu_seqlens = varlen ? cu : nullptr;
  const hipError_t e = gdn2::launch_backward(p, reinterpret_cast<hipStream_t>(stream));
  return e == hipSuccess ? GDN2_OK : GDN2_ERR_HIP;
}

}  // namespace
