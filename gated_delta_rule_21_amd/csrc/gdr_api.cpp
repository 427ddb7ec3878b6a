// C ABI of the gated delta-rule library: argument checks, then dispatch to the
// gfx950 kernels.  Every check runs before anything is enqueued.
#include <hip/hip_runtime.h>

#include <cstdarg>
#include <cstdint>
#include <cstdio>
#include <string>

#include "../../include/gdr.h"
#include "launchers.h"

namespace {

thread_local std::string g_last_error;

gdr_status fail(gdr_status st, const char* fmt, ...) {
  char buf[512];
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(buf, sizeof(buf), fmt, ap);
  va_end(ap);
  g_last_error = buf;
  return st;
}

struct Span {
  const char* name;
  uintptr_t lo, hi;   // [lo, hi); empty when lo == hi
};

bool overlaps(const Span& a, const Span& b) {
  if (a.lo == a.hi || b.lo == b.hi) return false;
  return a.lo < b.hi && b.lo < a.hi;
}

Span span(const char* name, const void* p, int64_t bytes) {
  uintptr_t lo = reinterpret_cast<uintptr_t>(p);
  return Span{name, lo, p ? lo + static_cast<uintptr_t>(bytes) : lo};
}

bool mul_ok(int64_t a, int64_t b, int64_t* out) {
  if (a < 0 || b < 0) return false;
  if (a != 0 && b > INT64_MAX / a) return false;
  *out = a * b;
  return true;
}

// Checks shared by both entry points.  Fills element counts per token-row.
gdr_status check_desc(const gdr_desc* d, bool decode) {
  if (!d) return fail(GDR_ERR_INVALID_ARG, "desc is NULL");
  if (d->io != GDR_F32 && d->io != GDR_BF16) return fail(GDR_ERR_INVALID_ARG, "io dtype %d is not GDR_F32/GDR_BF16", d->io);
  if (d->gate < GDR_GATE_NONE || d->gate > GDR_GATE_CHANNEL) return fail(GDR_ERR_INVALID_ARG, "gate %d is not a gdr_gate", d->gate);
  if (d->form != GDR_FORM_PAGE && d->form != GDR_FORM_LITERAL) return fail(GDR_ERR_INVALID_ARG, "form %d is not a gdr_form", d->form);
  if (d->B < 1) return fail(GDR_ERR_INVALID_ARG, "B = %lld must be >= 1", (long long)d->B);
  if (d->H < 1) return fail(GDR_ERR_INVALID_ARG, "H = %lld must be >= 1", (long long)d->H);
  if (decode) {
    if (d->T != 1) return fail(GDR_ERR_INVALID_ARG, "T = %lld: a decode step takes exactly one token", (long long)d->T);
  } else {
    if (d->T < 0) return fail(GDR_ERR_INVALID_ARG, "T = %lld must be >= 0", (long long)d->T);
    if (d->chunk != 0 && d->chunk != 64) return fail(GDR_ERR_UNSUPPORTED, "chunk = %d: only 64 is implemented", d->chunk);
  }
  if (d->d_k != 64 && d->d_k != 128) return fail(GDR_ERR_UNSUPPORTED, "d_k = %lld: supported 64, 128", (long long)d->d_k);
  if (d->d_v != 64 && d->d_v != 128) return fail(GDR_ERR_UNSUPPORTED, "d_v = %lld: supported 64, 128", (long long)d->d_v);
  if (!decode && d->io == GDR_F32 && d->d_k != 64 && d->gate == GDR_GATE_CHANNEL)
    return fail(GDR_ERR_UNSUPPORTED, "fp32 I/O chunk forward with a per-channel gate supports d_k = 64 only");
  int64_t bh, bth, x;
  if (!mul_ok(d->B, d->H, &bh) || !mul_ok(bh, d->T, &bth) || !mul_ok(bth, 128, &x) || !mul_ok(bh, 128 * 128 * 4, &x))
    return fail(GDR_ERR_INVALID_ARG, "sizes overflow");
  if (bh * 8 > INT32_MAX || bh * ((d->T + 63) / 64) > INT32_MAX)
    return fail(GDR_ERR_UNSUPPORTED, "B*H = %lld (x chunks) exceeds the grid limit", (long long)bh);
  // The kernels address one sequence's (b, h) slice with 32-bit byte offsets.
  const int64_t esz = d->io == GDR_BF16 ? 2 : 4;
  const int64_t dmax = d->d_k > d->d_v ? d->d_k : d->d_v;
  int64_t seq_bytes;
  if (!mul_ok(d->T, d->H, &seq_bytes) || !mul_ok(seq_bytes, dmax * esz, &seq_bytes) || seq_bytes > INT32_MAX)
    return fail(GDR_ERR_UNSUPPORTED, "T*H*max(d_k,d_v)*elem_size = %lld bytes exceeds 2^31 - 1 per sequence",
                (long long)seq_bytes);
  // ... and one sequence's workspace records the same way
  if (!decode && static_cast<int64_t>(gdr::chunk_workspace_bytes(1, d->T, 1, d->io, d->gate, static_cast<int>(d->d_k))) > INT32_MAX)
    return fail(GDR_ERR_UNSUPPORTED, "T = %lld: the per-sequence workspace exceeds 2^31 - 1 bytes", (long long)d->T);
  return GDR_OK;
}

// The backward: the forward's checks, then what this version implements.
gdr_status check_bwd_desc(const gdr_desc* d) {
  gdr_status st = check_desc(d, false);
  if (st != GDR_OK) return st;
  if (d->io != GDR_BF16) return fail(GDR_ERR_UNSUPPORTED, "chunk backward: bf16 I/O only");
  if (d->gate == GDR_GATE_CHANNEL && d->d_k != 128)
    return fail(GDR_ERR_UNSUPPORTED, "chunk backward: the per-channel gate needs d_k = 128");
  // one (sequence, head)'s chunk states are addressed with 32-bit byte offsets
  const int64_t per_seq = ((d->T + 63) / 64) * d->d_k * d->d_v * 2;
  if (per_seq > INT32_MAX)
    return fail(GDR_ERR_UNSUPPORTED, "T = %lld: the per-sequence chunk states exceed 2^31 - 1 bytes", (long long)d->T);
  return GDR_OK;
}

// Packed sequences: the descriptor's B is 1 and T counts all tokens.
gdr_status check_packed(const gdr_desc* d, int64_t n_seq) {
  if (n_seq < 1) return fail(GDR_ERR_INVALID_ARG, "n_seq = %lld must be >= 1", (long long)n_seq);
  if (d->B != 1) return fail(GDR_ERR_INVALID_ARG, "B = %lld: packed sequences take B = 1 (all tokens in T)", (long long)d->B);
  int64_t x;
  if (!mul_ok(n_seq, d->H, &x) || x * 8 > INT32_MAX || d->H * gdr::chunk_varlen_slots(d->T, n_seq) > INT32_MAX)
    return fail(GDR_ERR_UNSUPPORTED, "n_seq = %lld: exceeds the grid limit", (long long)n_seq);
  return GDR_OK;
}

// The backward's workspace: the transform's records (rec bytes), the chunk-start
// states (sb bytes), then the chunk-end state gradients (sb bytes).
void bwd_ws_layout(const gdr_desc* d, bool packed, int64_t n_seq, size_t* rec, size_t* sb) {
  const int dk = static_cast<int>(d->d_k), dv = static_cast<int>(d->d_v);
  *rec = packed ? gdr::chunk_varlen_records_bytes(d->T, n_seq, d->H, d->io, d->gate, dk)
                : gdr::chunk_workspace_bytes(d->B, d->T, d->H, d->io, d->gate, dk);
  *sb = packed ? gdr::chunk_bwd_varlen_state_bytes(d->T, n_seq, d->H, dk, dv)
               : gdr::chunk_bwd_state_bytes(d->B, d->T, d->H, dk, dv);
}

gdr_status check_align(const char* name, const void* p, uintptr_t a) {
  if (p && (reinterpret_cast<uintptr_t>(p) % a) != 0)
    return fail(GDR_ERR_ALIGNMENT, "%s = %p is not %u-byte aligned", name, p, (unsigned)a);
  return GDR_OK;
}

gdr_status check_no_overlap(const Span* outs, int n_out, const Span* all, int n_all) {
  for (int i = 0; i < n_out; ++i)
    for (int j = 0; j < n_all; ++j) {
      if (outs[i].name == all[j].name) continue;
      if (overlaps(outs[i], all[j]))
        return fail(GDR_ERR_INVALID_ARG, "%s overlaps %s", outs[i].name, all[j].name);
    }
  return GDR_OK;
}

}  // namespace

extern "C" {

const char* gdr_status_string(gdr_status s) {
  switch (s) {
    case GDR_OK: return "GDR_OK";
    case GDR_ERR_INVALID_ARG: return "GDR_ERR_INVALID_ARG: invalid argument";
    case GDR_ERR_UNSUPPORTED: return "GDR_ERR_UNSUPPORTED: configuration not implemented";
    case GDR_ERR_ALIGNMENT: return "GDR_ERR_ALIGNMENT: pointer misaligned";
    case GDR_ERR_WORKSPACE: return "GDR_ERR_WORKSPACE: workspace missing or too small";
    case GDR_ERR_HIP: return "GDR_ERR_HIP: HIP runtime error";
  }
  return "unknown gdr_status";
}

const char* gdr_last_error(void) { return g_last_error.c_str(); }

int gdr_version(void) { return 100; }

gdr_status gdr_chunk_fwd_workspace_size(const gdr_desc* d, size_t* bytes) {
  try {
    g_last_error.clear();
    if (!bytes) return fail(GDR_ERR_INVALID_ARG, "bytes is NULL");
    *bytes = 0;
    gdr_status st = check_desc(d, false);
    if (st != GDR_OK) return st;
    *bytes = gdr::chunk_workspace_bytes(d->B, d->T, d->H, d->io, d->gate, static_cast<int>(d->d_k));
    return GDR_OK;
  } catch (...) {
    return fail(GDR_ERR_INVALID_ARG, "internal error");
  }
}

}  // extern "C"

namespace {

// The forward over fixed-length batches (cu == nullptr) or packed sequences.  With
// `save` (the training forward) the workspace is the backward's, and the call also
// leaves there the chunk-start states the backward reads.
gdr_status chunk_fwd_impl(const gdr_desc* d, const int32_t* cu, int64_t n_seq, const void* q, const void* k,
                          const void* v, const void* beta, const void* log_a, const float* S0, void* o, float* S_T,
                          void* workspace, size_t workspace_bytes, void* stream, const void* kw = nullptr,
                          bool save = false) {
  gdr_status st = save ? check_bwd_desc(d) : check_desc(d, false);
  if (st != GDR_OK) return st;
  if (save && kw && d->gate == GDR_GATE_CHANNEL)
    return fail(GDR_ERR_UNSUPPORTED, "training forward with a write key: no gate or a scalar gate");
  const bool packed = cu != nullptr || n_seq != 0;
  if (packed) {
    if (!cu) return fail(GDR_ERR_INVALID_ARG, "cu_seqlens is NULL");
    if (n_seq < 1) return fail(GDR_ERR_INVALID_ARG, "n_seq = %lld must be >= 1", (long long)n_seq);
    if (d->B != 1) return fail(GDR_ERR_INVALID_ARG, "B = %lld: packed sequences take B = 1 (all tokens in T)", (long long)d->B);
    int64_t x;
    if (!mul_ok(n_seq, d->H, &x) || x * 8 > INT32_MAX || d->H * gdr::chunk_varlen_slots(d->T, n_seq) > INT32_MAX)
      return fail(GDR_ERR_UNSUPPORTED, "n_seq = %lld: exceeds the grid limit", (long long)n_seq);
  }
  const int64_t nseq = packed ? n_seq : d->B;        // sequences, and states in S0 / S_T
  const int dk_ = static_cast<int>(d->d_k), dv_ = static_cast<int>(d->d_v);
  const size_t ws_need =
      save ? (packed ? gdr::chunk_bwd_varlen_workspace_bytes(d->T, n_seq, d->H, dk_, dv_, d->gate)
                     : gdr::chunk_bwd_workspace_bytes(d->B, d->T, d->H, dk_, dv_, d->gate))
      : packed ? gdr::chunk_varlen_workspace_bytes(d->T, n_seq, d->H, d->io, d->gate, dk_)
               : gdr::chunk_workspace_bytes(d->B, d->T, d->H, d->io, d->gate, dk_);
  const int64_t esz = d->io == GDR_BF16 ? 2 : 4;
  const int64_t ntok = d->B * d->T * d->H;
  const bool any = d->T > 0;
  if (any) {
    if (!q) return fail(GDR_ERR_INVALID_ARG, "q is NULL");
    if (!k) return fail(GDR_ERR_INVALID_ARG, "k is NULL");
    if (!v) return fail(GDR_ERR_INVALID_ARG, "v is NULL");
    if (!beta) return fail(GDR_ERR_INVALID_ARG, "beta is NULL");
    if (!o) return fail(GDR_ERR_INVALID_ARG, "o is NULL");
    if (d->gate != GDR_GATE_NONE && !log_a) return fail(GDR_ERR_INVALID_ARG, "log_a is NULL but a gate is requested");
    if (!workspace) return fail(GDR_ERR_WORKSPACE, "workspace is NULL (%zu bytes needed)", ws_need);
    if (workspace_bytes < ws_need)
      return fail(GDR_ERR_WORKSPACE, "workspace_bytes = %zu, %zu needed", workspace_bytes, ws_need);
  }
  if (d->gate == GDR_GATE_NONE && log_a) return fail(GDR_ERR_INVALID_ARG, "log_a must be NULL for GDR_GATE_NONE");
  if ((st = check_align("q", q, 16)) || (st = check_align("k", k, 16)) || (st = check_align("v", v, 16)) ||
      (st = check_align("o", o, 16)) || (st = check_align("S0", S0, 16)) || (st = check_align("S_T", S_T, 16)) ||
      (st = check_align("beta", beta, esz)) || (st = check_align("log_a", log_a, esz)) ||
      (st = check_align("workspace", workspace, 16)) || (st = check_align("cu_seqlens", cu, 4)) ||
      (st = check_align("kw", kw, 16)))
    return st;
  const int64_t gate_w = d->gate == GDR_GATE_NONE ? 0 : d->gate == GDR_GATE_SCALAR ? 1 : d->d_k;
  const int64_t state_bytes = nseq * d->H * d->d_k * d->d_v * 4;
  Span all[] = {span("q", q, ntok * d->d_k * esz), span("k", k, ntok * d->d_k * esz),
                span("v", v, ntok * d->d_v * esz), span("beta", beta, ntok * esz),
                span("log_a", log_a, ntok * gate_w * esz), span("S0", S0, state_bytes),
                span("o", o, ntok * d->d_v * esz), span("S_T", S_T, state_bytes),
                span("workspace", d->T > 0 ? workspace : nullptr, static_cast<int64_t>(ws_need)),
                span("cu_seqlens", cu, packed ? (n_seq + 1) * 4 : 0),
                span("kw", kw, kw ? ntok * d->d_k * esz : 0)};
  Span outs[] = {all[6], all[7], all[8]};
  if (S_T && S0 == S_T) all[5].hi = all[5].lo;   // exact in-place update of the state is allowed
  if ((st = check_no_overlap(outs, 3, all, 11))) return st;

  gdr::ChunkParams p;
  p.q = q; p.k = k; p.v = v; p.beta = beta; p.log_a = log_a; p.S0 = S0; p.o = o; p.S_T = S_T;
  p.ws = workspace;
  p.B = nseq; p.T = d->T; p.H = d->H;
  p.d_k = static_cast<int>(d->d_k); p.d_v = static_cast<int>(d->d_v);
  p.io = d->io; p.gate = d->gate; p.literal = d->form == GDR_FORM_LITERAL;
  p.cu = cu;
  p.nslots = packed ? gdr::chunk_varlen_slots(d->T, n_seq) : 0;
  p.order = nullptr;
  p.kw = kw;
  if (save && d->T > 0) {
    size_t rec, sb;
    bwd_ws_layout(d, packed, n_seq, &rec, &sb);
    p.states = static_cast<char*>(workspace) + rec;
    // the packed order goes where the backward later writes its state gradients
    if (packed) p.order_out = reinterpret_cast<int32_t*>(static_cast<char*>(workspace) + rec + sb);
  }
  if (d->T == 0 && !S_T) return GDR_OK;
  hipError_t e = gdr::launch_chunk_fwd(p, static_cast<hipStream_t>(stream));
  if (e != hipSuccess) return fail(GDR_ERR_HIP, "chunk forward launch failed: %s", hipGetErrorString(e));
  return GDR_OK;
}

}  // namespace

extern "C" {

gdr_status gdr_chunk_fwd(const gdr_desc* d, const void* q, const void* k, const void* v, const void* beta,
                         const void* log_a, const float* S0, void* o, float* S_T, void* workspace,
                         size_t workspace_bytes, void* stream) {
  try {
    g_last_error.clear();
    return chunk_fwd_impl(d, nullptr, 0, q, k, v, beta, log_a, S0, o, S_T, workspace, workspace_bytes, stream);
  } catch (...) {
    return fail(GDR_ERR_INVALID_ARG, "internal error");
  }
}

gdr_status gdr_chunk_fwd_noalloc(const gdr_desc* d, const void* q, const void* k, const void* v, const void* beta,
                                 const void* log_a, const float* S0, void* o, float* S_T, void* stream) {
  try {
    g_last_error.clear();
    gdr_status st = check_desc(d, false);
    if (st != GDR_OK) return st;
    const size_t need = gdr::chunk_workspace_bytes(d->B, d->T, d->H, d->io, d->gate, static_cast<int>(d->d_k));
    if (need > gdr::STATIC_SCRATCH_BYTES)
      return fail(GDR_ERR_WORKSPACE, "this forward needs %zu bytes of scratch; the static scratch holds %zu",
                  need, gdr::STATIC_SCRATCH_BYTES);
    void* ws = nullptr;
    if (d->T > 0) {
      const hipError_t e = gdr::static_scratch(&ws);
      if (e != hipSuccess) return fail(GDR_ERR_HIP, "static scratch lookup failed: %s", hipGetErrorString(e));
    }
    return chunk_fwd_impl(d, nullptr, 0, q, k, v, beta, log_a, S0, o, S_T, ws, gdr::STATIC_SCRATCH_BYTES, stream);
  } catch (...) {
    return fail(GDR_ERR_INVALID_ARG, "internal error");
  }
}

gdr_status gdr_chunk_fwd_varlen_workspace_size(const gdr_desc* d, int64_t n_seq, size_t* bytes) {
  try {
    g_last_error.clear();
    if (!bytes) return fail(GDR_ERR_INVALID_ARG, "bytes is NULL");
    *bytes = 0;
    gdr_status st = check_desc(d, false);
    if (st != GDR_OK) return st;
    if (n_seq < 1) return fail(GDR_ERR_INVALID_ARG, "n_seq = %lld must be >= 1", (long long)n_seq);
    if (d->B != 1) return fail(GDR_ERR_INVALID_ARG, "B = %lld: packed sequences take B = 1 (all tokens in T)", (long long)d->B);
    *bytes = gdr::chunk_varlen_workspace_bytes(d->T, n_seq, d->H, d->io, d->gate, static_cast<int>(d->d_k));
    return GDR_OK;
  } catch (...) {
    return fail(GDR_ERR_INVALID_ARG, "internal error");
  }
}

gdr_status gdr_chunk_fwd_varlen(const gdr_desc* d, const int32_t* cu_seqlens, int64_t n_seq, const void* q,
                                const void* k, const void* v, const void* beta, const void* log_a, const float* S0,
                                void* o, float* S_T, void* workspace, size_t workspace_bytes, void* stream) {
  try {
    g_last_error.clear();
    if (!cu_seqlens) return fail(GDR_ERR_INVALID_ARG, "cu_seqlens is NULL");
    return chunk_fwd_impl(d, cu_seqlens, n_seq, q, k, v, beta, log_a, S0, o, S_T, workspace, workspace_bytes,
                          stream);
  } catch (...) {
    return fail(GDR_ERR_INVALID_ARG, "internal error");
  }
}

gdr_status gdr_chunk_fwd_varlen_wkey(const gdr_desc* d, const int32_t* cu_seqlens, int64_t n_seq, const void* q,
                                     const void* k, const void* kw, const void* v, const void* beta,
                                     const void* log_a, const float* S0, void* o, float* S_T, void* workspace,
                                     size_t workspace_bytes, void* stream) {
  try {
    g_last_error.clear();
    if (!cu_seqlens) return fail(GDR_ERR_INVALID_ARG, "cu_seqlens is NULL");
    if (!kw) return fail(GDR_ERR_INVALID_ARG, "kw is NULL");
    if (d && d->io != GDR_BF16) return fail(GDR_ERR_UNSUPPORTED, "write key chunk forward: bf16 I/O only");
    if (d && d->gate == GDR_GATE_CHANNEL && d->d_k != 128)
      return fail(GDR_ERR_UNSUPPORTED, "write key with a per-channel gate: d_k = 128 only");
    return chunk_fwd_impl(d, cu_seqlens, n_seq, q, k, v, beta, log_a, S0, o, S_T, workspace, workspace_bytes,
                          stream, kw);
  } catch (...) {
    return fail(GDR_ERR_INVALID_ARG, "internal error");
  }
}

}  // extern "C"

namespace {

gdr_status recurrent_step_impl(const gdr_desc* d, const void* q, const void* k, const void* kw, const void* v,
                               const void* beta, const void* log_a, const float* S, float* S_new, void* o,
                               void* stream) {
  gdr_status st = check_desc(d, true);
  if (st != GDR_OK) return st;
  const int64_t esz = d->io == GDR_BF16 ? 2 : 4;
  const int64_t n = d->B * d->H;
  if (!q) return fail(GDR_ERR_INVALID_ARG, "q is NULL");
  if (!k) return fail(GDR_ERR_INVALID_ARG, "k is NULL");
  if (!v) return fail(GDR_ERR_INVALID_ARG, "v is NULL");
  if (!beta) return fail(GDR_ERR_INVALID_ARG, "beta is NULL");
  if (!S) return fail(GDR_ERR_INVALID_ARG, "S is NULL");
  if (!S_new) return fail(GDR_ERR_INVALID_ARG, "S_new is NULL");
  if (!o) return fail(GDR_ERR_INVALID_ARG, "o is NULL");
  if (d->gate != GDR_GATE_NONE && !log_a) return fail(GDR_ERR_INVALID_ARG, "log_a is NULL but a gate is requested");
  if (d->gate == GDR_GATE_NONE && log_a) return fail(GDR_ERR_INVALID_ARG, "log_a must be NULL for GDR_GATE_NONE");
  if ((st = check_align("q", q, 16)) || (st = check_align("k", k, 16)) || (st = check_align("v", v, 16)) ||
      (st = check_align("o", o, 16)) || (st = check_align("S", S, 16)) || (st = check_align("S_new", S_new, 16)) ||
      (st = check_align("beta", beta, esz)) || (st = check_align("log_a", log_a, esz)) ||
      (st = check_align("kw", kw, 16)))
    return st;
  const int64_t gate_w = d->gate == GDR_GATE_NONE ? 0 : d->gate == GDR_GATE_SCALAR ? 1 : d->d_k;
  const int64_t state_bytes = n * d->d_k * d->d_v * 4;
  Span all[] = {span("q", q, n * d->d_k * esz), span("k", k, n * d->d_k * esz), span("v", v, n * d->d_v * esz),
                span("beta", beta, n * esz), span("log_a", log_a, n * gate_w * esz), span("S", S, state_bytes),
                span("o", o, n * d->d_v * esz), span("S_new", S_new, state_bytes),
                span("kw", kw, kw ? n * d->d_k * esz : 0)};
  Span outs[] = {all[6], all[7]};
  if (S == S_new) all[5].hi = all[5].lo;   // exact in-place update is allowed
  if ((st = check_no_overlap(outs, 2, all, 9))) return st;

  gdr::DecodeParams p;
  p.q = q; p.k = k; p.v = v; p.beta = beta; p.log_a = log_a; p.S = S; p.S_new = S_new; p.o = o;
  p.n_states = n;
  p.d_k = static_cast<int>(d->d_k); p.d_v = static_cast<int>(d->d_v);
  p.io = d->io; p.gate = d->gate; p.literal = d->form == GDR_FORM_LITERAL;
  p.kw = kw;
  hipError_t e = gdr::launch_decode_step(p, static_cast<hipStream_t>(stream));
  if (e != hipSuccess) return fail(GDR_ERR_HIP, "decode step launch failed: %s", hipGetErrorString(e));
  return GDR_OK;
}

}  // namespace

namespace {

// The backward over fixed-length batches (cu == nullptr) or packed sequences.
gdr_status chunk_bwd_impl(const gdr_desc* d, const int32_t* cu, int64_t n_seq, const void* q, const void* k,
                          const void* v, const void* beta, const void* log_a, const float* S0, const void* dO,
                          const float* dS_T, void* dq, void* dk, void* dv, void* dbeta, void* dlog_a, float* dS0,
                          void* workspace, size_t workspace_bytes, void* stream, const void* kw = nullptr,
                          void* dkw = nullptr, bool saved = false) {
  gdr_status st = check_bwd_desc(d);
  if (st != GDR_OK) return st;
  const bool wkey = kw != nullptr || dkw != nullptr;
  if (wkey && d->gate == GDR_GATE_CHANNEL)
    return fail(GDR_ERR_UNSUPPORTED, "backward with a write key: no gate or a scalar gate");
  const bool packed = cu != nullptr;
  if (packed && (st = check_packed(d, n_seq)) != GDR_OK) return st;
  const int64_t nseq = packed ? n_seq : d->B;       // sequences, and states in S0 / dS_T / dS0
  const bool gated = d->gate != GDR_GATE_NONE;
  const int dk_ = static_cast<int>(d->d_k), dv_ = static_cast<int>(d->d_v);
  const int64_t gate_width = d->gate == GDR_GATE_CHANNEL ? d->d_k : 1;   // log a values per token and head
  const size_t ws_need = d->T == 0 ? 0
                         : packed  ? gdr::chunk_bwd_varlen_workspace_bytes(d->T, n_seq, d->H, dk_, dv_, d->gate)
                                   : gdr::chunk_bwd_workspace_bytes(d->B, d->T, d->H, dk_, dv_, d->gate);
  if (d->T > 0) {
    const void* req[] = {q, k, v, beta, dO, dq, dk, dv, dbeta};
    const char* names[] = {"q", "k", "v", "beta", "dO", "dq", "dk", "dv", "dbeta"};
    for (int i = 0; i < 9; ++i)
      if (!req[i]) return fail(GDR_ERR_INVALID_ARG, "%s is NULL", names[i]);
    if (gated && !log_a) return fail(GDR_ERR_INVALID_ARG, "log_a is NULL but a gate is requested");
    if (gated && !dlog_a) return fail(GDR_ERR_INVALID_ARG, "dlog_a is NULL but a gate is requested");
    if (wkey && !kw) return fail(GDR_ERR_INVALID_ARG, "kw is NULL");
    if (wkey && !dkw) return fail(GDR_ERR_INVALID_ARG, "dkw is NULL");
    if (!workspace) return fail(GDR_ERR_WORKSPACE, "workspace is NULL (%zu bytes needed)", ws_need);
    if (workspace_bytes < ws_need)
      return fail(GDR_ERR_WORKSPACE, "workspace_bytes = %zu, %zu needed", workspace_bytes, ws_need);
  }
  if (!gated && log_a) return fail(GDR_ERR_INVALID_ARG, "log_a must be NULL for GDR_GATE_NONE");
  if (!gated && dlog_a) return fail(GDR_ERR_INVALID_ARG, "dlog_a must be NULL for GDR_GATE_NONE");
  if ((st = check_align("q", q, 16)) || (st = check_align("k", k, 16)) || (st = check_align("v", v, 16)) ||
      (st = check_align("dO", dO, 16)) || (st = check_align("dq", dq, 16)) || (st = check_align("dk", dk, 16)) ||
      (st = check_align("dv", dv, 16)) || (st = check_align("S0", S0, 16)) || (st = check_align("dS_T", dS_T, 16)) ||
      (st = check_align("dS0", dS0, 16)) || (st = check_align("beta", beta, 2)) ||
      (st = check_align("dbeta", dbeta, 2)) || (st = check_align("log_a", log_a, 2)) ||
      (st = check_align("dlog_a", dlog_a, 2)) || (st = check_align("workspace", workspace, 16)) ||
      (st = check_align("cu_seqlens", cu, 4)) || (st = check_align("kw", kw, 16)) || (st = check_align("dkw", dkw, 16)))
    return st;
  const int64_t ntok = d->B * d->T * d->H;
  const int64_t state_bytes = nseq * d->H * d->d_k * d->d_v * 4;
  Span all[] = {span("q", q, ntok * d->d_k * 2), span("k", k, ntok * d->d_k * 2),
                span("v", v, ntok * d->d_v * 2), span("beta", beta, ntok * 2),
                span("log_a", log_a, gated ? ntok * gate_width * 2 : 0), span("S0", S0, state_bytes),
                span("dO", dO, ntok * d->d_v * 2), span("dS_T", dS_T, state_bytes),
                span("cu_seqlens", cu, packed ? (n_seq + 1) * 4 : 0),
                span("dq", dq, ntok * d->d_k * 2), span("dk", dk, ntok * d->d_k * 2),
                span("dv", dv, ntok * d->d_v * 2), span("dbeta", dbeta, ntok * 2),
                span("dlog_a", dlog_a, gated ? ntok * gate_width * 2 : 0), span("dS0", dS0, state_bytes),
                span("workspace", d->T > 0 ? workspace : nullptr, static_cast<int64_t>(ws_need)),
                span("kw", kw, ntok * d->d_k * 2), span("dkw", dkw, ntok * d->d_k * 2)};
  Span outs[] = {all[9], all[10], all[11], all[12], all[13], all[14], all[15], all[17]};
  if (dS0 && dS0 == dS_T) all[7].hi = all[7].lo;   // the final-state gradient may be overwritten by dS0
  if ((st = check_no_overlap(outs, 8, all, 18))) return st;

  gdr::BwdParams p;
  gdr::ChunkParams& f = p.f;
  f.q = q; f.k = k; f.v = v; f.beta = beta; f.log_a = log_a; f.S0 = S0; f.o = nullptr; f.S_T = nullptr;
  f.ws = workspace;
  f.B = nseq; f.T = d->T; f.H = d->H;
  f.d_k = dk_; f.d_v = dv_;
  f.io = d->io; f.gate = d->gate; f.literal = d->form == GDR_FORM_LITERAL;
  f.cu = cu; f.nslots = packed ? gdr::chunk_varlen_slots(d->T, n_seq) : 0; f.order = nullptr; f.kw = kw;
  p.dO = dO; p.dS_T = dS_T; p.dq = dq; p.dk = dk; p.dv = dv; p.dbeta = dbeta; p.dlog_a = dlog_a; p.dS0 = dS0;
  p.dkw = dkw;
  p.saved = saved ? 1 : 0;
  size_t rec, sb;
  bwd_ws_layout(d, packed, n_seq, &rec, &sb);
  p.states = d->T > 0 ? static_cast<char*>(workspace) + rec : nullptr;
  p.dstates = d->T > 0 ? static_cast<char*>(workspace) + rec + sb : nullptr;
  if (d->T == 0 && !dS0) return GDR_OK;
  hipError_t e = gdr::launch_chunk_bwd(p, static_cast<hipStream_t>(stream));
  if (e != hipSuccess) return fail(GDR_ERR_HIP, "chunk backward launch failed: %s", hipGetErrorString(e));
  return GDR_OK;
}

}  // namespace

extern "C" {

gdr_status gdr_recurrent_step(const gdr_desc* d, const void* q, const void* k, const void* v, const void* beta,
                              const void* log_a, const float* S, float* S_new, void* o, void* stream) {
  try {
    g_last_error.clear();
    return recurrent_step_impl(d, q, k, nullptr, v, beta, log_a, S, S_new, o, stream);
  } catch (...) {
    return fail(GDR_ERR_INVALID_ARG, "internal error");
  }
}

gdr_status gdr_recurrent_step_wkey(const gdr_desc* d, const void* q, const void* k, const void* kw, const void* v,
                                   const void* beta, const void* log_a, const float* S, float* S_new, void* o,
                                   void* stream) {
  try {
    g_last_error.clear();
    if (!kw) return fail(GDR_ERR_INVALID_ARG, "kw is NULL");
    return recurrent_step_impl(d, q, k, kw, v, beta, log_a, S, S_new, o, stream);
  } catch (...) {
    return fail(GDR_ERR_INVALID_ARG, "internal error");
  }
}

gdr_status gdr_precond_scan(const gdr_desc* d, const void* k, const void* beta, const void* r, float eta,
                            const float* d0, void* kw, float* d_T, void* stream) {
  try {
    g_last_error.clear();
    if (!d) return fail(GDR_ERR_INVALID_ARG, "desc is NULL");
    if (d->io != GDR_F32 && d->io != GDR_BF16) return fail(GDR_ERR_INVALID_ARG, "io dtype %d is not GDR_F32/GDR_BF16", d->io);
    if (d->B < 1) return fail(GDR_ERR_INVALID_ARG, "B = %lld must be >= 1", (long long)d->B);
    if (d->H < 1) return fail(GDR_ERR_INVALID_ARG, "H = %lld must be >= 1", (long long)d->H);
    if (d->T < 0) return fail(GDR_ERR_INVALID_ARG, "T = %lld must be >= 0", (long long)d->T);
    if (d->d_k != 64 && d->d_k != 128) return fail(GDR_ERR_UNSUPPORTED, "d_k = %lld: supported 64, 128", (long long)d->d_k);
    if (!(eta == eta) || eta > 3.0e38f || eta < -3.0e38f) return fail(GDR_ERR_INVALID_ARG, "eta is not finite");
    const int64_t esz = d->io == GDR_BF16 ? 2 : 4;
    int64_t bh = 0, bth = 0, elems = 0, bytes = 0;
    if (!mul_ok(d->B, d->H, &bh) || !mul_ok(bh, d->T, &bth) || !mul_ok(bth, d->d_k, &elems) ||
        !mul_ok(elems, esz, &bytes))
      return fail(GDR_ERR_INVALID_ARG, "sizes overflow");
    if (bh > INT32_MAX) return fail(GDR_ERR_UNSUPPORTED, "B*H = %lld exceeds the grid limit", (long long)bh);
    if ((d->T + 128) * d->H * d->d_k * esz > INT32_MAX)   // 32-bit offsets within a sequence, two chunks past its end
      return fail(GDR_ERR_UNSUPPORTED, "(T + 128)*H*d_k*elem_size = %lld bytes exceeds 2^31 - 1 per sequence",
                  (long long)((d->T + 128) * d->H * d->d_k * esz));
    if (d->T > 0) {
      if (!k) return fail(GDR_ERR_INVALID_ARG, "k is NULL");
      if (!beta) return fail(GDR_ERR_INVALID_ARG, "beta is NULL");
      if (!kw) return fail(GDR_ERR_INVALID_ARG, "kw is NULL");
    }
    gdr_status st;
    if ((st = check_align("k", k, 16)) || (st = check_align("kw", kw, 16)) || (st = check_align("beta", beta, esz)) ||
        (st = check_align("r", r, esz)) || (st = check_align("d0", d0, 4)) || (st = check_align("d_T", d_T, 4)))
      return st;
    const int64_t dbytes = bh * d->d_k * 4;
    Span all[] = {span("k", d->T > 0 ? k : nullptr, bytes), span("beta", d->T > 0 ? beta : nullptr, bth * esz),
                  span("r", d->T > 0 ? r : nullptr, bth * esz), span("d0", d0, dbytes),
                  span("kw", d->T > 0 ? kw : nullptr, bytes), span("d_T", d_T, dbytes)};
    Span outs[] = {all[4], all[5]};
    if (d0 && d0 == d_T) all[3].hi = all[3].lo;   // exact in-place update is allowed
    if ((st = check_no_overlap(outs, 2, all, 6))) return st;

    gdr::PrecondParams p;
    p.k = k; p.beta = beta; p.r = r; p.d0 = d0; p.kw = kw; p.d_T = d_T;
    p.B = d->B; p.T = d->T; p.H = d->H;
    p.d_k = static_cast<int>(d->d_k); p.io = d->io; p.eta = eta;
    hipError_t e = gdr::launch_precond_scan(p, static_cast<hipStream_t>(stream));
    if (e != hipSuccess) return fail(GDR_ERR_HIP, "preconditioner scan launch failed: %s", hipGetErrorString(e));
    return GDR_OK;
  } catch (...) {
    return fail(GDR_ERR_INVALID_ARG, "internal error");
  }
}

namespace {
gdr_status check_precond_desc(const gdr_desc* d) {
  if (!d) return fail(GDR_ERR_INVALID_ARG, "desc is NULL");
  if (d->io != GDR_F32 && d->io != GDR_BF16) return fail(GDR_ERR_INVALID_ARG, "io dtype %d is not GDR_F32/GDR_BF16", d->io);
  if (d->B < 1) return fail(GDR_ERR_INVALID_ARG, "B = %lld must be >= 1", (long long)d->B);
  if (d->H < 1) return fail(GDR_ERR_INVALID_ARG, "H = %lld must be >= 1", (long long)d->H);
  if (d->T < 0) return fail(GDR_ERR_INVALID_ARG, "T = %lld must be >= 0", (long long)d->T);
  if (d->d_k != 64 && d->d_k != 128) return fail(GDR_ERR_UNSUPPORTED, "d_k = %lld: supported 64, 128", (long long)d->d_k);
  int64_t bh = 0, bth = 0, elems = 0;
  if (!mul_ok(d->B, d->H, &bh) || !mul_ok(bh, d->T, &bth) || !mul_ok(bth, d->d_k + 2, &elems) ||
      !mul_ok(elems, 4, &elems))
    return fail(GDR_ERR_INVALID_ARG, "sizes overflow");
  if (bh > INT32_MAX) return fail(GDR_ERR_UNSUPPORTED, "B*H = %lld exceeds the grid limit", (long long)bh);
  return GDR_OK;
}
}  // namespace

gdr_status gdr_precond_scan_bwd_workspace_size(const gdr_desc* d, size_t* bytes) {
  try {
    g_last_error.clear();
    if (!bytes) return fail(GDR_ERR_INVALID_ARG, "bytes is NULL");
    *bytes = 0;
    gdr_status st = check_precond_desc(d);
    if (st != GDR_OK) return st;
    *bytes = gdr::precond_scan_bwd_workspace_bytes(d->B, d->T, d->H, static_cast<int>(d->d_k));
    return GDR_OK;
  } catch (...) {
    return fail(GDR_ERR_INVALID_ARG, "internal error");
  }
}

gdr_status gdr_precond_scan_bwd(const gdr_desc* d, const void* k, const void* beta, const void* r, float eta,
                                const float* d0, const void* dkw, const float* dd_T, void* dk, void* dbeta, void* dr,
                                float* dd0, void* workspace, size_t workspace_bytes, void* stream) {
  try {
    g_last_error.clear();
    gdr_status st = check_precond_desc(d);
    if (st != GDR_OK) return st;
    if (!(eta == eta) || eta > 3.0e38f || eta < -3.0e38f) return fail(GDR_ERR_INVALID_ARG, "eta is not finite");
    const int64_t esz = d->io == GDR_BF16 ? 2 : 4;
    const int64_t bth = d->B * d->T * d->H;
    const size_t need = gdr::precond_scan_bwd_workspace_bytes(d->B, d->T, d->H, static_cast<int>(d->d_k));
    if (!r && dr) return fail(GDR_ERR_INVALID_ARG, "dr must be NULL without a retention r");
    if (d->T > 0) {
      const void* req[] = {k, beta, dk, dbeta};
      const char* names[] = {"k", "beta", "dk", "dbeta"};
      for (int i = 0; i < 4; ++i)
        if (!req[i]) return fail(GDR_ERR_INVALID_ARG, "%s is NULL", names[i]);
      if (!workspace) return fail(GDR_ERR_WORKSPACE, "workspace is NULL (%zu bytes needed)", need);
      if (workspace_bytes < need) return fail(GDR_ERR_WORKSPACE, "workspace_bytes = %zu, %zu needed", workspace_bytes, need);
    }
    if ((st = check_align("k", k, 16)) || (st = check_align("dkw", dkw, 16)) || (st = check_align("dk", dk, 16)) ||
        (st = check_align("beta", beta, esz)) || (st = check_align("r", r, esz)) ||
        (st = check_align("dbeta", dbeta, esz)) || (st = check_align("dr", dr, esz)) ||
        (st = check_align("d0", d0, 4)) || (st = check_align("dd_T", dd_T, 4)) || (st = check_align("dd0", dd0, 4)) ||
        (st = check_align("workspace", workspace, 16)))
      return st;
    const int64_t kbytes = bth * d->d_k * esz, dbytes = d->B * d->H * d->d_k * 4;
    const bool t0 = d->T > 0;
    Span all[] = {span("k", t0 ? k : nullptr, kbytes), span("beta", t0 ? beta : nullptr, bth * esz),
                  span("r", t0 ? r : nullptr, bth * esz), span("d0", d0, dbytes),
                  span("dkw", t0 ? dkw : nullptr, kbytes), span("dd_T", dd_T, dbytes),
                  span("dk", t0 ? dk : nullptr, kbytes), span("dbeta", t0 ? dbeta : nullptr, bth * esz),
                  span("dr", t0 ? dr : nullptr, bth * esz), span("dd0", dd0, dbytes),
                  span("workspace", t0 ? workspace : nullptr, static_cast<int64_t>(need))};
    Span outs[] = {all[6], all[7], all[8], all[9], all[10]};
    if (dd0 && dd0 == dd_T) all[5].hi = all[5].lo;   // dd0 may overwrite dd_T
    if ((st = check_no_overlap(outs, 5, all, 11))) return st;

    gdr::PrecondBwdParams p;
    p.f.k = k; p.f.beta = beta; p.f.r = r; p.f.d0 = d0; p.f.kw = nullptr; p.f.d_T = nullptr;
    p.f.B = d->B; p.f.T = d->T; p.f.H = d->H;
    p.f.d_k = static_cast<int>(d->d_k); p.f.io = d->io; p.f.eta = eta;
    p.dkw = dkw; p.dd_T = dd_T; p.dk = dk; p.dbeta = dbeta; p.dr = dr; p.dd0 = dd0;
    p.ws = static_cast<float*>(workspace);
    hipError_t e = gdr::launch_precond_scan_bwd(p, static_cast<hipStream_t>(stream));
    if (e != hipSuccess) return fail(GDR_ERR_HIP, "preconditioner scan backward launch failed: %s", hipGetErrorString(e));
    return GDR_OK;
  } catch (...) {
    return fail(GDR_ERR_INVALID_ARG, "internal error");
  }
}

gdr_status gdr_chunk_fwd_wkey(const gdr_desc* d, const void* q, const void* k, const void* kw, const void* v,
                              const void* beta, const void* log_a, const float* S0, void* o, float* S_T,
                              void* workspace, size_t workspace_bytes, void* stream) {
  try {
    g_last_error.clear();
    if (!kw) return fail(GDR_ERR_INVALID_ARG, "kw is NULL");
    if (d && d->io != GDR_BF16) return fail(GDR_ERR_UNSUPPORTED, "write key chunk forward: bf16 I/O only");
    if (d && d->gate == GDR_GATE_CHANNEL && d->d_k != 128)
      return fail(GDR_ERR_UNSUPPORTED, "write key with a per-channel gate: d_k = 128 only");
    return chunk_fwd_impl(d, nullptr, 0, q, k, v, beta, log_a, S0, o, S_T, workspace, workspace_bytes, stream, kw);
  } catch (...) {
    return fail(GDR_ERR_INVALID_ARG, "internal error");
  }
}

gdr_status gdr_chunk_bwd_workspace_size(const gdr_desc* d, size_t* bytes) {
  try {
    g_last_error.clear();
    if (!bytes) return fail(GDR_ERR_INVALID_ARG, "bytes is NULL");
    *bytes = 0;
    gdr_status st = check_bwd_desc(d);
    if (st != GDR_OK) return st;
    *bytes = d->T > 0 ? gdr::chunk_bwd_workspace_bytes(d->B, d->T, d->H, static_cast<int>(d->d_k), static_cast<int>(d->d_v),
                                                       d->gate)
                      : 0;
    return GDR_OK;
  } catch (...) {
    return fail(GDR_ERR_INVALID_ARG, "internal error");
  }
}

gdr_status gdr_chunk_bwd_varlen_workspace_size(const gdr_desc* d, int64_t n_seq, size_t* bytes) {
  try {
    g_last_error.clear();
    if (!bytes) return fail(GDR_ERR_INVALID_ARG, "bytes is NULL");
    *bytes = 0;
    gdr_status st = check_bwd_desc(d);
    if (st != GDR_OK) return st;
    if ((st = check_packed(d, n_seq)) != GDR_OK) return st;
    *bytes = d->T > 0 ? gdr::chunk_bwd_varlen_workspace_bytes(d->T, n_seq, d->H, static_cast<int>(d->d_k),
                                                              static_cast<int>(d->d_v), d->gate)
                      : 0;
    return GDR_OK;
  } catch (...) {
    return fail(GDR_ERR_INVALID_ARG, "internal error");
  }
}

gdr_status gdr_chunk_bwd(const gdr_desc* d, const void* q, const void* k, const void* v, const void* beta,
                         const void* log_a, const float* S0, const void* dO, const float* dS_T, void* dq, void* dk,
                         void* dv, void* dbeta, void* dlog_a, float* dS0, void* workspace, size_t workspace_bytes,
                         void* stream) {
  try {
    g_last_error.clear();
    return chunk_bwd_impl(d, nullptr, 0, q, k, v, beta, log_a, S0, dO, dS_T, dq, dk, dv, dbeta, dlog_a, dS0, workspace,
                          workspace_bytes, stream);
  } catch (...) {
    return fail(GDR_ERR_INVALID_ARG, "internal error");
  }
}

gdr_status gdr_chunk_bwd_wkey(const gdr_desc* d, const void* q, const void* k, const void* kw, const void* v,
                              const void* beta, const void* log_a, const float* S0, const void* dO, const float* dS_T,
                              void* dq, void* dk, void* dkw, void* dv, void* dbeta, void* dlog_a, float* dS0,
                              void* workspace, size_t workspace_bytes, void* stream) {
  try {
    g_last_error.clear();
    if (!kw) return fail(GDR_ERR_INVALID_ARG, "kw is NULL");
    if (!dkw) return fail(GDR_ERR_INVALID_ARG, "dkw is NULL");
    return chunk_bwd_impl(d, nullptr, 0, q, k, v, beta, log_a, S0, dO, dS_T, dq, dk, dv, dbeta, dlog_a, dS0, workspace,
                          workspace_bytes, stream, kw, dkw);
  } catch (...) {
    return fail(GDR_ERR_INVALID_ARG, "internal error");
  }
}

gdr_status gdr_chunk_bwd_varlen_wkey(const gdr_desc* d, const int32_t* cu_seqlens, int64_t n_seq, const void* q,
                                     const void* k, const void* kw, const void* v, const void* beta,
                                     const void* log_a, const float* S0, const void* dO, const float* dS_T, void* dq,
                                     void* dk, void* dkw, void* dv, void* dbeta, void* dlog_a, float* dS0,
                                     void* workspace, size_t workspace_bytes, void* stream) {
  try {
    g_last_error.clear();
    if (!cu_seqlens) return fail(GDR_ERR_INVALID_ARG, "cu_seqlens is NULL");
    if (!kw) return fail(GDR_ERR_INVALID_ARG, "kw is NULL");
    if (!dkw) return fail(GDR_ERR_INVALID_ARG, "dkw is NULL");
    return chunk_bwd_impl(d, cu_seqlens, n_seq, q, k, v, beta, log_a, S0, dO, dS_T, dq, dk, dv, dbeta, dlog_a, dS0,
                          workspace, workspace_bytes, stream, kw, dkw);
  } catch (...) {
    return fail(GDR_ERR_INVALID_ARG, "internal error");
  }
}

gdr_status gdr_chunk_fwd_save(const gdr_desc* d, const int32_t* cu_seqlens, int64_t n_seq, const void* q,
                              const void* k, const void* kw, const void* v, const void* beta, const void* log_a,
                              const float* S0, void* o, float* S_T, void* workspace, size_t workspace_bytes,
                              void* stream) {
  try {
    g_last_error.clear();
    if (!cu_seqlens && n_seq != 0) return fail(GDR_ERR_INVALID_ARG, "n_seq = %lld without cu_seqlens", (long long)n_seq);
    return chunk_fwd_impl(d, cu_seqlens, n_seq, q, k, v, beta, log_a, S0, o, S_T, workspace, workspace_bytes, stream,
                          kw, true);
  } catch (...) {
    return fail(GDR_ERR_INVALID_ARG, "internal error");
  }
}

gdr_status gdr_chunk_bwd_saved(const gdr_desc* d, const int32_t* cu_seqlens, int64_t n_seq, const void* q,
                               const void* k, const void* kw, const void* v, const void* beta, const void* log_a,
                               const float* S0, const void* dO, const float* dS_T, void* dq, void* dk, void* dkw,
                               void* dv, void* dbeta, void* dlog_a, float* dS0, void* workspace,
                               size_t workspace_bytes, void* stream) {
  try {
    g_last_error.clear();
    if (!cu_seqlens && n_seq != 0) return fail(GDR_ERR_INVALID_ARG, "n_seq = %lld without cu_seqlens", (long long)n_seq);
    if ((kw == nullptr) != (dkw == nullptr)) return fail(GDR_ERR_INVALID_ARG, "kw and dkw: both or neither");
    return chunk_bwd_impl(d, cu_seqlens, n_seq, q, k, v, beta, log_a, S0, dO, dS_T, dq, dk, dv, dbeta, dlog_a, dS0,
                          workspace, workspace_bytes, stream, kw, dkw, true);
  } catch (...) {
    return fail(GDR_ERR_INVALID_ARG, "internal error");
  }
}

gdr_status gdr_chunk_bwd_varlen(const gdr_desc* d, const int32_t* cu_seqlens, int64_t n_seq, const void* q,
                                const void* k, const void* v, const void* beta, const void* log_a, const float* S0,
                                const void* dO, const float* dS_T, void* dq, void* dk, void* dv, void* dbeta,
                                void* dlog_a, float* dS0, void* workspace, size_t workspace_bytes, void* stream) {
  try {
    g_last_error.clear();
    if (!cu_seqlens) return fail(GDR_ERR_INVALID_ARG, "cu_seqlens is NULL");
    return chunk_bwd_impl(d, cu_seqlens, n_seq, q, k, v, beta, log_a, S0, dO, dS_T, dq, dk, dv, dbeta, dlog_a, dS0,
                          workspace, workspace_bytes, stream);
  } catch (...) {
    return fail(GDR_ERR_INVALID_ARG, "internal error");
  }
}

}  // extern "C"
