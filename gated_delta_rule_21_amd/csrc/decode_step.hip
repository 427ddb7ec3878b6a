// Single-token decode step of the gated delta rule on gfx950.
//
// One token per (sequence, head) advances a constant-size fp32 state
// ("Moonshot AI's New Attention Architecture", §1: decoding keeps a fixed-size
// state instead of a growing cache; §2: the gated delta-rule update):
//
//     S~ = diag(a) S,   u = S~^T k,   delta = beta (v - u),
//     S' = S~ + k delta^T,   o = S'^T q = S~^T q + delta (k . q).
// With a write key kw ("OSDN: Improving Delta Rule with Provable Online
// Preconditioning in Linear Attention", §2.1: the right-preconditioned step)
// the state is written along kw instead: S' = S~ + kw delta^T, o gains
// delta (kw . q); the residual still reads along k.
//
// The step is bound by HBM bandwidth: each state (d_k*d_v*4 bytes) is read once
// and written once.  One 256-thread workgroup owns one state; each thread keeps
// its slice of the state in registers between the read and the write, so S can be
// updated in place.  Rows of the state are split across thread groups, columns
// across lanes (16-byte vector accesses, a full row per 32 or 16 lanes).
#include "device_common.h"
#include "launchers.h"

namespace gdr {

template <int IO, int GATE, int DK, int DV>
__global__ __launch_bounds__(256) void decode_step_kernel(DecodeParams p) {
  typedef typename Io<IO>::elem elem;
  constexpr int TPR = DV / 4;        // threads per state row (4 columns each)
  constexpr int RG = 256 / TPR;      // row groups
  constexpr int RPT = DK / RG;       // rows per thread
  constexpr int RG_PER_WAVE = 64 / TPR;
  static_assert(RPT * RG == DK, "rows must split evenly");

  const int64_t sid = blockIdx.x;    // state index n * H + h
  const int tid = threadIdx.x;
  const int cg = tid % TPR;
  const int rg = tid / TPR;
  const int wave = tid / 64;

  __shared__ float s_k[DK], s_q[DK], s_a[DK], s_kw[DK];
  __shared__ float s_u[4][DV], s_w[4][DV];
  __shared__ float s_kq;

  const elem* q = static_cast<const elem*>(p.q);
  const elem* k = static_cast<const elem*>(p.k);
  const elem* v = static_cast<const elem*>(p.v);
  const elem* beta = static_cast<const elem*>(p.beta);
  const elem* log_a = static_cast<const elem*>(p.log_a);

  // Issue the state reads first: they are the only large transfer.
  const float* Sp = p.S + sid * (DK * DV);
  float4 st[RPT];
#pragma unroll
  for (int m = 0; m < RPT; ++m)
    st[m] = *reinterpret_cast<const float4*>(Sp + (rg + RG * m) * DV + 4 * cg);

  if (tid < DK) {
    s_k[tid] = Io<IO>::load(k, sid * DK + tid);
    s_q[tid] = Io<IO>::load(q, sid * DK + tid);
    s_kw[tid] = p.kw ? Io<IO>::load(static_cast<const elem*>(p.kw), sid * DK + tid) : s_k[tid];
    if (GATE == GATE_CHANNEL) s_a[tid] = __expf(Io<IO>::load(log_a, sid * DK + tid));
  }
  float a_scalar = 1.f;
  if (GATE == GATE_SCALAR) a_scalar = __expf(Io<IO>::load(log_a, sid));
  const float b = Io<IO>::load(beta, sid);
  float vv[4];
#pragma unroll
  for (int j = 0; j < 4; ++j) vv[j] = Io<IO>::load(v, sid * DV + 4 * cg + j);
  __syncthreads();

  if (wave == 0) {  // (write key) . q, reduced across the first wave
    float kq = 0.f;
    for (int i = tid; i < DK; i += 64) kq += s_kw[i] * s_q[i];
#pragma unroll
    for (int off = 32; off > 0; off >>= 1) kq += __shfl_xor(kq, off);
    if (tid == 0) s_kq = kq;
  }

  // Decay, then partial u = S^T k (of the decayed or, literal ordering, the
  // previous state) and w = S~^T q over this thread's rows.
  float4 u = make_float4(0.f, 0.f, 0.f, 0.f), w = u;
#pragma unroll
  for (int m = 0; m < RPT; ++m) {
    const int i = rg + RG * m;
    const float ki = s_k[i], qi = s_q[i];
    float4 s = st[m];
    if (p.literal) { u.x += s.x * ki; u.y += s.y * ki; u.z += s.z * ki; u.w += s.w * ki; }
    if (GATE != GATE_NONE) {
      const float ai = (GATE == GATE_CHANNEL) ? s_a[i] : a_scalar;
      s.x *= ai; s.y *= ai; s.z *= ai; s.w *= ai;
    }
    if (!p.literal) { u.x += s.x * ki; u.y += s.y * ki; u.z += s.z * ki; u.w += s.w * ki; }
    w.x += s.x * qi; w.y += s.y * qi; w.z += s.z * qi; w.w += s.w * qi;
    st[m] = s;
  }
  // Reduce over the row groups of this wave (lanes sharing a column group).
#pragma unroll
  for (int off = TPR; off < 64; off <<= 1) {
    u.x += __shfl_xor(u.x, off); u.y += __shfl_xor(u.y, off);
    u.z += __shfl_xor(u.z, off); u.w += __shfl_xor(u.w, off);
    w.x += __shfl_xor(w.x, off); w.y += __shfl_xor(w.y, off);
    w.z += __shfl_xor(w.z, off); w.w += __shfl_xor(w.w, off);
  }
  if ((tid % 64) < TPR) {
    s_u[wave][4 * cg + 0] = u.x; s_u[wave][4 * cg + 1] = u.y;
    s_u[wave][4 * cg + 2] = u.z; s_u[wave][4 * cg + 3] = u.w;
    s_w[wave][4 * cg + 0] = w.x; s_w[wave][4 * cg + 1] = w.y;
    s_w[wave][4 * cg + 2] = w.z; s_w[wave][4 * cg + 3] = w.w;
  }
  __syncthreads();
  (void)RG_PER_WAVE;

  float d[4], wf[4];
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    const int c = 4 * cg + j;
    const float uc = s_u[0][c] + s_u[1][c] + s_u[2][c] + s_u[3][c];
    wf[j] = s_w[0][c] + s_w[1][c] + s_w[2][c] + s_w[3][c];
    d[j] = b * (vv[j] - uc);
  }

  // S' = S~ + k delta^T, written over the same addresses that were read, with
  // non-temporal stores (the state is not read again in this step; measured
  // faster than ordinary stores for this read-all-then-write-all pattern).
  float* Sn = p.S_new + sid * (DK * DV);
#pragma unroll
  for (int m = 0; m < RPT; ++m) {
    const int i = rg + RG * m;
    const float ki = s_kw[i];
    f32x4 s = {st[m].x + ki * d[0], st[m].y + ki * d[1], st[m].z + ki * d[2], st[m].w + ki * d[3]};
    __builtin_nontemporal_store(s, reinterpret_cast<f32x4*>(Sn + i * DV + 4 * cg));
  }
  if (rg == 0) {
    elem* o = static_cast<elem*>(p.o);
    const float kq = s_kq;
#pragma unroll
    for (int j = 0; j < 4; ++j) Io<IO>::store(o, sid * DV + 4 * cg + j, wf[j] + d[j] * kq);
  }
}

template <int IO, int GATE, int DK, int DV>
static hipError_t launch_decode_t(const DecodeParams& p, hipStream_t stream) {
  hipLaunchKernelGGL((decode_step_kernel<IO, GATE, DK, DV>), dim3(static_cast<unsigned>(p.n_states)),
                     dim3(256), 0, stream, p);
  return hipGetLastError();
}

template <int IO, int GATE>
static hipError_t launch_decode_g(const DecodeParams& p, hipStream_t stream) {
  if (p.d_k == 128 && p.d_v == 128) return launch_decode_t<IO, GATE, 128, 128>(p, stream);
  if (p.d_k == 128 && p.d_v == 64) return launch_decode_t<IO, GATE, 128, 64>(p, stream);
  if (p.d_k == 64 && p.d_v == 128) return launch_decode_t<IO, GATE, 64, 128>(p, stream);
  if (p.d_k == 64 && p.d_v == 64) return launch_decode_t<IO, GATE, 64, 64>(p, stream);
  return hipErrorInvalidValue;
}

template <int IO>
static hipError_t launch_decode_io(const DecodeParams& p, hipStream_t stream) {
  switch (p.gate) {
    case GATE_NONE: return launch_decode_g<IO, GATE_NONE>(p, stream);
    case GATE_SCALAR: return launch_decode_g<IO, GATE_SCALAR>(p, stream);
    case GATE_CHANNEL: return launch_decode_g<IO, GATE_CHANNEL>(p, stream);
  }
  return hipErrorInvalidValue;
}

hipError_t launch_decode_step(const DecodeParams& p, hipStream_t stream) {
  if (p.n_states == 0) return hipSuccess;
  return p.io == IO_BF16 ? launch_decode_io<IO_BF16>(p, stream) : launch_decode_io<IO_F32>(p, stream);
}

}  // namespace gdr
