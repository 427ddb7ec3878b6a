// Preconditioner scan of the preconditioned delta rule on gfx950.
//
// "OSDN: Improving Delta Rule with Provable Online Preconditioning in Linear
// Attention", §2.2: a first phase runs over the keys alone; each token's write
// key is the current diagonal preconditioner times the key, after which the
// preconditioner takes one online-gradient step on the closed-form surrogate
// h_t(d) = ((1 - beta_t <d, k_t^2>)^2 - 1) / (2 ||k_t||^2).  §2.3 (APF) scales
// the preconditioner by a per-token retention r_t.  Per (sequence, head):
//
//     kw_t    = d_t * k_t
//     d_{t+1} = r_t d_t + e_t w_t,     w_t = k_t^2,
//     e_t     = gam_t - alf_t <d_t, w_t>,   gam_t = eta beta_t / n_t,
//                                           alf_t = eta beta_t^2 / n_t,  n_t = ||k_t||^2
//
// (a descent step; a zero key adds nothing).  This is a delta rule whose state
// is the vector d: erase coefficient alf_t, key w_t, retention r_t.
//
// bf16 I/O: the chunkwise form of that recurrence (the same derivation as the
// chunkwise delta rule, with a state of width one).  With g_t the sum of
// log r_j over the chunk's tokens j < t, a chunk of 64 tokens starting from d_0:
//
//     x_t = <d_t, w_t> = e^{g_t} <w_t, d_0> + sum_{s<t} e^{g_t - g_{s+1}} e_s <w_t, w_s>
//     e   = (I + M)^{-1} b,   M_ts = alf_t e^{g_t - g_{s+1}} <w_t, w_s> (s < t),
//                             b_t  = gam_t - alf_t e^{g_t} <w_t, d_0>
//     d_t = e^{g_t} d_0 + sum_{s<t} e^{g_t - g_{s+1}} e_s w_s        (kw_t = d_t * k_t)
//     d_64 = e^{g_64} d_0 + sum_s e^{g_64 - g_{s+1}} e_s w_s.
//
// One 512-thread workgroup owns one (sequence, head) and walks its chunks in
// order, software-pipelined over neighbouring chunks (see the kernel).  The Gram
// matrix of the w_t and the product that forms every d_t run on
// MFMA with bf16 operands and fp32 accumulation; the unit lower triangular solve
// is a forward substitution by one wave (lane t holds row t of M, each step
// broadcasts e_s); the preconditioner itself, <w_t, d_0> and the chunk-end
// update stay in fp32 (w_t = k_t^2 is exact in fp32 for a bf16 key).
//
// fp32 I/O: a token-by-token scan, one wave per (sequence, head).
#include "chunk_common.h"

namespace gdr {

namespace {

template <int CTRL, int ROW_MASK = 0xF, bool BOUND_ZERO = false>
__device__ __forceinline__ float dpp(float old, float v) {
  return __int_as_float(__builtin_amdgcn_update_dpp(__float_as_int(old), __float_as_int(v), CTRL, ROW_MASK, 0xF,
                                                    BOUND_ZERO));
}

// Inclusive prefix sum over the 64 lanes of a wave (rows of 16 by shifts, then
// the row totals carried across rows).
__device__ __forceinline__ float wave_prefix_sum(float v) {
  v += dpp<0x111, 0xF, true>(0.f, v);   // row_shr:1
  v += dpp<0x112, 0xF, true>(0.f, v);   // row_shr:2
  v += dpp<0x114, 0xF, true>(0.f, v);   // row_shr:4
  v += dpp<0x118, 0xF, true>(0.f, v);   // row_shr:8
  v += dpp<0x142, 0xA>(0.f, v);         // row_bcast:15 into rows 1 and 3
  v += dpp<0x143, 0xC>(0.f, v);         // row_bcast:31 into rows 2 and 3
  return v;
}

// Sum over the wave, the same value returned to every lane.
__device__ __forceinline__ float wave_sum(float v) {
  return __int_as_float(__builtin_amdgcn_readlane(__float_as_int(wave_prefix_sum(v)), 63));
}

// Sum over aligned groups of four lanes, returned to all four.
__device__ __forceinline__ float quad_sum(float v) {
  v += dpp<0xB1>(0.f, v);   // quad_perm [1,0,3,2]
  v += dpp<0x4E>(0.f, v);   // quad_perm [2,3,0,1]
  return v;
}

}  // namespace

// ---------------------------------------------------------------------------
// fp32 I/O: token by token.  Lane l holds channels l*CPL .. l*CPL + CPL - 1.
// ---------------------------------------------------------------------------
template <int DK, bool HAS_R>
__global__ __launch_bounds__(64) void precond_scan_seq_kernel(PrecondParams p) {
  constexpr int CPL = DK / 64;
  constexpr int U = 16;   // tokens per block; the next block is loaded while this one runs
  const int64_t bh = blockIdx.x;
  const int64_t b = bh / p.H, h = bh - b * p.H;
  const int64_t T = p.T, H = p.H;
  const int lane = threadIdx.x;
  const float* __restrict__ k = static_cast<const float*>(p.k);
  const float* __restrict__ beta = static_cast<const float*>(p.beta);
  const float* __restrict__ r = static_cast<const float*>(p.r);
  float* __restrict__ kw = static_cast<float*>(p.kw);

  float d[CPL];
#pragma unroll
  for (int i = 0; i < CPL; ++i) d[i] = p.d0 ? p.d0[bh * DK + lane * CPL + i] : 1.f;

  float kc[U][CPL] = {}, bc[U] = {}, rc[U] = {}, kn[U][CPL] = {}, bn[U] = {}, rn[U] = {};
  // Tokens past the end read the last token (in bounds) and are skipped.
  auto load = [&](int64_t t0, float (&kx)[U][CPL], float (&bx)[U], float (&rx)[U]) {
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int64_t row = (b * T + (t0 + u < T ? t0 + u : T - 1)) * H + h;
#pragma unroll
      for (int i = 0; i < CPL; ++i) kx[u][i] = k[row * DK + lane * CPL + i];
      bx[u] = beta[row];
      rx[u] = HAS_R ? r[row] : 1.f;
    }
  };
  if (T > 0) load(0, kc, bc, rc);
  for (int64_t t0 = 0; t0 < T; t0 += U) {
    if (t0 + U < T) load(t0 + U, kn, bn, rn);
#pragma unroll
    for (int u = 0; u < U; ++u) {
      if (t0 + u >= T) break;
      const int64_t row = (b * T + t0 + u) * H + h;
      float w[CPL], x = 0.f, n = 0.f;
#pragma unroll
      for (int i = 0; i < CPL; ++i) {
        w[i] = kc[u][i] * kc[u][i];
        x = fmaf(d[i], w[i], x);
        n += w[i];
        kw[row * DK + lane * CPL + i] = d[i] * kc[u][i];
      }
      x = wave_sum(x);
      n = wave_sum(n);
      const float bt = bc[u];
      const float e = n > 0.f ? p.eta * bt * (1.f - bt * x) / n : 0.f;
#pragma unroll
      for (int i = 0; i < CPL; ++i) d[i] = fmaf(e, w[i], rc[u] * d[i]);
    }
#pragma unroll
    for (int u = 0; u < U; ++u) {
      bc[u] = bn[u];
      rc[u] = rn[u];
#pragma unroll
      for (int i = 0; i < CPL; ++i) kc[u][i] = kn[u][i];
    }
  }
  if (p.d_T) {
#pragma unroll
    for (int i = 0; i < CPL; ++i) p.d_T[bh * DK + lane * CPL + i] = d[i];
  }
}

// ---------------------------------------------------------------------------
// bf16 I/O: chunkwise and software-pipelined, one 512-thread workgroup (8 waves)
// per (sequence, head).  Iteration n of the chunk loop runs, between barriers:
//   1. wave 0: forward substitution of chunk n (the dependent chain), then two
//      tiles of the Gram matrix M of chunk n+1;  waves 1-4: output k~ of chunk
//      n-1;  waves 5-6: the rest of M of chunk n+1;  wave 7: stage chunk n+2
//      into LDS and prefetch chunk n+3;
//   2. all: partial sums of the chunk-end update of chunk n;
//   3. d_0 of chunk n+1;
//   4. all: <w_t, d_0> of chunk n+1.
// Only steps 1 (the substitution), 2, 3 and 4 are on the chain; the output,
// the Gram matrix and the staging of neighbouring chunks run beside it.  Key
// tiles are kept for four chunks (n-1 .. n+2) and w = k^2 is formed from them
// as operands are loaded.
// ---------------------------------------------------------------------------
template <int DK>
struct PsLayout {
  static constexpr int NW = 8, NT = 64 * NW;   // waves, threads
  static constexpr int LDK = DK + 8;           // bf16 row stride of the key tiles
  static constexpr int LM = CH + 4;            // fp32 row stride of M
  static constexpr int NKB = 4;                // key tiles of chunks n-1 .. n+2
  static constexpr int NP = DK / 2;            // channel pairs in the chunk-end update
  static constexpr int NQ = NT / NP;           // token groups in the chunk-end update
  static constexpr int TPQ = CH / NQ;          // tokens per group
  static constexpr int KV = DK / 32;           // 16-byte key pieces per loader lane and round
  static constexpr int CT = DK / 64;           // 16-channel output tiles per output wave
  static constexpr int PCH = DK / 8;           // channels per thread in <w_t, d_0>
  static constexpr size_t KB_BYTES = size_t(CH) * LDK * 2;
  static constexpr size_t M_BYTES = size_t(CH) * LM * 4;
  static constexpr size_t K_OFF = 0;
  static constexpr size_t M_OFF = K_OFF + NKB * KB_BYTES;
  static constexpr size_t D_OFF = M_OFF + 2 * M_BYTES;          // d_0, two chunks
  static constexpr size_t Q_OFF = D_OFF + size_t(2) * DK * 4;   // update partials [NQ][DK]
  static constexpr size_t T_OFF = Q_OFF + size_t(NQ) * DK * 4;  // per-token rows, four chunks
  // n_t, <w_t, d_0>, beta_t, g_t, g_{t+1}, e^{g_t}, e^{-g_{t+1}}, e_t (scaled), c_t
  static constexpr int TR_N = 0, TR_P = 1, TR_BETA = 2, TR_GEX = 3, TR_GIN = 4, TR_R = 5, TR_IR = 6, TR_EH = 7,
                       TR_C = 8, TR_ROWS = 9;
  static constexpr size_t TOK_FLOATS = size_t(TR_ROWS) * CH;
  static constexpr size_t BYTES = T_OFF + NKB * TOK_FLOATS * 4;
};

// The factored form of the decays (e^{g_t - g_{s+1}} = e^{g_t} e^{-g_{s+1}}) is
// used when the chunk's total log-retention is at least this; both factors then
// stay within fp32 range.  Below it, each entry takes its own exponential.
constexpr float PS_FACTOR_MIN_G = -80.f;

// bf16 squares of four bf16 keys (w = k^2 as an MFMA operand).
__device__ __forceinline__ bf16x4 ps_sq(bf16x4 k) {
  const f32x4 x = Op<IO_BF16>::f32(k);
  return to_bf16x4(f32x4{x[0] * x[0], x[1] * x[1], x[2] * x[2], x[3] * x[3]});
}

// Gram tiles, (R, J) blocks of W W^T with J <= R: four each for the two Gram
// waves, two for the substitution wave once its chain is done.
template <int W> struct PsGram;
template <> struct PsGram<0> {
  static constexpr int N = 4, NEED = 0x7;
  static constexpr int R[4] = {0, 1, 1, 2}, J[4] = {0, 0, 1, 0};
};
template <> struct PsGram<1> {
  static constexpr int N = 4, NEED = 0xF;
  static constexpr int R[4] = {3, 3, 3, 3}, J[4] = {0, 1, 2, 3};
};
template <> struct PsGram<2> {
  static constexpr int N = 2, NEED = 0x6;
  static constexpr int R[4] = {2, 2, 0, 0}, J[4] = {1, 2, 0, 0};
};

// M_ts = alf_t e^{g_t - g_{s+1}} <w_t, w_s> for s < t (0 elsewhere) into Ms.
template <int DK, bool HAS_R, int W, bool FACT>
__device__ __forceinline__ void precond_gram(const __bf16* Kb, float* Ms, const float* tok, float eta, int lr,
                                             int lg) {
  typedef PsLayout<DK> L;
  typedef Op<IO_BF16> op;
  typedef PsGram<W> G;
  f32x4 acc[G::N];
#pragma unroll
  for (int i = 0; i < G::N; ++i) acc[i] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
  for (int k0 = 0; k0 < DK; k0 += 32) {
    op::frag lo[4], hi[4];
#pragma unroll
    for (int R = 0; R < 4; ++R)
      if (G::NEED & (1 << R)) {
        const __bf16* row = Kb + (16 * R + lr) * L::LDK + k0 + 4 * lg;
        lo[R] = ps_sq(op::ld(row));
        hi[R] = ps_sq(op::ld(row + 16));
      }
#pragma unroll
    for (int i = 0; i < G::N; ++i)
      acc[i] = op::mma2(acc[i], lo[G::R[i]], hi[G::R[i]], lo[G::J[i]], hi[G::J[i]]);
  }
#pragma unroll
  for (int i = 0; i < G::N; ++i) {
    const int t4 = 16 * G::R[i] + 4 * lg, s = 16 * G::J[i] + lr;
    const f32x4 nn = *reinterpret_cast<const f32x4*>(tok + L::TR_N * CH + t4);
    const f32x4 be = *reinterpret_cast<const f32x4*>(tok + L::TR_BETA * CH + t4);
    const f32x4 rt = *reinterpret_cast<const f32x4*>(tok + L::TR_R * CH + t4);
    const f32x4 gx = *reinterpret_cast<const f32x4*>(tok + L::TR_GEX * CH + t4);
    const float irs = tok[L::TR_IR * CH + s], gs = tok[L::TR_GIN * CH + s];
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      // A zero key has a zero Gram row, so a clamped n_t is enough.
      const float alf = eta * be[q] * be[q] * __builtin_amdgcn_rcpf(fmaxf(nn[q], 1e-30f));
      float dec = 1.f;
      if (HAS_R) dec = FACT ? rt[q] * irs : __expf(fminf(gx[q] - gs, 0.f));
      Ms[(t4 + q) * L::LM + s] = (s < t4 + q ? 1.f : 0.f) * alf * dec * acc[i][q];
    }
  }
}

// Output of one output wave (ow = 0..3): k~_t = d_t * k_t for channel tiles
// CT*ow .. CT*ow + CT - 1 and all four 16-token blocks.  D^T = W^T L^T + d_0 e^{g_t}
// is formed as 16x16 tiles (rows: channels, columns: tokens), so each lane ends
// with four consecutive channels of one token.  FACT: D_t = e^{g_t} (d_0 +
// sum_{s<t} e_s e^{-g_{s+1}} w_s) (the EH row holds e_s e^{-g_{s+1}}); otherwise each
// L_ts = e^{g_t - g_{s+1}} e_s is formed with its own exponential (EH holds e_s).
template <int DK, bool FACT>
__device__ __forceinline__ void precond_output(const __bf16* Kb, const float* d0, const float* tok, rsrc_t kwr,
                                               uint32_t so, int64_t H, int64_t h, int ow, int lr, int lg) {
  typedef PsLayout<DK> L;
  typedef Op<IO_BF16> op;
  const float* teh = tok + L::TR_EH * CH;
  const float* tR = tok + L::TR_R * CH;
  op::frag ef[4], edf[4];   // factored operands: off-diagonal and diagonal (masked) blocks
  if (FACT) {
#pragma unroll
    for (int sb = 0; sb < 4; ++sb) {
      const f32x4 ev = *reinterpret_cast<const f32x4*>(teh + 16 * sb + 4 * lg);
      f32x4 dm;
#pragma unroll
      for (int j = 0; j < 4; ++j) dm[j] = 4 * lg + j < lr ? ev[j] : 0.f;
      ef[sb] = op::cvt(ev);
      edf[sb] = op::cvt(dm);
    }
  }
  auto bfrag = [&](int TB, int sb) -> op::frag {
    if (FACT) return sb < TB ? ef[sb] : edf[sb];
    const int t = 16 * TB + lr;
    const float gt = tok[L::TR_GEX * CH + t];
    const f32x4 gi = *reinterpret_cast<const f32x4*>(tok + L::TR_GIN * CH + 16 * sb + 4 * lg);
    const f32x4 ev = *reinterpret_cast<const f32x4*>(teh + 16 * sb + 4 * lg);
    f32x4 x;
#pragma unroll
    for (int j = 0; j < 4; ++j)
      x[j] = (16 * sb + 4 * lg + j < t ? 1.f : 0.f) * __expf(fminf(gt - gi[j], 0.f)) * ev[j];
    return op::cvt(x);
  };
#pragma unroll
  for (int ci = 0; ci < L::CT; ++ci) {
    const int c0 = 16 * (L::CT * ow + ci);
    op::frag af[4];
#pragma unroll
    for (int sb = 0; sb < 4; ++sb) af[sb] = ps_sq(op::ld_tr(Kb, L::LDK, 16 * sb, c0, lr, lg));
    const f32x4 dv = *reinterpret_cast<const f32x4*>(d0 + c0 + 4 * lg);
#pragma unroll
    for (int TB = 0; TB < 4; ++TB) {
      const int t = 16 * TB + lr;
      const float Rt = tR[t];
      const float pre = FACT ? 1.f : Rt, post = FACT ? Rt : 1.f;
      f32x4 acc = {pre * dv[0], pre * dv[1], pre * dv[2], pre * dv[3]};
#pragma unroll
      for (int sb = 0; sb + 1 <= TB; sb += 2)
        acc = op::mma2(acc, af[sb], af[sb + 1], bfrag(TB, sb), bfrag(TB, sb + 1));
      if ((TB & 1) == 0) acc = op::mma1(acc, af[TB], bfrag(TB, TB));
      const f32x4 kv = op::f32(op::ld(Kb + t * L::LDK + c0 + 4 * lg));
      const f32x4 o = {post * acc[0] * kv[0], post * acc[1] * kv[1], post * acc[2] * kv[2], post * acc[3] * kv[3]};
      const uint32_t voff = static_cast<uint32_t>((t * H + h) * DK + c0 + 4 * lg) * 2;
      buf_store8(__builtin_bit_cast(u32x2, to_bf16x4(o)), kwr, voff, so);
    }
  }
}

template <int DK, bool HAS_R>
__global__ __launch_bounds__(512) void precond_scan_chunk_kernel(PrecondParams p) {
  typedef PsLayout<DK> L;
  typedef Op<IO_BF16> op;
  typedef op::T bf;
  __shared__ __align__(16) unsigned char smem[L::BYTES];
  auto kbuf = [&](int64_t i) { return reinterpret_cast<bf*>(smem + L::K_OFF + (i & 3) * L::KB_BYTES); };
  auto mbuf = [&](int64_t i) { return reinterpret_cast<float*>(smem + L::M_OFF + (i & 1) * L::M_BYTES); };
  auto tbuf = [&](int64_t i) { return reinterpret_cast<float*>(smem + L::T_OFF) + (i & 3) * L::TOK_FLOATS; };
  float* dbuf = reinterpret_cast<float*>(smem + L::D_OFF);
  float* part = reinterpret_cast<float*>(smem + L::Q_OFF);

  const int tid = threadIdx.x;
  // the wave index is uniform: keeping it scalar makes every role test a scalar
  // branch (and keeps buffer offsets in scalar registers)
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6), lane = tid & 63;
  const int lr = lane & 15, lg = lane >> 4;
  const int64_t bh = blockIdx.x;
  const int64_t b = bh / p.H, h = bh - b * p.H;
  const int64_t T = p.T, H = p.H;
  const float eta = p.eta;
  const int64_t nch = (T + CH - 1) / CH;

  // Buffer ranges over this sequence's slab: loads past the last token return
  // zero and stores there are dropped, so the ragged last chunk needs no branch.
  const uint32_t slab = static_cast<uint32_t>(T * H);
  const rsrc_t kr = make_rsrc(static_cast<const uint16_t*>(p.k) + b * T * H * DK, slab * DK * 2);
  const rsrc_t kwr = make_rsrc(static_cast<uint16_t*>(p.kw) + b * T * H * DK, slab * DK * 2);
  const rsrc_t br = make_rsrc(static_cast<const uint16_t*>(p.beta) + b * T * H, slab * 2);
  const rsrc_t rr = make_rsrc(HAS_R ? static_cast<const uint16_t*>(p.r) + b * T * H : nullptr, HAS_R ? slab * 2 : 0);

  // Both M buffers zeroed once: blocks above the diagonal are never written.
  for (int i = tid; i < 2 * CH * L::LM; i += L::NT) reinterpret_cast<float*>(smem + L::M_OFF)[i] = 0.f;
  if (tid < DK) dbuf[tid] = p.d0 ? p.d0[bh * DK + tid] : 1.f;

  // ---- the staging wave (wave 7): lane (token 16i + lane/4, quarter lane%4) in
  // round i loads channels 8*(quarter + 4j) .. +7; lane also loads the factors of
  // token `lane`.  Loads for chunk c + 1 are issued as soon as chunk c is staged.
  const int sq = lane & 3, st = lane >> 2;
  u32x4 kreg[4][L::KV];
  uint16_t beta_r = 0, r_r = 0;
  auto load_chunk = [&](int64_t c) {
    const uint32_t so = __builtin_amdgcn_readfirstlane(static_cast<uint32_t>(c * CH * H * DK * 2));
    const uint32_t sb = __builtin_amdgcn_readfirstlane(static_cast<uint32_t>(c * CH * H * 2));
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
      for (int j = 0; j < L::KV; ++j)
        kreg[i][j] = buf_load16(kr, static_cast<uint32_t>(((16 * i + st) * H + h) * DK + 8 * (sq + 4 * j)) * 2, so);
    beta_r = buf_load2(br, static_cast<uint32_t>(lane * H + h) * 2, sb);
    if (HAS_R) r_r = buf_load2(rr, static_cast<uint32_t>(lane * H + h) * 2, sb);
  };
  auto stage = [&](int64_t c) {
    bf* Kb = kbuf(c);
    float* tk = tbuf(c);
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int t = 16 * i + st;
      float sn = 0.f;
#pragma unroll
      for (int j = 0; j < L::KV; ++j) {
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const float k0 = __uint_as_float(kreg[i][j][e] << 16), k1 = __uint_as_float(kreg[i][j][e] & 0xFFFF0000u);
          sn = fmaf(k0, k0, sn);
          sn = fmaf(k1, k1, sn);
        }
        *reinterpret_cast<u32x4*>(Kb + t * L::LDK + 8 * (sq + 4 * j)) = kreg[i][j];
      }
      sn = quad_sum(sn);
      if (sq == 0) tk[L::TR_N * CH + t] = sn;
    }
    const bool ok = c * CH + lane < T;
    const float lrv = HAS_R && ok ? __logf(bf16_bits_to_f32(r_r)) : 0.f;
    const float gin = HAS_R ? wave_prefix_sum(lrv) : 0.f;
    tk[L::TR_BETA * CH + lane] = bf16_bits_to_f32(beta_r);   // zero past the end
    tk[L::TR_GIN * CH + lane] = gin;
    tk[L::TR_GEX * CH + lane] = gin - lrv;
    tk[L::TR_R * CH + lane] = HAS_R ? __expf(gin - lrv) : 1.f;
    tk[L::TR_IR * CH + lane] = HAS_R ? __expf(-gin) : 1.f;   // read only by the factored form
  };
  auto factored = [&](int64_t c) {   // the chunk's total log-retention allows the factored form
    if (!HAS_R) return true;
    const float gC = __int_as_float(__builtin_amdgcn_readfirstlane(__float_as_int(tbuf(c)[L::TR_GIN * CH + CH - 1])));
    return gC >= PS_FACTOR_MIN_G;
  };
  if (wave == L::NW - 1 && nch > 0) load_chunk(0);
  __syncthreads();   // M zeroed, d_0 in place

  for (int64_t n = -2; n <= nch; ++n) {
    // ---- 1. substitution (n) | output (n-1) | Gram (n+1) | stage (n+2) --------------
    if (wave == 0) {
      if (n >= 0 && n < nch) {
        const float* tk = tbuf(n);
        float m[CH];
        const float* mrow = mbuf(n) + lane * L::LM;
#pragma unroll
        for (int i = 0; i < CH; i += 4) {
          const f32x4 v = *reinterpret_cast<const f32x4*>(mrow + i);
          m[i] = v[0]; m[i + 1] = v[1]; m[i + 2] = v[2]; m[i + 3] = v[3];
        }
        const float nn = tk[L::TR_N * CH + lane], be = tk[L::TR_BETA * CH + lane];
        const float gam = nn > 0.f ? eta * be * __builtin_amdgcn_rcpf(nn) : 0.f;   // alf_t = gam_t beta_t
        float acc = gam - gam * be * tk[L::TR_R * CH + lane] * tk[L::TR_P * CH + lane];
#pragma unroll
        for (int s = 0; s < CH; ++s) {
          const float es = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(acc), s));
          acc = fmaf(-m[s], es, acc);
        }
        const bool fact = factored(n);
        float* tkw = tbuf(n);
        // e_t e^{-g_{t+1}} for the factored output; e_t itself otherwise
        tkw[L::TR_EH * CH + lane] = fact && HAS_R ? acc * tk[L::TR_IR * CH + lane] : acc;
        tkw[L::TR_C * CH + lane] =
            HAS_R ? __expf(tk[L::TR_GIN * CH + CH - 1] - tk[L::TR_GIN * CH + lane]) * acc : acc;
      }
      if (n + 1 >= 0 && n + 1 < nch) {   // its share of the Gram matrix of chunk n+1
        const int64_t c = n + 1;
        if (factored(c)) precond_gram<DK, HAS_R, 2, true>(kbuf(c), mbuf(c), tbuf(c), eta, lr, lg);
        else precond_gram<DK, HAS_R, 2, false>(kbuf(c), mbuf(c), tbuf(c), eta, lr, lg);
      }
    } else if (wave <= 4) {
      if (n >= 1 && n <= nch) {
        const int64_t c = n - 1;
        const uint32_t so = __builtin_amdgcn_readfirstlane(static_cast<uint32_t>(c * CH * H * DK * 2));
        if (factored(c)) precond_output<DK, true>(kbuf(c), dbuf + (c & 1) * DK, tbuf(c), kwr, so, H, h, wave - 1, lr, lg);
        else precond_output<DK, false>(kbuf(c), dbuf + (c & 1) * DK, tbuf(c), kwr, so, H, h, wave - 1, lr, lg);
      }
    } else if (wave <= 6) {
      if (n + 1 >= 0 && n + 1 < nch) {
        const int64_t c = n + 1;
        const bool fact = factored(c);
        if (wave == 5) {
          if (fact) precond_gram<DK, HAS_R, 0, true>(kbuf(c), mbuf(c), tbuf(c), eta, lr, lg);
          else precond_gram<DK, HAS_R, 0, false>(kbuf(c), mbuf(c), tbuf(c), eta, lr, lg);
        } else {
          if (fact) precond_gram<DK, HAS_R, 1, true>(kbuf(c), mbuf(c), tbuf(c), eta, lr, lg);
          else precond_gram<DK, HAS_R, 1, false>(kbuf(c), mbuf(c), tbuf(c), eta, lr, lg);
        }
      }
    } else {
      if (n + 2 < nch) {
        stage(n + 2);
        if (n + 3 < nch) load_chunk(n + 3);
      }
    }
    __syncthreads();

    // ---- 2. partial sums of c_s w_s over token groups (chunk n) ----------------------
    if (n >= 0 && n < nch) {
      const bf* Kb = kbuf(n);
      const float* tc = tbuf(n) + L::TR_C * CH;
      const int cp = tid % L::NP, qd = tid / L::NP;
      float cs[L::TPQ];
      uint32_t ku[L::TPQ];
#pragma unroll
      for (int i = 0; i < L::TPQ; i += 4) {
        const f32x4 cv = *reinterpret_cast<const f32x4*>(tc + qd * L::TPQ + i);
#pragma unroll
        for (int q = 0; q < 4; ++q) cs[i + q] = cv[q];
      }
#pragma unroll
      for (int i = 0; i < L::TPQ; ++i)
        ku[i] = *reinterpret_cast<const uint32_t*>(Kb + (qd * L::TPQ + i) * L::LDK + 2 * cp);
      float a0 = 0.f, a1 = 0.f;
#pragma unroll
      for (int i = 0; i < L::TPQ; ++i) {
        const float k0 = __uint_as_float(ku[i] << 16), k1 = __uint_as_float(ku[i] & 0xFFFF0000u);
        a0 = fmaf(cs[i], k0 * k0, a0);
        a1 = fmaf(cs[i], k1 * k1, a1);
      }
      *reinterpret_cast<float2*>(part + qd * DK + 2 * cp) = make_float2(a0, a1);
    }
    __syncthreads();

    // ---- 3. d_0 of chunk n+1 = e^{g_64} d_0 + sum_s c_s w_s ------------------------
    if (n >= 0 && n < nch && tid < DK) {
      const float RC = HAS_R ? __expf(tbuf(n)[L::TR_GIN * CH + CH - 1]) : 1.f;
      float s = RC * dbuf[(n & 1) * DK + tid];
#pragma unroll
      for (int q = 0; q < L::NQ; ++q) s += part[q * DK + tid];
      dbuf[((n + 1) & 1) * DK + tid] = s;
    }
    __syncthreads();

    // ---- 4. <w_t, d_0> of chunk n+1, fp32: thread (token tid/8, eighth) -------------
    if (n + 1 >= 0 && n + 1 < nch) {
      const int64_t c = n + 1;
      const int t = tid >> 3, e8 = tid & 7;
      const bf* row = kbuf(c) + t * L::LDK + L::PCH * e8;
      const float* d0 = dbuf + (c & 1) * DK + L::PCH * e8;
      float sp = 0.f;
#pragma unroll
      for (int j = 0; j < L::PCH; j += 8) {
        const u32x4 kv = *reinterpret_cast<const u32x4*>(row + j);
        const f32x4 da = *reinterpret_cast<const f32x4*>(d0 + j);
        const f32x4 db = *reinterpret_cast<const f32x4*>(d0 + j + 4);
#pragma unroll
        for (int e = 0; e < 4; ++e) {
          const float k0 = __uint_as_float(kv[e] << 16), k1 = __uint_as_float(kv[e] & 0xFFFF0000u);
          sp = fmaf(k0 * k0, e < 2 ? da[2 * e] : db[2 * e - 4], sp);
          sp = fmaf(k1 * k1, e < 2 ? da[2 * e + 1] : db[2 * e - 3], sp);
        }
      }
      sp = quad_sum(sp);
      sp += dpp<0x141>(0.f, sp);   // row_half_mirror: the other quad of the 8
      if (e8 == 0) tbuf(c)[L::TR_P * CH + t] = sp;
    }
    __syncthreads();
  }
  if (p.d_T && tid < DK) p.d_T[bh * DK + tid] = dbuf[(nch & 1) * DK + tid];
}

template <int DK, bool HAS_R>
static hipError_t launch_chunk_t(const PrecondParams& p, hipStream_t stream) {
  constexpr size_t lds = PsLayout<DK>::BYTES;
  static_assert(lds <= 160 * 1024, "LDS budget");
  hipLaunchKernelGGL((precond_scan_chunk_kernel<DK, HAS_R>), dim3(static_cast<unsigned>(p.B * p.H)),
                     dim3(PsLayout<DK>::NT), 0, stream, p);
  return hipGetLastError();
}

template <int DK, bool HAS_R>
static hipError_t launch_seq_t(const PrecondParams& p, hipStream_t stream) {
  hipLaunchKernelGGL((precond_scan_seq_kernel<DK, HAS_R>), dim3(static_cast<unsigned>(p.B * p.H)), dim3(64), 0,
                     stream, p);
  return hipGetLastError();
}

hipError_t launch_precond_scan(const PrecondParams& p, hipStream_t stream) {
  if (p.B * p.H == 0) return hipSuccess;
  const bool hr = p.r != nullptr;
  if (p.io == IO_BF16) {
    if (p.d_k == 128) return hr ? launch_chunk_t<128, true>(p, stream) : launch_chunk_t<128, false>(p, stream);
    if (p.d_k == 64) return hr ? launch_chunk_t<64, true>(p, stream) : launch_chunk_t<64, false>(p, stream);
    return hipErrorInvalidValue;
  }
  if (p.d_k == 128) return hr ? launch_seq_t<128, true>(p, stream) : launch_seq_t<128, false>(p, stream);
  if (p.d_k == 64) return hr ? launch_seq_t<64, true>(p, stream) : launch_seq_t<64, false>(p, stream);
  return hipErrorInvalidValue;
}

}  // namespace gdr
