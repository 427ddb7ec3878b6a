// Chunkwise-parallel forward of the gated delta rule on gfx950 (one fused kernel).
//
// Method: "Moonshot AI's New Attention Architecture: Key Innovations Explained",
// §3 Hardware-Friendly Algorithm -- the sequence is cut into chunks of C = 64
// tokens; inside a chunk the work is dense (lower-triangular) matrix products,
// between chunks only the d_k x d_v state is passed on; §5 Practical
// Considerations -- the cumulative gate is kept in the log domain.  The update
// being computed is the per-channel gated delta rule of §2 of the same page
// (key-major state S, d_k rows, d_v columns):
//     S_t = (I - beta_t k_t k_t^T) diag(a_t) S_{t-1} + beta_t k_t v_t^T,  o_t = S_t^T q_t.
//
// Per chunk (rows r = 0..63, g_r = inclusive running sum of log a inside the chunk,
// S the state entering the chunk):
//   A     = strict_lower( diag(beta) (K*e^{g_read}) (K*e^{-g})^T )     g_read = g (decay
//           before the erase) or g_{r-1} (erase reads the undecayed state)
//   W     = (I + A)^{-1} diag(beta) (K*e^{g_read}),   U = (I + A)^{-1} diag(beta) V
//   Delta = U - W S
//   O     = (Q*e^{g}) S + lower_incl( (Q*e^{g}) (K*e^{-g})^T ) Delta
//   S'    = diag(e^{g_63}) S + (K*e^{g_63 - g})^T Delta
// (the correction terms W, U and the two state/output equations of §3; the
// query/key decay factors as derived from the §2 update, see the design notes).
//
// Work decomposition.  One workgroup of NW waves owns one (batch, head, d_v tile
// of 16*NW columns) and walks the chunks in order.  Wave w owns 16 state
// columns: its slice of S (d_k x 16, fp32) lives in MFMA accumulators for the
// whole sequence.  An accumulator tile (lane l: column l%16, rows 4(l/16)+s) is
// exactly the B-operand layout of the next product, so W*S, Q*S and the state
// update chain through registers without touching LDS.  The d_v-independent
// per-chunk work (log-gate scan, decayed operands, the 16x16 blocks of A and of
// the masked score matrix P, the four diagonal 16x16 inverses) is shared by the
// waves through LDS.  (I + A)^{-1} is never formed: each wave solves for its own
// columns of W and U by forward substitution over the four 16-row blocks
// (inverse diagonal block times right-hand side minus the blocks already solved).
//
// Numerics.  Decay factors are computed in the log domain.  For the score
// matrices the factor e^{g_r - g_j} is split at the first row of each 16-row
// block (e^{g_r - g_16R} on rows, e^{g_16J - g_j} on columns, and e^{g_16R - g_16J}
// on the column operand of blocks below the diagonal), so no operand exceeds the
// decay accumulated over 15 tokens.  Products run on bf16 MFMA with fp32
// accumulation for bf16 I/O and on fp32 MFMA for fp32 I/O; the state stays fp32.
#include "device_common.h"
#include "launchers.h"

namespace gdr {

constexpr int CH = 64;   // chunk length

template <int IO> struct Op;
template <> struct Op<IO_BF16> {
  typedef __bf16 T;
  typedef bf16x4 frag;
  static constexpr int PAD = 8;
  static __device__ __forceinline__ frag ld(const T* p) { return *reinterpret_cast<const frag*>(p); }
  static __device__ __forceinline__ void st(T* p, frag x) { *reinterpret_cast<frag*>(p) = x; }
  static __device__ __forceinline__ frag cvt(f32x4 x) { return to_bf16x4(x); }
  static __device__ __forceinline__ f32x4 f32(frag x) {
    f32x4 r;
    r[0] = static_cast<float>(x[0]); r[1] = static_cast<float>(x[1]);
    r[2] = static_cast<float>(x[2]); r[3] = static_cast<float>(x[3]);
    return r;
  }
  static __device__ __forceinline__ T from(float x) { return static_cast<__bf16>(x); }
  static __device__ __forceinline__ f32x4 mma2(f32x4 acc, frag a0, frag a1, frag b0, frag b1) {
    return mma_k32_bf16(acc, a0, a1, b0, b1);
  }
  static __device__ __forceinline__ f32x4 mma1(f32x4 acc, frag a, frag b) { return mma_k16_bf16(acc, a, b); }
};
template <> struct Op<IO_F32> {
  typedef float T;
  typedef f32x4 frag;
  static constexpr int PAD = 4;
  static __device__ __forceinline__ frag ld(const T* p) { return *reinterpret_cast<const frag*>(p); }
  static __device__ __forceinline__ void st(T* p, frag x) { *reinterpret_cast<frag*>(p) = x; }
  static __device__ __forceinline__ frag cvt(f32x4 x) { return x; }
  static __device__ __forceinline__ f32x4 f32(frag x) { return x; }
  static __device__ __forceinline__ T from(float x) { return x; }
  static __device__ __forceinline__ f32x4 mma2(f32x4 acc, frag a0, frag a1, frag b0, frag b1) {
    return mma_k16_f32(mma_k16_f32(acc, a0, b0), a1, b1);
  }
  static __device__ __forceinline__ f32x4 mma1(f32x4 acc, frag a, frag b) { return mma_k16_f32(acc, a, b); }
};

constexpr size_t cmax(size_t a, size_t b) { return a > b ? a : b; }

// LDS layout (bytes).  Regions that are dead by the time a later phase writes
// share storage: W over the row operand of A, the diagonal inverses over the
// column operand, and A and P over the log-gate scan buffer.
template <int IO, int GATE, int DK, int NW>
struct Layout {
  typedef typename Op<IO>::T T;
  static constexpr int PAD = Op<IO>::PAD;
  static constexpr int LDK = DK + PAD;    // row stride of [64][DK] tiles
  static constexpr int LCH = CH + PAD;    // row stride of [*][64] tiles
  static constexpr int LA = CH + 4;       // row stride of the fp32 A matrix
  static constexpr int LXI = 16 + PAD;    // row stride of the 16x16 inverses
  static constexpr int DVT = 16 * NW;
  static constexpr int NSEG = (64 * NW) / DK > 0 ? (64 * NW) / DK : 1;
  static constexpr size_t TILE_RM = size_t(CH) * LDK * sizeof(T);
  static constexpr size_t TILE_T = size_t(DK) * LCH * sizeof(T);
  static constexpr size_t XINV = size_t(4) * 16 * LXI * sizeof(T);
  static constexpr size_t A_BYTES = size_t(CH) * LA * 4;
  static constexpr size_t P_BYTES = size_t(CH) * LCH * sizeof(T);
  static constexpr size_t G_BYTES = GATE == GATE_CHANNEL ? size_t(CH) * DK * 4 : size_t(CH) * 4;
  static constexpr size_t OFF_XK = 0;                                   // X_K, then W
  static constexpr size_t OFF_Y = OFF_XK + TILE_RM;                     // Y, then inverses
  static constexpr size_t OFF_XQ = OFF_Y + cmax(TILE_RM, XINV);
  static constexpr size_t OFF_QH = OFF_XQ + TILE_RM;
  static constexpr size_t OFF_KRT = OFF_QH + TILE_RM;
  static constexpr size_t OFF_KDT = OFF_KRT + TILE_T;
  static constexpr size_t OFF_VT = OFF_KDT + TILE_T;
  static constexpr size_t OFF_G = OFF_VT + size_t(DVT) * LCH * sizeof(T);   // g, then A and P
  static constexpr size_t OFF_P = OFF_G + A_BYTES;
  static constexpr size_t OFF_BETA = OFF_G + cmax(G_BYTES, A_BYTES + P_BYTES);
  static constexpr size_t OFF_GAM = OFF_BETA + CH * 4;
  static constexpr size_t OFF_M = OFF_GAM + DK * 4;
  static constexpr size_t OFF_TOT = OFF_M + 6 * DK * 4;
  static constexpr size_t TOTAL = OFF_TOT + NSEG * DK * 4;
};

// (R, J) block pairs of the lower triangle (incl. diagonal) of a 4x4 block grid.
__device__ __forceinline__ void lower_pair(int t, int& R, int& J) {
  R = (t >= 1) + (t >= 3) + (t >= 6);
  J = t - R * (R + 1) / 2;
}
// Index of a strictly-lower pair (R > J) in 0..5.
__device__ __forceinline__ int strict_pair(int R, int J) { return R * (R - 1) / 2 + J; }

template <int IO, int GATE, int DK, int NW>
__global__ __launch_bounds__(NW * 64) void chunk_fwd_kernel(ChunkParams p, int n_tiles) {
  typedef Op<IO> O;
  typedef typename O::T T;
  typedef typename O::frag frag;
  typedef typename Io<IO>::elem elem;
  typedef Layout<IO, GATE, DK, NW> L;
  constexpr int NT = NW * 64;
  constexpr int DVT = 16 * NW;
  constexpr int DKT = DK / 16;
  constexpr int CBW = DKT / NW;          // 16-channel blocks of W solved per wave
  constexpr int LDK = L::LDK, LCH = L::LCH, LA = L::LA, LXI = L::LXI;
  static_assert(CBW >= 1 && CBW * NW == DKT, "channel blocks must split over waves");

  __shared__ __attribute__((aligned(16))) char smem[L::TOTAL];
  T* sXK = reinterpret_cast<T*>(smem + L::OFF_XK);
  T* sW = sXK;
  T* sY = reinterpret_cast<T*>(smem + L::OFF_Y);
  T* sXi = sY;
  T* sXQ = reinterpret_cast<T*>(smem + L::OFF_XQ);
  T* sQh = reinterpret_cast<T*>(smem + L::OFF_QH);
  T* sKrT = reinterpret_cast<T*>(smem + L::OFF_KRT);
  T* sKdT = reinterpret_cast<T*>(smem + L::OFF_KDT);
  T* sVT = reinterpret_cast<T*>(smem + L::OFF_VT);
  float* sG = reinterpret_cast<float*>(smem + L::OFF_G);
  float* sA = sG;
  T* sP = reinterpret_cast<T*>(smem + L::OFF_P);
  float* sBeta = reinterpret_cast<float*>(smem + L::OFF_BETA);
  float* sGam = reinterpret_cast<float*>(smem + L::OFF_GAM);
  float* sM = reinterpret_cast<float*>(smem + L::OFF_M);
  float* sTot = reinterpret_cast<float*>(smem + L::OFF_TOT);

  const elem* gq = static_cast<const elem*>(p.q);
  const elem* gk = static_cast<const elem*>(p.k);
  const elem* gv = static_cast<const elem*>(p.v);
  const elem* gbeta = static_cast<const elem*>(p.beta);
  const elem* gla = static_cast<const elem*>(p.log_a);
  elem* go = static_cast<elem*>(p.o);

  // Block -> (head, d_v tile).  Consecutive logical blocks land on one XCD (the
  // hardware deals block ids round-robin over 8 XCDs), so the tiles of one head
  // share that XCD's L2 for their common q, k, log_a reads.
  const int nblk = gridDim.x;
  int lb = blockIdx.x;
  if ((nblk & 7) == 0) lb = (blockIdx.x & 7) * (nblk >> 3) + (blockIdx.x >> 3);
  const int64_t bh = lb / n_tiles;
  const int tile = lb % n_tiles;
  const int64_t bb = bh / p.H, hh = bh % p.H;
  const int dv = p.d_v;
  const int col0 = tile * DVT;

  const int tid = threadIdx.x;
  const int wave = tid >> 6;
  const int lane = tid & 63;
  const int lr = lane & 15;
  const int lg = lane >> 4;
  const int scol = col0 + 16 * wave + lr;   // this lane's state / output column

  auto tok = [&](int64_t t) -> int64_t { return (bb * p.T + t) * p.H + hh; };
  auto G = [&](int r, int i) -> float {
    if (GATE == GATE_CHANNEL) return sG[r * DK + i];
    if (GATE == GATE_SCALAR) return sG[r];
    return 0.f;
  };

  // State slice: S[t][s] = S[16t + 4lg + s][scol].
  f32x4 S[DKT];
#pragma unroll
  for (int t = 0; t < DKT; ++t)
#pragma unroll
    for (int s = 0; s < 4; ++s)
      S[t][s] = p.S0 ? p.S0[(bh * DK + 16 * t + 4 * lg + s) * dv + scol] : 0.f;

  const int64_t nchunks = (p.T + CH - 1) / CH;
  for (int64_t n = 0; n < nchunks; ++n) {
    const int64_t t0 = n * CH;
    const int nrows = static_cast<int>(p.T - t0 < CH ? p.T - t0 : CH);

    // ---- (1) beta and the per-chunk cumulative log-gate -------------------------
    if (tid < CH) sBeta[tid] = tid < nrows ? Io<IO>::load(gbeta, tok(t0 + tid)) : 0.f;
    if (GATE == GATE_SCALAR) {
      if (wave == 0) {
        float x = lane < nrows ? Io<IO>::load(gla, tok(t0 + lane)) : 0.f;
#pragma unroll
        for (int off = 1; off < 64; off <<= 1) {
          const float y = __shfl_up(x, off);
          if (lane >= off) x += y;
        }
        sG[lane] = x;
      }
      __syncthreads();
      if (tid == 0) {
        sGam[0] = __expf(sG[CH - 1]);
#pragma unroll
        for (int R = 1; R < 4; ++R)
          for (int J = 0; J < R; ++J) sM[strict_pair(R, J)] = __expf(sG[16 * R] - sG[16 * J]);
      }
    } else if (GATE == GATE_CHANNEL) {
      for (int idx = tid; idx < CH * DK; idx += NT) {
        const int r = idx / DK, i = idx % DK;
        sG[idx] = r < nrows ? Io<IO>::load(gla, tok(t0 + r) * DK + i) : 0.f;
      }
      __syncthreads();
      constexpr int NSEG = L::NSEG;
      constexpr int SEGL = CH / NSEG;
      if (tid < NSEG * DK) {
        const int i = tid % DK, seg = tid / DK;
        float acc = 0.f;
        for (int r = seg * SEGL; r < (seg + 1) * SEGL; ++r) {
          acc += sG[r * DK + i];
          sG[r * DK + i] = acc;
        }
        sTot[seg * DK + i] = acc;
      }
      __syncthreads();
      if (NSEG > 1 && tid < NSEG * DK) {
        const int i = tid % DK, seg = tid / DK;
        float pre = 0.f;
        for (int s2 = 0; s2 < seg; ++s2) pre += sTot[s2 * DK + i];
        if (seg > 0)
          for (int r = seg * SEGL; r < (seg + 1) * SEGL; ++r) sG[r * DK + i] += pre;
      }
      __syncthreads();
      for (int i = tid; i < DK; i += NT) {
        sGam[i] = __expf(sG[(CH - 1) * DK + i]);
#pragma unroll
        for (int R = 1; R < 4; ++R)
          for (int J = 0; J < R; ++J) sM[strict_pair(R, J) * DK + i] = __expf(sG[16 * R * DK + i] - sG[16 * J * DK + i]);
      }
    } else {
      __syncthreads();
    }

    // ---- (2) decayed operands in LDS --------------------------------------------
    for (int idx = tid; idx < CH * (DK / 4); idx += NT) {
      const int r = idx / (DK / 4);
      const int i0 = (idx % (DK / 4)) * 4;
      const int R = r >> 4;
      float kk[4], qq[4];
      const bool live = r < nrows;
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        kk[j] = live ? Io<IO>::load(gk, tok(t0 + r) * DK + i0 + j) : 0.f;
        qq[j] = live ? Io<IO>::load(gq, tok(t0 + r) * DK + i0 + j) : 0.f;
      }
      const float be = sBeta[r];
      f32x4 xk, y, xq, qh;
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const int i = i0 + j;
        float e_xk = 1.f, e_y = 1.f, e_xq = 1.f, e_q = 1.f, e_kr = 1.f, e_kd = 1.f;
        if (GATE != GATE_NONE) {
          const float g = G(r, i), gR = G(16 * R, i), gC = G(CH - 1, i);
          const float gread = p.literal ? (r > 0 ? G(r - 1, i) : 0.f) : g;
          e_xk = __expf(gread - gR);
          e_y = __expf(gR - g);
          e_xq = __expf(g - gR);
          e_q = __expf(g);
          e_kr = __expf(gread);
          e_kd = __expf(gC - g);
        }
        xk[j] = be * kk[j] * e_xk;
        y[j] = kk[j] * e_y;
        xq[j] = qq[j] * e_xq;
        qh[j] = qq[j] * e_q;
        sKrT[i * LCH + r] = O::from(be * kk[j] * e_kr);
        sKdT[i * LCH + r] = O::from(kk[j] * e_kd);
      }
      O::st(sXK + r * LDK + i0, O::cvt(xk));
      O::st(sY + r * LDK + i0, O::cvt(y));
      O::st(sXQ + r * LDK + i0, O::cvt(xq));
      O::st(sQh + r * LDK + i0, O::cvt(qh));
    }
    for (int idx = tid; idx < CH * (DVT / 4); idx += NT) {
      const int r = idx / (DVT / 4);
      const int c0 = (idx % (DVT / 4)) * 4;
      const bool live = r < nrows;
      const float be = sBeta[r];
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        const float vv = live ? Io<IO>::load(gv, tok(t0 + r) * dv + col0 + c0 + j) : 0.f;
        sVT[(c0 + j) * LCH + r] = O::from(be * vv);
      }
    }
    __syncthreads();

    // ---- (3) 16x16 blocks of A (strictly lower) and P (lower incl. diagonal) ----
    for (int task = wave; task < 20; task += NW) {
      const bool isP = task >= 10;
      int R, J;
      lower_pair(task % 10, R, J);
      const T* rows = isP ? sXQ : sXK;
      f32x4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int kb = 0; kb < DK / 32; ++kb) {
        const int c = 32 * kb + 4 * lg;
        frag a0 = O::ld(rows + (16 * R + lr) * LDK + c);
        frag a1 = O::ld(rows + (16 * R + lr) * LDK + c + 16);
        frag b0 = O::ld(sY + (16 * J + lr) * LDK + c);
        frag b1 = O::ld(sY + (16 * J + lr) * LDK + c + 16);
        if (GATE != GATE_NONE && R > J) {
          const int pr = strict_pair(R, J);
          f32x4 m0, m1;
#pragma unroll
          for (int s = 0; s < 4; ++s) {
            m0[s] = GATE == GATE_CHANNEL ? sM[pr * DK + c + s] : sM[pr];
            m1[s] = GATE == GATE_CHANNEL ? sM[pr * DK + c + 16 + s] : sM[pr];
          }
          b0 = O::cvt(O::f32(b0) * m0);
          b1 = O::cvt(O::f32(b1) * m1);
        }
        acc = O::mma2(acc, a0, a1, b0, b1);
      }
#pragma unroll
      for (int s = 0; s < 4; ++s) {
        const int rr = 4 * lg + s;
        if (!isP) {
          sA[(16 * R + rr) * LA + 16 * J + lr] = (R == J && rr <= lr) ? 0.f : acc[s];
        } else {
          sP[(16 * R + rr) * LCH + 16 * J + lr] = O::from((R == J && rr < lr) ? 0.f : acc[s]);
        }
      }
    }
    __syncthreads();

    // ---- (4) inverses of the four unit-lower diagonal blocks of I + A -----------
    if (wave == 0) {
      const int R = lane >> 4, j = lane & 15;
      float x[16];
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        float acc = (i == j) ? 1.f : 0.f;
#pragma unroll
        for (int kk = 0; kk < i; ++kk) acc -= sA[(16 * R + i) * LA + 16 * R + kk] * x[kk];
        x[i] = acc;
      }
#pragma unroll
      for (int i = 0; i < 16; ++i) sXi[(16 * R + i) * LXI + j] = O::from(x[i]);
    }
    __syncthreads();

    // ---- (5) W and U by block forward substitution (per wave, own columns) ------
    // out_R = X_RR (rhs_R - sum_{J<R} A_RJ out_J), rhs taken from a transposed
    // [column][row] buffer.
    auto solve = [&](const T* rhsT, int colrow, f32x4* out) {
      frag outb[4];
#pragma unroll
      for (int R = 0; R < 4; ++R) {
        f32x4 acc = O::f32(O::ld(rhsT + colrow * LCH + 16 * R + 4 * lg));
        int J = 0;
#pragma unroll
        for (; J + 1 < R; J += 2) {
          const float* ar = sA + (16 * R + lr) * LA;
          f32x4 a0 = *reinterpret_cast<const f32x4*>(ar + 16 * J + 4 * lg);
          f32x4 a1 = *reinterpret_cast<const f32x4*>(ar + 16 * (J + 1) + 4 * lg);
          acc = O::mma2(acc, O::cvt(-a0), O::cvt(-a1), outb[J], outb[J + 1]);
        }
        if (J < R) {
          f32x4 a0 = *reinterpret_cast<const f32x4*>(sA + (16 * R + lr) * LA + 16 * J + 4 * lg);
          acc = O::mma1(acc, O::cvt(-a0), outb[J]);
        }
        f32x4 z = {0.f, 0.f, 0.f, 0.f};
        z = O::mma1(z, O::ld(sXi + (16 * R + lr) * LXI + 4 * lg), O::cvt(acc));
        out[R] = z;
        outb[R] = O::cvt(z);
      }
    };
#pragma unroll
    for (int cb = 0; cb < CBW; ++cb) {
      const int ch = (wave * CBW + cb) * 16;
      f32x4 w[4];
      solve(sKrT, ch + lr, w);
      // sW shares storage with the row operand of A, which is dead after (3).
#pragma unroll
      for (int R = 0; R < 4; ++R)
#pragma unroll
        for (int s = 0; s < 4; ++s) sW[(16 * R + 4 * lg + s) * LDK + ch + lr] = O::from(w[R][s]);
    }
    f32x4 U[4];
    solve(sVT, 16 * wave + lr, U);
    __syncthreads();

    // ---- (6) state pass and output for this wave's 16 columns ------------------
    frag Sb[DKT];
#pragma unroll
    for (int t = 0; t < DKT; ++t) Sb[t] = O::cvt(S[t]);
    frag Db[4];
#pragma unroll
    for (int R = 0; R < 4; ++R) {            // Delta = U - W S
      f32x4 ws = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int kb = 0; kb < DK / 32; ++kb) {
        const T* wr = sW + (16 * R + lr) * LDK + 32 * kb + 4 * lg;
        ws = O::mma2(ws, O::ld(wr), O::ld(wr + 16), Sb[2 * kb], Sb[2 * kb + 1]);
      }
      Db[R] = O::cvt(U[R] - ws);
    }
#pragma unroll
    for (int R = 0; R < 4; ++R) {            // O = (Q e^g) S + P Delta
      f32x4 oacc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int kb = 0; kb < DK / 32; ++kb) {
        const T* qr = sQh + (16 * R + lr) * LDK + 32 * kb + 4 * lg;
        oacc = O::mma2(oacc, O::ld(qr), O::ld(qr + 16), Sb[2 * kb], Sb[2 * kb + 1]);
      }
      const T* pr = sP + (16 * R + lr) * LCH + 4 * lg;
      int J = 0;
#pragma unroll
      for (; J + 1 <= R; J += 2) oacc = O::mma2(oacc, O::ld(pr + 16 * J), O::ld(pr + 16 * (J + 1)), Db[J], Db[J + 1]);
      if (J <= R) oacc = O::mma1(oacc, O::ld(pr + 16 * J), Db[J]);
#pragma unroll
      for (int s = 0; s < 4; ++s) {
        const int r = 16 * R + 4 * lg + s;
        if (r < nrows) Io<IO>::store(go, tok(t0 + r) * dv + scol, oacc[s]);
      }
    }
#pragma unroll
    for (int t = 0; t < DKT; ++t) {          // S' = diag(e^{g_63}) S + Kd^T Delta
      f32x4 acc = S[t];
      if (GATE == GATE_CHANNEL) {
#pragma unroll
        for (int s = 0; s < 4; ++s) acc[s] *= sGam[16 * t + 4 * lg + s];
      } else if (GATE == GATE_SCALAR) {
        acc = acc * sGam[0];
      }
      const T* kr = sKdT + (16 * t + lr) * LCH + 4 * lg;
      acc = O::mma2(acc, O::ld(kr), O::ld(kr + 16), Db[0], Db[1]);
      acc = O::mma2(acc, O::ld(kr + 32), O::ld(kr + 48), Db[2], Db[3]);
      S[t] = acc;
    }
    __syncthreads();                          // LDS is rewritten by the next chunk
  }

  if (p.S_T) {
#pragma unroll
    for (int t = 0; t < DKT; ++t)
#pragma unroll
      for (int s = 0; s < 4; ++s) p.S_T[(bh * DK + 16 * t + 4 * lg + s) * dv + scol] = S[t][s];
  }
}

template <int IO, int GATE, int DK, int NW>
static hipError_t launch_chunk_t(const ChunkParams& p, hipStream_t stream) {
  const int n_tiles = p.d_v / (16 * NW);
  const int64_t nblk = p.B * p.H * n_tiles;
  hipLaunchKernelGGL((chunk_fwd_kernel<IO, GATE, DK, NW>), dim3(static_cast<unsigned>(nblk)), dim3(NW * 64), 0,
                     stream, p, n_tiles);
  return hipGetLastError();
}

template <int IO, int GATE, int DK>
static hipError_t launch_chunk_dk(const ChunkParams& p, hipStream_t stream) {
  if constexpr (IO == IO_F32) {
    return launch_chunk_t<IO, GATE, DK, 2>(p, stream);
  } else {
    // Four waves (64 columns per workgroup) when that still gives at least one
    // workgroup per CU, otherwise two waves (32 columns) to fill the 256 CUs.
    const int64_t wg4 = p.B * p.H * (p.d_v / 64);
    if (wg4 >= 256) return launch_chunk_t<IO, GATE, DK, 4>(p, stream);
    return launch_chunk_t<IO, GATE, DK, 2>(p, stream);
  }
}

template <int IO, int GATE>
static hipError_t launch_chunk_g(const ChunkParams& p, hipStream_t stream) {
  if (p.d_k == 128) {
    if constexpr (IO == IO_F32) {
      return hipErrorInvalidValue;   // fp32 I/O: d_k = 64 only (LDS budget)
    } else {
      return launch_chunk_dk<IO, GATE, 128>(p, stream);
    }
  }
  if (p.d_k == 64) return launch_chunk_dk<IO, GATE, 64>(p, stream);
  return hipErrorInvalidValue;
}

template <int IO>
static hipError_t launch_chunk_io(const ChunkParams& p, hipStream_t stream) {
  switch (p.gate) {
    case GATE_NONE: return launch_chunk_g<IO, GATE_NONE>(p, stream);
    case GATE_SCALAR: return launch_chunk_g<IO, GATE_SCALAR>(p, stream);
    case GATE_CHANNEL: return launch_chunk_g<IO, GATE_CHANNEL>(p, stream);
  }
  return hipErrorInvalidValue;
}

hipError_t launch_chunk_fwd(const ChunkParams& p, hipStream_t stream) {
  if (p.B * p.H == 0) return hipSuccess;
  return p.io == IO_BF16 ? launch_chunk_io<IO_BF16>(p, stream) : launch_chunk_io<IO_F32>(p, stream);
}

}  // namespace gdr
