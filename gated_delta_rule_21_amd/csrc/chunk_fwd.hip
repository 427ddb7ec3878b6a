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
// query/key decay factors as derived from the §2 update).
//
// Work decomposition.  One workgroup of NW waves owns one (batch, head, d_v tile
// of 16*NW columns) and walks the chunks in order.  Wave w owns 16 state
// columns: its slice of S (d_k x 16, fp32) lives in MFMA accumulators for the
// whole sequence.  An accumulator tile (lane l: column l%16, rows 4(l/16)+s) is
// the operand layout of the next product, so W*S, the output and the state
// update chain through registers.  The d_v-independent per-chunk work (log-gate
// scan, the 16x16 blocks of A and of the masked score matrix P, the diagonal
// 16x16 inverses) is shared by the waves through LDS.  (I + A)^{-1} is never
// formed: each wave solves for its own columns of W and U by forward
// substitution over the four 16-row blocks.
//
// Memory.  q, k, v, beta and the log-gate are read once per chunk with buffer
// loads into registers one chunk ahead of their use; a buffer's range ends at
// the last token of the sequence, so the rows of a ragged last chunk read as
// zero.  Tiles sit row-major in LDS; products that contract over the chunk rows
// (the state update, the right-hand sides of W and U) read them with the gfx950
// LDS transpose load, so no transposed copy is made.  The output is computed
// transposed, so each lane stores four adjacent columns.
//
// Gates.  With no gate or a scalar gate the decay factors are per row and per
// column of the 64x64 intra-chunk matrices, so the products run on the raw
// q, k, v tiles and the factors are applied to the results (A and P element by
// element, the output and Delta row by row).  A per-channel gate sits inside
// the d_k contraction, so decayed operands are built first; for the score
// matrices the factor e^{g_r - g_j} is split at the first row of each 16-row
// block (e^{g_r - g_16R} on rows, e^{g_16J - g_j} on columns, e^{g_16R - g_16J} on
// the column operand of blocks below the diagonal), so no operand exceeds the
// decay accumulated over 15 tokens.
//
// Products run on bf16 MFMA with fp32 accumulation for bf16 I/O and on fp32
// MFMA for fp32 I/O; the state stays fp32.
#include <type_traits>

#include "device_common.h"
#include "launchers.h"

namespace gdr {

constexpr int CH = 64;   // chunk length

template <int IO> struct Op;
template <> struct Op<IO_BF16> {
  typedef __bf16 T;
  typedef bf16x4 frag;
  static constexpr int PAD = 8;      // row stride 4 (mod 32) dwords: fewest LDS bank conflicts (measured)
  static __device__ __forceinline__ frag ld(const T* p) { return *reinterpret_cast<const frag*>(p); }
  // Fragment holding M[r0 + 4*lg + s][c0 + lr], s = 0..3, of a row-major tile M:
  // the gfx950 LDS transpose load gathers it from 16 lanes' 8-byte reads.
  static __device__ __forceinline__ frag ld_tr(const T* m, int ld, int r0, int c0, int lr, int lg) {
    const T* a = m + (r0 + 4 * lg + (lr >> 2)) * ld + c0 + 4 * (lr & 3);
    typedef __attribute__((ext_vector_type(4))) short v4s;
    typedef __attribute__((address_space(3))) v4s lds_v4s;
    const v4s x = __builtin_amdgcn_ds_read_tr16_b64_v4i16((lds_v4s*)(const_cast<T*>(a)));
    return __builtin_bit_cast(frag, x);
  }
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
  static __device__ __forceinline__ frag ld_tr(const T* m, int ld, int r0, int c0, int lr, int lg) {
    frag f;
#pragma unroll
    for (int s = 0; s < 4; ++s) f[s] = m[(r0 + 4 * lg + s) * ld + c0 + lr];
    return f;
  }
  static __device__ __forceinline__ frag cvt(f32x4 x) { return x; }
  static __device__ __forceinline__ f32x4 f32(frag x) { return x; }
  static __device__ __forceinline__ T from(float x) { return x; }
  static __device__ __forceinline__ f32x4 mma2(f32x4 acc, frag a0, frag a1, frag b0, frag b1) {
    return mma_k16_f32(mma_k16_f32(acc, a0, b0), a1, b1);
  }
  static __device__ __forceinline__ f32x4 mma1(f32x4 acc, frag a, frag b) { return mma_k16_f32(acc, a, b); }
};

constexpr size_t cmax(size_t a, size_t b) { return a > b ? a : b; }

// LDS layout (bytes).  Row-major tiles: [64][DK] with stride LDK, the v tile
// [64][DVT] with stride LVT, the 64x64 matrices with stride LCH.
template <int IO, int GATE, int DK, int NW>
struct Layout {
  typedef typename Op<IO>::T T;
  static constexpr bool RAW = GATE != GATE_CHANNEL;   // products on raw q, k, v
  static constexpr int PAD = Op<IO>::PAD;
  static constexpr int LDK = DK + PAD;
  static constexpr int LCH = CH + PAD;
  static constexpr int LXI = 16 + (sizeof(T) == 2 ? 8 : 4);
  static constexpr int LSC = 20;                       // per-wave 16x16 fp32 scratch stride
  static constexpr int DVT = 16 * NW;
  static constexpr int LVT = DVT + PAD;
  static constexpr int NSEG = (64 * NW) / DK > 0 ? (64 * NW) / DK : 1;
  static constexpr size_t RM = size_t(CH) * LDK * sizeof(T);      // [64][DK]
  static constexpr size_t MM = size_t(CH) * LCH * sizeof(T);      // [64][64]
  static constexpr size_t XI_B = size_t(CH) * LXI * sizeof(T);
  static constexpr size_t V_B = size_t(CH) * LVT * sizeof(T);
  static constexpr size_t SC_B = size_t(NW) * 16 * LSC * 4;
  // common regions
  static constexpr size_t OFF_K = 0;                     // raw k (per-channel gate: X_K in place)
  static constexpr size_t OFF_Q = OFF_K + RM;            // raw q (per-channel gate: X_Q in place)
  static constexpr size_t OFF_V = OFF_Q + RM;            // raw v tile
  static constexpr size_t OFF_XI = OFF_V + V_B;          // inverses of the diagonal blocks
  static constexpr size_t OFF_SC = OFF_XI + XI_B;        // per-wave scratch of the inversion
  static constexpr size_t OFF_X = OFF_SC + SC_B;         // gate-dependent regions start here
  // raw gates
  static constexpr size_t R_W = OFF_X;
  static constexpr size_t R_A = R_W + RM;                // -A (off-diagonal blocks)
  static constexpr size_t R_P = R_A + MM;
  static constexpr size_t R_SMALL = R_P + MM;            // beta, g, g_read, e_w, e_o, e_d, gamma
  static constexpr size_t R_TOTAL = R_SMALL + 7 * CH * 4;
  // per-channel gate (W reuses X_K)
  static constexpr size_t C_Y = OFF_X;                   // column operand of the score blocks
  static constexpr size_t C_QH = C_Y + RM;               // q e^{g}
  static constexpr size_t C_KR = C_QH + RM;              // beta k e^{g_read}
  static constexpr size_t C_KD = C_KR + RM;              // k e^{g_63 - g}
  static constexpr size_t C_G = C_KD + RM;               // g [64][DK] fp32, then -A and P
  static constexpr size_t C_G_B = cmax(size_t(CH) * DK * 4, 2 * MM);
  static constexpr size_t C_BETA = C_G + C_G_B;
  static constexpr size_t C_GAM = C_BETA + CH * 4;
  static constexpr size_t C_M = C_GAM + DK * 4;
  static constexpr size_t C_TOT = C_M + 6 * DK * 4;
  static constexpr size_t C_TOTAL = C_TOT + NSEG * DK * 4;
  static constexpr size_t TOTAL = RAW ? R_TOTAL : C_TOTAL;
};

__device__ __forceinline__ int strict_pair(int R, int J) { return R * (R - 1) / 2 + J; }

// Ordering point for LDS traffic between the lanes of one wave.
__device__ __forceinline__ void wave_sync() {
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
  __builtin_amdgcn_wave_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
}

// (I + N)^{-1} of a strictly lower 16x16 block N held as an accumulator tile, by
// the finite Neumann product (I - N)(I + N^2)(I + N^4)(I + N^8) (N^16 = 0), on
// fp32 MFMA.  `scr` is this wave's 16x16 fp32 scratch, used to turn an
// accumulator tile into a row-major A operand.
__device__ __forceinline__ f32x4 unit_lower_inverse(f32x4 N, float* scr, int lr, int lg) {
  constexpr int LSC = 20;
  auto put = [&](f32x4 M) {
#pragma unroll
    for (int s = 0; s < 4; ++s) scr[(4 * lg + s) * LSC + lr] = M[s];
  };
  auto rows = [&]() -> f32x4 { return *reinterpret_cast<const f32x4*>(scr + lr * LSC + 4 * lg); };
  const f32x4 zero = {0.f, 0.f, 0.f, 0.f};
  f32x4 Y;
#pragma unroll
  for (int s = 0; s < 4; ++s) Y[s] = (4 * lg + s == lr ? 1.f : 0.f) - N[s];
  put(N);
  wave_sync();
  f32x4 a = rows();
  wave_sync();
  f32x4 P = mma_k16_f32(zero, a, N);          // N^2
  put(P);
  wave_sync();
  a = rows();
  wave_sync();
  Y = mma_k16_f32(Y, a, Y);                   // (I + N^2)(I - N)
  P = mma_k16_f32(zero, a, P);                // N^4
  put(P);
  wave_sync();
  a = rows();
  wave_sync();
  Y = mma_k16_f32(Y, a, Y);
  P = mma_k16_f32(zero, a, P);                // N^8
  put(P);
  wave_sync();
  a = rows();
  wave_sync();
  return mma_k16_f32(Y, a, Y);
}

template <int IO, int GATE, int DK, int NW>
__global__ __launch_bounds__(NW * 64) void chunk_fwd_kernel(ChunkParams p, int n_tiles) {
  typedef Op<IO> O;
  typedef typename O::T T;
  typedef typename O::frag frag;
  typedef typename Io<IO>::elem elem;
  typedef Layout<IO, GATE, DK, NW> L;
  constexpr bool RAW = L::RAW;
  constexpr int NT = NW * 64;
  constexpr int DVT = 16 * NW;
  constexpr int DKT = DK / 16;
  constexpr int CBW = DKT / NW;          // 16-channel blocks of W solved per wave
  constexpr int LDK = L::LDK, LCH = L::LCH, LXI = L::LXI, LVT = L::LVT;
  constexpr int ESZ = int(sizeof(elem));
  constexpr int EPV = 16 / ESZ;          // elements per 16-byte load
  constexpr int KROW = DK / EPV, VROW = DVT / EPV;
  constexpr int KV = CH * KROW / NT;     // 16-byte pieces of a k (q) tile per thread
  constexpr int VV = CH * VROW / NT;     // 16-byte pieces of the v tile per thread
  static_assert(CBW >= 1 && CBW * NW == DKT, "channel blocks must split over waves");
  static_assert(KV * NT == CH * KROW && VV * NT == CH * VROW && VV >= 1, "tile loads must split evenly");
  static_assert(L::TOTAL <= 163840, "LDS budget");

  __shared__ __attribute__((aligned(16))) char smem[L::TOTAL];
  T* sK = reinterpret_cast<T*>(smem + L::OFF_K);
  T* sQ = reinterpret_cast<T*>(smem + L::OFF_Q);
  T* sV = reinterpret_cast<T*>(smem + L::OFF_V);
  T* sXi = reinterpret_cast<T*>(smem + L::OFF_XI);
  float* sScr = reinterpret_cast<float*>(smem + L::OFF_SC);
  // raw-gate regions
  float* sSmall = reinterpret_cast<float*>(smem + L::R_SMALL);
  float* sBr = sSmall;              // beta
  float* sGr = sSmall + CH;         // g
  float* sGrd = sSmall + 2 * CH;    // g_read
  float* sEw = sSmall + 3 * CH;     // beta e^{g_read}   (right-hand side of W)
  float* sEo = sSmall + 4 * CH;     // e^{g}             (output rows)
  float* sEd = sSmall + 5 * CH;     // e^{g_63 - g}      (Delta rows in the state update)
  float* sGamR = sSmall + 6 * CH;   // e^{g_63}
  // per-channel regions
  T* sY = reinterpret_cast<T*>(smem + L::C_Y);
  T* sQh = reinterpret_cast<T*>(smem + L::C_QH);
  T* sKr = reinterpret_cast<T*>(smem + L::C_KR);
  T* sKd = reinterpret_cast<T*>(smem + L::C_KD);
  float* sG = reinterpret_cast<float*>(smem + L::C_G);
  float* sBc = reinterpret_cast<float*>(smem + L::C_BETA);
  float* sGamC = reinterpret_cast<float*>(smem + L::C_GAM);
  float* sM = reinterpret_cast<float*>(smem + L::C_M);
  float* sTot = reinterpret_cast<float*>(smem + L::C_TOT);
  // shared names
  T* sW = RAW ? reinterpret_cast<T*>(smem + L::R_W) : sK;   // X_K is dead once A and P exist
  T* sA = RAW ? reinterpret_cast<T*>(smem + L::R_A) : reinterpret_cast<T*>(smem + L::C_G);
  T* sP = RAW ? reinterpret_cast<T*>(smem + L::R_P) : reinterpret_cast<T*>(smem + L::C_G + L::MM);
  float* sBeta = RAW ? sBr : sBc;

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
  const int H = static_cast<int>(p.H);

  const int tid = threadIdx.x;
  const int wave = tid >> 6;
  const int lane = tid & 63;
  const int lr = lane & 15;
  const int lg = lane >> 4;
  const int scol = col0 + 16 * wave + lr;   // this lane's state column

  // Buffers over this sequence's (b, h) slice; each range ends after the last token.
  const int64_t row0 = bb * p.T * p.H + hh;            // token-row index of (b, t = 0, h)
  const uint32_t span = static_cast<uint32_t>(p.T > 0 ? (p.T - 1) * p.H + 1 : 0);   // rows in range
  const rsrc_t rk = make_rsrc(static_cast<const elem*>(p.k) + row0 * DK, span * DK * ESZ);
  const rsrc_t rq = make_rsrc(static_cast<const elem*>(p.q) + row0 * DK, span * DK * ESZ);
  const rsrc_t rv = make_rsrc(static_cast<const elem*>(p.v) + row0 * dv, span * dv * ESZ);
  const rsrc_t ro = make_rsrc(static_cast<const elem*>(p.o) + row0 * dv, span * dv * ESZ);
  const rsrc_t rb = make_rsrc(static_cast<const elem*>(p.beta) + row0, span * ESZ);
  const rsrc_t rl = make_rsrc(static_cast<const elem*>(p.log_a) + row0 * (GATE == GATE_CHANNEL ? DK : 1),
                              GATE == GATE_NONE ? 0u : span * (GATE == GATE_CHANNEL ? DK : 1) * ESZ);
  // per-thread byte offsets within a chunk (the chunk start goes in the scalar offset)
  uint32_t offk[KV], offv[VV];
#pragma unroll
  for (int v = 0; v < KV; ++v) {
    const int seg = tid + v * NT;
    offk[v] = static_cast<uint32_t>(((seg / KROW) * H * DK + (seg % KROW) * EPV) * ESZ);
  }
#pragma unroll
  for (int v = 0; v < VV; ++v) {
    const int seg = tid + v * NT;
    offv[v] = static_cast<uint32_t>(((seg / VROW) * H * dv + col0 + (seg % VROW) * EPV) * ESZ);
  }
  const uint32_t offb = static_cast<uint32_t>((tid % CH) * H * ESZ);

  // State slice: S[t][s] = S[16t + 4lg + s][scol].
  f32x4 S[DKT];
#pragma unroll
  for (int t = 0; t < DKT; ++t)
#pragma unroll
    for (int s = 0; s < 4; ++s)
      S[t][s] = p.S0 ? p.S0[(bh * DK + 16 * t + 4 * lg + s) * dv + scol] : 0.f;

  // ---- register prefetch of one chunk's inputs ----------------------------------
  u32x4 pk[KV], pq[KV], pl[GATE == GATE_CHANNEL ? KV : 1], pv[VV];
  float pb = 0.f, pls = 0.f;
  auto to_f32 = [&](uint32_t bits) -> float {
    if constexpr (IO == IO_BF16) return bf16_bits_to_f32(static_cast<uint16_t>(bits));
    else return __uint_as_float(bits);
  };
  auto prefetch = [&](int64_t m) __attribute__((always_inline)) {
    const uint32_t sk = static_cast<uint32_t>(m * CH * H * DK * ESZ);
    const uint32_t sv = static_cast<uint32_t>(m * CH * H * dv * ESZ);
    const uint32_t sb = static_cast<uint32_t>(m * CH * H * ESZ);
#pragma unroll
    for (int v = 0; v < KV; ++v) {
      pk[v] = buf_load16(rk, offk[v], sk);
      pq[v] = buf_load16(rq, offk[v], sk);
      if constexpr (GATE == GATE_CHANNEL) pl[v] = buf_load16(rl, offk[v], sk);
    }
#pragma unroll
    for (int v = 0; v < VV; ++v) pv[v] = buf_load16(rv, offv[v], sv);
    if (tid < CH) {
      if constexpr (IO == IO_BF16) {
        pb = to_f32(buf_load2(rb, offb, sb));
        if constexpr (GATE == GATE_SCALAR) pls = to_f32(buf_load2(rl, offb, sb));
      } else {
        pb = to_f32(buf_load4(rb, offb, sb));
        if constexpr (GATE == GATE_SCALAR) pls = to_f32(buf_load4(rl, offb, sb));
      }
    }
  };

  const int64_t nchunks = (p.T + CH - 1) / CH;
  if (nchunks > 0) prefetch(0);

  for (int64_t n = 0; n < nchunks; ++n) {
    const int64_t t0 = n * CH;

    // ---- (0) chunk from registers into LDS, per-chunk log-gate; next chunk's loads
#pragma unroll
    for (int v = 0; v < KV; ++v) {
      const int seg = tid + v * NT, row = seg / KROW, c = (seg % KROW) * EPV;
      *reinterpret_cast<u32x4*>(sK + row * LDK + c) = pk[v];
      *reinterpret_cast<u32x4*>(sQ + row * LDK + c) = pq[v];
      if constexpr (GATE == GATE_CHANNEL) {
#pragma unroll
        for (int j = 0; j < EPV; ++j) {
          const uint32_t w = pl[v][j * ESZ / 4];
          sG[row * DK + c + j] = to_f32(ESZ == 2 ? (w >> (16 * (j & 1))) & 0xffffu : w);
        }
      }
    }
#pragma unroll
    for (int v = 0; v < VV; ++v) {
      const int seg = tid + v * NT, row = seg / VROW, c = (seg % VROW) * EPV;
      *reinterpret_cast<u32x4*>(sV + row * LVT + c) = pv[v];
    }
    if constexpr (RAW) {
      if (wave == 0) {              // inclusive scan of the log-gate over the chunk rows
        float g = 0.f, gread = 0.f;
        if constexpr (GATE == GATE_SCALAR) {
          g = pls;
#pragma unroll
          for (int off = 1; off < 64; off <<= 1) {
            const float y = __shfl_up(g, off);
            if (lane >= off) g += y;
          }
          const float gprev = __shfl_up(g, 1);
          gread = p.literal ? (lane == 0 ? 0.f : gprev) : g;
        }
        const float gC = __shfl(g, 63);
        sBr[lane] = pb;
        sGr[lane] = g;
        sGrd[lane] = gread;
        sEw[lane] = pb * __expf(gread);
        sEo[lane] = __expf(g);
        sEd[lane] = __expf(gC - g);
        if (lane == 0) sGamR[0] = __expf(gC);
      }
    } else {
      if (tid < CH) sBc[tid] = pb;
    }
    if (n + 1 < nchunks) prefetch(n + 1);
    __syncthreads();

    if constexpr (!RAW) {
      // per-channel scan over the rows of each channel
      constexpr int NSEG = L::NSEG, SEGL = CH / NSEG;
      if (tid < NSEG * DK) {
        const int i = tid % DK, seg = tid / DK;
        float acc = 0.f;
#pragma unroll 8
        for (int r = seg * SEGL; r < (seg + 1) * SEGL; ++r) {
          acc += sG[r * DK + i];
          sG[r * DK + i] = acc;
        }
        sTot[seg * DK + i] = acc;
      }
      if constexpr (NSEG > 1) {
        __syncthreads();
        if (tid < NSEG * DK) {
          const int i = tid % DK, seg = tid / DK;
          float pre = 0.f;
          for (int s2 = 0; s2 < seg; ++s2) pre += sTot[s2 * DK + i];
          if (seg > 0)
            for (int r = seg * SEGL; r < (seg + 1) * SEGL; ++r) sG[r * DK + i] += pre;
        }
      }
      __syncthreads();
      // decayed operands; X_K and X_Q overwrite the raw tiles in place
      for (int i = tid; i < DK; i += NT) {
        sGamC[i] = __expf(sG[(CH - 1) * DK + i]);
#pragma unroll
        for (int R = 1; R < 4; ++R)
#pragma unroll
          for (int J = 0; J < R; ++J)
            sM[strict_pair(R, J) * DK + i] = __expf(sG[16 * R * DK + i] - sG[16 * J * DK + i]);
      }
      for (int task = tid; task < CH * (DK / 4); task += NT) {
        const int r = task / (DK / 4), i0 = (task % (DK / 4)) * 4, R = r >> 4;
        const f32x4 kk = O::f32(O::ld(sK + r * LDK + i0));
        const f32x4 qq = O::f32(O::ld(sQ + r * LDK + i0));
        const float be = sBeta[r];
        f32x4 xk, y, xq, qh, kr, kd;
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          const int i = i0 + j;
          const float g = sG[r * DK + i], gR = sG[16 * R * DK + i], gC = sG[(CH - 1) * DK + i];
          const float gread = p.literal ? (r > 0 ? sG[(r - 1) * DK + i] : 0.f) : g;
          xk[j] = be * kk[j] * __expf(gread - gR);
          y[j] = kk[j] * __expf(gR - g);
          xq[j] = qq[j] * __expf(g - gR);
          qh[j] = qq[j] * __expf(g);
          kr[j] = be * kk[j] * __expf(gread);
          kd[j] = kk[j] * __expf(gC - g);
        }
        *reinterpret_cast<frag*>(sK + r * LDK + i0) = O::cvt(xk);
        *reinterpret_cast<frag*>(sY + r * LDK + i0) = O::cvt(y);
        *reinterpret_cast<frag*>(sQ + r * LDK + i0) = O::cvt(xq);
        *reinterpret_cast<frag*>(sQh + r * LDK + i0) = O::cvt(qh);
        *reinterpret_cast<frag*>(sKr + r * LDK + i0) = O::cvt(kr);
        *reinterpret_cast<frag*>(sKd + r * LDK + i0) = O::cvt(kd);
      }
      __syncthreads();
    }

    // ---- (2) 16x16 blocks of A (strictly lower) and P (lower incl. diagonal) ------
    // Each wave forms the diagonal blocks of A it owns and inverts them in
    // registers; the 16 off-diagonal A blocks and P blocks are split evenly.
    auto block_product = [&](auto is_p, int R, int J) -> f32x4 {
      constexpr bool isP = decltype(is_p)::value;
      const T* rows = isP ? sQ : sK;
      const T* cols = RAW ? sK : sY;
      f32x4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int kb = 0; kb < DK / 32; ++kb) {
        const int c = 32 * kb + 4 * lg;
        frag a0 = O::ld(rows + (16 * R + lr) * LDK + c);
        frag a1 = O::ld(rows + (16 * R + lr) * LDK + c + 16);
        frag b0 = O::ld(cols + (16 * J + lr) * LDK + c);
        frag b1 = O::ld(cols + (16 * J + lr) * LDK + c + 16);
        if constexpr (GATE == GATE_CHANNEL) {
          if (R > J) {
            const float* m = sM + strict_pair(R, J) * DK + c;
            b0 = O::cvt(O::f32(b0) * *reinterpret_cast<const f32x4*>(m));
            b1 = O::cvt(O::f32(b1) * *reinterpret_cast<const f32x4*>(m + 16));
          }
        }
        acc = O::mma2(acc, a0, a1, b0, b1);
      }
      // decay and beta factors, then the causal mask
      const int j = 16 * J + lr;
#pragma unroll
      for (int s = 0; s < 4; ++s) {
        const int rr = 4 * lg + s, r = 16 * R + rr;
        float val = acc[s];
        if constexpr (GATE == GATE_SCALAR) val *= __expf((isP ? sGr[r] : sGrd[r]) - sGr[j]);
        if constexpr (RAW) {
          if (!isP) val *= sBr[r];
        }
        acc[s] = (R == J && (isP ? rr < lr : rr <= lr)) ? 0.f : val;
      }
      return acc;
    };
    for (int R = wave; R < 4; R += NW) {
      const f32x4 x = unit_lower_inverse(block_product(std::false_type{}, R, R), sScr + wave * 16 * L::LSC, lr, lg);
#pragma unroll
      for (int s = 0; s < 4; ++s) sXi[(16 * R + 4 * lg + s) * LXI + lr] = O::from(x[s]);
    }
    {
      // tasks [lo, hi) of the list: 6 strictly-lower A blocks, then 10 P blocks
      const int lo = 16 * wave / NW, hi = 16 * (wave + 1) / NW;
      for (int t = lo; t < (hi < 6 ? hi : 6); ++t) {
        const int R = 1 + (t >= 1) + (t >= 3), J = t - R * (R - 1) / 2;
        const f32x4 acc = block_product(std::false_type{}, R, J);
#pragma unroll
        for (int s = 0; s < 4; ++s) sA[(16 * R + 4 * lg + s) * LCH + 16 * J + lr] = O::from(-acc[s]);
      }
      for (int t = (lo > 6 ? lo : 6); t < hi; ++t) {
        const int u = t - 6;
        const int R = (u >= 1) + (u >= 3) + (u >= 6), J = u - R * (R + 1) / 2;
        const f32x4 acc = block_product(std::true_type{}, R, J);
#pragma unroll
        for (int s = 0; s < 4; ++s) sP[(16 * R + 4 * lg + s) * LCH + 16 * J + lr] = O::from(acc[s]);
      }
    }
    __syncthreads();

    // ---- (3) W and U by block forward substitution (per wave, own columns) --------
    // out_R = X_RR (rhs_R - sum_{J<R} A_RJ out_J); the CBW channel blocks of W and
    // the wave's block of U advance together.
    constexpr int NB = CBW + 1;
    f32x4 outf[NB][4];
    frag outb[NB][4];
    const T* wsrc = RAW ? sK : sKr;
#pragma unroll
    for (int R = 0; R < 4; ++R) {
      frag aR[3];
#pragma unroll
      for (int J = 0; J < R; ++J) aR[J] = O::ld(sA + (16 * R + lr) * LCH + 16 * J + 4 * lg);
      const frag xi = O::ld(sXi + (16 * R + lr) * LXI + 4 * lg);
#pragma unroll
      for (int c = 0; c < NB; ++c) {
        f32x4 acc;
        if (c < CBW) {
          acc = O::f32(O::ld_tr(wsrc, LDK, 16 * R, (wave * CBW + c) * 16, lr, lg));
          if constexpr (RAW) {
#pragma unroll
            for (int s = 0; s < 4; ++s) acc[s] *= sEw[16 * R + 4 * lg + s];
          }
        } else {
          acc = O::f32(O::ld_tr(sV, LVT, 16 * R, 16 * wave, lr, lg));
#pragma unroll
          for (int s = 0; s < 4; ++s) acc[s] *= sBeta[16 * R + 4 * lg + s];
        }
        int J = 0;
#pragma unroll
        for (; J + 1 < R; J += 2) acc = O::mma2(acc, aR[J], aR[J + 1], outb[c][J], outb[c][J + 1]);
        if (J < R) acc = O::mma1(acc, aR[J], outb[c][J]);
        f32x4 z = {0.f, 0.f, 0.f, 0.f};
        z = O::mma1(z, xi, O::cvt(acc));
        outf[c][R] = z;
        outb[c][R] = O::cvt(z);
      }
    }
#pragma unroll
    for (int c = 0; c < CBW; ++c) {
      const int ch = (wave * CBW + c) * 16 + lr;
#pragma unroll
      for (int R = 0; R < 4; ++R)
#pragma unroll
        for (int s = 0; s < 4; ++s) sW[(16 * R + 4 * lg + s) * LDK + ch] = O::from(outf[c][R][s]);
    }
    __syncthreads();

    // ---- (4) state pass and output for this wave's 16 columns ---------------------
    frag Sb[DKT];
#pragma unroll
    for (int t = 0; t < DKT; ++t) Sb[t] = O::cvt(S[t]);
    frag Db[4], Ds[4];
#pragma unroll
    for (int R = 0; R < 4; ++R) {            // Delta = U - W S
      f32x4 ws = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int kb = 0; kb < DK / 32; ++kb) {
        const T* wr = sW + (16 * R + lr) * LDK + 32 * kb + 4 * lg;
        ws = O::mma2(ws, O::ld(wr), O::ld(wr + 16), Sb[2 * kb], Sb[2 * kb + 1]);
      }
      const f32x4 d = outf[CBW][R] - ws;
      Db[R] = O::cvt(d);
      if constexpr (GATE == GATE_SCALAR) {
        f32x4 ds;
#pragma unroll
        for (int s = 0; s < 4; ++s) ds[s] = d[s] * sEd[16 * R + 4 * lg + s];
        Ds[R] = O::cvt(ds);
      } else {
        Ds[R] = Db[R];
      }
    }
    // O^T tile (rows = this wave's 16 columns, columns = 16 tokens):
    //   S^T (Q e^g)^T + Delta^T P^T; a lane ends up with 4 adjacent output columns.
    const T* qsrc = RAW ? sQ : sQh;
    const uint32_t so = static_cast<uint32_t>(t0 * H * dv * ESZ);
#pragma unroll
    for (int R = 0; R < 4; ++R) {
      f32x4 oq = {0.f, 0.f, 0.f, 0.f}, op = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int kb = 0; kb < DK / 32; ++kb) {
        const T* qr = qsrc + (16 * R + lr) * LDK + 32 * kb + 4 * lg;
        oq = O::mma2(oq, Sb[2 * kb], Sb[2 * kb + 1], O::ld(qr), O::ld(qr + 16));
      }
      const T* pr = sP + (16 * R + lr) * LCH + 4 * lg;
      int J = 0;
#pragma unroll
      for (; J + 1 <= R; J += 2) op = O::mma2(op, Db[J], Db[J + 1], O::ld(pr + 16 * J), O::ld(pr + 16 * (J + 1)));
      if (J <= R) op = O::mma1(op, Db[J], O::ld(pr + 16 * J));
      const int r = 16 * R + lr;
      f32x4 ov;
      if constexpr (GATE == GATE_SCALAR) ov = oq * sEo[r] + op; else ov = oq + op;
      // rows past the end of the sequence fall outside the buffer and are dropped
      const uint32_t voff = static_cast<uint32_t>((r * H * dv + col0 + 16 * wave + 4 * lg) * ESZ);
      if constexpr (IO == IO_BF16) {
        u32x2 w;
        w[0] = uint32_t(f32_to_bf16_bits(ov[0])) | (uint32_t(f32_to_bf16_bits(ov[1])) << 16);
        w[1] = uint32_t(f32_to_bf16_bits(ov[2])) | (uint32_t(f32_to_bf16_bits(ov[3])) << 16);
        buf_store8(w, ro, voff, so);
      } else {
        u32x4 w;
#pragma unroll
        for (int s = 0; s < 4; ++s) w[s] = __float_as_uint(ov[s]);
        buf_store16(w, ro, voff, so);
      }
    }
    // S' = diag(e^{g_63}) S + (K e^{g_63 - g})^T Delta
    const T* kdsrc = RAW ? sK : sKd;
#pragma unroll
    for (int t = 0; t < DKT; ++t) {
      f32x4 acc = S[t];
      if constexpr (GATE == GATE_CHANNEL) {
#pragma unroll
        for (int s = 0; s < 4; ++s) acc[s] *= sGamC[16 * t + 4 * lg + s];
      } else if constexpr (GATE == GATE_SCALAR) {
        acc = acc * sGamR[0];
      }
      acc = O::mma2(acc, O::ld_tr(kdsrc, LDK, 0, 16 * t, lr, lg), O::ld_tr(kdsrc, LDK, 16, 16 * t, lr, lg),
                    Ds[0], Ds[1]);
      acc = O::mma2(acc, O::ld_tr(kdsrc, LDK, 32, 16 * t, lr, lg), O::ld_tr(kdsrc, LDK, 48, 16 * t, lr, lg),
                    Ds[2], Ds[3]);
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
  if constexpr (IO == IO_F32 || GATE == GATE_CHANNEL) {
    return launch_chunk_t<IO, GATE, DK, 2>(p, stream);   // LDS budget: 32-column tiles
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
