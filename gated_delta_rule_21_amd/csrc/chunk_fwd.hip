// Chunkwise-parallel forward of the gated delta rule on gfx950: the sequential
// state pass and the output, given each chunk's T = (I + A)^{-1}, masked score
// matrix P and per-row gate factors from the per-chunk transform (chunk_prep.hip).
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
// S the state entering the chunk, T = (I + A)^{-1} and P from the per-chunk transform):
//   Delta = T diag(beta) (V - (K*e^{g_read}) S)
//           (= U - W S for the correction terms W = T diag(beta) K e^{g_read} and
//            U = T diag(beta) V of §3; applying T to the residual needs only the
//            64x64 T per chunk instead of W and U)
//   O     = (Q*e^{g}) S + P Delta,   P = lower_incl( (Q*e^{g}) (K*e^{-g})^T )
//   S'    = diag(e^{g_63}) S + (K*e^{g_63 - g})^T Delta
// g_read = g (decay before the erase) or g_{r-1} (erase reads the undecayed
// state); the query/key decay factors are those derived from the §2 update.
//
// Work decomposition.  One workgroup of NW waves owns one (batch, head, d_v tile
// of 16*NW columns) and walks the chunks in order.  Wave w owns 16 state
// columns: its slice of S (d_k x 16, fp32) lives in MFMA accumulators for the
// whole sequence.  An accumulator tile (lane l: column l%16, rows 4(l/16)+s) is
// the operand layout of the next product, so K S, the residual, T times it, the
// output and the state update chain through registers.
//
// Memory.  q, k, v and the chunk's workspace record (T, P, gate factors) are
// read once per chunk with buffer loads into registers one chunk ahead of
// their use (a per-channel gate also reads beta and log a); a buffer's range
// ends at the last token of the sequence, so the rows of a ragged last chunk read
// as zero and their stores are dropped.  Tiles sit row-major in LDS; products
// that contract over the chunk rows (the state update) read them with the gfx950
// LDS transpose load.  The output is computed transposed, so each lane stores
// four adjacent columns.
//
// Gates.  With no gate or a scalar gate the decay factors are per row, so the
// products run on the raw q, k tiles and the factors are applied to the rows
// of the results.  A per-channel gate sits inside the d_k contraction: the
// chunk's gate is scanned down each channel here and the decayed operands
// k e^{g_read}, q e^{g} and k e^{g_63 - g} are built before the products.
//
// Products run on bf16 MFMA with fp32 accumulation for bf16 I/O and on fp32
// MFMA for fp32 I/O; the state stays fp32.
#include <mutex>
#include <type_traits>

#include "chunk_common.h"
#include "launchers.h"

namespace gdr {

// LDS layout (bytes).  Row-major tiles: [64][DK] with stride LDK, the v tile
// [64][DVT] with stride LVT, the 64x64 matrices with stride LCH.
template <int IO, int GATE, int DK, int NW>
struct Layout {
  typedef typename Op<IO>::T T;
  static constexpr bool RAW = GATE != GATE_CHANNEL;   // products on raw q, k
  static constexpr int PAD = Op<IO>::PAD;
  static constexpr int LDK = DK + PAD;
  static constexpr int LCH = CH + PAD;
  static constexpr int DVT = 16 * NW;
  static constexpr int LVT = DVT + PAD;
  static constexpr int NSEG = (64 * NW) / DK > 0 ? (64 * NW) / DK : 1;
  static constexpr size_t RM = size_t(CH) * LDK * sizeof(T);      // [64][DK]
  static constexpr size_t MM = size_t(CH) * LCH * sizeof(T);      // [64][64]
  static constexpr size_t V_B = size_t(CH) * LVT * sizeof(T);
  static constexpr size_t OFF_K = 0;                     // raw k (per-channel: k e^{g_read})
  static constexpr size_t OFF_Q = OFF_K + RM;            // raw q (per-channel: q e^{g})
  static constexpr size_t OFF_V = OFF_Q + RM;            // raw v tile
  static constexpr size_t OFF_T = OFF_V + V_B;           // T^T, T = (I + A)^{-1}
  static constexpr size_t OFF_P = OFF_T + MM;            // P
  static constexpr size_t OFF_F = OFF_P + MM;            // beta, e^{g_read}, e^{g}, e^{g_63 - g}, e^{g_63}, g
  static constexpr size_t OFF_X = OFF_F + 6 * CH * 4;    // per-channel regions start here
  // no gate / scalar gate: the regions above, twice when that fits (chunk n is
  // read from one copy while chunk n+1 is written to the other)
  static constexpr int NB = (RAW && 2 * OFF_X <= 163840) ? 2 : 1;
  static constexpr size_t R_TOTAL = NB * OFF_X;
  // per-channel gate
  static constexpr size_t C_KD = OFF_X;                  // k e^{g_63 - g}
  static constexpr size_t C_G = C_KD + RM;               // g [64][DK] fp32
  static constexpr size_t C_GAM = C_G + size_t(CH) * DK * 4;
  static constexpr size_t C_TOT = C_GAM + DK * 4;
  static constexpr size_t C_TOTAL = C_TOT + NSEG * DK * 4;
  static constexpr size_t TOTAL = RAW ? R_TOTAL : C_TOTAL;
};

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
  constexpr int LDK = L::LDK, LCH = L::LCH, LVT = L::LVT;
  constexpr int ESZ = int(sizeof(elem));
  typedef WsRec<ESZ> W;
  constexpr int EPV = 16 / ESZ;          // elements per 16-byte load
  constexpr int KROW = DK / EPV, VROW = DVT / EPV;
  constexpr int KV = CH * KROW / NT;     // 16-byte pieces of a k (q) tile per thread
  constexpr int VV = CH * VROW / NT;     // 16-byte pieces of the v tile per thread
  constexpr int PPB = W::BLK * ESZ / 16; // 16-byte pieces per record block
  constexpr int PPR = PPB / 16;          // ... per block row
  constexpr int TV = (10 * PPB + NT - 1) / NT;   // pieces of the T (P) blocks per thread
  constexpr int FV = W::NF * CH * 4 / 16;        // pieces of the factor rows (threads 0..FV-1)
  static_assert(KV * NT == CH * KROW && VV * NT == CH * VROW && VV >= 1 && FV <= NT,
                "tile loads must split evenly");
  static_assert(L::TOTAL <= 163840, "LDS budget");

  constexpr int NB = L::NB;
  __shared__ __attribute__((aligned(16))) char smem[L::TOTAL];
  // per-channel regions
  T* sKd = reinterpret_cast<T*>(smem + L::C_KD);
  float* sG = reinterpret_cast<float*>(smem + L::C_G);
  float* sGamC = reinterpret_cast<float*>(smem + L::C_GAM);
  float* sTot = reinterpret_cast<float*>(smem + L::C_TOT);

  // Block -> (head, d_v tile).  Consecutive logical blocks land on one XCD (the
  // hardware deals block ids round-robin over 8 XCDs), so the tiles of one head
  // share that XCD's L2 for their common q, k and workspace reads.
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
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);   // uniform across the wave
  const int lane = tid & 63;
  const int lr = lane & 15;
  const int lg = lane >> 4;
  const int scol = col0 + 16 * wave + lr;   // this lane's state column

  // This sequence's tokens (a packed sequence's from the offset table) and records.
  const SeqSpan sq = seq_span(p, bb, hh);
  const int64_t nchunks = (sq.len + CH - 1) / CH;
  // Buffers over this sequence's (b, h) slice; each range ends after the last token.
  const int64_t row0 = sq.t0 * p.H + hh;               // token-row index of (b, t = 0, h)
  const uint32_t span = static_cast<uint32_t>(sq.len > 0 ? (sq.len - 1) * p.H + 1 : 0);   // rows in range
  const rsrc_t rk = make_rsrc(static_cast<const elem*>(p.k) + row0 * DK, span * DK * ESZ);
  const rsrc_t rq = make_rsrc(static_cast<const elem*>(p.q) + row0 * DK, span * DK * ESZ);
  const rsrc_t rv = make_rsrc(static_cast<const elem*>(p.v) + row0 * dv, span * dv * ESZ);
  const rsrc_t ro = make_rsrc(static_cast<const elem*>(p.o) + row0 * dv, span * dv * ESZ);
  const rsrc_t rb = make_rsrc(static_cast<const elem*>(p.beta) + row0, span * ESZ);
  const rsrc_t rl = make_rsrc(static_cast<const elem*>(p.log_a) + row0 * (GATE == GATE_CHANNEL ? DK : 1),
                              GATE == GATE_NONE ? 0u : span * (GATE == GATE_CHANNEL ? DK : 1) * ESZ);
  const rsrc_t rw = make_rsrc(static_cast<const char*>(p.ws) + sq.rec0 * W::BYTES,
                              static_cast<uint32_t>(nchunks * W::BYTES));
  static_assert(IO == IO_F32, "bf16 I/O runs the chain/helper kernel (chunk_state.hip)");
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
  u32x4 pk[KV], pq[KV], pl[GATE == GATE_CHANNEL ? KV : 1], pv[VV], pt[TV], pp[TV], pf;
  float pb = 0.f;
  auto to_f32 = [&](uint32_t bits) -> float {
    if constexpr (IO == IO_BF16) return bf16_bits_to_f32(static_cast<uint16_t>(bits));
    else return __uint_as_float(bits);
  };
  auto prefetch = [&](int64_t m) __attribute__((always_inline)) {
    const uint32_t sk = static_cast<uint32_t>(m * CH * H * DK * ESZ);
    const uint32_t sv = static_cast<uint32_t>(m * CH * H * dv * ESZ);
    const uint32_t sb = static_cast<uint32_t>(m * CH * H * ESZ);
    const uint32_t sw = static_cast<uint32_t>(m * W::BYTES);
#pragma unroll
    for (int v = 0; v < KV; ++v) {
      pk[v] = buf_load16(rk, offk[v], sk);
      pq[v] = buf_load16(rq, offk[v], sk);
      if constexpr (GATE == GATE_CHANNEL) pl[v] = buf_load16(rl, offk[v], sk);
    }
#pragma unroll
    for (int v = 0; v < VV; ++v) pv[v] = buf_load16(rv, offv[v], sv);
#pragma unroll
    for (int v = 0; v < TV; ++v) {
      const int pc = tid + v * NT;
      if (pc < 10 * PPB) {
        pt[v] = buf_load16(rw, W::T_OFF + static_cast<uint32_t>(pc * 16), sw);
        pp[v] = buf_load16(rw, W::P_OFF + static_cast<uint32_t>(pc * 16), sw);
      }
    }
    if constexpr (RAW) {
      if (tid < FV) pf = buf_load16(rw, W::F_OFF + static_cast<uint32_t>(tid * 16), sw);
    } else {
      if (tid < CH) pb = to_f32(IO == IO_BF16 ? buf_load2(rb, offb, sb) : buf_load4(rb, offb, sb));
    }
  };

  // the prefetched chunk from registers into one LDS copy
  auto store_chunk = [&](char* base) __attribute__((always_inline)) {
    T* dK = reinterpret_cast<T*>(base + L::OFF_K);
    T* dQ = reinterpret_cast<T*>(base + L::OFF_Q);
    T* dV = reinterpret_cast<T*>(base + L::OFF_V);
    T* dT = reinterpret_cast<T*>(base + L::OFF_T);
    T* dP = reinterpret_cast<T*>(base + L::OFF_P);
    float* dF = reinterpret_cast<float*>(base + L::OFF_F);
#pragma unroll
    for (int v = 0; v < KV; ++v) {
      const int seg = tid + v * NT, row = seg / KROW, c = (seg % KROW) * EPV;
      *reinterpret_cast<u32x4*>(dK + row * LDK + c) = pk[v];
      *reinterpret_cast<u32x4*>(dQ + row * LDK + c) = pq[v];
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
      *reinterpret_cast<u32x4*>(dV + row * LVT + c) = pv[v];
    }
#pragma unroll
    for (int v = 0; v < TV; ++v) {
      const int pc = tid + v * NT;
      if (pc < 10 * PPB) {                 // block u holds (T_RJ)^T and P_RJ: T^T and P tiles
        int R, J;
        tri_block(pc / PPB, R, J);
        const int a = (pc % PPB) / PPR, b0 = (pc % PPR) * EPV;
        *reinterpret_cast<u32x4*>(dT + (16 * J + a) * LCH + 16 * R + b0) = pt[v];
        *reinterpret_cast<u32x4*>(dP + (16 * R + a) * LCH + 16 * J + b0) = pp[v];
      }
    }
    if constexpr (RAW) {
      if (tid < FV) *reinterpret_cast<u32x4*>(dF + 4 * tid) = pf;
    } else {
      if (tid < CH) dF[tid] = pb;
    }
  };

  if (nchunks > 0) prefetch(0);
  if constexpr (NB == 2) {
    if (nchunks > 0) {
      store_chunk(smem);
      if (nchunks > 1) prefetch(1);
    }
    __syncthreads();
  }

  for (int64_t n = 0; n < nchunks; ++n) {
    const int64_t t0 = n * CH;
    char* cur = smem + (NB == 2 ? (n & 1) * L::OFF_X : 0);
    const T* sK = reinterpret_cast<const T*>(cur + L::OFF_K);
    const T* sQ = reinterpret_cast<const T*>(cur + L::OFF_Q);
    const T* sV = reinterpret_cast<const T*>(cur + L::OFF_V);
    const T* sT = reinterpret_cast<const T*>(cur + L::OFF_T);
    const T* sP = reinterpret_cast<const T*>(cur + L::OFF_P);
    const float* sF = reinterpret_cast<const float*>(cur + L::OFF_F);
    const float* sBeta = sF;                // beta
    const float* sEr = sF + CH;             // e^{g_read}    (rows of K S)
    const float* sEo = sF + 2 * CH;         // e^{g}         (output rows)
    const float* sEd = sF + 3 * CH;         // e^{g_63 - g}  (Delta rows in the state update)
    const float* sGamR = sF + 4 * CH;       // e^{g_63}

    // ---- next chunk's tiles into LDS and the loads after it; per-channel gate -------
    if constexpr (NB == 2) {
      // the other copy was last read in the previous chunk, before its closing barrier
      if (n + 1 < nchunks) {
        store_chunk(smem + ((n + 1) & 1) * L::OFF_X);
        if (n + 2 < nchunks) prefetch(n + 2);
      }
    } else {
      store_chunk(smem);
      if (n + 1 < nchunks) prefetch(n + 1);
      __syncthreads();
    }

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
      // decayed operands; k e^{g_read} and q e^{g} overwrite the raw tiles in place
      for (int i = tid; i < DK; i += NT) sGamC[i] = __expf(sG[(CH - 1) * DK + i]);
      for (int task = tid; task < CH * (DK / 4); task += NT) {
        const int r = task / (DK / 4), i0 = (task % (DK / 4)) * 4;
        const f32x4 kk = O::f32(O::ld(sK + r * LDK + i0));
        const f32x4 qq = O::f32(O::ld(sQ + r * LDK + i0));
        f32x4 kr, qh, kd;
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          const int i = i0 + j;
          const float g = sG[r * DK + i], gC = sG[(CH - 1) * DK + i];
          const float gread = p.literal ? (r > 0 ? sG[(r - 1) * DK + i] : 0.f) : g;
          kr[j] = kk[j] * __expf(gread);
          qh[j] = qq[j] * __expf(g);
          kd[j] = kk[j] * __expf(gC - g);
        }
        *reinterpret_cast<frag*>(const_cast<T*>(sK) + r * LDK + i0) = O::cvt(kr);
        *reinterpret_cast<frag*>(const_cast<T*>(sQ) + r * LDK + i0) = O::cvt(qh);
        *reinterpret_cast<frag*>(sKd + r * LDK + i0) = O::cvt(kd);
      }
      __syncthreads();
    }

    // ---- this wave's chain: residual, Delta = T R --------------------------------------
    frag Sb[DKT];
#pragma unroll
    for (int t = 0; t < DKT; ++t) Sb[t] = O::cvt(S[t]);
    frag Rb[4];
#pragma unroll
    for (int R = 0; R < 4; ++R) {            // R = diag(beta) (V - (K e^{g_read}) S)
      f32x4 x = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int kb = 0; kb < DK / 32; ++kb) {
        const T* kr = sK + (16 * R + lr) * LDK + 32 * kb + 4 * lg;
        x = O::mma2(x, O::ld(kr), O::ld(kr + 16), Sb[2 * kb], Sb[2 * kb + 1]);
      }
      const f32x4 vv = O::f32(O::ld_tr(sV, LVT, 16 * R, 16 * wave, lr, lg));
      f32x4 rr;
#pragma unroll
      for (int s = 0; s < 4; ++s) {
        const int r = 16 * R + 4 * lg + s;
        const float xs = GATE == GATE_SCALAR ? x[s] * sEr[r] : x[s];
        rr[s] = sBeta[r] * (vv[s] - xs);
      }
      Rb[R] = O::cvt(rr);
    }
    frag Db[4], Ds[4];
#pragma unroll
    for (int R = 0; R < 4; ++R) {            // Delta_R = sum_{m <= R} T_Rm R_m; rows of T from T^T
      f32x4 d = {0.f, 0.f, 0.f, 0.f};
      int m = 0;
#pragma unroll
      for (; m + 1 <= R; m += 2)
        d = O::mma2(d, O::ld_tr(sT, LCH, 16 * m, 16 * R, lr, lg), O::ld_tr(sT, LCH, 16 * (m + 1), 16 * R, lr, lg),
                    Rb[m], Rb[m + 1]);
      if (m <= R) d = O::mma1(d, O::ld_tr(sT, LCH, 16 * m, 16 * R, lr, lg), Rb[m]);
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
    const T* qsrc = sQ;
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
        buf_store8(__builtin_bit_cast(u32x2, to_bf16x4(ov)), ro, voff, so);
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
    __syncthreads();                          // this copy of LDS is rewritten after the next chunk
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

template <int IO, int GATE>
static hipError_t launch_chunk_g(const ChunkParams& p, hipStream_t stream) {
  // fp32 I/O: two waves, 32 columns per workgroup; at d_k = 128 one LDS copy of the
  // tiles (no double buffer), and no per-channel gate (its fp32 running sums of the
  // gate and third operand tile leave no room)
  if (p.d_k == 64) return launch_chunk_t<IO, GATE, 64, 2>(p, stream);
  if constexpr (GATE != GATE_CHANNEL)
    if (p.d_k == 128) return launch_chunk_t<IO, GATE, 128, 2>(p, stream);
  return hipErrorInvalidValue;
}

static hipError_t launch_chunk_f32(const ChunkParams& p, hipStream_t stream) {
  switch (p.gate) {
    case GATE_NONE: return launch_chunk_g<IO_F32, GATE_NONE>(p, stream);
    case GATE_SCALAR: return launch_chunk_g<IO_F32, GATE_SCALAR>(p, stream);
    case GATE_CHANNEL: return launch_chunk_g<IO_F32, GATE_CHANNEL>(p, stream);
  }
  return hipErrorInvalidValue;
}

hipError_t launch_chunk_fwd(const ChunkParams& p, hipStream_t stream) {
  if (p.B * p.H == 0) return hipSuccess;
  hipError_t e = launch_chunk_prep(p, stream);
  if (e != hipSuccess) return e;
  // bf16 I/O: chain and helper waves (chunk_state.hip); fp32 I/O: this file's kernel
  if (p.io == IO_BF16) {
    if (!p.cu) return launch_chunk_state_pipe(p, stream);
    // packed sequences: the state pass takes them longest first
    ChunkParams q = p;
    int32_t* order = p.order_out ? p.order_out
                                 : reinterpret_cast<int32_t*>(static_cast<char*>(p.ws) +
                                                              chunk_varlen_records_bytes(p.T, p.B, p.H, p.io, p.gate, p.d_k));
    q.order = order;
    if ((e = launch_varlen_order(q, order, stream)) != hipSuccess) return e;
    return launch_chunk_state_pipe(q, stream);
  }
  return launch_chunk_f32(p, stream);
}

size_t chunk_workspace_bytes(int64_t B, int64_t T, int64_t H, int io, int gate, int d_k) {
  const int64_t nchunks = (T + CH - 1) / CH;
  return static_cast<size_t>(B * H * nchunks) * rec_bytes(io, gate, d_k);
}

size_t chunk_varlen_records_bytes(int64_t T, int64_t n_seq, int64_t H, int io, int gate, int d_k) {
  return static_cast<size_t>(H * chunk_varlen_slots(T, n_seq)) * rec_bytes(io, gate, d_k);
}

size_t chunk_varlen_workspace_bytes(int64_t T, int64_t n_seq, int64_t H, int io, int gate, int d_k) {
  return chunk_varlen_records_bytes(T, n_seq, H, io, gate, d_k) + static_cast<size_t>((n_seq * 4 + 15) / 16 * 16);
}

// Rank of each packed sequence by length, longest first (ties by index): thread i
// counts the sequences that go before it.  The lengths pass through LDS in tiles.
// Above VARLEN_RANK_MAX sequences the order is the identity.
constexpr int64_t VARLEN_RANK_MAX = 16384;
__device__ __forceinline__ int64_t clamped_len(const ChunkParams& p, int64_t j) {   // as in seq_span
  int64_t a = p.cu[j], e = p.cu[j + 1];
  a = a < 0 ? 0 : (a > p.T ? p.T : a);
  e = e < a ? a : (e > p.T ? p.T : e);
  return e - a;
}

__global__ __launch_bounds__(256) void varlen_order_kernel(ChunkParams p, int32_t* order) {
  __shared__ int64_t tile[256];
  const int64_t i = static_cast<int64_t>(blockIdx.x) * 256 + threadIdx.x;
  const int64_t N = p.B;
  const int64_t li = i < N ? clamped_len(p, i) : 0;
  if (N > VARLEN_RANK_MAX) {
    if (i < N) order[i] = static_cast<int32_t>(i);
    return;
  }
  int64_t rank = 0;
  for (int64_t j0 = 0; j0 < N; j0 += 256) {
    __syncthreads();
    const int64_t j = j0 + threadIdx.x;
    if (j < N) tile[threadIdx.x] = clamped_len(p, j);
    __syncthreads();
    const int64_t n = N - j0 < 256 ? N - j0 : 256;
    for (int64_t t = 0; t < n; ++t) {
      const int64_t lj = tile[t];
      rank += (lj > li || (lj == li && j0 + t < i)) ? 1 : 0;
    }
  }
  if (i < N) order[rank] = static_cast<int32_t>(i);
}

hipError_t launch_varlen_order(const ChunkParams& p, int32_t* order, hipStream_t stream) {
  const unsigned nb = static_cast<unsigned>((p.B + 255) / 256);
  hipLaunchKernelGGL(varlen_order_kernel, dim3(nb), dim3(256), 0, stream, p, order);
  return hipGetLastError();
}

// ---------------------------------------------------------------------------------
// The workspace of the forward that allocates nothing (gdr_chunk_fwd_noalloc): the
// per-chunk records in one file-scope device array, a copy of which every GPU the
// library runs on holds until the process ends.  In host code `scratch` names a
// host-side stand-in, never the device memory: the device address of each GPU's
// copy is looked up once per device (with that device current) and kept here.
// ---------------------------------------------------------------------------------
static __device__ __align__(256) char scratch[STATIC_SCRATCH_BYTES];

hipError_t static_scratch(void** ptr) {
  constexpr int MAX_DEV = 64;
  static std::mutex mu;
  static void* addr[MAX_DEV] = {};
  int dev = -1;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  if (dev < 0 || dev >= MAX_DEV) return hipErrorInvalidDevice;
  std::lock_guard<std::mutex> lock(mu);
  if (!addr[dev]) {
    void* p = nullptr;
    e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess) return e;
    addr[dev] = p;
  }
  *ptr = addr[dev];
  return hipSuccess;
}

}  // namespace gdr
