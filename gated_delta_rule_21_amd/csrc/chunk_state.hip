// State pass of the chunkwise gated delta rule on gfx950 for bf16 I/O without a
// per-channel gate: chain waves and helper waves working side by side.
//
// "Moonshot AI's New Attention Architecture: Key Innovations Explained", §3
// Hardware-Friendly Algorithm: between chunks only the d_k x d_v state is
// passed on, and within a chunk the rest is dense lower-triangular products.
// Per chunk (rows r = 0..63, g_r = inclusive running sum of log a over the
// chunk, S the state entering it, T = (I + A)^{-1} from the per-chunk
// transform; scalar gate, so the decay factors are per row):
//   Delta = T diag(beta) (V - diag(e^{g_read}) K S)
//   O     = diag(e^{g}) Q S + P Delta,   P = lower_incl( e^{g_r - g_j} q_r . k_j )
//   S'    = e^{g_63} S + K^T diag(e^{g_63 - g}) Delta
//
// Only K S -> Delta -> S' lies on the sequential chain from chunk to chunk.
// One workgroup owns one (batch, head, d_v tile of 16*CG*NCH columns) and runs
// NCH chain waves and NHW helper waves, with one barrier per chunk:
//   chain wave c  (c < NCH) keeps CG groups of 16 columns of S in MFMA
//                 accumulators; every operand fragment it reads from LDS (rows
//                 of k, q, T, K^T and P) serves all its groups.  In the step of
//                 chunk n it first finishes the output of chunk n-1 (Q S and
//                 Delta of that chunk kept in registers, plus P of that chunk),
//                 then forms K S, Q S, the residual, Delta and the state update
//                 of chunk n;
//   helper wave h forms the rows of P of chunk n in row blocks h, h + NHW, ..,
//                 then moves chunk n+1 from registers into the other LDS copy and
//                 loads chunk n+2 (P first: it needs no memory, while the stores
//                 wait for loads issued a step earlier).
// The output of a chunk is written one step late, which is what lets P be
// formed beside the chain without a second barrier.  The tiles (k, q, v, T,
// per-row factors) and P are double-buffered in LDS.
//
// Operand layouts as elsewhere in this library: an accumulator tile (lane l:
// column l%16, rows 4(l/16)+s) is the B operand of the next product and, as the
// A operand, stands for its transpose; rows of T are read from T^T with the
// LDS transpose load; the output is formed transposed so each lane stores four
// adjacent columns.
#include <type_traits>

#include "chunk_common.h"
#include "launchers.h"

namespace gdr {

// LDS row strides (bf16 elements), measured on gfx950 at 8 waves per CU: reads
// of 8-byte row fragments (lane l: row l%16) run fastest (~121 B/clk) when a row
// is 2 or 6 (mod 8) dwords long, transpose reads (ds_read_b64_tr_b16) at 168 B/clk
// when it is 8 (mod 32) dwords and at 128 B/clk for most other lengths; the k
// tile is read both ways and takes 6 (mod 32) dwords (121 and 128 B/clk).
template <int DK, int DVT_, bool CHAN, bool KROW>
struct PipeLayout {
  static constexpr int LDK = DK + 12;                    // k: row and transpose reads (8-byte aligned rows)
  // With a write key, k is read by rows only (the transposed reads take the write
  // key): the measured row-read stride for k, and a tighter one for the write key,
  // bring 64 columns within the 160 KB of LDS.
  static constexpr int LDKK = KROW ? DK + 4 : LDK;       // stride of the k tile
  static constexpr int LDKD = KROW ? DK + 8 : LDK;       // stride of the third tile
  static constexpr int LDQ = DK + 4;                     // q: row reads (8-byte aligned rows)
  static constexpr int DVT = DVT_;
  static constexpr int LVT = DVT + 16;                   // v: transpose reads
  static constexpr int LCT = CH + 16;                    // T^T: transpose reads
  static constexpr int LCP = CH + 4;                     // P: row reads
  static constexpr size_t KB = size_t(CH) * LDKK * 2;
  static constexpr size_t KDB = size_t(CH) * LDKD * 2;
  static constexpr size_t QB = size_t(CH) * LDQ * 2;
  static constexpr size_t VB = size_t(CH) * LVT * 2;
  static constexpr size_t TB = size_t(CH) * LCT * 2;
  // one copy of a chunk's tiles
  static constexpr size_t B_K = 0;
  static constexpr size_t B_Q = B_K + KB;
  static constexpr size_t B_V = B_Q + QB;
  static constexpr size_t B_T = B_V + VB;                // T^T (the ten blocks on or above the diagonal)
  static constexpr size_t B_F = B_T + TB;                // factor rows of the workspace record
  static constexpr size_t B_KD = B_F + 6 * CH * 4;       // per-channel gate: k e^{g_63 - g} (transpose reads)
  static constexpr size_t BUF = B_KD + (CHAN ? KDB : 0);
  // P of chunk n in copy n % 2
  static constexpr size_t PB = size_t(CH) * LCP * 2;
  static constexpr size_t OFF_P = 2 * BUF;
  static constexpr size_t TOTAL = OFF_P + 2 * PB;
};

// SAVE: the training forward, which also stores the state entering every chunk
// (p.states); a kernel of its own, so the inference forward carries none of it.
template <int GATE, int DK, int NCH, int CG, int NHW, bool SAVE>
__global__ __launch_bounds__((NCH + NHW) * 64) void chunk_state_pipe_kernel(ChunkParams p, int n_tiles) {
  typedef Op<IO_BF16> O;
  typedef __bf16 T;
  typedef bf16x4 frag;
  typedef uint16_t elem;
  constexpr int DVT = 16 * CG * NCH;            // columns per workgroup
  constexpr bool CHAN = GATE == GATE_CHANNEL;
  constexpr bool WK = gate_wkey(GATE);            // write key: K^T and P take kw instead of k
  typedef PipeLayout<DK, DVT, CHAN || WK, WK> L;
  typedef WsRec<2> W;
  constexpr uint32_t RB = rec_bytes(IO_BF16, GATE, DK);   // bytes per chunk record
  constexpr int ESZ = 2, EPV = 8;
  constexpr int NH = NHW * 64;                   // helper threads
  constexpr int DKT = DK / 16;
  constexpr int LDKK = L::LDKK, LDKD = L::LDKD, LDQ = L::LDQ, LVT = L::LVT, LCT = L::LCT, LCP = L::LCP;
  constexpr int KROW = DK / EPV, VROW = DVT / EPV;
  constexpr int NKP = CH * KROW, NVP = CH * VROW; // 16-byte pieces of the k (q) tile, of the v tile
  constexpr int HK = (NKP + NH - 1) / NH;        // ... per helper thread (the last round guarded
  constexpr int HV = (NVP + NH - 1) / NH;        //     when the helpers do not divide them)
  constexpr int PPB = W::BLK * ESZ / 16, PPR = PPB / 16;
  constexpr int HT = (10 * PPB + NH - 1) / NH;   // ... of the T blocks
  constexpr int NFP = W::NF * CH * 4 / 16;       // pieces of the factor rows (helper threads 0..NFP-1)
  static_assert(NFP <= NH, "factor rows: one piece per helper thread");
  static_assert(L::TOTAL <= 163840, "LDS budget");

  __shared__ __attribute__((aligned(16))) char smem[L::TOTAL];
  auto p_tile = [&](int64_t n) __attribute__((always_inline)) {
    return reinterpret_cast<T*>(smem + L::OFF_P + (n & 1) * L::PB);
  };

  // Block -> (sequence, head, d_v tile).  Block ids are dealt round-robin over the
  // 8 XCDs and each XCD runs its share in order.  Fixed-length batches: consecutive
  // logical blocks on one XCD, so a head's tiles share that L2.  Packed sequences:
  // (sequence, head) items longest sequence first, item i on XCD i % 8 with its
  // tiles side by side there, so the longest chains start first everywhere.
  const int nblk = gridDim.x;
  int64_t bh;
  int tile;
  if (p.order && (p.B * p.H) % 8 == 0) {
    const int xcd = blockIdx.x & 7, pos = blockIdx.x >> 3;
    const int64_t item = static_cast<int64_t>(pos / n_tiles) * 8 + xcd;
    tile = pos % n_tiles;
    bh = static_cast<int64_t>(p.order[item / p.H]) * p.H + item % p.H;
  } else if (p.order) {
    const int64_t item = blockIdx.x / n_tiles;
    tile = blockIdx.x % n_tiles;
    bh = static_cast<int64_t>(p.order[item / p.H]) * p.H + item % p.H;
  } else {
    int lb = blockIdx.x;
    if ((nblk & 7) == 0) lb = (blockIdx.x & 7) * (nblk >> 3) + (blockIdx.x >> 3);
    bh = lb / n_tiles;
    tile = lb % n_tiles;
  }
  bh = uni64(bh);
  const int64_t bb = bh / p.H, hh = bh % p.H;
  const int dv = p.d_v;
  const int col0 = tile * DVT;
  const int H = static_cast<int>(p.H);

  const int tid = threadIdx.x;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);   // uniform across the wave
  const bool chain = wave < NCH;
  const int cw = chain ? wave : wave - NCH;      // chain: its columns 16 CG cw ..; helper: its index
  const int lane = tid & 63;
  const int lr = lane & 15;
  const int lg = lane >> 4;
  const int ht = tid - 64 * NCH;                 // helper thread index

  // this sequence's tokens (a packed sequence's come from the offset table)
  const SeqSpan sq = seq_span(p, bb, hh);
  const int64_t nchunks = (sq.len + CH - 1) / CH;
  const int64_t row0 = sq.t0 * p.H + hh;
  const uint32_t span = static_cast<uint32_t>(sq.len > 0 ? (sq.len - 1) * p.H + 1 : 0);
  const rsrc_t rk = make_rsrc(static_cast<const elem*>(p.k) + row0 * DK, span * DK * ESZ);
  const rsrc_t rq = make_rsrc(static_cast<const elem*>(p.q) + row0 * DK, span * DK * ESZ);
  const rsrc_t rkw = make_rsrc(static_cast<const elem*>(WK ? p.kw : p.k) + row0 * DK, span * DK * ESZ);
  const rsrc_t rv = make_rsrc(static_cast<const elem*>(p.v) + row0 * dv, span * dv * ESZ);
  const rsrc_t ro = make_rsrc(static_cast<const elem*>(p.o) + row0 * dv, span * dv * ESZ);
  const rsrc_t rw = make_rsrc(static_cast<const char*>(p.ws) + sq.rec0 * RB, static_cast<uint32_t>(nchunks * RB));

  // ---- helpers: loads one chunk ahead in registers, stores into an LDS copy ----------
  // Per-channel gate: k, q and k e^{g_63 - g} come decayed from the record (row-major
  // [64][d_k] each), and so does P, which is loaded a step after the tiles.
  u32x4 pk[HK], pq[HK], pkd[(CHAN || WK) ? HK : 1], pv[HV], pt[HT], pp[CHAN ? HT : 1], pf;
  auto prefetch = [&](int64_t m) __attribute__((always_inline)) {
    const uint32_t sk = static_cast<uint32_t>(m * CH * H * DK * ESZ);
    const uint32_t sv = static_cast<uint32_t>(m * CH * H * dv * ESZ);
    const uint32_t sw = static_cast<uint32_t>(m * RB);
#pragma unroll
    for (int v = 0; v < HK; ++v) {
      const int seg = ht + v * NH;
      if (NKP % NH != 0 && seg >= NKP) break;
      if constexpr (CHAN) {
        const uint32_t off = W::X_OFF + static_cast<uint32_t>(((seg / KROW) * DK + (seg % KROW) * EPV) * ESZ);
        pk[v] = buf_load16(rw, off, sw);
        pq[v] = buf_load16(rw, off + CH * DK * ESZ, sw);
        pkd[v] = buf_load16(rw, off + 2 * CH * DK * ESZ, sw);
      } else {
        const uint32_t off = static_cast<uint32_t>(((seg / KROW) * H * DK + (seg % KROW) * EPV) * ESZ);
        pk[v] = buf_load16(rk, off, sk);
        pq[v] = buf_load16(rq, off, sk);
        if constexpr (WK) pkd[v] = buf_load16(rkw, off, sk);
      }
    }
#pragma unroll
    for (int v = 0; v < HV; ++v) {
      const int seg = ht + v * NH;
      if (NVP % NH != 0 && seg >= NVP) break;
      pv[v] = buf_load16(rv, static_cast<uint32_t>(((seg / VROW) * H * dv + col0 + (seg % VROW) * EPV) * ESZ), sv);
    }
#pragma unroll
    for (int v = 0; v < HT; ++v) {
      const int pc = ht + v * NH;
      if (pc < 10 * PPB) pt[v] = buf_load16(rw, W::T_OFF + static_cast<uint32_t>(pc * 16), sw);
    }
    if (ht < NFP) pf = buf_load16(rw, W::F_OFF + static_cast<uint32_t>(ht * 16), sw);
  };
  auto prefetch_p = [&](int64_t m) __attribute__((always_inline)) {
    const uint32_t sw = static_cast<uint32_t>(m * RB);
#pragma unroll
    for (int v = 0; v < HT; ++v) {
      const int pc = ht + v * NH;
      if (pc < 10 * PPB) pp[v] = buf_load16(rw, W::P_OFF + static_cast<uint32_t>(pc * 16), sw);
    }
  };
  auto store_p = [&](T* sP) __attribute__((always_inline)) {
#pragma unroll
    for (int v = 0; v < HT; ++v) {
      const int pc = ht + v * NH;
      if (pc < 10 * PPB) {               // block u holds P_RJ: rows 16R.., columns 16J.. of P
        int R, J;
        tri_block(pc / PPB, R, J);
        const int a = (pc % PPB) / PPR, b0 = (pc % PPR) * EPV;
        u32x2* d2 = reinterpret_cast<u32x2*>(sP + (16 * R + a) * LCP + 16 * J + b0);   // 8-byte aligned rows
        d2[0] = u32x2{pp[v][0], pp[v][1]};
        d2[1] = u32x2{pp[v][2], pp[v][3]};
      }
    }
  };
  auto store_chunk = [&](char* base) __attribute__((always_inline)) {
    T* dK = reinterpret_cast<T*>(base + L::B_K);
    T* dQ = reinterpret_cast<T*>(base + L::B_Q);
    T* dV = reinterpret_cast<T*>(base + L::B_V);
    T* dT = reinterpret_cast<T*>(base + L::B_T);
#pragma unroll
    for (int v = 0; v < HK; ++v) {
      const int seg = ht + v * NH, row = seg / KROW, c = (seg % KROW) * EPV;
      if (NKP % NH != 0 && seg >= NKP) break;
      u32x2* k2 = reinterpret_cast<u32x2*>(dK + row * LDKK + c);    // k, q rows are 8-byte aligned
      k2[0] = u32x2{pk[v][0], pk[v][1]};
      k2[1] = u32x2{pk[v][2], pk[v][3]};
      u32x2* q2 = reinterpret_cast<u32x2*>(dQ + row * LDQ + c);
      q2[0] = u32x2{pq[v][0], pq[v][1]};
      q2[1] = u32x2{pq[v][2], pq[v][3]};
      if constexpr (CHAN || WK) {
        u32x2* d2 = reinterpret_cast<u32x2*>(reinterpret_cast<T*>(base + L::B_KD) + row * LDKD + c);
        d2[0] = u32x2{pkd[v][0], pkd[v][1]};
        d2[1] = u32x2{pkd[v][2], pkd[v][3]};
      }
    }
#pragma unroll
    for (int v = 0; v < HV; ++v) {
      const int seg = ht + v * NH, row = seg / VROW, c = (seg % VROW) * EPV;
      if (NVP % NH != 0 && seg >= NVP) break;
      *reinterpret_cast<u32x4*>(dV + row * LVT + c) = pv[v];
    }
#pragma unroll
    for (int v = 0; v < HT; ++v) {
      const int pc = ht + v * NH;
      if (pc < 10 * PPB) {               // block u holds (T_RJ)^T: rows 16J.., columns 16R.. of T^T
        int R, J;
        tri_block(pc / PPB, R, J);
        const int a = (pc % PPB) / PPR, b0 = (pc % PPR) * EPV;
        *reinterpret_cast<u32x4*>(dT + (16 * J + a) * LCT + 16 * R + b0) = pt[v];
      }
    }
    if (ht < NFP) *reinterpret_cast<u32x4*>(base + L::B_F + ht * 16) = pf;
  };

  // A chunk's LDS copy.
  struct Tiles {
    const T *K, *Q, *V, *Tt, *KD;
    // per-row factors; per-channel gate: beta, then e^{g_63} per channel from the row of er on
    const float *beta, *er, *eo, *ed, *gam, *g;
  };
  auto tiles = [&](int64_t n) __attribute__((always_inline)) {
    const char* cur = smem + (n & 1) * L::BUF;
    const float* f = reinterpret_cast<const float*>(cur + L::B_F);
    return Tiles{reinterpret_cast<const T*>(cur + L::B_K), reinterpret_cast<const T*>(cur + L::B_Q),
                 reinterpret_cast<const T*>(cur + L::B_V), reinterpret_cast<const T*>(cur + L::B_T),
                 reinterpret_cast<const T*>(cur + ((CHAN || WK) ? L::B_KD : L::B_K)),
                 f, f + CH, f + 2 * CH, f + 3 * CH, f + 4 * CH, f + 5 * CH};
  };

  // The two roles run separate loops with the same one barrier per chunk (the
  // role is uniform per wave), so neither keeps the other's registers live.
  if (chain) {
    // ---- chain waves: CG groups of 16 columns of S in MFMA accumulators --------------------
    // Every operand fragment read from LDS (rows of k, q, T, K^T, P) serves all CG groups.
    // The step is software-pipelined by hand: each stage issues the LDS reads of the
    // next one before its own products, and scheduling fences keep the compiler from
    // sinking those reads to their first use (which would expose the LDS latency on
    // every product).
    const int c0 = 16 * CG * cw;                // first column of this wave within the tile
    f32x4 S[CG][DKT];
#pragma unroll
    for (int g = 0; g < CG; ++g)
#pragma unroll
      for (int t = 0; t < DKT; ++t)
#pragma unroll
        for (int s = 0; s < 4; ++s)
          S[g][t][s] = p.S0 ? p.S0[(bh * DK + 16 * t + 4 * lg + s) * dv + col0 + c0 + 16 * g + lr] : 0.f;
    // the previous chunk's Q S (rows 16R + lr of O^T tiles), Delta and e^{g} of its rows
    f32x4 oq_prev[CG][4];
    frag db_prev[CG][4];
    float eo_prev[4];
#pragma unroll
    for (int R = 0; R < 4; ++R) {
      eo_prev[R] = 0.f;
#pragma unroll
      for (int g = 0; g < CG; ++g) {
        oq_prev[g][R] = f32x4{0.f, 0.f, 0.f, 0.f};
        db_prev[g][R] = O::cvt(oq_prev[g][R]);
      }
    }
    // Output voffset per (R, g); before the first chunk there is no output yet, and the
    // offset is pushed past the end of the buffer so the hardware drops those stores.
    uint32_t vo[4][CG];
#pragma unroll
    for (int R = 0; R < 4; ++R)
#pragma unroll
      for (int g = 0; g < CG; ++g)
        vo[R][g] = static_cast<uint32_t>(((16 * R + lr) * H * dv + col0 + c0 + 16 * g + 4 * lg) * ESZ);
    constexpr uint32_t DROP = 0x80000000u;     // beyond any sequence (at most 2^31 - 1 bytes)
    constexpr int NKB = DK / 32;
    // Training forward: the state entering each chunk, in bf16 and in the layout the
    // backward reads (four adjacent d_k values per lane, streaming stores).
    const uint32_t sbytes = static_cast<uint32_t>(dv * DK * 2);
    const rsrc_t rst = make_rsrc(SAVE ? static_cast<char*>(p.states) + sq.rec0 * sbytes : nullptr,
                                 SAVE ? static_cast<uint32_t>(nchunks * sbytes) : 0u);
    uint32_t sto[CG];
#pragma unroll
    for (int g = 0; g < CG; ++g) sto[g] = chunk_state_off(4 * lg, col0 + c0 + 16 * g + lr, dv);
    __syncthreads();                            // chunk 0 in LDS

    for (int64_t n = 0; n < nchunks; ++n) {
      const Tiles c = tiles(n);
      const T* sP = p_tile(n - 1);
      frag kf[2][2 * NKB], qf[2][2 * NKB];      // rows of k and q of one row block, double-buffered
      frag vt[4][CG];                           // v (transposed) of each row block
      f32x4 be[4], er[4];
      float eo[4];
      auto load_rows = [&](int b, int R) __attribute__((always_inline)) {
#pragma unroll
        for (int kb = 0; kb < NKB; ++kb) {
          const T* kr = c.K + (16 * R + lr) * LDKK + 32 * kb + 4 * lg;
          const T* qr = c.Q + (16 * R + lr) * LDQ + 32 * kb + 4 * lg;
          kf[b][2 * kb] = O::ld(kr);
          kf[b][2 * kb + 1] = O::ld(kr + 16);
          qf[b][2 * kb] = O::ld(qr);
          qf[b][2 * kb + 1] = O::ld(qr + 16);
        }
#pragma unroll
        for (int g = 0; g < CG; ++g) vt[R][g] = O::ld_tr(c.V, LVT, 16 * R, c0 + 16 * g, lr, lg);
        be[R] = *reinterpret_cast<const f32x4*>(c.beta + 16 * R + 4 * lg);
        er[R] = *reinterpret_cast<const f32x4*>(c.er + 16 * R + 4 * lg);
        eo[R] = gate_scalar(GATE) ? c.eo[16 * R + lr] : 1.f;
      };

      // stage A: P of the previous chunk, rows of block 0; S to bf16
      frag pf[10];
#pragma unroll
      for (int R = 0; R < 4; ++R)
#pragma unroll
        for (int J = 0; J <= R; ++J) pf[R * (R + 1) / 2 + J] = O::ld(sP + (16 * R + lr) * LCP + 16 * J + 4 * lg);
      load_rows(0, 0);
      frag Sb[CG][DKT];
#pragma unroll
      for (int g = 0; g < CG; ++g)
#pragma unroll
        for (int t = 0; t < DKT; ++t) Sb[g][t] = O::cvt(S[g][t]);
      if constexpr (SAVE) {
        const uint32_t so = static_cast<uint32_t>(n) * sbytes;
#pragma unroll
        for (int g = 0; g < CG; ++g)
#pragma unroll
          for (int t = 0; t < DKT; ++t)
            buf_store8_nt(__builtin_bit_cast(u32x2, Sb[g][t]), rst, sto[g] + chunk_state_off(16 * t, 0, dv), so);
      }

      // stages KS(R): K S and Q S of row block R; the residual of block R-1 (its K S has
      // had a stage to drain); the previous chunk's output after block 0
      f32x4 x[4][CG];
      frag Rb[CG][4];
      frag tf[10];                              // rows of T (from T^T)
      f32x4 ed[4];
      float gam = 1.f;
      auto resid = [&](int R) __attribute__((always_inline)) {
#pragma unroll
        for (int g = 0; g < CG; ++g) {
          const f32x4 vv = O::f32(vt[R][g]);
          f32x4 rr;
#pragma unroll
          for (int s = 0; s < 4; ++s)
            rr[s] = be[R][s] * (vv[s] - (gate_scalar(GATE) ? x[R][g][s] * er[R][s] : x[R][g][s]));
          Rb[g][R] = O::cvt(rr);
        }
      };
#pragma unroll
      for (int R = 0; R < 4; ++R) {
        __builtin_amdgcn_sched_barrier(0);
        if (R < 3) {
          load_rows((R + 1) & 1, R + 1);
        } else {
#pragma unroll
          for (int Rr = 0; Rr < 4; ++Rr)
#pragma unroll
            for (int m = 0; m <= Rr; ++m) tf[Rr * (Rr + 1) / 2 + m] = O::ld_tr(c.Tt, LCT, 16 * m, 16 * Rr, lr, lg);
#pragma unroll
          for (int Rr = 0; Rr < 4; ++Rr)
            ed[Rr] = gate_scalar(GATE) ? *reinterpret_cast<const f32x4*>(c.ed + 16 * Rr + 4 * lg)
                                         : f32x4{1.f, 1.f, 1.f, 1.f};
          if constexpr (gate_scalar(GATE)) gam = c.gam[0];
        }
        __builtin_amdgcn_sched_barrier(0);
        f32x4 oq[CG];
#pragma unroll
        for (int g = 0; g < CG; ++g) x[R][g] = oq[g] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int kb = 0; kb < NKB; ++kb)
#pragma unroll
          for (int g = 0; g < CG; ++g) {
            x[R][g] = O::mma2(x[R][g], kf[R & 1][2 * kb], kf[R & 1][2 * kb + 1], Sb[g][2 * kb], Sb[g][2 * kb + 1]);
            oq[g] = O::mma2(oq[g], Sb[g][2 * kb], Sb[g][2 * kb + 1], qf[R & 1][2 * kb], qf[R & 1][2 * kb + 1]);
          }
        if (R == 0) {
          // O^T tiles of chunk n-1: (Q S)^T e^{g} + Delta^T P^T, four adjacent columns per lane;
          // rows past the end of the sequence fall outside the buffer
          const uint32_t so = n > 0 ? static_cast<uint32_t>((n - 1) * CH * H * dv * ESZ) : 0u;
          const uint32_t drop = n > 0 ? 0u : DROP;
#pragma unroll
          for (int Ro = 0; Ro < 4; ++Ro) {
            f32x4 op[CG];
#pragma unroll
            for (int g = 0; g < CG; ++g) op[g] = f32x4{0.f, 0.f, 0.f, 0.f};
            int J = 0;
#pragma unroll
            for (; J + 1 <= Ro; J += 2)
#pragma unroll
              for (int g = 0; g < CG; ++g)
                op[g] = O::mma2(op[g], db_prev[g][J], db_prev[g][J + 1], pf[Ro * (Ro + 1) / 2 + J],
                                pf[Ro * (Ro + 1) / 2 + J + 1]);
            if (J <= Ro)
#pragma unroll
              for (int g = 0; g < CG; ++g) op[g] = O::mma1(op[g], db_prev[g][J], pf[Ro * (Ro + 1) / 2 + J]);
#pragma unroll
            for (int g = 0; g < CG; ++g) {
              const f32x4 ov = gate_scalar(GATE) ? oq_prev[g][Ro] * eo_prev[Ro] + op[g] : oq_prev[g][Ro] + op[g];
              buf_store8(__builtin_bit_cast(u32x2, to_bf16x4(ov)), ro, vo[Ro][g] + drop, so);
            }
          }
        } else {
          resid(R - 1);
        }
#pragma unroll
        for (int g = 0; g < CG; ++g) oq_prev[g][R] = oq[g];
        eo_prev[R] = eo[R];
      }

      // stage Delta: Delta_R = sum_{m <= R} T_Rm R_m; first rows of K^T for the update
      frag ktf[2][8];                           // K^T fragments of two 16-row tiles, double-buffered
      f32x4 gc[2][2];                           // per-channel gate: e^{g_63} of those rows of S
      auto load_kt = [&](int b, int tp) __attribute__((always_inline)) {
        if constexpr (CHAN)
#pragma unroll
          for (int h = 0; h < 2; ++h) gc[b][h] = *reinterpret_cast<const f32x4*>(c.er + 16 * (2 * tp + h) + 4 * lg);
#pragma unroll
        for (int h = 0; h < 2; ++h)
#pragma unroll
          for (int i = 0; i < 4; ++i) ktf[b][4 * h + i] = O::ld_tr(c.KD, LDKD, 16 * i, 16 * (2 * tp + h), lr, lg);
      };
      __builtin_amdgcn_sched_barrier(0);
      load_kt(0, 0);
      __builtin_amdgcn_sched_barrier(0);
      resid(3);
      frag Ds[CG][4];
#pragma unroll
      for (int R = 0; R < 4; ++R) {
        f32x4 d[CG];
#pragma unroll
        for (int g = 0; g < CG; ++g) d[g] = f32x4{0.f, 0.f, 0.f, 0.f};
        int m = 0;
#pragma unroll
        for (; m + 1 <= R; m += 2)
#pragma unroll
          for (int g = 0; g < CG; ++g)
            d[g] = O::mma2(d[g], tf[R * (R + 1) / 2 + m], tf[R * (R + 1) / 2 + m + 1], Rb[g][m], Rb[g][m + 1]);
        if (m <= R)
#pragma unroll
          for (int g = 0; g < CG; ++g) d[g] = O::mma1(d[g], tf[R * (R + 1) / 2 + m], Rb[g][m]);
#pragma unroll
        for (int g = 0; g < CG; ++g) {
          db_prev[g][R] = O::cvt(d[g]);
          Ds[g][R] = gate_scalar(GATE) ? O::cvt(d[g] * ed[R]) : db_prev[g][R];
        }
      }

      // stages U(tp): S' = e^{g_63} S + K^T diag(e^{g_63 - g}) Delta, two 16-row tiles each
#pragma unroll
      for (int tp = 0; tp < DKT / 2; ++tp) {
        __builtin_amdgcn_sched_barrier(0);
        if (tp + 1 < DKT / 2) load_kt((tp + 1) & 1, tp + 1);
        __builtin_amdgcn_sched_barrier(0);
#pragma unroll
        for (int h = 0; h < 2; ++h) {
          const int t = 2 * tp + h;
#pragma unroll
          for (int g = 0; g < CG; ++g) {
            f32x4 acc = S[g][t];
            if constexpr (gate_scalar(GATE)) acc = acc * gam;
            if constexpr (CHAN) acc = acc * gc[tp & 1][h];
            acc = O::mma2(acc, ktf[tp & 1][4 * h], ktf[tp & 1][4 * h + 1], Ds[g][0], Ds[g][1]);
            S[g][t] = O::mma2(acc, ktf[tp & 1][4 * h + 2], ktf[tp & 1][4 * h + 3], Ds[g][2], Ds[g][3]);
          }
        }
      }
      __builtin_amdgcn_sched_barrier(0);
      __syncthreads();                          // next chunk's tiles and this chunk's P in place
    }
    // output of the last chunk
    if (nchunks > 0) {
      const T* sP = p_tile(nchunks - 1);
      const uint32_t so = static_cast<uint32_t>((nchunks - 1) * CH * H * dv * ESZ);
#pragma unroll
      for (int R = 0; R < 4; ++R) {
        f32x4 op[CG];
#pragma unroll
        for (int g = 0; g < CG; ++g) op[g] = f32x4{0.f, 0.f, 0.f, 0.f};
        const T* pr = sP + (16 * R + lr) * LCP + 4 * lg;
#pragma unroll
        for (int J = 0; J <= R; ++J) {
          const frag p0 = O::ld(pr + 16 * J);
#pragma unroll
          for (int g = 0; g < CG; ++g) op[g] = O::mma1(op[g], db_prev[g][J], p0);
        }
#pragma unroll
        for (int g = 0; g < CG; ++g) {
          const f32x4 ov = gate_scalar(GATE) ? oq_prev[g][R] * eo_prev[R] + op[g] : oq_prev[g][R] + op[g];
          buf_store8(__builtin_bit_cast(u32x2, to_bf16x4(ov)), ro, vo[R][g], so);
        }
      }
    }
    if (p.S_T) {
#pragma unroll
      for (int g = 0; g < CG; ++g)
#pragma unroll
        for (int t = 0; t < DKT; ++t)
#pragma unroll
          for (int s = 0; s < 4; ++s)
            p.S_T[(bh * DK + 16 * t + 4 * lg + s) * dv + col0 + c0 + 16 * g + lr] = S[g][t][s];
    }
  } else {
    // ---- helper waves -------------------------------------------------------------------
    if (nchunks > 0) {
      prefetch(0);
      if constexpr (CHAN) prefetch_p(0);
      store_chunk(smem);
      if (nchunks > 1) prefetch(1);
    }
    __syncthreads();                            // chunk 0 in LDS

    for (int64_t n = 0; n < nchunks; ++n) {
      const Tiles c = tiles(n);
      // this helper's share of P of chunk n into copy n % 2 (copy n % 2 was last
      // read by the chain waves in the previous step, before the opening barrier)
      T* sP = p_tile(n);
      if constexpr (CHAN) {                     // P of chunk n from the record
        store_p(sP);
        if (n + 1 < nchunks) prefetch_p(n + 1);
      }
      // rows 16R.. of P: the rows of q are read once per row block, and with R a
      // compile-time constant the R + 1 blocks of the row are unrolled, so their
      // product chains and exponentials overlap instead of running one after another
      auto p_row = [&](auto RC) __attribute__((always_inline)) {
        constexpr int R = decltype(RC)::value;
        frag qf[DK / 16];
#pragma unroll
        for (int kb = 0; kb < DK / 32; ++kb) {
          qf[2 * kb] = O::ld(c.Q + (16 * R + lr) * LDQ + 32 * kb + 4 * lg);
          qf[2 * kb + 1] = O::ld(c.Q + (16 * R + lr) * LDQ + 32 * kb + 4 * lg + 16);
        }
        const int r = 16 * R + lr;
        const float gr = c.g[r];
#pragma unroll
        for (int J = 0; J <= R; ++J) {
          // (P_RJ)^T = K_J Q_R^T: lane holds P[16R + lr][16J + 4lg + s], four adjacent columns
          f32x4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
          for (int kb = 0; kb < DK / 32; ++kb) {
            const T* kr = c.KD + (16 * J + lr) * LDKD + 32 * kb + 4 * lg;   // k, or the write key
            acc = O::mma2(acc, O::ld(kr), O::ld(kr + 16), qf[2 * kb], qf[2 * kb + 1]);
          }
          const f32x4 gj = *reinterpret_cast<const f32x4*>(c.g + 16 * J + 4 * lg);
#pragma unroll
          for (int s = 0; s < 4; ++s) {
            float val = acc[s];
            if constexpr (gate_scalar(GATE)) val *= __expf(gr - gj[s]);
            acc[s] = (R == J && lr < 4 * lg + s) ? 0.f : val;
          }
          *reinterpret_cast<frag*>(sP + r * LCP + 16 * J + 4 * lg) = O::cvt(acc);
        }
      };
      if constexpr (!CHAN) {
        for (int R = cw; R < 4; R += NHW) {   // R = cw, cw + NHW, ..
          switch (R) {
            case 0: p_row(std::integral_constant<int, 0>()); break;
            case 1: p_row(std::integral_constant<int, 1>()); break;
            case 2: p_row(std::integral_constant<int, 2>()); break;
            default: p_row(std::integral_constant<int, 3>()); break;
          }
        }
      }
      // next chunk into the other LDS copy (last read before this step's opening
      // barrier), loads of the one after
      if (n + 1 < nchunks) {
        store_chunk(smem + ((n + 1) & 1) * L::BUF);
        if (n + 2 < nchunks) prefetch(n + 2);
      }
      __syncthreads();                          // next chunk's tiles and this chunk's P in place
    }
  }
}

template <int GATE, int DK, int NCH, int CG, int NHW>
static hipError_t launch_pipe_t(const ChunkParams& p, hipStream_t stream) {
  const int n_tiles = p.d_v / (16 * CG * NCH);
  const int64_t nblk = p.B * p.H * n_tiles;
  if (p.states)
    hipLaunchKernelGGL((chunk_state_pipe_kernel<GATE, DK, NCH, CG, NHW, true>), dim3(static_cast<unsigned>(nblk)),
                       dim3((NCH + NHW) * 64), 0, stream, p, n_tiles);
  else
    hipLaunchKernelGGL((chunk_state_pipe_kernel<GATE, DK, NCH, CG, NHW, false>), dim3(static_cast<unsigned>(nblk)),
                       dim3((NCH + NHW) * 64), 0, stream, p, n_tiles);
  return hipGetLastError();
}

template <int GATE, int DK>
static hipError_t launch_pipe_dk(const ChunkParams& p, hipStream_t stream) {
  // 32 columns per workgroup: 2 chain waves and 4 helpers (measured: 15-20% faster
  // than 2 helpers, as fast as 6, on the per-channel and the no-gate workloads).
  if constexpr (GATE == GATE_CHANNEL) {
    // per-channel gate: the third operand tile leaves LDS room for 32 columns only
    return launch_pipe_t<GATE, DK, 2, 1, 4>(p, stream);
  } else if constexpr (gate_wkey(GATE) && DK == 64) {
    return launch_pipe_t<GATE, DK, 2, 1, 4>(p, stream);
  } else {
    // 64 columns per workgroup when that still gives one workgroup per CU, else 32.
    // Measured on the gated workload (state pass): 4 chain waves of 16 columns with
    // 4 helpers is fastest; 2 chain waves of 32 columns (2 or 4 helpers) and 4
    // chain waves with 2 helpers were 8-50% slower (32-column chain waves run out
    // of registers).
    if (p.B * p.H * (p.d_v / 64) >= 256) return launch_pipe_t<GATE, DK, 4, 1, 4>(p, stream);
    return launch_pipe_t<GATE, DK, 2, 1, 4>(p, stream);
  }
}

template <int GATE>
static hipError_t launch_pipe_g(const ChunkParams& p, hipStream_t stream) {
  if (p.d_k == 128) return launch_pipe_dk<GATE, 128>(p, stream);
  if (p.d_k == 64) return launch_pipe_dk<GATE, 64>(p, stream);
  return hipErrorInvalidValue;
}

hipError_t launch_chunk_state_pipe(const ChunkParams& p, hipStream_t stream) {
  if (p.io != IO_BF16) return hipErrorInvalidValue;
  if (p.kw) {   // write key: the per-channel gate reads its write-key operands from the records
    if (p.gate == GATE_NONE) return launch_pipe_g<GATE_WKEY>(p, stream);
    if (p.gate == GATE_SCALAR) return launch_pipe_g<GATE_WKEY_SCALAR>(p, stream);
    if (p.gate != GATE_CHANNEL) return hipErrorInvalidValue;
  }
  if (p.gate == GATE_NONE) return launch_pipe_g<GATE_NONE>(p, stream);
  if (p.gate == GATE_SCALAR) return launch_pipe_g<GATE_SCALAR>(p, stream);
  if (p.gate == GATE_CHANNEL) return launch_pipe_g<GATE_CHANNEL>(p, stream);
  return hipErrorInvalidValue;
}

}  // namespace gdr
