// Backward pass of the chunkwise gated delta rule on gfx950: bf16 I/O, no gate or a
// scalar gate, decay before the erase (g_read = g below) or erase on the undecayed
// state (g_read_r = g_{r-1}, the A factor and the residual's decay read g_read),
// optionally with a separate write key ("OSDN: Improving Delta Rule with Provable
// Online Preconditioning in Linear Attention", §2.1: the erase reads along k, the
// write goes along kw; below, the column side of A and P, dDelta's key product and
// the state write then take KW, see bwd_chunk_kernel).
//
// The pages print no gradients; these are the reverse-mode derivatives of the
// chunk form of "Moonshot AI's New Attention Architecture: Key Innovations
// Explained", §3 Hardware-Friendly Algorithm (and §5: the gate stays in the log
// domain).  Per chunk (rows r = 0..63, g_r the running sum of log a inside the
// chunk, D_rj = e^{g_r - g_j}, S the state entering the chunk, dS' the gradient of
// the state leaving it, dO the gradient of the output):
//   forward   X = V - diag(e^{g_read}) K S,   Delta = T diag(beta) X,   T = (I + A)^{-1},
//             A = strict_lower(diag(beta) D_read * K K^T),   P = lower_incl(D * Q K^T),
//             O = diag(e^g) Q S + P Delta,   S' = e^{g_63} S + K^T diag(e^{g_63 - g}) Delta
//   reverse   dDelta = P^T dO + diag(e^{g_63 - g}) K dS',   dY = T^T dDelta,
//             dS = e^{g_63} dS' + Q^T diag(e^g) dO - K^T diag(beta e^g) dY
//   per chunk dv = diag(beta) dY,   dA = -strict_lower(dY Delta^T),   dP = lower_incl(dO Delta^T),
//             dq = (D * dP) K + diag(e^g) dO S^T,
//             dk = (beta D * dA) K + (beta D * dA)^T K + (D * dP)^T Q
//                  - diag(beta e^g) dY S^T + diag(e^{g_63 - g}) Delta dS'^T,
//             dbeta_r = sum_v dY X + sum_j dA_rj D_rj (K K^T)_rj,
//             dg_r = (row sums - column sums of dA * A and dP * P)_r
//                    - beta_r e^{g_r} k_r . (dY S^T)_r + e^{g_r} q_r . (dO S^T)_r - c_r,
//             c_r = e^{g_63 - g_r} k_r . (Delta dS'^T)_r,   dg_63 += sum_r c_r + e^{g_63} <dS', S>,
//             d log a_s = sum_{r >= s} dg_r.
//
// Three passes follow the per-chunk transform (chunk_prep.hip, which gives T and
// the gate factors of every chunk):
//   1. the states entering each chunk, in order (one workgroup per (sequence,
//      head, 64 state columns); the state in MFMA accumulators, as in the forward);
//   2. the gradients of the states leaving each chunk, in reverse order (the same
//      shape of work, dS in accumulators);
//   3. every chunk at once: the gradients of q, k, v, beta and log a.
// Passes 1 and 2 are independent and share one launch.  They store the states in
// bf16, the precision the forward's products read them in, in d_k tiles of 16 that
// are value-major (chunk_state_off) so that an accumulator lane writes four adjacent
// values and a store instruction 512 contiguous bytes.
//
// After a training forward (gdr_chunk_fwd_save), which leaves the transform's
// records and the chunk-start states in this workspace, neither the transform nor
// pass 1 runs; pass 2 then has the compute unit to itself and, without a per-channel
// gate or a write key, runs as bwd_rev_pipe_kernel (chain and helper waves).
//
// With a per-channel gate the two sequential passes here take the transform's
// decayed operands (k e^{g_read}, q e^{g}, k e^{g_63 - g}) and its P, and scale the
// state's rows by e^{g_63} of their channel; the per-chunk gradients of that gate
// are in chunk_bwd_chan.hip.  Operand fragments as described in bwd_common.h.
#include "bwd_common.h"
#include "launchers.h"

namespace gdr {

namespace {

// ---------------------------------------------------------------------------
// Passes 1 and 2: the sequential passes.  Neither reads what the other writes, so
// one launch runs both, and each compute unit holds a workgroup of each (their
// LDS together fits in one CU's 160 KB).  Four waves per workgroup, 16 state
// columns each.  LDS: pass 1 keeps two copies of one chunk's tiles (k, a 64-column
// v tile, T^T, the gate factors); pass 2 one copy (k, q, a 64-column dO tile, T^T,
// the factors) and P of the chunk.  Pass 1 reads k both ways, v and T^T transposed;
// pass 2 reads k and q both ways, dO and P transposed, T^T by rows.
// ---------------------------------------------------------------------------
// KD: a third key tile, the operand of the state update (pass 1) and of dDelta's key
// product (pass 2): k e^{g_63 - g} from the record (per-channel gate), or the write key.
template <int DK, bool REV, bool KD = false>
struct SeqLayout {
  static constexpr int LDK = ld_both(DK);
  static constexpr int LDV = ld_tr(64);
  static constexpr int LCT = REV ? ld_row(CH) : ld_tr(CH);
  static constexpr int LCP = ld_tr(CH);
  static constexpr size_t KB = size_t(CH) * LDK * 2;
  static constexpr size_t VB = size_t(CH) * LDV * 2;
  static constexpr size_t TB = size_t(CH) * LCT * 2;
  static constexpr size_t O_K = 0, O_Q = O_K + KB, O_V = O_Q + (REV ? KB : 0), O_T = O_V + VB, O_F = O_T + TB;
  static constexpr size_t O_KD = O_F + 6 * CH * 4;   // per-channel gate: k e^{g_63 - g}
  static constexpr size_t BUF = O_KD + (KD ? KB : 0);
  static constexpr size_t O_P = (REV ? 1 : 2) * BUF;
  static constexpr size_t TOTAL = O_P + (REV ? size_t(CH) * LCP * 2 : 0);
};

// One chunk's tiles in registers, then into one LDS copy: k (and q), the 64-column
// tile of v (or dO) from column col0, the T blocks and the factor rows of the record.
// Per-channel gate: k e^{g_read}, q e^{g} and k e^{g_63 - g} from the record in place
// of k and q, and (pass 2) the record's P.  With a write key (WK) its tile is the
// third key tile.
template <int DK, int NT, bool WITH_Q, bool CHAN = false, bool WK = false>
struct SeqStage {
  typedef SeqLayout<DK, WITH_Q, CHAN || WK> L;
  static constexpr uint32_t RB = rec_bytes(IO_BF16, CHAN ? GATE_CHANNEL : GATE_SCALAR, DK);
  static constexpr int KR = DK / 8;                  // 16-byte pieces per k row
  static constexpr int KP = CH * KR / NT;            // per thread
  static constexpr int VP = CH * 8 / NT;
  static constexpr int TP = (10 * 32 + NT - 1) / NT; // T blocks: 32 pieces each
  static_assert(KP * NT == CH * KR && VP * NT == CH * 8, "tile pieces split evenly");
  u32x4 k[KP], q[WITH_Q ? KP : 1], kd[CHAN || WK ? KP : 1], v[VP], t[TP], pp[CHAN && WITH_Q ? TP : 1], f;

  __device__ __forceinline__ void load(rsrc_t rk, rsrc_t rq, rsrc_t rv, rsrc_t rw, rsrc_t rkw, int64_t n, int tid,
                                       int H, int dv, int col0) {
    const uint32_t sk = static_cast<uint32_t>(n * CH * H * DK * 2);
    const uint32_t sv = static_cast<uint32_t>(n * CH * H * dv * 2);
    const uint32_t sw = static_cast<uint32_t>(n * RB);
#pragma unroll
    for (int i = 0; i < KP; ++i) {
      const int pc = tid + i * NT;
      if constexpr (CHAN) {
        const uint32_t off = W::X_OFF + static_cast<uint32_t>(((pc / KR) * DK + (pc % KR) * 8) * 2);
        k[i] = buf_load16(rw, off, sw);
        if constexpr (WITH_Q) q[i] = buf_load16(rw, off + CH * DK * 2, sw);
        kd[i] = buf_load16(rw, off + 2 * CH * DK * 2, sw);
      } else {
        const uint32_t off = static_cast<uint32_t>(((pc / KR) * H * DK + (pc % KR) * 8) * 2);
        k[i] = buf_load16(rk, off, sk);
        if constexpr (WITH_Q) q[i] = buf_load16(rq, off, sk);
        if constexpr (WK) kd[i] = buf_load16(rkw, off, sk);
      }
    }
#pragma unroll
    for (int i = 0; i < VP; ++i) {
      const int pc = tid + i * NT;
      v[i] = buf_load16(rv, static_cast<uint32_t>(((pc / 8) * H * dv + col0 + (pc % 8) * 8) * 2), sv);
    }
#pragma unroll
    for (int i = 0; i < TP; ++i) {
      const int pc = tid + i * NT;
      if (pc < 320) t[i] = buf_load16(rw, W::T_OFF + static_cast<uint32_t>(pc * 16), sw);
      if constexpr (CHAN && WITH_Q)
        if (pc < 320) pp[i] = buf_load16(rw, W::P_OFF + static_cast<uint32_t>(pc * 16), sw);
    }
    if (tid < 96) f = buf_load16(rw, W::F_OFF + static_cast<uint32_t>(tid * 16), sw);
  }

  __device__ __forceinline__ void store(char* base, int tid) const {
    T* dK = reinterpret_cast<T*>(base + L::O_K);
    T* dQ = reinterpret_cast<T*>(base + L::O_Q);
    T* dV = reinterpret_cast<T*>(base + L::O_V);
    T* dT = reinterpret_cast<T*>(base + L::O_T);
#pragma unroll
    for (int i = 0; i < KP; ++i) {
      const int pc = tid + i * NT;
      put16(dK + (pc / KR) * L::LDK + (pc % KR) * 8, k[i]);
      if constexpr (WITH_Q) put16(dQ + (pc / KR) * L::LDK + (pc % KR) * 8, q[i]);
      if constexpr (CHAN || WK) put16(reinterpret_cast<T*>(base + L::O_KD) + (pc / KR) * L::LDK + (pc % KR) * 8, kd[i]);
    }
#pragma unroll
    for (int i = 0; i < VP; ++i) {
      const int pc = tid + i * NT;
      put16(dV + (pc / 8) * L::LDV + (pc % 8) * 8, v[i]);
    }
#pragma unroll
    for (int i = 0; i < TP; ++i) {
      const int pc = tid + i * NT;
      if (pc < 320) {                    // block u holds (T_RJ)^T: the T^T tile, blocks on or above the diagonal
        int R, J;
        tri_block(pc / 32, R, J);
        const int a = (pc % 32) / 2, b0 = (pc % 2) * 8;
        put16(dT + (16 * J + a) * L::LCT + 16 * R + b0, t[i]);
        if constexpr (CHAN && WITH_Q)   // block u holds P_RJ: rows 16R.., columns 16J.. of P
          put16(reinterpret_cast<T*>(base + L::O_P) + (16 * R + a) * L::LCP + 16 * J + b0, pp[i]);
      }
    }
    if (tid < 96) *reinterpret_cast<u32x4*>(base + L::O_F + tid * 16) = f;
  }
};

// Pass 1: the state entering every chunk, stored in bf16 (chunk_state_off).  lb is the
// workgroup's (sequence, head, tile) index.  With a write key (WK) the update writes
// along it: S' = e^{g_63} S + KW^T (e^{g_63 - g} Delta).
template <int GATE, int DK, bool WK>
__device__ __forceinline__ void states_pass(const BwdParams& p, int n_tiles, int lb, char* smem) {
  constexpr bool CHAN = GATE == GATE_CHANNEL;
  constexpr uint32_t RB = rec_bytes(IO_BF16, GATE, DK);
  typedef SeqLayout<DK, false, CHAN || WK> L;
  constexpr int DKT = DK / 16, LDK = L::LDK, LDV = L::LDV, LCT = L::LCT;
  const ChunkParams& f = p.f;
  const int64_t bh = lb / n_tiles;
  const int tile = lb % n_tiles;
  const int64_t bb = bh / f.H, hh = bh % f.H;
  const int dv = f.d_v, H = static_cast<int>(f.H), col0 = tile * 64;
  const int tid = threadIdx.x;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int lane = tid & 63, lr = lane & 15, lg = lane >> 4;
  const int scol = col0 + 16 * wave + lr;
  const BwdSeq sq = bwd_seq_of(f, bb, hh);
  const int64_t nch = sq.nch;
  const Slice sl = sq.sl;
  const rsrc_t rk = sl.rs(f.k, DK), rv = sl.rs(f.v, dv), rkw = WK ? sl.rs(f.kw, DK) : rk;
  const rsrc_t rw = make_rsrc(static_cast<const char*>(f.ws) + sq.rec0 * RB, static_cast<uint32_t>(nch * RB));
  const uint32_t sbytes = static_cast<uint32_t>(dv * DK * 2);   // one chunk's state
  const rsrc_t rst = make_rsrc(static_cast<char*>(p.states) + sq.rec0 * sbytes, static_cast<uint32_t>(nch * sbytes));

  f32x4 S[DKT];   // S[t][s] = S[16t + 4lg + s][scol]
#pragma unroll
  for (int t = 0; t < DKT; ++t)
#pragma unroll
    for (int s = 0; s < 4; ++s) S[t][s] = f.S0 ? f.S0[(bh * DK + 16 * t + 4 * lg + s) * dv + scol] : 0.f;

  SeqStage<DK, 256, false, CHAN, WK> st;
  if (nch > 0) {
    st.load(rk, rk, rv, rw, rkw, 0, tid, H, dv, col0);
    st.store(smem, tid);
    if (nch > 1) st.load(rk, rk, rv, rw, rkw, 1, tid, H, dv, col0);
  }
  __syncthreads();
  for (int64_t n = 0; n < nch; ++n) {
    const char* cur = smem + (n & 1) * L::BUF;
    const T* sK = reinterpret_cast<const T*>(cur + L::O_K);
    const T* sV = reinterpret_cast<const T*>(cur + L::O_V);
    const T* sT = reinterpret_cast<const T*>(cur + L::O_T);
    const T* sKD = reinterpret_cast<const T*>(cur + (CHAN || WK ? L::O_KD : L::O_K));   // K^T of the update
    const float* sF = reinterpret_cast<const float*>(cur + L::O_F);
    if (n + 1 < nch) {   // the other copy was last read before the previous barrier
      st.store(smem + ((n + 1) & 1) * L::BUF, tid);
      if (n + 2 < nch) st.load(rk, rk, rv, rw, rkw, n + 2, tid, H, dv, col0);
    }
    const uint32_t so = static_cast<uint32_t>(n) * sbytes;
#pragma unroll
    for (int t = 0; t < DKT; ++t) buf_store8(bits8(S[t]), rst, chunk_state_off(16 * t + 4 * lg, scol, dv), so);

    frag Sb[DKT];
#pragma unroll
    for (int t = 0; t < DKT; ++t) Sb[t] = O::cvt(S[t]);
    frag Rb[4];
#pragma unroll
    for (int R = 0; R < 4; ++R) {        // diag(beta) X, X = V - diag(e^g) K S
      f32x4 x = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int kb = 0; kb < DK / 32; ++kb)
        x = O::mma2(x, rowf(sK, LDK, 16 * R, 32 * kb, lr, lg), rowf(sK, LDK, 16 * R, 32 * kb + 16, lr, lg),
                    Sb[2 * kb], Sb[2 * kb + 1]);
      const f32x4 vv = O::f32(colf(sV, LDV, 16 * R, 16 * wave, lr, lg));
      f32x4 rr;
#pragma unroll
      for (int s = 0; s < 4; ++s) {
        const int r = 16 * R + 4 * lg + s;
        rr[s] = sF[r] * (vv[s] - (GATE == GATE_SCALAR ? x[s] * sF[CH + r] : x[s]));
      }
      Rb[R] = O::cvt(rr);
    }
    frag Ds[4];
#pragma unroll
    for (int R = 0; R < 4; ++R) {        // Delta = T diag(beta) X, rows of T from T^T; then e^{g_63 - g}
      f32x4 d = {0.f, 0.f, 0.f, 0.f};
      int m = 0;
#pragma unroll
      for (; m + 1 <= R; m += 2)
        d = O::mma2(d, colf(sT, LCT, 16 * m, 16 * R, lr, lg), colf(sT, LCT, 16 * (m + 1), 16 * R, lr, lg), Rb[m],
                    Rb[m + 1]);
      if (m <= R) d = O::mma1(d, colf(sT, LCT, 16 * m, 16 * R, lr, lg), Rb[m]);
      if constexpr (GATE == GATE_SCALAR) {
#pragma unroll
        for (int s = 0; s < 4; ++s) d[s] *= sF[3 * CH + 16 * R + 4 * lg + s];
      }
      Ds[R] = O::cvt(d);
    }
#pragma unroll
    for (int t = 0; t < DKT; ++t) {      // S' = e^{g_63} S + K^T (e^{g_63 - g} Delta)
      f32x4 acc = S[t];
      if constexpr (GATE == GATE_SCALAR) acc = acc * sF[4 * CH];
      if constexpr (CHAN) {
#pragma unroll
        for (int s = 0; s < 4; ++s) acc[s] *= sF[CH + 16 * t + 4 * lg + s];
      }
      acc = O::mma2(acc, colf(sKD, LDK, 0, 16 * t, lr, lg), colf(sKD, LDK, 16, 16 * t, lr, lg), Ds[0], Ds[1]);
      acc = O::mma2(acc, colf(sKD, LDK, 32, 16 * t, lr, lg), colf(sKD, LDK, 48, 16 * t, lr, lg), Ds[2], Ds[3]);
      S[t] = acc;
    }
    __syncthreads();
  }
}

// Pass 2: the gradient of the state leaving every chunk, last chunk first, and dS0.
// One LDS copy of the chunk's tiles: the next chunk waits in registers and goes
// in after the step's last read.  With a write key (WK) P and dDelta's key product
// take it: P = lower_incl(D * Q KW^T), dDelta = diag(e^{g_63 - g}) KW dS' + P^T dO.
template <int GATE, int DK, bool WK>
__device__ __forceinline__ void reverse_pass(const BwdParams& p, int n_tiles, int lb, char* smem) {
  constexpr bool CHAN = GATE == GATE_CHANNEL;
  constexpr uint32_t RB = rec_bytes(IO_BF16, GATE, DK);
  typedef SeqLayout<DK, true, CHAN || WK> L;
  constexpr int DKT = DK / 16, LDK = L::LDK, LDV = L::LDV, LCT = L::LCT, LCP = L::LCP;
  const ChunkParams& f = p.f;
  const int64_t bh = lb / n_tiles;
  const int tile = lb % n_tiles;
  const int64_t bb = bh / f.H, hh = bh % f.H;
  const int dv = f.d_v, H = static_cast<int>(f.H), col0 = tile * 64;
  const int tid = threadIdx.x;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int lane = tid & 63, lr = lane & 15, lg = lane >> 4;
  const int scol = col0 + 16 * wave + lr;
  const BwdSeq sq = bwd_seq_of(f, bb, hh);
  const int64_t nch = sq.nch;
  const Slice sl = sq.sl;
  const rsrc_t rk = sl.rs(f.k, DK), rq = sl.rs(f.q, DK), rdo = sl.rs(p.dO, dv), rkw = WK ? sl.rs(f.kw, DK) : rk;
  const rsrc_t rw = make_rsrc(static_cast<const char*>(f.ws) + sq.rec0 * RB, static_cast<uint32_t>(nch * RB));
  const uint32_t sbytes = static_cast<uint32_t>(dv * DK * 2);
  const rsrc_t rds = make_rsrc(static_cast<char*>(p.dstates) + sq.rec0 * sbytes, static_cast<uint32_t>(nch * sbytes));
  T* sP = reinterpret_cast<T*>(smem + L::O_P);

  f32x4 dS[DKT];   // dS[t][s] = dS[16t + 4lg + s][scol]
#pragma unroll
  for (int t = 0; t < DKT; ++t)
#pragma unroll
    for (int s = 0; s < 4; ++s) dS[t][s] = p.dS_T ? p.dS_T[(bh * DK + 16 * t + 4 * lg + s) * dv + scol] : 0.f;

  SeqStage<DK, 256, true, CHAN, WK> st;
  if (nch > 0) {
    st.load(rk, rq, rdo, rw, rkw, nch - 1, tid, H, dv, col0);
    st.store(smem, tid);
  }
  __syncthreads();
  if (nch > 1) st.load(rk, rq, rdo, rw, rkw, nch - 2, tid, H, dv, col0);
  for (int64_t n = nch - 1; n >= 0; --n) {
    const char* cur = smem;
    const T* sK = reinterpret_cast<const T*>(cur + L::O_K);
    const T* sQ = reinterpret_cast<const T*>(cur + L::O_Q);
    const T* sO = reinterpret_cast<const T*>(cur + L::O_V);
    const T* sT = reinterpret_cast<const T*>(cur + L::O_T);
    const T* sKD = reinterpret_cast<const T*>(cur + (CHAN || WK ? L::O_KD : L::O_K));   // rows of dDelta's K
    const float* sF = reinterpret_cast<const float*>(cur + L::O_F);
    // P of this chunk, blocks u = wave, wave + 4, .. (row form: row 16R + lr); the
    // per-channel gate's P came with the tiles
    for (int u = wave; u < (CHAN ? 0 : 10); u += 4) {
      int R, J;
      tri_block(u, R, J);
      f32x4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int kb = 0; kb < DK / 32; ++kb)
        acc = O::mma2(acc, rowf(sKD, LDK, 16 * J, 32 * kb, lr, lg), rowf(sKD, LDK, 16 * J, 32 * kb + 16, lr, lg),
                      rowf(sQ, LDK, 16 * R, 32 * kb, lr, lg), rowf(sQ, LDK, 16 * R, 32 * kb + 16, lr, lg));
      const int r = 16 * R + lr;
#pragma unroll
      for (int s = 0; s < 4; ++s) {
        const int j = 16 * J + 4 * lg + s;
        float x = j <= r ? acc[s] : 0.f;
        if constexpr (GATE == GATE_SCALAR) x *= __expf(fminf(sF[5 * CH + r] - sF[5 * CH + j], 0.f));
        acc[s] = x;
      }
      st_row(sP, LCP, r, 16 * J + 4 * lg, acc);
    }
    __syncthreads();

    const uint32_t so = static_cast<uint32_t>(n) * sbytes;
#pragma unroll
    for (int t = 0; t < DKT; ++t) buf_store8(bits8(dS[t]), rds, chunk_state_off(16 * t + 4 * lg, scol, dv), so);

    frag dSb[DKT];
#pragma unroll
    for (int t = 0; t < DKT; ++t) dSb[t] = O::cvt(dS[t]);
    frag dOf[4], dOg[4];
#pragma unroll
    for (int kb = 0; kb < 4; ++kb) {
      dOf[kb] = colf(sO, LDV, 16 * kb, 16 * wave, lr, lg);
      if constexpr (GATE == GATE_SCALAR) {
        f32x4 x = O::f32(dOf[kb]);
#pragma unroll
        for (int s = 0; s < 4; ++s) x[s] *= sF[2 * CH + 16 * kb + 4 * lg + s];
        dOg[kb] = O::cvt(x);
      } else {
        dOg[kb] = dOf[kb];
      }
    }
    frag dDb[4];
#pragma unroll
    for (int M = 0; M < 4; ++M) {        // dDelta = diag(e^{g_63 - g}) K dS' + P^T dO
      f32x4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int kb = 0; kb < DK / 32; ++kb)
        acc = O::mma2(acc, rowf(sKD, LDK, 16 * M, 32 * kb, lr, lg), rowf(sKD, LDK, 16 * M, 32 * kb + 16, lr, lg),
                      dSb[2 * kb], dSb[2 * kb + 1]);
      if constexpr (GATE == GATE_SCALAR) {
#pragma unroll
        for (int s = 0; s < 4; ++s) acc[s] *= sF[3 * CH + 16 * M + 4 * lg + s];
      }
      int kb = M;
#pragma unroll
      for (; kb + 1 <= 3; kb += 2)
        acc = O::mma2(acc, colf(sP, LCP, 16 * kb, 16 * M, lr, lg), colf(sP, LCP, 16 * (kb + 1), 16 * M, lr, lg),
                      dOf[kb], dOf[kb + 1]);
      if (kb <= 3) acc = O::mma1(acc, colf(sP, LCP, 16 * kb, 16 * M, lr, lg), dOf[kb]);
      dDb[M] = O::cvt(acc);
    }
    frag Zb[4];
#pragma unroll
    for (int M = 0; M < 4; ++M) {        // dY = T^T dDelta; Z = -diag(beta e^g) dY
      f32x4 acc = {0.f, 0.f, 0.f, 0.f};
      int kb = M;
#pragma unroll
      for (; kb + 1 <= 3; kb += 2)
        acc = O::mma2(acc, rowf(sT, LCT, 16 * M, 16 * kb, lr, lg), rowf(sT, LCT, 16 * M, 16 * (kb + 1), lr, lg),
                      dDb[kb], dDb[kb + 1]);
      if (kb <= 3) acc = O::mma1(acc, rowf(sT, LCT, 16 * M, 16 * kb, lr, lg), dDb[kb]);
#pragma unroll
      for (int s = 0; s < 4; ++s) {
        const int r = 16 * M + 4 * lg + s;
        acc[s] *= -(GATE == GATE_SCALAR ? sF[r] * sF[CH + r] : sF[r]);
      }
      Zb[M] = O::cvt(acc);
    }
#pragma unroll
    for (int t = 0; t < DKT; ++t) {      // dS = e^{g_63} dS' + Q^T diag(e^g) dO + K^T Z
      f32x4 acc = dS[t];
      if constexpr (GATE == GATE_SCALAR) acc = acc * sF[4 * CH];
      if constexpr (CHAN) {
#pragma unroll
        for (int s = 0; s < 4; ++s) acc[s] *= sF[CH + 16 * t + 4 * lg + s];
      }
      acc = O::mma2(acc, colf(sQ, LDK, 0, 16 * t, lr, lg), colf(sQ, LDK, 16, 16 * t, lr, lg), dOg[0], dOg[1]);
      acc = O::mma2(acc, colf(sQ, LDK, 32, 16 * t, lr, lg), colf(sQ, LDK, 48, 16 * t, lr, lg), dOg[2], dOg[3]);
      acc = O::mma2(acc, colf(sK, LDK, 0, 16 * t, lr, lg), colf(sK, LDK, 16, 16 * t, lr, lg), Zb[0], Zb[1]);
      acc = O::mma2(acc, colf(sK, LDK, 32, 16 * t, lr, lg), colf(sK, LDK, 48, 16 * t, lr, lg), Zb[2], Zb[3]);
      dS[t] = acc;
    }
    __syncthreads();                    // this chunk's tiles and P are read
    if (n >= 1) {
      st.store(smem, tid);              // chunk n - 1, loaded during this step
      if (n >= 2) st.load(rk, rq, rdo, rw, rkw, n - 2, tid, H, dv, col0);
      __syncthreads();
    }
  }
  if (p.dS0) {
#pragma unroll
    for (int t = 0; t < DKT; ++t)
#pragma unroll
      for (int s = 0; s < 4; ++s) p.dS0[(bh * DK + 16 * t + 4 * lg + s) * dv + scol] = dS[t][s];
  }
}

// Passes 1 and 2 in one launch of 2 nseq workgroups: the first nseq take pass 1
// (mode 0); nseq workgroups of pass 1 alone (mode 1) or of pass 2 alone (mode 2).
template <int GATE, int DK, bool WK>
__global__ __launch_bounds__(256) void bwd_seq_kernel(BwdParams p, int n_tiles, int nseq, int mode) {
  constexpr bool KD = GATE == GATE_CHANNEL || WK;
  __shared__ __attribute__((aligned(16))) char smem[cmax(SeqLayout<DK, false, KD>::TOTAL, SeqLayout<DK, true, KD>::TOTAL)];
  const int b = blockIdx.x;
  const int role = mode == 0 ? b >= nseq : mode == 2;
  const int idx = mode == 0 ? b - role * nseq : b;
  if (role == 0) states_pass<GATE, DK, WK>(p, n_tiles, idx, smem);
  else reverse_pass<GATE, DK, WK>(p, n_tiles, idx, smem);
}

// Pass 2 with chain and helper waves (no gate or a scalar gate, no write key): four
// chain waves keep 16 columns of dS each in MFMA accumulators, four helper waves
// stage the tiles and form P one chunk ahead, with two copies of the tiles and of P
// in LDS and two barriers per chunk.  In the step of chunk n (copy b):
//   chain   | dS' out; dDelta = diag(e^{g_63 - g}) K dS' + P^T dO; dY = T^T dDelta;
//           |   Z = -diag(beta e^g) dY
//   helpers | chunk n - 1 from registers into copy 1 - b; loads of chunk n - 2
//   ------------------------------------------------------------------- barrier
//   chain   | dS = e^{g_63} dS' + Q^T diag(e^g) dO + K^T Z
//   helpers | P of chunk n - 1 from copy 1 - b into P copy 1 - b
//   ------------------------------------------------------------------- barrier
// Copy 1 - b and P copy 1 - b were last read by the chain in the step before,
// ahead of its closing barrier.  Only dDelta -> dY -> Z -> K^T Z lies on the chain
// from chunk to chunk; P, the staging and Q^T dO are off it or beside it.
template <int GATE, int DK>
struct RevPipeLayout {
  typedef SeqLayout<DK, true, false> S;   // one copy of the tiles (k, q, dO, T^T, factors) and P
  static constexpr size_t BUF = S::BUF;
  static constexpr size_t PB = size_t(CH) * S::LCP * 2;
  static constexpr size_t O_P = 2 * BUF;
  static constexpr size_t TOTAL = O_P + 2 * PB;
};

template <int GATE, int DK>
__global__ __launch_bounds__(512) void bwd_rev_pipe_kernel(BwdParams p, int n_tiles) {
  static_assert(GATE == GATE_NONE || GATE == GATE_SCALAR, "chain/helper reverse pass: no gate or a scalar gate");
  typedef SeqLayout<DK, true, false> S;
  typedef RevPipeLayout<GATE, DK> L;
  static_assert(L::TOTAL <= 163840, "LDS budget");
  constexpr uint32_t RB = rec_bytes(IO_BF16, GATE, DK);
  constexpr int DKT = DK / 16, LDK = S::LDK, LDV = S::LDV, LCT = S::LCT, LCP = S::LCP;
  __shared__ __attribute__((aligned(16))) char smem[L::TOTAL];
  const ChunkParams& f = p.f;
  const int lb = blockIdx.x;
  const int64_t bh = lb / n_tiles;
  const int tile = lb % n_tiles;
  const int64_t bb = bh / f.H, hh = bh % f.H;
  const int dv = f.d_v, H = static_cast<int>(f.H), col0 = tile * 64;
  const int tid = threadIdx.x;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const bool chain = wave < 4;
  const int lane = tid & 63, lr = lane & 15, lg = lane >> 4;
  const BwdSeq sq = bwd_seq_of(f, bb, hh);
  const int64_t nch = sq.nch;
  const Slice sl = sq.sl;
  const rsrc_t rk = sl.rs(f.k, DK), rq = sl.rs(f.q, DK), rdo = sl.rs(p.dO, dv);
  const rsrc_t rw = make_rsrc(static_cast<const char*>(f.ws) + sq.rec0 * RB, static_cast<uint32_t>(nch * RB));
  auto buf = [&](int64_t i) -> char* { return smem + (i & 1) * L::BUF; };
  auto pbuf = [&](int64_t i) -> T* { return reinterpret_cast<T*>(smem + L::O_P + (i & 1) * L::PB); };

  if (chain) {
    const int scol = col0 + 16 * wave + lr;
    const uint32_t sbytes = static_cast<uint32_t>(dv * DK * 2);
    const rsrc_t rds = make_rsrc(static_cast<char*>(p.dstates) + sq.rec0 * sbytes, static_cast<uint32_t>(nch * sbytes));
    f32x4 dS[DKT];   // dS[t][s] = dS[16t + 4lg + s][scol]
#pragma unroll
    for (int t = 0; t < DKT; ++t)
#pragma unroll
      for (int s = 0; s < 4; ++s) dS[t][s] = p.dS_T ? p.dS_T[(bh * DK + 16 * t + 4 * lg + s) * dv + scol] : 0.f;
    __syncthreads();                    // the last chunk's tiles in copy 0
    __syncthreads();                    // its P
    for (int64_t n = nch - 1; n >= 0; --n) {
      const int64_t i = nch - 1 - n;    // step index: the copy in use
      const char* cur = buf(i);
      const T* sK = reinterpret_cast<const T*>(cur + S::O_K);
      const T* sQ = reinterpret_cast<const T*>(cur + S::O_Q);
      const T* sO = reinterpret_cast<const T*>(cur + S::O_V);
      const T* sT = reinterpret_cast<const T*>(cur + S::O_T);
      const float* sF = reinterpret_cast<const float*>(cur + S::O_F);
      const T* sP = pbuf(i);

      const uint32_t so = static_cast<uint32_t>(n) * sbytes;
#pragma unroll
      for (int t = 0; t < DKT; ++t) buf_store8(bits8(dS[t]), rds, chunk_state_off(16 * t + 4 * lg, scol, dv), so);
      frag dSb[DKT];
#pragma unroll
      for (int t = 0; t < DKT; ++t) dSb[t] = O::cvt(dS[t]);
      frag dOf[4];
#pragma unroll
      for (int kb = 0; kb < 4; ++kb) dOf[kb] = colf(sO, LDV, 16 * kb, 16 * wave, lr, lg);
      // The products below read their LDS fragments one row block (or state tile) ahead,
      // and scheduling fences keep the compiler from sinking those reads to their use.
      frag kf[2][DK / 16], pf[2][4];    // rows of K of block M, columns of P^T of block M
      auto load_d = [&](int b, int M) __attribute__((always_inline)) {
#pragma unroll
        for (int kb = 0; kb < DK / 32; ++kb) {
          kf[b][2 * kb] = rowf(sK, LDK, 16 * M, 32 * kb, lr, lg);
          kf[b][2 * kb + 1] = rowf(sK, LDK, 16 * M, 32 * kb + 16, lr, lg);
        }
#pragma unroll
        for (int kb = 0; kb < 4; ++kb)
          if (kb >= M) pf[b][kb] = colf(sP, LCP, 16 * kb, 16 * M, lr, lg);
      };
      load_d(0, 0);
      frag dDb[4];
#pragma unroll
      for (int M = 0; M < 4; ++M) {     // dDelta = diag(e^{g_63 - g}) K dS' + P^T dO
        __builtin_amdgcn_sched_barrier(0);
        if (M < 3) load_d((M + 1) & 1, M + 1);
        __builtin_amdgcn_sched_barrier(0);
        f32x4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int kb = 0; kb < DK / 32; ++kb)
          acc = O::mma2(acc, kf[M & 1][2 * kb], kf[M & 1][2 * kb + 1], dSb[2 * kb], dSb[2 * kb + 1]);
        if constexpr (GATE == GATE_SCALAR) {
#pragma unroll
          for (int s = 0; s < 4; ++s) acc[s] *= sF[3 * CH + 16 * M + 4 * lg + s];
        }
        int kb = M;
#pragma unroll
        for (; kb + 1 <= 3; kb += 2) acc = O::mma2(acc, pf[M & 1][kb], pf[M & 1][kb + 1], dOf[kb], dOf[kb + 1]);
        if (kb <= 3) acc = O::mma1(acc, pf[M & 1][kb], dOf[kb]);
        dDb[M] = O::cvt(acc);
      }
      frag Zb[4];
#pragma unroll
      for (int M = 0; M < 4; ++M) {     // dY = T^T dDelta; Z = -diag(beta e^g) dY
        f32x4 acc = {0.f, 0.f, 0.f, 0.f};
        int kb = M;
#pragma unroll
        for (; kb + 1 <= 3; kb += 2)
          acc = O::mma2(acc, rowf(sT, LCT, 16 * M, 16 * kb, lr, lg), rowf(sT, LCT, 16 * M, 16 * (kb + 1), lr, lg),
                        dDb[kb], dDb[kb + 1]);
        if (kb <= 3) acc = O::mma1(acc, rowf(sT, LCT, 16 * M, 16 * kb, lr, lg), dDb[kb]);
#pragma unroll
        for (int s = 0; s < 4; ++s) {
          const int r = 16 * M + 4 * lg + s;
          acc[s] *= -(GATE == GATE_SCALAR ? sF[r] * sF[CH + r] : sF[r]);
        }
        Zb[M] = O::cvt(acc);
      }
      __syncthreads();                  // the helpers' copy of chunk n - 1 in place
      frag dOg[4];
#pragma unroll
      for (int kb = 0; kb < 4; ++kb) {
        if constexpr (GATE == GATE_SCALAR) {
          f32x4 x = O::f32(dOf[kb]);
#pragma unroll
          for (int s = 0; s < 4; ++s) x[s] *= sF[2 * CH + 16 * kb + 4 * lg + s];
          dOg[kb] = O::cvt(x);
        } else {
          dOg[kb] = dOf[kb];
        }
      }
      frag uf[2][8];                    // columns of Q^T and K^T of state tile t
      auto load_u = [&](int b, int t) __attribute__((always_inline)) {
#pragma unroll
        for (int m = 0; m < 4; ++m) {
          uf[b][m] = colf(sQ, LDK, 16 * m, 16 * t, lr, lg);
          uf[b][4 + m] = colf(sK, LDK, 16 * m, 16 * t, lr, lg);
        }
      };
      const float gam = GATE == GATE_SCALAR ? sF[4 * CH] : 1.f;
      load_u(0, 0);
#pragma unroll
      for (int t = 0; t < DKT; ++t) {   // dS = e^{g_63} dS' + Q^T diag(e^g) dO + K^T Z
        __builtin_amdgcn_sched_barrier(0);
        if (t + 1 < DKT) load_u((t + 1) & 1, t + 1);
        __builtin_amdgcn_sched_barrier(0);
        f32x4 acc = dS[t];
        if constexpr (GATE == GATE_SCALAR) acc = acc * gam;
        acc = O::mma2(acc, uf[t & 1][0], uf[t & 1][1], dOg[0], dOg[1]);
        acc = O::mma2(acc, uf[t & 1][2], uf[t & 1][3], dOg[2], dOg[3]);
        acc = O::mma2(acc, uf[t & 1][4], uf[t & 1][5], Zb[0], Zb[1]);
        acc = O::mma2(acc, uf[t & 1][6], uf[t & 1][7], Zb[2], Zb[3]);
        dS[t] = acc;
      }
      __builtin_amdgcn_sched_barrier(0);
      __syncthreads();                  // P of chunk n - 1 in place; this chunk's copies read
    }
    if (p.dS0) {
#pragma unroll
      for (int t = 0; t < DKT; ++t)
#pragma unroll
        for (int s = 0; s < 4; ++s) p.dS0[(bh * DK + 16 * t + 4 * lg + s) * dv + scol] = dS[t][s];
    }
  } else {
    const int ht = tid - 256, hw = wave - 4;
    SeqStage<DK, 256, true, false, false> st;
    // P of one chunk from its copy: blocks u = hw, hw + 4, .. (row form: row 16R + lr)
    auto form_p = [&](const char* c, T* sP) __attribute__((always_inline)) {
      const T* sK = reinterpret_cast<const T*>(c + S::O_K);
      const T* sQ = reinterpret_cast<const T*>(c + S::O_Q);
      const float* sF = reinterpret_cast<const float*>(c + S::O_F);
      for (int u = hw; u < 10; u += 4) {
        int R, J;
        tri_block(u, R, J);
        f32x4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int kb = 0; kb < DK / 32; ++kb)
          acc = O::mma2(acc, rowf(sK, LDK, 16 * J, 32 * kb, lr, lg), rowf(sK, LDK, 16 * J, 32 * kb + 16, lr, lg),
                        rowf(sQ, LDK, 16 * R, 32 * kb, lr, lg), rowf(sQ, LDK, 16 * R, 32 * kb + 16, lr, lg));
        const int r = 16 * R + lr;
#pragma unroll
        for (int s = 0; s < 4; ++s) {
          const int j = 16 * J + 4 * lg + s;
          float x = j <= r ? acc[s] : 0.f;
          if constexpr (GATE == GATE_SCALAR) x *= __expf(fminf(sF[5 * CH + r] - sF[5 * CH + j], 0.f));
          acc[s] = x;
        }
        st_row(sP, LCP, r, 16 * J + 4 * lg, acc);
      }
    };
    if (nch > 0) {
      st.load(rk, rq, rdo, rw, rk, nch - 1, ht, H, dv, col0);
      st.store(buf(0), ht);
      if (nch > 1) st.load(rk, rq, rdo, rw, rk, nch - 2, ht, H, dv, col0);
    }
    __syncthreads();                    // the last chunk's tiles in copy 0
    if (nch > 0) form_p(buf(0), pbuf(0));
    __syncthreads();                    // its P
    for (int64_t n = nch - 1; n >= 0; --n) {
      const int64_t i = nch - 1 - n;
      if (n >= 1) {
        st.store(buf(i + 1), ht);       // chunk n - 1 into the other copy
        if (n >= 2) st.load(rk, rq, rdo, rw, rk, n - 2, ht, H, dv, col0);
      }
      __syncthreads();                  // chunk n - 1 in place
      if (n >= 1) form_p(buf(i + 1), pbuf(i + 1));
      __syncthreads();                  // its P in place
    }
  }
}

// ---------------------------------------------------------------------------
// Pass 3: one workgroup of eight waves per chunk.  The d_v columns are taken in
// halves of 64 (the products over d_v accumulate across them).
// ---------------------------------------------------------------------------
// Every tile here is read both ways except dDelta (transposed only), Delta and dY
// (rows only).  With a write key (WK) its tile KW sits beside k; to make room,
// beta D * dA and the partial sums, which are only written after the d_v loop, take
// the place of dDelta, Delta and dY, which are only read inside it.
template <int DK, bool WK = false>
struct ChunkLayout {
  static constexpr int LDK = ld_both(DK);   // q, k, and the value-major states S^T, dS'^T
  static constexpr int LDV = ld_both(64);   // 64-column tiles: v then diag(beta) X, dO
  static constexpr int LDD = ld_tr(64);     // dDelta
  static constexpr int LDR = ld_row(64);    // Delta, dY
  static constexpr int LCP = ld_both(CH);   // 64 x 64 matrices
  static constexpr size_t KB = size_t(CH) * LDK * 2;
  static constexpr size_t VB = size_t(CH) * LDV * 2;
  static constexpr size_t CB = size_t(CH) * LCP * 2;
  static constexpr size_t O_Q = 0, O_K = O_Q + KB, O_KW = O_K + KB, O_T = O_KW + (WK ? KB : 0), O_F = O_T + CB;
  static constexpr size_t O_P = O_F + 6 * CH * 4;    // P, then D * dP
  static constexpr size_t O_AK0 = O_P + CB;          // beta D * dA (without a write key)
  static constexpr size_t O_V = O_AK0 + (WK ? 0 : CB);   // v half, then diag(beta) X
  static constexpr size_t O_DO = O_V + VB;
  static constexpr size_t O_DD = O_DO + VB;          // dDelta
  static constexpr size_t O_DL = O_DD + size_t(CH) * LDD * 2;   // Delta
  static constexpr size_t O_DY = O_DL + size_t(CH) * LDR * 2;   // dY
  static constexpr size_t O_S = O_DY + size_t(CH) * LDR * 2;    // S^T half [64][DK]
  static constexpr size_t O_DS = O_S + KB;           // dS'^T half
  // Partial row sums, each written by one wave and added in a fixed order (no
  // atomics, so the result does not depend on the order the waves run in):
  // dbeta over d_v tiles [4][64] and over column blocks [4][64]; dg row sums of the
  // A and of the P terms [4][64] each, column sums [4][64], and the row dots over
  // d_k tiles [DK / 16][64] twice (the terms of g_read and those of g); two per-wave
  // scalars [8] x 2.
  static constexpr size_t NRED = (4 + 4 + 4 + 4 + 4 + 2 * (DK / 16)) * CH + 16;
  static constexpr size_t O_AK = WK ? O_DD : O_AK0;
  static constexpr size_t O_RED = WK ? O_AK + CB : O_DS + KB;
  static constexpr size_t TOTAL = WK ? O_DS + KB : O_RED + NRED * 4;
  static_assert(!WK || O_RED + NRED * 4 <= O_S, "the post-loop tiles fit in the loop-only ones");
};

// One workgroup per chunk (the LDS admits one per compute unit).  With a write key
// (WK) the column side of the Gram and score blocks, dDelta's key product and the
// state write take KW, and the gradient of k splits into its read side (dk) and its
// write side (dkw):
//   dk  = (beta D * dA) KW - diag(beta e^{g_read}) dY S^T,
//   dkw = (beta D * dA)^T K + (D * dP)^T Q + diag(e^{g_63 - g}) Delta dS'^T,
//   dq  = (D * dP) KW + diag(e^g) dO S^T,
// and the chunk-end row dot c_r takes kw_r.
template <int GATE, int DK, int DV, bool WK>
__global__ __launch_bounds__(512) void bwd_chunk_kernel(BwdParams p) {
  typedef ChunkLayout<DK, WK> L;
  constexpr int NT = 512, NW = 8;
  constexpr int DKT = DK / 16, LDK = L::LDK, LDV = L::LDV, LDD = L::LDD, LDR = L::LDR, LCP = L::LCP;
  constexpr int KR = DK / 8, KP = CH * KR / NT;     // pieces of a [64][DK] tile per thread
  constexpr int NHALF = DV / 64;
  static_assert(KP * NT == CH * KR, "tile pieces split evenly");
  static_assert(L::TOTAL <= 163840, "LDS budget");
  constexpr bool G = GATE == GATE_SCALAR;
  __shared__ __attribute__((aligned(16))) char smem[L::TOTAL];
  T* sQ = reinterpret_cast<T*>(smem + L::O_Q);
  T* sK = reinterpret_cast<T*>(smem + L::O_K);
  T* sKW = reinterpret_cast<T*>(smem + (WK ? L::O_KW : L::O_K));   // the column-side key
  T* sT = reinterpret_cast<T*>(smem + L::O_T);
  const float* sF = reinterpret_cast<const float*>(smem + L::O_F);
  T* sP = reinterpret_cast<T*>(smem + L::O_P);
  T* sAk = reinterpret_cast<T*>(smem + L::O_AK);
  T* sV = reinterpret_cast<T*>(smem + L::O_V);
  T* sdO = reinterpret_cast<T*>(smem + L::O_DO);
  T* sdD = reinterpret_cast<T*>(smem + L::O_DD);
  T* sDl = reinterpret_cast<T*>(smem + L::O_DL);
  T* sdY = reinterpret_cast<T*>(smem + L::O_DY);
  T* sS = reinterpret_cast<T*>(smem + L::O_S);
  T* sdS = reinterpret_cast<T*>(smem + L::O_DS);
  float* rbX = reinterpret_cast<float*>(smem + L::O_RED);   // dbeta: [c][r], sum_v dY X of d_v tile c
  float* rbA = rbX + 4 * CH;            // dbeta: [J][r], the dA term of column block J
  float* rgA = rbA + 4 * CH;            // dg (g_read): [J][r], row sums of dA*A over column block J
  float* rgP = rgA + 4 * CH;            // dg: [J][r], row sums of dP*P over column block J
  float* rgC = rgP + 4 * CH;            // dg: [R][j], column sums of dA*A + dP*P over row block R
  float* rgK = rgC + 4 * CH;            // dg: [ic][r], the q and Delta dS'^T row dots over d_k tile ic
  float* rgX = rgK + (DK / 16) * CH;    // dg (g_read): [ic][r], the dY S^T row dot over d_k tile ic
  float* rcs = rgX + (DK / 16) * CH;    // [wave]: sum_r c_r
  float* rsd = rcs + 8;                 // [wave]: <dS', S>

  const ChunkParams& f = p.f;
  const int H = static_cast<int>(f.H);
  const int tid = threadIdx.x;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int lane = tid & 63, lr = lane & 15, lg = lane >> 4;
  constexpr uint32_t SBYTES = DV * DK * 2;          // one chunk's state

  // The workgroup's chunk: tasks as for the per-chunk transform (head fastest);
  // with packed sequences a slot past its sequence's end has no chunk.
  int64_t bb, n, hh;
  if (!prep_task(f, blockIdx.x, bb, n, hh)) return;
  const BwdSeq sq = bwd_seq_of(f, bb, hh);
  const int64_t nch = sq.nch;
  const Slice sl = sq.sl;
  {
    // q, k, the T blocks and the factor rows of the chunk
    u32x4 hq[KP], hk[KP], hkw[WK ? KP : 1], ht, hf;
    {
      const rsrc_t rq = sl.rs(f.q, DK), rk = sl.rs(f.k, DK), rkw = WK ? sl.rs(f.kw, DK) : rk;
      const rsrc_t rw = make_rsrc(static_cast<const char*>(f.ws) + sq.rec0 * W::BYTES, static_cast<uint32_t>(nch * W::BYTES));
      const uint32_t sk = static_cast<uint32_t>(n * CH * H * DK * 2), sw = static_cast<uint32_t>(n * W::BYTES);
#pragma unroll
      for (int i = 0; i < KP; ++i) {
        const int pc = tid + i * NT;
        const uint32_t off = static_cast<uint32_t>(((pc / KR) * H * DK + (pc % KR) * 8) * 2);
        hq[i] = buf_load16(rq, off, sk);
        hk[i] = buf_load16(rk, off, sk);
        if constexpr (WK) hkw[i] = buf_load16(rkw, off, sk);
      }
      if (tid < 320) ht = buf_load16(rw, W::T_OFF + static_cast<uint32_t>(tid * 16), sw);
      if (tid < 96) hf = buf_load16(rw, W::F_OFF + static_cast<uint32_t>(tid * 16), sw);
    }
    const rsrc_t rv = sl.rs(f.v, DV), rdo = sl.rs(p.dO, DV);
    const rsrc_t rdq = sl.rs(p.dq, DK), rdk = sl.rs(p.dk, DK), rdv = sl.rs(p.dv, DV);
    const rsrc_t rdkw = WK ? sl.rs(p.dkw, DK) : rdk;
    const rsrc_t rdb = sl.rs(p.dbeta, 1), rdl = sl.rs(p.dlog_a, G ? 1 : 0);
    const rsrc_t rst = make_rsrc(static_cast<const char*>(p.states) + sq.rec0 * SBYTES, static_cast<uint32_t>(nch * SBYTES));
    const rsrc_t rds = make_rsrc(static_cast<const char*>(p.dstates) + sq.rec0 * SBYTES, static_cast<uint32_t>(nch * SBYTES));
    const uint32_t sk = static_cast<uint32_t>(n * CH * H * DK * 2);   // chunk start in q, k (bytes)
    const uint32_t sv = static_cast<uint32_t>(n * CH * H * DV * 2);   // ... in v, dO
    const uint32_t ss = static_cast<uint32_t>(n) * SBYTES;
    const uint32_t sb = static_cast<uint32_t>(n * CH * H * 2);        // ... in beta, log a

    // one d_v half of v, dO, S^T, dS'^T
    u32x4 hv, hdo, hs[KP], hds[KP];
    float sdot = 0.f;                   // this thread's part of <dS', S>
    auto load_half = [&](int h) __attribute__((always_inline)) {
      hv = buf_load16(rv, static_cast<uint32_t>(((tid / 8) * H * DV + 64 * h + (tid % 8) * 8) * 2), sv);
      hdo = buf_load16(rdo, static_cast<uint32_t>(((tid / 8) * H * DV + 64 * h + (tid % 8) * 8) * 2), sv);
#pragma unroll
      for (int i = 0; i < KP; ++i) {   // piece pc: column 64 h + pc / KR of S, d_k values 8 (pc % KR) ..
        const int pc = tid + i * NT;
        const uint32_t off = chunk_state_off(8 * (pc % KR), 64 * h + pc / KR, DV);
        hs[i] = buf_load16(rst, off, ss);
        hds[i] = buf_load16(rds, off, ss);
      }
    };
    auto store_half = [&]() __attribute__((always_inline)) {
      put16(sV + (tid / 8) * LDV + (tid % 8) * 8, hv);
      put16(sdO + (tid / 8) * LDV + (tid % 8) * 8, hdo);
#pragma unroll
      for (int i = 0; i < KP; ++i) {
        const int pc = tid + i * NT;
        put16(sS + (pc / KR) * LDK + (pc % KR) * 8, hs[i]);
        put16(sdS + (pc / KR) * LDK + (pc % KR) * 8, hds[i]);
        if constexpr (G) {
#pragma unroll
          for (int j = 0; j < 4; ++j) {
            const uint32_t a = hs[i][j], b = hds[i][j];
            sdot += bf16_bits_to_f32(a & 0xffffu) * bf16_bits_to_f32(b & 0xffffu) +
                    bf16_bits_to_f32(a >> 16) * bf16_bits_to_f32(b >> 16);
          }
        }
      }
    };

    // ---- q, k, T, factors into LDS; the first d_v half is loaded meanwhile ----------
#pragma unroll
    for (int i = 0; i < KP; ++i) {
      const int pc = tid + i * NT;
      put16(sQ + (pc / KR) * LDK + (pc % KR) * 8, hq[i]);
      put16(sK + (pc / KR) * LDK + (pc % KR) * 8, hk[i]);
      if constexpr (WK) put16(sKW + (pc / KR) * LDK + (pc % KR) * 8, hkw[i]);
    }
    if (tid < 320) {
      int R, J;
      tri_block(tid / 32, R, J);
      const int a = (tid % 32) / 2, b0 = (tid % 2) * 8;
      put16(sT + (16 * J + a) * LCP + 16 * R + b0, ht);
    }
    if (tid < 96) *reinterpret_cast<u32x4*>(smem + L::O_F + tid * 16) = hf;
    load_half(0);
    __syncthreads();

    // ---- the wave's blocks of the 64 x 64 matrices: u = wave, wave + 8 (< 10) -------
    constexpr int NU = 2;
    f32x4 Gr[NU], QKr[NU], dAa[NU], dPa[NU];
#pragma unroll
    for (int i = 0; i < NU; ++i) {
      const int u = wave + NW * i;
      Gr[i] = QKr[i] = dAa[i] = dPa[i] = f32x4{0.f, 0.f, 0.f, 0.f};
      if (u < 10) {
        int R, J;
        tri_block(u, R, J);
#pragma unroll
        for (int kb = 0; kb < DK / 32; ++kb) {
          const frag b0 = rowf(sKW, LDK, 16 * J, 32 * kb, lr, lg), b1 = rowf(sKW, LDK, 16 * J, 32 * kb + 16, lr, lg);
          Gr[i] = O::mma2(Gr[i], b0, b1, rowf(sK, LDK, 16 * R, 32 * kb, lr, lg), rowf(sK, LDK, 16 * R, 32 * kb + 16, lr, lg));
          QKr[i] = O::mma2(QKr[i], b0, b1, rowf(sQ, LDK, 16 * R, 32 * kb, lr, lg), rowf(sQ, LDK, 16 * R, 32 * kb + 16, lr, lg));
        }
        const int r = 16 * R + lr;
        f32x4 pv;
#pragma unroll
        for (int s = 0; s < 4; ++s) {
          const int j = 16 * J + 4 * lg + s;
          float x = j <= r ? QKr[i][s] : 0.f;
          if constexpr (G) x *= __expf(fminf(sF[5 * CH + r] - sF[5 * CH + j], 0.f));
          pv[s] = x;
        }
        st_row(sP, LCP, r, 16 * J + 4 * lg, pv);
      }
    }
    store_half();                       // the first d_v half, loaded during the products above
    __syncthreads();
    if constexpr (NHALF > 1) load_half(1);

    // ---- per d_v half -------------------------------------------------------------------
    // 64 x d_k tiles: wave w owns row blocks M = 2 (w / 4) + mi (mi = 0, 1) and column
    // blocks ic = IC (w % 4) + j (j < IC), so fragments are shared along both
    constexpr int IC = DKT / 4, NX = 2 * IC;
    const int Mb = 2 * (wave >> 2), Ib = IC * (wave & 3);
    f32x4 dYS[NX], dOS[NX], DdS[NX];
#pragma unroll
    for (int i = 0; i < NX; ++i) dYS[i] = dOS[i] = DdS[i] = f32x4{0.f, 0.f, 0.f, 0.f};
    float dbx[2] = {0.f, 0.f};          // sum_v dY X for rows 16 M_i + lr
#pragma unroll
    for (int h = 0; h < NHALF; ++h) {
      if (h > 0) {
        store_half();
        __syncthreads();
      }
      // X = V - diag(e^g) K S (kept), diag(beta) X over the v tile;
      // dDelta = diag(e^{g_63 - g}) K dS' + P^T dO.  The wave's tiles (M, c) =
      // (wave / 4 + 2 i, wave % 4), i = 0, 1, share the column c.
      f32x4 Xr[2], KS2[2], KD2[2];
      {
        const int c = wave & 3;
#pragma unroll
        for (int i = 0; i < 2; ++i) KS2[i] = KD2[i] = f32x4{0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int kb = 0; kb < DK / 32; ++kb) {
          const frag s0 = rowf(sS, LDK, 16 * c, 32 * kb, lr, lg), s1 = rowf(sS, LDK, 16 * c, 32 * kb + 16, lr, lg);
          const frag d0 = rowf(sdS, LDK, 16 * c, 32 * kb, lr, lg), d1 = rowf(sdS, LDK, 16 * c, 32 * kb + 16, lr, lg);
#pragma unroll
          for (int i = 0; i < 2; ++i) {
            const int M = (wave >> 2) + 2 * i;
            const frag a0 = rowf(sK, LDK, 16 * M, 32 * kb, lr, lg), a1 = rowf(sK, LDK, 16 * M, 32 * kb + 16, lr, lg);
            KS2[i] = O::mma2(KS2[i], s0, s1, a0, a1);
            if constexpr (WK)
              KD2[i] = O::mma2(KD2[i], d0, d1, rowf(sKW, LDK, 16 * M, 32 * kb, lr, lg),
                               rowf(sKW, LDK, 16 * M, 32 * kb + 16, lr, lg));
            else
              KD2[i] = O::mma2(KD2[i], d0, d1, a0, a1);
          }
        }
      }
#pragma unroll
      for (int i = 0; i < 2; ++i) {
        const int t = wave + NW * i, M = t >> 2, c = t & 3;
        const int r = 16 * M + lr;
        const f32x4 ks = KS2[i];
        f32x4 kd = KD2[i];
        const f32x4 vv = O::f32(O::ld(sV + r * LDV + 16 * c + 4 * lg));
        const float er = G ? sF[CH + r] : 1.f;
        Xr[i] = vv - ks * er;
        st_row(sV, LDV, r, 16 * c + 4 * lg, Xr[i] * sF[r]);
        if constexpr (G) kd = kd * sF[3 * CH + r];
        int kb = M;
        for (; kb + 1 <= 3; kb += 2)
          kd = O::mma2(kd, colf(sdO, LDV, 16 * kb, 16 * c, lr, lg), colf(sdO, LDV, 16 * (kb + 1), 16 * c, lr, lg),
                       colf(sP, LCP, 16 * kb, 16 * M, lr, lg), colf(sP, LCP, 16 * (kb + 1), 16 * M, lr, lg));
        if (kb <= 3) kd = O::mma1(kd, colf(sdO, LDV, 16 * kb, 16 * c, lr, lg), colf(sP, LCP, 16 * kb, 16 * M, lr, lg));
        st_row(sdD, LDD, r, 16 * c + 4 * lg, kd);
      }
      __syncthreads();
      // Delta = T diag(beta) X, dY = T^T dDelta; dv = diag(beta) dY
#pragma unroll
      for (int i = 0; i < 2; ++i) {
        const int t = wave + NW * i, M = t >> 2, c = t & 3;
        const int r = 16 * M + lr;
        f32x4 dl = {0.f, 0.f, 0.f, 0.f}, dy = {0.f, 0.f, 0.f, 0.f};
        int kb = 0;
        for (; kb + 1 <= M; kb += 2)
          dl = O::mma2(dl, colf(sV, LDV, 16 * kb, 16 * c, lr, lg), colf(sV, LDV, 16 * (kb + 1), 16 * c, lr, lg),
                       colf(sT, LCP, 16 * kb, 16 * M, lr, lg), colf(sT, LCP, 16 * (kb + 1), 16 * M, lr, lg));
        if (kb <= M) dl = O::mma1(dl, colf(sV, LDV, 16 * kb, 16 * c, lr, lg), colf(sT, LCP, 16 * kb, 16 * M, lr, lg));
        kb = M;
        for (; kb + 1 <= 3; kb += 2)
          dy = O::mma2(dy, colf(sdD, LDD, 16 * kb, 16 * c, lr, lg), colf(sdD, LDD, 16 * (kb + 1), 16 * c, lr, lg),
                       rowf(sT, LCP, 16 * M, 16 * kb, lr, lg), rowf(sT, LCP, 16 * M, 16 * (kb + 1), lr, lg));
        if (kb <= 3) dy = O::mma1(dy, colf(sdD, LDD, 16 * kb, 16 * c, lr, lg), rowf(sT, LCP, 16 * M, 16 * kb, lr, lg));
        buf_store8(bits8(dy * sF[r]), rdv, static_cast<uint32_t>((r * H * DV + 64 * h + 16 * c + 4 * lg) * 2), sv);
#pragma unroll
        for (int s = 0; s < 4; ++s) dbx[i] += dy[s] * Xr[i][s];
        st_row(sDl, LDR, r, 16 * c + 4 * lg, dl);
        st_row(sdY, LDR, r, 16 * c + 4 * lg, dy);
      }
      __syncthreads();
      // dA += dY Delta^T, dP += dO Delta^T on the wave's blocks; dY S^T, dO S^T, Delta dS'^T
#pragma unroll
      for (int i = 0; i < NU; ++i) {
        const int u = wave + NW * i;
        if (u < 10) {
          int R, J;
          tri_block(u, R, J);
#pragma unroll
          for (int kb = 0; kb < 2; ++kb) {
            const frag b0 = rowf(sDl, LDR, 16 * J, 32 * kb, lr, lg), b1 = rowf(sDl, LDR, 16 * J, 32 * kb + 16, lr, lg);
            dAa[i] = O::mma2(dAa[i], b0, b1, rowf(sdY, LDR, 16 * R, 32 * kb, lr, lg), rowf(sdY, LDR, 16 * R, 32 * kb + 16, lr, lg));
            dPa[i] = O::mma2(dPa[i], b0, b1, rowf(sdO, LDV, 16 * R, 32 * kb, lr, lg), rowf(sdO, LDV, 16 * R, 32 * kb + 16, lr, lg));
          }
        }
      }
#pragma unroll
      for (int kb = 0; kb < 2; ++kb) {
        frag bs[IC][2], bd[IC][2];
#pragma unroll
        for (int j = 0; j < IC; ++j) {
          const int ic = Ib + j;
          bs[j][0] = colf(sS, LDK, 32 * kb, 16 * ic, lr, lg);
          bs[j][1] = colf(sS, LDK, 32 * kb + 16, 16 * ic, lr, lg);
          bd[j][0] = colf(sdS, LDK, 32 * kb, 16 * ic, lr, lg);
          bd[j][1] = colf(sdS, LDK, 32 * kb + 16, 16 * ic, lr, lg);
        }
#pragma unroll
        for (int mi = 0; mi < 2; ++mi) {
          const int M = Mb + mi;
          const frag y0 = rowf(sdY, LDR, 16 * M, 32 * kb, lr, lg), y1 = rowf(sdY, LDR, 16 * M, 32 * kb + 16, lr, lg);
          const frag o0 = rowf(sdO, LDV, 16 * M, 32 * kb, lr, lg), o1 = rowf(sdO, LDV, 16 * M, 32 * kb + 16, lr, lg);
          const frag e0 = rowf(sDl, LDR, 16 * M, 32 * kb, lr, lg), e1 = rowf(sDl, LDR, 16 * M, 32 * kb + 16, lr, lg);
#pragma unroll
          for (int j = 0; j < IC; ++j) {
            const int i = mi * IC + j;
            dYS[i] = O::mma2(dYS[i], bs[j][0], bs[j][1], y0, y1);
            dOS[i] = O::mma2(dOS[i], bs[j][0], bs[j][1], o0, o1);
            DdS[i] = O::mma2(DdS[i], bd[j][0], bd[j][1], e0, e1);
          }
        }
      }
      if (h + 1 < NHALF) __syncthreads();   // every read of this half's tiles is done
    }
    if constexpr (WK) __syncthreads();    // beta D * dA and the sums overwrite dDelta, Delta and dY

    // ---- beta D * dA and D * dP; dbeta and the row / column sums of dA*A and dP*P ------
#pragma unroll
    for (int i = 0; i < NU; ++i) {
      const int u = wave + NW * i;
      if (u < 10) {
        int R, J;
        tri_block(u, R, J);
        const int r = 16 * R + lr;
        const float br = sF[r];
        // the A factor e^{g_read_r - g_j}: g_read = g (decay before the erase) or
        // g_{r-1} (erase on the undecayed state; 0 at the chunk's first row)
        const float grd = p.f.literal ? (r > 0 ? sF[5 * CH + r - 1] : 0.f) : sF[5 * CH + r];
        f32x4 ak, pk;
        float db = 0.f, rsumA = 0.f, rsumP = 0.f;
        float csum[4];
#pragma unroll
        for (int s = 0; s < 4; ++s) {
          const int j = 16 * J + 4 * lg + s;
          const float DA = G ? __expf(fminf(grd - sF[5 * CH + j], 0.f)) : 1.f;
          const float DP = G ? __expf(fminf(sF[5 * CH + r] - sF[5 * CH + j], 0.f)) : 1.f;
          const float dA = j < r ? -dAa[i][s] : 0.f;
          const float dP = j <= r ? dPa[i][s] : 0.f;
          ak[s] = br * DA * dA;
          pk[s] = DP * dP;
          db += dA * DA * Gr[i][s];
          const float ea = ak[s] * Gr[i][s], ep = pk[s] * QKr[i][s];   // dA * A, dP * P
          rsumA += ea;
          rsumP += ep;
          csum[s] = ea + ep;
        }
        st_row(sAk, LCP, r, 16 * J + 4 * lg, ak);
        st_row(sP, LCP, r, 16 * J + 4 * lg, pk);
        db = lg_sum(db);
        if (lg == 0) rbA[J * CH + r] = db;
        if constexpr (G) {
          rsumA = lg_sum(rsumA);
          rsumP = lg_sum(rsumP);
          if (lg == 0) {
            rgA[J * CH + r] = rsumA;
            rgP[J * CH + r] = rsumP;
          }
#pragma unroll
          for (int s = 0; s < 4; ++s) {
            const float x = row16_sum(csum[s]);
            if (lr == 0) rgC[R * CH + 16 * J + 4 * lg + s] = x;
          }
        }
      }
    }
#pragma unroll
    for (int i = 0; i < 2; ++i) {       // tile (M, c) = ((wave + 8 i) / 4, wave % 4)
      const float x = lg_sum(dbx[i]);
      if (lg == 0) rbX[(wave & 3) * CH + 16 * ((wave >> 2) + 2 * i) + lr] = x;
    }
    if constexpr (G) {
      const float x = lg_sum(row16_sum(sdot));
      if (lane == 0) rsd[wave] = x;
    }
    __syncthreads();

    // ---- dk, dq -----------------------------------------------------------------------
    float csum = 0.f;
#pragma unroll
    for (int i = 0; i < NX; ++i) {
      const int mi = i / IC, j = i % IC;
      const int M = Mb + mi, ic = Ib + j;
      const int r = 16 * M + lr;
      f32x4 gk = {0.f, 0.f, 0.f, 0.f}, gq = {0.f, 0.f, 0.f, 0.f}, gw = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int kb = 0; kb < 4; ++kb) {
        const frag bk = colf(sK, LDK, 16 * kb, 16 * ic, lr, lg);
        const frag bw = WK ? colf(sKW, LDK, 16 * kb, 16 * ic, lr, lg) : bk;
        if (kb <= M) {                  // (beta D dA) KW, (D dP) KW: blocks on or left of the diagonal
          gk = O::mma1(gk, bw, rowf(sAk, LCP, 16 * M, 16 * kb, lr, lg));
          gq = O::mma1(gq, bw, rowf(sP, LCP, 16 * M, 16 * kb, lr, lg));
        }
        if (kb >= M) {                  // (beta D dA)^T K + (D dP)^T Q: blocks on or below it
          gw = O::mma1(gw, bk, colf(sAk, LCP, 16 * kb, 16 * M, lr, lg));
          gw = O::mma1(gw, colf(sQ, LDK, 16 * kb, 16 * ic, lr, lg), colf(sP, LCP, 16 * kb, 16 * M, lr, lg));
        }
      }
      const float br = sF[r];
      const float er = G ? sF[CH + r] : 1.f, eg = G ? sF[2 * CH + r] : 1.f, ed = G ? sF[3 * CH + r] : 1.f;
      const f32x4 dkr = gk - dYS[i] * (br * er);          // the read side
      const f32x4 dkw = gw + DdS[i] * ed;                 // the write side
      const f32x4 dq = gq + dOS[i] * eg;
      const uint32_t off = static_cast<uint32_t>((r * H * DK + 16 * ic + 4 * lg) * 2);
      if constexpr (WK) {
        buf_store8(bits8(dkr), rdk, off, sk);
        buf_store8(bits8(dkw), rdkw, off, sk);
      } else {
        buf_store8(bits8(dkr + dkw), rdk, off, sk);
      }
      buf_store8(bits8(dq), rdq, off, sk);
      if constexpr (G) {
        const f32x4 kk = O::f32(O::ld(sK + r * LDK + 16 * ic + 4 * lg));
        const f32x4 kwv = WK ? O::f32(O::ld(sKW + r * LDK + 16 * ic + 4 * lg)) : kk;
        const f32x4 qq = O::f32(O::ld(sQ + r * LDK + 16 * ic + 4 * lg));
        float a = 0.f, x = 0.f, c = 0.f;
#pragma unroll
        for (int s = 0; s < 4; ++s) {
          a += eg * qq[s] * dOS[i][s];
          x -= br * er * kk[s] * dYS[i][s];
          c += ed * kwv[s] * DdS[i][s];
        }
        a = lg_sum(a - c);
        x = lg_sum(x);
        if (lg == 0) {
          rgK[ic * CH + r] = a;
          rgX[ic * CH + r] = x;
        }
        csum += c;
      }
    }
    if constexpr (G) {
      const float x = lg_sum(row16_sum(csum));
      if (lane == 0) rcs[wave] = x;
    }
    __syncthreads();

    // ---- dbeta, d log a (suffix sums of dg over the chunk) ----------------------------
    if (wave == 0) {
      const int r = lane, Rr = r >> 4;
      const uint32_t off = static_cast<uint32_t>(lane * H * 2);
      float db = 0.f;
#pragma unroll
      for (int c = 0; c < 4; ++c) db += rbX[c * CH + r];
      for (int J = 0; J <= Rr; ++J) db += rbA[J * CH + r];
      buf_store2(f32_to_bf16_bits(db), rdb, off, sb);
      if constexpr (G) {
        float x = 0.f;
        for (int J = 0; J <= Rr; ++J) x += rgP[J * CH + r];
        for (int R = Rr; R < 4; ++R) x -= rgC[R * CH + r];
#pragma unroll
        for (int ic = 0; ic < DK / 16; ++ic) x += rgK[ic * CH + r];
        // terms of g_read_r': row r itself, or row r + 1 whose g_read is g_r
        const int rr = p.f.literal ? r + 1 : r;
        if (rr < CH) {
          const int Rq = rr >> 4;
          for (int J = 0; J <= Rq; ++J) x += rgA[J * CH + rr];
#pragma unroll
          for (int ic = 0; ic < DK / 16; ++ic) x += rgX[ic * CH + rr];
        }
        if (lane == CH - 1) {
          float cs = 0.f, sd = 0.f;
#pragma unroll
          for (int w = 0; w < NW; ++w) {
            cs += rcs[w];
            sd += rsd[w];
          }
          x += cs + sF[4 * CH] * sd;
        }
#pragma unroll
        for (int d = 1; d < 64; d <<= 1) {
          const float y = __shfl_down(x, d);
          if (lane + d < 64) x += y;
        }
        buf_store2(f32_to_bf16_bits(x), rdl, off, sb);
      }
    }
  }
}

// dS0 for sequences of no tokens: the incoming gradient (or zero) passes through.
__global__ void bwd_copy_state_kernel(const float* src, float* dst, int64_t n) {
  const int64_t i = static_cast<int64_t>(blockIdx.x) * blockDim.x + threadIdx.x;
  if (i < n) dst[i] = src ? src[i] : 0.f;
}

template <int GATE, int DK, bool WK>
hipError_t launch_bwd_t(const BwdParams& p, hipStream_t stream) {
  const ChunkParams& f = p.f;
  const int n_tiles = f.d_v / 64;
  const int64_t nseq = f.B * f.H * n_tiles;
  hipError_t e;
  bool rev_pipe = false;
  if constexpr (GATE != GATE_CHANNEL && !WK) rev_pipe = p.saved != 0;
  if (rev_pipe) {
    // the states came from the training forward: pass 2 alone, with chain and helper
    // waves.  (Both passes run side by side otherwise, a workgroup of each per compute
    // unit, which the chain/helper pass's LDS would not leave room for.)
    if constexpr (GATE != GATE_CHANNEL && !WK)
      hipLaunchKernelGGL((bwd_rev_pipe_kernel<GATE, DK>), dim3(static_cast<unsigned>(nseq)), dim3(512), 0, stream, p,
                         n_tiles);
  } else {
    hipLaunchKernelGGL((bwd_seq_kernel<GATE, DK, WK>), dim3(static_cast<unsigned>((p.saved ? 1 : 2) * nseq)),
                       dim3(256), 0, stream, p, n_tiles, static_cast<int>(nseq), p.saved ? 2 : 0);
  }
  e = hipGetLastError();
  if (e != hipSuccess) return e;
  if constexpr (GATE == GATE_CHANNEL) {
    static_assert(!WK, "per-channel gate: no write key");
    return launch_chunk_bwd_chan(p, stream);
  } else {
    const int64_t nch = (f.T + CH - 1) / CH;
    const unsigned grid = static_cast<unsigned>(f.cu ? f.H * f.nslots : f.B * f.H * nch);
    if (f.d_v == 128)
      hipLaunchKernelGGL((bwd_chunk_kernel<GATE, DK, 128, WK>), dim3(grid), dim3(512), 0, stream, p);
    else
      hipLaunchKernelGGL((bwd_chunk_kernel<GATE, DK, 64, WK>), dim3(grid), dim3(512), 0, stream, p);
    return hipGetLastError();
  }
}

template <int GATE, bool WK = false>
hipError_t launch_bwd_g(const BwdParams& p, hipStream_t stream) {
  if (p.f.d_k == 128) return launch_bwd_t<GATE, 128, WK>(p, stream);
  if constexpr (GATE != GATE_CHANNEL)   // the per-channel gate: d_k = 128 only
    if (p.f.d_k == 64) return launch_bwd_t<GATE, 64, WK>(p, stream);
  return hipErrorInvalidValue;
}

// The records follow the gate: with a per-channel gate they also hold the decayed
// operands the sequential passes read.
int rec_gate(int gate) { return gate == GATE_CHANNEL ? GATE_CHANNEL : GATE_SCALAR; }

}  // namespace

size_t chunk_bwd_state_bytes(int64_t B, int64_t T, int64_t H, int d_k, int d_v) {
  return static_cast<size_t>(B * H * ((T + CH - 1) / CH)) * static_cast<size_t>(d_k) * static_cast<size_t>(d_v) * 2u;
}

size_t chunk_bwd_workspace_bytes(int64_t B, int64_t T, int64_t H, int d_k, int d_v, int gate) {
  return chunk_workspace_bytes(B, T, H, IO_BF16, rec_gate(gate), d_k) + 2 * chunk_bwd_state_bytes(B, T, H, d_k, d_v);
}

size_t chunk_bwd_varlen_state_bytes(int64_t T, int64_t n_seq, int64_t H, int d_k, int d_v) {
  return static_cast<size_t>(H * chunk_varlen_slots(T, n_seq)) * static_cast<size_t>(d_k) * static_cast<size_t>(d_v) * 2u;
}

size_t chunk_bwd_varlen_workspace_bytes(int64_t T, int64_t n_seq, int64_t H, int d_k, int d_v, int gate) {
  return chunk_varlen_records_bytes(T, n_seq, H, IO_BF16, rec_gate(gate), d_k) +
         2 * chunk_bwd_varlen_state_bytes(T, n_seq, H, d_k, d_v);
}

hipError_t launch_chunk_bwd(const BwdParams& p, hipStream_t stream) {
  const ChunkParams& f = p.f;
  if (f.B * f.H == 0) return hipSuccess;
  if (f.io != IO_BF16 || (f.gate == GATE_CHANNEL && (f.d_k != 128 || f.kw))) return hipErrorInvalidValue;
  if (f.kw && !p.dkw) return hipErrorInvalidValue;
  if (f.T == 0) {
    if (!p.dS0) return hipSuccess;
    const int64_t n = f.B * f.H * f.d_k * f.d_v;
    hipLaunchKernelGGL(bwd_copy_state_kernel, dim3(static_cast<unsigned>((n + 255) / 256)), dim3(256), 0, stream, p.dS_T,
                       p.dS0, n);
    return hipGetLastError();
  }
  if (!p.saved) {   // else the records are the training forward's
    const hipError_t e = launch_chunk_prep(f, stream);   // with f.kw: T of the write-key Gram blocks
    if (e != hipSuccess) return e;
  }
  if (f.kw) {
    if (f.gate == GATE_NONE) return launch_bwd_g<GATE_NONE, true>(p, stream);
    if (f.gate == GATE_SCALAR) return launch_bwd_g<GATE_SCALAR, true>(p, stream);
    return hipErrorInvalidValue;
  }
  switch (f.gate) {
    case GATE_NONE: return launch_bwd_g<GATE_NONE>(p, stream);
    case GATE_SCALAR: return launch_bwd_g<GATE_SCALAR>(p, stream);
    case GATE_CHANNEL: return launch_bwd_g<GATE_CHANNEL>(p, stream);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace gdr
