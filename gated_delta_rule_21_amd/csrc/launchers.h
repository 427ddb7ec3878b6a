// Internal interface between the C-ABI layer (argument checks) and the kernels.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace gdr {

struct DecodeParams {
  const void* q;
  const void* k;
  const void* v;
  const void* beta;
  const void* log_a;
  const float* S;
  float* S_new;
  void* o;
  int64_t n_states;   // B * H
  int d_k, d_v;
  int io, gate, literal;
  const void* kw;     // write key [B, H, d_k] (the state is written along it), or null: along k
};

struct ChunkParams {
  const void* q;
  const void* k;
  const void* v;
  const void* beta;
  const void* log_a;
  const float* S0;    // may be null (zero initial state)
  void* o;
  float* S_T;         // may be null (not written)
  void* ws;           // per-chunk records of the transform (chunk_workspace_bytes)
  int64_t B, T, H;    // packed sequences: B = number of sequences, T = total tokens
  int d_k, d_v;
  int io, gate, literal;
  // Packed variable-length sequences (null for fixed-length batches): device int32
  // offsets cu[0..B], sequence b = tokens [cu[b], cu[b+1]) of [1, T, H, .] tensors;
  // nslots = records per head in the workspace (chunk_varlen_slots).
  const int32_t* cu;
  int64_t nslots;
  const int32_t* order;   // packed sequences: longest first (in the workspace, after the records)
  const void* kw;         // write key [B, T, H, d_k] (bf16), or null: the state is written along k
  // Training forward (bf16 state pass): the state entering every chunk, bf16 in
  // the backward's chunk-state layout (chunk_state_off), or null.
  void* states = nullptr;
  // Packed sequences: where the order is written (null: after the records in ws).
  int32_t* order_out = nullptr;
};

// Byte offset of element (d, v) of one chunk's bf16 state (d_k x d_v) in the
// per-chunk state records of the backward: d_k in tiles of 16, each tile value-major,
// [d_k / 16][d_v][16].  A lane holding four adjacent d of one column of an MFMA
// accumulator tile writes 8 bytes, and the 16 columns of a tile row are contiguous,
// so one store instruction covers 512 contiguous bytes.
__host__ __device__ constexpr uint32_t chunk_state_off(int d, int v, int d_v) {
  return static_cast<uint32_t>((((d >> 4) * d_v + v) * 16 + (d & 15)) * 2);
}

struct PrecondParams {
  const void* k;        // [B, T, H, d_k] io dtype
  const void* beta;     // [B, T, H] io dtype
  const void* r;        // [B, T, H] io dtype retention, or null (none)
  const float* d0;      // [B, H, d_k] starting preconditioner, or null (ones)
  void* kw;             // [B, T, H, d_k] io dtype write keys
  float* d_T;           // [B, H, d_k] final preconditioner, or null
  int64_t B, T, H;
  int d_k, io;
  float eta;
};
// Backward of the chunk forward (bf16 I/O, every gate -- a per-channel gate with
// d_k = 128 --, either form): f carries the forward's inputs, the workspace records
// (f.ws) and, for packed sequences, cu and nslots; o, S_T and order are unused.
struct BwdParams {
  ChunkParams f;
  const void* dO;       // [B, T, H, d_v] gradient of the output
  const float* dS_T;    // [B, H, d_k, d_v] gradient of the final state, or null (zero)
  void* dq;             // [B, T, H, d_k]
  void* dk;             // [B, T, H, d_k]; with a write key (f.kw) the read side only
  void* dkw;            // [B, T, H, d_k] gradient of the write key (f.kw set), else unused
  void* dv;             // [B, T, H, d_v]
  void* dbeta;          // [B, T, H]
  void* dlog_a;         // [B, T, H] (scalar gate), [B, T, H, d_k] (per-channel gate), else unused
  float* dS0;           // [B, H, d_k, d_v], or null (not written)
  void* states;         // B H ceil(T/64) chunk-start states, bf16, laid out by chunk_state_off
  void* dstates;        // the gradients of the chunk-end states, same layout
  // The records (f.ws) and the chunk-start states were left by a training forward
  // over the same inputs: no transform and no pass 1.
  int saved = 0;
};
// Reverse mode of the preconditioner scan (the gradients of <dkw, kw> + <dd_T, d_T>).
struct PrecondBwdParams {
  PrecondParams f;      // the forward's inputs (f.kw, f.d_T unused)
  const void* dkw;      // [B, T, H, d_k] io dtype gradient of kw, or null (zero)
  const float* dd_T;    // [B, H, d_k] gradient of d_T, or null (zero)
  void* dk;             // [B, T, H, d_k] io dtype
  void* dbeta;          // [B, T, H] io dtype
  void* dr;             // [B, T, H] io dtype (f.r set), or null (not written)
  float* dd0;           // [B, H, d_k], or null (not written)
  float* ws;            // precond_scan_bwd_workspace_bytes: d_t of every token, then (x_t, n_t)
};
size_t precond_scan_bwd_workspace_bytes(int64_t B, int64_t T, int64_t H, int d_k);
hipError_t launch_decode_step(const DecodeParams& p, hipStream_t stream);
// Preconditioner scan: one workgroup per (sequence, head).
hipError_t launch_precond_scan(const PrecondParams& p, hipStream_t stream);
hipError_t launch_precond_scan_bwd(const PrecondBwdParams& p, hipStream_t stream);
// Per-chunk transform (T tiles into p.ws), then the state pass; one stream, in order.
hipError_t launch_chunk_prep(const ChunkParams& p, hipStream_t stream);
hipError_t launch_chunk_state_pipe(const ChunkParams& p, hipStream_t stream);   // bf16 I/O
hipError_t launch_chunk_fwd(const ChunkParams& p, hipStream_t stream);
// B*H*ceil(T/64) records of the per-chunk transform (see WsRec in chunk_common.h)
size_t chunk_workspace_bytes(int64_t B, int64_t T, int64_t H, int io, int gate, int d_k);
// gdr_chunk_fwd_noalloc: the size of the static device array that holds its
// workspace, and that array's address on the current device (looked up once per
// device; the first call on a device loads it).
constexpr size_t STATIC_SCRATCH_BYTES = size_t(256) << 20;
hipError_t static_scratch(void** ptr);
// Packed sequences: record slots per head for n_seq sequences of T tokens in all
// (sequence b's chunks start at slot floor(cu[b] / 64) + b), and the workspace bytes:
// the records, then the order of the sequences by length (n_seq int32, 16-byte
// padded) in which the state pass takes them.
inline int64_t chunk_varlen_slots(int64_t T, int64_t n_seq) { return (T + 63) / 64 + n_seq; }
size_t chunk_varlen_records_bytes(int64_t T, int64_t n_seq, int64_t H, int io, int gate, int d_k);
size_t chunk_varlen_workspace_bytes(int64_t T, int64_t n_seq, int64_t H, int io, int gate, int d_k);
// Backward: the per-chunk transform into p.f.ws, then the three passes (p.saved:
// pass 2 and pass 3 only).
hipError_t launch_chunk_bwd(const BwdParams& p, hipStream_t stream);
// Bytes of one set of per-chunk states (bf16), and of the whole backward workspace:
// the transform's records, the chunk-start states, the chunk-end state gradients.
size_t chunk_bwd_state_bytes(int64_t B, int64_t T, int64_t H, int d_k, int d_v);
size_t chunk_bwd_workspace_bytes(int64_t B, int64_t T, int64_t H, int d_k, int d_v, int gate);
// Packed sequences: the records and the states by the slots of chunk_varlen_slots.
size_t chunk_bwd_varlen_state_bytes(int64_t T, int64_t n_seq, int64_t H, int d_k, int d_v);
size_t chunk_bwd_varlen_workspace_bytes(int64_t T, int64_t n_seq, int64_t H, int d_k, int d_v, int gate);
// The per-chunk gradients with a per-channel gate (d_k = 128), after the sequential passes.
hipError_t launch_chunk_bwd_chan(const BwdParams& p, hipStream_t stream);
// Longest-first order of packed sequences into `order` (n_seq int32).
hipError_t launch_varlen_order(const ChunkParams& p, int32_t* order, hipStream_t stream);

}  // namespace gdr
