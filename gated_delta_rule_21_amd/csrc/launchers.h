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
  int64_t B, T, H;
  int d_k, d_v;
  int io, gate, literal;
};

hipError_t launch_decode_step(const DecodeParams& p, hipStream_t stream);
// Per-chunk transform (T tiles into p.ws), then the state pass; one stream, in order.
hipError_t launch_chunk_prep(const ChunkParams& p, hipStream_t stream);
hipError_t launch_chunk_state_pipe(const ChunkParams& p, hipStream_t stream);   // bf16 I/O
hipError_t launch_chunk_fwd(const ChunkParams& p, hipStream_t stream);
// B*H*ceil(T/64) records of the per-chunk transform (see WsRec in chunk_common.h)
size_t chunk_workspace_bytes(int64_t B, int64_t T, int64_t H, int io, int gate, int d_k);

}  // namespace gdr
