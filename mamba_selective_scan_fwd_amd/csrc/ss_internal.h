// ss_internal.h -- kernel parameter blocks and launch entry points shared by
// the host ABI (ss_abi.cpp) and the kernel translation units.  Internal.
#pragma once

#include <hip/hip_runtime_api.h>
#include <stdint.h>

#include <utility>

#include "../../include/ss.h"

namespace ss {

// ss_fwd's validation and dispatch, with the workspace given explicitly (the
// C entry points ss_fwd and ss_fwd_noalloc both go through it).
ss_status fwd_checked(const ss_problem* p, const void* u, const void* delta, const float* A, const void* Bm,
                      const void* Cm, const float* D, const void* z, const float* delta_bias, const int32_t* lengths,
                      const int32_t* seq_idx, const float* h0, void* y, float* last_state, float* ckpt,
                      void* workspace, size_t workspace_bytes, void* stream);
size_t fwd_workspace_bytes(const ss_problem* p);  // the least workspace ss_fwd needs
ss_status fwd_check_problem(const ss_problem* p);

struct FwdParams {
  int32_t io;
  int32_t softplus;
  const void* u;
  const void* delta;
  const void* z;
  const void* Bm;
  const void* Cm;
  const float* A;
  const float* D;
  const float* bias;
  const int32_t* lengths;
  const int32_t* seq_idx;  // (batch, seqlen) document ids, or null
  const float* h0;         // (batch, dim, dstate) initial state, or null
  void* y;
  float* last_state;
  float* ckpt;
  // time-chunked scan (one launch): per (channel, chunk, state) the chunk's
  // pair (P, S) as one 64-bit word (P low), per (channel, group but the last,
  // state) the pair of a group of `group` consecutive chunks; nslots words
  // from `pairs` (through the group slots) are set to all ones, "not yet
  // published", before the launch; the error word in q_ctrl[1]
  uint64_t* pairs;
  uint64_t* gpairs;
  int64_t nslots;
  int32_t group;
  int32_t ngroups;
  int64_t batch, dim, dstate, seqlen;
  int64_t chunk_len;     // multiple of 64
  int64_t ch_blocks;     // ceil(dim / 16)
  int64_t ckpt_per_row;  // ceil(seqlen / 64)
  int32_t nchunks;
  // persistent work queue over (chunk, batch row, channel block) units (ragged
  // rows, or more row blocks than fit the GPU at once): null q_ctrl = off
  int32_t* q_ctrl;   // [0] next unit, [1] set when a wait gave up (also the time-chunked scan's)
  int32_t* q_flags;  // per (batch row, channel block, chunk): its final state is published
  float* q_carry;    // per (channel, chunk, state): the state after the chunk
  int64_t q_chunks;  // chunks per row (chunk_len steps each)
  int64_t q_grid;    // persistent workgroups
};

struct StepParams {
  int32_t io;
  int32_t softplus;
  const void* u;
  const void* delta;
  const void* z;
  const void* Bt;
  const void* Ct;
  const float* A;
  const float* D;
  const float* bias;
  const float* state_in;
  float* state_out;
  void* y;
  int64_t batch, dim, dstate;
};

struct BwdParams {
  int32_t io;
  int32_t softplus;
  const void* u;
  const void* delta;
  const void* z;
  const void* Bm;
  const void* Cm;
  const float* A;
  const float* D;
  const float* bias;
  const float* ckpt;
  const int32_t* seq_idx;  // (batch, seqlen) document ids, or null
  const void* dy;
  const float* dlast;      // (batch, dim, dstate) gradient from the final state, or null
  float* dh0;              // (batch, dim, dstate) gradient w.r.t. the initial state, or null
  void* du;
  void* ddelta;
  void* dz;
  float* dA;
  float* dB;
  float* dC;
  float* dD;
  float* dbias;
  float* gcarry;  // workspace: reverse carries per (channel, chunk, state)
  float* aggP;    // workspace: per-chunk decay product
  float* aggG;    // workspace: per-chunk state gradient from a zero carry
  int64_t batch, dim, dstate, seqlen;
  int64_t ch_blocks;
  int64_t nchunks;  // ceil(seqlen / 64)
};

struct ConvParams {
  int32_t io;
  int32_t width;  // W = d_conv, 1..4
  int32_t silu;
  const void* x;
  const float* w;     // (dim, W)
  const float* bias;  // (dim) or null
  const int32_t* seq_idx;
  const float* conv_init;  // (batch, dim, W-1) or null
  void* out;
  float* conv_final;       // (batch, dim, W-1) or null
  int64_t batch, dim, seqlen;
  int64_t tblocks;         // workgroups per row
};

struct ConvStepParams {
  int32_t io;
  int32_t width;
  int32_t silu;
  const void* x;  // (batch, dim)
  const float* w;
  const float* bias;
  const float* window_in;  // (batch, dim, W-1)
  float* window_out;
  void* out;               // (batch, dim)
  int64_t batch, dim;
};

struct SsdParams {
  int32_t io;        // SS_F16 or SS_BF16
  int32_t softplus;
  const void* x;     // (batch, seqlen, nheads, 64)
  const void* dt;    // (batch, seqlen, nheads)
  const float* A;    // (nheads)
  const void* Bm;    // (batch, seqlen, ngroups, dstate)
  const void* Cm;
  const float* D;        // (nheads) or null
  const void* z;         // like x, or null
  const float* dt_bias;  // (nheads) or null
  const int32_t* seq_idx;  // (batch, seqlen) document ids, or null
  const float* h0;       // (batch, nheads, 64, dstate) or null
  void* y;
  float* final_state;    // (batch, nheads, 64, dstate) or null
  // workspace
  uint16_t* ws_entry;    // (batch, nchunks, nheads, dstate, 64), I/O dtype bits: each chunk's entry state, [n][p]
  uint16_t* ws_cb;       // (batch, nchunks, ngroups, 256, 256) bf16: C B^T of each chunk
  int64_t batch, seqlen, nheads, ngroups, dstate, nchunks;
};

hipError_t launch_fwd(const FwdParams& p, int64_t nchunks, hipStream_t st);
int64_t device_cus();
hipError_t launch_ssd(const SsdParams& p, hipStream_t st);
hipError_t launch_conv(const ConvParams& p, hipStream_t st);
hipError_t launch_conv_step(const ConvStepParams& p, hipStream_t st);
int64_t conv_tblocks(int64_t seqlen);
hipError_t launch_step(const StepParams& p, hipStream_t st);
hipError_t launch_bwd(const BwdParams& p, hipStream_t st);
hipError_t launch_copy(const void* src, void* dst, int64_t bytes, hipStream_t st);
hipError_t launch_alu_probe(int32_t kind, int32_t workgroups, int32_t iters, int32_t lds_bytes, int64_t* out,
                            hipStream_t st);

}  // namespace ss
