// ss_fwd.hip -- selective-scan forward, decode step and chunk-carry kernels (gfx950).
//
// The recurrence (page "Mamba", Part IV Stages 4-6): per channel (b, d) and
// state n,  h_t[n] = exp(Delta_t A[d,n]) h_{t-1}[n] + Delta_t B[b,n,t] u_t,
// y_t = (sum_n C[b,n,t] h_t[n] + D[d] u_t) * SiLU(z_t),
// Delta_t = softplus(delta_t + bias[d]).
//
// Mapping on CDNA4.  One 64-lane wavefront holds 4 channels x 16 states:
// lane (c, n) keeps h[n] of channel c in a VGPR for the whole time walk.
// The per-(t, d) work (softplus, Delta*u, the skip, the gate, conversions)
// is spread over the 16 lanes of the channel's DPP row -- lane l owns the
// steps t = l (mod 16) -- and Delta_t, Delta_t*u_t reach the other lanes of
// the row through DPP row broadcasts folded into the multiplies.  The
// readout sum over n is a transpose through LDS: each step's products
// C[n,t] h_t[n] are written to a 16x16 tile per channel, and after 16 steps
// lane l adds up row t = l.  B and C tiles (shared by the 16 channels of a
// workgroup, which all belong to one batch row) are staged in LDS once per
// 64-step tile.  No MFMA: the work is an elementwise recurrence plus a
// 16-wide reduction, not a contraction.
//
// Time chunking (for problems with too few channels to fill 256 CUs): the
// sequence is cut into K chunks of a multiple of 64 steps.  Pass 1
// (ss_fwd_chunk_kernel<AGG>) computes for each chunk the pair (P, S) =
// (prod of exp(Delta A) over the chunk, state reached from the chunk's start
// with a zero carry; the first chunk starts from the caller's initial state), pass 2
// (ss_carry_kernel) scans the pairs with the associative operator
// (P1,S1) then (P2,S2) = (P2 P1, P2 S1 + S2) (page "Mamba", Part V, the
// combine for h_t = a_t h_{t-1} + b_t) to get each chunk's entry state, and
// pass 3 (ss_fwd_chunk_kernel<FINAL>) reruns every chunk from its entry state
// and writes y.  With K = 1 only pass 3 runs, from the initial state (zero
// unless given).
//
// Packed documents ("niverel-mamba" README, "seq_idx strict reset"): where
// the row's document id changes the state restarts from zero; the decay of
// that step is replaced by 0 (so a chunk holding a document start has P = 0).
// Tiles without a start run the plain code.
#include <type_traits>

#include "ss_device.h"
#include "ss_internal.h"

namespace ss {

hipError_t launch_carry(const float* aggP, const float* aggS, float* carry, int64_t nch, int32_t nchunks,
                        bool reverse, hipStream_t st);

namespace {

constexpr int kBCStride = kTile + 4;     // padded LDS row of the B tile (floats)
constexpr int kCTRow = 20;               // padded LDS row of the transposed C tile
constexpr int kPRow = 20;                // padded LDS row of the state tile (16 states + 4)
constexpr int kPChan = 16 * kPRow + 16;  // per-channel state tile; 336 = 16 mod 64 banks

// FINAL keeps C and the state tiles for the readout; the chunk-summary pass
// only needs B.
template <bool FINAL>
struct FwdSmem {
  float B[2][kStates][kBCStride];        // B[n][t], read by the state lanes
  float CT[2][kTile][kCTRow];            // C[t][n], read by the lane that owns step t
  float P[kWaves][kChPerWave * kPChan];  // h_t[n] of 16 steps, per channel
};
template <>
struct FwdSmem<false> {
  float B[2][kStates][kBCStride];
};
template <bool FINAL>
__device__ __forceinline__ float* state_tile(FwdSmem<FINAL>& sm, int wave) {
  if constexpr (FINAL) return sm.P[wave];
  else return nullptr;
}
template <bool FINAL>
__device__ __forceinline__ const float* ct_row(FwdSmem<FINAL>& sm, int buf, int l) {
  if constexpr (FINAL) return &sm.CT[buf][l][0];
  else return nullptr;
}

// Per-lane registers of the four steps this lane owns in a 64-step tile.
struct Owned {
  float dt[4];   // Delta_t (0 for masked steps)
  float dtu[4];  // Delta_t * u_t (0 for masked steps)
  float u[4];
  float z[4];
};

// Raw element bits of the owned steps of the next tile: loaded one tile
// ahead and converted only when used, so the loads stay in flight across a
// whole tile of compute.
template <int IO>
struct RawOwned {
  raw_t<IO> u[4], dl[4], z[4];
};

// Wave-uniform views of the operands: one buffer resource per tensor region
// (the 4 channel rows of this wave for u/delta/z/y, the batch row's (N, L)
// block for B/C).  Lanes address them with 32-bit byte offsets; accesses past
// the region return 0 / are dropped by the hardware range check.
struct Views {
  __amdgpu_buffer_rsrc_t u, dl, z, y, B, C;
};

template <int IO>
__device__ __forceinline__ void load_owned(RawOwned<IO>& r, const Views& v, uint32_t lane_elem0, int t0, int l) {
  constexpr uint32_t s = io_bytes<IO>();
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const uint32_t off = (lane_elem0 + (uint32_t)(t0 + 16 * i + l)) * s;
    r.u[i] = bload<IO>(v.u, off);
    r.dl[i] = bload<IO>(v.dl, off);
    r.z[i] = bload<IO>(v.z, off);  // a zero-size view when there is no gate
  }
}

// Staging of the B/C tile.  Thread (n, j) covers state row n.  With PAIR
// (16-bit data and an even seqlen, so that every element pair is 4-byte
// aligned) it loads two 32-bit words = steps t0 + 32k + 2j, +1 (k < 2);
// otherwise four single elements, steps t0 + j + 16k (k < 4).  Either way 16
// lanes cover a contiguous run of the row per load.
template <int IO, bool PAIR>
struct BCRaw {
  static constexpr int kN = PAIR ? 2 : 4;
  using T = std::conditional_t<PAIR, uint32_t, raw_t<IO>>;
  T b[kN], c[kN];
};

template <int IO, bool PAIR>
__device__ __forceinline__ void load_bc(BCRaw<IO, PAIR>& r, const Views& v, uint32_t seqlen, int t0, int tid,
                                        bool need_c) {
  constexpr uint32_t s = io_bytes<IO>();
  const int n = tid / 16, j = tid % 16;
#pragma unroll
  for (int k = 0; k < BCRaw<IO, PAIR>::kN; ++k) {
    if constexpr (PAIR) {
      const uint32_t off = ((uint32_t)n * seqlen + (uint32_t)(t0 + 32 * k + 2 * j)) * s;
      r.b[k] = __builtin_amdgcn_raw_buffer_load_b32(v.B, off, 0, 0);
      r.c[k] = need_c ? __builtin_amdgcn_raw_buffer_load_b32(v.C, off, 0, 0) : 0u;
    } else {
      const uint32_t off = ((uint32_t)n * seqlen + (uint32_t)(t0 + j + 16 * k)) * s;
      r.b[k] = bload<IO>(v.B, off);
      r.c[k] = need_c ? bload<IO>(v.C, off) : raw_t<IO>(0);
    }
  }
}

// B (row-major, for the state lanes) and C (transposed, for the step owners)
// of steps at or past the valid end are staged as exact zeros, so data past a
// row's length (padding, NaN) never reaches the state or the output.
template <int IO, bool PAIR, bool FINAL>
__device__ __forceinline__ void store_bc(FwdSmem<FINAL>& sm, int buf, const BCRaw<IO, PAIR>& r, int tid, int nvalid,
                                         bool n_ok) {
  const int n = tid / 16, j = tid % 16;
#pragma unroll
  for (int k = 0; k < BCRaw<IO, PAIR>::kN; ++k) {
    if constexpr (PAIR) {
      const int e = 32 * k + 2 * j;
      const bool ok0 = n_ok && e < nvalid, ok1 = n_ok && e + 1 < nvalid;
      const float b0 = bits_f32<IO>((raw_t<IO>)(r.b[k] & 0xffffu)), b1 = bits_f32<IO>((raw_t<IO>)(r.b[k] >> 16));
      *reinterpret_cast<float2*>(&sm.B[buf][n][e]) = make_float2(ok0 ? b0 : 0.0f, ok1 ? b1 : 0.0f);
      if constexpr (FINAL) {
        const float c0 = bits_f32<IO>((raw_t<IO>)(r.c[k] & 0xffffu)), c1 = bits_f32<IO>((raw_t<IO>)(r.c[k] >> 16));
        sm.CT[buf][e][n] = ok0 ? c0 : 0.0f;
        sm.CT[buf][e + 1][n] = ok1 ? c1 : 0.0f;
      }
    } else {
      const int e = j + 16 * k;
      const bool ok = n_ok && e < nvalid;
      sm.B[buf][n][e] = ok ? bits_f32<IO>(r.b[k]) : 0.0f;
      if constexpr (FINAL) sm.CT[buf][e][n] = ok ? bits_f32<IO>(r.c[k]) : 0.0f;
    }
  }
}

// Per-(t, d) work of the four owned steps: Delta, Delta*u (zero when masked).
template <int IO>
__device__ __forceinline__ void prep_owned(Owned& o, const RawOwned<IO>& r, int l, int nvalid, float bias,
                                           bool softplus, float& dt_sum) {
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const bool v = 16 * i + l < nvalid;
    const float u = bits_f32<IO>(r.u[i]);
    const float x = bits_f32<IO>(r.dl[i]) + bias;
    float dt = softplus ? softplus_f(x) : x;
    dt = v ? dt : 0.0f;
    o.dt[i] = dt;
    o.dtu[i] = v ? dt * u : 0.0f;
    o.u[i] = u;
    o.z[i] = bits_f32<IO>(r.z[i]);
    dt_sum += dt;
  }
}

// 16 steps of block I of the tile.  Lane (c, n) advances state n of channel c
// and (FINAL) leaves h_t[n] in column n of the channel's LDS state tile.  The
// block's 16 B values are read into registers up front, so no LDS wait sits
// between two steps of the recurrence.
template <int I, bool FINAL, bool RESET, int... J>
__device__ __forceinline__ void scan_block(float& h, const Owned& o, float A2, const float* sBrow, float* pcol,
                                           uint64_t starts, std::integer_sequence<int, J...>) {
  float bq[16];
  *reinterpret_cast<float4*>(&bq[0]) = *reinterpret_cast<const float4*>(sBrow + 16 * I + 0);
  *reinterpret_cast<float4*>(&bq[4]) = *reinterpret_cast<const float4*>(sBrow + 16 * I + 4);
  *reinterpret_cast<float4*>(&bq[8]) = *reinterpret_cast<const float4*>(sBrow + 16 * I + 8);
  *reinterpret_cast<float4*>(&bq[12]) = *reinterpret_cast<const float4*>(sBrow + 16 * I + 12);
  (
      [&] {
        const float a = reset_decay<RESET, 16 * I + J>(exp2_hw(row_bcast<J>(o.dt[I]) * A2), starts);
        h = fmaf(a, h, row_bcast<J>(o.dtu[I]) * bq[J]);
        if constexpr (FINAL) pcol[J * kPRow] = h;
      }(),
      ...);
  h = fresh(h);
  // keep the next block's exps from being hoisted here (register pressure)
  __builtin_amdgcn_sched_barrier(0);
}

__device__ __forceinline__ void wave_lds_sync() {
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
  __builtin_amdgcn_wave_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
}

// C[t][n] of the owned step 16 I + l (read before the block's scan, so the
// readout waits only for the state row)
struct CRow {
  float4 c0, c1, c2, c3;
};
__device__ __forceinline__ CRow load_crow(const float* crow) {
  CRow r;
  r.c0 = *reinterpret_cast<const float4*>(crow + 0);
  r.c1 = *reinterpret_cast<const float4*>(crow + 4);
  r.c2 = *reinterpret_cast<const float4*>(crow + 8);
  r.c3 = *reinterpret_cast<const float4*>(crow + 12);
  return r;
}

// Readout, skip, gate and store of the owned step 16 I + l of the tile:
// y0 = sum_n C[t][n] h_t[n] (four independent FMA chains).
template <int IO, int I>
__device__ __forceinline__ void finish_block(const Owned& o, const float* prow, const CRow& c, float Dd,
                                             bool need_z, const Views& v, uint32_t elem, int l, int nvalid,
                                             int nstop) {
  const float4 h0 = *reinterpret_cast<const float4*>(prow + 0);
  const float4 h1 = *reinterpret_cast<const float4*>(prow + 4);
  const float4 h2 = *reinterpret_cast<const float4*>(prow + 8);
  const float4 h3 = *reinterpret_cast<const float4*>(prow + 12);
  float y0 = c.c0.x * h0.x, y1 = c.c0.y * h0.y, y2 = c.c0.z * h0.z, y3 = c.c0.w * h0.w;
  y0 = fmaf(c.c1.x, h1.x, y0); y1 = fmaf(c.c1.y, h1.y, y1); y2 = fmaf(c.c1.z, h1.z, y2); y3 = fmaf(c.c1.w, h1.w, y3);
  y0 = fmaf(c.c2.x, h2.x, y0); y1 = fmaf(c.c2.y, h2.y, y1); y2 = fmaf(c.c2.z, h2.z, y2); y3 = fmaf(c.c2.w, h2.w, y3);
  y0 = fmaf(c.c3.x, h3.x, y0); y1 = fmaf(c.c3.y, h3.y, y1); y2 = fmaf(c.c3.z, h3.z, y2); y3 = fmaf(c.c3.w, h3.w, y3);
  float yv = fmaf(Dd, o.u[I], (y0 + y1) + (y2 + y3));
  if (need_z) yv *= silu_f(o.z[I]);
  const int tr = 16 * I + l;
  yv = tr < nvalid ? yv : 0.0f;
  const uint32_t off = tr < nstop ? (elem + (uint32_t)tr) * io_bytes<IO>() : kOffNone;
  bstore<IO>(v.y, off, yv);
}

template <int IO, bool FINAL, bool PAIR, bool SEQ>
__global__ void __launch_bounds__(kThreads) ss_fwd_chunk_kernel(FwdParams p) {
  __shared__ FwdSmem<FINAL> sm;
  constexpr uint32_t s = io_bytes<IO>();
  const int tid = threadIdx.x;
  const int wave = uniform(tid / 64);
  const int lane = tid % 64;
  const int cw = lane / 16;  // channel within the wave
  const int n = lane % 16;   // state index; also the time-owner index l
  const int l = n;

  // logical block -> (chunk, batch row, channel block).  Channel blocks vary
  // fastest: the blocks that share one batch row's B and C tiles run on one
  // XCD, so each row's B and C come from HBM about once.
  uint32_t lb = xcd_logical_block();
  const int64_t cb = lb % p.ch_blocks;
  lb /= p.ch_blocks;
  const int64_t b = lb % p.batch;
  const int64_t chunk = lb / p.batch + p.chunk_base;

  const int64_t d0 = cb * kChPerBlock + wave * kChPerWave;  // first channel of this wave
  const int64_t d = d0 + cw;
  const bool ch_ok = d < p.dim;
  const bool n_ok = n < p.dstate;
  const int64_t ch = b * p.dim + d;
  int64_t nch_w = p.dim - d0;
  nch_w = nch_w < 0 ? 0 : (nch_w > kChPerWave ? kChPerWave : nch_w);

  // time bounds (seqlen < 2^24, so 32-bit arithmetic is exact)
  const int L = (int)p.seqlen;
  int len = L;
  if (p.lengths) {
    const int v = p.lengths[b];
    len = v < 0 ? 0 : (v > L ? L : v);
  }
  const int t_begin = (int)(chunk * p.chunk_len);
  const int t_stop = t_begin + (int)p.chunk_len < L ? t_begin + (int)p.chunk_len : L;
  const int t_valid_end = t_stop < len ? t_stop : len;
  // tiles that hold at least one valid step; the rest of the chunk is zero-filled
  const int t_tile_end =
      t_valid_end > t_begin ? t_begin + ((t_valid_end - t_begin + kTile - 1) / kTile) * kTile : t_begin;

  const bool need_z = p.z != nullptr;
  const bool softplus = p.softplus != 0;
  const int64_t row0 = (b * p.dim + d0) * p.seqlen;  // element offset of the wave's first row
  const uint32_t wave_bytes = (uint32_t)(nch_w * p.seqlen) * s;
  Views v;
  v.u = make_rsrc(static_cast<const char*>(p.u) + row0 * s, wave_bytes);
  v.dl = make_rsrc(static_cast<const char*>(p.delta) + row0 * s, wave_bytes);
  const bool load_z = FINAL && need_z;
  v.z = make_rsrc(load_z ? static_cast<const char*>(p.z) + row0 * s : static_cast<const char*>(p.u),
                  load_z ? wave_bytes : 0u);
  v.y = make_rsrc(FINAL ? static_cast<const char*>(p.y) + row0 * s : static_cast<const char*>(p.u),
                  FINAL ? wave_bytes : 0u);
  const uint32_t bc_bytes = (uint32_t)(p.dstate * p.seqlen) * s;
  v.B = make_rsrc(static_cast<const char*>(p.Bm) + b * p.dstate * p.seqlen * s, bc_bytes);
  v.C = make_rsrc(static_cast<const char*>(p.Cm) + b * p.dstate * p.seqlen * s, bc_bytes);
  const uint32_t lane_elem0 = (uint32_t)cw * (uint32_t)L;
  const bool stage_n_ok = tid / 16 < p.dstate;

  const float A2 = (ch_ok && n_ok) ? p.A[d * p.dstate + n] * kLog2e : 0.0f;
  const float bias = (ch_ok && p.bias) ? p.bias[d] : 0.0f;
  const float Dd = (ch_ok && p.D) ? p.D[d] : 0.0f;

  // entry state: the caller's initial state for the first chunk (both
  // passes), the carried state for later chunks of the readout pass
  float h = 0.0f;
  if (chunk == 0) {
    if (p.h0 && ch_ok && n_ok) h = p.h0[ch * p.dstate + n];
  } else if (FINAL && p.carry && ch_ok) {
    h = p.carry[(ch * p.nchunks + chunk) * kStates + n];
  }

  // document ids of this row, one tile ahead like the other operands
  const __amdgpu_buffer_rsrc_t ids =
      make_rsrc(SEQ ? static_cast<const void*>(p.seq_idx + b * p.seqlen) : p.u, SEQ ? (uint32_t)L * 4u : 0u);
  uint32_t id_t = 0, id_prev = 0;
  bool any_start = false;  // a document starts inside this chunk (chunk decay = 0)

  float* pwave = state_tile<FINAL>(sm, wave) + cw * kPChan;
  float* pcol = pwave + n;                // column n of this channel's state tile
  const float* prow = pwave + l * kPRow;  // row l (step l of the block)

  float dt_sum = 0.0f;
  RawOwned<IO> raw;
  BCRaw<IO, PAIR> bcr;
  if (t_begin < t_tile_end) {
    if constexpr (SEQ) load_doc_ids(ids, t_begin + lane, id_t, id_prev);
    load_owned<IO>(raw, v, lane_elem0, t_begin, l);
    load_bc<IO, PAIR>(bcr, v, (uint32_t)L, t_begin, tid, FINAL);
    store_bc<IO, PAIR, FINAL>(sm, 0, bcr, tid, t_valid_end - t_begin, stage_n_ok);
  }
  __syncthreads();

  int buf = 0;
  for (int t0 = t_begin; t0 < t_tile_end; t0 += kTile) {
    const int nvalid = t_valid_end - t0;  // steps of this tile that advance the state
    const int nstop = t_stop - t0;        // steps of this tile that exist in the chunk
    Owned o;
    prep_owned<IO>(o, raw, l, nvalid, bias, softplus, dt_sum);
    if (FINAL && p.ckpt && ch_ok && n_ok) p.ckpt[(ch * p.ckpt_per_row + t0 / kTile) * p.dstate + n] = h;

    uint64_t starts = 0;
    if constexpr (SEQ) {
      starts = doc_starts(id_t, id_prev, t0 + lane, t_valid_end);
      any_start |= starts != 0;
    }

    const int t1 = t0 + kTile;
    const bool more = t1 < t_tile_end;
    if (more) {
      if constexpr (SEQ) load_doc_ids(ids, t1 + lane, id_t, id_prev);
      load_owned<IO>(raw, v, lane_elem0, t1, l);
      load_bc<IO, PAIR>(bcr, v, (uint32_t)L, t1, tid, FINAL);
    }

    const float* sBrow = &sm.B[buf][n][0];
    const float* sCT = ct_row<FINAL>(sm, buf, l);
    const uint32_t elem = lane_elem0 + (uint32_t)t0;
    constexpr auto seq = std::make_integer_sequence<int, 16>{};
    // the 64 steps of the tile; tiles in which a document starts take the
    // copy with the resets
    auto run_tile = [&](auto reset_tag) {
      constexpr bool RESET = decltype(reset_tag)::value;
#define SS_BLOCK(I)                                                                          \
      {                                                                                      \
        CRow cr;                                                                             \
        if constexpr (FINAL) cr = load_crow(sCT + 16 * (I) * kCTRow);                        \
        scan_block<I, FINAL, RESET>(h, o, A2, sBrow, pcol, starts, seq);                     \
        if constexpr (FINAL) {                                                               \
          wave_lds_sync();                                                                   \
          finish_block<IO, I>(o, prow, cr, Dd, need_z, v, elem, l, nvalid, nstop);           \
          wave_lds_sync();                                                                   \
        }                                                                                    \
      }
      SS_BLOCK(0)
      SS_BLOCK(1)
      SS_BLOCK(2)
      SS_BLOCK(3)
#undef SS_BLOCK
    };
    if constexpr (SEQ) {
      if (starts != 0) run_tile(std::true_type{});
      else run_tile(std::false_type{});
    } else {
      run_tile(std::false_type{});
    }

    if (more) store_bc<IO, PAIR, FINAL>(sm, buf ^ 1, bcr, tid, t_valid_end - t1, stage_n_ok);
    __syncthreads();
    buf ^= 1;
  }

  if (FINAL) {
    // steps past the row's length: y = 0, checkpoints hold the frozen state
    for (int t = t_tile_end + l; t < t_stop; t += 16) bstore<IO>(v.y, (lane_elem0 + (uint32_t)t) * s, 0.0f);
    if (p.ckpt && ch_ok && n_ok)
      for (int t0 = t_tile_end; t0 < t_stop; t0 += kTile)
        p.ckpt[(ch * p.ckpt_per_row + t0 / kTile) * p.dstate + n] = h;
    if (p.last_state && ch_ok && n_ok && chunk == p.nchunks - 1) p.last_state[ch * p.dstate + n] = h;
  } else if (ch_ok) {
    // chunk summary: P = exp(A * sum Delta) (= prod of the step decays), S = h
    const float dsum = row_sum(dt_sum);
    const int64_t k = (ch * p.nchunks + chunk) * kStates + n;
    p.aggP[k] = any_start ? 0.0f : exp2_hw(A2 * dsum);
    p.aggS[k] = h;
  }
}

// Pass 2: exclusive scan of the chunk pairs of one channel (forward: the
// entry state of every chunk; reverse = 1, the backward's carried state
// gradient: chunk c is visited as K-1-c).  256 threads per channel: thread
// (g, n), state n fastest so that 16 lanes read one chunk's 64 contiguous
// bytes, serially combines chunks [g*per, (g+1)*per) of state n; the value
// entering each group is then combined from the groups on its left through
// LDS, and each group replays its chunks from it.
__global__ void __launch_bounds__(256) ss_carry_kernel(const float* __restrict__ aggP, const float* __restrict__ aggS,
                                                       float* __restrict__ carry, int64_t nch, int32_t nchunks,
                                                       int32_t reverse) {
  __shared__ float sP[16][16], sS[16][16];
  const int tid = threadIdx.x;
  const int n = tid % 16, g = tid / 16;
  const int64_t ch = blockIdx.x;
  if (ch >= nch) return;  // uniform per workgroup
  const int per = (nchunks + 15) / 16;
  const int c0 = g * per < nchunks ? g * per : nchunks;
  const int c1 = c0 + per < nchunks ? c0 + per : nchunks;
  const int64_t base = ch * nchunks;
  auto slot = [&](int c) { return (base + (reverse ? nchunks - 1 - c : c)) * kStates + n; };

  // local pair over [c0, c1): applying it maps the value entering c0 to the
  // value leaving c1 - 1
  float P = 1.0f, S = 0.0f;
#pragma unroll 4
  for (int c = c0; c < c1; ++c) {
    const float pc = aggP[slot(c)];
    const float sc = aggS[slot(c)];
    S = fmaf(pc, S, sc);
    P *= pc;
  }
  sP[g][n] = P;
  sS[g][n] = S;
  __syncthreads();
  // the value entering group g: groups 0 .. g-1 applied in order to 0
  float E = 0.0f;
  for (int q = 0; q < g; ++q) E = fmaf(sP[q][n], E, sS[q][n]);
#pragma unroll 4
  for (int c = c0; c < c1; ++c) {
    carry[slot(c)] = E;
    E = fmaf(aggP[slot(c)], E, aggS[slot(c)]);
  }
}

// One decode step.  Lane (c, n) of the wave updates state n of channel c;
// the readout sum over n is a DPP row reduction.
template <int IO>
__global__ void __launch_bounds__(kThreads) ss_step_kernel(StepParams p) {
  const int tid = threadIdx.x;
  const int n = tid % 16;
  const int64_t ch = (int64_t)blockIdx.x * kChPerBlock + tid / 16;
  const bool ok = ch < p.batch * p.dim;
  const int64_t b = ok ? ch / p.dim : 0;
  const int64_t d = ok ? ch % p.dim : 0;
  const bool n_ok = n < p.dstate;

  const float u = ok ? load_io<IO>(p.u, ch) : 0.0f;
  const float dl = ok ? load_io<IO>(p.delta, ch) : 0.0f;
  const float bias = (ok && p.bias) ? p.bias[d] : 0.0f;
  const float x = dl + bias;
  const float dt = p.softplus ? softplus_f(x) : x;
  const float A2 = (ok && n_ok) ? p.A[d * p.dstate + n] * kLog2e : 0.0f;
  const float Bn = (ok && n_ok) ? load_io<IO>(p.Bt, b * p.dstate + n) : 0.0f;
  const float Cn = (ok && n_ok) ? load_io<IO>(p.Ct, b * p.dstate + n) : 0.0f;
  const float h0 = (ok && n_ok) ? p.state_in[ch * p.dstate + n] : 0.0f;
  // the skip weight and the gate are loaded with everything else, so the
  // step waits on one round of loads, not two
  const float Dd = (ok && p.D) ? p.D[d] : 0.0f;
  const float zv = (ok && p.z) ? load_io<IO>(p.z, ch) : 0.0f;
  const float h = fmaf(exp2_hw(dt * A2), h0, dt * u * Bn);
  const float y0 = row_sum(Cn * h);
  if (ok && n_ok) p.state_out[ch * p.dstate + n] = h;
  if (ok && n == 0) {
    float yv = y0 + (p.D ? Dd * u : 0.0f);
    if (p.z) yv *= silu_f(zv);
    store_io<IO>(p.y, ch, yv);
  }
}

// Plain device copy, 16 bytes per lane per iteration: the reference kernel
// for HBM bandwidth and for calibrating traffic counters.
__global__ void __launch_bounds__(256) ss_copy_kernel(const float4* __restrict__ src, float4* __restrict__ dst,
                                                      int64_t n16) {
  int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  const int64_t stride = (int64_t)gridDim.x * blockDim.x;
  for (; i < n16; i += stride) dst[i] = src[i];
}

template <int IO, bool PAIR, bool SEQ>
hipError_t launch_fwd_variant(const FwdParams& p, int64_t nchunks, hipStream_t st) {
  const int64_t blocks_per_chunk = p.batch * p.ch_blocks;
  if (nchunks > 1) {
    FwdParams q = p;
    q.chunk_base = 0;
    // pass 1: summaries of chunks 0 .. K-2 (the last chunk's summary is never needed)
    hipLaunchKernelGGL((ss_fwd_chunk_kernel<IO, false, PAIR, SEQ>),
                       dim3((uint32_t)(blocks_per_chunk * (nchunks - 1))), dim3(kThreads), 0, st, q);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    // pass 2: entry states
    e = launch_carry(p.aggP, p.aggS, p.carry, p.batch * p.dim, p.nchunks, false, st);
    if (e != hipSuccess) return e;
  }
  hipLaunchKernelGGL((ss_fwd_chunk_kernel<IO, true, PAIR, SEQ>), dim3((uint32_t)(blocks_per_chunk * nchunks)),
                     dim3(kThreads), 0, st, p);
  return hipGetLastError();
}

template <int IO, bool SEQ>
hipError_t launch_fwd_seq(const FwdParams& p, int64_t nchunks, hipStream_t st) {
  if constexpr (IO != SS_F32) {
    if (p.seqlen % 2 == 0) return launch_fwd_variant<IO, true, SEQ>(p, nchunks, st);
  }
  return launch_fwd_variant<IO, false, SEQ>(p, nchunks, st);
}

template <int IO>
hipError_t launch_fwd_io(const FwdParams& p, int64_t nchunks, hipStream_t st) {
  return p.seq_idx ? launch_fwd_seq<IO, true>(p, nchunks, st) : launch_fwd_seq<IO, false>(p, nchunks, st);
}

template <int IO>
hipError_t launch_step_io(const StepParams& p, hipStream_t st) {
  const int64_t nch = p.batch * p.dim;
  hipLaunchKernelGGL((ss_step_kernel<IO>), dim3((uint32_t)((nch + kChPerBlock - 1) / kChPerBlock)), dim3(kThreads),
                     0, st, p);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_fwd(const FwdParams& p, int64_t nchunks, hipStream_t st) {
  switch (p.io) {
    case SS_F32: return launch_fwd_io<SS_F32>(p, nchunks, st);
    case SS_F16: return launch_fwd_io<SS_F16>(p, nchunks, st);
    default: return launch_fwd_io<SS_BF16>(p, nchunks, st);
  }
}

hipError_t launch_step(const StepParams& p, hipStream_t st) {
  switch (p.io) {
    case SS_F32: return launch_step_io<SS_F32>(p, st);
    case SS_F16: return launch_step_io<SS_F16>(p, st);
    default: return launch_step_io<SS_BF16>(p, st);
  }
}

hipError_t launch_carry(const float* aggP, const float* aggS, float* carry, int64_t nch, int32_t nchunks,
                        bool reverse, hipStream_t st) {
  hipLaunchKernelGGL(ss_carry_kernel, dim3((uint32_t)nch), dim3(256), 0, st, aggP, aggS, carry, nch, nchunks,
                     (int32_t)(reverse ? 1 : 0));
  return hipGetLastError();
}

hipError_t launch_copy(const void* src, void* dst, int64_t bytes, hipStream_t st) {
  const int64_t n16 = bytes / 16;
  int64_t blocks = (n16 + 255) / 256;
  if (blocks > 256 * 16) blocks = 256 * 16;
  if (blocks < 1) blocks = 1;
  hipLaunchKernelGGL(ss_copy_kernel, dim3((uint32_t)blocks), dim3(256), 0, st,
                     reinterpret_cast<const float4*>(src), reinterpret_cast<float4*>(dst), n16);
  return hipGetLastError();
}

}  // namespace ss
