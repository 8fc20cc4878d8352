// ss_fwd.hip -- selective-scan forward: whole-row, time-chunked (look-back) and work-queue scans, decode step (gfx950).
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
// sequence is cut into K chunks of an even number of 64-step tiles, one
// workgroup per (chunk, 16-channel block), all in one launch
// (ss_fwd_lookback_kernel); the workgroup's two 256-thread halves take the
// two halves of the chunk at once.
// Each workgroup first scans its chunk from a zero state (the first chunk
// from the caller's initial state) to get the chunk's pair (P, S) = (prod of
// exp(Delta A) over the chunk, state reached); pairs compose with the
// associative operator (P1,S1) then (P2,S2) = (P2 P1, P2 S1 + S2) (page
// "Mamba", Part V, the combine for h_t = a_t h_{t-1} + b_t).  The pairs are
// published to the other workgroups in two levels: chunks form groups of G
// consecutive chunks; a workgroup composes the pairs of the chunks before it
// in its group, the last one of a group also publishes the group's pair, and
// every workgroup composes the pairs of the groups before its own.  That
// gives its chunk's entry state after two waits, whatever K; it then reruns
// its chunk from that state and writes y.  With K = 1 one workgroup per
// 16-channel block runs the whole row from the initial state (zero unless
// given) in ss_fwd_chunk_kernel.
//
// Packed documents ("niverel-mamba" README, "seq_idx strict reset"): where
// the row's document id changes the state restarts from zero; the decay of
// that step is replaced by 0 (so a chunk holding a document start has P = 0).
// Tiles without a start run the plain code.
#include <type_traits>

#include "ss_device.h"
#include "ss_internal.h"

namespace ss {

namespace {

// flags of a forward launch, fixed at compile time
constexpr int kFlSoftplus = 1;  // Delta = softplus(delta + bias)
constexpr int kFlGate = 2;      // y *= SiLU(z)

// A byte offset that puts every access of a tile out of range: added to a
// lane's offset inside its view (< 2^30: a view spans at most 16 rows of
// 2^24 four-byte elements) it stays below 2^32 and above every view's size,
// so loads return 0 and no branch is needed around the last tile's prefetch.
constexpr uint32_t kTileNone = 0x7fff0000u;

constexpr int kBCStride = kTile + 4;     // padded LDS row of the B tile (floats)
constexpr int kCTRow = 20;               // padded LDS row of the transposed C tile
// The state tile of a channel: 16 steps x 16 states, element (j, n) at
// j*16 + 4*((n>>2) ^ ((j>>2)&3)) + (n&3), channels 272 floats apart.  LDS has
// 32 banks and serves a 4-byte write a half-wave (two channels) at a time:
// 272 = 16 (mod 32) keeps the two channels of a step's write in different
// banks; the XOR swizzle lets the row reads (lane l reads step l's 16 states
// as 4 x 16 bytes, group k from position k ^ ((l>>2)&3), so the groups come
// back in order) run without conflicts too, which a padded row of 20 cannot
// give together with conflict-free writes (both checked with the
// bank-conflict counter on a one-wave probe).
constexpr int kPChan = 16 * 16 + 16;

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

// The channel within its 16-channel block that thread tid works on (wave w
// holds channels 4w .. 4w+3, 16 lanes each).
__device__ __forceinline__ int64_t ss_lane_channel(int tid, int64_t base) {
  return base + (tid / 64) * kChPerWave + (tid % 64) / 16;
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

template <int IO, bool GATE>
__device__ __forceinline__ void load_owned(RawOwned<IO>& r, const Views& v, uint32_t lane_off, uint32_t tile_off) {
  constexpr uint32_t s = io_bytes<IO>();
  const uint32_t base = lane_off + tile_off;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const uint32_t off = base + (uint32_t)(16 * i) * s;
    r.u[i] = bload<IO>(v.u, off);
    r.dl[i] = bload<IO>(v.dl, off);
    if constexpr (GATE) r.z[i] = bload<IO>(v.z, off);
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
__device__ __forceinline__ uint32_t bc_lane_off(uint32_t seqlen, int tid) {
  const int n = tid / 16, j = tid % 16;
  return ((uint32_t)n * seqlen + (uint32_t)(PAIR ? 2 * j : j)) * io_bytes<IO>();
}

template <int IO, bool PAIR>
__device__ __forceinline__ void load_bc(BCRaw<IO, PAIR>& r, const Views& v, uint32_t lane_off, uint32_t tile_off,
                                        bool need_c) {
  constexpr uint32_t s = io_bytes<IO>();
  const uint32_t base = lane_off + tile_off;
#pragma unroll
  for (int k = 0; k < BCRaw<IO, PAIR>::kN; ++k) {
    if constexpr (PAIR) {
      const uint32_t off = base + (uint32_t)(32 * k) * s;
      r.b[k] = __builtin_amdgcn_raw_buffer_load_b32(v.B, off, 0, 0);
      r.c[k] = need_c ? __builtin_amdgcn_raw_buffer_load_b32(v.C, off, 0, 0) : 0u;
    } else {
      const uint32_t off = base + (uint32_t)(16 * k) * s;
      r.b[k] = bload<IO>(v.B, off);
      r.c[k] = need_c ? bload<IO>(v.C, off) : raw_t<IO>(0);
    }
  }
}

// B (row-major, for the state lanes) and C (transposed, for the step owners)
// of steps at or past the valid end are staged as exact zeros, so data past a
// row's length (padding, NaN) never reaches the state or the output.  MASKED =
// false is the copy for a tile whose 64 steps all advance the state, staged
// with all 16 state rows present: every element is kept, so no per-lane
// compare or select is issued.
template <int IO, bool PAIR, bool FINAL, bool MASKED = true>
__device__ __forceinline__ void store_bc(FwdSmem<FINAL>& sm, int buf, const BCRaw<IO, PAIR>& r, int tid, int nvalid,
                                         bool n_ok) {
  const int n = tid / 16, j = tid % 16;
  if constexpr (!MASKED) {
    n_ok = true;
    nvalid = kTile;
  }
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

// Per-(t, d) work of the four owned steps: Delta, Delta*u (zero when masked;
// a FULL tile has no masked step).
template <int IO, int FL, bool FULL>
__device__ __forceinline__ void prep_owned(Owned& o, const RawOwned<IO>& r, int l, int nvalid, float bias,
                                           float& dt_sum) {
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const float u = bits_f32<IO>(r.u[i]);
    const float x = bits_f32<IO>(r.dl[i]) + bias;
    float dt = (FL & kFlSoftplus) ? softplus_f(x) : x;
    float dtu = dt * u;
    if constexpr (!FULL) {
      const bool ok = 16 * i + l < nvalid;
      dt = ok ? dt : 0.0f;
      dtu = ok ? dtu : 0.0f;
    }
    o.dt[i] = dt;
    o.dtu[i] = dtu;
    o.u[i] = u;
    if constexpr ((FL & kFlGate) != 0) o.z[i] = bits_f32<IO>(r.z[i]);
    dt_sum += dt;
  }
}

// 16 steps of block I of the tile.  Lane (c, n) advances state n of channel c
// and (FINAL) leaves h_t[n] in column n of the channel's LDS state tile.  The
// block's 16 B values are read into registers up front, so no LDS wait sits
// between two steps of the recurrence.
template <int I, bool FINAL, bool RESET, int... J>
__device__ __forceinline__ void scan_block(float& h, const Owned& o, float A2, const float* sBrow,
                                           float* const (&pcol)[4], uint64_t starts,
                                           std::integer_sequence<int, J...>) {
  float bq[16];
  *reinterpret_cast<float4*>(&bq[0]) = *reinterpret_cast<const float4*>(sBrow + 16 * I + 0);
  *reinterpret_cast<float4*>(&bq[4]) = *reinterpret_cast<const float4*>(sBrow + 16 * I + 4);
  *reinterpret_cast<float4*>(&bq[8]) = *reinterpret_cast<const float4*>(sBrow + 16 * I + 8);
  *reinterpret_cast<float4*>(&bq[12]) = *reinterpret_cast<const float4*>(sBrow + 16 * I + 12);
  (
      [&] {
        const float a = reset_decay<RESET, 16 * I + J>(exp2_hw(row_bcast<J>(o.dt[I]) * A2), starts);
        h = fmaf(a, h, row_bcast<J>(o.dtu[I]) * bq[J]);
        if constexpr (FINAL) pcol[J >> 2][J * 16] = h;  // element (J, n) of the swizzled tile
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
// y = sum_n C[t][n] h_t[n] + D u in two FMA chains (the skip starts the first).
// ybase is the byte offset of the lane's step 0 of the tile in its y row.
template <int IO, int I, int FL, bool FULL>
__device__ __forceinline__ void finish_block(const Owned& o, const float* const (&prow)[4], const CRow& c, float Dd,
                                             const Views& v, uint32_t ybase, int l, int nvalid, int nstop) {
  const float4 h0 = *reinterpret_cast<const float4*>(prow[0]);  // states 0..3 of step l
  const float4 h1 = *reinterpret_cast<const float4*>(prow[1]);
  const float4 h2 = *reinterpret_cast<const float4*>(prow[2]);
  const float4 h3 = *reinterpret_cast<const float4*>(prow[3]);
  float ya = fmaf(c.c0.x, h0.x, Dd * o.u[I]);
  float yb = c.c0.y * h0.y;
  ya = fmaf(c.c0.z, h0.z, ya); yb = fmaf(c.c0.w, h0.w, yb);
  ya = fmaf(c.c1.x, h1.x, ya); yb = fmaf(c.c1.y, h1.y, yb);
  ya = fmaf(c.c1.z, h1.z, ya); yb = fmaf(c.c1.w, h1.w, yb);
  ya = fmaf(c.c2.x, h2.x, ya); yb = fmaf(c.c2.y, h2.y, yb);
  ya = fmaf(c.c2.z, h2.z, ya); yb = fmaf(c.c2.w, h2.w, yb);
  ya = fmaf(c.c3.x, h3.x, ya); yb = fmaf(c.c3.y, h3.y, yb);
  ya = fmaf(c.c3.z, h3.z, ya); yb = fmaf(c.c3.w, h3.w, yb);
  float yv = ya + yb;
  if constexpr ((FL & kFlGate) != 0) yv *= silu_f(o.z[I]);
  uint32_t off = ybase + (uint32_t)(16 * I) * io_bytes<IO>();
  if constexpr (!FULL) {
    const int tr = 16 * I + l;
    yv = tr < nvalid ? yv : 0.0f;
    off = tr < nstop ? off : kOffNone;
  }
  bstore<IO>(v.y, off, yv);
}

// The scan of one time chunk [chunk * chunk_len, ...) of one (batch row,
// 16-channel block) by one workgroup, from the entry state h; on return h is
// the state after the chunk (after the row's last valid step), dt_sum the
// lane's sum of Delta over its owned steps and any_start whether a document
// starts inside the chunk.  The readout pass (FINAL) writes y for every step
// of the chunk (exact zeros past the row's length) and the checkpoints that
// fall in the chunk, including those past the row's length through
// ckpt_stop.  RANK: the waves lower their arbitration rank as they progress.
// The entry state is ready on the call (no hook), or a hook sets it once the
// chunk's first loads are in flight, so that their latency overlaps its waits
// for other workgroups.
struct EntryReady {
  __device__ void operator()(float&) const {}
};
template <int IO, bool FINAL, bool PAIR, bool SEQ, int FL, bool RANK, bool PAD = false, typename Entry = EntryReady>
__device__ __forceinline__ void scan_chunk(const FwdParams& p, FwdSmem<FINAL>& sm, int64_t b, int64_t cb,
                                           int64_t chunk, int ckpt_stop, float& h, float& dt_sum, bool& any_start,
                                           const Entry& entry = Entry{}, int iters = 0) {
  constexpr uint32_t s = io_bytes<IO>();
  const int tid = threadIdx.x % kThreads;  // within its 256-thread part of the workgroup
  const int wave = uniform(tid / 64);
  const int lane = tid % 64;
  const int cw = lane / 16;  // channel within the wave
  const int n = lane % 16;   // state index; also the time-owner index l
  const int l = n;

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

  constexpr bool GATE = FINAL && (FL & kFlGate) != 0;
  const int64_t row0 = (b * p.dim + d0) * p.seqlen;  // element offset of the wave's first row
  const uint32_t wave_bytes = (uint32_t)(nch_w * p.seqlen) * s;
  Views v;
  v.u = make_rsrc(static_cast<const char*>(p.u) + row0 * s, wave_bytes);
  v.dl = make_rsrc(static_cast<const char*>(p.delta) + row0 * s, wave_bytes);
  v.z = make_rsrc(GATE ? static_cast<const char*>(p.z) + row0 * s : static_cast<const char*>(p.u),
                  GATE ? wave_bytes : 0u);
  v.y = make_rsrc(FINAL ? static_cast<const char*>(p.y) + row0 * s : static_cast<const char*>(p.u),
                  FINAL ? wave_bytes : 0u);
  const uint32_t bc_bytes = (uint32_t)(p.dstate * p.seqlen) * s;
  v.B = make_rsrc(static_cast<const char*>(p.Bm) + b * p.dstate * p.seqlen * s, bc_bytes);
  v.C = make_rsrc(static_cast<const char*>(p.Cm) + b * p.dstate * p.seqlen * s, bc_bytes);
  const uint32_t lane_elem0 = (uint32_t)cw * (uint32_t)L;
  const uint32_t lane_off = (lane_elem0 + (uint32_t)l) * s;  // byte offset of the lane's owned step 0
  const uint32_t bc_off = bc_lane_off<IO, PAIR>((uint32_t)L, tid);
  const bool stage_n_ok = tid / 16 < p.dstate;
  const bool stage_all_n = p.dstate == kStates;  // uniform: every staged state row is valid

  const float A2 = (ch_ok && n_ok) ? p.A[d * p.dstate + n] * kLog2e : 0.0f;
  const float bias = (ch_ok && p.bias) ? p.bias[d] : 0.0f;
  const float Dd = (ch_ok && p.D) ? p.D[d] : 0.0f;

  // document ids of this row, one tile ahead like the other operands
  const __amdgpu_buffer_rsrc_t ids =
      make_rsrc(SEQ ? static_cast<const void*>(p.seq_idx + b * p.seqlen) : p.u, SEQ ? (uint32_t)L * 4u : 0u);
  uint32_t id_t = 0, id_prev = 0;

  // this lane's places in its channel's state tile: column n at rows of each
  // swizzle group (writes), the 4 state groups of row l (reads)
  float* pcol[4] = {};
  const float* prow[4] = {};
  if constexpr (FINAL) {
    float* const pwave = state_tile<FINAL>(sm, wave) + cw * kPChan;
#pragma unroll
    for (int c = 0; c < 4; ++c) {
      pcol[c] = pwave + 4 * ((n >> 2) ^ c) + (n & 3);
      prow[c] = pwave + l * 16 + 4 * (c ^ ((l >> 2) & 3));
    }
  }

  RawOwned<IO> raw, raw2;  // the tile's raw operands and the next tile's, alternating by pass
  BCRaw<IO, PAIR> bcr;
  if (t_begin < t_tile_end) {
    if constexpr (SEQ) load_doc_ids(ids, t_begin + lane, id_t, id_prev);
    load_owned<IO, GATE>(raw, v, lane_off, (uint32_t)t_begin * s);
    load_bc<IO, PAIR>(bcr, v, bc_off, (uint32_t)t_begin * s, FINAL);
  }
  entry(h);  // every thread calls it
  if (t_begin < t_tile_end) store_bc<IO, PAIR, FINAL>(sm, 0, bcr, tid, t_valid_end - t_begin, stage_n_ok);
  __syncthreads();
  int buf = 0;
  // at least `iters` passes of the loop, so that every part of a workgroup
  // meets the same barriers; passes past the chunk's last tile only sync
  const int own_tiles = (t_tile_end - t_begin) / kTile;
  const int n_iter = (PAD && iters > own_tiles) ? iters : own_tiles;
  // One pass per tile.  The two raw sets alternate (a pass converts one and
  // loads the next tile into the other), so the loop's back edge copies no
  // registers: with one set, this tile's lazily converted values and the next
  // tile's loads are live together and the back edge moves one into the other.
  int t0 = t_begin;
  auto pass = [&](const RawOwned<IO>& raw, RawOwned<IO>& raw_next) {
   if (!PAD || t0 < t_tile_end) {  // without PAD every pass has a tile
    const int nvalid = t_valid_end - t0;  // steps of this tile that advance the state
    const int nstop = t_stop - t0;        // steps of this tile that exist in the chunk
    if constexpr (RANK) rank_by_progress(t0 - t_begin, t_tile_end - t_begin);
    if (FINAL && p.ckpt && ch_ok && n_ok) p.ckpt[(ch * p.ckpt_per_row + t0 / kTile) * p.dstate + n] = h;

    uint64_t starts = 0;
    if constexpr (SEQ) {
      starts = doc_starts(id_t, id_prev, t0 + lane, t_valid_end);
      any_start |= starts != 0;
    }

    const int t1 = t0 + kTile;
    const bool more = t1 < t_tile_end;
    // the next tile's operands are loaded whether or not there is one: past
    // the last tile the offset is out of range and the loads return 0
    const uint32_t next_off = more ? (uint32_t)t1 * s : kTileNone;
    if constexpr (SEQ) {
      if (more) load_doc_ids(ids, t1 + lane, id_t, id_prev);
    }

    const float* sBrow = &sm.B[buf][n][0];
    const float* sCT = ct_row<FINAL>(sm, buf, l);
    const uint32_t ybase = lane_off + (uint32_t)t0 * s;
    constexpr auto seq = std::make_integer_sequence<int, 16>{};
    // the 64 steps of the tile: a tile whose steps all advance the state takes
    // the copy without masks, a tile in which a document starts the copy with
    // the resets
    auto run_tile = [&](auto reset_tag, auto full_tag) {
      constexpr bool RESET = decltype(reset_tag)::value;
      constexpr bool FULL = decltype(full_tag)::value;
      Owned o;
      prep_owned<IO, FL, FULL>(o, raw, l, nvalid, bias, dt_sum);
      load_owned<IO, GATE>(raw_next, v, lane_off, next_off);
      load_bc<IO, PAIR>(bcr, v, bc_off, next_off, FINAL);
#define SS_BLOCK(I)                                                                          \
      {                                                                                      \
        CRow cr;                                                                             \
        if constexpr (FINAL) cr = load_crow(sCT + 16 * (I) * kCTRow);                        \
        scan_block<I, FINAL, RESET>(h, o, A2, sBrow, pcol, starts, seq);                     \
        if constexpr (FINAL) {                                                               \
          wave_lds_sync();                                                                   \
          finish_block<IO, I, FL, FULL>(o, prow, cr, Dd, v, ybase, l, nvalid, nstop);        \
          wave_lds_sync();                                                                   \
        }                                                                                    \
      }
      SS_BLOCK(0)
      SS_BLOCK(1)
      SS_BLOCK(2)
      SS_BLOCK(3)
#undef SS_BLOCK
    };
    const bool full = t0 + kTile <= t_valid_end;
    if constexpr (SEQ) {
      if (starts != 0) {
        if (full) run_tile(std::true_type{}, std::true_type{});
        else run_tile(std::true_type{}, std::false_type{});
      } else {
        if (full) run_tile(std::false_type{}, std::true_type{});
        else run_tile(std::false_type{}, std::false_type{});
      }
    } else {
      if (full) run_tile(std::false_type{}, std::true_type{});
      else run_tile(std::false_type{}, std::false_type{});
    }

    if (more) {
      if (stage_all_n && t_valid_end - t1 >= kTile)
        store_bc<IO, PAIR, FINAL, false>(sm, buf ^ 1, bcr, tid, kTile, true);
      else
        store_bc<IO, PAIR, FINAL>(sm, buf ^ 1, bcr, tid, t_valid_end - t1, stage_n_ok);
    }
   }
    __syncthreads();
    buf ^= 1;
    t0 += kTile;
  };
  for (int it = 0; it < n_iter; it += 2) {
    pass(raw, raw2);
    if (it + 1 < n_iter) pass(raw2, raw);
  }

  if constexpr (FINAL) {
    // steps past the row's length: y = 0, checkpoints hold the frozen state
    for (int t = t_tile_end + l; t < t_stop; t += 16) bstore<IO>(v.y, (lane_elem0 + (uint32_t)t) * s, 0.0f);
    if (p.ckpt && ch_ok && n_ok)
      for (int t0 = t_tile_end; t0 < ckpt_stop; t0 += kTile)
        p.ckpt[(ch * p.ckpt_per_row + t0 / kTile) * p.dstate + n] = h;
  }
}

// One workgroup per (batch row, channel block): the whole row, from the
// caller's initial state, when time is not split.
template <int IO, bool PAIR, bool SEQ, int FL>
__global__ void __launch_bounds__(kThreads) ss_fwd_chunk_kernel(FwdParams p) {
  __shared__ FwdSmem<true> sm;
  const int n = threadIdx.x % 16;
  const int64_t d = ss_lane_channel(threadIdx.x, 0);
  // logical block -> (batch row, channel block).  Channel blocks vary
  // fastest: the blocks that share one batch row's B and C tiles run on one
  // XCD, so each row's B and C come from HBM about once.
  const uint32_t lb = xcd_logical_block();
  const uint32_t ncb = (uint32_t)p.ch_blocks;
  const int64_t b = lb / ncb;
  const int64_t cb = lb - (uint32_t)b * ncb;
  const int64_t dd = cb * kChPerBlock + d;
  const bool ch_ok = dd < p.dim, n_ok = n < p.dstate;
  const int64_t ch = b * p.dim + dd;

  float h = (p.h0 && ch_ok && n_ok) ? p.h0[ch * p.dstate + n] : 0.0f;
  float dt_sum = 0.0f;
  bool any_start = false;
  scan_chunk<IO, true, PAIR, SEQ, FL, true>(p, sm, b, cb, 0, (int)p.seqlen, h, dt_sum, any_start);
  if (p.last_state && ch_ok && n_ok) p.last_state[ch * p.dstate + n] = h;
}

// ---- persistent work queue (ragged rows, or more row blocks than fit) -------
// Units are (time chunk, batch row, channel block), handed out in that order
// by an atomic counter, the rows of a chunk longest first; a workgroup takes
// the next unit as soon as it is done with one, so the work of rows of any
// lengths spreads evenly over the GPU.  A unit starts from the state its row
// block reached at the end of the previous chunk, which the workgroup that
// ran that chunk published: the state, then a flag.  That unit was taken
// earlier, by a workgroup that is running, so the wait always ends; it is
// bounded all the same (kSpinLimit polls, then an error is recorded in
// q_ctrl[1] and the unit goes on).
//
// Only the state crosses workgroups (and XCDs, whose L2 caches are not
// coherent with one another).  It is moved with device-scope stores and
// loads, which go to the coherent level themselves, and the flag is raised
// only after every thread's store has completed (waitcnt, then the barrier).
// Release and acquire fences at device scope would also order every other
// store of the workgroup, by writing back and invalidating the whole L2 at
// each unit: measured on the ragged mamba-2.8b workload, 3.0 ms with them
// against 0.53 ms without.

constexpr int kQueueMaxRows = kThreads;  // rows ranked by length in one pass
constexpr int kSpinLimit = 1 << 18;

__device__ __forceinline__ int row_length(const FwdParams& p, int64_t b) {
  const int L = (int)p.seqlen;
  if (!p.lengths) return L;
  const int v = p.lengths[b];
  return v < 0 ? 0 : (v > L ? L : v);
}

// thread 0: wait until the flag is set, bounded
__device__ __forceinline__ void wait_published(const int32_t* flag, int32_t* err) {
  for (int i = 0; i < kSpinLimit; ++i) {
    if (__hip_atomic_load(flag, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) != 0) return;
    __builtin_amdgcn_s_sleep(2);
  }
  __hip_atomic_store(err, 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

template <int IO, bool PAIR, bool SEQ, int FL>
__global__ void __launch_bounds__(kThreads) ss_fwd_queue_kernel(FwdParams p) {
  __shared__ FwdSmem<true> sm;
  __shared__ int64_t s_unit;
  __shared__ int32_t s_order[kQueueMaxRows];
  const int tid = threadIdx.x;
  const int n = tid % 16, l = n;
  const int64_t Bsz = p.batch, cbs = p.ch_blocks, K = p.q_chunks;
  const int L = (int)p.seqlen;
  // rows by decreasing valid length, ties by index (batch <= kQueueMaxRows)
  if (tid < Bsz) {
    const int me = row_length(p, tid);
    int rank = 0;
    for (int64_t r = 0; r < Bsz; ++r) {
      const int o = row_length(p, r);
      rank += (o > me) || (o == me && r < tid);
    }
    s_order[rank] = tid;
  }
  const int64_t per_chunk = Bsz * cbs;
  const int64_t total = K * per_chunk;
  for (;;) {
    __syncthreads();  // the ranking is done; the previous unit is done with s_unit and the tiles
    if (tid == 0) s_unit = (int64_t)atomicAdd(reinterpret_cast<unsigned int*>(p.q_ctrl), 1u);
    __syncthreads();
    const int64_t unit = s_unit;
    if (unit >= total) break;
    const int64_t k = unit / per_chunk;
    const int64_t rem = unit % per_chunk;
    const int64_t b = s_order[rem / cbs];
    const int64_t cb = rem % cbs;
    const int len = row_length(p, b);
    const int64_t kv = len > 0 ? (len - 1) / p.chunk_len : 0;  // the row's last chunk with a valid step
    const int64_t d = ss_lane_channel(tid, cb * kChPerBlock);
    const bool ch_ok = d < p.dim, n_ok = n < p.dstate;
    const int64_t ch = b * p.dim + d;
    const int t_begin = (int)(k * p.chunk_len);
    const int t_stop = t_begin + (int)p.chunk_len < L ? t_begin + (int)p.chunk_len : L;
    if (k > kv) {
      // wholly past the row's length: y = 0 (the checkpoints and the final
      // state there were written by chunk kv)
      if (ch_ok)
        for (int t = t_begin + l; t < t_stop; t += 16) store_io<IO>(p.y, ch * p.seqlen + t, 0.0f);
      continue;
    }
    // the state the previous unit of this row block reached (waited for once
    // this unit's first loads are issued)
    auto entry = [&](float& h) {
      h = 0.0f;
      if (k == 0) {
        if (p.h0 && ch_ok && n_ok) h = p.h0[ch * p.dstate + n];
      } else {
        if (tid == 0) wait_published(p.q_flags + (b * cbs + cb) * K + (k - 1), p.q_ctrl + 1);
        __syncthreads();
        if (ch_ok)
          h = __hip_atomic_load(p.q_carry + (ch * K + (k - 1)) * kStates + n, __ATOMIC_RELAXED,
                                __HIP_MEMORY_SCOPE_AGENT);
      }
    };
    float h = 0.0f, dt_sum = 0.0f;
    bool any_start = false;
    // the row's last valid chunk also writes the checkpoints past its end
    scan_chunk<IO, true, PAIR, SEQ, FL, false>(p, sm, b, cb, k, k == kv ? L : t_stop, h, dt_sum, any_start, entry);
    if (k < kv) {
      if (ch_ok) __hip_atomic_store(p.q_carry + (ch * K + k) * kStates + n, h, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      __builtin_amdgcn_s_waitcnt(0);  // the state has reached the coherent level
      __syncthreads();
      if (tid == 0) __hip_atomic_store(p.q_flags + (b * cbs + cb) * K + k, 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    } else if (p.last_state && ch_ok && n_ok) {
      p.last_state[ch * p.dstate + n] = h;
    }
  }
}

// Clears the queue's counter, error word and flags before a launch (a kernel,
// not a memset, so that a captured graph replays it correctly).
__global__ void __launch_bounds__(256) ss_queue_clear_kernel(int32_t* ctrl, int32_t* flags, int64_t nflags) {
  const int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (i < 2) ctrl[i] = 0;
  for (int64_t j = i; j < nflags; j += (int64_t)gridDim.x * blockDim.x) flags[j] = 0;
}

// ---- time-chunked scan in one launch ----------------------------------------
// Workgroup i runs unit i of the order (chunk, batch row, channel block), so
// a workgroup waits only on workgroups numbered below it.  Those are running
// or done: the launch has at most 2 x 256 - 2 workgroups of 78 KB of LDS (two
// fit per CU), all resident at once on an otherwise idle GPU, and the hardware
// hands out workgroups in order of their number.  (An atomic counter handing
// out units would not need either fact, but its atomics serialise: the last
// unit of the long-sequence workload started 2.9 us after the first.)  Every
// wait is bounded all the same, so no launch can hang.
//
// A pair crosses workgroups (and XCDs, whose L2 caches are not coherent with
// one another) as one 64-bit word, P in the low half and S in the high half,
// stored and loaded with device-scope atomics, so the word is its own flag:
// before the launch every slot is set to kPairEmpty (both halves a NaN with
// every bit set, which the arithmetic does not produce), and a reader polls
// the slots it needs until none holds kPairEmpty (bounded: kSpinLimit polls,
// then the error word q_ctrl[1] is set and the wait ends).  No fence, no
// separate flag: one write and one read per hop.

constexpr uint64_t kPairEmpty = ~(uint64_t)0;
constexpr int kMaxGroup = 32;  // chunks per group, and groups, at most

__device__ __forceinline__ void publish_pair(uint64_t* slot, bool ok, float P, float S) {
  const uint64_t w = (uint64_t)__float_as_uint(P) | ((uint64_t)__float_as_uint(S) << 32);
  if (ok) __hip_atomic_store(slot, w, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// Composes, in order, the m (<= kMaxGroup) pairs at slot[k * stride] into
// (Pc, Sc) (one lane's own slots; nothing when !ok), waiting for each to be
// published; all m loads are in flight at once.
__device__ __forceinline__ void compose_published(const uint64_t* slot, int64_t stride, int m, bool ok, int32_t* err,
                                                  float& Pc, float& Sc) {
  if (!ok) return;
  uint64_t v[kMaxGroup];
#pragma unroll
  for (int k = 0; k < kMaxGroup; ++k)
    if (k < m) v[k] = __hip_atomic_load(slot + k * stride, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  for (int it = 0;; ++it) {
    bool pending = false;
#pragma unroll
    for (int k = 0; k < kMaxGroup; ++k) pending |= k < m && v[k] == kPairEmpty;
    if (!pending) break;
    if (it == kSpinLimit) {
      __hip_atomic_store(err, 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      break;
    }
    __builtin_amdgcn_s_sleep(2);
#pragma unroll
    for (int k = 0; k < kMaxGroup; ++k)
      if (k < m && v[k] == kPairEmpty)
        v[k] = __hip_atomic_load(slot + k * stride, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  }
#pragma unroll
  for (int k = 0; k < kMaxGroup; ++k) {
    if (k < m) {
      const float pk = __uint_as_float((uint32_t)v[k]), sk = __uint_as_float((uint32_t)(v[k] >> 32));
      Sc = fmaf(pk, Sc, sk);
      Pc *= pk;
    }
  }
}

// A workgroup is two 256-thread parts, each the four waves of the row block
// on one half of the chunk (the chunk is an even number of 64-step tiles):
// both halves scan at once, at two waves per SIMD, and meet in LDS, where
// the first half's pair gives the second half its entry state.
template <int IO, bool PAIR, bool SEQ, int FL>
__global__ void __launch_bounds__(2 * kThreads) ss_fwd_lookback_kernel(FwdParams p) {
  __shared__ FwdSmem<true> sm[2];
  __shared__ float sHalf[2][2][kThreads];  // each half's pair (P, S), per lane
  __shared__ float sEntry[kThreads];       // the chunk's entry state, per lane
  const int tid = threadIdx.x % kThreads, half = threadIdx.x / kThreads;  // half: uniform per wave
  const int n = tid % 16;
  // the launch has fewer than 2^23 workgroups: 32-bit index arithmetic (a
  // 64-bit division here delays the first loads by a few hundred cycles, on
  // a path that waits for other workgroups twice)
  const uint32_t nrb = (uint32_t)(p.batch * p.ch_blocks);  // (batch row, channel block) pairs
  const uint32_t ncb = (uint32_t)p.ch_blocks;
  const int64_t K = p.nchunks, NG = p.ngroups;
  const uint32_t G = (uint32_t)p.group;
  const uint32_t c32 = blockIdx.x / nrb, rb = blockIdx.x - c32 * nrb;
  const int64_t c = c32;
  const int64_t b = rb / ncb, cb = rb - (uint32_t)b * ncb;
  const int64_t d = ss_lane_channel(tid, cb * kChPerBlock);
  const bool ch_ok = d < p.dim, n_ok = n < p.dstate;
  const int64_t ch = b * p.dim + d;
  const int64_t g = c32 / G, i = c32 - (uint32_t)g * G;
  const int L = (int)p.seqlen;
  // this half as a chunk of its own: half the length, index 2c + half
  FwdParams q = p;
  q.chunk_len = p.chunk_len / 2;
  const int64_t sc = 2 * c + half;
  const int m = (int)(q.chunk_len / kTile);  // tiles per half
  const int sub_stop = (int)((sc + 1) * q.chunk_len) < L ? (int)((sc + 1) * q.chunk_len) : L;
  const float h_init = (c == 0 && p.h0 && ch_ok && n_ok) ? p.h0[ch * p.dstate + n] : 0.0f;
  uint64_t* const pairs = p.pairs + ch * K * kStates + n;                 // this lane's chunk slots
  uint64_t* const gpairs = p.gpairs + ch * (NG - 1) * kStates + n;       // and group slots

  // 1. each half's pair from a zero state (the first chunk's first half from
  // the initial state, with P = 0 so that the pair carries it), then the
  // chunk's, composed from both in LDS and published (the last chunk's is
  // never needed, but its second half needs the first half's pair)
  {
    float hh = half == 0 ? h_init : 0.0f, dt_sum = 0.0f;
    bool any_start = false;
    scan_chunk<IO, false, PAIR, SEQ, FL & kFlSoftplus, false, true>(q, reinterpret_cast<FwdSmem<false>&>(sm[half]), b,
                                                                    cb, sc, sub_stop, hh, dt_sum, any_start, EntryReady{}, m);
    const float A2 = (ch_ok && n_ok) ? p.A[d * p.dstate + n] * kLog2e : 0.0f;
    const float dsum = row_sum(dt_sum);
    sHalf[half][0][tid] = ((c == 0 && half == 0) || any_start) ? 0.0f : exp2_hw(A2 * dsum);
    sHalf[half][1][tid] = hh;
  }
  __syncthreads();  // both halves' pairs are in LDS; the shared tiles are free for the readout
  const float PA = sHalf[0][0][tid], SA = sHalf[0][1][tid];
  const float P = sHalf[1][0][tid] * PA, S = fmaf(sHalf[1][0][tid], SA, sHalf[1][1][tid]);
  if (half == 0 && c < K - 1) publish_pair(pairs + c * kStates, ch_ok, P, S);

  // 2-4 run inside the readout's start, once its first loads are in flight;
  // the first half waits, the second takes the entry state from it in LDS
  auto entry = [&](float& h) {
    if (half == 0) {
      // 2. the map from the group's entry to this chunk's entry: the pairs of
      // the group's chunks before this one
      float Pe = 1.0f, Se = 0.0f;
      if (i > 0) compose_published(pairs + g * G * kStates, kStates, (int)i, ch_ok, p.q_ctrl + 1, Pe, Se);
      // 3. the last chunk of a group that has a successor publishes the
      // group's pair (so the last group never does: ngroups - 1 group pairs)
      if (i == G - 1 && c < K - 1) publish_pair(gpairs + g * kStates, ch_ok, P * Pe, fmaf(P, Se, S));
      // 4. the state entering the group: the pairs of the groups before it,
      // applied to zero (the first chunk's pair holds the initial state)
      float Pg = 1.0f, H = 0.0f;
      if (g > 0) compose_published(gpairs, kStates, (int)g, ch_ok, p.q_ctrl + 1, Pg, H);
      sEntry[tid] = c == 0 ? h_init : fmaf(Pe, H, Se);
    }
    __syncthreads();  // every thread of both halves calls the hook once
    const float he = sEntry[tid];
    h = half == 0 ? he : fmaf(PA, he, SA);
  };

  // 5. rerun each half from its entry state and write y
  float h = 0.0f, dt_sum = 0.0f;
  bool any_start = false;
  scan_chunk<IO, true, PAIR, SEQ, FL, false, true>(q, sm[half], b, cb, sc, sub_stop, h, dt_sum, any_start, entry, m);
  if (p.last_state && ch_ok && n_ok && c == K - 1 && half == 1) p.last_state[ch * p.dstate + n] = h;
}

// Before a launch of the one-launch time-chunked scan: the error word to zero,
// every pair slot to kPairEmpty.
__global__ void __launch_bounds__(256) ss_pairs_clear_kernel(int32_t* ctrl, uint64_t* slots, int64_t n) {
  const int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (i < 2) ctrl[i] = 0;
  for (int64_t j = i; j < n; j += (int64_t)gridDim.x * blockDim.x) slots[j] = kPairEmpty;
}

// One decode step.  Lane (c, n) of the wave updates state n of channel c;
// the readout sum over n is a DPP row reduction.
template <int IO>
__global__ void __launch_bounds__(kThreads) ss_step_kernel(StepParams p) {
  const int tid = threadIdx.x;
  const int n = tid % 16;
  // the host keeps batch * dim below 2^26, so every index here fits 32 bits
  // (a 64-bit division here sits on the step's critical path)
  const uint32_t dim = (uint32_t)p.dim;
  const uint32_t ch = blockIdx.x * (uint32_t)kChPerBlock + (uint32_t)tid / 16u;
  const bool ok = ch < (uint32_t)(p.batch * p.dim);
  const uint32_t b = ok ? ch / dim : 0u;
  const uint32_t d = ok ? ch - b * dim : 0u;
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

template <int IO, bool PAIR, bool SEQ, int FL>
hipError_t launch_fwd_flags(const FwdParams& p, int64_t nchunks, hipStream_t st) {
  const int64_t blocks_per_chunk = p.batch * p.ch_blocks;
  if (nchunks > 1) {
    int64_t blocks = (p.nslots + 1023) / 1024;
    blocks = blocks < 1 ? 1 : (blocks > 1024 ? 1024 : blocks);
    hipLaunchKernelGGL(ss_pairs_clear_kernel, dim3((uint32_t)blocks), dim3(256), 0, st, p.q_ctrl, p.pairs, p.nslots);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    hipLaunchKernelGGL((ss_fwd_lookback_kernel<IO, PAIR, SEQ, FL>), dim3((uint32_t)(blocks_per_chunk * nchunks)),
                       dim3(2 * kThreads), 0, st, p);
    return hipGetLastError();
  }
  if (p.q_ctrl) {
    const int64_t nflags = blocks_per_chunk * p.q_chunks;
    int64_t blocks = (nflags + 255) / 256;
    blocks = blocks < 1 ? 1 : (blocks > 1024 ? 1024 : blocks);
    hipLaunchKernelGGL(ss_queue_clear_kernel, dim3((uint32_t)blocks), dim3(256), 0, st, p.q_ctrl, p.q_flags, nflags);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    hipLaunchKernelGGL((ss_fwd_queue_kernel<IO, PAIR, SEQ, FL>), dim3((uint32_t)p.q_grid), dim3(kThreads), 0, st, p);
    return hipGetLastError();
  }
  hipLaunchKernelGGL((ss_fwd_chunk_kernel<IO, PAIR, SEQ, FL>), dim3((uint32_t)blocks_per_chunk), dim3(kThreads), 0,
                     st, p);
  return hipGetLastError();
}

template <int IO, bool PAIR, bool SEQ>
hipError_t launch_fwd_variant(const FwdParams& p, int64_t nchunks, hipStream_t st) {
  const int fl = (p.softplus ? kFlSoftplus : 0) | (p.z ? kFlGate : 0);
  switch (fl) {
    case 0: return launch_fwd_flags<IO, PAIR, SEQ, 0>(p, nchunks, st);
    case kFlSoftplus: return launch_fwd_flags<IO, PAIR, SEQ, kFlSoftplus>(p, nchunks, st);
    case kFlGate: return launch_fwd_flags<IO, PAIR, SEQ, kFlGate>(p, nchunks, st);
    default: return launch_fwd_flags<IO, PAIR, SEQ, kFlSoftplus | kFlGate>(p, nchunks, st);
  }
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


}  // namespace ss
