// ss_bwd.hip -- selective-scan backward (gfx950).
//
// Gradient of the loss sum_t dy_t y_t through the recurrence of page
// "Mamba", Part IV Stages 4-6.  Per channel and state, the state gradient
// G_t = dy0_t C_t + a_{t+1} G_{t+1} (dy0 = dy * SiLU(z)) runs backwards in
// time; with it
//   dC_t += dy0_t h_t         dB_t += G_t Delta_t u_t      (summed over channels)
//   du_t  = Delta_t sum_n G_t B_t + dy0_t D
//   dDelta_t = u_t sum_n G_t B_t + sum_n A G_t a_t h_{t-1}
//   dA   += G_t a_t h_{t-1} Delta_t                         (summed over b, t)
//   ddelta_t = dDelta_t * sigmoid(delta_t + bias) when softplus is on.
// The forward states are not stored: they are recomputed chunk by chunk from
// the 64-step checkpoints ss_fwd wrote ("Mamba, on a laptop GPU", "The state
// lives in registers"; "Mamba", Part IV Stage 7).
//
// Passes (chunk = the 64 steps between two checkpoints):
//   AGG   per chunk: P = prod a_t over the chunk, Gz = the gradient leaving the
//         chunk's first step when nothing enters from the right;
//   carry the right-to-left exclusive scan of (P, Gz) gives the gradient
//         entering every chunk from the right (ss_carry_kernel, reversed);
//   MAIN  per chunk: recompute the chunk's 16-step block entry states from
//         the checkpoint, then per block (last first) recompute its 16 states
//         and walk them backwards with the true carried gradient, emit du, ddelta,
//         dz, accumulate dB/dC and dA/dD/dbias partials;
//   REDUCE sum the dA/dD/dbias partials over (batch row, chunk).
// Packed documents: the decay of a step that starts a new document is 0 in
// every recomputation and in the reverse walk, so no gradient crosses a
// document start.  The caller's gradient of the final state seeds the walk
// at the last step, and the gradient left after step 0 is returned as the
// gradient w.r.t. the initial state.
// Lane layout as the forward: a wavefront holds 4 channels x 16 states; the
// per-(t, d) work is owned by lane l = t mod 16 of the channel's row and
// broadcast with DPP; sums over states go through an LDS transpose; sums over
// channels (dB, dC) go through a [step][state][channel] LDS tile per wave,
// whose 4-channel sums each lane accumulates in registers over the
// workgroup's channel loop, then one cross-wave sum and one global atomic per
// element per workgroup (LDS float atomics serialise on gfx950).
#include <atomic>
#include <type_traits>

#include "ss_device.h"
#include "ss_internal.h"

namespace ss {

namespace {

// The carry pass: exclusive scan of the chunk pairs of one channel with the
// associative pair operator (page "Mamba", Part V, the combine for
// h_t = a_t h_{t-1} + b_t); reverse = 1, as the backward's carried state
// gradient runs, visits chunk c as K-1-c.  256 threads per channel: thread
// (g, n), state n fastest so that 16 lanes read one chunk's 64 contiguous
// bytes, serially combines chunks [g*per, (g+1)*per) of state n; the value
// entering each group is then combined from the groups on its left through
// LDS, and each group replays its chunks from it.  Only the first npairs
// visited chunks have a pair; no other pair is read.
__global__ void __launch_bounds__(256) ss_carry_kernel(const float* __restrict__ aggP, const float* __restrict__ aggS,
                                                       float* __restrict__ carry, int64_t nch, int32_t nchunks,
                                                       int32_t npairs, int32_t reverse) {
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
  const int c1p = c1 < npairs ? c1 : npairs;
#pragma unroll 4
  for (int c = c0; c < c1p; ++c) {
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
    if (c < c1p) E = fmaf(aggP[slot(c)], E, aggS[slot(c)]);
  }
}

hipError_t launch_carry(const float* aggP, const float* aggS, float* carry, int64_t nch, int32_t nchunks,
                        int32_t npairs, bool reverse, hipStream_t st) {
  hipLaunchKernelGGL(ss_carry_kernel, dim3((uint32_t)nch), dim3(256), 0, st, aggP, aggS, carry, nch, nchunks,
                     npairs, (int32_t)(reverse ? 1 : 0));
  return hipGetLastError();
}


constexpr int kBCStride = kTile + 4;
// Sum-over-states tiles: per channel 16 steps x 16 states, element (j, n) at
// j*16 + 4*((n>>2) ^ ((j>>2)&3)) + (n&3) (a swizzle that keeps both the
// per-step writes and the per-row reads free of bank conflicts); channels
// 272 floats apart (16 banks).
constexpr int kSChan = 16 * 16 + 16;
// Sum-over-channels tiles: per wave [16 steps][16 states][4 channels], the
// channel slot of states 8..15 swapped in pairs (cw ^ 2).  LDS has 32 banks
// and serves a 4-byte access a half-wave at a time; a half-wave is channels
// {0, 1} (or {2, 3}) x 16 states, which without the swap would put states n
// and n + 8 in the same banks (measured with the bank-conflict counter on a
// one-wave probe).  The channel sum adds the slots as (0 + 1) + (2 + 3),
// which the swap only reorders as a whole, so the sums are unchanged.
constexpr int kCTile = 16 * 16 * kChPerWave;

// AGG stages only the chunk's C (its B tile goes unused); MAIN uses B and C and
// adds its reduction tiles.
template <bool MAIN>
struct BwdSmem {
  float B[kStates][kBCStride];
  float C[kStates][kBCStride];
};
template <>
struct BwdSmem<true> {
  float B[kStates][kBCStride];
  float C[kStates][kBCStride];
  float T1[kWaves][kChPerWave * kSChan];  // G B, summed over states per step
  float T2[kWaves][kChPerWave * kSChan];  // A G a h_{t-1}, summed over states per step
  float T3[kWaves][kCTile];               // G Delta u, summed over channels per (step, state)
  float T4[kWaves][kCTile];               // dy0 h_t, summed over channels per (step, state)
};
static_assert(sizeof(float) * 2 * kWaves * kChPerWave * kSChan >= sizeof(float) * 2 * kWaves * kTile * kStates,
              "the sum-over-states tiles double as the cross-wave staging of dB/dC");

__device__ __forceinline__ int swz(int j, int n) { return j * 16 + 4 * ((n >> 2) ^ ((j >> 2) & 3)) + (n & 3); }

// values of the 4 steps t0 + 16 i + l this lane owns
struct BwdOwned {
  float dt[4], dtu[4], dy0[4], u[4], x[4], z[4], dy[4], y0[4];
  bool valid[4];
};

template <int IO>
struct BwdRaw {
  raw_t<IO> u[4], dl[4], z[4], dy[4];
};

struct BwdViews {
  __amdgpu_buffer_rsrc_t u, dl, z, dy, du, ddl, dz;
};

__device__ __forceinline__ void wave_lds_sync() {
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
  __builtin_amdgcn_wave_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
}

// sum of row l of a swizzled tile (the four 16-byte groups are read in a
// lane-dependent order so that lanes l, l+4, l+8, l+12 hit different banks)
__device__ __forceinline__ float row16_sum(const float* tile, int l) {
  const float* row = tile + l * 16;
  const int x = (l >> 2) & 3;
  const float4 r0 = *reinterpret_cast<const float4*>(row + 4 * (0 ^ x));
  const float4 r1 = *reinterpret_cast<const float4*>(row + 4 * (1 ^ x));
  const float4 r2 = *reinterpret_cast<const float4*>(row + 4 * (2 ^ x));
  const float4 r3 = *reinterpret_cast<const float4*>(row + 4 * (3 ^ x));
  return (((r0.x + r0.y) + (r0.z + r0.w)) + ((r1.x + r1.y) + (r1.z + r1.w))) +
         (((r2.x + r2.y) + (r2.z + r2.w)) + ((r3.x + r3.y) + (r3.z + r3.w)));
}

template <int IO>
__device__ __forceinline__ BwdViews make_views(const BwdParams& p, int64_t b, int64_t d0, bool need_z) {
  constexpr uint32_t s = io_bytes<IO>();
  int64_t nch_w = p.dim - d0;
  nch_w = nch_w < 0 ? 0 : (nch_w > kChPerWave ? kChPerWave : nch_w);
  const int64_t row0 = (b * p.dim + d0) * p.seqlen;
  const uint32_t bytes = (uint32_t)(nch_w * p.seqlen) * s;
  auto at = [&](const void* base) { return static_cast<const char*>(base) + row0 * s; };
  BwdViews v;
  v.u = make_rsrc(at(p.u), bytes);
  v.dl = make_rsrc(at(p.delta), bytes);
  v.dy = make_rsrc(at(p.dy), bytes);
  v.du = make_rsrc(at(p.du), bytes);
  v.ddl = make_rsrc(at(p.ddelta), bytes);
  v.z = make_rsrc(need_z ? at(p.z) : static_cast<const char*>(p.u), need_z ? bytes : 0u);
  v.dz = make_rsrc(need_z ? at(p.dz) : static_cast<const char*>(p.u), need_z ? bytes : 0u);
  return v;
}

template <int IO>
__device__ __forceinline__ void load_raw(BwdRaw<IO>& r, const BwdViews& v, uint32_t lane_elem0, int64_t t0, int l) {
  constexpr uint32_t s = io_bytes<IO>();
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const uint32_t off = (lane_elem0 + (uint32_t)(t0 + 16 * i + l)) * s;
    r.u[i] = bload<IO>(v.u, off);
    r.dl[i] = bload<IO>(v.dl, off);
    r.z[i] = bload<IO>(v.z, off);
    r.dy[i] = bload<IO>(v.dy, off);
  }
}

template <int IO>
__device__ __forceinline__ void prep(BwdOwned& o, const BwdRaw<IO>& r, int64_t t0, int l, int64_t t_end, float bias,
                                     bool softplus, bool need_z) {
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const bool v = t0 + 16 * i + l < t_end;
    const float u = bits_f32<IO>(r.u[i]);
    const float x = bits_f32<IO>(r.dl[i]) + bias;
    float dt = softplus ? softplus_f(x) : x;
    dt = v ? dt : 0.0f;
    const float z = bits_f32<IO>(r.z[i]);
    const float dy = v ? bits_f32<IO>(r.dy[i]) : 0.0f;
    o.dt[i] = dt;
    o.dtu[i] = v ? dt * u : 0.0f;
    o.dy0[i] = v ? (need_z ? dy * silu_f(z) : dy) : 0.0f;
    o.u[i] = u;
    o.x[i] = x;
    o.z[i] = z;
    o.dy[i] = dy;
    o.y0[i] = 0.0f;
    o.valid[i] = v;
  }
}

// ---- AGG: one chunk's gradient with a zero carry --------------------------------
// The reverse recurrence g_{t-1} = a_t (g_t + dy0_t C_t[n]) run from g = 0
// over the chunk, unrolled: the gradient reaching the chunk's entry is
// sum_t P_t dy0_t C_t[n], P_t = prod_{s <= t} a_s = exp2(A log2(e) cs_t), cs_t
// the chunk's running sum of Delta through step t (P_t = 0 from the chunk's
// first document start on).  The terms are independent of one another, so
// each step takes one FMA into the sum and nothing waits on the step before.
template <int I, bool RESET, int... J>
__device__ __forceinline__ void agg_block(float& G, const BwdOwned& o, float cs, float A2, const float* sCrow,
                                          int first, std::integer_sequence<int, J...>) {
  float4 c4;
  (
      [&] {
        constexpr int s = 16 * I + J;
        if constexpr (J % 4 == 0) c4 = *reinterpret_cast<const float4*>(sCrow + s);
        const float cj = (J % 4 == 0) ? c4.x : (J % 4 == 1) ? c4.y : (J % 4 == 2) ? c4.z : c4.w;
        float P = exp2_hw(row_bcast<J>(cs) * A2);
        if constexpr (RESET) P = s >= first ? 0.0f : P;
        G = fmaf(P, row_bcast<J>(o.dy0[I]) * cj, G);
      }(),
      ...);
  G = fresh(G);
  __builtin_amdgcn_sched_barrier(0);  // no hoisting across blocks (registers)
}

// ---- MAIN: forward recompute ---------------------------------------------------
// fwd_pass advances h through block I, keeping the block's 16 decays in
// as[0..16) (and, WITH_Y, leaving the readout terms C h in the sum-over-states
// tile); fwd_states recomputes block I's 16 states from its entry state and
// those decays into hs[0..16] just before the reverse walk needs them, so
// that only 17 states (not 65) are live at once, and no decay is taken twice.
template <int I, bool WITH_Y, bool RESET, int... J>
__device__ __forceinline__ void fwd_pass(float& h, float (&as)[16], const BwdOwned& o, float A2, const float* sBrow,
                                         const float* sCrow, float* t1c, int n, uint64_t starts,
                                         std::integer_sequence<int, J...>) {
  float4 b4, c4;
  (
      [&] {
        constexpr int s = 16 * I + J;
        if constexpr (J % 4 == 0) {
          b4 = *reinterpret_cast<const float4*>(sBrow + s);
          if constexpr (WITH_Y) c4 = *reinterpret_cast<const float4*>(sCrow + s);
        }
        const float bj = (J % 4 == 0) ? b4.x : (J % 4 == 1) ? b4.y : (J % 4 == 2) ? b4.z : b4.w;
        const float a = reset_decay<RESET, s>(exp2_hw(row_bcast<J>(o.dt[I]) * A2), starts);
        as[J] = a;
        h = fmaf(a, h, row_bcast<J>(o.dtu[I]) * bj);
        if constexpr (WITH_Y) {
          const float cj = (J % 4 == 0) ? c4.x : (J % 4 == 1) ? c4.y : (J % 4 == 2) ? c4.z : c4.w;
          t1c[swz(J, n)] = cj * h;
        }
      }(),
      ...);
  h = fresh(h);
  __builtin_amdgcn_sched_barrier(0);  // no hoisting across blocks (registers)
}

template <int I, int... J>
__device__ __forceinline__ void fwd_states(float (&hs)[17], const float (&as)[16], float h0, const BwdOwned& o,
                                           const float* sBrow, std::integer_sequence<int, J...>) {
  float4 b4;
  hs[0] = h0;
  (
      [&] {
        constexpr int s = 16 * I + J;
        if constexpr (J % 4 == 0) b4 = *reinterpret_cast<const float4*>(sBrow + s);
        const float bj = (J % 4 == 0) ? b4.x : (J % 4 == 1) ? b4.y : (J % 4 == 2) ? b4.z : b4.w;
        hs[J + 1] = fmaf(as[J], hs[J], row_bcast<J>(o.dtu[I]) * bj);
      }(),
      ...);
  hs[16] = fresh(hs[16]);
  __builtin_amdgcn_sched_barrier(0);
}

// ---- MAIN: reverse walk of block I -------------------------------------------
// Per step: the per-state terms G B and A G a h_{t-1} go to the sum-over-states
// tiles (their row sums give du and dDelta), the per-channel terms G Delta u
// and dy0 h_t to the sum-over-channels tiles (dB and dC).
template <int I, int... J>
__device__ __forceinline__ void bwd_block(float& g, float& dA_acc, const float (&hs)[17], const float (&as)[16],
                                          const BwdOwned& o, float Anat, const float* sBrow, const float* sCrow, float* t1c,
                                          float* t2c, float* t3w, float* t4w, int n, int cw,
                                          std::integer_sequence<int, J...>) {
  float4 b4, c4;
  // a copy of Delta u of its own, so that the broadcast folds into this block's
  // multiply instead of being shared (as a separate move) with the state recompute
  const float dtu_f = fresh(o.dtu[I]);
  (
      [&] {
        constexpr int jj = 15 - J;
        constexpr int s = 16 * I + jj;
        if constexpr (jj % 4 == 3) {  // steps s-3..s, read when the walk enters them
          b4 = *reinterpret_cast<const float4*>(sBrow + s - 3);
          c4 = *reinterpret_cast<const float4*>(sCrow + s - 3);
        }
        const float bqj = (jj % 4 == 0) ? b4.x : (jj % 4 == 1) ? b4.y : (jj % 4 == 2) ? b4.z : b4.w;
        const float cqj = (jj % 4 == 0) ? c4.x : (jj % 4 == 1) ? c4.y : (jj % 4 == 2) ? c4.z : c4.w;
        const float dtb = row_bcast<jj>(o.dt[I]);
        const float dy0b = row_bcast<jj>(o.dy0[I]);
        const float a = as[jj];               // decay of step s (0 at a document start)
        const float gh = fmaf(dy0b, cqj, g);  // dLoss/dh_t
        t4w[(jj * 16 + n) * kChPerWave + (cw ^ (2 * (n >> 3)))] = dy0b * hs[jj + 1];
        t3w[(jj * 16 + n) * kChPerWave + (cw ^ (2 * (n >> 3)))] = gh * row_bcast<jj>(dtu_f);
        t1c[swz(jj, n)] = gh * bqj;
        g = gh * a;                                 // to h_{t-1}
        const float q = g * hs[jj];                 // gh * a * h_{t-1}
        t2c[swz(jj, n)] = q * Anat;
        dA_acc = fmaf(q, dtb, dA_acc);
      }(),
      ...);
  g = fresh(g);
  dA_acc = fresh(dA_acc);
  __builtin_amdgcn_sched_barrier(0);  // no hoisting across blocks (registers)
}

// Sum of the wave's 4 channel rows for the (step, state) pairs this lane
// collects: step (lane>>4) + 4q, state lane&15, q < 4.
template <int I>
__device__ __forceinline__ void collect_block(float (&accB)[4][4], float (&accC)[4][4], const float* t3w,
                                              const float* t4w, int lane) {
#pragma unroll
  for (int q = 0; q < 4; ++q) {
    const int jj = (lane >> 4) + 4 * q, sn = lane & 15;
    const float4 b4 = *reinterpret_cast<const float4*>(t3w + (jj * 16 + sn) * kChPerWave);
    const float4 c4 = *reinterpret_cast<const float4*>(t4w + (jj * 16 + sn) * kChPerWave);
    accB[I][q] = fresh(accB[I][q] + ((b4.x + b4.y) + (b4.z + b4.w)));
    accC[I][q] = fresh(accC[I][q] + ((c4.x + c4.y) + (c4.z + c4.w)));
  }
}

// The per-lane scalars of one channel block (lane: channel d, state n).
struct BlockScalars {
  float A, bias, Dd, g_last, h_ck, g_in;
};
template <bool MAIN>
__device__ __forceinline__ void load_scalars(BlockScalars& s, const BwdParams& p, int64_t b, int64_t d, int64_t k,
                                             int64_t K, int n) {
  const bool ch_ok = d < p.dim, n_ok = n < p.dstate;
  const int64_t ch = b * p.dim + d;
  s.A = (ch_ok && n_ok) ? p.A[d * p.dstate + n] : 0.0f;
  s.bias = (ch_ok && p.bias) ? p.bias[d] : 0.0f;
  s.Dd = (ch_ok && p.D) ? p.D[d] : 0.0f;
  // gradient entering the chunk from the right with a zero carry; the last
  // chunk also receives the caller's gradient of the final state
  s.g_last = (k == K - 1 && p.dlast && ch_ok && n_ok) ? p.dlast[ch * p.dstate + n] : 0.0f;
  s.h_ck = (MAIN && ch_ok && n_ok) ? p.ckpt[(ch * K + k) * p.dstate + n] : 0.0f;
  s.g_in = (MAIN && k < K - 1 && ch_ok) ? p.gcarry[(ch * K + k) * kStates + n] : 0.0f;
}

// Work units are channel blocks in (batch row, chunk, block) order, block
// fastest.  Workgroup w takes the contiguous units [w U / W, (w + 1) U / W)
// of the U units over W workgroups, as segments that share a (batch row,
// chunk): each segment stages that chunk's B and C once, walks its channel
// blocks, and (MAIN) adds its dB/dC channel sums into the outputs.  AGG runs
// one unit per workgroup; MAIN runs one workgroup per resident slot, so every
// slot gets the same number of units (to within one).  The launch bounds ask
// for at least 2 (MAIN) or 7 (AGG) waves per SIMD: left free, the compiler
// takes MAIN past 256 registers, which leaves one wave per SIMD.
template <int IO, bool MAIN, bool SEQ>
__global__ void __launch_bounds__(kThreads, MAIN ? 2 : 7) ss_bwd_chunk_kernel(BwdParams p) {
  __shared__ BwdSmem<MAIN> sm;
  constexpr uint32_t s = io_bytes<IO>();
  const int tid = threadIdx.x;
  const int wave = uniform(tid / 64);
  const int lane = tid % 64;
  const int cw = lane / 16, n = lane % 16, l = n;

  const int64_t K = p.nchunks;
  const int64_t U = p.batch * K * p.ch_blocks;
  const int64_t W = gridDim.x;
  const int64_t w = xcd_logical_block();
  // AGG: exactly unit w (its grid is U workgroups)
  const int64_t u_begin = MAIN ? w * U / W : w;
  const int64_t u_end = MAIN ? (w + 1) * U / W : w + 1;
  const bool need_z = p.z != nullptr;
  const bool softplus = p.softplus != 0;
  const uint32_t L = (uint32_t)p.seqlen;
  const float* sBrow = &sm.B[n][0];
  const float* sCrow = &sm.C[n][0];
  constexpr auto seq = std::make_integer_sequence<int, 16>{};

  for (int64_t unit = u_begin; unit < u_end;) {
    const int64_t bk = unit / p.ch_blocks;
    const int64_t k = bk % K;
    const int64_t b = bk / K;
    const int64_t cb_begin = unit % p.ch_blocks;
    const int64_t cb_end =
        !MAIN ? cb_begin + 1 : (cb_begin + (u_end - unit) < p.ch_blocks ? cb_begin + (u_end - unit) : p.ch_blocks);
    unit += cb_end - cb_begin;

    const int64_t t0 = k * kTile;
    const int64_t t_end = t0 + kTile < p.seqlen ? t0 + kTile : p.seqlen;

    __syncthreads();  // the previous segment is done with the B/C and staging tiles
    // stage the chunk's B and C (shared by every channel of this batch row)
    {
      const uint32_t bc_bytes = (uint32_t)(p.dstate * p.seqlen) * s;
      const char* bbase = static_cast<const char*>(p.Bm) + b * p.dstate * p.seqlen * s;
      const char* cbase = static_cast<const char*>(p.Cm) + b * p.dstate * p.seqlen * s;
      const __amdgpu_buffer_rsrc_t rB = make_rsrc(bbase, bc_bytes), rC = make_rsrc(cbase, bc_bytes);
      const int sn = tid / 16, j = tid % 16;
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const int e = j + 16 * q;
        const bool ok = sn < p.dstate && t0 + e < t_end;
        const uint32_t off = ((uint32_t)sn * L + (uint32_t)(t0 + e)) * s;
        // AGG reads only C
        const float bv = MAIN ? bits_f32<IO>(bload<IO>(rB, off)) : 0.0f;
        const float cv = bits_f32<IO>(bload<IO>(rC, off));
        if constexpr (MAIN) sm.B[sn][e] = ok ? bv : 0.0f;
        sm.C[sn][e] = ok ? cv : 0.0f;
      }
    }
    // document starts among the chunk's steps (every wave computes the mask)
    uint64_t starts = 0;
    if constexpr (SEQ) {
      const __amdgpu_buffer_rsrc_t ids = make_rsrc(p.seq_idx + b * p.seqlen, L * 4u);
      uint32_t id_t, id_prev;
      load_doc_ids(ids, (int)t0 + lane, id_t, id_prev);
      starts = doc_starts(id_t, id_prev, (int)t0 + lane, (int)t_end);
    }
    __syncthreads();

    float accB[4][4], accC[4][4];
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
      for (int q = 0; q < 4; ++q) accB[i][q] = accC[i][q] = 0.0f;

    // Every load of a channel block is issued one block ahead, while the
    // previous block is computed: its inputs, its weights and (MAIN) its
    // checkpoint and carried gradient.  Loads complete in issue order for the
    // wait counter, so nothing else is loaded between two blocks' prefetches.
    const bool n_ok = n < p.dstate;
    const uint32_t lane_elem0 = (uint32_t)cw * L;
    BwdRaw<IO> raw;
    BlockScalars cur, nxt;
    if (cb_begin < cb_end) {
      load_scalars<MAIN>(cur, p, b, cb_begin * kChPerBlock + wave * kChPerWave + cw, k, K, n);
      load_raw<IO>(raw, make_views<IO>(p, b, cb_begin * kChPerBlock + wave * kChPerWave, need_z), lane_elem0, t0, l);
    }
    for (int64_t cb = cb_begin; cb < cb_end; ++cb) {
      const int64_t d0 = cb * kChPerBlock + wave * kChPerWave;
      const int64_t d = d0 + cw;
      const bool ch_ok = d < p.dim;
      const int64_t ch = b * p.dim + d;
      const BwdViews v = make_views<IO>(p, b, d0, need_z);

      const float A = cur.A;
      const float A2 = A * kLog2e;
      const float bias = cur.bias;
      const float Dd = cur.Dd;
      BwdOwned o;
      prep<IO>(o, raw, t0, l, t_end, bias, softplus, need_z);
      __builtin_amdgcn_sched_barrier(0);
      if (cb + 1 < cb_end) {
        load_scalars<MAIN>(nxt, p, b, d + kChPerBlock, k, K, n);
        load_raw<IO>(raw, make_views<IO>(p, b, d0 + kChPerBlock, need_z), lane_elem0, t0, l);
      }
      __builtin_amdgcn_sched_barrier(0);
      const int64_t wslot = ((ch * K + k) * kStates + n);
      const float g_last = cur.g_last;
      // chunks in which no document starts take the copy without the resets
      const bool reset = SEQ && starts != 0;
      if constexpr (!MAIN) {
        // running sums of Delta at the lane's owned steps 16 i + l
        float cs[4], run = 0.0f;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const float r = row_scan(o.dt[i]);
          cs[i] = run + r;
          run += row_bcast<15>(r);  // the block's total
        }
        const int first = starts != 0 ? (int)__builtin_ctzll(starts) : kTile;  // uniform
        float G = 0.0f;
        auto walk = [&](auto reset_tag) {
          constexpr bool R = decltype(reset_tag)::value;
          agg_block<0, R>(G, o, cs[0], A2, sCrow, first, seq);
          agg_block<1, R>(G, o, cs[1], A2, sCrow, first, seq);
          agg_block<2, R>(G, o, cs[2], A2, sCrow, first, seq);
          agg_block<3, R>(G, o, cs[3], A2, sCrow, first, seq);
        };
        if (reset) walk(std::bool_constant<SEQ>{});
        else walk(std::false_type{});
        // the whole chunk's decay, which also carries the caller's gradient of
        // the final state (last chunk) to the chunk's entry
        const float P = starts != 0 ? 0.0f : exp2_hw(A2 * run);
        if (ch_ok) {
          p.aggP[wslot] = P;
          p.aggG[wslot] = fmaf(P, g_last, G);
        }
      } else {
        float* t1c = sm.T1[wave] + cw * kSChan;  // this channel's sum-over-states tiles
        float* t2c = sm.T2[wave] + cw * kSChan;
        float* t3w = sm.T3[wave];
        float* t4w = sm.T4[wave];
        // first pass: entry state of each 16-step block (and y0 when gated)
        float hb[4], ac[4][16];  // block entry states, the chunk's decays
        float h = cur.h_ck;
        auto recompute = [&](auto reset_tag) {
          constexpr bool R = decltype(reset_tag)::value;
          if (need_z) {
#define SS_FWD_Y(I)                                                         \
    hb[I] = h;                                                                \
    fwd_pass<I, true, R>(h, ac[I], o, A2, sBrow, sCrow, t1c, n, starts, seq); \
    wave_lds_sync();                                                        \
    o.y0[I] = fmaf(Dd, o.u[I], row16_sum(t1c, l));                          \
    wave_lds_sync();
            SS_FWD_Y(0)
            SS_FWD_Y(1)
            SS_FWD_Y(2)
            SS_FWD_Y(3)
#undef SS_FWD_Y
          } else {
            hb[0] = h;
            fwd_pass<0, false, R>(h, ac[0], o, A2, sBrow, sCrow, t1c, n, starts, seq);
            hb[1] = h;
            fwd_pass<1, false, R>(h, ac[1], o, A2, sBrow, sCrow, t1c, n, starts, seq);
            hb[2] = h;
            fwd_pass<2, false, R>(h, ac[2], o, A2, sBrow, sCrow, t1c, n, starts, seq);
            hb[3] = h;
            fwd_pass<3, false, R>(h, ac[3], o, A2, sBrow, sCrow, t1c, n, starts, seq);  // its decays
          }
        };
        if (reset) recompute(std::bool_constant<SEQ>{});
        else recompute(std::false_type{});

        float g = (k < K - 1 && ch_ok) ? cur.g_in : g_last;
        float dA_acc = 0.0f, dD_acc = 0.0f, db_acc = 0.0f;
#define SS_BWD(I)                                                                                   \
    {                                                                                                 \
      float hs[17];                                                                                   \
      o.dt[I] = fresh(o.dt[I]);                                                                       \
      o.dtu[I] = fresh(o.dtu[I]);                                                                     \
      o.dy0[I] = fresh(o.dy0[I]);                                                                     \
      fwd_states<I>(hs, ac[I], hb[I], o, sBrow, seq);                                                 \
      bwd_block<I>(g, dA_acc, hs, ac[I], o, A, sBrow, sCrow, t1c, t2c, t3w, t4w, n, cw, seq);         \
      wave_lds_sync();                                                                                \
      const float sGB = row16_sum(t1c, l);                                                            \
      const float sQA = row16_sum(t2c, l);                                                            \
      collect_block<I>(accB, accC, t3w, t4w, lane);                                                   \
      const float du = fmaf(o.dt[I], sGB, o.dy0[I] * Dd);                                             \
      const float dD = fmaf(o.u[I], sGB, sQA);                                                        \
      float dx = softplus ? dD * sigmoid_f(o.x[I]) : dD;                                              \
      dx = o.valid[I] ? dx : 0.0f;                                                                    \
      const int64_t t = t0 + 16 * (I) + l;                                                            \
      const uint32_t off = (o.valid[I] && ch_ok) ? (lane_elem0 + (uint32_t)t) * s : kOffNone;         \
      bstore<IO>(v.du, off, o.valid[I] ? du : 0.0f);                                                  \
      bstore<IO>(v.ddl, off, dx);                                                                     \
      if (need_z) {                                                                                   \
        const float sz = sigmoid_f(o.z[I]);                                                           \
        const float dz = o.dy[I] * o.y0[I] * sz * fmaf(o.z[I], 1.0f - sz, 1.0f);                      \
        bstore<IO>(v.dz, off, o.valid[I] ? dz : 0.0f);                                                \
      }                                                                                               \
      dD_acc = fmaf(o.dy0[I], o.u[I], dD_acc);                                                        \
      db_acc += dx;                                                                                   \
      wave_lds_sync();                                                                                \
    }
        SS_BWD(3)
        SS_BWD(2)
        SS_BWD(1)
        SS_BWD(0)
#undef SS_BWD
        // the gradient left after step 0 is the gradient w.r.t. the initial state
        if (k == 0 && p.dh0 && ch_ok && n_ok) p.dh0[ch * p.dstate + n] = g;
        // partial sums of this (batch row, chunk) for the reduction pass
        const int64_t bk = b * K + k;
        if (ch_ok) p.aggP[(bk * p.dim + d) * kStates + n] = dA_acc;
        const float dDs = row_sum(dD_acc);
        const float dbs = row_sum(db_acc);
        if (ch_ok && n == 0) {
          p.aggG[bk * p.dim + d] = dDs;
          p.aggG[p.batch * K * p.dim + bk * p.dim + d] = dbs;
        }
      }
      cur = nxt;
    }

    if constexpr (MAIN) {
      // sum the four waves' channel sums, then one global add per element
      __syncthreads();
      float* stB = &sm.T1[0][0];                      // [wave][64 steps][16 states]
      float* stC = stB + kWaves * kTile * kStates;
#pragma unroll
      for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          const int st = 16 * i + (lane >> 4) + 4 * q, sn = lane & 15;
          stB[(wave * kTile + st) * kStates + sn] = accB[i][q];
          stC[(wave * kTile + st) * kStates + sn] = accC[i][q];
        }
      __syncthreads();
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        // (step, state) pair; the opaque copy keeps the compiler from holding
        // these addresses in registers (spilled) through the whole walk
        const int idx = opaque(tid) + kThreads * r;
        const int st = idx / kStates, sn = idx % kStates;
        float vb = 0.0f, vc = 0.0f;
#pragma unroll
        for (int w = 0; w < kWaves; ++w) {
          vb += stB[(w * kTile + st) * kStates + sn];
          vc += stC[(w * kTile + st) * kStates + sn];
        }
        if (sn < p.dstate && t0 + st < t_end) {
          const int64_t gi = (b * p.dstate + sn) * p.seqlen + t0 + st;
          unsafeAtomicAdd(p.dB + gi, vb);
          unsafeAtomicAdd(p.dC + gi, vc);
        }
      }
    }
  }  // segment
}

// Zero up to five float buffers in one launch (the atomic targets of the
// backward: dB, dC, dA, dD, dbias); a null buffer has count 0.
struct ZeroList {
  float* ptr[5];
  int64_t count[5];
};
__global__ void __launch_bounds__(256) ss_zero_kernel(ZeroList z) {
  const int64_t stride = (int64_t)gridDim.x * blockDim.x;
#pragma unroll
  for (int k = 0; k < 5; ++k)
    for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < z.count[k]; i += stride) z.ptr[k][i] = 0.0f;
}

// dA[d, n] = sum over (batch row, chunk) partials; dD, dbias likewise.  The
// (batch row, chunk) range is split over gridDim.y groups whose partial sums
// are added atomically into the zeroed outputs.
__global__ void __launch_bounds__(256) ss_bwd_reduce_kernel(const float* __restrict__ dApart,
                                                            const float* __restrict__ dDpart,
                                                            const float* __restrict__ dbpart, float* __restrict__ dA,
                                                            float* __restrict__ dD, float* __restrict__ dbias,
                                                            int64_t dim, int64_t dstate, int64_t nbk) {
  const int64_t idx = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  const int64_t d = idx / kStates;
  const int n = (int)(idx % kStates);
  if (d >= dim) return;
  const int64_t per = (nbk + gridDim.y - 1) / gridDim.y;
  const int64_t bk0 = (int64_t)blockIdx.y * per;
  const int64_t bk1 = bk0 + per < nbk ? bk0 + per : nbk;
  if (bk0 >= bk1) return;
  float acc = 0.0f;
#pragma unroll 8
  for (int64_t bk = bk0; bk < bk1; ++bk) acc += dApart[(bk * dim + d) * kStates + n];
  if (n < dstate) unsafeAtomicAdd(dA + d * dstate + n, acc);
  if (n == 0 && dD) {
    float s = 0.0f;
#pragma unroll 8
    for (int64_t bk = bk0; bk < bk1; ++bk) s += dDpart[bk * dim + d];
    unsafeAtomicAdd(dD + d, s);
  }
  if (n == 1 && dbias) {
    float s = 0.0f;
#pragma unroll 8
    for (int64_t bk = bk0; bk < bk1; ++bk) s += dbpart[bk * dim + d];
    unsafeAtomicAdd(dbias + d, s);
  }
}

// MAIN workgroups resident per CU: 76 KB of LDS and at most 256 registers per
// lane (2 waves per SIMD, held there by the kernel's launch bounds) each allow
// two.
constexpr int64_t kMainPerCu = 2;

hipError_t zero_outputs(const BwdParams& p, hipStream_t st) {
  ZeroList z{};
  const int64_t nbc = p.batch * p.dstate * p.seqlen;
  z.ptr[0] = p.dB; z.count[0] = nbc;
  z.ptr[1] = p.dC; z.count[1] = nbc;
  z.ptr[2] = p.dA; z.count[2] = p.dim * p.dstate;
  z.ptr[3] = p.dD; z.count[3] = p.dD ? p.dim : 0;
  z.ptr[4] = p.dbias; z.count[4] = p.dbias ? p.dim : 0;
  int64_t blocks = (nbc + 255) / 256;
  if (blocks > 4096) blocks = 4096;
  if (blocks < 1) blocks = 1;
  hipLaunchKernelGGL(ss_zero_kernel, dim3((uint32_t)blocks), dim3(256), 0, st, z);
  return hipGetLastError();
}

template <int IO, bool SEQ>
hipError_t launch_bwd_seq(const BwdParams& p, hipStream_t st) {
  const int64_t K = p.nchunks;
  hipError_t e = zero_outputs(p, st);  // every atomic target, before any kernel adds into it
  if (e != hipSuccess) return e;
  // MAIN: one workgroup per resident slot, each over an equal share of the
  // channel-block units (to within one), so that every slot finishes at about
  // the same time; a workgroup adds its dB/dC channel sums atomically once
  // per (batch row, chunk) it touches.
  const int64_t bk = p.batch * K;
  const int64_t units = bk * p.ch_blocks;
  const int64_t resident = kMainPerCu * device_cus();
  const dim3 grid((uint32_t)(units < resident ? units : resident));
  if (K > 1) {
    // AGG has nothing to reduce over channels: one channel block per workgroup
    hipLaunchKernelGGL((ss_bwd_chunk_kernel<IO, false, SEQ>), dim3((uint32_t)units), dim3(kThreads), 0, st, p);
    e = hipGetLastError();
    if (e != hipSuccess) return e;
    e = launch_carry(p.aggP, p.aggG, p.gcarry, p.batch * p.dim, (int32_t)K, (int32_t)K, true, st);
    if (e != hipSuccess) return e;
  }
  hipLaunchKernelGGL((ss_bwd_chunk_kernel<IO, true, SEQ>), grid, dim3(kThreads), 0, st, p);
  e = hipGetLastError();
  if (e != hipSuccess) return e;
  const int64_t threads = p.dim * kStates;
  // at most 16 groups of (batch row, chunk) partials: fewer atomic adds into
  // each output (16 measured faster than 8 or 33 on the backward workload)
  int64_t groups_y = (bk + 15) / 16;
  if (groups_y > 16) groups_y = 16;
  hipLaunchKernelGGL(ss_bwd_reduce_kernel, dim3((uint32_t)((threads + 255) / 256), (uint32_t)groups_y), dim3(256), 0,
                     st, p.aggP, p.aggG, p.aggG + p.batch * K * p.dim, p.dA, p.dD, p.dbias, p.dim, p.dstate, bk);
  return hipGetLastError();
}

template <int IO>
hipError_t launch_bwd_io(const BwdParams& p, hipStream_t st) {
  return p.seq_idx ? launch_bwd_seq<IO, true>(p, st) : launch_bwd_seq<IO, false>(p, st);
}

}  // namespace

// Compute units of the current device, asked once per device (256 if the
// runtime cannot say).
int64_t device_cus() {
  static std::atomic<int64_t> cached[64];
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return 256;
  int64_t v = cached[dev].load(std::memory_order_relaxed);
  if (v == 0) {
    int n = 0;
    v = (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) == hipSuccess && n > 0) ? n : 256;
    cached[dev].store(v, std::memory_order_relaxed);
  }
  return v;
}

hipError_t launch_bwd(const BwdParams& p, hipStream_t st) {
  switch (p.io) {
    case SS_F32: return launch_bwd_io<SS_F32>(p, st);
    case SS_F16: return launch_bwd_io<SS_F16>(p, st);
    default: return launch_bwd_io<SS_BF16>(p, st);
  }
}

}  // namespace ss
