// ss_ssd.hip -- Mamba-2 structured state-space (SSD) chunked scan on MFMA (gfx950).
//
// Page "Mamba" (walkthrough), "Deep dive: Mamba-2 and state-space duality":
// with A a scalar times the identity per head, the selective SSM of a head
// (state H[p][n], headdim P x dstate N, B and C shared by a group of heads)
//   H_t = a_t H_{t-1} + Delta_t x_t B_t^T,   y_t = H_t C_t + D x_t,
//   a_t = exp(Delta_t A_h),
// is also a masked quadratic attention, and the chunked algorithm computes it
// with dense matmuls: inside a chunk of Q = 256 steps the output is
//   Y_diag = (L o C B^T) (Delta x),  L[i, j] = exp(cs_i - cs_j) (j <= i),
// with cs the cumulative sum of Delta A over the chunk; between chunks one
// state is passed forward:
//   S_c = sum_j exp(cs_last - cs_j) Delta_j x_j B_j^T   (the chunk's own state)
//   H_in(c + 1) = exp(cs_last(c)) H_in(c) + S_c,  H_in(0) = h0,
//   Y_off = diag(exp(cs_i)) C H_in(c).
// Two kernels:
//   ssd_state_kernel  per (batch, head, slice of 32 states), walking the
//                     chunks in order: S_c on MFMA (K = Q) added into the
//                     decayed state held in the accumulators, each chunk's
//                     entry state written in the I/O dtype, the final state
//                     in fp32; after the walk the workgroups of a group
//                     share out its C B^T (summed in fp32, kept as bf16;
//                     once per group rather than per head);
//   ssd_scan_kernel   per (batch, chunk, head): Y_off = C H_in on MFMA, then
//                     per 64-step piece of the chunk's columns M = the decay-
//                     masked, Delta-scaled C B^T built in registers and
//                     Y_diag += M x on MFMA; D skip, SiLU(z) gate, store.
// MFMA: v_mfma_f32_16x16x32_{bf16,f16}, fp32 accumulation.  Operand lane
// layout (checked on the chip): A[m][k] in lane m + 16 (k / 8), element k % 8;
// B[k][n] in lane n + 16 (k / 8), element k % 8; D[m][n] in lane
// n + 16 (m / 4), element m % 4.  Operands whose k axis is time (x, B) are
// copied to LDS as time-major rows, the layout they have in memory, and read
// back as fragments with the transposing LDS read (tm_frag).
#include "ss_device.h"
#include "ss_internal.h"

namespace ss {
namespace {

constexpr int kQ = 256;      // chunk length
constexpr int kP = 64;       // headdim
constexpr int kJB = 64;      // time piece of a chunk staged at once
constexpr int kSsdThreads = 256;

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4v __attribute__((ext_vector_type(4)));

template <int IO> struct mfma_t;
template <> struct mfma_t<SS_BF16> {
  using V = bf16x8;
  static __device__ __forceinline__ f32x4 run(V a, V b, f32x4 c) {
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
  }
};
template <> struct mfma_t<SS_F16> {
  using V = f16x8;
  static __device__ __forceinline__ f32x4 run(V a, V b, f32x4 c) {
    return __builtin_amdgcn_mfma_f32_16x16x32_f16(a, b, c, 0, 0, 0);
  }
};

// 16-bit storage bits of v in the I/O dtype (round to nearest even)
template <int IO>
__device__ __forceinline__ uint16_t bits16(float v) {
  return __builtin_bit_cast(uint16_t, from_f32<IO>(v));
}
// two values packed low-first into one word of the I/O dtype (one packed
// hardware conversion, round to nearest even)
typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef _Float16 f16x2 __attribute__((ext_vector_type(2)));
template <int IO>
__device__ __forceinline__ uint32_t pack2(float lo, float hi) {
  if constexpr (IO == SS_BF16)
    return __builtin_bit_cast(uint32_t, __builtin_convertvector(f32x2{lo, hi}, bf16x2));
  else
    return __builtin_bit_cast(uint32_t, __builtin_convertvector(f32x2{lo, hi}, f16x2));
}
template <int IO>
__device__ __forceinline__ typename mfma_t<IO>::V as_vec(u32x4v w) {
  return __builtin_bit_cast(typename mfma_t<IO>::V, w);
}

// A range-checked view of the steps [t0, t0 + kQ) of one batch row: `at`
// points at step t0 (wave-uniform), `row` is the byte distance between
// steps, and steps at or past seqlen read as zeros through the hardware's
// range check.  No load is predicated, so none forces an early wait (a load
// under a branch must complete before the branch joins).  The host keeps a
// chunk of any operand below 2^31 bytes.
__device__ __forceinline__ __amdgpu_buffer_rsrc_t chunk_view(const void* at, int64_t row, int64_t t0, int64_t seqlen) {
  const int64_t n = seqlen - t0 < kQ ? seqlen - t0 : kQ;
  return make_rsrc(at, at ? (uint32_t)(n * row) : 0u);
}
__device__ __forceinline__ u32x4v vload16(__amdgpu_buffer_rsrc_t r, uint32_t off) {
  return __builtin_bit_cast(u32x4v, __builtin_amdgcn_raw_buffer_load_b128(r, off, 0, 0));
}
__device__ __forceinline__ uint2 vload8(__amdgpu_buffer_rsrc_t r, uint32_t off) {
  return __builtin_bit_cast(uint2, __builtin_amdgcn_raw_buffer_load_b64(r, off, 0, 0));
}

// Time-major tiles in LDS (row = step, W 16-bit columns, 16-byte chunks of a
// row rotated by (row / 4) so that both the row writes and the transposing
// reads below are free of bank conflicts).  Element offset of (row, col):
template <int W>
__device__ __forceinline__ int tm_off(int row, int col) {
  return row * W + 8 * ((col >> 3) ^ ((row >> 2) & (W / 8 - 1))) + (col & 7);
}
// An MFMA operand fragment whose k axis is time, read from a time-major
// tile with ds_read_b64_tr_b16 (gfx950; lane layout checked on the chip: in
// each group of 16 lanes, lane i receives element i % 4 of the 4-element
// reads of lanes i / 4 + 4q, q = 0..3).  Lane j of group g reads 4 columns
// c0 + 4 (j % 4) .. + 3 of row r0 + 8 g + 4 h + j / 4 (h = 0, 1), so lane i
// ends with column c0 + i at the 8 steps r0 + 8 g .. + 7: A[m = i][k] or
// B[k][n = i] of v_mfma_f32_16x16x32.
typedef short s16x4 __attribute__((ext_vector_type(4)));
typedef short s16x8 __attribute__((ext_vector_type(8)));
// For r0 a multiple of 32 the rotation does not depend on r0, so a lane's
// read address is r0 * W plus a per-lane offset: tm_lane_off gives it (h = 0
// for steps r0 + 8 g .. + 3, h = 1 for the next 4) and tm_frag reads the
// fragment at tile + r0 * W.
template <int W>
__device__ __forceinline__ int tm_lane_off(int c0, int h, int lane) {
  const int j = lane % 16, g = lane / 16;
  return tm_off<W>(8 * g + 4 * h + j / 4, c0 + 4 * (j % 4));
}
__device__ __forceinline__ u32x4v tm_frag(const uint16_t* at, int off_lo, int off_hi) {
  const s16x4 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((__attribute__((address_space(3))) s16x4*)(at + off_lo));
  const s16x4 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((__attribute__((address_space(3))) s16x4*)(at + off_hi));
  return __builtin_bit_cast(u32x4v, __builtin_shufflevector(lo, hi, 0, 1, 2, 3, 4, 5, 6, 7));
}

// Delta of this thread's step and the inclusive cumulative sum cs of Delta * A
// over the chunk (threads 0..255 = steps; steps past the sequence have Delta =
// 0).  cs goes to sCs; every thread of the workgroup must call it (it holds
// two barriers).
template <int IO>
__device__ __forceinline__ float chunk_cumsum(const SsdParams& p, float dt_raw, bool valid, float A, float bias,
                                              float* sCs, float* sWave) {
  const int tid = threadIdx.x, lane = tid % 64, wave = tid / 64;
  float delta = 0.0f;
  if (tid < kQ && valid) {
    const float xd = dt_raw + bias;
    delta = p.softplus ? softplus_f(xd) : xd;
  }
  float v = delta * A;
#pragma unroll
  for (int off = 1; off < 64; off <<= 1) {
    const float o = __shfl_up(v, off, 64);
    if (lane >= off) v += o;
  }
  if (tid < kQ && lane == 63) sWave[wave] = v;
  __syncthreads();
  if (tid < kQ) {
    float base = 0.0f;
    for (int w = 0; w < wave; ++w) base += sWave[w];
    sCs[tid] = v + base;
  }
  __syncthreads();
  return delta;
}

// cs for the whole chunk in every wave from the chunk's Delta (sDelta, one
// value per step): lane l takes steps 4 l .. 4 l + 3, sums them in order, and
// an inclusive scan of the lane totals (DPP row shifts 1, 2, 4, 8, then row
// broadcasts 15 and 31) gives each lane the sum of the steps before its own.
template <int CTRL, int ROW_MASK, bool BOUND_ZERO>
__device__ __forceinline__ float dpp_scan_step(float v) {
  return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), CTRL, ROW_MASK, 0xf, BOUND_ZERO));
}
__device__ __forceinline__ void wave_chunk_cumsum(const float* sDelta, float A, float (&delta)[4], float (&cs)[4]) {
  const int lane = threadIdx.x % 64;
  const float4 d4 = *reinterpret_cast<const float4*>(&sDelta[4 * lane]);
  delta[0] = d4.x; delta[1] = d4.y; delta[2] = d4.z; delta[3] = d4.w;
  float run = 0.0f;
#pragma unroll
  for (int e = 0; e < 4; ++e) {
    run = fmaf(delta[e], A, run);
    cs[e] = run;
  }
  float v = run;
  v += dpp_scan_step<0x111, 0xf, true>(v);   // row_shr:1
  v += dpp_scan_step<0x112, 0xf, true>(v);   // row_shr:2
  v += dpp_scan_step<0x114, 0xf, true>(v);   // row_shr:4
  v += dpp_scan_step<0x118, 0xf, true>(v);   // row_shr:8
  v += dpp_scan_step<0x142, 0xa, false>(v);  // row_bcast:15 into rows 1 and 3
  v += dpp_scan_step<0x143, 0xc, false>(v);  // row_bcast:31 into rows 2 and 3
  const float before = v - run;
#pragma unroll
  for (int e = 0; e < 4; ++e) cs[e] += before;
}

// ---- C B^T of a chunk, once per group -------------------------------------------
// CB[i][j] = sum_n C_i[n] B_j[n] (summed in fp32, stored as bf16) for the chunk's rows i and the columns j
// of every 64-step piece up to the one holding i (the causal half plus the rest
// of the diagonal pieces, so the output pass never reads an unwritten value):
// 160 tiles of 16 x 16.  Tile idx: row band R = rt / 4 holds 4 (R + 1) column
// tiles per row tile, and the bands start at idx 0, 16, 48, 96.
constexpr int kCbTiles = 160;
__device__ __forceinline__ void cb_tile_of(int idx, int& rt, int& jt) {
  const int R = idx < 16 ? 0 : idx < 48 ? 1 : idx < 96 ? 2 : 3;
  const int local = idx - 8 * R * (R + 1), ncols = 4 * (R + 1);
  rt = 4 * R + local / ncols;
  jt = local % ncols;
}
template <int IO, int N>
struct CbTile {
  u32x4v a[N / 32], b[N / 32];  // C rows 16 rt .., B rows 16 jt .. (8 states per lane and k-step)
  int rt, jt;
  __device__ __forceinline__ void load(const SsdParams& p, int64_t b_, int64_t c, int64_t g, int idx, int lane) {
    cb_tile_of(idx, rt, jt);
    const int64_t t0 = c * kQ, crow = p.ngroups * N * 2;
    const int64_t at = ((b_ * p.seqlen + t0) * p.ngroups + g) * N * 2;
    const auto cv = chunk_view(static_cast<const char*>(p.Cm) + at, crow, t0, p.seqlen);
    const auto bv = chunk_view(static_cast<const char*>(p.Bm) + at, crow, t0, p.seqlen);
    const uint32_t ri = (uint32_t)((16 * rt + lane % 16) * crow), rj = (uint32_t)((16 * jt + lane % 16) * crow);
#pragma unroll
    for (int ks = 0; ks < N / 32; ++ks) {
      const uint32_t n0 = (uint32_t)(32 * ks + 8 * (lane / 16)) * 2u;
      a[ks] = vload16(cv, ri + n0);
      b[ks] = vload16(bv, rj + n0);
    }
  }
  __device__ __forceinline__ void finish(const SsdParams& p, int64_t b_, int64_t c, int64_t g, int lane) {
    // the tile transposed, (B C^T)[j][i], so that a lane holds 4 consecutive
    // columns j = 16 jt + 4 (lane / 16) + r of one row i = 16 rt + lane % 16:
    // one 8-byte bf16 store per lane
    f32x4 acc = f32x4{0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
    for (int ks = 0; ks < N / 32; ++ks) acc = mfma_t<IO>::run(as_vec<IO>(b[ks]), as_vec<IO>(a[ks]), acc);
    uint16_t* CB = p.ws_cb + ((b_ * p.nchunks + c) * p.ngroups + g) * (int64_t)(kQ * kQ);
    *reinterpret_cast<uint2*>(CB + (16 * rt + lane % 16) * kQ + 16 * jt + 4 * (lane / 16)) =
        make_uint2(pack2<SS_BF16>(acc[0], acc[1]), pack2<SS_BF16>(acc[2], acc[3]));
  }
};

// ---- pass 1: chunk states and the state passed between chunks ---------------------
// Workgroup = (batch row, head, slice of 32 states).  It walks the chunks in
// order with its slice of the state H[p][n] (64 x 32) in the accumulators:
//   entry(c) = H   (stored in the I/O dtype for the output pass)
//   H <- exp(cs_last) H + sum_j exp(cs_last - cs_j) Delta_j x_j B_j^T
// The j-sum runs on the matrix cores: x * w and B are copied to LDS as
// time-major rows and read back as operand fragments with the transposing LDS
// read; wave w holds rows p in [16w, 16w + 16).  The next chunk's x, B and dt
// are loaded once this chunk's are in LDS, while it is being multiplied.  After
// the walk the waves of a group's workgroups (heads x slices x 4) share out
// the C B^T tiles of every chunk of the row.
constexpr int kNS = 32;  // states per slice
template <int IO, int N, bool SEQ>
__global__ void __launch_bounds__(kSsdThreads, 3) ssd_state_kernel(SsdParams p) {
  using M = mfma_t<IO>;
  constexpr int kSlices = N / kNS;
  __shared__ __attribute__((aligned(16))) float sW[kQ];
  __shared__ __attribute__((aligned(16))) float sDelta[kQ];
  __shared__ __attribute__((aligned(16))) uint16_t sX[kQ * kP];   // x * w, time-major (tm_off<64>)
  __shared__ __attribute__((aligned(16))) uint16_t sB[kQ * kNS];  // B of the slice, time-major (tm_off<32>)
  __shared__ int s_lr[2];  // SEQ: the chunk's last document start (-1: none), by chunk parity
  const int tid = threadIdx.x, lane = tid % 64, wave = tid / 64;
  const int64_t lb = xcd_logical_block();  // the workgroups of one row's group share B in an XCD's L2
  const int s = (int)(lb % kSlices);
  const int64_t h = (lb / kSlices) % p.nheads;
  const int64_t b = lb / (kSlices * p.nheads);
  const int64_t hpg = p.nheads / p.ngroups, g = h / hpg;
  const int64_t xrow = p.nheads * kP * 2, brow = p.ngroups * N * 2;
  const char* xbase = static_cast<const char*>(p.x) + ((b * p.seqlen) * p.nheads + h) * kP * 2;
  const char* bbase = static_cast<const char*>(p.Bm) + ((b * p.seqlen) * p.ngroups + g) * N * 2 + s * kNS * 2;
  const float A = p.A[h], bias = p.dt_bias ? p.dt_bias[h] : 0.0f;

  // x: 2048 16-byte pieces (step tid / 8 + 32 k, channels 8 (tid % 8) ..), eight per thread;
  // B: 1024 pieces (step tid / 4 + 64 k, states 8 (tid % 4) ..), four per thread
  const char* dtbase = static_cast<const char*>(p.dt) + (b * p.seqlen * p.nheads + h) * 2;
  // SEQ: the row's document ids through one range-checked view (step -1 and
  // steps past the row read as 0); step tid's id and its predecessor's
  const auto idv = make_rsrc(SEQ ? p.seq_idx + b * p.seqlen : nullptr, SEQ ? (uint32_t)(p.seqlen * 4) : 0u);
  uint32_t idr = 0, idpr = 0;
  u32x4v xr[8], br[4];
  raw_t<IO> dtr = 0;  // dt of step tid (raw bits)
  auto load_chunk = [&](int64_t c) {
    const int64_t t0 = c * kQ;
    if constexpr (SEQ) load_doc_ids(idv, (int)(t0 + tid), idr, idpr);
    const auto xv = chunk_view(xbase + t0 * xrow, xrow, t0, p.seqlen);
    const auto bv = chunk_view(bbase + t0 * brow, brow, t0, p.seqlen);
    const auto dv = chunk_view(dtbase + t0 * p.nheads * 2, p.nheads * 2, t0, p.seqlen);
#pragma unroll
    for (int k = 0; k < 8; ++k) xr[k] = vload16(xv, (uint32_t)((tid / 8 + 32 * k) * xrow + (tid % 8) * 16));
#pragma unroll
    for (int k = 0; k < 4; ++k) br[k] = vload16(bv, (uint32_t)((tid / 4 + 64 * k) * brow + (tid % 4) * 16));
    dtr = bload<IO>(dv, (uint32_t)(tid * p.nheads * 2));
  };

  // the state slice: lane holds p = 16 w + 4 (lane / 16) + r, n = 32 s + 16 nt + lane % 16
  f32x4 acc[2];
  const int64_t hbase = (b * p.nheads + h) * (int64_t)(kP * N);
#pragma unroll
  for (int nt = 0; nt < 2; ++nt)
#pragma unroll
    for (int r = 0; r < 4; ++r)
      acc[nt][r] = p.h0 ? p.h0[hbase + (16 * wave + 4 * (lane / 16) + r) * N + kNS * s + 16 * nt + lane % 16] : 0.0f;
  const int cb_slot = (int)(((h % hpg) * kSlices + s) * 4 + wave), cb_slots = (int)(hpg * kSlices * 4);
  // per-lane offsets of the fragment reads: x at channels 16 w .., B at states 16 nt ..
  const int xo0 = tm_lane_off<kP>(16 * wave, 0, lane), xo1 = tm_lane_off<kP>(16 * wave, 1, lane);
  const int bo[2][2] = {{tm_lane_off<kNS>(0, 0, lane), tm_lane_off<kNS>(0, 1, lane)},
                        {tm_lane_off<kNS>(16, 0, lane), tm_lane_off<kNS>(16, 1, lane)}};

  if (SEQ && tid < 2) s_lr[tid] = -1;
  __syncthreads();
  load_chunk(0);
  for (int64_t c = 0; c < p.nchunks; ++c) {
    const int64_t t0 = c * kQ;
    {  // Delta of step tid (0 past the sequence)
      float d = 0.0f;
      if (t0 + tid < p.seqlen) {
        const float xd = bits_f32<IO>(dtr) + bias;
        d = p.softplus ? softplus_f(xd) : xd;
      }
      sDelta[tid] = d;
      if constexpr (SEQ) {  // a document starts at step tid
        if (t0 + tid > 0 && t0 + tid < p.seqlen && idr != idpr) atomicMax(&s_lr[c & 1], tid);
      }
    }
    __syncthreads();
    // documents: only the steps from the chunk's last document start on feed
    // the state that leaves the chunk, and a start inside it drops the
    // entering state (the state is zero before every start)
    int lr = -1;
    if constexpr (SEQ) {
      lr = s_lr[c & 1];
      if (tid == 0) s_lr[(c + 1) & 1] = -1;
    }
    float delta[4], cs[4];
    wave_chunk_cumsum(sDelta, A, delta, cs);
    const float cs_last = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(cs[3]), 63));
    if (lane / 16 == wave) {  // this wave's quarter of the chunk: steps 4 lane .. 4 lane + 3
      float4 w;
      w.x = exp2_hw((cs_last - cs[0]) * kLog2e) * delta[0];  // 0 past the sequence (Delta = 0)
      w.y = exp2_hw((cs_last - cs[1]) * kLog2e) * delta[1];
      w.z = exp2_hw((cs_last - cs[2]) * kLog2e) * delta[2];
      w.w = exp2_hw((cs_last - cs[3]) * kLog2e) * delta[3];
      if constexpr (SEQ) {
        const int j = 4 * lane;
        w.x = j + 0 >= lr ? w.x : 0.0f;
        w.y = j + 1 >= lr ? w.y : 0.0f;
        w.z = j + 2 >= lr ? w.z : 0.0f;
        w.w = j + 3 >= lr ? w.w : 0.0f;
      }
      *reinterpret_cast<float4*>(&sW[4 * lane]) = w;
    }
    __syncthreads();
#pragma unroll
    for (int k = 0; k < 8; ++k) {  // x * w, one step per piece
      const int row = tid / 8 + 32 * k;
      const float sc = sW[row];
      u32x4v v;
#pragma unroll
      for (int q = 0; q < 4; ++q)
        v[q] = pack2<IO>(bits_f32<IO>((raw_t<IO>)(xr[k][q] & 0xffffu)) * sc,
                         bits_f32<IO>((raw_t<IO>)(xr[k][q] >> 16)) * sc);
      *reinterpret_cast<u32x4v*>(&sX[tm_off<kP>(row, 8 * (tid % 8))]) = v;
    }
#pragma unroll
    for (int k = 0; k < 4; ++k)
      *reinterpret_cast<u32x4v*>(&sB[tm_off<kNS>(tid / 4 + 64 * k, 8 * (tid % 4))]) = br[k];
    __syncthreads();
    if (c + 1 < p.nchunks) load_chunk(c + 1);  // lands while chunk c is multiplied

    // entry state of chunk c, then H <- decay H + S_c
    // stored [n][p]: the lane's 4 consecutive channels p of state n in one 8-byte store
    uint16_t* E = p.ws_entry + ((b * p.nchunks + c) * p.nheads + h) * (int64_t)(kP * N);
#pragma unroll
    for (int nt = 0; nt < 2; ++nt)
      *reinterpret_cast<uint2*>(&E[(kNS * s + 16 * nt + lane % 16) * kP + 16 * wave + 4 * (lane / 16)]) =
          make_uint2(pack2<IO>(acc[nt][0], acc[nt][1]), pack2<IO>(acc[nt][2], acc[nt][3]));
    const float decay = lr >= 0 ? 0.0f : exp2_hw(cs_last * kLog2e);
#pragma unroll
    for (int nt = 0; nt < 2; ++nt) acc[nt] *= decay;
#pragma unroll
    for (int ks = 0; ks < kQ; ks += 32) {
      const u32x4v a = tm_frag(sX + ks * kP, xo0, xo1);  // A[m = p][k = step]
#pragma unroll
      for (int nt = 0; nt < 2; ++nt) {
        const u32x4v bb = tm_frag(sB + ks * kNS, bo[nt][0], bo[nt][1]);  // B[k = step][n]
        acc[nt] = M::run(as_vec<IO>(a), as_vec<IO>(bb), acc[nt]);
      }
    }
    __syncthreads();
  }
  // C B^T of every chunk, shared out over the waves of the group's
  // workgroups after the walk (so that its operands hold no registers through
  // it), each tile's operands loaded while the previous tile is multiplied
  {
    const int64_t total = p.nchunks * kCbTiles;
    int64_t item = cb_slot;
    CbTile<IO, N> cur;
    if (item < total) cur.load(p, b, item / kCbTiles, g, (int)(item % kCbTiles), lane);
    while (item < total) {
      const int64_t nxt = item + cb_slots;
      CbTile<IO, N> nx;
      if (nxt < total) nx.load(p, b, nxt / kCbTiles, g, (int)(nxt % kCbTiles), lane);
      cur.finish(p, b, item / kCbTiles, g, lane);
      cur = nx;
      item = nxt;
    }
  }
  if (p.final_state) {
#pragma unroll
    for (int nt = 0; nt < 2; ++nt)
#pragma unroll
      for (int r = 0; r < 4; ++r)
        p.final_state[hbase + (16 * wave + 4 * (lane / 16) + r) * N + kNS * s + 16 * nt + lane % 16] = acc[nt][r];
  }
}

// ---- pass 3: outputs of a chunk -------------------------------------------------
// Y is built transposed, Y^T[p][i], so that each lane ends up with 4
// consecutive channels p of one step i.  The chunk's 256 rows are 8 blocks of
// 32; waves w and w + 4 take the two 16-row halves of blocks w and 7 - w, so
// every wave does the same causal work (block r needs column pieces
// 0 .. r / 2 of 64 steps).
//   Y^T = H_in C^T scaled by exp(cs_i)   (A = H_in from LDS, B = C^T)
//       + x^T M^T                        (A = x^T from LDS, B = M^T built in registers)
// with M[i][j] = CB[i][j] exp(cs_i - cs_j) Delta_j for j <= i.  Off the
// diagonal piece the decay factors through the piece's last step e:
// exp(cs_i - cs_e) * exp(cs_e - cs_j), both at most 1 there, so one exp per
// lane is enough; the diagonal piece takes the exp per element.  Global loads
// are issued ahead of their use: all prologue operands at once, each piece's
// CB two pieces ahead, the gate z right after the first block's first CB
// pieces (loads complete in issue order for the wait counter, so a load
// issued earlier than those would delay the first piece).
constexpr int kScanThreads = 512;
template <int IO, int N, bool SEQ>
__global__ void __launch_bounds__(kScanThreads, 4) ssd_scan_kernel(SsdParams p) {
  using M = mfma_t<IO>;
  __shared__ __attribute__((aligned(16))) float sDelta[kQ];
  __shared__ __attribute__((aligned(16))) float sCs[kQ];
  __shared__ __attribute__((aligned(16))) float sWp[kQ];           // exp(cs_e - cs_j) Delta_j, e = end of j's piece
  __shared__ float sWave[4];
  __shared__ __attribute__((aligned(16))) int sSeg[kQ];            // SEQ: document starts at or before each step
  __shared__ int sSegW[4];
  __shared__ __attribute__((aligned(16))) uint16_t sX[kQ * kP];    // x of the chunk, time-major (tm_off<64>)
  __shared__ __attribute__((aligned(16))) uint16_t sH[N * kP];     // entry state H_in, rows n of 64 p (tm_off<64>)
  const int tid = threadIdx.x, lane = tid % 64, wave = tid / 64;
  const int64_t lb = xcd_logical_block();  // the heads of one chunk run on one XCD and share its C, CB in L2
  const int64_t h = lb % p.nheads;
  const int64_t c = (lb / p.nheads) % p.nchunks;
  const int64_t b = lb / (p.nheads * p.nchunks);
  const int64_t g = h / (p.nheads / p.ngroups);
  const int64_t t0 = c * kQ;
  const int half = wave / 4;
  const int blk[2] = {wave % 4, 7 - wave % 4};
  const int64_t crow = p.ngroups * N * 2;  // bytes between steps of B and C
  const int64_t xrow = p.nheads * kP * 2;  // bytes between steps of x, z, y
  const char* cbase = static_cast<const char*>(p.Cm) + ((b * p.seqlen) * p.ngroups + g) * N * 2;
  const char* xbase = static_cast<const char*>(p.x) + ((b * p.seqlen) * p.nheads + h) * kP * 2;
  const uint16_t* Hin = p.ws_entry + ((b * p.nchunks + c) * p.nheads + h) * (int64_t)(kP * N);

  // ---- prologue: issue every operand load, then scan Delta A and fill LDS
  const auto xv = chunk_view(xbase + t0 * xrow, xrow, t0, p.seqlen);
  u32x4v xr[4];  // 16-byte pieces of x: step tid / 8 + 64 k, channels 8 (tid % 8) ..
#pragma unroll
  for (int k = 0; k < 4; ++k) xr[k] = vload16(xv, (uint32_t)((tid / 8 + 64 * k) * xrow + (tid % 8) * 16));
  constexpr int kHPieces = N * (kP / 8);  // 16-byte pieces of H_in (stored [n][p])
  constexpr int kHItems = (kHPieces + kScanThreads - 1) / kScanThreads;
  u32x4v hr[kHItems];
#pragma unroll
  for (int k = 0; k < kHItems; ++k) {
    const int item = tid + kScanThreads * k;
    hr[k] = item < kHPieces ? *reinterpret_cast<const u32x4v*>(Hin + item * 8) : u32x4v{0u, 0u, 0u, 0u};
  }
  const auto dv = chunk_view(static_cast<const char*>(p.dt) + ((b * p.seqlen + t0) * p.nheads + h) * 2, p.nheads * 2,
                             t0, p.seqlen);
  const raw_t<IO> dt_bits = bload<IO>(dv, tid < kQ ? (uint32_t)(tid * p.nheads * 2) : kOffNone);
  uint32_t idr = 0, idpr = 0;  // SEQ: document ids of step tid and of the step before it
  if constexpr (SEQ) {
    const auto idv = make_rsrc(p.seq_idx + b * p.seqlen, (uint32_t)(p.seqlen * 4));
    load_doc_ids(idv, (int)(t0 + tid), idr, idpr);
  }
  const auto cv = chunk_view(cbase + t0 * crow, crow, t0, p.seqlen);
  u32x4v cf[2][N / 32];
#pragma unroll
  for (int q = 0; q < 2; ++q)
#pragma unroll
    for (int ks = 0; ks < N / 32; ++ks)
      cf[q][ks] = vload16(cv, (uint32_t)((32 * blk[q] + 16 * half + lane % 16) * crow + (32 * ks + 8 * (lane / 16)) * 2));

  // x and H_in into LDS, then Delta and its cumulative sum (threads 0..255 = steps)
#pragma unroll
  for (int k = 0; k < 4; ++k) *reinterpret_cast<u32x4v*>(&sX[tm_off<kP>(tid / 8 + 64 * k, 8 * (tid % 8))]) = xr[k];
#pragma unroll
  for (int k = 0; k < kHItems; ++k) {
    const int item = tid + kScanThreads * k;
    if (item < kHPieces) *reinterpret_cast<u32x4v*>(&sH[tm_off<kP>(item / 8, 8 * (item % 8))]) = hr[k];
  }
  // documents: step i of the chunk sees the state entering the chunk only
  // before the chunk's first document start, and step j's input only from
  // the same document (no start in (j, i]): sSeg[i] counts the starts at or
  // before i (threads 0..255 = steps; per-wave counts in sSegW first)
  uint64_t starts = 0;
  if constexpr (SEQ) {
    starts = __builtin_amdgcn_ballot_w64(tid < kQ && t0 + tid > 0 && t0 + tid < p.seqlen && idr != idpr);
    if (tid < kQ && lane == 0) sSegW[wave] = (int)__builtin_popcountll(starts);
  }
  {
    const float delta = chunk_cumsum<IO>(p, bits_f32<IO>(dt_bits), tid < kQ && t0 + tid < p.seqlen, p.A[h],
                                         p.dt_bias ? p.dt_bias[h] : 0.0f, sCs, sWave);
    if (tid < kQ) {
      sDelta[tid] = delta;
      sWp[tid] = exp2_hw((sCs[tid | (kJB - 1)] - sCs[tid]) * kLog2e) * delta;
    }
  }
  if constexpr (SEQ) {
    if (tid < kQ) {  // sSegW is ordered by the barriers of the cumulative sum
      int before = 0;
      for (int w = 0; w < wave; ++w) before += sSegW[w];
      const uint64_t upto = lane == 63 ? ~0ull : ((2ull << lane) - 1);
      sSeg[tid] = before + (int)__builtin_popcountll(starts & upto);
    }
  }

  // ---- Y_off = H_in C^T, scaled by exp(cs_i)
  f32x4 acc[2][4];  // [block][p tile]: p = 16 pt + 4 (lane / 16) + r, i = 32 blk + 16 half + lane % 16
#pragma unroll
  for (int q = 0; q < 2; ++q)
#pragma unroll
    for (int pt = 0; pt < 4; ++pt) acc[q][pt] = f32x4{0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
  for (int ks = 0; ks < N / 32; ++ks) {
#pragma unroll
    for (int pt = 0; pt < 4; ++pt) {  // A[m = p][k = n] from the [n][p] tile
      const u32x4v hf = tm_frag(sH + 32 * ks * kP, tm_lane_off<kP>(16 * pt, 0, lane), tm_lane_off<kP>(16 * pt, 1, lane));
#pragma unroll
      for (int q = 0; q < 2; ++q) acc[q][pt] = M::run(as_vec<IO>(hf), as_vec<IO>(cf[q][ks]), acc[q][pt]);
    }
  }
#pragma unroll
  for (int q = 0; q < 2; ++q) {
    const float sc = exp2_hw(sCs[32 * blk[q] + 16 * half + lane % 16] * kLog2e);
#pragma unroll
    for (int pt = 0; pt < 4; ++pt) acc[q][pt] *= sc;
  }

  uint2 zv[2][4];
  __syncthreads();  // sDelta, sWp, sSeg
  if constexpr (SEQ) {  // the entering state reaches only the steps before the first start
#pragma unroll
    for (int q = 0; q < 2; ++q)
      if (sSeg[32 * blk[q] + 16 * half + lane % 16] != 0)
#pragma unroll
        for (int pt = 0; pt < 4; ++pt) acc[q][pt] = f32x4{0.0f, 0.0f, 0.0f, 0.0f};
  }

  // ---- Y_diag += x^T M^T, piece by piece (mask: the chunk holds a document
  // start, so M also keeps only pairs of steps of one document)
  const uint16_t* CBbase = p.ws_cb + ((b * p.nchunks + c) * p.ngroups + g) * (int64_t)(kQ * kQ);
  const bool mask = SEQ && sSeg[kQ - 1] != 0;  // uniform
#pragma unroll
  for (int q = 0; q < 2; ++q) {
    const int i = 32 * blk[q] + 16 * half + lane % 16;  // this lane's row (chunk-local)
    const int segi = SEQ ? sSeg[i] : 0;
    const int dpiece = 32 * blk[q] / kJB;               // the piece holding the block's rows (at most 3)
    const float csi = sCs[i];
    const uint16_t* cbrow = CBbase + i * kQ + 8 * (lane / 16);
    // CB of each piece (8 bf16 columns per lane and k-step), loaded two pieces ahead
    u32x4v cbv[kQ / kJB][2];
#pragma unroll
    for (int pc = 0; pc < 2; ++pc)
      if (pc <= dpiece)
#pragma unroll
        for (int ks = 0; ks < 2; ++ks) cbv[pc][ks] = *reinterpret_cast<const u32x4v*>(cbrow + kJB * pc + 32 * ks);
    if (q == 0) {  // the gate, loaded once the first pieces' C B^T are on their way
      // gate values for the epilogue: lane has channels 16 pt + 4 (lane / 16) .. + 3 of its step
      const auto zw = chunk_view(p.z ? static_cast<const char*>(p.z) + ((b * p.seqlen + t0) * p.nheads + h) * kP * 2
                                     : nullptr,
                                 xrow, t0, p.seqlen);
#pragma unroll
      for (int qq = 0; qq < 2; ++qq)
#pragma unroll
        for (int pt = 0; pt < 4; ++pt)
          zv[qq][pt] = vload8(zw, (uint32_t)((32 * blk[qq] + 16 * half + lane % 16) * xrow + (16 * pt + 4 * (lane / 16)) * 2));
    }
#pragma unroll
    for (int piece = 0; piece < kQ / kJB; ++piece) {
      if (piece > dpiece) break;
      const int jb = kJB * piece;
      if (piece + 2 < kQ / kJB && piece + 2 <= dpiece) {
#pragma unroll
        for (int ks = 0; ks < 2; ++ks)
          cbv[piece + 2][ks] = *reinterpret_cast<const u32x4v*>(cbrow + jb + 2 * kJB + 32 * ks);
      }
      const bool diag = piece == dpiece;
      const float ei = exp2_hw((csi - sCs[jb + kJB - 1]) * kLog2e);
#pragma unroll
      for (int ks = 0; ks < 2; ++ks) {
        const int j0 = jb + 32 * ks + 8 * (lane / 16);
        float cb[8];
#pragma unroll
        for (int e = 0; e < 4; ++e) {  // bf16 -> fp32: the high half of a 32-bit float
          cb[2 * e] = __builtin_bit_cast(float, cbv[piece][ks][e] << 16);
          cb[2 * e + 1] = __builtin_bit_cast(float, cbv[piece][ks][e] & 0xffff0000u);
        }
        float m[8];
        uint32_t same = 0xffu;  // bit e: step j0 + e is in row i's document
        if (mask) {
          const int4 s0 = *reinterpret_cast<const int4*>(&sSeg[j0]);
          const int4 s1 = *reinterpret_cast<const int4*>(&sSeg[j0 + 4]);
          same = (uint32_t)(s0.x == segi) | (uint32_t)(s0.y == segi) << 1 | (uint32_t)(s0.z == segi) << 2 |
                 (uint32_t)(s0.w == segi) << 3 | (uint32_t)(s1.x == segi) << 4 | (uint32_t)(s1.y == segi) << 5 |
                 (uint32_t)(s1.z == segi) << 6 | (uint32_t)(s1.w == segi) << 7;
        }
        if (diag) {
          const float4 c0 = *reinterpret_cast<const float4*>(&sCs[j0]);
          const float4 c1 = *reinterpret_cast<const float4*>(&sCs[j0 + 4]);
          const float4 d0 = *reinterpret_cast<const float4*>(&sDelta[j0]);
          const float4 d1 = *reinterpret_cast<const float4*>(&sDelta[j0 + 4]);
          const float csj[8] = {c0.x, c0.y, c0.z, c0.w, c1.x, c1.y, c1.z, c1.w};
          const float dj[8] = {d0.x, d0.y, d0.z, d0.w, d1.x, d1.y, d1.z, d1.w};
#pragma unroll
          for (int e = 0; e < 8; ++e) {
            const float v = cb[e] * exp2_hw((csi - csj[e]) * kLog2e) * dj[e];
            m[e] = j0 + e <= i && ((same >> e) & 1u) ? v : 0.0f;
          }
        } else {
          const float4 w0 = *reinterpret_cast<const float4*>(&sWp[j0]);
          const float4 w1 = *reinterpret_cast<const float4*>(&sWp[j0 + 4]);
          const float wj[8] = {w0.x, w0.y, w0.z, w0.w, w1.x, w1.y, w1.z, w1.w};
#pragma unroll
          for (int e = 0; e < 8; ++e) {
            m[e] = cb[e] * (wj[e] * ei);
            if (SEQ) m[e] = ((same >> e) & 1u) ? m[e] : 0.0f;
          }
        }
        u32x4v bop;
#pragma unroll
        for (int e = 0; e < 4; ++e)
          bop[e] = pack2<IO>(m[2 * e], m[2 * e + 1]);
#pragma unroll
        for (int pt = 0; pt < 4; ++pt) {  // A[m = p][k = step] = x^T, from the time-major tile
          const u32x4v xa = tm_frag(sX + (jb + 32 * ks) * kP, tm_lane_off<kP>(16 * pt, 0, lane),
                                    tm_lane_off<kP>(16 * pt, 1, lane));
          acc[q][pt] = M::run(as_vec<IO>(xa), as_vec<IO>(bop), acc[q][pt]);
        }
      }
    }
  }

  // ---- D skip (x from LDS), gate, store
  const float Dh = p.D ? p.D[h] : 0.0f;
#pragma unroll
  for (int q = 0; q < 2; ++q) {
    const int il = 32 * blk[q] + 16 * half + lane % 16;
    const int64_t t = t0 + il;
    if (t >= p.seqlen) continue;
#pragma unroll
    for (int pt = 0; pt < 4; ++pt) {
      const int p0 = 16 * pt + 4 * (lane / 16);
      const uint32_t zw[2] = {zv[q][pt].x, zv[q][pt].y};
      const uint2 xv = *reinterpret_cast<const uint2*>(&sX[tm_off<kP>(il, p0)]);  // x of channels p0 .. p0 + 3
      const uint32_t xw[2] = {xv.x, xv.y};
      uint32_t yw[2];
#pragma unroll
      for (int hw = 0; hw < 2; ++hw) {
        float yy[2];
#pragma unroll
        for (int s2 = 0; s2 < 2; ++s2) {
          const int r = 2 * hw + s2;
          float yv = fmaf(Dh, bits_f32<IO>((raw_t<IO>)((xw[hw] >> (16 * s2)) & 0xffffu)), acc[q][pt][r]);
          if (p.z) yv *= silu_f(bits_f32<IO>((raw_t<IO>)((zw[hw] >> (16 * s2)) & 0xffffu)));
          yy[s2] = yv;
        }
        yw[hw] = pack2<IO>(yy[0], yy[1]);
      }
      *reinterpret_cast<uint2*>(static_cast<char*>(p.y) + t * xrow + ((b * p.seqlen) * p.nheads + h) * kP * 2 +
                                p0 * 2) = make_uint2(yw[0], yw[1]);
    }
  }
}

template <int IO, int N, bool SEQ>
hipError_t launch_ssd_seq(const SsdParams& p, hipStream_t st) {
  hipLaunchKernelGGL((ssd_state_kernel<IO, N, SEQ>), dim3((uint32_t)(p.batch * p.nheads * (N / kNS))),
                     dim3(kSsdThreads), 0, st, p);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL((ssd_scan_kernel<IO, N, SEQ>), dim3((uint32_t)(p.batch * p.nchunks * p.nheads)),
                     dim3(kScanThreads), 0, st, p);
  return hipGetLastError();
}
template <int IO, int N>
hipError_t launch_ssd_n(const SsdParams& p, hipStream_t st) {
  return p.seq_idx ? launch_ssd_seq<IO, N, true>(p, st) : launch_ssd_seq<IO, N, false>(p, st);
}

template <int IO>
hipError_t launch_ssd_io(const SsdParams& p, hipStream_t st) {
  switch (p.dstate) {
    case 32: return launch_ssd_n<IO, 32>(p, st);
    case 64: return launch_ssd_n<IO, 64>(p, st);
    case 96: return launch_ssd_n<IO, 96>(p, st);
    default: return launch_ssd_n<IO, 128>(p, st);
  }
}

}  // namespace

hipError_t launch_ssd(const SsdParams& p, hipStream_t st) {
  return p.io == SS_F16 ? launch_ssd_io<SS_F16>(p, st) : launch_ssd_io<SS_BF16>(p, st);
}

}  // namespace ss
