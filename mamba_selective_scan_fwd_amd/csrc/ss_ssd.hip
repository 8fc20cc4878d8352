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
// Three kernels:
//   ssd_state_kernel  per (batch, chunk, head): S_c on MFMA (P x N, K = Q),
//                     and the chunk decay exp(cs_last);
//   ssd_pass_kernel   per (batch, head, state element): the chunk recurrence
//                     in fp32, writing each chunk's entry state (as the MFMA
//                     input dtype) and the final state;
//   ssd_scan_kernel   per (batch, chunk, head): Y_off = C H_in, then per
//                     64-step piece of the chunk's columns C B^T on MFMA,
//                     the decay mask in fp32, and Y_diag += M (Delta-scaled
//                     through the mask) x on MFMA; D skip, SiLU(z) gate, store.
// MFMA: v_mfma_f32_16x16x32_{bf16,f16}, fp32 accumulation.  Operand lane
// layout (checked on the chip): A[m][k] in lane m + 16 (k / 8), element k % 8;
// B[k][n] in lane n + 16 (k / 8), element k % 8; D[m][n] in lane
// n + 16 (m / 4), element m % 4.  Operands whose k axis is time are staged
// transposed in LDS (time is the slow axis in memory).
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

// Delta and the inclusive cumulative sum cs of Delta * A over the chunk's
// 256 steps (thread i = step i; steps past the sequence have Delta = 0).
template <int IO>
__device__ __forceinline__ void chunk_cumsum(const SsdParams& p, int64_t b, int64_t c, int64_t h, float A, float* sDelta,
                                             float* sCs, float* sWave) {
  const int tid = threadIdx.x, lane = tid % 64, wave = tid / 64;
  const int64_t t = c * kQ + tid;
  float delta = 0.0f;
  if (t < p.seqlen) {
    const float xd = load_io<IO>(p.dt, (b * p.seqlen + t) * p.nheads + h) + (p.dt_bias ? p.dt_bias[h] : 0.0f);
    delta = p.softplus ? softplus_f(xd) : xd;
  }
  float v = delta * A;
#pragma unroll
  for (int off = 1; off < 64; off <<= 1) {
    const float o = __shfl_up(v, off, 64);
    if (lane >= off) v += o;
  }
  if (lane == 63) sWave[wave] = v;
  sDelta[tid] = delta;
  __syncthreads();
  float base = 0.0f;
  for (int w = 0; w < wave; ++w) base += sWave[w];
  sCs[tid] = v + base;
  __syncthreads();
}

// Stage a 64-step piece of a (time x width) row-major 16-bit tensor into LDS
// transposed, dst[col][j] (j contiguous, row stride kXR): work item (jq, co)
// reads steps 4 jq .. 4 jq + 3 of columns 8 co .. 8 co + 7 with four 16-byte
// loads and writes each column's 4 steps with one 8-byte store.  `scale`
// (per step, optional) multiplies the values first.
template <int IO, int WIDTH, int kXR>
__device__ __forceinline__ void stage_transposed(uint16_t (*dst)[kXR], const char* base, int64_t row_stride_bytes,
                                                 int64_t t0, int64_t seqlen, const float* scale, int item) {
  constexpr int kOct = WIDTH / 8;
  const int jq = item / kOct, co = item % kOct;
  uint32_t w[4][4];
#pragma unroll
  for (int r = 0; r < 4; ++r) {
    const int64_t t = t0 + 4 * jq + r;
    u32x4v v = u32x4v{0u, 0u, 0u, 0u};
    if (t < seqlen) v = *reinterpret_cast<const u32x4v*>(base + t * row_stride_bytes + co * 16);
    if (scale) {
      const float sc = scale[4 * jq + r];
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        const float lo = bits_f32<IO>((raw_t<IO>)(v[q] & 0xffffu)) * sc;
        const float hi = bits_f32<IO>((raw_t<IO>)(v[q] >> 16)) * sc;
        v[q] = pack2<IO>(lo, hi);
      }
    }
#pragma unroll
    for (int q = 0; q < 4; ++q) w[r][q] = v[q];
  }
#pragma unroll
  for (int e = 0; e < 8; ++e) {  // column 8 co + e: its 4 steps
    const int q = e / 2, sh = 16 * (e % 2);
    const uint32_t a0 = (w[0][q] >> sh) & 0xffffu, a1 = (w[1][q] >> sh) & 0xffffu;
    const uint32_t a2 = (w[2][q] >> sh) & 0xffffu, a3 = (w[3][q] >> sh) & 0xffffu;
    uint2 pk;
    pk.x = a0 | (a1 << 16);
    pk.y = a2 | (a3 << 16);
    *reinterpret_cast<uint2*>(&dst[8 * co + e][4 * jq]) = pk;
  }
}

// ---- pass 1: the chunk's own state S_c[p][n] = sum_j w_j x_j[p] B_j[n] ----
// w_j = exp(cs_last - cs_j) Delta_j.  Every global operand of the chunk (x,
// B, dt) is loaded at once into registers, then moved to LDS transposed
// (time contiguous) two 64-step pieces at a time for the MFMAs: wave w takes
// rows p in [16w, 16w + 16) and all states n.  The workgroups of a group's
// heads also share out the group's C B^T: head k of the group takes the
// 16-row tiles k, k + heads_per_group, ...
template <int IO, int N>
__device__ __forceinline__ void cb_row_tile(const SsdParams& p, int64_t b, int64_t c, int64_t g, int rt, int lane,
                                            int wave) {
  using M = mfma_t<IO>;
  const int64_t t0 = c * kQ;
  const int64_t crow = p.ngroups * N * 2;
  const char* cbase = static_cast<const char*>(p.Cm) + ((b * p.seqlen) * p.ngroups + g) * N * 2;
  const char* bbase = static_cast<const char*>(p.Bm) + ((b * p.seqlen) * p.ngroups + g) * N * 2;
  auto frag = [&](const char* base, int64_t t, int n0) -> u32x4v {
    if (t >= p.seqlen) return u32x4v{0u, 0u, 0u, 0u};
    return *reinterpret_cast<const u32x4v*>(base + t * crow + n0 * 2);
  };
  // columns of every 64-step piece up to the one holding the row tile
  const int last_tile = 4 * (rt / 4) + 3;
  u32x4v af[N / 32], bf[4][N / 32];
#pragma unroll
  for (int ks = 0; ks < N / 32; ++ks) af[ks] = frag(cbase, t0 + 16 * rt + lane % 16, 32 * ks + 8 * (lane / 16));
#pragma unroll
  for (int u = 0; u < 4; ++u) {
    const int jt = wave + 4 * u;
#pragma unroll
    for (int ks = 0; ks < N / 32; ++ks)
      bf[u][ks] = jt <= last_tile ? frag(bbase, t0 + 16 * jt + lane % 16, 32 * ks + 8 * (lane / 16))
                                  : u32x4v{0u, 0u, 0u, 0u};
  }
  float* CB = p.ws_cb + ((b * p.nchunks + c) * p.ngroups + g) * (int64_t)(kQ * kQ);
#pragma unroll
  for (int u = 0; u < 4; ++u) {
    const int jt = wave + 4 * u;
    if (jt > last_tile) break;
    f32x4 acc = f32x4{0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
    for (int ks = 0; ks < N / 32; ++ks) acc = M::run(as_vec<IO>(af[ks]), as_vec<IO>(bf[u][ks]), acc);
    // lane holds rows i = 16 rt + 4 (lane / 16) + r of column j = 16 jt + lane % 16
#pragma unroll
    for (int r = 0; r < 4; ++r) CB[(16 * rt + 4 * (lane / 16) + r) * kQ + 16 * jt + lane % 16] = acc[r];
  }
}

template <int IO, int N>
__global__ void __launch_bounds__(kSsdThreads) ssd_state_kernel(SsdParams p) {
  using M = mfma_t<IO>;
  constexpr int kXR = 2 * kJB + 8;  // LDS row: two pieces of time, padded (272 B keeps 16-byte reads aligned)
  __shared__ __attribute__((aligned(16))) float sW[kQ];
  __shared__ float sDelta[kQ], sCs[kQ], sWave[4];
  __shared__ __attribute__((aligned(16))) uint16_t sXT[kP][kXR];  // (x * w)^T of two pieces: [p][j]
  __shared__ __attribute__((aligned(16))) uint16_t sBT[N][kXR];   // B^T of two pieces: [n][j]
  const int tid = threadIdx.x, lane = tid % 64, wave = tid / 64;
  const int64_t lb = xcd_logical_block();  // the heads of one chunk run on one XCD and share its B, C in L2
  const int64_t h = lb % p.nheads;
  const int64_t c = (lb / p.nheads) % p.nchunks;
  const int64_t b = lb / (p.nheads * p.nchunks);
  const int64_t hpg = p.nheads / p.ngroups;
  const int64_t g = h / hpg;
  const int64_t t0 = c * kQ;
  const int64_t xrow = p.nheads * kP * 2, brow = p.ngroups * N * 2;
  const char* xbase = static_cast<const char*>(p.x) + ((b * p.seqlen) * p.nheads + h) * kP * 2;
  const char* bbase = static_cast<const char*>(p.Bm) + ((b * p.seqlen) * p.ngroups + g) * N * 2;

  // x: 512 items (4 steps x 8 channels); item = tid + 256 k, piece 2 k + tid / 128
  u32x4v xr[2][4];
#pragma unroll
  for (int k = 0; k < 2; ++k) {
    const int item = tid + kSsdThreads * k, pc = item / 128, jq = (item % 128) / 8, co = item % 8;
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const int64_t t = t0 + 64 * pc + 4 * jq + r;
      xr[k][r] = t < p.seqlen ? *reinterpret_cast<const u32x4v*>(xbase + t * xrow + co * 16) : u32x4v{0u, 0u, 0u, 0u};
    }
  }
  // B: 8 N items (4 steps x 8 states), N / 32 per thread; item = tid + 256 k
  constexpr int kBI = N / 32;
  u32x4v br[kBI][4];
#pragma unroll
  for (int k = 0; k < kBI; ++k) {
    const int item = tid + kSsdThreads * k, pc = item / (2 * N), rem = item % (2 * N);
    const int jq = rem / (N / 8), co = rem % (N / 8);
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const int64_t t = t0 + 64 * pc + 4 * jq + r;
      br[k][r] = t < p.seqlen ? *reinterpret_cast<const u32x4v*>(bbase + t * brow + co * 16) : u32x4v{0u, 0u, 0u, 0u};
    }
  }
  chunk_cumsum<IO>(p, b, c, h, p.A[h], sDelta, sCs, sWave);  // ends with a barrier
  sW[tid] = exp2_hw((sCs[kQ - 1] - sCs[tid]) * kLog2e) * sDelta[tid];  // 0 past the sequence (Delta = 0)
  __syncthreads();

  f32x4 acc[N / 16];
#pragma unroll
  for (int i = 0; i < N / 16; ++i) acc[i] = f32x4{0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
  for (int round = 0; round < 2; ++round) {
    {  // x * w, transposed
      const int item = tid + kSsdThreads * round, pc = item / 128, jq = (item % 128) / 8, co = item % 8;
      uint32_t v[4][4];
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const float sc = sW[64 * pc + 4 * jq + r];
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          const float lo = bits_f32<IO>((raw_t<IO>)(xr[round][r][q] & 0xffffu)) * sc;
          const float hi = bits_f32<IO>((raw_t<IO>)(xr[round][r][q] >> 16)) * sc;
          v[r][q] = pack2<IO>(lo, hi);
        }
      }
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        const int q = e / 2, sh = 16 * (e % 2);
        uint2 pk;
        pk.x = ((v[0][q] >> sh) & 0xffffu) | (((v[1][q] >> sh) & 0xffffu) << 16);
        pk.y = ((v[2][q] >> sh) & 0xffffu) | (((v[3][q] >> sh) & 0xffffu) << 16);
        *reinterpret_cast<uint2*>(&sXT[8 * co + e][64 * (pc % 2) + 4 * jq]) = pk;
      }
    }
#pragma unroll
    for (int k = 0; k < kBI; ++k) {  // B, transposed
      const int item = tid + kSsdThreads * k, pc = item / (2 * N), rem = item % (2 * N);
      if (pc / 2 != round) continue;
      const int jq = rem / (N / 8), co = rem % (N / 8);
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        const int q = e / 2, sh = 16 * (e % 2);
        uint2 pk;
        pk.x = ((br[k][0][q] >> sh) & 0xffffu) | (((br[k][1][q] >> sh) & 0xffffu) << 16);
        pk.y = ((br[k][2][q] >> sh) & 0xffffu) | (((br[k][3][q] >> sh) & 0xffffu) << 16);
        *reinterpret_cast<uint2*>(&sBT[8 * co + e][64 * (pc % 2) + 4 * jq]) = pk;
      }
    }
    __syncthreads();
#pragma unroll
    for (int ks = 0; ks < 2 * kJB; ks += 32) {
      const int k0 = ks + 8 * (lane / 16);
      const u32x4v a = *reinterpret_cast<const u32x4v*>(&sXT[16 * wave + lane % 16][k0]);
#pragma unroll
      for (int nt = 0; nt < N / 16; ++nt) {
        const u32x4v bb = *reinterpret_cast<const u32x4v*>(&sBT[16 * nt + lane % 16][k0]);
        acc[nt] = M::run(as_vec<IO>(a), as_vec<IO>(bb), acc[nt]);
      }
    }
    __syncthreads();
  }
  // S_c[p][n]: lane holds rows p = 16 w + 4 (lane / 16) + r, column n = 16 nt + lane % 16
  float* S = p.ws_state + ((b * p.nchunks + c) * p.nheads + h) * (int64_t)(kP * N);
#pragma unroll
  for (int nt = 0; nt < N / 16; ++nt)
#pragma unroll
    for (int r = 0; r < 4; ++r) S[(16 * wave + 4 * (lane / 16) + r) * N + 16 * nt + lane % 16] = acc[nt][r];
  if (tid == 0) p.ws_decay[(b * p.nchunks + c) * p.nheads + h] = exp2_hw(sCs[kQ - 1] * kLog2e);
  // this head's share of the group's C B^T
  for (int64_t rt = h % hpg; rt < kQ / 16; rt += hpg) cb_row_tile<IO, N>(p, b, c, g, (int)rt, lane, wave);
}

// ---- pass 2: entry state of every chunk, H_in(c + 1) = decay_c H_in(c) + S_c ----
template <int IO>
__global__ void __launch_bounds__(256) ssd_pass_kernel(SsdParams p) {
  const int64_t per = (int64_t)kP * p.dstate;  // state elements per head
  const int64_t e = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (e >= p.batch * p.nheads * per) return;
  const int64_t bh = e / per, i = e % per;
  const int64_t b = bh / p.nheads, h = bh % p.nheads;
  float H = p.h0 ? p.h0[e] : 0.0f;  // h0 is (B, H, P, N): element e
  uint16_t* Hin = p.ws_entry;
  for (int64_t c = 0; c < p.nchunks; ++c) {
    const int64_t s = ((b * p.nchunks + c) * p.nheads + h) * per + i;
    Hin[s] = bits16<IO>(H);
    H = fmaf(p.ws_decay[(b * p.nchunks + c) * p.nheads + h], H, p.ws_state[s]);
  }
  if (p.final_state) p.final_state[e] = H;
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
// are issued ahead of their use: all prologue operands at once, the next
// piece's CB during the current piece, the gate z before the main loop.
constexpr int kScanThreads = 512;
template <int IO, int N>
__global__ void __launch_bounds__(kScanThreads) ssd_scan_kernel(SsdParams p) {
  using M = mfma_t<IO>;
  constexpr int kXR = kQ + 8;  // x^T row: 264 elements (528 B keeps 16-byte reads aligned)
  constexpr int kHR = N + 8;   // H_in row
  __shared__ __attribute__((aligned(16))) float sDelta[kQ];
  __shared__ __attribute__((aligned(16))) float sCs[kQ];
  __shared__ __attribute__((aligned(16))) float sWp[kQ];           // exp(cs_e - cs_j) Delta_j, e = end of j's piece
  __shared__ float sWave[4];
  __shared__ __attribute__((aligned(16))) uint16_t sXT[kP][kXR];   // x^T of the chunk: [p][j]
  __shared__ __attribute__((aligned(16))) uint16_t sH[kP][kHR];    // entry state H_in[p][n]
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
  const int pc = tid / 128, jq = (tid % 128) / 8, co = tid % 8;  // x item: steps 64 pc + 4 jq .. + 3, channels 8 co ..
  u32x4v xr[4];
#pragma unroll
  for (int r = 0; r < 4; ++r) {
    const int64_t t = t0 + 64 * pc + 4 * jq + r;
    xr[r] = t < p.seqlen ? *reinterpret_cast<const u32x4v*>(xbase + t * xrow + co * 16) : u32x4v{0u, 0u, 0u, 0u};
  }
  constexpr int kHPieces = kP * (N / 8);  // 16-byte pieces of H_in
  constexpr int kHItems = (kHPieces + kScanThreads - 1) / kScanThreads;
  u32x4v hr[kHItems];
#pragma unroll
  for (int k = 0; k < kHItems; ++k) {
    const int item = tid + kScanThreads * k;
    hr[k] = item < kHPieces ? *reinterpret_cast<const u32x4v*>(Hin + (item / (N / 8)) * N + 8 * (item % (N / 8)))
                            : u32x4v{0u, 0u, 0u, 0u};
  }
  float dt_raw = 0.0f;
  if (tid < kQ && t0 + tid < p.seqlen) dt_raw = load_io<IO>(p.dt, (b * p.seqlen + t0 + tid) * p.nheads + h);
  auto cfrag = [&](int64_t t, int n0) -> u32x4v {
    if (t >= p.seqlen) return u32x4v{0u, 0u, 0u, 0u};
    return *reinterpret_cast<const u32x4v*>(cbase + t * crow + n0 * 2);
  };
  u32x4v cf[2][N / 32];
#pragma unroll
  for (int q = 0; q < 2; ++q)
#pragma unroll
    for (int ks = 0; ks < N / 32; ++ks) cf[q][ks] = cfrag(t0 + 32 * blk[q] + 16 * half + lane % 16, 32 * ks + 8 * (lane / 16));

  {  // Delta and the inclusive cumulative sum of Delta A over the chunk (threads 0..255 = steps)
    float delta = 0.0f;
    if (tid < kQ && t0 + tid < p.seqlen) {
      const float xd = dt_raw + (p.dt_bias ? p.dt_bias[h] : 0.0f);
      delta = p.softplus ? softplus_f(xd) : xd;
    }
    float v = delta * p.A[h];
#pragma unroll
    for (int off = 1; off < 64; off <<= 1) {
      const float o = __shfl_up(v, off, 64);
      if (lane >= off) v += o;
    }
    if (tid < kQ) {
      if (lane == 63) sWave[wave] = v;
      sDelta[tid] = delta;
    }
    // x^T and H_in into LDS meanwhile
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      const int q = e / 2, sh = 16 * (e % 2);
      uint2 pk;
      pk.x = ((xr[0][q] >> sh) & 0xffffu) | (((xr[1][q] >> sh) & 0xffffu) << 16);
      pk.y = ((xr[2][q] >> sh) & 0xffffu) | (((xr[3][q] >> sh) & 0xffffu) << 16);
      *reinterpret_cast<uint2*>(&sXT[8 * co + e][64 * pc + 4 * jq]) = pk;
    }
#pragma unroll
    for (int k = 0; k < kHItems; ++k) {
      const int item = tid + kScanThreads * k;
      if (item < kHPieces) *reinterpret_cast<u32x4v*>(&sH[item / (N / 8)][8 * (item % (N / 8))]) = hr[k];
    }
    __syncthreads();
    if (tid < kQ) {
      float base = 0.0f;
      for (int w = 0; w < wave; ++w) base += sWave[w];
      sCs[tid] = v + base;
    }
    __syncthreads();
    if (tid < kQ) sWp[tid] = exp2_hw((sCs[tid | 63] - sCs[tid]) * kLog2e) * sDelta[tid];
  }

  // gate values for the epilogue: lane has channels 16 pt + 4 (lane / 16) .. + 3 of its step
  uint2 zv[2][4];
#pragma unroll
  for (int q = 0; q < 2; ++q) {
    const int64_t t = t0 + 32 * blk[q] + 16 * half + lane % 16;
#pragma unroll
    for (int pt = 0; pt < 4; ++pt)
      zv[q][pt] = (p.z && t < p.seqlen)
                      ? *reinterpret_cast<const uint2*>(static_cast<const char*>(p.z) + t * xrow +
                                                        ((b * p.seqlen) * p.nheads + h) * kP * 2 +
                                                        (16 * pt + 4 * (lane / 16)) * 2)
                      : make_uint2(0u, 0u);
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
    for (int pt = 0; pt < 4; ++pt) {
      const u32x4v hf = *reinterpret_cast<const u32x4v*>(&sH[16 * pt + lane % 16][32 * ks + 8 * (lane / 16)]);
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

  // ---- Y_diag += x^T M^T, piece by piece
  const float* CBbase = p.ws_cb + ((b * p.nchunks + c) * p.ngroups + g) * (int64_t)(kQ * kQ);
#pragma unroll
  for (int q = 0; q < 2; ++q) {
    const int i = 32 * blk[q] + 16 * half + lane % 16;  // this lane's row (chunk-local)
    const int dpiece = blk[q] / 2;                      // the piece holding the block's rows
    const float csi = sCs[i];
    const float* cbrow = CBbase + i * kQ + 8 * (lane / 16);
    float4 nxt[4];
#pragma unroll
    for (int k = 0; k < 4; ++k) nxt[k] = *reinterpret_cast<const float4*>(cbrow + 32 * (k / 2) + 4 * (k % 2));
    for (int piece = 0; piece <= dpiece; ++piece) {
      const int jb = 64 * piece;
      float4 cur[4];
#pragma unroll
      for (int k = 0; k < 4; ++k) cur[k] = nxt[k];
      if (piece < dpiece) {
#pragma unroll
        for (int k = 0; k < 4; ++k)
          nxt[k] = *reinterpret_cast<const float4*>(cbrow + jb + 64 + 32 * (k / 2) + 4 * (k % 2));
      }
      const bool diag = piece == dpiece;
      const float ei = exp2_hw((csi - sCs[jb + 63]) * kLog2e);
#pragma unroll
      for (int ks = 0; ks < 2; ++ks) {
        const int j0 = jb + 32 * ks + 8 * (lane / 16);
        const float cb[8] = {cur[2 * ks].x, cur[2 * ks].y, cur[2 * ks].z, cur[2 * ks].w,
                             cur[2 * ks + 1].x, cur[2 * ks + 1].y, cur[2 * ks + 1].z, cur[2 * ks + 1].w};
        float m[8];
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
            m[e] = j0 + e <= i ? v : 0.0f;
          }
        } else {
          const float4 w0 = *reinterpret_cast<const float4*>(&sWp[j0]);
          const float4 w1 = *reinterpret_cast<const float4*>(&sWp[j0 + 4]);
          const float wj[8] = {w0.x, w0.y, w0.z, w0.w, w1.x, w1.y, w1.z, w1.w};
#pragma unroll
          for (int e = 0; e < 8; ++e) m[e] = cb[e] * (wj[e] * ei);
        }
        u32x4v bop;
#pragma unroll
        for (int e = 0; e < 4; ++e)
          bop[e] = pack2<IO>(m[2 * e], m[2 * e + 1]);
#pragma unroll
        for (int pt = 0; pt < 4; ++pt) {
          const u32x4v xa = *reinterpret_cast<const u32x4v*>(&sXT[16 * pt + lane % 16][j0]);
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
      uint32_t yw[2];
#pragma unroll
      for (int hw = 0; hw < 2; ++hw) {
        float yy[2];
#pragma unroll
        for (int s2 = 0; s2 < 2; ++s2) {
          const int r = 2 * hw + s2;
          float yv = fmaf(Dh, bits_f32<IO>((raw_t<IO>)sXT[p0 + r][il]), acc[q][pt][r]);
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

template <int IO, int N>
hipError_t launch_ssd_n(const SsdParams& p, hipStream_t st) {
  const dim3 grid((uint32_t)(p.batch * p.nchunks * p.nheads));
  hipLaunchKernelGGL((ssd_state_kernel<IO, N>), grid, dim3(kSsdThreads), 0, st, p);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  const int64_t elems = p.batch * p.nheads * kP * N;
  hipLaunchKernelGGL((ssd_pass_kernel<IO>), dim3((uint32_t)((elems + 255) / 256)), dim3(256), 0, st, p);
  e = hipGetLastError();
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL((ssd_scan_kernel<IO, N>), grid, dim3(kScanThreads), 0, st, p);
  return hipGetLastError();
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
