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
        v[q] = (uint32_t)bits16<IO>(lo) | ((uint32_t)bits16<IO>(hi) << 16);
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
template <int IO, int N>
__global__ void __launch_bounds__(kSsdThreads) ssd_state_kernel(SsdParams p) {
  using M = mfma_t<IO>;
  constexpr int kXR = kJB + 8;  // padded LDS row (16-bit elements; 144 B keeps 16-byte reads aligned)
  __shared__ float sDelta[kQ], sCs[kQ], sWave[4], sW[kQ];
  __shared__ __attribute__((aligned(16))) uint16_t sXT[kP][kXR];  // (x * w)^T of one 64-step piece: [p][j]
  __shared__ __attribute__((aligned(16))) uint16_t sBT[N][kXR];   // B^T of the piece: [n][j]
  const int tid = threadIdx.x, lane = tid % 64, wave = tid / 64;
  const int64_t h = blockIdx.x % p.nheads;
  const int64_t c = (blockIdx.x / p.nheads) % p.nchunks;
  const int64_t b = blockIdx.x / (p.nheads * p.nchunks);
  const int64_t g = h / (p.nheads / p.ngroups);
  const float A = p.A[h];
  chunk_cumsum<IO>(p, b, c, h, A, sDelta, sCs, sWave);
  const float cs_last = sCs[kQ - 1];
  sW[tid] = exp2_hw((cs_last - sCs[tid]) * kLog2e) * sDelta[tid];  // 0 past the sequence (Delta = 0)
  __syncthreads();

  f32x4 acc[N / 16];
#pragma unroll
  for (int i = 0; i < N / 16; ++i) acc[i] = f32x4{0.0f, 0.0f, 0.0f, 0.0f};
  const char* xbase = static_cast<const char*>(p.x) + ((b * p.seqlen) * p.nheads + h) * kP * 2;
  const char* bbase = static_cast<const char*>(p.Bm) + ((b * p.seqlen) * p.ngroups + g) * N * 2;

  for (int jb = 0; jb < kQ; jb += kJB) {
    const int64_t t0 = c * kQ + jb;
    if (tid < 16 * (kP / 8))
      stage_transposed<IO, kP, kXR>(sXT, xbase, p.nheads * kP * 2, t0, p.seqlen, sW + jb, tid);
    if (tid < 16 * (N / 8))
      stage_transposed<IO, N, kXR>(sBT, bbase, p.ngroups * N * 2, t0, p.seqlen, nullptr, tid);
    __syncthreads();
    // wave w: rows p in [16w, 16w + 16), all N/16 column tiles; K = 64 in two steps
#pragma unroll
    for (int ks = 0; ks < kJB; ks += 32) {
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
  if (tid == 0) p.ws_decay[(b * p.nchunks + c) * p.nheads + h] = exp2_hw(cs_last * kLog2e);
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

// ---- C B^T of a chunk, once per group ---------------------------------------------
// CB[i][j] = sum_n C_i[n] B_j[n] in fp32 for the chunk's rows i and the columns j
// of every 64-step piece up to the one holding i (the causal half plus the rest
// of the diagonal pieces, so that the scan never reads an unwritten value).
// Workgroup = (batch, chunk, group, 16-row tile); wave w takes column tiles
// w, w + 4, ... .  Shared by all heads of the group.
template <int IO, int N>
__global__ void __launch_bounds__(kSsdThreads) ssd_cb_kernel(SsdParams p) {
  using M = mfma_t<IO>;
  const int lane = threadIdx.x % 64, wave = threadIdx.x / 64;
  const int rt = blockIdx.x % (kQ / 16);
  const int64_t bcg = blockIdx.x / (kQ / 16);
  const int64_t g = bcg % p.ngroups;
  const int64_t c = (bcg / p.ngroups) % p.nchunks;
  const int64_t b = bcg / (p.ngroups * p.nchunks);
  const int64_t t0 = c * kQ;
  const int64_t crow = p.ngroups * N * 2;
  const char* cbase = static_cast<const char*>(p.Cm) + ((b * p.seqlen) * p.ngroups + g) * N * 2;
  const char* bbase = static_cast<const char*>(p.Bm) + ((b * p.seqlen) * p.ngroups + g) * N * 2;
  auto frag = [&](const char* base, int64_t t, int n0) -> u32x4v {
    if (t >= p.seqlen) return u32x4v{0u, 0u, 0u, 0u};
    return *reinterpret_cast<const u32x4v*>(base + t * crow + n0 * 2);
  };
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
  float* CB = p.ws_cb + (bcg * kQ) * (int64_t)kQ;
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

// ---- pass 3: outputs of a chunk -------------------------------------------------
// Y is built transposed, Y^T[p][i], so that each lane ends up with 4
// consecutive channels p of one step i.  The chunk's 256 rows are 8 blocks of
// 32; wave w takes blocks w and 7 - w, so every wave does the same causal work
// (block r needs column pieces 0 .. r / 2 of 64 steps).
//   Y^T = diag-scaled H_in C^T       (entry state: A = H_in, B = C^T)
//       + x^T M^T                    (A = x^T from LDS, B = M^T built in registers)
// with M[i][j] = CB[i][j] exp(cs_i - cs_j) Delta_j for j <= i.  Off the
// diagonal piece the decay factors through the piece's last step e:
// exp(cs_i - cs_e) * exp(cs_e - cs_j), both at most 1 there, so only one exp
// per lane is needed; the diagonal piece takes the exp per element.
template <int IO, int N>
__global__ void __launch_bounds__(kSsdThreads) ssd_scan_kernel(SsdParams p) {
  using M = mfma_t<IO>;
  constexpr int kXR = kQ + 8;  // x^T row: 264 elements (528 B keeps 16-byte reads aligned)
  __shared__ __attribute__((aligned(16))) float sDelta[kQ];
  __shared__ __attribute__((aligned(16))) float sCs[kQ];
  __shared__ float sWave[4];
  __shared__ __attribute__((aligned(16))) float sWp[kQ];           // exp(cs_e - cs_j) Delta_j, e = end of j's piece
  __shared__ __attribute__((aligned(16))) uint16_t sXT[kP][kXR];   // x^T of the chunk: [p][j]
  const int tid = threadIdx.x, lane = tid % 64, wave = tid / 64;
  const int64_t h = blockIdx.x % p.nheads;
  const int64_t c = (blockIdx.x / p.nheads) % p.nchunks;
  const int64_t b = blockIdx.x / (p.nheads * p.nchunks);
  const int64_t g = h / (p.nheads / p.ngroups);
  const float A = p.A[h];
  const int64_t t0 = c * kQ;
  const char* xbase = static_cast<const char*>(p.x) + ((b * p.seqlen) * p.nheads + h) * kP * 2;
#pragma unroll
  for (int it = 0; it < 2; ++it)  // 512 work items: 4 pieces of 64 steps x 128
    stage_transposed<IO, kP, kXR>(reinterpret_cast<uint16_t(*)[kXR]>(&sXT[0][64 * (2 * it + tid / 128)]), xbase,
                                  p.nheads * kP * 2, t0 + 64 * (2 * it + tid / 128), p.seqlen, nullptr, tid % 128);
  chunk_cumsum<IO>(p, b, c, h, A, sDelta, sCs, sWave);  // ends with a barrier
  sWp[tid] = exp2_hw((sCs[tid | 63] - sCs[tid]) * kLog2e) * sDelta[tid];

  const char* cbase = static_cast<const char*>(p.Cm) + ((b * p.seqlen) * p.ngroups + g) * N * 2;
  const int64_t crow = p.ngroups * N * 2;
  auto cfrag = [&](int64_t t, int n0) -> u32x4v {
    if (t >= p.seqlen) return u32x4v{0u, 0u, 0u, 0u};
    return *reinterpret_cast<const u32x4v*>(cbase + t * crow + n0 * 2);
  };
  const int blk[2] = {wave, 7 - wave};
  f32x4 acc[2][4][2];  // [block][p tile][i tile]: p = 16 pt + 4 (lane / 16) + r, i = 32 blk + 16 it + lane % 16
  {
    const uint16_t* Hin = p.ws_entry + ((b * p.nchunks + c) * p.nheads + h) * (int64_t)(kP * N);
#pragma unroll
    for (int q = 0; q < 2; ++q)
#pragma unroll
      for (int pt = 0; pt < 4; ++pt)
#pragma unroll
        for (int it = 0; it < 2; ++it) acc[q][pt][it] = f32x4{0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
    for (int ks = 0; ks < N; ks += 32) {
      const int n0 = ks + 8 * (lane / 16);
      u32x4v hf[4], cf[2][2];
#pragma unroll
      for (int pt = 0; pt < 4; ++pt) hf[pt] = *reinterpret_cast<const u32x4v*>(Hin + (16 * pt + lane % 16) * N + n0);
#pragma unroll
      for (int q = 0; q < 2; ++q)
#pragma unroll
        for (int it = 0; it < 2; ++it) cf[q][it] = cfrag(t0 + 32 * blk[q] + 16 * it + lane % 16, n0);
#pragma unroll
      for (int q = 0; q < 2; ++q)
#pragma unroll
        for (int pt = 0; pt < 4; ++pt)
#pragma unroll
          for (int it = 0; it < 2; ++it)
            acc[q][pt][it] = M::run(as_vec<IO>(hf[pt]), as_vec<IO>(cf[q][it]), acc[q][pt][it]);
    }
    __syncthreads();  // sWp
#pragma unroll
    for (int q = 0; q < 2; ++q)
#pragma unroll
      for (int it = 0; it < 2; ++it) {
        const float sc = exp2_hw(sCs[32 * blk[q] + 16 * it + lane % 16] * kLog2e);
#pragma unroll
        for (int pt = 0; pt < 4; ++pt) acc[q][pt][it] *= sc;
      }
  }

  const float* CBbase = p.ws_cb + ((b * p.nchunks + c) * p.ngroups + g) * (int64_t)(kQ * kQ);
#pragma unroll
  for (int q = 0; q < 2; ++q) {
    const int i0 = 32 * blk[q];
    const int dpiece = blk[q] / 2;  // the piece holding this block's rows
    float csi[2];
    const float* cbrow[2];
#pragma unroll
    for (int it = 0; it < 2; ++it) {
      csi[it] = sCs[i0 + 16 * it + lane % 16];
      cbrow[it] = CBbase + (i0 + 16 * it + lane % 16) * kQ;
    }
    for (int piece = 0; piece <= dpiece; ++piece) {
      const int jb = 64 * piece;
      const bool diag = piece == dpiece;
      float ei[2];
#pragma unroll
      for (int it = 0; it < 2; ++it) ei[it] = exp2_hw((csi[it] - sCs[jb + 63]) * kLog2e);
#pragma unroll
      for (int ks = 0; ks < kJB; ks += 32) {
        const int j0 = jb + ks + 8 * (lane / 16);
        u32x4v xa[4];
#pragma unroll
        for (int pt = 0; pt < 4; ++pt) xa[pt] = *reinterpret_cast<const u32x4v*>(&sXT[16 * pt + lane % 16][j0]);
        const float4 w0 = *reinterpret_cast<const float4*>(&sWp[j0]);
        const float4 w1 = *reinterpret_cast<const float4*>(&sWp[j0 + 4]);
        const float wj[8] = {w0.x, w0.y, w0.z, w0.w, w1.x, w1.y, w1.z, w1.w};
#pragma unroll
        for (int it = 0; it < 2; ++it) {
          const int i = i0 + 16 * it + lane % 16;
          const float4 c0 = *reinterpret_cast<const float4*>(cbrow[it] + j0);
          const float4 c1 = *reinterpret_cast<const float4*>(cbrow[it] + j0 + 4);
          const float cb[8] = {c0.x, c0.y, c0.z, c0.w, c1.x, c1.y, c1.z, c1.w};
          float m[8];
          if (diag) {
#pragma unroll
            for (int e = 0; e < 8; ++e) {
              const int j = j0 + e;
              const float v = cb[e] * exp2_hw((csi[it] - sCs[j]) * kLog2e) * sDelta[j];
              m[e] = j <= i ? v : 0.0f;
            }
          } else {
#pragma unroll
            for (int e = 0; e < 8; ++e) m[e] = cb[e] * (wj[e] * ei[it]);
          }
          u32x4v bop;
#pragma unroll
          for (int e = 0; e < 4; ++e)
            bop[e] = (uint32_t)bits16<IO>(m[2 * e]) | ((uint32_t)bits16<IO>(m[2 * e + 1]) << 16);
#pragma unroll
          for (int pt = 0; pt < 4; ++pt) acc[q][pt][it] = M::run(as_vec<IO>(xa[pt]), as_vec<IO>(bop), acc[q][pt][it]);
        }
      }
    }
  }

  // D skip, gate, store: lane has channels 16 pt + 4 (lane / 16) .. + 3 of step i
  const float Dh = p.D ? p.D[h] : 0.0f;
#pragma unroll
  for (int q = 0; q < 2; ++q)
#pragma unroll
    for (int it = 0; it < 2; ++it) {
      const int64_t t = t0 + 32 * blk[q] + 16 * it + lane % 16;
      if (t >= p.seqlen) continue;
#pragma unroll
      for (int pt = 0; pt < 4; ++pt) {
        const int64_t idx = ((b * p.seqlen + t) * p.nheads + h) * kP + 16 * pt + 4 * (lane / 16);
        const uint2 xv = *reinterpret_cast<const uint2*>(static_cast<const uint16_t*>(p.x) + idx);
        uint2 zv = make_uint2(0u, 0u);
        if (p.z) zv = *reinterpret_cast<const uint2*>(static_cast<const uint16_t*>(p.z) + idx);
        const uint32_t xw[2] = {xv.x, xv.y}, zw[2] = {zv.x, zv.y};
        uint32_t yw[2];
#pragma unroll
        for (int hw = 0; hw < 2; ++hw) {
          float yy[2];
#pragma unroll
          for (int s2 = 0; s2 < 2; ++s2) {
            const float xf = bits_f32<IO>((raw_t<IO>)((xw[hw] >> (16 * s2)) & 0xffffu));
            float yv = fmaf(Dh, xf, acc[q][pt][it][2 * hw + s2]);
            if (p.z) yv *= silu_f(bits_f32<IO>((raw_t<IO>)((zw[hw] >> (16 * s2)) & 0xffffu)));
            yy[s2] = yv;
          }
          yw[hw] = (uint32_t)bits16<IO>(yy[0]) | ((uint32_t)bits16<IO>(yy[1]) << 16);
        }
        *reinterpret_cast<uint2*>(static_cast<uint16_t*>(p.y) + idx) = make_uint2(yw[0], yw[1]);
      }
    }
}

template <int IO, int N>
hipError_t launch_ssd_n(const SsdParams& p, hipStream_t st) {
  const dim3 grid((uint32_t)(p.batch * p.nchunks * p.nheads));
  hipLaunchKernelGGL((ssd_state_kernel<IO, N>), grid, dim3(kSsdThreads), 0, st, p);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL((ssd_cb_kernel<IO, N>), dim3((uint32_t)(p.batch * p.nchunks * p.ngroups * (kQ / 16))),
                     dim3(kSsdThreads), 0, st, p);
  e = hipGetLastError();
  if (e != hipSuccess) return e;
  const int64_t elems = p.batch * p.nheads * kP * N;
  hipLaunchKernelGGL((ssd_pass_kernel<IO>), dim3((uint32_t)((elems + 255) / 256)), dim3(256), 0, st, p);
  e = hipGetLastError();
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL((ssd_scan_kernel<IO, N>), grid, dim3(kSsdThreads), 0, st, p);
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
