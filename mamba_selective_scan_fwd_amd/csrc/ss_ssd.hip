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

// ---- pass 1: the chunk's own state S_c[p][n] = sum_j w_j x_j[p] B_j[n] ----
template <int IO, int N>
__global__ void __launch_bounds__(kSsdThreads) ssd_state_kernel(SsdParams p) {
  using M = mfma_t<IO>;
  constexpr int kXR = kJB + 8;  // padded LDS row (16-bit elements) of the transposed tiles
  __shared__ float sDelta[kQ], sCs[kQ], sWave[4];
  __shared__ uint16_t sXT[kP][kXR];  // (x * w)^T of one 64-step piece: [p][j]
  __shared__ uint16_t sBT[N][kXR];   // B^T of the piece: [n][j]
  const int tid = threadIdx.x, lane = tid % 64, wave = tid / 64;
  const int64_t h = blockIdx.x % p.nheads;
  const int64_t c = (blockIdx.x / p.nheads) % p.nchunks;
  const int64_t b = blockIdx.x / (p.nheads * p.nchunks);
  const int64_t g = h / (p.nheads / p.ngroups);
  const float A = p.A[h];
  chunk_cumsum<IO>(p, b, c, h, A, sDelta, sCs, sWave);
  const float cs_last = sCs[kQ - 1];

  f32x4 acc[N / 16];
#pragma unroll
  for (int i = 0; i < N / 16; ++i) acc[i] = f32x4{0.0f, 0.0f, 0.0f, 0.0f};

  for (int jb = 0; jb < kQ; jb += kJB) {
    // stage: thread covers step j = jb + tid / 4, 16 of the 64 headdim lanes and N/4 states
    {
      const int jj = tid / 4, part = tid % 4;
      const int64_t t = c * kQ + jb + jj;
      const bool ok = t < p.seqlen;
      const float w = ok ? exp2_hw((cs_last - sCs[jb + jj]) * kLog2e) * sDelta[jb + jj] : 0.0f;
#pragma unroll
      for (int q = 0; q < 16; ++q) {
        const int pp = part * 16 + q;
        const float xv = ok ? load_io<IO>(p.x, ((b * p.seqlen + t) * p.nheads + h) * kP + pp) : 0.0f;
        sXT[pp][jj] = bits16<IO>(xv * w);
      }
#pragma unroll
      for (int q = 0; q < N / 4; ++q) {
        const int n = part * (N / 4) + q;
        const float bv = ok ? load_io<IO>(p.Bm, ((b * p.seqlen + t) * p.ngroups + g) * N + n) : 0.0f;
        sBT[n][jj] = bits16<IO>(bv);
      }
    }
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

// ---- pass 3: outputs of a chunk -------------------------------------------------
template <int IO, int N>
__global__ void __launch_bounds__(kSsdThreads) ssd_scan_kernel(SsdParams p) {
  using M = mfma_t<IO>;
  constexpr int kXR = kJB + 8;
  constexpr int kMR = kJB + 8;
  __shared__ float sDelta[kQ], sCs[kQ], sWave[4];
  __shared__ uint16_t sXT[kP][kXR];              // x^T of one 64-step piece: [p][j]
  __shared__ uint16_t sM[4][64][kMR];            // per wave: masked, decayed C B^T block [i][j]
  const int tid = threadIdx.x, lane = tid % 64, wave = tid / 64;
  const int64_t h = blockIdx.x % p.nheads;
  const int64_t c = (blockIdx.x / p.nheads) % p.nchunks;
  const int64_t b = blockIdx.x / (p.nheads * p.nchunks);
  const int64_t g = h / (p.nheads / p.ngroups);
  const float A = p.A[h];
  chunk_cumsum<IO>(p, b, c, h, A, sDelta, sCs, sWave);

  const int row0 = 64 * wave;  // this wave's 64 rows (steps) of the chunk
  const int64_t t0 = c * kQ;
  // C fragment of row tile mt, k step ks: C[t][n], n = ks + 8 (lane / 16) .. + 7
  auto load_c = [&](int mt, int ks) -> u32x4v {
    const int64_t t = t0 + row0 + 16 * mt + lane % 16;
    if (t >= p.seqlen) return u32x4v{0u, 0u, 0u, 0u};
    const char* base = static_cast<const char*>(p.Cm) + (((b * p.seqlen + t) * p.ngroups + g) * N + ks + 8 * (lane / 16)) * 2;
    return *reinterpret_cast<const u32x4v*>(base);
  };

  // Y starts as Y_off = diag(exp(cs_i)) C H_in: acc[mt][nt], rows i = row0 + 16 mt + 4 (lane/16) + r, col p = 16 nt + lane%16
  f32x4 acc[4][4];
#pragma unroll
  for (int mt = 0; mt < 4; ++mt)
#pragma unroll
    for (int nt = 0; nt < 4; ++nt) acc[mt][nt] = f32x4{0.0f, 0.0f, 0.0f, 0.0f};
  {
    const uint16_t* Hin = p.ws_entry + ((b * p.nchunks + c) * p.nheads + h) * (int64_t)(kP * N);
#pragma unroll
    for (int ks = 0; ks < N; ks += 32) {
      u32x4v bfrag[4];
#pragma unroll
      for (int nt = 0; nt < 4; ++nt)  // B[k = n][col = p] = H_in[p][n]: 8 consecutive n
        bfrag[nt] = *reinterpret_cast<const u32x4v*>(Hin + (16 * nt + lane % 16) * N + ks + 8 * (lane / 16));
#pragma unroll
      for (int mt = 0; mt < 4; ++mt) {
        const u32x4v a = load_c(mt, ks);
#pragma unroll
        for (int nt = 0; nt < 4; ++nt) acc[mt][nt] = M::run(as_vec<IO>(a), as_vec<IO>(bfrag[nt]), acc[mt][nt]);
      }
    }
#pragma unroll
    for (int mt = 0; mt < 4; ++mt)
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const float sc = exp2_hw(sCs[row0 + 16 * mt + 4 * (lane / 16) + r] * kLog2e);
#pragma unroll
        for (int nt = 0; nt < 4; ++nt) acc[mt][nt][r] *= sc;
      }
  }

  // Y_diag: column pieces jb <= row0 (causal), all waves stage every piece
  for (int jb = 0; jb < kQ; jb += kJB) {
    {  // stage x^T of the piece: thread covers step jb + tid / 4 and 16 headdim lanes
      const int jj = tid / 4, part = tid % 4;
      const int64_t t = t0 + jb + jj;
      const bool ok = t < p.seqlen;
#pragma unroll
      for (int q = 0; q < 16; ++q) {
        const int pp = part * 16 + q;
        sXT[pp][jj] = ok ? bits16<IO>(load_io<IO>(p.x, ((b * p.seqlen + t) * p.nheads + h) * kP + pp)) : (uint16_t)0;
      }
    }
    __syncthreads();
    if (jb <= row0) {
      // C B^T block: rows i of this wave x the piece's 64 columns j
      f32x4 cb[4][4];
#pragma unroll
      for (int mt = 0; mt < 4; ++mt)
#pragma unroll
        for (int nt = 0; nt < 4; ++nt) cb[mt][nt] = f32x4{0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
      for (int ks = 0; ks < N; ks += 32) {
        u32x4v bfrag[4];
#pragma unroll
        for (int nt = 0; nt < 4; ++nt) {  // B[k = n][col = j] = B_j[n]
          const int64_t t = t0 + jb + 16 * nt + lane % 16;
          bfrag[nt] = t < p.seqlen ? *reinterpret_cast<const u32x4v*>(
                                         static_cast<const char*>(p.Bm) +
                                         (((b * p.seqlen + t) * p.ngroups + g) * N + ks + 8 * (lane / 16)) * 2)
                                   : u32x4v{0u, 0u, 0u, 0u};
        }
#pragma unroll
        for (int mt = 0; mt < 4; ++mt) {
          const u32x4v a = load_c(mt, ks);
#pragma unroll
          for (int nt = 0; nt < 4; ++nt) cb[mt][nt] = M::run(as_vec<IO>(a), as_vec<IO>(bfrag[nt]), cb[mt][nt]);
        }
      }
      // mask and decay: M[i][j] = CB[i][j] exp(cs_i - cs_j) Delta_j for j <= i, into LDS as [i][j]
#pragma unroll
      for (int nt = 0; nt < 4; ++nt) {
        const int j = jb + 16 * nt + lane % 16;
        const float csj = sCs[j], dj = sDelta[j];
#pragma unroll
        for (int mt = 0; mt < 4; ++mt)
#pragma unroll
          for (int r = 0; r < 4; ++r) {
            const int i = row0 + 16 * mt + 4 * (lane / 16) + r;
            const float m = j <= i ? cb[mt][nt][r] * exp2_hw((sCs[i] - csj) * kLog2e) * dj : 0.0f;
            sM[wave][16 * mt + 4 * (lane / 16) + r][16 * nt + lane % 16] = bits16<IO>(m);
          }
      }
      __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
      __builtin_amdgcn_wave_barrier();
      __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
      // Y += M (64 x 64, A from LDS) x^T-piece (B from LDS)
#pragma unroll
      for (int ks = 0; ks < kJB; ks += 32) {
        const int k0 = ks + 8 * (lane / 16);
        u32x4v bfrag[4];
#pragma unroll
        for (int nt = 0; nt < 4; ++nt) bfrag[nt] = *reinterpret_cast<const u32x4v*>(&sXT[16 * nt + lane % 16][k0]);
#pragma unroll
        for (int mt = 0; mt < 4; ++mt) {
          const u32x4v a = *reinterpret_cast<const u32x4v*>(&sM[wave][16 * mt + lane % 16][k0]);
#pragma unroll
          for (int nt = 0; nt < 4; ++nt) acc[mt][nt] = M::run(as_vec<IO>(a), as_vec<IO>(bfrag[nt]), acc[mt][nt]);
        }
      }
    }
    __syncthreads();
  }

  // D skip, gate, store
  const float Dh = p.D ? p.D[h] : 0.0f;
#pragma unroll
  for (int mt = 0; mt < 4; ++mt)
#pragma unroll
    for (int r = 0; r < 4; ++r) {
      const int64_t t = t0 + row0 + 16 * mt + 4 * (lane / 16) + r;
      if (t >= p.seqlen) continue;
#pragma unroll
      for (int nt = 0; nt < 4; ++nt) {
        const int64_t idx = ((b * p.seqlen + t) * p.nheads + h) * kP + 16 * nt + lane % 16;
        float yv = fmaf(Dh, load_io<IO>(p.x, idx), acc[mt][nt][r]);
        if (p.z) yv *= silu_f(load_io<IO>(p.z, idx));
        store_io<IO>(p.y, idx, yv);
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
