// ss_conv.hip -- depthwise causal conv1d + SiLU, the step before the scan (gfx950).
//
// Page "Mamba" (walkthrough), Part IV Stage 2: every channel d has its own
// filter of width W (d_conv, 4 by default), the input is padded on the left
// only, so output t sees inputs t-W+1 .. t, and a SiLU follows:
//   out[b,d,t] = silu(bias[d] + sum_{k<W} w[d,k] x[b,d,t-W+1+k]).
// Inputs before t = 0 come from an optional window conv_init (the last W-1
// inputs of the previous piece of the row), else 0.  With document ids
// ("niverel-mamba" README, "seq_idx strict reset": the convolution state
// resets with the scan's) an input from another document than step t's
// counts as 0.  conv_final receives the last W-1 inputs of each row, the
// window a decode step (ss_conv1d_step) continues from.
//
// The work is a streaming stencil, bound by HBM: one workgroup covers 1024
// consecutive steps of one row, each thread 4 steps 256 apart, so every
// load and store instruction of a wave touches 64 consecutive elements.  The
// W-1 earlier inputs of a step are read again with shifted offsets (they are
// L1/L2 hits), through a range-checked view of the row, so the row's edges
// need no branches.  All arithmetic is fp32.
#include "ss_device.h"
#include "ss_internal.h"

namespace ss {
namespace {

// element m of a small register array, m a runtime index (selects, no scratch)
template <int M>
__device__ __forceinline__ float pick(const float (&a)[M], int m) {
  float v = a[0];
#pragma unroll
  for (int i = 1; i < M; ++i) v = m == i ? a[i] : v;
  return v;
}

constexpr int kConvThreads = 256;
constexpr int kConvPerThread = 4;
constexpr int kConvSpan = kConvThreads * kConvPerThread;  // steps per workgroup

template <int IO, int W, bool SEQ, bool INIT>
__global__ void __launch_bounds__(kConvThreads) ss_conv1d_kernel(ConvParams p) {
  constexpr uint32_t s = io_bytes<IO>();
  const int tid = threadIdx.x;
  // the grid is below 2^23 workgroups: 32-bit index arithmetic (64-bit
  // divisions here delayed every workgroup's first loads)
  const uint32_t tb = (uint32_t)p.tblocks, dim = (uint32_t)p.dim;
  const uint32_t row32 = blockIdx.x / tb;
  const int64_t row = row32;  // b * dim + d
  const int t_base = (int)(blockIdx.x - row32 * tb) * kConvSpan;
  const int L = (int)p.seqlen;
  const uint32_t b32 = row32 / dim;
  const int64_t b = b32, d = row32 - b32 * dim;

  const __amdgpu_buffer_rsrc_t xr = make_rsrc(static_cast<const char*>(p.x) + row * p.seqlen * s, (uint32_t)L * s);
  const __amdgpu_buffer_rsrc_t yr = make_rsrc(static_cast<char*>(p.out) + row * p.seqlen * s, (uint32_t)L * s);
  const __amdgpu_buffer_rsrc_t ids =
      make_rsrc(SEQ ? static_cast<const void*>(p.seq_idx + b * p.seqlen) : p.x, SEQ ? (uint32_t)L * 4u : 0u);

  float w[W];
#pragma unroll
  for (int k = 0; k < W; ++k) w[k] = p.w[d * W + k];
  const float bias = p.bias ? p.bias[d] : 0.0f;
  float init[W > 1 ? W - 1 : 1];
  if constexpr (INIT) {
#pragma unroll
    for (int k = 0; k < W - 1; ++k) init[k] = p.conv_init[row * (W - 1) + k];
  }
  uint32_t first_id = 0;
  if constexpr (SEQ && INIT) first_id = __builtin_amdgcn_raw_buffer_load_b32(ids, 0u, 0, 0);

#pragma unroll
  for (int j = 0; j < kConvPerThread; ++j) {
    const int t = t_base + tid + kConvThreads * j;
    uint32_t id_t = 0;
    if constexpr (SEQ) id_t = __builtin_amdgcn_raw_buffer_load_b32(ids, (uint32_t)t * 4u, 0, 0);
    float pre = bias;
#pragma unroll
    for (int k = 0; k < W; ++k) {
      const int src = t - (W - 1) + k;
      float v = bits_f32<IO>(bload<IO>(xr, (uint32_t)src * s));  // 0 before the row (out of range)
      if constexpr (SEQ) {
        if (k < W - 1) {
          const uint32_t id_s = __builtin_amdgcn_raw_buffer_load_b32(ids, (uint32_t)src * 4u, 0, 0);
          v = (src < 0 || id_s == id_t) ? v : 0.0f;
        }
      }
      if constexpr (INIT) {
        if (k < W - 1) {
          bool use = src < 0;
          if constexpr (SEQ) use = use && id_t == first_id;
          v = use ? pick(init, W - 1 + src) : v;
        }
      }
      pre = fmaf(w[k], v, pre);
    }
    const float y = p.silu ? pre * sigmoid_f(pre) : pre;
    bstore<IO>(yr, t < L ? (uint32_t)t * s : kOffNone, y);
  }

  // the decode window: the row's last W-1 inputs, from the workgroup that ends the row
  if constexpr (W > 1) {
    if (p.conv_final && t_base + kConvSpan >= L && tid < W - 1) {
      const int src = L - (W - 1) + tid;
      float v = bits_f32<IO>(bload<IO>(xr, (uint32_t)src * s));
      if constexpr (SEQ) {
        const uint32_t id_last = __builtin_amdgcn_raw_buffer_load_b32(ids, (uint32_t)(L - 1) * 4u, 0, 0);
        const uint32_t id_s = __builtin_amdgcn_raw_buffer_load_b32(ids, (uint32_t)src * 4u, 0, 0);
        v = (src < 0 || id_s == id_last) ? v : 0.0f;
        if constexpr (INIT) {
          if (src < 0) v = id_last == first_id ? pick(init, W - 1 + src) : 0.0f;
        }
      } else if constexpr (INIT) {
        if (src < 0) v = pick(init, W - 1 + src);
      }
      p.conv_final[row * (W - 1) + tid] = v;
    }
  }
}

// Vector form for rows whose length is a multiple of 8 (every 8-step chunk
// of a row is 16-byte aligned and wholly inside or outside the row): a lane
// covers 8 consecutive steps with one 16-byte load (two for fp32), takes the
// W-1 earlier inputs from the 4 steps before its chunk (an 8-byte / 16-byte
// load that hits L1), and writes its 8 outputs with one 16-byte store (two
// for fp32).  A workgroup covers 2048 steps of one row.
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
constexpr int kVecPerLane = 8;
constexpr int kVecSpan = kConvThreads * kVecPerLane;

template <int IO>
__device__ __forceinline__ void load12(__amdgpu_buffer_rsrc_t r, int t0, float (&v)[12]) {
  // v[i] = x[t0 - 4 + i], i < 12
  if constexpr (IO == SS_F32) {
    const u32x4 a = __builtin_amdgcn_raw_buffer_load_b128(r, (uint32_t)(t0 - 4) * 4u, 0, 0);
    const u32x4 b = __builtin_amdgcn_raw_buffer_load_b128(r, (uint32_t)t0 * 4u, 0, 0);
    const u32x4 c = __builtin_amdgcn_raw_buffer_load_b128(r, (uint32_t)(t0 + 4) * 4u, 0, 0);
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      v[i] = __uint_as_float(a[i]);
      v[4 + i] = __uint_as_float(b[i]);
      v[8 + i] = __uint_as_float(c[i]);
    }
  } else {
    const u32x2 a = __builtin_amdgcn_raw_buffer_load_b64(r, (uint32_t)(t0 - 4) * 2u, 0, 0);
    const u32x4 b = __builtin_amdgcn_raw_buffer_load_b128(r, (uint32_t)t0 * 2u, 0, 0);
#pragma unroll
    for (int i = 0; i < 2; ++i) {
      v[2 * i] = bits_f32<IO>((raw_t<IO>)(a[i] & 0xffffu));
      v[2 * i + 1] = bits_f32<IO>((raw_t<IO>)(a[i] >> 16));
    }
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      v[4 + 2 * i] = bits_f32<IO>((raw_t<IO>)(b[i] & 0xffffu));
      v[4 + 2 * i + 1] = bits_f32<IO>((raw_t<IO>)(b[i] >> 16));
    }
  }
}

template <int IO>
__device__ __forceinline__ uint32_t pack2(float lo, float hi) {
  return (uint32_t)__builtin_bit_cast(uint16_t, from_f32<IO>(lo)) |
         ((uint32_t)__builtin_bit_cast(uint16_t, from_f32<IO>(hi)) << 16);
}

template <int IO>
__device__ __forceinline__ void store8(__amdgpu_buffer_rsrc_t r, int t0, const float (&y)[8]) {
  if constexpr (IO == SS_F32) {
    u32x4 a, b;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      a[i] = __float_as_uint(y[i]);
      b[i] = __float_as_uint(y[4 + i]);
    }
    __builtin_amdgcn_raw_buffer_store_b128(a, r, (uint32_t)t0 * 4u, 0, 0);
    __builtin_amdgcn_raw_buffer_store_b128(b, r, (uint32_t)(t0 + 4) * 4u, 0, 0);
  } else {
    u32x4 a;
#pragma unroll
    for (int i = 0; i < 4; ++i) a[i] = pack2<IO>(y[2 * i], y[2 * i + 1]);
    __builtin_amdgcn_raw_buffer_store_b128(a, r, (uint32_t)t0 * 2u, 0, 0);
  }
}

template <int IO, int W, bool SEQ, bool INIT>
__global__ void __launch_bounds__(kConvThreads) ss_conv1d_vec_kernel(ConvParams p) {
  constexpr uint32_t s = io_bytes<IO>();
  const int tid = threadIdx.x;
  // the grid is below 2^23 workgroups: 32-bit index arithmetic (64-bit
  // divisions here delayed every workgroup's first loads: 20.8 -> 19.8 us on
  // the mamba-130m x branch)
  const uint32_t tb = (uint32_t)p.tblocks, dim = (uint32_t)p.dim;
  const uint32_t row32 = blockIdx.x / tb;
  const int64_t row = row32;
  const int t0 = (int)(blockIdx.x - row32 * tb) * kVecSpan + kVecPerLane * tid;
  const int L = (int)p.seqlen;
  const uint32_t b32 = row32 / dim;
  const int64_t b = b32, d = row32 - b32 * dim;

  const __amdgpu_buffer_rsrc_t xr = make_rsrc(static_cast<const char*>(p.x) + row * p.seqlen * s, (uint32_t)L * s);
  const __amdgpu_buffer_rsrc_t yr = make_rsrc(static_cast<char*>(p.out) + row * p.seqlen * s, (uint32_t)L * s);

  float w[W];
#pragma unroll
  for (int k = 0; k < W; ++k) w[k] = p.w[d * W + k];
  const float bias = p.bias ? p.bias[d] : 0.0f;

  float xv[12];  // x[t0 - 4 .. t0 + 7]; 0 outside the row
  load12<IO>(xr, t0, xv);

  uint32_t idv[12];  // document ids of the same steps
  uint32_t first_id = 0;
  if constexpr (SEQ) {
    const __amdgpu_buffer_rsrc_t ids = make_rsrc(p.seq_idx + b * p.seqlen, (uint32_t)L * 4u);
#pragma unroll
    for (int q = 0; q < 3; ++q) {
      const u32x4 a = __builtin_amdgcn_raw_buffer_load_b128(ids, (uint32_t)(t0 - 4 + 4 * q) * 4u, 0, 0);
#pragma unroll
      for (int i = 0; i < 4; ++i) idv[4 * q + i] = a[i];
    }
    if constexpr (INIT) first_id = __builtin_amdgcn_raw_buffer_load_b32(ids, 0u, 0, 0);
  }
  float init[W > 1 ? W - 1 : 1];
  if constexpr (INIT) {
#pragma unroll
    for (int k = 0; k < W - 1; ++k) init[k] = p.conv_init[row * (W - 1) + k];
  }

  float y[kVecPerLane];
#pragma unroll
  for (int e = 0; e < kVecPerLane; ++e) {
    float pre = bias;
#pragma unroll
    for (int k = 0; k < W; ++k) {
      const int i = 4 + e - (W - 1) + k;  // index into xv / idv (compile-time)
      float v = xv[i];
      if constexpr (SEQ) {
        if (k < W - 1) v = (t0 + i - 4 < 0 || idv[i] == idv[4 + e]) ? v : 0.0f;
      }
      if constexpr (INIT) {
        if (k < W - 1) {
          const int src = t0 + i - 4;
          bool use = src < 0;
          if constexpr (SEQ) use = use && idv[4 + e] == first_id;
          v = use ? pick(init, W - 1 + src) : v;
        }
      }
      pre = fmaf(w[k], v, pre);
    }
    y[e] = p.silu ? pre * sigmoid_f(pre) : pre;
  }
  store8<IO>(yr, t0, y);

  if constexpr (W > 1) {
    if (p.conv_final && t0 + kVecPerLane >= L && t0 < L) {  // the lane holding the row's last step
#pragma unroll
      for (int j = 0; j < W - 1; ++j) {
        const int src = L - (W - 1) + j;
        const int i = src - t0 + 4;  // in 0..11 (L - t0 is 1..8)
        float v = 0.0f;
#pragma unroll
        for (int m = 0; m < 12; ++m) v = m == i ? xv[m] : v;
        if constexpr (SEQ) {
          uint32_t id_s = 0;
#pragma unroll
          for (int m = 0; m < 12; ++m) id_s = m == i ? idv[m] : id_s;
          uint32_t id_last = 0;
#pragma unroll
          for (int m = 4; m < 12; ++m) id_last = m == L - 1 - t0 + 4 ? idv[m] : id_last;
          v = (src < 0 || id_s == id_last) ? v : 0.0f;
          if constexpr (INIT) {
            if (src < 0) v = id_last == first_id ? pick(init, W - 1 + src) : 0.0f;
          }
        } else if constexpr (INIT) {
          if (src < 0) v = pick(init, W - 1 + src);
        }
        p.conv_final[row * (W - 1) + j] = v;
      }
    }
  }
}

// One decode step per (b, d): out = silu(bias + w . [window, x_t]); the
// window drops its oldest input and appends x_t.
template <int IO, int W>
__global__ void __launch_bounds__(256) ss_conv1d_step_kernel(ConvStepParams p) {
  const int64_t ch = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (ch >= p.batch * p.dim) return;
  // batch * dim < 2^31 (the host bounds the grid): a 32-bit remainder, off the
  // 64-bit division's longer path to the weight loads
  const int64_t d = (int64_t)((uint32_t)ch % (uint32_t)p.dim);
  float win[W];
#pragma unroll
  for (int k = 0; k < W - 1; ++k) win[k] = p.window_in[ch * (W - 1) + k];
  win[W - 1] = load_io<IO>(p.x, ch);
  float pre = p.bias ? p.bias[d] : 0.0f;
#pragma unroll
  for (int k = 0; k < W; ++k) pre = fmaf(p.w[d * W + k], win[k], pre);
  store_io<IO>(p.out, ch, p.silu ? pre * sigmoid_f(pre) : pre);
#pragma unroll
  for (int k = 0; k < W - 1; ++k) p.window_out[ch * (W - 1) + k] = win[k + 1];
}

template <int IO, int W, bool SEQ, bool INIT>
void launch_conv_kind(const ConvParams& p, hipStream_t st) {
  if (p.seqlen % kVecPerLane == 0) {
    ConvParams q = p;
    q.tblocks = (p.seqlen + kVecSpan - 1) / kVecSpan;
    hipLaunchKernelGGL((ss_conv1d_vec_kernel<IO, W, SEQ, INIT>), dim3((uint32_t)(p.batch * p.dim * q.tblocks)),
                       dim3(kConvThreads), 0, st, q);
  } else {
    hipLaunchKernelGGL((ss_conv1d_kernel<IO, W, SEQ, INIT>), dim3((uint32_t)(p.batch * p.dim * p.tblocks)),
                       dim3(kConvThreads), 0, st, p);
  }
}

template <int IO, int W>
hipError_t launch_conv_w(const ConvParams& p, hipStream_t st) {
  const bool seq = p.seq_idx != nullptr, init = p.conv_init != nullptr && W > 1;
  if (seq && init) launch_conv_kind<IO, W, true, true>(p, st);
  else if (seq) launch_conv_kind<IO, W, true, false>(p, st);
  else if (init) launch_conv_kind<IO, W, false, true>(p, st);
  else launch_conv_kind<IO, W, false, false>(p, st);
  return hipGetLastError();
}

template <int IO>
hipError_t launch_conv_io(const ConvParams& p, hipStream_t st) {
  switch (p.width) {
    case 1: return launch_conv_w<IO, 1>(p, st);
    case 2: return launch_conv_w<IO, 2>(p, st);
    case 3: return launch_conv_w<IO, 3>(p, st);
    default: return launch_conv_w<IO, 4>(p, st);
  }
}

template <int IO>
hipError_t launch_conv_step_io(const ConvStepParams& p, hipStream_t st) {
  const dim3 grid((uint32_t)((p.batch * p.dim + 255) / 256));
  switch (p.width) {
    case 1: hipLaunchKernelGGL((ss_conv1d_step_kernel<IO, 1>), grid, dim3(256), 0, st, p); break;
    case 2: hipLaunchKernelGGL((ss_conv1d_step_kernel<IO, 2>), grid, dim3(256), 0, st, p); break;
    case 3: hipLaunchKernelGGL((ss_conv1d_step_kernel<IO, 3>), grid, dim3(256), 0, st, p); break;
    default: hipLaunchKernelGGL((ss_conv1d_step_kernel<IO, 4>), grid, dim3(256), 0, st, p); break;
  }
  return hipGetLastError();
}

}  // namespace

int64_t conv_tblocks(int64_t seqlen) { return (seqlen + kConvSpan - 1) / kConvSpan; }

hipError_t launch_conv(const ConvParams& p, hipStream_t st) {
  switch (p.io) {
    case SS_F32: return launch_conv_io<SS_F32>(p, st);
    case SS_F16: return launch_conv_io<SS_F16>(p, st);
    default: return launch_conv_io<SS_BF16>(p, st);
  }
}

hipError_t launch_conv_step(const ConvStepParams& p, hipStream_t st) {
  switch (p.io) {
    case SS_F32: return launch_conv_step_io<SS_F32>(p, st);
    case SS_F16: return launch_conv_step_io<SS_F16>(p, st);
    default: return launch_conv_step_io<SS_BF16>(p, st);
  }
}

}  // namespace ss
